// ffn_mfma.hip — grouped int8 MFMA GEMMs of the prompt-chunk expert FFN over
// Q4_K experts (tokens grouped per expert; "Strata - the details", faster
// prompts: quantized expert kernels instead of FP16 expansion; one activation
// quantization per token, the "Strata-Sage-A1.5-GGUF" card's round-2 table).
//
// Arithmetic.  With activations quantized per (token, 256-block) as x = xd*xq
// and a Q4_K row block w = d*sc_j*q - dmin*m_j (sub-block j of 32 weights):
//   sum_k w_k x_k = xd * ( d * sum_j sc_j * S_j  -  dmin * sum_j m_j * X_j )
//   S_j = sum_{k in j} q_k xq_k,   X_j = sum_{k in j} xq_k.
// The 6-bit sub-block scale varies every 32 weights, so it cannot leave the
// K loop.  It is split into two 3-bit limbs, sc = 8*sh + sl, and the weights
// enter the int8 MFMA as the bytes q*sl and q*sh (both <= 105): two MFMAs per
// 32-deep K chunk, accumulated exactly in int32 over a 256-wide block, then
// acc_l + 8*acc_h is scaled once per block by d*xd in fp32.  The min term is a
// K = H/32 contraction: an fp16 MFMA of the per-32 activation sums X_j*xd
// (precomputed per token, fp16) with -dmin*m_j (fp16), added to the same fp32
// accumulators.
//
// MFMA layouts (v_mfma_i32_32x32x32_i8 and v_mfma_f32_32x32x16_f16): lane l
// supplies row l%32 of A (tokens) and column l%32 of B (weight rows); both use
// the same K positions for the same lane half and register byte; the result
// C[m][n] sits in lane n + 32*((m/4)%2), register 4*(m/8) + m%4.
//
// Work.  A tile is (expert, 32*MTILES tokens of its bucket); each tile is cut
// into 256-row blocks of the output.  Workgroups of 8 waves take one (tile,
// block); each wave owns 32 output rows (gate/up: the same 32 rows of both
// matrices, so SiLU(gate)*up is formed in registers).  The tile's activations
// sit in LDS for the whole K loop; weights stream from global memory straight
// into registers.  Work items are laid out (expert, token tile, block) and
// dealt to the 8 XCDs in contiguous ranges, so workgroups that share an
// expert's weights share an L2.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

constexpr int kMWaves = 8;
constexpr int kMThreads = kMWaves * kWave;
constexpr int kLdsPad = 16;  // bytes after each LDS row: consecutive rows start 4 banks apart
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t pk_mul_u16(uint32_t a, uint32_t b) {
    const v2u16 x = __builtin_bit_cast(v2u16, a), y = __builtin_bit_cast(v2u16, b);
    return __builtin_bit_cast(uint32_t, (v2u16)(x * y));
}

// Max / sum over the 32 lanes of a wave half (the same result in all of them).
__device__ __forceinline__ float half32_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
}

__device__ __forceinline__ int half32_sum(int v) {
    v += (int)dpp_u<0xB1>((uint32_t)v);
    v += (int)dpp_u<0x4E>((uint32_t)v);
    v += (int)dpp_u<0x141>((uint32_t)v);
    v += (int)dpp_u<0x140>((uint32_t)v);
    return v + __builtin_amdgcn_ds_swizzle(v, 0x401F);
}

// Work item of this workgroup: tile u and 256-row block nb.  Items are dealt
// to XCDs (blockIdx.x % 8) in contiguous ranges.  Returns false when idle.
__device__ __forceinline__ bool work_item(const int32_t* n_tiles, int nblocks, int& u, int& nb) {
    const int n_work = (*n_tiles) * nblocks;
    const int chunk = (n_work + kXcds - 1) / kXcds;
    const int xcd = blockIdx.x % kXcds, s = blockIdx.x / kXcds;
    if (s >= chunk) return false;
    const int w = xcd * chunk + s;
    if (w >= n_work) return false;
    u = w / nblocks;
    nb = w - u * nblocks;
    return true;
}

// Output row index of A-tile row m: token m of the tile (C-layout row of
// register v in this lane half).
__device__ __forceinline__ int c_row(int mt, int v, int h) { return mt * 32 + 8 * (v >> 2) + 4 * h + (v & 3); }

// Smallest power of two >= x (x finite, > 0); 1 otherwise.
__device__ __forceinline__ float pow2_ceil(float x) {
    if (!(x > 0.0f) || !(x < INFINITY)) return 1.0f;
    const uint32_t b = __float_as_uint(x);
    if ((b & 0x7FFFFFu) == 0 && (b >> 23) != 0) return x;
    const uint32_t e = (b >> 23) + 1;  // subnormal x: e = 1, i.e. 2^-126
    return e >= 255 ? 1.0f : __uint_as_float(e << 23);
}

// Q4_K x int8 grouped GEMM core.  For each of NT weight rows per lane
// (rowp[nt], a row of nsb Q4_K blocks) and the A tile in LDS (32*MTILES rows of
// int8, stride lda; per-256 scales xd_s[b*MT + m]; per-row power-of-two scales
// s_sc[m] and their inverses s_inv[m]; per-32 code sums in global memory, row
// pointer sums[mt] or null), sets
//   out[nt][mt][v] = sum_k w[n][k] * a[m][k]     (C layout).
template <int NT, int MTILES>
__device__ __forceinline__ void q4k_i8_core(const uint8_t* const* rowp, int nsb, const int8_t* lds_a, int lda,
                                            const float* xd_s, const float* s_sc, const float* s_inv,
                                            const int16_t* const* sums, v16f (&out)[NT][MTILES]) {
    constexpr int MT = 32 * MTILES;
    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane & 31, h = lane >> 5;
    const int8_t* a_lane = lds_a + n * lda + 16 * h;

#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) out[nt][mt][v] = 0.0f;

    // min term, two 256-blocks per MFMA (lane half h takes block 2*s2 + h):
    //   out = sum_{b,j} (-dmin_b m_bj / t) * (X_bj xd_b / s),  then out *= s * t,
    // with s a power of two per token row (>= its largest xd) and t one per
    // weight row (>= 63 * its largest dmin), so both operands stay within fp16
    // range.  Each operand is carried as an fp16 pair hi + lo (hi*hi + hi*lo +
    // lo*hi), which keeps the term to about 2^-22 relative.
    float t_sc[NT], t_inv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float mx = 0.0f;
        for (int b = 0; b < nsb; ++b)
            mx = fmaxf(mx, f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(rowp[nt] + (int64_t)b * 144 + 2)));
        t_sc[nt] = pow2_ceil(63.0f * mx);
        t_inv[nt] = 1.0f / t_sc[nt];
    }
    for (int s2 = 0; s2 < (nsb + 1) / 2; ++s2) {
        const int b = 2 * s2 + h;
        const bool ok = b < nsb;
        v8h Ah[MTILES], Al[MTILES];
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) {
            v8h z = {};
            Ah[mt] = z;
            Al[mt] = z;
            const int m = mt * 32 + n;
            if (ok && sums[mt]) {
                const uint4 raw = *reinterpret_cast<const uint4*>(sums[mt] + 8 * b);
                const float f = xd_s[b * MT + m] * s_inv[m];
                const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int16_t xs = (int16_t)((w4[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
                    const float av = (float)xs * f;
                    const _Float16 ah = (_Float16)av;
                    Ah[mt][i] = ah;
                    Al[mt][i] = (_Float16)(av - (float)ah);
                }
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            v8h Bh = {}, Bl = {};
            if (ok) {
                const uint4 v = *reinterpret_cast<const uint4*>(rowp[nt] + (int64_t)b * 144);
                const Q4KHead hh{v.x, v.y, v.z, v.w};
                const float dmin = q4k_dmin(hh);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    int sc, mn;
                    q4k_scale_min(hh, j, sc, mn);
                    const float bv = -(dmin * (float)mn) * t_inv[nt];
                    const _Float16 bh = (_Float16)bv;
                    Bh[j] = bh;
                    Bl[j] = (_Float16)(bv - (float)bh);
                }
            }
#pragma unroll
            for (int mt = 0; mt < MTILES; ++mt) {
                out[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah[mt], Bh, out[nt][mt], 0, 0, 0);
                out[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ah[mt], Bl, out[nt][mt], 0, 0, 0);
                out[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Al[mt], Bh, out[nt][mt], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 s4 = *reinterpret_cast<const float4*>(s_sc + mt * 32 + 8 * g + 4 * h);
            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) out[nt][mt][4 * g + r] *= sv[r] * t_sc[nt];
        }
    }

    for (int b = 0; b < nsb; ++b) {
        Q4KHead hd[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const uint4 v = *reinterpret_cast<const uint4*>(rowp[nt] + (int64_t)b * 144);
            hd[nt] = Q4KHead{v.x, v.y, v.z, v.w};
        }
        v16i accl[NT][MTILES], acch[NT][MTILES];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
                for (int v = 0; v < 16; ++v) accl[nt][mt][v] = acch[nt][mt][v] = 0;

#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint4 raw[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                raw[nt] = *reinterpret_cast<const uint4*>(rowp[nt] + (int64_t)b * 144 + 16 + 32 * c + 16 * h);
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                const int j = 2 * c + hi;
                v4i A[MTILES];
#pragma unroll
                for (int mt = 0; mt < MTILES; ++mt)
                    A[mt] = *reinterpret_cast<const v4i*>(a_lane + mt * 32 * lda + 256 * b + 32 * j);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    int sc, mn;
                    q4k_scale_min(hd[nt], j, sc, mn);
                    const uint32_t sl = (uint32_t)(sc & 7) * 0x10001u, sh = (uint32_t)(sc >> 3) * 0x10001u;
                    const uint32_t w4[4] = {raw[nt].x, raw[nt].y, raw[nt].z, raw[nt].w};
                    v4i Bl, Bh;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t q = (hi ? (w4[i] >> 4) : w4[i]) & 0x0F0F0F0Fu;
                        Bl[i] = (int)pk_mul_u16(q, sl);
                        Bh[i] = (int)pk_mul_u16(q, sh);
                    }
#pragma unroll
                    for (int mt = 0; mt < MTILES; ++mt) {
                        accl[nt][mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[mt], Bl, accl[nt][mt], 0, 0, 0);
                        acch[nt][mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[mt], Bh, acch[nt][mt], 0, 0, 0);
                    }
                }
            }
        }
        // scale the block: out += (acc_l + 8 acc_h) * d * xd
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 x4 = *reinterpret_cast<const float4*>(xd_s + b * MT + mt * 32 + 8 * g + 4 * h);
                const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const float d = q4k_d(hd[nt]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int v = 4 * g + r;
                        const int sm = accl[nt][mt][v] + (acch[nt][mt][v] << 3);
                        out[nt][mt][v] = fmaf((float)sm, d * xv[r], out[nt][mt][v]);
                    }
                }
            }
        }
    }
}

// Per-row scales of the min-term operand (threads < MT).
template <int MT>
__device__ __forceinline__ void row_scales(const float* xd_s, int nsb, float* s_sc, float* s_inv) {
    const int m = threadIdx.x;
    if (m >= MT) return;
    float mx = 0.0f;
    for (int b = 0; b < nsb; ++b) mx = fmaxf(mx, xd_s[b * MT + m]);
    const float sc = pow2_ceil(mx);
    s_sc[m] = sc;
    s_inv[m] = 1.0f / sc;
}

// Loads the A tile: rows src_row[m] (or zeros when < 0) of an int8 matrix with
// K columns, and their per-256 scales, into LDS.
template <int MTILES>
__device__ __forceinline__ void load_a_tile(const int8_t* __restrict__ q, const float* __restrict__ qd, int K,
                                            const int* s_src, int8_t* lds_a, int lda, float* xd_s) {
    constexpr int MT = 32 * MTILES;
    const int per_row = K / 16;
    for (int idx = threadIdx.x; idx < MT * per_row; idx += blockDim.x) {
        const int m = idx / per_row, c = idx - m * per_row;
        const int src = s_src[m];
        uint4 v = make_uint4(0, 0, 0, 0);
        if (src >= 0) v = *reinterpret_cast<const uint4*>(q + (int64_t)src * K + 16 * c);
        *reinterpret_cast<uint4*>(lds_a + m * lda + 16 * c) = v;
    }
    const int nsb = K / 256;
    for (int idx = threadIdx.x; idx < MT * nsb; idx += blockDim.x) {
        const int b = idx / MT, m = idx - b * MT;
        const int src = s_src[m];
        xd_s[b * MT + m] = src >= 0 ? qd[(int64_t)src * nsb + b] : 0.0f;
    }
}

// Rows of tile u: A-source row (token for gate/up, h row for down) and output
// row (pair id, or T*k + t for the shared expert), -1 when past the bucket.
template <int MT>
__device__ __forceinline__ void tile_rows(const MfmaArgs& a, int e, int m0, bool down, int* s_src, int* s_out) {
    const int tid = threadIdx.x;
    if (tid >= MT) return;
    const int npairs = a.T * a.k;
    int src = -1, orow = -1;
    if (e == a.E) {
        const int t = m0 + tid;
        if (t < a.T) {
            orow = npairs + t;
            src = down ? orow : t;
        }
    } else {
        const int p0 = a.offset[e], p1 = a.offset[e + 1];
        if (p0 < 0 || p1 < p0 || p1 > npairs) {
            if (tid == 0) raise_error(kErrPairRange);
        } else if (p0 + m0 + tid < p1) {
            const int p = a.pair[p0 + m0 + tid];
            if (p < 0 || p >= npairs) {
                raise_error(kErrPairRange);
            } else {
                orow = p;
                src = down ? p : p / a.k;
            }
        }
    }
    s_src[tid] = src;
    s_out[tid] = orow;
}

template <int MTILES>
__global__ void __launch_bounds__(kMThreads) gateup_mfma_kernel(MfmaArgs a) {
    constexpr int MT = 32 * MTILES;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ int s_src[MT], s_out[MT];
    __shared__ float s_red[kMWaves * MT];
    __shared__ __attribute__((aligned(16))) float s_id[MT];
    __shared__ float s_d[MT];
    __shared__ __attribute__((aligned(16))) float s_sc[MT];
    __shared__ float s_inv[MT];

    const int H = a.H, I = a.I, NB = I / 256;
    int u, nb;
    if (!work_item(a.n_tiles, NB, u, nb)) return;
    const int e = a.tile_e[u], m0 = a.tile_m0[u];
    const bool shared = (e == a.E);
    tile_rows<MT>(a, e, m0, false, s_src, s_out);
    __syncthreads();

    const int lda = H + kLdsPad;
    int8_t* lds_a = reinterpret_cast<int8_t*>(lds);
    float* xd_s = reinterpret_cast<float*>(lds + MT * lda);
    load_a_tile<MTILES>(a.xq, a.xd, H, s_src, lds_a, lda, xd_s);
    __syncthreads();
    row_scales<MT>(xd_s, H / 256, s_sc, s_inv);
    __syncthreads();

    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int n = lane & 31, h = lane >> 5;
    const int i = nb * 256 + wave * 32 + n;  // row of gate and up (column of h)
    const QMat G = shared ? a.sgate : a.gate, U = shared ? a.sup : a.up;
    const int64_t eo = shared ? 0 : (int64_t)e;
    const uint8_t* rowp[2] = {G.data + eo * G.expert_bytes + (int64_t)i * G.row_bytes,
                              U.data + eo * U.expert_bytes + (int64_t)i * U.row_bytes};
    const int16_t* sums[MTILES];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
        const int src = s_src[mt * 32 + n];
        sums[mt] = src >= 0 ? a.xs + (int64_t)src * (H / 32) : nullptr;
    }
    v16f acc[2][MTILES];
    q4k_i8_core<2, MTILES>(rowp, H / 256, lds_a, lda, xd_s, s_sc, s_inv, sums, acc);

    // h = silu(g) * u, then per-token amax over the 256 rows of this block
    float hv[MTILES][16];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float hh = silu_f32(acc[0][mt][v]) * acc[1][mt][v];
            hv[mt][v] = hh;
            float am = isfinite(hh) ? fabsf(hh) : INFINITY;
            am = half32_max(am);
            if (n == 0) s_red[wave * MT + c_row(mt, v, h)] = am;
        }
    }
    __syncthreads();
    if (threadIdx.x < MT) {
        const int m = threadIdx.x;
        float am = 0.0f;
        for (int w = 0; w < kMWaves; ++w) am = fmaxf(am, s_red[w * MT + m]);
        float id = 0.0f, d = 0.0f;
        if (!(am < INFINITY)) {
            if (s_out[m] >= 0) raise_error(kErrActNonFinite);
        } else if (am > 0.0f) {
            id = __fdiv_rn(127.0f, am);
            d = __fdiv_rn(am, 127.0f);
        }
        s_id[m] = id;
        s_d[m] = d;
        if (s_out[m] >= 0) a.hd[(int64_t)s_out[m] * NB + nb] = d;
    }
    __syncthreads();
    const int I32 = I / 32;
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 i4 = *reinterpret_cast<const float4*>(s_id + mt * 32 + 8 * g + 4 * h);
            const float iv[4] = {i4.x, i4.y, i4.z, i4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int v = 4 * g + r;
                const int m = c_row(mt, v, h);
                int q = 0;
                if (iv[r] != 0.0f) {
                    float qf = rintf(__fmul_rn(hv[mt][v], iv[r]));
                    qf = fminf(fmaxf(qf, -127.0f), 127.0f);
                    q = (int)qf;
                }
                const int orow = s_out[m];
                if (orow >= 0) a.hq[(int64_t)orow * I + i] = (int8_t)q;
                const int qs = half32_sum(q);
                if (n == 0 && orow >= 0) a.hs[(int64_t)orow * I32 + nb * 8 + wave] = (int16_t)qs;
            }
        }
    }
}

template <int MTILES>
__global__ void __launch_bounds__(kMThreads) down_mfma_kernel(MfmaArgs a) {
    constexpr int MT = 32 * MTILES;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ int s_src[MT], s_out[MT];
    __shared__ __attribute__((aligned(16))) float s_sc[MT];
    __shared__ float s_inv[MT];

    const int H = a.H, I = a.I, NB = H / 256;
    int u, ob;
    if (!work_item(a.n_tiles, NB, u, ob)) return;
    const int e = a.tile_e[u], m0 = a.tile_m0[u];
    const bool shared = (e == a.E);
    tile_rows<MT>(a, e, m0, true, s_src, s_out);
    __syncthreads();

    const int lda = I + kLdsPad;
    int8_t* lds_a = reinterpret_cast<int8_t*>(lds);
    float* hd_s = reinterpret_cast<float*>(lds + MT * lda);
    load_a_tile<MTILES>(a.hq, a.hd, I, s_src, lds_a, lda, hd_s);
    __syncthreads();
    row_scales<MT>(hd_s, I / 256, s_sc, s_inv);
    __syncthreads();

    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int n = lane & 31, h = lane >> 5;
    const int o = ob * 256 + wave * 32 + n;
    const QMat D = shared ? a.sdown : a.down;
    const int64_t eo = shared ? 0 : (int64_t)e;
    const uint8_t* rowp[1] = {D.data + eo * D.expert_bytes + (int64_t)o * D.row_bytes};
    const int16_t* sums[MTILES];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
        const int src = s_src[mt * 32 + n];
        sums[mt] = src >= 0 ? a.hs + (int64_t)src * (I / 32) : nullptr;
    }
    v16f acc[1][MTILES];
    q4k_i8_core<1, MTILES>(rowp, I / 256, lds_a, lda, hd_s, s_sc, s_inv, sums, acc);

    const int npairs = a.T * a.k;
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int orow = s_out[c_row(mt, v, h)];
            if (orow < 0) continue;
            if (orow < npairs)
                a.y_pair[(int64_t)orow * H + o] = acc[0][mt][v];
            else
                a.y_shared[(int64_t)(orow - npairs) * H + o] = acc[0][mt][v];
        }
    }
}

// xs[t][c] = sum_{l<32} xq[t][32c + l] (exact, |xs| <= 4064), one thread per (t, c).
__global__ void __launch_bounds__(256) act_sums_kernel(const int8_t* __restrict__ xq, int64_t n, int K,
                                                       int16_t* __restrict__ xs) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n) return;
    const int k32 = K / 32;
    const int64_t t = idx / k32;
    const int c = (int)(idx - t * k32);
    const uint4* p = reinterpret_cast<const uint4*>(xq + t * K + 32 * c);
    const uint4 v0 = p[0], v1 = p[1];
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int bsh = 0; bsh < 32; bsh += 8) s += (int)(int8_t)(w[i] >> bsh);
    xs[idx] = (int16_t)s;
}

// Tile list: tiles of 'mt' bucket entries per expert with count > 0, in
// ascending expert order, then the shared expert's tiles (e == E).
__global__ void __launch_bounds__(1024) mfma_tiles_kernel(const int32_t* __restrict__ count, int E, int T,
                                                          int npairs, int has_shared, int mt, int max_t,
                                                          int32_t* __restrict__ tile_e,
                                                          int32_t* __restrict__ tile_m0,
                                                          int32_t* __restrict__ n_tiles) {
    __shared__ int s_wave[kWave + 1];
    const int tid = threadIdx.x;
    int c = tid < E ? count[tid] : 0;
    if (c < 0 || c > npairs) {
        raise_error(kErrPairRange);
        c = 0;
    }
    const int nt = (c + mt - 1) / mt;
    int total = 0;
    const int start = block_exclusive_scan(nt, s_wave, total);
    // counts that sum past T*k cannot come from a routing call; never write past the list
    for (int i = 0; i < nt && start + i < max_t; ++i) {
        tile_e[start + i] = tid;
        tile_m0[start + i] = i * mt;
    }
    const int ns = has_shared ? (T + mt - 1) / mt : 0;
    for (int i = tid; i < ns && total + i < max_t; i += blockDim.x) {
        tile_e[total + i] = E;
        tile_m0[total + i] = i * mt;
    }
    if (tid == 0) {
        if (total + ns > max_t) raise_error(kErrPairRange);
        *n_tiles = min(total + ns, max_t);
    }
}

template <int MTILES>
size_t gateup_lds(int H) {
    return (size_t)(32 * MTILES) * (H + kLdsPad) + (size_t)(H / 256) * 32 * MTILES * sizeof(float);
}

int max_tiles(int T, int k, int E, int has_shared, int mt) {
    const int npairs = T * k;
    return (npairs + mt - 1) / mt + (E < npairs ? E : npairs) + (has_shared ? (T + mt - 1) / mt : 0);
}

unsigned grid_for(int works) { return (unsigned)((works + kXcds - 1) / kXcds * kXcds); }

template <int MTILES>
hipError_t launch_mfma_path(const MfmaArgs& a, hipStream_t s) {
    constexpr int MT = 32 * MTILES;
    const int maxt = max_tiles(a.T, a.k, a.E, a.has_shared, MT);
    mfma_tiles_kernel<<<1, 1024, 0, s>>>(a.count, a.E, a.T, a.T * a.k, a.has_shared, MT, maxt, a.tile_e,
                                         a.tile_m0, a.n_tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n_sums = (int64_t)a.T * (a.H / 32);
    act_sums_kernel<<<(unsigned)((n_sums + 255) / 256), 256, 0, s>>>(a.xq, n_sums, a.H, a.xs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    gateup_mfma_kernel<MTILES><<<grid_for(maxt * (a.I / 256)), kMThreads, gateup_lds<MTILES>(a.H), s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    down_mfma_kernel<MTILES><<<grid_for(maxt * (a.H / 256)), kMThreads, gateup_lds<MTILES>(a.I), s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool mfma_path_supported(int H, int I, int qg, int qu, int qd) {
    return qg == kQ4_K && qu == kQ4_K && qd == kQ4_K && H <= kMfmaMaxDim && I <= kMfmaMaxDim;
}

int mfma_tile_rows(int H, int I) { return (H <= 2048 && I <= 2048) ? 64 : 32; }

size_t mfma_tiles_bytes(int T, int k, int E, int has_shared, int H, int I) {
    const int mt = mfma_tile_rows(H, I);
    return 2 * sizeof(int32_t) * (size_t)max_tiles(T, k, E, has_shared, mt) + 256;
}

hipError_t launch_ffn_mfma(const MfmaArgs& a, hipStream_t s) {
    if (mfma_tile_rows(a.H, a.I) == 64) return launch_mfma_path<2>(a, s);
    return launch_mfma_path<1>(a, s);
}

}  // namespace moe
