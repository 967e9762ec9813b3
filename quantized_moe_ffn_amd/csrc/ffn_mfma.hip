// ffn_mfma.hip — grouped int8 MFMA GEMMs of the prompt-chunk expert FFN over
// Q4_K and Q5_K experts (tokens grouped per expert; "Strata - the details", faster
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
// acc_l + 8*acc_h is scaled once per block by d*xd in fp32.  The block's min
// term is one K = 16 fp16 MFMA pair: the lane halves carry the same eight
// sub-blocks, as the hi and lo fp16 parts of X_j*xd/s (X_j the exact per-32
// code sums; s a power of two >= the row's largest xd, so the operand stays
// below 4064), against the hi and lo parts of -dmin*m_j (exact); the four
// cross products keep the term to about 2^-22 relative.  1/s is folded into
// the row's block scales, and each finished row is multiplied by s.
//
// MFMA layouts (v_mfma_i32_32x32x32_i8, v_mfma_f32_32x32x16_f16): lane l
// supplies row l%32 of A (tokens) and column l%32 of B (weight rows); both use
// the same K positions for the same lane half and register byte; the result
// C[m][n] sits in lane n + 32*((m/4)%2), register 4*(m/8) + m%4.
//
// Work.  A tile is (expert, 32*MTILES tokens of its bucket).  Gate/up:
// workgroups of 8 waves take (tile, 256 rows of I); each wave owns 32 rows and
// runs them through gate, then up (so SiLU(gate)*up and the requantisation of
// h happen in registers).  Down: workgroups of 4 waves take (tile, 128 or 512
// rows of H), each wave 32 rows per round.  The tile's int8 activations, their per-256
// scales and per-32 sums sit in LDS for the whole K loop; weights stream from
// global memory into registers one 256-block ahead of use.  Work items are
// laid out (expert, token tile, row block) and dealt to the 8 XCDs in
// contiguous ranges, so workgroups that share an expert's weights share an L2.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kMWaves = 8;
constexpr int kMThreads = kMWaves * kWave;
constexpr int kLdsPad = 16;  // bytes after each LDS row: consecutive rows start 4 banks apart
constexpr int kXcds = 8;
constexpr int kHStride = 256 + 4;  // LDS row stride (floats) of the gate/up epilogue's h tile

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

// The A side of a tile in LDS.
struct TileLds {
    const int8_t* a;     // [MT][lda] int8 codes
    const float* xd;     // [nsb][MT] per-256 scales divided by the row's s
    const uint16_t* xs;  // [MT][xs_ld] fp16: hi parts of the K/32 values X*xd/s, then the lo parts
    const float* s;      // [MT] the rows' power-of-two s
    int lda, xs_ld, k32;
};

// Byte j (0..3) of v in both 16-bit halves: (v_j) | (v_j << 16).
__device__ __forceinline__ uint32_t byte_pair(uint32_t v, int j) {
    return __builtin_amdgcn_perm(0u, v, (0x0Cu << 24) | ((uint32_t)j << 16) | (0x0Cu << 8) | (uint32_t)j);
}

// One 256-block of a weight row, as a lane needs it: the 16-byte header and
// its four 16-byte quant slices (lane half h: bytes 32c + 16h .. + 15 of the
// quants); for Q5_K also the 16 fifth-bit bytes of those weights (qh bytes
// 16h .. 16h + 15: byte l holds the fifth bit of the low-nibble weight of
// chunk c in bit 2c and of the high-nibble weight in bit 2c + 1).
template <int QT>
struct MQuant;
template <>
struct MQuant<kQ4_K> {
    static constexpr int kBytes = 144, kQs = 16;
};
template <>
struct MQuant<kQ5_K> {
    static constexpr int kBytes = 176, kQs = 48;
};

struct BlockRegs {
    uint4 hdr;
    uint4 q[4];
    uint4 qh;
};

template <int QT>
__device__ __forceinline__ void load_block(const uint8_t* blk, int h, BlockRegs& r) {
    r.hdr = *reinterpret_cast<const uint4*>(blk);
#pragma unroll
    for (int c = 0; c < 4; ++c) r.q[c] = *reinterpret_cast<const uint4*>(blk + MQuant<QT>::kQs + 32 * c + 16 * h);
    if constexpr (QT == kQ5_K) r.qh = *reinterpret_cast<const uint4*>(blk + 16 + 16 * h);
}

// out[mt] += (this 256-block's contribution) for the lane's weight row and the
// tile's 32*MTILES rows, block index b of the row.
//
// Q5_K: the quants reach 31, and 7*31 does not fit an int8 byte, so the
// weights enter as sc*(q - 16) (limbs in -112..105).  A limb byte s*q (<= 217,
// from the same packed multiply) becomes s*(q - 16) by adding 128 - 16s to
// every byte, which cannot carry since the sum is s*(q - 16) + 128 in 16..233,
// and flipping bit 7 of every byte (the two's complement of the sum minus
// 128).  The 16*sc*X_j it takes away comes back through the min-term MFMA,
// whose weight side becomes 16*d*sc_j - dmin*m_j.
// How a block's products d*xd (the lane's row d against the tile rows' xd) are formed.
enum DxMode : int {
    kDxLanes = 0,      // each lane multiplies them, reading xd from LDS
    kDxRank1Pair = 1,  // one v_mfma_f32_32x32x1f32 for both 32-row tiles (32 result registers)
    kDxRank1Tile = 2,  // one v_mfma_f32_32x32x2f32 per tile (16 result registers)
};

template <int MTILES, int QT, int DX>
__device__ __forceinline__ void block_mma(const BlockRegs& br, int b, const TileLds& T, v16f (&out)[MTILES]) {
    static_assert(MTILES == 1 || MTILES == 2, "tiles of 32 or 64 rows");
    constexpr int MT = 32 * MTILES;
    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane & 31, h = lane >> 5;
    const Q4KHead hd{br.hdr.x, br.hdr.y, br.hdr.z, br.hdr.w};
    const int8_t* a_lane = T.a + n * T.lda + 256 * b + 16 * h;

    // the eight 6-bit scales and mins of the block, packed one per byte
    const uint32_t sc_lo = hd.h1 & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (hd.h3 & 0x0F0F0F0Fu) | ((hd.h1 >> 2) & 0x30303030u);
    const uint32_t mn_lo = hd.h2 & 0x3F3F3F3Fu;
    const uint32_t mn_hi = ((hd.h3 >> 4) & 0x0F0F0F0Fu) | ((hd.h2 >> 2) & 0x30303030u);
    const uint32_t sl4[2] = {sc_lo & 0x07070707u, sc_hi & 0x07070707u};
    const uint32_t sh4[2] = {(sc_lo >> 3) & 0x07070707u, (sc_hi >> 3) & 0x07070707u};

    v16i accl[MTILES], acch[MTILES];
    constexpr bool kFifth = QT == kQ5_K;
    const uint32_t hb4[4] = {br.qh.x, br.qh.y, br.qh.z, br.qh.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t w4[4] = {br.q[c].x, br.q[c].y, br.q[c].z, br.q[c].w};
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
            const int j = 2 * c + hi;
            const uint32_t sl = byte_pair(sl4[j >> 2], j & 3), sh = byte_pair(sh4[j >> 2], j & 3);
            // Q5_K: 128 - 16*s in every byte (s in both 16-bit halves of sl / sh)
            const uint32_t bias_l = kFifth ? 0x80808080u - ((sl | (sl << 8)) << 4) : 0u;
            const uint32_t bias_h = kFifth ? 0x80808080u - ((sh | (sh << 8)) << 4) : 0u;
            v4i Bl, Bh;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t q = (hi ? (w4[i] >> 4) : w4[i]) & 0x0F0F0F0Fu;
                if constexpr (kFifth) {
                    q |= ((hb4[i] >> j) & 0x01010101u) << 4;
                    Bl[i] = (int)((pk_mul_u16(q, sl) + bias_l) ^ 0x80808080u);
                    Bh[i] = (int)((pk_mul_u16(q, sh) + bias_h) ^ 0x80808080u);
                } else {
                    Bl[i] = (int)pk_mul_u16(q, sl);
                    Bh[i] = (int)pk_mul_u16(q, sh);
                }
            }
#pragma unroll
            for (int mt = 0; mt < MTILES; ++mt) {
                const v4i A = *reinterpret_cast<const v4i*>(a_lane + mt * 32 * T.lda + 32 * j);
                if (j == 0) {
                    const v16i z = {};
                    accl[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, Bl, z, 0, 0, 0);
                    acch[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, Bh, z, 0, 0, 0);
                } else {
                    accl[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, Bl, accl[mt], 0, 0, 0);
                    acch[mt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, Bh, acch[mt], 0, 0, 0);
                }
            }
        }
    }

    // min term: out += sum_j (-dmin m_j) (X_j xd / s), hi/lo fp16 pairs; lane
    // half 0 carries the hi parts of X_j xd / s, half 1 the lo parts (Q5_K:
    // 16 d sc_j - dmin m_j, each product exact, their sum rounded once)
    {
        const float dmin = q4k_dmin(hd);
        const float d16 = 16.0f * q4k_d(hd);
        v8h Bmh, Bml;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t mb = j < 4 ? mn_lo : mn_hi;
            float bv = -(dmin * (float)((mb >> (8 * (j & 3))) & 0xFFu));  // exact: 11 x 6 bits
            if constexpr (kFifth) {
                const uint32_t sb = j < 4 ? sc_lo : sc_hi;
                bv = fmaf(d16, (float)((sb >> (8 * (j & 3))) & 0xFFu), bv);
            }
            const _Float16 bh = (_Float16)bv;
            Bmh[j] = bh;
            Bml[j] = (_Float16)(bv - (float)bh);
        }
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) {
            const v8h Am =
                *reinterpret_cast<const v8h*>(T.xs + (mt * 32 + n) * T.xs_ld + h * T.k32 + 8 * b);
            out[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Am, Bmh, out[mt], 0, 0, 0);
            out[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Am, Bml, out[mt], 0, 0, 0);
        }
    }

    // main term: out += (acc_l + 8 acc_h) * (d * xd).  The products d * xd
    // form an outer product, which a rank-1 MFMA returns in the C layout of
    // the int32 accumulators, each product one fp32 multiply rounded once (the
    // bits of the lane's own d * xd).  kDxRank1Pair: v_mfma_f32_32x32x1f32, two
    // 32x32 blocks with K = 1; block mt takes xd of its 32 rows from lanes
    // 32*mt .. 32*mt + 31 and d of row n from lane n + 32*mt, into registers
    // 16*mt .. 16*mt + 15 (with one tile, block 1 repeats block 0, unused).
    // kDxRank1Tile: v_mfma_f32_32x32x2f32 per tile, K = 2 with the second K
    // slice (lanes 32..63) zero, so only 16 result registers are live at once.
    const float d = q4k_d(hd);
    if constexpr (DX == kDxRank1Tile) {
        const v16f z16 = {};
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) {
            const float xa = h ? 0.0f : T.xd[b * MT + mt * 32 + n];
            const v16f dx = __builtin_amdgcn_mfma_f32_32x32x2f32(xa, h ? 0.0f : d, z16, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int sm = accl[mt][v] + (acch[mt][v] << 3);
                out[mt][v] = fmaf((float)sm, dx[v], out[mt][v]);
            }
        }
    } else if constexpr (DX == kDxRank1Pair) {
        const float xa = T.xd[b * MT + (MTILES == 2 ? lane : n)];
        const v32f z32 = {};
        const v32f dx = __builtin_amdgcn_mfma_f32_32x32x1f32(xa, d, z32, 0, 0, 0);
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int sm = accl[mt][v] + (acch[mt][v] << 3);
                out[mt][v] = fmaf((float)sm, dx[16 * mt + v], out[mt][v]);
            }
        }
    } else {
#pragma unroll
        for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 x4 = *reinterpret_cast<const float4*>(T.xd + b * MT + mt * 32 + 8 * g + 4 * h);
                const float xv[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int v = 4 * g + r;
                    const int sm = accl[mt][v] + (acch[mt][v] << 3);
                    out[mt][v] = fmaf((float)sm, d * xv[r], out[mt][v]);
                }
            }
        }
    }
}

// out[mt][v] *= s of its row (C layout), turning the K loop's rows back to scale.
template <int MTILES>
__device__ __forceinline__ void apply_row_scale(const TileLds& T, v16f (&out)[MTILES]) {
    const int h = (threadIdx.x & (kWave - 1)) >> 5;
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 s4 = *reinterpret_cast<const float4*>(T.s + mt * 32 + 8 * g + 4 * h);
            out[mt][4 * g + 0] *= s4.x;
            out[mt][4 * g + 1] *= s4.y;
            out[mt][4 * g + 2] *= s4.z;
            out[mt][4 * g + 3] *= s4.w;
        }
    }
}

// Smallest power of two >= x (x finite, > 0); 1 otherwise.
__device__ __forceinline__ float pow2_ceil(float x) {
    if (!(x > 0.0f) || !(x < INFINITY)) return 1.0f;
    const uint32_t b = __float_as_uint(x);
    if ((b & 0x7FFFFFu) == 0 && (b >> 23) != 0) return x;
    const uint32_t e = (b >> 23) + 1;  // subnormal x: e = 1, i.e. 2^-126
    return e >= 255 ? 1.0f : __uint_as_float(e << 23);
}

// Loads the A side of tile: rows src_row[m] (zeros when < 0) of an int8 matrix
// with K columns, their per-256 scales, and their per-32 code sums.
template <int MTILES>
__device__ __forceinline__ void load_tile(const int8_t* __restrict__ q, const float* __restrict__ qd,
                                          const int16_t* __restrict__ qs, int K, const int* s_src, int8_t* lds_a,
                                          int lda, float* xd_s, uint16_t* xs_s, int xs_ld, float* s_sc) {
    constexpr int MT = 32 * MTILES;
    constexpr int kBatch = 8;
    const int tid = threadIdx.x, nthr = blockDim.x;
    // codes: thread -> (row m0 + j*rows_per_pass, 16-byte column c); K/16 <= 224 < nthr
    {
        const int per_row = K / 16;
        const int rows_per_pass = nthr / per_row;
        const int c = tid % per_row, m0 = tid / per_row;
        if (m0 < rows_per_pass) {
            for (int mb = m0; mb < MT; mb += kBatch * rows_per_pass) {
                // every load of the batch is issued before any is used: rows past
                // the bucket load row 0 and store zeros (a select at the store,
                // not a branch after each load, which would wait for it)
                uint4 v[kBatch];
                bool pad[kBatch];
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const int m = min(mb + i * rows_per_pass, MT - 1);
                    const int src = s_src[m];
                    pad[i] = src < 0;
                    v[i] = *reinterpret_cast<const uint4*>(q + (int64_t)max(src, 0) * K + 16 * c);
                }
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const int m = mb + i * rows_per_pass;
                    const uint32_t keep = pad[i] ? 0u : ~0u;
                    const uint4 w = make_uint4(v[i].x & keep, v[i].y & keep, v[i].z & keep, v[i].w & keep);
                    if (m < MT) *reinterpret_cast<uint4*>(lds_a + m * lda + 16 * c) = w;
                }
            }
        }
    }
    // per-256 scales [b][m], then each row's s and the scales divided by it
    const int nsb = K / 256;
    for (int idx = tid; idx < MT * nsb; idx += nthr) {
        const int b = idx / MT, m = idx % MT;
        const int src = s_src[m];
        xd_s[b * MT + m] = src >= 0 ? qd[(int64_t)src * nsb + b] : 0.0f;
    }
    __syncthreads();
    if (tid < MT) {
        float mx = 0.0f;
        for (int b = 0; b < nsb; ++b) mx = fmaxf(mx, xd_s[b * MT + tid]);
        const float sv = pow2_ceil(mx), inv = 1.0f / sv;  // powers of two: exact
        s_sc[tid] = sv;
        for (int b = 0; b < nsb; ++b) xd_s[b * MT + tid] *= inv;
    }
    __syncthreads();
    // per-32 values X*xd/s as fp16 hi/lo pairs: [m][0 .. K/32) hi, [m][K/32 .. 2K/32) lo.
    // A thread takes the eight sums of one 256-block of one row (one 16-byte
    // load; K/32 is a multiple of 8 and the rows start 16-byte aligned), all
    // scaled by that block's xd/s.
    const int k32 = K / 32, k256 = K / 256;
    for (int idx = tid; idx < MT * k256; idx += nthr) {
        const int m = idx / k256, b = idx - m * k256;
        const int src = s_src[m];
        const uint4 raw = *reinterpret_cast<const uint4*>(qs + (int64_t)max(src, 0) * k32 + 8 * b);
        const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
        const float sc = xd_s[b * MT + m];
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int16_t sv = (int16_t)(rw[t >> 1] >> (16 * (t & 1)));
            const float xv = src >= 0 ? (float)sv : 0.0f;
            const float v = xv * sc;
            const _Float16 vh = (_Float16)v;
            const uint32_t bh = __builtin_bit_cast(uint16_t, vh);
            const uint32_t bl = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)vh));
            if (t & 1) {
                hi[t >> 1] |= bh << 16;
                lo[t >> 1] |= bl << 16;
            } else {
                hi[t >> 1] = bh;
                lo[t >> 1] = bl;
            }
        }
        *reinterpret_cast<uint4*>(xs_s + m * xs_ld + 8 * b) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(xs_s + m * xs_ld + k32 + 8 * b) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
}

// LDS bytes of a tile's A side (dynamic part) for K columns.
template <int MTILES>
constexpr size_t tile_lds_bytes(int K) {
    return (size_t)(32 * MTILES) * (K + kLdsPad) + (size_t)(K / 256) * 32 * MTILES * sizeof(float) +
           (size_t)(32 * MTILES) * (2 * (K / 32) + 8) * sizeof(uint16_t);
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

// Carves the dynamic LDS into the tile's A side.
template <int MTILES>
__device__ __forceinline__ TileLds carve(unsigned char* lds, int K, const float* s_sc, int8_t*& a, float*& xd,
                                         uint16_t*& xs) {
    constexpr int MT = 32 * MTILES;
    const int lda = K + kLdsPad, xs_ld = 2 * (K / 32) + 8;
    a = reinterpret_cast<int8_t*>(lds);
    xd = reinterpret_cast<float*>(lds + (size_t)MT * lda);
    xs = reinterpret_cast<uint16_t*>(lds + (size_t)MT * lda + (size_t)(K / 256) * MT * sizeof(float));
    return TileLds{a, xd, xs, s_sc, lda, xs_ld, K / 32};
}

template <int MTILES, int QG>
__global__ void __launch_bounds__(kMThreads) gateup_mfma_kernel(MfmaArgs a) {
    constexpr int MT = 32 * MTILES;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ int s_src[MT], s_out[MT];
    __shared__ __attribute__((aligned(16))) float s_sc[MT];

    const int H = a.H, I = a.I, NB = I / 256, nsb = H / 256;
    int u, nb;
    if (!work_item(a.n_tiles, NB, u, nb)) return;
    const int e = a.tile_e[u], m0 = a.tile_m0[u];
    const bool shared = (e == a.E);
    tile_rows<MT>(a, e, m0, false, s_src, s_out);
    __syncthreads();

    int8_t* lds_a;
    float* xd_s;
    uint16_t* xs_s;
    const TileLds T = carve<MTILES>(lds, H, s_sc, lds_a, xd_s, xs_s);
    load_tile<MTILES>(a.xq, a.xd, a.xs, H, s_src, lds_a, T.lda, xd_s, xs_s, T.xs_ld, s_sc);
    __syncthreads();

    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int n = lane & 31, h = lane >> 5;
    const int i = nb * 256 + wave * 32 + n;  // row of gate and up (column of h)
    const QMat G = shared ? a.sgate : a.gate, U = shared ? a.sup : a.up;
    const int64_t eo = shared ? 0 : (int64_t)e;
    const uint8_t* rows[2] = {G.data + eo * G.expert_bytes + (int64_t)i * G.row_bytes,
                              U.data + eo * U.expert_bytes + (int64_t)i * U.row_bytes};

    // gate row, then up row: 2*nsb blocks, one block of prefetch
    v16f acc[MTILES], g_out[MTILES];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mt][v] = 0.0f;
    // blocks s = 0 .. 2*nsb-1 (gate row, then up row), loaded two ahead of use
    auto blk_ptr = [&](int sx) {
        const int r = sx >= nsb ? 1 : 0;
        return rows[r] + (int64_t)(sx - r * nsb) * MQuant<QG>::kBytes;
    };
    const int steps = 2 * nsb;
    auto step = [&](const BlockRegs& br, int sx) {
        block_mma<MTILES, QG, kDxRank1Pair>(br, sx >= nsb ? sx - nsb : sx, T, acc);
        if (sx == nsb - 1) {
            apply_row_scale<MTILES>(T, acc);
#pragma unroll
            for (int mt = 0; mt < MTILES; ++mt) {
                g_out[mt] = acc[mt];
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mt][v] = 0.0f;
            }
        }
    };
    // two register buffers alternate through a 2x unrolled loop (no copies of
    // registers that loads in flight still write); steps is even, so the body
    // has no conditional steps and the compiler can interleave them
    BlockRegs b0, b1;
    load_block<QG>(blk_ptr(0), h, b0);
    for (int s = 0; s < steps; s += 2) {
        load_block<QG>(blk_ptr(s + 1), h, b1);
        step(b0, s);
        load_block<QG>(blk_ptr(min(s + 2, steps - 1)), h, b0);
        step(b1, s + 1);
    }

    apply_row_scale<MTILES>(T, acc);
    // h = silu(g) * u goes through LDS (the tile is no longer needed), so that
    // each thread then owns one (token, 32-row block): the token's amax over
    // the 256 rows is a reduction over 8 neighbouring lanes, and the codes of
    // a block and their sum stay in one thread
    __syncthreads();
    float* s_h = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            s_h[c_row(mt, v, h) * kHStride + wave * 32 + n] = silu_f32(g_out[mt][v]) * acc[mt][v];
    __syncthreads();
    const int m = threadIdx.x >> 3, c32 = threadIdx.x & 7;
    if (m < MT) {   // whole waves past the tile's rows stay idle
        float hv[32];
        const float4* src = reinterpret_cast<const float4*>(s_h + m * kHStride + c32 * 32);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float4 f4 = src[j];
            hv[4 * j] = f4.x;
            hv[4 * j + 1] = f4.y;
            hv[4 * j + 2] = f4.z;
            hv[4 * j + 3] = f4.w;
        }
        bool fin = true;
        float am = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            fin = fin && isfinite(hv[j]);
            am = fmaxf(am, fabsf(hv[j]));
        }
        am = fin ? am : INFINITY;
        am = fmaxf(am, dpp_f<0xB1>(am));    // the token's 8 threads: quad swaps,
        am = fmaxf(am, dpp_f<0x4E>(am));
        am = fmaxf(am, dpp_f<0x141>(am));   // then the half-row mirror
        const int orow = s_out[m];
        float id = 0.0f, d = 0.0f;
        if (!(am < INFINITY)) {
            if (orow >= 0 && c32 == 0) raise_error(kErrActNonFinite);
        } else if (am > 0.0f) {
            id = __fdiv_rn(127.0f, am);
            d = __fdiv_rn(am, 127.0f);
        }
        uint32_t packed[8];
        int qsum = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t w = 0;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                int q = 0;
                if (id != 0.0f) q = (int)fminf(fmaxf(rintf(__fmul_rn(hv[4 * j + bb], id)), -127.0f), 127.0f);
                qsum += q;
                w |= ((uint32_t)q & 0xFFu) << (8 * bb);
            }
            packed[j] = w;
        }
        if (orow >= 0) {
            uint4* dst = reinterpret_cast<uint4*>(a.hq + (uint32_t)(orow * I + nb * 256 + c32 * 32));
            dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
            dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
            a.hs[(uint32_t)(orow * (I / 32) + nb * 8 + c32)] = (int16_t)qsum;
            if (c32 == 0) a.hd[(uint32_t)(orow * NB + nb)] = d;
        }
    }
}

constexpr int kDownRoundsMax = 4;  // 128-row rounds per down workgroup (large batches)
// Waves of a down workgroup.  Four (not eight) let a CU hold three workgroups,
// so each SIMD runs three waves instead of two: the down tile's LDS footprint
// (~39 KB at 64 tokens) allows it, and its registers stay within 168.
constexpr int kDownWaves = 4;

// PAIR16: the per-pair outputs go to y_pair_bf16 as bf16 (nearest even), not to y_pair.
template <int MTILES, int QD, bool PAIR16>
__global__ void __launch_bounds__(kDownWaves * kWave, MTILES == 1 ? 4 : 3) down_mfma_kernel(MfmaArgs a) {
    constexpr int MT = 32 * MTILES;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ int s_src[MT], s_out[MT];
    __shared__ __attribute__((aligned(16))) float s_sc[MT];
    __shared__ __attribute__((aligned(16))) int s_off[MT];  // element offset of the row's output, -1 past the bucket

    const int H = a.H, I = a.I, nsb = I / 256;
    constexpr int RR = 32 * kDownWaves;  // output rows per round: 32 per wave
    const int R = a.down_rounds;
    const int NB = (H / RR + R - 1) / R;
    int u, ob;
    if (!work_item(a.n_tiles, NB, u, ob)) return;
    const int e = a.tile_e[u], m0 = a.tile_m0[u];
    const bool shared = (e == a.E);
    tile_rows<MT>(a, e, m0, true, s_src, s_out);
    __syncthreads();
    const int npairs = a.T * a.k;
    // a tile is all routed pairs (rows of y_pair) or all shared-expert tokens
    // (rows T*k + t, stored as rows t of y_shared)
    if (threadIdx.x < MT) {
        const int orow = s_out[threadIdx.x];
        s_off[threadIdx.x] = orow >= 0 ? (orow - (shared ? npairs : 0)) * H : -1;
    }

    int8_t* lds_a;
    float* hd_s;
    uint16_t* hs_s;
    const TileLds T = carve<MTILES>(lds, I, s_sc, lds_a, hd_s, hs_s);
    load_tile<MTILES>(a.hq, a.hd, a.hs, I, s_src, lds_a, T.lda, hd_s, hs_s, T.xs_ld, s_sc);
    __syncthreads();

    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int n = lane & 31, h = lane >> 5;
    const QMat D = shared ? a.sdown : a.down;
    const int64_t eo = shared ? 0 : (int64_t)e;
    const int r0 = ob * R;
    const int nr = min(R, H / RR - r0);
    const uint8_t* base = D.data + eo * D.expert_bytes + (int64_t)(r0 * RR + wave * 32 + n) * D.row_bytes;
    const int64_t round_stride = (int64_t)RR * D.row_bytes;

    v16f acc[MTILES];
#pragma unroll
    for (int mt = 0; mt < MTILES; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mt][v] = 0.0f;
    auto blk_ptr = [&](int sx) {
        const int r = sx / nsb;
        return base + r * round_stride + (int64_t)(sx - r * nsb) * MQuant<QD>::kBytes;
    };
    const int steps = nr * nsb;
    auto step = [&](const BlockRegs& br, int sx) {
        const int r = sx / nsb, b = sx - r * nsb;
        block_mma<MTILES, QD, MTILES == 2 ? kDxRank1Tile : kDxLanes>(br, b, T, acc);
        if (b == nsb - 1) {
            apply_row_scale<MTILES>(T, acc);
            const int o = (r0 + r) * RR + wave * 32 + n;
#pragma unroll
            for (int mt = 0; mt < MTILES; ++mt) {
                // the output offsets of the lane's 16 rows (C layout: four runs
                // of four consecutive rows), read together
                int off[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int4 o4 = *reinterpret_cast<const int4*>(s_off + mt * 32 + 8 * g + 4 * h);
                    off[4 * g + 0] = o4.x;
                    off[4 * g + 1] = o4.y;
                    off[4 * g + 2] = o4.z;
                    off[4 * g + 3] = o4.w;
                }
                if (shared) {
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (off[v] >= 0) a.y_shared[(uint32_t)(off[v] + o)] = acc[mt][v];
                } else if constexpr (PAIR16) {
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (off[v] >= 0)
                            a.y_pair_bf16[(uint32_t)(off[v] + o)] = __builtin_bit_cast(uint16_t, (__bf16)acc[mt][v]);
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (off[v] >= 0) a.y_pair[(uint32_t)(off[v] + o)] = acc[mt][v];
                }
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[mt][v] = 0.0f;
            }
        }
    };
    BlockRegs b0, b1;
    load_block<QD>(blk_ptr(0), h, b0);
    int s = 0;
    for (; s + 1 < steps; s += 2) {
        load_block<QD>(blk_ptr(s + 1), h, b1);
        step(b0, s);
        load_block<QD>(blk_ptr(min(s + 2, steps - 1)), h, b0);
        step(b1, s + 1);
    }
    if (s < steps) step(b0, s);
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

// Tile list of a caller's routing (write_tile_list: 'mt' bucket entries per
// tile, experts in ascending order, then the shared expert's tiles, e == E).
__global__ void __launch_bounds__(1024) mfma_tiles_kernel(const int32_t* __restrict__ count, int E, int npairs,
                                                          TileList tl) {
    __shared__ int s_wave[kWave + 1];
    __shared__ int s_start[1024];
    const int tid = threadIdx.x;
    write_tile_list(tid < E ? count[tid] : 0, npairs, E, tl, s_wave, s_start);
}


int max_tiles(int T, int k, int E, int has_shared, int mt) {
    const int npairs = T * k;
    return (npairs + mt - 1) / mt + (E < npairs ? E : npairs) + (has_shared ? (T + mt - 1) / mt : 0);
}

unsigned grid_for(int works) { return (unsigned)((works + kXcds - 1) / kXcds * kXcds); }

template <int MTILES, int QD>
hipError_t launch_down(const MfmaArgs& a, int maxt, hipStream_t s) {
    constexpr int RR = 32 * kDownWaves;
    // rounds of RR output rows per down workgroup: four amortise the tile's LDS
    // load over 512 rows when there are work items to spare; small batches (a
    // few tokens per expert, few tiles) take one round so that the grid covers
    // the CUs
    MfmaArgs d = a;
    const int rounds_all = a.H / RR;
    d.down_rounds =
        (int64_t)maxt * ((rounds_all + kDownRoundsMax - 1) / kDownRoundsMax) >= 1024 ? kDownRoundsMax : 1;
    const int nb_down = (rounds_all + d.down_rounds - 1) / d.down_rounds;
    const dim3 gd(grid_for(maxt * nb_down));
    if (a.y_pair_bf16)
        down_mfma_kernel<MTILES, QD, true><<<gd, kDownWaves * kWave, tile_lds_bytes<MTILES>(a.I), s>>>(d);
    else
        down_mfma_kernel<MTILES, QD, false><<<gd, kDownWaves * kWave, tile_lds_bytes<MTILES>(a.I), s>>>(d);
    return hipGetLastError();
}

template <int MTILES, int QG, int QD>
hipError_t launch_mfma_path(const MfmaArgs& a, hipStream_t s) {
    constexpr int MT = 32 * MTILES;
    const int maxt = max_tiles(a.T, a.k, a.E, a.has_shared, MT);
    hipError_t e;
    if (!a.tiles_ready) {
        const TileList tl{a.tile_e, a.tile_m0, a.n_tiles, MT, maxt, a.T, a.has_shared};
        mfma_tiles_kernel<<<1, 1024, 0, s>>>(a.count, a.E, a.T * a.k, tl);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (!a.xs_ready) {
        const int64_t n_sums = (int64_t)a.T * (a.H / 32);
        act_sums_kernel<<<(unsigned)((n_sums + 255) / 256), 256, 0, s>>>(a.xq, n_sums, a.H, a.xs);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const size_t lds_gu = std::max(tile_lds_bytes<MTILES>(a.H), (size_t)MT * kHStride * sizeof(float));
    gateup_mfma_kernel<MTILES, QG><<<grid_for(maxt * (a.I / 256)), kMThreads, lds_gu, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_down<MTILES, QD>(a, maxt, s);
}

template <int MTILES, int QG>
hipError_t launch_mfma_qd(const MfmaArgs& a, hipStream_t s) {
    return a.down.qtype == kQ5_K ? launch_mfma_path<MTILES, QG, kQ5_K>(a, s) : launch_mfma_path<MTILES, QG, kQ4_K>(a, s);
}

template <int MTILES>
hipError_t launch_mfma_q(const MfmaArgs& a, hipStream_t s) {
    return a.gate.qtype == kQ5_K ? launch_mfma_qd<MTILES, kQ5_K>(a, s) : launch_mfma_qd<MTILES, kQ4_K>(a, s);
}

}  // namespace

// Gate and up in one of Q4_K and Q5_K (the same for both), down in either.
bool mfma_path_supported(int H, int I, int qg, int qu, int qd) {
    const bool kq_g = (qg == kQ4_K || qg == kQ5_K) && qu == qg;
    const bool kq_d = qd == kQ4_K || qd == kQ5_K;
    return kq_g && kq_d && H <= kMfmaMaxDim && I <= kMfmaMaxDim;
}

// The kernels index h and y rows with 32-bit element offsets.
bool mfma_rows_fit(int T, int k, int H, int I) {
    const int64_t rows = (int64_t)T * k + T;
    return rows * (H > I ? H : I) < ((int64_t)1 << 31);
}

// Tokens per tile: 64 when the LDS holds them (H, I <= 2048) and the experts
// average more than 32 tokens; else 32, so a batch of a few tokens per expert
// does not pay the MFMA and VALU work of 64 mostly empty rows.
int mfma_tile_rows(int T, int k, int E, int H, int I) {
    return (H <= 2048 && I <= 2048 && (int64_t)T * k > 32 * (int64_t)E) ? 64 : 32;
}

size_t mfma_tiles_bytes(int T, int k, int E, int has_shared, int H, int I) {
    const int mt = mfma_tile_rows(T, k, E, H, I);
    return 2 * sizeof(int32_t) * (size_t)max_tiles(T, k, E, has_shared, mt) + 256;
}

hipError_t launch_ffn_mfma(const MfmaArgs& a, hipStream_t s) {
    if (mfma_tile_rows(a.T, a.k, a.E, a.H, a.I) == 64) return launch_mfma_q<2>(a, s);
    return launch_mfma_q<1>(a, s);
}

}  // namespace moe
