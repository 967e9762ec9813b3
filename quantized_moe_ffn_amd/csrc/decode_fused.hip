// decode_fused.hip — the decode-sized layer (T <= 8 tokens, T*k <= 64) in two
// kernels:
//
//   K1 route + gate/up + SiLU: every wave recomputes the top-k of its token
//      from the router logits and issues the weight loads of each slot as soon
//      as the extraction round that names its expert ends; each workgroup
//      streams a tile of gate and up rows for up to two slots of one token
//      (or the shared expert for up to four tokens) and writes
//      h = silu(W_gate x) * (W_up x).  One extra workgroup writes the routing
//      results (idx, w, count, offset, pair, active, n_active) and a compact
//      table of the selected experts and weights for K2.
//   K2 down + combine: a workgroup owns a tile of output rows for every slot
//      of the layer (one slot per wave), so the routing-weighted sum over the k
//      slots (plus the shared expert) is formed in LDS in slot order and
//      written once: no float atomics, bitwise deterministic.
//
// Two launches per layer instead of four: on MI355X a small kernel costs a few
// microseconds of launch and drain, as much as streaming the ~14 MB of experts
// one Sage-A1.5-sized token touches ("Strata-Sage-A1.5-GGUF": 256 experts,
// top-8; Flash-Next, "Strata: a 125B MoE at 94 tok/s": 10 routed + 1 shared of
// 512).  The pages' own decode work moved the same way: fewer launches and
// host round trips in the verify pass ("Strata v0.1.39" release notes, Decode
// #646), register reductions in the decode chain ("Strata-Sage-A1.5-GGUF"
// round-2 table).
//
// Weight streaming (K1): a "slice" is 16 quant bytes of a Q4_K super-block =
// 16 weights of sub-block 2c (low nibbles) and 16 of sub-block 2c+1 (high
// nibbles); a Q5_K slice adds the 16 bytes holding those weights' fifth bits;
// a Q8_0 or Q5_1 row's lane takes one 34- or 24-byte block (32 weights) instead.  A unit of W
// waves covers P rows x (8*NB) slices per pass with
// 64*W == P*8*NB, so every lane keeps the same 32 columns for the whole kernel
// and holds those activations in registers (no LDS traffic for x).  Per slice a
// lane issues two 16-byte loads (super-block header + quants), decodes the two
// 6-bit scale/min pairs it needs and applies them once per 16 weights:
//   partial = d*(sc_lo*S_lo + sc_hi*S_hi) - dmin*(m_lo*X_lo + m_hi*X_hi).
#include <atomic>

#include "common.h"
#include "kernels.h"
#include "qblock.h"

namespace moe {

constexpr int kDecMaxT = 8;      // tokens handled by the fused decode path
constexpr int kShTok = 4;        // tokens per shared-expert group of the gate/up kernel
constexpr int kDecMaxPairs = 64; // T*k

template <int A, int B>
struct Gcd {
    static constexpr int value = Gcd<B, A % B>::value;
};
template <int A>
struct Gcd<A, 0> {
    static constexpr int value = A;
};

// Routing of up to kDecMaxT tokens: the expert and weight of every pair
// p = t*k + j in slot order.  One workgroup of K1 computes it and hands it to
// K2 through the workspace.
struct DecRoute {
    int sel[kDecMaxPairs];
    float w[kDecMaxPairs];
    float sg[kDecMaxT];   // sigmoid gate of the shared expert per token (when the layer has one)
};

static_assert(sizeof(DecRoute) <= kDecRouteTabBytes, "routing table size");

// Wave w selects the top-k of tokens w, w + nwaves, ...  Ends with __syncthreads().
template <int V>
__device__ __forceinline__ void dec_route(const float* __restrict__ logits, int T, int E, int k, int renorm, DecRoute& R) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int nwaves = blockDim.x / kWave;
    for (int t = wave; t < T; t += nwaves) {
        int e = -1;
        float w = 0.f;
        wave_topk<V>(logits + (int64_t)t * E, E, k, renorm != 0, e, w);
        if (lane < k) {
            R.sel[t * k + lane] = e;
            R.w[t * k + lane] = w;
        }
    }
    __syncthreads();
}

// The publishing workgroup of K1 writes the routing results in the layout
// moe_route_topk writes (active experts ascending, pairs grouped by expert).
__device__ __forceinline__ void dec_publish(const DecRoute& R, int T, int E, int k, const RoutingPtrs& r) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int P = T * k;
    if (wave == 0) {
        const int ep = lane < P ? R.sel[lane] : 0x7FFFFFFF;
        int below, same_before, ubelow, n_uniq;
        bool first;
        wave_buckets(ep, P, below, same_before, first, ubelow, n_uniq);
        if (lane < P) {
            r.idx[lane] = ep;
            r.w[lane] = R.w[lane];
            r.pair[below + same_before] = lane;
            if (first) r.active[ubelow] = ep;
        }
        if (lane == 0) *r.n_active = n_uniq;
    }
    for (int x = threadIdx.x; x <= E; x += blockDim.x) {
        int below = 0, cnt = 0;
        for (int q = 0; q < P; ++q) {
            below += (R.sel[q] < x);
            cnt += (R.sel[q] == x);
        }
        r.offset[x] = below;
        if (x < E) r.count[x] = cnt;
    }
}

// ---------------------------------------------------------------------------
// K1: route + gate/up + SiLU.
// ---------------------------------------------------------------------------
template <int NB, int PASSES>
struct K1Shape {
    static constexpr int G = Gcd<NB, 8>::value;
    static constexpr int W = NB / G;                       // waves per unit
    static constexpr int P = 8 / G;                        // rows per pass per unit
    static constexpr int UNITS = (4 + W - 1) / W;          // at least 4 waves (one per token)
    static constexpr int THREADS = 64 * W * UNITS;
    static constexpr int SLICES = 8 * NB;                  // slices per row
    static constexpr int ROWS = P * UNITS * PASSES;        // rows of the tile
    static constexpr bool IN_WAVE = (W == 1);              // a row's slices live in one wave
    static constexpr int GROUPS = IN_WAVE ? 1 : SLICES / 16;  // 16-lane groups per row otherwise
};

// Per-lane constants of the slice decode.  They are hidden from the compiler
// (an empty asm that claims to change them) so that it keeps the byte masks as
// written: a masked word then converts with one v_cvt_f32_ubyteN per weight
// instead of a bit-field extract plus a conversion.
//   scale word of the slice's sub-blocks: ((h1 >> sa) & ma) | (h3 & mb),
//   min word:                             ((h2 >> sa) & ma) | ((h3 >> 4) & mb),
// each holding the 6-bit values of sub-blocks 0-3 (c < 2) or 4-7 (c >= 2) in
// its bytes; sub-blocks 2c, 2c+1 are bytes 2(c%2), 2(c%2)+1, brought down by sh.
// For Q5_K also: the fifth bits of the slice's low- and high-nibble weights
// are bits 2c and 2c+1 of its qh bytes (f_lo, f_hi), isolated by m_one.
// A Q8_0 lane uses only sel8 and dsh8 (see q8_block_dot).
struct SliceKit {
    uint32_t m_lo, m_hi, sa, ma, mb, sh, f_lo, f_hi, m_one, sel8, dsh8;
};

// (the fifth-bit fields are kept only where a Q5_K slice uses them: three
// more live registers push some Q4_K kernels past an occupancy step)
template <bool kFifth = false>
__device__ __forceinline__ SliceKit slice_kit(int part) {
    const bool upper = part >= 4;
    const uint32_t c = (uint32_t)(part >> 1);
    SliceKit k{0x0F0F0F0Fu, 0xF0F0F0F0u, upper ? 2u : 0u, upper ? 0x30303030u : 0x3F3F3F3Fu,
               upper ? 0x0F0F0F0Fu : 0u, 8u * (uint32_t)(part & 2), 2u * c, 2u * c + 1u, 0x01010101u, 0u, 0u};
    asm volatile("" : "+v"(k.m_lo), "+v"(k.m_hi), "+v"(k.sa), "+v"(k.ma), "+v"(k.mb), "+v"(k.sh));
    if constexpr (kFifth) asm volatile("" : "+v"(k.f_lo), "+v"(k.f_hi), "+v"(k.m_one));
    return k;
}

// Super-block geometry of the k-quant formats the fused kernels stream: the
// block size and where a slice's 16 quant bytes start (Q4_K: after the 16-byte
// header; Q5_K: after the header and the 32 fifth-bit bytes).  A Q5_K slice
// also needs the 16 fifth-bit bytes of its weights, at 16 + 16*(part & 1).
template <int QT>
struct KQuant;
template <>
struct KQuant<kQ4_K> {
    static constexpr int kBytes = 144, kQs = 16;
    static constexpr bool kFifth = false;
};
template <>
struct KQuant<kQ5_K> {
    static constexpr int kBytes = 176, kQs = 48;
    static constexpr bool kFifth = true;
};

// The registers one slice takes: for a k-quant the super-block header, the 16
// quant bytes and, for Q5_K, the 16 fifth-bit bytes; for Q8_0 the nine dwords
// that hold the lane's 34-byte block.
struct KSlice {
    uint4 hdr, q, hb;
};

// Lane sl of a row: a k-quant row has 8 slices per 256-weight super-block
// (super-block sl/8, part sl%8); a Q8_0 row has one 32-weight block per lane
// (block sl, columns 32*sl .. 32*sl + 31).  Both give H/32 lanes per row.
// (Q5_1 rows, 24-byte blocks of 32 weights, are laid out per lane as Q8_0's.)
template <int QT>
constexpr bool kBlock32 = (QT == kQ8_0 || QT == kQ5_1);

template <int QT>
__device__ __forceinline__ int kslice_block_off(int sl) {
    if constexpr (QT == kQ8_0)
        return 34 * sl;
    else if constexpr (QT == kQ5_1)
        return 24 * sl;
    else
        return (sl >> 3) * KQuant<QT>::kBytes;
}

// First column of the lane's low and high halves (16 weights each).
template <int QT>
__device__ __forceinline__ int kslice_col_lo(int sl) {
    if constexpr (kBlock32<QT>)
        return 32 * sl;
    else
        return 256 * (sl >> 3) + q4k_slice_col_lo(sl & 7);
}
template <int QT>
__device__ __forceinline__ int kslice_col_hi(int sl) {
    if constexpr (kBlock32<QT>)
        return 32 * sl + 16;
    else
        return 256 * (sl >> 3) + q4k_slice_col_hi(sl & 7);
}

// A Q8_0 block sits at 34*sl bytes into a row whose start is 4-byte aligned,
// so it starts 2 bytes past a dword boundary exactly when sl is odd: the
// selector of v_perm_b32 that brings its quants into place, and the half of
// the first dword holding d.
template <int QT>
__device__ __forceinline__ SliceKit kslice_kit(int sl) {
    if constexpr (QT == kQ8_0) {
        SliceKit k{};
        const bool odd = (sl & 1) != 0;
        k.sel8 = odd ? 0x07060504u : 0x05040302u;
        k.dsh8 = odd ? 16u : 0u;
        return k;
    } else if constexpr (QT == kQ5_1) {
        return SliceKit{};
    } else {
        return slice_kit<KQuant<QT>::kFifth>(sl & 7);
    }
}

// blk = row start + kslice_block_off<QT>(sl)
template <int QT>
__device__ __forceinline__ void kslice_load(const uint8_t* blk, int sl, KSlice& r) {
    if constexpr (QT == kQ8_0) {
        const uint32_t* dw = reinterpret_cast<const uint32_t*>((uintptr_t)blk & ~(uintptr_t)3);
        r.hdr = make_uint4(dw[0], dw[1], dw[2], dw[3]);
        r.q = make_uint4(dw[4], dw[5], dw[6], dw[7]);
        r.hb = make_uint4(dw[8], 0u, 0u, 0u);
    } else if constexpr (QT == kQ5_1) {
        // 24 bytes at an 8-byte aligned offset: {d | m << 16, qh, qs[0..15]}
        const uint2* p = reinterpret_cast<const uint2*>(blk);
        const uint2 v0 = p[0], v1 = p[1], v2 = p[2];
        r.hdr = make_uint4(v0.x, v0.y, v1.x, v1.y);
        r.q = make_uint4(v2.x, v2.y, 0u, 0u);
    } else {
        const int part = sl & 7;
        r.hdr = *reinterpret_cast<const uint4*>(blk);
        r.q = *reinterpret_cast<const uint4*>(blk + KQuant<QT>::kQs + 16 * part);
        if constexpr (KQuant<QT>::kFifth) r.hb = *reinterpret_cast<const uint4*>(blk + 16 + 16 * (part & 1));
    }
}

// Dot products of one slice (16 quant bytes + its super-block header) with the
// lane's activations of nt tokens: acc[t] = sum over the slice's 32 weights.
// High nibbles are converted in place (16*q) and their scale carries the 1/16.
template <int TT>
__device__ __forceinline__ void q4k_slice_dot(const uint4 hv, const uint4 qv, const SliceKit& kit, int nt,
                                              const float (&xl)[TT][16], const float (&xh)[TT][16],
                                              const float (&sxl)[TT], const float (&sxh)[TT], float (&acc)[TT]) {
    const uint32_t scw = ((hv.y >> kit.sa) & kit.ma) | (hv.w & kit.mb);
    const uint32_t mnw = ((hv.z >> kit.sa) & kit.ma) | ((hv.w >> 4) & kit.mb);
    const uint32_t sc2 = scw >> kit.sh, mn2 = mnw >> kit.sh;
    const float d = f16_bits_to_f32(hv.x & 0xFFFFu), dmin = f16_bits_to_f32(hv.x >> 16);
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
    float ql[16], qh[16];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
        const uint32_t lo = qw[i4] & kit.m_lo, hi = qw[i4] & kit.m_hi;
        ql[4 * i4 + 0] = ubyte_f32<0>(lo);
        ql[4 * i4 + 1] = ubyte_f32<1>(lo);
        ql[4 * i4 + 2] = ubyte_f32<2>(lo);
        ql[4 * i4 + 3] = ubyte_f32<3>(lo);
        qh[4 * i4 + 0] = ubyte_f32<0>(hi);
        qh[4 * i4 + 1] = ubyte_f32<1>(hi);
        qh[4 * i4 + 2] = ubyte_f32<2>(hi);
        qh[4 * i4 + 3] = ubyte_f32<3>(hi);
    }
    const float dsl = d * ubyte_f32<0>(sc2), dsh = (d * 0.0625f) * ubyte_f32<1>(sc2);
    const float mml = dmin * ubyte_f32<0>(mn2), mmh = dmin * ubyte_f32<1>(mn2);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        acc[t] = 0.f;
        if (t < nt) {
            // four accumulation chains (even/odd weights of each sub-block)
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                s0 = fmaf(ql[j], xl[t][j], s0);
                s1 = fmaf(ql[j + 1], xl[t][j + 1], s1);
                s2 = fmaf(qh[j], xh[t][j], s2);
                s3 = fmaf(qh[j + 1], xh[t][j + 1], s3);
            }
            acc[t] = dsl * (s0 + s1) + dsh * (s2 + s3) - (mml * sxl[t] + mmh * sxh[t]);
        }
    }
}

// Q5_K: as q4k_slice_dot, with each quant's fifth bit OR-ed into bit 4 of
// its byte (q in 0..31, no in-place 16*q scaling for the high nibbles).
template <int TT>
__device__ __forceinline__ void q5k_slice_dot(const uint4 hv, const uint4 qv, const uint4 bv, const SliceKit& kit,
                                              int nt, const float (&xl)[TT][16], const float (&xh)[TT][16],
                                              const float (&sxl)[TT], const float (&sxh)[TT], float (&acc)[TT]) {
    const uint32_t scw = ((hv.y >> kit.sa) & kit.ma) | (hv.w & kit.mb);
    const uint32_t mnw = ((hv.z >> kit.sa) & kit.ma) | ((hv.w >> 4) & kit.mb);
    const uint32_t sc2 = scw >> kit.sh, mn2 = mnw >> kit.sh;
    const float d = f16_bits_to_f32(hv.x & 0xFFFFu), dmin = f16_bits_to_f32(hv.x >> 16);
    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
    const uint32_t hw[4] = {bv.x, bv.y, bv.z, bv.w};
    float ql[16], qh[16];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
        const uint32_t lo = (qw[i4] & kit.m_lo) | (((hw[i4] >> kit.f_lo) & kit.m_one) << 4);
        const uint32_t hi = ((qw[i4] >> 4) & kit.m_lo) | (((hw[i4] >> kit.f_hi) & kit.m_one) << 4);
        ql[4 * i4 + 0] = ubyte_f32<0>(lo);
        ql[4 * i4 + 1] = ubyte_f32<1>(lo);
        ql[4 * i4 + 2] = ubyte_f32<2>(lo);
        ql[4 * i4 + 3] = ubyte_f32<3>(lo);
        qh[4 * i4 + 0] = ubyte_f32<0>(hi);
        qh[4 * i4 + 1] = ubyte_f32<1>(hi);
        qh[4 * i4 + 2] = ubyte_f32<2>(hi);
        qh[4 * i4 + 3] = ubyte_f32<3>(hi);
    }
    const float dsl = d * ubyte_f32<0>(sc2), dsh = d * ubyte_f32<1>(sc2);
    const float mml = dmin * ubyte_f32<0>(mn2), mmh = dmin * ubyte_f32<1>(mn2);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        acc[t] = 0.f;
        if (t < nt) {
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                s0 = fmaf(ql[j], xl[t][j], s0);
                s1 = fmaf(ql[j + 1], xl[t][j + 1], s1);
                s2 = fmaf(qh[j], xh[t][j], s2);
                s3 = fmaf(qh[j + 1], xh[t][j + 1], s3);
            }
            acc[t] = dsl * (s0 + s1) + dsh * (s2 + s3) - (mml * sxl[t] + mmh * sxh[t]);
        }
    }
}

// Q8_0: the block's 32 int8 quants, each biased by 128 (a sign-bit flip of
// the byte) so it converts with v_cvt_f32_ubyteN; the bias comes back out as
// 128 * sum(x): acc = d * (sum (q + 128) x - 128 sum x).
template <int TT>
__device__ __forceinline__ void q8_block_dot(const KSlice& r, const SliceKit& kit, int nt,
                                             const float (&xl)[TT][16], const float (&xh)[TT][16],
                                             const float (&sxl)[TT], const float (&sxh)[TT], float (&acc)[TT]) {
    const uint32_t dw[9] = {r.hdr.x, r.hdr.y, r.hdr.z, r.hdr.w, r.q.x, r.q.y, r.q.z, r.q.w, r.hb.x};
    const float d = f16_bits_to_f32((dw[0] >> kit.dsh8) & 0xFFFFu);
    float q[32];
#pragma unroll
    for (int i4 = 0; i4 < 8; ++i4) {
        const uint32_t q4 = __builtin_amdgcn_perm(dw[i4 + 1], dw[i4], kit.sel8) ^ 0x80808080u;
        q[4 * i4 + 0] = ubyte_f32<0>(q4);
        q[4 * i4 + 1] = ubyte_f32<1>(q4);
        q[4 * i4 + 2] = ubyte_f32<2>(q4);
        q[4 * i4 + 3] = ubyte_f32<3>(q4);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        acc[t] = 0.f;
        if (t < nt) {
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                s0 = fmaf(q[j], xl[t][j], s0);
                s1 = fmaf(q[j + 1], xl[t][j + 1], s1);
                s2 = fmaf(q[16 + j], xh[t][j], s2);
                s3 = fmaf(q[16 + j + 1], xh[t][j + 1], s3);
            }
            acc[t] = d * (((s0 + s1) + (s2 + s3)) - 128.0f * (sxl[t] + sxh[t]));
        }
    }
}

// Q5_1: quant l of the block = low nibble of qs byte l + 16 * qh bit l, quant
// 16 + l = its high nibble + 16 * qh bit 16 + l.  Four qh bits go to bit 4 of
// four bytes at once: (v & 15) * 0x00204081 puts bit i of v at bit 8i (i + 7i)
// with no overlap between the shifted copies below bit 32 that survive the
// 0x01010101 mask.  acc = d * sum q x + m * sum x.
__device__ __forceinline__ uint32_t q51_spread4(uint32_t v) { return ((v & 15u) * 0x00204081u) & 0x01010101u; }

template <int TT>
__device__ __forceinline__ void q51_block_dot(const KSlice& r, int nt, const float (&xl)[TT][16],
                                              const float (&xh)[TT][16], const float (&sxl)[TT],
                                              const float (&sxh)[TT], float (&acc)[TT]) {
    const float d = f16_bits_to_f32(r.hdr.x & 0xFFFFu), m = f16_bits_to_f32(r.hdr.x >> 16);
    const uint32_t qh = r.hdr.y;
    const uint32_t qw[4] = {r.hdr.z, r.hdr.w, r.q.x, r.q.y};
    float ql[16], qv[16];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
        const uint32_t lo = (qw[i4] & 0x0F0F0F0Fu) | (q51_spread4(qh >> (4 * i4)) << 4);
        const uint32_t hi = ((qw[i4] >> 4) & 0x0F0F0F0Fu) | (q51_spread4(qh >> (16 + 4 * i4)) << 4);
        ql[4 * i4 + 0] = ubyte_f32<0>(lo);
        ql[4 * i4 + 1] = ubyte_f32<1>(lo);
        ql[4 * i4 + 2] = ubyte_f32<2>(lo);
        ql[4 * i4 + 3] = ubyte_f32<3>(lo);
        qv[4 * i4 + 0] = ubyte_f32<0>(hi);
        qv[4 * i4 + 1] = ubyte_f32<1>(hi);
        qv[4 * i4 + 2] = ubyte_f32<2>(hi);
        qv[4 * i4 + 3] = ubyte_f32<3>(hi);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        acc[t] = 0.f;
        if (t < nt) {
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                s0 = fmaf(ql[j], xl[t][j], s0);
                s1 = fmaf(ql[j + 1], xl[t][j + 1], s1);
                s2 = fmaf(qv[j], xh[t][j], s2);
                s3 = fmaf(qv[j + 1], xh[t][j + 1], s3);
            }
            acc[t] = d * ((s0 + s1) + (s2 + s3)) + m * (sxl[t] + sxh[t]);
        }
    }
}

template <int QT, int TT>
__device__ __forceinline__ void kslice_dot(const KSlice& r, const SliceKit& kit, int nt, const float (&xl)[TT][16],
                                           const float (&xh)[TT][16], const float (&sxl)[TT],
                                           const float (&sxh)[TT], float (&acc)[TT]) {
    if constexpr (QT == kQ8_0)
        q8_block_dot<TT>(r, kit, nt, xl, xh, sxl, sxh, acc);
    else if constexpr (QT == kQ5_1)
        q51_block_dot<TT>(r, nt, xl, xh, sxl, sxh, acc);
    else if constexpr (KQuant<QT>::kFifth)
        q5k_slice_dot<TT>(r.hdr, r.q, r.hb, kit, nt, xl, xh, sxl, sxh, acc);
    else
        q4k_slice_dot<TT>(r.hdr, r.q, kit, nt, xl, xh, sxl, sxh, acc);
}

template <int TT>
__device__ __forceinline__ void unpack_f4(const float4 (&v)[4], float (&o)[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[4 * i] = v[i].x;
        o[4 * i + 1] = v[i].y;
        o[4 * i + 2] = v[i].z;
        o[4 * i + 3] = v[i].w;
    }
}

// The streaming body of K1 for one expert slot: rows of gate and up of expert
// e (bank G/U), applied to the nt tokens s_tok[] (their x already loaded into
// xl4/xh4), h written to rows s_hrow[].
template <int NB, int PASSES, int TT, int QG>
__device__ __forceinline__ void dec_gateup_body(const DecArgs& a, const QMat& G, const QMat& U, int e, int nt,
                                                const int (&s_hrow)[TT], float4 (&xl4)[TT][4], float4 (&xh4)[TT][4],
                                                float* s_part) {
    using S = K1Shape<NB, PASSES>;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int unit = wave / S::W;
    const int f = (wave % S::W) * kWave + lane;         // flat lane inside the unit
    const int rr = f / S::SLICES;                        // row inside the pass
    const int sl = f % S::SLICES;
    const SliceKit kit = kslice_kit<QG>(sl);
    const int row0 = blockIdx.x * S::ROWS;

    const uint8_t* Gb = G.data + (int64_t)e * G.expert_bytes + kslice_block_off<QG>(sl);
    const uint8_t* Ub = U.data + (int64_t)e * U.expert_bytes + kslice_block_off<QG>(sl);
    KSlice rg[PASSES], ru[PASSES];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int i = row0 + (ps * S::UNITS + unit) * S::P + rr;
        const int ic = i < a.I ? i : a.I - 1;   // clamp: rows past I load a valid row and are not stored
        kslice_load<QG>(Gb + (int64_t)ic * G.row_bytes, sl, rg[ps]);
        kslice_load<QG>(Ub + (int64_t)ic * U.row_bytes, sl, ru[ps]);
    }
    float xl[TT][16], xh[TT][16], sxl[TT], sxh[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        sxl[t] = sxh[t] = 0.f;
        unpack_f4<TT>(xl4[t], xl[t]);
        unpack_f4<TT>(xh4[t], xh[t]);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            sxl[t] += xl[t][j];
            sxh[t] += xh[t][j];
        }
    }

#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int i = row0 + (ps * S::UNITS + unit) * S::P + rr;
        float pg[TT], pu[TT];
        kslice_dot<QG, TT>(rg[ps], kit, nt, xl, xh, sxl, sxh, pg);
        kslice_dot<QG, TT>(ru[ps], kit, nt, xl, xh, sxl, sxh, pu);
        if constexpr (S::IN_WAVE) {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                pg[t] = segment_sum<S::SLICES>(pg[t]);
                pu[t] = segment_sum<S::SLICES>(pu[t]);
            }
            if (sl == S::SLICES - 1 && i < a.I) {
#pragma unroll
                for (int t = 0; t < TT; ++t)
                    if (t < nt) a.h[(int64_t)s_hrow[t] * a.I + i] = silu_f32(pg[t]) * pu[t];
            }
        } else {
            // a row spans several waves: sums of 16-lane groups, then the row's groups in order
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                pg[t] = segment_sum<16>(pg[t]);
                pu[t] = segment_sum<16>(pu[t]);
            }
            if (ps > 0) __syncthreads();
            if ((lane & 15) == 15) {
                const int grp = sl >> 4;
#pragma unroll
                for (int t = 0; t < TT; ++t) {
                    s_part[((2 * t + 0) * S::P + rr) * S::GROUPS + grp] = pg[t];
                    s_part[((2 * t + 1) * S::P + rr) * S::GROUPS + grp] = pu[t];
                }
            }
            __syncthreads();
            const int job = threadIdx.x;   // one thread per (token, row)
            if (job < nt * S::P) {
                const int t = job / S::P, r2 = job % S::P;
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int q = 0; q < S::GROUPS; ++q) {
                    g += s_part[((2 * t + 0) * S::P + r2) * S::GROUPS + q];
                    u += s_part[((2 * t + 1) * S::P + r2) * S::GROUPS + q];
                }
                const int i2 = row0 + ps * S::P + r2;
                if (i2 < a.I) a.h[(int64_t)s_hrow[t] * a.I + i2] = silu_f32(g) * u;
            }
        }
    }
}

// The lane's 32 activation columns of token 0.
__device__ __forceinline__ void load_x0_slice(const DecArgs& a, int clo, int chi, float4 (&l4)[4], float4 (&h4)[4]) {
    const float4* pl = reinterpret_cast<const float4*>(a.x + clo);
    const float4* ph = reinterpret_cast<const float4*>(a.x + chi);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        l4[v] = pl[v];
        h4[v] = ph[v];
    }
}

// The lane's 32 activation columns of token `tok`.
template <int TT>
__device__ __forceinline__ void load_x_slice(const DecArgs& a, int tok, int clo, int chi, float4 (&l4)[4],
                                             float4 (&h4)[4]) {
    const float4* pl = reinterpret_cast<const float4*>(a.x + (int64_t)tok * a.H + clo);
    const float4* ph = reinterpret_cast<const float4*>(a.x + (int64_t)tok * a.H + chi);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        l4[v] = pl[v];
        h4[v] = ph[v];
    }
}

// ---------------------------------------------------------------------------
// K1: workgroup (tile of rows, group y).  Group y = t*Gk + q (y < T*Gk) owns
// the slots of token t with ranks q, q + Gk, ... (at most SM):
// every wave runs the token's top-k extraction itself and issues the loads of a slot
// right after the round that names its expert, so the weight traffic of the
// early slots overlaps the remaining rounds; the dot products then consume the
// slots in issue order.  Each (token, slot) pair streams its own expert rows:
// in a 3-token window nearly all 24 experts are distinct, so sharing loads
// between tokens would save little.  Two slots per group give about two waves
// per SIMD at one token (640 workgroups of 4 waves for top-8), so the dot
// products of one wave overlap the extraction rounds of another; the
// extraction itself is repeated by every wave.  Groups T*Gk .. T*Gk + ceil(T/4) - 1 (when
// the layer has a shared expert) each run it for 4 tokens against one load of
// its rows.  Grid row 0 holds one more workgroup that publishes the routing
// (and the table for K2); the groups take rows 1 and up.
// ---------------------------------------------------------------------------
template <int NB, int V, int TT, int SM, int QG>
__global__ void __launch_bounds__((K1Shape<NB, 1>::THREADS)) dec_gateup_pipe_kernel(DecArgs a, int Gk) {
    using S = K1Shape<NB, 1>;
    static_assert(TT <= kShTok, "shared-expert groups of at most kShTok tokens");
    constexpr int SP = SM > TT ? SM : TT;   // slots or tokens whose partial sums s_part holds
    // row 0 of the grid publishes (dispatched first, so it never waits for a
    // free slot behind the streaming workgroups); rows 1.. stream
    const int y = (int)blockIdx.y - 1;
    const int Gr = a.T * Gk;
    if (y < 0) {
        __shared__ DecRoute R;
        if (blockIdx.x != 0) return;
        dec_route<V>(a.logits, a.T, a.E, a.k, a.renorm, R);
        dec_publish(R, a.T, a.E, a.k, a.r);
        if (a.sgate_w) {   // one wave per token, as the separate gate kernel
            const int wave = threadIdx.x / kWave, nwaves = blockDim.x / kWave;
            for (int t = wave; t < a.T; t += nwaves) {
                const float v = shared_gate_wave(a.sgate_w, a.x + (int64_t)t * a.H, a.H);
                if ((threadIdx.x & (kWave - 1)) == 0) R.sg[t] = v;
            }
            __syncthreads();
        }
        const int* src = reinterpret_cast<const int*>(&R);
        for (int i = threadIdx.x; i < (int)(sizeof(DecRoute) / 4); i += blockDim.x) a.route_tab[i] = src[i];
        return;
    }
    __shared__ float s_part[S::IN_WAVE ? 1 : (2 * SP * S::P * S::GROUPS)];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int unit = wave / S::W;
    const int f = (wave % S::W) * kWave + lane;
    const int rr = f / S::SLICES;
    const int sl = f % S::SLICES;
    const SliceKit kit = kslice_kit<QG>(sl);
    const int clo = kslice_col_lo<QG>(sl);
    const int chi = kslice_col_hi<QG>(sl);
    const int i = blockIdx.x * S::ROWS + unit * S::P + rr;
    const int ic = i < a.I ? i : a.I - 1;   // rows past I load a valid row and are not stored

    if (y >= Gr) {
        // the shared expert: one load of its rows for tokens t0 .. t0 + TT - 1
        const int t0 = (y - Gr) * kShTok;
        const int nt = min(TT, a.T - t0);
        float4 xl4[TT][4], xh4[TT][4];
        int hrows[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const int tc = t0 + (t < nt ? t : nt - 1);
            load_x_slice<TT>(a, tc, clo, chi, xl4[t], xh4[t]);
            hrows[t] = a.T * a.k + tc;
        }
        dec_gateup_body<NB, 1, TT, QG>(a, a.sgate, a.sup, 0, nt, hrows, xl4, xh4, s_part);
        return;
    }

    const int tok = y / Gk, q = y - tok * Gk;
    // logits, then activations (neither depends on the routing): the logits
    // gate the extraction rounds, the activations are needed only once the
    // weights arrive, so they load behind the logits
    WaveExtract<V> ex;
    float xv[V];
    ex.issue(a.logits + (int64_t)tok * a.E, a.E, xv);
    float4 xl4[1][4], xh4[1][4];
    load_x_slice<1>(a, tok, clo, chi, xl4[0], xh4[0]);
    (void)ex.keys(a.E, xv);
    KSlice rg[SM], ru[SM];
    auto issue = [&](int m, int e) {
        const uint8_t* gr = a.gate.data + (int64_t)e * a.gate.expert_bytes + (int64_t)ic * a.gate.row_bytes +
                            kslice_block_off<QG>(sl);
        const uint8_t* ur = a.up.data + (int64_t)e * a.up.expert_bytes + (int64_t)ic * a.up.row_bytes +
                            kslice_block_off<QG>(sl);
        kslice_load<QG>(gr, sl, rg[m]);
        kslice_load<QG>(ur, sl, ru[m]);
    };
    int done = 0, win = 0;
#pragma unroll
    for (int m = 0; m < SM; ++m) {
        const int jt = q + m * Gk;
        if (jt < a.k) {
            while (done <= jt) {
                win = ex.next();
                ++done;
            }
            issue(m, win);
        }
    }

    float xl[1][16], xh[1][16], sxl[1], sxh[1];
    unpack_f4<1>(xl4[0], xl[0]);
    unpack_f4<1>(xh4[0], xh[0]);
    sxl[0] = sxh[0] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        sxl[0] += xl[0][j];
        sxh[0] += xh[0][j];
    }
    // h values of the slots, stored after the last slot: a store between the
    // slots would make the later loads wait for its completion
    float hv[SM];
#pragma unroll
    for (int m = 0; m < SM; ++m) {
        hv[m] = 0.f;
        const int jt = q + m * Gk;
        if (jt >= a.k) continue;
        float pg[1], pu[1];
        kslice_dot<QG, 1>(rg[m], kit, 1, xl, xh, sxl, sxh, pg);
        kslice_dot<QG, 1>(ru[m], kit, 1, xl, xh, sxl, sxh, pu);
        if constexpr (S::IN_WAVE) {
            pg[0] = segment_sum<S::SLICES>(pg[0]);
            pu[0] = segment_sum<S::SLICES>(pu[0]);
            hv[m] = silu_f32(pg[0]) * pu[0];
        } else {
            pg[0] = segment_sum<16>(pg[0]);
            pu[0] = segment_sum<16>(pu[0]);
            if ((lane & 15) == 15) {
                const int grp = sl >> 4;
                s_part[((2 * m + 0) * S::P + rr) * S::GROUPS + grp] = pg[0];
                s_part[((2 * m + 1) * S::P + rr) * S::GROUPS + grp] = pu[0];
            }
        }
    }
    if constexpr (S::IN_WAVE) {
        if (sl == S::SLICES - 1 && i < a.I) {
#pragma unroll
            for (int m = 0; m < SM; ++m) {
                const int jt = q + m * Gk;
                if (jt < a.k) a.h[(int64_t)(tok * a.k + jt) * a.I + i] = hv[m];
            }
        }
    } else {
        __syncthreads();
        // one thread per (slot, row): the row's 16-lane group sums in order
        for (int job = threadIdx.x; job < SM * S::P; job += blockDim.x) {
            const int m = job / S::P, r2 = job % S::P;
            const int jt = q + m * Gk;
            const int i2 = blockIdx.x * S::ROWS + r2;
            if (jt >= a.k || i2 >= a.I) continue;
            float gs = 0.f, us = 0.f;
#pragma unroll
            for (int g2 = 0; g2 < S::GROUPS; ++g2) {
                gs += s_part[((2 * m + 0) * S::P + r2) * S::GROUPS + g2];
                us += s_part[((2 * m + 1) * S::P + r2) * S::GROUPS + g2];
            }
            a.h[(int64_t)(tok * a.k + jt) * a.I + i2] = silu_f32(gs) * us;
        }
    }
}

// ---------------------------------------------------------------------------
// K2: down + combine.  A "slice" of a down row is 16 quant bytes of a Q4_K
// super-block (32 weights) or one 34-byte Q8_0 block (32 weights); NS slices
// per row, 64/NS rows per wave pass, PS passes per workgroup.  Slots
// are the (token, rank) pairs p = t*k + j (expert sel[p], h row p) and, with a
// shared expert, one slot per token t (h row T*k + t).  Each wave takes one
// slot at a time, all PS passes of it, with its weight and activation loads in
// flight together.  (Spreading a slot's passes over two waves, 16 waves for
// top-8 at one token, measured slower.)  Results go to LDS and the combine is
// formed in slot order.
// ---------------------------------------------------------------------------
constexpr int kK2MinPasses = 2;   // passes per workgroup: enough to cover H with
constexpr int kK2MaxPasses = 3;   // about one workgroup per CU
constexpr int kK2MaxThreads = 1024;

template <int QD, int NS, int PS>
__global__ void __launch_bounds__(kK2MaxThreads) dec_down_kernel(DecArgs a) {
    constexpr int RP = kWave / NS;              // rows per wave pass
    constexpr int RO = RP * PS;                 // output rows of the workgroup
    __shared__ DecRoute R;
    __shared__ float s_y[(kDecMaxPairs + kDecMaxT) * RO];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int nwaves = blockDim.x / kWave;
    const int T = a.T, k = a.k, P = T * k;
    const int o0 = blockIdx.x * RO;

    {   // the routing table written by the gate/up kernel's last workgroup
        int* dst = reinterpret_cast<int*>(&R);
        for (int i = threadIdx.x; i < (int)(sizeof(DecRoute) / 4); i += blockDim.x) dst[i] = a.route_tab[i];
    }
    __syncthreads();
    const int n_slots = P + (a.has_shared ? T : 0);
    const int rr = lane / NS, sl = lane % NS;
    const SliceKit kit = kslice_kit<QD>(sl);
    const int c_lo = kslice_col_lo<QD>(sl), c_hi = kslice_col_hi<QD>(sl);

    // one slot u at a time per wave: its PS passes of RP rows
    for (int u = wave; u < n_slots; u += nwaves) {
        bool live = true;
        const bool shared = u >= P;
        int e = 0;
        if (!shared) {
            e = R.sel[u];
            if (e < 0 || e >= a.E) {   // corrupted table: nothing is read through it
                if (lane == 0) raise_error(kErrExpertRange);
                live = false;
                e = 0;
            }
        }
        const QMat D = shared ? a.sdown : a.down;
        const uint8_t* Db = D.data + (int64_t)e * D.expert_bytes;
        const int64_t rowb = D.row_bytes;
        const int hrow = live ? u : 0;   // the h row of slot u is u
        // all weight loads, then the h loads
        KSlice rk[PS];
#pragma unroll
        for (int pp = 0; pp < PS; ++pp) {   // a dead slot loads expert 0's rows, never used
            const int o = o0 + pp * RP + rr;
            const int oc = o < a.H ? o : a.H - 1;
            kslice_load<QD>(Db + (int64_t)oc * rowb + kslice_block_off<QD>(sl), sl, rk[pp]);
        }
        float4 hl4[4], hh4[4];
        {
            const float4* pl = reinterpret_cast<const float4*>(a.h + (int64_t)hrow * a.I + c_lo);
            const float4* ph = reinterpret_cast<const float4*>(a.h + (int64_t)hrow * a.I + c_hi);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                hl4[v] = pl[v];
                hh4[v] = ph[v];
            }
        }
        if (!live) {   // the combine still reads the slot's rows: zeros, so out stays deterministic
#pragma unroll
            for (int pp = 0; pp < PS; ++pp)
                if (sl == NS - 1) s_y[u * RO + pp * RP + rr] = 0.f;
            continue;
        }
        float hl[1][16], hh[1][16], shl[1], shh[1];
        unpack_f4<1>(hl4, hl[0]);
        unpack_f4<1>(hh4, hh[0]);
        shl[0] = shh[0] = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            shl[0] += hl[0][j];
            shh[0] += hh[0][j];
        }
#pragma unroll
        for (int pp = 0; pp < PS; ++pp) {
            const int ps = pp;
            float acc[1];
            kslice_dot<QD, 1>(rk[pp], kit, 1, hl, hh, shl, shh, acc);
            acc[0] = segment_sum<NS>(acc[0]);
            if (sl == NS - 1) s_y[hrow * RO + ps * RP + rr] = acc[0];
        }
    }
    __syncthreads();
    // combine in slot order, then the shared expert; also publish y_pair / y_shared
    for (int job = threadIdx.x; job < T * RO; job += blockDim.x) {
        const int t = job / RO, r = job % RO, o = o0 + r;
        if (o >= a.H) continue;
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            const float y = s_y[(t * k + j) * RO + r];
            acc = fmaf(R.w[t * k + j], y, acc);
            if (a.y_pair) a.y_pair[(int64_t)(t * k + j) * a.H + o] = y;
        }
        if (a.has_shared) {
            const float ys = s_y[(P + t) * RO + r];
            const float sc = (a.shared_scale ? a.shared_scale[t] : 1.0f) * (a.sgate_w ? R.sg[t] : 1.0f);
            acc = fmaf(sc, ys, acc);
            if (a.y_shared) a.y_shared[(int64_t)t * a.H + o] = ys;
        }
        if (a.residual) acc += a.residual[(int64_t)t * a.H + o];   // may be out itself: read, then written
        a.out[(int64_t)t * a.H + o] = acc;
    }
}

// ---------------------------------------------------------------------------
// Expert-grouped decode FFN: batches past the two-kernel layer (T*k > 64) on
// fp32 activations.  The int8 path's tile list with kGrpTok pairs per tile
// (tiles of one expert's bucket, then the shared expert's token tiles) drives
// two kernels: a workgroup of the gate/up kernel streams a tile of the
// expert's rows once and applies it to the tile's tokens (the shared-expert
// body of K1 above), and a workgroup of the down kernel does the same with the
// tile's h rows, writing y_pair / y_shared for the combine.  An expert shared
// by several tokens of the batch is read once per tile of two of them, where
// the two-kernel layer reads it once per (token, rank) pair.
// ---------------------------------------------------------------------------
struct GroupTiles {
    const int32_t* tile_e;
    const int32_t* tile_m0;
    const int32_t* n_tiles;
    const int32_t* offset;
    const int32_t* pair;
};

// Pairs per tile of the expert-grouped kernels.  Two keep a wave's activation
// slices (32 floats per token) and its weight slices within ~120 VGPRs, so a
// SIMD holds four waves; four tokens per tile took 205-276 VGPRs.
constexpr int kGrpTok = 2;

// The tile's tokens (t < nt) and h rows; false (uniform across the workgroup)
// when the tile is past the list, empty, or its bucket entries are corrupt.
__device__ __forceinline__ bool group_tile(const DecArgs& a, const GroupTiles& g, int y, int& e, bool& shared,
                                           int& nt, int (&tok)[kGrpTok], int (&hrow)[kGrpTok]) {
    if (y >= *g.n_tiles) return false;
    e = g.tile_e[y];
    const int m0 = g.tile_m0[y];
    const int P = a.T * a.k;
    shared = e == a.E;
    if (shared) {
        nt = min(kGrpTok, a.T - m0);
        if (m0 < 0 || nt <= 0) return false;
#pragma unroll
        for (int t = 0; t < kGrpTok; ++t) {
            tok[t] = m0 + min(t, nt - 1);
            hrow[t] = P + tok[t];
        }
        return true;
    }
    if (e < 0 || e >= a.E) {
        if (threadIdx.x == 0) raise_error(kErrExpertRange);
        return false;
    }
    const int p0 = g.offset[e], p1 = g.offset[e + 1];
    if (p0 < 0 || p1 < p0 || p1 > P || m0 < 0) {
        if (threadIdx.x == 0) raise_error(kErrPairRange);
        return false;
    }
    nt = min(kGrpTok, p1 - p0 - m0);
    if (nt <= 0) return false;
#pragma unroll
    for (int t = 0; t < kGrpTok; ++t) {
        const int p = g.pair[p0 + m0 + min(t, nt - 1)];
        if (p < 0 || p >= P) {
            if (threadIdx.x == 0) raise_error(kErrPairRange);
            return false;
        }
        tok[t] = p / a.k;
        hrow[t] = p;
    }
    return true;
}

template <int NB, int PASSES, int QG>
__global__ void __launch_bounds__((K1Shape<NB, PASSES>::THREADS)) dec_gateup_grouped_kernel(DecArgs a, GroupTiles g) {
    using S = K1Shape<NB, PASSES>;
    constexpr int TT = kGrpTok;
    __shared__ float s_part[S::IN_WAVE ? 1 : (2 * TT * S::P * S::GROUPS)];
    int e, nt, tok[TT], hrow[TT];
    bool shared;
    if (!group_tile(a, g, blockIdx.y, e, shared, nt, tok, hrow)) return;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int sl = ((wave % S::W) * kWave + lane) % S::SLICES;
    const int clo = kslice_col_lo<QG>(sl), chi = kslice_col_hi<QG>(sl);
    float4 xl4[TT][4], xh4[TT][4];
#pragma unroll
    for (int t = 0; t < TT; ++t) load_x_slice<TT>(a, tok[t], clo, chi, xl4[t], xh4[t]);
    dec_gateup_body<NB, PASSES, TT, QG>(a, shared ? a.sgate : a.gate, shared ? a.sup : a.up, shared ? 0 : e, nt,
                                        hrow, xl4, xh4, s_part);
}

// Down: four waves, each PS passes of RP = 64/NS rows (NS lanes per row), all
// of its weight loads in flight before the tile's h slices are read.
constexpr int kGrpDownWaves = 4;

template <int QD, int NS, int PS>
__global__ void __launch_bounds__(kGrpDownWaves * kWave) dec_down_grouped_kernel(DecArgs a, GroupTiles g) {
    constexpr int RP = kWave / NS;
    constexpr int TT = kGrpTok;
    int e, nt, tok[TT], hrow[TT];
    bool shared;
    if (!group_tile(a, g, blockIdx.y, e, shared, nt, tok, hrow)) return;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int rr = lane / NS, sl = lane % NS;
    const SliceKit kit = kslice_kit<QD>(sl);
    const int c_lo = kslice_col_lo<QD>(sl), c_hi = kslice_col_hi<QD>(sl);
    const QMat D = shared ? a.sdown : a.down;
    const uint8_t* Db = D.data + (int64_t)(shared ? 0 : e) * D.expert_bytes + kslice_block_off<QD>(sl);
    const int o0 = (blockIdx.x * kGrpDownWaves + wave) * RP * PS;
    KSlice rk[PS];
#pragma unroll
    for (int pp = 0; pp < PS; ++pp) {
        const int o = o0 + pp * RP + rr;
        kslice_load<QD>(Db + (int64_t)(o < a.H ? o : a.H - 1) * D.row_bytes, sl, rk[pp]);
    }
    float4 hl4[TT][4], hh4[TT][4];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const float4* pl = reinterpret_cast<const float4*>(a.h + (int64_t)hrow[t] * a.I + c_lo);
        const float4* ph = reinterpret_cast<const float4*>(a.h + (int64_t)hrow[t] * a.I + c_hi);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            hl4[t][v] = pl[v];
            hh4[t][v] = ph[v];
        }
    }
    float hl[TT][16], hh[TT][16], shl[TT], shh[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        unpack_f4<TT>(hl4[t], hl[t]);
        unpack_f4<TT>(hh4[t], hh[t]);
        shl[t] = shh[t] = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            shl[t] += hl[t][j];
            shh[t] += hh[t][j];
        }
    }
#pragma unroll
    for (int pp = 0; pp < PS; ++pp) {
        const int o = o0 + pp * RP + rr;
        float acc[TT];
        kslice_dot<QD, TT>(rk[pp], kit, nt, hl, hh, shl, shh, acc);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            acc[t] = segment_sum<NS>(acc[t]);
            if (t < nt && sl == NS - 1 && o < a.H) {
                if (shared)
                    a.y_shared[(int64_t)tok[t] * a.H + o] = acc[t];
                else
                    a.y_pair[(int64_t)hrow[t] * a.H + o] = acc[t];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace {

// Workgroups of a K1 instance that the current device holds at once (per-CU
// occupancy times CUs), looked up once per instance and device; 0 if unknown.
constexpr int kDecMaxDevices = 64;

// Compute units of the current device, looked up once per device (256 on an
// MI355X; that value if the query fails).
int device_cus() {
    static std::atomic<int> cus[kDecMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDecMaxDevices) return 256;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

template <int NB, int V, int TT, int SM, int QG>
int k1_capacity() {
    static std::atomic<int> cap[kDecMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDecMaxDevices) return 0;
    int c = cap[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dec_gateup_pipe_kernel<NB, V, TT, SM, QG>,
                                                         K1Shape<NB, 1>::THREADS, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        c = per_cu * cus;
        cap[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

inline int k1_grid_rows(const DecArgs& a, int SM, int& Gk) {
    Gk = (a.k + SM - 1) / SM;                                         // groups per token
    const int n_sh = a.has_shared ? (a.T + kShTok - 1) / kShTok : 0;  // shared-expert groups
    return a.T * Gk + n_sh + 1;
}

template <int NB, int V, int TT, int SM, int QG>
hipError_t launch_k1_sm(const DecArgs& a, hipStream_t s) {
    using S = K1Shape<NB, 1>;
    int Gk;
    const int rows = k1_grid_rows(a, SM, Gk);
    dim3 grid((a.I + S::ROWS - 1) / S::ROWS, rows);
    dec_gateup_pipe_kernel<NB, V, TT, SM, QG><<<grid, S::THREADS, 0, s>>>(a, Gk);
    return hipGetLastError();
}

// Slots per group: the fewest of 2, 3, 4 whose grid the device holds at once.
// Fewer slots per wave shorten each wave's dot products and let waves of one
// SIMD overlap, but a grid that needs a second round of workgroups ends a
// whole workgroup duration later (the 3-token window at two slots: 1,664
// workgroups for 1,024 places).
template <int NB, int V, int TT, int QG>
hipError_t launch_k1_pipe(const DecArgs& a, hipStream_t s) {
    using S = K1Shape<NB, 1>;
    const int cols = (a.I + S::ROWS - 1) / S::ROWS;
    int Gk;
    if (cols * k1_grid_rows(a, 2, Gk) <= k1_capacity<NB, V, TT, 2, QG>()) return launch_k1_sm<NB, V, TT, 2, QG>(a, s);
    if (cols * k1_grid_rows(a, 3, Gk) <= k1_capacity<NB, V, TT, 3, QG>()) return launch_k1_sm<NB, V, TT, 3, QG>(a, s);
    return launch_k1_sm<NB, V, TT, 4, QG>(a, s);
}

template <int NB, int V, int QG>
hipError_t launch_k1_v(const DecArgs& a, hipStream_t s) {
    // the 4-token shared-expert branch costs registers; it runs only when the
    // layer has a shared expert and more than one token
    return (a.T == 1 || !a.has_shared) ? launch_k1_pipe<NB, V, 1, QG>(a, s) : launch_k1_pipe<NB, V, kShTok, QG>(a, s);
}

template <int NB, int QG>
hipError_t launch_k1_q(const DecArgs& a, hipStream_t s) {
    const int vpl = topk_vpl(a.E);
    if (vpl == 4) return launch_k1_v<NB, 4, QG>(a, s);
    if (vpl == 8) return launch_k1_v<NB, 8, QG>(a, s);
    return launch_k1_v<NB, 16, QG>(a, s);
}

template <int NB>
hipError_t launch_k1(const DecArgs& a, hipStream_t s) {
    if (a.gate.qtype == kQ5_K) return launch_k1_q<NB, kQ5_K>(a, s);
    if (a.gate.qtype == kQ8_0) return launch_k1_q<NB, kQ8_0>(a, s);
    if (a.gate.qtype == kQ5_1) return launch_k1_q<NB, kQ5_1>(a, s);
    return launch_k1_q<NB, kQ4_K>(a, s);
}

template <int QD, int NS, int PS>
hipError_t launch_k2p(const DecArgs& a, hipStream_t s) {
    constexpr int RO = (kWave / NS) * PS;
    const int slots = a.T * a.k + (a.has_shared ? a.T : 0);
    const int max_waves = kK2MaxThreads / kWave;
    // one slot per wave in flight; slots beyond 16 take further rounds
    const int waves = slots < 4 ? 4 : (slots > max_waves ? max_waves : slots);
    dec_down_kernel<QD, NS, PS><<<(a.H + RO - 1) / RO, waves * kWave, 0, s>>>(a);
    return hipGetLastError();
}

// Passes per workgroup: the fewest (at least two) that cover H in about one
// workgroup per CU, so no CU takes a second workgroup while others idle
// (H = 2,560 with 4-row passes: 214 workgroups of 3 passes, not 320 of 2).
template <int QD, int NS>
hipError_t launch_k2(const DecArgs& a, hipStream_t s) {
    constexpr int RP = kWave / NS;
    const int groups = (a.H + RP - 1) / RP;
    const int cus = device_cus();
    int ps = (groups + cus - 1) / cus;
    ps = ps < kK2MinPasses ? kK2MinPasses : (ps > kK2MaxPasses ? kK2MaxPasses : ps);
    return ps == 2 ? launch_k2p<QD, NS, 2>(a, s) : launch_k2p<QD, NS, 3>(a, s);
}

}  // namespace

// Shapes the fused decode path covers: Q4_K, Q5_K, Q8_0 or Q5_1 gate/up (the
// same format for both) with H/256 in {1, 2, 4, 8, 10}; down in any of those
// formats with 8, 16 or 32 lanes of 32 weights per row (I = 256, 512 or 1024);
// T <= 8, T*k <= 64.
bool dec_fused_supported(int T, int k, int H, int I, int qg, int qu, int qd) {
    auto known = [](int q) { return q == kQ4_K || q == kQ5_K || q == kQ8_0 || q == kQ5_1; };
    if (T < 1 || T > kDecMaxT || T * k > kDecMaxPairs) return false;
    if (!known(qg) || qu != qg || !known(qd)) return false;
    const int nb = H / 256;
    if (!(nb == 1 || nb == 2 || nb == 4 || nb == 8 || nb == 10)) return false;
    const int ns = I / 32;   // lanes per down row, every format
    return ns == 8 || ns == 16 || ns == 32;
}

namespace {

template <int QD>
hipError_t launch_k2_q(const DecArgs& a, hipStream_t s) {
    const int ns = a.I / 32;
    if (ns == 8) return launch_k2<QD, 8>(a, s);
    if (ns == 16) return launch_k2<QD, 16>(a, s);
    return launch_k2<QD, 32>(a, s);
}

}  // namespace

hipError_t launch_dec_fused(const DecArgs& a, hipStream_t s) {
    hipError_t e;
    switch (a.H / 256) {
        case 1: e = launch_k1<1>(a, s); break;
        case 2: e = launch_k1<2>(a, s); break;
        case 4: e = launch_k1<4>(a, s); break;
        case 8: e = launch_k1<8>(a, s); break;
        default: e = launch_k1<10>(a, s); break;
    }
    if (e != hipSuccess) return e;
    if (a.down.qtype == kQ4_K) return launch_k2_q<kQ4_K>(a, s);
    if (a.down.qtype == kQ5_K) return launch_k2_q<kQ5_K>(a, s);
    if (a.down.qtype == kQ5_1) return launch_k2_q<kQ5_1>(a, s);
    return launch_k2_q<kQ8_0>(a, s);
}

// ---------------------------------------------------------------------------
// The expert-grouped path's launcher.
// ---------------------------------------------------------------------------
namespace {

constexpr int kGrpPasses = 2;     // gate/up rows per wave (row passes)
constexpr int kGrpDownPasses = 2; // down row passes per wave

int grp_max_tiles(int T, int k, int E, int has_shared) {
    const int P = T * k;
    return (P + kGrpTok - 1) / kGrpTok + (E < P ? E : P) + (has_shared ? (T + kGrpTok - 1) / kGrpTok : 0);
}

template <int NB, int QG>
hipError_t launch_grp_gateup(const DecArgs& a, const GroupTiles& g, int maxt, hipStream_t s) {
    using S = K1Shape<NB, kGrpPasses>;
    const dim3 grid((a.I + S::ROWS - 1) / S::ROWS, maxt);
    dec_gateup_grouped_kernel<NB, kGrpPasses, QG><<<grid, S::THREADS, 0, s>>>(a, g);
    return hipGetLastError();
}

template <int QD>
hipError_t launch_grp_down(const DecArgs& a, const GroupTiles& g, int maxt, hipStream_t s) {
    constexpr int NS = 16, RO = kGrpDownWaves * (kWave / NS) * kGrpDownPasses;
    const dim3 grid((a.H + RO - 1) / RO, maxt);
    dec_down_grouped_kernel<QD, NS, kGrpDownPasses><<<grid, kGrpDownWaves * kWave, 0, s>>>(a, g);
    return hipGetLastError();
}

}  // namespace

// Shapes of the expert-grouped path: H = 2,048 or 2,560; Q4_K or Q5_K gate/up
// (the same for both); Q4_K, Q5_K or Q8_0 down with I = 512; batches past the
// two-kernel layer (T*k > 64).
bool dec_grouped_supported(int T, int k, int H, int I, int qg, int qu, int qd) {
    if (T < 1 || T * k <= kDecMaxPairs) return false;
    if (!(qg == kQ4_K || qg == kQ5_K) || qu != qg) return false;
    if (!(qd == kQ4_K || qd == kQ5_K || qd == kQ8_0)) return false;
    return (H == 2048 || H == 2560) && I == 512;
}

size_t dec_grouped_tiles_bytes(int T, int k, int E, int has_shared) {
    return 2 * sizeof(int32_t) * (size_t)grp_max_tiles(T, k, E, has_shared) + 256;
}

hipError_t launch_dec_grouped(const FfnArgs& f, hipStream_t s) {
    const int maxt = grp_max_tiles(f.T, f.k, f.E, f.has_shared);
    const size_t half = (dec_grouped_tiles_bytes(f.T, f.k, f.E, f.has_shared) - 256) / 2;
    int32_t* tile_e = f.tiles;
    int32_t* tile_m0 = f.tiles + half / sizeof(int32_t);
    int32_t* n_tiles = f.tiles + 2 * (half / sizeof(int32_t));
    const TileList tl{tile_e, tile_m0, n_tiles, kGrpTok, maxt, f.T, f.has_shared};
    mfma_tiles_kernel<<<1, 1024, 0, s>>>(f.count, f.E, f.T * f.k, tl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DecArgs a{};
    a.x = f.x;
    a.gate = f.gate;
    a.up = f.up;
    a.down = f.down;
    a.sgate = f.sgate;
    a.sup = f.sup;
    a.sdown = f.sdown;
    a.has_shared = f.has_shared;
    a.T = f.T;
    a.E = f.E;
    a.k = f.k;
    a.H = f.H;
    a.I = f.I;
    a.h = f.h;
    a.y_pair = f.y_pair;
    a.y_shared = f.y_shared;
    const GroupTiles g{tile_e, tile_m0, n_tiles, f.offset, f.pair};
    if (f.H == 2048)
        e = f.gate.qtype == kQ5_K ? launch_grp_gateup<8, kQ5_K>(a, g, maxt, s) : launch_grp_gateup<8, kQ4_K>(a, g, maxt, s);
    else
        e = f.gate.qtype == kQ5_K ? launch_grp_gateup<10, kQ5_K>(a, g, maxt, s)
                                  : launch_grp_gateup<10, kQ4_K>(a, g, maxt, s);
    if (e != hipSuccess) return e;
    if (f.down.qtype == kQ5_K) return launch_grp_down<kQ5_K>(a, g, maxt, s);
    if (f.down.qtype == kQ8_0) return launch_grp_down<kQ8_0>(a, g, maxt, s);
    return launch_grp_down<kQ4_K>(a, g, maxt, s);
}

}  // namespace moe
