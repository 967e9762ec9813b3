// qblock.h — device-side unpacking of Q4_K, Q5_K, Q8_0 and Q5_1 blocks, shared by the FFN
// kernels and the dequantization test hook (so the hook exercises the exact
// loads, nibble splits and scale decoding the FFN kernels use).
#pragma once

#include "common.h"

namespace moe {

// A Q4_K "slice": 16 quant bytes of one super-block = 16 weights of sub-block
// 2c (low nibbles) and 16 weights of sub-block 2c+1 (high nibbles), where the
// slice index part = 2c + half (0..7) selects qs[32c + 16*half .. +16].
//   low nibble  of byte i -> weight 64c + 16*half + i       (sub-block 2c)
//   high nibble of byte i -> weight 64c + 32 + 16*half + i  (sub-block 2c+1)
struct Q4KSlice {
    uint32_t q[4];          // the 16 quant bytes
    float d, dmin;          // super-block scales
    int sc_lo, m_lo;        // sub-block 2c
    int sc_hi, m_hi;        // sub-block 2c+1
};

__device__ __forceinline__ void q4k_load_slice(const uint8_t* __restrict__ blk, int part, Q4KSlice& s) {
    const uint4 hv = *reinterpret_cast<const uint4*>(blk);
    const uint4 qv = *reinterpret_cast<const uint4*>(blk + 16 + 16 * part);
    const Q4KHead h{hv.x, hv.y, hv.z, hv.w};
    s.q[0] = qv.x;
    s.q[1] = qv.y;
    s.q[2] = qv.z;
    s.q[3] = qv.w;
    s.d = q4k_d(h);
    s.dmin = q4k_dmin(h);
    const int c = part >> 1;
    q4k_scale_min(h, 2 * c, s.sc_lo, s.m_lo);
    q4k_scale_min(h, 2 * c + 1, s.sc_hi, s.m_hi);
}

// First weight index (within the super-block) of the low / high halves of a slice.
__device__ __forceinline__ int q4k_slice_col_lo(int part) { return 64 * (part >> 1) + 16 * (part & 1); }
__device__ __forceinline__ int q4k_slice_col_hi(int part) { return q4k_slice_col_lo(part) + 32; }

__device__ __forceinline__ int q4k_slice_qlo(const Q4KSlice& s, int i) {
    return (int)((s.q[i >> 2] >> (8 * (i & 3))) & 15u);
}
__device__ __forceinline__ int q4k_slice_qhi(const Q4KSlice& s, int i) {
    return (int)((s.q[i >> 2] >> (8 * (i & 3) + 4)) & 15u);
}

// A Q5_K slice: the Q4_K slice of the same part (Q5_K keeps Q4_K's header and
// quant layout, the quants 32 bytes further on) plus the 16 fifth-bit bytes of
// its weights: qh[16*half + i] holds the fifth bit of the low-nibble weight i
// in bit 2c and of the high-nibble weight i in bit 2c+1 (176-byte blocks:
// d, dmin, 12 scale bytes, qh[32], qs[128]).
struct Q5KSlice {
    Q4KSlice s;        // header fields and the 16 low-bit bytes
    uint32_t h[4];     // the 16 fifth-bit bytes
    int c;             // 64-weight chunk of the slice
};

__device__ __forceinline__ void q5k_load_slice(const uint8_t* __restrict__ blk, int part, Q5KSlice& s) {
    const uint4 hv = *reinterpret_cast<const uint4*>(blk);
    const uint4 bv = *reinterpret_cast<const uint4*>(blk + 16 + 16 * (part & 1));
    const uint4 qv = *reinterpret_cast<const uint4*>(blk + 48 + 16 * part);
    const Q4KHead h{hv.x, hv.y, hv.z, hv.w};
    s.s.q[0] = qv.x;
    s.s.q[1] = qv.y;
    s.s.q[2] = qv.z;
    s.s.q[3] = qv.w;
    s.s.d = q4k_d(h);
    s.s.dmin = q4k_dmin(h);
    s.c = part >> 1;
    q4k_scale_min(h, 2 * s.c, s.s.sc_lo, s.s.m_lo);
    q4k_scale_min(h, 2 * s.c + 1, s.s.sc_hi, s.s.m_hi);
    s.h[0] = bv.x;
    s.h[1] = bv.y;
    s.h[2] = bv.z;
    s.h[3] = bv.w;
}

__device__ __forceinline__ int q5k_slice_qlo(const Q5KSlice& s, int i) {
    return q4k_slice_qlo(s.s, i) + 16 * (int)((s.h[i >> 2] >> (8 * (i & 3) + 2 * s.c)) & 1u);
}
__device__ __forceinline__ int q5k_slice_qhi(const Q5KSlice& s, int i) {
    return q4k_slice_qhi(s.s, i) + 16 * (int)((s.h[i >> 2] >> (8 * (i & 3) + 2 * s.c + 1)) & 1u);
}

// Q8_0 block: 2-byte aligned (34-byte blocks), read as 17 halfwords.
struct Q80Block {
    float d;
    uint32_t q[8];  // 32 int8 quants, little-endian in 8 dwords
};

__device__ __forceinline__ void q80_load(const uint8_t* __restrict__ blk, Q80Block& b) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(blk);
    b.d = f16_bits_to_f32(p[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) b.q[i] = (uint32_t)p[1 + 2 * i] | ((uint32_t)p[2 + 2 * i] << 16);
}

__device__ __forceinline__ int q80_quant(const Q80Block& b, int i) {
    return (int)(int8_t)((b.q[i >> 2] >> (8 * (i & 3))) & 0xFFu);
}

// Q5_1 block: 24 bytes, 8-byte aligned (row starts and 24-byte blocks):
// fp16 d, fp16 m, a 32-bit word qh whose bit i is the fifth bit of quant i, and
// 16 bytes qs whose byte l holds the low four bits of quant l (low nibble) and
// of quant 16 + l (high nibble); w = d*q + m.
struct Q51Block {
    float d, m;
    uint32_t qh;
    uint32_t qs[4];
};

__device__ __forceinline__ void q51_load(const uint8_t* __restrict__ blk, Q51Block& b) {
    const uint2* p = reinterpret_cast<const uint2*>(blk);
    const uint2 v0 = p[0], v1 = p[1], v2 = p[2];
    b.d = f16_bits_to_f32(v0.x & 0xFFFFu);
    b.m = f16_bits_to_f32(v0.x >> 16);
    b.qh = v0.y;
    b.qs[0] = v1.x;
    b.qs[1] = v1.y;
    b.qs[2] = v2.x;
    b.qs[3] = v2.y;
}

__device__ __forceinline__ int q51_quant(const Q51Block& b, int i) {
    const int l = i & 15;
    const uint32_t byte = (b.qs[l >> 2] >> (8 * (l & 3))) & 0xFFu;
    const uint32_t low4 = i < 16 ? (byte & 15u) : (byte >> 4);
    return (int)(low4 | (((b.qh >> i) & 1u) << 4));
}

}  // namespace moe
