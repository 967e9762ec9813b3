// common.h — device helpers shared by the libmoe kernels (gfx950, wave64).
//
// Block formats (GGUF layouts; the pages name Q4_K and Q8_0 as expert formats,
// "Strata v0.1.31" release notes, Unsloth UD-Q4_K_XL bullet, and the
// "Strata-Sage-A1.5-GGUF" card's flag table, without a byte layout):
//   Q4_K, 144 B / 256 weights:
//     [0:2] d fp16 | [2:4] dmin fp16 | [4:16] s[12] | [16:144] qs[128]
//     sub-block j (weights 32j..32j+31): j < 4: sc = s[j] & 63, m = s[j+4] & 63
//       j >= 4: sc = (s[j+4] & 15) | (s[j-4] >> 6) << 4, m = (s[j+4] >> 4) | (s[j] >> 6) << 4
//     qs[32c+l]: low nibble = weight 64c+l, high nibble = weight 64c+32+l
//     w = d*sc*q - dmin*m
//   Q8_0, 34 B / 32 weights: [0:2] d fp16 | [2:34] q int8;  w = d*q
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kQ5_1 = 7;
constexpr int kQ8_0 = 8;
constexpr int kQ4_K = 12;
constexpr int kQ5_K = 13;
constexpr int kWave = 64;

// Bits of the per-device error word.
constexpr unsigned kErrExpertRange = 1u;   // an expert id outside [0, E)
constexpr unsigned kErrPairRange = 2u;     // bucket offsets / pair ids outside their range
constexpr unsigned kErrLogitNonFinite = 4u;
constexpr unsigned kErrActNonFinite = 8u;

extern __device__ unsigned int g_moe_err;

__device__ __forceinline__ void raise_error(unsigned bits) { atomicOr(&g_moe_err, bits); }

// IEEE binary16 bits -> fp32 (exact, subnormals included: v_cvt_f32_f16 with
// fp16 denormals enabled, the HIP default).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Q4_K header as four dwords: h0 = d | dmin << 16, h1 = s[0..3], h2 = s[4..7], h3 = s[8..11].
struct Q4KHead {
    uint32_t h0, h1, h2, h3;
};

__device__ __forceinline__ float q4k_d(const Q4KHead& h) { return f16_bits_to_f32(h.h0 & 0xFFFFu); }
__device__ __forceinline__ float q4k_dmin(const Q4KHead& h) { return f16_bits_to_f32(h.h0 >> 16); }

// 6-bit scale and min of sub-block j (0..7).
__device__ __forceinline__ void q4k_scale_min(const Q4KHead& h, int j, int& sc, int& m) {
    if (j < 4) {
        sc = (h.h1 >> (8 * j)) & 63;
        m = (h.h2 >> (8 * j)) & 63;
    } else {
        const int jj = j - 4;
        sc = ((h.h3 >> (8 * jj)) & 15) | (((h.h1 >> (8 * jj + 6)) & 3) << 4);
        m = ((h.h3 >> (8 * jj + 4)) & 15) | (((h.h2 >> (8 * jj + 6)) & 3) << 4);
    }
}

// Quant of weight i (0..255) from the 128 quant bytes viewed as 32 dwords.
__device__ __forceinline__ int q4k_quant(const uint32_t* qs32, int i) {
    const int c = i >> 6, l = i & 31, hi = (i >> 5) & 1;
    const int byte = 32 * c + l;
    const uint32_t b = (qs32[byte >> 2] >> (8 * (byte & 3))) & 0xFFu;
    return hi ? (int)(b >> 4) : (int)(b & 15u);
}

// DPP lane moves (no LDS round trip).  Lanes outside row_mask, or whose
// source is invalid, read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}

// Sum over aligned segments of SEG lanes (SEG in 4..64), in a fixed order:
// quad swaps, then half-row and row mirrors, then row broadcasts.  The segment
// total is valid in every lane for SEG <= 16, in the odd 16-lane row of each
// 32-lane half for SEG == 32, and in lanes 48..63 for SEG == 64; lane
// (segment end - 1) always holds it.
template <int SEG>
__device__ __forceinline__ float segment_sum(float v) {
    static_assert(SEG == 4 || SEG == 8 || SEG == 16 || SEG == 32 || SEG == 64, "segment size");
    v += dpp_f<0xB1>(v);                       // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);                       // quad_perm [2,3,0,1]
    if constexpr (SEG >= 8) v += dpp_f<0x141>(v);        // row_half_mirror
    if constexpr (SEG >= 16) v += dpp_f<0x140>(v);       // row_mirror
    if constexpr (SEG >= 32) v += dpp_f<0x142, 0xA>(v);  // row_bcast15 into rows 1, 3
    if constexpr (SEG >= 64) v += dpp_f<0x143, 0xC>(v);  // row_bcast31 into rows 2, 3
    return v;
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, true);
}

// Wave64 maximum of unsigned values, the same value in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u<0xB1>(v));
    v = max(v, dpp_u<0x4E>(v));
    v = max(v, dpp_u<0x141>(v));
    v = max(v, dpp_u<0x140>(v));
    v = max(v, dpp_u<0x142, 0xA>(v));
    v = max(v, dpp_u<0x143, 0xC>(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Wave64 sum, the same value in every lane, in a fixed order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
    v = segment_sum<64>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}


// Byte N of a dword as fp32 (one v_cvt_f32_ubyteN).
template <int N>
__device__ __forceinline__ float ubyte_f32(uint32_t v) {
    return (float)((v >> (8 * N)) & 0xFFu);
}

// silu(g) = g / (1 + e^-g), with the hardware reciprocal (about 1 ulp).  For
// g >= 17, 1 + e^-g rounds to 1 and the result is g exactly; for very negative
// g the reciprocal of +inf is 0 and the result is -0.
__device__ __forceinline__ float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Sigmoid gate of the shared expert for one token, by one wave:
// 1 / (1 + e^-z), z = g . x.  Lane l takes the float4 columns 4l, 4l + 256, ...
// in order and the wave adds the lanes with the fixed DPP tree, so every
// caller (the decode layer's routing workgroup, the separate gate kernel) gets
// the same bits.  g and x 16-byte aligned, H a multiple of 4.
__device__ __forceinline__ float shared_gate_wave(const float* __restrict__ g, const float* __restrict__ x, int H) {
    const int lane = threadIdx.x & (kWave - 1);
    float acc = 0.f;
    for (int c = 4 * lane; c < H; c += 4 * kWave) {
        const float4 gv = *reinterpret_cast<const float4*>(g + c);
        const float4 xv = *reinterpret_cast<const float4*>(x + c);
        acc = fmaf(gv.x, xv.x, acc);
        acc = fmaf(gv.y, xv.y, acc);
        acc = fmaf(gv.z, xv.z, acc);
        acc = fmaf(gv.w, xv.w, acc);
    }
    const float z = wave_sum(acc);
    return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

}  // namespace moe
