// quant.hip — per-token int8 activation quantisation, once per token and
// 256-wide block ("one quantization per token", the prompt-side expert stream
// of the "Strata-Sage-A1.5-GGUF" card's round-2 table; q8_1 activations kept
// finite, "Strata v0.1.39" release notes, fixes).
//
// Rule, evaluated in IEEE fp32: amax = max|x|; amax == 0 -> d = 0, q = 0;
// otherwise id = 127/amax (correctly rounded division), q = rint(x*id) with
// ties to even, clamped to +-127, d = amax/127.  A block holding a non-finite
// value raises the error word and is written as q = 0, d = 0.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kQBlocksPerWave = 4;   // blocks of one wave, loaded together

// Wave number wv quantises kQBlocksPerWave consecutive (row, 256-block)s: lane
// l holds elements 4l..4l+3 of each.  With xs non-null it also writes the exact
// sums of every 32 codes (int16, |sum| <= 4064), which the int8 MFMA GEMMs use.
__device__ void quantize_act_wave(int64_t wv, const float* __restrict__ x, int64_t n_blocks,
                                  int8_t* __restrict__ xq, float* __restrict__ xd, int16_t* __restrict__ xs) {
    const int64_t blk0 = wv * kQBlocksPerWave;
    const int lane = threadIdx.x & (kWave - 1);
    if (blk0 >= n_blocks) return;
    float4 v[kQBlocksPerWave];
#pragma unroll
    for (int b = 0; b < kQBlocksPerWave; ++b) {   // a block past the end reloads the last one, never stored
        const int64_t blk = blk0 + b < n_blocks ? blk0 + b : n_blocks - 1;
        v[b] = reinterpret_cast<const float4*>(x + blk * 256)[lane];
    }
#pragma unroll
    for (int b = 0; b < kQBlocksPerWave; ++b) {
        const int64_t blk = blk0 + b;
        if (blk >= n_blocks) break;
        const bool fin = isfinite(v[b].x) && isfinite(v[b].y) && isfinite(v[b].z) && isfinite(v[b].w);
        const bool all_fin = !__any(!fin);
        float amax = fmaxf(fmaxf(fabsf(v[b].x), fabsf(v[b].y)), fmaxf(fabsf(v[b].z), fabsf(v[b].w)));
        // |x| >= 0 orders as its bit pattern: the DPP maximum of unsigned values
        amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));
        char4 q = make_char4(0, 0, 0, 0);
        float d = 0.0f;
        if (!all_fin) {
            if (lane == 0) raise_error(kErrActNonFinite);
        } else if (amax > 0.0f) {
            const float id = __fdiv_rn(127.0f, amax);
            auto qz = [&](float a) -> signed char {
                float r = rintf(__fmul_rn(a, id));
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                return (signed char)(int)r;
            };
            q = make_char4(qz(v[b].x), qz(v[b].y), qz(v[b].z), qz(v[b].w));
            d = __fdiv_rn(amax, 127.0f);
        }
        reinterpret_cast<char4*>(xq + blk * 256)[lane] = q;
        if (lane == 0) xd[blk] = d;
        if (xs) {   // lanes 8c .. 8c + 7 hold codes 32c .. 32c + 31 (sums exact in fp32)
            const float s32 = segment_sum<8>((float)((int)q.x + (int)q.y + (int)q.z + (int)q.w));
            if ((lane & 7) == 7) xs[blk * 8 + (lane >> 3)] = (int16_t)(int)s32;
        }
    }
}

__global__ void __launch_bounds__(256) quantize_act_kernel(const float* __restrict__ x, int64_t n_blocks,
                                                           int8_t* __restrict__ xq, float* __restrict__ xd,
                                                           int16_t* __restrict__ xs) {
    quantize_act_wave((int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave, x, n_blocks, xq, xd, xs);
}

// Waves of quantize_act_wave that cover T rows of H (H a multiple of 256).
int64_t quantize_act_waves(int T, int H) {
    const int64_t n_blocks = (int64_t)T * (H / 256);
    return (n_blocks + kQBlocksPerWave - 1) / kQBlocksPerWave;
}

hipError_t launch_quantize_act(const float* x, int T, int H, int8_t* xq, float* xd, hipStream_t s,
                               int16_t* xs) {
    const int64_t n_blocks = (int64_t)T * (H / 256);
    const int64_t waves = quantize_act_waves(T, H);
    quantize_act_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, s>>>(x, n_blocks, xq, xd, xs);
    return hipGetLastError();
}

}  // namespace moe
