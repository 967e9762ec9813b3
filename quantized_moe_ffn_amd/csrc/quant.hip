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

// One wave per (row, 256-block): lane l holds elements 4l..4l+3.
__global__ void __launch_bounds__(256) quantize_act_kernel(const float* __restrict__ x, int64_t n_blocks,
                                                           int8_t* __restrict__ xq, float* __restrict__ xd) {
    const int64_t blk = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    if (blk >= n_blocks) return;
    const float4 v = reinterpret_cast<const float4*>(x + blk * 256)[lane];
    const bool fin = isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w);
    const bool all_fin = !__any(!fin);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = wave_max(amax);
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
        q = make_char4(qz(v.x), qz(v.y), qz(v.z), qz(v.w));
        d = __fdiv_rn(amax, 127.0f);
    }
    reinterpret_cast<char4*>(xq + blk * 256)[lane] = q;
    if (lane == 0) xd[blk] = d;
}

hipError_t launch_quantize_act(const float* x, int T, int H, int8_t* xq, float* xd, hipStream_t s) {
    const int64_t n_blocks = (int64_t)T * (H / 256);
    quantize_act_kernel<<<(unsigned)((n_blocks + 3) / 4), 256, 0, s>>>(x, n_blocks, xq, xd);
    return hipGetLastError();
}

}  // namespace moe
