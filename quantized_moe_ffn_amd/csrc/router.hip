// router.hip — router projection: logits[t][e] = sum_h W[e][h] * x[t][h] in
// fp32, the GPU stage in front of the top-k ("Strata - the details", "How it
// works": routers run on the GPU, their weights stay in VRAM).
//
// Two kernels, both summing each logit in a fixed order (bitwise
// deterministic, independent of the other tokens of the batch):
//   * decode batches (T <= kRouterGemvMaxT): one workgroup of 4 waves per
//     expert row; each thread holds its float4 columns of the row in registers
//     and the tokens are taken one after the other (a DPP wave sum, then the
//     four wave partials in order).  This is a read of E*H*4 bytes spread over
//     E workgroups.
//   * prompt chunks: fp32 MFMA (v_mfma_f32_32x32x2_f32) on tiles of 32 tokens x
//     32 experts per workgroup, operands loaded as float4 straight from global
//     memory: lane (row, half h) takes columns k0 + 4h .. k0 + 4h + 3 of its
//     token row and of its expert row, and the four MFMAs of the step pair
//     them up in the same order on both sides (MFMA i sums columns k0 + i and
//     k0 + 4 + i).  The four waves of a workgroup split the columns; 4,096
//     tokens x 256 experts make 1,024 workgroups, four waves per SIMD.  The
//     operands are gathered row by row (32 rows per load), not staged through
//     LDS, which keeps this kernel near 30% of the fp32 MFMA peak.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

typedef float v16f_r __attribute__((ext_vector_type(16)));

constexpr int kRouterGemvWaves = 4;

__global__ void __launch_bounds__(kRouterGemvWaves * kWave)
    router_gemv_kernel(const float* __restrict__ x, int T, int H, const float* __restrict__ w, int E,
                       float* __restrict__ logits) {
    __shared__ float s_part[kRouterGemvWaves][kRouterGemvMaxT];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    constexpr int kStride = 4 * kRouterGemvWaves * kWave;    // columns per sweep of the workgroup
    constexpr int kMaxChunks = kRouterMaxH / kStride;
    const float* wr = w + (int64_t)e * H;
    float4 wv[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int col = 4 * tid + c * kStride;
        wv[c] = col < H ? *reinterpret_cast<const float4*>(wr + col) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int t = 0; t < T; ++t) {
        const float* xr = x + (int64_t)t * H;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            const int col = 4 * tid + c * kStride;
            if (col < H) {
                const float4 xv = *reinterpret_cast<const float4*>(xr + col);
                acc = fmaf(wv[c].x, xv.x, acc);
                acc = fmaf(wv[c].y, xv.y, acc);
                acc = fmaf(wv[c].z, xv.z, acc);
                acc = fmaf(wv[c].w, xv.w, acc);
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) s_part[wave][t] = acc;
    }
    __syncthreads();
    if (tid < T) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < kRouterGemvWaves; ++q) s += s_part[q][tid];
        logits[(int64_t)tid * E + e] = s;
    }
}

constexpr int kRouterTile = 32;    // tokens x experts per tile (one MFMA block)
constexpr int kRouterGemmWaves = 4;

// Workgroup blockIdx.x takes token tile blockIdx.x / n_et and expert tile
// blockIdx.x % n_et; its four waves split the columns into four contiguous
// ranges of 8-column steps, and wave 0 adds the four partial tiles in wave
// order (fixed, so the result is deterministic).  Four waves per tile put four
// waves on each SIMD at the prompt-chunk shape; the loads of the next step are
// issued before the MFMAs of the current one.  (Loading a whole 128-byte line
// per lane and step, 32 MFMAs a step, measured slower.)
__global__ void __launch_bounds__(kRouterGemmWaves * kWave)
    router_gemm_kernel(const float* __restrict__ x, int T, int H, const float* __restrict__ w, int E,
                       float* __restrict__ logits, int n_et) {
    __shared__ float s_c[kRouterGemmWaves - 1][16][kWave];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int tt = blockIdx.x / n_et, et = blockIdx.x - tt * n_et;
    const int r = lane & 31, h = lane >> 5;
    const int t = tt * kRouterTile + r, e = et * kRouterTile + r;
    const int steps = H / 8;
    const int s0 = wave * steps / kRouterGemmWaves, s1 = (wave + 1) * steps / kRouterGemmWaves;
    // rows past T or E read a valid row (clamped) and are not stored
    const float* xr = x + (int64_t)min(t, T - 1) * H + 4 * h;
    const float* wr = w + (int64_t)min(e, E - 1) * H + 4 * h;
    v16f_r c = {};
    if (s0 < s1) {
        float4 a = *reinterpret_cast<const float4*>(xr + 8 * s0);
        float4 b = *reinterpret_cast<const float4*>(wr + 8 * s0);
        for (int st = s0; st < s1; ++st) {
            const int kn = 8 * (st + 1 < s1 ? st + 1 : st);
            const float4 an = *reinterpret_cast<const float4*>(xr + kn);
            const float4 bn = *reinterpret_cast<const float4*>(wr + kn);
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, c, 0, 0, 0);
            a = an;
            b = bn;
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s_c[wave - 1][v][lane] = c[v];
    }
    __syncthreads();
    if (wave != 0 || e >= E) return;
    // C[m][n] sits in lane n + 32*((m/4)%2), register 4*(m/8) + m%4
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        float acc = c[v];
#pragma unroll
        for (int q = 0; q < kRouterGemmWaves - 1; ++q) acc += s_c[q][v][lane];
        const int tok = tt * kRouterTile + 8 * (v >> 2) + 4 * h + (v & 3);
        if (tok < T) logits[(int64_t)tok * E + e] = acc;
    }
}

}  // namespace

hipError_t launch_router(const float* x, int T, int H, const float* w, int E, float* logits, hipStream_t s) {
    if (T <= kRouterGemvMaxT) {
        router_gemv_kernel<<<E, kRouterGemvWaves * kWave, 0, s>>>(x, T, H, w, E, logits);
    } else {
        const int n_et = (E + kRouterTile - 1) / kRouterTile;
        const int tiles = ((T + kRouterTile - 1) / kRouterTile) * n_et;
        router_gemm_kernel<<<tiles, kRouterGemmWaves * kWave, 0, s>>>(x, T, H, w, E, logits, n_et);
    }
    return hipGetLastError();
}

}  // namespace moe
