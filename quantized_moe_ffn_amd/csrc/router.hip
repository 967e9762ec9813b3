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
//   * prompt chunks: fp32 MFMA (v_mfma_f32_32x32x2_f32) on 64 x 64 tiles per
//     workgroup, the four waves splitting the columns and each running the
//     tile's four 32 x 32 blocks, with float4 operands loaded straight from
//     global memory (see router_gemm_kernel).  Staging 32-column slices
//     through LDS with one 32 x 32 block per wave measured slower.
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

constexpr int kRouterTile = 64;    // tokens x experts per workgroup
constexpr int kRouterGemmWaves = 4;

// Workgroup blockIdx.x takes token tile blockIdx.x / n_et and expert tile
// blockIdx.x % n_et (64 x 64, four 32 x 32 MFMA blocks).  Its four waves split
// the columns into four contiguous ranges of 8-column steps; each wave runs all
// four blocks, so four independent accumulation chains keep the MFMA pipe
// busy and each loaded float4 feeds two blocks.  Lane (row r, half h) loads
// columns k0 + 4h .. k0 + 4h + 3 of token rows r and r + 32 and of expert rows
// r and r + 32; MFMA i of the step sums columns k0 + i and k0 + 4 + i.  Wave 0
// adds the four partial tiles in wave order (fixed, so deterministic).
__global__ void __launch_bounds__(kRouterGemmWaves * kWave)
    router_gemm_kernel(const float* __restrict__ x, int T, int H, const float* __restrict__ w, int E,
                       float* __restrict__ logits, int n_et) {
    __shared__ float s_c[kRouterGemmWaves - 1][4][16][kWave];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int tt = blockIdx.x / n_et, et = blockIdx.x - tt * n_et;
    const int t0 = tt * kRouterTile, e0 = et * kRouterTile;
    const int r = lane & 31, h = lane >> 5;
    const int steps = H / 8;
    const int s0 = wave * steps / kRouterGemmWaves, s1 = (wave + 1) * steps / kRouterGemmWaves;
    // rows past T or E read a valid row (clamped) and are not stored
    const float* x0 = x + (int64_t)min(t0 + r, T - 1) * H + 4 * h;
    const float* x1 = x + (int64_t)min(t0 + r + 32, T - 1) * H + 4 * h;
    const float* w0 = w + (int64_t)min(e0 + r, E - 1) * H + 4 * h;
    const float* w1 = w + (int64_t)min(e0 + r + 32, E - 1) * H + 4 * h;
    v16f_r c[4] = {};   // blocks (token half, expert half): 00, 01, 10, 11
    if (s0 < s1) {
        float4 a0 = *reinterpret_cast<const float4*>(x0 + 8 * s0);
        float4 a1 = *reinterpret_cast<const float4*>(x1 + 8 * s0);
        float4 b0 = *reinterpret_cast<const float4*>(w0 + 8 * s0);
        float4 b1 = *reinterpret_cast<const float4*>(w1 + 8 * s0);
        for (int st = s0; st < s1; ++st) {
            // the next step's loads go out before this step's MFMAs
            const int kn = 8 * (st + 1 < s1 ? st + 1 : st);
            const float4 na0 = *reinterpret_cast<const float4*>(x0 + kn);
            const float4 na1 = *reinterpret_cast<const float4*>(x1 + kn);
            const float4 nb0 = *reinterpret_cast<const float4*>(w0 + kn);
            const float4 nb1 = *reinterpret_cast<const float4*>(w1 + kn);
            const float av[2][4] = {{a0.x, a0.y, a0.z, a0.w}, {a1.x, a1.y, a1.z, a1.w}};
            const float bv[2][4] = {{b0.x, b0.y, b0.z, b0.w}, {b1.x, b1.y, b1.z, b1.w}};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    c[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[q >> 1][i], bv[q & 1][i], c[q], 0, 0, 0);
            a0 = na0;
            a1 = na1;
            b0 = nb0;
            b1 = nb1;
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int v = 0; v < 16; ++v) s_c[wave - 1][q][v][lane] = c[q][v];
    }
    __syncthreads();
    if (wave != 0) return;
    // C[m][n] sits in lane n + 32*((m/4)%2), register 4*(m/8) + m%4
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = e0 + (q & 1) * 32 + r;
        if (e >= E) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float acc = c[q][v];
#pragma unroll
            for (int p = 0; p < kRouterGemmWaves - 1; ++p) acc += s_c[p][q][v][lane];
            const int tok = t0 + (q >> 1) * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            if (tok < T) logits[(int64_t)tok * E + e] = acc;
        }
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
