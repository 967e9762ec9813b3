// ffn_decode.hip — expert FFN with weights dequantized inside the dot products.
//
// The expert FFN of a routed MoE layer (Sage-A1.5: 256 experts / top-8, Q4_K
// down experts, "Strata-Sage-A1.5-GGUF" card; Flash-Next: 10 routed + 1 shared
// of 512, "Strata: a 125B MoE at 94 tok/s"), with the GGUF blocks decoded in
// registers rather than expanded to fp16 first ("Strata - the details", faster
// prompts: quantized kernels instead of FP16 expansion).
//
// Work split: one workgroup per (expert slot, tile of output rows).  Each
// workgroup streams its rows of the expert's matrices once and applies them to
// every token routed to that expert (tokens staged in LDS, kTokChunk at a time),
// so an expert shared by several tokens of a verify window is read once.
// Expert ids and token lists come from device memory (no host round trip).
//
// Dot products: a lane takes 16-byte quant slices of the row (32 weights each)
// and factors the Q4_K sub-block scale and min out of the inner sums:
//   sum_i w_i x_i = d * (sc_a S_a + sc_b S_b) - dmin * (m_a X_a + m_b X_b)
// with S = sum q*x, X = sum x over the lane's 16 weights of each sub-block;
// the wave then reduces across lanes with a butterfly (fixed order, so the
// result is bitwise deterministic).
#include "common.h"
#include "kernels.h"
#include "qblock.h"

namespace moe {

constexpr int kTokChunk = 4;
constexpr int kWaves = 4;

__device__ unsigned int g_moe_err = 0;

// Per-lane partial dots of one quantized row (cols weights) with nt vectors
// xs[t*xstride + c] held in LDS.
template <int QT>
__device__ __forceinline__ void row_partial(const uint8_t* __restrict__ row, int cols,
                                            const float* xs, int xstride, int nt,
                                            float acc[kTokChunk]) {
    const int lane = threadIdx.x & (kWave - 1);
    if constexpr (QT == kQ4_K) {
        const int nslices = (cols >> 8) * 8;
        for (int sidx = lane; sidx < nslices; sidx += kWave) {
            const int b = sidx >> 3, part = sidx & 7;
            Q4KSlice s;
            q4k_load_slice(row + (int64_t)b * 144, part, s);
            float qlo[16], qhi[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                qlo[i] = (float)q4k_slice_qlo(s, i);
                qhi[i] = (float)q4k_slice_qhi(s, i);
            }
            const int clo = 256 * b + q4k_slice_col_lo(part);
            const int chi = 256 * b + q4k_slice_col_hi(part);
            for (int t = 0; t < nt; ++t) {
                const float* xv = xs + t * xstride;
                float slo = 0.f, shi = 0.f, xlo = 0.f, xhi = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float a = xv[clo + i], c = xv[chi + i];
                    slo = fmaf(qlo[i], a, slo);
                    shi = fmaf(qhi[i], c, shi);
                    xlo += a;
                    xhi += c;
                }
                acc[t] += s.d * ((float)s.sc_lo * slo + (float)s.sc_hi * shi) -
                          s.dmin * ((float)s.m_lo * xlo + (float)s.m_hi * xhi);
            }
        }
    } else if constexpr (QT == kQ5_K) {
        const int nslices = (cols >> 8) * 8;
        for (int sidx = lane; sidx < nslices; sidx += kWave) {
            const int b = sidx >> 3, part = sidx & 7;
            Q5KSlice s;
            q5k_load_slice(row + (int64_t)b * 176, part, s);
            float qlo[16], qhi[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                qlo[i] = (float)q5k_slice_qlo(s, i);
                qhi[i] = (float)q5k_slice_qhi(s, i);
            }
            const int clo = 256 * b + q4k_slice_col_lo(part);
            const int chi = 256 * b + q4k_slice_col_hi(part);
            for (int t = 0; t < nt; ++t) {
                const float* xv = xs + t * xstride;
                float slo = 0.f, shi = 0.f, xlo = 0.f, xhi = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float a = xv[clo + i], c = xv[chi + i];
                    slo = fmaf(qlo[i], a, slo);
                    shi = fmaf(qhi[i], c, shi);
                    xlo += a;
                    xhi += c;
                }
                acc[t] += s.s.d * ((float)s.s.sc_lo * slo + (float)s.s.sc_hi * shi) -
                          s.s.dmin * ((float)s.s.m_lo * xlo + (float)s.s.m_hi * xhi);
            }
        }
    } else if constexpr (QT == kQ5_1) {
        // sum w x = d * sum q x + m * sum x over the block's 32 weights
        const int nblocks = cols >> 5;
        for (int b = lane; b < nblocks; b += kWave) {
            Q51Block blk;
            q51_load(row + (int64_t)b * 24, blk);
            float q[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) q[i] = (float)q51_quant(blk, i);
            for (int t = 0; t < nt; ++t) {
                const float* xv = xs + t * xstride + 32 * b;
                float sq = 0.f, sx = 0.f;
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    sq = fmaf(q[i], xv[i], sq);
                    sx += xv[i];
                }
                acc[t] += blk.d * sq + blk.m * sx;
            }
        }
    } else {
        const int nblocks = cols >> 5;
        for (int b = lane; b < nblocks; b += kWave) {
            Q80Block blk;
            q80_load(row + (int64_t)b * 34, blk);
            float q[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) q[i] = (float)q80_quant(blk, i);
            for (int t = 0; t < nt; ++t) {
                const float* xv = xs + t * xstride + 32 * b;
                float sacc = 0.f;
#pragma unroll
                for (int i = 0; i < 32; ++i) sacc = fmaf(q[i], xv[i], sacc);
                acc[t] += blk.d * sacc;
            }
        }
    }
}

// Resolves the expert slot of this workgroup.  Returns false when the slot is
// empty (or invalid: then the error word is raised).
struct SlotInfo {
    int e;          // expert index inside the bank (0 for the shared expert)
    int p0, p1;     // range in the pair list (shared: token range)
    bool shared;
};

__device__ __forceinline__ bool resolve_slot(const FfnArgs& a, int slot, SlotInfo& si) {
    si.shared = (slot == a.n_slots);
    if (si.shared) {
        si.e = 0;
        si.p0 = 0;
        si.p1 = a.T;
        return true;
    }
    if (slot >= *a.n_active) return false;
    si.e = a.active[slot];
    if (si.e < 0 || si.e >= a.E) {
        if (threadIdx.x == 0) raise_error(kErrExpertRange);
        return false;
    }
    si.p0 = a.offset[si.e];
    si.p1 = a.offset[si.e + 1];
    if (si.p0 < 0 || si.p1 < si.p0 || si.p1 > a.T * a.k) {
        if (threadIdx.x == 0) raise_error(kErrPairRange);
        return false;
    }
    return true;
}

// Token index and output row of the q-th entry of a slot (-1 if invalid).
__device__ __forceinline__ void slot_entry(const FfnArgs& a, const SlotInfo& si, int q, int& tok,
                                           int& hrow) {
    if (si.shared) {
        tok = q;
        hrow = a.T * a.k + q;
        return;
    }
    const int p = a.pair[q];
    if (p < 0 || p >= a.T * a.k) {
        raise_error(kErrPairRange);
        tok = -1;
        hrow = -1;
        return;
    }
    tok = p / a.k;
    hrow = p;
}

// gate/up + SiLU: h[row][i] = silu(g_i) * u_i for the rows i of this tile.
// xmode 0: x fp32; xmode 1: x = xd * xq (the int8 path's activations).
template <int QG, int QU, int RPW>
__global__ void __launch_bounds__(kWaves * kWave) gateup_decode_kernel(FfnArgs a, int xmode) {
    extern __shared__ float s_x[];  // [kTokChunk][H]
    __shared__ int s_tok[kTokChunk], s_row[kTokChunk];
    SlotInfo si;
    if (!resolve_slot(a, blockIdx.y, si)) return;
    const QMat G = si.shared ? a.sgate : a.gate;
    const QMat U = si.shared ? a.sup : a.up;
    const uint8_t* Gb = G.data + (int64_t)si.e * G.expert_bytes;
    const uint8_t* Ub = U.data + (int64_t)si.e * U.expert_bytes;
    const int H = a.H, I = a.I;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int i0 = blockIdx.x * (kWaves * RPW) + wave * RPW;
    for (int q0 = si.p0; q0 < si.p1; q0 += kTokChunk) {
        const int nt = min(kTokChunk, si.p1 - q0);
        __syncthreads();
        if (threadIdx.x < nt) {
            int tok, row;
            slot_entry(a, si, q0 + threadIdx.x, tok, row);
            s_tok[threadIdx.x] = tok;
            s_row[threadIdx.x] = row;
        }
        __syncthreads();
        for (int j = threadIdx.x; j < nt * H; j += blockDim.x) {
            const int t = j / H, c = j - t * H;
            const int tok = s_tok[t];
            float v = 0.f;
            if (tok >= 0) {
                v = xmode == 0 ? a.x[(int64_t)tok * H + c]
                               : a.xd[(int64_t)tok * (H >> 8) + (c >> 8)] * (float)a.xq[(int64_t)tok * H + c];
            }
            s_x[j] = v;
        }
        __syncthreads();
        for (int r = 0; r < RPW; ++r) {
            const int i = i0 + r;
            if (i >= I) break;
            float ag[kTokChunk] = {0.f, 0.f, 0.f, 0.f}, au[kTokChunk] = {0.f, 0.f, 0.f, 0.f};
            row_partial<QG>(Gb + (int64_t)i * G.row_bytes, H, s_x, H, nt, ag);
            row_partial<QU>(Ub + (int64_t)i * U.row_bytes, H, s_x, H, nt, au);
            for (int t = 0; t < nt; ++t) {
                const float g = wave_sum(ag[t]);
                const float u = wave_sum(au[t]);
                if (lane == 0 && s_row[t] >= 0) a.h[(int64_t)s_row[t] * I + i] = silu_f32(g) * u;
            }
        }
    }
}

// down: y[row][o] = sum_i W_down[o][i] * h[row][i] for the rows o of this tile.
// hmode 0: h fp32; hmode 1: h = hd * hq (the int8 path's quantized h).
template <int QD, int RPW>
__global__ void __launch_bounds__(kWaves * kWave) down_decode_kernel(FfnArgs a, int hmode) {
    extern __shared__ float s_h[];  // [kTokChunk][I]
    __shared__ int s_row[kTokChunk], s_tok[kTokChunk];
    SlotInfo si;
    if (!resolve_slot(a, blockIdx.y, si)) return;
    const QMat D = si.shared ? a.sdown : a.down;
    const uint8_t* Db = D.data + (int64_t)si.e * D.expert_bytes;
    const int H = a.H, I = a.I;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int o0 = blockIdx.x * (kWaves * RPW) + wave * RPW;
    for (int q0 = si.p0; q0 < si.p1; q0 += kTokChunk) {
        const int nt = min(kTokChunk, si.p1 - q0);
        __syncthreads();
        if (threadIdx.x < nt) {
            int tok, row;
            slot_entry(a, si, q0 + threadIdx.x, tok, row);
            s_tok[threadIdx.x] = tok;
            s_row[threadIdx.x] = row;
        }
        __syncthreads();
        for (int j = threadIdx.x; j < nt * I; j += blockDim.x) {
            const int t = j / I, c = j - t * I;
            const int row = s_row[t];
            float v = 0.f;
            if (row >= 0) {
                v = hmode == 0 ? a.h[(int64_t)row * I + c]
                               : a.hd[(int64_t)row * (I >> 8) + (c >> 8)] * (float)a.hq[(int64_t)row * I + c];
            }
            s_h[j] = v;
        }
        __syncthreads();
        for (int r = 0; r < RPW; ++r) {
            const int o = o0 + r;
            if (o >= H) break;
            float acc[kTokChunk] = {0.f, 0.f, 0.f, 0.f};
            row_partial<QD>(Db + (int64_t)o * D.row_bytes, I, s_h, I, nt, acc);
            for (int t = 0; t < nt; ++t) {
                const float y = wave_sum(acc[t]);
                if (lane == 0 && s_row[t] >= 0) {
                    if (si.shared)
                        a.y_shared[(int64_t)s_tok[t] * H + o] = y;
                    else
                        a.y_pair[(int64_t)s_row[t] * H + o] = y;
                }
            }
        }
    }
}

namespace {

constexpr int kGateRpw = 4;
constexpr int kDownRpw = 8;

template <int QG, int QU>
hipError_t launch_gateup_q(const FfnArgs& a, int xmode, hipStream_t s) {
    dim3 grid((a.I + kWaves * kGateRpw - 1) / (kWaves * kGateRpw), a.n_slots + (a.has_shared ? 1 : 0));
    size_t lds = (size_t)kTokChunk * a.H * sizeof(float);
    gateup_decode_kernel<QG, QU, kGateRpw><<<grid, kWaves * kWave, lds, s>>>(a, xmode);
    return hipGetLastError();
}

template <int QD>
hipError_t launch_down_q(const FfnArgs& a, int hmode, hipStream_t s) {
    dim3 grid((a.H + kWaves * kDownRpw - 1) / (kWaves * kDownRpw), a.n_slots + (a.has_shared ? 1 : 0));
    size_t lds = (size_t)kTokChunk * a.I * sizeof(float);
    down_decode_kernel<QD, kDownRpw><<<grid, kWaves * kWave, lds, s>>>(a, hmode);
    return hipGetLastError();
}

}  // namespace

// The shared expert may use other formats than the routed ones; the launch
// templates dispatch on the routed formats, and the kernels read the shared
// matrices' formats from the same template parameters, so both must agree
// (checked by the API layer).
namespace {

template <int QG>
hipError_t launch_gateup_g(const FfnArgs& a, int xmode, hipStream_t s) {
    if (a.up.qtype == kQ4_K) return launch_gateup_q<QG, kQ4_K>(a, xmode, s);
    if (a.up.qtype == kQ5_K) return launch_gateup_q<QG, kQ5_K>(a, xmode, s);
    if (a.up.qtype == kQ5_1) return launch_gateup_q<QG, kQ5_1>(a, xmode, s);
    return launch_gateup_q<QG, kQ8_0>(a, xmode, s);
}

}  // namespace

hipError_t launch_gateup(const FfnArgs& a, int xmode, hipStream_t s) {
    if (a.gate.qtype == kQ4_K) return launch_gateup_g<kQ4_K>(a, xmode, s);
    if (a.gate.qtype == kQ5_K) return launch_gateup_g<kQ5_K>(a, xmode, s);
    if (a.gate.qtype == kQ5_1) return launch_gateup_g<kQ5_1>(a, xmode, s);
    return launch_gateup_g<kQ8_0>(a, xmode, s);
}

hipError_t launch_down(const FfnArgs& a, int hmode, hipStream_t s) {
    if (a.down.qtype == kQ4_K) return launch_down_q<kQ4_K>(a, hmode, s);
    if (a.down.qtype == kQ5_K) return launch_down_q<kQ5_K>(a, hmode, s);
    if (a.down.qtype == kQ5_1) return launch_down_q<kQ5_1>(a, hmode, s);
    return launch_down_q<kQ8_0>(a, hmode, s);
}

hipError_t launch_ffn_decode(const FfnArgs& a, hipStream_t s) {
    // batches past the two-kernel layer: the expert-grouped kernels when the
    // shape is theirs (the caller gave them their tile-list workspace)
    if (a.tiles && ((uintptr_t)a.x % 16) == 0 &&
        dec_grouped_supported(a.T, a.k, a.H, a.I, a.gate.qtype, a.up.qtype, a.down.qtype))
        return launch_dec_grouped(a, s);
    hipError_t e = launch_gateup(a, 0, s);
    if (e != hipSuccess) return e;
    return launch_down(a, 0, s);
}

// ---------------------------------------------------------------------------
// Combine and the dequantization test hook.
// ---------------------------------------------------------------------------
// The per-pair rows as the combine reads them: fp32, or bf16 (the layer
// call's MOE_FFN_PAIR_BF16 hand-off, four values per uint2), widened exactly.
__device__ __forceinline__ float pair_value(float v) { return v; }
__device__ __forceinline__ float pair_value(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float4 pair_values(float4 v) { return v; }
__device__ __forceinline__ float4 pair_values(uint2 b) {
    return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u), __uint_as_float(b.y << 16),
                       __uint_as_float(b.y & 0xFFFF0000u));
}

// out may be the residual array itself (each element is read, then written, by
// one thread), so neither carries __restrict__.
template <typename YE>
__global__ void __launch_bounds__(256) combine_kernel(const YE* __restrict__ y_pair,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ y_shared,
                                                      const float* __restrict__ shared_scale,
                                                      const float* __restrict__ sgate, const float* residual,
                                                      int T, int k, int H, float* out) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)T * H) return;
    const int t = (int)(idx / H), o = (int)(idx - (int64_t)t * H);
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = fmaf(w[t * k + j], pair_value(y_pair[((int64_t)t * k + j) * H + o]), acc);
    if (y_shared) {
        const float sc = (shared_scale ? shared_scale[t] : 1.0f) * (sgate ? sgate[t] : 1.0f);
        acc = fmaf(sc, y_shared[(int64_t)t * H + o], acc);
    }
    if (residual) acc += residual[idx];
    out[idx] = acc;
}

// Four consecutive outputs per thread with 16-byte loads and stores (the same
// per-element summation order as combine_kernel, so the same bits). The pair
// rows of a token are loaded kRows at a time before any of them is summed, so a
// thread waits on one memory round trip per kRows rows, not one per row.
template <typename YE4>
__global__ void __launch_bounds__(256) combine4_kernel(const YE4* __restrict__ y_pair,
                                                       const float* __restrict__ w,
                                                       const float4* __restrict__ y_shared,
                                                       const float* __restrict__ shared_scale,
                                                       const float* __restrict__ sgate, const float4* residual,
                                                       int T, int k, int H4, float4* out) {
    constexpr int kRows = 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)T * H4) return;
    const int t = (int)(idx / H4), o = (int)(idx - (int64_t)t * H4);
    const YE4* yp = y_pair + (int64_t)t * k * H4 + o;
    const float* wt = w + (int64_t)t * k;
    float4 ys = make_float4(0.f, 0.f, 0.f, 0.f), rs = ys;
    float ss = 1.0f, sg = 1.0f;
    if (y_shared) {
        ys = y_shared[(int64_t)t * H4 + o];
        if (shared_scale) ss = shared_scale[t];
        if (sgate) sg = sgate[t];
    }
    if (residual) rs = residual[idx];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += kRows) {
        float4 y[kRows];
        float wj[kRows];
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            if (j0 + i < k) {
                y[i] = pair_values(yp[(int64_t)(j0 + i) * H4]);
                wj[i] = wt[j0 + i];
            }
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
            if (j0 + i < k) {
                acc.x = fmaf(wj[i], y[i].x, acc.x);
                acc.y = fmaf(wj[i], y[i].y, acc.y);
                acc.z = fmaf(wj[i], y[i].z, acc.z);
                acc.w = fmaf(wj[i], y[i].w, acc.w);
            }
        }
    }
    if (y_shared) {
        const float sc = ss * sg;
        acc.x = fmaf(sc, ys.x, acc.x);
        acc.y = fmaf(sc, ys.y, acc.y);
        acc.z = fmaf(sc, ys.z, acc.z);
        acc.w = fmaf(sc, ys.w, acc.w);
    }
    if (residual) {
        acc.x += rs.x;
        acc.y += rs.y;
        acc.z += rs.z;
        acc.w += rs.w;
    }
    out[idx] = acc;
}

// YE: the element type of y_pair (float or uint16_t bf16); YE4 four of them.
template <typename YE, typename YE4>
hipError_t launch_combine_rows(const YE* y_pair, const float* w, const float* y_shared, const float* shared_scale,
                               const float* sgate, const float* residual, int T, int k, int H, float* out,
                               hipStream_t s) {
    const auto al = [](const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; };
    if (H % 4 == 0 && al(y_pair, sizeof(YE4)) && al(out, 16) && (!y_shared || al(y_shared, 16)) &&
        (!residual || al(residual, 16))) {
        const int64_t n = (int64_t)T * (H / 4);
        combine4_kernel<YE4><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            reinterpret_cast<const YE4*>(y_pair), w, reinterpret_cast<const float4*>(y_shared), shared_scale, sgate,
            reinterpret_cast<const float4*>(residual), T, k, H / 4, reinterpret_cast<float4*>(out));
        return hipGetLastError();
    }
    const int64_t n = (int64_t)T * H;
    combine_kernel<YE><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(y_pair, w, y_shared, shared_scale, sgate, residual,
                                                                   T, k, H, out);
    return hipGetLastError();
}

hipError_t launch_combine(const float* y_pair, const float* w, const float* y_shared, const float* shared_scale,
                          const float* sgate, const float* residual, int T, int k, int H, float* out,
                          hipStream_t s) {
    return launch_combine_rows<float, float4>(y_pair, w, y_shared, shared_scale, sgate, residual, T, k, H, out, s);
}

hipError_t launch_combine_bf16(const uint16_t* y_pair, const float* w, const float* y_shared,
                               const float* shared_scale, const float* sgate, const float* residual, int T, int k,
                               int H, float* out, hipStream_t s) {
    return launch_combine_rows<uint16_t, uint2>(y_pair, w, y_shared, shared_scale, sgate, residual, T, k, H, out, s);
}

// One wave per token: s[t] = sigmoid(g . x_t) (shared_gate_wave).
__global__ void __launch_bounds__(256) shared_gate_kernel(const float* __restrict__ x, int T, int H,
                                                          const float* __restrict__ g, float* __restrict__ s) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (blockDim.x / kWave) + wave;
    if (t >= T) return;
    const float v = shared_gate_wave(g, x + (int64_t)t * H, H);
    if (lane == 0) s[t] = v;
}

hipError_t launch_shared_gate(const float* x, int T, int H, const float* g, float* s, hipStream_t st) {
    shared_gate_kernel<<<(unsigned)((T + 3) / 4), 4 * kWave, 0, st>>>(x, T, H, g, s);
    return hipGetLastError();
}

__global__ void __launch_bounds__(256) dequant_q4k_kernel(const uint8_t* __restrict__ blocks,
                                                          int64_t n_slices, float* __restrict__ out) {
    const int64_t sidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (sidx >= n_slices) return;
    const int64_t b = sidx >> 3;
    const int part = (int)(sidx & 7);
    Q4KSlice s;
    q4k_load_slice(blocks + b * 144, part, s);
    const float dlo = s.d * (float)s.sc_lo, mlo = s.dmin * (float)s.m_lo;
    const float dhi = s.d * (float)s.sc_hi, mhi = s.dmin * (float)s.m_hi;
    float* o = out + b * 256;
    const int clo = q4k_slice_col_lo(part), chi = q4k_slice_col_hi(part);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        o[clo + i] = dlo * (float)q4k_slice_qlo(s, i) - mlo;
        o[chi + i] = dhi * (float)q4k_slice_qhi(s, i) - mhi;
    }
}

__global__ void __launch_bounds__(256) dequant_q5k_kernel(const uint8_t* __restrict__ blocks,
                                                          int64_t n_slices, float* __restrict__ out) {
    const int64_t sidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (sidx >= n_slices) return;
    const int64_t b = sidx >> 3;
    const int part = (int)(sidx & 7);
    Q5KSlice s;
    q5k_load_slice(blocks + b * 176, part, s);
    const float dlo = s.s.d * (float)s.s.sc_lo, mlo = s.s.dmin * (float)s.s.m_lo;
    const float dhi = s.s.d * (float)s.s.sc_hi, mhi = s.s.dmin * (float)s.s.m_hi;
    float* o = out + b * 256;
    const int clo = q4k_slice_col_lo(part), chi = q4k_slice_col_hi(part);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        o[clo + i] = dlo * (float)q5k_slice_qlo(s, i) - mlo;
        o[chi + i] = dhi * (float)q5k_slice_qhi(s, i) - mhi;
    }
}

__global__ void __launch_bounds__(256) dequant_q80_kernel(const uint8_t* __restrict__ blocks,
                                                          int64_t n_blocks, float* __restrict__ out) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    Q80Block blk;
    q80_load(blocks + b * 34, blk);
#pragma unroll
    for (int i = 0; i < 32; ++i) out[b * 32 + i] = blk.d * (float)q80_quant(blk, i);
}

// w = fmaf(d, q, m): d*q is exact in fp32 (11 + 5 significant bits), so the
// weight is d*q + m rounded once.
__global__ void __launch_bounds__(256) dequant_q51_kernel(const uint8_t* __restrict__ blocks,
                                                          int64_t n_blocks, float* __restrict__ out) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= n_blocks) return;
    Q51Block blk;
    q51_load(blocks + b * 24, blk);
#pragma unroll
    for (int i = 0; i < 32; ++i) out[b * 32 + i] = fmaf(blk.d, (float)q51_quant(blk, i), blk.m);
}

hipError_t launch_dequant(const void* blocks, int qtype, int64_t n_weights, float* out, hipStream_t s) {
    if (qtype == kQ4_K) {
        const int64_t n = n_weights / 256 * 8;
        dequant_q4k_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const uint8_t*)blocks, n, out);
    } else if (qtype == kQ5_K) {
        const int64_t n = n_weights / 256 * 8;
        dequant_q5k_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const uint8_t*)blocks, n, out);
    } else if (qtype == kQ5_1) {
        const int64_t n = n_weights / 32;
        dequant_q51_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const uint8_t*)blocks, n, out);
    } else {
        const int64_t n = n_weights / 32;
        dequant_q80_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const uint8_t*)blocks, n, out);
    }
    return hipGetLastError();
}

}  // namespace moe
