// route.hip — top-k expert selection from router logits and per-expert bucketing.
//
// The router is a GPU stage on the pages ("Strata - the details", "How it works":
// routers live in VRAM; the decode verify pass routes each token of a window).
// Selection: descending logit, ties to the lower expert index, IEEE comparison
// (-0 and +0 tie).  Weights: softmax over the k selected logits (renormalised),
// or the plain softmax over all E taken at the selected slots.
// Bucketing: pairs p = t*k + j grouped by expert, ascending p within an expert
// (a stable counting sort), so every later stage is deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

// Larger key <=> larger logit.  -0 is folded onto +0 so they tie; NaNs get a
// place in the total order of bit patterns (and raise the error word).
__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key.
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Extraction engine: one wave, the E (<= 64*V) logits of one token, lane l
// owning experts l, l+64, ...  Each lane caches the largest key it still holds
// (best) and the lowest v holding it (bv), so a round is one DPP wave maximum
// of best, a ballot, and a readlane of the winner's bv.  Ties: equal keys
// resolve to the lower expert index (lower v first, since e = lane + 64*v, then
// the lower lane).  Key 0 marks taken or absent experts; real keys are >= 1.
// Rounds return the slots in descending-logit order.  No LDS traffic.
// Up to kSortedV keys per lane, each lane sorts its keys once (descending,
// equal keys by ascending v), so the winner of a round only shifts its list
// by one and its next best is already at the front; with more keys per lane
// the winner clears the taken key and rescans.
constexpr int kSortedV = 8;

template <int V>
struct WaveExtract {
    uint32_t key[V];
    int vi[V];   // sorted lists: the v of key[i]
    uint32_t best;
    int bv;
    // Stable descending sort of the lane's keys: odd-even transposition, whose
    // compare-exchanges touch neighbours only and swap on a strictly larger key,
    // so equal keys keep their ascending-v order.
    __device__ __forceinline__ void sort_keys() {
#pragma unroll
        for (int v = 0; v < V; ++v) vi[v] = v;
#pragma unroll
        for (int ph = 0; ph < V; ++ph) {
#pragma unroll
            for (int i = ph & 1; i + 1 < V; i += 2) {
                const bool sw = key[i + 1] > key[i];
                const uint32_t ka = key[i], kb = key[i + 1];
                const int ia = vi[i], ib = vi[i + 1];
                key[i] = sw ? kb : ka;
                key[i + 1] = sw ? ka : kb;
                vi[i] = sw ? ib : ia;
                vi[i + 1] = sw ? ia : ib;
            }
        }
        best = key[0];
        bv = vi[0];
    }
    __device__ __forceinline__ void refresh() {
        best = key[0];
#pragma unroll
        for (int v = 1; v < V; ++v) best = max(best, key[v]);
        bv = V - 1;
#pragma unroll
        for (int v = V - 2; v >= 0; --v)
            if (key[v] == best) bv = v;
    }
    // Issues the logit loads (clamped index, all in flight at once).
    __device__ __forceinline__ void issue(const float* __restrict__ lg, int E, float (&xv)[V]) {
        const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int e = lane + kWave * v;
            xv[v] = lg[e < E ? e : E - 1];
        }
    }
    // Loads the logits and keys them.  Returns true in lanes that hold a
    // non-finite logit.
    __device__ __forceinline__ bool load(const float* __restrict__ lg, int E, float (&xv)[V]) {
        issue(lg, E, xv);
        return keys(E, xv);
    }
    // Keys the issued logits (waits for them).
    __device__ __forceinline__ bool keys(int E, const float (&xv)[V]) {
        const int lane = threadIdx.x & (kWave - 1);
        bool bad = false;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            // no short-circuit: a branch here lets the compiler move the
            // load of v into it, behind later loads
            const bool in = lane + kWave * v < E;
            const uint32_t kk = max(order_key(xv[v]), 1u);
            bad |= in & !isfinite(xv[v]);
            key[v] = in ? kk : 0u;
        }
        if constexpr (V <= kSortedV) {
            sort_keys();
        } else {
            refresh();
        }
        return bad;
    }
    // The expert of the next slot; M receives its key.  Branch-free except for
    // the rare case of a key held by several lanes.
    __device__ __forceinline__ int next(uint32_t& M) {
        const int lane = threadIdx.x & (kWave - 1);
        M = wave_max_u32(best);
        const bool hold = best == M;
        const uint64_t lanes = __ballot(hold);
        int wl = (int)__builtin_ctzll(lanes);
        int wv = __builtin_amdgcn_readlane(bv, wl);
        // one holder (the usual case): it is the winner, known without the
        // scalar lane search, so the next round's maximum need not wait for it
        bool mine = hold;
        if (__popcll(lanes) != 1) {
            // the lowest (v, lane) among the lanes holding M: a wave minimum of
            // 64*v + lane over those lanes
            const uint32_t cand = hold ? (uint32_t)(kWave * bv + lane) : 0xFFFFFFFFu;
            const uint32_t c = ~wave_max_u32(~cand);
            wl = (int)(c & (kWave - 1));
            wv = (int)(c / kWave);
            mine = lane == wl;
        }
        if constexpr (V <= kSortedV) {
            // the winning lane's taken key is its front one (wv is its bv):
            // shift its list by one
#pragma unroll
            for (int v = 0; v + 1 < V; ++v) {
                key[v] = mine ? key[v + 1] : key[v];
                vi[v] = mine ? vi[v + 1] : vi[v];
            }
            key[V - 1] = mine ? 0u : key[V - 1];
            best = key[0];
            bv = vi[0];
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v) key[v] = (mine && v == wv) ? 0u : key[v];
            refresh();
        }
        return wl + kWave * wv;
    }
    __device__ __forceinline__ int next() {
        uint32_t M;
        return next(M);
    }
};

// One wave selects the top-k of one token's E logits and computes the routing
// weights.  Returns, in lane j < k, the expert of slot j and its weight; other
// lanes get -1 / 0.  Raises kErrLogitNonFinite for a NaN or infinite logit.
template <int V>
__device__ __forceinline__ void wave_topk(const float* __restrict__ lg, int E, int k, bool renorm, int& out_e,
                                          float& out_w) {
    const int lane = threadIdx.x & (kWave - 1);
    WaveExtract<V> ex;
    float xv[V];
    if (__any(ex.load(lg, E, xv))) {
        if (lane == 0) raise_error(kErrLogitNonFinite);
    }
    int my_e = -1;
    float my_l = 0.0f, top = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t M;
        const int e = ex.next(M);
        const float val = key_value(M);
        if (j == 0) top = val;
        if (lane == j) {
            my_e = e;
            my_l = val;
        }
    }
    if (renorm) {
        const float ex2 = (lane < k) ? expf(my_l - top) : 0.0f;
        const float sum = wave_sum(ex2);
        out_w = (lane < k) ? ex2 / sum : 0.0f;
    } else {
        float part = 0.0f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int e = lane + kWave * v;
            if (e < E) part += expf(xv[v] - top);
        }
        const float sum = wave_sum(part);
        out_w = (lane < k) ? expf(my_l - top) / sum : 0.0f;
    }
    out_e = my_e;
}

// Values per lane for E experts (the kernels are instantiated for 4, 8, 16).
inline int topk_vpl(int E) { return E <= 256 ? 4 : (E <= 512 ? 8 : 16); }

// Buckets of up to 64 (token, slot) pairs inside one wave: lane p holds the
// expert e of pair p (p < P).  Computes, with readlane loops (no LDS):
//   below  = pairs with a smaller expert, same_before = earlier pairs of e,
//   first  = p is e's first pair, ubelow = distinct experts smaller than e,
//   n_uniq = distinct experts.
// Then pair p goes to position below + same_before of the pair list and, if
// first, e is active entry ubelow with its pairs starting at below.
__device__ __forceinline__ void wave_buckets(int e, int P, int& below, int& same_before, bool& first, int& ubelow,
                                             int& n_uniq) {
    const int lane = threadIdx.x & (kWave - 1);
    const bool mine = lane < P;
    below = 0;
    same_before = 0;
    for (int q = 0; q < P; ++q) {
        const int eq = __builtin_amdgcn_readlane(e, q);
        below += (eq < e);
        same_before += (q < lane && eq == e);
    }
    first = mine && same_before == 0;
    const uint64_t fm = __ballot(first);
    ubelow = 0;
    for (int q = 0; q < P; ++q) {
        if ((fm >> q) & 1ull) {
            const int eq = __builtin_amdgcn_readlane(e, q);
            ubelow += (eq < e);
        }
    }
    n_uniq = __popcll(fm);
}

// Block-wide exclusive scan of n <= blockDim.x ints held one per thread.
// Returns the exclusive prefix for this thread and writes the total.
__device__ int block_exclusive_scan(int v, int* s_wave, int& total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int w = (lane < nwaves) ? s_wave[lane] : 0;
        int wi = w;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(wi, off, kWave);
            if (lane >= off) wi += o;
        }
        if (lane < nwaves) s_wave[lane] = wi - w;  // exclusive wave offsets
        if (lane == nwaves - 1) s_wave[kWave] = wi;
    }
    __syncthreads();
    const int res = s_wave[wave] + incl - v;
    total = s_wave[kWave];
    __syncthreads();
    return res;
}

// The MFMA GEMMs' tile list from the bucket counts: expert e's ceil(count/mt)
// tiles in expert order, then the shared expert's tiles over all T tokens.
// Every thread of the workgroup calls it (blockDim.x >= E); thread e < E passes
// count[e], the others 0.  s_start holds E ints of LDS.  Each thread writes
// list entries j = tid, tid + blockDim.x, ..., finding the expert of entry j
// as the last e whose first entry is <= j (experts without tiles share the
// next expert's first entry, so the last such e is the one with tiles).
// Counts past npairs cannot come from a routing pass: they raise
// kErrPairRange, and the list never grows past max_t.
__device__ void write_tile_list(int c, int npairs, int E, const TileList& tl, int* s_wave, int* s_start) {
    const int tid = threadIdx.x;
    if (c < 0 || c > npairs) {
        raise_error(kErrPairRange);
        c = 0;
    }
    const int nt = (c + tl.mt - 1) / tl.mt;
    int total = 0;
    const int start = block_exclusive_scan(nt, s_wave, total);
    if (tid < E) s_start[tid] = start;
    __syncthreads();
    const int ns = tl.has_shared ? (tl.T + tl.mt - 1) / tl.mt : 0;
    const int n = min(total + ns, tl.max_t);
    for (int j = tid; j < n; j += blockDim.x) {
        int e = E, m0 = (j - total) * tl.mt;
        if (j < total) {
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_start[mid] <= j)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            e = lo;
            m0 = (j - s_start[lo]) * tl.mt;
        }
        tl.tile_e[j] = e;
        tl.tile_m0[j] = m0;
    }
    if (tid == 0) {
        if (total + ns > tl.max_t) raise_error(kErrPairRange);
        *tl.n_tiles = n;
    }
}

// ---------------------------------------------------------------------------
// Small batches (T*k <= kSmallPairs): top-k and bucketing in one workgroup.
// ---------------------------------------------------------------------------
template <int V>
__global__ void __launch_bounds__(1024) route_small_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int renorm,
                                                           RoutingPtrs r) {
    __shared__ int s_idx[kSmallPairs];
    __shared__ int s_count[1024];
    __shared__ int s_off[1024];
    __shared__ int s_wave[kWave + 1];
    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid & (kWave - 1);
    const int nwaves = blockDim.x / kWave;
    const int P = T * k;
    for (int e = tid; e < E; e += blockDim.x) s_count[e] = 0;
    for (int t = wave; t < T; t += nwaves) {
        int e;
        float w;
        wave_topk<V>(logits + (int64_t)t * E, E, k, renorm != 0, e, w);
        if (lane < k) {
            r.idx[t * k + lane] = e;
            r.w[t * k + lane] = w;
            s_idx[t * k + lane] = e;
        }
    }
    __syncthreads();
    for (int p = tid; p < P; p += blockDim.x) atomicAdd(&s_count[s_idx[p]], 1);
    __syncthreads();
    // offsets and the active list: E <= 1024 = blockDim.x
    int total_pairs, n_act;
    const int c = (tid < E) ? s_count[tid] : 0;
    const int off = block_exclusive_scan(c, s_wave, total_pairs);
    const int apos = block_exclusive_scan((tid < E && c > 0) ? 1 : 0, s_wave, n_act);
    if (tid < E) {
        s_off[tid] = off;
        r.count[tid] = c;
        r.offset[tid] = off;
        if (c > 0) r.active[apos] = tid;
    }
    if (tid == 0) {
        r.offset[E] = total_pairs;
        *r.n_active = n_act;
    }
    __syncthreads();
    // stable placement: rank = earlier pairs of the same expert
    for (int p = tid; p < P; p += blockDim.x) {
        const int e = s_idx[p];
        int rank = 0;
        for (int q = 0; q < p; ++q) rank += (s_idx[q] == e);
        r.pair[s_off[e] + rank] = p;
    }
}

// ---------------------------------------------------------------------------
// Large batches: one wave per token, then a tiled stable counting sort.
// ---------------------------------------------------------------------------
template <int V>
__device__ void route_token_wave(int t, const float* __restrict__ logits, int E, int k, int renorm, int32_t* idx,
                                 float* w) {
    const int lane = threadIdx.x & (kWave - 1);
    int e;
    float wt;
    wave_topk<V>(logits + (int64_t)t * E, E, k, renorm != 0, e, wt);
    if (lane < k) {
        idx[(int64_t)t * k + lane] = e;
        w[(int64_t)t * k + lane] = wt;
    }
}

template <int V>
__global__ void __launch_bounds__(256) route_tokens_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int renorm, int32_t* idx,
                                                           float* w) {
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    route_token_wave<V>(t, logits, E, k, renorm, idx, w);
}

// A layer call's prompt chunk: the per-token top-k and the activation
// quantisation read and write disjoint arrays, so one launch carries both.
// Workgroups below nr route four tokens each; the rest quantise x.
template <int V>
__global__ void __launch_bounds__(256) route_quant_kernel(const float* __restrict__ logits, int T, int E,
                                                          int k, int renorm, int32_t* idx, float* w, int nr,
                                                          const float* __restrict__ x, int64_t n_blocks,
                                                          int8_t* __restrict__ xq, float* __restrict__ xd,
                                                          int16_t* __restrict__ xs) {
    const int wave = threadIdx.x / kWave;
    if ((int)blockIdx.x < nr) {
        const int t = blockIdx.x * (blockDim.x / kWave) + wave;
        if (t < T) route_token_wave<V>(t, logits, E, k, renorm, idx, w);
        return;
    }
    quantize_act_wave((int64_t)(blockIdx.x - nr) * (blockDim.x / kWave) + wave, x, n_blocks, xq, xd, xs);
}

// Per tile of kTilePairs pairs: histogram over experts and each pair's rank
// among the earlier pairs of its expert inside the tile.
__global__ void __launch_bounds__(kTilePairs) bucket_tile_kernel(const int32_t* __restrict__ idx, int P,
                                                                 int E, int32_t* tile_hist,
                                                                 int32_t* rank) {
    __shared__ int s_e[kTilePairs];
    __shared__ int s_h[1024];
    const int tile = blockIdx.x, tid = threadIdx.x;
    const int p = tile * kTilePairs + tid;
    for (int e = tid; e < E; e += blockDim.x) s_h[e] = 0;
    const int e = (p < P) ? idx[p] : -1;
    s_e[tid] = e;
    __syncthreads();
    if (p < P) atomicAdd(&s_h[e], 1);
    int rk = 0;
    for (int q = 0; q < tid; ++q) rk += (s_e[q] == e);
    if (p < P) rank[p] = rk;
    __syncthreads();
    for (int x = tid; x < E; x += blockDim.x) tile_hist[(int64_t)tile * E + x] = s_h[x];
}

// One workgroup: per-expert totals, offsets, tile bases and the active list.
// G = blockDim/E threads share an expert (thread t: expert t % E, chunk t / E
// of the tiles): each sums its chunk, the chunk sums meet in LDS, and each
// then writes its chunk's exclusive prefixes from the sum of the chunks
// before it; a chunk's values stay in registers between the two passes when
// it holds at most kB tiles (one round trip each way instead of one per 16
// tiles).  With tl.mt > 0 the totals also give the MFMA tile list.
__global__ void __launch_bounds__(1024) bucket_scan_kernel(int n_tiles, int E, int P,
                                                           int32_t* tile_hist, RoutingPtrs r, TileList tl) {
    __shared__ int s_wave[kWave + 1];
    __shared__ int s_part[1024];
    constexpr int kB = 32;
    const int t = threadIdx.x;
    const int G = max(1, (int)blockDim.x / E);
    const int q = t / E, e = t - q * E;
    const bool act = q < G;
    const int chunk = (n_tiles + G - 1) / G;
    const int lo = q * chunk, hi = min(n_tiles, lo + chunk);
    int hv[kB];
    int sum = 0;
    if (act) {
        for (int t0 = lo; t0 < hi; t0 += kB) {
#pragma unroll
            for (int i = 0; i < kB; ++i) hv[i] = t0 + i < hi ? tile_hist[(int64_t)(t0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kB; ++i) sum += hv[i];
        }
    }
    s_part[t] = act ? sum : 0;
    __syncthreads();
    int base = 0, run = 0;
    if (act) {
        for (int qq = 0; qq < G; ++qq) {
            const int v = s_part[qq * E + e];
            base += qq < q ? v : 0;
            run += v;
        }
        int c = base;
        for (int t0 = lo; t0 < hi; t0 += kB) {
            if (hi - lo > kB) {   // more than one batch: the registers hold the last one only
#pragma unroll
                for (int i = 0; i < kB; ++i) hv[i] = t0 + i < hi ? tile_hist[(int64_t)(t0 + i) * E + e] : 0;
            }
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                if (t0 + i < hi) {
                    tile_hist[(int64_t)(t0 + i) * E + e] = c;
                    c += hv[i];
                }
            }
        }
    }
    // threads t < E (chunk 0) hold their expert's total in run
    int total, n_act;
    const int mine = t < E ? run : 0;
    const int off = block_exclusive_scan(mine, s_wave, total);
    const int apos = block_exclusive_scan((t < E && run > 0) ? 1 : 0, s_wave, n_act);
    if (t < E) {
        r.count[t] = run;
        r.offset[t] = off;
        if (run > 0) r.active[apos] = t;
    }
    if (t == 0) {
        r.offset[E] = total;
        *r.n_active = n_act;
    }
    if (tl.mt > 0) write_tile_list(mine, P, E, tl, s_wave, s_part);   // s_part is free again
}

// pair[offset[e] + (pairs of e in earlier tiles) + rank of p in its tile] = p
__global__ void __launch_bounds__(256) bucket_scatter_kernel(const int32_t* __restrict__ idx, int P,
                                                             int E, const int32_t* __restrict__ tile_base,
                                                             const int32_t* __restrict__ offset,
                                                             const int32_t* __restrict__ rank,
                                                             int32_t* pair) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= P) return;
    const int tile = p / kTilePairs;
    const int e = idx[p];
    pair[offset[e] + tile_base[(int64_t)tile * E + e] + rank[p]] = p;
}

hipError_t launch_route(const float* logits, int T, int E, int k, int renorm, const RoutingPtrs& r,
                        void* ws, hipStream_t s, RouteExtras* ex) {
    const int P = T * k;
    const int vpl = topk_vpl(E);
    if (ex) ex->tiles_written = false;
    if (P <= kSmallPairs) {
        if (vpl == 4)
            route_small_kernel<4><<<1, 1024, 0, s>>>(logits, T, E, k, renorm, r);
        else if (vpl == 8)
            route_small_kernel<8><<<1, 1024, 0, s>>>(logits, T, E, k, renorm, r);
        else
            route_small_kernel<16><<<1, 1024, 0, s>>>(logits, T, E, k, renorm, r);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || !ex) return e;
        return launch_quantize_act(ex->x, T, ex->H, ex->xq, ex->xd, s, ex->xs);
    }
    const int n_tiles = (P + kTilePairs - 1) / kTilePairs;
    int32_t* tile_hist = (int32_t*)ws;
    int32_t* rank = tile_hist + (size_t)n_tiles * E;
    const int nr = (T + 3) / 4;
    if (ex) {
        const int64_t n_blocks = (int64_t)T * (ex->H / 256);
        const unsigned grid = (unsigned)(nr + (quantize_act_waves(T, ex->H) + 3) / 4);
        if (vpl == 4)
            route_quant_kernel<4><<<grid, 256, 0, s>>>(logits, T, E, k, renorm, r.idx, r.w, nr, ex->x, n_blocks,
                                                       ex->xq, ex->xd, ex->xs);
        else if (vpl == 8)
            route_quant_kernel<8><<<grid, 256, 0, s>>>(logits, T, E, k, renorm, r.idx, r.w, nr, ex->x, n_blocks,
                                                       ex->xq, ex->xd, ex->xs);
        else
            route_quant_kernel<16><<<grid, 256, 0, s>>>(logits, T, E, k, renorm, r.idx, r.w, nr, ex->x, n_blocks,
                                                        ex->xq, ex->xd, ex->xs);
    } else if (vpl == 4) {
        route_tokens_kernel<4><<<nr, 256, 0, s>>>(logits, T, E, k, renorm, r.idx, r.w);
    } else if (vpl == 8) {
        route_tokens_kernel<8><<<nr, 256, 0, s>>>(logits, T, E, k, renorm, r.idx, r.w);
    } else {
        route_tokens_kernel<16><<<nr, 256, 0, s>>>(logits, T, E, k, renorm, r.idx, r.w);
    }
    bucket_tile_kernel<<<n_tiles, kTilePairs, 0, s>>>(r.idx, P, E, tile_hist, rank);
    TileList tl{};
    if (ex && ex->tiles.mt > 0) tl = ex->tiles;
    bucket_scan_kernel<<<1, 1024, 0, s>>>(n_tiles, E, P, tile_hist, r, tl);
    bucket_scatter_kernel<<<(P + 255) / 256, 256, 0, s>>>(r.idx, P, E, tile_hist, r.offset, rank, r.pair);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && ex) ex->tiles_written = tl.mt > 0;
    return e;
}

size_t route_workspace_bytes(int T, int E, int k) {
    const int64_t P = (int64_t)T * k;
    if (P <= kSmallPairs) return 0;
    const int64_t n_tiles = (P + kTilePairs - 1) / kTilePairs;
    return (size_t)(n_tiles * E + P) * sizeof(int32_t);
}

}  // namespace moe
