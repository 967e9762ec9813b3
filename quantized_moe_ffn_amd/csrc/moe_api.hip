// moe_api.hip — the C ABI of libmoe (declared in include/moe.h): argument
// validation, workspace layout and dispatch to the kernels.  Nothing here
// allocates, frees or synchronises (except moe_check_device_errors).
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"

// Workspace of moe_forward_noalloc: a device array of the library, one copy per
// GPU, held until the process ends.  Host code never passes its name to a
// kernel or a copy (on the host the name is only a stand-in for the symbol):
// the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

moe_status ok() {
    g_last_error[0] = '\0';
    return MOE_OK;
}

moe_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MOE_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// Reads and clears the current device's error word (the stream already synchronised).
// Returns MOE_ERR_DEVICE, with a message that starts with `what`, if it was set.
moe_status take_error_word(const char* what) {
    unsigned int word = 0, zero = 0;
    hipError_t e = hipMemcpyFromSymbol(&word, HIP_SYMBOL(moe::g_moe_err), sizeof(word), 0, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return from_hip(e, "read the device error word");
    if (word == 0) return ok();
    e = hipMemcpyToSymbol(HIP_SYMBOL(moe::g_moe_err), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
    if (e != hipSuccess) return from_hip(e, "clear the device error word");
    return fail(MOE_ERR_DEVICE, "%sdevice error word 0x%x:%s%s%s%s", what, word,
                (word & moe::kErrExpertRange) ? " expert id out of range;" : "",
                (word & moe::kErrPairRange) ? " bucket offsets or pair ids out of range;" : "",
                (word & moe::kErrLogitNonFinite) ? " non-finite router logit;" : "",
                (word & moe::kErrActNonFinite) ? " non-finite activation;" : "");
}

// MOE_SYNC_DEBUG=1 in the environment (read at every call): each call that
// enqueued work synchronises its stream and checks the device error word
// before it returns, so an asynchronous fault or a kernel-detected error is
// reported by the call that caused it.  Skipped while the stream is being
// captured into a graph (a synchronisation would end the capture).
moe_status finish(moe_status st, hipStream_t stream, const char* what) {
    if (st != MOE_OK) return st;
    const char* v = getenv("MOE_SYNC_DEBUG");
    if (!v || strcmp(v, "1") != 0) return st;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return from_hip(e, "MOE_SYNC_DEBUG: query stream capture");
    if (cs != hipStreamCaptureStatusNone) return st;
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "%s (MOE_SYNC_DEBUG): stream synchronize: HIP error %d (%s)", what,
                                     (int)e, hipGetErrorString(e));
    char prefix[160];
    snprintf(prefix, sizeof(prefix), "%s (MOE_SYNC_DEBUG): ", what);
    return take_error_word(prefix);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Device address of `scratch` on the device of `stream`, looked up once per
// device with that device current, and kept.
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kScratchDevices];
std::mutex g_scratch_mu;

moe_status scratch_address(hipStream_t stream, void** out) {
    int dev = 0, cur = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return from_hip(e, "moe_forward_noalloc: device of the stream");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(MOE_ERR_UNSUPPORTED, "moe_forward_noalloc: device %d (supported: 0..%d)", dev, kScratchDevices - 1);
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_acquire);
        if (!p) {
            if ((e = hipGetDevice(&cur)) != hipSuccess) return from_hip(e, "moe_forward_noalloc: current device");
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
                return from_hip(e, "moe_forward_noalloc: make the stream's device current");
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
            if (e != hipSuccess) return from_hip(e, "moe_forward_noalloc: hipGetSymbolAddress(scratch)");
            if (e2 != hipSuccess) return from_hip(e2, "moe_forward_noalloc: restore the current device");
            if (!p || ((uintptr_t)p % 256) != 0)
                return fail(MOE_ERR_DEVICE, "moe_forward_noalloc: scratch address %p is not 256-byte aligned", p);
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return ok();
}

bool known_qtype(int qt) { return qt == MOE_Q4_K || qt == MOE_Q5_K || qt == MOE_Q8_0 || qt == MOE_Q5_1; }
int blk_weights(int qt) { return (qt == MOE_Q8_0 || qt == MOE_Q5_1) ? 32 : 256; }
int blk_bytes(int qt) { return qt == MOE_Q4_K ? 144 : (qt == MOE_Q5_K ? 176 : (qt == MOE_Q5_1 ? 24 : 34)); }
// Q4_K, Q5_K blocks are 16-byte multiples; Q5_1 blocks (24 bytes) are read as 8-byte words
size_t blk_align(int qt) { return qt == MOE_Q8_0 ? 2 : (qt == MOE_Q5_1 ? 8 : 16); }

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kMaxDim = 3584;   // H and I: LDS staging of kTokChunk rows of fp32 (< 64 KB)
constexpr int kAutoDecodeMaxT = 8;   // AUTO: fp-activation path up to this many tokens

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Validates one projection; rows x cols weights per expert, n_experts experts.
moe_status check_qmatrix(const moe_qmatrix& m, const char* name, int rows, int cols, int n_experts) {
    if (!m.data) return fail(MOE_ERR_INVALID_ARGUMENT, "%s.data is NULL", name);
    if (!known_qtype(m.qtype))
        return fail(MOE_ERR_UNSUPPORTED, "%s.qtype = %d: supported are Q4_K (%d), Q5_K (%d), Q8_0 (%d) and Q5_1 (%d)",
                    name, m.qtype, MOE_Q4_K, MOE_Q5_K, MOE_Q8_0, MOE_Q5_1);
    if (m.rows != rows || m.cols != cols)
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s is %d x %d, expected %d x %d", name, m.rows, m.cols,
                    rows, cols);
    if (cols % blk_weights(m.qtype) != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s.cols = %d is not a multiple of the block size %d", name,
                    cols, blk_weights(m.qtype));
    const int64_t rb = (int64_t)cols / blk_weights(m.qtype) * blk_bytes(m.qtype);
    if (m.row_bytes != rb)
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s.row_bytes = %lld, expected %lld", name,
                    (long long)m.row_bytes, (long long)rb);
    if (n_experts > 1 && m.expert_bytes < (int64_t)rows * rb)
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s.expert_bytes = %lld < rows*row_bytes = %lld", name,
                    (long long)m.expert_bytes, (long long)rows * rb);
    const size_t al = blk_align(m.qtype);
    if (!aligned(m.data, al) || (m.expert_bytes % (int64_t)al) != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s: data and expert_bytes must be %zu-byte aligned", name, al);
    return MOE_OK;
}

moe::QMat to_qmat(const moe_qmatrix& m) {
    return moe::QMat{(const uint8_t*)m.data, m.row_bytes, m.expert_bytes, m.qtype};
}

struct FfnWorkspace {
    size_t h, hq, hd, xs, hs, tiles, total;
    bool mfma;
    bool grouped;   // decode path, expert-grouped kernels: tiles holds their tile list
};

// The int8 path runs as grouped int8 MFMA GEMMs for k-quant experts (Q4_K or
// Q5_K gate/up, Q4_K or Q5_K down); the shared expert's formats equal the
// routed ones (validate_layer).
bool int8_uses_mfma(const moe_layer* L) {
    return moe::mfma_path_supported(L->hidden, L->inter, L->gate.qtype, L->up.qtype, L->down.qtype);
}

FfnWorkspace ffn_ws_layout(const moe_layer* L, int T, int k, uint32_t path) {
    const size_t rows = (size_t)T * k + (L->has_shared ? T : 0);
    FfnWorkspace w{};
    w.mfma = path == MOE_FFN_INT8 && int8_uses_mfma(L) && moe::mfma_rows_fit(T, k, L->hidden, L->inter);
    w.grouped = path == MOE_FFN_DECODE && moe::dec_grouped_supported(T, k, L->hidden, L->inter, L->gate.qtype,
                                                                      L->up.qtype, L->down.qtype);
    size_t off = 0;
    w.h = 0;
    if (!w.mfma) off += align_up(rows * L->inter * sizeof(float), 256);
    if (w.grouped) {
        w.tiles = off;
        off += align_up(moe::dec_grouped_tiles_bytes(T, k, L->n_experts, L->has_shared ? 1 : 0), 256);
    }
    w.hq = off;
    w.hd = off;
    if (path == MOE_FFN_INT8) {
        w.hq = off;
        off += align_up(rows * L->inter, 256);
        w.hd = off;
        off += align_up(rows * (L->inter / 256) * sizeof(float), 256);
        if (w.mfma) {
            w.xs = off;
            off += align_up((size_t)T * (L->hidden / 32) * 2, 256);
            w.hs = off;
            off += align_up(rows * (L->inter / 32) * 2, 256);
            w.tiles = off;
            off += align_up(moe::mfma_tiles_bytes(T, k, L->n_experts, L->has_shared, L->hidden, L->inter), 256);
        }
    }
    w.total = off;
    return w;
}

void set_ffn_ws(moe::FfnArgs& a, char* base, const FfnWorkspace& w) {
    a.h = (float*)(base + w.h);
    a.hq = (int8_t*)(base + w.hq);
    a.hd = (float*)(base + w.hd);
    a.xs = w.mfma ? (int16_t*)(base + w.xs) : nullptr;
    a.hs = w.mfma ? (int16_t*)(base + w.hs) : nullptr;
    a.tiles = (w.mfma || w.grouped) ? (int32_t*)(base + w.tiles) : nullptr;
}

struct ForwardWorkspace {
    size_t route, ffn, xq, xd, tab, sg, yp, total;
    bool yp_bf16;   // yp holds bf16 per-pair outputs (else fp32); used with MOE_FFN_PAIR_BF16
};

// ffn_flags of the layer calls: a path selector, optionally with MOE_FFN_PAIR_BF16.
bool split_ffn_flags(uint32_t flags, uint32_t& sel, bool& pair_ws) {
    pair_ws = (flags & MOE_FFN_PAIR_BF16) != 0;
    sel = flags & ~(uint32_t)MOE_FFN_PAIR_BF16;
    return sel == MOE_FFN_AUTO || sel == MOE_FFN_DECODE || sel == MOE_FFN_INT8;
}

ForwardWorkspace forward_ws_layout(const moe_layer* L, int T, int k, uint32_t path, bool pair_ws) {
    ForwardWorkspace w{};
    size_t off = 0;
    w.route = off;
    off += align_up(moe::route_workspace_bytes(T, L->n_experts, k), 256);
    w.ffn = off;
    off += align_up(ffn_ws_layout(L, T, k, path).total, 256);
    w.xq = off;
    off += align_up((size_t)T * L->hidden, 256);
    w.xd = off;
    off += align_up((size_t)T * (L->hidden / 256) * sizeof(float), 256);
    w.tab = off;
    off += moe::kDecRouteTabBytes;
    w.sg = off;   // shared-expert gate values of the separate stages
    off += align_up((size_t)T * sizeof(float), 256);
    w.yp = off;   // the per-pair outputs when the caller does not take them
    w.yp_bf16 = ffn_ws_layout(L, T, k, path).mfma;
    if (pair_ws) off += align_up((size_t)T * k * L->hidden * (w.yp_bf16 ? 2 : 4), 256);
    w.total = off;
    return w;
}

uint32_t resolve_path(uint32_t flags, int T) {
    if (flags == MOE_FFN_AUTO) return T <= kAutoDecodeMaxT ? MOE_FFN_DECODE : MOE_FFN_INT8;
    return flags;
}

moe_status validate_layer(const moe_layer* L, int32_t T, int32_t k, const float* y_shared) {
    if (!L) return fail(MOE_ERR_INVALID_ARGUMENT, "layer descriptor is NULL");
    const int E = L->n_experts, H = L->hidden, I = L->inter;
    if (E < 1 || E > kMaxExperts) return fail(MOE_ERR_INVALID_ARGUMENT, "n_experts = %d: need 1..%d", E, kMaxExperts);
    if (H < 256 || H % 256 || I < 256 || I % 256)
        return fail(MOE_ERR_INVALID_ARGUMENT, "hidden = %d, inter = %d: both must be positive multiples of 256", H, I);
    if (H > kMaxDim || I > kMaxDim)
        return fail(MOE_ERR_UNSUPPORTED, "hidden = %d, inter = %d: the library supports up to %d", H, I, kMaxDim);
    if (T < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d: need at least one token", T);
    if (k < 1 || k > E || k > kMaxTopK)
        return fail(MOE_ERR_INVALID_ARGUMENT, "k = %d: need 1 <= k <= min(E = %d, %d)", k, E, kMaxTopK);
    if ((int64_t)T * k > (int64_t)1 << 30)
        return fail(MOE_ERR_INVALID_ARGUMENT, "T*k = %lld is too large", (long long)T * k);
    moe_status st;
    if ((st = check_qmatrix(L->gate, "gate", I, H, E)) != MOE_OK) return st;
    if ((st = check_qmatrix(L->up, "up", I, H, E)) != MOE_OK) return st;
    if ((st = check_qmatrix(L->down, "down", H, I, E)) != MOE_OK) return st;
    if (L->has_shared) {
        if ((st = check_qmatrix(L->sh_gate, "sh_gate", I, H, 1)) != MOE_OK) return st;
        if ((st = check_qmatrix(L->sh_up, "sh_up", I, H, 1)) != MOE_OK) return st;
        if ((st = check_qmatrix(L->sh_down, "sh_down", H, I, 1)) != MOE_OK) return st;
        if (L->sh_gate.qtype != L->gate.qtype || L->sh_up.qtype != L->up.qtype || L->sh_down.qtype != L->down.qtype)
            return fail(MOE_ERR_UNSUPPORTED, "the shared expert must use the routed experts' formats "
                        "(gate %d/%d, up %d/%d, down %d/%d)", L->sh_gate.qtype, L->gate.qtype,
                        L->sh_up.qtype, L->up.qtype, L->sh_down.qtype, L->down.qtype);
        if (!y_shared) return fail(MOE_ERR_INVALID_ARGUMENT, "layer has a shared expert but y_shared is NULL");
    }
    return MOE_OK;
}

void fill_ffn_args(moe::FfnArgs& a, const moe_layer* L, int T, int k) {
    a.gate = to_qmat(L->gate);
    a.up = to_qmat(L->up);
    a.down = to_qmat(L->down);
    a.has_shared = L->has_shared ? 1 : 0;
    if (a.has_shared) {
        a.sgate = to_qmat(L->sh_gate);
        a.sup = to_qmat(L->sh_up);
        a.sdown = to_qmat(L->sh_down);
    }
    a.H = L->hidden;
    a.I = L->inter;
    a.T = T;
    a.k = k;
    a.E = L->n_experts;
    a.n_slots = (int)((int64_t)T * k < a.E ? (int64_t)T * k : a.E);
}

bool aligned16_bank(const moe_qmatrix& m) { return aligned(m.data, 16) && (m.expert_bytes % 16) == 0; }

// The two-kernel decode path applies: shapes it is built for, 16-byte aligned
// banks and activations, and the decode arithmetic selected.
bool use_fused_decode(const moe_layer* L, int T, int k, const float* x, uint32_t path) {
    if (path != MOE_FFN_DECODE || !aligned(x, 16)) return false;
    if (!moe::dec_fused_supported(T, k, L->hidden, L->inter, L->gate.qtype, L->up.qtype, L->down.qtype)) return false;
    if (!aligned16_bank(L->gate) || !aligned16_bank(L->up) || !aligned16_bank(L->down)) return false;
    if (L->has_shared && (!aligned16_bank(L->sh_gate) || !aligned16_bank(L->sh_up) || !aligned16_bank(L->sh_down)))
        return false;
    return true;
}

// The router stage of moe_forward_router: the router matrix.
struct RouterStage {
    const float* w;
};

// moe_forward_ep, and with rt the layer from x and the router matrix (logits
// are then written by moe_router_logits' kernel ahead of the layer).
moe_status forward_impl(const moe_layer* L, const float* logits, const float* x, int32_t T, int32_t k,
                        uint32_t route_flags, uint32_t ffn_flags, const moe_routing* r, float* y_pair,
                        float* y_shared, const float* shared_scale, const moe_epilogue* ep, float* out,
                        void* workspace, size_t ws_bytes, hipStream_t stream, const RouterStage* rt) {
    moe_status st = validate_layer(L, T, k, y_shared);
    if (st != MOE_OK) return st;
    const float* sgate_w = ep ? ep->shared_gate : nullptr;
    const float* residual = ep ? ep->residual : nullptr;
    if (sgate_w && !L->has_shared)
        return fail(MOE_ERR_INVALID_ARGUMENT, "epilogue shared_gate given for a layer without a shared expert");
    if (shared_scale && !L->has_shared)
        return fail(MOE_ERR_INVALID_ARGUMENT, "shared_scale given for a layer without a shared expert");
    if ((sgate_w && !aligned(sgate_w, 16)) || (residual && !aligned(residual, 4)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "epilogue: shared_gate must be 16-byte aligned, residual 4-byte aligned");
    if (residual && (residual == y_pair || residual == y_shared))
        return fail(MOE_ERR_INVALID_ARGUMENT, "epilogue: residual must not alias y_pair or y_shared");
    uint32_t sel = 0;
    bool pair_ws = false;
    if (!split_ffn_flags(ffn_flags, sel, pair_ws))
        return fail(MOE_ERR_INVALID_ARGUMENT,
                    "ffn_flags = 0x%x: use MOE_FFN_AUTO, MOE_FFN_DECODE or MOE_FFN_INT8, optionally with "
                    "MOE_FFN_PAIR_BF16",
                    ffn_flags);
    if (!logits || !x || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "logits, x or out is NULL");
    if (!y_pair && !pair_ws) return fail(MOE_ERR_INVALID_ARGUMENT, "y_pair is NULL (allowed with MOE_FFN_PAIR_BF16)");
    if (pair_ws) y_pair = nullptr;   // not touched
    if (!aligned(logits, 4) || !aligned(x, 16) || !aligned(out, 4) || !aligned(y_pair, 4) ||
        (y_shared && !aligned(y_shared, 4)) || (shared_scale && !aligned(shared_scale, 4)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "x must be 16-byte aligned, the other fp32 arrays 4-byte aligned");
    if (route_flags & ~(uint32_t)MOE_ROUTE_RENORM)
        return fail(MOE_ERR_INVALID_ARGUMENT, "route_flags = 0x%x: only MOE_ROUTE_RENORM is defined", route_flags);
    if (!r || !r->idx || !r->w || !r->count || !r->offset || !r->pair || !r->active || !r->n_active)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_routing or one of its arrays is NULL");
    const uint32_t path = resolve_path(sel, T);
    const ForwardWorkspace wl = forward_ws_layout(L, T, k, path, pair_ws);
    if (!workspace || ws_bytes < wl.total)
        return fail(MOE_ERR_WORKSPACE, "forward workspace: %zu bytes given, %zu needed", ws_bytes, wl.total);
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    char* ws = (char*)workspace;
    moe::RoutingPtrs rp{r->idx, r->w, r->count, r->offset, r->pair, r->active, r->n_active};
    const int renorm = (route_flags & MOE_ROUTE_RENORM) ? 1 : 0;
    if (rt) {
        const hipError_t e0 = moe::launch_router(x, T, L->hidden, rt->w, L->n_experts, (float*)logits, stream);
        if (e0 != hipSuccess) return from_hip(e0, "moe_forward_router: router launch");
    }

    if (use_fused_decode(L, T, k, x, path)) {
        moe::DecArgs d{};
        d.logits = logits;
        d.x = x;
        d.gate = to_qmat(L->gate);
        d.up = to_qmat(L->up);
        d.down = to_qmat(L->down);
        d.has_shared = L->has_shared ? 1 : 0;
        if (d.has_shared) {
            d.sgate = to_qmat(L->sh_gate);
            d.sup = to_qmat(L->sh_up);
            d.sdown = to_qmat(L->sh_down);
        }
        d.T = T;
        d.E = L->n_experts;
        d.k = k;
        d.H = L->hidden;
        d.I = L->inter;
        d.renorm = renorm;
        d.r = rp;
        d.h = (float*)(ws + wl.ffn);
        d.y_pair = y_pair;
        d.y_shared = y_shared;
        d.shared_scale = shared_scale;
        d.sgate_w = sgate_w;
        d.residual = residual;
        d.out = out;
        d.route_tab = (int*)(ws + wl.tab);
        return finish(from_hip(moe::launch_dec_fused(d, stream), "moe_forward (decode) launch"), stream,
                      rt ? "moe_forward_router" : "moe_forward");
    }

    moe::FfnArgs a{};
    fill_ffn_args(a, L, T, k);
    a.count = r->count;
    a.offset = r->offset;
    a.pair = r->pair;
    a.active = r->active;
    a.n_active = r->n_active;
    a.x = x;
    a.xq = (int8_t*)(ws + wl.xq);
    a.xd = (float*)(ws + wl.xd);
    set_ffn_ws(a, ws + wl.ffn, ffn_ws_layout(L, T, k, path));
    // the per-pair outputs: the caller's y_pair, or with MOE_FFN_PAIR_BF16 the
    // workspace (bf16 on the MFMA GEMMs, fp32 on the other stages)
    float* yp32 = y_pair;
    uint16_t* yp16 = nullptr;
    if (pair_ws) {
        if (wl.yp_bf16)
            yp16 = (uint16_t*)(ws + wl.yp);
        else
            yp32 = (float*)(ws + wl.yp);
    }
    a.y_pair = yp32;
    a.y_pair_bf16 = yp16;
    a.y_shared = y_shared;
    hipError_t e;
    if (path == MOE_FFN_INT8) {
        // The routing launches also quantise x (with the MFMA GEMMs' per-32 code
        // sums when a.xs is set) and, on large batches, write the tile list.
        moe::RouteExtras ex{};
        ex.x = x;
        ex.H = L->hidden;
        ex.xq = (int8_t*)a.xq;
        ex.xd = (float*)a.xd;
        ex.xs = a.xs;
        ex.tiles = moe::int8_tile_list(a);
        e = moe::launch_route(logits, T, L->n_experts, k, renorm, rp, ws + wl.route, stream, &ex);
        if (e != hipSuccess) return from_hip(e, "moe_forward: routing and quantisation launch");
        a.xs_ready = a.xs ? 1 : 0;
        a.tiles_ready = ex.tiles_written ? 1 : 0;
        e = moe::launch_ffn_int8(a, stream);
    } else {
        e = moe::launch_route(logits, T, L->n_experts, k, renorm, rp, ws + wl.route, stream);
        if (e != hipSuccess) return from_hip(e, "moe_forward: routing launch");
        e = moe::launch_ffn_decode(a, stream);
    }
    if (e != hipSuccess) return from_hip(e, "moe_forward: expert FFN launch");
    float* sg = nullptr;
    if (sgate_w) {
        sg = (float*)(ws + wl.sg);
        e = moe::launch_shared_gate(x, T, L->hidden, sgate_w, sg, stream);
        if (e != hipSuccess) return from_hip(e, "moe_forward: shared-expert gate launch");
    }
    const float* ysh = L->has_shared ? y_shared : nullptr;
    e = yp16 ? moe::launch_combine_bf16(yp16, r->w, ysh, shared_scale, sg, residual, T, k, L->hidden, out, stream)
             : moe::launch_combine(yp32, r->w, ysh, shared_scale, sg, residual, T, k, L->hidden, out, stream);
    return finish(from_hip(e, "moe_forward: combine launch"), stream, "moe_forward");
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_last_error; }

size_t moe_route_workspace_bytes(int32_t T, int32_t E, int32_t k) {
    if (T < 1 || E < 1 || k < 1) return 0;
    return moe::route_workspace_bytes(T, E, k);
}

moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, uint32_t flags,
                          const moe_routing* r, void* workspace, size_t ws_bytes, hipStream_t stream) {
    if (!logits) return fail(MOE_ERR_INVALID_ARGUMENT, "logits is NULL");
    if (!aligned(logits, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "logits must be 4-byte aligned");
    if (T < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d: need at least one token", T);
    if (E < 1 || E > kMaxExperts)
        return fail(MOE_ERR_INVALID_ARGUMENT, "E = %d: need 1 <= E <= %d", E, kMaxExperts);
    if (k < 1 || k > E || k > kMaxTopK)
        return fail(MOE_ERR_INVALID_ARGUMENT, "k = %d: need 1 <= k <= min(E = %d, %d)", k, E, kMaxTopK);
    if (flags & ~(uint32_t)MOE_ROUTE_RENORM)
        return fail(MOE_ERR_INVALID_ARGUMENT, "flags = 0x%x: only MOE_ROUTE_RENORM is defined", flags);
    if ((int64_t)T * k > (int64_t)1 << 30)
        return fail(MOE_ERR_INVALID_ARGUMENT, "T*k = %lld is too large", (long long)T * k);
    if (!r || !r->idx || !r->w || !r->count || !r->offset || !r->pair || !r->active || !r->n_active)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_routing or one of its arrays is NULL");
    const size_t need = moe::route_workspace_bytes(T, E, k);
    if (need && (!workspace || ws_bytes < need))
        return fail(MOE_ERR_WORKSPACE, "routing workspace: %zu bytes given, %zu needed", ws_bytes, need);
    if (need && !aligned(workspace, 4)) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 4-byte aligned");
    moe::RoutingPtrs rp{r->idx, r->w, r->count, r->offset, r->pair, r->active, r->n_active};
    return finish(from_hip(moe::launch_route(logits, T, E, k, (flags & MOE_ROUTE_RENORM) ? 1 : 0, rp, workspace,
                                             stream),
                           "moe_route_topk launch"),
                  stream, "moe_route_topk");
}

moe_status moe_quantize_act(const float* x, int32_t T, int32_t H, int8_t* xq, float* xd, hipStream_t stream) {
    if (!x || !xq || !xd) return fail(MOE_ERR_INVALID_ARGUMENT, "x, xq or xd is NULL");
    if (T < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d: need at least one token", T);
    if (H < 256 || H % 256 != 0) return fail(MOE_ERR_INVALID_ARGUMENT, "H = %d: must be a positive multiple of 256", H);
    if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(xd, 4))
        return fail(MOE_ERR_INVALID_ARGUMENT, "x must be 16-byte aligned, xq and xd 4-byte aligned");
    return finish(from_hip(moe::launch_quantize_act(x, T, H, xq, xd, stream), "moe_quantize_act launch"), stream,
                  "moe_quantize_act");
}

moe_status moe_router_logits(const float* x, int32_t T, int32_t H, const float* w_router, int32_t E,
                             float* logits, hipStream_t stream) {
    if (!x || !w_router || !logits) return fail(MOE_ERR_INVALID_ARGUMENT, "x, w_router or logits is NULL");
    if (T < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d: need at least one token", T);
    if (E < 1 || E > kMaxExperts) return fail(MOE_ERR_INVALID_ARGUMENT, "E = %d: need 1..%d", E, kMaxExperts);
    if (H < 8 || H % 8 != 0 || H > moe::kRouterMaxH)
        return fail(MOE_ERR_INVALID_ARGUMENT, "H = %d: must be a positive multiple of 8, at most %d", H,
                    moe::kRouterMaxH);
    if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(logits, 4))
        return fail(MOE_ERR_INVALID_ARGUMENT, "x and w_router must be 16-byte aligned, logits 4-byte aligned");
    return finish(from_hip(moe::launch_router(x, T, H, w_router, E, logits, stream), "moe_router_logits launch"),
                  stream, "moe_router_logits");
}

size_t moe_ffn_workspace_bytes(const moe_layer* L, int32_t T, int32_t k, uint32_t flags) {
    if (!L || T < 1 || k < 1) return 0;
    return ffn_ws_layout(L, T, k, resolve_path(flags, T)).total;
}


moe_status moe_expert_ffn_q(const moe_layer* L, const moe_routing* r, int32_t T, int32_t k, const float* x,
                            const int8_t* xq, const float* xd, uint32_t flags, float* y_pair, float* y_shared,
                            void* workspace, size_t ws_bytes, hipStream_t stream) {
    moe_status st = validate_layer(L, T, k, y_shared);
    if (st != MOE_OK) return st;
    if (!r || !r->count || !r->offset || !r->pair || !r->active || !r->n_active)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_routing or one of count/offset/pair/active/n_active is NULL");
    if (!y_pair) return fail(MOE_ERR_INVALID_ARGUMENT, "y_pair is NULL");
    if (flags != MOE_FFN_AUTO && flags != MOE_FFN_DECODE && flags != MOE_FFN_INT8)
        return fail(MOE_ERR_INVALID_ARGUMENT, "flags = 0x%x: use MOE_FFN_AUTO, MOE_FFN_DECODE or MOE_FFN_INT8", flags);
    const uint32_t path = resolve_path(flags, T);
    if (path == MOE_FFN_DECODE && !x) return fail(MOE_ERR_INVALID_ARGUMENT, "decode path needs x (fp32 [T][H])");
    if (path == MOE_FFN_INT8 && (!xq || !xd))
        return fail(MOE_ERR_INVALID_ARGUMENT, "int8 path needs xq and xd from moe_quantize_act");
    if (path == MOE_FFN_INT8 && !aligned(xq, 16))
        return fail(MOE_ERR_INVALID_ARGUMENT, "xq must be 16-byte aligned");
    if ((x && !aligned(x, 4)) || (xd && !aligned(xd, 4)) || !aligned(y_pair, 4) || (y_shared && !aligned(y_shared, 4)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "fp32 arrays must be 4-byte aligned");
    const FfnWorkspace wl = ffn_ws_layout(L, T, k, path);
    if (!workspace || ws_bytes < wl.total)
        return fail(MOE_ERR_WORKSPACE, "FFN workspace: %zu bytes given, %zu needed", ws_bytes, wl.total);
    if (!aligned(workspace, 256)) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");

    moe::FfnArgs a{};
    fill_ffn_args(a, L, T, k);
    a.count = r->count;
    a.offset = r->offset;
    a.pair = r->pair;
    a.active = r->active;
    a.n_active = r->n_active;
    a.x = x;
    a.xq = xq;
    a.xd = xd;
    set_ffn_ws(a, (char*)workspace, wl);
    a.y_pair = y_pair;
    a.y_shared = y_shared;
    if (path == MOE_FFN_DECODE)
        return finish(from_hip(moe::launch_ffn_decode(a, stream), "moe_expert_ffn_q (decode) launch"), stream,
                      "moe_expert_ffn_q");
    return finish(from_hip(moe::launch_ffn_int8(a, stream), "moe_expert_ffn_q (int8) launch"), stream,
                  "moe_expert_ffn_q");
}

size_t moe_forward_workspace_bytes(const moe_layer* L, int32_t T, int32_t k, uint32_t ffn_flags) {
    uint32_t sel = 0;
    bool pair_ws = false;
    if (!L || T < 1 || k < 1 || !split_ffn_flags(ffn_flags, sel, pair_ws)) return 0;
    return forward_ws_layout(L, T, k, resolve_path(sel, T), pair_ws).total;
}

moe_status moe_forward(const moe_layer* L, const float* logits, const float* x, int32_t T, int32_t k,
                       uint32_t route_flags, uint32_t ffn_flags, const moe_routing* r, float* y_pair,
                       float* y_shared, const float* shared_scale, float* out, void* workspace, size_t ws_bytes,
                       hipStream_t stream) {
    return moe_forward_ep(L, logits, x, T, k, route_flags, ffn_flags, r, y_pair, y_shared, shared_scale, nullptr,
                          out, workspace, ws_bytes, stream);
}

moe_status moe_forward_ep(const moe_layer* L, const float* logits, const float* x, int32_t T, int32_t k,
                          uint32_t route_flags, uint32_t ffn_flags, const moe_routing* r, float* y_pair,
                          float* y_shared, const float* shared_scale, const moe_epilogue* ep, float* out,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
    return forward_impl(L, logits, x, T, k, route_flags, ffn_flags, r, y_pair, y_shared, shared_scale, ep, out,
                        workspace, ws_bytes, stream, nullptr);
}

moe_status moe_forward_router(const moe_layer* L, const float* x, const float* w_router, float* logits, int32_t T,
                              int32_t k, uint32_t route_flags, uint32_t ffn_flags, const moe_routing* r,
                              float* y_pair, float* y_shared, const float* shared_scale, float* out, void* workspace,
                              size_t ws_bytes, hipStream_t stream) {
    if (!L) return fail(MOE_ERR_INVALID_ARGUMENT, "layer descriptor is NULL");
    if (!w_router || !aligned(w_router, 16))
        return fail(MOE_ERR_INVALID_ARGUMENT, "w_router is NULL or not 16-byte aligned");
    if (L->hidden > moe::kRouterMaxH)
        return fail(MOE_ERR_UNSUPPORTED, "hidden = %d: the router supports up to %d", L->hidden, moe::kRouterMaxH);
    const RouterStage rt{w_router};
    return forward_impl(L, logits, x, T, k, route_flags, ffn_flags, r, y_pair, y_shared, shared_scale, nullptr, out,
                        workspace, ws_bytes, stream, &rt);
}

moe_status moe_shared_gate(const float* x, int32_t T, int32_t H, const float* gate_w, float* s,
                           hipStream_t stream) {
    if (!x || !gate_w || !s) return fail(MOE_ERR_INVALID_ARGUMENT, "x, gate_w or s is NULL");
    if (T < 1 || H < 4 || H % 4)
        return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d, H = %d: need T >= 1 and H a positive multiple of 4", T, H);
    if (!aligned(x, 16) || !aligned(gate_w, 16) || !aligned(s, 4))
        return fail(MOE_ERR_INVALID_ARGUMENT, "x and gate_w must be 16-byte aligned, s 4-byte aligned");
    return finish(from_hip(moe::launch_shared_gate(x, T, H, gate_w, s, stream), "moe_shared_gate launch"), stream,
                  "moe_shared_gate");
}

moe_status moe_combine(const float* y_pair, const float* w, const float* y_shared, const float* shared_scale,
                       int32_t T, int32_t k, int32_t H, float* out, hipStream_t stream) {
    if (!y_pair || !w || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "y_pair, w or out is NULL");
    if (T < 1 || k < 1 || k > kMaxTopK || H < 1)
        return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d, k = %d, H = %d: need T >= 1, 1 <= k <= %d, H >= 1", T, k, H,
                    kMaxTopK);
    if (shared_scale && !y_shared)
        return fail(MOE_ERR_INVALID_ARGUMENT, "shared_scale given without y_shared");
    if (!aligned(y_pair, 4) || !aligned(w, 4) || !aligned(out, 4) || (y_shared && !aligned(y_shared, 4)) ||
        (shared_scale && !aligned(shared_scale, 4)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "fp32 arrays must be 4-byte aligned");
    return finish(from_hip(moe::launch_combine(y_pair, w, y_shared, shared_scale, nullptr, nullptr, T, k, H, out,
                                               stream),
                           "moe_combine launch"),
                  stream, "moe_combine");
}

moe_status moe_combine_ep(const float* y_pair, const float* w, const float* y_shared, const float* shared_scale,
                          const float* shared_gate_s, const float* residual, int32_t T, int32_t k, int32_t H,
                          float* out, hipStream_t stream) {
    if (!y_pair || !w || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "y_pair, w or out is NULL");
    if (T < 1 || k < 1 || k > kMaxTopK || H < 1)
        return fail(MOE_ERR_INVALID_ARGUMENT, "T = %d, k = %d, H = %d: need T >= 1, 1 <= k <= %d, H >= 1", T, k, H,
                    kMaxTopK);
    if ((shared_scale || shared_gate_s) && !y_shared)
        return fail(MOE_ERR_INVALID_ARGUMENT, "shared_scale or shared_gate_s given without y_shared");
    if (residual && (residual == y_pair || residual == y_shared))
        return fail(MOE_ERR_INVALID_ARGUMENT, "residual must not alias y_pair or y_shared");
    if (!aligned(y_pair, 4) || !aligned(w, 4) || !aligned(out, 4) || (y_shared && !aligned(y_shared, 4)) ||
        (shared_scale && !aligned(shared_scale, 4)) || (shared_gate_s && !aligned(shared_gate_s, 4)) ||
        (residual && !aligned(residual, 4)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "fp32 arrays must be 4-byte aligned");
    return finish(from_hip(moe::launch_combine(y_pair, w, y_shared, shared_scale, shared_gate_s, residual, T, k, H,
                                               out, stream),
                           "moe_combine_ep launch"),
                  stream, "moe_combine_ep");
}

moe_status moe_dequant_q(const void* blocks, int32_t qtype, int64_t n_weights, float* out, hipStream_t stream) {
    if (!blocks || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "blocks or out is NULL");
    if (!known_qtype(qtype))
        return fail(MOE_ERR_UNSUPPORTED, "qtype = %d: supported are Q4_K (%d), Q5_K (%d), Q8_0 (%d) and Q5_1 (%d)",
                    qtype, MOE_Q4_K, MOE_Q5_K, MOE_Q8_0, MOE_Q5_1);
    if (n_weights < 0 || n_weights % blk_weights(qtype) != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "n_weights = %lld is not a multiple of the block size %d",
                    (long long)n_weights, blk_weights(qtype));
    if (!aligned(blocks, blk_align(qtype)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "blocks must be %d-byte aligned", (int)blk_align(qtype));
    if (n_weights == 0) return ok();
    return finish(from_hip(moe::launch_dequant(blocks, qtype, n_weights, out, stream), "moe_dequant_q launch"), stream,
                  "moe_dequant_q");
}

moe_status moe_check_device_errors(hipStream_t stream) {
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return from_hip(e, "moe_check_device_errors: stream synchronize");
    return take_error_word("");
}

moe_status moe_forward_noalloc(const moe_layer* L, const float* logits, const float* x, int32_t T, int32_t k,
                               uint32_t route_flags, uint32_t ffn_flags, const moe_routing* r, float* y_pair,
                               float* y_shared, const float* shared_scale, float* out, hipStream_t stream) {
    moe_status st = validate_layer(L, T, k, y_shared);
    if (st != MOE_OK) return st;
    uint32_t sel = 0;
    bool pair_ws = false;
    if (!split_ffn_flags(ffn_flags, sel, pair_ws))
        return fail(MOE_ERR_INVALID_ARGUMENT,
                    "ffn_flags = 0x%x: use MOE_FFN_AUTO, MOE_FFN_DECODE or MOE_FFN_INT8, optionally with "
                    "MOE_FFN_PAIR_BF16",
                    ffn_flags);
    const size_t need = forward_ws_layout(L, T, k, resolve_path(sel, T), pair_ws).total;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_WORKSPACE,
                    "moe_forward_noalloc: T = %d, k = %d needs %zu bytes of workspace; its static scratch holds %zu "
                    "(use moe_forward with a caller-owned workspace)",
                    T, k, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if ((st = scratch_address(stream, &ws)) != MOE_OK) return st;
    return moe_forward(L, logits, x, T, k, route_flags, ffn_flags, r, y_pair, y_shared, shared_scale, out, ws,
                       (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
