// ffn_int8.hip — the int8-activation expert FFN (prompt chunks).
//
// Quantisation points, as on the pages' prompt path ("one quantization per
// token", the "Strata-Sage-A1.5-GGUF" card's round-2 table; quantized expert
// kernels instead of FP16 expansion, "Strata - the details", faster prompts):
// token activations enter as xq/xd (moe_quantize_act), and h = silu(g)*u is
// re-quantized per (pair, 256-wide block of I) with the same rule before the
// down projection.
//
// Q4_K or Q5_K gate/up with Q4_K or Q5_K down run as grouped int8 MFMA GEMMs
// (ffn_mfma.hip).  Other format mixes evaluate both projections with the
// decode path's in-register dequantization on x = xd*xq and h = hd*hq.
#include "common.h"
#include "kernels.h"

namespace moe {

TileList int8_tile_list(const FfnArgs& a) {
    TileList t{};
    // (the shared expert's formats equal the routed ones: checked by the API layer)
    if (!a.tiles || !mfma_path_supported(a.H, a.I, a.gate.qtype, a.up.qtype, a.down.qtype)) return t;
    const size_t half = (mfma_tiles_bytes(a.T, a.k, a.E, a.has_shared, a.H, a.I) - 256) / 2;
    t.tile_e = a.tiles;
    t.tile_m0 = a.tiles + half / sizeof(int32_t);
    t.n_tiles = a.tiles + 2 * (half / sizeof(int32_t));
    t.mt = mfma_tile_rows(a.T, a.k, a.E, a.H, a.I);
    t.max_t = max_tiles(a.T, a.k, a.E, a.has_shared, t.mt);
    t.T = a.T;
    t.has_shared = a.has_shared;
    return t;
}

hipError_t launch_ffn_int8(const FfnArgs& a, hipStream_t s) {
    const TileList tl = int8_tile_list(a);
    if (tl.mt > 0) {
        MfmaArgs m{};
        m.gate = a.gate;
        m.up = a.up;
        m.down = a.down;
        m.sgate = a.sgate;
        m.sup = a.sup;
        m.sdown = a.sdown;
        m.has_shared = a.has_shared;
        m.H = a.H;
        m.I = a.I;
        m.T = a.T;
        m.k = a.k;
        m.E = a.E;
        m.count = a.count;
        m.offset = a.offset;
        m.pair = a.pair;
        m.xq = a.xq;
        m.xd = a.xd;
        m.xs = a.xs;
        m.hq = a.hq;
        m.hd = a.hd;
        m.hs = a.hs;
        m.y_pair = a.y_pair;
        m.y_shared = a.y_shared;
        m.xs_ready = a.xs_ready;
        m.tile_e = tl.tile_e;
        m.tile_m0 = tl.tile_m0;
        m.n_tiles = tl.n_tiles;
        m.tiles_ready = a.tiles_ready;
        m.y_pair_bf16 = a.y_pair_bf16;
        return launch_ffn_mfma(m, s);
    }
    if (a.y_pair_bf16) return hipErrorInvalidValue;   // bf16 pair outputs come from the MFMA GEMMs only
    hipError_t e = launch_gateup(a, 1, s);
    if (e != hipSuccess) return e;
    const int rows = a.T * a.k + (a.has_shared ? a.T : 0);
    e = launch_quantize_act(a.h, rows, a.I, a.hq, a.hd, s);
    if (e != hipSuccess) return e;
    return launch_down(a, 1, s);
}

}  // namespace moe
