// ffn_int8.hip — the int8-activation expert FFN (prompt chunks).
//
// Quantisation points, as on the pages' prompt path ("one quantization per
// token", the "Strata-Sage-A1.5-GGUF" card's round-2 table; quantized expert
// kernels instead of FP16 expansion, "Strata - the details", faster prompts):
// token activations enter as xq/xd (moe_quantize_act), and h = silu(g)*u is
// re-quantized per (pair, 256-wide block of I) with the same rule before the
// down projection.
//
// This version evaluates both projections with the decode path's in-register
// dequantization on x = xd*xq and h = hd*hq.
#include "common.h"
#include "kernels.h"

namespace moe {

hipError_t launch_ffn_int8(const FfnArgs& a, void* ws_extra, hipStream_t s) {
    (void)ws_extra;
    hipError_t e = launch_gateup(a, 1, s);
    if (e != hipSuccess) return e;
    const int rows = a.T * a.k + (a.has_shared ? a.T : 0);
    e = launch_quantize_act(a.h, rows, a.I, a.hq, a.hd, s);
    if (e != hipSuccess) return e;
    return launch_down(a, 1, s);
}

size_t ffn_int8_extra_bytes(int T, int k, int E, int H, int I) {
    (void)T; (void)k; (void)E; (void)H; (void)I;
    return 0;
}

}  // namespace moe
