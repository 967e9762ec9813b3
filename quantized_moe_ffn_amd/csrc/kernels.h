// kernels.h — internal launchers of libmoe (host side of the kernel files).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kSmallPairs = 256;  // T*k up to this: routing + bucketing in one workgroup
constexpr int kTilePairs = 256;   // tile of the large-batch counting sort

struct RoutingPtrs {
    int32_t* idx;
    float* w;
    int32_t* count;
    int32_t* offset;
    int32_t* pair;
    int32_t* active;
    int32_t* n_active;
};

// One projection of a bank, as the kernels see it.
struct QMat {
    const uint8_t* data;
    int64_t row_bytes;
    int64_t expert_bytes;
    int qtype;
};

struct FfnArgs {
    QMat gate, up, down;           // routed banks
    QMat sgate, sup, sdown;        // shared expert (used when has_shared)
    int has_shared;
    int H, I, T, k, E;
    const int32_t* count;
    const int32_t* offset;
    const int32_t* pair;
    const int32_t* active;
    const int32_t* n_active;
    const float* x;                // [T][H] fp32 (decode path)
    const int8_t* xq;              // [T][H] int8 (int8 path)
    const float* xd;               // [T][H/256]
    float* h;                      // workspace [T*k + T][I] fp32 (decode path)
    int8_t* hq;                    // workspace [T*k + T][I] int8 (int8 path)
    float* hd;                     // workspace [T*k + T][I/256]
    float* y_pair;                 // [T*k][H]
    float* y_shared;               // [T][H]
    int n_slots;                   // min(E, T*k) routed expert slots
    int16_t* xs;                   // workspace [T][H/32]: per-32 sums of xq (int8 MFMA path)
    int16_t* hs;                   // workspace [T*k + T][I/32]: per-32 sums of hq (int8 MFMA path)
    int32_t* tiles;                // workspace: MFMA tile list (mfma_tiles_bytes)
    int xs_ready;                  // xs already holds the per-32 sums of xq
    int tiles_ready;               // the tile list in tiles is already written (by the routing launches)
    uint16_t* y_pair_bf16;         // non-null: the MFMA GEMMs write the per-pair outputs here as bf16
                                   // [T*k][H] instead of y_pair
};

// The MFMA GEMMs' work list: tile i of expert e covers rows mt*i .. mt*i + mt - 1
// of e's bucket; the shared expert's tiles (expert index E) cover all T tokens.
struct TileList {
    int32_t* tile_e;
    int32_t* tile_m0;
    int32_t* n_tiles;
    int mt;                        // tokens per tile; 0: no tile list
    int max_t;                     // capacity of tile_e / tile_m0
    int T;
    int has_shared;
};

// The grouped int8 MFMA GEMMs of the int8 path (Q4_K gate/up/down).
constexpr int kMfmaMaxDim = 3584;

struct MfmaArgs {
    QMat gate, up, down, sgate, sup, sdown;
    int has_shared, H, I, T, k, E;
    const int32_t* count;
    const int32_t* offset;
    const int32_t* pair;
    const int8_t* xq;              // [T][H]
    const float* xd;               // [T][H/256]
    int16_t* xs;                   // [T][H/32] per-32 sums of xq
    int8_t* hq;                    // [T*k + T][I]
    float* hd;                     // [T*k + T][I/256]
    int16_t* hs;                   // [T*k + T][I/32] per-32 sums of hq
    float* y_pair;                 // [T*k][H]
    float* y_shared;               // [T][H]
    int32_t* tile_e;
    int32_t* tile_m0;
    int32_t* n_tiles;
    int down_rounds;               // 128-row rounds per down workgroup (set by the launcher)
    int xs_ready;                  // xs already holds the per-32 sums of xq (written with the codes)
    int tiles_ready;               // tile_e / tile_m0 / n_tiles already hold the tile list
    uint16_t* y_pair_bf16;         // non-null: y_pair is written here as bf16 (nearest even) instead
};

bool mfma_path_supported(int H, int I, int qg, int qu, int qd);
bool mfma_rows_fit(int T, int k, int H, int I);
int mfma_tile_rows(int T, int k, int E, int H, int I);
size_t mfma_tiles_bytes(int T, int k, int E, int has_shared, int H, int I);
hipError_t launch_ffn_mfma(const MfmaArgs& a, hipStream_t s);

// The two-kernel decode layer (route + gate/up + SiLU; down + combine).
struct DecArgs {
    const float* logits;  // [T][E]
    const float* x;       // [T][H]
    QMat gate, up, down, sgate, sup, sdown;
    int has_shared;
    int T, E, k, H, I, renorm;
    RoutingPtrs r;
    float* h;             // [T*k + T][I]
    float* y_pair;        // [T*k][H] or null
    float* y_shared;      // [T][H] or null
    const float* shared_scale;
    const float* sgate_w; // [H] or null: sigmoid gate of the shared expert
    const float* residual;// [T][H] or null: added to out last
    float* out;           // [T][H]
    int* route_tab;       // workspace: the routing table K1 hands to K2 (kDecRouteTabBytes)
};

constexpr int kDecRouteTabBytes = 4096;

bool dec_fused_supported(int T, int k, int H, int I, int qg, int qu, int qd);
hipError_t launch_dec_fused(const DecArgs& a, hipStream_t s);

// The expert-grouped decode FFN (batches past the two-kernel layer): tile list
// (in f.tiles, dec_grouped_tiles_bytes), gate/up, down; y_pair / y_shared out.
bool dec_grouped_supported(int T, int k, int H, int I, int qg, int qu, int qd);
size_t dec_grouped_tiles_bytes(int T, int k, int E, int has_shared);
hipError_t launch_dec_grouped(const FfnArgs& f, hipStream_t s);

// The int8 path's other two prologue stages, carried by the routing launches of
// a layer call: quantisation of x (launch_quantize_act's rule and outputs) and,
// with tiles.mt > 0, the MFMA tile list (written from the bucket counts).
struct RouteExtras {
    const float* x;                // [T][H], 16-byte aligned
    int H;
    int8_t* xq;
    float* xd;
    int16_t* xs;                   // may be null (no per-32 sums)
    TileList tiles;
    bool tiles_written;            // set by launch_route
};

hipError_t launch_route(const float* logits, int T, int E, int k, int renorm, const RoutingPtrs& r,
                        void* ws, hipStream_t s, RouteExtras* ex = nullptr);
size_t route_workspace_bytes(int T, int E, int k);

hipError_t launch_gateup(const FfnArgs& a, int xmode, hipStream_t s);
hipError_t launch_down(const FfnArgs& a, int hmode, hipStream_t s);
hipError_t launch_ffn_decode(const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn_int8(const FfnArgs& a, hipStream_t s);
// The tile list launch_ffn_int8's MFMA GEMMs would use (mt = 0 when it takes another path).
TileList int8_tile_list(const FfnArgs& a);

constexpr int kRouterGemvMaxT = 16;   // router: tokens up to which the matrix-vector kernel runs
constexpr int kRouterMaxH = 8192;     // router: largest hidden size
hipError_t launch_router(const float* x, int T, int H, const float* w, int E, float* logits, hipStream_t s);

// xs non-null: also the int16 sums of every 32 codes (xs [T][H/32])
hipError_t launch_quantize_act(const float* x, int T, int H, int8_t* xq, float* xd, hipStream_t s,
                               int16_t* xs = nullptr);
// out = sum_j w_j y_pair_j (slot order) + (shared_scale * sgate) * y_shared + residual;
// null arrays drop their term (a null scale or gate is 1).
hipError_t launch_combine(const float* y_pair, const float* w, const float* y_shared, const float* shared_scale,
                          const float* sgate, const float* residual, int T, int k, int H, float* out,
                          hipStream_t s);
// The same with the per-pair rows in bf16 (8-byte aligned), widened exactly to fp32.
hipError_t launch_combine_bf16(const uint16_t* y_pair, const float* w, const float* y_shared,
                               const float* shared_scale, const float* sgate, const float* residual, int T, int k,
                               int H, float* out, hipStream_t s);
// s[t] = 1 / (1 + exp(-(g . x_t))), one wave per token
hipError_t launch_shared_gate(const float* x, int T, int H, const float* g, float* s, hipStream_t st);
hipError_t launch_dequant(const void* blocks, int qtype, int64_t n_weights, float* out, hipStream_t s);

}  // namespace moe
