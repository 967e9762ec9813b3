/*
 * moe.h — C ABI of libmoe: the routed mixture-of-experts FFN over GGUF
 * block-quantized expert weights, on AMD Instinct MI355X (gfx950).
 *
 * The method is the per-layer expert path the Strata pages keep returning to:
 * router logits -> top-k expert selection -> per-expert token buckets -> expert
 * FFN with the weights dequantized inside the dot products (gate and up
 * projections, SiLU(gate)*up, down projection) -> routing-weighted combine, with
 * an optional always-on shared expert.  Sources: "Strata-Sage-A1.5-GGUF" (model
 * card: 256 experts / top-8, Q4_K down experts), "Strata: a 125B MoE at 94
 * tok/s on a 12 GB Card" (sparsity table: 512 experts, 10 routed + 1 shared,
 * hidden 2,560), "Strata v0.1.31" release notes (Unsloth UD-Q4_K_XL bullet:
 * Q4_K / Q8_0 experts, dequantizers bit-exact, dot products within float
 * rounding), "Strata - the details" ("How it works": routers and shared
 * experts on the GPU; MTP verify windows of up to 3 drafts; prompt chunks).
 *
 * Conventions for every call
 *  - Every array argument is a DEVICE pointer owned by the caller; nothing is
 *    retained after the call returns.  Descriptor structs (moe_qmatrix,
 *    moe_layer, moe_routing) live in HOST memory and are read during the call.
 *  - Every call that takes a stream only enqueues work on it: no call
 *    allocates or frees memory, and none synchronises (except
 *    moe_check_device_errors, which is documented to).
 *  - Arguments are validated before anything is enqueued.  On failure the call
 *    returns a non-zero moe_status, enqueues nothing, and moe_last_error()
 *    (per host thread) names the failed check and the numbers involved.
 *  - Errors found by kernels (an expert id out of range in routing buffers
 *    passed in, a non-finite router logit or activation) set a per-device
 *    error word; the kernel then skips the offending item without touching
 *    memory out of bounds.  moe_check_device_errors reports and clears it.
 *  - Results are bitwise deterministic run to run, and a token's result does
 *    not depend on which other tokens share its experts.
 *  - With MOE_SYNC_DEBUG=1 in the environment (read at every call), each call
 *    that enqueues work synchronises its stream and checks the device error
 *    word before returning, so it reports its own asynchronous faults and
 *    kernel-detected errors (MOE_ERR_DEVICE).  Not done while the stream is
 *    being captured into a graph.
 *  - All sizes are element counts unless named *_bytes.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1, /* a shape, pointer, alignment or flag check failed */
    MOE_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement     */
    MOE_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required       */
    MOE_ERR_DEVICE = 4            /* a HIP call failed, or a kernel set the error word */
} moe_status;

/* Block formats, numbered as in GGUF.  The pages name these formats (the
 * "Strata v0.1.31" Unsloth bullet; Q4_K down experts on the Sage-A1.5 card) and
 * give no byte layout; the public GGUF layouts are used:
 *   MOE_Q4_K: 144-byte super-block of 256 weights: fp16 d, fp16 dmin, 12 bytes
 *             packing eight 6-bit scales and eight 6-bit mins, 128 bytes of
 *             4-bit quants; w = d*sc*q - dmin*m per 32-weight sub-block.
 *   MOE_Q5_K: 176-byte super-block of 256 weights: Q4_K's header, then 32
 *             bytes holding the fifth bit of every quant, then the low 4 bits
 *             as Q4_K's quants; q in 0..31, w = d*sc*q - dmin*m.
 *   MOE_Q8_0: 34-byte block of 32 weights: fp16 d, 32 int8 q; w = d*q.
 *   MOE_Q5_1: 24-byte block of 32 weights: fp16 d, fp16 m, a 32-bit
 *             little-endian word whose bit i is the fifth bit of quant i, 16
 *             bytes of low 4 bits (byte l: quant l in the low nibble, quant
 *             16+l in the high nibble); q in 0..31, w = d*q + m.
 * Q4_K and Q5_K banks must be 16-byte aligned, Q5_1 banks 8-byte aligned,
 * Q8_0 banks 2-byte aligned.  The two-kernel decode layer takes gate/up in
 * any of the four formats (one format for both) with down in any of them;
 * the int8 MFMA GEMMs take Q4_K or Q5_K gate/up with Q4_K or Q5_K down; past
 * eight tokens (T*k > 64) the decode path's expert-grouped kernels take Q4_K or
 * Q5_K gate/up with Q4_K, Q5_K or Q8_0 down at H = 2048 or 2560, I = 512
 * (16-byte aligned x); other mixes run on the general kernels of the chosen
 * path. */
enum { MOE_Q5_1 = 7, MOE_Q8_0 = 8, MOE_Q4_K = 12, MOE_Q5_K = 13 };

/* moe_route_topk flags */
enum { MOE_ROUTE_RENORM = 1u }; /* weights = softmax over the k selected logits */

/* moe_expert_ffn_q path selection */
enum {
    MOE_FFN_AUTO = 0u,   /* decode path up to 8 tokens, int8 path above               */
    MOE_FFN_DECODE = 1u, /* fp32 activations, weights dequantized in registers        */
    MOE_FFN_INT8 = 2u,   /* int8 activations (moe_quantize_act); grouped int8 MFMA GEMMs
                            when gate, up and down are Q4_K or Q5_K */
    /* The layer calls only (moe_forward and its variants), OR-ed with one of the
     * above: y_pair is not returned (it may be NULL) and the per-pair outputs
     * reach the combine through the workspace.  On the int8 MFMA GEMMs they are
     * kept as bf16 (rounded to nearest even), which halves their write and read
     * (T*k*H*2 bytes each way instead of *4).  The combine then sums the bf16
     * values widened to fp32, so out moves by at most 2^-8 * sum_j |w_j*y_j| per
     * element (bf16's unit roundoff), inside the int8 path's 5e-3 tolerance
     * ("Strata - the details", "How it works": the per-expert outputs and the
     * weighted sum stay on the GPU).  The other paths keep the per-pair outputs
     * in fp32 and give the same out as without the flag. */
    MOE_FFN_PAIR_BF16 = 16u
};

/* One projection of an expert bank: n_experts matrices of rows x cols weights,
 * each row a contiguous run of blocks (cols contiguous), rows back to back,
 * experts expert_bytes apart.  row_bytes must equal cols/B*S for the format's
 * block of B weights and S bytes; rows must be 16-byte aligned (Q4_K) or the
 * row start 2-byte aligned (Q8_0); data must be 256-byte aligned. */
typedef struct moe_qmatrix {
    const void* data;
    int32_t qtype;
    int32_t rows;
    int32_t cols;
    int32_t reserved;
    int64_t row_bytes;
    int64_t expert_bytes;
} moe_qmatrix;

/* One MoE layer: routed banks gate/up [E][I][H] and down [E][H][I]; when
 * has_shared != 0 the sh_* matrices hold the always-on shared expert (one
 * expert each, same H and I). */
typedef struct moe_layer {
    int32_t n_experts; /* E */
    int32_t hidden;    /* H, a multiple of 256 */
    int32_t inter;     /* I, a multiple of 256 */
    int32_t has_shared;
    moe_qmatrix gate, up, down;
    moe_qmatrix sh_gate, sh_up, sh_down;
} moe_layer;

/* Routing results, all device arrays written by moe_route_topk.
 *   idx [T][k] int32   selected experts, slot j in descending logit order
 *   w   [T][k] fp32    routing weights
 *   count [E], offset [E+1] int32: pairs per expert and their exclusive sums
 *   pair [T*k] int32   pair ids p = t*k + j grouped by expert (ascending expert,
 *                      ascending p within an expert)
 *   active [min(E, T*k)] int32  experts with count > 0, ascending
 *   n_active [1] int32 */
typedef struct moe_routing {
    int32_t* idx;
    float* w;
    int32_t* count;
    int32_t* offset;
    int32_t* pair;
    int32_t* active;
    int32_t* n_active;
} moe_routing;

/* Bytes of device workspace moe_route_topk needs for T tokens, E experts, top-k. */
size_t moe_route_workspace_bytes(int32_t T, int32_t E, int32_t k);

/* Top-k expert selection from router logits plus per-expert bucketing.
 * logits: fp32 [T][E].  Selection order: descending logit, ties to the lower
 * expert index, IEEE comparison (-0 and +0 tie).  With MOE_ROUTE_RENORM the
 * weights are the softmax over the k selected logits; without it, the softmax
 * over all E logits taken at the k selected experts.
 * Checks: 1 <= T; 1 <= k <= min(E, 16); E <= 1024; logits 4-byte aligned; every
 * moe_routing pointer non-null; ws_bytes >= moe_route_workspace_bytes.
 * A non-finite logit sets the device error word (results for that token are
 * still written, ordered by the total order of the bit patterns). */
moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, uint32_t flags,
                          const moe_routing* r, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/* Router projection, the GPU stage in front of the top-k ("Strata - the
 * details", "How it works": routers run on the GPU with their weights in
 * VRAM):  logits[t][e] = sum_h w_router[e][h] * x[t][h], no bias.
 * x fp32 [T][H], w_router fp32 [E][H] (rows contiguous), logits fp32 [T][E];
 * all device pointers owned by the caller.  Sums are fp32 in a fixed order:
 * up to 16 tokens a matrix-vector kernel, above that fp32 MFMA tiles of 32
 * tokens x 32 experts.  Bitwise deterministic; within each of the two kernels
 * a token's logits depend on its own row only (the kernel follows from T).
 * Checks: T >= 1; 1 <= E <= 1024; 8 <= H <= 8192, H % 8 == 0; x and w_router
 * 16-byte aligned, logits 4-byte aligned. */
moe_status moe_router_logits(const float* x, int32_t T, int32_t H, const float* w_router, int32_t E,
                             float* logits, hipStream_t stream);

/* Per-token int8 activation quantisation, once per token and 256-wide block
 * (the "one quantization per token" of the Sage-A1.5 card's round-2 table):
 * amax = max|x|; amax == 0 gives d = 0 and q = 0; otherwise id = 127/amax
 * (IEEE fp32, correctly rounded), q = rint(x*id) (ties to even) clamped to
 * +-127, d = amax/127.  x fp32 [T][H] -> xq int8 [T][H], xd fp32 [T][H/256].
 * Checks: T >= 1, H % 256 == 0, pointers non-null.  A non-finite x sets the
 * device error word and that block is written as q = 0, d = 0 (codes stay
 * finite, as the "Strata v0.1.39" fixes require of q8_1 activations). */
moe_status moe_quantize_act(const float* x, int32_t T, int32_t H, int8_t* xq, float* xd,
                            hipStream_t stream);

/* Bytes of device workspace moe_expert_ffn_q needs. */
size_t moe_ffn_workspace_bytes(const moe_layer* L, int32_t T, int32_t k, uint32_t flags);

/* Expert FFN for every routed (token, slot) pair, and for the shared expert.
 *   y_pair[p] = W_down[e] * (silu(W_gate[e] x_t) .* (W_up[e] x_t)),  e = idx[p], t = p / k
 *   y_shared[t] = the same with the shared expert's matrices (when has_shared).
 * Weights are dequantized inside the dot products.  Decode path: x fp32 [T][H].
 * Int8 path: xq/xd from moe_quantize_act (xq 16-byte aligned); h is
 * re-quantized per (pair, 256-wide block of I) with moe_quantize_act's rule for
 * the int8 down projection.  With gate/up Q4_K or Q5_K and down Q4_K or Q5_K
 * (and (T*k + T)*max(H, I) < 2^31) both projections run as grouped int8 MFMA
 * GEMMs over the tokens of each expert; there the min term is carried in fp16,
 * so every block's dmin*m (Q4_K), or 16*d*sc - dmin*m (Q5_K, whose quants
 * enter as q - 16), must stay below 65504 in magnitude (dmin below 1039; for
 * Q5_K also d below 64).  Other format mixes use the decode path's kernels on
 * the dequantized int8 activations.  y_pair fp32
 * [T*k][H]; y_shared fp32 [T][H] (required iff has_shared).  r must hold the
 * result of moe_route_topk for the same T, k and E (read on the device: no host
 * synchronisation).
 * Checks: shapes consistent with L; H, I multiples of 256; qtypes supported
 * (gate/up/down: Q4_K, Q5_K, Q8_0 or Q5_1); alignment; workspace size. */
moe_status moe_expert_ffn_q(const moe_layer* L, const moe_routing* r, int32_t T, int32_t k,
                            const float* x, const int8_t* xq, const float* xd, uint32_t flags,
                            float* y_pair, float* y_shared, void* workspace, size_t ws_bytes,
                            hipStream_t stream);

/* Routing-weighted combine:
 *   out[t] = sum_{j<k} w[t][j] * y_pair[t*k+j]  (+ s_t * y_shared[t])
 * summed in slot order, then the shared expert; s_t = shared_scale[t], or 1
 * when shared_scale is NULL; y_shared may be NULL (no shared expert).
 * All fp32 and 4-byte aligned; out [T][H].  No residual, norm or bias. */
moe_status moe_combine(const float* y_pair, const float* w, const float* y_shared,
                       const float* shared_scale, int32_t T, int32_t k, int32_t H, float* out,
                       hipStream_t stream);

/* Routing-weighted combine with the layer epilogue:
 *   out[t] = sum_{j<k} w[t][j] * y_pair[t*k+j] + s_t * y_shared[t] + residual[t]
 * in that order (slot order, then the shared expert, then the residual), with
 * s_t = shared_scale[t] * shared_gate_s[t] (a NULL factor is 1; both need
 * y_shared).  shared_gate_s [T] holds the gate values moe_shared_gate writes.
 * residual [T][H] or NULL; out may be the residual array itself (an in-place
 * update of the residual stream) but must not alias y_pair or y_shared.  With
 * shared_gate_s and residual NULL this is moe_combine, bit for bit.  All
 * arrays fp32 and 4-byte aligned. */
moe_status moe_combine_ep(const float* y_pair, const float* w, const float* y_shared,
                          const float* shared_scale, const float* shared_gate_s, const float* residual,
                          int32_t T, int32_t k, int32_t H, float* out, hipStream_t stream);

/* Sigmoid gate of a shared expert ("Strata - the details", "How it works":
 * shared experts and the gated-residual weights stay on the GPU; the gate's
 * form is a reading: one fp32 weight vector per layer):
 *   s[t] = 1 / (1 + exp(-(gate_w . x[t])))
 * x fp32 [T][H] and gate_w fp32 [H], both 16-byte aligned; s fp32 [T].  The dot
 * is summed in a fixed order by one wave per token; moe_forward_ep computes the
 * same bits inside the decode layer.  Checks: T >= 1, H a positive multiple of
 * 4, non-null pointers, alignment. */
moe_status moe_shared_gate(const float* x, int32_t T, int32_t H, const float* gate_w, float* s,
                           hipStream_t stream);

/* Bytes of device workspace moe_forward needs (for the path ffn_flags selects,
 * with room for the per-pair outputs when it carries MOE_FFN_PAIR_BF16). */
size_t moe_forward_workspace_bytes(const moe_layer* L, int32_t T, int32_t k, uint32_t ffn_flags);

/* The whole layer: routing (as moe_route_topk, results written to r), expert
 * FFN (as moe_expert_ffn_q, from fp32 x; on the int8 path x is quantized with
 * moe_quantize_act's rule into the workspace) and combine (as moe_combine),
 * enqueued on one stream.  For decode batches (T <= 8, T*k <= 64, gate/up of
 * one format with H/256 in {1,2,4,8,10}, down rows of 8, 16 or 32 32-weight
 * blocks, 16-byte aligned banks) the layer runs as two
 * kernels: routing fused into the gate/up kernel (each wave recomputes the
 * top-k of its token) and the combine fused into the down kernel (formed in
 * slot order in LDS); other shapes run the separate stages.  Same results
 * contract as the three calls (bitwise
 * deterministic; combine in slot order).  y_pair [T*k][H] is written unless
 * ffn_flags carries MOE_FFN_PAIR_BF16 (then it may be NULL and is not touched);
 * y_shared [T][H] is required iff the layer has a shared expert;
 * shared_scale [T] or NULL (non-NULL needs a shared expert).  x must be
 * 16-byte aligned.  Checks: those of
 * moe_route_topk and moe_expert_ffn_q; ws_bytes >= moe_forward_workspace_bytes. */
moe_status moe_forward(const moe_layer* L, const float* logits, const float* x, int32_t T, int32_t k,
                       uint32_t route_flags, uint32_t ffn_flags, const moe_routing* r, float* y_pair,
                       float* y_shared, const float* shared_scale, float* out, void* workspace,
                       size_t ws_bytes, hipStream_t stream);

/* The layer epilogue of moe_forward_ep.  NULL members drop their term. */
typedef struct moe_epilogue {
    const float* residual;    /* fp32 [T][H]: added to out last; may be out itself */
    const float* shared_gate; /* fp32 [H], 16-byte aligned: the shared expert is scaled by
                                 sigmoid(shared_gate . x_t) (times shared_scale[t] when given);
                                 needs a layer with a shared expert */
} moe_epilogue;

/* moe_forward followed by the epilogue (ep NULL: moe_forward exactly): the
 * combine becomes moe_combine_ep's, with the gate values computed from x as
 * moe_shared_gate does.  On the two-kernel decode layer both are fused: the
 * routing workgroup of the gate/up kernel computes the gate, the down kernel
 * adds the residual while it forms the combine; elsewhere a gate kernel and
 * the combine kernel do it.  The gate values are the same bits on both, and
 * the epilogue equals moe_forward with those values as shared_scale followed
 * by one fp32 add of the residual, bit for bit.  Extra checks: shared_gate
 * needs has_shared; residual must not alias y_pair or y_shared. */
moe_status moe_forward_ep(const moe_layer* L, const float* logits, const float* x, int32_t T, int32_t k,
                          uint32_t route_flags, uint32_t ffn_flags, const moe_routing* r, float* y_pair,
                          float* y_shared, const float* shared_scale, const moe_epilogue* ep, float* out,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/* The layer from the activations and the router matrix, in one call: the
 * router projection of moe_router_logits (its kernel, so the same bits, written
 * to logits fp32 [T][E]), then moe_forward on those logits with moe_forward's
 * arguments, workspace (moe_forward_workspace_bytes), checks and results
 * contract.  Router matrices are a GPU stage in front of the top-k ("Strata -
 * the details", "How it works").  w_router fp32 [E][H], 16-byte aligned;
 * H <= 8192.  No epilogue (see moe_forward_ep). */
moe_status moe_forward_router(const moe_layer* L, const float* x, const float* w_router, float* logits, int32_t T,
                              int32_t k, uint32_t route_flags, uint32_t ffn_flags, const moe_routing* r,
                              float* y_pair, float* y_shared, const float* shared_scale, float* out, void* workspace,
                              size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): moe_forward
 * with its workspace taken from a static device array of the library,
 * MOE_NOALLOC_SCRATCH_BYTES per GPU, held by each GPU the library runs on until
 * the process ends.  Same arguments, checks, results and contract as
 * moe_forward, without workspace/ws_bytes.  Rejects (MOE_ERR_WORKSPACE, nothing
 * enqueued) a call whose moe_forward_workspace_bytes exceeds the array: every
 * decode batch fits, and int8-path batches up to about a thousand tokens of a
 * hidden-2048 / top-8 / intermediate-512 layer (about two hundred with
 * MOE_FFN_PAIR_BF16, whose per-pair outputs then take room in the array too).
 * Calls no allocating routine.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and give wrong results;
 * serialise them.  The array needs no clearing: each call writes every byte of
 * it that it reads. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
moe_status moe_forward_noalloc(const moe_layer* L, const float* logits, const float* x, int32_t T, int32_t k,
                               uint32_t route_flags, uint32_t ffn_flags, const moe_routing* r, float* y_pair,
                               float* y_shared, const float* shared_scale, float* out, hipStream_t stream);

/* Test hook: dequantize n_weights weights of contiguous blocks to fp32 with the
 * unpacking helpers of the general (unfused) kernels.  Each value is the exact
 * d*sc*q - dmin*m (Q4_K, Q5_K), d*q (Q8_0) or d*q + m (Q5_1) rounded once to
 * fp32.  The two-kernel decode layer and the int8 MFMA GEMMs unpack the same
 * blocks with code of their own (per-lane slices; 3-bit scale limbs); those
 * are pinned by layers whose every result is exact.  n_weights must be a
 * multiple of the block size. */
moe_status moe_dequant_q(const void* blocks, int32_t qtype, int64_t n_weights, float* out,
                         hipStream_t stream);

/* Synchronises `stream`, then reads and clears the current device's error
 * word.  Returns MOE_ERR_DEVICE (and a message naming the flags) if set. */
moe_status moe_check_device_errors(hipStream_t stream);

/* Message for the last failed call on this host thread ("" if none). */
const char* moe_last_error(void);

int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
