/*
 * moe_oracle.c — CPU oracle for the routed mixture-of-experts FFN over GGUF
 * block-quantized expert weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library, and the product path never
 * calls it.
 *
 * It is deliberately plain and slow: every weight is unpacked from its bytes
 * by the format definition, every sum is accumulated in fp64 in index order,
 * and nothing is blocked, fused or reordered beyond what the definitions say.
 * The only concession to speed is an OpenMP "parallel for" over independent
 * output rows (each row's sum is still a plain sequential loop).
 *
 * What the pages fix and what is read into them
 * ---------------------------------------------
 * The pages name the method but print none of its equations:
 *  - "Strata-Sage-A1.5-GGUF" (model card, intro and round-1 flag table): a
 *    256-expert / top-8 MoE shipped as Q4_K_M, whose down-projection experts
 *    are Q4_K.
 *  - "Strata: a 125B MoE at 94 tok/s on a 12 GB Card" (sparsity table): 512
 *    experts per layer, 10 routed + 1 shared active, hidden size 2,560.
 *  - "Strata v0.1.31" release notes (Unsloth UD-Q4_K_XL bullet): experts in
 *    Q4_K and Q8_0 (among others) run natively; the GPU dequantizers match the
 *    reference dequantizer bit for bit, and the dot products match the CPU
 *    "within float rounding".
 *  - "Strata - the details" ("How it works"): routers and shared experts live
 *    on the GPU; prompts run in chunks of up to 8,192 tokens.
 *  - "Strata v0.1.39" release notes (fixes): the activations quantized for the
 *    GPU dot products are kept finite.
 * The readings taken where the pages are silent (each function says which):
 *  R-layout  Q4_K, Q5_K, Q5_1 and Q8_0 byte layouts are the public GGUF
 *            ones (Q5_K and Q5_1: among the expert formats of the Unsloth
 *            UD-Q4_K_XL files the "Strata v0.1.31" release notes say run
 *            natively).
 *  R-topk    top-k by logit, descending, ties to the lower expert index,
 *            IEEE comparison (so -0 == +0 is a tie).
 *  R-softmax routing weights are the softmax over the k selected logits
 *            (softmax over all E renormalised over the k); without the
 *            renormalise flag, the plain softmax over all E at the k slots.
 *  R-ffn     expert FFN = W_down * (silu(W_gate x) .* (W_up x)),
 *            silu(g) = g / (1 + exp(-g)).
 *  R-combine out_t = sum_j w_tj * y_tj (slot order) + s_t * y_shared_t; no
 *            norm or bias.
 *  R-epilogue the layer's optional epilogue: the shared expert scaled by a
 *            sigmoid gate 1/(1 + exp(-(g . x_t))) of the token's hidden state
 *            (one vector g per layer; the pages keep shared experts and the
 *            "gated-residual" weights on the GPU, "Strata - the details", "How
 *            it works"), and the residual stream added to the layer output.
 *  R-router  router logits are a plain projection of the token's hidden
 *            state by an fp32 [E][H] router matrix: logit_e = sum_h W[e][h]
 *            x[h], no bias ("Strata - the details", "How it works": routers
 *            are a GPU stage; their weights live in VRAM).
 *  R-quant   activations quantized once per token, per 256-wide block:
 *            amax = max|x|; amax == 0 gives d = 0, q = 0; otherwise
 *            id = 127/amax, q = rint(x*id) (ties to even) clamped to +-127,
 *            d = amax/127.  For token activations this is evaluated in IEEE
 *            fp32 (the codes must match the GPU bit for bit); for the
 *            intermediate h of the int8 path it is evaluated in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_Q5_1 7
#define ORC_Q8_0 8
#define ORC_Q4_K 12
#define ORC_Q5_K 13

int orc_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the parallel loops from now on (n >= 1); for a single-thread
 * baseline of the same code. */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------- */
/* IEEE binary16 -> fp64, exact for every bit pattern (incl. subnormals).     */
/* Q4_K's d/dmin and Q8_0's d are stored as binary16 (R-layout).             */
/* ------------------------------------------------------------------------- */
double orc_fp16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int mant = h & 0x3FF;
    double v;
    if (expo == 0) {
        v = ldexp((double)mant, -24);               /* subnormal: m * 2^-24 */
    } else if (expo == 31) {
        v = mant ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + mant), expo - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------------------- */
/* Q4_K super-block (R-layout): 144 bytes for 256 weights.                   */
/*   [0:2]   d     fp16                                                     */
/*   [2:4]   dmin  fp16                                                     */
/*   [4:16]  s[12] eight 6-bit scales and eight 6-bit mins, packed          */
/*   [16:144] qs[128] 4-bit quants                                          */
/* Sub-block j (0..7) holds weights 32j..32j+31.                            */
/*   j < 4 : sc = s[j] & 63,  m = s[j+4] & 63                                */
/*   j >= 4: sc = (s[j+4] & 15) | ((s[j-4] >> 6) << 4)                       */
/*           m  = (s[j+4] >> 4) | ((s[j]   >> 6) << 4)                       */
/* Quants: byte qs[32c+l] holds weight 64c+l in its low nibble and weight   */
/* 64c+32+l in its high nibble (c = 0..3, l = 0..31).                       */
/* Weight value: w = d*sc*q - dmin*m.                                        */
/* ------------------------------------------------------------------------- */
void orc_q4k_unpack(const uint8_t* blk, uint16_t* d_bits, uint16_t* dmin_bits,
                    int32_t* sc, int32_t* m, int32_t* q) {
    const uint8_t* s = blk + 4;
    const uint8_t* qs = blk + 16;
    *d_bits = rd16(blk);
    *dmin_bits = rd16(blk + 2);
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            m[j] = s[j + 4] & 63;
        } else {
            sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            m[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
    }
    for (int c = 0; c < 4; ++c) {
        for (int l = 0; l < 32; ++l) {
            q[64 * c + l] = qs[32 * c + l] & 15;
            q[64 * c + 32 + l] = qs[32 * c + l] >> 4;
        }
    }
}

/* Inverse of orc_q4k_unpack: fields -> 144 bytes.  Field ranges: sc, m in
 * 0..63, q in 0..15.  Together with unpack this is a bijection between the
 * 144 bytes and the fields (96 bits of scales/mins fill the 12 bytes exactly). */
void orc_q4k_pack(uint16_t d_bits, uint16_t dmin_bits, const int32_t* sc,
                  const int32_t* m, const int32_t* q, uint8_t* blk) {
    uint8_t* s = blk + 4;
    uint8_t* qs = blk + 16;
    blk[0] = (uint8_t)(d_bits & 0xFF);
    blk[1] = (uint8_t)(d_bits >> 8);
    blk[2] = (uint8_t)(dmin_bits & 0xFF);
    blk[3] = (uint8_t)(dmin_bits >> 8);
    for (int j = 0; j < 4; ++j) {
        /* low 6 bits: sc_j / m_j ; top 2 bits: the high bits of sc_{j+4} / m_{j+4} */
        s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        s[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
        s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
    }
    for (int c = 0; c < 4; ++c)
        for (int l = 0; l < 32; ++l)
            qs[32 * c + l] = (uint8_t)((q[64 * c + l] & 15) | ((q[64 * c + 32 + l] & 15) << 4));
}

/* Dequantize n_blocks Q4_K super-blocks into 256*n_blocks fp64 weights.
 * Every product here is exact in fp64 (d has 11 significant bits), so each
 * weight is the exact value of the format's definition. */
void orc_q4k_dequant(const uint8_t* blocks, int64_t n_blocks, double* out) {
    for (int64_t b = 0; b < n_blocks; ++b) {
        uint16_t db, dmb;
        int32_t sc[8], m[8], q[256];
        orc_q4k_unpack(blocks + 144 * b, &db, &dmb, sc, m, q);
        double d = orc_fp16_to_f64(db), dmin = orc_fp16_to_f64(dmb);
        for (int i = 0; i < 256; ++i) {
            int j = i / 32;
            out[256 * b + i] = d * sc[j] * q[i] - dmin * m[j];
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Q5_K super-block (R-layout): 176 bytes for 256 weights.                   */
/*   [0:2]    d     fp16                                                    */
/*   [2:4]    dmin  fp16                                                    */
/*   [4:16]   s[12] the 6-bit scales and mins, packed as in Q4_K            */
/*   [16:48]  qh[32] the fifth (high) bit of every quant                    */
/*   [48:176] qs[128] the low 4 bits, laid out as Q4_K's quants             */
/* Quant of weight 64c+l:    (qs[32c+l] & 15) + 16 * bit 2c   of qh[l]      */
/* Quant of weight 64c+32+l: (qs[32c+l] >> 4) + 16 * bit 2c+1 of qh[l]      */
/* (c = 0..3, l = 0..31); q in 0..31.  Weight value: w = d*sc*q - dmin*m.    */
/* ------------------------------------------------------------------------- */
void orc_q5k_unpack(const uint8_t* blk, uint16_t* d_bits, uint16_t* dmin_bits,
                    int32_t* sc, int32_t* m, int32_t* q) {
    const uint8_t* s = blk + 4;
    const uint8_t* qh = blk + 16;
    const uint8_t* qs = blk + 48;
    *d_bits = rd16(blk);
    *dmin_bits = rd16(blk + 2);
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            m[j] = s[j + 4] & 63;
        } else {
            sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            m[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
    }
    for (int c = 0; c < 4; ++c) {
        for (int l = 0; l < 32; ++l) {
            q[64 * c + l] = (qs[32 * c + l] & 15) + 16 * ((qh[l] >> (2 * c)) & 1);
            q[64 * c + 32 + l] = (qs[32 * c + l] >> 4) + 16 * ((qh[l] >> (2 * c + 1)) & 1);
        }
    }
}

/* Inverse of orc_q5k_unpack: fields (sc, m in 0..63, q in 0..31) -> 176
 * bytes; with unpack a bijection (the 8 qh bits of byte l are the fifth bits
 * of weights l, 32+l, 64+l, ..., 224+l in that order). */
void orc_q5k_pack(uint16_t d_bits, uint16_t dmin_bits, const int32_t* sc,
                  const int32_t* m, const int32_t* q, uint8_t* blk) {
    uint8_t* s = blk + 4;
    uint8_t* qh = blk + 16;
    uint8_t* qs = blk + 48;
    blk[0] = (uint8_t)(d_bits & 0xFF);
    blk[1] = (uint8_t)(d_bits >> 8);
    blk[2] = (uint8_t)(dmin_bits & 0xFF);
    blk[3] = (uint8_t)(dmin_bits >> 8);
    for (int j = 0; j < 4; ++j) {
        s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        s[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
        s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
    }
    for (int l = 0; l < 32; ++l) {
        int h = 0;
        for (int c = 0; c < 4; ++c) {
            h |= ((q[64 * c + l] >> 4) & 1) << (2 * c);
            h |= ((q[64 * c + 32 + l] >> 4) & 1) << (2 * c + 1);
        }
        qh[l] = (uint8_t)h;
    }
    for (int c = 0; c < 4; ++c)
        for (int l = 0; l < 32; ++l)
            qs[32 * c + l] = (uint8_t)((q[64 * c + l] & 15) | ((q[64 * c + 32 + l] & 15) << 4));
}

/* Dequantize n_blocks Q5_K super-blocks (exact in fp64, as for Q4_K). */
void orc_q5k_dequant(const uint8_t* blocks, int64_t n_blocks, double* out) {
    for (int64_t b = 0; b < n_blocks; ++b) {
        uint16_t db, dmb;
        int32_t sc[8], m[8], q[256];
        orc_q5k_unpack(blocks + 176 * b, &db, &dmb, sc, m, q);
        double d = orc_fp16_to_f64(db), dmin = orc_fp16_to_f64(dmb);
        for (int i = 0; i < 256; ++i) {
            int j = i / 32;
            out[256 * b + i] = d * sc[j] * q[i] - dmin * m[j];
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Q8_0 block (R-layout): 34 bytes for 32 weights: fp16 d, then 32 int8 q.   */
/* Weight value: w = d*q.                                                    */
/* ------------------------------------------------------------------------- */
void orc_q80_dequant(const uint8_t* blocks, int64_t n_blocks, double* out) {
    for (int64_t b = 0; b < n_blocks; ++b) {
        const uint8_t* blk = blocks + 34 * b;
        double d = orc_fp16_to_f64(rd16(blk));
        for (int i = 0; i < 32; ++i)
            out[32 * b + i] = d * (double)(int8_t)blk[2 + i];
    }
}

/* ------------------------------------------------------------------------- */
/* Q5_1 block (R-layout): 24 bytes for 32 weights.                           */
/*   [0:2]  d   fp16                                                        */
/*   [2:4]  m   fp16 (an offset added to every weight)                       */
/*   [4:8]  qh  32-bit little-endian word: bit i is the fifth bit of weight i*/
/*   [8:24] qs[16] the low 4 bits: byte l holds weight l in its low nibble   */
/*          and weight 16+l in its high nibble                               */
/* Quant of weight l:    (qs[l] & 15) + 16 * bit l      of qh                */
/* Quant of weight 16+l: (qs[l] >> 4) + 16 * bit (16+l) of qh   (l = 0..15); */
/* q in 0..31.  Weight value: w = d*q + m.                                   */
/* ------------------------------------------------------------------------- */
void orc_q51_unpack(const uint8_t* blk, uint16_t* d_bits, uint16_t* m_bits, int32_t* q) {
    const uint8_t* qs = blk + 8;
    uint32_t qh = (uint32_t)blk[4] | ((uint32_t)blk[5] << 8) | ((uint32_t)blk[6] << 16) | ((uint32_t)blk[7] << 24);
    *d_bits = rd16(blk);
    *m_bits = rd16(blk + 2);
    for (int l = 0; l < 16; ++l) {
        q[l] = (qs[l] & 15) + 16 * (int32_t)((qh >> l) & 1u);
        q[16 + l] = (qs[l] >> 4) + 16 * (int32_t)((qh >> (16 + l)) & 1u);
    }
}

/* Inverse of orc_q51_unpack: fields (q in 0..31) -> 24 bytes; with unpack a
 * bijection between the bytes and (d bits, m bits, q[32]). */
void orc_q51_pack(uint16_t d_bits, uint16_t m_bits, const int32_t* q, uint8_t* blk) {
    uint32_t qh = 0;
    blk[0] = (uint8_t)(d_bits & 0xFF);
    blk[1] = (uint8_t)(d_bits >> 8);
    blk[2] = (uint8_t)(m_bits & 0xFF);
    blk[3] = (uint8_t)(m_bits >> 8);
    for (int i = 0; i < 32; ++i) qh |= (uint32_t)((q[i] >> 4) & 1) << i;
    for (int b = 0; b < 4; ++b) blk[4 + b] = (uint8_t)(qh >> (8 * b));
    for (int l = 0; l < 16; ++l) blk[8 + l] = (uint8_t)((q[l] & 15) | ((q[16 + l] & 15) << 4));
}

/* Dequantize n_blocks Q5_1 blocks into 32*n_blocks fp64 weights.  d*q and m
 * are multiples of 2^-24 below 2^21 in magnitude, so d*q + m is exact in
 * fp64: each weight is the exact value of the definition. */
void orc_q51_dequant(const uint8_t* blocks, int64_t n_blocks, double* out) {
    for (int64_t b = 0; b < n_blocks; ++b) {
        uint16_t db, mb;
        int32_t q[32];
        orc_q51_unpack(blocks + 24 * b, &db, &mb, q);
        double d = orc_fp16_to_f64(db), m = orc_fp16_to_f64(mb);
        for (int i = 0; i < 32; ++i) out[32 * b + i] = d * q[i] + m;
    }
}

static int blk_weights(int qtype) { return (qtype == ORC_Q8_0 || qtype == ORC_Q5_1) ? 32 : 256; }
static int blk_bytes(int qtype) {
    return qtype == ORC_Q4_K ? 144 : (qtype == ORC_Q5_K ? 176 : (qtype == ORC_Q5_1 ? 24 : 34));
}

/* One row of a quantized matrix (cols weights) -> fp64. */
static void dequant_row(const uint8_t* row, int qtype, int cols, double* out) {
    int64_t nb = cols / blk_weights(qtype);
    if (qtype == ORC_Q4_K)
        orc_q4k_dequant(row, nb, out);
    else if (qtype == ORC_Q5_K)
        orc_q5k_dequant(row, nb, out);
    else if (qtype == ORC_Q5_1)
        orc_q51_dequant(row, nb, out);
    else
        orc_q80_dequant(row, nb, out);
}

/* ------------------------------------------------------------------------- */
/* Router projection (R-router): x fp32 [T][H], W fp32 [E][H] -> fp64 [T][E] */
/* logits, each a sequential fp64 sum over h.                                */
/* ------------------------------------------------------------------------- */
void orc_router_logits(const float* x, int32_t T, int32_t H, const float* W, int32_t E, double* out) {
#pragma omp parallel for schedule(static)
    for (int64_t te = 0; te < (int64_t)T * E; ++te) {
        const int64_t t = te / E, e = te % E;
        const float* xr = x + t * H;
        const float* wr = W + e * H;
        double acc = 0.0;
        for (int32_t h = 0; h < H; ++h) acc += (double)wr[h] * (double)xr[h];
        out[te] = acc;
    }
}

/* ------------------------------------------------------------------------- */
/* Routing: top-k expert selection from router logits (R-topk, R-softmax).   */
/* logits fp32 [T][E] -> idx [T][k] (slot order = descending logit), w [T][k]*/
/* ------------------------------------------------------------------------- */
void orc_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                    int32_t* idx, double* w) {
    char* taken = (char*)malloc((size_t)E);
    for (int32_t t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        memset(taken, 0, (size_t)E);
        /* k passes of a plain arg-max; scanning ascending with a strict '>'
           keeps the lower index on ties (and treats -0 and +0 as equal). */
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            idx[(int64_t)t * k + j] = best;
        }
        double* wt = w + (int64_t)t * k;
        if (renorm) {
            double top = (double)l[idx[(int64_t)t * k]];
            double sum = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                wt[j] = exp((double)l[idx[(int64_t)t * k + j]] - top);
                sum += wt[j];
            }
            for (int32_t j = 0; j < k; ++j) wt[j] /= sum;
        } else {
            double top = (double)l[idx[(int64_t)t * k]];
            double sum = 0.0;
            for (int32_t e = 0; e < E; ++e) sum += exp((double)l[e] - top);
            for (int32_t j = 0; j < k; ++j) wt[j] = exp((double)l[idx[(int64_t)t * k + j]] - top) / sum;
        }
    }
    free(taken);
}

/* ------------------------------------------------------------------------- */
/* Bucketing of (token, slot) pairs per expert.  Pair id p = t*k + j.        */
/* count[e], offset[e] (exclusive prefix sum, offset[E] = T*k), pair[] lists */
/* the pairs grouped by expert in ascending expert id and ascending p within  */
/* an expert; active[] lists the experts with count > 0, ascending.          */
/* ------------------------------------------------------------------------- */
void orc_bucket(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* count,
                int32_t* offset, int32_t* pair, int32_t* active, int32_t* n_active) {
    int32_t P = T * k;
    for (int32_t e = 0; e < E; ++e) count[e] = 0;
    for (int32_t p = 0; p < P; ++p) count[idx[p]]++;
    offset[0] = 0;
    for (int32_t e = 0; e < E; ++e) offset[e + 1] = offset[e] + count[e];
    int32_t pos = 0, na = 0;
    for (int32_t e = 0; e < E; ++e) {
        for (int32_t p = 0; p < P; ++p)
            if (idx[p] == e) pair[pos++] = p;
        if (count[e] > 0) active[na++] = e;
    }
    *n_active = na;
}

/* ------------------------------------------------------------------------- */
/* Activation quantisation, evaluated in IEEE fp32 (R-quant).                */
/* x fp32 [T][H] -> xq int8 [T][H], xd fp32 [T][H/256].                      */
/* This file is compiled without fast-math or FP contraction, so each        */
/* operation below is one correctly rounded fp32 operation.                  */
/* ------------------------------------------------------------------------- */
void orc_quant_act_f32(const float* x, int32_t T, int32_t H, int8_t* xq, float* xd) {
    int32_t nb = H / 256;
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t b = 0; b < nb; ++b) {
            const float* v = x + (int64_t)t * H + 256 * b;
            int8_t* q = xq + (int64_t)t * H + 256 * b;
            float amax = 0.0f;
            for (int i = 0; i < 256; ++i) {
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            if (amax == 0.0f) {
                xd[(int64_t)t * nb + b] = 0.0f;
                for (int i = 0; i < 256; ++i) q[i] = 0;
                continue;
            }
            float id = 127.0f / amax;
            for (int i = 0; i < 256; ++i) {
                float prod = v[i] * id;
                float r = rintf(prod);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                q[i] = (int8_t)r;
            }
            xd[(int64_t)t * nb + b] = amax / 127.0f;
        }
    }
}

/* The same rule in fp64, applied in place to one vector of n (multiple of
 * 256) values: v <- dequant(quant(v)).  Used for h on the int8 path. */
static void quant_dequant_f64(double* v, int32_t n) {
    for (int32_t b = 0; b < n / 256; ++b) {
        double* u = v + 256 * b;
        double amax = 0.0;
        for (int i = 0; i < 256; ++i)
            if (fabs(u[i]) > amax) amax = fabs(u[i]);
        if (amax == 0.0) {
            for (int i = 0; i < 256; ++i) u[i] = 0.0;
            continue;
        }
        double id = 127.0 / amax, d = amax / 127.0;
        for (int i = 0; i < 256; ++i) {
            double r = rint(u[i] * id);
            if (r > 127.0) r = 127.0;
            if (r < -127.0) r = -127.0;
            u[i] = d * r;
        }
    }
}

/* silu(g) = g / (1 + exp(-g)) (R-ffn).  For very negative g, exp(-g) is +inf
 * and the quotient is -0, so no NaN arises for finite g. */
double orc_silu(double g) { return g / (1.0 + exp(-g)); }

/* ------------------------------------------------------------------------- */
/* Expert FFN for a list of (token, expert) pairs (R-ffn).                   */
/*                                                                           */
/* Weights: three banks, each [n_experts][rows][row_bytes] with stride       */
/* *_expert_bytes between experts: gate and up are [I][H], down is [H][I].   */
/* mode 0 (fp path): x is the token's activation, read from x_f32 [T][H].    */
/* mode 1 (int8 path): the token's activation is dequant(quant_f32(x)),      */
/*   i.e. xd[b]*xq[i] with xq/xd from orc_quant_act_f32 on the token's row,  */
/*   and h is replaced by dequant(quant_f64(h)) per 256-wide block before    */
/*   the down projection (the quantisation points of an int8 down GEMM).     */
/* Output: y [n_pairs][H] fp64.                                              */
/* ------------------------------------------------------------------------- */
void orc_expert_ffn(const uint8_t* gate, const uint8_t* up, const uint8_t* down,
                    int32_t qt_gate, int32_t qt_up, int32_t qt_down,
                    int64_t gate_expert_bytes, int64_t up_expert_bytes, int64_t down_expert_bytes,
                    int32_t H, int32_t I, int32_t n_pairs, const int32_t* pair_expert,
                    const int32_t* pair_token, int32_t mode, const float* x_f32, double* y) {
    int64_t gate_row = (int64_t)(H / blk_weights(qt_gate)) * blk_bytes(qt_gate);
    int64_t up_row = (int64_t)(H / blk_weights(qt_up)) * blk_bytes(qt_up);
    int64_t down_row = (int64_t)(I / blk_weights(qt_down)) * blk_bytes(qt_down);
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    int8_t* xq = (int8_t*)malloc((size_t)H);
    float* xd = (float*)malloc(sizeof(float) * (size_t)(H / 256 + 1));
    for (int32_t p = 0; p < n_pairs; ++p) {
        int64_t e = pair_expert[p], t = pair_token[p];
        if (mode == 1) orc_quant_act_f32(x_f32 + t * H, 1, H, xq, xd);
        for (int32_t c = 0; c < H; ++c) {
            if (mode == 0)
                xv[c] = (double)x_f32[t * H + c];
            else
                xv[c] = (double)xd[c / 256] * (double)xq[c];
        }
        const uint8_t* G = gate + e * gate_expert_bytes;
        const uint8_t* U = up + e * up_expert_bytes;
        const uint8_t* D = down + e * down_expert_bytes;
#pragma omp parallel for schedule(static)
        for (int32_t i = 0; i < I; ++i) {
            double* wr = (double*)malloc(sizeof(double) * (size_t)H);
            double g = 0.0, u = 0.0;
            dequant_row(G + i * gate_row, qt_gate, H, wr);
            for (int32_t c = 0; c < H; ++c) g += wr[c] * xv[c];
            dequant_row(U + i * up_row, qt_up, H, wr);
            for (int32_t c = 0; c < H; ++c) u += wr[c] * xv[c];
            h[i] = orc_silu(g) * u;
            free(wr);
        }
        if (mode == 1) quant_dequant_f64(h, I);
#pragma omp parallel for schedule(static)
        for (int32_t o = 0; o < H; ++o) {
            double* wr = (double*)malloc(sizeof(double) * (size_t)I);
            double acc = 0.0;
            dequant_row(D + o * down_row, qt_down, I, wr);
            for (int32_t i = 0; i < I; ++i) acc += wr[i] * h[i];
            y[(int64_t)p * H + o] = acc;
            free(wr);
        }
    }
    free(xv);
    free(h);
    free(xq);
    free(xd);
}

/* ------------------------------------------------------------------------- */
/* Routing-weighted combine (R-combine).                                     */
/* y_pair [T*k][H] (pair p = t*k + j), w [T][k], y_shared [T][H] or NULL,    */
/* shared_scale [T] or NULL (= 1).  out [T][H].                              */
/* ------------------------------------------------------------------------- */
/* Combine with the layer epilogue (R-epilogue): the shared expert's weight is
 * s_t = shared_scale[t] * gate[t] (each factor 1 when its array is NULL; gate
 * holds the sigmoid values of orc_shared_gate), and the residual stream, when
 * given, is added last:
 *   out_t = sum_j w_tj * y_tj + s_t * y_shared_t + residual_t. */
void orc_combine_ep(const double* y_pair, const double* w, const double* y_shared,
                    const double* shared_scale, const double* gate, const double* residual,
                    int32_t T, int32_t k, int32_t H, double* out) {
    for (int32_t t = 0; t < T; ++t) {
        for (int32_t o = 0; o < H; ++o) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j)
                acc += w[(int64_t)t * k + j] * y_pair[((int64_t)t * k + j) * H + o];
            if (y_shared) {
                double s = (shared_scale ? shared_scale[t] : 1.0) * (gate ? gate[t] : 1.0);
                acc += s * y_shared[(int64_t)t * H + o];
            }
            if (residual) acc += residual[(int64_t)t * H + o];
            out[(int64_t)t * H + o] = acc;
        }
    }
}

void orc_combine(const double* y_pair, const double* w, const double* y_shared,
                 const double* shared_scale, int32_t T, int32_t k, int32_t H, double* out) {
    orc_combine_ep(y_pair, w, y_shared, shared_scale, NULL, NULL, T, k, H, out);
}

/* Sigmoid gate of the shared expert (R-epilogue): one weight vector g [H]
 * per layer, gate_t = 1 / (1 + exp(-(g . x_t))) with the dot a sequential fp64
 * sum over h.  x fp32 [T][H], g fp32 [H] -> out fp64 [T]. */
void orc_shared_gate(const float* x, int32_t T, int32_t H, const float* g, double* out) {
    for (int32_t t = 0; t < T; ++t) {
        double z = 0.0;
        for (int32_t h = 0; h < H; ++h) z += (double)g[h] * (double)x[(int64_t)t * H + h];
        out[t] = 1.0 / (1.0 + exp(-z));
    }
}
