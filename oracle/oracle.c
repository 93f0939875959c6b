/*
 * oracle.c -- plain, slow, scalar fp64 CPU reference for block-sparse
 * attention decoding.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file: it is used by the test-suite, by the smoke check and by
 * the CPU-baseline leg of the benchmark, and by nothing else.  It shares no
 * code, header, table or helper with the GPU library.
 *
 * Every function works on ONE sequence and ONE KV head at a time, on plain
 * contiguous arrays:
 *     K[t*d + i], V[t*d + i]   token t, channel i   (float; the values are the
 *                              exact stored values, e.g. bf16 widened)
 *     q[h*d + i]               query head h of the GQA group, channel i
 * All arithmetic is in double.  Nothing is blocked, fused or reordered beyond
 * what the definitions below state; everything is recomputed from scratch.
 *
 * Sources (page title, then section):
 *  [ReSA]   "Rectified Sparse Attention for Efficient Long-Sequence
 *           Generation" (research.elamur.ai summary page), sections "Summary"
 *           and "Key points".
 *  [SeerR]  "SeerAttention-R: Sparse Attention Adaptation for Long Reasoning"
 *           (mlsanity.com page), section "Abstract (arXiv)".
 *  [SAS]    "Simple Attention Sparsification" (hyper.ai page), section
 *           "Method" (the o_SAS equation, the softmax gates over the
 *           candidate blocks, the unit gate of the current block and the
 *           Top-K discretisation).
 *  [FD]     Flash-Decoding, cited in the [ReSA] page's reference list.
 *
 * Readings the pages leave open are marked READING and are listed, with the
 * reason for each, in the design notes of the repository.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

static int64_t orc_nblocks(int64_t T, int b) { return (T + b - 1) / b; }

/* ------------------------------------------------------------------------ */
/* 1. Block descriptors                                                      */
/* ------------------------------------------------------------------------ */

/* [ReSA] "Summary": each memory block is described Quest-style by the
 * channel-wise minimum and maximum of its keys.  READING: a block covers
 * tokens [j*b, min((j+1)*b, T)); a partial last block uses only the tokens
 * present.  mn, mx: [NB][d]. */
ORC_API void orc_desc_minmax(const float* K, int64_t T, int d, int b,
                             double* mn, double* mx) {
    int64_t NB = orc_nblocks(T, b);
    for (int64_t j = 0; j < NB; ++j) {
        int64_t t0 = j * b;
        int64_t t1 = (j + 1) * (int64_t)b;
        if (t1 > T) t1 = T;
        for (int i = 0; i < d; ++i) {
            double lo = K[t0 * d + i];
            double hi = lo;
            for (int64_t t = t0 + 1; t < t1; ++t) {
                double v = K[t * d + i];
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            mn[j * d + i] = lo;
            mx[j * d + i] = hi;
        }
    }
}

/* [SeerR] "Abstract (arXiv)": the plug-in gate scores blocks from pooled
 * keys, without pooling the query.  READING: the pooled key of a block is the
 * mean of its keys.  mean: [NB][d]. */
ORC_API void orc_desc_mean(const float* K, int64_t T, int d, int b,
                           double* mean) {
    int64_t NB = orc_nblocks(T, b);
    for (int64_t j = 0; j < NB; ++j) {
        int64_t t0 = j * b;
        int64_t t1 = (j + 1) * (int64_t)b;
        if (t1 > T) t1 = T;
        for (int i = 0; i < d; ++i) {
            double s = 0.0;
            for (int64_t t = t0; t < t1; ++t) s += K[t * d + i];
            mean[j * d + i] = s / (double)(t1 - t0);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* 2. Group block scores                                                     */
/* ------------------------------------------------------------------------ */

/* [ReSA] "Summary": min/max descriptors score the blocks, and one block
 * selection is shared by all query heads of a GQA group.  READING: the score
 * of block j for head h is sum_i max(q_hi*mn_ji, q_hi*mx_ji) -- the largest
 * value q_h.k can take for any k inside the block's channel-wise box -- and
 * the group score is the sum over the G heads of the group.  s: [nblk]. */
ORC_API void orc_score_quest(const float* q, int G, int d, const double* mn,
                             const double* mx, int64_t nblk, double* s) {
    for (int64_t j = 0; j < nblk; ++j) {
        double acc = 0.0;
        for (int h = 0; h < G; ++h) {
            for (int i = 0; i < d; ++i) {
                double a = (double)q[h * d + i] * mn[j * d + i];
                double c = (double)q[h * d + i] * mx[j * d + i];
                acc += (a > c) ? a : c;
            }
        }
        s[j] = acc;
    }
}

/* [SeerR] "Abstract (arXiv)": a lightweight linear plug-in gate over pooled
 * keys; [SAS] "Method": s = R_theta(q, {K_B}).  READING: one linear map
 * W [d][d] (row r = output channel r) applied to the sum of the group's query
 * heads, dotted with the block's mean key:
 *     u = sum_h q_h;  w = W u;  s_j = w . mean_j.   s: [nblk]. */
ORC_API void orc_score_gate(const float* q, int G, int d, const float* W,
                            const double* mean, int64_t nblk, double* s) {
    double* u = (double*)malloc(sizeof(double) * (size_t)d);
    double* w = (double*)malloc(sizeof(double) * (size_t)d);
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int h = 0; h < G; ++h) acc += q[h * d + i];
        u[i] = acc;
    }
    for (int r = 0; r < d; ++r) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += (double)W[r * d + i] * u[i];
        w[r] = acc;
    }
    for (int64_t j = 0; j < nblk; ++j) {
        double acc = 0.0;
        for (int r = 0; r < d; ++r) acc += w[r] * mean[j * d + r];
        s[j] = acc;
    }
    free(u);
    free(w);
}

/* ------------------------------------------------------------------------ */
/* 3. How many blocks to keep                                                */
/* ------------------------------------------------------------------------ */

/* [ReSA] "Key points": a dynamic top-n that always keeps the recent local
 * blocks and never keeps fewer than a minimum count; the kept set is sized by
 * the sparsity p (ablated at 0.9/0.95/0.98).  [SeerR] "Abstract (arXiv)":
 * the kept set may instead be given as a token budget (4K tokens).
 * READING: p is the fraction SKIPPED, given in basis points so that no
 * floating point enters the count; local blocks count towards n:
 *     n_req = budget / b                     (budget_tokens > 0)
 *           = ceil((10000 - bp) * NB / 10000) (otherwise)
 *     n     = min(NB, max(n_req, n_min, min(n_local, NB))). */
ORC_API int64_t orc_block_count(int64_t NB, int b, int64_t budget_tokens,
                                int sparsity_bp, int n_local, int n_min) {
    int64_t n_req;
    if (budget_tokens > 0)
        n_req = budget_tokens / b;
    else
        n_req = ((int64_t)(10000 - sparsity_bp) * NB + 9999) / 10000;
    int64_t nl = (n_local < NB) ? n_local : NB;
    int64_t n = n_req;
    if (n_min > n) n = n_min;
    if (nl > n) n = nl;
    if (n > NB) n = NB;
    return n;
}

/* ------------------------------------------------------------------------ */
/* 4. Top-n selection                                                        */
/* ------------------------------------------------------------------------ */

/* [ReSA] "Key points" (recent local blocks always kept); [SAS] "Method"
 * (the current block is always retained; at inference the ranking is cut to
 * discrete Top-K block indices).  The last min(n_local, NB) blocks are kept;
 * the other n - n_local' are taken from the candidates 0..NB-n_local'-1 by
 * repeated arg-max under the order (score descending, index ascending).
 * READING: ties go to the lower index; the result is emitted ascending and
 * padded with -1 up to idx_cap.  Returns the number of kept blocks. */
ORC_API int64_t orc_select(const double* s, int64_t NB, int64_t n,
                           int n_local, int32_t* idx, int64_t idx_cap) {
    int64_t nl = (n_local < NB) ? n_local : NB;
    int64_t nc = NB - nl;
    unsigned char* keep = (unsigned char*)calloc((size_t)(NB > 0 ? NB : 1), 1);
    for (int64_t j = nc; j < NB; ++j) keep[j] = 1;
    for (int64_t pick = 0; pick < n - nl; ++pick) {
        int64_t best = -1;
        for (int64_t j = 0; j < nc; ++j) {
            if (keep[j]) continue;
            if (best < 0 || s[j] > s[best]) best = j; /* '>' keeps lower index on ties */
        }
        if (best < 0) break;
        keep[best] = 1;
    }
    int64_t c = 0;
    for (int64_t j = 0; j < NB; ++j)
        if (keep[j]) idx[c++] = (int32_t)j;
    for (int64_t k = c; k < idx_cap; ++k) idx[k] = -1;
    free(keep);
    return c;
}

/* ------------------------------------------------------------------------ */
/* 5. Exact softmax attention over the kept blocks                           */
/* ------------------------------------------------------------------------ */

/* [ReSA] "Summary" (attention over the selected blocks only); [SAS]
 * "Method" (non-selected blocks are masked out of an exact softmax).  For a
 * single query head q [d]: the attended tokens are the union of
 * [j*b, min((j+1)*b, T)) over the kept blocks j; two passes:
 *     z_t = scale * q.K_t,  m = max z,  l = sum exp(z_t - m),
 *     o = sum exp(z_t - m) V_t / l,  lse = m + ln l   (natural log).
 * o: [d]. */
ORC_API void orc_attend(const float* q, const float* K, const float* V,
                        int64_t T, int d, int b, const int32_t* idx,
                        int64_t nidx, double scale, double* o, double* lse) {
    double m = -INFINITY;
    for (int64_t k = 0; k < nidx; ++k) {
        int64_t t0 = (int64_t)idx[k] * b;
        int64_t t1 = t0 + b;
        if (t1 > T) t1 = T;
        for (int64_t t = t0; t < t1; ++t) {
            double z = 0.0;
            for (int i = 0; i < d; ++i) z += (double)q[i] * K[t * d + i];
            z *= scale;
            if (z > m) m = z;
        }
    }
    double l = 0.0;
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    for (int64_t k = 0; k < nidx; ++k) {
        int64_t t0 = (int64_t)idx[k] * b;
        int64_t t1 = t0 + b;
        if (t1 > T) t1 = T;
        for (int64_t t = t0; t < t1; ++t) {
            double z = 0.0;
            for (int i = 0; i < d; ++i) z += (double)q[i] * K[t * d + i];
            z *= scale;
            double p = exp(z - m);
            l += p;
            for (int i = 0; i < d; ++i) o[i] += p * V[t * d + i];
        }
    }
    for (int i = 0; i < d; ++i) o[i] /= l;
    *lse = m + log(l);
}

/* Dense softmax attention of one query head over tokens [0, n_tok): the
 * textbook definition, written separately from orc_attend so that the two
 * can be checked against each other. */
ORC_API void orc_dense_attend(const float* q, const float* K, const float* V,
                              int64_t n_tok, int d, double scale, double* o,
                              double* lse) {
    double* z = (double*)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1));
    double m = -INFINITY;
    for (int64_t t = 0; t < n_tok; ++t) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += (double)q[i] * K[t * d + i];
        z[t] = scale * acc;
        if (z[t] > m) m = z[t];
    }
    /* z is overwritten by the weights exp(z_t - m); every sum below still
     * runs over t in order, so o and lse are those of the per-channel form
     * sum_t exp(z_t - m) V[t][i], value for value */
    double l = 0.0;
    for (int64_t t = 0; t < n_tok; ++t) {
        z[t] = exp(z[t] - m);
        l += z[t];
    }
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    for (int64_t t = 0; t < n_tok; ++t)
        for (int i = 0; i < d; ++i) o[i] += z[t] * V[t * d + i];
    for (int i = 0; i < d; ++i) o[i] /= l;
    *lse = m + log(l);
    free(z);
}

/* ------------------------------------------------------------------------ */
/* 6. Rectification                                                          */
/* ------------------------------------------------------------------------ */

/* [ReSA] "Summary": after every f generated tokens those tokens are
 * re-encoded in one dense parallel pass whose keys/values overwrite their
 * cache entries (and, through them, the block descriptors, which this oracle
 * always recomputes from scratch).  READING: the caller supplies the
 * re-encoded k_new/v_new [f][d]; the order is overwrite, then causal dense
 * attention of query i (position T-f+i) over tokens 0..T-f+i.
 * K, V [T][d] are modified in place.  q: [G][f][d]; o: [G][f][d];
 * lse: [G][f]. */
ORC_API void orc_rectify(const float* q, int G, int f, float* K, float* V,
                         int64_t T, int d, const float* k_new,
                         const float* v_new, double scale, double* o,
                         double* lse) {
    for (int i = 0; i < f; ++i) {
        for (int c = 0; c < d; ++c) {
            K[(T - f + i) * d + c] = k_new[i * d + c];
            V[(T - f + i) * d + c] = v_new[i * d + c];
        }
    }
    for (int h = 0; h < G; ++h) {
        for (int i = 0; i < f; ++i) {
            orc_dense_attend(q + ((int64_t)h * f + i) * d, K, V, T - f + i + 1,
                             d, scale, o + ((int64_t)h * f + i) * d,
                             lse + (int64_t)h * f + i);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* 7. One whole sparse decode step for one (sequence, KV head) group        */
/* ------------------------------------------------------------------------ */

/* The plain definition of a decode step after the new token has been
 * appended (the query attends to its own token): rebuild all descriptors,
 * score the candidate blocks, count, select, attend for each of the G query
 * heads.  desc_kind 0 = min/max (Quest), 1 = mean-pooled keys with gate W.
 * idx: [idx_cap]; returns the kept count.  o: [G][d]; lse: [G];
 * scores (optional, may be NULL): [NB] with the candidates' scores (the local
 * blocks' entries are left as NaN). */
ORC_API int64_t orc_decode_group(const float* q, int G, const float* K,
                                 const float* V, int64_t T, int d, int b,
                                 int desc_kind, const float* W,
                                 int64_t budget_tokens, int sparsity_bp,
                                 int n_local, int n_min, double scale,
                                 int32_t* idx, int64_t idx_cap, double* o,
                                 double* lse, double* scores) {
    int64_t NB = orc_nblocks(T, b);
    int64_t nl = (n_local < NB) ? n_local : NB;
    double* s = (double*)malloc(sizeof(double) * (size_t)NB);
    for (int64_t j = 0; j < NB; ++j) s[j] = NAN;
    if (desc_kind == 0) {
        double* mn = (double*)malloc(sizeof(double) * (size_t)(NB * d));
        double* mx = (double*)malloc(sizeof(double) * (size_t)(NB * d));
        orc_desc_minmax(K, T, d, b, mn, mx);
        orc_score_quest(q, G, d, mn, mx, NB - nl, s);
        free(mn);
        free(mx);
    } else {
        double* mean = (double*)malloc(sizeof(double) * (size_t)(NB * d));
        orc_desc_mean(K, T, d, b, mean);
        orc_score_gate(q, G, d, W, mean, NB - nl, s);
        free(mean);
    }
    int64_t n = orc_block_count(NB, b, budget_tokens, sparsity_bp, n_local, n_min);
    int64_t cnt = orc_select(s, NB, n, n_local, idx, idx_cap);
    for (int h = 0; h < G; ++h)
        orc_attend(q + (int64_t)h * d, K, V, T, d, b, idx, cnt, scale,
                   o + (int64_t)h * d, lse + h);
    if (scores) memcpy(scores, s, sizeof(double) * (size_t)NB);
    free(s);
    return cnt;
}

/* ------------------------------------------------------------------------ */
/* 8. Log-gate bias of the selected blocks (SAS)                            */
/* ------------------------------------------------------------------------ */

/* [SAS] "Method": the context is split into one always-retained current
 * block B_0, whose gate stays g_0 = 1, and C historical blocks, whose
 * selector scores s become normalised gates g = softmax(s) over all C of
 * them; the logits of a selected historical block's tokens get log g added
 * inside the softmax.
 * READING: g = softmax(tau * s) with tau > 0 (tau = 1 is the page's form;
 * the scores here are the method's block scores, not a trained selector's
 * logits, so their scale is left to the caller).  n_current trailing blocks
 * keep the unit gate: 1 is the page's B_0 (every other block, a kept local
 * one included, is historical: it is scored, enters the normaliser and gets
 * its log-gate), n_current = n_local treats every local block as current.
 * s: [NB] with blocks 0..NB-n_current-1 scored; idx/cnt: a selection as
 * orc_select returns it; bias: [cnt], log g of each selected block. */
ORC_API void orc_gate_bias(const double* s, int64_t NB, int n_current, double tau,
                           const int32_t* idx, int64_t cnt, double* bias) {
    int64_t nu = (n_current < NB) ? n_current : NB;
    int64_t nc = NB - nu;
    /* log sum_c exp(tau s_c), with the largest term factored out */
    double m = -INFINITY;
    for (int64_t c = 0; c < nc; ++c)
        if (tau * s[c] > m) m = tau * s[c];
    double z = 0.0;
    for (int64_t c = 0; c < nc; ++c) z += exp(tau * s[c] - m);
    double log_norm = m + log(z);
    for (int64_t k = 0; k < cnt; ++k) {
        int64_t j = idx[k];
        bias[k] = (j >= nc) ? 0.0 : tau * s[j] - log_norm;
    }
}

/* [SAS] "Method", the o_SAS equation: softmax over the selected blocks'
 * tokens of z_t + bias(block of t), z_t = scale q.k_t; two passes, exact.
 * bias: [nidx], the additive logit bias of each selected block. */
ORC_API void orc_attend_biased(const float* q, const float* K, const float* V,
                               int64_t T, int d, int b, const int32_t* idx,
                               int64_t nidx, const double* bias, double scale,
                               double* o, double* lse) {
    double m = -INFINITY;
    for (int64_t k = 0; k < nidx; ++k) {
        int64_t t0 = (int64_t)idx[k] * b;
        int64_t t1 = t0 + b;
        if (t1 > T) t1 = T;
        for (int64_t t = t0; t < t1; ++t) {
            double z = 0.0;
            for (int i = 0; i < d; ++i) z += (double)q[i] * K[t * d + i];
            z = z * scale + bias[k];
            if (z > m) m = z;
        }
    }
    double l = 0.0;
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    for (int64_t k = 0; k < nidx; ++k) {
        int64_t t0 = (int64_t)idx[k] * b;
        int64_t t1 = t0 + b;
        if (t1 > T) t1 = T;
        for (int64_t t = t0; t < t1; ++t) {
            double z = 0.0;
            for (int i = 0; i < d; ++i) z += (double)q[i] * K[t * d + i];
            z = z * scale + bias[k];
            double p = exp(z - m);
            l += p;
            for (int i = 0; i < d; ++i) o[i] += p * V[t * d + i];
        }
    }
    for (int i = 0; i < d; ++i) o[i] /= l;
    *lse = m + log(l);
}

/* A whole decode step with the SAS log-gate bias: orc_decode_group's
 * descriptors, scores, count and selection, then the scores of every
 * historical block (all but the n_current trailing ones, see orc_gate_bias)
 * and the biased attention.
 * bias (optional, may be NULL): [idx_cap] receives log g of each selected
 * block. */
ORC_API int64_t orc_decode_group_gated(const float* q, int G, const float* K,
                                       const float* V, int64_t T, int d, int b,
                                       int desc_kind, const float* W,
                                       int64_t budget_tokens, int sparsity_bp,
                                       int n_local, int n_min, int n_current,
                                       double scale, double tau, int32_t* idx,
                                       int64_t idx_cap, double* o, double* lse,
                                       double* bias) {
    int64_t NB = orc_nblocks(T, b);
    double* s = (double*)malloc(sizeof(double) * (size_t)(NB > 0 ? NB : 1));
    double* o0 = (double*)malloc(sizeof(double) * (size_t)G * d);
    double* l0 = (double*)malloc(sizeof(double) * (size_t)G);
    int64_t cnt = orc_decode_group(q, G, K, V, T, d, b, desc_kind, W, budget_tokens,
                                   sparsity_bp, n_local, n_min, scale, idx, idx_cap,
                                   o0, l0, s);
    /* the historical blocks' scores (the candidates' and those of the kept
     * local blocks before the current ones), same definition as the
     * selection's */
    int64_t nu = (n_current < NB) ? n_current : NB;
    if (desc_kind == 0) {
        double* mn = (double*)malloc(sizeof(double) * (size_t)((NB > 0 ? NB : 1) * d));
        double* mx = (double*)malloc(sizeof(double) * (size_t)((NB > 0 ? NB : 1) * d));
        orc_desc_minmax(K, T, d, b, mn, mx);
        orc_score_quest(q, G, d, mn, mx, NB - nu, s);
        free(mn);
        free(mx);
    } else {
        double* mean = (double*)malloc(sizeof(double) * (size_t)((NB > 0 ? NB : 1) * d));
        orc_desc_mean(K, T, d, b, mean);
        orc_score_gate(q, G, d, W, mean, NB - nu, s);
        free(mean);
    }
    double* g = (double*)malloc(sizeof(double) * (size_t)(cnt > 0 ? cnt : 1));
    orc_gate_bias(s, NB, (int)nu, tau, idx, cnt, g);
    for (int h = 0; h < G; ++h)
        orc_attend_biased(q + (int64_t)h * d, K, V, T, d, b, idx, cnt, g, scale,
                          o + (int64_t)h * d, lse + h);
    if (bias)
        for (int64_t k = 0; k < cnt; ++k) bias[k] = g[k];
    free(g);
    free(l0);
    free(o0);
    free(s);
    return cnt;
}
