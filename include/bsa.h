/*
 * bsa.h -- C ABI of the block-sparse attention decoding library (libbsa.so,
 * HIP kernels for AMD gfx950 / MI355X).
 *
 * The method (sources cited per entry point below):
 *   * every block of b consecutive cached tokens carries a key descriptor --
 *     the channel-wise min and max of its keys (Quest style) or the sum of its
 *     keys (mean pooling for a linear plug-in gate);
 *   * the descriptors are scored against the current query, one score per
 *     block for a whole GQA group of query heads;
 *   * a dynamic top-n keeps the recent local blocks, a minimum count, and the
 *     best-scoring remaining blocks;
 *   * exact softmax attention runs over the kept blocks only (split over the
 *     kept tokens, partial results merged by log-sum-exp);
 *   * every f generated tokens, rectification overwrites the last f tokens'
 *     keys/values with re-encoded ones, refreshes the affected descriptors and
 *     runs causal dense attention of those f queries over the whole cache.
 *
 * Sources: "Rectified Sparse Attention for Efficient Long-Sequence
 * Generation" (research.elamur.ai summary), sections "Summary" and "Key
 * points"; "SeerAttention-R: Sparse Attention Adaptation for Long Reasoning"
 * (mlsanity.com), section "Abstract (arXiv)"; "Simple Attention
 * Sparsification" (hyper.ai), section "Method"; Flash-Decoding and
 * PagedAttention as cited in the ReSA page's reference list.
 *
 * ---------------------------------------------------------------------------
 * General contract (all entry points)
 * ---------------------------------------------------------------------------
 * Ownership.  The caller allocates every buffer (device memory unless stated):
 *   pools, page table, sequence lengths, descriptors, selection lists,
 *   outputs and workspace.  The library allocates nothing, frees nothing and
 *   keeps no state between calls (the one exception is the per-GPU scratch
 *   array of bsa_sparse_decode_static, a device variable of fixed size that
 *   the library's code object holds).  Pointers must stay valid until the
 *   work enqueued on `stream` has completed.
 * Streams.  Every call validates its arguments on the host, enqueues kernels
 *   on `stream` (0 = the null stream) and returns.  The library never
 *   synchronises.  Calls on one cache must be ordered by the caller (the
 *   usual way: one stream).
 * Errors.  Argument checks run before any HIP call; a failed check returns
 *   its status and enqueues nothing.  BSA_ERR_HIP reports a launch error
 *   (hipGetLastError after the launches).  Device-side contracts (listed per
 *   call, e.g. seq_lens[b] <= max_blocks*block, page ids < num_pages) are not
 *   checked on the device; breaking them is undefined behaviour.
 * Checked build.  libbsa_checked.so exports the same entry points, built with
 *   BSA_CHECKED=1.  Each call first drains `stream`, copies the device values
 *   its contracts bound to the host and returns BSA_ERR_CONTRACT, enqueuing
 *   nothing, if one of these is broken:
 *     every call:   0 <= seq_lens[s] <= max_blocks*block, and every block
 *                   holding tokens has a page id >= 0 (the pool size is the
 *                   caller's, so the upper bound is not checked);
 *     append:       seq_lens[s] >= n_new (bsa_append_select and
 *                   bsa_append_select_decode: >= 1);
 *     decode:       0 <= cnt <= n_max, the first cnt ids of each idx row are
 *                   distinct and below ceil(seq_lens[s] / block), and their
 *                   gate biases (gated call) are finite;
 *     rectify:      seq_lens[s] >= f.
 *   A failed copy returns BSA_ERR_HIP.  The checked build synchronises on
 *   every call: it is for debugging and cannot be captured into a graph.
 * Numbers.  q and o use the KV dtype; lse is fp32, the natural log of the sum
 *   over attended tokens of exp(softmax_scale * q.k); accumulation is fp32.
 *
 * ---------------------------------------------------------------------------
 * Memory layout
 * ---------------------------------------------------------------------------
 * Pages.  One page holds one block: b tokens of one KV head.  The pools are
 *   k_pool, v_pool: [num_pages][Hkv][b*d] elements of the KV dtype.
 *   Logical block j of sequence s lives in page page_table[s*max_blocks + j].
 *   Inside a page (b*d elements) token t (0 <= t < b), channel i sits at
 *     fp32 K and V:  t*d + i                      (row major)
 *     bf16 K:        ((t/16)*(d/32) + i/32)*512 + ((t%16) + 16*((i%32)/8))*8 + i%8
 *     bf16 V:        ((t/32)*(d/16) + i/16)*512 + ((i%16) + 16*g)*8 + e
 *                    where u = t%32, g = (u%16)/4, e = (u%4) + 4*(u/16)
 *   The bf16 orders make every 1 KiB of a page exactly one 64-lane operand of
 *   the gfx950 bf16 matrix instructions, so the attention kernels read pages
 *   with fully coalesced 16-byte loads.  Tokens [32r, 32r+32) of a page are
 *   one contiguous 32*d run in both K and V.  bsa_build_block_desc writes
 *   pages in this order from row-major [tokens][d] input; callers never need
 *   to compute it themselves.
 * Descriptors.  desc is indexed by LOGICAL block:
 *   MINMAX:   [B][Hkv][max_blocks][2][d] in the KV dtype (min row, then max
 *             row; min/max of stored values is exact in that dtype);
 *   MEANPOOL: [B][Hkv][max_blocks][d] fp32 running SUM of the block's keys in
 *             token order (the mean is sum / tokens-in-block).
 * Sequence lengths.  seq_lens[B] (int32, device) is the number of tokens in
 *   each sequence's cache INCLUDING any tokens being appended by the current
 *   call; the caller advances it (the library only reads it).
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef BSA_API
#define BSA_API __attribute__((visibility("default")))
#endif

typedef enum bsa_status {
    BSA_OK = 0,
    BSA_ERR_NULL = 1,        /* a required pointer is NULL */
    BSA_ERR_SHAPE = 2,       /* B/Hq/Hkv/d/block/max_blocks inconsistent */
    BSA_ERR_UNSUPPORTED = 3, /* dtype, d, block or descriptor kind not built */
    BSA_ERR_PARAM = 4,       /* selection / rectify parameter out of range */
    BSA_ERR_WORKSPACE = 5,   /* ws too small (see bsa_workspace_size) */
    BSA_ERR_HIP = 6,         /* a kernel launch failed */
    BSA_ERR_CONTRACT = 7     /* checked build only: a device-side input breaks
                                its contract (see "Checked build" above) */
} bsa_status;

typedef enum bsa_dtype { BSA_DTYPE_F32 = 0, BSA_DTYPE_BF16 = 1 } bsa_dtype;

typedef enum bsa_desc_kind {
    BSA_DESC_MINMAX = 0,   /* channel-wise min/max (Quest) */
    BSA_DESC_MEANPOOL = 1  /* key sum -> mean, scored through a gate W */
} bsa_desc_kind;

typedef enum bsa_op {
    BSA_OP_SELECT = 1,
    BSA_OP_DECODE = 2,
    BSA_OP_RECTIFY = 3,
    BSA_OP_STEP = 4     /* bsa_append_select_decode, by n_max */
} bsa_op;

/* Problem shape.  Supported: 1 <= Hq/Hkv <= 16 with Hq % Hkv == 0;
 * d in {64, 128}; block in {32, 64, 128, 256}; 1 <= max_blocks <= 32768. */
typedef struct bsa_layout {
    int32_t B;           /* sequences in the batch */
    int32_t Hq;          /* query heads */
    int32_t Hkv;         /* KV heads; query head h uses KV head h / (Hq/Hkv) */
    int32_t d;           /* head dimension */
    int32_t block;       /* b: tokens per block == tokens per page */
    int32_t max_blocks;  /* page-table row length (capacity per sequence) */
    int32_t kv_dtype;    /* bsa_dtype */
    int32_t desc_kind;   /* bsa_desc_kind */
} bsa_layout;

/* The paged cache.  All pointers are device pointers. */
typedef struct bsa_cache {
    void* k_pool;               /* [num_pages][Hkv][block*d] */
    void* v_pool;               /* [num_pages][Hkv][block*d] */
    const int32_t* page_table;  /* [B][max_blocks] physical page ids */
    const int32_t* seq_lens;    /* [B] tokens in each sequence */
    void* desc;                 /* descriptors, see the layout notes above */
} bsa_cache;

/* Selection parameters ("Rectified Sparse Attention ...", Key points: dynamic
 * top-n with recent local blocks and a minimum count; "SeerAttention-R ...",
 * Abstract: token budget).  With NB = ceil(T/b) blocks in a sequence:
 *   n_req = budget_tokens / b                         if budget_tokens > 0
 *         = ceil((10000 - sparsity_bp) * NB / 10000)  otherwise
 *   n     = min(NB, max(n_req, n_min, min(n_local, NB)))
 * The last min(n_local, NB) blocks are always kept; the rest of the n are
 * the best-scoring other blocks, ties to the lower block index.
 *
 * Log-gate bias ("Simple Attention Sparsification", Method: the context is
 * one always-retained current block, whose gate is 1, and historical
 * blocks, whose gates are a softmax over all their scores; log g is added to
 * a kept block's logits).  The last gate_current blocks are current (1, the
 * page's single current block, when gate_current is 0 or 1; at most
 * n_local); every other block is historical and is scored, a kept local one
 * included.  When gate_bias is set, the selecting call also writes, at the
 * position of each kept block j in idx,
 *   bias = log softmax(gate_tau * s)_j  over ALL H = NB - gate_current
 *          historical blocks,
 * 0 for a current block and 0 for the -1 padding; computed in fp32 from the
 * fp32 scores as gate_tau * (s_j - max s) - ln sum_h exp(gate_tau * (s_h -
 * max s)).  bsa_sparse_decode_gated consumes it.  The selection itself
 * (which blocks are kept) does not depend on the gate settings. */
typedef struct bsa_select_params {
    int32_t budget_tokens;  /* >= 0; 0 selects the sparsity rule */
    int32_t sparsity_bp;    /* p (fraction skipped) in basis points, [0, 10000) */
    int32_t n_local;        /* >= 1: the current (possibly partial) block is local */
    int32_t n_min;          /* >= 0 */
    int32_t n_max;          /* row length of idx; must be >= n for NB = max_blocks */
    const void* gate_w;     /* MEANPOOL only: W [d][d] bf16, row r = output
                               channel r; NULL for MINMAX */
    float gate_tau;         /* >= 0, finite; read only when gate_bias is set */
    float* gate_bias;       /* NULL, or device fp32 [B][Hkv][n_max], OUT: the
                               log-gate bias of each entry of idx (below) */
    int32_t gate_current;   /* read only when gate_bias is set: trailing
                               blocks with the unit gate, 0..n_local (0 = 1) */
} bsa_select_params;

/* ---------------------------------------------------------------------------
 * bsa_build_block_desc -- write tokens into the paged cache and maintain the
 * block descriptors ("Rectified Sparse Attention ...", Summary: Quest-style
 * min/max block descriptors; "SeerAttention-R ...", Abstract: pooled keys
 * for a plug-in gate; PagedAttention for the page table).
 *
 * Append mode (k_new and v_new non-NULL): k_new, v_new are row-major
 *   [B][Hkv][n_new][d] in the KV dtype.  Token i of sequence s goes to
 *   position seq_lens[s] - n_new + i (the caller has already advanced
 *   seq_lens).  Descriptors of every block these positions touch are updated:
 *   a block first opened by this call is initialised from the new tokens, a
 *   block opened earlier is merged with them (min/max, or the running key sum
 *   in token order).  n_new = 1 is the per-step decode append; n_new = T is a
 *   prefill.  range_begin must be NULL.
 * Rebuild mode (k_new == v_new == NULL): descriptors of every block that
 *   overlaps [range_begin[s], seq_lens[s]) are recomputed from scratch from
 *   the cache contents.  range_begin: device int32 [B], or NULL for 0.
 *   n_new is ignored.
 * Device contract: n_new <= seq_lens[s] <= max_blocks*block.
 * Errors: BSA_ERR_NULL, BSA_ERR_SHAPE, BSA_ERR_UNSUPPORTED, BSA_ERR_PARAM
 *   (n_new < 1 in append mode, or only one of k_new/v_new given),
 *   BSA_ERR_HIP.
 * ------------------------------------------------------------------------- */
BSA_API bsa_status bsa_build_block_desc(const bsa_layout* layout, const bsa_cache* cache,
                                const void* k_new, const void* v_new,
                                int32_t n_new, const int32_t* range_begin,
                                hipStream_t stream);

/* ---------------------------------------------------------------------------
 * bsa_select_blocks -- score every non-local block of every (sequence, KV
 * head) group against the group's query heads and keep the top-n
 * ("Rectified Sparse Attention ...", Summary: min/max descriptors score the
 * blocks, one selection per GQA group; Key points: dynamic top-n;
 * "Simple Attention Sparsification", Method: the current block is always
 * retained and inference keeps discrete Top-K block indices).
 *
 * Scores, per group (sequence s, KV head k, heads h of the group):
 *   MINMAX:   s_j = sum_h sum_i max(q_hi * min_ji, q_hi * max_ji)
 *   MEANPOOL: s_j = (W (sum_h q_h)) . (sum_j / tokens_j)
 * computed in fp32.
 * q: [B][Hq][d] in the KV dtype.
 * idx: [B][Hkv][n_max] int32, OUT: kept block ids ascending, padded with -1.
 * cnt: [B][Hkv] int32, OUT: n.  An empty sequence (seq_lens[s] = 0) has no
 *   block: cnt = 0 and its idx rows are all -1.
 * ws: workspace of at least bsa_workspace_size(layout, BSA_OP_SELECT, n_max)
 *   bytes (holds the scores; contents need no initialisation).
 * gate_bias (optional): see bsa_select_params.
 * Errors: BSA_ERR_NULL, BSA_ERR_SHAPE, BSA_ERR_UNSUPPORTED, BSA_ERR_PARAM
 *   (n_local < 1, n_min < 0, budget_tokens < 0, sparsity_bp outside
 *   [0, 10000), n_max too small, gate_w missing for MEANPOOL, gate_tau
 *   negative or not finite or gate_current outside [0, n_local] while
 *   gate_bias is set),
 *   BSA_ERR_WORKSPACE, BSA_ERR_HIP.
 * ------------------------------------------------------------------------- */
BSA_API bsa_status bsa_select_blocks(const bsa_layout* layout, const bsa_cache* cache,
                             const void* q, const bsa_select_params* params,
                             int32_t* idx, int32_t* cnt, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * bsa_append_select -- the per-step pair bsa_build_block_desc (append mode,
 * one token per sequence) then bsa_select_blocks, in two kernel launches
 * instead of three: the new token lands in the last block, which is local
 * and never scored, so writing it and scoring the other blocks run side by
 * side in one launch.  Same references as the two calls it stands for.
 * Results are identical to the two calls made in that order.
 * k_new, v_new: [B][Hkv][1][d] in the KV dtype (the caller has already
 *   advanced seq_lens by one).  Other arguments as in bsa_select_blocks.
 * Errors: those of both calls.
 * ------------------------------------------------------------------------- */
BSA_API bsa_status bsa_append_select(const bsa_layout* layout, const bsa_cache* cache,
                             const void* k_new, const void* v_new, const void* q,
                             const bsa_select_params* params, int32_t* idx,
                             int32_t* cnt, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * bsa_sparse_decode -- exact softmax attention of each query head over the
 * tokens of its group's kept blocks ("Rectified Sparse Attention ...",
 * Summary: group block-sparse attention; "Simple Attention Sparsification",
 * Method: non-selected blocks masked, online softmax; Flash-Decoding: split
 * over the keys, partials merged by log-sum-exp).
 *   o_h = sum_t exp(z_t - lse_h) v_t,  z_t = softmax_scale * q_h . k_t,
 *   lse_h = ln sum_t exp(z_t), t over the kept blocks' tokens (< seq_lens).
 * q: [B][Hq][d]; idx/cnt: as written by bsa_select_blocks with row length
 * n_max (any ascending or not, duplicate-free list of valid block ids works).
 * o: [B][Hq][d] in the KV dtype, OUT.  lse: [B][Hq] fp32, OUT.  A group with
 *   cnt = 0 (e.g. an empty sequence) attends to nothing: o = 0, lse = -inf.
 * ws: at least bsa_workspace_size(layout, BSA_OP_DECODE, n_max) bytes.
 * Errors: BSA_ERR_NULL, BSA_ERR_SHAPE, BSA_ERR_UNSUPPORTED, BSA_ERR_PARAM
 *   (n_max < 1, softmax_scale not finite and > 0), BSA_ERR_WORKSPACE,
 *   BSA_ERR_HIP.
 * ------------------------------------------------------------------------- */
BSA_API bsa_status bsa_sparse_decode(const bsa_layout* layout, const bsa_cache* cache,
                             const void* q, const int32_t* idx,
                             const int32_t* cnt, int32_t n_max,
                             float softmax_scale, void* o, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * bsa_append_select_decode -- one whole decode step of one layer:
 * bsa_append_select (append one token per sequence, score, keep the top-n)
 * then bsa_sparse_decode over the kept blocks (with
 * bsa_sparse_decode_gated's log-gate bias when params->gate_bias is set).
 * Same references as those calls ("Rectified Sparse Attention ...",
 * Summary and Key points; "Simple Attention Sparsification", Method).
 * Results (the cache, idx, cnt, gate_bias, o, lse) are identical to those
 * calls made in that order with the same arguments.  For bf16 caches whose
 * rows hold at most 8192 candidate blocks (max_blocks - n_local <= 8192),
 * with n_max <= 4096 and no gate_bias, the selection runs inside the decode
 * launch: every decode workgroup selects its group's kept blocks from the
 * scores, which saves the top-n launch and a dependent round trip; other
 * cases make the four launches of the two calls.
 * k_new, v_new: [B][Hkv][1][d]; q: [B][Hq][d] (KV dtype; the caller has
 *   already advanced seq_lens by one).  idx, cnt: OUT, as bsa_select_blocks
 *   writes them (row length params->n_max).  o, lse: OUT, as
 *   bsa_sparse_decode.
 * ws: at least bsa_workspace_size(layout, BSA_OP_STEP, params->n_max) bytes
 *   (the scores, then the decode's split partials; no initialisation).
 * Errors: those of bsa_append_select and bsa_sparse_decode.
 * ------------------------------------------------------------------------- */
BSA_API bsa_status bsa_append_select_decode(const bsa_layout* layout,
                             const bsa_cache* cache, const void* k_new,
                             const void* v_new, const void* q,
                             const bsa_select_params* params, int32_t* idx,
                             int32_t* cnt, float softmax_scale, void* o,
                             float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * bsa_sparse_decode_gated -- bsa_sparse_decode with an additive logit bias
 * per kept block ("Simple Attention Sparsification", Method: the o_SAS
 * equation, softmax(q K_S^T + log g_S) V_S over the kept blocks S):
 *   z_t = softmax_scale * q_h . k_t + gate_bias[k]   for t in block idx[k],
 * o_h and lse_h as in bsa_sparse_decode over these z_t.
 * gate_bias: device fp32 [B][Hkv][n_max], the row layout of idx; entry k
 *   biases every token of block idx[k] (as written by a selecting call with
 *   bsa_select_params.gate_bias set; any finite values work).  Entries at
 *   positions >= cnt are not read.
 * Other arguments, workspace and errors as in bsa_sparse_decode
 *   (BSA_ERR_NULL also for a NULL gate_bias).
 * ------------------------------------------------------------------------- */
BSA_API bsa_status bsa_sparse_decode_gated(const bsa_layout* layout,
                             const bsa_cache* cache, const void* q,
                             const int32_t* idx, const int32_t* cnt,
                             const float* gate_bias, int32_t n_max,
                             float softmax_scale, void* o, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * bsa_sparse_decode_static -- bsa_sparse_decode without a workspace
 * argument, for callers that cannot allocate device memory around the call
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The split partials go to a scratch array of
 * BSA_STATIC_SCRATCH_BYTES that the library holds in a file-scope device
 * variable: one copy per GPU, kept until the process ends.  The call
 * allocates nothing and frees nothing; on its first use on a device (with
 * that device current) it looks up the device address of that device's
 * copy once.  `stream` must belong to the current device.
 * Results are bit-identical to bsa_sparse_decode with the same arguments.
 * Every call on one GPU shares that GPU's scratch array, and the array keeps
 * the last call's contents: calls whose work may overlap on one GPU (other
 * streams, other host threads) race and give undefined results; order them
 * on one stream.  Nothing in the array needs to start at zero.
 * Arguments as in bsa_sparse_decode.
 * Errors: as bsa_sparse_decode; BSA_ERR_WORKSPACE when the call needs more
 *   than BSA_STATIC_SCRATCH_BYTES (bsa_workspace_size(layout, BSA_OP_DECODE,
 *   n_max) > BSA_STATIC_SCRATCH_BYTES; use bsa_sparse_decode with a caller
 *   workspace then); BSA_ERR_HIP if the scratch address cannot be looked up.
 * ------------------------------------------------------------------------- */
#define BSA_STATIC_SCRATCH_BYTES (16u << 20)
BSA_API bsa_status bsa_sparse_decode_static(const bsa_layout* layout,
                             const bsa_cache* cache, const void* q,
                             const int32_t* idx, const int32_t* cnt,
                             int32_t n_max, float softmax_scale, void* o,
                             float* lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * bsa_rectify_chunk -- ReSA rectification of the last f tokens of every
 * sequence ("Rectified Sparse Attention ...", Summary: every f generated
 * tokens are re-encoded in one dense pass that overwrites their KV entries
 * and block keys; Key points: f in {16, 32, 64, 128}).  In stream order:
 *   1. K/V at positions [T-f, T) (T = seq_lens[s]) <- k_new, v_new;
 *   2. descriptors of the blocks overlapping [T-f, T) are recomputed from
 *      scratch;
 *   3. query i (position T-f+i) of head h attends densely and causally to
 *      tokens 0..T-f+i of the rewritten cache.
 * q: [B][Hq][f][d]; k_new, v_new: [B][Hkv][f][d] (KV dtype, row major).
 * o: [B][Hq][f][d] KV dtype, OUT; lse: [B][Hq][f] fp32, OUT.
 * ws: at least bsa_workspace_size(layout, BSA_OP_RECTIFY, f) bytes.
 * Device contract: f <= seq_lens[s].
 * Errors: BSA_ERR_NULL, BSA_ERR_SHAPE, BSA_ERR_UNSUPPORTED, BSA_ERR_PARAM
 *   (f < 1, f > max_blocks*block, G*f > 4096, softmax_scale not finite and
 *   > 0), BSA_ERR_WORKSPACE, BSA_ERR_HIP.
 * ------------------------------------------------------------------------- */
BSA_API bsa_status bsa_rectify_chunk(const bsa_layout* layout, const bsa_cache* cache,
                             const void* q, const void* k_new,
                             const void* v_new, int32_t f, float softmax_scale,
                             void* o, float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* Workspace bytes needed by an operation (op = bsa_op), for the given
 * n_max (SELECT, DECODE, STEP) or f (RECTIFY).  Returns 0 for an invalid layout or
 * op.  Host-only; makes no HIP call. */
BSA_API size_t bsa_workspace_size(const bsa_layout* layout, int32_t op,
                          int32_t n_max_or_f);

/* Blocks kept for NB blocks under `params` (the n of bsa_select_params), the
 * host-side twin of the device rule; -1 for invalid parameters.  Callers use
 * it to size n_max: n_max = bsa_block_count(params, max_blocks, block). */
BSA_API int32_t bsa_block_count(const bsa_select_params* params, int32_t NB,
                        int32_t block);

/* Static description of a status code.  Never NULL. */
BSA_API const char* bsa_status_string(bsa_status status);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
