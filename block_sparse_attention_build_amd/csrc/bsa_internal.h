// bsa_internal.h -- host-side launch interface between the C ABI
// (bsa_abi.hip) and the kernel files.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

struct CacheArgs {
    void* k_pool;
    void* v_pool;
    const int32_t* page_table;
    const int32_t* seq_lens;
    void* desc;
    int B, Hq, Hkv, G, d, block, max_blocks;
    int dtype;      // kF32 / kBF16
    int desc_kind;  // kMinMax / kMeanPool
};

// kv_write modes
constexpr int kModeAppend = 0;     // write new tokens, merge into descriptors
constexpr int kModeOverwrite = 1;  // write new tokens, rebuild touched descriptors
constexpr int kModeRebuild = 2;    // no write, rebuild descriptors of a range

hipError_t launch_kv_write(const CacheArgs& c, int mode, const void* k_new, const void* v_new,
                           int n_new, const int32_t* range_begin, hipStream_t stream);

struct SelectArgs {
    const void* q;
    const void* gate_w;
    int budget_tokens, sparsity_bp, n_local, n_min, n_max;
    int32_t* idx;
    int32_t* cnt;
    float* scores;  // workspace [B*Hkv][score_stride(max_blocks)]
    float gate_tau;
    float* gate_bias;  // nullptr, or [B*Hkv][n_max]: log-gate bias per idx entry
    int gate_current;  // with gate_bias: trailing blocks with the unit gate (>= 1)
};
hipError_t launch_select(const CacheArgs& c, const SelectArgs& s, hipStream_t stream);
// Append of one token per sequence (kModeAppend, n_new = 1) and selection,
// the append sharing the scoring launch.
hipError_t launch_append_select(const CacheArgs& c, const void* k_new, const void* v_new,
                                const SelectArgs& s, hipStream_t stream);
// The append and the scores of launch_append_select without the top-n
// launch (the decode kernel then selects in-workgroup: DecodeArgs.scores).
hipError_t launch_append_score_only(const CacheArgs& c, const void* k_new, const void* v_new,
                                    const SelectArgs& s, hipStream_t stream);
// keys-per-thread bucket of the top-n kernel for a given max_blocks (0 = too many)
int topn_keys_per_thread(int max_blocks);
// row stride (floats) of the score workspace: max_blocks rounded up to 4
int score_stride(int max_blocks);

struct DecodeArgs {
    const void* q;
    const int32_t* idx;
    const int32_t* cnt;
    int n_max;
    int splits;  // S: partials per (sequence, query head)
    float scale_log2;  // softmax_scale * log2(e)
    const float* bias;  // nullptr, or [B*Hkv][n_max]: natural-log logit bias per idx entry
    float* o_part;     // [B*Hq][S][d]
    float* lse_part;   // [B*Hq][S]  (base-2 log-sum-exp of the scaled logits)
    void* o;
    float* lse;
    // In-workgroup selection (bf16, no bias, decode_selects() true): with
    // scores set, every decode workgroup selects its group's kept blocks
    // from the score row itself, idx/cnt above are ignored, and the first
    // split of each group writes the kept list to idx_out/cnt_out.
    const float* scores = nullptr;  // [B*Hkv][score_stride]
    int score_stride = 0;
    int budget_tokens = 0, sparsity_bp = 0, n_local = 1, n_min = 0;
    int32_t* idx_out = nullptr;     // [B*Hkv][n_max]
    int32_t* cnt_out = nullptr;     // [B*Hkv]
};
hipError_t launch_decode(const CacheArgs& c, const DecodeArgs& a, hipStream_t stream);
int decode_splits(const CacheArgs& c, int n_max);
// In-workgroup selection: candidate blocks per sequence (max_blocks minus the
// local blocks) up to which the decode kernel can select (up to sixteen per
// thread), and the longest kept list it holds in LDS beside the unit
// partials (so that the decode's units are cut as in bsa_sparse_decode).
constexpr int kDecodeSelectSlots = 8192;
constexpr int kDecodeSelectMaxKept = 4096;
// Whether launch_decode can select in-workgroup for this layout.
bool decode_selects(const CacheArgs& c, int n_local, int n_max);

struct RectifyArgs {
    const void* q;      // [B][Hq][f][d]
    const void* k_new;  // [B][Hkv][f][d]
    const void* v_new;
    int f;
    int splits;           // fp32: token chunks per group
    int chunk_tiles;      // fp32: 32-token tiles per chunk
    int wgs;              // bf16: workgroups launched (even shares of all tiles)
    int rows_per_wg;      // bf16: rows of a row group
    int sets;             // bf16: sets of workgroups (one row group each) in the 256-row shape, else 1
    float scale_log2;
    float* o_part;        // bf16: [slot][rows_per_wg][d]; fp32: [B*Hq*f][S][d]
    float* lse_part;      // bf16: [slot][rows_per_wg];    fp32: [B*Hq*f][S]
    void* o;
    float* lse;
};
// Sizes of the partial results of one rectify call (floats) and the launch
// shape they follow.
struct RectifyPlan {
    int64_t o_floats;
    int64_t lse_floats;
    int splits, chunk_tiles;  // fp32 path
    int wgs, rows_per_wg, sets;  // bf16 path
};
hipError_t launch_rectify(const CacheArgs& c, const RectifyArgs& a, hipStream_t stream);
void rectify_plan(const CacheArgs& c, int f, RectifyPlan* plan);

// Merge S partials of `rows` rows into o (KV dtype) and lse (natural log).
hipError_t launch_combine(int dtype, int d, int rows, int splits, const float* o_part,
                          const float* lse_part, void* o, float* lse, hipStream_t stream);
// Same, but row r merges only the splits covering [0, seq_lens[r / rows_per_seq]).
hipError_t launch_combine_ragged(int dtype, int d, int rows, int splits, const float* o_part,
                                 const float* lse_part, void* o, float* lse,
                                 const int32_t* seq_lens, int rows_per_seq,
                                 int tokens_per_split, hipStream_t stream);

}  // namespace bsa
