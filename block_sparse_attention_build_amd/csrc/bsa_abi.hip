// bsa_abi.hip -- the extern "C" surface declared in include/bsa.h.
// Every entry point validates its arguments on the host before any HIP call,
// carves its workspace, enqueues its kernels on the caller's stream and
// returns; nothing is allocated, nothing is synchronised.
//
// Built with BSA_CHECKED=1 (libbsa_checked.so), every entry point also
// verifies the device-side contracts it states before enqueuing anything:
// it drains the stream, copies the values the contracts bound (sequence
// lengths, page ids in use, kept counts and ids, biases) to the host and
// returns BSA_ERR_CONTRACT if one is broken.  That build synchronises on
// every call, so it is for debugging, not for graph capture.
#include <math.h>
#include <stddef.h>

#include <atomic>
#include <mutex>

#ifndef BSA_CHECKED
#define BSA_CHECKED 0
#endif
#if BSA_CHECKED
#include <vector>
#endif

#include "../../include/bsa.h"
#include "bsa_device.h"
#include "bsa_internal.h"

using namespace bsa;

// Scratch memory of bsa_sparse_decode_static: one copy of this array per GPU,
// held until the process ends.  In host code `scratch` is only a stand-in
// for the symbol: its device address (per device) comes from
// hipGetSymbolAddress, and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[BSA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// The device address of the current device's copy of `scratch`, resolved on
// the first call on that device (with that device current) and kept.
bsa_status static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BSA_ERR_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BSA_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return BSA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bsa_status check_layout(const bsa_layout* L) {
    if (!L) return BSA_ERR_NULL;
    if (L->B < 1 || L->Hq < 1 || L->Hkv < 1 || L->max_blocks < 1) return BSA_ERR_SHAPE;
    if (L->Hq % L->Hkv != 0) return BSA_ERR_SHAPE;
    if (L->Hq / L->Hkv > 16) return BSA_ERR_UNSUPPORTED;
    if (L->d != 64 && L->d != 128) return BSA_ERR_UNSUPPORTED;
    if (L->block != 32 && L->block != 64 && L->block != 128 && L->block != 256)
        return BSA_ERR_UNSUPPORTED;
    if (L->kv_dtype != BSA_DTYPE_F32 && L->kv_dtype != BSA_DTYPE_BF16) return BSA_ERR_UNSUPPORTED;
    if (L->desc_kind != BSA_DESC_MINMAX && L->desc_kind != BSA_DESC_MEANPOOL)
        return BSA_ERR_UNSUPPORTED;
    if (L->max_blocks > 32768) return BSA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(L->max_blocks) * L->block > (1ll << 30)) return BSA_ERR_UNSUPPORTED;
    return BSA_OK;
}

bsa_status check_cache(const bsa_cache* C) {
    if (!C) return BSA_ERR_NULL;
    if (!C->k_pool || !C->v_pool || !C->page_table || !C->seq_lens || !C->desc)
        return BSA_ERR_NULL;
    return BSA_OK;
}

CacheArgs make_args(const bsa_layout* L, const bsa_cache* C) {
    CacheArgs a;
    a.k_pool = C ? C->k_pool : nullptr;
    a.v_pool = C ? C->v_pool : nullptr;
    a.page_table = C ? C->page_table : nullptr;
    a.seq_lens = C ? C->seq_lens : nullptr;
    a.desc = C ? C->desc : nullptr;
    a.B = L->B;
    a.Hq = L->Hq;
    a.Hkv = L->Hkv;
    a.G = L->Hq / L->Hkv;
    a.d = L->d;
    a.block = L->block;
    a.max_blocks = L->max_blocks;
    a.dtype = L->kv_dtype == BSA_DTYPE_BF16 ? kBF16 : kF32;
    a.desc_kind = L->desc_kind == BSA_DESC_MINMAX ? kMinMax : kMeanPool;
    return a;
}

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

struct DecodeWs {
    size_t o_part, lse_part, total;
    int splits;
};
DecodeWs decode_ws(const CacheArgs& c, int n_max) {
    DecodeWs w;
    w.splits = decode_splits(c, n_max);
    const size_t rows = static_cast<size_t>(c.B) * c.Hq;
    w.o_part = 0;
    w.lse_part = align_up(rows * w.splits * c.d * sizeof(float));
    w.total = w.lse_part + align_up(rows * w.splits * sizeof(float));
    return w;
}

struct RectifyWs {
    size_t o_part, lse_part, total;
    RectifyPlan plan;
};
RectifyWs rectify_ws(const CacheArgs& c, int f) {
    RectifyWs w;
    rectify_plan(c, f, &w.plan);
    w.o_part = 0;
    w.lse_part = align_up(static_cast<size_t>(w.plan.o_floats) * sizeof(float));
    w.total = w.lse_part + align_up(static_cast<size_t>(w.plan.lse_floats) * sizeof(float));
    return w;
}

size_t select_ws(const CacheArgs& c) {
    return align_up(static_cast<size_t>(c.B) * c.Hkv * score_stride(c.max_blocks) * sizeof(float));
}

bsa_status check_select_params(const bsa_layout* L, const bsa_select_params* P) {
    if (!P) return BSA_ERR_NULL;
    if (P->n_local < 1 || P->n_min < 0 || P->budget_tokens < 0) return BSA_ERR_PARAM;
    if (P->budget_tokens == 0 && (P->sparsity_bp < 0 || P->sparsity_bp >= 10000))
        return BSA_ERR_PARAM;
    if (L->desc_kind == BSA_DESC_MEANPOOL && !P->gate_w) return BSA_ERR_PARAM;
    if (P->n_max < 1) return BSA_ERR_PARAM;
    const int need = block_count(L->max_blocks, L->block, P->budget_tokens, P->sparsity_bp,
                                 P->n_local, P->n_min);
    if (P->n_max < need) return BSA_ERR_PARAM;
    if (P->gate_bias && !(isfinite(P->gate_tau) && P->gate_tau >= 0.f)) return BSA_ERR_PARAM;
    if (P->gate_bias && (P->gate_current < 0 || P->gate_current > P->n_local)) return BSA_ERR_PARAM;
    return BSA_OK;
}

bsa_status hip_status(hipError_t e) { return e == hipSuccess ? BSA_OK : BSA_ERR_HIP; }

// ---------------------------------------------------------------------------
// Device-side contracts, verified on the host (checked builds).  Each check
// returns BSA_OK at once in the default build.
// ---------------------------------------------------------------------------
#if BSA_CHECKED
// n elements at src, after the work already enqueued on the stream
template <typename T>
bool fetch(std::vector<T>& dst, const void* src, size_t n, hipStream_t stream) {
    dst.assign(n, T());
    if (n == 0) return true;
    if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
        return false;
    return hipStreamSynchronize(stream) == hipSuccess;
}

int blocks_of(int32_t T, int block) { return (T + block - 1) / block; }
#endif

// lo <= seq_lens[s] <= max_blocks*block for every sequence, and a
// non-negative page id for every block that holds tokens.  T_out (checked
// builds) receives the lengths.
#if BSA_CHECKED
bsa_status contract_cache(const CacheArgs& c, int64_t lo, hipStream_t stream,
                          std::vector<int32_t>* T_out = nullptr) {
    std::vector<int32_t> T, pt;
    if (!fetch(T, c.seq_lens, c.B, stream)) return BSA_ERR_HIP;
    const int64_t cap = static_cast<int64_t>(c.max_blocks) * c.block;
    for (int s = 0; s < c.B; ++s)
        if (T[s] < lo || T[s] > cap) return BSA_ERR_CONTRACT;
    if (!fetch(pt, c.page_table, static_cast<size_t>(c.B) * c.max_blocks, stream))
        return BSA_ERR_HIP;
    for (int s = 0; s < c.B; ++s)
        for (int j = 0; j < blocks_of(T[s], c.block); ++j)
            if (pt[static_cast<size_t>(s) * c.max_blocks + j] < 0) return BSA_ERR_CONTRACT;
    if (T_out) *T_out = T;
    return BSA_OK;
}
#else
bsa_status contract_cache(const CacheArgs&, int64_t, hipStream_t) { return BSA_OK; }
#endif

// The kept lists of a decode: 0 <= cnt <= n_max, and the first cnt entries
// of each idx row are distinct block ids below ceil(seq_lens / block), with
// finite biases when a bias is given.
#if BSA_CHECKED
bsa_status contract_kept(const CacheArgs& c, const int32_t* idx, const int32_t* cnt,
                         const float* bias, int n_max, hipStream_t stream) {
    std::vector<int32_t> T, ci, ix;
    std::vector<float> bs;
    bsa_status st = contract_cache(c, 0, stream, &T);
    if (st != BSA_OK) return st;
    const size_t groups = static_cast<size_t>(c.B) * c.Hkv;
    if (!fetch(ci, cnt, groups, stream) || !fetch(ix, idx, groups * n_max, stream))
        return BSA_ERR_HIP;
    if (bias && !fetch(bs, bias, groups * n_max, stream)) return BSA_ERR_HIP;
    for (size_t g = 0; g < groups; ++g) {
        const int nb = blocks_of(T[g / c.Hkv], c.block);
        if (ci[g] < 0 || ci[g] > n_max) return BSA_ERR_CONTRACT;
        std::vector<char> seen(nb, 0);
        for (int k = 0; k < ci[g]; ++k) {
            const int32_t j = ix[g * n_max + k];
            if (j < 0 || j >= nb || seen[j]) return BSA_ERR_CONTRACT;
            seen[j] = 1;
            if (bias && !isfinite(bs[g * n_max + k])) return BSA_ERR_CONTRACT;
        }
    }
    return BSA_OK;
}
#else
bsa_status contract_kept(const CacheArgs&, const int32_t*, const int32_t*, const float*, int,
                         hipStream_t) {
    return BSA_OK;
}
#endif

// Host-side checks of a decode call, workspace aside.
bsa_status check_decode(const bsa_layout* layout, const bsa_cache* cache, const void* q,
                        const int32_t* idx, const int32_t* cnt, int32_t n_max,
                        float softmax_scale, const void* o, const float* lse) {
    bsa_status st = check_layout(layout);
    if (st != BSA_OK) return st;
    if ((st = check_cache(cache)) != BSA_OK) return st;
    if (!q || !idx || !cnt || !o || !lse) return BSA_ERR_NULL;
    if (n_max < 1 || n_max > layout->max_blocks) return BSA_ERR_PARAM;
    if (!scale_ok(softmax_scale)) return BSA_ERR_PARAM;
    return BSA_OK;
}

bsa_status sparse_decode(const bsa_layout* layout, const bsa_cache* cache, const void* q,
                         const int32_t* idx, const int32_t* cnt, const float* bias, int32_t n_max,
                         float softmax_scale, void* o, float* lse, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    bsa_status st = check_decode(layout, cache, q, idx, cnt, n_max, softmax_scale, o, lse);
    if (st != BSA_OK) return st;
    if (!ws) return BSA_ERR_NULL;
    const CacheArgs c = make_args(layout, cache);
    const DecodeWs w = decode_ws(c, n_max);
    if (ws_bytes < w.total) return BSA_ERR_WORKSPACE;
    if ((st = contract_kept(c, idx, cnt, bias, n_max, stream)) != BSA_OK) return st;
    DecodeArgs a;
    a.q = q;
    a.idx = idx;
    a.cnt = cnt;
    a.n_max = n_max;
    a.splits = w.splits;
    a.scale_log2 = softmax_scale * kLog2e;
    a.bias = bias;
    a.o_part = reinterpret_cast<float*>(static_cast<char*>(ws) + w.o_part);
    a.lse_part = reinterpret_cast<float*>(static_cast<char*>(ws) + w.lse_part);
    a.o = o;
    a.lse = lse;
    return hip_status(launch_decode(c, a, stream));
}

}  // namespace

extern "C" {

const char* bsa_status_string(bsa_status status) {
    switch (status) {
        case BSA_OK: return "ok";
        case BSA_ERR_NULL: return "a required pointer is NULL";
        case BSA_ERR_SHAPE: return "inconsistent shape (B, Hq, Hkv, max_blocks)";
        case BSA_ERR_UNSUPPORTED: return "unsupported dtype, head dim, block size or descriptor kind";
        case BSA_ERR_PARAM: return "parameter out of range";
        case BSA_ERR_WORKSPACE: return "workspace too small";
        case BSA_ERR_HIP: return "HIP kernel launch failed";
        case BSA_ERR_CONTRACT: return "a device-side input breaks its contract (checked build)";
    }
    return "unknown status";
}

int32_t bsa_block_count(const bsa_select_params* params, int32_t NB, int32_t block) {
    if (!params || NB < 0 || block < 1) return -1;
    if (params->n_local < 1 || params->n_min < 0 || params->budget_tokens < 0) return -1;
    if (params->budget_tokens == 0 && (params->sparsity_bp < 0 || params->sparsity_bp >= 10000))
        return -1;
    return block_count(NB, block, params->budget_tokens, params->sparsity_bp, params->n_local,
                       params->n_min);
}

size_t bsa_workspace_size(const bsa_layout* layout, int32_t op, int32_t n_max_or_f) {
    if (check_layout(layout) != BSA_OK || n_max_or_f < 1) return 0;
    const CacheArgs c = make_args(layout, nullptr);
    switch (op) {
        case BSA_OP_SELECT: return select_ws(c);
        case BSA_OP_DECODE: return decode_ws(c, n_max_or_f).total;
        case BSA_OP_RECTIFY: return rectify_ws(c, n_max_or_f).total;
        case BSA_OP_STEP: return select_ws(c) + decode_ws(c, n_max_or_f).total;
        default: return 0;
    }
}

bsa_status bsa_build_block_desc(const bsa_layout* layout, const bsa_cache* cache,
                                const void* k_new, const void* v_new, int32_t n_new,
                                const int32_t* range_begin, hipStream_t stream) {
    bsa_status st = check_layout(layout);
    if (st != BSA_OK) return st;
    if ((st = check_cache(cache)) != BSA_OK) return st;
    const bool append = (k_new != nullptr) || (v_new != nullptr);
    if (append) {
        if (!k_new || !v_new) return BSA_ERR_PARAM;
        if (n_new < 1 || static_cast<int64_t>(n_new) >
                             static_cast<int64_t>(layout->max_blocks) * layout->block)
            return BSA_ERR_PARAM;
        if (range_begin) return BSA_ERR_PARAM;
    }
    const CacheArgs c = make_args(layout, cache);
    if ((st = contract_cache(c, append ? n_new : 0, stream)) != BSA_OK) return st;
    return hip_status(launch_kv_write(c, append ? kModeAppend : kModeRebuild, k_new, v_new,
                                      append ? n_new : 0, range_begin, stream));
}

bsa_status bsa_select_blocks(const bsa_layout* layout, const bsa_cache* cache, const void* q,
                             const bsa_select_params* params, int32_t* idx, int32_t* cnt,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
    bsa_status st = check_layout(layout);
    if (st != BSA_OK) return st;
    if ((st = check_cache(cache)) != BSA_OK) return st;
    if (!q || !idx || !cnt || !ws) return BSA_ERR_NULL;
    if ((st = check_select_params(layout, params)) != BSA_OK) return st;
    const CacheArgs c = make_args(layout, cache);
    if (topn_keys_per_thread(c.max_blocks) == 0) return BSA_ERR_UNSUPPORTED;
    if (ws_bytes < select_ws(c)) return BSA_ERR_WORKSPACE;
    if ((st = contract_cache(c, 0, stream)) != BSA_OK) return st;
    SelectArgs s;
    s.q = q;
    s.gate_w = params->gate_w;
    s.budget_tokens = params->budget_tokens;
    s.sparsity_bp = params->sparsity_bp;
    s.n_local = params->n_local;
    s.n_min = params->n_min;
    s.n_max = params->n_max;
    s.idx = idx;
    s.cnt = cnt;
    s.scores = static_cast<float*>(ws);
    s.gate_tau = params->gate_tau;
    s.gate_bias = params->gate_bias;
    s.gate_current = params->gate_current > 1 ? params->gate_current : 1;
    return hip_status(launch_select(c, s, stream));
}

bsa_status bsa_append_select(const bsa_layout* layout, const bsa_cache* cache, const void* k_new,
                             const void* v_new, const void* q, const bsa_select_params* params,
                             int32_t* idx, int32_t* cnt, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
    bsa_status st = check_layout(layout);
    if (st != BSA_OK) return st;
    if ((st = check_cache(cache)) != BSA_OK) return st;
    if (!k_new || !v_new || !q || !idx || !cnt || !ws) return BSA_ERR_NULL;
    if ((st = check_select_params(layout, params)) != BSA_OK) return st;
    const CacheArgs c = make_args(layout, cache);
    if (topn_keys_per_thread(c.max_blocks) == 0) return BSA_ERR_UNSUPPORTED;
    if (ws_bytes < select_ws(c)) return BSA_ERR_WORKSPACE;
    if ((st = contract_cache(c, 1, stream)) != BSA_OK) return st;
    SelectArgs s;
    s.q = q;
    s.gate_w = params->gate_w;
    s.budget_tokens = params->budget_tokens;
    s.sparsity_bp = params->sparsity_bp;
    s.n_local = params->n_local;
    s.n_min = params->n_min;
    s.n_max = params->n_max;
    s.idx = idx;
    s.cnt = cnt;
    s.scores = static_cast<float*>(ws);
    s.gate_tau = params->gate_tau;
    s.gate_bias = params->gate_bias;
    s.gate_current = params->gate_current > 1 ? params->gate_current : 1;
    return hip_status(launch_append_select(c, k_new, v_new, s, stream));
}

bsa_status bsa_append_select_decode(const bsa_layout* layout, const bsa_cache* cache,
                                    const void* k_new, const void* v_new, const void* q,
                                    const bsa_select_params* params, int32_t* idx, int32_t* cnt,
                                    float softmax_scale, void* o, float* lse, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
    bsa_status st = check_layout(layout);
    if (st != BSA_OK) return st;
    if ((st = check_cache(cache)) != BSA_OK) return st;
    if (!k_new || !v_new || !q || !idx || !cnt || !o || !lse || !ws) return BSA_ERR_NULL;
    if ((st = check_select_params(layout, params)) != BSA_OK) return st;
    if (params->n_max > layout->max_blocks) return BSA_ERR_PARAM;
    if (!scale_ok(softmax_scale)) return BSA_ERR_PARAM;
    const CacheArgs c = make_args(layout, cache);
    if (topn_keys_per_thread(c.max_blocks) == 0) return BSA_ERR_UNSUPPORTED;
    const size_t sel_bytes = select_ws(c);
    const DecodeWs w = decode_ws(c, params->n_max);
    if (ws_bytes < sel_bytes + w.total) return BSA_ERR_WORKSPACE;
    if ((st = contract_cache(c, 1, stream)) != BSA_OK) return st;
    SelectArgs s;
    s.q = q;
    s.gate_w = params->gate_w;
    s.budget_tokens = params->budget_tokens;
    s.sparsity_bp = params->sparsity_bp;
    s.n_local = params->n_local;
    s.n_min = params->n_min;
    s.n_max = params->n_max;
    s.idx = idx;
    s.cnt = cnt;
    s.scores = static_cast<float*>(ws);
    s.gate_tau = params->gate_tau;
    s.gate_bias = params->gate_bias;
    s.gate_current = params->gate_current > 1 ? params->gate_current : 1;
    char* dws = static_cast<char*>(ws) + sel_bytes;
    DecodeArgs a;
    a.q = q;
    a.idx = idx;
    a.cnt = cnt;
    a.n_max = params->n_max;
    a.splits = w.splits;
    a.scale_log2 = softmax_scale * kLog2e;
    a.bias = params->gate_bias;
    a.o_part = reinterpret_cast<float*>(dws + w.o_part);
    a.lse_part = reinterpret_cast<float*>(dws + w.lse_part);
    a.o = o;
    a.lse = lse;
    const bool in_wg = !params->gate_bias && decode_selects(c, params->n_local, params->n_max);
    if (!in_wg) {
        if ((st = hip_status(launch_append_select(c, k_new, v_new, s, stream))) != BSA_OK)
            return st;
        if ((st = contract_kept(c, idx, cnt, a.bias, a.n_max, stream)) != BSA_OK) return st;
        return hip_status(launch_decode(c, a, stream));
    }
    if ((st = hip_status(launch_append_score_only(c, k_new, v_new, s, stream))) != BSA_OK)
        return st;
    a.scores = s.scores;
    a.score_stride = score_stride(c.max_blocks);
    a.budget_tokens = params->budget_tokens;
    a.sparsity_bp = params->sparsity_bp;
    a.n_local = params->n_local;
    a.n_min = params->n_min;
    a.idx_out = idx;
    a.cnt_out = cnt;
    return hip_status(launch_decode(c, a, stream));
}

bsa_status bsa_sparse_decode(const bsa_layout* layout, const bsa_cache* cache, const void* q,
                             const int32_t* idx, const int32_t* cnt, int32_t n_max,
                             float softmax_scale, void* o, float* lse, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
    return sparse_decode(layout, cache, q, idx, cnt, nullptr, n_max, softmax_scale, o, lse, ws,
                         ws_bytes, stream);
}

bsa_status bsa_sparse_decode_gated(const bsa_layout* layout, const bsa_cache* cache,
                                   const void* q, const int32_t* idx, const int32_t* cnt,
                                   const float* gate_bias, int32_t n_max, float softmax_scale,
                                   void* o, float* lse, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
    if (!gate_bias) return BSA_ERR_NULL;
    return sparse_decode(layout, cache, q, idx, cnt, gate_bias, n_max, softmax_scale, o, lse, ws,
                         ws_bytes, stream);
}

bsa_status bsa_sparse_decode_static(const bsa_layout* layout, const bsa_cache* cache,
                                    const void* q, const int32_t* idx, const int32_t* cnt,
                                    int32_t n_max, float softmax_scale, void* o, float* lse,
                                    hipStream_t stream) {
    bsa_status st = check_decode(layout, cache, q, idx, cnt, n_max, softmax_scale, o, lse);
    if (st != BSA_OK) return st;
    if (decode_ws(make_args(layout, cache), n_max).total > BSA_STATIC_SCRATCH_BYTES)
        return BSA_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = static_scratch(&ws)) != BSA_OK) return st;
    return sparse_decode(layout, cache, q, idx, cnt, nullptr, n_max, softmax_scale, o, lse, ws,
                         BSA_STATIC_SCRATCH_BYTES, stream);
}

bsa_status bsa_rectify_chunk(const bsa_layout* layout, const bsa_cache* cache, const void* q,
                             const void* k_new, const void* v_new, int32_t f,
                             float softmax_scale, void* o, float* lse, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
    bsa_status st = check_layout(layout);
    if (st != BSA_OK) return st;
    if ((st = check_cache(cache)) != BSA_OK) return st;
    if (!q || !k_new || !v_new || !o || !lse || !ws) return BSA_ERR_NULL;
    if (f < 1 || static_cast<int64_t>(f) > static_cast<int64_t>(layout->max_blocks) * layout->block)
        return BSA_ERR_PARAM;
    if ((layout->Hq / layout->Hkv) * f > 4096) return BSA_ERR_PARAM;
    if (!scale_ok(softmax_scale)) return BSA_ERR_PARAM;
    const CacheArgs c = make_args(layout, cache);
    const RectifyWs w = rectify_ws(c, f);
    if (ws_bytes < w.total) return BSA_ERR_WORKSPACE;
    if ((st = contract_cache(c, f, stream)) != BSA_OK) return st;
    RectifyArgs a;
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.f = f;
    a.splits = w.plan.splits;
    a.chunk_tiles = w.plan.chunk_tiles;
    a.wgs = w.plan.wgs;
    a.rows_per_wg = w.plan.rows_per_wg;
    a.sets = w.plan.sets;
    a.scale_log2 = softmax_scale * kLog2e;
    a.o_part = reinterpret_cast<float*>(static_cast<char*>(ws) + w.o_part);
    a.lse_part = reinterpret_cast<float*>(static_cast<char*>(ws) + w.lse_part);
    a.o = o;
    a.lse = lse;
    return hip_status(launch_rectify(c, a, stream));
}

}  // extern "C"
