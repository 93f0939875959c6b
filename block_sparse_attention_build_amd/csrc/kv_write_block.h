// kv_write_block.h -- device body of the KV write / descriptor update
// (kv_write.hip), shared with the fused append + score kernel (select.hip).
//
// "Rectified Sparse Attention for Efficient Long-Sequence Generation",
// Summary (block keys); "SeerAttention-R", Abstract (pooled keys).
//
// One workgroup owns one (sequence, KV head, logical block): it copies the
// block's new tokens from the row-major source into the page (in the page's
// matrix-operand order), then one thread per channel walks the block's
// tokens in order to update or rebuild that channel's descriptor.  New-token
// values are read from the source, older ones from the cache, so there is no
// read-after-write hazard inside the workgroup.  Work per step is a few KiB,
// so the body is latency-bound: every thread keeps KB loads in flight.
#pragma once

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

constexpr int kKvBatch = 8;  // loads in flight per thread (default)

struct KvWriteParams {
    CacheArgs c;
    int mode;
    const void* k_new;
    const void* v_new;
    int n_new;
    const int32_t* range_begin;
};

// One (sequence, KV head, block) of the write: bx = block offset from the
// first touched block, grp = sequence * Hkv + KV head; NT threads, KB loads
// in flight per thread.
template <int DT, int DESC, int NT, int KB = kKvBatch>
__device__ __forceinline__ void kv_write_block(const KvWriteParams& p, int bx, int grp) {
    typedef typename Elem<DT>::T E;
    const CacheArgs& c = p.c;
    const int s = grp / c.Hkv;
    const int kvh = grp - s * c.Hkv;
    const int T = c.seq_lens[s];
    int lo;
    if (p.mode == kModeRebuild)
        lo = p.range_begin ? p.range_begin[s] : 0;
    else
        lo = T - p.n_new;
    if (lo < 0) lo = 0;
    if (lo >= T) return;
    const int j = lo / c.block + bx;
    const int tb0 = j * c.block;
    if (tb0 >= T) return;
    const int tb1 = min(tb0 + c.block, T);
    const int d = c.d;
    const int64_t page = c.page_table[static_cast<int64_t>(s) * c.max_blocks + j];
    const int64_t page_off = (page * c.Hkv + kvh) * static_cast<int64_t>(c.block) * d;
    E* kp = static_cast<E*>(c.k_pool) + page_off;
    E* vp = static_cast<E*>(c.v_pool) + page_off;
    const bool writes = p.mode != kModeRebuild;
    // source rows of this group: [n_new][d]
    const E* ks = writes ? static_cast<const E*>(p.k_new) + static_cast<int64_t>(grp) * p.n_new * d
                         : nullptr;
    const E* vs = writes ? static_cast<const E*>(p.v_new) + static_cast<int64_t>(grp) * p.n_new * d
                         : nullptr;

    if (writes) {
        // copy: KB independent source loads per thread before the stores
        // (the stores could alias the sources as far as the compiler knows,
        // so without the batching every load would wait for the last store)
        const int w0 = max(tb0, lo);
        const int nel = (tb1 - w0) * d;
        const E* ksrc = ks + static_cast<int64_t>(w0 - lo) * d;
        const E* vsrc = vs + static_cast<int64_t>(w0 - lo) * d;
        for (int e0 = threadIdx.x; e0 < nel; e0 += KB * NT) {
            E kb[KB], vb[KB];
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const int e = e0 + u * NT;
                if (e < nel) {
                    kb[u] = ksrc[e];
                    vb[u] = vsrc[e];
                }
            }
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const int e = e0 + u * NT;
                if (e < nel) {
                    const int tt = e / d;
                    const int i = e - tt * d;
                    const int t = w0 - tb0 + tt;
                    kp[k_off<DT>(t, i, d)] = kb[u];
                    vp[v_off<DT>(t, i, d)] = vb[u];
                }
            }
        }
    }

    // descriptor of block j, one thread per channel; the block's keys are
    // read KB tokens at a time (independent loads), then folded in token
    // order
    const bool merge = (p.mode == kModeAppend) && (tb0 < lo);
    const int t_first = merge ? lo : tb0;
    const int64_t drow = static_cast<int64_t>(grp) * c.max_blocks + j;
    for (int i = threadIdx.x; i < d; i += NT) {
        float mn = 0.f, mx = 0.f, acc = 0.f;
        bool have = merge;
        if (merge) {
            if (DESC == kMinMax) {
                const E* dp = static_cast<const E*>(c.desc) + drow * 2 * d;
                mn = Elem<DT>::load(dp, i);
                mx = Elem<DT>::load(dp, d + i);
            } else {
                acc = static_cast<const float*>(c.desc)[drow * d + i];
            }
        }
        for (int t0 = t_first; t0 < tb1; t0 += KB) {
            float v[KB];
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const int t = t0 + u;
                v[u] = 0.f;
                if (t < tb1)
                    v[u] = (writes && t >= lo) ? Elem<DT>::load(ks, static_cast<int64_t>(t - lo) * d + i)
                                               : Elem<DT>::load(kp, k_off<DT>(t - tb0, i, d));
            }
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                if (t0 + u >= tb1) break;
                if (DESC == kMinMax) {
                    mn = (!have || v[u] < mn) ? v[u] : mn;
                    mx = (!have || v[u] > mx) ? v[u] : mx;
                    have = true;
                } else {
                    acc += v[u];
                }
            }
        }
        if (DESC == kMinMax) {
            E* dp = static_cast<E*>(c.desc) + drow * 2 * d;
            Elem<DT>::store(dp, i, mn);  // exact: mn/mx are stored values
            Elem<DT>::store(dp, d + i, mx);
        } else {
            static_cast<float*>(c.desc)[drow * d + i] = acc;
        }
    }
}

}  // namespace bsa
