// kv_write.hip -- write tokens into the paged KV cache and maintain the
// per-block key descriptors in the same pass.
//
// Descriptors ("Rectified Sparse Attention for Efficient Long-Sequence
// Generation", Summary): Quest-style channel-wise min and max of the keys of
// each block; for the plug-in gate ("SeerAttention-R", Abstract) the pooled
// key of the block, kept here as the fp32 running sum of its keys in token
// order (mean = sum / tokens).
//
// One workgroup owns one (sequence, KV head, logical block): it copies the
// block's new tokens from the row-major source into the page (in the page's
// matrix-operand order), then one thread per channel walks the block's
// tokens in order to update or rebuild that channel's descriptor.  New-token
// values are read from the source, older ones from the cache, so there is no
// read-after-write hazard inside the workgroup.  Work per step is a few KiB,
// so the kernel is latency-bound: every thread keeps kBatch loads in flight.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

constexpr int kThreads = 128;
constexpr int kBatch = 8;  // loads in flight per thread

struct KvWriteParams {
    CacheArgs c;
    int mode;
    const void* k_new;
    const void* v_new;
    int n_new;
    const int32_t* range_begin;
};

template <int DT, int DESC>
__global__ __launch_bounds__(kThreads) void kv_write_kernel(KvWriteParams p) {
    typedef typename Elem<DT>::T E;
    const CacheArgs& c = p.c;
    const int grp = blockIdx.y;  // sequence * Hkv + kv head
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
    const int j = lo / c.block + static_cast<int>(blockIdx.x);
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
        // copy: kBatch independent source loads per thread before the stores
        // (the stores could alias the sources as far as the compiler knows,
        // so without the batching every load would wait for the last store)
        const int w0 = max(tb0, lo);
        const int nel = (tb1 - w0) * d;
        const E* ksrc = ks + static_cast<int64_t>(w0 - lo) * d;
        const E* vsrc = vs + static_cast<int64_t>(w0 - lo) * d;
        for (int e0 = threadIdx.x; e0 < nel; e0 += kBatch * kThreads) {
            E kb[kBatch], vb[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = e0 + u * kThreads;
                if (e < nel) {
                    kb[u] = ksrc[e];
                    vb[u] = vsrc[e];
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = e0 + u * kThreads;
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
    // read kBatch tokens at a time (independent loads), then folded in token
    // order
    const bool merge = (p.mode == kModeAppend) && (tb0 < lo);
    const int t_first = merge ? lo : tb0;
    const int64_t drow = static_cast<int64_t>(grp) * c.max_blocks + j;
    for (int i = threadIdx.x; i < d; i += kThreads) {
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
        for (int t0 = t_first; t0 < tb1; t0 += kBatch) {
            float v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int t = t0 + u;
                v[u] = 0.f;
                if (t < tb1)
                    v[u] = (writes && t >= lo) ? Elem<DT>::load(ks, static_cast<int64_t>(t - lo) * d + i)
                                               : Elem<DT>::load(kp, k_off<DT>(t - tb0, i, d));
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
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

template <int DT, int DESC>
hipError_t launch_t(const KvWriteParams& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((kv_write_kernel<DT, DESC>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_write(const CacheArgs& c, int mode, const void* k_new, const void* v_new,
                           int n_new, const int32_t* range_begin, hipStream_t stream) {
    KvWriteParams p{c, mode, k_new, v_new, n_new, range_begin};
    int gx;
    if (mode == kModeRebuild)
        gx = c.max_blocks;
    else
        gx = min((n_new + c.block - 1) / c.block + 1, c.max_blocks);
    dim3 grid(gx, c.B * c.Hkv);
    if (c.dtype == kBF16)
        return c.desc_kind == kMinMax ? launch_t<kBF16, kMinMax>(p, grid, stream)
                                      : launch_t<kBF16, kMeanPool>(p, grid, stream);
    return c.desc_kind == kMinMax ? launch_t<kF32, kMinMax>(p, grid, stream)
                                  : launch_t<kF32, kMeanPool>(p, grid, stream);
}

}  // namespace bsa
