// kv_write.hip -- write tokens into the paged KV cache and maintain the
// per-block key descriptors in the same pass.
//
// Descriptors ("Rectified Sparse Attention for Efficient Long-Sequence
// Generation", Summary): Quest-style channel-wise min and max of the keys of
// each block; for the plug-in gate ("SeerAttention-R", Abstract) the pooled
// key of the block, kept here as the fp32 running sum of its keys in token
// order (mean = sum / tokens).
//
// The per-block body lives in kv_write_block.h (shared with the fused
// append + score kernel); this file launches it on its own.
#include "bsa_device.h"
#include "bsa_internal.h"
#include "kv_write_block.h"

namespace bsa {

namespace {

constexpr int kThreads = 128;
// loads in flight per thread: a rectify overwrite or a rebuild walks whole
// blocks with few workgroups, so its time is the number of dependent
// round trips (a 64-token block in two instead of eight)
constexpr int kBatch = 32;

template <int DT, int DESC>
__global__ __launch_bounds__(kThreads) void kv_write_kernel(KvWriteParams p) {
    kv_write_block<DT, DESC, kThreads, kBatch>(p, static_cast<int>(blockIdx.x),
                                               static_cast<int>(blockIdx.y));
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
