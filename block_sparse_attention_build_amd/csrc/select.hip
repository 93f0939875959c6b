// select.hip -- group block scoring and top-n block selection.
//
// "Rectified Sparse Attention for Efficient Long-Sequence Generation",
// Summary: min/max block descriptors score the memory blocks and every query
// head of a GQA group shares one block selection; Key points: dynamic top-n
// keeping the recent local blocks and a minimum count.  "Simple Attention
// Sparsification", Method: the current block is always retained and, at
// inference, the ranking becomes discrete Top-K block indices.
//
// Kernel 1 (score): streams the descriptors of every candidate (non-local)
//   block, one group per grid row, many workgroups per group so that long
//   contexts spread over the whole chip.
//   Min/max score.  With m <= M per channel, max(q*m, q*M) equals
//   max(q,0)*M + min(q,0)*m, so the group score
//       sum_h sum_i max(q_hi m_i, q_hi M_i)
//   equals  Q+ . M + Q- . m  with  Q+_i = sum_h max(q_hi, 0),
//   Q-_i = sum_h min(q_hi, 0)  -- one 2d-long dot product per block instead
//   of G of them.  Mean-pool score: (W sum_h q_h) . sum_j / tokens_j.
//   Scores are fp32.  Each block's descriptor row is read by a run of lanes
//   with 16-byte loads and reduced with cross-lane adds.
// Kernel 2 (top-n): one 1024-thread workgroup per group holds the candidate
//   scores in registers as order-preserving uint32 keys, finds the n-th
//   largest key with an MSB-first radix select over LDS histograms (digits
//   taken from key - min_key so that the first digit already spreads the
//   keys), then compacts the kept blocks in ascending index order with two
//   block-wide prefix scans (ties at the threshold go to the lower index),
//   appends the local blocks and pads with -1.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreIters = 8;
constexpr int kTopnThreads = 1024;
constexpr int kTopnWaves = kTopnThreads / kWave;

struct ScoreParams {
    CacheArgs c;
    SelectArgs s;
};

// 16-byte chunk of descriptor elements as floats
template <int DE>  // descriptor element kind: kF32 / kBF16
struct Chunk;
template <>
struct Chunk<kBF16> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const void* p, float* out) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            out[2 * k] = __uint_as_float(w[k] << 16);
            out[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
};
template <>
struct Chunk<kF32> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const void* p, float* out) {
        const floatx4 w = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = w[k];
    }
};

template <int DT, int DESC, int D>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreParams p) {
    typedef typename Elem<DT>::T E;
    constexpr int DE = DESC == kMinMax ? DT : kF32;  // descriptor element type
    constexpr int EPL = Chunk<DE>::N;                 // elements per lane
    constexpr int LPB = D / EPL;                      // lanes per block row
    constexpr int BPI = kScoreThreads / LPB;          // blocks per iteration
    constexpr int BPW = BPI * kScoreIters;            // blocks per workgroup
    const CacheArgs& c = p.c;
    const SelectArgs& a = p.s;
    const int grp = blockIdx.y;
    const int s = grp / c.Hkv;
    const int kvh = grp - s * c.Hkv;
    const int T = c.seq_lens[s];
    const int NB = (T + c.block - 1) / c.block;
    const int nl = min(a.n_local, NB);
    const int NC = NB - nl;
    const int c0 = blockIdx.x * BPW;
    if (c0 >= NC) return;
    const int c1 = min(c0 + BPW, NC);
    const int tid = threadIdx.x;
    const int lp = tid % LPB;      // lane position inside the block row
    const int slot = tid / LPB;    // which block of the iteration
    const int ch0 = lp * EPL;      // first channel of this lane

    const E* qg = static_cast<const E*>(a.q) + (static_cast<int64_t>(s) * c.Hq + kvh * c.G) * D;
    float wa[EPL], wb[EPL];
    if (DESC == kMinMax) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float qp = 0.f, qm = 0.f;
            for (int h = 0; h < c.G; ++h) {
                const float x = Elem<DT>::load(qg, h * D + ch0 + e);
                qp += fmaxf(x, 0.f);
                qm += fminf(x, 0.f);
            }
            wa[e] = qp;  // pairs with the max row
            wb[e] = qm;  // pairs with the min row
        }
    } else {
        __shared__ float u_s[D];
        for (int i = tid; i < D; i += kScoreThreads) {
            float acc = 0.f;
            for (int h = 0; h < c.G; ++h) acc += Elem<DT>::load(qg, h * D + i);
            u_s[i] = acc;
        }
        __syncthreads();
        const uint16_t* W = static_cast<const uint16_t*>(a.gate_w);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const uint16_t* wr = W + (ch0 + e) * D;
            float acc = 0.f;
            for (int k = 0; k < D; ++k) acc += bf2f(wr[k]) * u_s[k];
            wa[e] = acc;
            wb[e] = 0.f;
        }
    }

    float* out = a.scores + static_cast<int64_t>(grp) * c.max_blocks;
    const int64_t row0 = static_cast<int64_t>(grp) * c.max_blocks;
    for (int jb = c0; jb < c1; jb += BPI) {
        const int j = jb + slot;
        if (j >= c1) break;  // whole lane run leaves together
        float part = 0.f;
        if (DESC == kMinMax) {
            const E* dp = static_cast<const E*>(c.desc) + (row0 + j) * 2 * D;
            float mn[EPL], mx[EPL];
            Chunk<DE>::load(dp + ch0, mn);
            Chunk<DE>::load(dp + D + ch0, mx);
#pragma unroll
            for (int e = 0; e < EPL; ++e) part += wa[e] * mx[e] + wb[e] * mn[e];
        } else {
            const float* dp = static_cast<const float*>(c.desc) + (row0 + j) * D;
            float sm[EPL];
            Chunk<kF32>::load(dp + ch0, sm);
#pragma unroll
            for (int e = 0; e < EPL; ++e) part += wa[e] * sm[e];
        }
        part = group_sum<LPB>(part);
        if (lp == 0) {
            if (DESC == kMeanPool) {
                const int ntok = min(c.block, T - j * c.block);
                part = part / static_cast<float>(ntok);
            }
            out[j] = part;
        }
    }
}

// ----------------------------- top-n ---------------------------------------

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m, 64)));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m, 64)));
    return v;
}
__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}
// Exclusive prefix sum over all kTopnThreads threads; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
    const int w = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if ((threadIdx.x & 63) == 63) wsum[w] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < kTopnWaves; ++k) {
        const int t = wsum[k];
        before += (k < w) ? t : 0;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

struct TopnParams {
    CacheArgs c;
    SelectArgs s;
};

template <int KPT>
__global__ __launch_bounds__(kTopnThreads) void topn_kernel(TopnParams p) {
    const CacheArgs& c = p.c;
    const SelectArgs& a = p.s;
    __shared__ int hist[256];
    __shared__ int wsum[kTopnWaves];
    __shared__ uint32_t red_min[kTopnWaves], red_max[kTopnWaves];
    __shared__ int s_digit, s_above;

    const int grp = blockIdx.x;
    const int s = grp / c.Hkv;
    const int tid = threadIdx.x;
    const int T = c.seq_lens[s];
    const int NB = (T + c.block - 1) / c.block;
    const int nl = min(a.n_local, NB);
    const int NC = NB - nl;
    const int n = block_count(NB, c.block, a.budget_tokens, a.sparsity_bp, a.n_local, a.n_min);
    const int K = n - nl;  // candidates to pick
    int32_t* out = a.idx + static_cast<int64_t>(grp) * a.n_max;
    const float* sc = a.scores + static_cast<int64_t>(grp) * c.max_blocks;

    const int base = tid * KPT;
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const int j = base + r;
        key[r] = (j < NC) ? float_key(sc[j]) : 0u;
    }

    // mode: 0 = none, 1 = all candidates, 2 = threshold
    int mode = (K <= 0) ? 0 : (K >= NC ? 1 : 2);
    uint32_t tau = 0;
    int need_eq = 0;
    if (mode == 2) {
        uint32_t lmin = 0xffffffffu, lmax = 0u;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            if (base + r < NC) {
                lmin = min(lmin, key[r]);
                lmax = max(lmax, key[r]);
            }
        }
        lmin = wave_min_u32(lmin);
        lmax = wave_max_u32(lmax);
        if ((tid & 63) == 0) {
            red_min[tid >> 6] = lmin;
            red_max[tid >> 6] = lmax;
        }
        __syncthreads();
        uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
        for (int w = 0; w < kTopnWaves; ++w) {
            kmin = min(kmin, red_min[w]);
            kmax = max(kmax, red_max[w]);
        }
        const uint32_t range = kmax - kmin;
        uint32_t prefix = 0;  // over key - kmin
        int krem = K;
        int shift = (range == 0u) ? 0 : 32 - __clz(static_cast<int>(range));
        while (shift > 0) {
            const int dbits = min(8, shift);
            shift -= dbits;
            const int hi = shift + dbits;  // bits above the digit must match prefix
            for (int b = tid; b < 256; b += kTopnThreads) hist[b] = 0;
            __syncthreads();
#pragma unroll
            for (int r = 0; r < KPT; ++r) {
                if (base + r < NC) {
                    const uint32_t kr = key[r] - kmin;
                    const bool alive = hi >= 32 || ((kr >> hi) == (prefix >> hi));
                    if (alive) atomicAdd(&hist[(kr >> shift) & ((1u << dbits) - 1u)], 1);
                }
            }
            __syncthreads();
            // suffix counts over the digits: thread t < 256 looks at digit 255 - t
            // (waves 0..3 are whole waves, so the in-wave scan is well formed)
            int h = 0, incl = 0;
            if (tid < 256) {
                h = hist[255 - tid];
                incl = wave_incl_scan(h);
                if ((tid & 63) == 63) wsum[tid >> 6] = incl;
            }
            __syncthreads();
            if (tid < 256) {
                int before = 0;
                for (int w = 0; w < (tid >> 6); ++w) before += wsum[w];
                const int ge = before + incl;  // keys whose digit >= 255 - tid
                if (ge >= krem && ge - h < krem) {  // exactly one thread
                    s_digit = 255 - tid;
                    s_above = ge - h;
                }
            }
            __syncthreads();
            prefix |= static_cast<uint32_t>(s_digit) << shift;
            krem -= s_above;
            __syncthreads();
        }
        tau = kmin + prefix;
        need_eq = krem;
    }

    // compaction in ascending index order
    int total = 0;
    int n_eq = 0;
    if (mode == 2) {
#pragma unroll
        for (int r = 0; r < KPT; ++r) n_eq += (base + r < NC && key[r] == tau) ? 1 : 0;
    }
    int eq_rank = block_excl_scan(n_eq, wsum, &total);
    bool sel[KPT];
    int n_sel = 0;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const bool valid = base + r < NC;
        bool take;
        if (mode == 0)
            take = false;
        else if (mode == 1)
            take = valid;
        else if (valid && key[r] > tau)
            take = true;
        else if (valid && key[r] == tau) {
            take = eq_rank < need_eq;
            ++eq_rank;
        } else
            take = false;
        sel[r] = take;
        n_sel += take ? 1 : 0;
    }
    int pos = block_excl_scan(n_sel, wsum, &total);
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        if (sel[r]) out[pos++] = base + r;
    }
    // local blocks follow the picked candidates (their ids are the largest)
    for (int t = tid; t < nl; t += kTopnThreads) out[total + t] = NC + t;
    for (int t = total + nl + tid; t < a.n_max; t += kTopnThreads) out[t] = -1;
    if (tid == 0) a.cnt[grp] = total + nl;
}

template <int DT, int DESC, int D>
hipError_t launch_score(const ScoreParams& p, hipStream_t stream) {
    constexpr int DE = DESC == kMinMax ? DT : kF32;
    constexpr int EPL = DE == kBF16 ? 8 : 4;
    constexpr int BPW = (kScoreThreads / (D / EPL)) * kScoreIters;
    dim3 grid((p.c.max_blocks + BPW - 1) / BPW, p.c.B * p.c.Hkv);
    hipLaunchKernelGGL((score_kernel<DT, DESC, D>), grid, dim3(kScoreThreads), 0, stream, p);
    return hipGetLastError();
}

template <int DT, int DESC>
hipError_t launch_score_d(const ScoreParams& p, hipStream_t stream) {
    return p.c.d == 64 ? launch_score<DT, DESC, 64>(p, stream) : launch_score<DT, DESC, 128>(p, stream);
}

template <int KPT>
hipError_t launch_topn_k(const TopnParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((topn_kernel<KPT>), dim3(p.c.B * p.c.Hkv), dim3(kTopnThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int topn_keys_per_thread(int max_blocks) {
    for (int k = 1; k <= 32; k <<= 1)
        if (k * kTopnThreads >= max_blocks) return k;
    return 0;
}

hipError_t launch_select(const CacheArgs& c, const SelectArgs& s, hipStream_t stream) {
    ScoreParams sp{c, s};
    hipError_t err;
    if (c.dtype == kBF16)
        err = c.desc_kind == kMinMax ? launch_score_d<kBF16, kMinMax>(sp, stream)
                                     : launch_score_d<kBF16, kMeanPool>(sp, stream);
    else
        err = c.desc_kind == kMinMax ? launch_score_d<kF32, kMinMax>(sp, stream)
                                     : launch_score_d<kF32, kMeanPool>(sp, stream);
    if (err != hipSuccess) return err;
    TopnParams tp{c, s};
    switch (topn_keys_per_thread(c.max_blocks)) {
        case 1: return launch_topn_k<1>(tp, stream);
        case 2: return launch_topn_k<2>(tp, stream);
        case 4: return launch_topn_k<4>(tp, stream);
        case 8: return launch_topn_k<8>(tp, stream);
        case 16: return launch_topn_k<16>(tp, stream);
        case 32: return launch_topn_k<32>(tp, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bsa
