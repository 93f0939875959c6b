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
//   with 16-byte loads and reduced with DPP row adds; the group's query
//   weights are formed once per workgroup in LDS.  A variant also carries
//   the decode step's append (one extra workgroup per group, see
//   append_score_kernel).
// Kernel 2 (top-n): one 1024-thread workgroup per group holds the candidate
//   scores in registers as order-preserving uint32 keys and finds the n-th
//   largest key with an MSB-first radix select (digits taken from
//   key - min_key so that the first digit already spreads the keys): the
//   first pass histograms every key (per-wave LDS histograms), the keys left
//   in the threshold's digit are gathered into an LDS list and wave 0
//   finishes the search on it.  The kept blocks are then compacted in
//   ascending index order with one block-wide prefix scan (ties at the
//   threshold go to the lower index), the local blocks appended and the row
//   padded with -1.  Keys per thread are sized for the capacity; slots past
//   the row's candidates hold the key 0 (below every real key), and waves
//   holding only such keys skip the per-key work.  With a gate-bias output
//   ("Simple Attention Sparsification", Method: softmax gates over the
//   candidate blocks, log g added to a kept block's logits) the kernel also
//   forms the softmax normaliser over all candidates and writes each kept
//   block's log-gate beside its id.
#include "bsa_device.h"
#include "bsa_internal.h"
#include "kv_write_block.h"

namespace bsa {

namespace {

#ifndef BSA_SCORE_THREADS
#define BSA_SCORE_THREADS 256
#endif
constexpr int kScoreThreads = BSA_SCORE_THREADS;
#ifndef BSA_SCORE_ITERS
#define BSA_SCORE_ITERS 8
#endif
constexpr int kScoreIters = BSA_SCORE_ITERS;
constexpr int kTopnThreads = 1024;
constexpr int kTopnWaves = kTopnThreads / kWave;
constexpr int kAliveCap = 2048;  // keys gathered after the first radix pass
struct ScoreParams {
    CacheArgs c;
    SelectArgs s;
    int stride;  // score row stride (floats)
};

// 16-byte chunk of descriptor elements as floats
template <int DE>  // descriptor element kind: kF32 / kBF16
struct Chunk;
template <>
struct Chunk<kBF16> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void unpack(const u32x4 w, float* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            out[2 * k] = __uint_as_float(w[k] << 16);
            out[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void load(const void* p, float* out) {
        unpack(*reinterpret_cast<const u32x4*>(p), out);
    }
};
template <>
struct Chunk<kF32> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void unpack(const u32x4 w, float* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = __uint_as_float(w[k]);
    }
    static __device__ __forceinline__ void load(const void* p, float* out) {
        unpack(*reinterpret_cast<const u32x4*>(p), out);
    }
};

// Descriptor row geometry: BR bytes per block (both rows for min/max), read
// as 16-byte pieces, LPB = BR/16 lanes per block, so that one wave load
// instruction covers 64/LPB whole blocks = one contiguous KiB.  A lane of a
// min/max block owns 8 (bf16) or 4 (fp32) channels of either the min row
// (paired with Q-) or the max row (paired with Q+); a mean-pool lane owns 4
// channels of the key sum (paired with W sum_h q_h).
template <int DT, int DESC, int D>
struct ScoreGeom {
    static constexpr int ES = (DESC == kMinMax) ? (DT == kBF16 ? 2 : 4) : 4;  // bytes/elem
    static constexpr int EPL = 16 / ES;                                          // elems/lane
    static constexpr int BR = (DESC == kMinMax ? 2 : 1) * D * ES;                // bytes/block
    static constexpr int LPB = BR / 16;                                          // lanes/block
    static constexpr int BPL = kWave / LPB;                // blocks per wave load
    static constexpr int BPW = BPL * (kScoreThreads / kWave) * kScoreIters;  // blocks per WG
};

// How a scoring workgroup forms the group's query weights (step 0 and 2
// below): per-thread loads of up to 16 or up to 4 heads summed into LDS
// behind a barrier, or (min/max, up to 4 heads) per-lane loads of the
// lane's own channels with no LDS and no barrier.  The per-lane form does
// 8x the VALU work, which a launch that fills the chip hides behind its
// descriptor stream (a 512K-token select of 8 groups, 1032 workgroups:
// 15.85 -> 15.56 us per call) and a small one does not (a 32K-token one,
// 72 workgroups: 8.17 -> 8.29 us).
constexpr int kQ16 = 0, kQ4 = 1, kQLane = 2;
constexpr int kQLaneMinWorkgroups = 256;

template <int DESC>
int score_qv(int G, int workgroups) {
    if (G > 4) return kQ16;
    return (DESC == kMinMax && workgroups >= kQLaneMinWorkgroups) ? kQLane : kQ4;
}

// Scores of the candidate blocks [bx * BPW, (bx + 1) * BPW) of group grp.
template <int DT, int DESC, int D, int QV>
__device__ __forceinline__ void score_block(const ScoreParams& p, int bx, int grp) {
    typedef typename Elem<DT>::T E;
    typedef ScoreGeom<DT, DESC, D> Gm;
    constexpr int EPL = Gm::EPL, LPB = Gm::LPB, BPL = Gm::BPL;
    constexpr int DE = (Gm::ES == 2) ? kBF16 : kF32;
    const CacheArgs& c = p.c;
    const SelectArgs& a = p.s;
    const int s = grp / c.Hkv;
    const int kvh = grp - s * c.Hkv;
    const int c0 = bx * Gm::BPW;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lp = lane % LPB;   // lane position inside the block's bytes
    const int bl = lane / LPB;   // which block of the wave load
    // channels of this lane and which descriptor row it reads
    const bool max_row = (DESC == kMinMax) && (lp * 16 >= D * Gm::ES);
    const int ch0 = (lp * EPL) % D;

    // 0. the group's queries (G <= 16 values per thread, known before any
    //    load), requested ahead of the descriptors: the sums in step 2 then
    //    wait for these alone, in one round trip, while the descriptors are
    //    still arriving (a loop over the heads with a load per iteration would
    //    wait for every descriptor load, then make one trip per head).
    //    Min/max with up to 4 heads: each lane instead reads, per head, the
    //    16 bytes of the channels it scores and forms its own weights, so
    //    the weights need no LDS and no workgroup barrier.
    constexpr int kMaxG = (QV == kQ16) ? 16 : 4;
    constexpr bool kLaneW = QV == kQLane;
    static_assert(!kLaneW || DESC == kMinMax, "per-lane weights are min/max only");
    const E* qg = static_cast<const E*>(a.q) + (static_cast<int64_t>(s) * c.Hq + kvh * c.G) * D;
    // the sequence length, in the same round trip (a scalar load would be
    // placed after the descriptors have arrived and cost a trip of its own)
    const int T_v = load_int_vgpr(c.seq_lens + s);
    // (every thread issues all kMaxG loads, heads past G at head 0's address:
    //  no branch and no select waits on a loaded value here; groups of up to
    //  4 heads have instances of their own, with 4 loads per thread instead
    //  of 16)
    const int qi = tid % D;
    typename Elem<DT>::T qraw[kLaneW ? 1 : kMaxG];
    u32x4 qc[kLaneW ? kMaxG : 1];
    if constexpr (kLaneW) {
#pragma unroll
        for (int h = 0; h < kMaxG; ++h)
            qc[h] = *reinterpret_cast<const u32x4*>(qg + (h < c.G ? h : 0) * D + ch0);
    } else {
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) qraw[h] = qg[(h < c.G ? h : 0) * D + qi];
    }

    // 1. descriptor loads next, before anything they do not depend on is
    //    known: indices are clamped to the descriptor array (max_blocks rows),
    //    results past the candidates are discarded below, so every load of
    //    the workgroup is in flight while the length arrives.
    const char* base = static_cast<const char*>(c.desc) +
                       (static_cast<int64_t>(grp) * c.max_blocks) * Gm::BR + lp * 16;
    float x[kScoreIters][EPL];
#pragma unroll
    for (int it = 0; it < kScoreIters; ++it) {
        const int j = min(c0 + (it * (kScoreThreads / kWave) + wave) * BPL + bl, c.max_blocks - 1);
        Chunk<DE>::load(base + static_cast<int64_t>(j) * Gm::BR, x[it]);
    }
    // mean-pool: the gate matrix (row-major bf16), requested with the
    // descriptors since it depends on nothing else.  It is read in 16-byte
    // pieces, LPR lanes per row, so that every wave load covers whole rows.
    constexpr int LPR = D / 8;                    // lanes per gate row
    constexpr int RPI = kWave / LPR;              // rows per wave load
    constexpr int NWV = kScoreThreads / kWave;    // waves per workgroup
    constexpr int NI = D / (NWV * RPI);           // loads per thread
    static_assert(NI * NWV * RPI == D, "gate matrix split");
    u32x4 wl[NI];
    if (DESC == kMeanPool) {
        const uint16_t* wg = static_cast<const uint16_t*>(a.gate_w) + (lane % LPR) * 8;
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            const int r = (k * NWV + wave) * RPI + lane / LPR;
            wl[k] = *reinterpret_cast<const u32x4*>(wg + r * D);
        }
    }
    // Every load above is issued before anything waits for one: without
    // this fence (the LDS path's barrier is one too) the compiler moves the
    // length's early exit ahead of the loads and sinks each query load into
    // the test of its head, making one round trip per load.
    asm volatile("" ::: "memory");
    // 2. the group's query weights, once per workgroup, into LDS:
    //    min/max: Q-_i = sum_h min(q_hi, 0) (pairs with the min row) and
    //             Q+_i = sum_h max(q_hi, 0) (pairs with the max row);
    //    mean-pool: u_i = sum_h q_hi, then w = W u.
    //    (heads summed in order h = 0..G-1)
    __shared__ float qw[2 * D];
    if constexpr (kLaneW) {
        // formed per lane below
    } else if (DESC == kMinMax) {
        if (tid < 2 * D) {
            const bool upper = tid >= D;
            float acc = 0.f;
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
                const float xq = Elem<DT>::load(qraw, h);
                if (h < c.G) acc += upper ? fmaxf(xq, 0.f) : fminf(xq, 0.f);
            }
            qw[tid] = acc;
        }
    } else {
        if (tid < D) {
            float acc = 0.f;
#pragma unroll
            for (int h = 0; h < kMaxG; ++h)
                if (h < c.G) acc += Elem<DT>::load(qraw, h);
            qw[tid] = acc;
        }
    }
    const int T = __builtin_amdgcn_readfirstlane(T_v);
    const int NB = (T + c.block - 1) / c.block;
    // scored: the candidates, and with a log-gate bias every historical
    // block (all but the gate_current trailing ones, kept local ones included)
    const int NC = NB - min(a.gate_bias ? a.gate_current : a.n_local, NB);
    if constexpr (!kLaneW) __syncthreads();
    if (c0 >= NC) return;  // uniform across the workgroup
    float wv[EPL];
    if constexpr (kLaneW) {
        // the same sums as the LDS path forms, head by head from 0
#pragma unroll
        for (int e = 0; e < EPL; ++e) wv[e] = 0.f;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            float qv[EPL];
            Chunk<DE>::unpack(qc[h], qv);
            if (h < c.G) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) wv[e] += max_row ? fmaxf(qv[e], 0.f) : fminf(qv[e], 0.f);
            }
        }
    } else if (DESC == kMinMax) {
        const float* src = qw + (max_row ? D : 0) + ch0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) wv[e] = src[e];
    } else {
        // w = W u in LDS: each lane forms the 8-channel piece of the rows
        // it loaded above, then the LPR pieces of a row are added in
        // channel order (rows padded by one float against bank conflicts)
        __shared__ float w_part[D * (LPR + 1)];
        __shared__ float w_s[D];
        {
            const int j = lane % LPR;
            float uv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) uv[e] = qw[8 * j + e];
#pragma unroll
            for (int k = 0; k < NI; ++k) {
                const int r = (k * NWV + wave) * RPI + lane / LPR;
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc += __uint_as_float(wl[k][e] << 16) * uv[2 * e];
                    acc += __uint_as_float(wl[k][e] & 0xffff0000u) * uv[2 * e + 1];
                }
                w_part[r * (LPR + 1) + j] = acc;
            }
        }
        __syncthreads();
        if (tid < D) {
            float acc = 0.f;
#pragma unroll
            for (int jj = 0; jj < LPR; ++jj) acc += w_part[tid * (LPR + 1) + jj];
            w_s[tid] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPL; ++e) wv[e] = w_s[ch0 + e];
    }

    float part[kScoreIters];
#pragma unroll
    for (int it = 0; it < kScoreIters; ++it) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc += wv[e] * x[it][e];
        part[it] = acc;
    }
    float* out = a.scores + static_cast<int64_t>(grp) * p.stride;
#pragma unroll
    for (int it = 0; it < kScoreIters; ++it) {
        const float tot = group_sum_last<LPB>(part[it]);
        const int j = c0 + (it * (kScoreThreads / kWave) + wave) * BPL + bl;
        if (lp == LPB - 1 && j < NC) {
            float v = tot;
            if (DESC == kMeanPool) v = v / static_cast<float>(min(c.block, T - j * c.block));
            out[j] = v;
        }
    }
}

template <int DT, int DESC, int D, int QV>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(ScoreParams p) {
    score_block<DT, DESC, D, QV>(p, static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y));
}

// Append of one token per sequence fused with the scoring: workgroups
// x < score_gx score, the others write the new token and update the
// descriptor of its block.  The two roles touch disjoint data -- the token
// lands in the last block, which is local and never scored -- so they can
// share one launch.
template <int DT, int DESC, int D, int QV>
__global__ __launch_bounds__(kScoreThreads) void append_score_kernel(ScoreParams sp, KvWriteParams kp,
                                                                     int score_gx) {
    const int bx = static_cast<int>(blockIdx.x);
    if (bx < score_gx)
        score_block<DT, DESC, D, QV>(sp, bx, static_cast<int>(blockIdx.y));
    else
        kv_write_block<DT, DESC, kScoreThreads>(kp, bx - score_gx, static_cast<int>(blockIdx.y));
}

// ----------------------------- top-n ---------------------------------------

struct TopnParams {
    CacheArgs c;
    SelectArgs s;
    int stride;  // score row stride (floats), a multiple of 4
};

template <int KPT>
__global__ __launch_bounds__(kTopnThreads) void topn_kernel(TopnParams p) {
    const CacheArgs& c = p.c;
    const SelectArgs& a = p.s;
    // one private histogram per wave (LDS atomics then only collide within
    // a wave instruction, not across the 16 waves), summed into hsum
    __shared__ int hist[kTopnWaves][256];
    __shared__ int hsum[256];
    __shared__ int wsum[kTopnWaves];
    __shared__ uint32_t alive_s[kAliveCap];  // key - kmin of the keys alive after pass 1
    __shared__ int n_alive_s;
    __shared__ uint32_t res_s[2];
    __shared__ uint32_t red_min[kTopnWaves], red_max[kTopnWaves];
    __shared__ float red_z[kTopnWaves];
    __shared__ float red_x[kTopnWaves];  // largest extra historical score per wave
    __shared__ uint32_t w0keys[KPT * kWave];  // wave 0's keys, slot r * 64 + lane

    const int grp = blockIdx.x;
    const int s = grp / c.Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int32_t* out = a.idx + static_cast<int64_t>(grp) * a.n_max;
    const float* sc = a.scores + static_cast<int64_t>(grp) * p.stride;
    const int base = tid * KPT;

    // the sequence length with a buffer load (a VGPR until it is needed) and
    // every score group of the thread, all in one round trip: the score loads
    // depend on nothing but the row's capacity (a multiple of 4; groups past
    // it read the row's first group), and nothing waits for a load until all
    // have been issued (a load followed by its conversion would wait for it
    // before the next load went out)
    const int T_v = load_int_vgpr(c.seq_lens + s);
    floatx4 v[KPT >= 4 ? KPT / 4 : 1];
    float v1[KPT >= 4 ? 1 : KPT];
    if constexpr (KPT >= 4) {
#pragma unroll
        for (int r = 0; r < KPT; r += 4) {
            const int g0 = (base + r + 4 <= p.stride) ? base + r : 0;
            v[r / 4] = *reinterpret_cast<const floatx4*>(sc + g0);
        }
    } else {
#pragma unroll
        for (int r = 0; r < KPT; ++r) v1[r] = sc[(base + r < p.stride) ? base + r : 0];
    }
    const int T = __builtin_amdgcn_readfirstlane(T_v);
    const int NB = (T + c.block - 1) / c.block;
    const int nl = min(a.n_local, NB);
    const int NC = NB - nl;
    const int n = block_count(NB, c.block, a.budget_tokens, a.sparsity_bp, a.n_local, a.n_min);
    const int K = n - nl;  // candidates to pick

    // Slots past the candidates hold the key 0, below every real key (the
    // scores are never NaN, so the smallest real key, that of -inf, is
    // 0x007fffff).  It never passes key > tau or key == tau (tau >= the
    // smallest real key) and is skipped by the radix passes' key != 0 test,
    // so no phase needs a per-key bounds test.
    // A wave whose first slot is past the candidates holds only the key 0
    // (KPT is sized for the capacity, the row for the current length): such
    // a wave skips every per-key loop below but takes part in every barrier.
    const bool live = wave * kWave * KPT < NC;  // wave-uniform
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) key[r] = 0u;
    if constexpr (KPT >= 4) {
        // the groups loaded above; slots past the candidates get the key 0
        if (live) {
#pragma unroll
            for (int r = 0; r < KPT; r += 4)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    key[r + k] = (base + r + k < NC) ? float_key(v[r / 4][k]) : 0u;
        }
    } else if (live) {
#pragma unroll
        for (int r = 0; r < KPT; ++r)
            key[r] = (base + r < NC) ? float_key(v1[r]) : 0u;
    }

    // mode: 0 = pick none, 1 = pick every candidate, 2 = threshold select
    const int mode = (K <= 0) ? 0 : (K >= NC ? 1 : 2);

    // Log-gate bias ("Simple Attention Sparsification", Method): gates are
    // softmax(tau * s) over all NC candidates, so a kept candidate's bias is
    // tau * (s_j - smax) - ln sum_c exp(tau * (s_c - smax)).  smax is the
    // largest key, which the threshold select reduces anyway; each wave's
    // part of the sum goes to red_z and is added up after a barrier the
    // select already has.  In the threshold select the parts are formed
    // while wave 0 alone finishes the radix passes and the other waves
    // would only wait: wave 1 also forms wave 0's part, from a copy of
    // wave 0's keys in LDS.
    // Only picked candidates carry a bias, so with nothing picked there is
    // no normaliser to form.
    float* bias_out = a.gate_bias ? a.gate_bias + static_cast<int64_t>(grp) * a.n_max : nullptr;
    const float tau_l2 = a.gate_tau * kLog2e;
    float g_smax = 0.f, g_lnz = 0.f;
    // Historical blocks past the candidates: the kept local blocks before the
    // gate_current current ones.  They are scored (after the candidates in
    // the score row), enter the normaliser and carry their own log-gate;
    // thread t handles extras t, t + 1024, ... (usually none or one).
    const int n_extra = bias_out ? max(0, nl - min(a.gate_current, NB)) : 0;
    // a normaliser is needed when some kept block is historical
    const bool gated = bias_out != nullptr && (mode != 0 || n_extra > 0);  // uniform
    // this wave's part of sum_h exp(tau * (s_h - smax)), into red_z[wave]
    auto gate_sum_part = [&]() __attribute__((always_inline)) {
        float z = 0.f;
        if (live) {
#pragma unroll
            for (int r = 0; r < KPT; ++r)
                if (key[r] != 0u)
                    z += __builtin_amdgcn_exp2f(tau_l2 * (key_float(key[r]) - g_smax));
        }
        for (int e = tid; e < n_extra; e += kTopnThreads)
            z += __builtin_amdgcn_exp2f(tau_l2 * (sc[NC + e] - g_smax));
        z = wave_sum(z);
        if (lane == 0) red_z[wave] = z;
    };
    // the largest extra score of this thread (-inf if none), for smax
    auto extra_max = [&]() __attribute__((always_inline)) {
        float m = -INFINITY;
        for (int e = tid; e < n_extra; e += kTopnThreads) m = fmaxf(m, sc[NC + e]);
        return m;
    };
    // wave 0's part, formed by another wave from w0keys (the same terms in
    // the same order as wave 0 would add them)
    auto gate_sum_wave0 = [&]() __attribute__((always_inline)) {
        float z = 0.f;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const uint32_t k = w0keys[r * kWave + lane];
            if (k != 0u) z += __builtin_amdgcn_exp2f(tau_l2 * (key_float(k) - g_smax));
        }
        // and the extras wave 0's threads hold
        for (int e = lane; e < n_extra; e += kTopnThreads)
            z += __builtin_amdgcn_exp2f(tau_l2 * (sc[NC + e] - g_smax));
        z = wave_sum(z);
        if (lane == 0) red_z[0] = z;
    };
    auto gate_finish = [&]() __attribute__((always_inline)) {  // after a barrier
        float zt = 0.f;
#pragma unroll
        for (int w = 0; w < kTopnWaves; ++w) zt += red_z[w];
        g_lnz = logf(zt);
    };
    auto gate = [&](uint32_t k) __attribute__((always_inline)) {
        return a.gate_tau * (key_float(k) - g_smax) - g_lnz;
    };

    if (mode != 2 && gated) {
        uint32_t lmax = 0u;
        if (live) {
#pragma unroll
            for (int r = 0; r < KPT; ++r) lmax = max(lmax, key[r]);
        }
        const float xm = extra_max();
        if (xm != -INFINITY) lmax = max(lmax, float_key(xm));
        lmax = wave_max_u32(lmax);
        if (lane == 0) red_max[wave] = lmax;
        __syncthreads();
        uint32_t kmx = 0u;
#pragma unroll
        for (int w = 0; w < kTopnWaves; ++w) kmx = max(kmx, red_max[w]);
        g_smax = key_float(kmx);
        gate_sum_part();
        __syncthreads();
        gate_finish();
    }
    if (mode == 1) {
        if (live) {
#pragma unroll
            for (int r = 0; r < KPT; ++r) {
                if (base + r < NC) {
                    out[base + r] = base + r;
                    if (gated) bias_out[base + r] = gate(key[r]);
                }
            }
        }
    }
    uint32_t tau = 0;
    int need_eq = 0;
    if (mode == 2) {
        // minimum of key - 1 (the sentinel wraps to the top), maximum of key
        uint32_t lmin = 0xffffffffu, lmax = 0u;
        if (live) {
#pragma unroll
            for (int r = 0; r < KPT; ++r) {
                lmin = min(lmin, key[r] - 1u);
                lmax = max(lmax, key[r]);
            }
        }
        lmin = wave_min_u32(lmin);
        lmax = wave_max_u32(lmax);
        // the normaliser's maximum also covers the extra historical blocks
        const float xm = gated ? wave_max(extra_max()) : -INFINITY;
        if (lane == 0) {
            red_min[wave] = lmin;
            red_max[wave] = lmax;
            red_x[wave] = xm;
        }
        __syncthreads();
        uint32_t kmin = 0xffffffffu, kmax = 0u;
        float xmax = -INFINITY;
#pragma unroll
        for (int w = 0; w < kTopnWaves; ++w) {
            kmin = min(kmin, red_min[w]);
            kmax = max(kmax, red_max[w]);
            xmax = fmaxf(xmax, red_x[w]);
        }
        kmin += 1u;
        g_smax = fmaxf(key_float(kmax), xmax);
        bool z_pending = gated;  // the normaliser's parts are still to form
        const uint32_t range = kmax - kmin;
        uint32_t prefix = 0;  // of key - kmin, above the current digit
        int krem = K;
        int shift = (range == 0u) ? 0 : 32 - __clz(static_cast<int>(range));
        // digit search, by every wave on its own copy of the answer: lane L
        // covers digits 255-4L .. 252-4L (descending), counts are suffix sums;
        // returns the digit holding the krem-th largest alive key and how
        // many alive keys lie in higher digits
        auto find_digit = [&](const int* h, int& digit, int& above) __attribute__((always_inline)) {
            find_digit256(h, krem, lane, digit, above);
        };
        // one radix pass over every key of the workgroup
        auto block_pass = [&]() __attribute__((always_inline)) {
            const int dbits = min(8, shift);
            shift -= dbits;
            const int hi = shift + dbits;
            int* hw = hist[wave];
#pragma unroll
            for (int i = 0; i < 4; ++i) hw[lane + 64 * i] = 0;  // nobody reads it now
            if (live) {
#pragma unroll
                for (int r = 0; r < KPT; ++r) {
                    const uint32_t kr = key[r] - kmin;
                    const bool alive = key[r] != 0u && (hi >= 32 || ((kr >> hi) == (prefix >> hi)));
                    if (alive) atomicAdd(&hw[(kr >> shift) & ((1u << dbits) - 1u)], 1);
                }
            }
            if (tid == 0) n_alive_s = 0;  // for the alive-key list below
            __syncthreads();
            if (tid < 256) {
                int t = 0;
#pragma unroll
                for (int w = 0; w < kTopnWaves; ++w) t += hist[w][tid];
                hsum[tid] = t;
            }
            __syncthreads();
            int digit, above;
            find_digit(hsum, digit, above);
            prefix |= static_cast<uint32_t>(digit) << shift;
            krem -= above;
            return digit;
        };

        // The first pass runs over every key.  The keys still alive after it
        // (those in the threshold's digit) are usually a few percent of them:
        // they are gathered into LDS and the remaining passes run on that list
        // in wave 0 alone, with no workgroup barriers.  A list too long for
        // the buffer keeps to whole-workgroup passes.
        if (shift > 0) {
            const int d1 = block_pass();
            const int n_alive = hsum[d1];
            if (shift > 0 && n_alive <= kAliveCap) {
                // list slots: a lane mask of the alive keys, a wave prefix of
                // the lane counts and one LDS atomic per wave for its base
                if (live) {
                    uint32_t am = 0u;
#pragma unroll
                    for (int r = 0; r < KPT; ++r) {
                        const uint32_t kr = key[r] - kmin;
                        am |= (key[r] != 0u && (kr >> shift) == (prefix >> shift)) ? (1u << r) : 0u;
                    }
                    const int cnt_l = __builtin_popcount(am);
                    const int incl = wave_incl_scan(cnt_l);
                    int wbase = 0;
                    if (lane == 63) wbase = atomicAdd(&n_alive_s, incl);
                    int at = __builtin_amdgcn_readlane(wbase, 63) + incl - cnt_l;
#pragma unroll
                    for (int r = 0; r < KPT; ++r) {
                        if (am & (1u << r)) alive_s[at++] = key[r] - kmin;
                    }
                }
                if (z_pending && wave == 0) {
#pragma unroll
                    for (int r = 0; r < KPT; ++r) w0keys[r * kWave + lane] = key[r];
                }
                __syncthreads();
                if (wave == 0) {
                    __builtin_amdgcn_s_setprio(2);  // the other waves only wait for it
                    while (shift > 0) {
                        const int dbits = min(8, shift);
                        shift -= dbits;
                        const int hi = shift + dbits;
                        int* hw = hist[0];
#pragma unroll
                        for (int i = 0; i < 4; ++i) hw[lane + 64 * i] = 0;
                        for (int i = lane; i < n_alive; i += kWave) {
                            const uint32_t kr = alive_s[i];
                            if ((kr >> hi) == (prefix >> hi))
                                atomicAdd(&hw[(kr >> shift) & ((1u << dbits) - 1u)], 1);
                        }
                        int digit, above;
                        find_digit(hw, digit, above);
                        prefix |= static_cast<uint32_t>(digit) << shift;
                        krem -= above;
                    }
                    if (lane == 0) {
                        res_s[0] = prefix;
                        res_s[1] = static_cast<uint32_t>(krem);
                    }
                    __builtin_amdgcn_s_setprio(0);
                } else if (z_pending) {
                    gate_sum_part();
                    if (wave == 1) gate_sum_wave0();
                }
                z_pending = false;
                __syncthreads();
                prefix = res_s[0];
                krem = static_cast<int>(res_s[1]);
                shift = 0;
            }
            while (shift > 0) block_pass();
        }
        tau = kmin + prefix;
        need_eq = krem;
        if (z_pending) gate_sum_part();  // added up after the scan's barrier below

        // one packed scan: (keys > tau) << 16 | (keys == tau), per thread;
        // the positions of those keys are kept as bit masks
        uint32_t gt_m = 0u, eq_m = 0u;
        if (live) {
#pragma unroll
            for (int r = 0; r < KPT; ++r) {
                gt_m |= (key[r] > tau) ? (1u << r) : 0u;
                eq_m |= (key[r] == tau) ? (1u << r) : 0u;
            }
        }
        const int n_eq = __builtin_popcount(eq_m);
        const int packed = (__builtin_popcount(gt_m) << 16) | n_eq;
        const int incl = wave_incl_scan(packed);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        if (gated) gate_finish();
        int before = 0;
#pragma unroll
        for (int w = 0; w < kTopnWaves; ++w) before += (w < wave) ? wsum[w] : 0;
        const int excl = before + incl - packed;
        const int eq_rank = excl & 0xffff;
        int pos = (excl >> 16) + min(eq_rank, need_eq);
        // this thread's keys equal to tau are ranked eq_rank, eq_rank + 1, ...
        // (ascending index); those ranked below need_eq are taken
        uint32_t take_m = gt_m;
        for (int k = max(0, min(need_eq - eq_rank, n_eq)); k > 0; --k) {
            take_m |= eq_m & (0u - eq_m);
            eq_m &= eq_m - 1u;
        }
        // only the taken keys, lowest index first.  The rows are written
        // through buffer descriptors sized to n_max entries: a store takes a
        // 32-bit byte offset, and the hardware drops a store past the row
        // (pos >= n_max), which replaces the bounds test.
        const __amdgpu_buffer_rsrc_t out_rs = __builtin_amdgcn_make_buffer_rsrc(
            out, 0, a.n_max * static_cast<int>(sizeof(int32_t)), kBufferWord3);
        int off = pos * static_cast<int>(sizeof(int32_t));
        if (gated) {
            const __amdgpu_buffer_rsrc_t bias_rs = __builtin_amdgcn_make_buffer_rsrc(
                bias_out, 0, a.n_max * static_cast<int>(sizeof(float)), kBufferWord3);
            // a taken key's bias needs the key itself: the keys are walked in
            // groups of four, so picking one out of the registers takes a
            // three-step select chain (no dynamic register indexing)
            constexpr int GS = KPT < 4 ? KPT : 4;
#pragma unroll
            for (int g0 = 0; g0 < KPT; g0 += GS) {
                uint32_t m = (take_m >> g0) & ((1u << GS) - 1u);
                while (m != 0u) {
                    const int rr = __builtin_ctz(m);
                    uint32_t kk = key[g0];
#pragma unroll
                    for (int i = 1; i < GS; ++i) kk = (rr == i) ? key[g0 + i] : kk;
                    __builtin_amdgcn_raw_buffer_store_b32(base + g0 + rr, out_rs, off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gate(kk)), bias_rs, off,
                                                          0, 0);
                    off += static_cast<int>(sizeof(int32_t));
                    m &= m - 1u;
                }
            }
        } else {
            while (take_m != 0u) {
                __builtin_amdgcn_raw_buffer_store_b32(base + __builtin_ctz(take_m), out_rs, off, 0,
                                                      0);
                off += static_cast<int>(sizeof(int32_t));
                take_m &= take_m - 1u;
            }
        }
    }
    const int picked = (mode == 0) ? 0 : K;
    // local blocks follow the picked candidates (their ids are the largest)
    for (int t = tid; t < nl; t += kTopnThreads) out[picked + t] = NC + t;
    for (int t = picked + nl + tid; t < a.n_max; t += kTopnThreads) out[t] = -1;
    if (bias_out) {
        // the extra historical blocks lead the local blocks; the current
        // blocks and the padding get 0
        for (int t = picked + tid; t < a.n_max; t += kTopnThreads) {
            const int e = t - picked;
            bias_out[t] = (e < n_extra)
                              ? a.gate_tau * (sc[NC + e] - g_smax) - g_lnz
                              : 0.f;
        }
    }
    if (tid == 0) a.cnt[grp] = picked + nl;
}

template <int DT, int DESC, int D>
hipError_t launch_score(const ScoreParams& p, hipStream_t stream) {
    constexpr int BPW = ScoreGeom<DT, DESC, D>::BPW;
    dim3 grid((p.c.max_blocks + BPW - 1) / BPW, p.c.B * p.c.Hkv);
    switch (score_qv<DESC>(p.c.G, static_cast<int>(grid.x * grid.y))) {
        case kQLane:
            if constexpr (DESC == kMinMax) {
                hipLaunchKernelGGL((score_kernel<DT, DESC, D, kQLane>), grid, dim3(kScoreThreads), 0,
                                   stream, p);
                break;
            }
            [[fallthrough]];
        case kQ4:
            hipLaunchKernelGGL((score_kernel<DT, DESC, D, kQ4>), grid, dim3(kScoreThreads), 0, stream, p);
            break;
        default:
            hipLaunchKernelGGL((score_kernel<DT, DESC, D, kQ16>), grid, dim3(kScoreThreads), 0, stream, p);
    }
    return hipGetLastError();
}

template <int DT, int DESC>
hipError_t launch_score_d(const ScoreParams& p, hipStream_t stream) {
    return p.c.d == 64 ? launch_score<DT, DESC, 64>(p, stream) : launch_score<DT, DESC, 128>(p, stream);
}

template <int DT, int DESC, int D>
hipError_t launch_append_score(const ScoreParams& sp, const KvWriteParams& kp, hipStream_t stream) {
    constexpr int BPW = ScoreGeom<DT, DESC, D>::BPW;
    const int score_gx = (sp.c.max_blocks + BPW - 1) / BPW;
    // one token per sequence touches one block
    dim3 grid(score_gx + 1, sp.c.B * sp.c.Hkv);
    switch (score_qv<DESC>(sp.c.G, static_cast<int>(grid.x * grid.y))) {
        case kQLane:
            if constexpr (DESC == kMinMax) {
                hipLaunchKernelGGL((append_score_kernel<DT, DESC, D, kQLane>), grid, dim3(kScoreThreads),
                                   0, stream, sp, kp, score_gx);
                break;
            }
            [[fallthrough]];
        case kQ4:
            hipLaunchKernelGGL((append_score_kernel<DT, DESC, D, kQ4>), grid, dim3(kScoreThreads), 0,
                               stream, sp, kp, score_gx);
            break;
        default:
            hipLaunchKernelGGL((append_score_kernel<DT, DESC, D, kQ16>), grid, dim3(kScoreThreads), 0,
                               stream, sp, kp, score_gx);
    }
    return hipGetLastError();
}

template <int DT, int DESC>
hipError_t launch_append_score_d(const ScoreParams& sp, const KvWriteParams& kp, hipStream_t stream) {
    return sp.c.d == 64 ? launch_append_score<DT, DESC, 64>(sp, kp, stream)
                        : launch_append_score<DT, DESC, 128>(sp, kp, stream);
}

template <int KPT>
hipError_t launch_topn_k(const TopnParams& p, hipStream_t stream) {
    static_assert(KPT >= 4 || KPT == 1 || KPT == 2, "keys per thread");
    hipLaunchKernelGGL((topn_kernel<KPT>), dim3(p.c.B * p.c.Hkv), dim3(kTopnThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int score_stride(int max_blocks) { return (max_blocks + 3) & ~3; }

int topn_keys_per_thread(int max_blocks) {
    for (int k = 1; k <= 32; k <<= 1)
        if (k * kTopnThreads >= max_blocks) return k;
    return 0;
}

namespace {

hipError_t launch_topn(const CacheArgs& c, const SelectArgs& s, hipStream_t stream) {
    TopnParams tp{c, s, score_stride(c.max_blocks)};
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

}  // namespace

hipError_t launch_select(const CacheArgs& c, const SelectArgs& s, hipStream_t stream) {
    ScoreParams sp{c, s, score_stride(c.max_blocks)};
    hipError_t err;
    if (c.dtype == kBF16)
        err = c.desc_kind == kMinMax ? launch_score_d<kBF16, kMinMax>(sp, stream)
                                     : launch_score_d<kBF16, kMeanPool>(sp, stream);
    else
        err = c.desc_kind == kMinMax ? launch_score_d<kF32, kMinMax>(sp, stream)
                                     : launch_score_d<kF32, kMeanPool>(sp, stream);
    if (err != hipSuccess) return err;
    return launch_topn(c, s, stream);
}

hipError_t launch_append_score_only(const CacheArgs& c, const void* k_new, const void* v_new,
                                    const SelectArgs& s, hipStream_t stream) {
    ScoreParams sp{c, s, score_stride(c.max_blocks)};
    KvWriteParams kp{c, kModeAppend, k_new, v_new, 1, nullptr};
    if (c.dtype == kBF16)
        return c.desc_kind == kMinMax ? launch_append_score_d<kBF16, kMinMax>(sp, kp, stream)
                                      : launch_append_score_d<kBF16, kMeanPool>(sp, kp, stream);
    return c.desc_kind == kMinMax ? launch_append_score_d<kF32, kMinMax>(sp, kp, stream)
                                  : launch_append_score_d<kF32, kMeanPool>(sp, kp, stream);
}

hipError_t launch_append_select(const CacheArgs& c, const void* k_new, const void* v_new,
                                const SelectArgs& s, hipStream_t stream) {
    const hipError_t err = launch_append_score_only(c, k_new, v_new, s, stream);
    if (err != hipSuccess) return err;
    return launch_topn(c, s, stream);
}

}  // namespace bsa
