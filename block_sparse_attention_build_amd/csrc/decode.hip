// decode.hip -- exact softmax attention over the kept blocks (split over the
// kept tokens) and the log-sum-exp merge of the partial results.
//
// "Rectified Sparse Attention for Efficient Long-Sequence Generation",
// Summary: group block-sparse attention, all query heads of a GQA group
// reading the same kept blocks.  "Simple Attention Sparsification", Method:
// non-selected blocks are masked out of an exact, online softmax.
// Flash-Decoding (cited in the ReSA page's references): split the keys,
// merge the partial (o, lse) pairs.
//
// bf16 path (the bandwidth-critical kernel).  One workgroup = 8 waves = one
// (sequence, KV head, split), one workgroup per CU; the split is a contiguous
// range of 32-token tiles of the group's kept-block list, cut into units of
// unit_tiles tiles that the waves claim from an LDS counter.
// Per tile a wave issues 16-byte loads of 8 KiB of K and 8 KiB of V (d=128):
// every load instruction reads one contiguous KiB because the page layout
// stores each KiB as one matrix-core operand.  The wave then computes
//   S^T (32 tokens x 16 head columns) = K Q^T   with v_mfma_f32_16x16x32_bf16
// (the group's G <= 16 heads padded to 16 columns), an online softmax per
// head column (max across the 4 lane groups with two shuffles), and
//   O (16 heads x d) += P V
// where P is exactly the S^T accumulator the lane already holds (the V page
// layout orders tokens to match), split into bf16 hi + lo parts so that the
// weights keep ~16 mantissa bits.  K and V are read once per group, never
// once per head.  Each unit leaves a partial (max, sum, O) in LDS; the units
// are merged in unit order and the workgroup writes one normalised partial
// (o, base-2 lse) per head, which the merge kernel combines across splits.
// The gated instance ("Simple Attention Sparsification", Method: the o_SAS
// equation) adds each kept block's log-gate bias to its tokens' logits; the
// bias rides along with the block's page id, one wave-uniform value per tile.
//
// fp32 path.  Same split structure, plain VALU arithmetic (no fp32 matrix
// operand layout is defined for the pages); used by the small fp32 cases.
#include <math.h>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

// Tuning: threads per workgroup, waves per SIMD the bf16 kernel is
// register-limited to, and the number of workgroups a decode call aims for
// (one resident round on 256 CUs).
#ifndef BSA_DECODE_WAVES_PER_EU
#define BSA_DECODE_WAVES_PER_EU 2
#endif
#ifndef BSA_DECODE_TARGET_WGS
#define BSA_DECODE_TARGET_WGS 256
#endif
#ifndef BSA_DECODE_UNIT_LDS
#define BSA_DECODE_UNIT_LDS (112 * 1024)  // LDS bytes for the per-unit partials
#endif
#ifndef BSA_DECODE_UNITS_PER_SPLIT
#define BSA_DECODE_UNITS_PER_SPLIT 8  // units a split is cut into: one per wave
#endif
#ifndef BSA_DECODE_MAX_UNIT
#define BSA_DECODE_MAX_UNIT 8  // most tiles per unit, unless the LDS slots need more
#endif
constexpr int kLdsBytes = 160 * 1024;      // LDS of one CU
constexpr int kMaxSplitBlocks = 4096;      // kept blocks one split may cover
constexpr int kThreads = 256;     // fp32 kernel
constexpr int kWaves = kThreads / kWave;
constexpr int kDecThreads = 512;  // bf16 kernel: 8 waves

struct DecodeParams {
    CacheArgs c;
    DecodeArgs a;
    int max_blocks_per_wg;  // LDS slots for a split's block/page ids
    int unit_tiles;         // bf16: tiles per unit of work
    int max_units;          // bf16: LDS slots for unit partials
};

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// K and V tiles are read once per call: streaming (nontemporal) loads keep
// them from displacing reused lines in L2 and the last-level cache
__device__ __forceinline__ u32x4 ldg16_stream(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Merge the per-wave (m, l, O) held in LDS and write one partial per head.
// sm/sl: [kWaves][16]; so: [kWaves][G][D].
__device__ __forceinline__ void merge_waves_and_store(const float* sm, const float* sl,
                                                      const float* so, int G, int D,
                                                      float* o_part, float* lse_part,
                                                      int64_t head_row0, int S, int split) {
    for (int k = threadIdx.x; k < G * D; k += kThreads) {
        const int h = k / D;
        const int ch = k - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w * 16 + h]);
        const int64_t row = head_row0 + h;
        float* op = o_part + (row * S + split) * D;
        if (M == -INFINITY) {
            op[ch] = 0.f;
            if (ch == 0) lse_part[row * S + split] = -INFINITY;
            continue;
        }
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = exp2f(sm[w * 16 + h] - M);
            L += sl[w * 16 + h] * sc;
            acc += so[(w * G + h) * D + ch] * sc;
        }
        op[ch] = acc / L;
        if (ch == 0) lse_part[row * S + split] = M + log2f(L);
    }
}

// In-workgroup selection, for rows of at most KPT * kDecThreads candidate
// blocks.  Thread t holds the keys of blocks t, t + kDecThreads, ... (row r
// of the thread is block t + r * kDecThreads), so every score and page-id
// load of a row is one coalesced wave load.  The rule is the top-n kernel's
// ("Rectified Sparse Attention ...", Key points: dynamic top-n with local
// blocks and a minimum count; "Simple Attention Sparsification", Method:
// discrete Top-K with the current block always kept): n = block_count(NB),
// the nl = min(n_local, NB) last blocks, and the n - nl candidates of largest
// score (ties to the lower index), found by an MSB-first radix select over
// order-preserving uint32 keys.  The kept ids and their page ids go to
// kept/kept_page (LDS, ascending); returns n.  pg[r]: page id of the thread's
// block in row r; lpg: page id of local block tid (tid < nl).  scratch: LDS,
// kSelScratchInts ints, free again on return.  Ends with a barrier.
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kSelAliveCap = 1024;  // keys gathered after the first radix pass
constexpr int kSelMaxRows = 16;     // candidate rows per thread
constexpr int kSelScratchInts =
    kDecWaves * 256 + 256 + 2 * kDecWaves + 4 + kSelAliveCap + kSelMaxRows * kDecWaves;
static_assert(kSelMaxRows * kDecThreads == kDecodeSelectSlots, "candidate capacity");

template <int KPT>
__device__ __forceinline__ int select_kept(const DecodeArgs& a, int T, int block,
                                           const float (&sc)[KPT], const int (&pg)[KPT], int lpg,
                                           int* scratch, int* kept, int* kept_page) {
    static_assert(KPT <= kSelMaxRows, "rows per thread");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int* hist = scratch;                  // [kDecWaves][256] digit counts, one per wave
    int* hsum = hist + kDecWaves * 256;   // [256] their sum
    int* red = hsum + 256;                // [2][kDecWaves] min, max
    int* misc = red + 2 * kDecWaves;      // [4] alive-list length, prefix, keys left
    uint32_t* alive = reinterpret_cast<uint32_t*>(misc + 4);  // [kSelAliveCap] key - kmin
    int* rowcnt = misc + 4 + kSelAliveCap;  // [KPT][kDecWaves] packed (> tau) << 16 | (== tau)
    const int NB = (T + block - 1) / block;
    const int nl = min(a.n_local, NB);
    const int NC = NB - nl;
    const int n = block_count(NB, block, a.budget_tokens, a.sparsity_bp, a.n_local, a.n_min);
    const int K = n - nl;  // candidates to pick (0 <= K <= NC)
    // slots that are not candidates hold the key 0, below every real key
    uint32_t key[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) key[r] = (tid + r * kDecThreads < NC) ? float_key(sc[r]) : 0u;
    // keys > tau are taken, and the first need_eq keys == tau (by index):
    // K = 0 takes nothing (no key exceeds 0xffffffff), K = NC every candidate
    uint32_t tau = (K == 0) ? 0xffffffffu : 0u;
    int need_eq = 0;
    if (K > 0 && K < NC) {  // uniform
        uint32_t lmin = 0xffffffffu, lmax = 0u;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            lmin = min(lmin, key[r] - 1u);  // the key 0 wraps to the top
            lmax = max(lmax, key[r]);
        }
        lmin = wave_min_u32(lmin);
        lmax = wave_max_u32(lmax);
        if (lane == 0) {
            red[wave] = static_cast<int>(lmin);
            red[kDecWaves + wave] = static_cast<int>(lmax);
        }
        __syncthreads();
        uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
            kmin = min(kmin, static_cast<uint32_t>(red[w]));
            kmax = max(kmax, static_cast<uint32_t>(red[kDecWaves + w]));
        }
        kmin += 1u;
        const uint32_t range = kmax - kmin;
        uint32_t prefix = 0;  // of key - kmin, above the current digit
        int krem = K;         // keys still to take at or below the prefix
        int shift = (range == 0u) ? 0 : 32 - __clz(static_cast<int>(range));
        // a wave whose row-0 blocks are all past the candidates holds only keys 0
        const bool live = wave * kWave < NC;  // wave-uniform
        // one radix pass over every key of the workgroup; returns the digit
        auto block_pass = [&]() __attribute__((always_inline)) {
            const int dbits = min(8, shift);
            shift -= dbits;
            const int hi = shift + dbits;
            const uint32_t dmask = (1u << dbits) - 1u;
            int* hw = hist + wave * 256;
#pragma unroll
            for (int i = 0; i < 4; ++i) hw[lane + 64 * i] = 0;  // nobody reads it now
            if (live) {
#pragma unroll
                for (int r = 0; r < KPT; ++r) {
                    const uint32_t kr = key[r] - kmin;
                    if (key[r] != 0u && (hi >= 32 || (kr >> hi) == (prefix >> hi)))
                        atomicAdd(&hw[(kr >> shift) & dmask], 1);
                }
            }
            if (tid == 0) misc[0] = 0;  // the alive list below starts empty
            __syncthreads();
            if (tid < 256) {
                int t = 0;
#pragma unroll
                for (int w = 0; w < kDecWaves; ++w) t += hist[w * 256 + tid];
                hsum[tid] = t;
            }
            __syncthreads();
            int digit, above;
            find_digit256(hsum, krem, lane, digit, above);
            prefix |= static_cast<uint32_t>(digit) << shift;
            krem -= above;
            return digit;
        };
        // The first pass runs over every key.  The keys still alive after it
        // (those in the threshold's digit, usually a small fraction) are
        // gathered into LDS and wave 0 finishes the remaining passes on that
        // list alone, with no workgroup barriers; a list too long for the
        // buffer keeps to whole-workgroup passes.
        if (shift > 0) {
            const int d1 = block_pass();
            const int n_alive = hsum[d1];
            if (shift > 0 && n_alive <= kSelAliveCap) {
                if (live) {
                    // list slots: a lane mask of the alive keys, a wave prefix
                    // of the lane counts and one LDS atomic per wave
                    uint32_t am = 0u;
#pragma unroll
                    for (int r = 0; r < KPT; ++r) {
                        const uint32_t kr = key[r] - kmin;
                        am |= (key[r] != 0u && (kr >> shift) == (prefix >> shift)) ? (1u << r) : 0u;
                    }
                    const int cnt_l = __builtin_popcount(am);
                    const int incl_l = wave_incl_scan(cnt_l);
                    int wbase = 0;
                    if (lane == 63) wbase = atomicAdd(&misc[0], incl_l);
                    int at = __builtin_amdgcn_readlane(wbase, 63) + incl_l - cnt_l;
#pragma unroll
                    for (int r = 0; r < KPT; ++r)
                        if (am & (1u << r)) alive[at++] = key[r] - kmin;
                }
                __syncthreads();
                if (wave == 0) {
                    while (shift > 0) {
                        const int dbits = min(8, shift);
                        shift -= dbits;
                        const int hi = shift + dbits;
                        int* hw = hist;
#pragma unroll
                        for (int i = 0; i < 4; ++i) hw[lane + 64 * i] = 0;
                        for (int i = lane; i < n_alive; i += kWave) {
                            const uint32_t kr = alive[i];
                            if ((kr >> hi) == (prefix >> hi))
                                atomicAdd(&hw[(kr >> shift) & ((1u << dbits) - 1u)], 1);
                        }
                        int digit, above;
                        find_digit256(hw, krem, lane, digit, above);
                        prefix |= static_cast<uint32_t>(digit) << shift;
                        krem -= above;
                    }
                    if (lane == 0) {
                        misc[1] = static_cast<int>(prefix);
                        misc[2] = krem;
                    }
                }
                __syncthreads();
                prefix = static_cast<uint32_t>(misc[1]);
                krem = misc[2];
                shift = 0;
            }
            while (shift > 0) block_pass();
        }
        tau = kmin + prefix;
        need_eq = krem;
    }
    // Positions in the ascending kept list, which runs row by row (row r
    // holds blocks r * kDecThreads .. + kDecThreads - 1) and, in a row, wave
    // by wave and lane by lane.  Per (row, wave): the counts of keys > tau
    // and == tau, packed, from ballots; every wave then forms the exclusive
    // prefix of those counts in list order, and a key's place adds its
    // lane's rank in the row's ballots.
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const uint64_t mg = __ballot(key[r] > tau);
        const uint64_t me = __ballot(key[r] == tau);
        if (lane == 0) rowcnt[r * kDecWaves + wave] = (__popcll(mg) << 16) | __popcll(me);
    }
    __syncthreads();
    // lane l holds entries l and l + 64 of the (row, wave) list (at most
    // 16 x 8 = 128 entries); pre0/pre1: their exclusive prefixes
    constexpr int NE = KPT * kDecWaves;
    const int e0 = (lane < NE) ? rowcnt[lane] : 0;
    const int e1 = (lane + 64 < NE) ? rowcnt[lane + 64] : 0;
    const int inc0 = wave_incl_scan(e0);
    const int tot0 = __builtin_amdgcn_readlane(inc0, 63);
    const int pre0 = inc0 - e0;
    const int pre1 = tot0 + wave_incl_scan(e1) - e1;
    // the ballots below are formed again rather than kept from the counting
    // loop (2 x KPT 64-bit masks would not fit in scalar registers)
#pragma unroll
    for (int r = 0; r < KPT; ++r) asm volatile("" : "+v"(key[r]));
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const int c = tid + r * kDecThreads;
        const bool g = key[r] > tau, e = key[r] == tau;
        const uint64_t mg = __ballot(g);
        const uint64_t me = __ballot(e);
        const int idx_e = r * kDecWaves + wave;  // wave-uniform
        const int lsrc = __builtin_amdgcn_readfirstlane(idx_e & 63);
        const int pre = (idx_e < 64) ? __builtin_amdgcn_readlane(pre0, lsrc)
                                     : __builtin_amdgcn_readlane(pre1, lsrc);
        if (g || e) {
            const int below_g = (pre >> 16) + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                static_cast<uint32_t>(mg >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mg), 0u)));
            const int below_e = (pre & 0xffff) + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                static_cast<uint32_t>(me >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(me), 0u)));
            if (g || below_e < need_eq) {
                const int pos = below_g + min(below_e, need_eq);
                kept[pos] = c;
                kept_page[pos] = pg[r];
            }
        }
    }
    // the local blocks follow the K picked candidates (their ids are the largest)
    if (tid < nl) {
        kept[K + tid] = NC + tid;
        kept_page[K + tid] = lpg;
    }
    __syncthreads();
    return n;
}

// The bf16 kernel: one workgroup of kDecThreads (8 waves) per (sequence, KV
// head, split), one workgroup per CU.  The split's kept tiles are cut into
// units of unit_tiles tiles (about one per wave); waves claim units one at a
// time from an LDS counter, so a wave that the hardware serves faster takes
// any spare unit.  Each unit leaves its own partial (running max, sum,
// unnormalised O) in LDS, and the units are merged in unit order at the
// end, so the result does not depend on which wave took which unit.
//
// SELK > 0: the workgroup first selects its group's kept blocks from the
// score row (select_kept, SELK blocks per thread), with every block's page id
// requested in the same round trip as the scores, so the split's ids and
// page ids are in LDS without a further trip.  The first split of each group
// also writes the kept list to idx_out/cnt_out.
template <int D, int BLK, bool GATE, int SELK>
__global__ __launch_bounds__(kDecThreads)
__attribute__((amdgpu_waves_per_eu(BSA_DECODE_WAVES_PER_EU, 8))) void decode_bf16_kernel(
    DecodeParams p) {
    constexpr bool SEL = SELK > 0;
    constexpr int NK = SEL ? SELK : 1;
    static_assert(!(GATE && SEL), "the in-workgroup selection writes no bias");
    constexpr int KS = D / 32;   // k-steps of the QK product
    constexpr int NT = D / 16;   // column tiles of the PV product
    constexpr int TPB = BLK / 32;
    extern __shared__ float smem[];
    const int MU = p.max_units;
    const int G = p.c.G;
    float* um = smem;                    // [MU][16] running max per unit and head column
    float* ul = um + MU * 16;            // [MU][16] running sum
    float* uo = ul + MU * 16;            // [MU][G][D] unnormalised O
    int* s_blk = reinterpret_cast<int*>(uo + MU * G * D);  // [max_blocks_per_wg]
    int* s_page = s_blk + p.max_blocks_per_wg;              // [max_blocks_per_wg]
    float* s_bias = reinterpret_cast<float*>(s_page + p.max_blocks_per_wg);  // GATE only
    __shared__ int s_next;

    const CacheArgs& c = p.c;
    const DecodeArgs& a = p.a;
    const int split = blockIdx.x;
    const int grp = blockIdx.y;
    const int s = grp / c.Hkv;
    const int kvh = grp - s * c.Hkv;
    const int S = a.splits;
    // The split ranges cover n_max blocks (known before any load), so the
    // block ids, the kept count, the length and the queries are requested
    // together.
    const int U = a.n_max * TPB;
    const int u0 = static_cast<int>(static_cast<int64_t>(U) * split / S);
    const int u1 = static_cast<int>(static_cast<int64_t>(U) * (split + 1) / S);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int col = lane & 15;

    // SEL: the length, this thread's NK scores and their blocks' page ids
    // (one coalesced wave load per row), requested before the queries; slots
    // past the row read its first entry
    int T_v = 0;
    float sc[NK];
    int pg[NK];
    const int32_t* prow = c.page_table + static_cast<int64_t>(s) * c.max_blocks;
    if constexpr (SEL) {
        T_v = load_int_vgpr(c.seq_lens + s);
        const float* srow = a.scores + static_cast<int64_t>(grp) * a.score_stride;
#pragma unroll
        for (int r = 0; r < NK; ++r) {
            const int cb = threadIdx.x + r * kDecThreads;
            sc[r] = srow[cb < a.score_stride ? cb : 0];
            pg[r] = prow[cb < c.max_blocks ? cb : 0];
        }
    }

    // B operand of S^T = K Q^T: lane (g, col) holds q[head col][32ks + 8g .. +8]
    bf16x8 qb[KS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                             (static_cast<int64_t>(s) * c.Hq + kvh * G + col) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (col < G) w = ldg16(qp + ks * 32 + g * 8);
            qb[ks] = __builtin_bit_cast(bf16x8, w);
        }
    }

    // block ids and page ids of this split, resolved once (two dependent
    // round trips for the whole workgroup instead of two per tile)
    const int pb0 = u0 / TPB;
    // s_blk / s_page hold the split's entries from pb0 on, or (SEL) the
    // whole kept list
    const int id0 = SEL ? 0 : pb0;
    int cnt, T;
    if constexpr (SEL) {
        T = __builtin_amdgcn_readfirstlane(T_v);
        // the local blocks' page ids (thread j: local block j), requested now
        // and first needed at the end of the selection
        const int NBs = (T + BLK - 1) / BLK;
        const int nls = min(a.n_local, NBs);
        const int lpg = (static_cast<int>(threadIdx.x) < nls) ? prow[NBs - nls + threadIdx.x] : 0;
        // the selection's scratch lies in the unit partials' LDS, written
        // only after it
        cnt = select_kept<NK>(a, T, BLK, sc, pg, lpg, reinterpret_cast<int*>(smem), s_blk, s_page);
        if (split == 0) {
            int32_t* orow = a.idx_out + static_cast<int64_t>(grp) * a.n_max;
            for (int i = threadIdx.x; i < a.n_max; i += kDecThreads)
                orow[i] = (i < cnt) ? s_blk[i] : -1;
            if (threadIdx.x == 0) a.cnt_out[grp] = cnt;
        }
        if (threadIdx.x == 0) s_next = 0;
        __syncthreads();
    } else {
        const int32_t* idxrow = a.idx + static_cast<int64_t>(grp) * a.n_max;
        const int32_t* ptrow = prow;
        const int nblk = (u1 > u0) ? (u1 - 1) / TPB - pb0 + 1 : 0;
        cnt = a.cnt[grp];
        T = c.seq_lens[s];
        for (int i = threadIdx.x; i < nblk; i += kDecThreads) {
            const int blk = idxrow[pb0 + i];
            const bool kept = pb0 + i < cnt;
            s_blk[i] = kept ? blk : 0;
            s_page[i] = kept ? ptrow[blk] : 0;
            if (GATE) s_bias[i] = kept ? a.bias[static_cast<int64_t>(grp) * a.n_max + pb0 + i] * kLog2e : 0.f;
        }
        if (threadIdx.x == 0) s_next = 0;
        __syncthreads();
    }

    // the kept tiles of the split, in units
    const int uend = min(u1, cnt * TPB);
    const int UT = p.unit_tiles;
    const int n_units = (uend > u0) ? (uend - u0 + UT - 1) / UT : 0;

    floatx4 oacc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) oacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const uint16_t* kpool = static_cast<const uint16_t*>(c.k_pool);
    const uint16_t* vpool = static_cast<const uint16_t*>(c.v_pool);
    const float sl2 = a.scale_log2;
    const uint16_t* kl = kpool + lane * 8;
    const uint16_t* vl = vpool + lane * 8;
    u32x4 kr[2 * KS], vr[NT];
    auto grab = [&]() __attribute__((always_inline)) {
        int v = 0;
        if (lane == 0) v = atomicAdd(&s_next, 1);
        return __builtin_amdgcn_readfirstlane(v);
    };
    // tile u -> (element offset of its 32-token run, tokens valid in it,
    // base-2 logit bias of its block)
    auto resolve = [&](int u, int64_t& off, int& nvalid, float& b2) __attribute__((always_inline)) {
        const int pi = u / TPB;
        const int r = u - pi * TPB;
        const int blk = __builtin_amdgcn_readfirstlane(s_blk[pi - id0]);
        const int page = __builtin_amdgcn_readfirstlane(s_page[pi - id0]);
        b2 = GATE ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_bias[pi - id0])))
                  : 0.f;
        nvalid = T - (blk * BLK + 32 * r);
        off = (static_cast<int64_t>(page) * c.Hkv + kvh) * static_cast<int64_t>(BLK * D) + 32 * r * D;
    };
    auto load_k = [&](int64_t off) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 2 * KS; ++k) kr[k] = ldg16_stream(kl + off + k * 512);
    };
    auto load_v = [&](int64_t off) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NT; ++n) vr[n] = ldg16_stream(vl + off + n * 512);
    };
    // one tile: QK, online softmax, PV; NEXT: also issue the next tile's loads
    auto step = [&](const int nvalid, const float b2, const bool next, const int64_t off_nxt)
                    __attribute__((always_inline)) {
        floatx4 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kr[mt * KS + ks]), qb[ks], sacc[mt], 0, 0, 0);
        }
        if (next) load_k(off_nxt);
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int tok = (k < 4) ? (4 * g + k) : (16 + 4 * g + k - 4);
            const float z = GATE ? fmaf(sacc[k >> 2][k & 3], sl2, b2) : sacc[k >> 2][k & 3] * sl2;
            x[k] = (tok < nvalid) ? z : -INFINITY;
        }
        float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                           fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        if (__ballot(tmax > m_run) != 0) {  // some head's running max grows
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
            // O rows are heads 4g+e; their alpha lives in lane 4g+e
            float al[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * g + e, 64);
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) oacc[n][e] *= al[e];
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;  // nothing seen yet
        float pr[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) pr[k] = __builtin_amdgcn_exp2f(x[k] - m_use);
        l_run += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
        // P = hi + lo, both bf16 (round to nearest even in hardware)
        bf16x8 ph, pl;
#pragma unroll
        for (int k = 0; k < 8; ++k) ph[k] = static_cast<__bf16>(pr[k]);
#pragma unroll
        for (int k = 0; k < 8; ++k) pl[k] = static_cast<__bf16>(pr[k] - static_cast<float>(ph[k]));
        // token slots past the end may hold anything (even NaN): zero them
        uint32_t keep[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t0 = (2 * k < 4) ? (4 * g + 2 * k) : (16 + 4 * g + 2 * k - 4);
            keep[k] = (t0 < nvalid ? 0x0000ffffu : 0u) | (t0 + 1 < nvalid ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            u32x4 vm = vr[n];
#pragma unroll
            for (int k = 0; k < 4; ++k) vm[k] &= keep[k];
            const bf16x8 vb = __builtin_bit_cast(bf16x8, vm);
            oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, oacc[n], 0, 0, 0);
            oacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, oacc[n], 0, 0, 0);
        }
        if (next) load_v(off_nxt);
    };
    // the finished unit's partial to LDS, and a fresh state
    auto flush = [&](int unit) __attribute__((always_inline)) {
        float l_tot = l_run + __shfl_xor(l_run, 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        if (g == 0) {
            um[unit * 16 + col] = m_run;
            ul[unit * 16 + col] = l_tot;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int h = 4 * g + e;
            if (h < G) {
#pragma unroll
                for (int n = 0; n < NT; ++n) uo[(unit * G + h) * D + n * 16 + col] = oacc[n][e];
            }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) oacc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
    };

    // Tile loop, software-pipelined across unit boundaries: the next tile's
    // K loads are issued as soon as QK has consumed the current K registers
    // and its V loads as soon as PV has consumed V; the next unit is claimed
    // while the last tile of the current one is being computed.  Every load
    // in the steady-state body is unconditional (the last tile is a separate
    // call without next-tile loads), so the compiler's wait counters only
    // wait for the registers each step needs.  Tile addressing is
    // wave-uniform.
    int unit = grab();
    if (unit < n_units) {
        int t = u0 + unit * UT;
        int t_end = min(t + UT, uend);
        int64_t off = 0;
        int nv = 0;
        float b2 = 0.f;
        resolve(t, off, nv, b2);
        load_k(off);
        load_v(off);
        while (true) {
            int nt = t + 1, nunit = unit, nend = t_end;
            if (nt >= t_end) {  // last tile of the unit: claim the next one
                nunit = grab();
                nt = u0 + nunit * UT;
                nend = min(nt + UT, uend);
            }
            if (nunit >= n_units) break;
            int64_t off_nxt = 0;
            int nv_nxt = 0;
            float b2_nxt = 0.f;
            resolve(nt, off_nxt, nv_nxt, b2_nxt);
            step(nv, b2, true, off_nxt);
            if (nunit != unit) flush(unit);
            unit = nunit;
            t = nt;
            t_end = nend;
            nv = nv_nxt;
            b2 = b2_nxt;
        }
        step(nv, b2, false, 0);
        flush(unit);
    }
    __syncthreads();

    // merge of the units, in unit order, into one partial per head: the
    // per-head maximum and every unit's weight 2^(m_u - M) are formed once
    // (the weights overwrite um), then each output channel sums over the
    // units with several LDS reads in flight
    __shared__ float s_M[16];
    if (threadIdx.x < 16) {
        float M = -INFINITY;
#pragma unroll 8
        for (int u = 0; u < n_units; ++u) M = fmaxf(M, um[u * 16 + threadIdx.x]);
        s_M[threadIdx.x] = M;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n_units * 16; i += kDecThreads) {
        const float M = s_M[i & 15];
        um[i] = (M == -INFINITY) ? 0.f : exp2f(um[i] - M);
    }
    __syncthreads();
    const int64_t head_row0 = static_cast<int64_t>(s) * c.Hq + kvh * G;
    for (int k = threadIdx.x; k < G * D; k += kDecThreads) {
        const int h = k / D;
        const int ch = k - h * D;
        const float M = s_M[h];
        const int64_t row = head_row0 + h;
        float* op = a.o_part + (row * S + split) * D;
        if (M == -INFINITY) {
            op[ch] = 0.f;
            if (ch == 0) a.lse_part[row * S + split] = -INFINITY;
            continue;
        }
        float L = 0.f, acc = 0.f;
#pragma unroll 8
        for (int u = 0; u < n_units; ++u) {
            const float sc = um[u * 16 + h];
            L += ul[u * 16 + h] * sc;
            acc += uo[(u * G + h) * D + ch] * sc;
        }
        op[ch] = acc / L;
        if (ch == 0) a.lse_part[row * S + split] = M + log2f(L);
    }
}

// fp32 caches: same split, plain arithmetic.  Lane t < 32 owns token t of a
// tile for the logits; every lane owns channels lane, lane+64 for O.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_f32_kernel(DecodeParams p) {
    constexpr int CPL = D / 64;  // output channels per lane
    extern __shared__ float smem[];
    float* sm = smem;
    float* sl = sm + kWaves * 16;
    float* so = sl + kWaves * 16;  // [kWaves][G][D]
    float* qs = so + kWaves * p.c.G * D;  // [G][D]

    const CacheArgs& c = p.c;
    const DecodeArgs& a = p.a;
    const int split = blockIdx.x;
    const int grp = blockIdx.y;
    const int s = grp / c.Hkv;
    const int kvh = grp - s * c.Hkv;
    const int G = c.G;
    const int T = c.seq_lens[s];
    const int BLK = c.block;
    const int TPB = BLK / 32;
    const int U = a.cnt[grp] * TPB;
    const int S = a.splits;
    const int u0 = static_cast<int>(static_cast<int64_t>(U) * split / S);
    const int u1 = static_cast<int>(static_cast<int64_t>(U) * (split + 1) / S);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;

    const float* qg = static_cast<const float*>(a.q) + (static_cast<int64_t>(s) * c.Hq + kvh * G) * D;
    for (int k = threadIdx.x; k < G * D; k += kThreads) qs[k] = qg[k];
    __syncthreads();

    float m[16], l[16], o[16][CPL];
#pragma unroll
    for (int h = 0; h < 16; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) o[h][k] = 0.f;
    }
    const float* kpool = static_cast<const float*>(c.k_pool);
    const float* vpool = static_cast<const float*>(c.v_pool);
    const int32_t* idxrow = a.idx + static_cast<int64_t>(grp) * a.n_max;
    const int32_t* ptrow = c.page_table + static_cast<int64_t>(s) * c.max_blocks;

    for (int u = u0 + wave; u < u1; u += kWaves) {
        const int pi = u / TPB;
        const int r = u - pi * TPB;
        const int blk = idxrow[pi];
        const int tok0 = blk * BLK + 32 * r;
        const int nvalid = min(32, T - tok0);
        if (nvalid <= 0) continue;
        const int64_t page = ptrow[blk];
        const float b2 = a.bias ? a.bias[static_cast<int64_t>(grp) * a.n_max + pi] * kLog2e : 0.f;
        const float* kt = kpool + (page * c.Hkv + kvh) * static_cast<int64_t>(BLK * D) + 32 * r * D;
        const float* vt = vpool + (page * c.Hkv + kvh) * static_cast<int64_t>(BLK * D) + 32 * r * D;
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            if (h >= G) continue;  // (not break: keeps the loop unrollable)
            float z = -INFINITY;
            if (lane < nvalid) {
                float acc = 0.f;
                for (int i = 0; i < D; ++i) acc += qs[h * D + i] * kt[lane * D + i];
                z = fmaf(acc, a.scale_log2, b2);
            }
            const float mt = wave_max(z);
            const float m_new = fmaxf(m[h], mt);
            const float alpha = exp2f(m[h] - m_new);
            const float pz = (lane < nvalid) ? exp2f(z - m_new) : 0.f;
            l[h] = l[h] * alpha + wave_sum(pz);
            m[h] = m_new;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int ch = lane + 64 * k;
                float acc = o[h][k] * alpha;
                for (int t = 0; t < nvalid; ++t) acc += __shfl(pz, t, 64) * vt[t * D + ch];
                o[h][k] = acc;
            }
        }
    }
    if (lane < 16) {
        float mv = -INFINITY, lv = 0.f;
#pragma unroll
        for (int h = 0; h < 16; ++h)
            if (h == lane) {
                mv = m[h];
                lv = l[h];
            }
        sm[wave * 16 + lane] = mv;
        sl[wave * 16 + lane] = lv;
    }
#pragma unroll
    for (int h = 0; h < 16; ++h) {
        if (h >= G) continue;
#pragma unroll
        for (int k = 0; k < CPL; ++k) so[(wave * G + h) * D + lane + 64 * k] = o[h][k];
    }
    __syncthreads();
    merge_waves_and_store(sm, sl, so, G, D, a.o_part, a.lse_part,
                          static_cast<int64_t>(s) * c.Hq + kvh * G, S, split);
}

// Merge of the partial (o, base-2 lse) pairs of each row, in a fixed order.
// Row `row` merges its first S splits, or, when seq_lens is given, only the
// splits that cover [0, seq_lens[row / rows_per_seq]) at tokens_per_split
// tokens each (the others were never written).  Grid: rows x (d / 64); the
// 256 threads take 64 channels x 4 split lanes.  Every partial o a thread
// needs is loaded in the same round trip as the lse values (kCombBatch per
// lane at a time); the split weights 2^(lse_k - M) are formed once M is
// known, and the 4 lane sums (o and weights) are added in fixed order.
constexpr int kCombThreads = 256;
constexpr int kCombCh = 64;                         // channels per workgroup
constexpr int kCombLanes = kCombThreads / kCombCh;  // split lanes per channel
constexpr int kCombBatch = 16;                      // o loads in flight per lane

template <int DT>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    int d, int S, const float* __restrict__ o_part, const float* __restrict__ lse_part, void* o,
    float* lse, const int32_t* seq_lens, int rows_per_seq, int tokens_per_split) {
    extern __shared__ float lse_s[];  // [S] partial lse of the row
    __shared__ float red[kCombThreads / kWave];
    __shared__ float part_sum[kCombLanes][kCombCh];
    __shared__ float part_w[kCombLanes];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    int Sv = S;
    if (seq_lens) {
        const int T = seq_lens[row / rows_per_seq];
        Sv = min(S, (T + tokens_per_split - 1) / tokens_per_split);
    }
    const int cl = tid % kCombCh;
    const int lane_k = tid / kCombCh;
    const int ch = blockIdx.y * kCombCh + cl;
    const float* op = o_part + row * S * d + ch;
    const float* lp = lse_part + row * S;
    // first batch of partial o values, in flight together with the lse loads
    float ov[kCombBatch];
#pragma unroll
    for (int u = 0; u < kCombBatch; ++u) {
        const int k = lane_k + kCombLanes * u;
        ov[u] = (k < Sv) ? op[static_cast<int64_t>(k) * d] : 0.f;
    }
    float m = -INFINITY;
    for (int k = tid; k < Sv; k += kCombThreads) {
        const float v = lp[k];
        lse_s[k] = v;
        m = fmaxf(m, v);
    }
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kCombThreads / kWave; ++w) M = fmaxf(M, red[w]);
    float acc = 0.f, wsum = 0.f;
    if (M != -INFINITY) {
        for (int k0 = 0; k0 < Sv; k0 += kCombLanes * kCombBatch) {
            if (k0 > 0) {  // more splits than one batch covers
#pragma unroll
                for (int u = 0; u < kCombBatch; ++u) {
                    const int k = k0 + lane_k + kCombLanes * u;
                    ov[u] = (k < Sv) ? op[static_cast<int64_t>(k) * d] : 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < kCombBatch; ++u) {
                const int k = k0 + lane_k + kCombLanes * u;
                if (k < Sv) {
                    const float wk = exp2f(lse_s[k] - M);
                    acc += wk * ov[u];
                    wsum += wk;
                }
            }
        }
    }
    part_sum[lane_k][cl] = acc;
    if (cl == 0) part_w[lane_k] = wsum;
    __syncthreads();
    if (lane_k == 0) {
        float tot = 0.f, L = 0.f;
#pragma unroll
        for (int p2 = 0; p2 < kCombLanes; ++p2) {
            tot += part_sum[p2][cl];
            L += part_w[p2];
        }
        const bool empty = (M == -INFINITY);
        Elem<DT>::store(static_cast<typename Elem<DT>::T*>(o), row * d + ch, empty ? 0.f : tot / L);
        if (ch == 0) lse[row] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
    }
}

template <int D, int BLK>
hipError_t launch_bf16(DecodeParams p, hipStream_t stream) {
    const bool gate = p.a.bias != nullptr;
    const bool sel = p.a.scores != nullptr;
    if (gate && sel) return hipErrorInvalidValue;
    // SEL: candidate blocks of the longest possible row
    const int cand = p.c.max_blocks - min(p.a.n_local, p.c.max_blocks);
    // SEL: the whole kept list (at most n_max entries) stays in LDS
    if (sel) p.max_blocks_per_wg = max(p.max_blocks_per_wg, p.a.n_max);
    // units: about one per wave, of 2 to BSA_DECODE_MAX_UNIT tiles (fewer,
    // longer units mean fewer partials to flush and merge, and waves that
    // the hardware serves faster still take the spare units); longer units
    // only when the split has more units than the LDS holds partial slots
    const int tiles = (p.a.n_max * (BLK / 32) + p.a.splits - 1) / p.a.splits;
    const int unit_bytes = static_cast<int>(sizeof(float)) * (32 + p.c.G * D);
    // the split's block ids, page ids (and biases) take what they need; the
    // unit partials get the configured budget or what remains of the CU's LDS
    const int id_bytes = (gate ? 3 : 2) * static_cast<int>(sizeof(int)) * p.max_blocks_per_wg;
    const int budget = min(BSA_DECODE_UNIT_LDS, kLdsBytes - 256 - id_bytes);
    const int slots = budget / unit_bytes;
    int ut = (tiles + BSA_DECODE_UNITS_PER_SPLIT - 1) / BSA_DECODE_UNITS_PER_SPLIT;
    ut = min(max(ut, 2), BSA_DECODE_MAX_UNIT);
    ut = max(ut, (tiles + slots - 1) / slots);
    p.unit_tiles = ut;
    p.max_units = (tiles + ut - 1) / ut;
    // SEL: the selection's scratch lies in the unit partials' slots
    if (sel) {
        const int sel_bytes = static_cast<int>(sizeof(int)) * kSelScratchInts;
        p.max_units = max(p.max_units, (sel_bytes + unit_bytes - 1) / unit_bytes);
    }
    const size_t shm = static_cast<size_t>(unit_bytes) * p.max_units + id_bytes;
    dim3 grid(p.a.splits, p.c.B * p.c.Hkv);
    if (gate)
        hipLaunchKernelGGL((decode_bf16_kernel<D, BLK, true, 0>), grid, dim3(kDecThreads), shm,
                           stream, p);
    else if (!sel)
        hipLaunchKernelGGL((decode_bf16_kernel<D, BLK, false, 0>), grid, dim3(kDecThreads), shm,
                           stream, p);
    else if (cand <= 2 * kDecThreads)
        hipLaunchKernelGGL((decode_bf16_kernel<D, BLK, false, 2>), grid, dim3(kDecThreads), shm,
                           stream, p);
    else if (cand <= 4 * kDecThreads)
        hipLaunchKernelGGL((decode_bf16_kernel<D, BLK, false, 4>), grid, dim3(kDecThreads), shm,
                           stream, p);
    else if (cand <= 8 * kDecThreads)
        hipLaunchKernelGGL((decode_bf16_kernel<D, BLK, false, 8>), grid, dim3(kDecThreads), shm,
                           stream, p);
    else
        hipLaunchKernelGGL((decode_bf16_kernel<D, BLK, false, 16>), grid, dim3(kDecThreads), shm,
                           stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(const DecodeParams& p, hipStream_t stream) {
    switch (p.c.block) {
        case 32: return launch_bf16<D, 32>(p, stream);
        case 64: return launch_bf16<D, 64>(p, stream);
        case 128: return launch_bf16<D, 128>(p, stream);
        case 256: return launch_bf16<D, 256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_f32(const DecodeParams& p, hipStream_t stream) {
    const size_t shm = sizeof(float) * (2 * kWaves * 16 + kWaves * p.c.G * D + p.c.G * D);
    dim3 grid(p.a.splits, p.c.B * p.c.Hkv);
    hipLaunchKernelGGL((decode_f32_kernel<D>), grid, dim3(kThreads), shm, stream, p);
    return hipGetLastError();
}

}  // namespace

int decode_splits(const CacheArgs& c, int n_max) {
    // about BSA_DECODE_TARGET_WGS workgroups over the chip (one per CU for
    // the bf16 kernel), at least 4 tiles in every split, and at most
    // kMaxSplitBlocks blocks in a split (their ids are staged in LDS).
    const int groups = c.B * c.Hkv;
    const int tiles = n_max * (c.block / 32);
    int S = (BSA_DECODE_TARGET_WGS + groups - 1) / groups;
    const int cap = (tiles + 3) / 4;
    if (S > cap) S = cap;
    const int least = (n_max + kMaxSplitBlocks - 1) / kMaxSplitBlocks;
    if (S < least) S = least;
    if (S < 1) S = 1;
    return S;
}

bool decode_selects(const CacheArgs& c, int n_local, int n_max) {
    const int cand = c.max_blocks - min(n_local, c.max_blocks);
    return c.dtype == kBF16 && cand <= kDecodeSelectSlots && n_max <= kDecodeSelectMaxKept;
}

hipError_t launch_combine_ragged(int dtype, int d, int rows, int splits, const float* o_part,
                                 const float* lse_part, void* o, float* lse,
                                 const int32_t* seq_lens, int rows_per_seq,
                                 int tokens_per_split, hipStream_t stream) {
    const size_t shm = sizeof(float) * static_cast<size_t>(splits);
    const dim3 grid(rows, d / kCombCh);
    if (dtype == kBF16)
        hipLaunchKernelGGL((combine_kernel<kBF16>), grid, dim3(kCombThreads), shm, stream, d,
                           splits, o_part, lse_part, o, lse, seq_lens, rows_per_seq,
                           tokens_per_split);
    else
        hipLaunchKernelGGL((combine_kernel<kF32>), grid, dim3(kCombThreads), shm, stream, d,
                           splits, o_part, lse_part, o, lse, seq_lens, rows_per_seq,
                           tokens_per_split);
    return hipGetLastError();
}

hipError_t launch_combine(int dtype, int d, int rows, int splits, const float* o_part,
                          const float* lse_part, void* o, float* lse, hipStream_t stream) {
    return launch_combine_ragged(dtype, d, rows, splits, o_part, lse_part, o, lse, nullptr, 1, 1,
                                 stream);
}

hipError_t launch_decode(const CacheArgs& c, const DecodeArgs& a, hipStream_t stream) {
    // a split covers at most ceil(n_max*TPB / S) tiles, which touch at most
    // that many / TPB + 1 blocks (+1 more when it starts inside a block)
    const int tpb = c.block / 32;
    const int tiles = (a.n_max * tpb + a.splits - 1) / a.splits;
    DecodeParams p{c, a, tiles / tpb + 2, 0, 0};
    if (a.scores && !decode_selects(c, a.n_local, a.n_max)) return hipErrorInvalidValue;
    hipError_t err;
    if (c.dtype == kBF16)
        err = c.d == 64 ? launch_bf16_d<64>(p, stream) : launch_bf16_d<128>(p, stream);
    else
        err = c.d == 64 ? launch_f32<64>(p, stream) : launch_f32<128>(p, stream);
    if (err != hipSuccess) return err;
    return launch_combine(c.dtype, c.d, c.B * c.Hq, a.splits, a.o_part, a.lse_part, a.o, a.lse,
                          stream);
}

}  // namespace bsa
