// rectify.hip -- dense causal attention of the f re-encoded queries of every
// sequence over its whole cache (ReSA rectification).
//
// "Rectified Sparse Attention for Efficient Long-Sequence Generation",
// Summary: after every f generated tokens those tokens are re-encoded in one
// parallel dense pass that overwrites their KV entries and block keys; Key
// points: f in {16, 32, 64, 128}.  The overwrite and the descriptor refresh
// run first (kv_write.hip, overwrite mode); this file computes, for query i of
// head h (position T-f+i), softmax attention over tokens 0..T-f+i.
//
// bf16 path: the only dense contraction of the method.  Rows = the G*f
// queries of a GQA group.  The tiles of all groups are dealt out in equal
// contiguous shares to a fixed number of workgroups (stream-K), so ragged
// lengths cost no load imbalance; each run of a share inside one group yields
// one partial (o, base-2 lse) per row, merged afterwards in list order.  K/V
// tiles (32 tokens, 16 KiB at d = 128) stream through an LDS ring fed by
// direct global->LDS copies.  Two shapes:
//  - up to 128 rows (row groups of 64 with 4 waves or 128 with 8 waves, two
//    workgroups per CU): one 16-row tile per wave on v_mfma_f32_16x16x32_bf16,
//    a 4-stage ring two tiles ahead, one workgroup barrier per tile;
//  - more rows: row groups of 256 on v_mfma_f32_32x32x16_bf16, one workgroup
//    of 8 waves per CU running a ping-pong schedule (below).
// Both take the online softmax with a lazily moved reference max and P in
// bf16.
//
// fp32 path: fixed token chunks per workgroup, plain VALU arithmetic, the
// chunk merge of decode.hip.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
#ifndef BSA_RECTIFY_CHUNK_TILES
#define BSA_RECTIFY_CHUNK_TILES 64
#endif
#ifndef BSA_RECTIFY_STAGES
#define BSA_RECTIFY_STAGES 4
#endif
#ifndef BSA_RECTIFY_WAVES_PER_EU
#define BSA_RECTIFY_WAVES_PER_EU 4
#endif
constexpr float kRebase = 8.f;  // log2 headroom before the running max is moved
constexpr int kChunkTiles = BSA_RECTIFY_CHUNK_TILES;  // 32-token tiles per workgroup
constexpr int kStages = BSA_RECTIFY_STAGES;           // tiles in flight per workgroup (LDS ring)

struct RectifyParams {
    CacheArgs c;
    RectifyArgs a;
};

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Direct copy of 16 bytes per lane from global memory into LDS: lane L's
// bytes land at lds + 16 L (lds is wave-uniform; it goes into M0).  Written
// in asm so that the compiler does not treat it as an LDS write it must
// drain before every LDS read; the kernels order it themselves with explicit
// vector-memory waits and barriers.  The instruction has no register output.
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds) {
    // the low 32 bits of a generic LDS address are the LDS offset
    const uint32_t m0 =
        __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
    // (an M0 write needs one wait state before an LDS-DMA load reads it)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---------------------------------------------------------------------------
// Work split of the bf16 path (stream-K style).  The attention of one call is
// a set of groups (sequence, KV head, row group) in that order, group g
// holding the ceil(T/32) tiles of its sequence; the groups' tiles, laid end
// to end, form one list of N tiles.  Workgroup w of W takes the tiles
// [w N / W, (w+1) N / W), whatever groups they belong to, so every workgroup
// gets the same work however ragged the lengths are.  Each maximal run of a
// workgroup's tiles inside one group (a "piece") yields one partial (o, lse)
// per row, stored in slot g + w: along the list, every new piece moves to
// the next group, the next workgroup or both, so g + w grows strictly and
// slots never collide; there are fewer than (groups + W).
// ---------------------------------------------------------------------------
constexpr int kStreamWGs = 512;       // two workgroups per CU on a 256-CU part
constexpr int kMinTilesPerWG = 16;    // fewer workgroups for small calls
constexpr int kMaxTilesPerWG = 256;   // bounds the per-piece page list

__device__ __forceinline__ int ntiles_of(int T) { return (T + 31) / 32; }

// Workgroups used for N tiles when `launched` were launched (launched is at
// least ceil(N_max / kMaxTilesPerWG) for the cache's capacity N_max).
__device__ __forceinline__ int stream_wgs(int64_t N, int launched) {
    if (N <= 0) return 0;
    const int64_t lo = (N + kMaxTilesPerWG - 1) / kMaxTilesPerWG;
    const int64_t hi = min(static_cast<int64_t>(kStreamWGs), (N + kMinTilesPerWG - 1) / kMinTilesPerWG);
    return static_cast<int>(min(max(lo, hi), static_cast<int64_t>(launched)));
}
__device__ __forceinline__ int64_t wg_begin(int w, int64_t N, int W) {
    return static_cast<int64_t>(w) * N / W;
}
// the workgroup whose range holds tile x: the largest w with wg_begin(w) <= x
__device__ __forceinline__ int wg_owner(int64_t x, int64_t N, int W) {
    return static_cast<int>(((x + 1) * W + N - 1) / N - 1);
}

// Wave-wide scan over the sequences: total tiles N of all groups, and (when
// x >= 0) the sequence holding list position x with the list position of its
// first tile.  per_seq = groups per sequence (Hkv * row groups).  Every lane
// returns the same values.
struct SeqHit {
    int64_t N;
    int s;           // -1 if x is not in the list
    int64_t start;   // list position of sequence s's first tile
};
__device__ __forceinline__ SeqHit seq_scan(const int32_t* seq_lens, int B, int per_seq, int64_t x) {
    const int lane = threadIdx.x & 63;
    SeqHit h{0, -1, 0};
    for (int s0 = 0; s0 < B; s0 += kWave) {
        const int sq = s0 + lane;
        const long long per = (sq < B) ? static_cast<long long>(ntiles_of(seq_lens[sq])) * per_seq : 0;
        long long incl = per;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const long long y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        const int64_t excl = h.N + incl - per;
        const uint64_t m = __ballot(h.s < 0 && x >= excl && x < h.N + incl);
        if (m != 0) {
            const int L = __builtin_ctzll(m);
            h.s = s0 + L;
            h.start = __shfl(static_cast<long long>(excl), L, 64);
        }
        h.N += __shfl(incl, 63, 64);
    }
    return h;
}

// Eight waves of one row tile each fit two workgroups per CU (four waves per
// SIMD, at most 128 VGPRs); the other shapes run one.
template <int D, int BLK, int RTW, int NS, int NW>
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu((RTW == 1 && NW == 8) ? BSA_RECTIFY_WAVES_PER_EU : 1)))
void rectify_bf16_kernel(RectifyParams p) {
    constexpr int KS = D / 32;
    constexpr int NT = D / 16;
    constexpr int TILE_EL = 32 * D;             // elements of K (or V) per tile
    constexpr int CH = 2 * TILE_EL / 512;       // 1 KiB chunks per tile, K then V
    constexpr int CPW = CH / NW;                // chunks each wave copies
    constexpr int RWG = 16 * RTW * NW;          // rows per workgroup (row group)
    static_assert(CPW >= 1 && CPW * NW == CH, "chunks split evenly over the waves");
    // NS-stage ring of tiles in LDS, filled by direct global->LDS copies
    // (copy16_to_lds): each wave copies CPW KiB chunks per tile, NS-2 tiles
    // ahead of the one being computed, without using registers.
    __shared__ __attribute__((aligned(16))) uint16_t ring[NS][2 * TILE_EL];
    __shared__ int s_page[kMaxTilesPerWG * 32 / BLK + 2];
    __shared__ long long s_loc[4];

    const CacheArgs& c = p.c;
    const RectifyArgs& a = p.a;
    const int G = c.G;
    const int f = a.f;
    const int R = G * f;
    const int Z = (R + RWG - 1) / RWG;  // row groups per KV head
    const int per_seq = c.Hkv * Z;
    const int wave = threadIdx.x >> 6;
    const int w = blockIdx.x;

    if (wave == 0) {
        const SeqHit tot = seq_scan(c.seq_lens, c.B, per_seq, -1);
        const int W = stream_wgs(tot.N, gridDim.x);
        int64_t x0 = 0, x1 = 0;
        SeqHit h{tot.N, -1, 0};
        if (w < W) {
            x0 = wg_begin(w, tot.N, W);
            x1 = wg_begin(w + 1, tot.N, W);
            h = seq_scan(c.seq_lens, c.B, per_seq, x0);
        }
        if ((threadIdx.x & 63) == 0) {
            s_loc[0] = (w < W && x1 > x0) ? h.s : -1;
            s_loc[1] = x0 - h.start;  // position inside sequence s's groups
            s_loc[2] = x1 - x0;       // tiles of this workgroup
        }
    }
    __syncthreads();
    // (values read from LDS are wave-uniform; readfirstlane keeps them, and
    // all the piece bookkeeping derived from them, in scalar registers)
    int s = __builtin_amdgcn_readfirstlane(static_cast<int>(s_loc[0]));
    if (s < 0) return;  // no tiles for this workgroup (uniform)
    const int64_t pos0 = s_loc[1];
    const int64_t left0 = s_loc[2];
    int64_t left = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(left0 >> 32))) << 32) |
                   static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(left0)));
    int nts = ntiles_of(c.seq_lens[s]);
    int gl = __builtin_amdgcn_readfirstlane(static_cast<int>(pos0 / nts));  // group inside the sequence
    int off = __builtin_amdgcn_readfirstlane(static_cast<int>(pos0 - static_cast<int64_t>(gl) * nts));

    const uint16_t* kpool = static_cast<const uint16_t*>(c.k_pool);
    const uint16_t* vpool = static_cast<const uint16_t*>(c.v_pool);
    const float sl2 = a.scale_log2;
    const float rebase = kRebase / sl2;  // in raw score units

    while (true) {
        // ---- one piece: tiles [t0, t1) of group (s, kvh, zg) ----
        // The thread index is re-derived per piece behind an empty asm, so the
        // compiler cannot hoist thread-dependent values (epilogue addresses,
        // mask offsets) out of the piece loop, where they would stay live
        // through the tile loop and cost registers.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int g = lane >> 4;
        const int col = lane & 15;
        const int kvh = gl / Z;
        const int zg = gl - kvh * Z;
        const int T = c.seq_lens[s];
        const int t0 = off;
        const int nt = static_cast<int>(min(left, static_cast<int64_t>(nts - off)));
        const int t1 = t0 + nt;
        const int64_t slot = static_cast<int64_t>(s) * per_seq + gl + w;
        const int64_t row_base = (static_cast<int64_t>(s) * c.Hq + kvh * G) * f;  // row r = 0
        const int rt0 = (zg * NW + wave) * RTW;  // first 16-row tile of this wave

        __syncthreads();  // the previous piece is done with s_page and the ring
        // page ids of the piece's blocks (tiles are 32 tokens, blocks BLK tokens)
        const int32_t* ptrow = c.page_table + static_cast<int64_t>(s) * c.max_blocks;
        const int blk0 = (32 * t0) / BLK;
        const int nblk = (32 * (t1 - 1)) / BLK - blk0 + 1;
        for (int i = tid; i < nblk; i += NW * kWave) s_page[i] = ptrow[blk0 + i];

        // B operand of S^T = K Q^T for each row tile: row rt*16 + col
        bf16x8 qb[RTW][KS];
        int pos[RTW];  // query position of the row held in column `col`
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            const int r = (rt0 + rt) * 16 + col;
            pos[rt] = (r < R) ? T - f + (r % f) : T - 1;
            const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (row_base + r) * D;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (r < R) v = ldg16(qp + ks * 32 + g * 8);
                qb[rt][ks] = __builtin_bit_cast(bf16x8, v);
            }
        }
        floatx4 oacc[RTW][NT];
        float m_run[RTW], l_run[RTW], nms[RTW];  // raw running max, sum, -max*scale
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            m_run[rt] = -INFINITY;
            l_run[rt] = 0.f;
            nms[rt] = 0.f;
#pragma unroll
            for (int n = 0; n < NT; ++n) oacc[rt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        // retire the query and page-table loads before the copy ring starts, so
        // that no wait for them lands inside the loop (where it would also drain
        // the copies in flight)
        wait_vmcnt<0>();
        __syncthreads();  // s_page

        // queue the copies of tile t into ring stage buf
        auto issue = [&](int t, int buf) __attribute__((always_inline)) {
            const int tok0 = 32 * t;
            const int blk = tok0 / BLK;
            const int page = __builtin_amdgcn_readfirstlane(s_page[blk - blk0]);
            const int64_t goff = (static_cast<int64_t>(page) * c.Hkv + kvh) * static_cast<int64_t>(BLK * D) +
                                 (tok0 - blk * BLK) * D + lane * 8;
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int ch = wave * CPW + i;
                const uint16_t* src = (ch < CH / 2) ? kpool + goff + ch * 512
                                                    : vpool + goff + (ch - CH / 2) * 512;
                copy16_to_lds(src, &ring[buf][ch * 512]);
            }
        };

        // One barrier per tile.  Tiles are copied DIST = NS - 2 ahead, so the
        // stage refilled in iteration k last held tile k - 2; every wave has
        // finished computing tile k - 2 before it reached the barrier of
        // iteration k - 1, which the refilling wave has passed.
        constexpr int DIST = NS - 2;
        static_assert(DIST >= 1, "ring stages");
#pragma unroll
        for (int k = 0; k < DIST; ++k)
            if (k < nt) issue(t0 + k, k);
        for (int k = 0; k < nt; ++k) {
            const int t = t0 + k;
            const uint16_t* st = ring[k % NS];
            if (k + DIST < nt) {
                issue(t + DIST, (k + DIST) % NS);
                wait_vmcnt<CPW * DIST>();  // this wave's copies of tile k have landed
            } else {
                wait_vmcnt<0>();
            }
            __builtin_amdgcn_s_barrier();  // ... and every other wave's
            asm volatile("" ::: "memory");  // no LDS read moves above this point
            const uint16_t* ks_lds = st + lane * 8;
            const uint16_t* vs_lds = st + TILE_EL + lane * 8;
            u32x4 kr[2 * KS];
#pragma unroll
            for (int kk = 0; kk < 2 * KS; ++kk) kr[kk] = *reinterpret_cast<const u32x4*>(ks_lds + kk * 512);
            const int tok0 = 32 * t;
            const int nvalid = T - tok0;  // >= 1
            u32x4 vr[NT];
            // S^T of every row tile first: the matrix cores work on the later
            // row tiles' products while the softmax of the first one runs
            floatx4 sacc_rt[RTW][2];
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    sacc_rt[rt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        sacc_rt[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, kr[mt * KS + ks]), qb[rt][ks], sacc_rt[rt][mt],
                            0, 0, 0);
                }
            // V operands are read once the K operands are consumed, which
            // keeps both out of registers at the same time
            asm volatile("" ::: "memory");
#pragma unroll
            for (int n = 0; n < NT; ++n) vr[n] = *reinterpret_cast<const u32x4*>(vs_lds + n * 512);
            if (nvalid < 32) {  // zero V of the tokens past T (ragged last tile)
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const int tok = (kk < 4) ? (4 * g + kk) : (16 + 4 * g + kk - 4);
                    if (tok >= nvalid) {
                        const uint32_t keep = (kk & 1) ? 0x0000ffffu : 0xffff0000u;
#pragma unroll
                        for (int n = 0; n < NT; ++n) vr[n][kk >> 1] &= keep;
                    }
                }
            }
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
                // raw scores; the scale is folded into the exponent below
                float x[8];
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) x[kk] = sacc_rt[rt][kk >> 2][kk & 3];
                if (tok0 + 31 > T - f) {  // the causal mask only bites in the last f tokens
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) {
                        const int tok = tok0 + ((kk < 4) ? (4 * g + kk) : (16 + 4 * g + kk - 4));
                        x[kk] = (tok <= pos[rt]) ? x[kk] : -INFINITY;
                    }
                }
                float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                   fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
                tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
                // The reference point of the exponentials moves only when a row's
                // score exceeds it by more than kRebase (log2 units), so most tiles
                // skip the accumulator rescale; p stays below 2^kRebase, which the
                // fp32 sums and the bf16 P operand carry without loss of range.
                if (__ballot(tmax > m_run[rt] + rebase) != 0) {
                    const float m_new = fmaxf(m_run[rt], tmax);
                    // a row that has seen nothing keeps its (zero) state
                    const float alpha = (m_new == -INFINITY)
                                            ? 1.f
                                            : __builtin_amdgcn_exp2f((m_run[rt] - m_new) * sl2);
                    l_run[rt] *= alpha;
                    m_run[rt] = m_new;
                    nms[rt] = (m_new == -INFINITY) ? 0.f : -m_new * sl2;
                    float al[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * g + e, 64);
#pragma unroll
                    for (int n = 0; n < NT; ++n)
#pragma unroll
                        for (int e = 0; e < 4; ++e) oacc[rt][n][e] *= al[e];
                }
                float pr[8];
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) pr[kk] = __builtin_amdgcn_exp2f(fmaf(x[kk], sl2, nms[rt]));
                l_run[rt] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
                bf16x8 ph;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) ph[kk] = static_cast<__bf16>(pr[kk]);
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    oacc[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        ph, __builtin_bit_cast(bf16x8, vr[n]), oacc[rt][n], 0, 0, 0);
            }
        }

        // partials of this wave's rows for the piece, in slot `slot`
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            float l_tot = l_run[rt] + __shfl_xor(l_run[rt], 16, 64);
            l_tot += __shfl_xor(l_tot, 32, 64);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 4 * g + e;  // row inside the tile held in element e
                const float L = __shfl(l_tot, rr, 64);
                const float M = __shfl(m_run[rt], rr, 64);
                const int r = (rt0 + rt) * 16 + rr;
                if (r >= R) continue;
                const int64_t prow = slot * RWG + (r - zg * RWG);
                float* op = a.o_part + prow * D;
                const bool empty = (M == -INFINITY);
#pragma unroll
                for (int n = 0; n < NT; ++n) op[n * 16 + col] = empty ? 0.f : oacc[rt][n][e] / L;
                if (col == 0) a.lse_part[prow] = empty ? -INFINITY : M * sl2 + log2f(L);
            }
        }

        // ---- next piece ----
        left -= nt;
        if (left <= 0) break;
        off = 0;
        if (++gl == per_seq) {
            gl = 0;
            do {
                ++s;
                nts = ntiles_of(c.seq_lens[s]);
            } while (nts == 0);  // tiles remain, so a non-empty sequence follows
        }
    }
}

// ---------------------------------------------------------------------------
// 256-row shape (more than 128 rows per KV head): one workgroup of 8 waves per
// CU, two 16-row tiles per wave, an 8-stage LDS ring.
//
// Ping-pong schedule.  Waves 0-3 (group A) and 4-7 (group B) share the four
// SIMDs pairwise and work half a tile apart: in every phase (the span between
// two workgroup barriers) one wave of each SIMD runs its matrix products
// while the other runs the exponentials of its softmax, so the matrix cores
// and the VALU are busy at the same time instead of in turn.  32x32x16 MFMAs
// take half the issue slots of 16x16x32 ones for the same work, which leaves
// the other wave's VALU nearly its full rate.  Per wave and tile k, the VALU
// phase reads K(k+1) from LDS and takes exp2 of tile k's scores (from the
// previous matrix phase); the matrix phase computes S(k+1) = K(k+1) Q^T and
// O += P(k-1) V(k-1) (16 MFMAs), with tile k's row sums and bf16 P and the
// LDS reads of V(k) placed between them.  Group A's phases are 2k (VALU) and
// 2k+1 (matrix); group B's are 2k+1 and 2k+2.  Only group A copies tiles into
// the ring: tile k + NS - 3 in its VALU phase k (where it waits for group B's
// matrix phase anyway), and it waits for its copies of tile k+1 before the
// barrier that opens phase 2k; the last use of a stage (group B's PV of the
// tile it held, phase 2k - 2) ends before the stage is refilled.
//
// The softmax takes no maximum on its common path: the exponentials use the
// current reference max, and only when some lane's sum of its sixteen
// exponentials exceeds 2^kRebase (or is not finite) does the wave take the
// slow path, which finds the tile's row maxima (a permlane swap with the lane
// holding the row's other half), moves the reference, rescales O and the row
// sums and recomputes P.  The reference starts at +inf in exponent units, so the first
// tile of every piece takes the slow path.
//
// More than 256 rows go to further sets of workgroups, one row group each.
// Every set runs the same stream-K split of the same tile list, so workgroup w
// of every set reads the same tiles at about the same time; the set size is a
// multiple of 8, which puts those workgroups on one XCD (workgroups are dealt
// to the eight XCDs in turn), so the later reads of a tile hit that XCD's L2
// instead of HBM.  Page ids come from the page table by scalar loads issued
// one tile before they are used.
// ---------------------------------------------------------------------------
constexpr int kWideRows = 256;  // rows per workgroup: 8 waves x two 16-row tiles
constexpr int kWideStages = 8;  // LDS ring stages (16 KiB each at d = 128)
constexpr int kWideWGs = 256;   // workgroups resident at once: one per CU
constexpr float kPmax = 256.f;  // 2^kRebase: largest lane sum of exponentials on the fast path

int wide_sets(int R) { return (R + kWideRows - 1) / kWideRows; }
int wide_set_wgs(int Z) {
    const int w = (kWideWGs / Z) / 8 * 8;
    return w < 8 ? 8 : w;
}
// workgroups of a set that take tiles, for N tiles in the list
__device__ __forceinline__ int wide_wgs(int64_t N, int per_set) {
    if (N <= 0) return 0;
    return static_cast<int>(min(static_cast<int64_t>(per_set), (N + kMinTilesPerWG - 1) / kMinTilesPerWG));
}

// Maximum of v and the value in lane ^ 32, returned to both lanes.
__device__ __forceinline__ float half_swap_max(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Workgroup barrier that no instruction is scheduled across (the phases of
// the ping-pong must stay on their side of it) and no LDS access moves across.
__device__ __forceinline__ void phase_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int D, int BLK>
__global__ __launch_bounds__(8 * kWave) void rectify_wide_kernel(RectifyParams p) {
    constexpr int NW = 8;
    constexpr int NS = kWideStages;
    constexpr int DIST = NS - 3;
    constexpr int KQ = D / 16;   // k steps of S^T = K Q^T (16 channels each)
    constexpr int NB = D / 32;   // 32-channel column blocks of O
    constexpr int TILE_EL = 32 * D;
    constexpr int CH = 2 * TILE_EL / 512;  // 1 KiB chunks per tile, K then V
    constexpr int CPW = CH / (NW / 2);     // chunks each group-A wave copies
    static_assert(CPW >= 1 && CPW * (NW / 2) == CH, "chunks split evenly over group A");
    static_assert((NS & (NS - 1)) == 0, "ring stages: a power of two");
    __shared__ __attribute__((aligned(16))) uint16_t ring[NS][2 * TILE_EL];
    __shared__ long long s_loc[4];

    const CacheArgs& c = p.c;
    const RectifyArgs& a = p.a;
    const int G = c.G;
    const int f = a.f;
    const int R = G * f;
    const int per_set = a.wgs / a.sets;
    const int z = blockIdx.x / per_set;  // set = row group
    const int w = blockIdx.x - z * per_set;
    const int per_seq = c.Hkv;
    const int64_t slot_base = static_cast<int64_t>(z) * (static_cast<int64_t>(c.B) * c.Hkv + per_set);

    if (threadIdx.x < kWave) {
        const SeqHit tot = seq_scan(c.seq_lens, c.B, per_seq, -1);
        const int W = wide_wgs(tot.N, per_set);
        int64_t x0 = 0, x1 = 0;
        SeqHit h{tot.N, -1, 0};
        if (w < W) {
            x0 = wg_begin(w, tot.N, W);
            x1 = wg_begin(w + 1, tot.N, W);
            h = seq_scan(c.seq_lens, c.B, per_seq, x0);
        }
        if (threadIdx.x == 0) {
            s_loc[0] = (w < W && x1 > x0) ? h.s : -1;
            s_loc[1] = x0 - h.start;
            s_loc[2] = x1 - x0;
        }
    }
    __syncthreads();
    int s = __builtin_amdgcn_readfirstlane(static_cast<int>(s_loc[0]));
    if (s < 0) return;
    const int64_t pos0 = s_loc[1];
    const int64_t left0 = s_loc[2];
    int64_t left = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(left0 >> 32))) << 32) |
                   static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(left0)));
    int nts = ntiles_of(c.seq_lens[s]);
    int gl = __builtin_amdgcn_readfirstlane(static_cast<int>(pos0 / nts));
    int off = __builtin_amdgcn_readfirstlane(static_cast<int>(pos0 - static_cast<int64_t>(gl) * nts));

    const uint16_t* kpool = static_cast<const uint16_t*>(c.k_pool);
    const uint16_t* vpool = static_cast<const uint16_t*>(c.v_pool);
    const float sl2 = a.scale_log2;

    while (true) {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const bool grp_a = wave < NW / 2;
        const int hf = lane >> 5;  // lane half
        const int l32 = lane & 31;
        const int kvh = gl;
        const int T = c.seq_lens[s];
        const int t0 = off;
        const int nt = static_cast<int>(min(left, static_cast<int64_t>(nts - off)));
        const int64_t slot = slot_base + static_cast<int64_t>(s) * per_seq + gl + w;
        const int64_t row_base = (static_cast<int64_t>(s) * c.Hq + kvh * G) * f;  // row r = 0
        const int r_wave = z * kWideRows + wave * 32;                               // first row of this wave
        const int32_t* ptrow = c.page_table + static_cast<int64_t>(s) * c.max_blocks;
        // page ids by scalar loads (constant address space: the table is
        // never written by this kernel)
        const __attribute__((address_space(4))) int32_t* ptrow_s =
            (const __attribute__((address_space(4))) int32_t*)(ptrow);
        const int64_t head_off = static_cast<int64_t>(kvh) * (BLK * D) + lane * 8;
        // per-lane LDS element offsets of the K (A operand) and V (B operand)
        // pieces inside a ring stage, from the page's operand order
        const int k_lane = (l32 >> 4) * (D / 32) * 512 + ((lane & 15) + 16 * hf) * 8;
        const int v_lane = TILE_EL + (l32 >> 4) * 512 + (lane & 15) * 8 + hf * 128;

        __syncthreads();  // the previous piece is done with the ring

        // B operand of S^T = K Q^T: row r_wave + l32, channels 16 kq + 8 hf ..
        const int r_me = r_wave + l32;
        const int pos = (r_me < R) ? T - f + (r_me % f) : T - 1;  // query position of the lane's row
        bf16x8 qb[KQ];
        {
            const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (row_base + r_me) * D + 8 * hf;
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (r_me < R) v = ldg16(qp + kq * 16);
                qb[kq] = __builtin_bit_cast(bf16x8, v);
            }
        }
        floatx16 oacc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[nb][e] = 0.f;
        float m_run = -INFINITY, l_run = 0.f;
        float nms = INFINITY;  // forces the slow path on the first tile
        wait_vmcnt<0>();

        auto page_of = [&](int t) __attribute__((always_inline)) {
            return ptrow_s[__builtin_amdgcn_readfirstlane((32 * t) / BLK)];
        };
        // group A: queue the copies of tile t (page id pg) into ring stage buf
        auto issue = [&](int t, int buf, int pg) __attribute__((always_inline)) {
            const int tok0 = 32 * t;
            const int64_t goff = static_cast<int64_t>(pg) * c.Hkv * (BLK * D) + head_off + (tok0 % BLK) * D;
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int ch = wave * CPW + i;
                const uint16_t* src = (ch < CH / 2) ? kpool + goff + ch * 512
                                                    : vpool + goff + (ch - CH / 2) * 512;
                copy16_to_lds(src, &ring[buf][ch * 512]);
            }
        };
        auto read_k = [&](u32x4* kr, int buf) __attribute__((always_inline)) {
            const uint16_t* st = ring[buf] + k_lane;
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq)
                kr[kq] = *reinterpret_cast<const u32x4*>(st + (kq >> 1) * 512 + (kq & 1) * 256);
        };
        auto read_v = [&](u32x4* vr, int buf) __attribute__((always_inline)) {
            const uint16_t* st = ring[buf] + v_lane;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    vr[2 * nb + m] = *reinterpret_cast<const u32x4*>(st + nb * 1024 + m * 256);
        };

        const int t_last = t0 + nt - 1;
        // Page id of the next tile to copy: pg_load is the scalar load in
        // flight, pg_next its value.  Scalar and LDS loads share one wait
        // counter, so the value is taken over right after the matrix phase
        // has waited for its LDS operands anyway, never where LDS reads are
        // still in flight.
        int pg_load = 0, pg_next = 0;
        if (grp_a) {
#pragma unroll
            for (int k = 0; k < DIST; ++k)
                if (k < nt) issue(t0 + k, k, page_of(t0 + k));
            pg_next = page_of(min(t0 + DIST, t_last));
            pg_load = pg_next;
            if (nt >= DIST)
                wait_vmcnt<CPW * (DIST - 1)>();
            else
                wait_vmcnt<0>();
        }
        phase_barrier();  // tile 0 is in the ring

        // S^T of tile 0 of the piece (both groups): accumulator element 4j + i
        // holds token 8j + 4 hf + i of the tile for the lane's row
        floatx16 sc;
        u32x4 kr[KQ];
        u32x4 vr[2 * NB];
        read_k(kr, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq)
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr[kq]), qb[kq], sc, 0, 0, 0);
        bf16x8 pk[2], pprev[2];  // P of tokens {8m + 4hf + i, 16 + 8m + 4hf + i}: the A operands of PV
        // A reference moved in the VALU phase of tile k applies to O once
        // PV(k-1) is in it: at the start of the next VALU phase (or before
        // the last PV).  O's element 4j + i of every block is row 8j + 4hf + i
        // and takes the factor of the lane holding that row.
        bool resc_pending = false;
        float alpha_pending = 1.f;
        auto rescale_o = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float al = __shfl(alpha_pending, 8 * (e >> 2) + 4 * hf + (e & 3), 64);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) oacc[nb][e] *= al;
            }
            resc_pending = false;
        };
        if (!grp_a) phase_barrier();  // group B runs one phase behind

        // tiles from k_mask on reach into the causal tail [T - f + 1, T)
        const int k_mask = max(0, min(nt, (T - f + 1) / 32 - t0));
        // one tile: VALU phase (LDS reads for the next matrix phase, softmax of
        // tile k), then matrix phase (S(k+1), O += P(k-1) V(k-1))
        auto iter = [&](int k, auto mask_tag) __attribute__((always_inline)) {
            constexpr bool masked = decltype(mask_tag)::value;
            const int t = t0 + k;
            if (grp_a) {
                // this wave's copies of tile k + 1 have landed (tiles up to
                // k - 1 + DIST are queued)
                if (k + DIST - 1 < nt)
                    wait_vmcnt<CPW * (DIST - 2)>();
                else
                    wait_vmcnt<0>();
            }
            phase_barrier();
            // ---- VALU phase: K(k+1) from LDS, exponentials of tile k ----
            read_k(kr, (k + 1) & (NS - 1));
            if (grp_a && k + DIST < nt) {
                issue(t + DIST, (k + DIST) & (NS - 1), pg_next);
                pg_load = page_of(min(t + DIST + 1, t_last));
            }
            __builtin_amdgcn_sched_barrier(0);  // the reads go out first; the softmax hides their latency
            if (resc_pending) rescale_o();
            const int tok_lane = 32 * t + 4 * hf;
            float pr[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float x = sc[e];
                if (masked) x = (tok_lane + 8 * (e >> 2) + (e & 3) <= pos) ? x : -INFINITY;
                pr[e] = __builtin_amdgcn_exp2f(fmaf(x, sl2, nms));
            }
            // the lane's sum of exponentials at most 2^kRebase, so every one
            // is (NaN and inf fail the test); the sum feeds the row sum too
            float ls = (((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]))) +
                       (((pr[8] + pr[9]) + (pr[10] + pr[11])) + ((pr[12] + pr[13]) + (pr[14] + pr[15])));
            float alpha = 1.f;
            const bool resc = __ballot(!(ls <= kPmax)) != 0;  // uniform
            if (resc) {
                // slow path: find the row maxima of the tile, move the reference
                float x[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    x[e] = sc[e];
                    if (masked) x[e] = (tok_lane + 8 * (e >> 2) + (e & 3) <= pos) ? x[e] : -INFINITY;
                }
                float tmax = x[0];
#pragma unroll
                for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, x[e]);
                tmax = half_swap_max(tmax);  // the row's other 16 tokens sit in lane ^ 32
                const float m_new = fmaxf(m_run, tmax);
                const bool none = (m_new == -INFINITY);  // the row has seen no token yet
                alpha = none ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * sl2);
                m_run = m_new;
                nms = none ? INFINITY : -m_new * sl2;
                const float nm = none ? 0.f : nms;
#pragma unroll
                for (int e = 0; e < 16; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(x[e], sl2, nm));
                ls = (((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]))) +
                     (((pr[8] + pr[9]) + (pr[10] + pr[11])) + ((pr[12] + pr[13]) + (pr[14] + pr[15])));
            }
            resc_pending = resc;
            alpha_pending = alpha;
            // ---- matrix phase: S(k+1), O += P(k-1) V(k-1); the row sums and
            // bf16 P of tile k and the V(k) reads fill the gaps ----
            phase_barrier();
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq)
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr[kq]), qb[kq], sc, 0, 0, 0);
            asm volatile("s_mov_b32 %0, %1" : "=s"(pg_next) : "s"(pg_load));
            l_run = l_run * alpha + ls;
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pk[m][i] = static_cast<__bf16>(pr[4 * m + i]);
                    pk[m][4 + i] = static_cast<__bf16>(pr[4 * m + 8 + i]);
                }
            if (k > 0) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int m = 0; m < 2; ++m)
                        oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            pprev[m], __builtin_bit_cast(bf16x8, vr[2 * nb + m]), oacc[nb], 0, 0, 0);
            }
            read_v(vr, k & (NS - 1));  // V(k) for the next matrix phase
            // interleave: the S MFMAs with the VALU work, the PV MFMAs with
            // the V reads that replace their operands
#pragma unroll
            for (int i = 0; i < KQ; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
#pragma unroll
            for (int i = 0; i < 2 * NB; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            pprev[0] = pk[0];
            pprev[1] = pk[1];
        };
        int k = 0;
        for (; k < k_mask; ++k) iter(k, std::false_type{});
        for (; k < nt; ++k) iter(k, std::true_type{});
        if (grp_a) phase_barrier();  // group A ends one phase earlier
        if (resc_pending) rescale_o();

        // PV of the piece's last tile (the only one that can run past T;
        // its V was read in the last matrix phase)
        {
            const int nvalid = T - 32 * t_last;
            if (nvalid < 32) {
                // zero V of the tokens past T: k-slot e of m holds token
                // 8m + 4hf + e (e < 4) or 16 + 8m + 4hf + e - 4
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tok = 8 * m + 4 * hf + (e & 3) + 16 * (e >> 2);
                        if (tok >= nvalid) {
                            const uint32_t keep = (e & 1) ? 0x0000ffffu : 0xffff0000u;
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb) vr[2 * nb + m][e >> 1] &= keep;
                        }
                    }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        pprev[m], __builtin_bit_cast(bf16x8, vr[2 * nb + m]), oacc[nb], 0, 0, 0);
        }

        // partials of this wave's rows for the piece, in slot `slot`: element
        // 4j + i of block nb is row 8j + 4 hf + i, channel 32 nb + l32
        const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int rr = 8 * (e >> 2) + 4 * hf + (e & 3);
            const float L = __shfl(l_tot, rr, 64);
            const float M = __shfl(m_run, rr, 64);
            const int r = r_wave + rr;
            if (r >= R) continue;
            const int64_t prow = slot * kWideRows + (r - z * kWideRows);
            float* op = a.o_part + prow * D + l32;
            const bool empty = (M == -INFINITY);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) op[nb * 32] = empty ? 0.f : oacc[nb][e] / L;
            if (l32 == 0) a.lse_part[prow] = empty ? -INFINITY : M * sl2 + log2f(L);
        }

        left -= nt;
        if (left <= 0) break;
        off = 0;
        if (++gl == per_seq) {
            gl = 0;
            do {
                ++s;
                nts = ntiles_of(c.seq_lens[s]);
            } while (nts == 0);
        }
    }
}

// Merge of the pieces of every row of the bf16 path, in list order.  One
// workgroup per 16 rows of a row group: 16 threads per row, each owning d/16
// channels; the row's pieces (one partial per slot, RWG partial rows apart)
// are read four at a time and weighted by 2^(lse_k - M).  WIDE: the
// 256-row shape, whose row groups are sets of workgroups over one list of
// (sequence, KV head) groups; otherwise the row groups are groups of the
// list.
template <int RWG, int D, bool WIDE>
__global__ __launch_bounds__(256) void rectify_merge_kernel(RectifyParams p) {
    constexpr int CPT = D / 16;  // channels per thread
    static_assert(CPT % 4 == 0, "float4 channel groups");
    __shared__ long long s_loc[2];
    const CacheArgs& c = p.c;
    const RectifyArgs& a = p.a;
    const int R = c.G * a.f;
    const int Z = (R + RWG - 1) / RWG;
    const int per_seq = WIDE ? c.Hkv : c.Hkv * Z;
    const int nrb = (R + 15) / 16;
    const int grp = blockIdx.x / nrb;  // s * Hkv + kvh
    const int r0 = (blockIdx.x - grp * nrb) * 16;
    const int s = grp / c.Hkv;
    const int kvh = grp - s * c.Hkv;
    const int zg = r0 / RWG;  // the 16 rows share a row group (RWG is a multiple of 16)
    const int tid = threadIdx.x;
    if (tid < kWave) {
        const SeqHit tot = seq_scan(c.seq_lens, c.B, per_seq, -1);
        const SeqHit pre = seq_scan(c.seq_lens, s, per_seq, -1);  // tiles of sequences < s
        if (tid == 0) {
            s_loc[0] = tot.N;
            s_loc[1] = pre.N;
        }
    }
    __syncthreads();
    const int64_t N = s_loc[0];
    const int nts = ntiles_of(c.seq_lens[s]);
    const int per_set = WIDE ? a.wgs / a.sets : a.wgs;
    const int W = WIDE ? wide_wgs(N, per_set) : stream_wgs(N, a.wgs);
    const int gl = WIDE ? kvh : kvh * Z + zg;
    const int64_t start = s_loc[1] + static_cast<int64_t>(gl) * nts;
    const int64_t slot_base =
        WIDE ? static_cast<int64_t>(zg) * (static_cast<int64_t>(c.B) * c.Hkv + per_set) : 0;
    int w0 = 0, npieces = 0;
    if (nts > 0) {
        w0 = wg_owner(start, N, W);
        npieces = wg_owner(start + nts - 1, N, W) - w0 + 1;
    }
    const int row = tid >> 4;
    const int q = tid & 15;
    const int r = r0 + row;
    const bool valid = r < R;
    const int64_t prow0 = (slot_base + static_cast<int64_t>(s) * per_seq + gl + w0) * RWG + (r - zg * RWG);
    const float* lp = a.lse_part + prow0;
    float M = -INFINITY;
    if (valid)
        for (int k = q; k < npieces; k += 16) M = fmaxf(M, lp[static_cast<int64_t>(k) * RWG]);
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 16));
    float acc[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) acc[i] = 0.f;
    float L = 0.f;
    if (valid && M != -INFINITY) {
        const float* op = a.o_part + prow0 * D + q * CPT;
        for (int k0 = 0; k0 < npieces; k0 += 4) {
            float lv[4];
            floatx4 ov[4][CPT / 4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t k = k0 + u;
                lv[u] = -INFINITY;
                if (k < npieces) {
                    lv[u] = lp[k * RWG];
#pragma unroll
                    for (int v = 0; v < CPT / 4; ++v)
                        ov[u][v] = *reinterpret_cast<const floatx4*>(op + k * RWG * D + 4 * v);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (k0 + u >= npieces) break;
                const float wk = exp2f(lv[u] - M);
                L += wk;
#pragma unroll
                for (int v = 0; v < CPT / 4; ++v)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[4 * v + e] += wk * ov[u][v][e];
            }
        }
    }
    if (!valid) return;
    const bool empty = (M == -INFINITY);
    const int64_t orow = (static_cast<int64_t>(s) * c.Hq + kvh * c.G) * a.f + r;
    typedef typename Elem<kBF16>::T E;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
        Elem<kBF16>::store(static_cast<E*>(a.o), orow * D + q * CPT + i, empty ? 0.f : acc[i] / L);
    if (q == 0) a.lse[orow] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
}

// fp32 caches: one wave per row at a time, lane t < 32 owns token t of a tile.
template <int D>
__global__ __launch_bounds__(kThreads) void rectify_f32_kernel(RectifyParams p) {
    constexpr int CPL = D / 64;
    const CacheArgs& c = p.c;
    const RectifyArgs& a = p.a;
    const int split = blockIdx.x;
    const int grp = blockIdx.y;
    const int s = grp / c.Hkv;
    const int kvh = grp - s * c.Hkv;
    const int G = c.G;
    const int f = a.f;
    const int R = G * f;
    const int T = c.seq_lens[s];
    const int S = a.splits;
    const int BLK = c.block;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t row_base = (static_cast<int64_t>(s) * c.Hq + kvh * G) * f;
    const int ntiles = (T + 31) / 32;
    const int t0 = split * a.chunk_tiles;
    const int t1 = min(t0 + a.chunk_tiles, ntiles);
    if (t0 >= t1) return;
    const float* kpool = static_cast<const float*>(c.k_pool);
    const float* vpool = static_cast<const float*>(c.v_pool);
    const int32_t* ptrow = c.page_table + static_cast<int64_t>(s) * c.max_blocks;

    for (int r = blockIdx.z * kWaves + wave; r < R; r += kWaves * gridDim.z) {
        const int posr = T - f + (r % f);
        const float* qr = static_cast<const float*>(a.q) + (row_base + r) * D;
        float m = -INFINITY, l = 0.f, o[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) o[k] = 0.f;
        for (int t = t0; t < t1; ++t) {
            const int tok0 = 32 * t;
            const int blk = tok0 / BLK;
            const int64_t page = ptrow[blk];
            const int64_t off = (page * c.Hkv + kvh) * static_cast<int64_t>(BLK * D) + (tok0 - blk * BLK) * D;
            const int nvis = min(32, posr + 1 - tok0);  // tokens this row may see
            if (nvis <= 0) break;
            float z = -INFINITY;
            if (lane < nvis) {
                float acc = 0.f;
                for (int i = 0; i < D; ++i) acc += qr[i] * kpool[off + lane * D + i];
                z = acc * a.scale_log2;
            }
            const float mt = wave_max(z);
            const float m_new = fmaxf(m, mt);
            const float alpha = exp2f(m - m_new);
            const float pz = (lane < nvis) ? exp2f(z - m_new) : 0.f;
            l = l * alpha + wave_sum(pz);
            m = m_new;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                float acc = o[k] * alpha;
                for (int tt = 0; tt < nvis; ++tt)
                    acc += __shfl(pz, tt, 64) * vpool[off + tt * D + lane + 64 * k];
                o[k] = acc;
            }
        }
        const int64_t row = row_base + r;
        float* op = a.o_part + (row * S + split) * D;
        const bool empty = (m == -INFINITY);
#pragma unroll
        for (int k = 0; k < CPL; ++k) op[lane + 64 * k] = empty ? 0.f : o[k] / l;
        if (lane == 0) a.lse_part[row * S + split] = empty ? -INFINITY : m + log2f(l);
    }
}

// Rows (G*f) per workgroup: up to 64 with 4 waves, up to 128 with 8 waves of
// one 16-row tile each (two workgroups per CU), more in the 256-row shape
// (one workgroup per CU, row groups of 256 in co-scheduled sets).
int rows_per_wg(int R) { return R <= 64 ? 64 : (R <= 128 ? 128 : kWideRows); }

template <int D, int BLK, int RTW, int NW>
hipError_t launch_bf16(const RectifyParams& p, hipStream_t stream) {
    constexpr int RWG = 16 * RTW * NW;
    if (p.a.rows_per_wg != RWG || p.a.sets != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rectify_bf16_kernel<D, BLK, RTW, kStages, NW>), dim3(p.a.wgs),
                       dim3(NW * kWave), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int R = p.c.G * p.a.f;
    const int64_t wgs = static_cast<int64_t>(p.c.B) * p.c.Hkv * ((R + 15) / 16);
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rectify_merge_kernel<RWG, D, false>), dim3(static_cast<uint32_t>(wgs)), dim3(256),
                       0, stream, p);
    return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_wide(const RectifyParams& p, hipStream_t stream) {
    const int R = p.c.G * p.a.f;
    if (p.a.rows_per_wg != kWideRows || p.a.sets != wide_sets(R) || p.a.wgs % p.a.sets != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((rectify_wide_kernel<D, BLK>), dim3(p.a.wgs), dim3(8 * kWave), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t wgs = static_cast<int64_t>(p.c.B) * p.c.Hkv * ((R + 15) / 16);
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rectify_merge_kernel<kWideRows, D, true>), dim3(static_cast<uint32_t>(wgs)),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_bf16_r(const RectifyParams& p, hipStream_t stream) {
    const int R = p.c.G * p.a.f;
    if (R <= 64) return launch_bf16<D, BLK, 1, 4>(p, stream);
    if (R <= 128) return launch_bf16<D, BLK, 1, 8>(p, stream);
    return launch_wide<D, BLK>(p, stream);
}

template <int D>
hipError_t launch_bf16_d(const RectifyParams& p, hipStream_t stream) {
    switch (p.c.block) {
        case 32: return launch_bf16_r<D, 32>(p, stream);
        case 64: return launch_bf16_r<D, 64>(p, stream);
        case 128: return launch_bf16_r<D, 128>(p, stream);
        case 256: return launch_bf16_r<D, 256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_f32(const RectifyParams& p, hipStream_t stream) {
    const int R = p.c.G * p.a.f;
    const int zr = (R + 63) / 64;
    dim3 grid(p.a.splits, p.c.B * p.c.Hkv, zr);
    hipLaunchKernelGGL((rectify_f32_kernel<D>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

void rectify_plan(const CacheArgs& c, int f, RectifyPlan* pl) {
    const int64_t max_tokens = static_cast<int64_t>(c.max_blocks) * c.block;
    const int64_t tiles = (max_tokens + 31) / 32;
    *pl = RectifyPlan{};
    if (c.dtype == kBF16) {
        const int R = c.G * f;
        const int rwg = rows_per_wg(R);
        pl->rows_per_wg = rwg;
        int64_t slots;
        if (rwg == kWideRows) {
            // sets of workgroups, each over the list of (sequence, KV head) groups
            const int Z = wide_sets(R);
            const int per_set = wide_set_wgs(Z);
            pl->sets = Z;
            pl->wgs = Z * per_set;
            slots = static_cast<int64_t>(Z) * (static_cast<int64_t>(c.B) * c.Hkv + per_set);
        } else {
            const int64_t groups = static_cast<int64_t>(c.B) * c.Hkv * ((R + rwg - 1) / rwg);
            const int64_t n_max = groups * tiles;
            const int64_t wgs = std::max<int64_t>(kStreamWGs, (n_max + kMaxTilesPerWG - 1) / kMaxTilesPerWG);
            pl->sets = 1;
            pl->wgs = static_cast<int>(std::min<int64_t>(wgs, 0x7fffffff));
            slots = groups + wgs;
        }
        pl->o_floats = slots * rwg * c.d;
        pl->lse_floats = slots * rwg;
    } else {
        pl->chunk_tiles = kChunkTiles;
        pl->splits = static_cast<int>((tiles + kChunkTiles - 1) / kChunkTiles);
        const int64_t rows = static_cast<int64_t>(c.B) * c.Hq * f;
        pl->o_floats = rows * pl->splits * c.d;
        pl->lse_floats = rows * pl->splits;
    }
}

hipError_t launch_rectify(const CacheArgs& c, const RectifyArgs& a, hipStream_t stream) {
    // 1. overwrite [T-f, T) and rebuild the descriptors of the blocks it touches
    hipError_t err = launch_kv_write(c, kModeOverwrite, a.k_new, a.v_new, a.f, nullptr, stream);
    if (err != hipSuccess) return err;
    RectifyParams p{c, a};
    // 2. causal dense attention over even shares of all tiles, then the merge
    if (c.dtype == kBF16) return c.d == 64 ? launch_bf16_d<64>(p, stream) : launch_bf16_d<128>(p, stream);
    // fp32: chunks of kChunkTiles tiles, then the merge of the chunks covering
    // [0, T) of each sequence
    err = c.d == 64 ? launch_f32<64>(p, stream) : launch_f32<128>(p, stream);
    if (err != hipSuccess) return err;
    return launch_combine_ragged(c.dtype, c.d, c.B * c.Hq * a.f, a.splits, a.o_part, a.lse_part,
                                 a.o, a.lse, c.seq_lens, c.Hq * a.f, 32 * a.chunk_tiles, stream);
}

}  // namespace bsa
