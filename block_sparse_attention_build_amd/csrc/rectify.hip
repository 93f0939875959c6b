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
// bf16 path: the only dense contraction of the method, on
// v_mfma_f32_16x16x32_bf16.  Rows = the G*f queries of a GQA group (G*f = 128
// for G = 4, f = 32).  One workgroup = (sequence, KV head, chunk of 32-token
// tiles, group of up to 64*RTW rows); each of its 4 waves owns RTW 16-row
// tiles.  K/V tiles (16 KiB at d = 128) are copied once per workgroup from HBM
// into a double-buffered LDS stage with coalesced 16-byte loads (the next
// tile's loads are in flight while the current one is computed) and every
// wave reads its matrix operands from LDS with conflict-free 16-byte reads.
// Per tile and 16-row tile: S^T = K Q^T (2 x d/32 MFMAs), causal mask, online
// softmax, O += P V with P split into bf16 hi + lo (2 x d/16 x 2 MFMAs).
// Each wave writes normalised partials (o, base-2 lse) for its own rows; the
// log-sum-exp merge (decode.hip) combines the chunks.
//
// fp32 path: same chunking, plain VALU arithmetic.
#include <math.h>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunkTiles = 64;  // 2048 tokens per workgroup
constexpr int kStages = 4;       // tiles in flight per workgroup (LDS ring)

struct RectifyParams {
    CacheArgs c;
    RectifyArgs a;
};

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Partials of rows that see no token of this chunk.
__device__ __forceinline__ void store_empty(float* o_part, float* lse_part, int64_t row, int S,
                                            int split, int D, int ch) {
    o_part[(row * S + split) * D + ch] = 0.f;
    if (ch == 0) lse_part[row * S + split] = -INFINITY;
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
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int D, int BLK, int RTW, int NS, int NW>
__global__ __launch_bounds__(NW * kWave) void rectify_bf16_kernel(RectifyParams p) {
    constexpr int KS = D / 32;
    constexpr int NT = D / 16;
    constexpr int TILE_EL = 32 * D;             // elements of K (or V) per tile
    constexpr int CH = 2 * TILE_EL / 512;       // 1 KiB chunks per tile, K then V
    constexpr int CPW = CH / NW;                // chunks each wave copies
    static_assert(CPW >= 1 && CPW * NW == CH, "chunks split evenly over the waves");
    // NS-stage ring of tiles in LDS, filled by direct global->LDS copies
    // (copy16_to_lds): each wave copies CPW KiB chunks per tile, NS-1 tiles
    // ahead of the one being computed, without using registers.
    __shared__ __attribute__((aligned(16))) uint16_t ring[NS][2 * TILE_EL];
    __shared__ int s_page[kChunkTiles * 32 / 32 + 2];

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
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int col = lane & 15;
    const int64_t row_base = (static_cast<int64_t>(s) * c.Hq + kvh * G) * f;  // output row of r = 0
    const int rt0 = (blockIdx.z * NW + wave) * RTW;  // first 16-row tile of this wave

    const int ntiles = (T + 31) / 32;
    const int t0 = split * a.chunk_tiles;
    const int t1 = min(t0 + a.chunk_tiles, ntiles);
    if (t0 >= t1) return;  // the merge only reads the chunks that cover [0, T)
    const int nt = t1 - t0;

    // page ids of the chunk's blocks (tiles are 32 tokens, blocks BLK tokens)
    const int32_t* ptrow = c.page_table + static_cast<int64_t>(s) * c.max_blocks;
    const int blk0 = (32 * t0) / BLK;
    const int nblk = (32 * (t1 - 1)) / BLK - blk0 + 1;
    for (int i = threadIdx.x; i < nblk; i += NW * kWave) s_page[i] = ptrow[blk0 + i];

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
            u32x4 w = {0u, 0u, 0u, 0u};
            if (r < R) w = ldg16(qp + ks * 32 + g * 8);
            qb[rt][ks] = __builtin_bit_cast(bf16x8, w);
        }
    }
    floatx4 oacc[RTW][NT];
    float m_run[RTW], l_run[RTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        m_run[rt] = -INFINITY;
        l_run[rt] = 0.f;
#pragma unroll
        for (int n = 0; n < NT; ++n) oacc[rt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    const uint16_t* kpool = static_cast<const uint16_t*>(c.k_pool);
    const uint16_t* vpool = static_cast<const uint16_t*>(c.v_pool);
    const float sl2 = a.scale_log2;
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
        const int64_t off = (static_cast<int64_t>(page) * c.Hkv + kvh) * static_cast<int64_t>(BLK * D) +
                            (tok0 - blk * BLK) * D + lane * 8;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const int ch = wave * CPW + i;
            const uint16_t* src = (ch < CH / 2) ? kpool + off + ch * 512
                                                : vpool + off + (ch - CH / 2) * 512;
            copy16_to_lds(src, &ring[buf][ch * 512]);
        }
    };

#pragma unroll
    for (int k = 0; k < NS - 1; ++k)
        if (k < nt) issue(t0 + k, k);
    for (int k = 0; k < nt; ++k) {
        const int t = t0 + k;
        const uint16_t* st = ring[k % NS];
        // every wave is done reading the stage refilled next (it held tile k-1)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (k + NS - 1 < nt) {
            issue(t + NS - 1, (k + NS - 1) % NS);
            wait_vmcnt<CPW * (NS - 1)>();  // this wave's copies of tile k have landed
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
        u32x4 vr[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) vr[n] = *reinterpret_cast<const u32x4*>(vs_lds + n * 512);
        const int tok0 = 32 * t;
        const int nvalid = T - tok0;  // >= 1
        if (nvalid < 32) {
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
            floatx4 sacc[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                sacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, kr[mt * KS + ks]), qb[rt][ks], sacc[mt], 0, 0, 0);
            }
            float x[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) x[kk] = sacc[kk >> 2][kk & 3] * sl2;
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
            if (__ballot(tmax > m_run[rt]) != 0) {  // some row's running max grows
                const float m_new = fmaxf(m_run[rt], tmax);
                const float alpha = __builtin_amdgcn_exp2f(m_run[rt] - m_new);
                l_run[rt] *= alpha;
                m_run[rt] = m_new;
                float al[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * g + e, 64);
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) oacc[rt][n][e] *= al[e];
            }
            const float m_use = (m_run[rt] == -INFINITY) ? 0.f : m_run[rt];  // row sees nothing yet
            float pr[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) pr[kk] = __builtin_amdgcn_exp2f(x[kk] - m_use);
            l_run[rt] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
            bf16x8 ph, pl;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) ph[kk] = static_cast<__bf16>(pr[kk]);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                pl[kk] = static_cast<__bf16>(pr[kk] - static_cast<float>(ph[kk]));
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const bf16x8 vb = __builtin_bit_cast(bf16x8, vr[n]);
                oacc[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, oacc[rt][n], 0, 0, 0);
                oacc[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, oacc[rt][n], 0, 0, 0);
            }
        }    }

    // partials for this wave's rows
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
            const int64_t row = row_base + r;
            float* op = a.o_part + (row * S + split) * D;
            const bool empty = (M == -INFINITY);
#pragma unroll
            for (int n = 0; n < NT; ++n) op[n * 16 + col] = empty ? 0.f : oacc[rt][n][e] / L;
            if (col == 0) a.lse_part[row * S + split] = empty ? -INFINITY : M + log2f(L);
        }
    }
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

template <int D, int BLK, int RTW, int NW>
hipError_t launch_bf16(const RectifyParams& p, hipStream_t stream) {
    const int R = p.c.G * p.a.f;
    const int rows_per_wg = 16 * RTW * NW;
    dim3 grid(p.a.splits, p.c.B * p.c.Hkv, (R + rows_per_wg - 1) / rows_per_wg);
    hipLaunchKernelGGL((rectify_bf16_kernel<D, BLK, RTW, kStages, NW>), grid, dim3(NW * kWave), 0,
                       stream, p);
    return hipGetLastError();
}

// Rows (G*f) per workgroup: up to 64 with 4 waves, up to 128 with 8 waves of
// one 16-row tile each (two waves per SIMD), 256 with 8 waves of two tiles;
// more rows take several workgroups along z.
template <int D, int BLK>
hipError_t launch_bf16_r(const RectifyParams& p, hipStream_t stream) {
    const int R = p.c.G * p.a.f;
    if (R <= 64) return launch_bf16<D, BLK, 1, 4>(p, stream);
    if (R <= 128) return launch_bf16<D, BLK, 1, 8>(p, stream);
    return launch_bf16<D, BLK, 2, 8>(p, stream);
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

void rectify_splits(const CacheArgs& c, int f, int* splits, int* chunk_tiles) {
    (void)f;
    const int64_t max_tokens = static_cast<int64_t>(c.max_blocks) * c.block;
    const int64_t tiles = (max_tokens + 31) / 32;
    *chunk_tiles = kChunkTiles;
    *splits = static_cast<int>((tiles + kChunkTiles - 1) / kChunkTiles);
}

hipError_t launch_rectify(const CacheArgs& c, const RectifyArgs& a, hipStream_t stream) {
    // 1. overwrite [T-f, T) and rebuild the descriptors of the blocks it touches
    hipError_t err = launch_kv_write(c, kModeOverwrite, a.k_new, a.v_new, a.f, nullptr, stream);
    if (err != hipSuccess) return err;
    // 2. causal dense attention, split over token chunks
    RectifyParams p{c, a};
    if (c.dtype == kBF16)
        err = c.d == 64 ? launch_bf16_d<64>(p, stream) : launch_bf16_d<128>(p, stream);
    else
        err = c.d == 64 ? launch_f32<64>(p, stream) : launch_f32<128>(p, stream);
    if (err != hipSuccess) return err;
    // 3. merge the chunks (only the chunks covering [0, T) of each sequence)
    return launch_combine_ragged(c.dtype, c.d, c.B * c.Hq * a.f, a.splits, a.o_part, a.lse_part,
                                 a.o, a.lse, c.seq_lens, c.Hq * a.f, 32 * a.chunk_tiles, stream);
}

}  // namespace bsa
