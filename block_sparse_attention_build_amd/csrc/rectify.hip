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

template <int D, int BLK, int RTW>
__global__ __launch_bounds__(kThreads) void rectify_bf16_kernel(RectifyParams p) {
    constexpr int KS = D / 32;
    constexpr int NT = D / 16;
    constexpr int TILE_EL = 32 * D;          // elements of K (or V) per tile
    constexpr int CHUNKS = TILE_EL / 8;      // 16-byte pieces per tile
    constexpr int PER_T = CHUNKS / kThreads; // pieces per thread (K or V)
    __shared__ __attribute__((aligned(16))) uint16_t stage[2][2 * TILE_EL];

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
    const int rt0 = (blockIdx.z * kWaves + wave) * RTW;  // first 16-row tile of this wave

    const int ntiles = (T + 31) / 32;
    const int t0 = split * a.chunk_tiles;
    const int t1 = min(t0 + a.chunk_tiles, ntiles);
    if (t0 >= t1) return;  // the merge only reads the chunks that cover [0, T)

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
    const int32_t* ptrow = c.page_table + static_cast<int64_t>(s) * c.max_blocks;
    const float sl2 = a.scale_log2;

    u32x4 pre_k[PER_T], pre_v[PER_T];
    auto fetch = [&](int t) {
        const int tok0 = 32 * t;
        const int blk = tok0 / BLK;
        const int64_t page = ptrow[blk];
        const int64_t off = (page * c.Hkv + kvh) * static_cast<int64_t>(BLK * D) + (tok0 - blk * BLK) * D;
#pragma unroll
        for (int k = 0; k < PER_T; ++k) {
            const int piece = threadIdx.x + k * kThreads;
            pre_k[k] = ldg16(kpool + off + piece * 8);
            pre_v[k] = ldg16(vpool + off + piece * 8);
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int k = 0; k < PER_T; ++k) {
            const int piece = threadIdx.x + k * kThreads;
            *reinterpret_cast<u32x4*>(&stage[buf][piece * 8]) = pre_k[k];
            *reinterpret_cast<u32x4*>(&stage[buf][TILE_EL + piece * 8]) = pre_v[k];
        }
    };

    fetch(t0);
    stash(0);
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
        const int buf = (t - t0) & 1;
        if (t + 1 < t1) fetch(t + 1);
        const uint16_t* ks_lds = &stage[buf][lane * 8];
        const uint16_t* vs_lds = &stage[buf][TILE_EL + lane * 8];
        u32x4 kr[2 * KS];
#pragma unroll
        for (int k = 0; k < 2 * KS; ++k) kr[k] = *reinterpret_cast<const u32x4*>(ks_lds + k * 512);
        u32x4 vr[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) vr[n] = *reinterpret_cast<const u32x4*>(vs_lds + n * 512);
        const int tok0 = 32 * t;
        const int nvalid = T - tok0;  // >= 1
        if (nvalid < 32) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int tok = (k < 4) ? (4 * g + k) : (16 + 4 * g + k - 4);
                if (tok >= nvalid) {
                    const uint32_t keep = (k & 1) ? 0x0000ffffu : 0xffff0000u;
#pragma unroll
                    for (int n = 0; n < NT; ++n) vr[n][k >> 1] &= keep;
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
            float tmax = -INFINITY;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int tok = tok0 + ((k < 4) ? (4 * g + k) : (16 + 4 * g + k - 4));
                const float v = sacc[k >> 2][k & 3] * sl2;
                x[k] = (tok <= pos[rt]) ? v : -INFINITY;
                tmax = fmaxf(tmax, x[k]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m_run[rt], tmax);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // row sees nothing yet
            const float alpha = exp2f(m_run[rt] - m_use);
            float pr[8];
            float psum = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                pr[k] = exp2f(x[k] - m_use);
                psum += pr[k];
            }
            l_run[rt] = l_run[rt] * alpha + psum;
            m_run[rt] = m_new;
            float al[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * g + e, 64);
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) oacc[rt][n][e] *= al[e];
            u32x4 phi, plo;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint16_t h0 = f2bf(pr[2 * k]);
                const uint16_t h1 = f2bf(pr[2 * k + 1]);
                phi[k] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
                plo[k] = pack_bf2(pr[2 * k] - bf2f(h0), pr[2 * k + 1] - bf2f(h1));
            }
            const bf16x8 ph = __builtin_bit_cast(bf16x8, phi);
            const bf16x8 pl = __builtin_bit_cast(bf16x8, plo);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const bf16x8 vb = __builtin_bit_cast(bf16x8, vr[n]);
                oacc[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, oacc[rt][n], 0, 0, 0);
                oacc[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, oacc[rt][n], 0, 0, 0);
            }
        }
        if (t + 1 < t1) stash(buf ^ 1);
        __syncthreads();
    }

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

template <int D, int BLK, int RTW>
hipError_t launch_bf16(const RectifyParams& p, hipStream_t stream) {
    const int R = p.c.G * p.a.f;
    const int rows_per_wg = 64 * RTW;
    dim3 grid(p.a.splits, p.c.B * p.c.Hkv, (R + rows_per_wg - 1) / rows_per_wg);
    hipLaunchKernelGGL((rectify_bf16_kernel<D, BLK, RTW>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_bf16_r(const RectifyParams& p, hipStream_t stream) {
    const int R = p.c.G * p.a.f;
    if (R <= 64) return launch_bf16<D, BLK, 1>(p, stream);
    if (R <= 128) return launch_bf16<D, BLK, 2>(p, stream);
    return launch_bf16<D, BLK, 4>(p, stream);
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
