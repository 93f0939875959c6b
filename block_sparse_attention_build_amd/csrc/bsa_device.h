// bsa_device.h -- device-side building blocks shared by the libbsa kernels:
// storage types, bf16 conversion, the page layouts, wave reductions.
// gfx950 (CDNA4) only: wave64, bf16 matrix-core instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

constexpr int kWave = 64;

// dtype tags (match bsa_dtype)
constexpr int kF32 = 0;
constexpr int kBF16 = 1;
// descriptor kinds (match bsa_desc_kind)
constexpr int kMinMax = 0;
constexpr int kMeanPool = 1;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 values are carried as their 16-bit patterns.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}
// Two fp32 -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return static_cast<uint32_t>(f2bf(lo)) | (static_cast<uint32_t>(f2bf(hi)) << 16);
}

template <int DT> struct Elem;
template <> struct Elem<kF32> {
    typedef float T;
    static __device__ __forceinline__ float load(const T* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = v; }
    static __device__ __forceinline__ T from(float v) { return v; }
};
template <> struct Elem<kBF16> {
    typedef uint16_t T;
    static __device__ __forceinline__ float load(const T* p, int64_t i) { return bf2f(p[i]); }
    static __device__ __forceinline__ void store(T* p, int64_t i, float v) { p[i] = f2bf(v); }
    static __device__ __forceinline__ T from(float v) { return f2bf(v); }
};

// ---------------------------------------------------------------------------
// Page layouts (element offsets inside one page of b tokens x d channels).
// fp32: row major.  bf16: every 512 elements (1 KiB) are one 64-lane operand
// of v_mfma_f32_16x16x32_bf16, lane L holding 8 consecutive elements at
// L*8.  For a 16x32 (rows x k) operand the lane of (row r, k) is r + 16*(k/8)
// and its element is k%8.
//   K: operand A of S^T = K Q^T: rows = 16 tokens, k = 32 channels;
//      chunk = (t/16)*(d/32) + i/32.
//   V: operand B of O = P V: k = 32 tokens, columns = 16 channels;
//      chunk = (t/32)*(d/16) + i/16.  Within the 32 tokens, token slot
//      (lane group g, element e) holds token 4g+e (e < 4) or 16+4g+e-4
//      (e >= 4): exactly the tokens the S^T accumulator of lane group g
//      holds after two 16-token row tiles, so P needs no data movement.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int k_off_bf16(int t, int i, int d) {
    return (((t >> 4) * (d >> 5) + (i >> 5)) << 9) + (((t & 15) + (((i & 31) >> 3) << 4)) << 3) +
           (i & 7);
}
__host__ __device__ __forceinline__ int v_off_bf16(int t, int i, int d) {
    const int u = t & 31;
    const int g = (u & 15) >> 2;
    const int e = (u & 3) + ((u >> 4) << 2);
    return (((t >> 5) * (d >> 4) + (i >> 4)) << 9) + (((i & 15) + (g << 4)) << 3) + e;
}
template <int DT>
__host__ __device__ __forceinline__ int k_off(int t, int i, int d) {
    return DT == kBF16 ? k_off_bf16(t, i, d) : t * d + i;
}
template <int DT>
__host__ __device__ __forceinline__ int v_off(int t, int i, int d) {
    return DT == kBF16 ? v_off_bf16(t, i, d) : t * d + i;
}

// ---------------------------------------------------------------------------
// Wave helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, WIDTH);
    return v;
}

// ---------------------------------------------------------------------------
// DPP wave primitives (GFX9 data-parallel primitives: row_shr:n moves a value
// n lanes up inside each row of 16 lanes, row_bcast:15 hands lane 15 of a row
// to the next row, row_bcast:31 hands lane 31 to rows 2 and 3).  They run
// on the VALU with no LDS round trip, unlike the generic lane shuffles.
// Lanes with no source keep `old`, which is the operation's identity.
// ---------------------------------------------------------------------------
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_move(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += dpp_move<kDppRowShr1, 0xf>(0, x);
    x += dpp_move<kDppRowShr2, 0xf>(0, x);
    x += dpp_move<kDppRowShr4, 0xf>(0, x);
    x += dpp_move<kDppRowShr8, 0xf>(0, x);
    x += dpp_move<kDppRowBcast15, 0xa>(0, x);
    x += dpp_move<kDppRowBcast31, 0xc>(0, x);
    return x;
}

// Sum of float v over each run of W consecutive lanes (W = 16, 32 or 64),
// left in the run's last lane (the other lanes hold partial sums).
template <int W>
__device__ __forceinline__ float group_sum_last(float v) {
    static_assert(W == 16 || W == 32 || W == 64, "run width");
    auto add = [](float a, int b) { return a + __int_as_float(b); };
    v = add(v, dpp_move<kDppRowShr1, 0xf>(0, __float_as_int(v)));
    v = add(v, dpp_move<kDppRowShr2, 0xf>(0, __float_as_int(v)));
    v = add(v, dpp_move<kDppRowShr4, 0xf>(0, __float_as_int(v)));
    v = add(v, dpp_move<kDppRowShr8, 0xf>(0, __float_as_int(v)));
    if (W >= 32) v = add(v, dpp_move<kDppRowBcast15, 0xa>(0, __float_as_int(v)));
    if (W >= 64) v = add(v, dpp_move<kDppRowBcast31, 0xc>(0, __float_as_int(v)));
    return v;
}

// Minimum / maximum of an unsigned value over the wave, returned to every lane.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    int x = static_cast<int>(v);
    auto mn = [](int a, int b) { return static_cast<int>(min(static_cast<uint32_t>(a), static_cast<uint32_t>(b))); };
    x = mn(x, dpp_move<kDppRowShr1, 0xf>(x, x));
    x = mn(x, dpp_move<kDppRowShr2, 0xf>(x, x));
    x = mn(x, dpp_move<kDppRowShr4, 0xf>(x, x));
    x = mn(x, dpp_move<kDppRowShr8, 0xf>(x, x));
    x = mn(x, dpp_move<kDppRowBcast15, 0xa>(x, x));
    x = mn(x, dpp_move<kDppRowBcast31, 0xc>(x, x));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 63));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    int x = static_cast<int>(v);
    auto mx = [](int a, int b) { return static_cast<int>(max(static_cast<uint32_t>(a), static_cast<uint32_t>(b))); };
    x = mx(x, dpp_move<kDppRowShr1, 0xf>(x, x));
    x = mx(x, dpp_move<kDppRowShr2, 0xf>(x, x));
    x = mx(x, dpp_move<kDppRowShr4, 0xf>(x, x));
    x = mx(x, dpp_move<kDppRowShr8, 0xf>(x, x));
    x = mx(x, dpp_move<kDppRowBcast15, 0xa>(x, x));
    x = mx(x, dpp_move<kDppRowBcast31, 0xc>(x, x));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 63));
}
// Maximum / sum of a float over the wave, returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
    auto mx = [](float a, int b) { return fmaxf(a, __int_as_float(b)); };
    v = mx(v, dpp_move<kDppRowShr1, 0xf>(__float_as_int(v), __float_as_int(v)));
    v = mx(v, dpp_move<kDppRowShr2, 0xf>(__float_as_int(v), __float_as_int(v)));
    v = mx(v, dpp_move<kDppRowShr4, 0xf>(__float_as_int(v), __float_as_int(v)));
    v = mx(v, dpp_move<kDppRowShr8, 0xf>(__float_as_int(v), __float_as_int(v)));
    v = mx(v, dpp_move<kDppRowBcast15, 0xa>(__float_as_int(v), __float_as_int(v)));
    v = mx(v, dpp_move<kDppRowBcast31, 0xc>(__float_as_int(v), __float_as_int(v)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum_last<64>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data
// format, no swizzle): accesses through it are range-checked against the
// descriptor's byte count
constexpr int kBufferWord3 = 0x00020000;

// One int read with a vector (buffer) load, left in a VGPR until the caller
// takes it with readfirstlane at its use: the load joins the round trip of
// the vector loads issued with it, where a scalar load would be placed at
// its first use and waited for on its own.
__device__ __forceinline__ int load_int_vgpr(const int32_t* p) {
    return __builtin_amdgcn_raw_buffer_load_b32(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(p), 0,
                                          static_cast<int>(sizeof(int32_t)), kBufferWord3),
        0, 0, 0);
}

// One digit step of an MSB-first radix select, by one wave (every lane gets
// the answer): h is a 256-bin histogram of the alive keys' current digit;
// returns the digit that holds the krem-th largest alive key and how many
// alive keys lie in higher digits.  Lane L covers digits 255-4L .. 252-4L
// (descending); the counts are suffix sums.
__device__ __forceinline__ void find_digit256(const int* h, int krem, int lane, int& digit,
                                              int& above) {
    int c4[4], hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = h[255 - 4 * lane - i];
    c4[0] = hv[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) c4[i] = c4[i - 1] + hv[i];
    const int incl = wave_incl_scan(c4[3]);
    const int excl = incl - c4[3];
    int found_i = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ge = excl + c4[i];  // keys whose digit >= this one
        if (ge >= krem && ge - hv[i] < krem) found_i = i;
    }
    const uint64_t bal = __ballot(found_i >= 0);
    const int src = __ffsll(static_cast<unsigned long long>(bal)) - 1;  // exactly one lane
    const int my_digit = 255 - 4 * lane - (found_i < 0 ? 0 : found_i);
    const int my_above = excl + (found_i <= 0 ? 0 : c4[found_i - 1]);
    digit = __builtin_amdgcn_readlane(my_digit, src);
    above = __builtin_amdgcn_readlane(my_above, src);
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key);
// -0.0 is folded onto +0.0 first.  Inputs are not NaN.
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float a key came from (-0 comes back as +0).
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Kept-block count for NB blocks ("Rectified Sparse Attention ...", Key
// points: dynamic top-n with local blocks and a minimum count; the token
// budget of "SeerAttention-R", Abstract).  p is the skipped fraction in basis
// points; the local blocks count towards n.
__host__ __device__ __forceinline__ int block_count(int NB, int block, int budget_tokens,
                                                    int sparsity_bp, int n_local, int n_min) {
    int n_req;
    if (budget_tokens > 0)
        n_req = budget_tokens / block;
    else
        n_req = static_cast<int>((static_cast<int64_t>(10000 - sparsity_bp) * NB + 9999) / 10000);
    const int nl = n_local < NB ? n_local : NB;
    int n = n_req;
    if (n_min > n) n = n_min;
    if (nl > n) n = nl;
    if (n > NB) n = NB;
    return n;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace bsa
