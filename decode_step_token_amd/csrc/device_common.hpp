// Device helpers shared by the sampler kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dst {

constexpr int kWave = 64;
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;

// Prepare's clamps ("The engine and the sampler", section "The sampler"):
// MIN_T = MIN_P = 1e-6 as float32.
constexpr float kMinT = 1e-6f;
constexpr float kMinP = 1e-6f;

// ------------------------------------------------------------ loads --

// Load through the global address space (global_load_*, not flat_load_*):
// flat loads also count against the LDS wait counter, which serialises the
// streaming loop against its LDS traffic.
template <typename T>
__device__ __forceinline__ T ld_global(const void* p) {
    return *reinterpret_cast<const __attribute__((address_space(1))) T*>(
        reinterpret_cast<uintptr_t>(p));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load (the HIP vector classes cannot be built from a global reference).
__device__ __forceinline__ uint4 ld_global_u4(const void* p) {
    const u32x4_t v = ld_global<u32x4_t>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte streaming load: the line is not kept in the caches for reuse, so a
// row read once does not push other lines (instructions, tables) out of L2.
__device__ __forceinline__ uint4 ld_global_u4_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(
        reinterpret_cast<const __attribute__((address_space(1))) u32x4_t*>(reinterpret_cast<uintptr_t>(p)));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- values --

// Order-preserving 32-bit key of a float: larger float -> larger key; -0.0
// is folded onto +0.0 so that the two compare equal, as floats do.
__device__ __forceinline__ uint32_t f32_key(float x) {
    uint32_t b = __float_as_uint(x);
    b = (b == 0x80000000u) ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_f32(uint32_t k) {
    uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(b);
}

__device__ __forceinline__ float bf16_bits_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

template <int DT>
struct Elem;

template <>
struct Elem<kDtypeF32> {
    using scalar_t = float;
    static constexpr int kVec = 4;  // 16-byte loads
    __device__ static __forceinline__ float at(const void* row, int64_t i) {
        return ld_global<float>(static_cast<const float*>(row) + i);
    }
    // Loads kVec consecutive values starting at i (16-byte aligned).
    __device__ static __forceinline__ void vec(const void* row, int64_t i, float* out) {
        const uint4 v = ld_global_u4(static_cast<const float*>(row) + i);
        out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
        out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
    }
};

template <>
struct Elem<kDtypeBF16> {
    using scalar_t = uint16_t;
    static constexpr int kVec = 8;  // 16-byte loads
    __device__ static __forceinline__ float at(const void* row, int64_t i) {
        return bf16_bits_f32(ld_global<uint16_t>(static_cast<const uint16_t*>(row) + i));
    }
    __device__ static __forceinline__ void vec(const void* row, int64_t i, float* out) {
        const uint4 v = ld_global_u4(static_cast<const uint16_t*>(row) + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[2 * j] = __uint_as_float(w[j] << 16);
            out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
};

// ------------------------------------------------------------ parameters --

struct RowParams {
    bool greedy;
    float T;      // effective temperature
    int k;        // effective top-k (V when disabled)
    float p;      // effective top-p (1 when disabled)
    bool top_p;   // p < 1
    float min_p;  // effective min_p (0 when disabled)
};

// Sampler.prepare's per-request clamps, evaluated on the device.  A row is
// greedy when its temperature is not above MIN_T (NaN included); top_k < 1
// or >= V disables top-k; top_p is clamped to [MIN_P, 1] (NaN -> MIN_P);
// min_p (the pages' exercise) is off unless above 0 (NaN: off), at most 1.
__device__ __forceinline__ RowParams row_params(const float* temperature, const int32_t* top_k,
                                                const float* top_p, const float* min_p, int b,
                                                int V) {
    RowParams r;
    if (temperature == nullptr) {
        r.greedy = true; r.T = kMinT; r.k = 1; r.p = 1.0f; r.top_p = false; r.min_p = 0.0f;
        return r;
    }
    const float t = ld_global<float>(temperature + b);
    r.greedy = !(t > kMinT);
    r.T = r.greedy ? kMinT : t;
    int k = top_k ? ld_global<int32_t>(top_k + b) : 0;
    r.k = (k < 1 || k >= V) ? V : k;
    float p = top_p ? ld_global<float>(top_p + b) : 1.0f;
    p = fminf(fmaxf(p, kMinP), 1.0f);
    r.p = p;
    r.top_p = p < 1.0f;
    const float mp = min_p ? ld_global<float>(min_p + b) : 0.0f;
    r.min_p = mp > 0.0f ? fminf(mp, 1.0f) : 0.0f;
    if (r.greedy) { r.k = 1; r.top_p = false; r.min_p = 0.0f; }
    return r;
}

// ---------------------------------------------------------------- Philox --
// Philox-4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw, SC'11): each round
// multiplies counter words 0 and 2 by the two Philox constants, swaps the
// 64-bit halves into place and xors in the round key, which is then bumped by
// the Weyl increments.

struct Philox4x64 {
    uint64_t x0, x1, x2, x3;
};

__device__ __forceinline__ Philox4x64 philox4x64_10(Philox4x64 c, uint64_t k0, uint64_t k1) {
    constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull;
    constexpr uint64_t M1 = 0xCA5A826395121157ull;
    constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull;
    constexpr uint64_t W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t lo0 = M0 * c.x0, hi0 = __umul64hi(M0, c.x0);
        const uint64_t lo1 = M1 * c.x2, hi1 = __umul64hi(M1, c.x2);
        Philox4x64 n;
        n.x0 = hi1 ^ c.x1 ^ k0;
        n.x1 = lo1;
        n.x2 = hi0 ^ c.x3 ^ k1;
        n.x3 = lo0;
        c = n;
        k0 += W0;
        k1 += W1;
    }
    return c;
}

// The request's stream: key (seed, 0), counter (uid, step, 0, 0); word 0.
__device__ __forceinline__ uint64_t request_word(uint64_t seed, int64_t uid, uint64_t step) {
    Philox4x64 c{static_cast<uint64_t>(uid), step, 0ull, 0ull};
    return philox4x64_10(c, seed, 0ull).x0;
}

// 24-bit dyadic uniform in [0, 1), exact in float and double.
__device__ __forceinline__ double uniform24(uint64_t word) {
    return static_cast<double>(word >> 40) * (1.0 / 16777216.0);
}

// ------------------------------------------------------------ barriers --
// A workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load of the wave (its release fence covers all
// address spaces), which drains a prefetch that is still in flight; this one
// waits for the wave's LDS operations alone (s_waitcnt lgkmcnt(0): vmcnt and
// expcnt fields at their maximum) and keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

// ------------------------------------------------- DPP wave64 reductions --
// Cross-lane data movement through DPP (no LDS round trip): quad swaps, row
// half-mirror and mirror combine within a 16-lane row, then row_bcast15 /
// row_bcast31 fold the four rows so that lane 63 holds the result, which is
// read back into a scalar register.

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v),
                                                             CTRL, ROW_MASK, 0xf, false));
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float old, float v) {
    return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(old), __float_as_uint(v)));
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double old, double v) {
    const uint64_t o = static_cast<uint64_t>(__double_as_longlong(old));
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK>(static_cast<uint32_t>(o), static_cast<uint32_t>(b));
    const uint32_t hi = dpp_u32<CTRL, ROW_MASK>(static_cast<uint32_t>(o >> 32), static_cast<uint32_t>(b >> 32));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

constexpr int kDppXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;

// Maximum over the 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v, v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v, v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v, v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v, v));
    v = fmaxf(v, dpp_f32<kDppBcast15, 0xa>(-INFINITY, v));
    v = fmaxf(v, dpp_f32<kDppBcast31, 0xc>(-INFINITY, v));
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(v)), 63)));
}

// Sum over the 64 lanes, returned wave-uniform.
__device__ __forceinline__ double wave_sum_dpp(double v) {
    v += dpp_f64<kDppXor1>(v, v);
    v += dpp_f64<kDppXor2>(v, v);
    v += dpp_f64<kDppHalfMirror>(v, v);
    v += dpp_f64<kDppMirror>(v, v);
    v += dpp_f64<kDppBcast15, 0xa>(0.0, v);
    v += dpp_f64<kDppBcast31, 0xc>(0.0, v);
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b)), 63));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b >> 32)), 63));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Inclusive prefix sum over the 64 lanes (lane order) through DPP: shifts of
// 1, 2, 4, 8 within each 16-lane row, then the row_bcast15 / row_bcast31
// carries across rows.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32_zero(uint32_t v) {
    // lanes without a source read 0 (bound_ctrl)
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xf, true));
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64_zero(double v) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = dpp_u32_zero<CTRL, ROW_MASK>(static_cast<uint32_t>(b));
    const uint32_t hi = dpp_u32_zero<CTRL, ROW_MASK>(static_cast<uint32_t>(b >> 32));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

constexpr int kDppShr1 = 0x111;
constexpr int kDppShr2 = 0x112;
constexpr int kDppShr4 = 0x114;
constexpr int kDppShr8 = 0x118;

__device__ __forceinline__ uint32_t wave_scan_u32_dpp(uint32_t v) {
    v += dpp_u32_zero<kDppShr1>(v);
    v += dpp_u32_zero<kDppShr2>(v);
    v += dpp_u32_zero<kDppShr4>(v);
    v += dpp_u32_zero<kDppShr8>(v);
    v += dpp_u32_zero<kDppBcast15, 0xa>(v);
    v += dpp_u32_zero<kDppBcast31, 0xc>(v);
    return v;
}

__device__ __forceinline__ double wave_scan_f64_dpp(double v) {
    v += dpp_f64_zero<kDppShr1>(v);
    v += dpp_f64_zero<kDppShr2>(v);
    v += dpp_f64_zero<kDppShr4>(v);
    v += dpp_f64_zero<kDppShr8>(v);
    v += dpp_f64_zero<kDppBcast15, 0xa>(v);
    v += dpp_f64_zero<kDppBcast31, 0xc>(v);
    return v;
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = readlane_u32(static_cast<uint32_t>(b), lane);
    const uint32_t hi = readlane_u32(static_cast<uint32_t>(b >> 32), lane);
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v, v));
    v = max(v, dpp_u32<kDppXor2>(v, v));
    v = max(v, dpp_u32<kDppHalfMirror>(v, v));
    v = max(v, dpp_u32<kDppMirror>(v, v));
    v = max(v, dpp_u32<kDppBcast15, 0xa>(0u, v));
    v = max(v, dpp_u32<kDppBcast31, 0xc>(0u, v));
    return readlane_u32(v, 63);
}

// Maximum of a 64-bit value over the 64 lanes (wave-uniform result).
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
    auto step = [](uint64_t x, uint32_t olo, uint32_t ohi) {
        const uint64_t o = (static_cast<uint64_t>(ohi) << 32) | olo;
        return o > x ? o : x;
    };
    uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    v = step(v, dpp_u32<kDppXor1>(lo, lo), dpp_u32<kDppXor1>(hi, hi));
    lo = static_cast<uint32_t>(v); hi = static_cast<uint32_t>(v >> 32);
    v = step(v, dpp_u32<kDppXor2>(lo, lo), dpp_u32<kDppXor2>(hi, hi));
    lo = static_cast<uint32_t>(v); hi = static_cast<uint32_t>(v >> 32);
    v = step(v, dpp_u32<kDppHalfMirror>(lo, lo), dpp_u32<kDppHalfMirror>(hi, hi));
    lo = static_cast<uint32_t>(v); hi = static_cast<uint32_t>(v >> 32);
    v = step(v, dpp_u32<kDppMirror>(lo, lo), dpp_u32<kDppMirror>(hi, hi));
    lo = static_cast<uint32_t>(v); hi = static_cast<uint32_t>(v >> 32);
    v = step(v, dpp_u32<kDppBcast15, 0xa>(0u, lo), dpp_u32<kDppBcast15, 0xa>(0u, hi));
    lo = static_cast<uint32_t>(v); hi = static_cast<uint32_t>(v >> 32);
    v = step(v, dpp_u32<kDppBcast31, 0xc>(0u, lo), dpp_u32<kDppBcast31, 0xc>(0u, hi));
    lo = readlane_u32(static_cast<uint32_t>(v), 63);
    hi = readlane_u32(static_cast<uint32_t>(v >> 32), 63);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Rank of this lane among the set bits of `mask` below it.
__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// ------------------------------------------------------ wave64 reductions --

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        T w = __shfl_xor(v, o, kWave);
        v = v > w ? v : w;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        T w = __shfl_xor(v, o, kWave);
        v = v < w ? v : w;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Inclusive prefix sum across the wave (lane order).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        T w = __shfl_up(v, o, kWave);
        if (lane >= o) v += w;
    }
    return v;
}

// Block-wide helpers.  `scratch` must hold BLOCK/64 + 1 elements of T and is
// reused across calls: each call starts and ends with __syncthreads().
template <int BLOCK, typename T>
__device__ __forceinline__ T block_max(T v, T* scratch) {
    constexpr int NW = BLOCK / kWave;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) scratch[wid] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) r = r > scratch[i] ? r : scratch[i];
    __syncthreads();
    return r;
}

template <int BLOCK, typename T>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
    constexpr int NW = BLOCK / kWave;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) scratch[wid] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) r += scratch[i];
    __syncthreads();
    return r;
}

// Exclusive prefix over the block in thread order; *total receives the sum.
template <int BLOCK, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* scratch, T* total) {
    constexpr int NW = BLOCK / kWave;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const T incl = wave_incl_scan(v);
    T excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = T(0);
    __syncthreads();
    if (lane == kWave - 1) scratch[wid] = incl;
    __syncthreads();
    T before = T(0), all = T(0);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        before += (i < wid) ? scratch[i] : T(0);
        all += scratch[i];
    }
    __syncthreads();
    *total = all;
    return before + excl;
}

}  // namespace dst
