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
        return static_cast<const float*>(row)[i];
    }
    // Loads kVec consecutive values starting at i (16-byte aligned).
    __device__ static __forceinline__ void vec(const void* row, int64_t i, float* out) {
        float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(row) + i);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
};

template <>
struct Elem<kDtypeBF16> {
    using scalar_t = uint16_t;
    static constexpr int kVec = 8;  // 16-byte loads
    __device__ static __forceinline__ float at(const void* row, int64_t i) {
        return bf16_bits_f32(static_cast<const uint16_t*>(row)[i]);
    }
    __device__ static __forceinline__ void vec(const void* row, int64_t i, float* out) {
        uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + i);
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
};

// Sampler.prepare's per-request clamps, evaluated on the device.  A row is
// greedy when its temperature is not above MIN_T (NaN included); top_k < 1
// or >= V disables top-k; top_p is clamped to [MIN_P, 1] (NaN -> MIN_P).
__device__ __forceinline__ RowParams row_params(const float* temperature, const int32_t* top_k,
                                                const float* top_p, int b, int V) {
    RowParams r;
    if (temperature == nullptr) {
        r.greedy = true; r.T = kMinT; r.k = 1; r.p = 1.0f; r.top_p = false;
        return r;
    }
    const float t = temperature[b];
    r.greedy = !(t > kMinT);
    r.T = r.greedy ? kMinT : t;
    int k = top_k ? top_k[b] : 0;
    r.k = (k < 1 || k >= V) ? V : k;
    float p = top_p ? top_p[b] : 1.0f;
    p = fminf(fmaxf(p, kMinP), 1.0f);
    r.p = p;
    r.top_p = p < 1.0f;
    if (r.greedy) { r.k = 1; r.top_p = false; }
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
