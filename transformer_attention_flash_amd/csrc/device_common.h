// device_common.h -- small CDNA4 device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// log2(e): scores are pre-multiplied by scale*log2(e) so every exponential is
// a single v_exp_f32 (2^x).
constexpr float kLog2e = 1.4426950408889634f;

// Finite stand-in for -infinity as the initial running max, so that
// exp2(m_old - m_new) is 1 (not NaN) while a row has seen only masked keys.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Vector of N floats for N in {1, 2, 4}: the per-lane slice of a row.
template <int N> struct VecN;
template <> struct VecN<1> { typedef float type; };
template <> struct VecN<2> { typedef f32x2 type; };
template <> struct VecN<4> { typedef f32x4 type; };

template <int N>
__device__ __forceinline__ float vget(const typename VecN<N>::type &x, int i) {
    if constexpr (N == 1) {
        return x;
    } else {
        return x[i];
    }
}

template <int N>
__device__ __forceinline__ void vset(typename VecN<N>::type &x, int i, float val) {
    if constexpr (N == 1) {
        x = val;
    } else {
        x[i] = val;
    }
}

// Cross-lane combines without an LDS round trip.  v_permlane32_swap returns,
// in every lane l, the values of lanes l and l ^ 32 (one in each result), so
// combining its two results needs no lane mask; a swizzle swaps the 16-lane
// halves of each 32-lane group.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16(float x) {
    return __uint_as_float(__builtin_amdgcn_ds_swizzle(__float_as_uint(x), 0x401F));  // lane l ^ 16
}
// Over the four lanes i, i + 16, i + 32, i + 48.
__device__ __forceinline__ float max4(float x) { return max_xor32(fmaxf(x, xor16(x))); }
__device__ __forceinline__ float sum4(float x) { return sum_xor32(x + xor16(x)); }

}  // namespace attn
