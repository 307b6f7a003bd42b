// Device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx2 __attribute__((ext_vector_type(2)));

namespace lwo {

constexpr int kWave = 64;

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }   // v_cvt_pk_bf16_f32: nearest-even

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// tanh(t) = 1 - 2 / (exp(2t) + 1), with exp(2t) = 2^(2t log2 e) on v_exp_f32.
// Inline (no call, so kernels holding large accumulator sets do not spill);
// absolute error about 1e-7, saturating to +-1 for |t| > 44 without NaN.
__device__ __forceinline__ float tanh_fast(float t) {
    const float e = __builtin_amdgcn_exp2f(fminf(t * 2.8853900817779268f, 126.0f));   // 2 log2(e)
    return 1.0f - 2.0f / (e + 1.0f);
}

__device__ __forceinline__ float gelu_tanh(float u) {
    // 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))
    const float k0 = 0.7978845608028654f;
    return 0.5f * u * (1.0f + tanh_fast(k0 * (u + 0.044715f * u * u * u)));
}

__device__ __forceinline__ float silu(float u) { return u / (1.0f + expf(-u)); }

// Two floats -> two OCP e4m3 codes (round to nearest even) in the low 16 bits.
// Inputs are clamped to +-448 first, so the hardware's out-of-range rule never applies.
__device__ __forceinline__ uint32_t pack2_e4m3(float a, float b) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

}  // namespace lwo
