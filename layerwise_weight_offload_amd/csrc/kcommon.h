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

// k-tiled activation rows (the operand form of the tiled weights): a matrix of
// M rows of R bytes (R a multiple of 64) stored as 64-row x 64-byte tiles, the
// tiles of one 64-row band in column order, so that one 64-byte stage of a
// 64-row band is 4 KB of consecutive memory.  Byte c of row m sits at the
// offset below; the buffer spans whole bands (rows rounded up to 64).
__host__ __device__ __forceinline__ size_t ktiled_off(int m, size_t c, size_t R) {
    return (size_t)(m >> 6) * R * 64 + (c >> 6) * 4096 + (size_t)(m & 63) * 64 + (c & 63);
}

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }   // v_cvt_pk_bf16_f32: nearest-even

// Cross-lane reductions with DPP moves (VALU, no LDS round trip).  dpp<C, R>
// returns, in the lanes of the 16-lane rows enabled by R, the value of the
// lane that DPP control C selects, and `old` in the other rows.
template <int C, int R = 0xF>
__device__ __forceinline__ float dpp(float v, float old) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), C, R, 0xF, false));
}

// op over each 16-lane row, left in every lane of the row: quad_perm [1,0,3,2]
// and [2,3,0,1] combine the lanes of a quad, row_half_mirror the two quads of
// an 8-lane half, row_mirror the two halves.
template <typename Op>
__device__ __forceinline__ float row16_reduce(float v, Op op) {
    v = op(v, dpp<0xB1>(v, 0.0f));
    v = op(v, dpp<0x4E>(v, 0.0f));
    v = op(v, dpp<0x141>(v, 0.0f));
    return op(v, dpp<0x140>(v, 0.0f));
}

// op over the wavefront, returned as a wave-uniform value: row_bcast15 folds
// row 0 into row 1 and row 2 into row 3, row_bcast31 rows 0-1 into rows 2-3,
// and lane 63 then holds the result (`id`: op's identity, for the rows a
// broadcast leaves unchanged).
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op, float id) {
    v = row16_reduce(v, op);
    v = op(v, dpp<0x142, 0xA>(v, id));
    v = op(v, dpp<0x143, 0xC>(v, id));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce(v, [](float a, float b) { return a + b; }, 0.0f);
}

__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); }, -INFINITY);
}

// tanh(t) = 1 - 2 / (exp(2t) + 1), with exp(2t) = 2^(2t log2 e) on v_exp_f32.
// Inline (no call, so kernels holding large accumulator sets do not spill);
// absolute error a few 1e-7, saturating to +-1 for |t| > 44 without NaN.  The
// reciprocal is the hardware one (v_rcp_f32, about 1 ulp): a correctly rounded
// division costs about ten instructions per element in the GELU epilogue.
__device__ __forceinline__ float tanh_fast(float t) {
    const float e = __builtin_amdgcn_exp2f(fminf(t * 2.8853900817779268f, 126.0f));   // 2 log2(e)
    return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
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
