// Dense MFMA throughput probe: the ceiling the block kernels are measured
// against besides the published peak.  Every wavefront runs `iters` rounds
// of four independent accumulator chains of v_mfma_f32_32x32x16_bf16 (bf16)
// or v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3, unit scales) on register
// operands, so the matrix cores never wait for memory or for one another;
// each lane stores one sum so that nothing is optimised away.
#include "kcommon.h"
#include "kernels.h"

namespace lwo {

template <bool FP8>
__global__ __launch_bounds__(256) void k_mfma_peak(int iters, float* sink) {
    const int tid = blockIdx.x * 256 + threadIdx.x;
    // operands from the lane id: finite, small, not foldable
    const int base = 0x3c003c00 ^ (threadIdx.x & 7);   // bf16 pairs near 1.0; e4m3 bytes are finite
    intx4 a4 = {base, base + 1, base + 2, base + 3};
    intx4 b4 = {base + 4, base + 5, base + 6, base + 7};
    floatx16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (FP8) {
                const intx8 a8 = {a4[0], a4[1], a4[2], a4[3], a4[0], a4[1], a4[2], a4[3]};
                const intx8 b8 = {b4[0], b4[1], b4[2], b4[3], b4[0], b4[1], b4[2], b4[3]};
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[c], 0, 0, 0, 127, 0, 127);
            } else {
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                                 __builtin_bit_cast(bf16x8, b4), acc[c], 0, 0, 0);
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[tid] = s;
}

hipError_t launch_mfma_peak(bool fp8, int blocks, int iters, float* sink, hipStream_t st) {
    if (fp8) LWO_KL((k_mfma_peak<true>), blocks, 256, 0, st, iters, sink);
    else LWO_KL((k_mfma_peak<false>), blocks, 256, 0, st, iters, sink);
    return hipGetLastError();
}

}  // namespace lwo
