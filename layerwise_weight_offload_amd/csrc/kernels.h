// Host-side launchers of the gfx950 kernels (all enqueue on `st` and return
// the launch status; shapes are checked by the callers in block.hip).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lwo {

// Events the next kernel launch records at its own start and end (the
// dispatch's timestamps, so no gap between launches is counted).  The kernel
// timer sets them around exactly one launch; null otherwise (plain launch).
struct LaunchEvents { hipEvent_t start = nullptr, stop = nullptr; };
LaunchEvents& launch_events();   // per host thread

// kern<<<grid, block, shmem, st>>>(args...), with the launch events above.
#define LWO_KL(kern, grid, block, shmem, st, ...)                                                  \
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(block), (shmem), (st), ::lwo::launch_events().start, \
                          ::lwo::launch_events().stop, 0u, __VA_ARGS__)

// Epilogue of a linear layer Y = A W^T: v = acc (* w_scale[n / seg] * a_scale[m]) + bias[n], then
//   EPI_STORE  out[m, n] = v                       (act dtype)
//   EPI_GELU   out[m, n] = GELU_tanh(v)            (act dtype)
//   EPI_GATED  xr[m, n] += gate[(m / rows_per_batch) * gate_ld + n] * v   (fp32 residual)
//   EPI_RESID  xr[m, n] += v                                              (fp32 residual)
enum EpiKind { EPI_STORE = 0, EPI_GELU = 1, EPI_GATED = 2, EPI_RESID = 3 };

struct GemmArgs {
    const void* a;          // [M, K], lda = K: row-major, or k-tiled when a_tiled (bf16/fp8)
    const void* w;          // [N, K] (a Linear weight [out, in]): row-major for fp32, 64x64-byte tiles for bf16/fp8
    int M, N, K;
    int dtype;              // lwo_dtype of A and W: F32, BF16, or FP8_E4M3 (A codes + per-row a_scale)
    int act_dtype;          // dtype of bias and of `out`
    int epi;                // EpiKind
    const void* bias;       // [N] act dtype or null
    void* out; int ldo;     // EPI_STORE / EPI_GELU target
    float* xr; int ldx;     // EPI_GATED / EPI_RESID residual
    const float* gate; int gate_ld; int rows_per_batch;
    const float* w_scale; int w_seg;   // fp8: per-segment weight scale (segment = w_seg output columns)
    const float* a_scale;              // fp8: per-row activation scale
    int a_tiled;            // A in k-tiled rows (ktiled_off, R = K bytes)
    int out_tiled;          // EPI_STORE / EPI_GELU: out in k-tiled rows (R = ldo bf16)
};

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);

struct AttnArgs {
    const void* q; int ldq;     // row (b*Tq + t) holds head h at column h*dh
    const void* k; int ldk;     // row (b*Tk + t)
    const void* v; int ldv;
    void* o; int ldo;           // row (b*Tq + t); k-tiled rows (R = ldo bf16) when o_tiled
    int o_tiled;
    int B, H, Tq, Tk, dh;
    int dtype;                  // F32 or BF16 (q, k, v, o)
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t st);   // dtype F32 (launch_attention calls it)

hipError_t launch_to_f32(const void* x, int dt, float* xr, size_t n, hipStream_t st);
hipError_t launch_from_f32(const float* xr, void* x, int dt, size_t n, hipStream_t st);
// SiLU of the conditioning vector [n], to fp32 (once per step, DiT kind).
hipError_t launch_silu(const void* in, int dt, float* out, int n, hipStream_t st);
// mod [B, 6D] = silu_cond [B, D] x w^T + b (the DiT adaLN linear; w [6D, D] and b in dtype dt).
hipError_t launch_mod_dit(const float* silu_cond, const void* w, const void* b, int dt, float* mod, int B, int D,
                          hipStream_t st);
hipError_t launch_mod_video(const void* cond, const void* table, int dt, float* mod, int B, int D, hipStream_t st);
// LayerNorm of the fp32 rows xr [M, D]; with mod, y = LN(x)(1 + mod[b, scale_chunk]) + mod[b, shift_chunk]
// where b = row / T.  out_dt F32/BF16 writes `out`; FP8_E4M3 writes codes to `out` and row scales to out_scale.
// out_tiled (BF16, FP8): `out` in k-tiled rows (ktiled_off, R = D elements).
hipError_t launch_ln(const float* xr, int M, int D, int T, const float* mod, int shift_chunk, int scale_chunk,
                     void* out, int out_dt, float* out_scale, int out_tiled, hipStream_t st);
// In-place RMSNorm of columns [0, D) (gain gq) and [D, 2D) (gain gk) of qkv rows (row stride 3D).
hipError_t launch_rmsnorm_qk(void* qkv, int dt, int M, int D, const void* gq, const void* gk, hipStream_t st);
// bf16 rows [M, N] -> e4m3 codes and per-row scales (dynamic amax / 448); codes_tiled: codes in k-tiled rows.
hipError_t launch_quant_rows(const void* in, int M, int N, uint8_t* codes, float* scales, int codes_tiled,
                             hipStream_t st);
hipError_t launch_checksum(const void* dev, uint64_t bytes, uint64_t* acc, hipStream_t st);
hipError_t launch_checksum_compare(uint64_t* acc, uint64_t expect, hipStream_t st);
hipError_t launch_zero_u64(uint64_t* p, int n, hipStream_t st);
// MFMA throughput probe: `blocks` x 256 threads, 4 * iters MFMAs per wavefront, one float per thread to sink.
hipError_t launch_mfma_peak(bool fp8, int blocks, int iters, float* sink, hipStream_t st);

}  // namespace lwo
