// Row-wise and elementwise kernels of the DiT block (HBM-bound): residual
// conversion, adaLN modulation, LayerNorm (+ modulation, + fp8 row
// quantisation), q/k RMSNorm, fp8 row quantisation and the slot checksum.
//
// The row kernels keep their row in registers, so LayerNorm takes its mean
// and variance in two exact passes and the quantiser its amax and codes
// without re-reading HBM: one 64-lane wavefront per row (q/k RMSNorm, fp8
// quantisation, LayerNorm up to 2048 wide) or two per row, each with half of
// it (wider LayerNorm); four wavefronts share a 256-thread workgroup.
#include "../../include/lwo.h"
#include "kcommon.h"
#include "kernels.h"

namespace lwo {

__device__ __forceinline__ float4 load4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 load4(const bf16* p) {
    bf16x4 v = *(const bf16x4*)p;
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}
__device__ __forceinline__ void store4(float* p, float4 v) { *(float4*)p = v; }
__device__ __forceinline__ void store4(bf16* p, float4 v) {
    bf16x4 o;
    o[0] = (bf16)v.x; o[1] = (bf16)v.y; o[2] = (bf16)v.z; o[3] = (bf16)v.w;
    *(bf16x4*)p = o;
}

// ------------------------------------------------------------------ residual conversion

template <typename T>
__global__ void k_to_f32(const T* __restrict__ x, float* __restrict__ xr, size_t n4) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i < n4; i += (size_t)gridDim.x * blockDim.x) store4(xr + 4 * i, load4(x + 4 * i));
}

template <typename T>
__global__ void k_from_f32(const float* __restrict__ xr, T* __restrict__ x, size_t n4) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i < n4; i += (size_t)gridDim.x * blockDim.x) store4(x + 4 * i, load4(xr + 4 * i));
}

static int grid_for(size_t n, int per_block) {
    size_t g = (n + per_block - 1) / per_block;
    return (int)(g < 8192 ? (g ? g : 1) : 8192);
}

hipError_t launch_to_f32(const void* x, int dt, float* xr, size_t n, hipStream_t st) {
    size_t n4 = n / 4;
    if (dt == LWO_F32) LWO_KL((k_to_f32<float>), grid_for(n4, 256), 256, 0, st, (const float*)x, xr, n4);
    else LWO_KL((k_to_f32<bf16>), grid_for(n4, 256), 256, 0, st, (const bf16*)x, xr, n4);
    return hipGetLastError();
}

hipError_t launch_from_f32(const float* xr, void* x, int dt, size_t n, hipStream_t st) {
    size_t n4 = n / 4;
    if (dt == LWO_F32) LWO_KL((k_from_f32<float>), grid_for(n4, 256), 256, 0, st, xr, (float*)x, n4);
    else LWO_KL((k_from_f32<bf16>), grid_for(n4, 256), 256, 0, st, xr, (bf16*)x, n4);
    return hipGetLastError();
}

// ------------------------------------------------------------------ adaLN modulation

// DiT kind: mod[b, n] = sum_k SiLU(cond[b, k]) W[n, k] + bias[n], n < 6D.
// SiLU(cond) [B, D] in fp32, once per step: every block's adaLN GEMV reads it.
template <typename T>
__global__ void k_silu(const T* __restrict__ in, float* __restrict__ out, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) out[i] = silu(to_f(in[i]));
}

// A GEMV over the [6D, D] weight, bound by reading it once: 16 lanes own one
// row, a workgroup of NT threads owns NT / 16 rows (512: the DiT-XL matrix in
// one round of workgroups, one per CU).  K goes in windows of CL 16-byte loads
// per lane, CL sized to the row (the DiT-XL row is 9 loads).  Each thread first
// loads its share of the window's SiLU(cond) (computed once per step, up to
// four batches), then issues the weight loads, then stages the SiLU values
// into LDS: both sets of loads are in flight together, so the window costs one
// memory round trip, and the products of a load start as soon as it lands.
// For that every load is unconditional (a lane past the row end re-reads the
// row's last 16 bytes, a SiLU value past the window end goes to a spare LDS
// slot), so the compiler's wait counts are exact instead of draining all loads
// at the first use; the scheduling barrier and the weight pointer without
// __restrict__ keep the weight loads ahead of the workgroup barrier (loads
// through a restrict pointer are free to sink to their use).  The bias is read
// with the rest, once.  ONE: a single window and at most four batches, so the
// kernel is straight-line code (a loop would make its head wait for every
// load still in flight, the bias's included).
template <typename T, int NT, int CL, bool ONE>
__global__ __launch_bounds__(NT) void k_mod_dit(const float* __restrict__ sc_in, const T* w,
                                                 const T* __restrict__ bias, float* __restrict__ mod, int B, int D) {
    constexpr int EV = 16 / sizeof(T);                  // elements per 16-byte load (8 bf16, 4 f32)
    constexpr int WIN = CL * 16 * EV;                   // window elements
    constexpr int SPT = (4 * WIN + NT - 1) / NT;        // SiLU values per thread and window (four batches)
    __shared__ __attribute__((aligned(16))) float scf[4 * WIN + kWave];
    float (*sc)[WIN] = (float (*)[WIN])scf;
    const int n = blockIdx.x * (NT / 16) + threadIdx.x / 16, l16 = threadIdx.x % 16;
    const int nr = min(n, 6 * D - 1);
    const T* wr = w + (size_t)nr * D;
    const T bq = bias[nr];
    const int nbb = ONE ? 1 : (B + 3) / 4, nwin = ONE ? 1 : (D + WIN - 1) / WIN;
    for (int bb = 0; bb < nbb; ++bb) {
        const int b0 = bb * 4, nb = min(4, B - b0);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int wi = 0; wi < nwin; ++wi) {
            const int k0 = wi * WIN, wn = min(WIN, D - k0);
            float sv[SPT];
#pragma unroll
            for (int t = 0; t < SPT; ++t) {
                const int q = t * NT + threadIdx.x, j = q / WIN, kk = q % WIN;
                sv[t] = sc_in[j < nb && kk < wn ? (size_t)(b0 + j) * D + k0 + kk : 0];
            }
            intx4 raw[CL];
#pragma unroll
            for (int i = 0; i < CL; ++i) raw[i] = *(const intx4*)(wr + min(k0 + (i * 16 + l16) * EV, D - EV));
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();                            // the previous window's reads are done
#pragma unroll
            for (int t = 0; t < SPT; ++t) {
                const int q = t * NT + threadIdx.x, j = q / WIN, kk = q % WIN;
                scf[j < nb && kk < wn ? j * WIN + kk : 4 * WIN + threadIdx.x % kWave] = sv[t];
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < CL; ++i) {
                const int kk = (i * 16 + l16) * EV;
                if (k0 + kk >= D) break;
                float wv[EV];
                if constexpr (EV == 8) {
                    const bf16x8 v = __builtin_bit_cast(bf16x8, raw[i]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) wv[e] = (float)v[e];
                } else {
                    const float4 v = __builtin_bit_cast(float4, raw[i]);
                    wv[0] = v.x; wv[1] = v.y; wv[2] = v.z; wv[3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (j >= nb) break;
#pragma unroll
                    for (int e = 0; e < EV; ++e) acc[j] = fmaf(wv[e], sc[j][kk + e], acc[j]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float v = row16_reduce(acc[j], [](float a, float b) { return a + b; });
            if (l16 == 0 && n < 6 * D && j < nb) mod[(size_t)(b0 + j) * 6 * D + n] = v + to_f(bq);
        }
    }
}

// Video kind: mod[b, i, d] = cond[b, i, d] + table[i, d].
template <typename T>
__global__ void k_mod_video(const T* __restrict__ cond, const T* __restrict__ table, float* __restrict__ mod,
                            int B, int D) {
    const int n = 6 * D;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < B * n; i += gridDim.x * blockDim.x)
        mod[i] = to_f(cond[i]) + to_f(table[i % n]);
}

hipError_t launch_silu(const void* in, int dt, float* out, int n, hipStream_t st) {
    const int g = grid_for((size_t)n, 256);
    if (dt == LWO_F32) LWO_KL((k_silu<float>), g, 256, 0, st, (const float*)in, out, n);
    else LWO_KL((k_silu<bf16>), g, 256, 0, st, (const bf16*)in, out, n);
    return hipGetLastError();
}

template <typename T>
static hipError_t mod_dit_dispatch(const float* silu_cond, const T* w, const T* b, float* mod, int B, int D,
                                   hipStream_t st) {
    constexpr int EV = 16 / sizeof(T);
    const int nch = (D + 16 * EV - 1) / (16 * EV);      // 16-byte loads per lane for one row
    const dim3 grid((6 * D + 31) / 32);
#define LWO_MOD_CASE(C)                                                                                     \
    if (B <= 4 && nch <= C) {                                                                               \
        LWO_KL((k_mod_dit<T, 512, C, true>), grid, 512, 0, st, silu_cond, w, b, mod, B, D);                  \
        return hipGetLastError();                                                                           \
    }
    LWO_MOD_CASE(2) LWO_MOD_CASE(4) LWO_MOD_CASE(5) LWO_MOD_CASE(9) LWO_MOD_CASE(16)
#undef LWO_MOD_CASE
    LWO_KL((k_mod_dit<T, 512, 16, false>), grid, 512, 0, st, silu_cond, w, b, mod, B, D);
    return hipGetLastError();
}

hipError_t launch_mod_dit(const float* silu_cond, const void* w, const void* b, int dt, float* mod, int B, int D,
                          hipStream_t st) {
    if (D < 8 || D % 8) return hipErrorInvalidValue;
    if (dt == LWO_F32) return mod_dit_dispatch(silu_cond, (const float*)w, (const float*)b, mod, B, D, st);
    return mod_dit_dispatch(silu_cond, (const bf16*)w, (const bf16*)b, mod, B, D, st);
}

hipError_t launch_mod_video(const void* cond, const void* table, int dt, float* mod, int B, int D, hipStream_t st) {
    int g = grid_for((size_t)B * 6 * D, 256);
    if (dt == LWO_F32) LWO_KL((k_mod_video<float>), g, 256, 0, st, (const float*)cond, (const float*)table, mod, B, D);
    else LWO_KL((k_mod_video<bf16>), g, 256, 0, st, (const bf16*)cond, (const bf16*)table, mod, B, D);
    return hipGetLastError();
}

// ------------------------------------------------------------------ LayerNorm (+ modulation, + fp8)

// OUT: 0 float, 1 bf16, 2 fp8 codes + row scale.  WPR wavefronts share a row.
// WPR 2 (wide rows): each wavefront holds half of the row in registers (the
// first half has the odd float4 chunk, NV4 chunks per lane, >= ceil(D / 8) / 64),
// which keeps the register count, and so the wavefronts per SIMD, where the
// HBM stream needs them; their partial sums meet in LDS and are added in a fixed
// order (first half + second half).  WPR 1 (rows up to 2048 wide): one
// wavefront holds the whole row, so the statistics need no LDS exchange and no
// barrier, and the modulation's scale and shift are loaded with the row
// instead of after the statistics.  The choice depends on D only, so every
// output type and layout of one width sees the same floats.
// k-tiled output (`tiled`): the workgroup's RPW rows (consecutive rows inside one
// 64-row tile) are staged in LDS (RPW x D x out bytes of dynamic LDS) and
// written as runs of RPW x 64 bytes, 16 bytes per lane.
template <int OUT, bool MOD, int NV4, int WPR>
__global__ __launch_bounds__(256) void k_ln(const float* __restrict__ xr, int M, int D, int T,
                                            const float* __restrict__ mod, int shc, int scc,
                                            void* __restrict__ out, float* __restrict__ out_scale, int tiled) {
    constexpr int RPW = 4 / WPR;                        // rows per workgroup
    constexpr bool PF = MOD && WPR == 1;                // scale and shift loaded with the row
    __shared__ float red[3][RPW][WPR];                  // [quantity][row of the workgroup][half]
    extern __shared__ __attribute__((aligned(16))) unsigned char ln_rows[];   // k-tiled output staging
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int rw = wave / WPR, hf = wave % WPR;         // row within the workgroup, half of the row
    const int row = blockIdx.x * RPW + rw;
    const bool live = row < M;
    const int n4 = D / 4, nh0 = WPR == 2 ? (n4 + 1) / 2 : n4;
    const int nh = hf ? n4 - nh0 : nh0, c0 = hf ? nh0 : 0;   // float4 chunks of this half, first chunk
    const float* x = xr + (size_t)(live ? row : 0) * D;
    const int bi = (live ? row : 0) / T;
    const float* shift = MOD ? mod + ((size_t)bi * 6 + shc) * D : nullptr;
    const float* scale = MOD ? mod + ((size_t)bi * 6 + scc) * D : nullptr;
    float4 v[NV4], scv[PF ? NV4 : 1], shv[PF ? NV4 : 1];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
        const int c = lane + kWave * i;
        v[i] = live && c < nh ? load4(x + 4 * (c0 + c)) : make_float4(0.f, 0.f, 0.f, 0.f);
        if constexpr (PF) {
            if (c < nh) { scv[i] = load4(scale + 4 * (c0 + c)); shv[i] = load4(shift + 4 * (c0 + c)); }
        }
    }
#pragma unroll
    for (int i = 0; i < NV4; ++i) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    s = wave_sum(s);
    if constexpr (WPR == 2) {
        if (lane == 0) red[0][rw][hf] = s;
        __syncthreads();
        s = red[0][rw][0] + red[0][rw][1];
    }
    const float mean = s / (float)D;
    float s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
        const int c = lane + kWave * i;
        if (c < nh) {
            float a = v[i].x - mean, b = v[i].y - mean, cc = v[i].z - mean, d = v[i].w - mean;
            s2 += (a * a + b * b) + (cc * cc + d * d);
        }
    }
    s2 = wave_sum(s2);
    if constexpr (WPR == 2) {
        if (lane == 0) red[1][rw][hf] = s2;
        __syncthreads();
        s2 = red[1][rw][0] + red[1][rw][1];
    }
    const float rstd = 1.0f / sqrtf(s2 / (float)D + 1e-6f);
    constexpr int OB = OUT == 0 ? 4 : OUT == 1 ? 2 : 1; // output bytes per element
    unsigned char* stage = ln_rows + (size_t)rw * D * OB;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
        const int c = lane + kWave * i, cc4 = c0 + c;
        float4 y = make_float4((v[i].x - mean) * rstd, (v[i].y - mean) * rstd, (v[i].z - mean) * rstd,
                               (v[i].w - mean) * rstd);
        if (MOD && c < nh) {
            float4 sc, sh;
            if constexpr (PF) { sc = scv[i]; sh = shv[i]; }
            else { sc = load4(scale + 4 * cc4); sh = load4(shift + 4 * cc4); }
            y.x = y.x * (1.0f + sc.x) + sh.x;
            y.y = y.y * (1.0f + sc.y) + sh.y;
            y.z = y.z * (1.0f + sc.z) + sh.z;
            y.w = y.w * (1.0f + sc.w) + sh.w;
        }
        if (OUT == 2) {
            if (c < nh) amax = fmaxf(amax, fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w))));
            v[i] = y;
        } else if (live && c < nh) {
            if (OUT == 0) store4((float*)out + (size_t)row * D + 4 * cc4, y);
            else if (tiled) store4((bf16*)stage + 4 * cc4, y);
            else store4((bf16*)out + (size_t)row * D + 4 * cc4, y);
        }
    }
    if (OUT == 2) {
        amax = wave_max(amax);
        if constexpr (WPR == 2) {
            if (lane == 0) red[2][rw][hf] = amax;
            __syncthreads();
            amax = fmaxf(red[2][rw][0], red[2][rw][1]);
        }
        const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
        uint8_t* o = (uint8_t*)out + (size_t)row * D;
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
            const int c = lane + kWave * i;
            if (live && c < nh) {
                uint32_t lo = pack2_e4m3(v[i].x * inv, v[i].y * inv), hi = pack2_e4m3(v[i].z * inv, v[i].w * inv);
                uint8_t* dst = tiled ? stage + 4 * (c0 + c) : o + 4 * (c0 + c);
                *(uint32_t*)dst = lo | (hi << 16);
            }
        }
        if (live && lane == 0 && hf == 0) out_scale[row] = amax > 0.0f ? amax / 448.0f : 1.0f;
    }
    if (OUT != 0 && tiled) {
        __syncthreads();
        const int R = D * OB, nq = (R / 64) * 4 * RPW;  // 16-byte pieces of the staged rows
        const int r0 = blockIdx.x * RPW;
        unsigned char* g = (unsigned char*)out + ktiled_off(r0, 0, (size_t)R);   // row r0 + k follows at +64 k
        for (int q = threadIdx.x; q < nq; q += blockDim.x) {
            const int j = q / (4 * RPW), p = q % (4 * RPW), rr = p >> 2;
            if (r0 + rr >= M) continue;
            *(uint4*)(g + (size_t)j * 4096 + 16 * p) = *(const uint4*)(ln_rows + (size_t)rr * R + 64 * j + 16 * (p & 3));
        }
    }
}

template <int OUT, bool MOD>
static hipError_t ln_dispatch(const float* xr, int M, int D, int T, const float* mod, int shc, int scc, void* out,
                              float* out_scale, int tiled, hipStream_t st) {
    const bool one = D <= 2048;                         // one wavefront per row
    const int rpw = one ? 4 : 2;
    const int need = one ? (D / 4 + kWave - 1) / kWave : ((D / 4 + 1) / 2 + kWave - 1) / kWave;
    dim3 grid((M + rpw - 1) / rpw);
    const size_t shm = tiled ? (size_t)rpw * D * (OUT == 1 ? 2 : 1) : 0;   // staged rows
#define LWO_LN_CASE(NV)                                                                                     \
    if (need <= NV) {                                                                                       \
        if constexpr (NV <= 8) {                        /* one wavefront per row: need <= 8 */              \
            if (one) {                                                                                      \
                LWO_KL((k_ln<OUT, MOD, NV, 1>), grid, 256, shm, st, xr, M, D, T, mod, shc, scc, out, out_scale, tiled); \
                return hipGetLastError();                                                                   \
            }                                                                                               \
        }                                                                                                   \
        LWO_KL((k_ln<OUT, MOD, NV, 2>), grid, 256, shm, st, xr, M, D, T, mod, shc, scc, out, out_scale, tiled);     \
        return hipGetLastError();                                                                           \
    }
    LWO_LN_CASE(1) LWO_LN_CASE(2) LWO_LN_CASE(3) LWO_LN_CASE(4) LWO_LN_CASE(5) LWO_LN_CASE(6) LWO_LN_CASE(8)
    LWO_LN_CASE(10) LWO_LN_CASE(12) LWO_LN_CASE(16)
#undef LWO_LN_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_ln(const float* xr, int M, int D, int T, const float* mod, int shift_chunk, int scale_chunk,
                     void* out, int out_dt, float* out_scale, int out_tiled, hipStream_t st) {
    if (M <= 0) return hipSuccess;   // no rows: nothing to launch (a zero grid is an invalid launch)
    const bool m = mod != nullptr;
    const int tl = out_dt == LWO_F32 ? 0 : out_tiled;
    if (out_dt == LWO_F32) return m ? ln_dispatch<0, true>(xr, M, D, T, mod, shift_chunk, scale_chunk, out, out_scale, 0, st)
                                    : ln_dispatch<0, false>(xr, M, D, T, mod, 0, 0, out, out_scale, 0, st);
    if (out_dt == LWO_BF16) return m ? ln_dispatch<1, true>(xr, M, D, T, mod, shift_chunk, scale_chunk, out, out_scale, tl, st)
                                     : ln_dispatch<1, false>(xr, M, D, T, mod, 0, 0, out, out_scale, tl, st);
    return m ? ln_dispatch<2, true>(xr, M, D, T, mod, shift_chunk, scale_chunk, out, out_scale, tl, st)
             : ln_dispatch<2, false>(xr, M, D, T, mod, 0, 0, out, out_scale, tl, st);
}

// ------------------------------------------------------------------ q/k RMSNorm

template <typename T, int NV4>
__global__ __launch_bounds__(256) void k_rmsnorm_qk(T* __restrict__ qkv, int M, int D, const T* __restrict__ gq,
                                                    const T* __restrict__ gk) {
    const int w = blockIdx.x * 4 + threadIdx.x / kWave;   // (row, part)
    const int lane = threadIdx.x % kWave;
    if (w >= 2 * M) return;
    const int row = w >> 1, part = w & 1;
    T* x = qkv + (size_t)row * 3 * D + (size_t)part * D;
    const T* g = part ? gk : gq;
    const int n4 = D / 4;
    float4 v[NV4];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
        const int c = lane + kWave * i;
        v[i] = c < n4 ? load4(x + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
        s += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
    }
    const float r = 1.0f / sqrtf(wave_sum(s) / (float)D + 1e-6f);
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
        const int c = lane + kWave * i;
        if (c < n4) {
            const float4 gv = load4(g + 4 * c);
            store4(x + 4 * c, make_float4(v[i].x * r * gv.x, v[i].y * r * gv.y, v[i].z * r * gv.z, v[i].w * r * gv.w));
        }
    }
}

// bf16 rows with 16-byte accesses, kept as raw bf16 in registers (half the
// registers of a float copy): the same arithmetic, in the same order, as above.
template <int NV8>
__global__ __launch_bounds__(256) void k_rmsnorm_qk_b8(bf16* __restrict__ qkv, int M, int D, const bf16* __restrict__ gq,
                                                       const bf16* __restrict__ gk) {
    const int w = blockIdx.x * 4 + threadIdx.x / kWave;   // (row, part)
    const int lane = threadIdx.x % kWave;
    if (w >= 2 * M) return;
    const int row = w >> 1, part = w & 1;
    bf16* x = qkv + (size_t)row * 3 * D + (size_t)part * D;
    const bf16* g = part ? gk : gq;
    const int n8 = D / 8;
    bf16x8 v[NV8];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NV8; ++i) {
        const int c = lane + kWave * i;
        if (c < n8) {
            v[i] = *(const bf16x8*)(x + 8 * c);
#pragma unroll
            for (int e = 0; e < 8; e += 4) {
                const float a = (float)v[i][e], b = (float)v[i][e + 1], cc = (float)v[i][e + 2], d = (float)v[i][e + 3];
                s += (a * a + b * b) + (cc * cc + d * d);
            }
        }
    }
    const float r = 1.0f / sqrtf(wave_sum(s) / (float)D + 1e-6f);
#pragma unroll
    for (int i = 0; i < NV8; ++i) {
        const int c = lane + kWave * i;
        if (c < n8) {
            const bf16x8 gv = *(const bf16x8*)(g + 8 * c);
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)v[i][e] * r * (float)gv[e]);
            *(bf16x8*)(x + 8 * c) = o;
        }
    }
}

template <typename T>
static hipError_t rms_dispatch(T* qkv, int M, int D, const T* gq, const T* gk, hipStream_t st) {
    const int need = (D / 4 + kWave - 1) / kWave;
    dim3 grid((2 * M + 3) / 4);
#define LWO_RMS_CASE(NV)                                                          \
    if (need <= NV) {                                                             \
        LWO_KL((k_rmsnorm_qk<T, NV>), grid, 256, 0, st, qkv, M, D, gq, gk);             \
        return hipGetLastError();                                                 \
    }
    LWO_RMS_CASE(1) LWO_RMS_CASE(2) LWO_RMS_CASE(4) LWO_RMS_CASE(8) LWO_RMS_CASE(12) LWO_RMS_CASE(16)
    LWO_RMS_CASE(20) LWO_RMS_CASE(24) LWO_RMS_CASE(32)
#undef LWO_RMS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_rmsnorm_qk(void* qkv, int dt, int M, int D, const void* gq, const void* gk, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    if (dt == LWO_F32) return rms_dispatch<float>((float*)qkv, M, D, (const float*)gq, (const float*)gk, st);
    if (D % 8 == 0) {
        const int need = (D / 8 + kWave - 1) / kWave;
        dim3 grid((2 * M + 3) / 4);
#define LWO_RMS8_CASE(NV)                                                                                    \
    if (need <= NV) {                                                                                        \
        LWO_KL((k_rmsnorm_qk_b8<NV>), grid, 256, 0, st, (bf16*)qkv, M, D, (const bf16*)gq, (const bf16*)gk);  \
        return hipGetLastError();                                                                            \
    }
        LWO_RMS8_CASE(1) LWO_RMS8_CASE(2) LWO_RMS8_CASE(4) LWO_RMS8_CASE(6) LWO_RMS8_CASE(8) LWO_RMS8_CASE(10)
        LWO_RMS8_CASE(12) LWO_RMS8_CASE(16)
#undef LWO_RMS8_CASE
    }
    return rms_dispatch<bf16>((bf16*)qkv, M, D, (const bf16*)gq, (const bf16*)gk, st);
}

// ------------------------------------------------------------------ fp8 row quantisation

// One wavefront per row: amax over the row, then codes = e4m3(x * (448 / amax)), scale = amax / 448.
__global__ __launch_bounds__(256) void k_quant_rows(const bf16* __restrict__ in, int M, int N,
                                                    uint8_t* __restrict__ codes, float* __restrict__ scales, int tiled) {
    const int row = blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (row >= M) return;
    const bf16* x = in + (size_t)row * N;
    float amax = 0.0f;
    for (int c = lane; c < N / 8; c += kWave) {
        bf16x8 v = *(const bf16x8*)(x + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[e]));
    }
    amax = wave_max(amax);
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
    uint8_t* o = codes + (size_t)row * N;
    for (int c = lane; c < N / 8; c += kWave) {
        bf16x8 v = *(const bf16x8*)(x + 8 * c);
        uint32_t w0 = pack2_e4m3((float)v[0] * inv, (float)v[1] * inv) | (pack2_e4m3((float)v[2] * inv, (float)v[3] * inv) << 16);
        uint32_t w1 = pack2_e4m3((float)v[4] * inv, (float)v[5] * inv) | (pack2_e4m3((float)v[6] * inv, (float)v[7] * inv) << 16);
        *(uint2*)(tiled ? codes + ktiled_off(row, (size_t)8 * c, (size_t)N) : o + 8 * c) = make_uint2(w0, w1);
    }
    if (lane == 0) scales[row] = amax > 0.0f ? amax / 448.0f : 1.0f;
}

// The same with the row held in registers between the two passes (one HBM read).
template <int NV8>
__global__ __launch_bounds__(256) void k_quant_rows_reg(const bf16* __restrict__ in, int M, int N,
                                                        uint8_t* __restrict__ codes, float* __restrict__ scales,
                                                        int tiled) {
    const int row = blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (row >= M) return;
    const bf16* x = in + (size_t)row * N;
    const int n8 = N / 8;
    bf16x8 v[NV8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV8; ++i) {
        const int c = lane + kWave * i;
        if (c < n8) {
            v[i] = *(const bf16x8*)(x + 8 * c);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[i][e]));
        }
    }
    amax = wave_max(amax);
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
    uint8_t* o = codes + (size_t)row * N;
#pragma unroll
    for (int i = 0; i < NV8; ++i) {
        const int c = lane + kWave * i;
        if (c < n8) {
            const bf16x8 u = v[i];
            uint32_t w0 = pack2_e4m3((float)u[0] * inv, (float)u[1] * inv) | (pack2_e4m3((float)u[2] * inv, (float)u[3] * inv) << 16);
            uint32_t w1 = pack2_e4m3((float)u[4] * inv, (float)u[5] * inv) | (pack2_e4m3((float)u[6] * inv, (float)u[7] * inv) << 16);
            *(uint2*)(tiled ? codes + ktiled_off(row, (size_t)8 * c, (size_t)N) : o + 8 * c) = make_uint2(w0, w1);
        }
    }
    if (lane == 0) scales[row] = amax > 0.0f ? amax / 448.0f : 1.0f;
}

hipError_t launch_quant_rows(const void* in, int M, int N, uint8_t* codes, float* scales, int codes_tiled,
                             hipStream_t st) {
    if (M <= 0) return hipSuccess;
    const int need = (N / 8 + kWave - 1) / kWave;
#define LWO_Q_CASE(NV)                                                                                         \
    if (need <= NV) {                                                                                          \
        LWO_KL((k_quant_rows_reg<NV>), (M + 3) / 4, 256, 0, st, (const bf16*)in, M, N, codes, scales,          \
               codes_tiled);                                                                                   \
        return hipGetLastError();                                                                              \
    }
    LWO_Q_CASE(1) LWO_Q_CASE(2) LWO_Q_CASE(4) LWO_Q_CASE(8) LWO_Q_CASE(10) LWO_Q_CASE(16) LWO_Q_CASE(28)
#undef LWO_Q_CASE
    LWO_KL((k_quant_rows), (M + 3) / 4, 256, 0, st, (const bf16*)in, M, N, codes, scales, codes_tiled);
    return hipGetLastError();
}

// ------------------------------------------------------------------ slot checksum

__device__ __forceinline__ uint64_t splitmix64_next(uint64_t s) {
    uint64_t z = s + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// acc[0] += sum_i SplitMix64(w_i ^ (i * golden)) over n words (integer sum: any order gives the same bits).
__global__ __launch_bounds__(256) void k_checksum(const uint64_t* __restrict__ w, uint64_t n,
                                                  unsigned long long* __restrict__ acc) {
    uint64_t s = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
        s += splitmix64_next(w[i] ^ (i * 0x9E3779B97F4A7C15ull));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor((unsigned long long)s, o);
    if ((threadIdx.x % kWave) == 0) atomicAdd(acc, (unsigned long long)s);
}

__global__ void k_checksum_compare(unsigned long long* acc, unsigned long long expect) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && acc[0] != expect) atomicAdd(acc + 1, 1ull);
}

__global__ void k_zero_u64(unsigned long long* p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

hipError_t launch_checksum(const void* dev, uint64_t bytes, uint64_t* acc, hipStream_t st) {
    const uint64_t n = bytes / 8;
    int g = (int)((n + 256 * 16 - 1) / (256 * 16));
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    LWO_KL((k_checksum), g, 256, 0, st, (const uint64_t*)dev, n, (unsigned long long*)acc);
    return hipGetLastError();
}

hipError_t launch_checksum_compare(uint64_t* acc, uint64_t expect, hipStream_t st) {
    LWO_KL((k_checksum_compare), 1, 64, 0, st, (unsigned long long*)acc, (unsigned long long)expect);
    return hipGetLastError();
}

hipError_t launch_zero_u64(uint64_t* p, int n, hipStream_t st) {
    LWO_KL((k_zero_u64), (n + 63) / 64, 64, 0, st, (unsigned long long*)p, n);
    return hipGetLastError();
}

}  // namespace lwo
