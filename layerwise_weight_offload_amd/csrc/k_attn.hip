// Softmax attention without a mask (self- and cross-attention of the DiT
// block): O = softmax(Q K^T / sqrt(d)) V per (batch, head), streamed over key
// tiles with an online softmax so the T x T score matrix never exists.
//
// k_attn_bf16 (gfx950 MFMA): a 256-thread workgroup owns 128 queries of one
// (batch, head), 32 per wavefront.  Per 64-key tile:
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = the
//          wavefront's Q fragments kept in registers for the whole kernel;
//          the accumulator layout puts one query in each lane (column), so
//          the row max and row sum are in-lane reductions plus one swap
//          between the two 32-lane halves;
//   O^T += V^T P^T: B = the probabilities straight from the S^T registers
//          (rounded to bf16), A = V^T read from an LDS tile stored
//          transposed; the key order inside each MFMA k-step follows the
//          accumulator layout, identically on both operands.
// Head dims 64, 72 and 128: the QK^T contraction is padded with zeros to a
// multiple of 16 and the PV output to a multiple of 32 columns (72 -> 80 and
// 96); padded columns are never stored.  Key and query tails are masked.
//
// k_attn_f32: one query per lane with fp32 FMA, for the fp32 workloads.
#include <math.h>

#include "../../include/lwo.h"
#include "kcommon.h"
#include "kernels.h"

namespace lwo {

template <int DH>
__global__ __launch_bounds__(256) void k_attn_bf16(AttnArgs a) {
    constexpr int DK = (DH + 15) / 16 * 16;
    constexpr int DN = (DH + 31) / 32 * 32;
    constexpr int KS = DK / 16, NT = DN / 32;
    constexpr int BN = 64;
    constexpr int KST = DK + 8;     // K tile row stride (elements): 16-byte pad
    constexpr int VST = BN + 8;     // V^T tile row stride (elements)
    __shared__ __attribute__((aligned(16))) bf16 Ks[BN * KST];
    __shared__ __attribute__((aligned(16))) bf16 Vt[DN * VST];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int l32 = lane % 32, half = lane / 32;
    const int h = blockIdx.y, b = blockIdx.z;
    const int Tq = a.Tq, Tk = a.Tk;
    const int qi = blockIdx.x * 128 + wave * 32 + l32;
    const bf16* Q = (const bf16*)a.q;
    const bf16* K = (const bf16*)a.k;
    const bf16* V = (const bf16*)a.v;
    const intx4 z = {0, 0, 0, 0};

    intx4 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int d0 = s * 16 + half * 8;
        qf[s] = (qi < Tq && d0 < DH) ? *(const intx4*)(Q + (size_t)(b * Tq + qi) * a.ldq + h * DH + d0) : z;
    }
    floatx16 oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] = 0.0f;
    float m_i = -INFINITY, l_i = 0.0f;
    const float sl2 = 1.4426950408889634f / sqrtf((float)DH);   // log2(e) / sqrt(d)

    for (int key0 = 0; key0 < Tk; key0 += BN) {
        __syncthreads();
        for (int c = tid; c < BN * (DK / 8); c += 256) {
            const int key = c / (DK / 8), d0 = (c % (DK / 8)) * 8;
            const intx4 v = (key0 + key < Tk && d0 < DH)
                                ? *(const intx4*)(K + (size_t)(b * Tk + key0 + key) * a.ldk + h * DH + d0) : z;
            *(intx4*)&Ks[key * KST + d0] = v;
        }
        for (int c = tid; c < BN * (DN / 8); c += 256) {
            const int key = c % BN, d0 = (c / BN) * 8;
            const intx4 v = (key0 + key < Tk && d0 < DH)
                                ? *(const intx4*)(V + (size_t)(b * Tk + key0 + key) * a.ldv + h * DH + d0) : z;
            const bf16x8 vv = __builtin_bit_cast(bf16x8, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) Vt[(d0 + e) * VST + key] = vv[e];
        }
        __syncthreads();

        floatx16 s[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const intx4*)&Ks[(t * 32 + l32) * KST + st * 16 + half * 8]);
                s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, __builtin_bit_cast(bf16x8, qf[st]), s[t], 0, 0, 0);
            }
        }
        // s[t][r]: key key0 + 32t + 8(r/4) + 4*half + r%4, query qi
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + t * 32 + 8 * (r / 4) + 4 * half + (r % 4);
                const float v = key < Tk ? s[t][r] * sl2 : -INFINITY;
                s[t][r] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_i, mx);
        const float corr = exp2f(m_i - m_new);
        float rs = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2f(s[t][r] - m_new);
                s[t][r] = p;
                rs += p;
            }
        rs += __shfl_xor(rs, 32);
        l_i = l_i * corr + rs;
        m_i = m_new;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[nt][r] *= corr;

#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 pf;
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[e] = (bf16)s[t][ks * 8 + e];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const bf16* vr = &Vt[(nt * 32 + l32) * VST + t * 32 + ks * 16 + half * 4];
                    const bf16x4 lo = *(const bf16x4*)vr, hi = *(const bf16x4*)(vr + 8);
                    const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    oacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[nt], 0, 0, 0);
                }
            }
    }

    if (qi >= Tq) return;
    const float inv = 1.0f / l_i;
    bf16* O = (bf16*)a.o + (size_t)(b * Tq + qi) * a.ldo + h * DH;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = nt * 32 + 8 * g + 4 * half;
            if (d0 < DH) {
                bf16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (bf16)(oacc[nt][4 * g + e] * inv);
                *(bf16x4*)(O + d0) = o;
            }
        }
}

template <int DH>
__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
    __shared__ float Ks[32][DH];
    __shared__ float Vs[32][DH];
    const int lane = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int qi = blockIdx.x * 64 + lane;
    const float* Q = (const float*)a.q;
    const float* K = (const float*)a.k;
    const float* V = (const float*)a.v;
    float q[DH], o[DH];
    const float scale = 1.0f / sqrtf((float)DH);
#pragma unroll
    for (int d = 0; d < DH; ++d) {
        q[d] = qi < a.Tq ? Q[(size_t)(b * a.Tq + qi) * a.ldq + h * DH + d] * scale : 0.0f;
        o[d] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    for (int key0 = 0; key0 < a.Tk; key0 += 32) {
        __syncthreads();
        for (int i = lane; i < 32 * DH; i += 64) {
            const int key = i / DH, d = i % DH;
            const bool ok = key0 + key < a.Tk;
            Ks[key][d] = ok ? K[(size_t)(b * a.Tk + key0 + key) * a.ldk + h * DH + d] : 0.0f;
            Vs[key][d] = ok ? V[(size_t)(b * a.Tk + key0 + key) * a.ldv + h * DH + d] : 0.0f;
        }
        __syncthreads();
        const int nk = min(32, a.Tk - key0);
        for (int j = 0; j < nk; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int d = 0; d < DH; ++d) s += q[d] * Ks[j][d];
            const float mn = fmaxf(m, s);
            const float c = expf(m - mn), p = expf(s - mn);
            l = l * c + p;
#pragma unroll
            for (int d = 0; d < DH; ++d) o[d] = o[d] * c + p * Vs[j][d];
            m = mn;
        }
    }
    if (qi >= a.Tq) return;
    float* O = (float*)a.o + (size_t)(b * a.Tq + qi) * a.ldo + h * DH;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < DH; ++d) O[d] = o[d] * inv;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
    if (a.Tq <= 0 || a.B <= 0) return hipSuccess;
    if (a.Tk <= 0) return hipErrorInvalidValue;
    if (a.dtype == LWO_BF16) {
        dim3 grid((a.Tq + 127) / 128, a.H, a.B);
        switch (a.dh) {
            case 64: k_attn_bf16<64><<<grid, 256, 0, st>>>(a); break;
            case 72: k_attn_bf16<72><<<grid, 256, 0, st>>>(a); break;
            case 128: k_attn_bf16<128><<<grid, 256, 0, st>>>(a); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        dim3 grid((a.Tq + 63) / 64, a.H, a.B);
        switch (a.dh) {
            case 64: k_attn_f32<64><<<grid, 64, 0, st>>>(a); break;
            case 72: k_attn_f32<72><<<grid, 64, 0, st>>>(a); break;
            case 128: k_attn_f32<128><<<grid, 64, 0, st>>>(a); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace lwo
