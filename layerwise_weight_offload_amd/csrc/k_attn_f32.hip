// Softmax attention in fp32 for the fp32 workloads (the same operation as
// k_attn.hip: O = softmax(Q K^T / sqrt(d)) V per (batch, head), without a mask).
#include <math.h>

#include "../../include/lwo.h"
#include "kcommon.h"
#include "kernels.h"

namespace lwo {

// fp32: eight lanes per query, each holding an eighth of the head's columns
// of q and of the output; the score is the eight partial dot products summed
// by three lane exchanges (the same bits in all eight lanes), then every lane
// runs the same online softmax in base-2 units (log2 e folded into the query
// scale; v_exp_f32 is accurate to about one ulp).  8 queries per 64-lane
// workgroup, 32-key tiles in LDS shared by all of them.
template <int DH>
__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
    constexpr int QL = 8, DS = DH / QL;   // lanes per query, columns per lane
    static_assert(DH % QL == 0, "head dim");
    __shared__ __attribute__((aligned(16))) float Ks[32][DH];
    __shared__ __attribute__((aligned(16))) float Vs[32][DH];
    const int lane = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int qi = blockIdx.x * (64 / QL) + lane / QL, d0 = (lane % QL) * DS;
    const float* Q = (const float*)a.q;
    const float* K = (const float*)a.k;
    const float* V = (const float*)a.v;
    float q[DS], o[DS];
    const float scale = 1.4426950408889634f / sqrtf((float)DH);   // log2(e) / sqrt(d)
#pragma unroll
    for (int d = 0; d < DS; ++d) {
        q[d] = qi < a.Tq ? Q[(size_t)(b * a.Tq + qi) * a.ldq + h * DH + d0 + d] * scale : 0.0f;
        o[d] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    // A 32-key tile is 32 DH / 4 float4s per operand, NV4 per lane: all of them are
    // loaded before any is stored, so their latencies overlap.
    constexpr int C4 = DH / 4, NV4 = (32 * C4 + 63) / 64;
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int key0 = 0; key0 < a.Tk; key0 += 32) {
        float4 kv[NV4], vv[NV4];
#pragma unroll
        for (int u = 0; u < NV4; ++u) {
            const int i4 = lane + 64 * u, key = i4 / C4, c4 = i4 % C4;
            const bool ok = i4 < 32 * C4 && key0 + key < a.Tk;
            kv[u] = ok ? *(const float4*)(K + (size_t)(b * a.Tk + key0 + key) * a.ldk + h * DH + 4 * c4) : z4;
            vv[u] = ok ? *(const float4*)(V + (size_t)(b * a.Tk + key0 + key) * a.ldv + h * DH + 4 * c4) : z4;
        }
        __syncthreads();                             // the previous tile's reads are done
#pragma unroll
        for (int u = 0; u < NV4; ++u) {
            const int i4 = lane + 64 * u, key = i4 / C4, c4 = i4 % C4;
            if (i4 < 32 * C4) {
                *(float4*)&Ks[key][4 * c4] = kv[u];
                *(float4*)&Vs[key][4 * c4] = vv[u];
            }
        }
        __syncthreads();
        const int nk = min(32, a.Tk - key0);
        for (int j = 0; j < nk; ++j) {
            float s = 0.0f;
#pragma unroll
            for (int d = 0; d < DS; ++d) s += q[d] * Ks[j][d0 + d];
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            const float mn = fmaxf(m, s);
            const float c = __builtin_amdgcn_exp2f(m - mn), p = __builtin_amdgcn_exp2f(s - mn);
            l = l * c + p;
#pragma unroll
            for (int d = 0; d < DS; ++d) o[d] = o[d] * c + p * Vs[j][d0 + d];
            m = mn;
        }
    }
    if (qi >= a.Tq) return;
    float* O = (float*)a.o + (size_t)(b * a.Tq + qi) * a.ldo + h * DH + d0;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < DS; ++d) O[d] = o[d] * inv;
}

hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t st) {
    if (a.Tq <= 0 || a.B <= 0) return hipSuccess;
    if (a.Tk <= 0) return hipErrorInvalidValue;
    dim3 grid((a.Tq + 7) / 8, a.H, a.B);   // 8 queries per workgroup
    switch (a.dh) {
        case 64: LWO_KL((k_attn_f32<64>), grid, 64, 0, st, a); break;
        case 72: LWO_KL((k_attn_f32<72>), grid, 64, 0, st, a); break;
        case 128: LWO_KL((k_attn_f32<128>), grid, 64, 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lwo
