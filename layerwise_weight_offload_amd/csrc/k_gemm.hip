// Linear layers of the DiT block, Y = A W^T with a fused epilogue (bias,
// GELU-tanh, gated or plain residual add into the fp32 residual stream).
//
// k_gemm_deep takes bf16 (v_mfma_f32_32x32x16_bf16, or v_mfma_f32_16x16x32_bf16
// for the 256x256 tiles) or OCP fp8 e4m3 (v_mfma_scale_f32_32x32x64_f8f6f4 with
// unit block scales) operands and accumulates in fp32.  Both operands are K-contiguous: [M,K]
// activations, row-major or k-tiled, and [N,K] weights tiled in 64-row x
// 64-byte tiles (the block layout's tiled weights), so a stage of weight rows
// (and of k-tiled activation rows, which the block's own producers write) is
// one run of consecutive memory, loaded with 128-byte requests where a
// row-major stage takes 64-byte ones; each lane's MFMA fragment is one or two
// 16-byte LDS reads from a row.  No split-K: every output is produced by one lane in a
// fixed order, so results are deterministic run to run.  Tiles of 256x256,
// 256x128, 128x128 or 128x64 by problem size; direct-to-LDS loads three
// stages ahead; LDS-staged vector epilogue (details at the kernel).
// * k_gemm_f32: fp32 FMA tiles (64x64, 4x4 per thread) for the fp32
//   workloads, where bf16 rounding would exceed a 1e-4 tolerance.
#include <type_traits>

#include "../../include/lwo.h"
#include "kcommon.h"
#include "kernels.h"

namespace lwo {

template <int EPI, typename ActT>
__device__ __forceinline__ void epilogue(const GemmArgs& g, int m, int n, float v) {
    if (g.bias) v += to_f(((const ActT*)g.bias)[n]);
    if (EPI == EPI_STORE) {
        ((ActT*)g.out)[(size_t)m * g.ldo + n] = from_f<ActT>(v);
    } else if (EPI == EPI_GELU) {
        ((ActT*)g.out)[(size_t)m * g.ldo + n] = from_f<ActT>(gelu_tanh(v));
    } else if (EPI == EPI_GATED) {
        float* x = g.xr + (size_t)m * g.ldx + n;
        *x += g.gate[(size_t)(m / g.rows_per_batch) * g.gate_ld + n] * v;
    } else {
        float* x = g.xr + (size_t)m * g.ldx + n;
        *x += v;
    }
}

// ------------------------------------------------------------------ fp32 FMA tiles

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs g) {
    __shared__ float As[16][64 + 4];
    __shared__ float Ws[16][64 + 4];
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const float* A = (const float*)g.a;
    const float* W = (const float*)g.w;
    const int lr = tid / 4, lk = (tid % 4) * 4;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < g.K; k0 += 16) {
        const float4 av = (m0 + lr < g.M) ? *(const float4*)(A + (size_t)(m0 + lr) * g.K + k0 + lk) : z;
        const float4 wv = (n0 + lr < g.N) ? *(const float4*)(W + (size_t)(n0 + lr) * g.K + k0 + lk) : z;
        __syncthreads();
        As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
        Ws[lk + 0][lr] = wv.x; Ws[lk + 1][lr] = wv.y; Ws[lk + 2][lr] = wv.z; Ws[lk + 3][lr] = wv.w;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; b[i] = Ws[kk][tx * 4 + i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m < g.M && n < g.N) epilogue<EPI, float>(g, m, n, acc[i][j]);
        }
}

// A T x T tile (T = 32 or 64) with K split four ways inside a 1024-thread
// workgroup, for grids too small to fill the chip with k_gemm_f32: group kg
// (256 threads, (T / 16) x (T / 16) outputs each) sums k in [kg Kq, (kg + 1) Kq)
// in k order, and group 0 adds the other groups' partial tiles in group order
// (through LDS) before the epilogue, so the results do not depend on timing.
template <int EPI, int T>
__global__ __launch_bounds__(1024) void k_gemm_f32_splitk(GemmArgs g) {
    constexpr int KG = 4, R = T / 16, LPR = 256 / T, LW = 16 / LPR;   // outputs per thread side; loaders per row; floats each
    static_assert(T == 32 || T == 64, "tile");
    __shared__ float As[KG][16][T + 4];
    __shared__ float Ws[KG][16][T + 4];
    __shared__ float red[KG - 1][T][T + 1];
    const int kg = threadIdx.x / 256, tid = threadIdx.x % 256, tx = tid % 16, ty = tid / 16;
    const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
    const float* A = (const float*)g.a;
    const float* W = (const float*)g.w;
    const int lr = tid / LPR, lk = (tid % LPR) * LW;
    const int Kq = (g.K / 16 + KG - 1) / KG * 16;   // every group runs Kq / 16 steps; columns past K read zeros
    const int kb = kg * Kq;
    float acc[R][R];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[i][j] = 0.0f;
    for (int k0 = kb; k0 < kb + Kq; k0 += 16) {
        const bool kin = k0 < g.K;
        float av[LW], wv[LW];
#pragma unroll
        for (int e = 0; e < LW; ++e) {
            av[e] = (kin && m0 + lr < g.M) ? A[(size_t)(m0 + lr) * g.K + k0 + lk + e] : 0.0f;
            wv[e] = (kin && n0 + lr < g.N) ? W[(size_t)(n0 + lr) * g.K + k0 + lk + e] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < LW; ++e) { As[kg][lk + e][lr] = av[e]; Ws[kg][lk + e][lr] = wv[e]; }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            float a[R], b[R];
#pragma unroll
            for (int i = 0; i < R; ++i) { a[i] = As[kg][kk][ty * R + i]; b[i] = Ws[kg][kk][tx * R + i]; }
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int j = 0; j < R; ++j) acc[i][j] += a[i] * b[j];
        }
    }
    if (kg > 0) {
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int j = 0; j < R; ++j) red[kg - 1][ty * R + i][tx * R + j] = acc[i][j];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) {
            float v = acc[i][j];
#pragma unroll
            for (int r = 0; r < KG - 1; ++r) v += red[r][ty * R + i][tx * R + j];
            const int m = m0 + ty * R + i, n = n0 + tx * R + j;
            if (m < g.M && n < g.N) epilogue<EPI, float>(g, m, n, v);
        }
}

// ------------------------------------------------------------------ MFMA tiles (bf16 / fp8)

// Tile index -> (tile row, tile col).  Workgroups are handed to the 8 XCDs
// round-robin, so consecutive ids land on different L2s; the remap gives each
// XCD a contiguous run of tiles, and inside that run tiles go in groups of
// kGroupM tile rows (column-major within a group) so that the A rows and the
// W columns a group touches stay in that XCD's L2.
constexpr int kXcds = 8, kGroupM = 8;

__device__ __forceinline__ void tile_of(int pid, int nt_m, int nt_n, int& tm, int& tn) {
    const int total = nt_m * nt_n;
    const int x = pid % kXcds, idx = pid / kXcds;
    const int base = total / kXcds, rem = total % kXcds;
    const int t = x * base + min(x, rem) + idx;      // bijection of [0, total)
    const int per_group = kGroupM * nt_n;
    const int g = t / per_group, first_m = g * kGroupM;
    const int gsz = min(nt_m - first_m, kGroupM);
    const int r = t % per_group;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

// ------------------------------------------------------------------ deep prefetch, direct-to-LDS

// BM x BN outputs per 256-thread workgroup (BM, BN in {64, 128, 256}, BM >=
// 128): 2x2 wavefronts, each owning (BM/2) x (BN/2) = TM x TN MFMA 32x32
// blocks.  K advances in 64-byte stages (32 bf16 or 64 fp8 elements) held in
// four LDS buffers; each stage is fetched with global_load_lds three stages
// ahead of its use, so about three stages of MFMA work cover the load
// latency.  The wait before a stage is `s_waitcnt vmcnt(2 L)` (this
// wavefront's L loads per stage for the two later stages may still be in
// flight) followed by a plain s_barrier: the workgroup barrier of the
// language would also drain those later loads.  LDS rows are 64 bytes (four
// 16-byte chunks); chunk c of row r sits at c ^ f(r).  Which f keeps a
// fragment read on distinct banks depends on the lanes' row/chunk pattern
// (measured on gfx950 with the LDS bank-conflict counter and with a timing
// probe of ds_read_b128 at eight wavefronts per CU):
//  * 32x32 blocks (lane l: row l % 32, chunk l / 32): f(r) = (r >> 2) & 3 is
//    conflict-free, (r >> 1) & 3 and r & 3 are not;
//  * 16x16x32 blocks (lane l: row l % 16, chunk l / 16): (r >> 1) & 3 is
//    conflict-free, (r >> 2) & 3 takes two cycles per read.
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz64_m16(int r) { return (r >> 1) & 3; }

// 16-byte LDS read issued as an instruction the compiler does not track: its
// completion is awaited explicitly (lds_wait), so the compiler's own waits,
// which cannot tell the buffers in flight from the one being read, stay out
// of the loop.  The low 32 bits of a generic LDS address are the LDS offset.
__device__ __forceinline__ intx4 lds_read16(const unsigned char* p) {
    intx4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"((uint32_t)(uintptr_t)p));
    return v;
}


// The gated epilogue in two forms: EPI_GATED reads one gate row per tile and
// serves shapes where no tile spans two batches (one batch, or rows per batch
// a multiple of the tile height); EPI_GATED_ROWS reads the gate row of each
// output row.  Kept apart so that the common form has no per-row load behind a
// branch: the compiler's wait after such a branch drains every load in flight.
constexpr int EPI_GATED_ROWS = 4;

template <int BM, int BN, int SB, bool FP8, int EPI, int NWN = 2, bool M16 = false>
__global__ __launch_bounds__(128 * NWN) void k_gemm_deep(GemmArgs g) {
    // 2 x NWN wavefronts, each owning (BM/2) x (BN/NWN) outputs = TM x TN MFMA blocks of RB x RB
    // (RB = 32: v_mfma_f32_32x32x16_bf16 / the fp8 32x32x64; RB = 16: v_mfma_f32_16x16x32_bf16).
    static_assert(!(M16 && FP8), "16x16 blocks: bf16 only");
    constexpr int RB = M16 ? 16 : 32;
    constexpr int NW = 2 * NWN;
    constexpr int TM = BM / (2 * RB), TN = BN / (RB * NWN);
    constexpr int TS = BM / 64;                      // 32-row slices of a wavefront's block (epilogue)
    constexpr int DIST = 3;                          // prefetch distance (4 buffers); SB = stage bytes per row
    constexpr int KS = (FP8 || M16) ? SB / 64 : SB / 32;   // MFMA k-steps per stage
    constexpr int CPR = SB / 16, RPI = kWave / CPR;  // 16-byte chunks per row, rows per load instruction
    constexpr int LIA = BM / (NW * RPI), LIW = BN / (NW * RPI);   // load instructions per wavefront per operand
    constexpr int VM = 2 * (LIA + LIW);              // loads of the two stages after the one awaited
    // Tail stages (a stage count that is not a multiple of four) cost registers
    // in the large-tile kernels, so only the small-tile ones carry them.
    constexpr bool TAIL = BM == 128;
    static_assert(BM >= 128 && BN >= 64 && BM <= 256 && BN <= 256 && TN >= 1 && LIA >= 1 && LIW >= 1, "tile");
    static_assert(SB == 64 || SB == 128, "stage depth");
    constexpr int AB = BM * SB, WB = BN * SB;        // bytes of one stage buffer per operand
    static_assert(4 * (AB + WB) <= 160 * 1024, "LDS");
    // Chunk c of row r sits at c ^ swz(r): 64-byte rows as described above;
    // 128-byte rows (r >> 1) & 7 (rows r and r + 1 are half the banks apart).
    auto swz = [](int r) { return SB == 64 ? (M16 ? swz64_m16(r) : swz64(r)) : (r >> 1) & 7; };
    // Four buffers per operand as separate arrays, used with compile-time
    // indices (the k loop is unrolled by four): the compiler can then tell the
    // buffer a load fills from the one being read, and does not stall every
    // LDS read on the loads still in flight.
    __shared__ __attribute__((aligned(1024))) unsigned char A_0[AB], A_1[AB], A_2[AB], A_3[AB];
    __shared__ __attribute__((aligned(1024))) unsigned char W_0[WB], W_1[WB], W_2[WB], W_3[WB];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / NWN, wn = wave % NWN, l32 = lane % 32, half = lane / 32;
    int tmi, tni;
    tile_of(blockIdx.x, (g.M + BM - 1) / BM, (g.N + BN - 1) / BN, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const size_t rowA = (size_t)g.K * (FP8 ? 1 : 2);
    const unsigned char* A0 = (const unsigned char*)g.a + (size_t)m0 * rowA;
    const unsigned char* W0 = (const unsigned char*)g.w;
    // Rows past M or N re-read the last row (finite data); their outputs are not stored.
    // W is tiled: 64-row x 64-byte tiles, those of one 64-row band in k order,
    // so row n's 64 bytes at stage byte kb + 64 t sit at
    // (n / 64) * rowA * 64 + (kb / 64 + t) * 4096 + (n % 64) * 64, and one stage
    // of a 64-row band is 4 KB (64-byte stages) or 8 KB (128-byte) of
    // consecutive memory.  offW holds the part that does not move with kb; the
    // stage's own part is kb * 64.
    // A is row-major, or k-tiled like W (g.a_tiled): then the band of m0 (a
    // multiple of 64) starts at m0 * rowA as well, and a stage moves by kb * 64.
    uint32_t offA[LIA], offW[LIW];
#pragma unroll
    for (int i = 0; i < LIA; ++i) {
        const int r = (wave * LIA + i) * RPI + lane / CPR;
        const int m = min(r, g.M - 1 - m0), ch = (lane % CPR) ^ swz(r);
        offA[i] = g.a_tiled ? (uint32_t)((m >> 6) * rowA * 64) + (uint32_t)((ch >> 2) * 4096 + (m & 63) * 64 + (ch & 3) * 16)
                            : (uint32_t)(m * rowA) + (uint32_t)(ch * 16);
    }
    const int ash = g.a_tiled ? 6 : 0;
#pragma unroll
    for (int i = 0; i < LIW; ++i) {
        const int r = (wave * LIW + i) * RPI + lane / CPR;
        const int n = n0 + min(r, g.N - 1 - n0), ch = (lane % CPR) ^ swz(r);
        offW[i] = (uint32_t)((n >> 6) * rowA * 64) + (uint32_t)((ch >> 2) * 4096 + (n & 63) * 64 + (ch & 3) * 16);
    }
    auto abuf = [&](auto b) -> unsigned char* {
        if constexpr (decltype(b)::value == 0) return A_0;
        else if constexpr (decltype(b)::value == 1) return A_1;
        else if constexpr (decltype(b)::value == 2) return A_2;
        else return A_3;
    };
    auto wbuf = [&](auto b) -> unsigned char* {
        if constexpr (decltype(b)::value == 0) return W_0;
        else if constexpr (decltype(b)::value == 1) return W_1;
        else if constexpr (decltype(b)::value == 2) return W_2;
        else return W_3;
    };
    auto issue = [&](auto b, int kb) {
        unsigned char* ad = abuf(b);
        unsigned char* wd = wbuf(b);
#pragma unroll
        for (int i = 0; i < LIA; ++i)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(A0 + offA[i] + (kb << ash)),
                                             (__attribute__((address_space(3))) void*)(ad + (wave * LIA + i) * RPI * SB),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < LIW; ++i)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(W0 + offW[i] + kb * 64),
                                             (__attribute__((address_space(3))) void*)(wd + (wave * LIW + i) * RPI * SB),
                                             16, 0, 0);
    };

    using AccT = std::conditional_t<M16, floatx4, floatx16>;
    constexpr int NACC = M16 ? 4 : 16;
    AccT acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.0f;

    // Fragments: bf16 one 16-byte read per operand block and k-step, fp8 two.
    constexpr int RP = FP8 ? 2 : 1;                  // reads per fragment
    constexpr int NR = (TM + TN) * RP;               // reads per k-step
    intx4 fa[2][TM][RP], fb[2][TN][RP];
    auto reads = [&](int slot, const unsigned char* as, const unsigned char* ws, int ks) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * (BM / 2) + i * RB + (M16 ? lane % 16 : l32), sw = swz(row);
#pragma unroll
            for (int q = 0; q < RP; ++q) {
                const int c = M16 ? ks * 4 + lane / 16 : (FP8 ? ks * 4 + half * 2 + q : ks * 2 + half);
                fa[slot][i][q] = lds_read16(as + row * SB + ((c ^ sw) * 16));
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * (BN / NWN) + j * RB + (M16 ? lane % 16 : l32), sw = swz(row);
#pragma unroll
            for (int q = 0; q < RP; ++q) {
                const int c = M16 ? ks * 4 + lane / 16 : (FP8 ? ks * 4 + half * 2 + q : ks * 2 + half);
                fb[slot][j][q] = lds_read16(ws + row * SB + ((c ^ sw) * 16));
            }
        }
    };
    // Wait until at most `pending` LDS reads are outstanding (0 or NR, a literal after
    // inlining); the fragments of `slot` pass through the wait so the MFMAs that use
    // them cannot move above it.
    auto lds_wait = [&](int slot, int pending) {
        if (pending == 0) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fa[slot][0][0]));
        else asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(fa[slot][0][0]) : "i"(NR));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int q = 0; q < RP; ++q) asm volatile("" : "+v"(fa[slot][i][q]));
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < RP; ++q) asm volatile("" : "+v"(fb[slot][j][q]));
    };
    auto mma = [&](int slot) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (FP8) {
                    const intx4 a0 = fa[slot][i][0], a1 = fa[slot][i][1], b0 = fb[slot][j][0], b1 = fb[slot][j][1];
                    const intx8 av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                    const intx8 bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                    // formats 0/0: e4m3 x e4m3; scale exponents 127 = 2^0
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 0, 0, 0, 127, 0, 127);
                } else if constexpr (M16) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[slot][i][0]),
                                                                        __builtin_bit_cast(bf16x8, fb[slot][j][0]),
                                                                        acc[i][j], 0, 0, 0);
                } else {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[slot][i][0]),
                                                                        __builtin_bit_cast(bf16x8, fb[slot][j][0]),
                                                                        acc[i][j], 0, 0, 0);
                }
            }
    };
    // Single-k-step stages (KS = 1: the 16x16x32 tiles and fp8): the stage's
    // reads go out as the B fragments, then the A fragments in NG groups of
    // rows; the MFMAs of each group of rows start as soon as its fragments
    // have landed, so only the first group's read latency is exposed.
    constexpr int NG = (KS == 1 && TM % 4 == 0) ? 4 : 1, GR = TM / NG;   // groups, A rows per group
    // Group 0 of a stage: the B fragments and A rows [0, GR); the rest: A rows [GR, TM).
    auto reads_group0 = [&](const unsigned char* as, const unsigned char* ws) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * (BN / NWN) + j * RB + (M16 ? lane % 16 : l32), sw = swz(row);
#pragma unroll
            for (int q = 0; q < RP; ++q) {
                const int c = M16 ? lane / 16 : (FP8 ? half * 2 + q : half);
                fb[0][j][q] = lds_read16(ws + row * SB + ((c ^ sw) * 16));
            }
        }
#pragma unroll
        for (int i = 0; i < GR; ++i) {
            const int row = wm * (BM / 2) + i * RB + (M16 ? lane % 16 : l32), sw = swz(row);
#pragma unroll
            for (int q = 0; q < RP; ++q) {
                const int c = M16 ? lane / 16 : (FP8 ? half * 2 + q : half);
                fa[0][i][q] = lds_read16(as + row * SB + ((c ^ sw) * 16));
            }
        }
    };
    auto reads_rest = [&](const unsigned char* as) {
#pragma unroll
        for (int i = GR; i < TM; ++i) {
            const int row = wm * (BM / 2) + i * RB + (M16 ? lane % 16 : l32), sw = swz(row);
#pragma unroll
            for (int q = 0; q < RP; ++q) {
                const int c = M16 ? lane / 16 : (FP8 ? half * 2 + q : half);
                fa[0][i][q] = lds_read16(as + row * SB + ((c ^ sw) * 16));
            }
        }
    };
    // Wait until the fragments of row group gi have landed (the later groups'
    // GR RP reads each may still be outstanding); the waited fragments pass
    // through the wait so that the MFMAs using them stay below it.
    auto wait_group = [&](int g) {   // g: a literal after inlining
        if (g == 0) asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"((NG - 1) * GR * RP) : "memory");
        else if (g == 1) asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(NG > 2 ? (NG - 2) * GR * RP : 0) : "memory");
        else if (g == 2) asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(NG > 3 ? (NG - 3) * GR * RP : 0) : "memory");
        else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (g == 0) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < RP; ++q) asm volatile("" : "+v"(fb[0][j][q]));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
            if (i / GR == g)
#pragma unroll
                for (int q = 0; q < RP; ++q) asm volatile("" : "+v"(fa[0][i][q]));
    };
    auto mma_rows = [&](int g) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if (i / GR != g) continue;
                if constexpr (FP8) {
                    const intx4 a0 = fa[0][i][0], a1 = fa[0][i][1], b0 = fb[0][j][0], b1 = fb[0][j][1];
                    const intx8 av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                    const intx8 bv = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 0, 0, 0, 127, 0, 127);
                } else if constexpr (M16) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[0][i][0]),
                                                                        __builtin_bit_cast(bf16x8, fb[0][j][0]),
                                                                        acc[i][j], 0, 0, 0);
                } else {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[0][i][0]),
                                                                        __builtin_bit_cast(bf16x8, fb[0][j][0]),
                                                                        acc[i][j], 0, 0, 0);
                }
            }
    };

    const int nk = (int)(rowA / SB);
    // Stages of four k-steps (bf16, 128-byte stages) read the next stage's
    // first fragments during their last MFMAs ("look-ahead", below): measured
    // 3-5% faster on the tiles that use them.  With two k-steps per stage the
    // 256-row tiles ran 2-3% slower that way, and with one (fp8, 64-byte
    // stages) both fragment slots would be live at once, beyond the 256x256
    // tile's registers; those stages read at their own start.
    // Grouped look-ahead (below) for the fp8 single-k-step stages: 3-4% faster
    // on the 32760-token fp8 products, 1-3% slower on the 16x16x32 bf16 ones,
    // which read their groups at the stage start (A/B on one machine, same output bits).
    constexpr bool LOOK = KS >= 4 || (NG > 1 && FP8);
    // Look-ahead stage: multiply the tiles in buffer B = kt % 4 while the next
    // k-step's fragments are read, the first of them having been read at the
    // end of the previous stage.  Before its last k-step: wait for this
    // wavefront's loads of stage kt + 1 (those of kt + 2 and kt + 3 may still
    // be outstanding), then a barrier.  The barrier makes every wavefront's
    // loads of stage kt + 1 visible, and it follows every wavefront's last read
    // of buffer B, which is then refilled with stage kt + 4.  Stage kt + 1's
    // first fragments are read while the last MFMAs of stage kt run, so no
    // stage starts on an LDS read.
    // Plain stage: wait for its own tiles (loads of the two later stages may be
    // outstanding) and barrier, refill the buffer freed one stage ago (three
    // stages ahead), then read and multiply, the reads for k-step ks + 1 in
    // flight while the MFMAs of k-step ks run.
    auto stage = [&](auto b, int kt) {
        constexpr int B = decltype(b)::value;
        const unsigned char* as = abuf(b);
        const unsigned char* ws = wbuf(b);
        if constexpr (LOOK && NG > 1) {
            // Grouped look-ahead (one k-step per stage): group 0 of this stage was
            // read at the end of the previous one; read the other rows, multiply
            // each group as it lands, and before the last group wait for stage
            // kt + 1's loads and barrier (every wavefront is then done reading
            // buffer B, which takes stage kt + 4); after the last group's MFMAs
            // read group 0 of stage kt + 1 into the registers they freed.
            using Next = std::integral_constant<int, (B + 1) % 4>;
            reads_rest(as);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                wait_group(g);
                if (g == NG - 1) {
                    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(VM) : "memory");
                    issue(b, min(kt + 4, nk - 1) * SB);
                }
                mma_rows(g);
                __builtin_amdgcn_sched_barrier(0);   // group g's MFMAs stay between its wait and the next
            }
            __builtin_amdgcn_sched_barrier(0);   // the last MFMAs read B and A rows before the reads reuse them
            reads_group0(abuf(Next{}), wbuf(Next{}));
        } else if constexpr (LOOK) {
            using Next = std::integral_constant<int, (B + 1) % 4>;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int sl = ks & 1;   // KS is a multiple of 4
                if (ks + 1 < KS) {
                    reads(sl ^ 1, as, ws, ks + 1);
                    lds_wait(sl, NR);
                } else {
                    lds_wait(sl, 0);
                    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(VM) : "memory");
                    issue(b, min(kt + 4, nk - 1) * SB);
                    reads(sl ^ 1, abuf(Next{}), wbuf(Next{}), 0);
                }
                mma(sl);
            }
        } else if constexpr (NG > 1) {
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(VM) : "memory");
            issue(std::integral_constant<int, (B + DIST) % 4>{}, min(kt + DIST, nk - 1) * SB);
            reads_group0(as, ws);
            reads_rest(as);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                wait_group(g);
                mma_rows(g);
            }
        } else {
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(VM) : "memory");
            issue(std::integral_constant<int, (B + DIST) % 4>{}, min(kt + DIST, nk - 1) * SB);
            reads(0, as, ws, 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 1 < KS) {
                    reads((ks + 1) & 1, as, ws, ks + 1);
                    lds_wait(ks & 1, NR);
                } else {
                    lds_wait(ks & 1, 0);
                }
                mma(ks & 1);
            }
        }
    };

    // Stage kt uses buffer kt % 4; past the end issue() re-loads the last stage
    // into a buffer no later stage reads (and the last look-ahead reads that
    // buffer; the values are not used).  Look-ahead: stages 0..3 in flight,
    // stage 0 visible to every wavefront and its first fragments read before
    // the loop.  Plain: stages 0..2 in flight.
    // The epilogue's per-row and per-column operands (bias, fp8 row and weight
    // scales) are loaded here, ahead of the first stages, held in registers
    // through the k loop and put in LDS after it, so the epilogue reads no
    // global memory but the residual.  Every thread loads (clamped indices), so
    // no branch disturbs the compiler's wait counts.
    static_assert(128 * NWN >= BM && 128 * NWN >= BN, "a thread per epilogue row and column");
    __shared__ __attribute__((aligned(16))) float ep_as[FP8 ? BM : 1], ep_ws[FP8 ? BN : 1];
    __shared__ __attribute__((aligned(16))) bf16 ep_bias[BN];
    const bf16* bsrc = g.bias ? (const bf16*)g.bias : (const bf16*)g.w;   // W: any 8 readable bytes
    const bf16x4 ep_bv = *(const bf16x4*)(bsrc + min(n0 + 4 * min(tid, BN / 4 - 1), g.N - 4));
    float ep_asv = 0.0f, ep_wsv = 0.0f;
    if constexpr (FP8) {
        ep_asv = g.a_scale[min(m0 + min(tid, BM - 1), g.M - 1)];
        ep_wsv = g.w_scale[min(n0 + min(tid, BN - 1), g.N - 1) / g.w_seg];
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, min(1, nk - 1) * SB);
    issue(std::integral_constant<int, 2>{}, min(2, nk - 1) * SB);
    if constexpr (LOOK) {
        issue(std::integral_constant<int, 3>{}, min(3, nk - 1) * SB);
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"i"(VM + LIA + LIW) : "memory");
        if constexpr (NG > 1) reads_group0(abuf(std::integral_constant<int, 0>{}), wbuf(std::integral_constant<int, 0>{}));
        else reads(0, abuf(std::integral_constant<int, 0>{}), wbuf(std::integral_constant<int, 0>{}), 0);
    }
    // Without TAIL the launcher guarantees nk % 4 == 0.
    int kt = 0;
    for (; kt + 4 <= nk; kt += 4) {
        stage(std::integral_constant<int, 0>{}, kt);
        stage(std::integral_constant<int, 1>{}, kt + 1);
        stage(std::integral_constant<int, 2>{}, kt + 2);
        stage(std::integral_constant<int, 3>{}, kt + 3);
    }
    if constexpr (TAIL) {
        if (kt < nk) stage(std::integral_constant<int, 0>{}, kt);
        if (kt + 1 < nk) stage(std::integral_constant<int, 1>{}, kt + 1);
        if (kt + 2 < nk) stage(std::integral_constant<int, 2>{}, kt + 2);
    }
    if constexpr (LOOK) {   // the last look-ahead reads are still in flight into the fragment registers
        lds_wait(0, 0);
        lds_wait(1, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the trailing re-loads before the workgroup ends
    if (tid < BN / 4) *(bf16x4*)&ep_bias[4 * tid] = g.bias ? ep_bv : bf16x4{0, 0, 0, 0};
    if constexpr (FP8) {
        if (tid < BM) ep_as[tid] = ep_asv;
        if (tid < BN) ep_ws[tid] = ep_wsv;
    }
    __syncthreads();                                    // every wavefront is done with the stage buffers

    // Lane and wavefront indices derived again after the k loop, through an asm
    // statement, so that the compiler does not keep the k loop's copies (and
    // values computed from them) alive across it.
    int etid = threadIdx.x;
    asm volatile("" : "+v"(etid));
    const int ewave = etid / kWave, elane = etid % kWave, ewm = ewave / NWN, ewn = ewave % NWN;
    const int el32 = elane % 32, ehalf = elane / 32;
    // Epilogue through LDS.  Per 32-row slice of its block, a wavefront writes
    // the fp32 accumulators into its own buffer (row stride CW floats), reads
    // them back as row-contiguous float4s (CH lanes per row, RPP rows per
    // pass) and applies the epilogue with 8- or 16-byte global accesses.  The
    // residual forms load the fp32 residual rows of slice i + 1 before slice
    // i's LDS round trip, so the slices' load latencies overlap, and read the
    // gate row once when the tile's rows all lie in one batch.  Every load is
    // unconditional (rows past M and columns past N read row M - 1 and column
    // 0, and only the stores are masked), so the compiler's wait counts are
    // exact: a load under a lane condition makes the waits that follow it drain
    // every load in flight, which had put each residual load of the prefetch
    // one round trip behind the previous one.
    constexpr int CW = BN / NWN, CH = CW / 4, RPP = kWave / CH, NP = 32 / RPP, PB = NP < 8 ? NP : 8;
    constexpr bool RES = EPI >= EPI_GATED;
    static_assert((NW / 4) * 32 * CW * 4 <= AB, "epilogue staging fits the A buffers");
    float* lds = (float*)((ewave % 4 == 0 ? A_0 : ewave % 4 == 1 ? A_1 : ewave % 4 == 2 ? A_2 : A_3) +
                          (ewave / 4) * 32 * CW * 4);
    const int c4 = elane % CH, rr = elane / CH;           // float4 column chunk and row-in-pass of this elane
    const int nb = n0 + ewn * CW + 4 * c4;               // its first output column (CW = BN / NWN)
    const bool ncol = nb < g.N;                         // N % 8 == 0: all four columns valid
    const int nbl = ncol ? nb : 0;                      // the column its loads read
    const int mw = m0 + ewm * (BM / 2);                  // first row of this wavefront's block
    const int nl = nb - n0;                             // its first column within the tile (< BN)
    const bf16x4 bb = *(const bf16x4*)&ep_bias[nl];
    const float4 bias4 = make_float4((float)bb[0], (float)bb[1], (float)bb[2], (float)bb[3]);
    float4 ws4 = make_float4(1.f, 1.f, 1.f, 1.f);
    if constexpr (FP8) ws4 = *(const float4*)&ep_ws[nl];
    float4 xq[2][NP];                                   // residual rows of two slices (residual forms)
    auto load_x = [&](int i, float4 (&dst)[NP]) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int m = min(mw + i * 32 + p * RPP + rr, g.M - 1);
            dst[p] = *(const float4*)(g.xr + (size_t)m * g.ldx + nbl);
        }
    };
    float4 g1 = make_float4(1.f, 1.f, 1.f, 1.f);     // the tile's gate row (EPI_GATED)
    if constexpr (EPI == EPI_GATED) g1 = *(const float4*)(g.gate + (size_t)(m0 / g.rows_per_batch) * g.gate_ld + nbl);
    if constexpr (RES) load_x(0, xq[0]);
#pragma unroll
    for (int i = 0; i < TS; ++i) {
        if constexpr (RES) {
            if (i + 1 < TS) load_x(i + 1, xq[(i + 1) % 2]);
        }
        if constexpr (M16) {   // 16x16 blocks 2i, 2i + 1: elane holds column elane % 16, rows 4 (elane / 16) + r
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        lds[(sb * 16 + 4 * (elane / 16) + r) * CW + j * 16 + elane % 16] = acc[2 * i + sb][j][r];
        } else {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    lds[(8 * (r / 4) + 4 * ehalf + (r % 4)) * CW + j * 32 + el32] = acc[i][j][r];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // own slice only: no cross-wavefront sync
#pragma unroll
        for (int h = 0; h < NP / PB; ++h) {
            float4 v[PB];
            int mrow[PB];
#pragma unroll
            for (int it = 0; it < PB; ++it) {
                const int row = (h * PB + it) * RPP + rr;
                mrow[it] = mw + i * 32 + row;
                float4 a4 = *(const float4*)&lds[row * CW + 4 * c4];
                if (FP8) {
                    const float as = ep_as[mrow[it] - m0];
                    a4 = make_float4(a4.x * ws4.x * as, a4.y * ws4.y * as, a4.z * ws4.z * as, a4.w * ws4.w * as);
                }
                v[it] = make_float4(a4.x + bias4.x, a4.y + bias4.y, a4.z + bias4.z, a4.w + bias4.w);
            }
#pragma unroll
            for (int it = 0; it < PB; ++it) {
                if (!ncol || mrow[it] >= g.M) continue;
                const float4 y = v[it];
                if constexpr (EPI <= EPI_GELU) {
                    bf16x4 o;
                    if (EPI == EPI_GELU) {
                        o[0] = (bf16)gelu_tanh(y.x); o[1] = (bf16)gelu_tanh(y.y);
                        o[2] = (bf16)gelu_tanh(y.z); o[3] = (bf16)gelu_tanh(y.w);
                    } else {
                        o[0] = (bf16)y.x; o[1] = (bf16)y.y; o[2] = (bf16)y.z; o[3] = (bf16)y.w;
                    }
                    bf16* dst = g.out_tiled ? (bf16*)((char*)g.out + ktiled_off(mrow[it], (size_t)2 * nb, (size_t)2 * g.ldo))
                                            : (bf16*)g.out + (size_t)mrow[it] * g.ldo + nb;
                    *(bf16x4*)dst = o;
                } else {
                    const float4 x = xq[i % 2][h * PB + it];
                    float4 gg = g1;
                    if constexpr (EPI == EPI_GATED_ROWS)
                        gg = *(const float4*)(g.gate + (size_t)(mrow[it] / g.rows_per_batch) * g.gate_ld + nb);
                    *(float4*)(g.xr + (size_t)mrow[it] * g.ldx + nb) =
                        make_float4(x.x + gg.x * y.x, x.y + gg.y * y.y, x.z + gg.z * y.z, x.w + gg.w * y.w);
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next slice overwrites
    }
}

// ------------------------------------------------------------------ launch

template <int EPI, int BM, int BN, int SB, bool F8, int NWN = 2, bool M16 = false>
static void launch_deep(const GemmArgs& g, int grid, int threads, hipStream_t st) {
    if constexpr (EPI == EPI_GATED) {
        if (g.rows_per_batch < g.M && g.rows_per_batch % BM) {   // a batch boundary inside some tile
            LWO_KL((k_gemm_deep<BM, BN, SB, F8, EPI_GATED_ROWS, NWN, M16>), grid, threads, 0, st, g);
            return;
        }
    }
    LWO_KL((k_gemm_deep<BM, BN, SB, F8, EPI, NWN, M16>), grid, threads, 0, st, g);
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, hipStream_t st) {
    if (g.dtype == LWO_F32) {
        dim3 grid((g.N + 63) / 64, (g.M + 63) / 64);
        // Under 64 tiles of 64x64 a few CUs would each run one wavefront per SIMD
        // down the whole of K: 32x32 tiles (four times the workgroups), K split four ways.
        if (grid.x * grid.y < 64 && g.K >= 64) {
            dim3 g32((g.N + 31) / 32, (g.M + 31) / 32);
            LWO_KL((k_gemm_f32_splitk<EPI, 32>), g32, 1024, 0, st, g);
        } else {
            LWO_KL((k_gemm_f32<EPI>), grid, 256, 0, st, g);
        }
        return hipGetLastError();
    }
    // K rows are a multiple of 128 bytes (argument checks); the 256-row tiles
    // unroll the k loop by four 64-byte stages without a tail.
    const bool rows256 = (size_t)g.K * (g.dtype == LWO_BF16 ? 2 : 1) % 256 == 0;
    auto tiles = [&](int bm, int bn) { return ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn); };
    const bool f8 = g.dtype != LWO_BF16;
    // Tile choice (measured on the block shapes): the largest tile that still
    // gives most CUs a workgroup.  256x256 and 256x128 hold one workgroup per
    // CU (LDS), 128x128 two (64-byte stages) or one (128-byte stages), 128x64 one.
    const int t256 = tiles(256, 256), t256x128 = tiles(256, 128), t128 = tiles(128, 128);
    if (rows256 && t256 >= 256) {   // eight wavefronts: two per SIMD
        // bf16 on 16x16x32 MFMAs: half the accumulator traffic per flop of the
        // 32x32x16 form, which these power-limited products turn into speed
        // (32760-token products 1-4% faster, same results bit for bit).
        if (f8) launch_deep<EPI, 256, 256, 64, true, 4>(g, t256, 512, st);
        else launch_deep<EPI, 256, 256, 64, false, 4, true>(g, t256, 512, st);
    } else if (rows256 && t256x128 >= 192 && t256x128 <= 256) {
        if (f8) launch_deep<EPI, 256, 128, 64, true>(g, t256x128, 256, st);
        else launch_deep<EPI, 256, 128, 64, false>(g, t256x128, 256, st);
    } else if (t128 > 256) {   // two 64 KB workgroups per CU
        if (f8) launch_deep<EPI, 128, 128, 64, true>(g, t128, 256, st);
        else launch_deep<EPI, 128, 128, 64, false>(g, t128, 256, st);
    } else if (t128 >= 128) {  // one workgroup per CU: 128-byte stages keep more bytes in flight
        if (f8) launch_deep<EPI, 128, 128, 128, true, 4>(g, t128, 512, st);
        else launch_deep<EPI, 128, 128, 128, false, 4>(g, t128, 512, st);
    } else {
        const int t = tiles(128, 64);
        if (f8) launch_deep<EPI, 128, 64, 128, true>(g, t, 256, st);
        else launch_deep<EPI, 128, 64, 128, false>(g, t, 256, st);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
    if (g.M <= 0) return hipSuccess;
    const int kq = g.dtype == LWO_F32 ? 16 : (g.dtype == LWO_BF16 ? 64 : 128);
    if (g.N <= 0 || g.K <= 0 || g.K % kq) return hipErrorInvalidValue;
    if (g.dtype != LWO_F32 && g.act_dtype != LWO_BF16) return hipErrorInvalidValue;
    if ((g.a_tiled || g.out_tiled) && g.dtype == LWO_F32) return hipErrorInvalidValue;   // fp32 tiles read rows
    if (g.out_tiled && (g.epi > EPI_GELU || g.ldo % 32)) return hipErrorInvalidValue;    // whole 64-byte tile rows
    switch (g.epi) {
        case EPI_STORE: return launch_epi<EPI_STORE>(g, st);
        case EPI_GELU: return launch_epi<EPI_GELU>(g, st);
        case EPI_GATED: return launch_epi<EPI_GATED>(g, st);
        default: return launch_epi<EPI_RESID>(g, st);
    }
}

}  // namespace lwo
