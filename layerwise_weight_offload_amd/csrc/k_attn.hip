// Softmax attention without a mask (self- and cross-attention of the DiT
// block): O = softmax(Q K^T / sqrt(d)) V per (batch, head), streamed over key
// tiles with an online softmax so the T x T score matrix never exists.
//
// k_attn_tr (bf16, gfx950 MFMA v_mfma_f32_32x32x16_bf16), per wavefront 32
// queries, per 64-key tile:
//   S^T = K Q^T: A = K rows from LDS, B = the wavefront's Q fragments kept in
//          registers for the whole kernel; the accumulator layout puts one
//          query in each lane (column), so the row max and row sum are
//          in-lane reductions plus one swap between the two 32-lane halves;
//   O^T += V^T P^T: B = the probabilities straight from the S^T registers
//          (rounded to bf16), A = V^T fragments read transposed from the
//          row-major V tile; the key order inside each MFMA k-step follows
//          the accumulator layout, identically on both operands.
// Head dims 64, 72 and 128: QK^T is padded with zeros to a multiple of 16
// and the PV output to a multiple of 32 columns (72 -> 80 and 96); padded
// columns are never stored.  Key and query tails are masked.
//
// The fp32 kernel is in k_attn_f32.hip.
#include <math.h>

#include <type_traits>

#include "../../include/lwo.h"
#include "kcommon.h"
#include "kernels.h"

namespace lwo {

// ------------------------------------------------------------------ direct-to-LDS tiles, transpose reads

// k_attn_tr<DH, NW>: NW wavefronts own 32 NW queries of one (batch, head),
// 32 per wavefront, with the S^T = K Q^T / O^T += V^T P^T formulation above.
// Per 64-key tile:
//  * K and V land in LDS with global_load_lds (16 bytes per lane, no
//    register round trip), double-buffered: the tile after the current one
//    is in flight while the current one is multiplied.  A row is NC 16-byte
//    chunks (NC = 16, 12, 8 for d = 128, 72, 64: d 72 is read as 80 columns
//    by QK and 96 by PV); chunks past the head's data hold a copy of its last
//    chunk, so every value read is finite: padded K columns meet zero Q
//    columns and padded V columns only feed outputs that are not stored.
//    Chunk c of row r sits at c ^ fK(r) in K and c ^ fV(r) in V, chosen per
//    row pitch so that the rows one fragment read touches fall on distinct
//    banks.
//  * V^T fragments come from ds_read_b64_tr_b16: within each group of 16
//    lanes, lane 4y + c addresses four consecutive 16-bit values and lane j
//    receives value j % 4 of lanes j / 4, 4 + j / 4, 8 + j / 4, 12 + j / 4.
//    With lane 4y + c pointing at key K0 + y, columns d0 + 4c .. d0 + 4c + 3,
//    lane j gets V[K0 .. K0 + 3][d0 + j]: four keys of one output column, in
//    the key order of the probability operand.
//  * The softmax reference point (the row max in base-2 exponent units) is
//    set on a wavefront's first tile and then kept: the probabilities and the
//    row sum share it, so any reference gives the same result up to rounding.
//    A tile takes no row max unless its row sum passes 2^32 in some lane (a
//    score far above the reference); such a tile recomputes its scores from
//    LDS, moves the reference to the row max and rescales O and the row sum.

// LDS reads issued as instructions the compiler does not track (their
// completion is awaited with explicit lgkmcnt waits, so loads still in flight
// into the other buffer do not stall them); `off` must fold to a constant.
#define LDS_RD128(v, addr, off) asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(off))
#define LDS_RD64_TR16(v, addr, off) asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(off))

template <int DH> struct TrGeom;
template <> struct TrGeom<128> {   // 256-byte rows: every row starts on bank 0
    static constexpr int NC = 16;
    static __device__ int fk(int r) { return r & 15; }
    static __device__ int fv(int r) { return 4 * (r & 3); }
};
template <> struct TrGeom<72> {    // 192-byte rows: rows r, r+4, r+8, r+12 share banks
    static constexpr int NC = 12;
    static __device__ int fk(int r) { return (r >> 2) & 3; }   // permutes within aligned groups of 4: stays < 12
    static __device__ int fv(int) { return 0; }               // four consecutive rows already disjoint
};
template <> struct TrGeom<64> {    // 128-byte rows: rows r, r+2 share banks
    static constexpr int NC = 8;
    static __device__ int fk(int r) { return (r >> 1) & 7; }
    static __device__ int fv(int r) { return 4 * ((r >> 1) & 1); }
};

// KSP = 2 splits the key tiles of one query tile between two groups of NW
// wavefronts (the first and the second half of the tiles, each group with its
// own K/V buffers), so a grid of few query tiles still puts two wavefronts on
// every SIMD; the groups' softmax states and accumulators merge through LDS at
// the end (the merge is exact: O and the row sum share each group's reference
// point, both rescaled to the larger one).
template <int DH, int NW, int KSP = 1>
__global__ __launch_bounds__(NW * KSP * 64, 2) void k_attn_tr(AttnArgs a) {
    using G = TrGeom<DH>;
    constexpr int BN = 64, QW = 32, NC = G::NC, PITCH = NC * 16, NVALID = DH / 8;
    constexpr int KS = (DH + 15) / 16, NT = (DH + 31) / 32;   // QK k-steps, PV output tiles of 32 columns
    constexpr int LI = NC / NW;                      // load instructions per wavefront per operand and tile
    static_assert(NC % NW == 0 && 2 * KS <= NC && 4 * NT <= NC, "geometry");
    constexpr int TB = BN * PITCH;                   // bytes per K or V tile
    constexpr int KOFF = 0, VOFF = 2 * TB;           // K buffers at 0, TB; V buffers at 2 TB, 3 TB (per group)
    static_assert(KSP == 1 || KSP == 2, "key split");
    __shared__ __attribute__((aligned(1024))) unsigned char lds_all[KSP * 4 * TB];

    const int tid = threadIdx.x, wave = (tid / kWave) % NW, lane = tid % kWave;
    const int grp = tid / (kWave * NW);              // key group (0 unless KSP = 2)
    unsigned char* const smem = lds_all + grp * 4 * TB;
    const int l32 = lane % 32, half = lane / 32;
    // Workgroups go to the 8 XCDs round-robin by linear id.  Each XCD gets a
    // contiguous run of (query tile, head, batch) work instead, so its L2
    // streams the keys and values of few heads: on the 32760-token stack this
    // halves the bytes the kernel fetches from memory (5.7 -> 3.0 GB per
    // launch) at the same speed.  The map is a bijection of the grid.
    int qt, h, b;
    {
        const int nx = gridDim.x, ny = gridDim.y;
        const int total = nx * ny * gridDim.z;
        const int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
        const int x = id % 8, idx = id / 8, base = total / 8, rem = total % 8;
        const int t = x * base + min(x, rem) + idx;
        qt = t % nx;
        h = (t / nx) % ny;
        b = t / (nx * ny);
    }
    const int Tq = a.Tq, Tk = a.Tk;
    const int qi = qt * (NW * QW) + wave * QW + l32;
    const unsigned char* Kg = (const unsigned char*)a.k + ((size_t)b * Tk * a.ldk + h * DH) * 2;
    const unsigned char* Vg = (const unsigned char*)a.v + ((size_t)b * Tk * a.ldv + h * DH) * 2;

    // Loads: instruction q = wave LI + i fills chunk positions 64 q .. 64 q + 63 of
    // the tile (row p / NC, position p % NC), one per lane.
    int lrow[LI], kcol[LI], vcol[LI];
#pragma unroll
    for (int i = 0; i < LI; ++i) {
        const int p = (wave * LI + i) * 64 + lane;
        const int r = p / NC, cp = p % NC;
        lrow[i] = r;
        kcol[i] = min(cp ^ G::fk(r), NVALID - 1) * 16;
        vcol[i] = min(cp ^ G::fv(r), NVALID - 1) * 16;
    }
    auto issue = [&](auto buf, int key0) {
        constexpr int B = decltype(buf)::value;
#pragma unroll
        for (int i = 0; i < LI; ++i) {
            const size_t key = (size_t)min(key0 + lrow[i], Tk - 1);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Kg + key * a.ldk * 2 + kcol[i]),
                                             (__attribute__((address_space(3))) void*)(smem + KOFF + B * TB + (wave * LI + i) * 1024),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Vg + key * a.ldv * 2 + vcol[i]),
                                             (__attribute__((address_space(3))) void*)(smem + VOFF + B * TB + (wave * LI + i) * 1024),
                                             16, 0, 0);
        }
    };

    const intx4 z = {0, 0, 0, 0};
    intx4 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int d0 = s * 16 + half * 8;
        qf[s] = (qi < Tq && d0 < DH) ? *(const intx4*)((const bf16*)a.q + (size_t)(b * Tq + qi) * a.ldq + h * DH + d0) : z;
    }

    floatx16 oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] = 0.0f;
    float m_i = -INFINITY, l_i = 0.0f;
    const float sl2 = 1.4426950408889634f / sqrtf((float)DH);   // log2(e) / sqrt(d)

    // Per-lane LDS addresses; buffer and key offsets go into the instruction.
    const uint32_t sbase = (uint32_t)(uintptr_t)smem;
    uint32_t kaddr[KS], vaddr[NT];
#pragma unroll
    for (int st = 0; st < KS; ++st)   // K row t*32 + l32 (fk(row) == fk(l32)), chunk 2 st + half
        kaddr[st] = sbase + KOFF + l32 * PITCH + (((2 * st + half) ^ G::fk(l32)) * 16);
    {
        const int j16 = lane % 16, ty = j16 / 4, tc = j16 % 4, g2 = (lane / 16) % 2;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)   // V row t*32 + 16 ks + 4 half + ty (+ 8): fv(row) == fv(ty)
            vaddr[nt] = sbase + VOFF + (4 * half + ty) * PITCH + ((4 * nt + 2 * g2 + tc / 2) ^ G::fv(ty)) * 16 +
                        8 * (tc % 2);
    }

    // `first`: the wavefront's first tile (m_i = -inf in every lane).
    auto tile = [&](auto buf, int key0, bool first) {
        constexpr int BO = decltype(buf)::value * TB;
        floatx16 s[2];
        // ---- S^T = K Q^T for 64 keys (computed again from the same LDS tile
        // on the rare path below); keys past Tk are masked to -inf
        auto scores = [&]() {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
            if constexpr (KS == 8) {
                // four batches of four k-steps (batch u: 32-key half u / 2, k-steps
                // 4 (u % 2) .. + 3); two batches in flight
                intx4 kf[2][4];
#define KREAD(u)                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                         \
        LDS_RD128(kf[(u) % 2][i], kaddr[4 * ((u) % 2) + i], BO + ((u) / 2) * 32 * PITCH);
                KREAD(0);
                KREAD(1);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (u < 3) asm volatile("s_waitcnt lgkmcnt(4)" ::: "memory");
                    else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        asm volatile("" : "+v"(kf[u % 2][i]));
                        s[u / 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[u % 2][i]),
                                                                           __builtin_bit_cast(bf16x8, qf[4 * (u % 2) + i]),
                                                                           s[u / 2], 0, 0, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);   // keep batch u's MFMAs ahead of the reads that reuse its registers
                    if (u == 0) { KREAD(2); }
                    if (u == 1) { KREAD(3); }
                }
#undef KREAD
            } else {
                // both 32-key halves in flight, then the MFMAs of each
                intx4 kf[2][KS];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int st = 0; st < KS; ++st) LDS_RD128(kf[t][st], kaddr[st], BO + t * 32 * PITCH);
                asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(KS) : "memory");
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    if (t == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                    for (int st = 0; st < KS; ++st) {
                        asm volatile("" : "+v"(kf[t][st]));
                        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[t][st]),
                                                                       __builtin_bit_cast(bf16x8, qf[st]), s[t], 0, 0, 0);
                    }
                }
            }
            // s[t][r]: key key0 + 32t + 8(r/4) + 4 half + r%4, query qi
            if (key0 + BN > Tk) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (key0 + t * 32 + 8 * (r / 4) + 4 * half + (r % 4) >= Tk) s[t][r] = -INFINITY;
            }
        };
        scores();
        // V^T fragments of keys 0..31 (16 keys per k-step): read now, in flight
        // during the softmax below, whose two-half reductions use a lane swap
        // (VALU) rather than an LDS permute so that nothing waits for them early.
#define VREAD(T, KS, VF)                                                                  \
    _Pragma("unroll") for (int nt = 0; nt < NT; ++nt) {                                   \
        LDS_RD64_TR16(VF[KS][nt][0], vaddr[nt], BO + ((T) * 32 + 16 * (KS)) * PITCH);     \
        LDS_RD64_TR16(VF[KS][nt][1], vaddr[nt], BO + ((T) * 32 + 16 * (KS) + 8) * PITCH); \
    }
        intx2 va[2][NT][2], vb[2][NT][2];
        VREAD(0, 0, va);
        VREAD(0, 1, va);
        __builtin_amdgcn_sched_barrier(0);   // issue them before the softmax, not where PV needs them
        auto swap_halves = [](float x, auto op) {
            const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            return op(__uint_as_float(p[0]), __uint_as_float(p[1]));
        };

        // ---- Probabilities against the current reference point m_i (base-2
        // exponent units) and their row sum, taken from the bf16 values the PV
        // products use (two at a time, a dot product against (1, 1)).  The
        // reference point does not follow the row max tile by tile: any m_i
        // gives the same O and row sum up to rounding, as both share it, so the
        // max is only taken when the probabilities would grow too large.  A tile
        // whose row sum passes 2^32 in some lane (a score far above m_i, or the
        // first tile, where m_i = -inf) recomputes its scores from the tile still
        // in LDS, moves m_i to the row max, rescales O and the row sum, and
        // recomputes the probabilities; the first tile goes straight to the max,
        // and every other tile skips it.
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        bf16x8 pf[2][2];
        float rs;
        auto probs = [&]() {
            const float nm = -m_i;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[t][r] = __builtin_amdgcn_exp2f(fmaf(s[t][r], sl2, nm));
            const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
            float r0 = 0.0f, r1 = 0.0f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pf[t][ks][e] = (bf16)s[t][ks * 8 + e];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bf16x2_t pp = {pf[t][ks][2 * e], pf[t][ks][2 * e + 1]};
                        if (ks == 0) r0 = __builtin_amdgcn_fdot2_f32_bf16(pp, one, r0, false);
                        else r1 = __builtin_amdgcn_fdot2_f32_bf16(pp, one, r1, false);
                    }
                }
            rs = r0 + r1;
        };
        bool redo = first;
        if (!first) {
            probs();
            redo = __ballot(!(rs <= 0x1p32f)) != 0;   // NaN-safe: a NaN sum takes this path too
            if (redo) scores();
        }
        if (redo) {
            float mx = s[0][0];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
            mx = swap_halves(mx, [](float u, float v) { return fmaxf(u, v); }) * sl2;
            const float m_new = fmaxf(m_i, mx);
            const float corr = __builtin_amdgcn_exp2f(m_i - m_new);   // 0 on the first tile, 1 where m_i stays
            l_i *= corr;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[nt][r] *= corr;
            m_i = m_new;
            probs();
        }

        // ---- O^T += V^T P^T, one k-step (16 keys) at a time.  Keys 32..63's
        // fragments are read while keys 0..31's MFMAs run; every wait leaves at
        // most 2 NT reads outstanding (the counter holds 15).
        auto pv = [&](int t, int ks, intx2 (&vf)[2][NT][2]) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                asm volatile("" : "+v"(vf[ks][nt][0]), "+v"(vf[ks][nt][1]));
                const intx4 v4 = {vf[ks][nt][0][0], vf[ks][nt][0][1], vf[ks][nt][1][0], vf[ks][nt][1][1]};
                oacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v4), pf[t][ks], oacc[nt], 0, 0, 0);
            }
        };
        VREAD(1, 0, vb);
        asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(2 * NT) : "memory");   // keys 0..31 landed
        VREAD(1, 1, vb);
        pv(0, 0, va);
        pv(0, 1, va);
        asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(2 * NT) : "memory");   // keys 32..47
        pv(1, 0, vb);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        pv(1, 1, vb);
        l_i += swap_halves(rs, [](float u, float v) { return u + v; });
#undef VREAD
    };

    // Group g takes tiles [g nt0, min((g + 1) nt0, ntile)); every wavefront runs the
    // same nt0 iterations so that the barriers match, skipping tiles past its range.
    const int ntile = (Tk + BN - 1) / BN, nt0 = (ntile + KSP - 1) / KSP;
    const int t0 = grp * nt0, tend = min(t0 + nt0, ntile);
    if (t0 < tend) issue(std::integral_constant<int, 0>{}, t0 * BN);
    for (int j = 0; j < nt0; j += 2) {
        // Tile j in buffer 0: its loads are this wavefront's only outstanding ones; the
        // barrier publishes every wavefront's loads and frees buffer 1 for tile j + 1.
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (t0 + j + 1 < tend) issue(std::integral_constant<int, 1>{}, (t0 + j + 1) * BN);
        if (t0 + j < tend) tile(std::integral_constant<int, 0>{}, (t0 + j) * BN, j == 0);
        if (j + 1 >= nt0) break;
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (t0 + j + 2 < tend) issue(std::integral_constant<int, 0>{}, (t0 + j + 2) * BN);
        if (t0 + j + 1 < tend) tile(std::integral_constant<int, 1>{}, (t0 + j + 1) * BN, false);
    }

    if constexpr (KSP == 2) {
        // Group 1 leaves m, l and its accumulators in LDS (lane-contiguous per
        // wavefront) and ends; group 0 merges them into its own.
        constexpr int NF = NT * 16 + 2;
        static_assert(NW * NF * kWave * 4 <= KSP * 4 * TB, "merge fits the tile buffers");
        float* red = (float*)lds_all + wave * NF * kWave;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();                             // every wavefront is done with the tile buffers
        if (grp == 1) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) red[(nt * 16 + r) * kWave + lane] = oacc[nt][r];
            red[(NT * 16) * kWave + lane] = m_i;
            red[(NT * 16 + 1) * kWave + lane] = l_i;
        }
        __syncthreads();
        if (grp == 1) return;
        const float m1 = red[(NT * 16) * kWave + lane], l1 = red[(NT * 16 + 1) * kWave + lane];
        const float m = fmaxf(m_i, m1);
        const float c0 = __builtin_amdgcn_exp2f(m_i - m), c1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[nt][r] = oacc[nt][r] * c0 + red[(nt * 16 + r) * kWave + lane] * c1;
        l_i = l_i * c0 + l1 * c1;
    }

    if (qi >= Tq) return;
    const float inv = 1.0f / l_i;
    const int orow = b * Tq + qi;
    bf16* O = (bf16*)a.o + (size_t)orow * a.ldo + h * DH;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d0 = nt * 32 + 8 * g + 4 * half;
            if (d0 < DH) {
                bf16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (bf16)(oacc[nt][4 * g + e] * inv);
                // k-tiled output: 8 bytes at an 8-byte column offset stay inside one 64-byte tile row
                bf16* dst = a.o_tiled ? (bf16*)((char*)a.o + ktiled_off(orow, (size_t)2 * (h * DH + d0), (size_t)2 * a.ldo))
                                      : O + d0;
                *(bf16x4*)dst = o;
            }
        }
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
    if (a.Tq <= 0 || a.B <= 0) return hipSuccess;
    if (a.Tk <= 0) return hipErrorInvalidValue;
    if (a.dtype == LWO_BF16) {
        // d 64 / 72: four wavefronts per 128 queries leave one wavefront per SIMD
        // when there are at most as many query tiles as CUs; then the key tiles
        // are split over two groups of wavefronts (at least two tiles each).
        const long qtiles = (long)((a.Tq + 127) / 128) * a.H * a.B;
        const bool ksplit = qtiles <= 256 && a.Tk > 2 * 64;
        switch (a.dh) {
            case 64:
                if (ksplit) LWO_KL((k_attn_tr<64, 4, 2>), dim3((a.Tq + 127) / 128, a.H, a.B), 512, 0, st, a);
                else LWO_KL((k_attn_tr<64, 4>), dim3((a.Tq + 127) / 128, a.H, a.B), 256, 0, st, a);
                break;
            case 72:
                if (ksplit) LWO_KL((k_attn_tr<72, 4, 2>), dim3((a.Tq + 127) / 128, a.H, a.B), 512, 0, st, a);
                else LWO_KL((k_attn_tr<72, 4>), dim3((a.Tq + 127) / 128, a.H, a.B), 256, 0, st, a);
                break;
            case 128:
                // Few key tiles (cross-attention over a 512-token context): four
                // wavefronts, two workgroups per CU, so one workgroup's prologue
                // and epilogue overlap the other's tiles (32760 x 512: 0.55 ->
                // 0.51 ms); long key ranges keep eight wavefronts per workgroup.
                if (a.Tk <= 1024) LWO_KL((k_attn_tr<128, 4>), dim3((a.Tq + 127) / 128, a.H, a.B), 256, 0, st, a);
                else LWO_KL((k_attn_tr<128, 8>), dim3((a.Tq + 255) / 256, a.H, a.B), 512, 0, st, a);
                break;
            default: return hipErrorInvalidValue;
        }
    } else {
        return launch_attention_f32(a, st);
    }
    return hipGetLastError();
}

}  // namespace lwo
