// One DiT block's forward as a sequence of kernel launches on the compute
// stream, reading weights through zero-copy views into a slot (or the
// resident region): every parameter is `slot base + layout offset`, so the
// weights are never repacked on the device ("Distributed Layerwise Offload",
// "Registered runtime-cache transfer": parameters are views at offsets of one
// flat device buffer).
//
// The residual stream stays in fp32 for the whole step; LayerNorm outputs,
// projections and attention outputs are in the activation dtype (or e4m3
// codes with per-row scales when the linears are fp8).
#include <algorithm>
#include <cstdio>

#include "kernels.h"
#include "lwo_internal.h"

namespace lwo {

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Lay the workspace out from `base` (nullptr: only size it); returns its bytes.
size_t workspace_carve(const lwo_model_desc& d, void* base, Workspace* ws) {
    const size_t M = (size_t)d.batch * d.tokens, D = d.hidden, F = d.ffn;
    const size_t Mp = (M + 63) / 64 * 64;   // buffers that may hold k-tiled rows span whole 64-row bands
    const size_t Mc = (size_t)d.batch * d.ctx_tokens;
    const size_t ae = dtype_bytes(d.act_dtype);
    const bool video = d.kind == LWO_KIND_VIDEO, fp8 = d.linear_dtype == LWO_FP8_E4M3;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const size_t o_xr = take(M * D * 4), o_mod = take((size_t)d.batch * 6 * D * 4), o_h = take(Mp * D * ae);
    const size_t o_silu = video ? 0 : take((size_t)d.batch * D * 4);
    const size_t o_big = take(Mp * std::max(3 * D, F) * ae), o_attn = take(Mp * D * ae);
    const size_t o_cq = video ? take(M * D * ae) : 0, o_ckv = video ? take(Mc * 2 * D * ae) : 0;
    const size_t o_q8 = fp8 ? take(Mp * std::max(D, F)) : 0, o_q8s = fp8 ? take(std::max(M, Mc) * 4) : 0;
    const size_t o_c8 = fp8 ? take(Mc * D) : 0, o_c8s = fp8 ? take(Mc * 4) : 0;
    const size_t o_sums = take(16);
    if (!base) return off;
    char* b = (char*)base;
    ws->base = base;
    ws->bytes = off;
    ws->xr = (float*)(b + o_xr);
    ws->mod = (float*)(b + o_mod);
    ws->silu_cond = video ? nullptr : (float*)(b + o_silu);
    ws->h = b + o_h;
    ws->big = b + o_big;
    ws->attn = b + o_attn;
    ws->cq = video ? b + o_cq : nullptr;
    ws->ckv = video ? b + o_ckv : nullptr;
    ws->q8 = fp8 ? (uint8_t*)(b + o_q8) : nullptr;
    ws->q8_scale = fp8 ? (float*)(b + o_q8s) : nullptr;
    ws->ctx8 = fp8 ? (uint8_t*)(b + o_c8) : nullptr;
    ws->ctx8_scale = fp8 ? (float*)(b + o_c8s) : nullptr;
    ws->sums = (uint64_t*)(b + o_sums);
    return off;
}

lwo_status workspace_alloc(const lwo_model_desc& d, Workspace* ws) {
    const size_t bytes = workspace_carve(d, nullptr, nullptr);
    void* base = nullptr;
    if (hipMalloc(&base, bytes) != hipSuccess) {
        set_error("hipMalloc of the activation workspace (" + std::to_string(bytes) + " bytes) failed");
        return LWO_ENOMEM;
    }
    workspace_carve(d, base, ws);
    LWO_HIP_TRY(hipMemset(ws->sums, 0, 16));
    return LWO_OK;
}

void workspace_free(Workspace* ws) {
    if (ws->base) (void)hipFree(ws->base);
    *ws = Workspace();
}

// ------------------------------------------------------------------ kernel timing

LaunchEvents& launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}

hipEvent_t KernelTimer::get() {
    hipEvent_t e = nullptr;
    if (!pool.empty()) { e = pool.back(); pool.pop_back(); return e; }
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

int KernelTimer::cls(const char* name) {
    for (size_t i = 0; i < agg.size(); ++i)
        if (agg[i].name == name) return (int)i;
    agg.push_back(Agg());
    agg.back().name = name;
    return (int)agg.size() - 1;
}

lwo_status KernelTimer::collect() {
    for (Rec& r : pending) {
        LWO_HIP_TRY(hipEventSynchronize(r.b));
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {   // the operation launched nothing (empty shape)
            (void)hipGetLastError();
            pool.push_back(r.a);
            pool.push_back(r.b);
            continue;
        }
        Agg& a = agg[r.cls];
        a.launches++;
        a.ms += ms;
        a.flops += r.flops;
        a.bytes += r.bytes;
        pool.push_back(r.a);
        pool.push_back(r.b);
    }
    pending.clear();
    return LWO_OK;
}

void KernelTimer::reset() {
    for (Rec& r : pending) { pool.push_back(r.a); pool.push_back(r.b); }
    pending.clear();
    agg.clear();
}

void KernelTimer::destroy() {
    reset();
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
    pool.clear();
}

#define LWO_LAUNCH(expr)                                                                  \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess) {                                                           \
            set_error(std::string("kernel launch failed: ") + #expr + ": " + hipGetErrorString(e_)); \
            return LWO_EHIP;                                                              \
        }                                                                                 \
    } while (0)

lwo_status enqueue_step_begin(const lwo_model_desc& d, const Workspace& ws, const void* x, const void* cond,
                              const void* ctx, hipStream_t st) {
    const size_t n = (size_t)d.batch * d.tokens * d.hidden;
    LWO_LAUNCH(launch_to_f32(x, d.act_dtype, ws.xr, n, st));
    if (d.kind == LWO_KIND_DIT)   // SiLU(cond) feeds the adaLN linear of every block: once per step
        LWO_LAUNCH(launch_silu(cond, d.act_dtype, ws.silu_cond, d.batch * d.hidden, st));
    if (d.linear_dtype == LWO_FP8_E4M3)   // the context feeds the cross K/V linears of every block: quantise once
        LWO_LAUNCH(launch_quant_rows(ctx, d.batch * d.ctx_tokens, d.hidden, ws.ctx8, ws.ctx8_scale, 0, st));
    return LWO_OK;
}

lwo_status enqueue_step_end(const lwo_model_desc& d, const Workspace& ws, void* x, hipStream_t st) {
    const size_t n = (size_t)d.batch * d.tokens * d.hidden;
    LWO_LAUNCH(launch_from_f32(ws.xr, x, d.act_dtype, n, st));
    return LWO_OK;
}

static GemmArgs gemm_args(const lwo_model_desc& d, const void* a, const void* w, int M, int N, int K, int epi,
                          const void* bias) {
    GemmArgs g{};
    g.a = a; g.w = w; g.M = M; g.N = N; g.K = K;
    g.dtype = d.linear_dtype;
    g.act_dtype = d.act_dtype;
    g.epi = epi;
    g.bias = bias;
    g.rows_per_batch = d.tokens;
    // The block's own activations reach the MFMA linears k-tiled (the caller's context rows are the exception).
    g.a_tiled = d.linear_dtype != LWO_F32;
    return g;
}

lwo_status enqueue_block(const lwo_model_desc& d, const BlockPtrs& p, const Workspace& ws, const void* cond,
                         const void* ctx, hipStream_t st, KernelTimer* kt) {
    const int B = d.batch, T = d.tokens, D = d.hidden, F = d.ffn, H = d.heads, dh = D / H;
    const int M = B * T, Mc = B * d.ctx_tokens;
    const int act = d.act_dtype, ae = dtype_bytes(act);
    const bool fp8 = d.linear_dtype == LWO_FP8_E4M3;
    // Activations that feed an MFMA linear are written k-tiled by their producer:
    // LayerNorm, and with bf16 linears the attention output and the GELU output
    // (with fp8 linears those two stay row-major for the row quantiser, which
    // writes the codes k-tiled).
    const int tl = d.linear_dtype != LWO_F32, tl16 = tl && !fp8;
    const int h_dt = fp8 ? LWO_FP8_E4M3 : act;      // LayerNorm output dtype feeding a linear
    void* h_buf = fp8 ? (void*)ws.q8 : ws.h;
    char* big = (char*)ws.big;
    const float* mod = ws.mod;
    const float* wsc = p.w_scale;

    // fp8: one weight scale per tensor.  The fused QKV (and cross K|V) GEMMs
    // span several tensors, one per D output columns; the others span one.
    auto fp8_in = [&](GemmArgs& g, int scale_idx, const float* a_scale, bool fused) {
        if (!fp8) return;
        g.w_scale = wsc + scale_idx;
        g.w_seg = fused ? D : g.N;
        g.a_scale = a_scale;
    };
    // Timing wrapper: the one kernel `launch` enqueues records its own start and
    // end into two events, attributed to the kernel class `name`.
    auto timed = [&](const char* name, double flops, double bytes, auto&& launch) -> hipError_t {
        if (!kt || !kt->on) return launch();
        KernelTimer::Rec r{kt->cls(name), kt->get(), kt->get(), flops, bytes};
        if (!r.a || !r.b) return hipErrorOutOfMemory;
        launch_events() = LaunchEvents{r.a, r.b};
        const hipError_t e = launch();
        launch_events() = LaunchEvents{};
        kt->pending.push_back(r);
        return e;
    };
    const char* dtn = act == LWO_F32 ? "f32" : (fp8 ? "fp8" : "bf16");
    // One timing class per call site (the product and its epilogue), so that a
    // class's launches all have one shape.
    auto gemm = [&](const char* site, const GemmArgs& g) {
        static const char* epn[] = {"store", "gelu", "gated", "resid"};
        char name[48];
        snprintf(name, sizeof(name), "gemm_%s_%s_%s", dtn, site, epn[g.epi]);
        const double ea = dtype_bytes(g.dtype), eo = g.epi <= EPI_GELU ? ae : 8.0;
        const double bytes = (double)g.M * g.K * ea + (double)g.N * g.K * ea + (double)g.M * g.N * eo;
        return timed(name, 2.0 * g.M * g.N * g.K, bytes, [&] { return launch_gemm(g, st); });
    };
    auto attn = [&](const char* site, const void* q, int ldq, const void* k, const void* v, int ldkv, int Tk) {
        AttnArgs a{};
        a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldkv; a.v = v; a.ldv = ldkv;
        a.o = ws.attn; a.ldo = D; a.o_tiled = tl16;
        a.B = B; a.H = H; a.Tq = T; a.Tk = Tk; a.dh = dh; a.dtype = act;
        char name[48];
        snprintf(name, sizeof(name), "attn_%s_%s_d%d", site, act == LWO_F32 ? "f32" : "bf16", dh);
        const double flops = 4.0 * B * H * (double)T * Tk * dh;
        const double bytes = (double)B * ((double)T * D * 2 + 2.0 * Tk * D) * ae;
        return timed(name, flops, bytes, [&] { return launch_attention(a, st); });
    };
    auto ln = [&](const float* m, int shc, int scc, void* out, int out_dt, float* osc) {
        const double bytes = (double)M * D * (4 + dtype_bytes(out_dt)) + (m ? 2.0 * B * D * 4 : 0.0);
        return timed(m ? "layernorm_mod" : "layernorm", 0.0, bytes,
                     [&] { return launch_ln(ws.xr, M, D, T, m, shc, scc, out, out_dt, osc, tl, st); });
    };
    auto quant = [&](const void* in, int rows, int n, uint8_t* codes, float* sc) {
        return timed("quant_rows_fp8", 0.0, (double)rows * n * 3,
                     [&] { return launch_quant_rows(in, rows, n, codes, sc, tl, st); });
    };

    if (d.kind == LWO_KIND_DIT) {
        LWO_LAUNCH(timed("adaln_modulation", 2.0 * B * 6 * D * D, 6.0 * D * D * ae,
                         [&] { return launch_mod_dit(ws.silu_cond, p.ada_w, p.ada_b, act, ws.mod, B, D, st); }));
        LWO_LAUNCH(ln(mod, 0, 1, ws.h, act, nullptr));
        GemmArgs g = gemm_args(d, ws.h, p.q_w, M, 3 * D, D, EPI_STORE, p.qkv_b);
        g.out = big; g.ldo = 3 * D;
        LWO_LAUNCH(gemm("qkv", g));
        LWO_LAUNCH(attn("self", big, 3 * D, big + (size_t)D * ae, big + (size_t)2 * D * ae, 3 * D, T));
        g = gemm_args(d, ws.attn, p.o_w, M, D, D, EPI_GATED, p.o_b);
        g.xr = ws.xr; g.ldx = D; g.gate = mod + 2 * D; g.gate_ld = 6 * D;
        LWO_LAUNCH(gemm("o", g));
        LWO_LAUNCH(ln(mod, 3, 4, ws.h, act, nullptr));
        g = gemm_args(d, ws.h, p.fc1_w, M, F, D, EPI_GELU, p.fc1_b);
        g.out = big; g.ldo = F; g.out_tiled = tl16;
        LWO_LAUNCH(gemm("fc1", g));
        g = gemm_args(d, big, p.fc2_w, M, D, F, EPI_GATED, p.fc2_b);
        g.xr = ws.xr; g.ldx = D; g.gate = mod + 5 * D; g.gate_ld = 6 * D;
        LWO_LAUNCH(gemm("fc2", g));
        return LWO_OK;
    }

    // video kind
    LWO_LAUNCH(timed("modulation_add", 6.0 * B * D, 6.0 * B * D * (2 * ae + 4),
                     [&] { return launch_mod_video(cond, p.mod_table, act, ws.mod, B, D, st); }));
    LWO_LAUNCH(ln(mod, 0, 1, h_buf, h_dt, ws.q8_scale));
    GemmArgs g = gemm_args(d, h_buf, p.q_w, M, 3 * D, D, EPI_STORE, p.qkv_b);
    g.out = big; g.ldo = 3 * D;
    fp8_in(g, 0, ws.q8_scale, true);
    LWO_LAUNCH(gemm("qkv", g));
    LWO_LAUNCH(timed("rmsnorm_qk", 0.0, 4.0 * M * D * ae,
                     [&] { return launch_rmsnorm_qk(big, act, M, D, p.q_norm, p.k_norm, st); }));
    LWO_LAUNCH(attn("self", big, 3 * D, big + (size_t)D * ae, big + (size_t)2 * D * ae, 3 * D, T));
    const void* a_in = ws.attn;
    if (fp8) { LWO_LAUNCH(quant(ws.attn, M, D, ws.q8, ws.q8_scale)); a_in = ws.q8; }
    g = gemm_args(d, a_in, p.o_w, M, D, D, EPI_GATED, p.o_b);
    g.xr = ws.xr; g.ldx = D; g.gate = mod + 2 * D; g.gate_ld = 6 * D;
    fp8_in(g, 3, ws.q8_scale, false);
    LWO_LAUNCH(gemm("o", g));

    // cross-attention: ungated, plain LayerNorm on the queries, keys/values from the context
    LWO_LAUNCH(ln(nullptr, 0, 0, h_buf, h_dt, ws.q8_scale));
    g = gemm_args(d, h_buf, p.cq_w, M, D, D, EPI_STORE, p.cq_b);
    g.out = ws.cq; g.ldo = D;
    fp8_in(g, 4, ws.q8_scale, false);
    LWO_LAUNCH(gemm("cq", g));
    g = gemm_args(d, fp8 ? (const void*)ws.ctx8 : ctx, p.ck_w, Mc, 2 * D, D, EPI_STORE, p.ckv_b);
    g.out = ws.ckv; g.ldo = 2 * D; g.a_tiled = 0;
    fp8_in(g, 5, ws.ctx8_scale, true);
    LWO_LAUNCH(gemm("ckv", g));
    const char* ckv = (const char*)ws.ckv;
    LWO_LAUNCH(attn("cross", ws.cq, D, ckv, ckv + (size_t)D * ae, 2 * D, d.ctx_tokens));
    a_in = ws.attn;
    if (fp8) { LWO_LAUNCH(quant(ws.attn, M, D, ws.q8, ws.q8_scale)); a_in = ws.q8; }
    g = gemm_args(d, a_in, p.co_w, M, D, D, EPI_RESID, p.co_b);
    g.xr = ws.xr; g.ldx = D;
    fp8_in(g, 7, ws.q8_scale, false);
    LWO_LAUNCH(gemm("co", g));

    // FFN
    LWO_LAUNCH(ln(mod, 3, 4, h_buf, h_dt, ws.q8_scale));
    g = gemm_args(d, h_buf, p.fc1_w, M, F, D, EPI_GELU, p.fc1_b);
    g.out = big; g.ldo = F; g.out_tiled = tl16;
    fp8_in(g, 8, ws.q8_scale, false);
    LWO_LAUNCH(gemm("fc1", g));
    a_in = big;
    if (fp8) { LWO_LAUNCH(quant(big, M, F, ws.q8, ws.q8_scale)); a_in = ws.q8; }
    g = gemm_args(d, a_in, p.fc2_w, M, D, F, EPI_GATED, p.fc2_b);
    g.xr = ws.xr; g.ldx = D; g.gate = mod + 5 * D; g.gate_ld = 6 * D;
    fp8_in(g, 9, ws.q8_scale, false);
    LWO_LAUNCH(gemm("fc2", g));
    return LWO_OK;
}

lwo_status enqueue_checksum(const void* dev, uint64_t bytes, uint64_t* acc, hipStream_t st) {
    LWO_LAUNCH(launch_checksum(dev, bytes, acc, st));
    return LWO_OK;
}

lwo_status enqueue_checksum_compare(uint64_t* acc, uint64_t expect, hipStream_t st) {
    LWO_LAUNCH(launch_checksum_compare(acc, expect, st));
    return LWO_OK;
}

lwo_status enqueue_zero_u64(uint64_t* p, int n, hipStream_t st) {
    LWO_LAUNCH(launch_zero_u64(p, n, st));
    return LWO_OK;
}

}  // namespace lwo
