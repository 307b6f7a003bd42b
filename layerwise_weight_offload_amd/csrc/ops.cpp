// Single-kernel entry points of the C ABI: argument validation, then the
// same launchers the denoise step uses.
#include "kernels.h"
#include "lwo_internal.h"

using namespace lwo;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

lwo_status bad(const std::string& m) {
    set_error(m);
    return LWO_EINVAL;
}

lwo_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) {
        set_error(std::string(what) + ": " + hipGetErrorString(e));
        return LWO_EHIP;
    }
    return LWO_OK;
}

}  // namespace

extern "C" lwo_status lwo_op_linear(int32_t dtype, int32_t epilogue, const void* a, const float* a_scale,
                                    const void* w, const float* w_scale, int32_t w_seg, const void* bias, int32_t M,
                                    int32_t N, int32_t K, void* out, int32_t ldo, float* xr, int32_t ldx,
                                    const float* gate, int32_t gate_ld, int32_t rows_per_gate, int32_t a_layout,
                                    int32_t out_layout, void* stream) {
    try {
        clear_error();
        if (dtype != LWO_F32 && dtype != LWO_BF16 && dtype != LWO_FP8_E4M3) return bad("linear: dtype");
        if (epilogue < EPI_STORE || epilogue > EPI_RESID) return bad("linear: epilogue");
        if (M < 0 || N < 1 || K < 1) return bad("linear: sizes");
        const int kq = dtype == LWO_F32 ? 16 : (dtype == LWO_BF16 ? 64 : 128);
        if (K % kq) return bad("linear: K must be a multiple of " + std::to_string(kq));
        if (N % 8) return bad("linear: N must be a multiple of 8");
        if (dtype != LWO_F32 && N % 64) return bad("linear: N must be a multiple of 64 (tiled bf16/fp8 weights)");
        if (!a || !w || !aligned16(a) || !aligned16(w)) return bad("linear: a and w must be 16-byte aligned device pointers");
        if (bias && ((uintptr_t)bias & 7u)) return bad("linear: bias must be 8-byte aligned");
        if (dtype == LWO_FP8_E4M3 && (!a_scale || !w_scale || w_seg < 1)) return bad("linear: fp8 needs a_scale, w_scale and w_seg");
        if (epilogue <= EPI_GELU) {
            if (!out || ldo < N || ldo % 8 || !aligned16(out)) return bad("linear: out (16-byte aligned) and ldo >= N, a multiple of 8, required");
        } else {
            if (!xr || ldx < N || ldx % 8 || !aligned16(xr)) return bad("linear: xr (16-byte aligned) and ldx >= N, a multiple of 8, required");
            if (epilogue == EPI_GATED && (!gate || gate_ld < N || gate_ld % 8 || rows_per_gate < 1 || !aligned16(gate)))
                return bad("linear: gate (16-byte aligned), gate_ld >= N (a multiple of 8) and rows_per_gate required");
        }
        if ((a_layout != LWO_ROWS && a_layout != LWO_KTILED) || (out_layout != LWO_ROWS && out_layout != LWO_KTILED))
            return bad("linear: a_layout and out_layout must be LWO_ROWS or LWO_KTILED");
        if (dtype == LWO_F32 && (a_layout || out_layout)) return bad("linear: k-tiled operands need BF16 or FP8");
        if (out_layout && (epilogue > EPI_GELU || ldo % 32))
            return bad("linear: a k-tiled out needs epilogue 0 or 1 and ldo a multiple of 32");
        if (!stream) return bad("linear: stream is NULL");
        GemmArgs g{};
        g.a = a; g.w = w; g.M = M; g.N = N; g.K = K; g.dtype = dtype;
        g.act_dtype = dtype == LWO_F32 ? LWO_F32 : LWO_BF16;
        g.epi = epilogue; g.bias = bias; g.out = out; g.ldo = ldo; g.xr = xr; g.ldx = ldx;
        g.gate = gate; g.gate_ld = gate_ld; g.rows_per_batch = rows_per_gate > 0 ? rows_per_gate : 1;
        g.w_scale = w_scale; g.w_seg = w_seg > 0 ? w_seg : 1; g.a_scale = a_scale;
        g.a_tiled = a_layout; g.out_tiled = out_layout;
        return launched(launch_gemm(g, (hipStream_t)stream), "linear");
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_op_linear");
    } catch (const std::exception& e) {
        return fail_exception("lwo_op_linear", e.what());
    } catch (...) {
        return fail_exception("lwo_op_linear", "unknown exception");
    }
}

extern "C" lwo_status lwo_op_attention(int32_t dtype, const void* q, int32_t ldq, const void* k, int32_t ldk,
                                       const void* v, int32_t ldv, void* o, int32_t ldo, int32_t batch, int32_t heads,
                                       int32_t tq, int32_t tk, int32_t head_dim, int32_t o_layout, void* stream) {
    try {
        clear_error();
        if (dtype != LWO_F32 && dtype != LWO_BF16) return bad("attention: dtype must be F32 or BF16");
        if (head_dim != 64 && head_dim != 72 && head_dim != 128) return bad("attention: head_dim must be 64, 72 or 128");
        if (batch < 1 || heads < 1 || tq < 0 || tk < 1) return bad("attention: sizes");
        const int D = heads * head_dim;
        if (ldq < D || ldk < D || ldv < D || ldo < D) return bad("attention: leading dimensions must cover heads*head_dim");
        if (ldq % 8 || ldk % 8 || ldv % 8 || ldo % 8) return bad("attention: leading dimensions must be multiples of 8");
        if (!q || !k || !v || !o || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
            return bad("attention: pointers must be 16-byte aligned device pointers");
        if (o_layout != LWO_ROWS && o_layout != LWO_KTILED) return bad("attention: o_layout must be LWO_ROWS or LWO_KTILED");
        if (o_layout && (dtype != LWO_BF16 || ldo % 32)) return bad("attention: a k-tiled o needs BF16 and ldo a multiple of 32");
        if (!stream) return bad("attention: stream is NULL");
        AttnArgs a{};
        a.q = q; a.ldq = ldq; a.k = k; a.ldk = ldk; a.v = v; a.ldv = ldv; a.o = o; a.ldo = ldo;
        a.B = batch; a.H = heads; a.Tq = tq; a.Tk = tk; a.dh = head_dim; a.dtype = dtype; a.o_tiled = o_layout;
        return launched(launch_attention(a, (hipStream_t)stream), "attention");
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_op_attention");
    } catch (const std::exception& e) {
        return fail_exception("lwo_op_attention", e.what());
    } catch (...) {
        return fail_exception("lwo_op_attention", "unknown exception");
    }
}

extern "C" lwo_status lwo_op_layernorm(const float* x, int32_t M, int32_t D, int32_t rows_per_batch, const float* mod,
                                       int32_t shift_chunk, int32_t scale_chunk, void* out, int32_t out_dtype,
                                       float* out_scale, int32_t out_layout, void* stream) {
    try {
        clear_error();
        if (M < 0 || D < 4 || D % 4 || D > 8192) return bad("layernorm: D must be a multiple of 4 and at most 8192");
        if (out_dtype != LWO_F32 && out_dtype != LWO_BF16 && out_dtype != LWO_FP8_E4M3) return bad("layernorm: out_dtype");
        if (!x || !out || !aligned16(x) || !aligned16(out)) return bad("layernorm: x and out must be 16-byte aligned");
        if (mod && (rows_per_batch < 1 || shift_chunk < 0 || shift_chunk > 5 || scale_chunk < 0 || scale_chunk > 5 || !aligned16(mod)))
            return bad("layernorm: modulation arguments");
        if (out_dtype == LWO_FP8_E4M3 && !out_scale) return bad("layernorm: fp8 output needs out_scale");
        if (out_layout != LWO_ROWS && out_layout != LWO_KTILED) return bad("layernorm: out_layout must be LWO_ROWS or LWO_KTILED");
        if (out_layout && (out_dtype == LWO_F32 || (D * (out_dtype == LWO_BF16 ? 2 : 1)) % 64))
            return bad("layernorm: a k-tiled out needs BF16 or FP8 rows of a multiple of 64 bytes");
        if (!stream) return bad("layernorm: stream is NULL");
        return launched(launch_ln(x, M, D, rows_per_batch > 0 ? rows_per_batch : 1, mod, shift_chunk, scale_chunk, out,
                                  out_dtype, out_scale, out_layout, (hipStream_t)stream), "layernorm");
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_op_layernorm");
    } catch (const std::exception& e) {
        return fail_exception("lwo_op_layernorm", e.what());
    } catch (...) {
        return fail_exception("lwo_op_layernorm", "unknown exception");
    }
}

extern "C" lwo_status lwo_op_quantize_rows(const void* in, int32_t M, int32_t N, uint8_t* codes, float* scales,
                                           int32_t codes_layout, void* stream) {
    try {
        clear_error();
        if (M < 0 || N < 8 || N % 8) return bad("quantize_rows: N must be a positive multiple of 8");
        if (!in || !codes || !scales || !aligned16(in) || ((uintptr_t)codes & 7u)) return bad("quantize_rows: pointers");
        if (codes_layout != LWO_ROWS && codes_layout != LWO_KTILED)
            return bad("quantize_rows: codes_layout must be LWO_ROWS or LWO_KTILED");
        if (codes_layout && N % 64) return bad("quantize_rows: k-tiled codes need N a multiple of 64");
        if (!stream) return bad("quantize_rows: stream is NULL");
        return launched(launch_quant_rows(in, M, N, codes, scales, codes_layout, (hipStream_t)stream), "quantize_rows");
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_op_quantize_rows");
    } catch (const std::exception& e) {
        return fail_exception("lwo_op_quantize_rows", e.what());
    } catch (...) {
        return fail_exception("lwo_op_quantize_rows", "unknown exception");
    }
}

extern "C" lwo_status lwo_op_rmsnorm_qk(int32_t dtype, void* qkv, int32_t M, int32_t D, const void* gq, const void* gk,
                                        void* stream) {
    try {
        clear_error();
        if (dtype != LWO_F32 && dtype != LWO_BF16) return bad("rmsnorm_qk: dtype");
        if (M < 0 || D < 4 || D % 4 || D > 8192) return bad("rmsnorm_qk: D must be a multiple of 4 and at most 8192");
        if (!qkv || !gq || !gk || !aligned16(qkv) || !aligned16(gq) || !aligned16(gk)) return bad("rmsnorm_qk: pointers");
        if (!stream) return bad("rmsnorm_qk: stream is NULL");
        return launched(launch_rmsnorm_qk(qkv, dtype, M, D, gq, gk, (hipStream_t)stream), "rmsnorm_qk");
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_op_rmsnorm_qk");
    } catch (const std::exception& e) {
        return fail_exception("lwo_op_rmsnorm_qk", e.what());
    } catch (...) {
        return fail_exception("lwo_op_rmsnorm_qk", "unknown exception");
    }
}

extern "C" lwo_status lwo_probe_mfma(int32_t dtype, int32_t blocks, int32_t iters, float* sink, uint64_t sink_floats,
                                     void* stream, double* flops) {
    try {
        clear_error();
        if (dtype != LWO_BF16 && dtype != LWO_FP8_E4M3) return bad("probe_mfma: dtype must be BF16 or FP8_E4M3");
        if (blocks < 1 || blocks > 65536 || iters < 1 || iters > 1000000) return bad("probe_mfma: blocks or iters out of range");
        if (!sink || ((uintptr_t)sink & 3u) || sink_floats < (uint64_t)blocks * 256) return bad("probe_mfma: sink");
        if (!stream) return bad("probe_mfma: stream is NULL");
        if (flops) *flops = (double)blocks * 4 /* wavefronts */ * 4.0 * iters * (dtype == LWO_BF16 ? 32768.0 : 131072.0);
        return launched(launch_mfma_peak(dtype == LWO_FP8_E4M3, blocks, iters, sink, (hipStream_t)stream), "probe_mfma");
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_probe_mfma");
    } catch (const std::exception& e) {
        return fail_exception("lwo_probe_mfma", e.what());
    } catch (...) {
        return fail_exception("lwo_probe_mfma", "unknown exception");
    }
}
