// Block layout, host packing codecs, host checksum and descriptor checks.
//
// The flat per-block extent follows the offload design of keeping each
// block's parameters as flattened pinned host tensors ("CPU Offloading for
// Diffusion Models", "Layerwise (Blockwise) Offloading / How It Works") and
// of placing every parameter at an offset of one flat buffer ("Distributed
// Layerwise Offload", "Registered runtime-cache transfer").  Per-tensor fp8
// weights carry one float32 scale each, finalised before offload
// ("Distributed Layerwise Offload", "Feature compatibility").
#include <cmath>
#include <cstring>
#include <mutex>

#include "lwo_internal.h"

namespace lwo {

// ------------------------------------------------------------------ errors

static thread_local std::string g_err;

void set_error(const std::string& msg) { g_err = msg; }
void clear_error() { g_err.clear(); }

// No C++ exception crosses the C ABI: every entry point catches what its
// body throws and reports it through these (which themselves never throw).
lwo_status fail_alloc(const char* where) noexcept {
    try {
        g_err = std::string(where) + ": out of host memory";
    } catch (...) {
        g_err.clear();
    }
    return LWO_ENOMEM;
}

lwo_status fail_exception(const char* where, const char* what) noexcept {
    try {
        g_err = std::string(where) + ": " + what;
    } catch (...) {
        g_err.clear();
    }
    return LWO_EIO;
}

int dtype_bytes(int dt) { return dt == LWO_F32 ? 4 : dt == LWO_BF16 ? 2 : 1; }

int Layout::find(const char* name) const {
    for (size_t i = 0; i < tensors.size(); ++i)
        if (tensors[i].name == name) return (int)i;
    return -1;
}

lwo_status validate_desc(const lwo_model_desc* d) {
    if (!d) { set_error("desc is NULL"); return LWO_EINVAL; }
    auto bad = [](const char* m) { set_error(std::string("invalid model desc: ") + m); return LWO_EINVAL; };
    if (d->kind != LWO_KIND_DIT && d->kind != LWO_KIND_VIDEO) return bad("kind");
    if (d->n_blocks < 1 || d->n_blocks > 100000) return bad("n_blocks");
    if (d->heads < 1 || d->hidden < 1 || d->hidden % d->heads) return bad("hidden must be heads * head_dim");
    int hd = d->hidden / d->heads;
    if (hd != 64 && hd != 72 && hd != 128) return bad("head dim must be 64, 72 or 128");
    if (d->ffn < 1) return bad("ffn");
    if (d->batch < 1 || d->tokens < 1) return bad("batch/tokens");
    if ((int64_t)d->batch * d->tokens > (int64_t)1 << 26) return bad("batch*tokens too large");
    if (d->kind == LWO_KIND_VIDEO && d->ctx_tokens < 1) return bad("video kind needs ctx_tokens >= 1");
    if (d->kind == LWO_KIND_DIT && d->ctx_tokens != 0) return bad("DiT kind has no context (ctx_tokens = 0)");
    if (d->act_dtype != LWO_F32 && d->act_dtype != LWO_BF16) return bad("act_dtype must be F32 or BF16");
    if (d->linear_dtype == LWO_FP8_E4M3) {
        if (d->act_dtype != LWO_BF16 || d->kind != LWO_KIND_VIDEO) return bad("fp8 linears need the video kind with bf16 activations");
        if (d->hidden % 128 || d->ffn % 128) return bad("fp8 linears need hidden and ffn multiples of 128");
    } else if (d->linear_dtype != d->act_dtype) {
        return bad("linear_dtype must equal act_dtype or be FP8_E4M3");
    }
    if (d->hidden % 64 || d->ffn % 64) return bad("hidden and ffn must be multiples of 64");
    if (d->hidden > 8192) return bad("hidden above 8192 is not supported by the row kernels");
    return LWO_OK;
}

static void add(Layout& L, uint64_t& off, const char* name, int r0, int r1, int dtype) {
    TensorSlot t;
    t.name = name;
    off = (off + kTensorAlign - 1) / kTensorAlign * kTensorAlign;
    t.offset = off;
    t.rank = r1 ? 2 : 1;
    t.shape[0] = r0;
    t.shape[1] = r1;
    t.dtype = dtype;
    t.bytes = (uint64_t)r0 * (uint64_t)(r1 ? r1 : 1) * (uint64_t)dtype_bytes(dtype);
    // GEMM weights in bf16/fp8 are stored in the order the GEMM reads them;
    // the DiT modulation matrix is read by a GEMV and stays row-major.
    const size_t len = std::strlen(name);
    t.tiled = len > 2 && std::strcmp(name + len - 2, ".w") == 0 && dtype != LWO_F32 && std::strcmp(name, "ada.w") != 0;
    off += t.bytes;
    L.tensors.push_back(t);
}

Layout make_layout(const lwo_model_desc& d) {
    Layout L;
    uint64_t off = 0;
    const int D = d.hidden, F = d.ffn, a = d.act_dtype, w = d.linear_dtype;
    if (d.kind == LWO_KIND_DIT) {
        add(L, off, "ada.w", 6 * D, D, w);
        add(L, off, "ada.b", 6 * D, 0, a);
        add(L, off, "attn.q.w", D, D, w);
        add(L, off, "attn.k.w", D, D, w);
        add(L, off, "attn.v.w", D, D, w);
        add(L, off, "attn.qkv.b", 3 * D, 0, a);
        add(L, off, "attn.o.w", D, D, w);
        add(L, off, "attn.o.b", D, 0, a);
        add(L, off, "ffn.fc1.w", F, D, w);
        add(L, off, "ffn.fc1.b", F, 0, a);
        add(L, off, "ffn.fc2.w", D, F, w);
        add(L, off, "ffn.fc2.b", D, 0, a);
    } else {
        add(L, off, "mod.table", 6, D, a);
        add(L, off, "attn.q.w", D, D, w);
        add(L, off, "attn.k.w", D, D, w);
        add(L, off, "attn.v.w", D, D, w);
        add(L, off, "attn.qkv.b", 3 * D, 0, a);
        add(L, off, "attn.q.norm", D, 0, a);
        add(L, off, "attn.k.norm", D, 0, a);
        add(L, off, "attn.o.w", D, D, w);
        add(L, off, "attn.o.b", D, 0, a);
        add(L, off, "cross.q.w", D, D, w);
        add(L, off, "cross.q.b", D, 0, a);
        add(L, off, "cross.k.w", D, D, w);
        add(L, off, "cross.v.w", D, D, w);
        add(L, off, "cross.kv.b", 2 * D, 0, a);
        add(L, off, "cross.o.w", D, D, w);
        add(L, off, "cross.o.b", D, 0, a);
        add(L, off, "ffn.fc1.w", F, D, w);
        add(L, off, "ffn.fc1.b", F, 0, a);
        add(L, off, "ffn.fc2.w", D, F, w);
        add(L, off, "ffn.fc2.b", D, 0, a);
        if (w == LWO_FP8_E4M3) add(L, off, "linear.scales", 10, 0, LWO_F32);
    }
    L.extent_bytes = (off + kExtentAlign - 1) / kExtentAlign * kExtentAlign;
    return L;
}

BlockPtrs block_ptrs(const Layout& L, const lwo_model_desc& d, const char* base) {
    BlockPtrs p;
    std::memset(&p, 0, sizeof(p));
    auto at = [&](const char* n) -> const void* {
        int i = L.find(n);
        return i < 0 ? nullptr : (const void*)(base + L.tensors[i].offset);
    };
    p.q_w = at("attn.q.w"); p.k_w = at("attn.k.w"); p.v_w = at("attn.v.w"); p.qkv_b = at("attn.qkv.b");
    p.o_w = at("attn.o.w"); p.o_b = at("attn.o.b");
    p.fc1_w = at("ffn.fc1.w"); p.fc1_b = at("ffn.fc1.b"); p.fc2_w = at("ffn.fc2.w"); p.fc2_b = at("ffn.fc2.b");
    if (d.kind == LWO_KIND_DIT) {
        p.ada_w = at("ada.w"); p.ada_b = at("ada.b");
    } else {
        p.mod_table = at("mod.table"); p.q_norm = at("attn.q.norm"); p.k_norm = at("attn.k.norm");
        p.cq_w = at("cross.q.w"); p.cq_b = at("cross.q.b"); p.ck_w = at("cross.k.w"); p.cv_w = at("cross.v.w");
        p.ckv_b = at("cross.kv.b"); p.co_w = at("cross.o.w"); p.co_b = at("cross.o.b");
        p.w_scale = (const float*)at("linear.scales");
    }
    return p;
}

// ------------------------------------------------------------------ tiled weights

// Byte (n, c) of a row-major [N, R bytes] matrix goes to tile (n / 64, c / 64)
// at ((n / 64) * (R / 64) + c / 64) * 4096, row n % 64, byte c % 64 of the
// tile: each tile row is 64 consecutive bytes of the source row.
void tile_rows(const unsigned char* src, int N, uint64_t R, unsigned char* dst) {
    const uint64_t tiles_per_band = R / 64;
    for (int n = 0; n < N; ++n) {
        const unsigned char* row = src + (uint64_t)n * R;
        unsigned char* band = dst + (uint64_t)(n / 64) * tiles_per_band * 4096 + (uint64_t)(n % 64) * 64;
        for (uint64_t t = 0; t < tiles_per_band; ++t) std::memcpy(band + t * 4096, row + t * 64, 64);
    }
}

// ------------------------------------------------------------------ codecs

static inline uint32_t f2u(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = f2u(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))   // NaN -> quiet NaN, sign kept
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);
    u += 0x7FFFu + ((u >> 16) & 1u);                              // round half to even on bit 16
    return (uint16_t)(u >> 16);
}

// OCP E4M3 ("FN"): bias 7, 3 mantissa bits, max 448, no infinities.
uint8_t f32_to_e4m3_rne_sat(float f) {
    uint32_t u = f2u(f);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    if (std::isnan(f)) return 0x7F;
    float a = std::fabs(f);
    if (a >= 448.0f) return sign | 0x7E;
    if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
        int m = (int)std::nearbyintf(a * 512.0f);   // exact scaling, then round half to even
        return sign | (uint8_t)m;              // m == 8 is the smallest normal, code 0x08
    }
    int e = (int)((u >> 23) & 0xFFu) - 127;     // -6 .. 8
    uint32_t mant = u & 0x7FFFFFu;
    uint32_t keep = mant >> 20, rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) {
        if (++keep == 8u) { keep = 0; ++e; }
    }
    if (e > 8 || (e == 8 && keep == 7u)) return sign | 0x7E;
    return sign | (uint8_t)(((e + 7) << 3) | (int)keep);
}

static inline uint64_t splitmix64_next(uint64_t s) {
    uint64_t z = s + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t extent_checksum_host(const void* p, uint64_t bytes) {
    const unsigned char* c = (const unsigned char*)p;
    uint64_t n = bytes / 8, acc = 0;
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t w;
        std::memcpy(&w, c + 8 * i, 8);
        acc += splitmix64_next(w ^ (i * 0x9E3779B97F4A7C15ull));
    }
    return acc;
}

}  // namespace lwo

using namespace lwo;

extern "C" lwo_status lwo_block_layout(const lwo_model_desc* desc, lwo_tensor_info* out, int32_t cap,
                                       int32_t* n, uint64_t* extent_bytes) {
    try {
        clear_error();
        LWO_TRY(validate_desc(desc));
        Layout L = make_layout(*desc);
        if (n) *n = (int32_t)L.tensors.size();
        if (extent_bytes) *extent_bytes = L.extent_bytes;
        if (!out) return cap == 0 ? LWO_OK : (set_error("out is NULL"), LWO_EINVAL);
        if (cap < (int32_t)L.tensors.size()) { set_error("cap smaller than the tensor count"); return LWO_EINVAL; }
        for (size_t i = 0; i < L.tensors.size(); ++i) {
            const TensorSlot& t = L.tensors[i];
            lwo_tensor_info& o = out[i];
            std::memset(&o, 0, sizeof(o));
            std::strncpy(o.name, t.name.c_str(), sizeof(o.name) - 1);
            o.offset = t.offset;
            o.bytes = t.bytes;
            o.rank = t.rank;
            o.shape[0] = t.shape[0];
            o.shape[1] = t.shape[1];
            o.dtype = t.dtype;
            o.tiled = t.tiled ? 1 : 0;
        }
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_block_layout");
    } catch (const std::exception& e) {
        return fail_exception("lwo_block_layout", e.what());
    } catch (...) {
        return fail_exception("lwo_block_layout", "unknown exception");
    }
}

extern "C" lwo_status lwo_pack_block(const lwo_model_desc* desc, const float* const* tensors, int32_t n_tensors,
                                     void* dst, uint64_t dst_bytes) {
    try {
        clear_error();
        LWO_TRY(validate_desc(desc));
        Layout L = make_layout(*desc);
        const bool fp8 = desc->linear_dtype == LWO_FP8_E4M3;
        const int n_in = (int)L.tensors.size() - (fp8 ? 1 : 0);
        if (!tensors || n_tensors != n_in) { set_error("pack: expected " + std::to_string(n_in) + " tensors"); return LWO_EINVAL; }
        if (!dst || dst_bytes < L.extent_bytes) { set_error("pack: destination too small"); return LWO_EINVAL; }
        for (int i = 0; i < n_in; ++i)
            if (!tensors[i]) { set_error("pack: tensor " + L.tensors[i].name + " is NULL"); return LWO_EINVAL; }
        unsigned char* out = (unsigned char*)dst;
        std::memset(out, 0, L.extent_bytes);
        float scales[10];
        int n_scales = 0;
        std::vector<unsigned char> rowmajor;
        for (int i = 0; i < n_in; ++i) {
            const TensorSlot& t = L.tensors[i];
            const uint64_t n = t.bytes / (uint64_t)dtype_bytes(t.dtype);
            const float* src = tensors[i];
            // A tiled tensor is encoded row-major into a scratch buffer, then tiled.
            if (t.tiled) rowmajor.resize(t.bytes);
            unsigned char* o = t.tiled ? rowmajor.data() : out + t.offset;
            if (t.dtype == LWO_F32) {
                std::memcpy(o, src, t.bytes);
            } else if (t.dtype == LWO_BF16) {
                uint16_t* ob = (uint16_t*)o;
                for (uint64_t j = 0; j < n; ++j) ob[j] = f32_to_bf16_rne(src[j]);
            } else {
                float amax = 0.0f;
                for (uint64_t j = 0; j < n; ++j) amax = std::fmax(amax, std::fabs(src[j]));
                const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
                for (uint64_t j = 0; j < n; ++j) o[j] = f32_to_e4m3_rne_sat(src[j] / s);
                scales[n_scales++] = s;
            }
            if (t.tiled) tile_rows(rowmajor.data(), t.shape[0], (uint64_t)t.shape[1] * dtype_bytes(t.dtype), out + t.offset);
        }
        if (fp8) {
            const TensorSlot& t = L.tensors.back();
            if (n_scales != 10) { set_error("pack: expected ten fp8 weight matrices"); return LWO_EINVAL; }
            std::memcpy(out + t.offset, scales, sizeof(scales));
        }
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_pack_block");
    } catch (const std::exception& e) {
        return fail_exception("lwo_pack_block", e.what());
    } catch (...) {
        return fail_exception("lwo_pack_block", "unknown exception");
    }
}

extern "C" lwo_status lwo_tile_weight(int32_t dtype, const void* src, int32_t N, int32_t K, void* dst) {
    try {
        clear_error();
        if (dtype != LWO_BF16 && dtype != LWO_FP8_E4M3) { set_error("tile_weight: dtype must be BF16 or FP8_E4M3"); return LWO_EINVAL; }
        const uint64_t R = (uint64_t)(K > 0 ? K : 0) * (uint64_t)dtype_bytes(dtype);
        if (N < 1 || K < 1 || N % 64 || R % 64) { set_error("tile_weight: N must be a multiple of 64 and K * element bytes of 64"); return LWO_EINVAL; }
        if (!src || !dst) { set_error("tile_weight: null pointer"); return LWO_EINVAL; }
        tile_rows((const unsigned char*)src, N, R, (unsigned char*)dst);
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_tile_weight");
    } catch (const std::exception& e) {
        return fail_exception("lwo_tile_weight", e.what());
    } catch (...) {
        return fail_exception("lwo_tile_weight", "unknown exception");
    }
}

extern "C" lwo_status lwo_extent_checksum(const void* host, uint64_t bytes, uint64_t* sum) {
    try {
        clear_error();
        if (!sum || (bytes && !host) || bytes % 8) { set_error("checksum: bad arguments"); return LWO_EINVAL; }
        *sum = extent_checksum_host(host, bytes);
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_extent_checksum");
    } catch (const std::exception& e) {
        return fail_exception("lwo_extent_checksum", e.what());
    } catch (...) {
        return fail_exception("lwo_extent_checksum", "unknown exception");
    }
}

extern "C" const char* lwo_last_error(void) { return g_err.c_str(); }
