// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <exception>
#include <new>
#include <string>
#include <vector>

#include "../../include/lwo.h"

namespace lwo {

// ------------------------------------------------------------------ errors

void set_error(const std::string& msg);
lwo_status fail_alloc(const char* where) noexcept;                     // LWO_ENOMEM
lwo_status fail_exception(const char* where, const char* what) noexcept;  // LWO_EIO
void clear_error();

#define LWO_HIP_TRY(expr)                                                              \
    do {                                                                               \
        hipError_t e_ = (expr);                                                        \
        if (e_ != hipSuccess) {                                                        \
            ::lwo::set_error(std::string(#expr) + ": " + hipGetErrorString(e_));       \
            return LWO_EHIP;                                                           \
        }                                                                              \
    } while (0)

#define LWO_TRY(expr)                                                                  \
    do {                                                                               \
        lwo_status s_ = (expr);                                                        \
        if (s_ != LWO_OK) return s_;                                                   \
    } while (0)

// ------------------------------------------------------------------ layout

constexpr uint64_t kTensorAlign = 256;
constexpr uint64_t kExtentAlign = 4096;

struct TensorSlot {
    std::string name;
    uint64_t offset = 0, bytes = 0;
    int rank = 1;
    int shape[2] = {0, 0};
    int dtype = LWO_F32;
    bool tiled = false;   // 64-row x 64-byte tiles (bf16/fp8 GEMM weights)
};

struct Layout {
    std::vector<TensorSlot> tensors;   // in block order
    uint64_t extent_bytes = 0;
    int find(const char* name) const;  // index or -1
};

lwo_status validate_desc(const lwo_model_desc* d);
Layout make_layout(const lwo_model_desc& d);
int dtype_bytes(int dt);

// Host codecs (library side): float -> bf16 bits, float -> e4m3 code.
uint16_t f32_to_bf16_rne(float f);
uint8_t f32_to_e4m3_rne_sat(float f);
uint64_t extent_checksum_host(const void* p, uint64_t bytes);

// ------------------------------------------------------------------ kernels

// Device pointers of one block's tensors (inside a slot or the resident region).
struct BlockPtrs {
    const float* w_scale;    // fp8: ten per-tensor scales (device, weight-matrix order), else null
    // DiT kind
    const void* ada_w; const void* ada_b;
    // both kinds
    const void* q_w; const void* k_w; const void* v_w; const void* qkv_b;
    const void* o_w; const void* o_b;
    const void* fc1_w; const void* fc1_b; const void* fc2_w; const void* fc2_b;
    // video kind
    const void* mod_table; const void* q_norm; const void* k_norm;
    const void* cq_w; const void* cq_b; const void* ck_w; const void* cv_w; const void* ckv_b;
    const void* co_w; const void* co_b;
};

BlockPtrs block_ptrs(const Layout& L, const lwo_model_desc& d, const char* base);

// Activation workspace for one denoise step.
struct Workspace {
    float* xr = nullptr;        // fp32 residual [M, D]
    float* mod = nullptr;       // fp32 modulation [B, 6, D]
    float* silu_cond = nullptr; // DiT kind: SiLU(cond) [B, D] fp32, once per step
    void* h = nullptr;          // LN output [M, D] act dtype
    void* big = nullptr;        // [M, max(3D, F)] act dtype: qkv, then FFN hidden
    void* attn = nullptr;       // attention output [M, D] act dtype
    void* cq = nullptr;         // cross-attention queries [M, D]
    void* ckv = nullptr;        // cross-attention keys|values [B*Tc, 2D]
    uint8_t* q8 = nullptr;      // fp8 activation codes [M, max(D, F)]
    float* q8_scale = nullptr;  // per-row fp8 scales [max(M, B*Tc)]
    uint8_t* ctx8 = nullptr;    // fp8 context codes [B*Tc, D]
    float* ctx8_scale = nullptr;
    uint64_t* sums = nullptr;   // checksum scratch [2]: running sum, mismatch count
    size_t bytes = 0;
    void* base = nullptr;
};

lwo_status workspace_alloc(const lwo_model_desc& d, Workspace* ws);
// The workspace's layout from base (device); with base == nullptr it only
// returns the bytes it needs.
size_t workspace_carve(const lwo_model_desc& d, void* base, Workspace* ws);
void workspace_free(Workspace* ws);

// Optional per-kernel timing: events around each launch, aggregated per kernel symbol.
struct KernelTimer {
    struct Rec { int cls; hipEvent_t a, b; double flops, bytes; };
    struct Agg { std::string name; uint64_t launches = 0; double ms = 0, flops = 0, bytes = 0; };
    bool on = false;
    std::vector<Rec> pending;
    std::vector<Agg> agg;
    std::vector<hipEvent_t> pool;
    hipEvent_t get();
    int cls(const char* name);
    lwo_status collect();   // synchronise pending events into agg
    void reset();
    void destroy();
};

// Enqueue one block's forward on `stream` (kt may be null).
lwo_status enqueue_block(const lwo_model_desc& d, const BlockPtrs& p, const Workspace& ws,
                         const void* cond, const void* ctx, hipStream_t stream, KernelTimer* kt);

// Step prologue/epilogue: x (act dtype) -> fp32 residual (and, DiT kind, SiLU(cond)
// for every block's adaLN linear; fp8 linears: the context's e4m3 codes), and back.
lwo_status enqueue_step_begin(const lwo_model_desc& d, const Workspace& ws, const void* x, const void* cond,
                              const void* ctx, hipStream_t st);
lwo_status enqueue_step_end(const lwo_model_desc& d, const Workspace& ws, void* x, hipStream_t stream);

// Checksum of `bytes` (multiple of 8) device bytes; adds into acc[0].  When
// expect is given, a second kernel compares acc[0] with *expect_host and
// increments acc[1] on mismatch (acc[0] is reset by the caller).
lwo_status enqueue_checksum(const void* dev, uint64_t bytes, uint64_t* acc, hipStream_t stream);
lwo_status enqueue_checksum_compare(uint64_t* acc, uint64_t expect, hipStream_t stream);
lwo_status enqueue_zero_u64(uint64_t* p, int n, hipStream_t stream);

}  // namespace lwo
