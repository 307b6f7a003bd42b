// lwo_run_blocks_noalloc: one denoise step over device-resident block extents
// that allocates nothing.  The activation workspace (the fp32 residual, the
// modulation, LayerNorm, QKV/FFN and attention outputs, fp8 codes) lives in a
// file-scope device array instead of memory the library allocates; every GPU
// the library runs on holds its own copy of the array until the process ends.
//
// Host code never uses the array's name as an address: on the host it is a
// stand-in symbol, not device memory.  The first call on a device looks the
// array's device address up with hipGetSymbolAddress (with that device
// current) and keeps it per device; kernels take that address.
#include <mutex>

#include "lwo_internal.h"

using namespace lwo;

namespace {

constexpr uint64_t kScratchBytes = 64ull << 20;   // LWO_NOALLOC_SCRATCH_BYTES in include/lwo.h
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The array's address on `dev` (current), looked up once per device.
lwo_status scratch_on(int dev, void** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_error(std::string("hipGetSymbolAddress of the no-alloc scratch array: ") + hipGetErrorString(e));
            return LWO_EHIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return LWO_OK;
}

}  // namespace

extern "C" lwo_status lwo_run_blocks_noalloc(const lwo_model_desc* desc, const void* const* blocks, int32_t n_blocks,
                                             void* x, const void* cond, const void* ctx, void* hip_stream) {
    try {
        clear_error();
        LWO_TRY(validate_desc(desc));
        const lwo_model_desc& d = *desc;
        if (n_blocks < 1 || !blocks) { set_error("noalloc: n_blocks >= 1 block pointers required"); return LWO_EINVAL; }
        for (int b = 0; b < n_blocks; ++b)
            if (!blocks[b] || ((uintptr_t)blocks[b] % 256)) {
                set_error("noalloc: block " + std::to_string(b) + " is NULL or not 256-byte aligned");
                return LWO_EINVAL;
            }
        if (!hip_stream) { set_error("noalloc: stream is NULL"); return LWO_EINVAL; }
        if (!x || !cond) { set_error("noalloc: x and cond are required"); return LWO_EINVAL; }
        if (d.kind == LWO_KIND_VIDEO && !ctx) { set_error("noalloc: video kind needs ctx"); return LWO_EINVAL; }
        if (d.kind == LWO_KIND_DIT && ctx) { set_error("noalloc: DiT kind takes no ctx"); return LWO_EINVAL; }
        const size_t need = workspace_carve(d, nullptr, nullptr);
        if (need > kScratchBytes) {
            set_error("noalloc: the step's workspace needs " + std::to_string(need) + " bytes, more than the " +
                      std::to_string(kScratchBytes) + "-byte scratch array");
            return LWO_EINVAL;
        }
        hipStream_t st = (hipStream_t)hip_stream;
        int dev = -1, prev = -1;
        LWO_HIP_TRY(hipStreamGetDevice(st, &dev));
        if (dev < 0 || dev >= kMaxDevices) { set_error("noalloc: device ordinal out of range"); return LWO_EINVAL; }
        LWO_HIP_TRY(hipGetDevice(&prev));
        // The stream's device is made current for the symbol lookup and the
        // launches; the caller's current device is restored on every return.
        struct Restore { int d; ~Restore() { if (d >= 0) (void)hipSetDevice(d); } } restore{prev};
        LWO_HIP_TRY(hipSetDevice(dev));
        void* base = nullptr;
        LWO_TRY(scratch_on(dev, &base));
        Workspace ws;
        workspace_carve(d, base, &ws);
        LWO_TRY(enqueue_zero_u64(ws.sums, 2, st));   // the checksum counters start at zero (no memset node)
        const Layout lay = make_layout(d);
        LWO_TRY(enqueue_step_begin(d, ws, x, cond, ctx, st));
        for (int b = 0; b < n_blocks; ++b)
            LWO_TRY(enqueue_block(d, block_ptrs(lay, d, (const char*)blocks[b]), ws, cond, ctx, st, nullptr));
        LWO_TRY(enqueue_step_end(d, ws, x, st));
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_run_blocks_noalloc");
    } catch (const std::exception& e) {
        return fail_exception("lwo_run_blocks_noalloc", e.what());
    } catch (...) {
        return fail_exception("lwo_run_blocks_noalloc", "unknown exception");
    }
}
