// The block store: host weight extents, the two-slot device arena, the copy
// stream with its readiness events, and the ring that streams blocks
// through the slots during a denoise step.
//
// Design sources (offloader documentation pages):
//  * "CPU Offloading for Diffusion Models", "Layerwise (Blockwise) Offloading
//    / How It Works": a dedicated copy stream prefetches block i+1 while
//    block i computes, parameters are kept as flattened pinned host tensors,
//    and the last block prefetches block 0 (execution-flow table).
//  * "Distributed Layerwise Offload", "Startup and runtime sequence": a pair
//    of device buffers, each as large as the biggest block that streams;
//    compute waits for the current buffer's readiness, the next block goes to the alternate
//    slot, the first block is primed at enable; "Feature compatibility":
//    resident leading layers; "Registered runtime-cache transfer" and
//    "Failure and lifecycle boundaries": page-aligned, coalesced, budgeted,
//    read-only, all-or-nothing host registration, and shutdown order
//    (synchronise, unregister, then release).
//  * "CPU Offloading", "Cross-strategy invariants": a device buffer is only
//    reused once the kernels and copies that depend on it have finished; "Shared
//    lifecycle": a failed enable leaves no partial state.
//  * "Distributed Layerwise Offload", "Host backing and transfer
//    composition" and "Runtime cache": with pageable (e.g. mmap) host
//    storage and no registration, every streamed block is packed into one of
//    two bounded pinned host staging slots and copied from there; a zero
//    registration budget or a failed (rolled back) registration keeps that
//    staging path.
//  * "Distributed Layerwise Offload", "AllGather path" and "Host backing and
//    transfer composition" (ordinary runtime tensors, group larger than one):
//    each rank keeps about 1/group of every streamed block pinned, copies its
//    shard of the next block to the device, and the group's all-gather on a
//    communication stream completes the slot while the current block runs.
//    SHARD mode is one rank's share of that on one GPU: the rank's shard is
//    the only host memory and the only host -> device copy; the other shards,
//    which the all-gather would bring from the peers, come from a device
//    region that stands in for them (copied on a separate gather stream).
#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <cstring>
#include <mutex>
#include <thread>

#include "lwo_internal.h"

using namespace lwo;

// Host copy workers for STAGED mode: one extent copy is split into equal
// parts, one per worker plus the calling thread, which waits for all of them.
struct PackPool {
    std::vector<std::thread> th;
    std::mutex mu;
    std::condition_variable go, done;
    uint64_t gen = 0;
    int left = 0;
    bool stop = false;
    char* dst = nullptr;
    const char* src = nullptr;
    uint64_t bytes = 0;

    void part(int i) {
        const int parts = (int)th.size() + 1;
        const uint64_t a = bytes * (uint64_t)i / parts / 64 * 64;
        const uint64_t b = (i + 1 == parts) ? bytes : bytes * (uint64_t)(i + 1) / parts / 64 * 64;
        if (b > a) std::memcpy(dst + a, src + a, b - a);
    }
    void start(int workers) {
        for (int i = 0; i < workers; ++i)
            th.emplace_back([this, i] {
                uint64_t seen = 0;
                for (;;) {
                    std::unique_lock<std::mutex> lk(mu);
                    go.wait(lk, [&] { return stop || gen != seen; });
                    if (stop) return;
                    seen = gen;
                    lk.unlock();
                    part(i + 1);
                    lk.lock();
                    if (--left == 0) done.notify_one();
                }
            });
    }
    void copy(char* d, const char* s_, uint64_t n) {
        {
            std::lock_guard<std::mutex> lk(mu);
            dst = d;
            src = s_;
            bytes = n;
            left = (int)th.size();
            ++gen;
        }
        go.notify_all();
        part(0);
        std::unique_lock<std::mutex> lk(mu);
        done.wait(lk, [&] { return left == 0; });
    }
    void shutdown() {
        {
            std::lock_guard<std::mutex> lk(mu);
            stop = true;
        }
        go.notify_all();
        for (auto& t : th) t.join();
        th.clear();
        stop = false;
    }
};

struct lwo_store {
    lwo_model_desc d{};                   // the stack: shared shapes, largest ffn, fp8 if any block type is
    std::vector<lwo_model_desc> tdesc;    // per block type
    std::vector<Layout> tlay;             // per block type
    std::vector<int> btype;               // per block: its type
    std::vector<uint64_t> bext;           // per block: extent bytes of its type
    std::vector<uint64_t> dext;           // per block: device bytes (bext, or the shard-padded extent)
    std::vector<uint64_t> roff;           // per block: offset in the resident region (prefix sums of dext)
    uint64_t max_ext = 0;                 // slot and staging size (largest dext)
    // SHARD: this rank's share of an all-gather group
    int group = 1, rank = 0;
    uint64_t shard = 0;                   // bytes of one shard (dext / group)
    char* peer = nullptr;                 // device: per block the group-1 other shards, back to back
    hipStream_t gather = nullptr;         // stand-in for the communication stream
    hipEvent_t shard_done[2] = {nullptr, nullptr};
    uint64_t gather_bytes = 0;
    int device = 0;
    int host_mode = LWO_HOST_PIN_COPY;    // mode in effect
    std::vector<void*> host;              // per-block host extent
    bool host_owned = false;              // PIN_COPY: allocated with hipHostMalloc
    char* stage[2] = {nullptr, nullptr};  // STAGED: two pinned staging slots of extent_bytes
    hipEvent_t stage_done[2] = {nullptr, nullptr};   // end of the last device copy out of each
    bool stage_busy[2] = {false, false};
    int stage_next = 0;
    PackPool pool;
    int pack_threads = 0;                 // workers besides the calling thread
    uint64_t pack_bytes = 0;
    double pack_ms = 0;
    std::vector<uint64_t> reg_base, reg_len;
    std::vector<uint64_t> host_sums;      // lazily computed host checksums
    bool sums_ready = false;
    char* slot[2] = {nullptr, nullptr};
    int slot_block[2] = {-1, -1};         // block held (or being received) by each slot
    char* resident = nullptr;
    int k = 0;
    int head_slot = 0;                    // slot holding (or receiving) block k
    hipStream_t copy = nullptr;
    hipEvent_t copy_done[2] = {nullptr, nullptr};
    hipEvent_t compute_done[2] = {nullptr, nullptr};
    Workspace ws;
    bool validation = false;
    bool timing = false;
    std::vector<hipEvent_t> tev;          // timing events, two per copy of the last step
    int n_timed = 0;
    uint64_t h2d_copies = 0, h2d_bytes = 0, steps = 0;
    double build_ms = 0;
    KernelTimer kt;
    int max_inflight = 1;                 // pacing depth of run (0: no host wait)
    hipEvent_t step_done[16] = {};        // completion of recent steps, ring indexed by step number
    bool dead = false;
};

// ------------------------------------------------------------------ registration

extern "C" lwo_status lwo_register_ranges(const void* const* ptrs, const uint64_t* bytes, int32_t n, uint64_t page,
                                          uint64_t budget, lwo_register_fn reg, lwo_unregister_fn unreg, void* user,
                                          uint64_t* out_base, uint64_t* out_len, int32_t cap, int32_t* n_out) {
    try {
        clear_error();
        if (n < 0 || (n && (!ptrs || !bytes)) || !reg || !unreg || page == 0 || (page & (page - 1))) {
            set_error("register: bad arguments (page must be a power of two)");
            return LWO_EINVAL;
        }
        // page-align every range outward, then coalesce overlapping or adjacent ranges
        std::vector<std::pair<uint64_t, uint64_t>> r;   // [begin, end)
        for (int i = 0; i < n; ++i) {
            if (!bytes[i]) continue;
            uint64_t b = (uint64_t)(uintptr_t)ptrs[i];
            uint64_t e = b + bytes[i];
            r.emplace_back(b & ~(page - 1), (e + page - 1) & ~(page - 1));
        }
        std::sort(r.begin(), r.end());
        std::vector<std::pair<uint64_t, uint64_t>> c;
        for (auto& x : r) {
            if (!c.empty() && x.first <= c.back().second) c.back().second = std::max(c.back().second, x.second);
            else c.push_back(x);
        }
        uint64_t total = 0;
        for (auto& x : c) total += x.second - x.first;
        if (n_out) *n_out = (int32_t)c.size();
        if (cap < (int32_t)c.size() || (!c.empty() && (!out_base || !out_len))) {
            set_error("register: output capacity smaller than the coalesced range count");
            return LWO_EINVAL;
        }
        if (total > budget) {   // checked before any registration call
            set_error("register: " + std::to_string(total) + " bytes exceed the budget of " + std::to_string(budget));
            return LWO_EBUDGET;
        }
        for (size_t i = 0; i < c.size(); ++i) {
            if (reg(user, (void*)(uintptr_t)c[i].first, c[i].second - c[i].first) != 0) {
                bool rb_ok = true;
                for (size_t j = i; j-- > 0;)
                    if (unreg(user, (void*)(uintptr_t)c[j].first) != 0) rb_ok = false;
                if (!rb_ok) {
                    set_error("register: range " + std::to_string(i) + " failed and a rollback unregister failed; "
                              "the ranges that could not be unregistered must stay mapped");
                    return LWO_EROLLBACK;
                }
                set_error("register: range " + std::to_string(i) + " failed; all earlier ranges were unregistered");
                return LWO_EREGISTER;
            }
        }
        for (size_t i = 0; i < c.size(); ++i) {
            out_base[i] = c[i].first;
            out_len[i] = c[i].second - c[i].first;
        }
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_register_ranges");
    } catch (const std::exception& e) {
        return fail_exception("lwo_register_ranges", e.what());
    } catch (...) {
        return fail_exception("lwo_register_ranges", "unknown exception");
    }
}

static int32_t hip_register_cb(void*, void* base, uint64_t bytes) {
    return hipHostRegister(base, bytes, hipHostRegisterReadOnly) == hipSuccess ? 0 : 1;
}
static int32_t hip_unregister_cb(void*, void* base) {
    return hipHostUnregister(base) == hipSuccess ? 0 : 1;
}

// ------------------------------------------------------------------ teardown

static void release(lwo_store* s) {
    if (!s) return;
    (void)hipSetDevice(s->device);
    if (s->copy) (void)hipStreamSynchronize(s->copy);
    if (s->gather) (void)hipStreamSynchronize(s->gather);
    (void)hipDeviceSynchronize();   // compute that may still read a slot runs on caller streams
    if (s->host_mode == LWO_HOST_REGISTER) {
        for (size_t i = s->reg_base.size(); i-- > 0;) (void)hipHostUnregister((void*)(uintptr_t)s->reg_base[i]);
        s->reg_base.clear();
        s->reg_len.clear();
    }
    if (s->host_owned)
        for (void* p : s->host)
            if (p) (void)hipHostFree(p);
    s->host.clear();
    s->pool.shutdown();
    for (int i = 0; i < 2; ++i) {
        if (s->stage[i]) (void)hipHostFree(s->stage[i]);
        if (s->stage_done[i]) (void)hipEventDestroy(s->stage_done[i]);
    }
    for (int i = 0; i < 2; ++i) {
        if (s->slot[i]) (void)hipFree(s->slot[i]);
        if (s->copy_done[i]) (void)hipEventDestroy(s->copy_done[i]);
        if (s->compute_done[i]) (void)hipEventDestroy(s->compute_done[i]);
    }
    for (hipEvent_t e : s->tev) (void)hipEventDestroy(e);
    for (hipEvent_t e : s->step_done)
        if (e) (void)hipEventDestroy(e);
    if (s->resident) (void)hipFree(s->resident);
    if (s->peer) (void)hipFree(s->peer);
    for (hipEvent_t e : s->shard_done)
        if (e) (void)hipEventDestroy(e);
    if (s->gather) (void)hipStreamDestroy(s->gather);
    s->kt.destroy();
    workspace_free(&s->ws);
    if (s->copy) (void)hipStreamDestroy(s->copy);
    delete s;
}

// ------------------------------------------------------------------ helpers

// Enqueue the transfer of block b into dst (device, dext[b] bytes) and record
// `done` on the stream that finishes it (optional timing events around the
// host -> device copy only).  STAGED: wait until the device copy last issued
// from the next staging slot is done (the host is about to overwrite it), pack
// the pageable extent into it, then copy.  SHARD: copy this rank's pinned
// shard to its offset of dst on the copy stream; the gather stream waits for
// it and copies the other shards from the peer region around it.
static lwo_status h2d_block(lwo_store* s, char* dst, int b, hipEvent_t done, hipEvent_t t0 = nullptr,
                            hipEvent_t t1 = nullptr) {
    const uint64_t ext = s->host_mode == LWO_HOST_SHARD ? s->shard : s->bext[b];
    const char* src = (const char*)s->host[b];
    int q = -1;
    if (s->host_mode == LWO_HOST_STAGED) {
        q = s->stage_next;
        s->stage_next ^= 1;
        if (s->stage_busy[q]) LWO_HIP_TRY(hipEventSynchronize(s->stage_done[q]));
        const auto c0 = std::chrono::steady_clock::now();
        s->pool.copy(s->stage[q], src, ext);
        s->pack_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - c0).count();
        s->pack_bytes += ext;
        src = s->stage[q];
    }
    char* at = s->host_mode == LWO_HOST_SHARD ? dst + (uint64_t)s->rank * s->shard : dst;
    if (t0) LWO_HIP_TRY(hipEventRecord(t0, s->copy));
    LWO_HIP_TRY(hipMemcpyAsync(at, src, ext, hipMemcpyHostToDevice, s->copy));
    if (t1) LWO_HIP_TRY(hipEventRecord(t1, s->copy));
    if (q >= 0) {
        LWO_HIP_TRY(hipEventRecord(s->stage_done[q], s->copy));
        s->stage_busy[q] = true;
    }
    s->h2d_copies++;
    s->h2d_bytes += ext;
    if (s->host_mode != LWO_HOST_SHARD || s->group == 1) {
        if (done) LWO_HIP_TRY(hipEventRecord(done, s->copy));
        return LWO_OK;
    }
    // The all-gather stand-in: shards [0, rank) and (rank, group) of block b.
    const int sl = (dst == s->slot[1]) ? 1 : 0;
    LWO_HIP_TRY(hipEventRecord(s->shard_done[sl], s->copy));
    LWO_HIP_TRY(hipStreamWaitEvent(s->gather, s->shard_done[sl], 0));
    const uint64_t below = (uint64_t)s->rank * s->shard, above = s->dext[b] - below - s->shard;
    const char* pb = s->peer + (uint64_t)b * (s->dext[b] - s->shard);
    if (below) LWO_HIP_TRY(hipMemcpyAsync(dst, pb, below, hipMemcpyDeviceToDevice, s->gather));
    if (above) LWO_HIP_TRY(hipMemcpyAsync(dst + below + s->shard, pb + below, above, hipMemcpyDeviceToDevice, s->gather));
    s->gather_bytes += below + above;
    if (done) LWO_HIP_TRY(hipEventRecord(done, s->gather));
    return LWO_OK;
}

// Wait on the host until every transfer stream of the store has drained.
static lwo_status sync_transfers(lwo_store* s) {
    LWO_HIP_TRY(hipStreamSynchronize(s->copy));
    if (s->gather) LWO_HIP_TRY(hipStreamSynchronize(s->gather));
    return LWO_OK;
}

static lwo_status prime_head(lwo_store* s) {
    // Block k goes to slot 0 on the copy stream ([DLO] prime the first block).
    s->head_slot = 0;
    s->slot_block[0] = s->slot_block[1] = -1;
    if (s->k >= s->d.n_blocks) return LWO_OK;
    LWO_TRY(h2d_block(s, s->slot[0], s->k, s->copy_done[0]));
    s->slot_block[0] = s->k;
    return LWO_OK;
}

static void compute_host_sums(lwo_store* s) {
    if (s->sums_ready) return;
    const int n = s->d.n_blocks;
    s->host_sums.assign(n, 0);
    unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    std::vector<std::thread> th;
    for (unsigned t = 0; t < nt; ++t)
        th.emplace_back([s, t, nt, n] {
            for (int b = (int)t; b < n; b += (int)nt) s->host_sums[b] = extent_checksum_host(s->host[b], s->bext[b]);
        });
    for (auto& x : th) x.join();
    s->sums_ready = true;
}

static lwo_status check_store(lwo_store* s) {
    if (!s) { set_error("store is NULL"); return LWO_EINVAL; }
    if (s->dead) { set_error("store is not usable after a failed call"); return LWO_ESTATE; }
    return LWO_OK;
}

// ------------------------------------------------------------------ build

static lwo_status build_staged(lwo_store* s, const lwo_block_source* src);
static lwo_status build_shard(lwo_store* s, const lwo_block_source* src);
static lwo_status build_device(lwo_store* s);

static lwo_status build(lwo_store* s, const lwo_block_source* src, int mode, uint64_t budget) {
    const int n = s->d.n_blocks;
    LWO_HIP_TRY(hipSetDevice(s->device));
    s->host.assign(n, nullptr);
    if (mode == LWO_HOST_PIN_COPY) {
        s->host_owned = true;
        for (int b = 0; b < n; ++b) {
            const uint64_t ext = s->bext[b];
            void* p = nullptr;
            if (hipHostMalloc(&p, ext, hipHostMallocDefault) != hipSuccess || !p) {
                set_error("hipHostMalloc of block " + std::to_string(b) + " (" + std::to_string(ext) + " bytes) failed");
                return LWO_ENOMEM;
            }
            s->host[b] = p;
            if (src->extents) {
                if (!src->extents[b]) { set_error("extent " + std::to_string(b) + " is NULL"); return LWO_EINVAL; }
                std::memcpy(p, src->extents[b], ext);
            } else if (src->fill(src->user, b, p, ext) != 0) {
                set_error("fill callback failed for block " + std::to_string(b));
                return LWO_EINVAL;
            }
        }
    } else if (mode == LWO_HOST_SHARD) {
        return build_shard(s, src);
    } else if (mode == LWO_HOST_REGISTER && budget > 0) {
        if (!src->extents) { set_error("REGISTER mode needs caller extents"); return LWO_EINVAL; }
        const uint64_t page = 4096;
        std::vector<uint64_t> lens(s->bext);
        for (int b = 0; b < n; ++b) {
            if (!src->extents[b] || ((uintptr_t)src->extents[b] % page)) {
                set_error("REGISTER mode needs page-aligned extents (block " + std::to_string(b) + ")");
                return LWO_EINVAL;
            }
            s->host[b] = const_cast<void*>(src->extents[b]);
        }
        std::vector<uint64_t> base(n), len(n);
        int32_t nr = 0;
        lwo_status st = lwo_register_ranges(src->extents, lens.data(), n, page, budget, hip_register_cb,
                                            hip_unregister_cb, nullptr, base.data(), len.data(), n, &nr);
        if (st == LWO_EBUDGET || st == LWO_EREGISTER) {   // nothing stays registered: keep the staging path
            (void)hipGetLastError();
            s->host_mode = LWO_HOST_STAGED;
            return build_staged(s, src);
        }
        if (st != LWO_OK) return st;   // LWO_EROLLBACK: a range may still be registered
        s->reg_base.assign(base.begin(), base.begin() + nr);
        s->reg_len.assign(len.begin(), len.begin() + nr);
        for (int b = 0; b < n; ++b) {   // every extent must now be known to HIP as registered host memory
            unsigned int flags = 0;
            if (hipHostGetFlags(&flags, s->host[b]) != hipSuccess) {
                set_error("registered extent " + std::to_string(b) + " is not recognised as pinned");
                return LWO_EREGISTER;
            }
        }
    } else {   // STAGED, or REGISTER with a zero budget
        s->host_mode = LWO_HOST_STAGED;
        return build_staged(s, src);
    }
    return build_device(s);
}

// STAGED: borrow the caller's pageable extents, allocate the two pinned staging slots.
static lwo_status build_staged(lwo_store* s, const lwo_block_source* src) {
    const uint64_t ext = s->max_ext;
    if (!src->extents) { set_error("STAGED mode needs caller extents"); return LWO_EINVAL; }
    for (int b = 0; b < s->d.n_blocks; ++b) {
        if (!src->extents[b]) { set_error("extent " + std::to_string(b) + " is NULL"); return LWO_EINVAL; }
        s->host[b] = const_cast<void*>(src->extents[b]);
    }
    for (int i = 0; i < 2; ++i) {
        if (hipHostMalloc((void**)&s->stage[i], ext, hipHostMallocDefault) != hipSuccess || !s->stage[i]) {
            s->stage[i] = nullptr;
            set_error("hipHostMalloc of a staging slot failed");
            return LWO_ENOMEM;
        }
        LWO_HIP_TRY(hipEventCreateWithFlags(&s->stage_done[i], hipEventDisableTiming));
    }
    s->pack_threads = (int)std::max(0u, std::min(7u, std::thread::hardware_concurrency() / 2));
    s->pool.start(s->pack_threads);
    return build_device(s);
}

// SHARD: read each block's whole extent once (from the caller's extents or the
// fill callback, into a pinned scratch extent padded with zeros to the shard
// multiple), checksum it, keep this rank's shard in pinned host memory and
// place the other shards in the peer region on the device.
static lwo_status build_shard(lwo_store* s, const lwo_block_source* src) {
    const int n = s->d.n_blocks;
    const uint64_t dx = s->dext[0], sh = s->shard, ext = s->bext[0];
    s->host_owned = true;   // the shards allocated so far are released on failure
    char* tmp = nullptr;
    if (hipHostMalloc((void**)&tmp, dx, hipHostMallocDefault) != hipSuccess || !tmp) {
        set_error("hipHostMalloc of the shard build's scratch extent failed");
        return LWO_ENOMEM;
    }
    struct Free { char* p; ~Free() { if (p) (void)hipHostFree(p); } } guard{tmp};
    if (s->group > 1) {
        const uint64_t bytes = (uint64_t)n * (dx - sh);
        if (hipMalloc(&s->peer, bytes) != hipSuccess) {
            s->peer = nullptr;
            set_error("hipMalloc of the peer-shard region (" + std::to_string(bytes) + " bytes) failed");
            return LWO_ENOMEM;
        }
        LWO_HIP_TRY(hipStreamCreateWithFlags(&s->gather, hipStreamNonBlocking));
        for (hipEvent_t& e : s->shard_done) LWO_HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    }
    s->host_sums.assign(n, 0);
    for (int b = 0; b < n; ++b) {
        if (src->extents) {
            if (!src->extents[b]) { set_error("extent " + std::to_string(b) + " is NULL"); return LWO_EINVAL; }
            std::memcpy(tmp, src->extents[b], ext);
        } else if (src->fill(src->user, b, tmp, ext) != 0) {
            set_error("fill callback failed for block " + std::to_string(b));
            return LWO_EINVAL;
        }
        std::memset(tmp + ext, 0, dx - ext);
        s->host_sums[b] = extent_checksum_host(tmp, ext);
        void* p = nullptr;
        if (hipHostMalloc(&p, sh, hipHostMallocDefault) != hipSuccess || !p) {
            set_error("hipHostMalloc of shard " + std::to_string(b) + " (" + std::to_string(sh) + " bytes) failed");
            return LWO_ENOMEM;
        }
        s->host[b] = p;
        const uint64_t below = (uint64_t)s->rank * sh;
        std::memcpy(p, tmp + below, sh);
        if (s->group > 1) {
            char* pb = s->peer + (uint64_t)b * (dx - sh);
            if (below) LWO_HIP_TRY(hipMemcpy(pb, tmp, below, hipMemcpyHostToDevice));
            if (dx - below - sh) LWO_HIP_TRY(hipMemcpy(pb + below, tmp + below + sh, dx - below - sh, hipMemcpyHostToDevice));
        }
    }
    s->sums_ready = true;
    return build_device(s);
}

// Device arena, workspace, copy stream and events; prime the head block.
static lwo_status build_device(lwo_store* s) {
    const uint64_t ext = s->max_ext;
    for (int i = 0; i < 2; ++i) {
        if (hipMalloc(&s->slot[i], ext) != hipSuccess) { s->slot[i] = nullptr; set_error("hipMalloc of a slot failed"); return LWO_ENOMEM; }
        LWO_HIP_TRY(hipEventCreateWithFlags(&s->copy_done[i], hipEventDisableTiming));
        LWO_HIP_TRY(hipEventCreateWithFlags(&s->compute_done[i], hipEventDisableTiming));
    }
    LWO_TRY(workspace_alloc(s->d, &s->ws));
    LWO_HIP_TRY(hipStreamCreateWithFlags(&s->copy, hipStreamNonBlocking));
    for (hipEvent_t& e : s->step_done) LWO_HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    LWO_TRY(prime_head(s));
    LWO_TRY(sync_transfers(s));
    return LWO_OK;
}

// Shared by the build calls: block b has descriptor types[block_type[b]].
static lwo_status build_store(const lwo_model_desc* types, int32_t n_types, const int32_t* block_type, int32_t n_blocks,
                              const lwo_block_source* src, int32_t host_mode, uint64_t register_budget,
                              int32_t device, lwo_store** out, int32_t group = 1, int32_t rank = 0) {
    if (!out) { set_error("out is NULL"); return LWO_EINVAL; }
    *out = nullptr;
    if (!types || n_types < 1 || !block_type || n_blocks < 1) { set_error("stack: types, block_type and n_blocks >= 1 required"); return LWO_EINVAL; }
    std::vector<lwo_model_desc> td(types, types + n_types);
    for (int t = 0; t < n_types; ++t) {
        td[t].n_blocks = n_blocks;
        LWO_TRY(validate_desc(&td[t]));
        const lwo_model_desc& a = td[0], &c = td[t];
        if (c.kind != a.kind || c.hidden != a.hidden || c.batch != a.batch || c.tokens != a.tokens ||
            c.ctx_tokens != a.ctx_tokens || c.act_dtype != a.act_dtype) {
            set_error("block type " + std::to_string(t) + " differs from type 0 in kind, hidden, batch, tokens, "
                      "ctx_tokens or act_dtype");
            return LWO_EINVAL;
        }
    }
    for (int b = 0; b < n_blocks; ++b)
        if (block_type[b] < 0 || block_type[b] >= n_types) { set_error("block_type[" + std::to_string(b) + "] out of range"); return LWO_EINVAL; }
    if (!src || (!src->extents && !src->fill)) { set_error("block source has neither extents nor fill"); return LWO_EINVAL; }
    if (host_mode != LWO_HOST_PIN_COPY && host_mode != LWO_HOST_REGISTER && host_mode != LWO_HOST_STAGED &&
        host_mode != LWO_HOST_SHARD) {
        set_error("host_mode");
        return LWO_EINVAL;
    }
    if (host_mode == LWO_HOST_SHARD && (n_types != 1 || group < 1 || group > 64 || rank < 0 || rank >= group)) {
        set_error("shard store: one block type, 1 <= group <= 64 and 0 <= rank < group required");
        return LWO_EINVAL;
    }
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) {
        set_error("device " + std::to_string(device) + " is not available");
        return LWO_EINVAL;
    }
    auto t0 = std::chrono::steady_clock::now();
    lwo_store* s = new (std::nothrow) lwo_store();
    if (!s) { set_error("out of host memory"); return LWO_ENOMEM; }
    // An exception part-way (host memory) must not leak the partial store either.
    lwo_status st = LWO_OK;
    try {
        s->tdesc = td;
        for (const lwo_model_desc& t : td) s->tlay.push_back(make_layout(t));
        s->btype.assign(block_type, block_type + n_blocks);
        s->d = td[0];
        for (const lwo_model_desc& t : td) {
            s->d.ffn = std::max(s->d.ffn, t.ffn);
            if (t.linear_dtype == LWO_FP8_E4M3) s->d.linear_dtype = LWO_FP8_E4M3;
        }
        uint64_t off = 0;
        for (int b = 0; b < n_blocks; ++b) {
            s->bext.push_back(s->tlay[block_type[b]].extent_bytes);
            // SHARD: the extent padded to group equal shards of whole pages
            const uint64_t unit = (uint64_t)group * 4096;
            s->dext.push_back(host_mode == LWO_HOST_SHARD ? (s->bext[b] + unit - 1) / unit * unit : s->bext[b]);
            s->roff.push_back(off);
            off += s->dext[b];
            s->max_ext = std::max(s->max_ext, s->dext[b]);
        }
        s->group = group;
        s->rank = rank;
        s->shard = s->dext[0] / group;
        s->device = device;
        s->host_mode = host_mode;
        st = build(s, src, host_mode, register_budget);
    } catch (...) {
        release(s);
        throw;
    }
    if (st != LWO_OK) {
        std::string msg;
        try {
            msg = lwo_last_error();
        } catch (...) {
        }
        release(s);   // fail closed: nothing of the partial build survives
        set_error(msg);
        return st;
    }
    s->build_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    *out = s;
    return LWO_OK;
}

extern "C" lwo_status lwo_build_block_store(const lwo_model_desc* desc, const lwo_block_source* src, int32_t host_mode,
                                            uint64_t register_budget, int32_t device, lwo_store** out) {
    try {
        clear_error();
        if (!out) { set_error("out is NULL"); return LWO_EINVAL; }
        *out = nullptr;
        LWO_TRY(validate_desc(desc));
        std::vector<int32_t> bt(desc->n_blocks, 0);
        return build_store(desc, 1, bt.data(), desc->n_blocks, src, host_mode, register_budget, device, out);
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_build_block_store");
    } catch (const std::exception& e) {
        return fail_exception("lwo_build_block_store", e.what());
    } catch (...) {
        return fail_exception("lwo_build_block_store", "unknown exception");
    }
}

extern "C" lwo_status lwo_build_mixed_store(const lwo_model_desc* types, int32_t n_types, const int32_t* block_type,
                                            int32_t n_blocks, const lwo_block_source* src, int32_t host_mode,
                                            uint64_t register_budget, int32_t device, lwo_store** out) {
    try {
        clear_error();
        return build_store(types, n_types, block_type, n_blocks, src, host_mode, register_budget, device, out);
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_build_mixed_store");
    } catch (const std::exception& e) {
        return fail_exception("lwo_build_mixed_store", e.what());
    } catch (...) {
        return fail_exception("lwo_build_mixed_store", "unknown exception");
    }
}

extern "C" lwo_status lwo_build_shard_store(const lwo_model_desc* desc, const lwo_block_source* src, int32_t group,
                                            int32_t rank, int32_t device, lwo_store** out) {
    try {
        clear_error();
        if (!out) { set_error("out is NULL"); return LWO_EINVAL; }
        *out = nullptr;
        LWO_TRY(validate_desc(desc));
        std::vector<int32_t> bt(desc->n_blocks, 0);
        return build_store(desc, 1, bt.data(), desc->n_blocks, src, LWO_HOST_SHARD, 0, device, out, group, rank);
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_build_shard_store");
    } catch (const std::exception& e) {
        return fail_exception("lwo_build_shard_store", e.what());
    } catch (...) {
        return fail_exception("lwo_build_shard_store", "unknown exception");
    }
}

extern "C" lwo_status lwo_destroy_block_store(lwo_store* s) {
    try {
        clear_error();
        release(s);
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_destroy_block_store");
    } catch (const std::exception& e) {
        return fail_exception("lwo_destroy_block_store", e.what());
    } catch (...) {
        return fail_exception("lwo_destroy_block_store", "unknown exception");
    }
}

// ------------------------------------------------------------------ resident prefix

extern "C" lwo_status lwo_set_resident_prefix(lwo_store* s, int32_t k) {
    try {
        clear_error();
        LWO_TRY(check_store(s));
        if (k < 0 || k > s->d.n_blocks) { set_error("resident prefix out of range"); return LWO_EINVAL; }
        LWO_HIP_TRY(hipSetDevice(s->device));
        LWO_TRY(sync_transfers(s));
        LWO_HIP_TRY(hipDeviceSynchronize());
        char* region = nullptr;
        if (k > 0) {
            const uint64_t bytes = s->roff[k - 1] + s->dext[k - 1];
            if (hipMalloc(&region, bytes) != hipSuccess) {
                set_error("hipMalloc of the resident region (" + std::to_string(bytes) + " bytes) failed");
                return LWO_ENOMEM;   // previous prefix stays in effect
            }
            for (int b = 0; b < k; ++b) {
                if (h2d_block(s, region + s->roff[b], b, nullptr) != LWO_OK) {
                    (void)sync_transfers(s);
                    (void)hipFree(region);
                    set_error("copy of resident block " + std::to_string(b) + " failed");
                    return LWO_EHIP;
                }
            }
            if (sync_transfers(s) != LWO_OK) {
                (void)hipFree(region);
                set_error("copy of the resident prefix failed");
                return LWO_EHIP;
            }
        }
        if (s->resident) (void)hipFree(s->resident);
        s->resident = region;
        s->k = k;
        LWO_TRY(prime_head(s));
        LWO_TRY(sync_transfers(s));
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_set_resident_prefix");
    } catch (const std::exception& e) {
        return fail_exception("lwo_set_resident_prefix", e.what());
    } catch (...) {
        return fail_exception("lwo_set_resident_prefix", "unknown exception");
    }
}

// ------------------------------------------------------------------ the step

static lwo_status validate_slot(lwo_store* s, const char* base, int block, hipStream_t st) {
    LWO_TRY(enqueue_zero_u64(s->ws.sums, 1, st));
    LWO_TRY(enqueue_checksum(base, s->bext[block], s->ws.sums, st));
    return enqueue_checksum_compare(s->ws.sums, s->host_sums[block], st);
}

static lwo_status run_step(lwo_store* s, void* x, const void* cond, const void* ctx, hipStream_t st) {
    const lwo_model_desc& d = s->d;
    const int n = d.n_blocks, k = s->k, m = n - k;
    auto run_block = [&](int b, const char* base) {
        const lwo_model_desc& bd = s->tdesc[s->btype[b]];
        return enqueue_block(bd, block_ptrs(s->tlay[s->btype[b]], bd, base), s->ws, cond, ctx, st, &s->kt);
    };
    LWO_TRY(enqueue_step_begin(d, s->ws, x, cond, ctx, st));
    for (int b = 0; b < k; ++b) {
        LWO_TRY(run_block(b, s->resident + s->roff[b]));
    }
    if (m > 0) {
        for (hipEvent_t e : s->tev) (void)hipEventDestroy(e);
        s->tev.clear();
        s->n_timed = 0;
        int cur = s->head_slot;
        for (int j = k; j < n; ++j) {
            if (s->slot_block[cur] != j) { set_error("ring state corrupted"); return LWO_ESTATE; }
            // RAW: the block's bytes must have landed before its kernels read them.
            LWO_HIP_TRY(hipStreamWaitEvent(st, s->copy_done[cur], 0));
            if (s->validation) LWO_TRY(validate_slot(s, s->slot[cur], j, st));
            // The block's kernels go in before the prefetch call: the runtime may
            // block the host inside hipMemcpyAsync when many copies are queued,
            // and the compute queue must not starve meanwhile.
            LWO_TRY(run_block(j, s->slot[cur]));
            LWO_HIP_TRY(hipEventRecord(s->compute_done[cur], st));
            int nxt = cur;
            if (m > 1) {
                const int nb = (j + 1 < n) ? j + 1 : k;   // circular: the last block prefetches block k
                nxt = 1 - cur;
                if (s->slot_block[nxt] != nb) {
                    // WAR: the alternate slot's previous block must have finished computing.
                    LWO_HIP_TRY(hipStreamWaitEvent(s->copy, s->compute_done[nxt], 0));
                    hipEvent_t e0 = nullptr, e1 = nullptr;
                    if (s->timing) {
                        LWO_HIP_TRY(hipEventCreate(&e0));
                        LWO_HIP_TRY(hipEventCreate(&e1));
                        s->tev.push_back(e0);
                        s->tev.push_back(e1);
                        s->n_timed++;
                    }
                    LWO_TRY(h2d_block(s, s->slot[nxt], nb, s->copy_done[nxt], e0, e1));
                    s->slot_block[nxt] = nb;
                }
            }
            cur = nxt;
        }
        s->head_slot = cur;   // the slot holding (or receiving) block k for the next step
    }
    LWO_TRY(enqueue_step_end(d, s->ws, x, st));
    LWO_HIP_TRY(hipEventRecord(s->step_done[s->steps % 16], st));
    s->steps++;
    return LWO_OK;
}

extern "C" lwo_status lwo_run_denoise_step(lwo_store* s, void* x, const void* cond, const void* ctx, void* hip_stream) {
    try {
        clear_error();
        LWO_TRY(check_store(s));
        if (!hip_stream) { set_error("run needs a non-null stream (the legacy null stream would serialise with the copy stream)"); return LWO_EINVAL; }
        if (!x || !cond) { set_error("x and cond are required"); return LWO_EINVAL; }
        if (s->d.kind == LWO_KIND_VIDEO && !ctx) { set_error("video kind needs ctx"); return LWO_EINVAL; }
        if (s->d.kind == LWO_KIND_DIT && ctx) { set_error("DiT kind takes no ctx"); return LWO_EINVAL; }
        LWO_HIP_TRY(hipSetDevice(s->device));
        if (s->max_inflight > 0 && s->steps >= (uint64_t)s->max_inflight)   // pacing: bound host run-ahead
            LWO_HIP_TRY(hipEventSynchronize(s->step_done[(s->steps - s->max_inflight) % 16]));
        lwo_status st = run_step(s, x, cond, ctx, (hipStream_t)hip_stream);
        if (st != LWO_OK) s->dead = true;   // the ring's events no longer describe the slots
        return st;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_run_denoise_step");
    } catch (const std::exception& e) {
        return fail_exception("lwo_run_denoise_step", e.what());
    } catch (...) {
        return fail_exception("lwo_run_denoise_step", "unknown exception");
    }
}

// ------------------------------------------------------------------ validation and stats

extern "C" lwo_status lwo_set_max_inflight(lwo_store* s, int32_t max_inflight) {
    try {
        clear_error();
        LWO_TRY(check_store(s));
        if (max_inflight < 0 || max_inflight > 16) { set_error("max_inflight must be 0..16"); return LWO_EINVAL; }
        s->max_inflight = max_inflight;
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_set_max_inflight");
    } catch (const std::exception& e) {
        return fail_exception("lwo_set_max_inflight", e.what());
    } catch (...) {
        return fail_exception("lwo_set_max_inflight", "unknown exception");
    }
}

extern "C" lwo_status lwo_set_validation(lwo_store* s, int32_t on) {
    try {
        clear_error();
        LWO_TRY(check_store(s));
        if (on) compute_host_sums(s);
        s->validation = on != 0;
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_set_validation");
    } catch (const std::exception& e) {
        return fail_exception("lwo_set_validation", e.what());
    } catch (...) {
        return fail_exception("lwo_set_validation", "unknown exception");
    }
}

extern "C" lwo_status lwo_set_copy_timing(lwo_store* s, int32_t on) {
    try {
        clear_error();
        LWO_TRY(check_store(s));
        s->timing = on != 0;
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_set_copy_timing");
    } catch (const std::exception& e) {
        return fail_exception("lwo_set_copy_timing", e.what());
    } catch (...) {
        return fail_exception("lwo_set_copy_timing", "unknown exception");
    }
}

extern "C" lwo_status lwo_copy_times(lwo_store* s, float* ms, int32_t cap, int32_t* n) {
    try {
        clear_error();
        LWO_TRY(check_store(s));
        LWO_HIP_TRY(hipSetDevice(s->device));
        LWO_TRY(sync_transfers(s));
        int cnt = s->n_timed;
        if (n) *n = cnt;
        for (int i = 0; i < cnt && i < cap && ms; ++i)
            LWO_HIP_TRY(hipEventElapsedTime(&ms[i], s->tev[2 * i], s->tev[2 * i + 1]));
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_copy_times");
    } catch (const std::exception& e) {
        return fail_exception("lwo_copy_times", e.what());
    } catch (...) {
        return fail_exception("lwo_copy_times", "unknown exception");
    }
}

extern "C" lwo_status lwo_block_checksum(lwo_store* s, int32_t block, uint64_t* host_sum, uint64_t* slot_sum) {
    try {
        clear_error();
        LWO_TRY(check_store(s));
        if (block < 0 || block >= s->d.n_blocks || !host_sum || !slot_sum) { set_error("bad block or output"); return LWO_EINVAL; }
        LWO_HIP_TRY(hipSetDevice(s->device));
        LWO_HIP_TRY(hipDeviceSynchronize());
        compute_host_sums(s);
        const uint64_t ext = s->bext[block];
        const char* base = nullptr;
        if (block < s->k) {
            base = s->resident + s->roff[block];
        } else if (s->slot_block[0] == block || s->slot_block[1] == block) {
            base = s->slot[s->slot_block[0] == block ? 0 : 1];
        } else {
            // borrow the slot the ring is not about to read
            int sl = 1 - s->head_slot;
            LWO_TRY(h2d_block(s, s->slot[sl], block, s->copy_done[sl]));
            LWO_HIP_TRY(hipStreamWaitEvent(s->copy, s->copy_done[sl], 0));
            s->slot_block[sl] = block;
            base = s->slot[sl];
        }
        LWO_TRY(enqueue_zero_u64(s->ws.sums, 1, s->copy));
        LWO_TRY(enqueue_checksum(base, ext, s->ws.sums, s->copy));
        uint64_t got = 0;
        LWO_HIP_TRY(hipMemcpyAsync(&got, s->ws.sums, 8, hipMemcpyDeviceToHost, s->copy));
        LWO_HIP_TRY(hipStreamSynchronize(s->copy));
        *host_sum = s->host_sums[block];
        *slot_sum = got;
        if (got != s->host_sums[block]) { set_error("slot checksum differs from the host extent"); return LWO_ECHECKSUM; }
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_block_checksum");
    } catch (const std::exception& e) {
        return fail_exception("lwo_block_checksum", e.what());
    } catch (...) {
        return fail_exception("lwo_block_checksum", "unknown exception");
    }
}

extern "C" lwo_status lwo_set_kernel_timing(lwo_store* s, int32_t on) {
    try {
        clear_error();
        LWO_TRY(check_store(s));
        LWO_HIP_TRY(hipSetDevice(s->device));
        LWO_HIP_TRY(hipDeviceSynchronize());
        s->kt.reset();
        s->kt.on = on != 0;
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_set_kernel_timing");
    } catch (const std::exception& e) {
        return fail_exception("lwo_set_kernel_timing", e.what());
    } catch (...) {
        return fail_exception("lwo_set_kernel_timing", "unknown exception");
    }
}

extern "C" lwo_status lwo_kernel_stats(lwo_store* s, lwo_kernel_stat* out, int32_t cap, int32_t* n) {
    try {
        clear_error();
        LWO_TRY(check_store(s));
        LWO_HIP_TRY(hipSetDevice(s->device));
        LWO_TRY(s->kt.collect());
        const int cnt = (int)s->kt.agg.size();
        if (n) *n = cnt;
        if (!out && cap == 0) return LWO_OK;   // count query
        if (cnt > cap || !out) { set_error("kernel_stats: capacity too small"); return LWO_EINVAL; }
        for (int i = 0; i < cnt; ++i) {
            const KernelTimer::Agg& a = s->kt.agg[i];
            std::memset(&out[i], 0, sizeof(out[i]));
            std::strncpy(out[i].name, a.name.c_str(), sizeof(out[i].name) - 1);
            out[i].launches = a.launches;
            out[i].total_ms = a.ms;
            out[i].flops = a.flops;
            out[i].bytes = a.bytes;
        }
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_kernel_stats");
    } catch (const std::exception& e) {
        return fail_exception("lwo_kernel_stats", e.what());
    } catch (...) {
        return fail_exception("lwo_kernel_stats", "unknown exception");
    }
}

extern "C" lwo_status lwo_get_stats(lwo_store* s, lwo_stats* o) {
    try {
        clear_error();
        if (!s || !o) { set_error("NULL argument"); return LWO_EINVAL; }
        LWO_HIP_TRY(hipSetDevice(s->device));
        LWO_HIP_TRY(hipDeviceSynchronize());
        std::memset(o, 0, sizeof(*o));
        const uint64_t ext = s->max_ext;
        uint64_t all = 0, big = 0;
        for (uint64_t e : s->bext) { all += e; big = std::max(big, e); }
        o->extent_bytes = big;
        o->slot_bytes = ext;
        o->device_weight_bytes = 2 * ext + (s->k ? s->roff[s->k - 1] + s->dext[s->k - 1] : 0);
        o->workspace_bytes = s->ws.bytes;
        o->host_bytes = s->host_mode == LWO_HOST_STAGED ? 0
                        : s->host_mode == LWO_HOST_SHARD ? (uint64_t)s->d.n_blocks * s->shard : all;
        o->group = s->group;
        o->rank = s->rank;
        o->shard_bytes = s->host_mode == LWO_HOST_SHARD ? s->shard : 0;
        o->gather_bytes = s->gather_bytes;
        o->peer_device_bytes = s->peer ? (uint64_t)s->d.n_blocks * (s->dext[0] - s->shard) : 0;
        o->staging_bytes = s->host_mode == LWO_HOST_STAGED ? 2 * ext : 0;
        o->pack_bytes = s->pack_bytes;
        o->pack_ms = s->pack_ms;
        o->pack_threads = s->host_mode == LWO_HOST_STAGED ? s->pack_threads + 1 : 0;
        o->h2d_copies = s->h2d_copies;
        o->h2d_bytes = s->h2d_bytes;
        o->steps = s->steps;
        uint64_t mism = 0;
        if (s->ws.sums) LWO_HIP_TRY(hipMemcpy(&mism, s->ws.sums + 1, 8, hipMemcpyDeviceToHost));
        o->checksum_mismatches = mism;
        o->registered_ranges = s->reg_base.size();
        for (uint64_t l : s->reg_len) o->registered_bytes += l;
        o->resident_prefix = s->k;
        o->head_slot = s->head_slot;
        o->host_mode = s->host_mode;
        o->validation = s->validation;
        o->build_ms = s->build_ms;
        return LWO_OK;
    } catch (const std::bad_alloc&) {
        return fail_alloc("lwo_get_stats");
    } catch (const std::exception& e) {
        return fail_exception("lwo_get_stats", e.what());
    } catch (...) {
        return fail_exception("lwo_get_stats", "unknown exception");
    }
}
