/*
 * lwo.h - C ABI of the layerwise weight-offload library for one MI355X GPU.
 *
 * A diffusion transformer's blocks keep their weights in host memory, one
 * flat extent per block, and are streamed into exactly two device slots by
 * hipMemcpyAsync on a dedicated copy stream; the copy of block i+1 overlaps
 * the forward of block i, and the last streamed block prefetches the first
 * one again.  Sources (pages of the offloader documentation of a diffusion
 * serving engine):
 *   [LW]  "CPU Offloading for Diffusion Models", section "Layerwise
 *         (Blockwise) Offloading / How It Works" and its execution-flow
 *         table (prefetch next block on a copy stream, last block prefetches
 *         block 0, flattened pinned host tensors).
 *   [DLO] "Distributed Layerwise Offload": "Components and ownership",
 *         "Startup and runtime sequence" (a pair of device buffers as large
 *         as the biggest streamed block, readiness events, prime the first
 *         block), "Registered runtime-cache transfer" (page-align, coalesce,
 *         budget check before mutation, read-only registration, all-or-
 *         nothing rollback, unregister before unmap), "Failure and lifecycle
 *         boundaries", "Feature compatibility" (resident leading layers,
 *         per-tensor fp8 linears).
 *   [ARCH] "CPU Offloading": "Shared lifecycle" (a failed enable leaves no
 *         partial state) and "Cross-strategy invariants" (device storage is
 *         not reused until dependent work completes).
 *
 * Conventions for every call:
 *   - returns lwo_status; LWO_OK is 0; no C++ exception crosses the ABI:
 *     host memory exhaustion inside a call returns LWO_ENOMEM, any other
 *     internal exception (e.g. a thread that cannot start) LWO_EIO;
 *   - on failure nothing is left half-built, and lwo_last_error() returns a
 *     thread-local message describing the last failure on this thread;
 *   - pointers documented as "device" are HIP device pointers on the
 *     store's device; "host" pointers are ordinary process memory;
 *   - a store is used from one host thread at a time.
 *
 * Block layout (shared with the flat extents the caller may provide): every
 * tensor starts at a multiple of 256 bytes, the extent is a multiple of 4096
 * bytes, gaps are zero.  Weight matrices ("*.w", [out, in]) are in the
 * linear dtype; biases, norm gains and modulation tables in the activation
 * dtype; with fp8 linears ten float32 per-tensor scales follow every other
 * tensor, in weight-matrix order.  lwo_block_layout() lists the tensors and
 * offsets.
 *
 * Tiled weights: a bf16 or fp8 matrix that a block GEMM multiplies (every
 * "*.w" except the DiT kind's "ada.w") is stored in tiles of 64 rows x 64
 * bytes (32 bf16 or 64 fp8 elements of a row), the order in which the GEMM
 * reads it.  For W [N, K] with R = K * element bytes per row (N a multiple
 * of 64, R of 64), the byte at row n, row byte c of the row-major matrix
 * sits at
 *     ((n / 64) * (R / 64) + c / 64) * 4096 + (n % 64) * 64 + c % 64,
 * so the tiles of one 64-row band follow each other along K, and a 64-row,
 * 64-byte stage of the GEMM is 4 KB of consecutive memory.  Row-major
 * matrices stacked along N (q|k|v) tile to the tiled stacked matrix.
 * lwo_block_layout() marks these tensors (tiled = 1); float32 matrices and
 * "ada.w" stay row-major.
 *
 * Block math (the workload's transformer block; LN is LayerNorm with eps
 * 1e-6 and no affine, GELU is the tanh form):
 *   DiT kind:   m = Lin_ada(SiLU(cond)) -> shift1 scale1 gate1 shift2 scale2 gate2
 *               x += gate1 * Lin_o(Attn(Lin_qkv(LN(x)(1+scale1)+shift1)))
 *               x += gate2 * Lin_fc2(GELU(Lin_fc1(LN(x)(1+scale2)+shift2)))
 *   video kind: m = cond + M_block (same six chunks); q and k pass through
 *               RMSNorm (eps 1e-6, gain) over the hidden width; after the
 *               self-attention branch an ungated cross-attention branch
 *               x += Lin_co(Attn(Lin_cq(LN(x)), Lin_ck(ctx), Lin_cv(ctx)));
 *               then the FFN branch as above.
 */
#ifndef LWO_H
#define LWO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lwo_status {
    LWO_OK = 0,
    LWO_EINVAL = 1,      /* bad argument, descriptor, alignment or size */
    LWO_ENOMEM = 2,      /* host or device allocation failed */
    LWO_EHIP = 3,        /* a HIP runtime call failed (message names it) */
    LWO_EBUDGET = 4,     /* registration needs more than the budget; nothing was registered */
    LWO_EREGISTER = 5,   /* a range failed to register; earlier ranges were rolled back */
    LWO_EROLLBACK = 6,   /* a rollback unregister failed: the process must not unmap the range */
    LWO_ESTATE = 7,      /* call not valid in the store's current state */
    LWO_ECHECKSUM = 8,   /* slot bytes differ from the host extent, or a cache entry from its digests */
    LWO_ETIMEOUT = 9,    /* a wait with a time limit expired (another writer holds a cache lock) */
    LWO_EIO = 10         /* a file, lock or mapping operation failed (message names it) */
} lwo_status;

typedef enum lwo_dtype { LWO_F32 = 0, LWO_BF16 = 1, LWO_FP8_E4M3 = 2 } lwo_dtype;
typedef enum lwo_block_kind { LWO_KIND_DIT = 0, LWO_KIND_VIDEO = 1 } lwo_block_kind;
/* Activation row layout of the single-kernel entry points (project addition,
 * a storage order only: no value changes).  LWO_ROWS: row-major with the
 * stated leading dimension.  LWO_KTILED: the tiled-weight order above applied
 * to activation rows, with R = leading dimension * element bytes (a multiple
 * of 64) and the rows rounded up to a multiple of 64: the byte at row m, row
 * byte c sits at ((m / 64) * (R / 64) + c / 64) * 4096 + (m % 64) * 64 +
 * c % 64.  The buffer spans ceil(M / 64) * 64 rows; the padding rows of the
 * last band are never read or written.  A denoise step writes the
 * activations that feed its bf16/fp8 linears in this order, so each
 * 64-byte GEMM stage of them is 4 KB of consecutive memory. */
typedef enum lwo_layout { LWO_ROWS = 0, LWO_KTILED = 1 } lwo_layout;
typedef enum lwo_host_mode {
    LWO_HOST_PIN_COPY = 0, LWO_HOST_REGISTER = 1, LWO_HOST_STAGED = 2,
    LWO_HOST_SHARD = 3     /* one rank's share of an all-gather group (lwo_build_shard_store) */
} lwo_host_mode;

/* Shape of the block stack and of one denoise step's activations.
 * Constraints (LWO_EINVAL otherwise): n_blocks >= 1; hidden = heads * head
 * dim with head dim in {64, 72, 128}; batch, tokens >= 1; video kind needs
 * ctx_tokens >= 1, DiT kind ctx_tokens = 0; act_dtype F32 or BF16;
 * linear_dtype equal to act_dtype, or FP8_E4M3 with act BF16 and the video
 * kind; hidden and ffn are multiples of 64 (of 128 with FP8 linears). */
typedef struct lwo_model_desc {
    int32_t kind;          /* lwo_block_kind */
    int32_t n_blocks;
    int32_t hidden;        /* D */
    int32_t heads;         /* H */
    int32_t ffn;           /* F */
    int32_t batch;         /* B */
    int32_t tokens;        /* T */
    int32_t ctx_tokens;    /* Tc (video kind) */
    int32_t act_dtype;     /* lwo_dtype */
    int32_t linear_dtype;  /* lwo_dtype */
} lwo_model_desc;

typedef struct lwo_tensor_info {
    char name[32];         /* e.g. "attn.q.w" */
    uint64_t offset;       /* byte offset inside the block extent */
    uint64_t bytes;
    int32_t rank;          /* 1 or 2 */
    int32_t shape[2];
    int32_t dtype;         /* lwo_dtype */
    int32_t tiled;         /* 1: stored in 64-row x 64-byte tiles (above); 0: row-major */
} lwo_tensor_info;

/* Where build takes each block's flat extent from.
 *   extents != NULL: extents[b] points to extent_bytes of host memory in the
 *     layout above.  PIN_COPY reads them during the call only.  REGISTER
 *     and STAGED borrow them until destroy (immutable, mapped until
 *     lwo_destroy_block_store returns; REGISTER needs them page-aligned).
 *   extents == NULL (PIN_COPY only): fill(user, b, dst, extent_bytes) is
 *     called once per block, in order, to write block b's extent into the
 *     store's pinned host memory dst (e.g. with lwo_pack_block); a non-zero
 *     return aborts the build with LWO_EINVAL. */
typedef struct lwo_block_source {
    const void* const* extents;
    int32_t (*fill)(void* user, int32_t block, void* dst, uint64_t extent_bytes);
    void* user;
} lwo_block_source;

typedef struct lwo_stats {
    uint64_t extent_bytes;       /* bytes of one block extent (the largest, for a mixed stack) */
    uint64_t slot_bytes;         /* bytes of each of the two device slots */
    uint64_t device_weight_bytes;/* resident prefix + two slots */
    uint64_t workspace_bytes;    /* activation workspace on the device */
    uint64_t host_bytes;         /* pinned or registered host bytes */
    uint64_t h2d_copies;         /* hipMemcpyAsync calls issued for blocks (total) */
    uint64_t h2d_bytes;          /* bytes those copies moved (total) */
    uint64_t steps;              /* denoise steps run */
    uint64_t checksum_mismatches;/* validation mode: blocks whose slot checksum differed */
    uint64_t registered_ranges;  /* REGISTER mode: coalesced ranges registered */
    uint64_t registered_bytes;
    int32_t resident_prefix;     /* k */
    int32_t head_slot;           /* slot holding (or receiving) block k */
    int32_t host_mode;           /* lwo_host_mode in effect */
    int32_t validation;          /* 1 if per-block checksums run before each block */
    double build_ms;             /* wall time of lwo_build_block_store */
    uint64_t staging_bytes;      /* STAGED: the two pinned staging slots */
    uint64_t pack_bytes;         /* STAGED: bytes packed host -> staging (total) */
    double pack_ms;              /* STAGED: host wall time spent packing (total) */
    int32_t pack_threads;        /* STAGED: threads that pack one extent */
    int32_t reserved;
    int32_t group;               /* SHARD: all-gather group size (1 otherwise) */
    int32_t rank;                /* SHARD: this store's rank in the group (0 otherwise) */
    uint64_t shard_bytes;        /* SHARD: bytes of one block's shard (the extent padded to group * 4096, / group) */
    uint64_t gather_bytes;       /* SHARD: bytes the gather stand-in copied into slots (total) */
    uint64_t peer_device_bytes;  /* SHARD: device bytes of the region standing in for the other ranks' shards */
} lwo_stats;

/* --- layout and packing (host only, no GPU needed) ---------------------- */

/* Tensor table of one block for desc: writes up to cap entries to out (out
 * may be NULL with cap 0 to query), the count to *n and the extent size to
 * *extent_bytes.  LWO_EINVAL if cap is too small (count is still written).
 * Source: [LW] flattened per-block host tensors; [DLO] "Registered
 * runtime-cache transfer" (each tensor at an offset of one flat buffer). */
lwo_status lwo_block_layout(const lwo_model_desc* desc, lwo_tensor_info* out, int32_t cap,
                            int32_t* n, uint64_t* extent_bytes);

/* Flatten one block: tensors[i] (host, float32, row-major, in the order of
 * lwo_block_layout, excluding the fp8 scale table) are converted to their
 * stored dtype and written at their offsets in dst (host, dst_bytes >=
 * extent_bytes), tiled where the table says so; padding is zeroed.  bf16 rounds to nearest-even; fp8 uses
 * one scale per tensor, s = amax|w| / 448 (1 for an all-zero tensor), codes
 * = e4m3(w / s) rounded to nearest-even and saturated, and the scales go to
 * "linear.scales".  Source: [DLO] "Feature compatibility" (per-tensor fp8
 * linears finalised before offload); [LW] flattened tensors. */
lwo_status lwo_pack_block(const lwo_model_desc* desc, const float* const* tensors, int32_t n_tensors,
                          void* dst, uint64_t dst_bytes);

/* Rearrange a row-major weight [N, K] of dtype BF16 or FP8_E4M3 (host, N * K
 * elements) into the tiled order above (host dst, the same size, not
 * overlapping src), the form lwo_op_linear takes.  LWO_EINVAL for another
 * dtype, N not a multiple of 64, K * element bytes not a multiple of 64, or a
 * null pointer. */
lwo_status lwo_tile_weight(int32_t dtype, const void* src, int32_t N, int32_t K, void* dst);

/* Position-weighted SplitMix64 sum over a host buffer (bytes % 8 == 0):
 * sum_i SplitMix64(w_i ^ (i * 0x9E3779B97F4A7C15)) mod 2^64 over the
 * little-endian 64-bit words w_i.  The device computes the same sum over a
 * slot.  Writes *sum. */
lwo_status lwo_extent_checksum(const void* host, uint64_t bytes, uint64_t* sum);

/* --- registration lifecycle (host only; the callbacks make it testable) -- */

typedef int32_t (*lwo_register_fn)(void* user, void* base, uint64_t bytes);   /* 0 = success */
typedef int32_t (*lwo_unregister_fn)(void* user, void* base);                /* 0 = success */

/* [DLO] "Registered runtime-cache transfer" and "Failure and lifecycle
 * boundaries": page-align each [ptr, ptr+bytes) outward to `page`, coalesce
 * overlapping or adjacent ranges, check the total against budget before
 * calling reg at all (LWO_EBUDGET, no calls), then call reg on each range in
 * address order.  If reg fails on a range, every range already registered is
 * passed to unreg in reverse order and LWO_EREGISTER is returned; if an
 * unreg fails during that rollback, LWO_EROLLBACK is returned and the
 * remaining ranges stay registered (the caller must not unmap them).  On
 * success the coalesced ranges are written to out_base/out_len (cap
 * entries; LWO_EINVAL before any reg call if cap is too small) and their
 * count to *n_out. */
lwo_status lwo_register_ranges(const void* const* ptrs, const uint64_t* bytes, int32_t n, uint64_t page,
                               uint64_t budget, lwo_register_fn reg, lwo_unregister_fn unreg, void* user,
                               uint64_t* out_base, uint64_t* out_len, int32_t cap, int32_t* n_out);

/* --- persisted flat-block files (host only, no GPU needed) --------------
 * [DLO] "Runtime cache": one content-addressed entry per block stack,
 * published atomically, mapped read-only as the host backing of a store.
 * Entry <dir>/<key>/ holds blocks.bin (block b's extent at b * stride, stride
 * = extent_bytes rounded up to 4096, zero padded, so every extent is
 * page-aligned in the mapping) and manifest.json (format, descriptor, tensor
 * table, per-block SHA-256 digests, content digest).  The key is the
 * lower-case hex SHA-256 of the canonical layout text followed by the 32-byte
 * block digests in order. */

typedef struct lwo_cache lwo_cache;   /* an open, validated, mapped entry */

/* FIPS 180-4 SHA-256 of bytes at data into out32[32]. */
lwo_status lwo_sha256(const void* data, uint64_t bytes, uint8_t* out32);

/* Publish the stack read from src (extents, or fill called twice per block:
 * once to hash, once to write) under dir, creating dir if needed.  Takes an
 * exclusive flock on <dir>/<key>.lock, polling up to wait_ms
 * (LWO_ETIMEOUT).  If the entry exists it is joined (*created = 0).
 * Otherwise temporaries <dir>/.tmp-<key>-* left by dead writers are removed,
 * the files are written and fsynced in a fresh temporary directory, which is
 * renamed to <dir>/<key> (*created = 1).  key_out receives the key
 * (65 bytes with the terminating NUL).  On error nothing is published. */
lwo_status lwo_cache_publish(const char* dir, const lwo_model_desc* desc, const lwo_block_source* src,
                             uint32_t wait_ms, char* key_out, int32_t* created);

/* Open <dir>/<key>: the manifest must describe desc's layout (LWO_EINVAL
 * otherwise) and its digests must give the key (LWO_ECHECKSUM);
 * blocks.bin is mapped read-only and shared; with verify != 0 every block's
 * SHA-256 is recomputed from the mapping (LWO_ECHECKSUM on a mismatch). */
lwo_status lwo_cache_open(const char* dir, const char* key, const lwo_model_desc* desc, int32_t verify,
                          lwo_cache** out);

/* The n_blocks extent pointers inside the mapping (page-aligned, valid until
 * lwo_cache_close); out == NULL and cap == 0 only sets *n. */
lwo_status lwo_cache_extents(const lwo_cache* cache, const void** out, int32_t cap, int32_t* n);

/* Unmap and close.  A store built on the extents must be destroyed first. */
lwo_status lwo_cache_close(lwo_cache* cache);

/* --- the store ----------------------------------------------------------- */

typedef struct lwo_store lwo_store;   /* opaque */

/* [LW], [DLO] "Startup and runtime sequence": set up the host weight store
 * (PIN_COPY: one hipHostMalloc extent per block filled from src; REGISTER:
 * the caller's extents registered read-only through lwo_register_ranges with
 * hipHostRegister, all-or-nothing within register_budget bytes; STAGED, see
 * below), the device
 * arena (two slots of extent_bytes; no resident prefix), the activation
 * workspace, a non-blocking copy stream at default priority and the
 * readiness events, then prime block 0 into slot 0.  On `device` (HIP
 * ordinal).  On any failure everything allocated so far is released and
 * *out is NULL.
 * [DLO] "Host backing and transfer composition", "Runtime cache": STAGED
 * borrows the caller's pageable extents (e.g. an mmap of a flat block file)
 * and allocates two pinned staging slots of extent_bytes; every block copy
 * first waits until the device copy last issued from the next staging slot
 * has finished, packs the extent into it on the host (split over
 * pack_threads threads; the calling thread blocks meanwhile) and then copies
 * it to the device on the copy stream.  REGISTER with register_budget == 0,
 * or whose registration fails and is rolled back (LWO_EBUDGET,
 * LWO_EREGISTER), continues as STAGED; lwo_stats.host_mode reports the mode
 * in effect.  A failed rollback (LWO_EROLLBACK) still fails the build. */
lwo_status lwo_build_block_store(const lwo_model_desc* desc, const lwo_block_source* src,
                                 int32_t host_mode, uint64_t register_budget, int32_t device,
                                 lwo_store** out);

/* [LW] "How It Works" (models with several block types, streamed through
 * the same slots) and [DLO] "Startup and runtime sequence" (slots sized for
 * the largest streamed block): a stack of n_blocks blocks where block b has
 * descriptor types[block_type[b]] (its n_blocks field is ignored).  All types
 * share kind, hidden, batch, tokens, ctx_tokens and act_dtype (LWO_EINVAL
 * otherwise, checked before any device call); heads, ffn and linear_dtype
 * may differ.  Each block's extent has its own type's layout and size
 * (lwo_block_layout of the type); extents[b] / fill(.., b, .., bytes) use
 * that size.  The slots and staging slots hold the largest extent, the
 * resident region the sum of the prefix's extents, the workspace the largest
 * ffn.  Otherwise as lwo_build_block_store, which is the one-type case. */
lwo_status lwo_build_mixed_store(const lwo_model_desc* types, int32_t n_types, const int32_t* block_type,
                                 int32_t n_blocks, const lwo_block_source* src, int32_t host_mode,
                                 uint64_t register_budget, int32_t device, lwo_store** out);

/* [DLO] "AllGather path" and "Host backing and transfer composition" (the
 * row for ordinary runtime tensors with a group larger than one): one rank's
 * share of the sharded ring, on one GPU.  Each block's extent is padded with
 * zeros to a multiple of group * 4096 bytes (shard_bytes = padded / group;
 * shards cut across tensor boundaries) and rank `rank` keeps only shard
 * `rank` of every block in pinned host memory: about extent / group bytes
 * per block.  The ring is lwo_build_block_store's, with one change per
 * streamed block: the copy stream copies the rank's shard host -> device to
 * its offset rank * shard_bytes of the slot, and a second (gather) stream
 * waits for that copy and then completes the slot with the other group - 1
 * shards, the all-gather's result.  On one GPU the shards the peers would
 * send over the all-gather come from a device region holding them
 * (peer_device_bytes = n_blocks * (padded - shard_bytes)), copied device to
 * device; the compute stream waits for the gather's event exactly as it
 * waits for a whole-block copy.  Host -> device bytes per step are thus
 * n_streamed * shard_bytes (lwo_stats.h2d_bytes counts those only;
 * gather_bytes the rest).  With group 1 the one shard is the whole extent and
 * nothing is gathered.
 *   src: the caller's extents (read during the call) or fill (called once per
 *        block, in order, with a scratch extent of extent_bytes), as for
 *        PIN_COPY; each extent is read once, checksummed for validation and
 *        split.
 *   LWO_EINVAL: group outside [1, 64], rank outside [0, group), or as
 *   lwo_build_block_store.  Everything else (resident prefix, validation,
 *   timing, stats, destroy) works as for the other host modes; copy timing
 *   covers the shard's host -> device copy. */
lwo_status lwo_build_shard_store(const lwo_model_desc* desc, const lwo_block_source* src, int32_t group,
                                 int32_t rank, int32_t device, lwo_store** out);

/* [DLO] "Feature compatibility" (resident leading layers): keep blocks
 * 0..k-1 in a device-resident region and stream blocks k..n_blocks-1
 * through the two slots (0 <= k <= n_blocks; k = n_blocks streams nothing).
 * Synchronises the store's streams, reallocates the resident region, copies
 * the prefix and primes block k into slot 0.  The two slots stay allocated.
 * On failure the previous prefix stays in effect. */
lwo_status lwo_set_resident_prefix(lwo_store* store, int32_t k);

/* One denoise step over every block, enqueued on hip_stream (a non-null
 * hipStream_t of the store's device) and returned without waiting:
 *   x    device, [batch, tokens, hidden] in act_dtype, updated in place;
 *   cond device, DiT kind [batch, hidden], video kind [batch, 6, hidden],
 *        act_dtype;
 *   ctx  device, [batch, ctx_tokens, hidden] act_dtype (video kind), NULL
 *        for the DiT kind.
 * Blocks run in order: the resident prefix, then the ring over blocks
 * k..n-1 where, for each streamed block j, the compute stream waits for
 * slot(j)'s copy event, the copy stream waits until the other slot's last
 * block has finished computing and then copies the next block (j+1, or k
 * after the last) into it ([LW] execution-flow table; [DLO] readiness
 * events; [ARCH] no reuse before dependent work completes).  With a single
 * streamed block it stays in its slot and nothing is copied.  The last
 * prefetch stays in flight across calls.  Caller keeps x, cond, ctx valid
 * until the stream drains.  Device faults surface as LWO_EHIP at a later
 * synchronising call.
 * Pacing: before enqueuing, the call waits on the host until at most
 * max_inflight - 1 earlier steps of this store are still executing (default
 * max_inflight 1: the previous step has finished).  The next step's first
 * block is already in its slot (the circular prefetch), so the device does
 * not idle; unbounded host run-ahead measured slower on MI355X (queued
 * cross-stream waits stall the copy engine). */
lwo_status lwo_run_denoise_step(lwo_store* store, void* x, const void* cond, const void* ctx,
                                void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one
 * denoise step over n_blocks device-resident block extents, with the same
 * kernels, in the same order, as lwo_run_denoise_step with every block
 * resident, and no allocation of any kind on the device.
 *   blocks  n_blocks device pointers (256-byte aligned), block b's extent in
 *           the layout of lwo_block_layout(desc) (e.g. lwo_pack_block's bytes
 *           copied to the device); caller-owned, read only;
 *   x, cond, ctx as for lwo_run_denoise_step (x updated in place);
 *   hip_stream a non-null stream; the call runs on that stream's device
 *           (made current during the call; the caller's current device is
 *           restored before it returns).
 * The step's activation workspace lives in a file-scope device array of
 * LWO_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends.  Every call on one GPU uses that GPU's one array
 * and leaves its contents behind: calls that overlap on one GPU (two streams,
 * or two threads) race and corrupt each other's results; serialise them.
 * LWO_EINVAL if the descriptor's workspace (it grows with batch * tokens *
 * max(3 * hidden, ffn)) exceeds the array, for a bad pointer or a NULL
 * stream, before anything is enqueued.  Nothing is synchronised. */
#define LWO_NOALLOC_SCRATCH_BYTES (64ull << 20)
lwo_status lwo_run_blocks_noalloc(const lwo_model_desc* desc, const void* const* blocks, int32_t n_blocks, void* x,
                                  const void* cond, const void* ctx, void* hip_stream);

/* Set the pacing depth of lwo_run_denoise_step (1..16, or 0 for no host
 * wait at all). */
lwo_status lwo_set_max_inflight(lwo_store* store, int32_t max_inflight);

/* Validation mode (on != 0): before each streamed block the compute stream
 * checksums the slot on the device and compares it with the host extent's
 * sum taken at build; mismatches are counted in lwo_stats.
 * Source: [ARCH] "Cross-strategy invariants" (while a parameter is offloaded
 * its host copy is the single authoritative one, so a slot must hold exactly
 * those bytes); the checksum itself is a project addition (the pages name no
 * check), a position-weighted SplitMix64 sum (lwo_extent_checksum). */
lwo_status lwo_set_validation(lwo_store* store, int32_t on);

/* Synchronise, copy block `block` into a slot (or use its resident copy),
 * checksum it on the device and compare with the host extent's checksum.
 * Writes both sums; LWO_ECHECKSUM if they differ.  Leaves the ring primed
 * as it was.  Source: as lwo_set_validation ([ARCH] "Cross-strategy
 * invariants"); a project addition for checking one block on demand. */
lwo_status lwo_block_checksum(lwo_store* store, int32_t block, uint64_t* host_sum, uint64_t* slot_sum);

/* Per-copy timing: when on, every block copy is bracketed by timing events on
 * the copy stream; lwo_copy_times returns the durations (ms) of the copies
 * issued by the most recent step (after synchronising), up to cap, count in
 * *n. */
lwo_status lwo_set_copy_timing(lwo_store* store, int32_t on);
lwo_status lwo_copy_times(lwo_store* store, float* ms, int32_t cap, int32_t* n);

/* Per-kernel timing: when on, every kernel a step enqueues for a block is
 * bracketed by timing events on the compute stream.  lwo_kernel_stats
 * synchronises and returns, per kernel (one entry per kernel symbol), the
 * launches, their total duration and their total algorithmic flops and HBM
 * bytes since timing was switched on (or last reset by on = 1 again).  cap
 * entries at most (out may be NULL with cap 0 to query the count); count in
 * *n (LWO_EINVAL if cap is too small). */
typedef struct lwo_kernel_stat {
    char name[48];
    uint64_t launches;
    double total_ms;
    double flops;          /* algorithmic: 2MNK per GEMM, 4 B H Tq Tk d per attention */
    double bytes;          /* algorithmic HBM bytes: operands read once, results written once */
} lwo_kernel_stat;

lwo_status lwo_set_kernel_timing(lwo_store* store, int32_t on);
lwo_status lwo_kernel_stats(lwo_store* store, lwo_kernel_stat* out, int32_t cap, int32_t* n);

/* Synchronise the store's copy stream and snapshot its counters.  A project
 * addition: the pages publish no figures ([DLO] "Validation status": hardware
 * and performance claims need fresh measurements), and these counters (bytes
 * copied per step, host and device residency, the host mode in effect after
 * a registration fallback, [DLO] "Host backing and transfer composition")
 * are what such measurements read. */
lwo_status lwo_get_stats(lwo_store* store, lwo_stats* out);

/* [DLO] "Failure and lifecycle boundaries": synchronise outstanding device
 * work, unregister host ranges (REGISTER mode), free pinned host memory, the
 * arena, workspace, events and copy stream.  NULL is a no-op.  In REGISTER
 * mode the caller may unmap its extents once this returns. */
lwo_status lwo_destroy_block_store(lwo_store* store);

/* --- single kernels ------------------------------------------------------
 * The kernels a denoise step enqueues, callable one at a time on `stream`
 * (device pointers; nothing is synchronised).  They let a caller compose its
 * own block or check one kernel at full size.  Arguments are validated
 * before launch (LWO_EINVAL: null or misaligned pointer, a leading dimension
 * smaller than the row, an unsupported size); device pointers must be
 * 16-byte aligned and leading dimensions multiples of 8 elements. */

/* Linear layer Y = A W^T + bias with a fused epilogue (the workload's
 * Linear(out, in) with weight [N, K]):
 *   epilogue 0: out[m, n] = Y               1: out[m, n] = GELU_tanh(Y)
 *            2: xr[m, n] += gate[(m / rows_per_gate) * gate_ld + n] * Y
 *            3: xr[m, n] += Y
 * dtype F32: A, W, bias, out float32.  BF16: A, W, bias, out bf16.
 * FP8_E4M3: A and W e4m3 codes, Y = (A W^T) * w_scale[n / w_seg] *
 * a_scale[m] + bias with bias and out bf16.  xr and gate are float32.
 * K must be a multiple of 16 (F32), 64 (BF16) or 128 (FP8); lda = K.  W is
 * row-major (ldw = K) for F32 and tiled (the block layout's tiled weights,
 * lwo_tile_weight) for BF16 and FP8, with N a multiple of 64.  a_layout: A
 * in LWO_ROWS or (BF16, FP8) LWO_KTILED order; out_layout: `out` of
 * epilogues 0 and 1 in LWO_ROWS or (BF16, FP8; ldo a multiple of 32)
 * LWO_KTILED order. */
lwo_status lwo_op_linear(int32_t dtype, int32_t epilogue, const void* a, const float* a_scale, const void* w,
                         const float* w_scale, int32_t w_seg, const void* bias, int32_t M, int32_t N, int32_t K,
                         void* out, int32_t ldo, float* xr, int32_t ldx, const float* gate, int32_t gate_ld,
                         int32_t rows_per_gate, int32_t a_layout, int32_t out_layout, void* stream);

/* Softmax attention without a mask, per batch b and head h:
 * O[b, t, h*d:(h+1)*d] = softmax(Q_bh K_bh^T / sqrt(d)) V_bh, rows of Q/O at
 * b*Tq + t, rows of K/V at b*Tk + t, head h in columns [h*d, (h+1)*d).
 * dtype F32 or BF16 for q, k, v, o; head_dim 64, 72 or 128.  o_layout:
 * LWO_ROWS, or LWO_KTILED (BF16, ldo a multiple of 32; rows b*Tq + t). */
lwo_status lwo_op_attention(int32_t dtype, const void* q, int32_t ldq, const void* k, int32_t ldk, const void* v,
                            int32_t ldv, void* o, int32_t ldo, int32_t batch, int32_t heads, int32_t tq,
                            int32_t tk, int32_t head_dim, int32_t o_layout, void* stream);

/* Row LayerNorm (eps 1e-6, no affine) of float32 x [M, D] (row stride D);
 * with mod ([B, 6, D] float32, b = row / rows_per_batch) the result is
 * LN(x)(1 + mod[b, scale_chunk]) + mod[b, shift_chunk].  out_dtype F32/BF16
 * writes out [M, D]; FP8_E4M3 writes e4m3 codes to out and per-row scales
 * amax/448 to out_scale (codes = e4m3(y * 448 / amax), float32 arithmetic).
 * out_layout: LWO_ROWS, or LWO_KTILED for BF16/FP8 rows of a multiple of 64
 * bytes (scales stay one float per row). */
lwo_status lwo_op_layernorm(const float* x, int32_t M, int32_t D, int32_t rows_per_batch, const float* mod,
                            int32_t shift_chunk, int32_t scale_chunk, void* out, int32_t out_dtype,
                            float* out_scale, int32_t out_layout, void* stream);

/* bf16 rows [M, N] (row-major) -> e4m3 codes [M, N] and per-row scales (as
 * above); codes_layout LWO_ROWS, or LWO_KTILED with N a multiple of 64. */
lwo_status lwo_op_quantize_rows(const void* in, int32_t M, int32_t N, uint8_t* codes, float* scales,
                                int32_t codes_layout, void* stream);

/* In place on rows of width 3D (q | k | v): q <- RMSNorm(q) * gq and
 * k <- RMSNorm(k) * gk over the D features (eps 1e-6); dtype F32 or BF16. */
lwo_status lwo_op_rmsnorm_qk(int32_t dtype, void* qkv, int32_t M, int32_t D, const void* gq, const void* gk,
                             void* stream);

/* Dense MFMA throughput probe.  It is a measurement, not a step of the
 * method: block kernels are set against the published dense peak and, for
 * context, against what the matrix cores sustain at the clock they run at
 * under full load.  It enqueues `blocks` workgroups of 256 threads (4 or more
 * per CU fill every SIMD).  Each wavefront runs 4 * iters independent MFMAs
 * on register operands: dtype BF16 uses v_mfma_f32_32x32x16_bf16 (32768
 * flops each), FP8_E4M3 uses v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales
 * (131072 flops each).  `sink` (device, caller-owned, at least blocks * 256
 * floats) receives one float per thread.  *flops returns the launch's flop
 * count; the caller divides it by the time it measures on `stream`.
 * LWO_EINVAL for another dtype, blocks outside [1, 65536], iters outside
 * [1, 10^6], a short or misaligned sink, or a NULL stream. */
lwo_status lwo_probe_mfma(int32_t dtype, int32_t blocks, int32_t iters, float* sink, uint64_t sink_floats, void* stream,
                          double* flops);

/* Thread-local description of the last failure ("" if none).  A project
 * addition: [DLO] "Failure and lifecycle boundaries" and [ARCH] "Shared
 * lifecycle" require failures to surface without partial state; the status
 * code says which failure, this text says where. */
const char* lwo_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LWO_H */
