"""ctypes marshalling for liblwo.so (see include/lwo.h for every contract)."""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
import weakref

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblwo.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -m layerwise_weight_offload_amd.build "
                      f"or __graft_entry__.build()); there is no fallback implementation")

# PyTorch ships its own HIP runtime library.  When it is installed, load it
# before liblwo.so so that the library binds to that same runtime: a process
# that uses both (tests, bench.py) then has one HIP runtime whichever package
# it imports first.  Two runtimes in one process do not share devices.  The
# binding uses nothing from PyTorch.
try:
    import torch  # noqa: F401
except ImportError:
    pass

_lib = C.CDLL(LIB_PATH)

# enums (include/lwo.h)
F32, BF16, FP8_E4M3 = 0, 1, 2
ROWS, KTILED = 0, 1   # lwo_layout
KIND_DIT, KIND_VIDEO = 0, 1
HOST_PIN_COPY, HOST_REGISTER, HOST_STAGED, HOST_SHARD = 0, 1, 2, 3
STATUS = {0: "LWO_OK", 1: "LWO_EINVAL", 2: "LWO_ENOMEM", 3: "LWO_EHIP", 4: "LWO_EBUDGET",
          5: "LWO_EREGISTER", 6: "LWO_EROLLBACK", 7: "LWO_ESTATE", 8: "LWO_ECHECKSUM", 9: "LWO_ETIMEOUT",
          10: "LWO_EIO"}

DTYPES = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}


class LwoError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class _Desc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("kind", "n_blocks", "hidden", "heads", "ffn", "batch", "tokens",
                                         "ctx_tokens", "act_dtype", "linear_dtype")]


class _TensorInfo(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("offset", C.c_uint64), ("bytes", C.c_uint64), ("rank", C.c_int32),
                ("shape", C.c_int32 * 2), ("dtype", C.c_int32), ("tiled", C.c_int32)]


_FILL = C.CFUNCTYPE(C.c_int32, C.c_void_p, C.c_int32, C.c_void_p, C.c_uint64)
_REG = C.CFUNCTYPE(C.c_int32, C.c_void_p, C.c_void_p, C.c_uint64)
_UNREG = C.CFUNCTYPE(C.c_int32, C.c_void_p, C.c_void_p)


class _Source(C.Structure):
    _fields_ = [("extents", C.POINTER(C.c_void_p)), ("fill", _FILL), ("user", C.c_void_p)]


class _Stats(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in ("extent_bytes", "slot_bytes", "device_weight_bytes", "workspace_bytes",
                                          "host_bytes", "h2d_copies", "h2d_bytes", "steps", "checksum_mismatches",
                                          "registered_ranges", "registered_bytes")] + \
               [(n, C.c_int32) for n in ("resident_prefix", "head_slot", "host_mode", "validation")] + \
               [("build_ms", C.c_double), ("staging_bytes", C.c_uint64), ("pack_bytes", C.c_uint64),
                ("pack_ms", C.c_double), ("pack_threads", C.c_int32), ("reserved", C.c_int32),
                ("group", C.c_int32), ("rank", C.c_int32), ("shard_bytes", C.c_uint64), ("gather_bytes", C.c_uint64),
                ("peer_device_bytes", C.c_uint64)]


class _KStat(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_uint64), ("total_ms", C.c_double), ("flops", C.c_double),
                ("bytes", C.c_double)]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_P = C.c_void_p
_lib_block_layout = _sig("lwo_block_layout", C.c_int, C.POINTER(_Desc), C.POINTER(_TensorInfo), C.c_int32,
                         C.POINTER(C.c_int32), C.POINTER(C.c_uint64))
_lib_pack_block = _sig("lwo_pack_block", C.c_int, C.POINTER(_Desc), C.POINTER(C.c_void_p), C.c_int32, _P, C.c_uint64)
_lib_tile_weight = _sig("lwo_tile_weight", C.c_int, C.c_int32, _P, C.c_int32, C.c_int32, _P)
_lib_extent_checksum = _sig("lwo_extent_checksum", C.c_int, _P, C.c_uint64, C.POINTER(C.c_uint64))
_lib_register_ranges = _sig("lwo_register_ranges", C.c_int, C.POINTER(C.c_void_p), C.POINTER(C.c_uint64), C.c_int32,
                            C.c_uint64, C.c_uint64, _REG, _UNREG, _P, C.POINTER(C.c_uint64),
                            C.POINTER(C.c_uint64), C.c_int32, C.POINTER(C.c_int32))
_lib_build = _sig("lwo_build_block_store", C.c_int, C.POINTER(_Desc), C.POINTER(_Source), C.c_int32, C.c_uint64,
                  C.c_int32, C.POINTER(_P))
_lib_build_mixed = _sig("lwo_build_mixed_store", C.c_int, C.POINTER(_Desc), C.c_int32, C.POINTER(C.c_int32), C.c_int32,
                        C.POINTER(_Source), C.c_int32, C.c_uint64, C.c_int32, C.POINTER(_P))
_lib_build_shard = _sig("lwo_build_shard_store", C.c_int, C.POINTER(_Desc), C.POINTER(_Source), C.c_int32, C.c_int32,
                        C.c_int32, C.POINTER(_P))
_lib_run_noalloc = _sig("lwo_run_blocks_noalloc", C.c_int, C.POINTER(_Desc), C.POINTER(C.c_void_p), C.c_int32, _P, _P,
                        _P, _P)
_lib_set_prefix = _sig("lwo_set_resident_prefix", C.c_int, _P, C.c_int32)
_lib_run = _sig("lwo_run_denoise_step", C.c_int, _P, _P, _P, _P, _P)
_lib_set_validation = _sig("lwo_set_validation", C.c_int, _P, C.c_int32)
_lib_set_max_inflight = _sig("lwo_set_max_inflight", C.c_int, _P, C.c_int32)
_lib_block_checksum = _sig("lwo_block_checksum", C.c_int, _P, C.c_int32, C.POINTER(C.c_uint64), C.POINTER(C.c_uint64))
_lib_set_copy_timing = _sig("lwo_set_copy_timing", C.c_int, _P, C.c_int32)
_lib_copy_times = _sig("lwo_copy_times", C.c_int, _P, C.POINTER(C.c_float), C.c_int32, C.POINTER(C.c_int32))
_lib_get_stats = _sig("lwo_get_stats", C.c_int, _P, C.POINTER(_Stats))
_lib_set_kernel_timing = _sig("lwo_set_kernel_timing", C.c_int, _P, C.c_int32)
_lib_kernel_stats = _sig("lwo_kernel_stats", C.c_int, _P, C.POINTER(_KStat), C.c_int32, C.POINTER(C.c_int32))
_lib_destroy = _sig("lwo_destroy_block_store", C.c_int, _P)
_lib_last_error = _sig("lwo_last_error", C.c_char_p)
_lib_sha256 = _sig("lwo_sha256", C.c_int, _P, C.c_uint64, C.c_char_p)
_lib_cache_publish = _sig("lwo_cache_publish", C.c_int, C.c_char_p, C.POINTER(_Desc), C.POINTER(_Source), C.c_uint32,
                          C.c_char_p, C.POINTER(C.c_int32))
_lib_cache_open = _sig("lwo_cache_open", C.c_int, C.c_char_p, C.c_char_p, C.POINTER(_Desc), C.c_int32, C.POINTER(_P))
_lib_cache_extents = _sig("lwo_cache_extents", C.c_int, _P, C.POINTER(C.c_void_p), C.c_int32, C.POINTER(C.c_int32))
_lib_cache_close = _sig("lwo_cache_close", C.c_int, _P)
_I = C.c_int32
_lib_op_linear = _sig("lwo_op_linear", C.c_int, _I, _I, _P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _I, _P, _I, _P, _I, _I,
                      _I, _I, _P)
_lib_op_attention = _sig("lwo_op_attention", C.c_int, _I, _P, _I, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _P)
_lib_op_layernorm = _sig("lwo_op_layernorm", C.c_int, _P, _I, _I, _I, _P, _I, _I, _P, _I, _P, _I, _P)
_lib_op_quantize_rows = _sig("lwo_op_quantize_rows", C.c_int, _P, _I, _I, _P, _P, _I, _P)
_lib_op_rmsnorm_qk = _sig("lwo_op_rmsnorm_qk", C.c_int, _I, _P, _I, _I, _P, _P, _P)
_lib_probe_mfma = _sig("lwo_probe_mfma", C.c_int, _I, _I, _I, _P, C.c_uint64, _P, C.POINTER(C.c_double))

EXPORTED = ["lwo_block_layout", "lwo_pack_block", "lwo_tile_weight", "lwo_extent_checksum", "lwo_register_ranges",
            "lwo_build_block_store", "lwo_build_mixed_store", "lwo_build_shard_store", "lwo_set_resident_prefix", "lwo_run_denoise_step", "lwo_run_blocks_noalloc", "lwo_set_max_inflight",
            "lwo_set_validation",
            "lwo_block_checksum", "lwo_set_copy_timing", "lwo_copy_times", "lwo_set_kernel_timing",
            "lwo_kernel_stats", "lwo_get_stats", "lwo_op_linear", "lwo_op_attention", "lwo_op_layernorm",
            "lwo_op_quantize_rows", "lwo_op_rmsnorm_qk", "lwo_probe_mfma",
            "lwo_destroy_block_store", "lwo_last_error", "lwo_sha256", "lwo_cache_publish", "lwo_cache_open",
            "lwo_cache_extents", "lwo_cache_close"]


def exported_symbols() -> list[str]:
    return list(EXPORTED)


def _v(p):
    return C.c_void_p(p) if p else None


def op_linear(dtype, epilogue, a, w, M, N, K, stream, *, a_scale=0, w_scale=0, w_seg=0, bias=0, out=0, ldo=0,
              xr=0, ldx=0, gate=0, gate_ld=0, rows_per_gate=0, a_layout=ROWS, out_layout=ROWS):
    """All pointers are device addresses (ints); see lwo_op_linear."""
    _check(_lib_op_linear(dtype, epilogue, _v(a), _v(a_scale), _v(w), _v(w_scale), w_seg, _v(bias), M, N, K,
                          _v(out), ldo, _v(xr), ldx, _v(gate), gate_ld, rows_per_gate, a_layout, out_layout,
                          _v(stream)))


def op_attention(dtype, q, ldq, k, ldk, v, ldv, o, ldo, batch, heads, tq, tk, head_dim, stream, *, o_layout=ROWS):
    _check(_lib_op_attention(dtype, _v(q), ldq, _v(k), ldk, _v(v), ldv, _v(o), ldo, batch, heads, tq, tk, head_dim,
                             o_layout, _v(stream)))


def op_layernorm(x, M, D, out, out_dtype, stream, *, mod=0, rows_per_batch=1, shift_chunk=0, scale_chunk=0,
                 out_scale=0, out_layout=ROWS):
    _check(_lib_op_layernorm(_v(x), M, D, rows_per_batch, _v(mod), shift_chunk, scale_chunk, _v(out), out_dtype,
                             _v(out_scale), out_layout, _v(stream)))


def op_quantize_rows(inp, M, N, codes, scales, stream, *, codes_layout=ROWS):
    _check(_lib_op_quantize_rows(_v(inp), M, N, _v(codes), _v(scales), codes_layout, _v(stream)))


def op_rmsnorm_qk(dtype, qkv, M, D, gq, gk, stream):
    _check(_lib_op_rmsnorm_qk(dtype, _v(qkv), M, D, _v(gq), _v(gk), _v(stream)))


def probe_mfma(dtype, blocks, iters, sink, sink_floats, stream) -> float:
    """Enqueue the MFMA throughput probe; returns the launch's flop count (see lwo_probe_mfma)."""
    fl = C.c_double(0.0)
    _check(_lib_probe_mfma(dtype, blocks, iters, _v(sink), sink_floats, _v(stream), C.byref(fl)))
    return fl.value


def last_error() -> str:
    return (_lib_last_error() or b"").decode()


def _check(status: int) -> None:
    if status != 0:
        raise LwoError(status, last_error())


@dataclasses.dataclass(frozen=True)
class ModelDesc:
    kind: int
    n_blocks: int
    hidden: int
    heads: int
    ffn: int
    batch: int
    tokens: int
    ctx_tokens: int
    act_dtype: int
    linear_dtype: int

    @classmethod
    def from_workload(cls, w) -> "ModelDesc":
        """From any object with the lwo_synth.Workload fields."""
        return cls(KIND_DIT if w.kind == "dit" else KIND_VIDEO, w.n_blocks, w.hidden, w.heads, w.ffn, w.batch,
                   w.tokens, w.ctx_tokens, DTYPES[w.act_dtype], DTYPES[w.linear_dtype])

    def _c(self) -> _Desc:
        return _Desc(*dataclasses.astuple(self))


def block_layout(desc: ModelDesc):
    """([dict(name, offset, bytes, shape, dtype, tiled)], extent_bytes)."""
    d = desc._c()
    n = C.c_int32()
    ext = C.c_uint64()
    _check(_lib_block_layout(C.byref(d), None, 0, C.byref(n), C.byref(ext)))
    arr = (_TensorInfo * n.value)()
    _check(_lib_block_layout(C.byref(d), arr, n.value, C.byref(n), C.byref(ext)))
    out = [dict(name=t.name.decode(), offset=t.offset, bytes=t.bytes, shape=tuple(t.shape[:t.rank]), dtype=t.dtype,
                tiled=bool(t.tiled)) for t in arr]
    return out, ext.value


def tile_weight(dtype: int, w: np.ndarray) -> np.ndarray:
    """Row-major weight [N, K] (bf16 as uint16 or fp8 codes as uint8, host)
    -> a new uint8 array in the tiled order that op_linear takes."""
    w = np.ascontiguousarray(w)
    if w.ndim != 2:
        raise ValueError("tile_weight: w must be 2-D")
    out = np.empty(w.nbytes, dtype=np.uint8)
    _check(_lib_tile_weight(dtype, w.ctypes.data, w.shape[0], w.shape[1], out.ctypes.data))
    return out


def pack_block(desc: ModelDesc, tensors, dst=None, dst_bytes: int | None = None):
    """Flatten float32 tensors into one extent.  dst: a writable buffer, or an
    integer address of dst_bytes writable bytes; returns a new uint8 array if
    dst is None."""
    _, ext = block_layout(desc)
    arrs = [np.ascontiguousarray(t, dtype=np.float32) for t in tensors]
    ptrs = (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    out = None
    if dst is None:
        out = np.empty(ext, dtype=np.uint8)
        addr, cap = out.ctypes.data, ext
    elif isinstance(dst, int):
        if dst_bytes is None:
            raise ValueError("dst_bytes is required with an address")
        addr, cap = dst, dst_bytes
    else:
        view = np.frombuffer(dst, dtype=np.uint8)
        addr, cap = view.ctypes.data, view.size
    _check(_lib_pack_block(C.byref(desc._c()), ptrs, len(arrs), C.c_void_p(addr), cap))
    return out


def extent_checksum(buf) -> int:
    a = np.frombuffer(buf, dtype=np.uint8)
    s = C.c_uint64()
    _check(_lib_extent_checksum(C.c_void_p(a.ctypes.data), a.size, C.byref(s)))
    return s.value


def register_ranges(ptrs, sizes, page, budget, reg, unreg, cap=64):
    """Drive the registration lifecycle with Python callbacks reg(base, len) ->
    int and unreg(base) -> int (0 = success).  Returns [(base, len)]."""
    n = len(ptrs)
    P = (C.c_void_p * max(n, 1))(*ptrs)
    S = (C.c_uint64 * max(n, 1))(*sizes)
    rcb = _REG(lambda user, base, ln: int(reg(int(base or 0), int(ln))))
    ucb = _UNREG(lambda user, base: int(unreg(int(base or 0))))
    ob = (C.c_uint64 * cap)()
    ol = (C.c_uint64 * cap)()
    nout = C.c_int32()
    _check(_lib_register_ranges(P, S, n, page, budget, rcb, ucb, None, ob, ol, cap, C.byref(nout)))
    return [(ob[i], ol[i]) for i in range(nout.value)]


@dataclasses.dataclass
class Stats:
    extent_bytes: int
    slot_bytes: int
    device_weight_bytes: int
    workspace_bytes: int
    host_bytes: int
    h2d_copies: int
    h2d_bytes: int
    steps: int
    checksum_mismatches: int
    registered_ranges: int
    registered_bytes: int
    resident_prefix: int
    head_slot: int
    host_mode: int
    validation: int
    build_ms: float
    staging_bytes: int
    pack_bytes: int
    pack_ms: float
    pack_threads: int
    reserved: int
    group: int
    rank: int
    shard_bytes: int
    gather_bytes: int
    peer_device_bytes: int


class Store:
    """Owner of one lwo_store handle (destroy() or context-manager exit frees it)."""

    def __init__(self, handle, desc: ModelDesc, keepalive=None):
        self._h = handle
        self.desc = desc
        self._keep = keepalive

    @property
    def handle(self) -> int:
        return self._h.value or 0

    def _live(self):
        if not self._h:
            raise LwoError(7, "store already destroyed")
        return self._h

    def set_resident_prefix(self, k: int) -> None:
        _check(_lib_set_prefix(self._live(), k))

    def run_denoise_step(self, x: int, cond: int, ctx: int | None, stream: int) -> None:
        """x, cond, ctx: device addresses; stream: hipStream_t as an integer."""
        _check(_lib_run(self._live(), C.c_void_p(x), C.c_void_p(cond), C.c_void_p(ctx) if ctx else None,
                        C.c_void_p(stream)))

    def set_max_inflight(self, n: int) -> None:
        """Pacing depth of run_denoise_step (0: never wait on the host)."""
        _check(_lib_set_max_inflight(self._live(), n))

    def set_validation(self, on: bool) -> None:
        _check(_lib_set_validation(self._live(), 1 if on else 0))

    def block_checksum(self, block: int):
        hs, ss = C.c_uint64(), C.c_uint64()
        st = _lib_block_checksum(self._live(), block, C.byref(hs), C.byref(ss))
        if st not in (0, 8):
            _check(st)
        return hs.value, ss.value

    def set_copy_timing(self, on: bool) -> None:
        _check(_lib_set_copy_timing(self._live(), 1 if on else 0))

    def copy_times(self, cap: int = 4096) -> list[float]:
        buf = (C.c_float * cap)()
        n = C.c_int32()
        _check(_lib_copy_times(self._live(), buf, cap, C.byref(n)))
        return [buf[i] for i in range(min(n.value, cap))]

    def set_kernel_timing(self, on: bool) -> None:
        """Switch per-kernel timing on (resetting the totals) or off."""
        _check(_lib_set_kernel_timing(self._live(), 1 if on else 0))

    def kernel_stats(self) -> list[dict]:
        """[dict(name, launches, total_ms, flops, bytes)] since timing was switched on."""
        n = C.c_int32()
        _check(_lib_kernel_stats(self._live(), None, 0, C.byref(n)))
        arr = (_KStat * max(n.value, 1))()
        _check(_lib_kernel_stats(self._live(), arr, n.value, C.byref(n)))
        return [dict(name=k.name.decode(), launches=k.launches, total_ms=k.total_ms, flops=k.flops, bytes=k.bytes)
                for k in arr[:n.value]]

    def stats(self) -> Stats:
        s = _Stats()
        _check(_lib_get_stats(self._live(), C.byref(s)))
        return Stats(*[getattr(s, f[0]) for f in _Stats._fields_])

    def destroy(self) -> None:
        if self._h:
            _check(_lib_destroy(self._h))
            self._h = None
            self._keep = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _source(extents=None, fill=None):
    """A lwo_block_source over host buffers/addresses or a fill(b, dst_addr, nbytes) callback, and the
    Python objects it points into (keep them alive while the library may use the source)."""
    src = _Source()
    keep = []
    if extents is not None:
        addrs = [e if isinstance(e, int) else np.frombuffer(e, dtype=np.uint8).ctypes.data for e in extents]
        arr = (C.c_void_p * len(addrs))(*addrs)
        keep.append((arr, extents))
        src.extents = C.cast(arr, C.POINTER(C.c_void_p))
        src.fill = _FILL()
    else:
        def _fill(user, b, dst, nbytes):
            try:
                fill(int(b), int(dst), int(nbytes))
                return 0
            except Exception:   # reported through the library's status
                import traceback
                traceback.print_exc()
                return 1
        cb = _FILL(_fill)
        keep.append(cb)
        src.extents = C.POINTER(C.c_void_p)()
        src.fill = cb
    return src, keep


def sha256(buf) -> bytes:
    """The library's SHA-256 of a bytes-like object."""
    a = np.frombuffer(buf, dtype=np.uint8)
    out = C.create_string_buffer(32)
    _check(_lib_sha256(a.ctypes.data if a.size else None, a.size, out))
    return out.raw


def cache_publish(directory: str, desc: ModelDesc, extents=None, fill=None, wait_ms: int = 10000):
    """Publish the block stack under directory; returns (key, created)."""
    src, keep = _source(extents, fill)
    key = C.create_string_buffer(65)
    created = C.c_int32()
    _check(_lib_cache_publish(os.fsencode(directory), C.byref(desc._c()), C.byref(src), wait_ms, key,
                              C.byref(created)))
    del keep
    return key.value.decode(), bool(created.value)


class CacheExtents(list):
    """Page-aligned extent addresses inside an open entry's mapping.  The list
    holds its entry, so a store that keeps the list keeps the entry too."""

    def __init__(self, addrs, entry):
        super().__init__(addrs)
        self.entry = entry


class CacheEntry:
    """An open, validated entry mapped read-only; extents() are page-aligned addresses in the mapping.
    close() refuses while a store built on those extents is alive (its copies read the mapping)."""

    def __init__(self, handle, n):
        self._h = handle
        self.n_blocks = n
        self._borrowers = weakref.WeakSet()

    def extents(self) -> CacheExtents:
        if not self._h:
            raise LwoError(7, "cache entry is closed")
        arr = (C.c_void_p * self.n_blocks)()
        n = C.c_int32()
        _check(_lib_cache_extents(self._h, arr, self.n_blocks, C.byref(n)))
        return CacheExtents([int(arr[i]) for i in range(n.value)], self)

    def borrow(self, store) -> None:
        """Record a store (anything with a `handle`, non-zero while it is alive) that reads the mapping."""
        self._borrowers.add(store)

    def close(self) -> None:
        if self._h:
            live = [s for s in self._borrowers if getattr(s, "handle", 0)]
            if live:
                raise LwoError(7, f"{len(live)} store(s) built on this entry's extents are still alive: "
                                  "destroy them before closing the entry")
            _check(_lib_cache_close(self._h))
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def cache_open(directory: str, key: str, desc: ModelDesc, verify: bool = True) -> CacheEntry:
    h = C.c_void_p()
    _check(_lib_cache_open(os.fsencode(directory), key.encode(), C.byref(desc._c()), int(verify), C.byref(h)))
    return CacheEntry(h, desc.n_blocks)


def build_block_store(desc: ModelDesc, extents=None, fill=None, host_mode: int = HOST_PIN_COPY,
                      register_budget: int = 0, device: int = 0) -> Store:
    """extents: list of host buffers/addresses (one per block), or fill(b, dst_addr, nbytes) -> None
    writing block b's flat extent into the store's pinned memory.  REGISTER and STAGED borrow the
    extents: the returned store keeps the Python objects alive until it is destroyed."""
    src, keep = _source(extents, fill)
    h = C.c_void_p()
    _check(_lib_build(C.byref(desc._c()), C.byref(src), host_mode, register_budget, device, C.byref(h)))
    store = Store(h, desc, keepalive=keep if host_mode in (HOST_REGISTER, HOST_STAGED) else None)
    if isinstance(extents, CacheExtents) and host_mode in (HOST_REGISTER, HOST_STAGED):
        extents.entry.borrow(store)
    return store


def build_mixed_store(types, block_type, extents=None, fill=None, host_mode: int = HOST_PIN_COPY,
                      register_budget: int = 0, device: int = 0) -> Store:
    """A stack whose block b has descriptor types[block_type[b]]; extents[b] / fill use that type's extent size."""
    types = list(types)
    bt = list(block_type)
    src, keep = _source(extents, fill)
    arr = (_Desc * len(types))(*[t._c() for t in types])
    tarr = (C.c_int32 * len(bt))(*bt)
    h = C.c_void_p()
    _check(_lib_build_mixed(arr, len(types), tarr, len(bt), C.byref(src), host_mode, register_budget, device,
                            C.byref(h)))
    n_desc = dataclasses.replace(types[0], n_blocks=len(bt))
    return Store(h, n_desc, keepalive=keep if host_mode in (HOST_REGISTER, HOST_STAGED) else None)


def build_shard_store(desc: ModelDesc, group: int, rank: int, extents=None, fill=None, device: int = 0) -> Store:
    """One rank's share of an all-gather group (see lwo_build_shard_store): only shard `rank` of every block is
    pinned on the host; the other shards stand in on the device for what the all-gather would bring."""
    src, keep = _source(extents, fill)
    h = C.c_void_p()
    _check(_lib_build_shard(C.byref(desc._c()), C.byref(src), group, rank, device, C.byref(h)))
    del keep
    return Store(h, desc)


NOALLOC_SCRATCH_BYTES = 64 << 20


def run_blocks_noalloc(desc: ModelDesc, blocks, x: int, cond: int, ctx: int | None, stream: int) -> None:
    """One step over device-resident extents (device addresses) with no device allocation
    (see lwo_run_blocks_noalloc)."""
    arr = (C.c_void_p * max(len(blocks), 1))(*[int(b) for b in blocks])
    _check(_lib_run_noalloc(C.byref(desc._c()), arr, len(blocks), C.c_void_p(x), C.c_void_p(cond),
                            C.c_void_p(ctx) if ctx else None, C.c_void_p(stream)))
