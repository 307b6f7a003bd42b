"""The flat per-block extent: tensor order, offsets and packing.

Test infrastructure (see the package docstring); not imported by the library.

"CPU Offloading for Diffusion Models", section "Layerwise (Blockwise)
Offloading / How It Works", keeps each block's parameters as flattened
tensors in pinned host memory; "Distributed Layerwise Offload", section
"Registered runtime-cache transfer", places every parameter at an offset of
one flattened device buffer and page-aligns host ranges.  The concrete layout
is this project's choice (the pages give none):

* tensors in block order (below), each starting at a multiple of 256 bytes;
* the extent is rounded up to a multiple of 4096 bytes; gaps are zero;
* a weight matrix ``*.w`` is stored in the linear dtype, every other tensor
  (bias, norm gain, modulation table) in the activation dtype;
* a bf16 or fp8 weight matrix other than the DiT kind's ``ada.w`` is stored
  tiled: its row-major bytes, viewed as 64-row x 64-byte tiles, are written
  tile after tile, the tiles of each 64-row band in order along a row and the
  bands in row order; inside a tile its 64 rows of 64 bytes follow each other.
  float32 matrices and ``ada.w`` are row-major;
* with fp8 linears, the ten per-tensor float32 scales follow every other
  tensor, in the order the weight matrices appear.

Block order, DiT kind (D hidden, F FFN width):
  ada.w[6D,D] ada.b[6D] attn.q.w[D,D] attn.k.w attn.v.w attn.qkv.b[3D]
  attn.o.w[D,D] attn.o.b[D] ffn.fc1.w[F,D] ffn.fc1.b[F] ffn.fc2.w[D,F] ffn.fc2.b[D]
Block order, video kind:
  mod.table[6,D] attn.q.w attn.k.w attn.v.w attn.qkv.b[3D] attn.q.norm[D]
  attn.k.norm[D] attn.o.w attn.o.b cross.q.w cross.q.b cross.k.w cross.v.w
  cross.kv.b[2D] cross.o.w cross.o.b ffn.fc1.w ffn.fc1.b ffn.fc2.w ffn.fc2.b
  [linear.scales[10] f32 when the linears are fp8]
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import codecs

TENSOR_ALIGN = 256
EXTENT_ALIGN = 4096

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


@dataclasses.dataclass(frozen=True)
class Slot:
    name: str
    offset: int
    nbytes: int
    shape: tuple
    dtype: str


def _names_shapes(kind: str, D: int, F: int):
    if kind == "dit":
        return [
            ("ada.w", (6 * D, D)), ("ada.b", (6 * D,)),
            ("attn.q.w", (D, D)), ("attn.k.w", (D, D)), ("attn.v.w", (D, D)), ("attn.qkv.b", (3 * D,)),
            ("attn.o.w", (D, D)), ("attn.o.b", (D,)),
            ("ffn.fc1.w", (F, D)), ("ffn.fc1.b", (F,)),
            ("ffn.fc2.w", (D, F)), ("ffn.fc2.b", (D,)),
        ]
    if kind == "video":
        return [
            ("mod.table", (6, D)),
            ("attn.q.w", (D, D)), ("attn.k.w", (D, D)), ("attn.v.w", (D, D)), ("attn.qkv.b", (3 * D,)),
            ("attn.q.norm", (D,)), ("attn.k.norm", (D,)),
            ("attn.o.w", (D, D)), ("attn.o.b", (D,)),
            ("cross.q.w", (D, D)), ("cross.q.b", (D,)),
            ("cross.k.w", (D, D)), ("cross.v.w", (D, D)), ("cross.kv.b", (2 * D,)),
            ("cross.o.w", (D, D)), ("cross.o.b", (D,)),
            ("ffn.fc1.w", (F, D)), ("ffn.fc1.b", (F,)),
            ("ffn.fc2.w", (D, F)), ("ffn.fc2.b", (D,)),
        ]
    raise ValueError(kind)


def tiled(name: str, dtype: str) -> bool:
    return name.endswith(".w") and dtype in ("bf16", "fp8") and name != "ada.w"


def tile_bytes(rows: np.ndarray) -> np.ndarray:
    """[N, R] uint8 row-major bytes -> flat uint8 in the tiled order above."""
    N, R = rows.shape
    assert N % 64 == 0 and R % 64 == 0, (N, R)
    return np.ascontiguousarray(rows.reshape(N // 64, 64, R // 64, 64).transpose(0, 2, 1, 3)).reshape(-1)


def untile_bytes(flat: np.ndarray, N: int, R: int) -> np.ndarray:
    """Inverse of tile_bytes: flat tiled bytes -> [N, R] row-major bytes."""
    return np.ascontiguousarray(flat.reshape(N // 64, R // 64, 64, 64).transpose(0, 2, 1, 3)).reshape(N, R)


def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def block_layout(kind: str, D: int, F: int, act: str, lin: str):
    """(list of Slot, extent_bytes)."""
    slots = []
    off = 0
    for name, shape in _names_shapes(kind, D, F):
        dt = lin if name.endswith(".w") else act
        n = int(np.prod(shape)) * ELEM_BYTES[dt]
        off = _round_up(off, TENSOR_ALIGN)
        slots.append(Slot(name, off, n, tuple(shape), dt))
        off += n
    if lin == "fp8":
        n_w = sum(1 for s in slots if s.name.endswith(".w"))
        off = _round_up(off, TENSOR_ALIGN)
        slots.append(Slot("linear.scales", off, 4 * n_w, (n_w,), "f32"))
        off += 4 * n_w
    return slots, _round_up(off, EXTENT_ALIGN)


def layout_for(w):
    return block_layout(w.kind, w.hidden, w.ffn, w.act_dtype, w.linear_dtype)


def pack_block(w, tensors) -> bytes:
    """Pack one block's float32 tensors (generator order) into its extent."""
    slots, ext = layout_for(w)
    buf = np.zeros(ext, dtype=np.uint8)
    by_name = {s.name: s for s in slots}
    scales = []
    names = [n for n, _ in _names_shapes(w.kind, w.hidden, w.ffn)]
    for name, t in zip(names, tensors):
        s = by_name[name]
        t = np.ascontiguousarray(t, dtype=np.float32)
        assert t.shape == s.shape, (name, t.shape, s.shape)
        if s.dtype == "f32":
            raw = t.view(np.uint8).reshape(-1)
        elif s.dtype == "bf16":
            raw = codecs.bf16_encode(t).view(np.uint8).reshape(-1)
        else:
            codes, sc = codecs.quantize_tensor_e4m3(t)
            raw = codes.reshape(-1)
            scales.append(sc)
        if tiled(s.name, s.dtype):
            raw = tile_bytes(raw.reshape(s.shape[0], -1))
        buf[s.offset:s.offset + s.nbytes] = raw
    if w.linear_dtype == "fp8":
        s = by_name["linear.scales"]
        buf[s.offset:s.offset + s.nbytes] = np.asarray(scales, dtype=np.float32).view(np.uint8)
    return buf.tobytes()


def unpack_block(w, extent: bytes) -> dict:
    """Decode a packed extent into float64 tensors (fp8 weights dequantised
    with their per-tensor scale as one multiply)."""
    slots, ext = layout_for(w)
    b = np.frombuffer(extent, dtype=np.uint8)
    assert b.size == ext
    out = {}
    raw = {}
    for s in slots:
        seg = b[s.offset:s.offset + s.nbytes]
        if tiled(s.name, s.dtype):
            seg = untile_bytes(seg, s.shape[0], s.nbytes // s.shape[0]).reshape(-1)
        if s.dtype == "f32":
            v = seg.view(np.float32).astype(np.float64)
        elif s.dtype == "bf16":
            v = codecs.bf16_decode(seg.view(np.uint16))
        else:
            v = None
            raw[s.name] = seg
        if v is not None:
            out[s.name] = v.reshape(s.shape)
    if w.linear_dtype == "fp8":
        sc = out.pop("linear.scales").reshape(-1)
        wnames = [s.name for s in slots if s.name.endswith(".w")]
        for i, name in enumerate(wnames):
            shape = next(s.shape for s in slots if s.name == name)
            out[name] = (codecs.e4m3_decode(raw[name]) * np.float64(np.float32(sc[i]))).reshape(shape)
        out["_scales"] = sc.astype(np.float32)
    return out


def _rows_parallel(fn, t: np.ndarray, threads: int) -> np.ndarray:
    """fn applied to row ranges of t on a thread pool and concatenated; only
    for elementwise fn, where splitting the rows cannot change a value."""
    if threads <= 1 or t.ndim < 2 or t.shape[0] < 2 * threads:
        return fn(t)
    import concurrent.futures as fut
    step = (t.shape[0] + threads - 1) // threads
    with fut.ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda i: fn(t[i:i + step]), range(0, t.shape[0], step)))
    return np.concatenate(parts, axis=0)


def stored_params(w, tensors, threads: int = 1) -> dict:
    """The float64 tensors unpack_block(w, pack_block(w, tensors)) returns,
    formed from the generator's float32 tensors without building the extent:
    each tensor is rounded to its stored dtype (bf16 grid rounding; fp8 with
    quantize_tensor_e4m3's per-tensor scale s, the code's value times s as
    one multiply).  Tiling only moves bytes, so it does not enter.  Pinned
    equal to the pack/unpack round trip for every kind and dtype; the GPU
    parity tests of full-size stacks use it because packing hundreds of
    millions of weights through the byte codecs is slow.  ``threads`` splits
    the elementwise rounding of large tensors over row ranges."""
    slots, _ = layout_for(w)
    by_name = {s.name: s for s in slots}
    names = [n for n, _ in _names_shapes(w.kind, w.hidden, w.ffn)]
    out, scales = {}, []
    for name, t in zip(names, tensors):
        s = by_name[name]
        t = np.ascontiguousarray(t, dtype=np.float32)
        assert t.shape == s.shape, (name, t.shape, s.shape)
        if s.dtype == "f32":
            out[name] = t.astype(np.float64)
        elif s.dtype == "bf16":
            out[name] = _rows_parallel(codecs.bf16_round_grid, t, threads)
        else:
            amax = np.float32(np.max(np.abs(t))) if t.size else np.float32(0.0)
            sc = np.float32(amax / np.float32(codecs.E4M3_MAX)) if amax > 0 else np.float32(1.0)
            out[name] = _rows_parallel(lambda r: codecs.e4m3_round_grid((r / sc).astype(np.float32)) * np.float64(sc),
                                       t, threads)
            scales.append(sc)
    if w.linear_dtype == "fp8":
        out["_scales"] = np.asarray(scales, dtype=np.float32)
    return out
