"""Seeded synthetic workloads for layerwise weight offload of a DiT block stack.

This module only draws random numbers and names shapes.  It holds no part of
the block computation, the storage codecs or the block layout: the HIP
library and the CPU oracle each implement those on their own, and both take
their inputs from here.

Workloads (sizes follow the offload design page's targets for a diffusion
transformer: a tiny DiT, a DiT-XL-shaped stack, and a 14B-class video DiT):

* ``dit_tiny_fp32``   4 blocks, D=256, H=4, F=1024, B=1, T=64, fp32
* ``dit_xl_bf16``     28 blocks, D=1152, H=16 (d=72), F=4608, B=2, T=1024, bf16
* ``video14b_bf16``   40 blocks, D=5120, H=40 (d=128), F=13824, B=1,
                      T=32760 (21x30x52 latent patches), 512 context tokens
* ``video14b_t256``   the same stack at T=256 (transfer-bound)
* ``video14b_fp8``    the same stack with per-tensor fp8 e4m3 linear weights
* ``video14b_t256_fp8`` the fp8 stack at T=256

plus small variants (suffix ``_t``) whose shapes span several kernel tiles
with ragged tails, used by the parity tests, and small mixed stacks of two
block types (``MixedStack``).

Draw recipe (one stream per block, one for the step inputs):

* block ``b`` of a workload with seed ``s`` uses
  ``numpy.random.Generator(PCG64(SeedSequence([s, b])))`` and draws, tensor by
  tensor in block order, ``standard_normal(shape, float32) * 0.02`` for every
  weight, bias and modulation table; norm gains are ones, or
  ``1 + 0.1 * standard_normal`` when ``gamma_jitter`` is set;
* the step inputs use ``SeedSequence([s, 1_000_000])`` and draw x [B,T,D],
  then cond ([B,D] for the DiT kind, [B,6,D] for the video kind), then (video
  kind only) ctx [B,Tc,D], all standard normal float32.

fp8 weight codes and scales are *not* produced here: quantisation is part of
packing a block, which each side implements itself.
"""
from __future__ import annotations

import concurrent.futures as _fut
import dataclasses
import os

import numpy as np

KIND_DIT = "dit"
KIND_VIDEO = "video"

INPUT_STREAM = 1_000_000


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "dit" or "video"
    n_blocks: int
    hidden: int
    heads: int
    ffn: int
    batch: int
    tokens: int
    ctx_tokens: int      # 0 for the DiT kind
    act_dtype: str       # "f32" or "bf16"
    linear_dtype: str    # "f32", "bf16" or "fp8"
    seed: int
    gamma_jitter: bool = False
    resident_prefix: int = 0

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: dict[str, Workload] = {}


def _add(w: Workload) -> None:
    WORKLOADS[w.name] = w


# Full-size workloads.
_add(Workload("dit_tiny_fp32", KIND_DIT, 4, 256, 4, 1024, 1, 64, 0, "f32", "f32", 101))
_add(Workload("dit_xl_bf16", KIND_DIT, 28, 1152, 16, 4608, 2, 1024, 0, "bf16", "bf16", 102))
_add(Workload("video14b_bf16", KIND_VIDEO, 40, 5120, 40, 13824, 1, 32760, 512, "bf16", "bf16", 103))
_add(Workload("video14b_t256", KIND_VIDEO, 40, 5120, 40, 13824, 1, 256, 512, "bf16", "bf16", 103))
_add(Workload("video14b_t256_k8", KIND_VIDEO, 40, 5120, 40, 13824, 1, 256, 512, "bf16", "bf16", 103,
              resident_prefix=8))
_add(Workload("video14b_fp8", KIND_VIDEO, 40, 5120, 40, 13824, 1, 32760, 512, "bf16", "fp8", 103))
# the fp8 stack at 256 tokens: end-to-end parity of all 40 blocks with fp8 linears
_add(Workload("video14b_t256_fp8", KIND_VIDEO, 40, 5120, 40, 13824, 1, 256, 512, "bf16", "fp8", 103))

# Small variants for parity: several tiles along every axis and ragged tails.
_add(Workload("dit_t_fp32", KIND_DIT, 3, 576, 8, 2304, 2, 200, 0, "f32", "f32", 201))
_add(Workload("dit_t_bf16", KIND_DIT, 3, 576, 8, 2304, 2, 200, 0, "bf16", "bf16", 202))
_add(Workload("dit_t64_bf16", KIND_DIT, 3, 256, 4, 1024, 1, 333, 0, "bf16", "bf16", 203))
_add(Workload("video_t_fp32", KIND_VIDEO, 3, 256, 4, 1024, 1, 200, 40, "f32", "f32", 301, gamma_jitter=True))
_add(Workload("video_t_bf16", KIND_VIDEO, 3, 256, 2, 1024, 1, 300, 40, "bf16", "bf16", 302, gamma_jitter=True))
_add(Workload("video_t_fp8", KIND_VIDEO, 3, 256, 2, 1024, 1, 300, 40, "bf16", "fp8", 303, gamma_jitter=True))


def get(name: str) -> Workload:
    return WORKLOADS[name]


# Mixed stacks: several block types streamed through one ring.  Block b of a
# stack draws its tensors as block b of its type's workload (all types share
# the stack's seed), so the recipe above is unchanged.
@dataclasses.dataclass(frozen=True)
class MixedStack:
    name: str
    types: tuple          # Workload per block type; they share kind, hidden, batch, tokens, ctx, act dtype, seed
    block_type: tuple     # type index of each block, in stack order

    @property
    def n_blocks(self) -> int:
        return len(self.block_type)

    def type_of(self, b: int) -> Workload:
        return self.types[self.block_type[b]].with_(n_blocks=self.n_blocks)

    @property
    def inputs(self) -> Workload:
        """The workload whose step inputs the stack takes (shared by every type)."""
        return self.types[0].with_(n_blocks=self.n_blocks)


MIXED: dict[str, MixedStack] = {}


def _mix(name: str, types, block_type) -> None:
    MIXED[name] = MixedStack(name, tuple(types), tuple(block_type))


# two DiT block types of different sizes (head dims 64 and 128, FFN 1024 and 512), fp32
_mix("dit_mixed_fp32", [Workload("dit_mixed_fp32.a", KIND_DIT, 1, 256, 4, 1024, 1, 96, 0, "f32", "f32", 401),
                        Workload("dit_mixed_fp32.b", KIND_DIT, 1, 256, 2, 512, 1, 96, 0, "f32", "f32", 401)],
     [0, 1, 1, 0, 1])
# two DiT block types (head dims 72 and 64, FFN 2304 and 1152), bf16, ragged tokens
_mix("dit_mixed_bf16", [Workload("dit_mixed_bf16.a", KIND_DIT, 1, 576, 8, 2304, 2, 200, 0, "bf16", "bf16", 402),
                        Workload("dit_mixed_bf16.b", KIND_DIT, 1, 576, 9, 1152, 2, 200, 0, "bf16", "bf16", 402)],
     [1, 0, 0, 1, 0])
# video blocks with bf16 and with fp8 linears (extents of different sizes)
_mix("video_mixed_fp8", [Workload("video_mixed_fp8.a", KIND_VIDEO, 1, 256, 2, 1024, 1, 300, 40, "bf16", "bf16", 403,
                                  gamma_jitter=True),
                         Workload("video_mixed_fp8.b", KIND_VIDEO, 1, 256, 2, 512, 1, 300, 40, "bf16", "fp8", 403,
                                  gamma_jitter=True)],
     [0, 1, 0, 1])
# the 40-block video stack at 256 tokens with bf16 and fp8 linears alternating (extents of 702.7 and 351.5 MB)
_mix("video14b_t256_mixed",
     [Workload("video14b_t256_mixed.a", KIND_VIDEO, 1, 5120, 40, 13824, 1, 256, 512, "bf16", "bf16", 103),
      Workload("video14b_t256_mixed.b", KIND_VIDEO, 1, 5120, 40, 13824, 1, 256, 512, "bf16", "fp8", 103)],
     [0, 1] * 20)


def get_mixed(name: str) -> MixedStack:
    return MIXED[name]


def tensor_inventory(w: Workload) -> list[tuple[str, tuple[int, ...]]]:
    """Names and shapes of one block's drawn tensors, in draw order.

    Only the tensors the generator draws are listed (the fp8 scale table is
    derived while packing, not drawn)."""
    D, F = w.hidden, w.ffn
    if w.kind == KIND_DIT:
        return [
            ("ada.w", (6 * D, D)), ("ada.b", (6 * D,)),
            ("attn.q.w", (D, D)), ("attn.k.w", (D, D)), ("attn.v.w", (D, D)),
            ("attn.qkv.b", (3 * D,)),
            ("attn.o.w", (D, D)), ("attn.o.b", (D,)),
            ("ffn.fc1.w", (F, D)), ("ffn.fc1.b", (F,)),
            ("ffn.fc2.w", (D, F)), ("ffn.fc2.b", (D,)),
        ]
    return [
        ("mod.table", (6, D)),
        ("attn.q.w", (D, D)), ("attn.k.w", (D, D)), ("attn.v.w", (D, D)),
        ("attn.qkv.b", (3 * D,)),
        ("attn.q.norm", (D,)), ("attn.k.norm", (D,)),
        ("attn.o.w", (D, D)), ("attn.o.b", (D,)),
        ("cross.q.w", (D, D)), ("cross.q.b", (D,)),
        ("cross.k.w", (D, D)), ("cross.v.w", (D, D)), ("cross.kv.b", (2 * D,)),
        ("cross.o.w", (D, D)), ("cross.o.b", (D,)),
        ("ffn.fc1.w", (F, D)), ("ffn.fc1.b", (F,)),
        ("ffn.fc2.w", (D, F)), ("ffn.fc2.b", (D,)),
    ]


def block_tensors(w: Workload, b: int) -> list[np.ndarray]:
    """Draw block ``b``'s tensors (float32, C-contiguous) in inventory order."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, b])))
    out = []
    for name, shape in tensor_inventory(w):
        if name.endswith(".norm"):
            if w.gamma_jitter:
                g = rng.standard_normal(shape, dtype=np.float32)
                out.append((np.float32(1.0) + np.float32(0.1) * g).astype(np.float32))
            else:
                out.append(np.ones(shape, dtype=np.float32))
        else:
            t = rng.standard_normal(shape, dtype=np.float32)
            t *= np.float32(0.02)
            out.append(t)
    return out


def iter_blocks(w, threads: int | None = None):
    """Yield (b, tensors) for every block of a Workload or a MixedStack (block
    b drawn with its own type), drawing ahead on a thread pool (numpy's
    generators release the GIL while filling large arrays)."""
    threads = threads or min(16, os.cpu_count() or 1)
    ahead = max(1, min(threads, 4))
    type_of = w.type_of if isinstance(w, MixedStack) else (lambda b: w)
    with _fut.ThreadPoolExecutor(max_workers=threads) as ex:
        futs = {}
        for b in range(min(ahead, w.n_blocks)):
            futs[b] = ex.submit(block_tensors, type_of(b), b)
        for b in range(w.n_blocks):
            nb = b + ahead
            if nb < w.n_blocks:
                futs[nb] = ex.submit(block_tensors, type_of(nb), nb)
            yield b, futs.pop(b).result()


def step_inputs(w: Workload):
    """(x, cond, ctx) as float32; ctx is None for the DiT kind."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, INPUT_STREAM])))
    x = rng.standard_normal((w.batch, w.tokens, w.hidden), dtype=np.float32)
    if w.kind == KIND_DIT:
        cond = rng.standard_normal((w.batch, w.hidden), dtype=np.float32)
        ctx = None
    else:
        cond = rng.standard_normal((w.batch, 6, w.hidden), dtype=np.float32)
        ctx = rng.standard_normal((w.batch, w.ctx_tokens, w.hidden), dtype=np.float32)
    return x, cond, ctx
