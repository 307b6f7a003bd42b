"""Helpers for GPU tests: build a store from a seeded workload, place the
step inputs on the device, run steps on a non-default stream, and compute
the oracle's answer on the same inputs."""
from __future__ import annotations

import concurrent.futures as _fut
import os
import time

import numpy as np

import lwo_synth
from oracle import dit as o_dit
from oracle import layout as o_layout


def torch_dtype(w):
    import torch
    return torch.float32 if w.act_dtype == "f32" else torch.bfloat16


def make_store(lwo, w, k=0, tensors=None):
    """tensors: optional callable b -> list of float32 arrays (defaults to the generator)."""
    desc = lwo.ModelDesc.from_workload(w)
    get = tensors or (lambda b: lwo_synth.block_tensors(w, b))

    def fill(b, dst, n):
        lwo.pack_block(desc, get(b), dst=dst, dst_bytes=n)

    store = lwo.build_block_store(desc, fill=fill)
    if k:
        store.set_resident_prefix(k)
    return store


def device_inputs(w, inputs=None):
    """(x, cond, ctx) torch tensors on cuda:0 in the activation dtype."""
    import torch
    x, cond, ctx = inputs if inputs is not None else lwo_synth.step_inputs(w)
    dt = torch_dtype(w)
    to = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0").to(dt).contiguous()
    return to(x), to(cond), to(ctx)


def run_steps(store, x, cond, ctx, steps=1, stream=None):
    """Run `steps` denoise steps in place on x (a torch tensor); returns x."""
    import torch
    s = stream or torch.cuda.Stream()
    torch.cuda.current_stream().synchronize()
    for _ in range(steps):
        store.run_denoise_step(x.data_ptr(), cond.data_ptr(), ctx.data_ptr() if ctx is not None else None,
                               s.cuda_stream)
    s.synchronize()
    return x


def to_f64(t) -> np.ndarray:
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def oracle_out(w, tensors=None, inputs=None, steps=1):
    """The oracle's x after `steps` passes over all blocks, on the library's inputs
    (the bf16 rounding of the draws for a bf16 workload)."""
    get = tensors or (lambda b: lwo_synth.block_tensors(w, b))
    ext = [o_layout.pack_block(w, get(b)) for b in range(w.n_blocks)]
    x, cond, ctx = o_dit.decode_inputs(w, *(inputs if inputs is not None else lwo_synth.step_inputs(w)))
    x0 = x
    for _ in range(steps):
        x = o_dit.stack_forward(w, ext, x, cond, ctx)
        if w.act_dtype == "bf16":   # the step hands x back in the activation dtype
            from oracle import codecs
            x = codecs.bf16_round(x.astype(np.float32))
    return x0, x


def build_with_oracle(lwo, w, fp8_act: bool = False):
    """Build w's store (PIN_COPY) and, in the same pass over the generator's
    blocks, run the oracle's stack forward on the same drawn tensors, so that
    each block is drawn once and host memory holds one block's float32 and
    float64 tensors at a time besides the store.  The oracle takes the stored
    values from oracle.layout.stored_params and runs on a worker thread while
    the library packs the next extent.  Returns (store, x0, want): the
    oracle's input and its output after one pass over every block, in
    float64, with the bf16 rounding of the output for a bf16 workload."""
    desc = lwo.ModelDesc.from_workload(w)
    x0, cond, ctx = o_dit.decode_inputs(w, *lwo_synth.step_inputs(w))
    threads = min(16, os.cpu_count() or 1)
    blocks = lwo_synth.iter_blocks(w, threads=threads)
    pool = _fut.ThreadPoolExecutor(max_workers=1)
    state = {"x": x0, "job": None}
    t0 = time.perf_counter()

    def advance(b, t):
        p = o_layout.stored_params(w, t, threads=threads)
        state["x"] = o_dit.block_forward(w, state["x"], cond, ctx, p, fp8_act=fp8_act)
        if b % 4 == 3 or b == w.n_blocks - 1:
            print(f"[oracle] {w.name}: block {b + 1}/{w.n_blocks} at {time.perf_counter() - t0:.0f} s", flush=True)

    def fill(b, dst, n):
        bb, t = next(blocks)
        assert bb == b
        if state["job"] is not None:
            state["job"].result()        # the oracle runs the blocks in order
        state["job"] = pool.submit(advance, b, t)
        lwo.pack_block(desc, t, dst=dst, dst_bytes=n)

    try:
        store = lwo.build_block_store(desc, fill=fill)
        state["job"].result()
    finally:
        pool.shutdown(wait=True)
    want = state["x"]
    if w.act_dtype == "bf16":   # the step hands x back in the activation dtype
        from oracle import codecs
        want = codecs.bf16_round(want.astype(np.float32))
    return store, x0, want


def row_col_errors(got: np.ndarray, want: np.ndarray):
    """Largest error of any token row and of any feature column of [..., D]
    outputs (rows = every leading index), each relative to a typical row or
    column: a row's L2 error over that row's own norm (rows are alike), and a
    column's L2 error over the root-mean-square column norm of the whole
    tensor.  Columns are not alike: the residual stream's columns carry a
    value shared by every row (most of a column's norm deep in a stack), so
    a column whose shared value is near zero has a small norm of its own and
    a large error relative to it, while its error is ordinary.  A wrong row or
    column shows an error of order 1 under either measure, even when the
    whole-tensor figure hides it."""
    g = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(want, np.float64).reshape(-1, want.shape[-1])
    d = g - r
    rows = np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-300)
    col_rms = max(np.linalg.norm(r) / np.sqrt(r.shape[1]), 1e-300)
    cols = np.linalg.norm(d, axis=0) / col_rms
    return float(rows.max()), float(cols.max())
