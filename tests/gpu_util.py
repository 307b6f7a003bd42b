"""Helpers for GPU tests: build a store from a seeded workload, place the
step inputs on the device, run steps on a non-default stream, and compute
the oracle's answer on the same inputs."""
from __future__ import annotations

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
