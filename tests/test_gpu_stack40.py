"""GPU parity of the 40-block 14B-class video stack (hidden 5120, 40 heads,
FFN 13824, 512 context tokens) at 256 tokens, end to end through the C ABI,
against the float64 oracle over every output element.

* bf16 linears: one step streamed from block 0, with the first 8 blocks
  resident, and with all 40 resident must give the same bits; the output is
  held to the stated 2e-2 relative L2 (3e-2 on the update).
* fp8 linears (per-tensor e4m3 weights, the 32760-token fp8 stack's weights
  at 256 tokens): the stated 5e-2 against the plain oracle (stored weights,
  exact activations).  The kernels also quantise every linear's input per
  row; the oracle that does the same lies 4.2e-2 from the plain one after
  the first block and 4.5-4.6e-2 after 20-40 (the error hardly compounds:
  each block's update is of the size of the residual stream and its
  quantisation error is fresh, about 4% of it).  The GPU measures 4.60e-2
  over the 40 blocks, so the bound holds with about 8% headroom and is not
  widened.
* every row (token) of the output is also held to 1.5 times the whole-tensor
  bound and every column (feature) to 5 times it, a column's error taken
  relative to the tensor's root-mean-square column norm (gpu_util.
  row_col_errors): a wrong row or column shows an error of order 1 there.
  Rows are alike; a few columns carry about 4 times the whole tensor's error,
  because a linear's input column that a per-column shift dominates rounds
  the same way in every row (the oracle with emulated fp8 activations shows
  0.155-0.183 against 0.042-0.045 over 1-20 blocks).

The oracle runs block by block beside the store's build, on the same drawn
tensors (tests/gpu_util.build_with_oracle), so host memory holds the pinned
store plus one block at a time.
"""
import numpy as np
import pytest

import lwo_synth
from oracle import dit as o_dit

from .conftest import gpu_available
from .gpu_util import build_with_oracle, device_inputs, row_col_errors, run_steps, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _run(st, w, k):
    import torch
    st.set_resident_prefix(k)
    x, cond, ctx = device_inputs(w)
    run_steps(st, x, cond, ctx)
    bits = x.cpu().view(-1).view(torch.int16).numpy().copy()
    return x, bits


def _check(name, got, x0, want, tol_out, tol_delta):
    e_out = o_dit.rel_l2(got, want)
    e_delta = o_dit.rel_l2(got - x0, want - x0)
    e_row, e_col = row_col_errors(got, want)
    print(f"[stack40] {name}: rel_l2(out)={e_out:.3e} rel_l2(update)={e_delta:.3e} "
          f"max row {e_row:.3e} max column {e_col:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert e_out <= tol_out and e_delta <= tol_delta, (e_out, e_delta)
    assert e_row <= 1.5 * tol_out and e_col <= 5 * tol_out, (e_row, e_col)


def test_video14b_t256_bf16_stack_streamed_prefix_resident(lib):
    w = lwo_synth.get("video14b_t256")
    print(f"[stack40] {w.name}: building the store and the oracle", flush=True)
    st, x0, want = build_with_oracle(lib, w)
    with st:
        outs = {}
        for k in (0, 8, 40):
            print(f"[stack40] {w.name}: step with k={k}", flush=True)
            x, outs[k] = _run(st, w, k)
            if k == 0:
                got = to_f64(x).reshape(want.shape)
            del x
    assert np.array_equal(outs[8], outs[0]) and np.array_equal(outs[40], outs[0])
    _check(w.name, got, x0, want, 2e-2, 3e-2)


def test_video14b_t256_fp8_stack(lib):
    w = lwo_synth.get("video14b_t256_fp8")
    print(f"[stack40] {w.name}: building the store and the oracle", flush=True)
    st, x0, want = build_with_oracle(lib, w)
    with st:
        x, b0 = _run(st, w, 0)
        got = to_f64(x).reshape(want.shape)
        del x
        _, b40 = _run(st, w, 40)
    assert np.array_equal(b0, b40)
    _check(w.name, got, x0, want, 5e-2, 5e-2)
