"""GPU parity through the C ABI: streamed execution against the float64 oracle,
streamed == resident bit for bit, slot bytes == host bytes.

Tolerances (relative L2 over the whole output, float64).  Every token row is
also held to 1.5 times the output bound and every feature column to 5 times
it (a column's error relative to the tensor's root-mean-square column norm,
tests/gpu_util.row_col_errors), so that a wrong row or column, which the
whole-tensor figure can hide, fails (its error is of order 1).  Rows are alike
(the worst row measures 1.1 times the whole tensor); columns are not: where a
linear's input column is dominated by a per-column shift, it rounds the same
way in every row and its error does not average out, so a few columns carry
3-4 times the whole tensor's error.  The oracle with emulated fp8 activations
shows the same against the plain oracle (worst column 0.155-0.183 against
0.042-0.045 over 1-20 blocks of the 256-token video stack), so this is the
arithmetic, not the kernels.
  * fp32 workloads: 1e-4 on x_out and on the block-stack update x_out - x_in
    (fp32 accumulation over K <= 4608 gives ~1e-6; the bound is the stated one);
  * bf16 workloads: 2e-2 on x_out (the stated bound) and 3e-2 on the update:
    every GEMM input is rounded to bf16 (relative 2^-9 per element), the
    attention probabilities are rounded to bf16, and the output returns in
    bf16, so a few 1e-3 per block is expected; 3e-2 leaves room for three
    blocks without admitting a wrong term (a wrong term moves the update by
    O(1)).  The full 28-block DiT-XL step measures 3.2e-3 on x_out and 3.8e-3
    on the update, well inside the same bounds.
"""
import numpy as np
import pytest

import lwo_synth
from oracle import dit as o_dit

from .conftest import gpu_available
from .gpu_util import device_inputs, make_store, oracle_out, row_col_errors, run_steps, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _parity(lwo, name, tol_out, tol_delta, k=0, steps=1, w=None):
    w = w or lwo_synth.get(name)
    print(f"[parity] {name} k={k} steps={steps}", flush=True)
    x0, want = oracle_out(w, steps=steps)
    with make_store(lwo, w, k=k) as st:
        x, cond, ctx = device_inputs(w)
        run_steps(st, x, cond, ctx, steps=steps)
        got = to_f64(x).reshape(want.shape)
    assert np.isfinite(got).all()
    e_out = o_dit.rel_l2(got, want)
    e_delta = o_dit.rel_l2(got - x0, want - x0)
    e_row, e_col = row_col_errors(got, want)
    print(f"[parity] {name}: rel_l2(out)={e_out:.3e} rel_l2(update)={e_delta:.3e} max row {e_row:.3e} "
          f"max column {e_col:.3e}", flush=True)
    assert e_out <= tol_out and e_delta <= tol_delta, (e_out, e_delta)
    assert e_row <= 1.5 * tol_out and e_col <= 5 * tol_out, (e_row, e_col)


def test_dit_tiny_fp32_full(lib):
    _parity(lib, "dit_tiny_fp32", 1e-4, 1e-4)


def test_dit_xl_full_step(lib):
    """The DiT-XL stack at its full size (28 blocks, hidden 1152, 2 x 1024 tokens), streamed from
    block 0 as the bench runs it, against the float64 oracle over every output element."""
    _parity(lib, "dit_xl_bf16", 2e-2, 3e-2)


@pytest.mark.parametrize("base,change,tol_out,tol_delta", [
    ("dit_t64_bf16", dict(batch=5, tokens=64, n_blocks=2), 2e-2, 3e-2),                      # two batch groups
    ("dit_t_fp32", dict(hidden=1152, heads=9, ffn=4608, tokens=96, n_blocks=1), 1e-4, 1e-4),  # two windows
])
def test_dit_modulation_looping_form(lib, base, change, tol_out, tol_delta):
    """DiT shapes whose adaLN GEMV runs its looping form: more than four batches (the SiLU values staged
    in groups of four), and a row longer than sixteen 16-byte loads per lane (fp32 at 1152 wide: two
    windows).  The DiT-XL, tiny and 200-token shapes take the single-window form."""
    w = lwo_synth.get(base).with_(**change)
    _parity(lib, f"{base} {change}", tol_out, tol_delta, w=w)


@pytest.mark.parametrize("name,tol_out,tol_delta", [("video14b_bf16", 2e-2, 3e-2), ("video14b_fp8", 5e-2, 5e-2)])
def test_video14b_block_full_size_sampled_rows(lib, name, tol_out, tol_delta):
    """One block of the 14B-class video stack at its full size (D 5120, 40 heads, FFN 13824, 32760 tokens,
    512 context tokens; bf16, or fp8 linears), run through the store, against the float64 oracle on 64
    output rows (keys and values over all 32760 tokens), including the first and last query tiles and the
    ragged last one.  With fp8 linears the output is held to the stated 5e-2 against the plain oracle
    (stored weights, exact activations), and the update must be closer to the oracle that also quantises
    each linear's input per row than to the plain one (see test_fp8_video for its 4e-2 bound)."""
    from oracle import codecs
    from oracle import layout as o_layout
    w = lwo_synth.get(name).with_(n_blocks=1)
    rng = np.random.default_rng(7)
    T = w.tokens
    rows = np.unique(np.concatenate([rng.integers(0, T, 56), [0, 1, 127, 128, T // 2, 255 * 128, T - 2, T - 1]]))
    print(f"[parity] {name} block 0 at full size, {rows.size} sampled rows", flush=True)
    with make_store(lib, w) as st:
        x, cond, ctx = device_inputs(w)
        run_steps(st, x, cond, ctx)
        got = to_f64(x).reshape(w.batch, T, w.hidden)[:, rows]
        del x, cond, ctx
    x0, c0, ctx0 = o_dit.decode_inputs(w, *lwo_synth.step_inputs(w))
    params = o_layout.unpack_block(w, o_layout.pack_block(w, lwo_synth.block_tensors(w, 0)))
    bf = lambda a: codecs.bf16_round(a.astype(np.float32))   # the step hands x back in bf16
    want = bf(o_dit.video_block_rows(x0, c0, ctx0, params, w.heads, rows))
    xr = x0[:, rows]
    assert np.isfinite(got).all()
    e_out = o_dit.rel_l2(got, want)
    e_delta = o_dit.rel_l2(got - xr, want - xr)
    e_row, e_col = row_col_errors(got, want)
    print(f"[parity] {name} block: rel_l2(out)={e_out:.3e} rel_l2(update)={e_delta:.3e} max row {e_row:.3e} "
          f"max column {e_col:.3e}", flush=True)
    assert e_out <= tol_out and e_delta <= tol_delta, (e_out, e_delta)
    assert e_row <= 1.5 * tol_out and e_col <= 5 * tol_out, (e_row, e_col)
    if w.linear_dtype == "fp8":
        emul = bf(o_dit.video_block_rows(x0, c0, ctx0, params, w.heads, rows, fp8_act=True))
        e_emul = o_dit.rel_l2(got - xr, emul - xr)
        print(f"[parity] {name} block: update vs emulated fp8 activations {e_emul:.3e}", flush=True)
        assert e_emul <= 4e-2 and e_emul < e_delta, (e_emul, e_delta)


@pytest.mark.parametrize("name", ["dit_t_fp32", "video_t_fp32"])
def test_fp32_ragged(lib, name):
    _parity(lib, name, 1e-4, 1e-4)


@pytest.mark.parametrize("name", ["dit_t_bf16", "dit_t64_bf16", "video_t_bf16"])
def test_bf16_ragged(lib, name):
    _parity(lib, name, 2e-2, 3e-2)


def test_two_steps_fp32(lib):
    _parity(lib, "dit_t_fp32", 1e-4, 1e-4, steps=2)


@pytest.mark.parametrize("name,ks", [("dit_t_bf16", (0, 1, 2, 3)), ("video_t_fp32", (0, 1, 3)),
                                     ("dit_tiny_fp32", (0, 1, 4))])
def test_streamed_equals_resident(lib, name, ks):
    """Same kernels on the same bytes: every resident prefix gives identical bits,
    over three consecutive steps (odd ring lengths flip the slot parity)."""
    w = lwo_synth.get(name)
    outs = {}
    for k in ks:
        print(f"[resident] {name} k={k}", flush=True)
        with make_store(lib, w, k=k) as st:
            x, cond, ctx = device_inputs(w)
            run_steps(st, x, cond, ctx, steps=3)
            outs[k] = x.cpu().view(-1).view(dtype=__import__("torch").int16 if w.act_dtype == "bf16" else
                                             __import__("torch").int32).numpy().copy()
    ref = outs[ks[0]]
    for k in ks[1:]:
        assert np.array_equal(outs[k], ref), k


def test_slot_checksums_and_validation(lib):
    w = lwo_synth.get("video_t_bf16")
    from oracle import checksum as o_ck
    from oracle import layout as o_layout
    with make_store(lib, w) as st:
        for b in range(w.n_blocks):
            hs, ss = st.block_checksum(b)
            assert hs == ss == o_ck.extent_checksum(o_layout.pack_block(w, lwo_synth.block_tensors(w, b)))
        st.set_validation(True)
        x, cond, ctx = device_inputs(w)
        run_steps(st, x, cond, ctx, steps=2)
        s = st.stats()
        assert s.validation == 1 and s.checksum_mismatches == 0


def test_copy_schedule_and_arena(lib):
    """Two slots sized to the extent; one prime copy, then one copy per streamed block per step."""
    w = lwo_synth.get("dit_t_fp32")   # 3 blocks
    with make_store(lib, w) as st:
        s0 = st.stats()
        assert s0.h2d_copies == 1 and s0.device_weight_bytes == 2 * s0.extent_bytes
        x, cond, ctx = device_inputs(w)
        run_steps(st, x, cond, ctx, steps=2)
        s = st.stats()
        assert s.h2d_copies == 1 + 2 * 3 and s.h2d_bytes == s.h2d_copies * s.extent_bytes
        st.set_resident_prefix(1)
        s = st.stats()
        assert s.resident_prefix == 1 and s.device_weight_bytes == 3 * s.extent_bytes
        c0 = s.h2d_copies
        run_steps(st, x, cond, ctx, steps=2)   # ring of two: both blocks stay in the two slots
        assert st.stats().h2d_copies == c0 + 1


def test_zero_gate_identity_gpu(lib):
    w = lwo_synth.get("dit_t_bf16")
    D = w.hidden

    def tensors(b):
        t = lwo_synth.block_tensors(w, b)
        for g in (2, 5):
            t[0][g * D:(g + 1) * D] = 0   # ada.w gate rows
            t[1][g * D:(g + 1) * D] = 0   # ada.b gate entries
        return t

    with make_store(lib, w, tensors=tensors) as st:
        x, cond, ctx = device_inputs(w)
        x_in = x.clone()
        run_steps(st, x, cond, ctx, steps=2)
        assert bool((x == x_in).all())


def test_run_argument_errors(lib):
    w = lwo_synth.get("dit_tiny_fp32")
    with make_store(lib, w) as st:
        x, cond, ctx = device_inputs(w)
        with pytest.raises(lib.LwoError):
            st.run_denoise_step(x.data_ptr(), cond.data_ptr(), None, 0)          # null stream
        with pytest.raises(lib.LwoError):
            st.run_denoise_step(x.data_ptr(), cond.data_ptr(), x.data_ptr(), 1)   # ctx on the DiT kind
        with pytest.raises(lib.LwoError):
            st.set_resident_prefix(w.n_blocks + 1)


def test_fp8_video(lib):
    """fp8 linears: against the plain oracle (weights dequantised, activations
    exact) within the stated 5e-2 on the output.  Against the oracle that also
    quantises each linear's input per row (the approximation the kernels
    make) the update must be closer than against the plain oracle, and within
    4e-2: the kernels' bf16 intermediates differ from float64 by ~2^-9, which
    moves ~2^-9 / 2^-3 = 1.6% of the quantised elements across an e4m3
    rounding boundary (one code, 6-12% of the element), i.e. ~1% relative
    noise per fp8 GEMM input, seven fp8 GEMMs per block, three blocks."""
    w = lwo_synth.get("video_t_fp8")
    print("[parity] video_t_fp8", flush=True)
    from oracle import layout as o_layout
    ext = [o_layout.pack_block(w, lwo_synth.block_tensors(w, b)) for b in range(w.n_blocks)]
    x0, cond, ctx = o_dit.decode_inputs(w, *lwo_synth.step_inputs(w))
    plain = o_dit.stack_forward(w, ext, x0, cond, ctx)
    emul = o_dit.stack_forward(w, ext, x0, cond, ctx, fp8_act=True)
    with make_store(lib, w) as st:
        x, c, cx = device_inputs(w)
        run_steps(st, x, c, cx)
        got = to_f64(x).reshape(plain.shape)
    e_plain = o_dit.rel_l2(got, plain)
    e_emul = o_dit.rel_l2(got - x0, emul - x0)
    e_plain_upd = o_dit.rel_l2(got - x0, plain - x0)
    print(f"[parity] fp8: rel_l2(out, plain)={e_plain:.3e} update vs plain={e_plain_upd:.3e} "
          f"update vs emulated={e_emul:.3e}", flush=True)
    assert e_plain <= 5e-2 and e_emul <= 4e-2 and e_emul < e_plain_upd


def test_pacing_depth_does_not_change_results(lib):
    """Host pacing only changes when steps are enqueued, never what they compute."""
    w = lwo_synth.get("video_t_bf16")
    import torch
    outs = []
    for depth in (1, 0, 3):
        with make_store(lib, w) as st:
            st.set_max_inflight(depth)
            x, cond, ctx = device_inputs(w)
            run_steps(st, x, cond, ctx, steps=4)
            outs.append(x.cpu().view(torch.int16).numpy().copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    with make_store(lib, w) as st:
        with pytest.raises(lib.LwoError):
            st.set_max_inflight(17)
