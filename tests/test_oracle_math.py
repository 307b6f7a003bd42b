"""Pins for the oracle's block math (CPU only): closed forms, brute force,
library routines and structural identities."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import lwo_synth
from oracle import dit, layout


# ------------------------------------------------------------------ norms / activations

def test_layer_norm_closed_form():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((7, 33)) * 3 + 5
    y = dit.layer_norm(z)
    var = z.var(axis=-1)
    np.testing.assert_allclose(y.mean(axis=-1), 0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).mean(axis=-1), var / (var + 1e-6), rtol=1e-12)
    assert np.all(dit.layer_norm(np.full((2, 9), 3.25)) == 0)
    ref = Fn.layer_norm(torch.from_numpy(z), (33,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_rms_norm_closed_form():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 40)) * 2
    y = dit.rms_norm(z, np.ones(40))
    ms = (z ** 2).mean(axis=-1)
    np.testing.assert_allclose((y ** 2).mean(axis=-1), ms / (ms + 1e-6), rtol=1e-12)
    g = rng.standard_normal(40)
    np.testing.assert_allclose(dit.rms_norm(z, g), y * g, rtol=1e-13)
    # scale invariance (up to eps)
    np.testing.assert_allclose(dit.rms_norm(7 * z, g), dit.rms_norm(z, g), rtol=1e-6)


def test_gelu_silu_against_library():
    u = np.linspace(-12, 12, 2001)
    ref = Fn.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    np.testing.assert_allclose(dit.gelu_tanh(u), ref, rtol=1e-13, atol=1e-15)
    assert dit.gelu_tanh(np.array([0.0]))[0] == 0
    np.testing.assert_allclose(dit.silu(u), Fn.silu(torch.from_numpy(u)).numpy(), rtol=1e-13, atol=1e-15)
    assert dit.silu(np.array([0.0]))[0] == 0


# ------------------------------------------------------------------ attention

def _attention_loops(q, k, v, heads):
    """Element-by-element softmax attention in pure Python floats."""
    B, Tq, D = q.shape
    Tk = k.shape[1]
    d = D // heads
    out = np.zeros((B, Tq, D))
    for b in range(B):
        for h in range(heads):
            for i in range(Tq):
                s = [sum(q[b, i, h * d + c] * k[b, j, h * d + c] for c in range(d)) / math.sqrt(d)
                     for j in range(Tk)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = sum(e)
                for c in range(d):
                    out[b, i, h * d + c] = sum(e[j] * v[b, j, h * d + c] for j in range(Tk)) / tot
    return out


@pytest.mark.parametrize("d,heads,Tq,Tk", [(8, 2, 5, 7), (9, 3, 4, 4), (16, 1, 3, 11)])
def test_attention_brute_force(d, heads, Tq, Tk):
    rng = np.random.default_rng(d * 100 + Tq)
    D = d * heads
    q = rng.standard_normal((2, Tq, D))
    k = rng.standard_normal((2, Tk, D))
    v = rng.standard_normal((2, Tk, D))
    np.testing.assert_allclose(dit.attention(q, k, v, heads), _attention_loops(q, k, v, heads), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d", [64, 72, 128])
def test_attention_library_and_invariants(d):
    rng = np.random.default_rng(d)
    heads, Tq, Tk = 2, 50, 70
    D = heads * d
    q = rng.standard_normal((1, Tq, D)) * 2
    k = rng.standard_normal((1, Tk, D)) * 2
    v = rng.standard_normal((1, Tk, D))
    got = dit.attention(q, k, v, heads, q_chunk=16)
    th = lambda a, T: torch.from_numpy(a).reshape(1, T, heads, d).transpose(1, 2)
    ref = Fn.scaled_dot_product_attention(th(q, Tq), th(k, Tk), th(v, Tk)).transpose(1, 2).reshape(1, Tq, D).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
    # V = 1 gives exactly-1 outputs up to rounding (rows of P sum to one)
    ones = dit.attention(q, k, np.ones_like(v), heads)
    np.testing.assert_allclose(ones, 1.0, atol=1e-12)
    # sampled rows agree with the full computation
    rows = dit.attention_rows(q[0, [0, 17, 49]], k[0], v[0], heads)
    np.testing.assert_allclose(rows, got[0, [0, 17, 49]], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ blocks

def _params(w, b=0, seed_shift=0):
    t = lwo_synth.block_tensors(w.with_(seed=w.seed + seed_shift), b)
    names = [n for n, _ in lwo_synth.tensor_inventory(w)]
    return {n: a.astype(np.float64) for n, a in zip(names, t)}


def _small(kind):
    if kind == "dit":
        return lwo_synth.Workload("pin_dit", "dit", 1, 32, 2, 64, 2, 9, 0, "f32", "f32", 7)
    return lwo_synth.Workload("pin_video", "video", 1, 32, 2, 64, 2, 9, 5, "f32", "f32", 8, gamma_jitter=True)


def _inputs(w):
    x, c, ctx = lwo_synth.step_inputs(w)
    return x.astype(np.float64), c.astype(np.float64), None if ctx is None else ctx.astype(np.float64)


def test_dit_zero_gate_identity():
    w = _small("dit")
    p = _params(w)
    D = w.hidden
    for g in (2, 5):   # gate1, gate2 chunks of the modulation
        p["ada.w"][g * D:(g + 1) * D] = 0
        p["ada.b"][g * D:(g + 1) * D] = 0
    x, c, _ = _inputs(w)
    assert np.array_equal(dit.dit_block(x, c, p, w.heads), x)


def test_video_block_rows_equal_the_full_block():
    """The sampled-row video block (keys and values over every token, every
    other step on the chosen rows) gives the full block's rows, in any row
    order and with repeats, for both batches."""
    w = _small("video")
    p = _params(w)
    x, c, ctx = _inputs(w)
    for fp8_act in (False, True):
        full = dit.video_block(x, c, ctx, p, w.heads, fp8_act=fp8_act)
        for rows in ([0], [8, 0, 3], [2, 2, 7], list(range(w.tokens))):
            got = dit.video_block_rows(x, c, ctx, p, w.heads, rows, fp8_act=fp8_act)
            np.testing.assert_allclose(got, full[:, rows], rtol=1e-12, atol=1e-12)


def test_video_zero_gate_identity():
    w = _small("video")
    p = _params(w)
    x, c, ctx = _inputs(w)
    for g in (2, 5):
        c[:, g] = 0
        p["mod.table"][g] = 0
    p["cross.o.w"][:] = 0
    p["cross.o.b"][:] = 0
    assert np.array_equal(dit.video_block(x, c, ctx, p, w.heads), x)


def test_dit_bias_path_ignores_ada_weight_at_zero_cond():
    w = _small("dit")
    p = _params(w)
    x, c, _ = _inputs(w)
    c[:] = 0
    y1 = dit.dit_block(x, c, p, w.heads)
    p["ada.w"] = np.random.default_rng(9).standard_normal(p["ada.w"].shape)
    assert np.array_equal(dit.dit_block(x, c, p, w.heads), y1)


def _set_mod(p, D, vals):
    """Make the DiT modulation constant: ada.w = 0 and ada.b = chunks."""
    p["ada.w"][:] = 0
    p["ada.b"][:] = np.concatenate(vals)


def test_dit_attention_branch_special_case():
    """scale1 = -1 makes the attention input the constant row shift1, so every
    token attends to identical keys and gets v = Lin_v(shift1); with gate2 = 0
    the block adds gate1 * Lin_o(Lin_v(shift1)) to every token."""
    w = _small("dit")
    p = _params(w)
    D = w.hidden
    rng = np.random.default_rng(11)
    sh1, g1 = rng.standard_normal(D), rng.standard_normal(D)
    _set_mod(p, D, [sh1, -np.ones(D), g1, rng.standard_normal(D), rng.standard_normal(D), np.zeros(D)])
    x, c, _ = _inputs(w)
    y = dit.dit_block(x, c, p, w.heads)
    v = p["attn.v.w"] @ sh1 + p["attn.qkv.b"][2 * D:]
    want = g1 * (p["attn.o.w"] @ v + p["attn.o.b"])
    np.testing.assert_allclose(y - x, np.broadcast_to(want, x.shape), rtol=1e-10, atol=1e-12)


def test_dit_ffn_branch_special_case():
    """scale2 = -1 and gate1 = 0: every token gains gate2 * Lin_fc2(GELU(Lin_fc1(shift2)))."""
    w = _small("dit")
    p = _params(w)
    D = w.hidden
    rng = np.random.default_rng(12)
    sh2, g2 = rng.standard_normal(D), rng.standard_normal(D)
    _set_mod(p, D, [rng.standard_normal(D), rng.standard_normal(D), np.zeros(D), sh2, -np.ones(D), g2])
    x, c, _ = _inputs(w)
    y = dit.dit_block(x, c, p, w.heads)
    u = p["ffn.fc1.w"] @ sh2 + p["ffn.fc1.b"]
    want = g2 * (p["ffn.fc2.w"] @ dit.gelu_tanh(u) + p["ffn.fc2.b"])
    np.testing.assert_allclose(y - x, np.broadcast_to(want, x.shape), rtol=1e-10, atol=1e-12)


def test_video_cross_branch_single_context_token():
    """With one context token every query gets Lin_cv(ctx); with both gates zero
    the block adds Lin_co(Lin_cv(ctx)) (cross-attention is ungated)."""
    w = _small("video").with_(ctx_tokens=1)
    p = _params(w)
    D = w.hidden
    x, c, ctx = _inputs(w)
    c[:, 2] = 0
    c[:, 5] = 0
    p["mod.table"][2] = 0
    p["mod.table"][5] = 0
    y = dit.video_block(x, c, ctx, p, w.heads)
    for b in range(w.batch):
        v = p["cross.v.w"] @ ctx[b, 0] + p["cross.kv.b"][D:]
        want = p["cross.o.w"] @ v + p["cross.o.b"]
        np.testing.assert_allclose(y[b] - x[b], np.broadcast_to(want, x[b].shape), rtol=1e-10, atol=1e-12)


def test_video_qk_rmsnorm_invariance():
    """Scaling Lin_q (or Lin_k) by a positive factor leaves the block unchanged
    (up to the eps inside RMSNorm) because q and k are RMS-normalised; changing
    the norm gain does change it."""
    w = _small("video")
    p = _params(w)
    x, c, ctx = _inputs(w)
    y = dit.video_block(x, c, ctx, p, w.heads)
    D = w.hidden
    for name, sl in (("attn.q.w", slice(0, D)), ("attn.k.w", slice(D, 2 * D))):
        p2 = {k: v.copy() for k, v in p.items()}
        p2[name] *= 3.0
        p2["attn.qkv.b"][sl] *= 3.0
        # eps = 1e-6 against a mean square of about 1e-2 leaves ~1e-4 relative slack
        np.testing.assert_allclose(dit.video_block(x, c, ctx, p2, w.heads), y, rtol=0, atol=2e-6)
    p3 = {k: v.copy() for k, v in p.items()}
    p3["attn.q.norm"] *= 2.0
    assert np.abs(dit.video_block(x, c, ctx, p3, w.heads) - y).max() > 1e-3


@pytest.mark.parametrize("kind", ["dit", "video"])
def test_token_permutation_equivariance_and_batch_independence(kind):
    w = _small(kind)
    p = _params(w)
    x, c, ctx = _inputs(w)
    y = dit.block_forward(w, x, c, ctx, p)
    perm = np.random.default_rng(5).permutation(w.tokens)
    yp = dit.block_forward(w, x[:, perm], c, ctx, p)
    np.testing.assert_allclose(yp, y[:, perm], rtol=1e-12, atol=1e-12)
    y0 = dit.block_forward(w, x[:1], c[:1], None if ctx is None else ctx[:1], p)
    np.testing.assert_allclose(y0, y[:1], rtol=1e-12, atol=1e-12)


def test_stack_is_blocks_in_order():
    w = lwo_synth.get("dit_t_fp32").with_(tokens=12, n_blocks=3)
    ext = [layout.pack_block(w, lwo_synth.block_tensors(w, b)) for b in range(w.n_blocks)]
    x, c, ctx = dit.decode_inputs(w, *lwo_synth.step_inputs(w))
    y = dit.stack_forward(w, ext, x, c, ctx)
    z = x
    for b in (0, 1, 2):
        z = dit.block_forward(w, z, c, ctx, layout.unpack_block(w, ext[b]))
    assert np.array_equal(y, z)
    # order matters
    z2 = dit.stack_forward(w, ext, x, c, ctx, blocks=[1, 0, 2])
    assert np.abs(z2 - y).max() > 0


def _mixed_small(name, tokens=12):
    m = lwo_synth.get_mixed(name)
    return lwo_synth.MixedStack(m.name, tuple(t.with_(tokens=tokens) for t in m.types), m.block_type)


def test_mixed_stack_reduces_to_uniform_stack():
    """A mixed stack whose types are all the same workload is the uniform stack."""
    w = lwo_synth.get("dit_t_fp32").with_(tokens=12, n_blocks=3)
    m = lwo_synth.MixedStack("same", (w, w), (0, 1, 0))
    ext = [layout.pack_block(w, lwo_synth.block_tensors(w, b)) for b in range(3)]
    x, c, ctx = dit.decode_inputs(w, *lwo_synth.step_inputs(w))
    assert np.array_equal(dit.stack_forward_mixed(m, ext, x, c, ctx), dit.stack_forward(w, ext, x, c, ctx))


@pytest.mark.parametrize("name", ["dit_mixed_fp32", "video_mixed_fp8"])
def test_mixed_stack_uses_each_blocks_type_and_order(name):
    m = _mixed_small(name)
    ext = [layout.pack_block(m.type_of(b), lwo_synth.block_tensors(m.type_of(b), b)) for b in range(m.n_blocks)]
    assert len({len(e) for e in ext}) == 2   # two extent sizes in one stack
    x, c, ctx = dit.decode_inputs(m.inputs, *lwo_synth.step_inputs(m.inputs))
    y = dit.stack_forward_mixed(m, ext, x, c, ctx)
    assert np.isfinite(y).all() and np.abs(y - x).max() > 0
    # order matters
    rev = lwo_synth.MixedStack(m.name, m.types, tuple(reversed(m.block_type)))
    y2 = dit.stack_forward_mixed(rev, [ext[b] for b in reversed(range(m.n_blocks))], x, c, ctx)
    assert np.abs(y2 - y).max() > 0
    # a zero-gated block of either type is the identity, in a stack of the other type's blocks
    for t in (0, 1):
        wb = m.type_of(list(m.block_type).index(t))
        tens = lwo_synth.block_tensors(wb, 0)
        p = layout.unpack_block(wb, layout.pack_block(wb, tens))
        D = wb.hidden
        if wb.kind == "dit":
            for g in (2, 5):
                p["ada.w"][g * D:(g + 1) * D] = 0
                p["ada.b"][g * D:(g + 1) * D] = 0
            cz = c
        else:
            cz = c.copy()
            for g in (2, 5):
                cz[:, g] = 0
                p["mod.table"][g] = 0
            p["cross.o.w"][:] = 0
            p["cross.o.b"][:] = 0
        assert np.array_equal(dit.block_forward(wb, y, cz, ctx, p), y)
