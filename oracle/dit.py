"""Float64 forward of the DiT block stack with every weight resident.

Test infrastructure (see the package docstring); not imported by the library.

Offloading streams block weights but leaves each block's forward untouched
("CPU Offloading for Diffusion Models", section "Layerwise (Blockwise)
Offloading / How It Works", execution-flow table: block i computes while
block i+1 is prefetched; the computation of block i is the model's own).  The
block math below is the workload definition of the diffusion transformers
being offloaded (adaLN-zero DiT blocks; a video DiT block with q/k RMSNorm and
cross-attention to a text context).  Readings taken where the definition is
open are listed in the design notes and repeated at each function.

Conventions: row-major; ``Lin(z) = z @ W.T + b`` with W of shape
[out, in]; heads split the feature axis contiguously (head h owns features
[h*d, (h+1)*d)).
"""
from __future__ import annotations

import math

import numpy as np

from . import codecs, layout

LN_EPS = 1e-6
RMS_EPS = 1e-6


# ------------------------------------------------------------------ pieces

def layer_norm(z: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """(z - mean) / sqrt(var + eps) over the last axis; biased variance, no
    affine parameters."""
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + eps)


def rms_norm(z: np.ndarray, gamma: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """z / sqrt(mean(z^2) + eps) * gamma over the last axis."""
    return z / np.sqrt((z * z).mean(axis=-1, keepdims=True) + eps) * gamma


def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def linear(z: np.ndarray, w: np.ndarray, b: np.ndarray | None) -> np.ndarray:
    y = z @ w.T
    return y if b is None else y + b


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, heads: int, q_chunk: int = 2048) -> np.ndarray:
    """Multi-head softmax attention without a mask.

    q [B,Tq,D], k and v [B,Tk,D] -> [B,Tq,D].  Per (batch, head):
    S = q_h k_h^T / sqrt(d); P = softmax over keys (shifted by the row
    maximum); O = P v_h.  Query rows are taken in chunks only to bound
    memory; every chunk sees every key, so the result is exact."""
    B, Tq, D = q.shape
    d = D // heads
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        for h in range(heads):
            sl = slice(h * d, (h + 1) * d)
            kh = k[b, :, sl]
            vh = v[b, :, sl]
            for s in range(0, Tq, q_chunk):
                qh = q[b, s:s + q_chunk, sl]
                S = (qh @ kh.T) * scale
                S -= S.max(axis=-1, keepdims=True)
                P = np.exp(S)
                P /= P.sum(axis=-1, keepdims=True)
                out[b, s:s + q_chunk, sl] = P @ vh
    return out


def attention_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, heads: int) -> np.ndarray:
    """The same attention for a few query rows q_rows [n, D] of one batch
    element against keys k, v [Tk, D]; used to sample full-size outputs."""
    n, D = q_rows.shape
    d = D // heads
    out = np.empty((n, D))
    for h in range(heads):
        sl = slice(h * d, (h + 1) * d)
        S = (q_rows[:, sl] @ k[:, sl].T) / math.sqrt(d)
        S -= S.max(axis=-1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=-1, keepdims=True)
        out[:, sl] = P @ v[:, sl]
    return out


def chunks6(m: np.ndarray):
    """Split modulation [B, 6, D] into shift1, scale1, gate1, shift2, scale2,
    gate2, each [B, 1, D] (broadcast over tokens)."""
    return [m[:, i, None, :] for i in range(6)]


# ------------------------------------------------------------------ blocks

def dit_block(x: np.ndarray, cond: np.ndarray, p: dict, heads: int) -> np.ndarray:
    """adaLN-zero DiT block.

    m = Lin_ada(SiLU(cond)) gives, in this order, shift1, scale1, gate1,
    shift2, scale2, gate2 (each [B, D]);
    h = LN(x)(1 + scale1) + shift1;  [q|k|v] = Lin_qkv(h);
    x = x + gate1 * Lin_o(Attn(q, k, v));
    h = LN(x)(1 + scale2) + shift2;
    x = x + gate2 * Lin_fc2(GELU(Lin_fc1(h)))."""
    B, T, D = x.shape
    m = linear(silu(cond), p["ada.w"], p["ada.b"]).reshape(B, 6, D)
    sh1, sc1, g1, sh2, sc2, g2 = chunks6(m)
    h = layer_norm(x) * (1.0 + sc1) + sh1
    wqkv = np.concatenate([p["attn.q.w"], p["attn.k.w"], p["attn.v.w"]], axis=0)
    qkv = linear(h, wqkv, p["attn.qkv.b"])
    q, k, v = qkv[..., :D], qkv[..., D:2 * D], qkv[..., 2 * D:]
    a = attention(q, k, v, heads)
    x = x + g1 * linear(a, p["attn.o.w"], p["attn.o.b"])
    h = layer_norm(x) * (1.0 + sc2) + sh2
    x = x + g2 * linear(gelu_tanh(linear(h, p["ffn.fc1.w"], p["ffn.fc1.b"])), p["ffn.fc2.w"], p["ffn.fc2.b"])
    return x


def fp8_activation(z: np.ndarray, stored_bf16: bool) -> np.ndarray:
    """Emulate the input of an fp8 linear: the activation (rounded to bf16
    first when it is stored in bf16 before quantisation) is quantised per row
    to e4m3 with scale amax/448 in float32 and dequantised exactly."""
    z32 = z.astype(np.float32)
    if stored_bf16:
        z32 = codecs.bf16_round(z32).astype(np.float32)
    q, s = codecs.quantize_rows_e4m3(z32)
    return codecs.e4m3_decode(q) * s.astype(np.float64)[..., None]


def video_block(x: np.ndarray, cond: np.ndarray, ctx: np.ndarray, p: dict, heads: int,
                fp8_act: bool = False) -> np.ndarray:
    """Video DiT block.

    m = cond + M_blk (cond [B,6,D], the block's own [6,D] table); same chunk
    order as the DiT kind;
    h = LN(x)(1 + scale1) + shift1;
    q = RMS_gq(Lin_q(h)), k = RMS_gk(Lin_k(h)) over the full hidden width,
    v = Lin_v(h);  x = x + gate1 * Lin_o(Attn(q, k, v));
    x = x + Lin_co(Attn(Lin_cq(LN(x)), Lin_ck(ctx), Lin_cv(ctx)))  (ungated);
    h = LN(x)(1 + scale2) + shift2;  x = x + gate2 * Lin_fc2(GELU(Lin_fc1(h))).

    fp8_act=True additionally quantises the input of every linear per row to
    e4m3 (the approximation an fp8 GEMM makes; see fp8_activation)."""
    B, T, D = x.shape
    qa = (lambda z, stored_bf16=False: fp8_activation(z, stored_bf16)) if fp8_act else (lambda z, stored_bf16=False: z)
    m = cond + p["mod.table"][None, :, :]
    sh1, sc1, g1, sh2, sc2, g2 = chunks6(m)
    h = qa(layer_norm(x) * (1.0 + sc1) + sh1)
    bq, bk, bv = p["attn.qkv.b"][:D], p["attn.qkv.b"][D:2 * D], p["attn.qkv.b"][2 * D:]
    q = rms_norm(linear(h, p["attn.q.w"], bq), p["attn.q.norm"])
    k = rms_norm(linear(h, p["attn.k.w"], bk), p["attn.k.norm"])
    v = linear(h, p["attn.v.w"], bv)
    x = x + g1 * linear(qa(attention(q, k, v, heads), True), p["attn.o.w"], p["attn.o.b"])
    cq = linear(qa(layer_norm(x)), p["cross.q.w"], p["cross.q.b"])
    bck, bcv = p["cross.kv.b"][:D], p["cross.kv.b"][D:]
    ctx_in = qa(ctx, True)
    ck = linear(ctx_in, p["cross.k.w"], bck)
    cv = linear(ctx_in, p["cross.v.w"], bcv)
    x = x + linear(qa(attention(cq, ck, cv, heads), True), p["cross.o.w"], p["cross.o.b"])
    h = qa(layer_norm(x) * (1.0 + sc2) + sh2)
    x = x + g2 * linear(qa(gelu_tanh(linear(h, p["ffn.fc1.w"], p["ffn.fc1.b"])), True), p["ffn.fc2.w"], p["ffn.fc2.b"])
    return x


def video_block_rows(x: np.ndarray, cond: np.ndarray, ctx: np.ndarray, p: dict, heads: int,
                     rows, fp8_act: bool = False) -> np.ndarray:
    """video_block's output at token indices ``rows`` only (every batch),
    [B, len(rows), D].  Self-attention's keys and values need every token;
    every other step of the block (the per-row fp8 quantisation included)
    acts on each token's row alone, so it is taken on the selected rows.  The
    steps and their order are video_block's."""
    B, T, D = x.shape
    rows = np.asarray(rows)
    qa = (lambda z, stored_bf16=False: fp8_activation(z, stored_bf16)) if fp8_act else (lambda z, stored_bf16=False: z)
    m = cond + p["mod.table"][None, :, :]
    sh1, sc1, g1, sh2, sc2, g2 = chunks6(m)
    h = qa(layer_norm(x) * (1.0 + sc1) + sh1)                  # every token: keys and values
    bq, bk, bv = p["attn.qkv.b"][:D], p["attn.qkv.b"][D:2 * D], p["attn.qkv.b"][2 * D:]
    k = rms_norm(linear(h, p["attn.k.w"], bk), p["attn.k.norm"])
    v = linear(h, p["attn.v.w"], bv)
    xr = x[:, rows]
    q = rms_norm(linear(h[:, rows], p["attn.q.w"], bq), p["attn.q.norm"])
    del h
    xr = xr + g1 * linear(qa(attention(q, k, v, heads), True), p["attn.o.w"], p["attn.o.b"])
    cq = linear(qa(layer_norm(xr)), p["cross.q.w"], p["cross.q.b"])
    bck, bcv = p["cross.kv.b"][:D], p["cross.kv.b"][D:]
    ctx_in = qa(ctx, True)
    ck = linear(ctx_in, p["cross.k.w"], bck)
    cv = linear(ctx_in, p["cross.v.w"], bcv)
    xr = xr + linear(qa(attention(cq, ck, cv, heads), True), p["cross.o.w"], p["cross.o.b"])
    hr = qa(layer_norm(xr) * (1.0 + sc2) + sh2)
    return xr + g2 * linear(qa(gelu_tanh(linear(hr, p["ffn.fc1.w"], p["ffn.fc1.b"])), True), p["ffn.fc2.w"],
                            p["ffn.fc2.b"])


def block_forward(w, x, cond, ctx, params: dict, fp8_act: bool = False) -> np.ndarray:
    if w.kind == "dit":
        return dit_block(x, cond, params, w.heads)
    return video_block(x, cond, ctx, params, w.heads, fp8_act=fp8_act)


# ------------------------------------------------------------------ stack

def decode_inputs(w, x, cond, ctx):
    """Inputs as the library receives them: float32 for an fp32 workload,
    the bf16 rounding of the float32 draws otherwise; returned as float64."""
    def dec(a):
        if a is None:
            return None
        a = np.asarray(a, dtype=np.float32)
        return codecs.bf16_round(a) if w.act_dtype == "bf16" else a.astype(np.float64)
    return dec(x), dec(cond), dec(ctx)


def stack_forward(w, extents, x, cond, ctx, blocks=None, fp8_act: bool = False) -> np.ndarray:
    """Apply blocks (default: all) in order to float64 inputs.

    ``extents`` is a sequence (or callable b -> bytes) giving each block's
    packed extent; the weights the oracle uses are decoded from it, so they
    are exactly the stored values."""
    blocks = range(w.n_blocks) if blocks is None else blocks
    for b in blocks:
        ext = extents(b) if callable(extents) else extents[b]
        params = layout.unpack_block(w, ext)
        x = block_forward(w, x, cond, ctx, params, fp8_act=fp8_act)
    return x


def stack_forward_mixed(m, extents, x, cond, ctx, fp8_act: bool = False) -> np.ndarray:
    """A stack of several block types applied in order: block b is decoded and
    run with its own type's workload ``m.type_of(b)`` (the per-block reading of
    a model with several block types streamed through one ring).  ``fp8_act``
    applies to the blocks whose linears are fp8."""
    for b in range(m.n_blocks):
        wb = m.type_of(b)
        ext = extents(b) if callable(extents) else extents[b]
        params = layout.unpack_block(wb, ext)
        x = block_forward(wb, x, cond, ctx, params, fp8_act=fp8_act and wb.linear_dtype == "fp8")
    return x


def rel_l2(y: np.ndarray, ref: np.ndarray) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    return float(np.linalg.norm((y - ref).ravel()) / (den if den > 0 else 1.0))
