"""Single kernels through the C ABI at the full workload shapes, checked
element by element on sampled outputs that the float64 oracle computes one
by one, and exhaustively at the smaller shapes.

Tolerances are derived from the arithmetic:
  * linear, bf16 or fp8 operands: the oracle uses the exact operand values, the
    kernel accumulates in fp32 (error <= ~K * 2^-24 * sum|a_i w_i|, bounded here
    by 1e-5 * sum|a_i w_i|) and rounds the result to bf16 (2^-9 relative); the
    check is |got - ref| <= 2^-8 |ref| + 1e-5 sum|a_i w_i| (+ the GELU slope);
  * attention: probabilities enter the PV product rounded to bf16 (2^-9
    relative each) and the output is rounded to bf16, so
    |got - ref| <= 2^-8 (sum_j p_j |v_j| + |ref|) + 1e-5;
  * LayerNorm / RMSNorm to bf16: 2^-8 relative + 1e-5;
  * fp8 row quantisation: codes bit-exact (the decision is taken in float32
    on both sides from the same float32/bf16 input).
"""
import math

import numpy as np
import pytest

from oracle import codecs
from oracle import dit as o_dit

from .conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

F32, BF16, FP8 = 0, 1, 2


def _torch():
    import torch
    return torch


def _bf16_dev(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to("cuda:0")


def _f64(t):
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def _stream():
    torch = _torch()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    return s


def _tiled_dev(lib, dtype, w_dev):
    """Device copy of a row-major bf16 (torch) or fp8 (uint8 codes) weight in
    the tiled order op_linear takes, made on the host by lwo_tile_weight."""
    torch = _torch()
    host = w_dev.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == BF16 else w_dev.cpu().numpy()
    return torch.from_numpy(lib.tile_weight(dtype, host)).to("cuda:0")


def _sample(rng, M, N, n):
    m = np.concatenate([rng.integers(0, M, n - 4), [0, M - 1, M - 1, (M // 128) * 128 % M]])
    nn = np.concatenate([rng.integers(0, N, n - 4), [0, N - 1, 0, N - 1]])
    return m.astype(np.int64), nn.astype(np.int64)


# ------------------------------------------------------------------ linear (bf16)

@pytest.mark.parametrize("M,N,K,epi", [
    (32760, 15360, 5120, 0),     # video fused QKV
    (32760, 5120, 13824, 2),     # video FFN down-projection, gated residual
    (32760, 13824, 5120, 1),     # video FFN up-projection, GELU
    (512, 10240, 5120, 0),       # video cross K|V from the context
    (32760, 5120, 5120, 3),      # video cross output projection, plain residual
    (2048, 1152, 4608, 2),       # DiT-XL FFN down, gated
    (2048, 3456, 1152, 0),       # DiT-XL QKV
    (2048, 1152, 1152, 2),       # DiT-XL attention output, gated
    (2048, 4608, 1152, 1),       # DiT-XL FFN up, GELU
    (256, 15360, 5120, 0),       # video at 256 tokens: QKV
    (256, 5120, 13824, 2),       # video at 256 tokens: FFN down, gated
    (200, 576, 2304, 1),         # ragged M and N
    (2000, 1088, 576, 2),        # gated, 128x128 tiles with ragged M and N and a stage tail
    (2048, 1152, 128, 3),        # residual, 128x128 tiles with fewer stages than the loads in flight
    (4096, 5120, 1024, 2),       # gated, 256x256 tiles, two batches split on a tile boundary (one gate row a tile)
])
def test_linear_bf16_sampled(lib, M, N, K, epi):
    torch = _torch()
    print(f"[linear bf16] M={M} N={N} K={K} epi={epi}", flush=True)
    rng = np.random.default_rng(M * 7 + N + K)
    a32 = rng.standard_normal((M, K), dtype=np.float32)
    w32 = (rng.standard_normal((N, K), dtype=np.float32) * 0.02).astype(np.float32)
    b32 = (rng.standard_normal(N, dtype=np.float32) * 0.02).astype(np.float32)
    a, w, b = _bf16_dev(a32), _bf16_dev(w32), _bf16_dev(b32)
    wt = _tiled_dev(lib, BF16, w)
    del a32, w32
    s = _stream()
    out = xr = gate = None
    T = max(1, M // 2)   # two "batches" for the gate
    if epi <= 1:
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        lib.op_linear(BF16, epi, a.data_ptr(), wt.data_ptr(), M, N, K, s.cuda_stream, bias=b.data_ptr(),
                      out=out.data_ptr(), ldo=N)
    else:
        x0 = rng.standard_normal((M, N), dtype=np.float32)
        xr = torch.from_numpy(x0).to("cuda:0")
        gate = torch.from_numpy(rng.standard_normal((2, 6 * N), dtype=np.float32)).to("cuda:0") if epi == 2 else None
        lib.op_linear(BF16, epi, a.data_ptr(), wt.data_ptr(), M, N, K, s.cuda_stream, bias=b.data_ptr(),
                      xr=xr.data_ptr(), ldx=N, gate=gate.data_ptr() if gate is not None else 0, gate_ld=6 * N,
                      rows_per_gate=T)
    s.synchronize()
    ms, ns = _sample(rng, M, N, 512)
    A = _f64(a[torch.from_numpy(ms).to("cuda:0")])
    W = _f64(w[torch.from_numpy(ns).to("cuda:0")])
    bias = _f64(b)[ns]
    y = np.einsum("ik,ik->i", A, W) + bias
    mag = np.einsum("ik,ik->i", np.abs(A), np.abs(W)) + np.abs(bias)
    if epi == 0:
        ref, got, tol = y, _f64(out)[ms, ns], 2.0 ** -8 * np.abs(y) + 1e-5 * mag
    elif epi == 1:
        ref = o_dit.gelu_tanh(y)
        got = _f64(out)[ms, ns]
        tol = 2.0 ** -8 * np.abs(ref) + 1.2e-5 * mag + 1e-6
    else:
        g = _f64(gate)[ms // T, ns] if epi == 2 else 1.0
        ref = x0[ms, ns].astype(np.float64) + g * y
        got = _f64(xr)[ms, ns]
        tol = 1e-5 * np.abs(g) * mag + 1e-6 * np.abs(ref) + 1e-6
    err = np.abs(got - ref)
    print(f"[linear bf16] max err/tol = {np.max(err / tol):.3f}", flush=True)
    assert np.all(err <= tol), (np.argmax(err / tol), float(np.max(err / tol)))


# ------------------------------------------------------------------ linear (fp8)

@pytest.mark.parametrize("M,N,K,seg", [(32760, 15360, 5120, 5120), (32760, 5120, 13824, 5120), (300, 1024, 256, 1024),
                                       (2048, 1152, 4608, 1152),    # 144 tiles of 128x128, one per CU
                                       (2048, 3456, 1024, 1152),    # 216 tiles of 256x128 (grouped look-ahead)
                                       (2000, 1088, 640, 64)])      # ragged M and N (a half tile of weight rows)
def test_linear_fp8_sampled(lib, M, N, K, seg):
    torch = _torch()
    print(f"[linear fp8] M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + N + K)
    a_codes, a_sc = codecs.quantize_rows_e4m3(rng.standard_normal((M, K), dtype=np.float32))
    w_codes = codecs.e4m3_encode(rng.standard_normal((N, K), dtype=np.float32) * np.float32(60))
    w_sc = (rng.uniform(0.5, 2.0, N // seg) * 1e-3).astype(np.float32)
    b32 = (rng.standard_normal(N, dtype=np.float32) * 0.02).astype(np.float32)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
    a, w, asc, wsc, b = dev(a_codes), dev(lib.tile_weight(FP8, w_codes)), dev(a_sc), dev(w_sc), _bf16_dev(b32)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    s = _stream()
    lib.op_linear(FP8, 0, a.data_ptr(), w.data_ptr(), M, N, K, s.cuda_stream, a_scale=asc.data_ptr(),
                  w_scale=wsc.data_ptr(), w_seg=seg, bias=b.data_ptr(), out=out.data_ptr(), ldo=N)
    s.synchronize()
    ms, ns = _sample(rng, M, N, 512)
    A = codecs.e4m3_decode(a_codes[ms])
    W = codecs.e4m3_decode(w_codes[ns])
    scale = w_sc[ns // seg].astype(np.float64) * a_sc[ms].astype(np.float64)
    bias = codecs.bf16_round(b32)[ns]
    y = np.einsum("ik,ik->i", A, W) * scale + bias
    mag = np.einsum("ik,ik->i", np.abs(A), np.abs(W)) * scale + np.abs(bias)
    got = _f64(out)[ms, ns]
    err = np.abs(got - y)
    tol = 2.0 ** -8 * np.abs(y) + 1e-5 * mag
    print(f"[linear fp8] max err/tol = {np.max(err / tol):.3f}", flush=True)
    assert np.all(err <= tol)


# ------------------------------------------------------------------ attention

def _attn_case(lib, dtype, B, H, Tq, Tk, d, fused_qkv, n_rows, seed):
    torch = _torch()
    rng = np.random.default_rng(seed)
    D = H * d
    tdt = torch.bfloat16 if dtype == BF16 else torch.float32
    conv = (lambda a: _bf16_dev(a)) if dtype == BF16 else (lambda a: torch.from_numpy(a).to("cuda:0"))
    if fused_qkv:   # q | k | v in one [B*T, 3D] buffer, as the self-attention step lays them out
        qkv = conv(rng.standard_normal((B * Tq, 3 * D), dtype=np.float32))
        q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
        ld_q = ld_k = ld_v = 3 * D
    else:
        q = conv(rng.standard_normal((B * Tq, D), dtype=np.float32))
        kv = conv(rng.standard_normal((B * Tk, 2 * D), dtype=np.float32))
        k, v = kv[:, :D], kv[:, D:]
        ld_q, ld_k, ld_v = D, 2 * D, 2 * D
    o = torch.empty((B * Tq, D), dtype=tdt, device="cuda:0")
    s = _stream()
    lib.op_attention(dtype, q.data_ptr(), ld_q, k.data_ptr(), ld_k, v.data_ptr(), ld_v, o.data_ptr(), D, B, H, Tq, Tk,
                     d, s.cuda_stream)
    s.synchronize()
    got_all = _f64(o)
    worst = 0.0
    for b in range(B):
        rows = np.unique(np.concatenate([rng.integers(0, Tq, max(n_rows - 3, 1)), [0, Tq - 1, (Tq - 1) // 128 * 128]]))
        Q = _f64(q[b * Tq + torch.from_numpy(rows).to("cuda:0")])
        K = _f64(k[b * Tk:(b + 1) * Tk])
        V = _f64(v[b * Tk:(b + 1) * Tk])
        ref = o_dit.attention_rows(Q, K, V, H)
        # sum_j p_j |v_j| per (row, head, column)
        mag = o_dit.attention_rows(Q, K, np.abs(V), H)
        got = got_all[b * Tq + rows]
        if dtype == BF16:
            tol = 2.0 ** -8 * (mag + np.abs(ref)) + 1e-5
        else:
            tol = 1e-5 * (mag + np.abs(ref)) + 1e-6
        r = np.max(np.abs(got - ref) / tol)
        worst = max(worst, float(r))
        assert np.all(np.abs(got - ref) <= tol), (b, float(r))
    print(f"[attention] B={B} H={H} Tq={Tq} Tk={Tk} d={d}: max err/tol = {worst:.3f}", flush=True)


@pytest.mark.parametrize("B,H,Tq,Tk,d,fused,rows", [
    (1, 40, 32760, 32760, 128, True, 24),     # video self-attention
    (1, 40, 32760, 512, 128, False, 64),      # video cross-attention
    (1, 40, 256, 256, 128, True, 256),        # video at 256 tokens: every row
    (2, 16, 1024, 1024, 72, True, 1024),      # DiT-XL: every row
    (1, 4, 333, 333, 64, True, 333),          # ragged, d 64
    (2, 2, 200, 40, 72, False, 200),          # cross with fewer keys than one tile
    (2, 3, 77, 40, 128, False, 77),           # d 128: one partial query block, one partial key tile
    (1, 2, 300, 130, 128, True, 300),         # d 128: ragged queries, three key tiles, the last partial
    (1, 3, 129, 128, 128, False, 129),        # d 128: two full key tiles (even tile count)
    (2, 2, 64, 64, 128, True, 64),            # d 128: one full key tile
    (1, 2, 520, 700, 128, False, 520),        # d 128: eleven key tiles, three query blocks
    # d 128 beyond 1024 keys (eight-wavefront workgroups): odd and even tile counts, partial last tiles
    (2, 2, 300, 1025, 128, False, 300),       # 17 key tiles, the last with one key
    (2, 1, 130, 1057, 128, False, 130),       # 17 tiles, the last with 33 keys (its second half one key)
    (1, 2, 1100, 1100, 128, True, 1100),      # 18 tiles, the last with 12 keys; ragged queries, every row
    (1, 2, 200, 1120, 128, False, 200),       # 18 tiles, the last with 32 keys (its second half empty)
    (1, 3, 513, 1152, 128, False, 513),       # 18 full tiles, three query blocks, one row in the last
    (2, 2, 100, 150, 72, False, 100),         # key tiles split over two groups: the second has one partial tile
    (1, 16, 2100, 300, 72, False, 48),        # d 72 with more query tiles than CUs: no key split
    (1, 64, 600, 200, 64, False, 48),         # d 64 with more query tiles than CUs: no key split
])
def test_attention_bf16(lib, B, H, Tq, Tk, d, fused, rows):
    print(f"[attention bf16] B={B} H={H} Tq={Tq} Tk={Tk} d={d}", flush=True)
    _attn_case(lib, BF16, B, H, Tq, Tk, d, fused, rows, seed=Tq + Tk + d)


@pytest.mark.parametrize("pattern,d,Tk", [("growing", 128, 1100), ("growing", 72, 1000), ("late_key", 128, 1100),
                                          ("late_key", 64, 700)])
def test_attention_bf16_reference_point_moves(lib, pattern, d, Tk):
    """Scores that rise far above the first tiles' maximum: the kernel's
    probabilities are taken against a reference point that it moves only when
    a tile's row sum passes 2^32, so these inputs must take that path (key
    norms growing 30x along the keys, or one key in the last tile scaled to
    dominate about half of the queries) and still match the oracle."""
    torch = _torch()
    print(f"[attention bf16 reference] {pattern} d={d} Tk={Tk}", flush=True)
    rng = np.random.default_rng(Tk + d + len(pattern))
    B, H, Tq = 1, 2, 300
    D = H * d
    q32 = rng.standard_normal((B * Tq, D), dtype=np.float32)
    k32 = rng.standard_normal((B * Tk, D), dtype=np.float32)
    if pattern == "growing":
        k32 *= (1.0 + 30.0 * np.arange(Tk, dtype=np.float32) / Tk)[:, None]
    else:
        k32[Tk - 3] = 2000.0 / np.sqrt(d)
    v32 = rng.standard_normal((B * Tk, D), dtype=np.float32)
    q, k, v = _bf16_dev(q32), _bf16_dev(k32), _bf16_dev(v32)
    o = torch.empty((B * Tq, D), dtype=torch.bfloat16, device="cuda:0")
    s = _stream()
    lib.op_attention(BF16, q.data_ptr(), D, k.data_ptr(), D, v.data_ptr(), D, o.data_ptr(), D, B, H, Tq, Tk, d,
                     s.cuda_stream)
    s.synchronize()
    Q, K, V = _f64(q), _f64(k), _f64(v)
    ref = o_dit.attention_rows(Q, K, V, H)
    mag = o_dit.attention_rows(Q, K, np.abs(V), H)
    got = _f64(o)
    tol = 2.0 ** -8 * (mag + np.abs(ref)) + 1e-5
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    print(f"[attention bf16 reference] max err/tol = {np.max(err / tol):.3f}", flush=True)
    assert np.all(err <= tol), float(np.max(err / tol))


@pytest.mark.parametrize("B,H,Tq,Tk,d", [(1, 4, 64, 64, 64), (2, 8, 200, 200, 72), (1, 2, 77, 40, 128)])
def test_attention_f32(lib, B, H, Tq, Tk, d):
    _attn_case(lib, F32, B, H, Tq, Tk, d, Tq == Tk, Tq, seed=d + Tq)


# ------------------------------------------------------------------ row kernels

@pytest.mark.parametrize("M,D", [(32760, 5120), (2048, 1152), (333, 256),
                                 (203, 2048),    # the widest rows of one wavefront each, a 4-row workgroup short of rows
                                 (131, 2112)])   # the narrowest of two wavefronts per row (five float4 chunks a lane)
def test_layernorm_modulated_and_fp8(lib, M, D):
    torch = _torch()
    print(f"[layernorm] M={M} D={D}", flush=True)
    rng = np.random.default_rng(M + D)
    x = (rng.standard_normal((M, D), dtype=np.float32) * 3 + 1).astype(np.float32)
    B = 2 if M % 2 == 0 else 1
    mod = rng.standard_normal((B, 6, D), dtype=np.float32) * 0.5
    xd = torch.from_numpy(x).to("cuda:0")
    md = torch.from_numpy(mod).to("cuda:0")
    s = _stream()
    o16 = torch.empty((M, D), dtype=torch.bfloat16, device="cuda:0")
    o32 = torch.empty((M, D), dtype=torch.float32, device="cuda:0")
    o8 = torch.empty((M, D), dtype=torch.uint8, device="cuda:0")
    sc8 = torch.empty(M, dtype=torch.float32, device="cuda:0")
    T = M // B
    kw = dict(mod=md.data_ptr(), rows_per_batch=T, shift_chunk=3, scale_chunk=4)
    lib.op_layernorm(xd.data_ptr(), M, D, o16.data_ptr(), BF16, s.cuda_stream, **kw)
    lib.op_layernorm(xd.data_ptr(), M, D, o32.data_ptr(), F32, s.cuda_stream, **kw)
    lib.op_layernorm(xd.data_ptr(), M, D, o8.data_ptr(), FP8, s.cuda_stream, out_scale=sc8.data_ptr(), **kw)
    s.synchronize()
    bi = np.arange(M) // T
    ref = o_dit.layer_norm(x.astype(np.float64)) * (1 + mod[bi, 4].astype(np.float64)) + mod[bi, 3]
    got16, got32 = _f64(o16), _f64(o32)
    assert np.all(np.abs(got32 - ref) <= 1e-5 * (np.abs(ref) + 1))
    assert np.all(np.abs(got16 - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)
    # fp8 output: the same float32 row values, quantised; codes decided in float32 on both sides
    codes, scales = codecs.quantize_rows_e4m3(o32.cpu().numpy())
    assert np.array_equal(sc8.cpu().numpy(), scales)
    assert np.array_equal(o8.cpu().numpy(), codes)


@pytest.mark.parametrize("M,N", [(32760, 5120), (32760, 13824), (300, 256)])
def test_quantize_rows_bit_exact(lib, M, N):
    torch = _torch()
    rng = np.random.default_rng(M + N)
    x = rng.standard_normal((M, N), dtype=np.float32) * np.exp(rng.uniform(-3, 3, (M, 1))).astype(np.float32)
    x[min(3, M - 1)] = 0.0
    xd = _bf16_dev(x)
    codes = torch.empty((M, N), dtype=torch.uint8, device="cuda:0")
    sc = torch.empty(M, dtype=torch.float32, device="cuda:0")
    s = _stream()
    lib.op_quantize_rows(xd.data_ptr(), M, N, codes.data_ptr(), sc.data_ptr(), s.cuda_stream)
    s.synchronize()
    ref_codes, ref_sc = codecs.quantize_rows_e4m3(xd.float().cpu().numpy())
    assert np.array_equal(sc.cpu().numpy(), ref_sc)
    assert np.array_equal(codes.cpu().numpy(), ref_codes)


@pytest.mark.parametrize("M,D,dtype", [(32760, 5120, BF16), (300, 256, F32)])
def test_rmsnorm_qk(lib, M, D, dtype):
    torch = _torch()
    rng = np.random.default_rng(M + D)
    qkv = rng.standard_normal((M, 3 * D), dtype=np.float32) * 2
    gq = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    gk = (1 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    conv = _bf16_dev if dtype == BF16 else (lambda a: torch.from_numpy(a).to("cuda:0"))
    t, gqd, gkd = conv(qkv), conv(gq), conv(gk)
    before = _f64(t)
    s = _stream()
    lib.op_rmsnorm_qk(dtype, t.data_ptr(), M, D, gqd.data_ptr(), gkd.data_ptr(), s.cuda_stream)
    s.synchronize()
    got = _f64(t)
    gq64, gk64 = _f64(gqd), _f64(gkd)
    ref_q = o_dit.rms_norm(before[:, :D], gq64)
    ref_k = o_dit.rms_norm(before[:, D:2 * D], gk64)
    rel = 2.0 ** -8 if dtype == BF16 else 1e-5
    assert np.all(np.abs(got[:, :D] - ref_q) <= rel * np.abs(ref_q) + 1e-5)
    assert np.all(np.abs(got[:, D:2 * D] - ref_k) <= rel * np.abs(ref_k) + 1e-5)
    assert np.array_equal(got[:, 2 * D:], before[:, 2 * D:])   # v untouched


def test_ops_with_no_rows_write_nothing(lib):
    """M = 0 (and Tq = 0) is a valid, empty call: it returns OK and leaves every output as it was."""
    torch = _torch()
    print("[empty] M = 0 for every op", flush=True)
    s = _stream()
    a = torch.zeros(64 * 64, dtype=torch.bfloat16, device="cuda:0")
    w = torch.zeros(64 * 128, dtype=torch.uint8, device="cuda:0")
    sc = torch.ones(64, dtype=torch.float32, device="cuda:0")
    sent = torch.full((4096,), 7.0, dtype=torch.float32, device="cuda:0")
    s8 = torch.full((4096,), 7, dtype=torch.uint8, device="cuda:0")
    lib.op_linear(BF16, 0, a.data_ptr(), a.data_ptr(), 0, 64, 64, s.cuda_stream, out=sent.data_ptr(), ldo=64)
    lib.op_linear(BF16, 2, a.data_ptr(), a.data_ptr(), 0, 64, 64, s.cuda_stream, xr=sent.data_ptr(), ldx=64,
                  gate=sc.data_ptr(), gate_ld=64, rows_per_gate=1)
    lib.op_linear(FP8, 0, w.data_ptr(), w.data_ptr(), 0, 64, 128, s.cuda_stream, a_scale=sc.data_ptr(),
                  w_scale=sc.data_ptr(), w_seg=64, out=sent.data_ptr(), ldo=64)
    lib.op_attention(BF16, a.data_ptr(), 64, a.data_ptr(), 64, a.data_ptr(), 64, sent.data_ptr(), 64, 1, 1, 0, 4, 64,
                     s.cuda_stream)
    lib.op_layernorm(sent.data_ptr(), 0, 64, sent.data_ptr(), BF16, s.cuda_stream)
    lib.op_layernorm(sent.data_ptr(), 0, 64, s8.data_ptr(), FP8, s.cuda_stream, out_scale=sent.data_ptr())
    lib.op_quantize_rows(a.data_ptr(), 0, 64, s8.data_ptr(), sent.data_ptr(), s.cuda_stream)
    lib.op_rmsnorm_qk(BF16, sent.data_ptr(), 0, 64, a.data_ptr(), a.data_ptr(), s.cuda_stream)
    lib.op_rmsnorm_qk(F32, sent.data_ptr(), 0, 64, sent.data_ptr(), sent.data_ptr(), s.cuda_stream)
    s.synchronize()
    assert bool((sent == 7.0).all()) and bool((s8 == 7).all())


def test_op_argument_validation(lib):
    torch = _torch()
    a = torch.zeros(64 * 64, dtype=torch.bfloat16, device="cuda:0")
    s = _stream()
    with pytest.raises(lib.LwoError):   # K not a multiple of 64
        lib.op_linear(BF16, 0, a.data_ptr(), a.data_ptr(), 8, 8, 32, s.cuda_stream, out=a.data_ptr(), ldo=8)
    with pytest.raises(lib.LwoError):   # N not a multiple of 64 (tiled bf16 weights)
        lib.op_linear(BF16, 0, a.data_ptr(), a.data_ptr(), 8, 96, 64, s.cuda_stream, out=a.data_ptr(), ldo=96)
    with pytest.raises(lib.LwoError):   # misaligned pointer
        lib.op_linear(BF16, 0, a.data_ptr() + 2, a.data_ptr(), 8, 8, 64, s.cuda_stream, out=a.data_ptr(), ldo=8)
    with pytest.raises(lib.LwoError):   # head dim 96
        lib.op_attention(BF16, a.data_ptr(), 96, a.data_ptr(), 96, a.data_ptr(), 96, a.data_ptr(), 96, 1, 1, 4, 4,
                         96, s.cuda_stream)


# ------------------------------------------------------------------ MFMA throughput probe

def test_probe_mfma_counts_and_rejects(lib):
    torch = _torch()
    s = _stream()
    sink = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    for dt, per in ((BF16, 32768), (FP8, 131072)):
        fl = lib.probe_mfma(dt, 8, 10, sink.data_ptr(), sink.numel(), s.cuda_stream)
        s.synchronize()
        assert fl == 8 * 4 * 4 * 10 * per
        assert bool(torch.isfinite(sink).all())
    with pytest.raises(lib.LwoError):
        lib.probe_mfma(F32, 8, 10, sink.data_ptr(), sink.numel(), s.cuda_stream)
    with pytest.raises(lib.LwoError):   # sink shorter than blocks * 256 floats
        lib.probe_mfma(BF16, 9, 10, sink.data_ptr(), sink.numel(), s.cuda_stream)
