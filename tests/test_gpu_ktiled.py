"""The k-tiled activation layout (LWO_KTILED) through the C ABI.

The layout only moves bytes: a kernel that reads or writes k-tiled rows
must produce the same bits as with row-major rows.  Each case runs both
forms on the same device inputs and compares every output element bit for
bit, and checks sampled outputs against the float64 oracle with the
tolerances of test_gpu_ops (derived there from the arithmetic).  The
host-side tiling is the oracle's definition of the tiled order
(oracle.layout.tile_bytes), applied to rows padded to whole 64-row bands.
Padding rows of a k-tiled output hold a sentinel that must survive.
"""
import numpy as np
import pytest

from oracle import codecs
from oracle import dit as o_dit
from oracle import layout as o_layout

from .conftest import gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

F32, BF16, FP8 = 0, 1, 2
ROWS, KTILED = 0, 1
SENT = 0x5A


def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    return s


def _bytes(t):
    """[M, n] device tensor -> [M, n * element bytes] uint8 host array."""
    torch = _torch()
    return t.contiguous().view(torch.uint8).cpu().numpy().reshape(t.shape[0], -1)


def _pad64(m):
    return (m + 63) // 64 * 64


def _tile_dev(rows_u8):
    """Row-major bytes [M, R] -> device uint8 buffer of the k-tiled order (rows padded with SENT)."""
    torch = _torch()
    M, R = rows_u8.shape
    full = np.full((_pad64(M), R), SENT, np.uint8)
    full[:M] = rows_u8
    return torch.from_numpy(o_layout.tile_bytes(full)).to("cuda:0")


def _untile(buf, M, R):
    """Device k-tiled buffer -> (row-major bytes [M, R], padding rows' bytes)."""
    rows = o_layout.untile_bytes(buf.cpu().numpy(), _pad64(M), R)
    return rows[:M], rows[M:]


def _tiled_out(M, R):
    torch = _torch()
    return torch.full((_pad64(M) * R,), SENT, dtype=torch.uint8, device="cuda:0")


def _bf16_f64(u16):
    """bf16 bit patterns (uint16) -> float64 values."""
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ linear

@pytest.mark.parametrize("M,N,K,epi", [
    (32760, 15360, 5120, 0),     # video fused QKV: 256x256 tiles, 16x16x32 MFMAs
    (32760, 13824, 5120, 1),     # video FFN up, GELU, k-tiled output as well
    (2048, 1152, 4608, 2),       # DiT-XL FFN down, gated: 128x128 tiles, 128-byte stages
    (2048, 3456, 1152, 0),       # DiT-XL QKV: 256x128 tiles
    (2000, 1088, 576, 2),        # ragged M (a partial band) and N, a stage tail
    (200, 576, 2304, 1),         # ragged M below one tile, k-tiled GELU output with padding rows
    (130, 512, 128, 3),          # 128x64 tiles, plain residual
])
def test_linear_bf16_ktiled(lib, M, N, K, epi):
    torch = _torch()
    print(f"[ktiled linear bf16] M={M} N={N} K={K} epi={epi}", flush=True)
    rng = np.random.default_rng(M * 3 + N + K)
    a = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to(torch.bfloat16).to("cuda:0")
    w = torch.from_numpy(rng.standard_normal((N, K), dtype=np.float32) * 0.02).to(torch.bfloat16).to("cuda:0")
    b = torch.from_numpy(rng.standard_normal(N, dtype=np.float32) * 0.02).to(torch.bfloat16).to("cuda:0")
    wt = torch.from_numpy(lib.tile_weight(BF16, _bytes(w).view(np.uint16))).to("cuda:0")
    at = _tile_dev(_bytes(a))
    s = _stream()
    if epi <= 1:
        ref_out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        t_out = _tiled_out(M, 2 * N)
        lib.op_linear(BF16, epi, a.data_ptr(), wt.data_ptr(), M, N, K, s.cuda_stream, bias=b.data_ptr(),
                      out=ref_out.data_ptr(), ldo=N)
        lib.op_linear(BF16, epi, at.data_ptr(), wt.data_ptr(), M, N, K, s.cuda_stream, bias=b.data_ptr(),
                      out=t_out.data_ptr(), ldo=N, a_layout=KTILED, out_layout=KTILED)
        s.synchronize()
        got, pad = _untile(t_out, M, 2 * N)
        want = _bytes(ref_out)
        assert np.all(pad == SENT)
    else:
        x0 = torch.from_numpy(rng.standard_normal((M, N), dtype=np.float32)).to("cuda:0")
        gate = torch.from_numpy(rng.standard_normal((2, 6 * N), dtype=np.float32)).to("cuda:0")
        xa, xb = x0.clone(), x0.clone()
        kw = dict(bias=b.data_ptr(), ldx=N, gate=gate.data_ptr() if epi == 2 else 0, gate_ld=6 * N,
                  rows_per_gate=max(1, M // 2))
        lib.op_linear(BF16, epi, a.data_ptr(), wt.data_ptr(), M, N, K, s.cuda_stream, xr=xa.data_ptr(), **kw)
        lib.op_linear(BF16, epi, at.data_ptr(), wt.data_ptr(), M, N, K, s.cuda_stream, xr=xb.data_ptr(),
                      a_layout=KTILED, **kw)
        s.synchronize()
        got, want = xb.cpu().numpy(), xa.cpu().numpy()
    assert np.array_equal(got, want), "k-tiled A must give the row-major result bit for bit"
    # sampled oracle check of the k-tiled call
    ms = np.concatenate([rng.integers(0, M, 60), [0, M - 1]])
    ns = np.concatenate([rng.integers(0, N, 60), [N - 1, 0]])
    A = a[torch.from_numpy(ms).to("cuda:0")].double().cpu().numpy()
    W = w[torch.from_numpy(ns).to("cuda:0")].double().cpu().numpy()
    bias = b.double().cpu().numpy()[ns]
    y = np.einsum("ik,ik->i", A, W) + bias
    mag = np.einsum("ik,ik->i", np.abs(A), np.abs(W)) + np.abs(bias)
    if epi <= 1:
        ref = y if epi == 0 else o_dit.gelu_tanh(y)
        g = _bf16_f64(got.view(np.uint16)[ms, ns])
        tol = 2.0 ** -8 * np.abs(ref) + 1.2e-5 * mag + 1e-6
    else:
        gv = gate.double().cpu().numpy()[ms // max(1, M // 2), ns] if epi == 2 else 1.0
        ref = x0.double().cpu().numpy()[ms, ns] + gv * y
        g = got[ms, ns].astype(np.float64)
        tol = 1e-5 * np.abs(gv) * mag + 1e-6 * np.abs(ref) + 1e-6
    assert np.all(np.abs(g - ref) <= tol), float(np.max(np.abs(g - ref) / tol))


@pytest.mark.parametrize("M,N,K,seg", [(32760, 5120, 13824, 5120), (2048, 3456, 1024, 1152), (300, 1024, 256, 1024)])
def test_linear_fp8_ktiled(lib, M, N, K, seg):
    torch = _torch()
    print(f"[ktiled linear fp8] M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M + 2 * N + K)
    a_codes, a_sc = codecs.quantize_rows_e4m3(rng.standard_normal((M, K), dtype=np.float32))
    w_codes = codecs.e4m3_encode(rng.standard_normal((N, K), dtype=np.float32) * np.float32(60))
    w_sc = (rng.uniform(0.5, 2.0, N // seg) * 1e-3).astype(np.float32)
    b32 = (rng.standard_normal(N, dtype=np.float32) * 0.02).astype(np.float32)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")
    a, at = dev(a_codes), _tile_dev(a_codes)
    w, asc, wsc = dev(lib.tile_weight(FP8, w_codes)), dev(a_sc), dev(w_sc)
    b = torch.from_numpy(b32).to(torch.bfloat16).to("cuda:0")
    o1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    o2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    s = _stream()
    kw = dict(a_scale=asc.data_ptr(), w_scale=wsc.data_ptr(), w_seg=seg, bias=b.data_ptr(), ldo=N)
    lib.op_linear(FP8, 0, a.data_ptr(), w.data_ptr(), M, N, K, s.cuda_stream, out=o1.data_ptr(), **kw)
    lib.op_linear(FP8, 0, at.data_ptr(), w.data_ptr(), M, N, K, s.cuda_stream, out=o2.data_ptr(), a_layout=KTILED,
                  **kw)
    s.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    ms = np.concatenate([rng.integers(0, M, 60), [M - 1]])
    ns = np.concatenate([rng.integers(0, N, 60), [N - 1]])
    A, W = codecs.e4m3_decode(a_codes[ms]), codecs.e4m3_decode(w_codes[ns])
    scale = w_sc[ns // seg].astype(np.float64) * a_sc[ms].astype(np.float64)
    bias = codecs.bf16_round(b32)[ns]
    y = np.einsum("ik,ik->i", A, W) * scale + bias
    mag = np.einsum("ik,ik->i", np.abs(A), np.abs(W)) * scale + np.abs(bias)
    got = o2.double().cpu().numpy()[ms, ns]
    assert np.all(np.abs(got - y) <= 2.0 ** -8 * np.abs(y) + 1e-5 * mag)


# ------------------------------------------------------------------ attention output

@pytest.mark.parametrize("B,H,Tq,Tk,d,fused", [
    (1, 40, 32760, 32760, 128, True),    # video self-attention (eight-wavefront workgroups)
    (1, 40, 32760, 512, 128, False),     # video cross-attention
    (2, 16, 1024, 1024, 72, True),       # DiT-XL
    (1, 2, 300, 130, 128, True),         # ragged queries: a partial band
    (2, 4, 100, 150, 72, False),         # key split over two groups, rows b * Tq + t across a band edge
    (1, 4, 333, 333, 64, True),          # d 64
])
def test_attention_ktiled_output(lib, B, H, Tq, Tk, d, fused):
    torch = _torch()
    print(f"[ktiled attention] B={B} H={H} Tq={Tq} Tk={Tk} d={d}", flush=True)
    rng = np.random.default_rng(B + H + Tq + Tk + d)
    D = H * d
    conv = lambda x: torch.from_numpy(x).to(torch.bfloat16).to("cuda:0")
    if fused:
        qkv = conv(rng.standard_normal((B * Tq, 3 * D), dtype=np.float32))
        q, k, v, ldq, ldkv = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:], 3 * D, 3 * D
    else:
        q = conv(rng.standard_normal((B * Tq, D), dtype=np.float32))
        kv = conv(rng.standard_normal((B * Tk, 2 * D), dtype=np.float32))
        k, v, ldq, ldkv = kv[:, :D], kv[:, D:], D, 2 * D
    o = torch.empty((B * Tq, D), dtype=torch.bfloat16, device="cuda:0")
    ot = _tiled_out(B * Tq, 2 * D)
    s = _stream()
    args = (q.data_ptr(), ldq, k.data_ptr(), ldkv, v.data_ptr(), ldkv)
    lib.op_attention(BF16, *args, o.data_ptr(), D, B, H, Tq, Tk, d, s.cuda_stream)
    lib.op_attention(BF16, *args, ot.data_ptr(), D, B, H, Tq, Tk, d, s.cuda_stream, o_layout=KTILED)
    s.synchronize()
    got, pad = _untile(ot, B * Tq, 2 * D)
    assert np.array_equal(got, _bytes(o)), "k-tiled output must hold the row-major result bit for bit"
    assert np.all(pad == SENT)
    gotf = _bf16_f64(got.view(np.uint16))
    for b in range(B):
        rows = np.unique(np.concatenate([rng.integers(0, Tq, 6), [0, Tq - 1]]))
        Q = q[b * Tq + torch.from_numpy(rows).to("cuda:0")].double().cpu().numpy()
        K = k[b * Tk:(b + 1) * Tk].double().cpu().numpy()
        V = v[b * Tk:(b + 1) * Tk].double().cpu().numpy()
        ref = o_dit.attention_rows(Q, K, V, H)
        mag = o_dit.attention_rows(Q, K, np.abs(V), H)
        assert np.all(np.abs(gotf[b * Tq + rows] - ref) <= 2.0 ** -8 * (mag + np.abs(ref)) + 1e-5)


# ------------------------------------------------------------------ row kernels

@pytest.mark.parametrize("M,D", [(32760, 5120), (2048, 1152), (333, 256),
                                 (203, 2048),    # the widest rows of one wavefront each, a 4-row workgroup short of rows
                                 (131, 2112)])   # the narrowest of two wavefronts per row (five float4 chunks a lane)
def test_layernorm_ktiled(lib, M, D):
    torch = _torch()
    print(f"[ktiled layernorm] M={M} D={D}", flush=True)
    rng = np.random.default_rng(M + 5 * D)
    x = (rng.standard_normal((M, D), dtype=np.float32) * 3 + 1).astype(np.float32)
    B = 2 if M % 2 == 0 else 1
    mod = rng.standard_normal((B, 6, D), dtype=np.float32) * 0.5
    xd, md = torch.from_numpy(x).to("cuda:0"), torch.from_numpy(mod).to("cuda:0")
    s = _stream()
    kw = dict(mod=md.data_ptr(), rows_per_batch=M // B, shift_chunk=0, scale_chunk=1)
    o16 = torch.empty((M, D), dtype=torch.bfloat16, device="cuda:0")
    t16 = _tiled_out(M, 2 * D)
    o8 = torch.empty((M, D), dtype=torch.uint8, device="cuda:0")
    t8 = _tiled_out(M, D)
    sc_a = torch.empty(M, dtype=torch.float32, device="cuda:0")
    sc_b = torch.empty(M, dtype=torch.float32, device="cuda:0")
    lib.op_layernorm(xd.data_ptr(), M, D, o16.data_ptr(), BF16, s.cuda_stream, **kw)
    lib.op_layernorm(xd.data_ptr(), M, D, t16.data_ptr(), BF16, s.cuda_stream, out_layout=KTILED, **kw)
    lib.op_layernorm(xd.data_ptr(), M, D, o8.data_ptr(), FP8, s.cuda_stream, out_scale=sc_a.data_ptr(), **kw)
    lib.op_layernorm(xd.data_ptr(), M, D, t8.data_ptr(), FP8, s.cuda_stream, out_scale=sc_b.data_ptr(),
                     out_layout=KTILED, **kw)
    s.synchronize()
    g16, p16 = _untile(t16, M, 2 * D)
    g8, p8 = _untile(t8, M, D)
    assert np.array_equal(g16, _bytes(o16)) and np.array_equal(g8, o8.cpu().numpy())
    assert np.array_equal(sc_a.cpu().numpy(), sc_b.cpu().numpy())
    assert np.all(p16 == SENT) and np.all(p8 == SENT)
    rows = np.concatenate([rng.integers(0, M, 32), [0, M - 1]])
    bi = rows // (M // B)
    ref = o_dit.layer_norm(x[rows].astype(np.float64)) * (1 + mod[bi, 1].astype(np.float64)) + mod[bi, 0]
    got = _bf16_f64(g16.view(np.uint16)[rows])
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


@pytest.mark.parametrize("M,N", [(32760, 5120), (300, 256)])
def test_quantize_rows_ktiled(lib, M, N):
    torch = _torch()
    rng = np.random.default_rng(M + 3 * N)
    x = rng.standard_normal((M, N), dtype=np.float32) * np.exp(rng.uniform(-3, 3, (M, 1))).astype(np.float32)
    xd = torch.from_numpy(x).to(torch.bfloat16).to("cuda:0")
    codes = _tiled_out(M, N)
    sc = torch.empty(M, dtype=torch.float32, device="cuda:0")
    s = _stream()
    lib.op_quantize_rows(xd.data_ptr(), M, N, codes.data_ptr(), sc.data_ptr(), s.cuda_stream, codes_layout=KTILED)
    s.synchronize()
    got, pad = _untile(codes, M, N)
    ref_codes, ref_sc = codecs.quantize_rows_e4m3(xd.float().cpu().numpy())
    assert np.array_equal(got, ref_codes) and np.array_equal(sc.cpu().numpy(), ref_sc)
    assert np.all(pad == SENT)


def test_ktiled_argument_validation(lib):
    torch = _torch()
    a = torch.zeros(64 * 256, dtype=torch.bfloat16, device="cuda:0")
    f = torch.zeros(64 * 256, dtype=torch.float32, device="cuda:0")
    s = _stream()
    p, st = a.data_ptr(), s.cuda_stream
    bad = [
        lambda: lib.op_linear(F32, 0, f.data_ptr(), f.data_ptr(), 8, 64, 64, st, out=f.data_ptr(), ldo=64,
                              a_layout=KTILED),                                   # fp32 has no k-tiled form
        lambda: lib.op_linear(BF16, 2, p, p, 8, 64, 64, st, xr=f.data_ptr(), ldx=64, gate=f.data_ptr(),
                              gate_ld=64, rows_per_gate=1, out_layout=KTILED),    # residual epilogue, no out
        lambda: lib.op_linear(BF16, 0, p, p, 8, 64, 64, st, out=p, ldo=72, out_layout=KTILED),   # ldo % 32
        lambda: lib.op_linear(BF16, 0, p, p, 8, 64, 64, st, out=p, ldo=64, a_layout=2),          # unknown layout
        lambda: lib.op_attention(F32, f.data_ptr(), 64, f.data_ptr(), 64, f.data_ptr(), 64, f.data_ptr(), 64, 1, 1,
                                 4, 4, 64, st, o_layout=KTILED),
        lambda: lib.op_layernorm(f.data_ptr(), 4, 64, f.data_ptr(), F32, st, out_layout=KTILED),
        lambda: lib.op_layernorm(f.data_ptr(), 4, 48, p, FP8, st, out_scale=f.data_ptr(), out_layout=KTILED),
        lambda: lib.op_quantize_rows(p, 4, 72, p, f.data_ptr(), st, codes_layout=KTILED),
    ]
    for i, call in enumerate(bad):
        with pytest.raises(lib.LwoError):
            print(f"[ktiled validation] case {i}", flush=True)
            call()


@pytest.mark.parametrize("M", [1, 63, 65])
def test_ktiled_band_edges(lib, M):
    """One row, one row short of a band, one row past a band: every k-tiled producer and the
    linear that reads its output give the row-major bits, and no padding byte is written."""
    torch = _torch()
    print(f"[ktiled edges] M={M}", flush=True)
    rng = np.random.default_rng(M)
    D, N = 256, 128
    s = _stream()
    x = torch.from_numpy(rng.standard_normal((M, D), dtype=np.float32)).to("cuda:0")
    rows16 = torch.empty((M, D), dtype=torch.bfloat16, device="cuda:0")
    t16 = _tiled_out(M, 2 * D)
    lib.op_layernorm(x.data_ptr(), M, D, rows16.data_ptr(), BF16, s.cuda_stream)
    lib.op_layernorm(x.data_ptr(), M, D, t16.data_ptr(), BF16, s.cuda_stream, out_layout=KTILED)
    codes = _tiled_out(M, D)
    sc = torch.empty(M, dtype=torch.float32, device="cuda:0")
    lib.op_quantize_rows(rows16.data_ptr(), M, D, codes.data_ptr(), sc.data_ptr(), s.cuda_stream, codes_layout=KTILED)
    w = torch.from_numpy(rng.standard_normal((N, D), dtype=np.float32) * 0.05).to(torch.bfloat16).to("cuda:0")
    wt = torch.from_numpy(lib.tile_weight(BF16, _bytes(w).view(np.uint16))).to("cuda:0")
    y_rows = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    y_t = _tiled_out(M, 2 * N)
    lib.op_linear(BF16, 1, rows16.data_ptr(), wt.data_ptr(), M, N, D, s.cuda_stream, out=y_rows.data_ptr(), ldo=N)
    lib.op_linear(BF16, 1, t16.data_ptr(), wt.data_ptr(), M, N, D, s.cuda_stream, out=y_t.data_ptr(), ldo=N,
                  a_layout=KTILED, out_layout=KTILED)
    s.synchronize()
    g16, p16 = _untile(t16, M, 2 * D)
    g8, p8 = _untile(codes, M, D)
    gy, py = _untile(y_t, M, 2 * N)
    assert np.array_equal(g16, _bytes(rows16)) and np.all(p16 == SENT)
    ref_codes, ref_sc = codecs.quantize_rows_e4m3(rows16.float().cpu().numpy())
    assert np.array_equal(g8, ref_codes) and np.array_equal(sc.cpu().numpy(), ref_sc) and np.all(p8 == SENT)
    assert np.array_equal(gy, _bytes(y_rows)) and np.all(py == SENT)
