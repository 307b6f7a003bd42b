"""bench.py's host logic (no GPU): the one-GPU guard, the algorithmic FLOP
count it divides by, and the committed HBM-traffic record it reports only
while the kernel sources are the ones the counters were taken on."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

import lwo_synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def _linear(M, N, K):
    return 2.0 * M * N * K


@pytest.mark.parametrize("name", ["dit_xl_bf16", "dit_tiny_fp32", "video14b_bf16", "video14b_t256"])
def test_block_flops_is_the_sum_over_the_block_products(name):
    """Every product of the block written out one by one: adaLN GEMV (DiT), QKV,
    attention QK^T and PV, out-projection, cross q / K|V / attention / output
    (video), FFN up and down."""
    w = lwo_synth.get(name)
    B, T, D, F, Tc = w.batch, w.tokens, w.hidden, w.ffn, w.ctx_tokens
    M = B * T
    f = _linear(M, 3 * D, D) + 2 * (2.0 * B * T * T * D) + _linear(M, D, D) + _linear(M, F, D) + _linear(M, D, F)
    if w.kind == "dit":
        f += _linear(B, 6 * D, D)
    else:
        f += _linear(M, D, D) + _linear(B * Tc, 2 * D, D) + 2 * (2.0 * B * T * Tc * D) + _linear(M, D, D)
    assert _bench().block_flops(w) == pytest.approx(f, rel=1e-12)


def test_block_flops_at_the_stated_sizes():
    # DiT-XL-shaped: 65.26 GF of linears + 9.66 GF of attention; 14B-class video: 41,957 GF
    b = _bench()
    assert b.block_flops(lwo_synth.get("dit_xl_bf16")) / 1e9 == pytest.approx(74.93, abs=0.01)
    assert b.block_flops(lwo_synth.get("video14b_bf16")) / 1e9 == pytest.approx(41957, abs=1)


def test_published_peaks():
    b = _bench()
    assert b.MFMA_PEAK_TFLOPS == {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3} and b.HBM_PEAK_GBPS == 8000.0


def test_traffic_record_follows_the_kernel_sources(tmp_path):
    """A record applies while the sources it names hash to its sources_sha256
    and stops applying (None) once one byte of them changes; other labels or
    workloads find nothing.  Checked on a record written here, so the test does
    not depend on whether the committed record is current."""
    import hashlib
    import json
    b = _bench()
    src = "layerwise_weight_offload_amd/csrc"
    os.makedirs(tmp_path / src)
    names = [f"{src}/{f}" for f in ("k_gemm.hip", "kcommon.h", "kernels.h")]
    h = hashlib.sha256()
    for n in names:
        shutil.copy(os.path.join(ROOT, n), tmp_path / n)
        h.update(open(tmp_path / n, "rb").read())
    rec = {"label": "gemm_bf16_gated", "workload": "dit_xl_bf16", "sources": names, "sources_sha256": h.hexdigest(),
           "hbm_bytes_per_launch": 123456789}
    os.makedirs(tmp_path / "profiles")
    (tmp_path / "profiles" / "note.md").write_text("# note\n\n```json\n" + json.dumps(rec) + "\n```\n")
    b.ROOT = str(tmp_path)
    assert b.committed_traffic("gemm_bf16_gated", "dit_xl_bf16") == 123456789
    assert b.committed_traffic("gemm_bf16_gated", "no_such_workload") is None
    assert b.committed_traffic("gemm_bf16_gelu", "dit_xl_bf16") is None
    with open(tmp_path / names[1], "a") as fh:   # one byte more in a header the kernel includes
        fh.write("\n")
    assert b.committed_traffic("gemm_bf16_gated", "dit_xl_bf16") is None


def test_committed_traffic_record_is_well_formed():
    """The committed record parses, names existing sources and is at least the
    algorithmic traffic when current (None means the kernel changed since)."""
    b = _bench()
    got = b.committed_traffic("attn_self_bf16_d128", "video14b_bf16")
    assert got is None or (isinstance(got, int) and got > 0)


def test_cpu_baseline_runs_each_block_with_its_own_type():
    """The mixed-stack baseline decodes and runs block b with its own type: on
    a small fp32 stack it matches the oracle's mixed stack over all blocks."""
    import numpy as np
    from oracle import dit as o_dit
    from oracle import layout as o_layout
    b = _bench()
    m = lwo_synth.get_mixed("dit_mixed_fp32")
    r = b.cpu_baseline(m.inputs, 1e9, type_of=m.type_of)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["sample"].startswith(f"{m.n_blocks} of {m.n_blocks} blocks")
    # the same per-block decode, checked against the oracle's mixed stack
    x, cond, ctx = o_dit.decode_inputs(m.inputs, *lwo_synth.step_inputs(m.inputs))
    ext = [o_layout.pack_block(m.type_of(i), lwo_synth.block_tensors(m.type_of(i), i)) for i in range(m.n_blocks)]
    y = x
    for i in range(m.n_blocks):
        y = o_dit.stack_forward(m.type_of(i), [ext[i]], y, cond, ctx, blocks=[0])
    assert np.array_equal(y, o_dit.stack_forward_mixed(m, ext, x, cond, ctx))


def test_cpu_baseline_row_extrapolation_branch():
    """Blocks above the FLOP limit are timed at two query-row counts and
    extrapolated to every row; the float64 extra is reported beside it."""
    b = _bench()
    w = lwo_synth.get("video_t_bf16")
    r = b.cpu_baseline(w, 1e9, max_block_flops=0.0)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["float64_value"] > 0
    assert "query rows" in r["sample"] and f"x {w.n_blocks} blocks" in r["sample"]
