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
    b = _bench()
    got = b.committed_traffic("gemm_bf16_gated", "dit_xl_bf16")
    assert isinstance(got, int) and got > 37306368   # at least the algorithmic bytes per launch
    assert b.committed_traffic("gemm_bf16_gated", "no_such_workload") is None
    # a copy of the tree whose kernel source differs by one byte: the record no longer applies
    shutil.copytree(os.path.join(ROOT, "profiles"), tmp_path / "profiles")
    src = "layerwise_weight_offload_amd/csrc"
    os.makedirs(tmp_path / src)
    for f in ("k_gemm.hip", "kcommon.h", "kernels.h"):
        shutil.copy(os.path.join(ROOT, src, f), tmp_path / src / f)
    b.ROOT = str(tmp_path)
    assert b.committed_traffic("gemm_bf16_gated", "dit_xl_bf16") == got
    with open(tmp_path / src / "k_gemm.hip", "a") as fh:
        fh.write("\n")
    assert b.committed_traffic("gemm_bf16_gated", "dit_xl_bf16") is None
