"""The C-ABI library on the host (no GPU): exported symbols, block layout,
packing and checksum bit-exact against the oracle, descriptor validation and
the all-or-nothing registration lifecycle."""
import os
import re
import subprocess

import numpy as np
import pytest

import lwo_synth
from oracle import checksum as o_checksum
from oracle import layout as o_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lwo.h")

DT = {"f32": 0, "bf16": 1, "fp8": 2}


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lwo_[a-z0-9_]+)\s*\(", src)) - {"lwo_register_fn", "lwo_unregister_fn"})


def test_library_exports_every_declared_symbol(lib):
    declared = _declared()
    assert "lwo_run_denoise_step" in declared and "lwo_build_block_store" in declared
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lwo_\w+)", out))
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    assert sorted(lib.exported_symbols()) == declared


@pytest.mark.parametrize("name", sorted(lwo_synth.WORKLOADS))
def test_layout_matches_oracle(lib, name):
    w = lwo_synth.get(name)
    got, ext = lib.block_layout(lib.ModelDesc.from_workload(w))
    want, want_ext = o_layout.layout_for(w)
    assert ext == want_ext
    assert [(t["name"], t["offset"], t["bytes"], t["shape"], t["dtype"], t["tiled"]) for t in got] == \
           [(s.name, s.offset, s.nbytes, tuple(s.shape), DT[s.dtype], o_layout.tiled(s.name, s.dtype)) for s in want]


@pytest.mark.parametrize("dtype,N,K", [(1, 64, 32), (1, 192, 1152), (2, 128, 64), (2, 64, 448)])
def test_tile_weight_matches_oracle(lib, dtype, N, K):
    rng = np.random.default_rng(N + K)
    w = rng.integers(0, 1 << 16, (N, K), dtype=np.uint16) if dtype == 1 else rng.integers(0, 256, (N, K), dtype=np.uint8)
    got = lib.tile_weight(dtype, w)
    want = o_layout.tile_bytes(w.view(np.uint8).reshape(N, -1))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype,N,K", [(0, 64, 64), (1, 100, 64), (1, 64, 16), (2, 64, 32), (1, 0, 64)])
def test_tile_weight_rejects(lib, dtype, N, K):
    w = np.zeros((max(N, 1), K), dtype=np.uint16 if dtype != 2 else np.uint8)
    with pytest.raises(lib.LwoError) as e:
        if N == 0:
            lib._binding._check(lib._binding._lib_tile_weight(dtype, w.ctypes.data, 0, K, w.ctypes.data))
        else:
            lib.tile_weight(dtype, w)
    assert e.value.name == "LWO_EINVAL"


def _edge_tensors(w, b):
    """Generator draws with a few planted rounding edge cases."""
    t = lwo_synth.block_tensors(w, b)
    edges = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0, 1e-30, -1e-30, 3e38, 2 ** -130,
                      0.5 + 2 ** -10, 7.0, 15.5], dtype=np.float32)
    for a in t:
        n = min(a.size, edges.size)
        a.reshape(-1)[:n] = edges[:n] * (0.02 if a.size > 4096 else 1.0)
    return t


@pytest.mark.parametrize("name", ["dit_t_fp32", "dit_t_bf16", "video_t_fp32", "video_t_bf16", "video_t_fp8",
                                  "dit_tiny_fp32"])
def test_pack_bit_exact_vs_oracle(lib, name):
    w = lwo_synth.get(name)
    desc = lib.ModelDesc.from_workload(w)
    for b in range(2):
        t = lwo_synth.block_tensors(w, b) if b == 0 else _edge_tensors(w, b)
        got = lib.pack_block(desc, t)
        want = np.frombuffer(o_layout.pack_block(w, t), np.uint8)
        assert got.size == want.size
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (name, b, bad[:10])


def test_fp8_pack_ties_and_saturation(lib):
    """Values exactly between two e4m3 codes, scaled so that w / s lands on them."""
    w = lwo_synth.get("video_t_fp8")
    desc = lib.ModelDesc.from_workload(w)
    t = lwo_synth.block_tensors(w, 0)
    q = t[1]   # attn.q.w: force amax = 448 so s = 1 and codes are the values themselves
    from oracle import codecs
    pos = codecs.E4M3_VALUES[:127]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([[448.0], mids, -mids, pos, -pos]).astype(np.float32)
    q.reshape(-1)[:vals.size] = vals
    q.reshape(-1)[vals.size:] = 0.0
    got = lib.pack_block(desc, t)
    want = np.frombuffer(o_layout.pack_block(w, t), np.uint8)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("nbytes", [0, 8, 4096, 1 << 20])
def test_checksum_matches_oracle(lib, nbytes):
    buf = np.random.default_rng(nbytes).integers(0, 256, nbytes, dtype=np.uint8).tobytes()
    assert lib.extent_checksum(buf) == o_checksum.extent_checksum(buf)


def test_checksum_of_packed_extent(lib):
    w = lwo_synth.get("dit_t_bf16")
    ext = lib.pack_block(lib.ModelDesc.from_workload(w), lwo_synth.block_tensors(w, 0))
    assert lib.extent_checksum(ext) == o_checksum.extent_checksum(ext.tobytes())


@pytest.mark.parametrize("field,value", [("heads", 3), ("hidden", 200), ("n_blocks", 0), ("tokens", 0),
                                         ("act_dtype", 2), ("ctx_tokens", 5), ("linear_dtype", 2), ("ffn", 100)])
def test_descriptor_validation(lib, field, value):
    import dataclasses
    w = lwo_synth.get("dit_t_bf16")
    d = dataclasses.replace(lib.ModelDesc.from_workload(w), **{field: value})
    with pytest.raises(lib.LwoError) as e:
        lib.block_layout(d)
    assert e.value.name == "LWO_EINVAL" and "invalid model desc" in str(e.value)


def test_pack_rejects_bad_arguments(lib):
    w = lwo_synth.get("dit_t_fp32")
    desc = lib.ModelDesc.from_workload(w)
    t = lwo_synth.block_tensors(w, 0)
    with pytest.raises(lib.LwoError):
        lib.pack_block(desc, t[:-1])
    with pytest.raises(lib.LwoError):
        lib.pack_block(desc, t, dst=bytearray(16))


def test_build_fails_closed_without_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    w = lwo_synth.get("dit_tiny_fp32")
    desc = lib.ModelDesc.from_workload(w)
    calls = []
    with pytest.raises(lib.LwoError) as e:
        lib.build_block_store(desc, fill=lambda b, dst, n: calls.append(b))
    assert e.value.name == "LWO_EINVAL" and "not available" in str(e.value)
    assert calls == []


# ------------------------------------------------------------------ registration lifecycle

class FakePlatform:
    def __init__(self, fail_at=None, unreg_fail=()):
        self.fail_at = fail_at
        self.unreg_fail = set(unreg_fail)
        self.log = []
        self.live = {}

    def reg(self, base, ln):
        i = len([x for x in self.log if x[0] == "reg"])
        self.log.append(("reg", base, ln))
        if self.fail_at is not None and i == self.fail_at:
            return 1
        self.live[base] = ln
        return 0

    def unreg(self, base):
        self.log.append(("unreg", base))
        if base in self.unreg_fail:
            return 1
        self.live.pop(base)
        return 0


P = 4096


def test_register_aligns_and_coalesces(lib):
    f = FakePlatform()
    ptrs = [10 * P + 100, 10 * P + 3000, 12 * P, 20 * P + 5, 13 * P - 1]
    sizes = [50, 2000, 10, P, 2]
    got = lib.register_ranges(ptrs, sizes, P, 1 << 40, f.reg, f.unreg)
    # [10P, 11P) + [10P, 12P) + [12P, 13P) + [12P, 14P) (13P-1 .. 13P+1 touches two pages) merge to
    # [10P, 14P); [20P+5, 21P+5) becomes [20P, 22P) and stays apart
    assert got == [(10 * P, 4 * P), (20 * P, 2 * P)]
    assert [x for x in f.log if x[0] == "reg"] == [("reg", 10 * P, 4 * P), ("reg", 20 * P, 2 * P)]


def test_register_budget_checked_before_any_call(lib):
    f = FakePlatform()
    with pytest.raises(lib.LwoError) as e:
        lib.register_ranges([0, 4 * P], [P, P], P, 2 * P - 1, f.reg, f.unreg)
    assert e.value.name == "LWO_EBUDGET"
    assert f.log == []
    assert lib.register_ranges([0, 4 * P], [P, P], P, 2 * P, f.reg, f.unreg) == [(0, P), (4 * P, P)]


@pytest.mark.parametrize("fail_at", [0, 1, 3])
def test_register_failure_rolls_back_in_reverse(lib, fail_at):
    f = FakePlatform(fail_at=fail_at)
    ptrs = [i * 4 * P for i in range(5)]
    with pytest.raises(lib.LwoError) as e:
        lib.register_ranges(ptrs, [P] * 5, P, 1 << 40, f.reg, f.unreg)
    assert e.value.name == "LWO_EREGISTER"
    assert f.live == {}
    unregs = [x[1] for x in f.log if x[0] == "unreg"]
    assert unregs == [ptrs[j] for j in range(fail_at - 1, -1, -1)]


def test_register_rollback_failure_is_reported(lib):
    ptrs = [i * 4 * P for i in range(4)]
    f = FakePlatform(fail_at=3, unreg_fail={ptrs[1]})
    with pytest.raises(lib.LwoError) as e:
        lib.register_ranges(ptrs, [P] * 4, P, 1 << 40, f.reg, f.unreg)
    assert e.value.name == "LWO_EROLLBACK"
    assert set(f.live) == {ptrs[1]}      # the range that could not be unregistered stays registered
    assert [x[1] for x in f.log if x[0] == "unreg"] == [ptrs[2], ptrs[1], ptrs[0]]


def test_struct_layouts_match_header(lib, tmp_path):
    """The binding's ctypes mirrors have the C header's sizes and field offsets
    (compiled with the host C compiler against include/lwo.h)."""
    import ctypes as C
    from layerwise_weight_offload_amd import _binding as B
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    structs = {"lwo_model_desc": B._Desc, "lwo_tensor_info": B._TensorInfo, "lwo_block_source": B._Source,
               "lwo_stats": B._Stats, "lwo_kernel_stat": B._KStat}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "lwo.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f in py._fields_:
            lines.append(f'  printf("{cname} {f[0]} %zu\\n", offsetof({cname}, {f[0]}));')
    lines.append("  return 0; }")
    src = tmp_path / "sizes.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "sizes"
    subprocess.run(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {(ln.split()[0], ln.split()[1]): int(ln.split()[2]) for ln in out if ln.strip()}
    for cname, py in structs.items():
        assert got[(cname, "size")] == C.sizeof(py), cname
        for f in py._fields_:
            assert got[(cname, f[0])] == getattr(py, f[0]).offset, (cname, f[0])


def test_mixed_build_validation_before_device(lib):
    """Mixed stacks: inconsistent types or bad indices fail with LWO_EINVAL before
    any device call (so the checks run on a host without a GPU); a consistent
    stack gets as far as the device check."""
    m = lwo_synth.get_mixed("dit_mixed_bf16")
    a, b = (lib.ModelDesc.from_workload(t) for t in m.types)
    src = [np.zeros(8, np.uint8)] * 5
    import dataclasses
    for types, bt in [([a, dataclasses.replace(b, hidden=512)], [0, 1]),      # hidden differs
                      ([a, dataclasses.replace(b, tokens=100)], [0, 1]),      # tokens differ
                      ([a, dataclasses.replace(b, kind=1, ctx_tokens=8)], [0, 1]),
                      ([a, b], [0, 2]),                                       # type index out of range
                      ([a, b], []),                                           # no blocks
                      ([a, dataclasses.replace(b, heads=7)], [0, 1])]:        # invalid head dim
        with pytest.raises(lib.LwoError) as e:
            lib.build_mixed_store(types, bt, extents=src[:max(len(bt), 1)])
        assert e.value.status == 1, (types, bt, str(e.value))
    if not os.path.exists("/dev/kfd"):
        with pytest.raises(lib.LwoError) as e:
            lib.build_mixed_store([a, b], list(m.block_type), extents=src)
        assert "device" in str(e.value)


def test_build_rejects_scratch_in_asm_read_kernels():
    """The kernels that await inline-asm LDS reads by hand must not spill; the
    build parses hipcc's resource-usage remarks and names any that do."""
    import importlib.util
    path = os.path.join(ROOT, "layerwise_weight_offload_amd", "build.py")
    spec = importlib.util.spec_from_file_location("lwo_build_under_test", path)
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    pre = "/x/k.hip:13:1: remark: "
    tail = " [-Rpass-analysis=kernel-resource-usage]"
    text = "\n".join([
        pre + "Function Name: _ZN3lwo11k_gemm_deepILi256ELi256ELi64ELb0ELi0ELi4EEEvNS_8GemmArgsE" + tail,
        pre + "    ScratchSize [bytes/lane]: 0" + tail,
        pre + "Function Name: _ZN3lwo9k_attn_trILi128ELi8ELi1EEEvNS_8AttnArgsE" + tail,
        pre + "    ScratchSize [bytes/lane]: 16" + tail,
        pre + "Function Name: _ZN3lwo10k_attn_f32ILi128EEEvNS_8AttnArgsE" + tail,   # plain loads: allowed
        pre + "    ScratchSize [bytes/lane]: 36" + tail,
    ])
    bad = b._scratch_users(text)
    assert len(bad) == 1 and "k_attn_tr" in bad[0] and "16 bytes" in bad[0]


def test_shard_build_validation_before_device(lib):
    """Shard stores: a group outside [1, 64] or a rank outside [0, group) fails
    with LWO_EINVAL before any device call; valid arguments get as far as the
    device check."""
    w = lwo_synth.get("dit_tiny_fp32")
    desc = lib.ModelDesc.from_workload(w)
    src = [np.zeros(8, np.uint8)] * w.n_blocks
    for g, r in [(0, 0), (65, 0), (2, 2), (3, -1)]:
        with pytest.raises(lib.LwoError) as e:
            lib.build_shard_store(desc, g, r, extents=src)
        assert e.value.status == 1 and "shard" in str(e.value), (g, r, str(e.value))
    if not os.path.exists("/dev/kfd"):
        with pytest.raises(lib.LwoError) as e:
            lib.build_shard_store(desc, 4, 3, extents=src)
        assert "device" in str(e.value)


def test_op_layout_arguments_rejected_before_any_device_call(lib):
    """The single-kernel entry points check their row-layout arguments (LWO_ROWS / LWO_KTILED) before
    touching a device: every call below fails validation with LWO_EINVAL and a message, on a host with no
    GPU.  The pointers are 16-byte aligned stand-ins that are never dereferenced."""
    P, S = 0x100000, 0x200000   # stand-in device pointer and stream handle
    F32, BF16, FP8, KT = 0, 1, 2, 1
    bad = [
        ("linear: k-tiled operands need BF16 or FP8",
         lambda: lib.op_linear(F32, 0, P, P, 64, 64, 64, S, out=P, ldo=64, a_layout=KT)),
        ("linear: a k-tiled out needs epilogue 0 or 1",
         lambda: lib.op_linear(BF16, 2, P, P, 64, 64, 64, S, xr=P, ldx=64, gate=P, gate_ld=64, rows_per_gate=1,
                               out_layout=KT)),
        ("linear: a k-tiled out needs", lambda: lib.op_linear(BF16, 0, P, P, 64, 64, 64, S, out=P, ldo=72,
                                                              out_layout=KT)),
        ("linear: a_layout and out_layout", lambda: lib.op_linear(BF16, 0, P, P, 64, 64, 64, S, out=P, ldo=64,
                                                                  a_layout=2)),
        ("attention: a k-tiled o needs BF16",
         lambda: lib.op_attention(F32, P, 64, P, 64, P, 64, P, 64, 1, 1, 4, 4, 64, S, o_layout=KT)),
        ("attention: o_layout", lambda: lib.op_attention(BF16, P, 64, P, 64, P, 64, P, 64, 1, 1, 4, 4, 64, S,
                                                         o_layout=-1)),
        ("layernorm: a k-tiled out needs", lambda: lib.op_layernorm(P, 4, 64, P, F32, S, out_layout=KT)),
        ("layernorm: a k-tiled out needs", lambda: lib.op_layernorm(P, 4, 48, P, FP8, S, out_scale=P,
                                                                    out_layout=KT)),
        ("quantize_rows: k-tiled codes need N a multiple of 64",
         lambda: lib.op_quantize_rows(P, 4, 72, P, P, S, codes_layout=KT)),
    ]
    for msg, call in bad:
        with pytest.raises(lib.LwoError) as e:
            call()
        assert e.value.status == 1 and msg in str(e.value), (msg, str(e.value))
