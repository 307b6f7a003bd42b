"""STAGED host mode ("Distributed Layerwise Offload", "Host backing and
transfer composition"): pageable caller extents are packed into one of two
pinned staging slots, then copied to the device slot.  The bytes that reach
the slots are the same as in PIN_COPY, so every output must be bit-identical;
the oracle bounds are those of the other parity tests."""
import numpy as np
import pytest

import lwo_synth
from oracle import checksum as o_ck
from oracle import dit as o_dit
from oracle import layout as o_layout

from .conftest import gpu_available
from .gpu_util import device_inputs, oracle_out, run_steps, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _pageable_extents(lib, w):
    desc = lib.ModelDesc.from_workload(w)
    _, ext = lib.block_layout(desc)
    out = []
    for b in range(w.n_blocks):
        buf = np.empty(ext, np.uint8)   # ordinary (pageable) host memory
        lib.pack_block(desc, lwo_synth.block_tensors(w, b), dst=buf.ctypes.data, dst_bytes=ext)
        out.append(buf)
    return desc, out


def _bits(w, x):
    import torch
    return x.cpu().view(-1).view(torch.int16 if w.act_dtype == "bf16" else torch.int32).numpy().copy()


@pytest.mark.parametrize("name,steps", [("dit_t_fp32", 3), ("video_t_bf16", 3)])
def test_staged_equals_pin_copy(lib, name, steps):
    w = lwo_synth.get(name)
    print(f"[staged] {name}", flush=True)
    desc, exts = _pageable_extents(lib, w)
    outs = {}
    for mode in (lib.HOST_PIN_COPY, lib.HOST_STAGED):
        with lib.build_block_store(desc, extents=exts, host_mode=mode) as st:
            x, c, cx = device_inputs(w)
            run_steps(st, x, c, cx, steps=steps)
            outs[mode] = _bits(w, x)
            s = st.stats()
            assert s.host_mode == mode
            if mode == lib.HOST_STAGED:
                assert s.staging_bytes == 2 * s.extent_bytes and s.host_bytes == 0
                assert s.pack_bytes == s.h2d_bytes and s.pack_threads >= 1
                assert s.h2d_copies == 1 + steps * w.n_blocks   # prime + one per streamed block per step
    assert np.array_equal(outs[lib.HOST_PIN_COPY], outs[lib.HOST_STAGED])


def test_staged_parity_vs_oracle(lib):
    w = lwo_synth.get("video_t_fp32")
    desc, exts = _pageable_extents(lib, w)
    x0, want = oracle_out(w, steps=2)
    with lib.build_block_store(desc, extents=exts, host_mode=lib.HOST_STAGED) as st:
        x, c, cx = device_inputs(w)
        run_steps(st, x, c, cx, steps=2)
        got = to_f64(x).reshape(want.shape)
    e = o_dit.rel_l2(got, want)
    print(f"[staged] video_t_fp32 two steps: rel_l2 {e:.3e}", flush=True)
    assert e <= 1e-4 and o_dit.rel_l2(got - x0, want - x0) <= 1e-4


def test_staged_resident_prefix_checksums_and_validation(lib):
    w = lwo_synth.get("dit_t_bf16")   # 3 blocks
    desc, exts = _pageable_extents(lib, w)
    with lib.build_block_store(desc, extents=exts, host_mode=lib.HOST_STAGED) as st:
        st.set_resident_prefix(1)
        for b in range(w.n_blocks):
            hs, ss = st.block_checksum(b)
            assert hs == ss == o_ck.extent_checksum(o_layout.pack_block(w, lwo_synth.block_tensors(w, b)))
        st.set_validation(True)
        x, c, cx = device_inputs(w)
        run_steps(st, x, c, cx, steps=2)
        s = st.stats()
        assert s.validation == 1 and s.checksum_mismatches == 0 and s.resident_prefix == 1
    with lib.build_block_store(desc, extents=exts, host_mode=lib.HOST_PIN_COPY) as ref:
        ref.set_resident_prefix(1)
        xr, c, cx = device_inputs(w)
        run_steps(ref, xr, c, cx, steps=2)
    assert np.array_equal(_bits(w, x), _bits(w, xr))


def test_register_with_zero_budget_continues_staged(lib):
    """A zero registration budget never registers anything and keeps the staging path."""
    w = lwo_synth.get("dit_tiny_fp32")
    desc, exts = _pageable_extents(lib, w)
    with lib.build_block_store(desc, extents=exts, host_mode=lib.HOST_REGISTER, register_budget=0) as st:
        s = st.stats()
        assert s.host_mode == lib.HOST_STAGED and s.registered_ranges == 0 and s.staging_bytes == 2 * s.extent_bytes
        x, c, cx = device_inputs(w)
        run_steps(st, x, c, cx, steps=1)
    with lib.build_block_store(desc, extents=exts, host_mode=lib.HOST_PIN_COPY) as ref:
        xr, c, cx = device_inputs(w)
        run_steps(ref, xr, c, cx, steps=1)
    assert np.array_equal(_bits(w, x), _bits(w, xr))


def test_staged_needs_extents(lib):
    w = lwo_synth.get("dit_tiny_fp32")
    desc = lib.ModelDesc.from_workload(w)
    with pytest.raises(lib.LwoError):
        lib.build_block_store(desc, fill=lambda b, d, n: None, host_mode=lib.HOST_STAGED)


def test_cache_backed_staged_store(lib, tmp_path):
    """Publish the stack as a flat-block file, map it back (verified) and stream
    from the mapping through the staging slots: same bits as PIN_COPY."""
    w = lwo_synth.get("video_t_bf16")
    desc, exts = _pageable_extents(lib, w)
    key, created = lib.cache_publish(str(tmp_path), desc, extents=exts)
    assert created
    del exts
    with lib.cache_open(str(tmp_path), key, desc, verify=True) as entry:
        with lib.build_block_store(desc, extents=entry.extents(), host_mode=lib.HOST_STAGED) as st:
            x, c, cx = device_inputs(w)
            run_steps(st, x, c, cx, steps=2)
            with pytest.raises(lib.LwoError):   # the store still reads the mapping
                entry.close()
            for b in range(w.n_blocks):
                hs, ss = st.block_checksum(b)
                assert hs == ss == o_ck.extent_checksum(o_layout.pack_block(w, lwo_synth.block_tensors(w, b)))
    desc2, exts2 = _pageable_extents(lib, w)
    with lib.build_block_store(desc2, extents=exts2, host_mode=lib.HOST_PIN_COPY) as ref:
        xr, c, cx = device_inputs(w)
        run_steps(ref, xr, c, cx, steps=2)
    assert np.array_equal(_bits(w, x), _bits(w, xr))
