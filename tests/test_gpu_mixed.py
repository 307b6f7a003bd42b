"""Mixed block stacks: several block types with different extent sizes
streamed through one ring (slots sized to the largest).  Parity against the
oracle's per-block-type stack; the tolerances are those of the uniform
stacks (fp32 1e-4; bf16 2e-2 on the output, 3e-2 on the update; fp8 5e-2
against the plain oracle and 4e-2 against the one that also quantises the
fp8 blocks' activations)."""
import numpy as np
import pytest

import lwo_synth
from oracle import checksum as o_ck
from oracle import dit as o_dit
from oracle import layout as o_layout

from .conftest import gpu_available
from .gpu_util import device_inputs, run_steps, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _oracle_ext(m):
    return [o_layout.pack_block(m.type_of(b), lwo_synth.block_tensors(m.type_of(b), b)) for b in range(m.n_blocks)]


def _store(lib, m, k=0, host_mode=None, pageable=False):
    types = [lib.ModelDesc.from_workload(t) for t in m.types]
    if pageable:
        exts = []
        for b in range(m.n_blocks):
            d = lib.ModelDesc.from_workload(m.type_of(b))
            _, n = lib.block_layout(d)
            buf = np.empty(n, np.uint8)
            lib.pack_block(d, lwo_synth.block_tensors(m.type_of(b), b), dst=buf.ctypes.data, dst_bytes=n)
            exts.append(buf)
        st = lib.build_mixed_store(types, m.block_type, extents=exts,
                                   host_mode=lib.HOST_STAGED if host_mode is None else host_mode)
    else:
        def fill(b, dst, n):
            wb = m.type_of(b)
            lib.pack_block(lib.ModelDesc.from_workload(wb), lwo_synth.block_tensors(wb, b), dst=dst, dst_bytes=n)
        st = lib.build_mixed_store(types, m.block_type, fill=fill)
    if k:
        st.set_resident_prefix(k)
    return st


def _bits(m, x):
    import torch
    return x.cpu().view(-1).view(torch.int16 if m.inputs.act_dtype == "bf16" else torch.int32).numpy().copy()


@pytest.mark.parametrize("name,tol_out,tol_upd", [("dit_mixed_fp32", 1e-4, 1e-4), ("dit_mixed_bf16", 2e-2, 3e-2)])
def test_mixed_parity(lib, name, tol_out, tol_upd):
    m = lwo_synth.get_mixed(name)
    print(f"[mixed] {name}", flush=True)
    x0, cond, ctx = o_dit.decode_inputs(m.inputs, *lwo_synth.step_inputs(m.inputs))
    want = o_dit.stack_forward_mixed(m, _oracle_ext(m), x0, cond, ctx)
    with _store(lib, m) as st:
        x, c, cx = device_inputs(m.inputs)
        run_steps(st, x, c, cx)
        got = to_f64(x).reshape(want.shape)
        s = st.stats()
        sizes = [lib.block_layout(lib.ModelDesc.from_workload(t))[1] for t in m.types]
        assert s.extent_bytes == s.slot_bytes == max(sizes) and s.device_weight_bytes == 2 * max(sizes)
    e_out, e_upd = o_dit.rel_l2(got, want), o_dit.rel_l2(got - x0, want - x0)
    print(f"[mixed] {name}: rel_l2(out)={e_out:.3e} rel_l2(update)={e_upd:.3e}", flush=True)
    assert e_out <= tol_out and e_upd <= tol_upd


def test_mixed_fp8_and_bf16_blocks(lib):
    m = lwo_synth.get_mixed("video_mixed_fp8")
    x0, cond, ctx = o_dit.decode_inputs(m.inputs, *lwo_synth.step_inputs(m.inputs))
    ext = _oracle_ext(m)
    plain = o_dit.stack_forward_mixed(m, ext, x0, cond, ctx)
    emul = o_dit.stack_forward_mixed(m, ext, x0, cond, ctx, fp8_act=True)
    with _store(lib, m) as st:
        x, c, cx = device_inputs(m.inputs)
        run_steps(st, x, c, cx)
        got = to_f64(x).reshape(plain.shape)
    e_plain = o_dit.rel_l2(got, plain)
    e_emul = o_dit.rel_l2(got - x0, emul - x0)
    e_plain_upd = o_dit.rel_l2(got - x0, plain - x0)
    print(f"[mixed] fp8+bf16: out vs plain {e_plain:.3e}, update vs plain {e_plain_upd:.3e}, vs emulated {e_emul:.3e}",
          flush=True)
    assert e_plain <= 5e-2 and e_emul <= 4e-2 and e_emul < e_plain_upd


def test_mixed_streamed_equals_resident_and_checksums(lib):
    m = lwo_synth.get_mixed("dit_mixed_bf16")
    outs = {}
    for k in (0, 2, 5):
        with _store(lib, m, k=k) as st:
            x, c, cx = device_inputs(m.inputs)
            run_steps(st, x, c, cx, steps=3)
            outs[k] = _bits(m, x)
            if k == 2:
                ext = _oracle_ext(m)
                for b in range(m.n_blocks):
                    hs, ss = st.block_checksum(b)
                    assert hs == ss == o_ck.extent_checksum(ext[b])
                s = st.stats()
                assert s.device_weight_bytes == 2 * s.extent_bytes + len(ext[0]) + len(ext[1])
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[0], outs[5])


def test_mixed_staged_equals_pin_copy(lib):
    m = lwo_synth.get_mixed("video_mixed_fp8")
    res = []
    for pageable in (False, True):
        with _store(lib, m, pageable=pageable) as st:
            st.set_validation(True)
            x, c, cx = device_inputs(m.inputs)
            run_steps(st, x, c, cx, steps=2)
            res.append(_bits(m, x))
            assert st.stats().checksum_mismatches == 0
    assert np.array_equal(res[0], res[1])
