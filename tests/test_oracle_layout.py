"""Pins for the oracle's block layout and packer (CPU only)."""
import numpy as np
import pytest

import lwo_synth
from oracle import codecs, layout


@pytest.mark.parametrize("name", sorted(lwo_synth.WORKLOADS))
def test_layout_invariants(name):
    w = lwo_synth.get(name)
    slots, ext = layout.layout_for(w)
    end = 0
    for s in slots:
        assert s.offset % 256 == 0 and s.offset >= end
        assert s.nbytes == int(np.prod(s.shape)) * layout.ELEM_BYTES[s.dtype]
        end = s.offset + s.nbytes
    assert ext % 4096 == 0 and end <= ext < end + 4096
    inv = lwo_synth.tensor_inventory(w)
    assert [(n, tuple(sh)) for n, sh in inv] == [(s.name, s.shape) for s in slots][:len(inv)]


def _closed_form_bytes(kind, D, F, act, lin):
    """Unpadded payload: (#linear weights) * lin + (#other) * act (+ scales)."""
    e = layout.ELEM_BYTES
    if kind == "dit":
        n_lin = 6 * D * D + 4 * D * D + 2 * D * F
        n_oth = 6 * D + 3 * D + D + F + D
        return n_lin * e[lin] + n_oth * e[act]
    n_lin = 8 * D * D + 2 * D * F
    n_oth = 6 * D + 3 * D + 2 * D + D + D + 2 * D + D + F + D
    return n_lin * e[lin] + n_oth * e[act] + (40 if lin == "fp8" else 0)


@pytest.mark.parametrize("name,expect", [
    ("dit_tiny_fp32", 4_733_952), ("dit_xl_bf16", 47_810_304),
    ("video14b_bf16", 702_747_648), ("video14b_fp8", 351_474_728)])
def test_extent_sizes_closed_form(name, expect):
    w = lwo_synth.get(name)
    slots, ext = layout.layout_for(w)
    payload = sum(s.nbytes for s in slots)
    assert payload == _closed_form_bytes(w.kind, w.hidden, w.ffn, w.act_dtype, w.linear_dtype) == expect
    end = slots[-1].offset + slots[-1].nbytes
    assert ext == (end + 4095) // 4096 * 4096


@pytest.mark.parametrize("name", ["dit_t_fp32", "dit_t_bf16", "video_t_fp8"])
def test_pack_unpack_roundtrip(name):
    w = lwo_synth.get(name)
    t = lwo_synth.block_tensors(w, 1)
    ext = layout.pack_block(w, t)
    slots, n = layout.layout_for(w)
    assert len(ext) == n
    p = layout.unpack_block(w, ext)
    names = [nm for nm, _ in lwo_synth.tensor_inventory(w)]
    for nm, a in zip(names, t):
        got = p[nm]
        a = a.astype(np.float64)
        dt = next(s.dtype for s in slots if s.name == nm)
        if dt == "f32":
            assert np.array_equal(got, a)
        elif dt == "bf16":
            assert np.all(np.abs(got - a) <= np.abs(a) * 2.0 ** -8)
        else:
            sc = float(np.max(np.abs(a)) / 448)
            assert np.all(np.abs(got - a) <= np.maximum(np.abs(a) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6))
    # padding is zero
    b = np.frombuffer(ext, np.uint8)
    covered = np.zeros(n, bool)
    for s in slots:
        covered[s.offset:s.offset + s.nbytes] = True
    assert not b[~covered].any()


def test_fp8_scales_follow_weights_in_order():
    w = lwo_synth.get("video_t_fp8")
    t = lwo_synth.block_tensors(w, 0)
    ext = layout.pack_block(w, t)
    slots, _ = layout.layout_for(w)
    sc_slot = slots[-1]
    assert sc_slot.name == "linear.scales" and sc_slot.offset > max(s.offset for s in slots[:-1])
    sc = np.frombuffer(ext[sc_slot.offset:sc_slot.offset + 40], np.float32)
    names = [nm for nm, _ in lwo_synth.tensor_inventory(w)]
    wl = [a for nm, a in zip(names, t) if nm.endswith(".w")]
    assert len(wl) == 10
    for i, a in enumerate(wl):
        assert sc[i] == np.float32(np.max(np.abs(a)) / np.float32(448))
