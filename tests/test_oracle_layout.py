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


def test_tile_bytes_hand_positions():
    """A 128 x 128-byte matrix makes 2 x 2 tiles of 4096 bytes: tile (band 0,
    bytes 0-63) first, then (band 0, bytes 64-127), then band 1 likewise; in
    a tile, row after row of 64 bytes.  Offsets below are worked by hand."""
    rows = (np.arange(128 * 128, dtype=np.int64).reshape(128, 128) * 7919 % 251).astype(np.uint8)
    flat = layout.tile_bytes(rows)
    assert flat.size == 128 * 128
    assert np.array_equal(flat[0:64], rows[0, 0:64])
    assert np.array_equal(flat[64:128], rows[1, 0:64])
    assert np.array_equal(flat[4032:4096], rows[63, 0:64])
    assert np.array_equal(flat[4096:4160], rows[0, 64:128])
    assert np.array_equal(flat[4096 + 5 * 64:4096 + 6 * 64], rows[5, 64:128])
    assert np.array_equal(flat[8192:8256], rows[64, 0:64])
    assert np.array_equal(flat[12288 + 63 * 64:16384], rows[127, 64:128])
    assert np.array_equal(layout.untile_bytes(flat, 128, 128), rows)


def test_tile_bytes_is_a_permutation_and_keeps_bands():
    """Every tile row is 64 consecutive source bytes; a 64-row band's tiles
    hold exactly that band's rows, so matrices stacked along N tile to the
    stacked tiled matrix."""
    rng = np.random.default_rng(5)
    a, b = rng.integers(0, 256, (64, 192), dtype=np.uint8), rng.integers(0, 256, (128, 192), dtype=np.uint8)
    stacked = layout.tile_bytes(np.concatenate([a, b]))
    assert np.array_equal(stacked, np.concatenate([layout.tile_bytes(a), layout.tile_bytes(b)]))
    assert np.array_equal(np.sort(stacked), np.sort(np.concatenate([a, b]).reshape(-1)))


@pytest.mark.parametrize("name", ["dit_t_bf16", "video_t_fp8"])
def test_pack_tiles_gemm_weights_only(name):
    """bf16/fp8 GEMM weights are tiled; the DiT modulation matrix and every
    non-matrix tensor keep their row-major bytes."""
    w = lwo_synth.get(name)
    t = lwo_synth.block_tensors(w, 0)
    ext = np.frombuffer(layout.pack_block(w, t), np.uint8)
    slots, _ = layout.layout_for(w)
    names = [nm for nm, _ in lwo_synth.tensor_inventory(w)]
    for nm, a in zip(names, t):
        s = next(x for x in slots if x.name == nm)
        seg = ext[s.offset:s.offset + s.nbytes]
        if s.dtype == "bf16":
            raw = codecs.bf16_encode(a).view(np.uint8).reshape(-1)
        elif s.dtype == "fp8":
            raw = codecs.quantize_tensor_e4m3(a)[0].reshape(-1)
        else:
            continue
        if nm.endswith(".w") and nm != "ada.w":
            assert layout.tiled(nm, s.dtype)
            assert not np.array_equal(seg, raw)
            assert np.array_equal(seg, layout.tile_bytes(raw.reshape(s.shape[0], -1)))
        else:
            assert not layout.tiled(nm, s.dtype)
            assert np.array_equal(seg, raw)


@pytest.mark.parametrize("name", ["dit_tiny_fp32", "dit_t_bf16", "video_t_fp32", "video_t_bf16", "video_t_fp8"])
def test_stored_params_equal_the_pack_unpack_round_trip(name):
    w = lwo_synth.get(name)
    t = lwo_synth.block_tensors(w, 2)
    want = layout.unpack_block(w, layout.pack_block(w, t))
    for threads in (1, 3):
        got = layout.stored_params(w, t, threads=threads)
        assert sorted(got) == sorted(want)
        for k in want:
            assert got[k].dtype == want[k].dtype and np.array_equal(got[k], want[k]), (k, threads)
