"""One rank's share of the all-gather shard path ("Distributed Layerwise
Offload", "AllGather path" and "Host backing and transfer composition"): the
store pins only shard `rank` of every block, copies it host -> device into
its offset of the slot, and a gather stream completes the slot with the other
shards (held on the device in place of the peers).  The slot then holds the
block's extent byte for byte, so every output must be bit-identical to the
PIN_COPY store's, the slot checksum must equal the oracle's extent checksum,
and the host bytes and host -> device bytes per step must be the shard's."""
import numpy as np
import pytest

import lwo_synth
from oracle import checksum as o_ck
from oracle import dit as o_dit
from oracle import layout as o_layout

from .conftest import gpu_available
from .gpu_util import device_inputs, make_store, oracle_out, row_col_errors, run_steps, to_f64

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _bits(w, x):
    import torch
    return x.cpu().view(-1).view(torch.int16 if w.act_dtype == "bf16" else torch.int32).numpy().copy()


def _shard_store(lib, w, g, r):
    desc = lib.ModelDesc.from_workload(w)

    def fill(b, dst, n):
        lib.pack_block(desc, lwo_synth.block_tensors(w, b), dst=dst, dst_bytes=n)

    return lib.build_shard_store(desc, g, r, fill=fill)


def _reference_bits(lib, w, k=0, steps=3):
    with make_store(lib, w, k=k) as st:
        x, c, cx = device_inputs(w)
        run_steps(st, x, c, cx, steps=steps)
        return _bits(w, x)


@pytest.mark.parametrize("name,g,r", [("video_t_bf16", 1, 0), ("video_t_bf16", 2, 1), ("video_t_bf16", 3, 0),
                                      ("video_t_bf16", 3, 2), ("video_t_bf16", 8, 5), ("dit_t_fp32", 4, 3)])
def test_shard_equals_pin_copy_and_slot_bytes(lib, name, g, r):
    w = lwo_synth.get(name)
    print(f"[shard] {name} group={g} rank={r}", flush=True)
    ref = _reference_bits(lib, w)
    with _shard_store(lib, w, g, r) as st:
        s0 = st.stats()
        ext = s0.extent_bytes
        unit = g * 4096
        padded = (o_layout.layout_for(w)[1] + unit - 1) // unit * unit
        assert s0.host_mode == lib.HOST_SHARD and s0.group == g and s0.rank == r
        assert s0.slot_bytes == padded and s0.shard_bytes == padded // g
        assert s0.host_bytes == w.n_blocks * s0.shard_bytes
        assert s0.peer_device_bytes == w.n_blocks * (padded - s0.shard_bytes)
        x, c, cx = device_inputs(w)
        run_steps(st, x, c, cx, steps=3)
        s = st.stats()
        # one prime copy, then one shard per streamed block per step
        assert s.h2d_copies == 1 + 3 * w.n_blocks and s.h2d_bytes == s.h2d_copies * s.shard_bytes
        assert s.gather_bytes == s.h2d_copies * (padded - s.shard_bytes)
        assert np.array_equal(_bits(w, x), ref)
        for b in range(w.n_blocks):
            hs, ss = st.block_checksum(b)
            assert hs == ss == o_ck.extent_checksum(o_layout.pack_block(w, lwo_synth.block_tensors(w, b)))
        assert ext == o_layout.layout_for(w)[1]


def test_shard_with_resident_prefix_and_validation(lib):
    w = lwo_synth.get("video_t_bf16")
    ref = _reference_bits(lib, w, k=1)
    with _shard_store(lib, w, 4, 1) as st:
        st.set_resident_prefix(1)
        st.set_validation(True)
        x, c, cx = device_inputs(w)
        run_steps(st, x, c, cx, steps=3)
        s = st.stats()
        assert s.validation == 1 and s.checksum_mismatches == 0 and s.resident_prefix == 1
        assert np.array_equal(_bits(w, x), ref)


def test_shard_fp8_against_oracle(lib):
    """fp8 linears through a group of 4, rank 2: the same bits as PIN_COPY and
    the stated 5e-2 against the plain oracle."""
    w = lwo_synth.get("video_t_fp8")
    ref = _reference_bits(lib, w, steps=1)
    x0, want = oracle_out(w)
    with _shard_store(lib, w, 4, 2) as st:
        x, c, cx = device_inputs(w)
        run_steps(st, x, c, cx, steps=1)
        assert np.array_equal(_bits(w, x), ref)
        got = to_f64(x).reshape(want.shape)
    e = o_dit.rel_l2(got, want)
    e_row, _ = row_col_errors(got, want)
    print(f"[shard] video_t_fp8 group 4 rank 2: rel_l2 {e:.3e}, max row {e_row:.3e}", flush=True)
    assert e <= 5e-2 and e_row <= 7.5e-2
