"""lwo_run_blocks_noalloc (no device allocation; the workspace lives in the
library's per-GPU scratch array) against lwo_run_denoise_step with every
block resident: the same kernels in the same order on the same bytes, so the
outputs must be identical bit for bit.  Two calls in a row on one GPU, the
second with fewer tokens than the first (the array keeps the first call's
contents), then a descriptor whose workspace exceeds the array is refused
before anything is enqueued."""
import numpy as np
import pytest

import lwo_synth

from .conftest import gpu_available
from .gpu_util import device_inputs, make_store, run_steps

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _bits(w, x):
    import torch
    return x.cpu().view(-1).view(torch.int16 if w.act_dtype == "bf16" else torch.int32).numpy().copy()


def _device_extents(lib, w):
    import torch
    desc = lib.ModelDesc.from_workload(w)
    out = []
    for b in range(w.n_blocks):
        ext = lib.pack_block(desc, lwo_synth.block_tensors(w, b))
        out.append(torch.from_numpy(ext).to("cuda:0"))
    return desc, out


def _resident_step_bits(lib, w):
    with make_store(lib, w, k=w.n_blocks) as st:
        x, c, cx = device_inputs(w)
        run_steps(st, x, c, cx, steps=1)
        return _bits(w, x)


@pytest.mark.parametrize("name,small_tokens", [("video_t_bf16", 100), ("dit_t_fp32", 57), ("video_t_fp8", 130)])
def test_noalloc_equals_resident_step_twice(lib, name, small_tokens):
    import torch
    w_big = lwo_synth.get(name)
    w_small = w_big.with_(tokens=small_tokens)
    s = torch.cuda.Stream()
    for w in (w_big, w_small):
        print(f"[noalloc] {name} tokens={w.tokens}", flush=True)
        desc, exts = _device_extents(lib, w)
        x, c, cx = device_inputs(w)
        torch.cuda.synchronize()
        lib.run_blocks_noalloc(desc, [e.data_ptr() for e in exts], x.data_ptr(), c.data_ptr(),
                               cx.data_ptr() if cx is not None else None, s.cuda_stream)
        s.synchronize()
        assert torch.cuda.current_device() == 0   # the caller's current device is left as it was
        got = _bits(w, x)
        assert np.array_equal(got, _resident_step_bits(lib, w)), (name, w.tokens)


def test_noalloc_refuses_a_workspace_beyond_the_array(lib):
    import torch
    w = lwo_synth.get("video14b_bf16")          # 32760 tokens: a workspace of about 1.6 GB
    desc = lib.ModelDesc.from_workload(w)
    buf = torch.zeros(1 << 12, dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.Stream()
    with pytest.raises(lib.LwoError) as e:
        lib.run_blocks_noalloc(desc, [buf.data_ptr()] * 2, buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                               s.cuda_stream)
    assert e.value.status == 1 and "scratch" in str(e.value)
    with pytest.raises(lib.LwoError):
        lib.run_blocks_noalloc(desc, [buf.data_ptr()], buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), 0)
