"""CPU oracle for layerwise weight offload of a DiT block stack.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this package.  The library under
``layerwise_weight_offload_amd`` never imports it, and it imports nothing
from the library: the two share no code.  Inputs come from ``lwo_synth``.

Offloading changes where block weights live, not what a block computes
("CPU Offloading for Diffusion Models", section "Layerwise (Blockwise)
Offloading / How It Works": each block runs its ordinary forward once its
weights are on the device).  The oracle therefore is the plain definition:
every block's weights resident, blocks applied in order, in float64.

Modules
  codecs    bf16 and OCP fp8 e4m3 storage codecs (encode/decode)
  layout    the flat per-block extent: tensor order, offsets, packing
  checksum  position-weighted SplitMix64 sum over a block extent
  dit       LayerNorm, RMSNorm, GELU-tanh, SiLU, attention, both block kinds

Every function here is pinned by tests in ``tests/test_oracle_*.py`` against
closed forms, brute force, library routines or published values.  The
whole-stack output is pinned only through those component pins and the
structural identities (zero gates, bias path); the pages print no worked
numbers for it.
"""
