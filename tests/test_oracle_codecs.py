"""Pins for the oracle's storage codecs and checksum (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import checksum, codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ------------------------------------------------------------------ bf16

def _bf16_torch(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_encode_matches_torch_random():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    np.testing.assert_array_equal(codecs.bf16_encode(x), _bf16_torch(x))


def test_bf16_encode_ties_and_specials():
    # exact halfway cases: 1 + 2^-8 (tie, even neighbour is 1.0), 1 + 3*2^-8 (tie, rounds up)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 3.3895314e38,
                     3.3961776e38, -3.3961776e38, 3.3961773e38, 3.4e38, np.finfo(np.float32).max,
                     np.inf, -np.inf, 0.0, -0.0, 1e-45, 65504.0], dtype=np.float32)
    np.testing.assert_array_equal(codecs.bf16_encode(ties), _bf16_torch(ties))
    assert codecs.bf16_encode(np.array([1 + 2 ** -8], np.float32))[0] == 0x3F80
    assert codecs.bf16_encode(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 0x3F82
    nan = codecs.bf16_encode(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_bf16_decode_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = codecs.bf16_decode(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# ------------------------------------------------------------------ e4m3

def test_e4m3_landmarks_from_spec():
    for code, val in _golden_lines("e4m3_landmarks.txt"):
        c = int(code, 16)
        v = float(val)
        got = codecs.E4M3_VALUES[c]
        assert got == v and np.signbit(got) == np.signbit(v), (code, got, v)
    assert np.isnan(codecs.E4M3_VALUES[0x7F]) and np.isnan(codecs.E4M3_VALUES[0xFF])
    assert np.isfinite(codecs.E4M3_VALUES[[c for c in range(256) if c & 0x7F != 0x7F]]).all()


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-12, 6, 100_000))).astype(np.float32)
    x = np.clip(x, -464, 464).astype(np.float32)   # torch's cast is NaN beyond the 448/480 midpoint
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codecs.e4m3_encode(x), ref)
    # every exact value and every midpoint between neighbours
    pos = codecs.E4M3_VALUES[:127]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    allv = np.concatenate([pos, -pos, mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(allv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codecs.e4m3_encode(allv), ref)


def test_e4m3_saturates():
    x = np.array([449, 480, 1e6, -1e30, np.inf], dtype=np.float32)
    np.testing.assert_array_equal(codecs.e4m3_encode(x), [0x7E, 0x7E, 0x7E, 0xFE, 0x7E])


def test_quantize_tensor_error_bound():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 96)) * 0.02).astype(np.float32)
    codes, s = codecs.quantize_tensor_e4m3(w)
    assert s == np.float32(np.max(np.abs(w)) / np.float32(448))
    deq = codecs.e4m3_decode(codes) * np.float64(s)
    # relative half-ulp of e4m3 normals is 2^-4; subnormal steps are 2^-10 absolute (in code units)
    err = np.abs(deq - w.astype(np.float64))
    bound = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * float(s)) * (1 + 1e-6)
    assert (err <= bound).all()
    assert np.max(np.abs(codecs.e4m3_decode(codes))) == 448.0
    z_codes, z_s = codecs.quantize_tensor_e4m3(np.zeros((3, 4), np.float32))
    assert z_s == 1.0 and not z_codes.any()


def test_quantize_rows_matches_definition():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 37)).astype(np.float32)
    x[2] = 0
    codes, s = codecs.quantize_rows_e4m3(x)
    assert s[2] == 1.0 and not codes[2].any()
    for r in (0, 1, 3, 4):
        amax = np.float32(np.max(np.abs(x[r])))
        assert s[r] == np.float32(amax / np.float32(448))
        assert np.abs(codecs.e4m3_decode(codes[r])).max() == 448.0
        ref = torch.from_numpy((x[r] * np.float32(np.float32(448) / amax)).astype(np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(codes[r], ref)


# ------------------------------------------------------------------ checksum

def test_splitmix64_published_sequence():
    want = [int(ln[0], 16) for ln in _golden_lines("splitmix64_seed0.txt")]
    gamma = 0x9E3779B97F4A7C15
    # output k of the generator started at 0 is the finaliser of k*gamma, i.e. next() from state (k-1)*gamma
    states = np.array([((k - 1) * gamma) % 2 ** 64 for k in (1, 2, 3)], dtype=np.uint64)
    got = [int(v) for v in checksum.splitmix64_next(states)]
    assert got == want


def _checksum_brute(buf: bytes) -> int:
    """Pure-Python integer version of the definition, for tiny inputs."""
    M = 2 ** 64
    g = 0x9E3779B97F4A7C15
    tot = 0
    for i in range(len(buf) // 8):
        w = int.from_bytes(buf[8 * i:8 * i + 8], "little")
        z = (w ^ (i * g % M)) % M
        z = (z + g) % M
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) % M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) % M
        z = z ^ (z >> 31)
        tot = (tot + z) % M
    return tot


def test_checksum_brute_force_and_properties():
    rng = np.random.default_rng(4)
    buf = rng.integers(0, 256, 8 * 257, dtype=np.uint8).tobytes()
    assert checksum.extent_checksum(buf) == _checksum_brute(buf)
    assert checksum.extent_checksum(b"") == 0
    # position weighting: swapping two different words changes the sum
    a = bytearray(buf)
    a[0:8], a[8:16] = buf[8:16], buf[0:8]
    assert checksum.extent_checksum(bytes(a)) != checksum.extent_checksum(buf)
    # a single flipped bit changes the sum
    a = bytearray(buf)
    a[1000] ^= 0x10
    assert checksum.extent_checksum(bytes(a)) != checksum.extent_checksum(buf)
    with pytest.raises(ValueError):
        checksum.extent_checksum(b"1234567")


# ------------------------------------------------------------------ grid rounding (fast stored values)

def _bf16_neighbourhood() -> np.ndarray:
    """Every bf16 pattern with several low halves: exact values, the smallest
    steps above them, the ties just below/at/above the midpoint and the last
    pattern before the next value (float32 bit patterns, both signs)."""
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0, 1, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    return u.view(np.float32)


def test_bf16_round_grid_equals_the_pattern_codec():
    x = _bf16_neighbourhood()
    want = codecs.bf16_round(x)
    got = codecs.bf16_round_grid(x)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), x[~same][:8]
    assert (np.signbit(got) == np.signbit(want))[~np.isnan(want)].all()
    rng = np.random.default_rng(11)
    y = (rng.standard_normal(300_000) * np.exp(rng.uniform(-90, 88, 300_000))).astype(np.float32)
    np.testing.assert_array_equal(codecs.bf16_round_grid(y), codecs.bf16_round(y))
    # largest finite bf16, the overflow tie, and the subnormal steps
    edge = np.array([3.3895314e38, 3.3961776e38, -3.3961776e38, 2 ** -133, 1.5 * 2 ** -133, 2 ** -134,
                     2.5 * 2 ** -133, 1e-45], dtype=np.float32)
    np.testing.assert_array_equal(codecs.bf16_round_grid(edge), codecs.bf16_round(edge))


def test_e4m3_round_grid_equals_the_table_codec():
    pos = codecs.E4M3_VALUES[:127]
    mids = (pos[1:] + pos[:-1]) / 2
    nudge = np.concatenate([mids * (1 - 2 ** -20), mids * (1 + 2 ** -20)])
    rng = np.random.default_rng(12)
    wide = rng.standard_normal(200_000) * np.exp(rng.uniform(-16, 8, 200_000))
    x = np.concatenate([pos, -pos, mids, -mids, nudge, -nudge, wide, [0.0, -0.0, 448.0, 449.0, 464.0, 480.0,
                                                                    1e9, -1e9, np.inf, -np.inf, np.nan]])
    want = codecs.e4m3_decode(codecs.e4m3_encode(x))
    got = codecs.e4m3_round_grid(x)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), x[~same][:8]
    assert (np.signbit(got) == np.signbit(want))[~np.isnan(want)].all()


# ------------------------------------------------------------------ the fp8 activation emulation

@pytest.mark.parametrize("stored_bf16", [False, True])
def test_fp8_activation_matches_torch_casts(stored_bf16):
    """oracle.dit.fp8_activation against torch: (optionally) a bf16 cast of the
    float32 rows, the per-row scale amax/448 in float32, a float8_e4m3fn cast
    of the rows times 448/amax, and the codes' values times the scale."""
    from oracle import dit
    rng = np.random.default_rng(13)
    z = rng.standard_normal((9, 200)) * np.exp(rng.uniform(-4, 4, (9, 1)))
    z[4] = 0.0
    z[6, :] = 1e-3
    got = dit.fp8_activation(z, stored_bf16)
    t = torch.from_numpy(z.astype(np.float32))
    if stored_bf16:
        t = t.to(torch.bfloat16).to(torch.float32)
    amax = t.abs().amax(dim=1)
    nz = amax > 0
    scale = torch.where(nz, amax / 448.0, torch.ones_like(amax))
    inv = torch.where(nz, 448.0 / torch.where(nz, amax, torch.ones_like(amax)), torch.zeros_like(amax))
    codes = (t * inv[:, None]).to(torch.float8_e4m3fn)
    want = codes.to(torch.float64) * scale.to(torch.float64)[:, None]
    np.testing.assert_array_equal(got, want.numpy())
    assert not got[4].any()


def test_fp8_activation_bf16_pre_rounding_is_observable():
    """The bf16 rounding before quantisation changes the code when it moves a
    value across an e4m3 rounding boundary: with row amax 448 the scale is 1,
    and 1 + 1/16 + 2^-10 (just above the e4m3 midpoint 1 + 1/16 between 1 and
    1.125) rounds to bf16 1 + 1/16 exactly, a tie that goes to the even code 1.0."""
    from oracle import dit
    v = np.array([[1.0 + 2 ** -4 + 2 ** -10, 448.0]])
    assert dit.fp8_activation(v, False)[0, 0] == 1.125
    assert dit.fp8_activation(v, True)[0, 0] == 1.0
