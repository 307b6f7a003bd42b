"""Persisted flat-block files (host only): SHA-256 against hashlib and the
published FIPS 180-2 example digests, the entry format, joining, corruption
and layout checks, and the publication protocol under concurrency, stale
temporaries, a held lock and a writer that dies holding the lock."""
import ctypes
import fcntl
import hashlib
import json
import multiprocessing as mp
import os
import shutil

import numpy as np
import pytest

import lwo_synth

ETIMEOUT, EINVAL, ECHECKSUM = 9, 1, 8


def _extents(lib, name):
    w = lwo_synth.get(name)
    desc = lib.ModelDesc.from_workload(w)
    _, ext = lib.block_layout(desc)
    bufs = []
    for b in range(w.n_blocks):
        buf = np.empty(ext, np.uint8)
        lib.pack_block(desc, lwo_synth.block_tensors(w, b), dst=buf.ctypes.data, dst_bytes=ext)
        bufs.append(buf)
    return desc, ext, bufs


@pytest.mark.parametrize("n", [0, 1, 3, 55, 56, 57, 63, 64, 65, 119, 120, 128, 1000, 65536 + 7])
def test_sha256_matches_hashlib(lib, n):
    data = np.random.default_rng(n).integers(0, 256, n, dtype=np.uint8).tobytes()
    assert lib.sha256(data) == hashlib.sha256(data).digest()


def test_sha256_published_examples(lib):
    # FIPS 180-2, appendix B.1 and B.2, and the empty message
    assert lib.sha256(b"abc").hex() == "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad"
    assert lib.sha256(b"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq").hex() == \
        "248d6a61d20638b8e5c026930c3e6039a33ce45964ff2167f6ecedd419db06c1"
    assert lib.sha256(b"").hex() == "e3b0c44298fc1c149afbf4c8996fb92427ae41e4649b934ca495991b7852b855"


def test_publish_open_roundtrip(lib, tmp_path):
    desc, ext, bufs = _extents(lib, "dit_tiny_fp32")
    key, created = lib.cache_publish(str(tmp_path), desc, extents=bufs)
    assert created and len(key) == 64
    entry = tmp_path / key
    man = json.loads((entry / "manifest.json").read_text())
    stride = (ext + 4095) // 4096 * 4096
    assert man["format"] == "lwo-flat-blocks-2" and man["key"] == key == man["content_digest"]
    assert man["n_blocks"] == desc.n_blocks and man["extent_bytes"] == ext and man["stride"] == stride
    assert (entry / "blocks.bin").stat().st_size == stride * desc.n_blocks == man["file_bytes"]
    digests = [hashlib.sha256(b.tobytes()).digest() for b in bufs]
    assert man["block_sha256"] == [d.hex() for d in digests]
    assert hashlib.sha256(man["meta"].encode() + b"".join(digests)).hexdigest() == key
    assert [(t["name"], t["tiled"]) for t in man["tensors"]] == \
           [(t["name"], t["tiled"]) for t in lib.block_layout(desc)[0]]
    raw = (entry / "blocks.bin").read_bytes()
    for b, buf in enumerate(bufs):   # extent then zero padding to the stride
        assert raw[b * stride:b * stride + ext] == buf.tobytes()
        assert raw[b * stride + ext:(b + 1) * stride] == bytes(stride - ext)
    assert not [p for p in os.listdir(tmp_path) if p.startswith(".tmp-")]
    with lib.cache_open(str(tmp_path), key, desc, verify=True) as c:
        addrs = c.extents()
        assert len(addrs) == desc.n_blocks and all(a % 4096 == 0 for a in addrs)
        for a, buf in zip(addrs, bufs):
            assert ctypes.string_at(a, ext) == buf.tobytes()


def test_publish_joins_and_fill_gives_same_key(lib, tmp_path):
    desc, ext, bufs = _extents(lib, "dit_tiny_fp32")
    key, created = lib.cache_publish(str(tmp_path), desc, extents=bufs)
    key2, created2 = lib.cache_publish(str(tmp_path), desc, extents=bufs)
    assert created and not created2 and key2 == key
    calls = []

    def fill(b, dst, n):
        calls.append(b)
        ctypes.memmove(dst, bufs[b].ctypes.data, n)

    key3, created3 = lib.cache_publish(str(tmp_path / "other"), desc, fill=fill)
    assert key3 == key and created3 and calls == list(range(desc.n_blocks)) * 2   # hash pass, write pass
    bufs[1][100] ^= 1   # different bytes -> different entry
    key4, _ = lib.cache_publish(str(tmp_path), desc, extents=bufs)
    assert key4 != key


def test_open_detects_corruption_and_other_layouts(lib, tmp_path):
    desc, ext, bufs = _extents(lib, "dit_tiny_fp32")
    key, _ = lib.cache_publish(str(tmp_path / "a"), desc, extents=bufs)
    shutil.copytree(tmp_path / "a" / key, tmp_path / "b" / key)
    with open(tmp_path / "b" / key / "blocks.bin", "r+b") as f:
        f.seek(ext + 4096 + 17)   # inside block 1 (stride >= ext)
        byte = f.read(1)
        f.seek(-1, 1)
        f.write(bytes([byte[0] ^ 0x40]))
    with pytest.raises(lib.LwoError) as e:
        lib.cache_open(str(tmp_path / "b"), key, desc, verify=True)
    assert e.value.status == ECHECKSUM
    lib.cache_open(str(tmp_path / "b"), key, desc, verify=False).close()   # unverified open maps it
    other = lib.ModelDesc.from_workload(lwo_synth.get("dit_t_fp32"))
    with pytest.raises(lib.LwoError) as e:
        lib.cache_open(str(tmp_path / "a"), key, other, verify=False)
    assert e.value.status == EINVAL
    with pytest.raises(lib.LwoError) as e:
        lib.cache_open(str(tmp_path / "a"), "0" * 64, desc)
    man = json.loads((tmp_path / "a" / key / "manifest.json").read_text())
    man["block_sha256"][0] = "0" * 64   # digests no longer give the key
    shutil.copytree(tmp_path / "a" / key, tmp_path / "c" / key)
    (tmp_path / "c" / key / "manifest.json").write_text(json.dumps(man))
    with pytest.raises(lib.LwoError) as e:
        lib.cache_open(str(tmp_path / "c"), key, desc, verify=False)
    assert e.value.status in (ECHECKSUM, 10)


def _publisher(directory, name, q):
    import layerwise_weight_offload_amd as lib
    desc, ext, bufs = _extents(lib, name)
    q.put(lib.cache_publish(directory, desc, extents=bufs, wait_ms=60000))


def test_concurrent_publishers_write_once(lib, tmp_path):
    ctx = mp.get_context("spawn")
    q = ctx.Queue()
    ps = [ctx.Process(target=_publisher, args=(str(tmp_path), "dit_tiny_fp32", q)) for _ in range(4)]
    for p in ps:
        p.start()
    res = [q.get(timeout=120) for _ in ps]
    for p in ps:
        p.join(timeout=60)
        assert p.exitcode == 0
    assert len({k for k, _ in res}) == 1 and sum(c for _, c in res) == 1
    key = res[0][0]
    assert sorted(os.listdir(tmp_path)) == sorted([key, key + ".lock"])
    desc = lib.ModelDesc.from_workload(lwo_synth.get("dit_tiny_fp32"))
    lib.cache_open(str(tmp_path), key, desc, verify=True).close()


def test_stale_temporary_is_removed(lib, tmp_path):
    desc, ext, bufs = _extents(lib, "dit_tiny_fp32")
    key, _ = lib.cache_publish(str(tmp_path / "probe"), desc, extents=bufs)
    stale = tmp_path / f".tmp-{key}-424242-7"
    stale.mkdir()
    (stale / "blocks.bin").write_bytes(b"partial")
    key2, created = lib.cache_publish(str(tmp_path), desc, extents=bufs)
    assert key2 == key and created and not stale.exists()


def _hold_lock_and_die(path):
    fd = os.open(path, os.O_RDWR | os.O_CREAT, 0o644)
    fcntl.flock(fd, fcntl.LOCK_EX)
    os._exit(0)   # dies holding the lock; the kernel releases it


def test_held_lock_times_out_and_dead_writer_releases(lib, tmp_path):
    desc, ext, bufs = _extents(lib, "dit_tiny_fp32")
    key, _ = lib.cache_publish(str(tmp_path / "probe"), desc, extents=bufs)
    lock = tmp_path / f"{key}.lock"
    fd = os.open(lock, os.O_RDWR | os.O_CREAT, 0o644)
    fcntl.flock(fd, fcntl.LOCK_EX)
    try:
        with pytest.raises(lib.LwoError) as e:
            lib.cache_publish(str(tmp_path), desc, extents=bufs, wait_ms=100)
        assert e.value.status == ETIMEOUT and not (tmp_path / key).exists()
    finally:
        fcntl.flock(fd, fcntl.LOCK_UN)
        os.close(fd)
    p = mp.get_context("spawn").Process(target=_hold_lock_and_die, args=(str(lock),))
    p.start()
    p.join(timeout=60)
    key2, created = lib.cache_publish(str(tmp_path), desc, extents=bufs, wait_ms=5000)
    assert key2 == key and created


def test_close_refuses_while_a_borrowing_store_lives(lib, tmp_path):
    """The extents list keeps its entry alive, and the entry cannot be unmapped
    while a store that reads its extents is alive (a stand-in object with a
    live handle plays the store here; the GPU test builds a real one)."""
    import gc
    desc, ext, bufs = _extents(lib, "dit_tiny_fp32")
    key, _ = lib.cache_publish(str(tmp_path), desc, extents=bufs)
    entry = lib.cache_open(str(tmp_path), key, desc, verify=True)
    addrs = entry.extents()
    assert addrs.entry is entry

    class Borrower:
        handle = 1

    store = Borrower()
    entry.borrow(store)
    with pytest.raises(lib.LwoError) as e:
        entry.close()
    assert e.value.status == 7
    assert ctypes.string_at(addrs[0], ext) == bufs[0].tobytes()   # still mapped
    store.handle = 0                                               # destroyed
    entry.close()
    with pytest.raises(lib.LwoError):
        entry.extents()
    # a dropped store no longer blocks closing
    entry = lib.cache_open(str(tmp_path), key, desc, verify=False)
    s2 = Borrower()
    entry.borrow(s2)
    del s2
    gc.collect()
    entry.close()
