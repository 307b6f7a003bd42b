#!/usr/bin/env python3
"""Denoise-step benchmark of layerwise weight offload on one MI355X.

One step = one pass of the whole block stack over one batch of synthetic
input: every streamed block's weights are copied host -> device through the
two slots while the previous block computes.  Default workload: the
14B-class video DiT stack (40 blocks, D 5120, 40 heads of 128, FFN 13824,
32760 tokens, 512 context tokens, bf16), all 40 blocks streamed: the largest
workload that fits one GPU, and the one whose per-block compute must hide the
next block's copy.

Timed regions (HIP events recorded on the stream the library enqueues on):
  resident  blocks 0..L-1 kept on the device (no copies)       -> T_res
  streamed  blocks k..L-1 streamed through the two slots        -> T_str (the value)
  kernels   resident again, with per-kernel events              -> roofline of the dominant kernel
plus a pinned-memory H2D peak (hipMemcpyAsync from hipHostMalloc'd memory,
block-sized and 1 GiB copies, best of 10) and the oracle's time on the host
for a bounded sample of blocks.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise-step ms streamed vs resident; H2D GB/s; overlap %; block TFLOP/s"
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
HBM_PEAK_GBPS = 8000.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def pinned_peak(torch, nbytes: int, stream, reps: int = 10) -> float:
    """Best-of-reps GB/s of one hipMemcpyAsync of nbytes from pinned host memory."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    best = 0.0
    with torch.cuda.stream(stream):
        for _ in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src, non_blocking=True)
            e1.record(stream)
            e1.synchronize()
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return best


def copy_calibration(torch) -> int:
    """Three dispatches of a plain streaming kernel (y = 1.0 * x over 2^28 fp32):
    each reads and writes exactly 1 GiB, so what FETCH_SIZE / WRITE_SIZE report
    for it gives the scale from those counters to HBM bytes."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise y = 1.0 * x", "dispatches": 3, "read_bytes": 4 * n,
                      "write_bytes": 4 * n}), flush=True)
    return 0


def committed_traffic(label: str, workload: str):
    """HBM bytes per launch of `label` on `workload` from a committed rocprofv3
    counter summary (profiles/*.md, a fenced json block), or None when there is
    none or the kernel sources changed since the counters were taken."""
    import glob
    import hashlib
    import re
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for blk in re.findall(r"```json\n(.*?)\n```", open(path).read(), re.S):
            try:
                rec = json.loads(blk)
            except ValueError:
                continue
            if rec.get("label") != label or rec.get("workload") != workload:
                continue
            h = hashlib.sha256()
            for src in rec.get("sources", []):
                with open(os.path.join(ROOT, src), "rb") as f:
                    h.update(f.read())
            if h.hexdigest() != rec.get("sources_sha256"):
                return None
            return rec.get("hbm_bytes_per_launch")
    return None


def block_flops(w) -> float:
    """Algorithmic FLOPs of one block: 2MNK per linear, 4 B H Tq Tk d per attention."""
    B, T, D, F, Tc = w.batch, w.tokens, w.hidden, w.ffn, w.ctx_tokens
    M = B * T
    gemm = 2.0 * M * D * (3 * D + D + 2 * F)
    attn = 4.0 * B * T * T * D
    if w.kind == "video":
        gemm += 2.0 * M * D * (2 * D) + 2.0 * B * Tc * D * 2 * D
        attn += 4.0 * B * T * Tc * D
    else:
        gemm += 2.0 * B * D * 6 * D
    return gemm + attn


def _f32_params(p: dict) -> dict:
    return {k: v.astype(np.float32) for k, v in p.items() if not k.startswith("_")}


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(w, seconds: float, max_block_flops: float = 2.5e12, type_of=None):
    """The oracle (every weight resident, NumPy float32 with BLAS on every
    host core) timed on a bounded sample of the step.

    Blocks up to max_block_flops: whole blocks of the step in order while the
    time budget lasts, per-block time x the block count.  Larger blocks (the
    32760-token video blocks): the oracle's block evaluated at r query rows
    (oracle.dit.video_block_rows: LayerNorm, K and V over every token, the
    rest of the block for the r rows against all keys and values), timed at
    two row counts.  Its cost is affine in r, so the two points extrapolate to
    all rows of one full-shape block, then x the block count.  float64 (the
    precision of the parity oracle) is timed the same way as an extra.
    type_of(b): block b's workload in a mixed stack (w gives the inputs)."""
    import lwo_synth
    from oracle import dit as o_dit
    from oracle import layout as o_layout
    cores = int(_threads())
    threads = min(16, os.cpu_count() or 1)
    x64, c64, ctx64 = o_dit.decode_inputs(w, *lwo_synth.step_inputs(w))
    if block_flops(w) <= max_block_flops:
        x = x64.astype(np.float32)
        cond = c64.astype(np.float32)
        ctx = None if ctx64 is None else ctx64.astype(np.float32)
        done, spent = 0, 0.0
        while done < w.n_blocks and (done == 0 or spent < seconds):
            wb = w if type_of is None else type_of(done)
            p = _f32_params(o_layout.stored_params(wb, lwo_synth.block_tensors(wb, done), threads=threads))
            t0 = time.perf_counter()
            x = o_dit.block_forward(wb, x, cond, ctx, p)
            spent += time.perf_counter() - t0
            done += 1
            log(f"oracle block {done}: {spent:.1f} s so far")
        return {"value": round(spent / done * 1e3 * w.n_blocks, 1), "unit": "ms", "cores": cores, "kind": "oracle",
                "sample": f"{done} of {w.n_blocks} blocks of one step timed ({spent:.1f} s), per-block time x "
                          f"{w.n_blocks}; NumPy float32, {cores} BLAS threads"}
    assert w.kind == "video"
    p64 = o_layout.stored_params(w, lwo_synth.block_tensors(w, 0), threads=threads)

    def timed_rows(dt, n):
        rows = np.arange(n)
        p = p64 if dt == np.float64 else _f32_params(p64)
        args = [a.astype(dt) for a in (x64, c64, ctx64)]
        t0 = time.perf_counter()
        o_dit.video_block_rows(*args, p, w.heads, rows)
        return time.perf_counter() - t0

    out = {}
    for dt, (r1, r2) in ((np.float32, (256, 1024)), (np.float64, (64, 256))):
        r2 = min(r2, w.tokens)
        r1 = min(r1, r2 // 2)
        t1, t2 = timed_rows(dt, r1), timed_rows(dt, r2)
        per_block = t1 + (t2 - t1) * (w.tokens - r1) / (r2 - r1)
        out[dt] = (per_block, t1, t2, r1, r2)
        log(f"oracle block 0, {np.dtype(dt).name}: {r1} rows {t1:.1f} s, {r2} rows {t2:.1f} s -> "
            f"{per_block:.0f} s for all {w.tokens} rows")
    pb, t1, t2, r1, r2 = out[np.float32]
    pb64 = out[np.float64][0]
    return {"value": round(pb * 1e3 * w.n_blocks, 1), "unit": "ms", "cores": cores, "kind": "oracle",
            "sample": f"block 0 at full shape (all {w.tokens} tokens for K/V, queries against all keys) evaluated "
                      f"at {r1} and {r2} query rows ({t1:.1f} s and {t2:.1f} s), its affine cost in the rows "
                      f"extrapolated to all {w.tokens} rows, x {w.n_blocks} blocks; NumPy float32, {cores} BLAS "
                      f"threads",
            "float64_value": round(pb64 * 1e3 * w.n_blocks, 1),
            "float64_sample": f"the same at {out[np.float64][3]} and {out[np.float64][4]} rows in float64"}


def mfma_probe(torch, lwo, s, reps: int = 3) -> dict:
    """Sustained dense MFMA rate of lwo_probe_mfma (bf16 and fp8, three
    workgroups of four wavefronts per CU, the most its registers let one CU
    hold at once, independent accumulator chains): what the matrix cores
    deliver at the clock they hold under full load.  Best of `reps`."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 3 * cus
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    out = {"blocks": blocks}
    for name, dt, iters in (("bf16", lwo.BF16, 20000), ("fp8", lwo.FP8_E4M3, 5000)):
        lwo.probe_mfma(dt, blocks, iters, sink.data_ptr(), sink.numel(), s.cuda_stream)   # warm-up
        best = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fl = lwo.probe_mfma(dt, blocks, iters, sink.data_ptr(), sink.numel(), s.cuda_stream)
            e1.record(s)
            e1.synchronize()
            best = max(best, fl / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        out[name + "_tflops"] = round(best, 1)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="video14b_bf16")
    ap.add_argument("--resident-prefix", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--host-mode", choices=("pin_copy", "staged"), default="pin_copy",
                    help="pin_copy: pinned host extents; staged: pageable extents packed through two pinned "
                         "staging slots")
    ap.add_argument("--cache-dir", default=None,
                    help="with --host-mode staged: publish the stack as a flat-block file under this directory, "
                         "map it back (verified) and stream from the mapping")
    ap.add_argument("--shard", default=None, metavar="G:R",
                    help="one rank's share of an all-gather group of G: only shard R of every block is pinned and "
                         "copied host -> device; the other shards stand in on the device")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain elementwise copy of known size (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2

    import torch

    import layerwise_weight_offload_amd as lwo
    import lwo_synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(torch)
    mixed = lwo_synth.MIXED.get(args.workload)
    if mixed is not None:   # a stack of several block types (extents of different sizes)
        if args.host_mode != "pin_copy":
            print("bench.py: mixed stacks are measured in pin_copy mode", file=sys.stderr)
            return 2
        w = mixed.inputs
        L = mixed.n_blocks
        k = 0 if args.resident_prefix is None else args.resident_prefix
        tdescs = [lwo.ModelDesc.from_workload(t.with_(n_blocks=L)) for t in mixed.types]
        text = [lwo.block_layout(d)[1] for d in tdescs]
        desc_of = lambda b: tdescs[mixed.block_type[b]]
        ext_of = [text[t] for t in mixed.block_type]
        type_of = mixed.type_of
    else:
        w = lwo_synth.get(args.workload)
        k = w.resident_prefix if args.resident_prefix is None else args.resident_prefix
        L = w.n_blocks
        desc = lwo.ModelDesc.from_workload(w)
        desc_of = lambda b: desc
        ext_of = [lwo.block_layout(desc)[1]] * L
        type_of = None
    ext = max(ext_of)

    # ---- build the store from the seeded generator (drawn ahead on host threads)
    blocks = lwo_synth.iter_blocks(mixed if mixed is not None else w)

    def fill(b, dst, n):
        bb, t = next(blocks)
        assert bb == b
        lwo.pack_block(desc_of(b), t, dst=dst, dst_bytes=n)
        if b % 8 == 7 or b == L - 1:
            log(f"packed block {b + 1}/{L}")

    shard = None
    if args.shard:
        if mixed is not None or args.host_mode != "pin_copy":
            print("bench.py: --shard takes a one-type stack and no --host-mode", file=sys.stderr)
            return 2
        g, r = (int(v) for v in args.shard.split(":"))
        shard = (g, r)
    t0 = time.perf_counter()
    if shard is not None:
        store = lwo.build_shard_store(desc, shard[0], shard[1], fill=fill)
    elif args.host_mode == "staged":
        pageable = []
        for b in range(L):
            buf = np.empty(ext, np.uint8)   # ordinary pageable host memory
            fill(b, buf.ctypes.data, ext)
            pageable.append(buf)
        cache_entry = None
        if args.cache_dir:
            t1 = time.perf_counter()
            key, created = lwo.cache_publish(args.cache_dir, desc, extents=pageable)
            del pageable
            cache_entry = lwo.cache_open(args.cache_dir, key, desc, verify=True)
            pageable = cache_entry.extents()
            log(f"flat-block file {key[:12]}... ({'published' if created else 'joined'}) and verified mapping in "
                f"{time.perf_counter() - t1:.1f} s")
        store = lwo.build_block_store(desc, extents=pageable, host_mode=lwo.HOST_STAGED)
    elif mixed is not None:
        store = lwo.build_mixed_store(tdescs, mixed.block_type, fill=fill)
    else:
        store = lwo.build_block_store(desc, fill=fill)
    log(f"built {L} extents of {', '.join(f'{e / 1e6:.2f}' for e in sorted(set(ext_of)))} MB ({args.host_mode}) "
        f"in {time.perf_counter() - t0:.1f} s")

    dt = torch.float32 if w.act_dtype == "f32" else torch.bfloat16
    xs, cs, cxs = lwo_synth.step_inputs(w)
    x0 = torch.from_numpy(xs).to("cuda:0").to(dt)
    cond = torch.from_numpy(cs).to("cuda:0").to(dt)
    ctx = None if cxs is None else torch.from_numpy(cxs).to("cuda:0").to(dt)
    x = x0.clone()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()

    def region(steps: int, warmup: int) -> float:
        x.copy_(x0)
        torch.cuda.synchronize()
        for _ in range(warmup):
            store.run_denoise_step(x.data_ptr(), cond.data_ptr(), ctx.data_ptr() if ctx is not None else None,
                                   s.cuda_stream)
        s.synchronize()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(steps):
            store.run_denoise_step(x.data_ptr(), cond.data_ptr(), ctx.data_ptr() if ctx is not None else None,
                                   s.cuda_stream)
        e1.record(s)
        e1.synchronize()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    # ---- all resident
    store.set_resident_prefix(L)
    t_res = region(args.steps, args.warmup)
    log(f"resident: {t_res:.3f} ms/step")

    # ---- per-kernel timing (resident, same kernels)
    store.set_kernel_timing(True)
    region(args.steps, 0)
    kstats = store.kernel_stats()
    store.set_kernel_timing(False)

    # ---- streamed
    store.set_resident_prefix(k)
    t_str = region(args.steps, args.warmup)
    log(f"streamed (k={k}): {t_str:.3f} ms/step")
    store.set_copy_timing(True)
    region(1, 0)
    copy_ms = store.copy_times()
    store.set_copy_timing(False)
    st = store.stats()

    # ---- pinned H2D peak (copies of the size the ring issues: an extent, or a shard)
    peak_block = pinned_peak(torch, st.shard_bytes if shard is not None else ext, s)
    peak_gib = pinned_peak(torch, 1 << 30, s, reps=5)
    peak = max(peak_block, peak_gib)
    log(f"pinned H2D peak: block-sized {peak_block:.1f} GB/s, 1 GiB {peak_gib:.1f} GB/s")
    probe = mfma_probe(torch, lwo, s)
    log(f"MFMA probe: bf16 {probe['bf16_tflops']} TFLOP/s, fp8 {probe['fp8_tflops']} TFLOP/s sustained")

    m = L - k
    copies_per_step = m if m >= 3 else 0
    if shard is not None:   # only the rank's shard crosses the host link
        ext_of = [st.shard_bytes] * L
    bytes_per_step = sum(ext_of[k:]) if copies_per_step else 0
    h2d_gbps = bytes_per_step / (t_str * 1e-3) / 1e9 if bytes_per_step else 0.0
    t_copy = bytes_per_step / (peak_block * 1e9) * 1e3 if bytes_per_step else 0.0
    overlap = None
    if t_copy > 0:
        overlap = max(0.0, min(1.0, (t_res + t_copy - t_str) / min(t_res, t_copy)))
    # A step copies blocks k+1 .. L-1, then block k for the next step.
    copy_order = list(range(k + 1, L)) + [k]
    per_copy = [ext_of[copy_order[i % len(copy_order)]] / (c * 1e-3) / 1e9 for i, c in enumerate(copy_ms) if c > 0]

    steps_timed = args.steps
    flops_step = sum(kk["flops"] for kk in kstats) / steps_timed
    block_tflops = flops_step / (t_res * 1e-3) / 1e12
    lin_dt = w.linear_dtype if w.linear_dtype != "f32" else "f32"
    dom = max(kstats, key=lambda kk: kk["total_ms"])
    avg_ms = dom["total_ms"] / dom["launches"]
    if dom["flops"] > 0:
        kdt = "fp8" if "fp8" in dom["name"] else ("f32" if "f32" in dom["name"] else "bf16")
        ach = dom["flops"] / dom["launches"] / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS[kdt], "unit": "TFLOP/s",
                "frac": round(ach / MFMA_PEAK_TFLOPS[kdt], 4)}
        if kdt in ("bf16", "fp8"):   # context: the sustained rate the probe measured on this GPU
            roof.update({"probe_peak": probe[kdt + "_tflops"], "frac_of_probe": round(ach / probe[kdt + "_tflops"], 4)})
    else:
        ach = dom["bytes"] / dom["launches"] / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4)}
    roof.update({"kernel": dom["name"], "avg_launch_ms": round(avg_ms, 4), "launches_per_step": dom["launches"] // steps_timed,
                 "algorithmic_bytes_per_launch": round(dom["bytes"] / dom["launches"]),
                 "traffic": committed_traffic(dom["name"], args.workload)})

    kernels = {kk["name"]: {"ms_per_step": round(kk["total_ms"] / steps_timed, 4),
                            "launches_per_step": kk["launches"] // steps_timed,
                            "tflops": round(kk["flops"] / (kk["total_ms"] * 1e-3) / 1e12, 1) if kk["flops"] else None,
                            "gbps": round(kk["bytes"] / (kk["total_ms"] * 1e-3) / 1e9, 1)}
               for kk in sorted(kstats, key=lambda kk: -kk["total_ms"])}

    cpu = None
    if not args.no_cpu_baseline:
        store.destroy()   # release pinned host memory before the oracle allocates
        cpu = cpu_baseline(w, args.cpu_seconds, type_of=type_of)

    out = {
        "metric": METRIC, "value": round(t_str, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_str, 3), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8+bf16"}[
            "fp8" if mixed is not None and any(t.linear_dtype == "fp8" for t in mixed.types) else w.linear_dtype],
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) inputs)",
        "config": {"workload": args.workload, "kind": w.kind, "blocks": L, "hidden": w.hidden, "heads": w.heads,
                   "ffn": w.ffn, "batch": w.batch, "tokens": w.tokens, "ctx_tokens": w.ctx_tokens,
                   "act_dtype": w.act_dtype, "linear_dtype": w.linear_dtype, "resident_prefix": k,
                   "streamed_blocks": m, "host_mode": args.host_mode + ("+file" if args.cache_dir else ""),
                   "extent_bytes": ext},
        "resident_ms": round(t_res, 3),
        "streamed_over_resident": round(t_str / t_res, 4),
        "h2d_gbps": round(h2d_gbps, 2),
        "pinned_peak_gbps": round(peak, 2),
        "pinned_peak_block_gbps": round(peak_block, 2),
        "h2d_frac_of_pinned_peak": round(h2d_gbps / peak_block, 4) if bytes_per_step else None,
        "per_copy_gbps_median": round(float(np.median(per_copy)), 2) if per_copy else None,
        "copy_ms_if_serial": round(t_copy, 3),
        "overlap_pct": None if overlap is None else round(100 * overlap, 1),
        "block_tflops": round(block_tflops, 2),
        "block_mfma_frac": round(block_tflops / MFMA_PEAK_TFLOPS[lin_dt if lin_dt != "fp8" else "bf16"], 4),
        "h2d_copies_total": st.h2d_copies,
        "pack_gbps": round(st.pack_bytes / (st.pack_ms * 1e-3) / 1e9, 2) if st.pack_ms > 0 else None,
        "pack_threads": st.pack_threads or None,
        "build_s": round(st.build_ms / 1e3, 2),
        "roofline": roof,
        "mfma_probe": probe,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    if shard is not None:
        cm = sorted(copy_ms)
        out["config"]["host_mode"] = "shard"
        out["shard"] = {"group": shard[0], "rank": shard[1], "shard_bytes": st.shard_bytes,
                        "host_pinned_bytes": st.host_bytes, "h2d_bytes_per_step": bytes_per_step,
                        "gather_bytes_per_step": copies_per_step * (st.slot_bytes - st.shard_bytes),
                        "peer_device_bytes": st.peer_device_bytes,
                        "shard_copy_ms_median": round(cm[len(cm) // 2], 4) if cm else None,
                        "note": "the other ranks' shards come from a device region in place of the all-gather"}
    if mixed is not None:
        out["config"]["types"] = [{"heads": t.heads, "ffn": t.ffn, "linear_dtype": t.linear_dtype, "extent_bytes": e}
                                  for t, e in zip(mixed.types, text)]
        out["config"]["block_type"] = list(mixed.block_type)
    line = json.dumps(out)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
