"""Benchmark of the streaming frame-to-cache step on one MI355X.

Workload: one attention layer at the LingBot-Map frame shape -- 1004 tokens per
frame, 16 heads x 64 dims, bf16, scale_frames 8, sliding window 64 frames,
keyframe interval 1 -- streamed frame by frame with frame-correlated Q/K/V.
The first 72 frames fill the cache (8 scale frames attended jointly, then
frame by frame); every later frame is a steady-state step:

    append(frame) -> evict(oldest) -> attend(1004 queries over 72,288 cached tokens)

Untimed: the fill and ``--warmup`` steps.  Timed: exactly ``--steps`` steps,
bracketed by device synchronisation, with nothing recorded between the calls;
the inputs of every timed frame are generated into HBM before the clock
starts.  Then ``--steps`` more steps with HIP events around every call and
its attention kernel give the per-call split (an event record costs the GPU a
few microseconds, so those steps are not the timed ones).  With the defaults
the stream is 322 frames long (72 + 10 + 2 x 120).

Printed: one JSON line (metric frames/s per layer) with the attention kernel's
roofline position (MFMA-bound; algorithmic FLOP = 4*H*D*n_q*N per call) and
the CPU oracle timed on this host as a baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk/CU)
PEAK_HBM_GBS = 8000.0
PEAK_SCLK_MHZ = 2400.0  # the clock the bf16 peak assumes
ATTEND_SOURCE = os.path.join(ROOT, "bounded_kv_cache_stream_amd", "csrc", "attend.hip")
KERNELS_FILE = os.path.join(ROOT, "profiles", "kernels_stream.json")  # written by profile_bench.py


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=120)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--splits", type=int, default=0, help="split-KV partitions (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=["stream", "clces", "append", "long", "budget", "diversity"],
                    default="stream",
                    help="stream: the attention step (default); clces: score_and_compact on the 24-layer "
                         "cache; append: one frame's page write for 24 layers in one launch; long: the "
                         "10,000-frame keyframe-interval-4 stream, sustained; budget: the 24-layer "
                         "token-budget stack (append, attend, score_and_compact per layer); diversity: the "
                         "stack with diversity-scored per-head pruning and softmax layer budgets")
    ap.add_argument("--layers", type=int, default=0, help="diversity workload: layers (default 24)")
    ap.add_argument("--per-head", type=int, default=0,
                    help="diversity workload: mean tokens kept per head and layer (default 128,512)")
    ap.add_argument("--tau", type=float, default=1.0, help="diversity workload: softmax temperature")
    ap.add_argument("--special", type=int, default=0,
                    help="stream / long workloads: special tokens per frame kept across evictions (0 = off)")
    ap.add_argument("--frames", type=int, default=0, help="long workload: frames to run (0 = the full 10,000)")
    ap.add_argument("--merge", action="store_true",
                    help="budget / diversity workloads: merge ragged pages after each compaction / prune")
    ap.add_argument("--defer", action="store_true",
                    help="budget / clces workloads: score_and_compact returns once enqueued (KV_CLCES_DEFER); the next call "
                         "on the layer applies the new page lengths")
    ap.add_argument("--reuse-ranks", action=argparse.BooleanOptionalAction, default=True,
                    help="clces workload: each step ranks only its own layer and reuses the earlier steps' ranks of "
                         "the other window layers, the per-frame rank history of StreamCacheVGGT 2.1.4 "
                         "(KV_CLCES_REUSE_RANKS; every layer holds the same whole frames). Default on; "
                         "--no-reuse-ranks ranks every window layer in every step")
    ap.add_argument("--fused", action="store_true",
                    help="stream/long/budget workloads: one kv_append_attend call per frame and layer (the page "
                         "write shares the "
                         "table-upload launch) instead of append, evict and attend")
    ap.add_argument("--tiling", choices=["auto", "page", "packed"], default="auto",
                    help="KV tiles of the bf16 attention (kv_set_attend_tiling): auto (default), 64-token tiles "
                         "per page, or packed across page ends")
    ap.add_argument("--heads", type=int, default=0,
                    help="stream workload: heads per GPU (default 16; 2 = one GPU's share when 8 GPUs split the heads)")
    ap.add_argument("--sclk", action="store_true",
                    help="stream workload: sample the shader clock with rocm-smi during the timed steps (use "
                         "--steps 20000 or so: one read takes about half a second)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def calib_copy(mib, dev):
    """One device-to-device copy of `mib` MiB: a kernel of known traffic, for the counter calibration."""
    import torch
    if not mib:
        return
    src = torch.empty(mib * (1 << 20), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


class ClockSampler:
    """Samples the GPU's current shader clock (rocm-smi's sclk level, read in a child process) in a thread
    while the timed steps run.  One read takes about half a second, so a timed region of a few seconds is
    needed for a useful median."""

    PATTERN = re.compile(r"sclk clock level: \S+ \((\d+)Mhz\)")

    def __init__(self):
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)

    def _loop(self):
        while not self._stop.is_set():
            try:
                r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=10)
            except (OSError, subprocess.SubprocessError):
                return
            m = self.PATTERN.search(r.stdout)
            if m:
                self.samples.append((time.perf_counter(), int(m.group(1))))
            self._stop.wait(0.05)

    def start(self):
        self._thread.start()

    def stop(self, t0, t1):
        """Stops sampling; the summary of the reads that completed between t0 and t1 (perf_counter)."""
        self._stop.set()
        self._thread.join()
        mhz = sorted(v for t, v in self.samples if t0 <= t <= t1)
        if not mhz:
            return {"median": None, "samples": 0, "note": "no read completed inside the timed steps"}
        return {"median": mhz[len(mhz) // 2], "min": mhz[0], "max": mhz[-1], "samples": len(mhz),
                "source": "rocm-smi current sclk level, read during the timed steps"}


TILINGS = {"auto": 0, "page": 1, "packed": 2}  # KV_TILING_AUTO, KV_TILING_PAGE, KV_TILING_PACKED


def recorded_counters(heads, splits):
    """The attention kernel's HBM bytes and MFMA utilisation per call from the committed rocprofv3 summary
    (profile_bench.py), if it was taken with this attention source at this shape (16 heads, the library's
    split count); else None."""
    try:
        with open(KERNELS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16", {}).get("attend.hip") != source_hash(ATTEND_SOURCE) or heads != 16 or splits:
        return None
    # the kernel is a template (tiles per page or packed): the stream's pages take one instantiation
    k = next((v for n, v in rec.get("kernels", {}).items() if "attend_bf16_kernel" in n), None)
    if not k or "fetch_bytes" not in k or "write_bytes" not in k:
        return None
    return {"traffic": k["fetch_bytes"] + k["write_bytes"], "mfma_util_pct": k.get("mfma_util_pct"),
            "rocprof_kernel_avg_us": k["avg_us"], "summary": os.path.relpath(KERNELS_FILE, ROOT)}


def cpu_baseline(frames_kv, q_frame, attended, min_seconds=10.0, max_frames=6):
    """The fp64 oracle on this host: steady-state frames (all 1004 queries over 72 frames), repeated until
    about `min_seconds` of CPU work (at most `max_frames` frames)."""
    import numpy as np
    from oracle import attention, window
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    sim = window.WindowCache(8, 64, 1, 73)
    for t in range(attended[-1] + 1):  # policy bookkeeping of the whole stream so far
        sim.append(t)
        sim.evict()
        sim.attended()
    n = 0
    while True:
        K = np.concatenate([frames_kv[f][0] for f in attended]).astype(np.float64)
        V = np.concatenate([frames_kv[f][1] for f in attended]).astype(np.float64)
        attention.attend(q_frame.astype(np.float64), K, V, 1.0)
        n += 1
        sec = time.perf_counter() - t0
        if sec >= min_seconds or n >= max_frames:
            break
    return {"value": n / sec, "unit": "frames/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} steady-state frame{'s' if n > 1 else ''}: 1004 queries x {K.shape[0]} cached tokens x 16 heads each, fp64 "
                      f"numpy, plus the window-policy simulation of {attended[-1] + 1} frames ({sec:.1f} s)"}


def moved_tokens(keep_mask_pages):
    """Rows the page compaction moves: with n kept slots in a page, the kept slots at or past n."""
    n = 0
    for m in keep_mask_pages:
        kept = sum(1 for k in m if k)
        n += sum(1 for i in range(kept, len(m)) if m[i])
    return n


def run_clces(args):
    """score_and_compact on 24 layers x 72 frames x 1004 tokens, W=5, lambda=0.5, keep 50%."""
    import numpy as np
    import torch

    from bounded_kv_cache_stream_amd import kvstream as kv
    from bounded_kv_cache_stream_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[3]
    T, H, L, F, K = w["tokens"], w["heads"], w["layers"], w["cache_frames"], w["keep"]
    N = F * T
    cfg = kv.make_config(num_layers=L, num_heads=H, page_tokens=T, scale_frames=0, sliding_window=0,
                         keyframe_interval=1, pages_per_layer=F, max_queries=T, max_splits=8, max_window=5)
    cache = kv.KVCache(cfg, device=dev)
    cache.set_tiling(TILINGS[args.tiling])
    for l in range(L):
        for t in range(F):
            _, k, v = synth.iid_frame(3, l, t, (T, H, 64), device=dev, dtype=torch.bfloat16)
            cache.append(l, t, k, v)
    table = torch.from_numpy(synth.raw_scores(3, N, L)).to(dev)
    keep = torch.empty(K, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    times = []
    returns = []
    moved = 0
    if args.defer:
        # deferred steps back to back on the stream: the 24 calls' stream time over 24 (events), then the
        # keep sets of every layer, read once all steps are done
        keeps = [torch.empty(K, dtype=torch.int32, device=dev) for _ in range(L)]
        stream = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for l in range(L):
            cache.score_and_compact(l, table, w["clces_window"], w["lam"], K, keep_ids=keeps[l], defer=True,
                                    reuse_ranks=args.reuse_ranks)
        e1.record(stream)
        torch.cuda.synchronize()
        cache.sync()
        times = [e0.elapsed_time(e1) / 1e3 / L] * L
        for l in range(L):
            kept = set(keeps[l].cpu().numpy().tolist())
            moved += moved_tokens([[(t * T + j) in kept for j in range(T)] for t in range(F)])
    else:
        for l in range(L):
            t0 = time.perf_counter()
            cache.score_and_compact(l, table, w["clces_window"], w["lam"], K, keep_ids=keep,
                                    reuse_ranks=args.reuse_ranks)
            t1 = time.perf_counter()  # the call returns once the new page lengths are known
            torch.cuda.synchronize()  # the rows have moved
            times.append(time.perf_counter() - t0)
            returns.append(t1 - t0)
            kept = set(keep.cpu().numpy().tolist())
            moved += moved_tokens([[(t * T + j) in kept for j in range(T)] for t in range(F)])
    calib_copy(args.calib_copy_mib, dev)
    times.sort()
    med = times[len(times) // 2]
    bytes_per_layer = moved / L * 2 * H * 64 * 2 * 2  # read + write of K and V rows, bf16
    cpu = None
    if not args.no_cpu_baseline:
        cpu = clces_cpu_baseline(synth.raw_scores(3, N, L), T, F, K, w)
    print(json.dumps({
        "metric": "score_and_compact us per layer (CLCES W=5, lambda=0.5, keep 50%)"
                  + (", deferred: stream time of 24 back-to-back calls / 24" if args.defer else "")
                  + (", ranks of earlier layers reused" if args.reuse_ranks else ", every window layer ranked"),
        "value": med * 1e6,
        "unit": "us", "higher_is_better": False, "n_gpus": 1, "steps": L, "dtype": "fp64 score / bf16 pages",
        "data": "synthetic (seeded chi-square raw scores, iid N(0,1) K/V)",
        "config": {"workload": w["name"], "layers": L, "tokens": N, "keep": K, "window": w["clces_window"],
                   "reuse_ranks": args.reuse_ranks},
        "p90_us": times[int(0.9 * (L - 1))] * 1e6,
        "call_return_us": sorted(returns)[L // 2] * 1e6 if returns else None,
        "moved_tokens_per_layer": moved / L,
        "compaction_bytes_per_layer": bytes_per_layer,
        "rooflines_recorded": clces_rooflines(N, w["clces_window"], L, bytes_per_layer, args.reuse_ranks),
        "cpu_baseline": cpu,
    }), flush=True)


CLCES_SOURCE = os.path.join(ROOT, "bounded_kv_cache_stream_amd", "csrc", "clces.hip")
# written by profile_bench.py: ranks reused (the default), and every window layer ranked in every step
CLCES_KERNELS = {True: os.path.join(ROOT, "profiles", "kernels_clces.json"),
                 False: os.path.join(ROOT, "profiles", "kernels_clces_rerank.json")}


def clces_rooflines(N, W, L, compaction_bytes, reuse):
    """HBM position of the scoring kernels and of the compaction, from the committed rocprofv3 record of this
    workload (per call: every kernel's mean time x its launches per call), if clces.hip still hashes as
    recorded; else None.  Algorithmic bytes of the scoring per call: gather 12 B per key and ranked layer
    + 4 B per token (raw score, id, order key; the current score), fuse 12 B per token, two
    select passes and mark and index 8 B per token each (48 B per token in all), and per key and ranked layer
    the rank method the record shows: block sort + counts (sort: key read, sorted key, index and block rank
    written, 16 B; counts: sorted key and index read once, G = min(8, blocks) count slices written, 8 + 4 G B;
    fuse: 1 + G slices read and the rank written, 4 G + 8 B), 44 + 8 G B; or four radix passes of 20 B (counts
    read, key and value read and written) and the rank read by fuse, 96 B.  A window layer whose ranks are
    reused costs fuse one 4 B rank read per key.  Layer l has min(W, l + 1) window layers; with reuse it ranks
    one of them (its own), else all of them; the bytes are the mean over the L calls.  The record must have
    been taken in the same mode (its command names --reuse-ranks exactly when reuse is on)."""
    try:
        with open(CLCES_KERNELS[bool(reuse)]) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16", {}).get("clces.hip") != source_hash(CLCES_SOURCE):
        return None
    if any("--reuse-ranks" in c.split() for c in rec.get("commands", [])) != bool(reuse):
        return None
    ks = rec.get("kernels", {})
    calls = next((e["used"] for k, e in ks.items() if k.startswith("prep_kernel")), None)
    if not calls:
        return None
    score_us, compact_us = 0.0, 0.0
    for k, e in ks.items():
        per_call = e["avg_us"] * e["used"] / calls
        if "compact_kernel" in k:
            compact_us += per_call
        elif any(k.startswith(n) for n in ("prep_kernel", "gather_kernel", "rank_hist_kernel", "rank_scatter_kernel",
                                             "rank_sort_kernel", "rank_count_kernel", "fuse_kernel",
                                             "select_pass_kernel", "select_finish_kernel", "mark_kernel",
                                             "index_kernel")):
            score_us += per_call
    per_rank = 44 + 8 * min(8, (N + 2047) // 2048) if any(k.startswith("rank_count_kernel") for k in ks) else 96
    n_win = [min(W, l + 1) for l in range(L)]
    n_rank = [1 if reuse else n for n in n_win]
    score_bytes = N * (sum(per_rank * r + 4 * (n - r) for n, r in zip(n_win, n_rank)) / L + 48)
    out = {"source": os.path.relpath(CLCES_KERNELS[bool(reuse)], ROOT)}
    for name, by, us in (("scoring", score_bytes, score_us), ("compaction", compaction_bytes, compact_us)):
        gbs = by / (us * 1e-6) / 1e9 if us else None
        out[name] = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS if gbs else None, "bytes_per_call": by, "kernels_us_per_call": us}
    return out


def clces_cpu_baseline(scores, T, F, K, w):
    """The oracle's CLCES step (ranks, fuse, top-k, page compaction of the token ids) on the host, for the
    last layer (5 window layers); K/V rows are not moved by the oracle, so this times the scoring only."""
    import os as _os

    from oracle import budget
    L = scores.shape[1]
    t0 = time.perf_counter()
    b = budget.BudgetCache(L - 1, T, K, F, window=w["clces_window"], lam=w["lam"])
    for t in range(F):
        b.append(t)
    b.score_and_compact(scores)
    dt = time.perf_counter() - t0
    return {"value": dt * 1e6, "unit": "us", "cores": len(_os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"one layer's CLCES step (N = {F * T}, window 5) in float64 numpy, token ids compacted"}


def run_append(args):
    """kv_append_frame_layers: one 1004-token frame of 24 layers (197.4 MB read + written) per step."""
    import torch

    from bounded_kv_cache_stream_amd import kvstream as kv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, T, H, D = 24, 1004, 16, 64
    cfg = kv.make_config(num_layers=L, num_heads=H, page_tokens=T, scale_frames=0, sliding_window=4,
                         keyframe_interval=1, pages_per_layer=5, max_queries=T, max_splits=4)
    cache = kv.KVCache(cfg, device=dev)
    cache.set_tiling(TILINGS[args.tiling])
    frames = [(torch.randn(L, T, H, D, device=dev).bfloat16(), torch.randn(L, T, H, D, device=dev).bfloat16())
              for _ in range(4)]
    stream = torch.cuda.current_stream(dev)

    def step(t, evp=None):
        k, v = frames[t % 4]
        if evp is not None:
            evp[0].record(stream)
        cache.append_layers(0, t, k, v)
        if evp is not None:
            evp[1].record(stream)
        for l in range(L):
            cache.evict(l)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + i, ev[i])
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2]
    calib_copy(args.calib_copy_mib, dev)
    nbytes = 2 * 2 * L * T * H * D * 2  # K and V, read and written, bf16
    t0 = time.perf_counter()
    for l in range(L):
        cache.evict(l)
    evict_us = (time.perf_counter() - t0) / L * 1e6
    print(json.dumps({
        "metric": "page write GB/s (one 1004-token frame x 24 layers per launch)", "value": nbytes / (med * 1e-3) / 1e9,
        "unit": "GB/s", "higher_is_better": True, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "dtype": "bf16", "data": "synthetic N(0,1)", "config": {"workload": "append_l24_t1004_h16_d64", "layers": L},
        "ms_per_launch_median": med, "bytes_per_launch": nbytes,
        "roofline": {"bound": "hbm", "achieved": nbytes / (med * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "evict_host_us_per_layer": evict_us,
    }), flush=True)


def run_long(args):
    """The 10,000-frame stream with keyframe interval 4: append+evict+attend for every frame, timed whole.

    Inputs come from a ring of 64 AR(1) frames generated in HBM before the clock starts (the values do
    not change the work; the policy, page table and attended set follow the frame index)."""
    import torch

    from bounded_kv_cache_stream_amd import kvstream as kv
    from bounded_kv_cache_stream_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[2]
    T, H, D, S, Wf, k = w["tokens"], w["heads"], w["head_dim"], w["scale_frames"], w["window"], w["keyframe_interval"]
    F = args.frames or w["frames"]
    sp = args.special
    special_pages = (F * sp + (T // max(sp, 1)) * max(sp, 1) - 1) // ((T // max(sp, 1)) * max(sp, 1)) + 1 if sp else 0
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=S, sliding_window=Wf,
                         keyframe_interval=k, pages_per_layer=S + Wf + 1 + special_pages, max_queries=S * T,
                         max_splits=16, special_tokens=sp)
    cache = kv.KVCache(cfg, device=dev)
    cache.set_tiling(TILINGS[args.tiling])
    ar = synth.AR1Stream(2, 0, (T, H, D), device=dev)
    ring = [ar.next() for _ in range(64)]
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    out_scale = torch.empty((S * T, H, D), dtype=torch.bfloat16, device=dev)
    scale_q = [ring[t][0] for t in range(S)]
    q_scale = torch.cat(scale_q)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for t in range(F):
        q, kk, vv = ring[t % 64]
        if args.fused and t >= S - 1:
            if t == S - 1:
                cache.append_attend(0, t, kk, vv, q_scale, 1.0, out=out_scale)
            else:
                cache.append_attend(0, t, kk, vv, q, 1.0, out=out)
            continue
        cache.append(0, t, kk, vv)
        cache.evict(0)
        if t == S - 1:
            cache.attend(0, q_scale, 1.0, out=out_scale)
        elif t >= S:
            cache.attend(0, q, 1.0, out=out)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1)
    info = cache.info(0)
    print(json.dumps({
        "metric": "frames/sec sustained over the keyframe-interval-4 stream (append+evict+attend, 1 layer)"
                  + (", one fused call per frame" if args.fused else ""),
        "value": F / (ms / 1e3), "unit": "frames/s", "higher_is_better": True, "n_gpus": 1, "frames": F,
        "ms_per_frame": ms / F, "dtype": "bf16", "data": "synthetic (ring of 64 seeded AR(1) frames, bf16)",
        "config": {"workload": w["name"].replace("_h16_", f"_h{H}_") + (f"_sp{sp}" if sp else ""),
                   "tokens_per_frame": T, "heads": H, "head_dim": D, "scale_frames": S,
                   "sliding_window": Wf, "keyframe_interval": k, "special_tokens": sp, "fused": args.fused},
        "final_persisted_frames": info["persisted_frames"], "final_special_tokens": info["special_tokens"],
        "wall_s": wall}), flush=True)


def run_budget(args):
    """The 24-layer token-budget stack: per frame and layer append -> attend -> score_and_compact.

    Frames 0..warmup-1 fill the cache (the budget of 128,512 tokens is reached at frame 128); the next
    `steps` frames are timed with nothing recorded between the calls, and `steps` more carry HIP events
    around each call for the per-call split.  K/V/Q come
    from a ring of 8 AR(1) frames per layer in HBM; the raw-score table covers every token id."""
    import numpy as np
    import torch

    from bounded_kv_cache_stream_amd import kvstream as kv
    from bounded_kv_cache_stream_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[4]
    T, H, D, L, B = w["tokens"], w["heads"], w["head_dim"], w["layers"], w["budget"]
    warm = max(args.warmup, 140)
    F = warm + 2 * args.steps  # the timed frames, then as many with events for the per-call split
    cfg = kv.make_config(num_layers=L, num_heads=H, page_tokens=T, scale_frames=0, sliding_window=0,
                         keyframe_interval=1, pages_per_layer=F, max_queries=T, max_splits=16,
                         max_window=w["clces_window"])
    cache = kv.KVCache(cfg, device=dev)
    cache.set_tiling(TILINGS[args.tiling])
    table = torch.from_numpy(synth.raw_scores(4, F * T, L)).to(dev)
    rings = []
    for l in range(L):
        ar = synth.AR1Stream(4, l, (T, H, D), device=dev)
        rings.append([ar.next() for _ in range(8)])
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = {name: [] for name in ("append", "attend", "score", "merge")}

    def frame(t, timed):
        for l in range(L):
            q, k, v = rings[l][t % 8]
            marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if timed else None
            if timed:
                marks[0].record(stream)
            if args.fused:
                # one call: the page write shares the table-upload launch
                if timed:
                    marks[1].record(stream)
                cache.append_attend(l, t, k, v, q, w["sm_scale"], out=out)
            else:
                cache.append(l, t, k, v)
                if timed:
                    marks[1].record(stream)
                cache.attend(l, q, w["sm_scale"], out=out)
            if timed:
                marks[2].record(stream)
            cache.score_and_compact(l, table, w["clces_window"], w["lam"], B, defer=args.defer)
            if timed:
                marks[3].record(stream)
            if args.merge:
                cache.merge_pages(l)
            if timed:
                marks[4].record(stream)
                ev["append"].append((marks[0], marks[1]))
                ev["attend"].append((marks[1], marks[2]))
                ev["score"].append((marks[2], marks[3]))
                ev["merge"].append((marks[3], marks[4]))

    for t in range(warm):
        frame(t, False)
    torch.cuda.synchronize()
    n_tok = cache.info(0)["tokens"]
    wall0 = time.perf_counter()
    for t in range(warm, warm + args.steps):
        frame(t, False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for t in range(warm + args.steps, F):
        frame(t, True)
    torch.cuda.synchronize()
    split = {name: float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e3 for name, pairs in ev.items()}
    attended = n_tok + T
    flops = 4.0 * H * D * T * attended
    pages = [cache.info(l)["persisted_frames"] for l in range(L)]
    ids, lens, _ = cache.page_table(L - 1)
    tiles = (sum(lens) + T + 63) // 64  # the attention packs the tokens into 64-token tiles across page ends
    print(json.dumps({
        "metric": "frames/sec of the 24-layer token-budget stack (append, attend, score_and_compact"
                  + (" deferred" if args.defer else "") + (", merge_pages" if args.merge else "")
                  + (", append + attend in one kv_append_attend call" if args.fused else "") + " per layer)",
        "value": args.steps / wall, "unit": "frames/s", "higher_is_better": True, "n_gpus": 1, "steps": args.steps,
        "warmup": warm, "ms_per_frame": wall / args.steps * 1e3, "dtype": "bf16",
        "data": "synthetic (ring of 8 seeded AR(1) frames per layer, chi-square raw scores)",
        "config": {"workload": w["name"], "layers": L, "tokens_per_frame": T, "heads": H, "head_dim": D,
                   "budget": B, "attended_tokens": attended, "clces_window": w["clces_window"], "lam": w["lam"]},
        "page_merge": bool(args.merge), "pages_per_layer_mean": float(np.mean(pages)),
        "attend_tiles_layer23": tiles, "attend_tile_fill": attended / (64.0 * tiles),
        "us_per_layer": split,
        "attend_tflops": flops / (split["attend"] * 1e-6) / 1e12,
        "attend_frac_bf16_peak": flops / (split["attend"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}), flush=True)


def run_diversity(args):
    """The diversity-pruned stack: per frame, append the frame to every layer (one launch), score every
    layer (its mean diversity), split the total budget over the layers with the tempered softmax, prune
    every layer to its per-head top-K, then attend every layer over the pages each head kept.

    Frame 0 is the anchor (scale_frames = 1).  The total budget is layers x heads x per_head tokens; the
    untimed frames run until every layer has pruned at least 8 times.  K/V/Q come from a ring of 8 AR(1)
    frames per layer in HBM.  The `steps` timed frames record nothing between the phases; `steps` more
    frames carry HIP events around each phase for the split.  The batched scoring and prune each wait once
    for all layers (they read back the means, the new lengths and the error flags); the prune reuses the
    keys of the scoring."""
    import numpy as np
    import torch

    from bounded_kv_cache_stream_amd import kvstream as kv
    from bounded_kv_cache_stream_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, per_head, tau = args.layers or 24, args.per_head or 128512, args.tau
    T, H, D = synth.TOKENS_PER_FRAME, 16, 64
    total = L * H * per_head
    warm = max(args.warmup, 2 * ((per_head + T - 1) // T) + 9)
    F = warm + 2 * args.steps  # the timed frames, then as many with events for the phase split
    cfg = kv.make_config(num_layers=L, num_heads=H, page_tokens=T, scale_frames=1, sliding_window=0,
                         keyframe_interval=1, pages_per_layer=F, max_queries=T, max_splits=16)
    cache = kv.KVCache(cfg, device=dev)
    cache.set_tiling(TILINGS[args.tiling])
    rings_q, rings_k, rings_v = [], [], []
    ars = [synth.AR1Stream(5, l, (T, H, D), device=dev) for l in range(L)]
    for i in range(8):
        fr = [a.next() for a in ars]
        rings_q.append([f[0] for f in fr])
        rings_k.append(torch.stack([f[1] for f in fr]).contiguous())
        rings_v.append(torch.stack([f[2] for f in fr]).contiguous())
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    cand = np.zeros((L, H), dtype=np.int64)  # candidates per head after the frame's append
    kept = np.zeros((L, H), dtype=np.int64)
    log = {"score": [], "prune": [], "merge": [], "attend": [], "append": [], "cand": [], "kept": [],
           "budgets": []}

    def frame(t, timed):
        # timed: HIP events between the phases, for the split
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(6)] if timed else None
        rec = (lambda i: marks[i].record(stream)) if timed else (lambda i: None)  # noqa: E731
        rec(0)
        cache.append_layers(0, t, rings_k[t % 8], rings_v[t % 8])
        rec(1)
        cand[:] = kept + (T if t > 0 else 0)
        means = cache.diversity_score_layers(0, L)
        rec(2)
        budgets = kv.kv_layer_budgets(means, tau, total, H)
        cache.diversity_prune_layers(0, budgets, out=kept)
        rec(3)
        if args.merge:
            cache.merge_pages_layers(0, L)
        rec(4)
        for l in range(L):
            cache.attend(l, rings_q[t % 8][l], 1.0, out=out)
        rec(5)
        if timed:
            log["append"].append((marks[0], marks[1]))
            log["score"].append((marks[1], marks[2]))
            log["prune"].append((marks[2], marks[3]))
            log["merge"].append((marks[3], marks[4]))
            log["attend"].append((marks[4], marks[5]))
            log["cand"].append(cand.copy())
            log["kept"].append(kept.copy())
            log["budgets"].append(budgets)

    for t in range(warm):
        frame(t, False)
    torch.cuda.synchronize()
    assert min(cache.info(l)["prunes"] for l in range(L)) >= 8, "the untimed frames must reach every budget"
    wall0 = time.perf_counter()
    for t in range(warm, warm + args.steps):
        frame(t, False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for t in range(warm + args.steps, F):
        frame(t, True)
    torch.cuda.synchronize()
    split = {k: float(np.mean([a.elapsed_time(b) for a, b in log[k]])) * 1e3
             for k in ("append", "score", "prune", "merge", "attend")}
    cand_rows = float(np.mean([c.sum() for c in log["cand"]]))  # candidate rows (head x token) per frame
    kept_rows = float(np.mean([k.sum() for k in log["kept"]]))
    score_bytes = 2.0 * cand_rows * D * 2  # two passes over every candidate key row, bf16
    attn_flops = float(np.mean([4.0 * D * T * (k.sum() + L * H * T) for k in log["kept"]]))
    pages = [cache.info(l)["persisted_frames"] for l in range(L)]
    hl = np.array(cache.head_lengths(L // 2))
    tiles = (hl.sum(axis=0) + 63) // 64  # per head: tokens packed into 64-token tiles across page ends
    result = {
        "metric": f"frames/sec of the {L}-layer diversity-pruned stack (append, score, budgets, prune, "
                  + ("page merge, " if args.merge else "") + "attend)",
        "value": args.steps / wall, "unit": "frames/s", "higher_is_better": True, "n_gpus": 1,
        "steps": args.steps, "warmup": warm, "ms_per_frame": wall / args.steps * 1e3, "dtype": "bf16",
        "data": "synthetic (ring of 8 seeded AR(1) frames per layer)",
        "config": {"workload": f"diversity_l{L}_h{H}_d{D}_t{T}_k{per_head}_tau{tau:g}"
                               + ("_merge" if args.merge else ""), "layers": L,
                   "tokens_per_frame": T, "heads": H, "head_dim": D, "per_head_budget_mean": per_head,
                   "total_budget": total, "tau": tau, "anchor_frames": 1},
        "us_per_frame": split,
        "candidates_per_frame": cand_rows, "kept_per_frame": kept_rows,
        "budget_spread": [int(min(log["budgets"][-1])), int(max(log["budgets"][-1]))],
        "pages_per_layer_mean": float(np.mean(pages)),
        "merges_per_layer_mean": float(np.mean([cache.info(l)["merges"] for l in range(L)])),
        "attend_tile_fill_mid_layer": float(hl.sum(axis=0).mean() / (64.0 * tiles.mean())),
        "roofline": {"bound": "hbm", "achieved": score_bytes / (split["score"] * 1e-6) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": score_bytes / (split["score"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
                     "traffic": None, "kernel": "kv_diversity_score_layers (div_sum + div_score per layer, two "
                                                "reads of every candidate key; includes the small kernels "
                                                "and the one read-back)",
                     "bytes_per_frame": score_bytes},
        "attend_tflops": attn_flops / (split["attend"] * 1e-6) / 1e12,
        "attend_frac_bf16_peak": attn_flops / (split["attend"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = diversity_cpu_baseline(L, T, H, per_head)
    print(json.dumps(result), flush=True)


def diversity_cpu_baseline(L, T, H, per_head):
    """The oracle's diversity step for one layer (scores of every candidate of every head in float64, the
    per-head top-K and the per-page, per-head compaction of the token ids) at the state where the
    candidates first exceed the budget: the anchor plus ceil(per_head / T) + 1 frames."""
    import os as _os

    import numpy as np

    from oracle import diversity
    n_frames = (per_head + T - 1) // T + 2
    rng = np.random.default_rng(5)
    keys = {f: rng.standard_normal((T, H, 64)).astype(np.float32) for f in range(n_frames)}
    c = diversity.DiversityCache(H, T, n_frames)
    for f in range(n_frames):
        c.append(f)
    t0 = time.perf_counter()
    c.prune(lambda f, h: keys[f][:, h, :], per_head)
    dt = time.perf_counter() - t0
    return {"value": 1.0 / (L * dt), "unit": "frames/s", "cores": len(_os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"one layer's score + top-K + compaction ({H} heads x {(n_frames - 1) * T} candidates, "
                      f"{dt:.1f} s), scaled to {L} layers; attention and page writes not included"}


def main():
    args = parse()
    if args.workload == "clces":
        return run_clces(args)
    if args.workload == "append":
        return run_append(args)
    if args.workload == "long":
        return run_long(args)
    if args.workload == "budget":
        return run_budget(args)
    if args.workload == "diversity":
        return run_diversity(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the path shards by head across GPUs "
                                   "without any exchange (attention, page writes and compaction are per head); there is no multi-GPU mode",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from bounded_kv_cache_stream_amd import kvstream as kv
    from bounded_kv_cache_stream_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[1]
    T, H, D = w["tokens"], args.heads or w["heads"], w["head_dim"]
    S, Wf = w["scale_frames"], w["window"]
    sp = args.special
    cfg = kv.make_config(num_layers=1, num_heads=H, page_tokens=T, scale_frames=S, sliding_window=Wf,
                         keyframe_interval=1, pages_per_layer=S + Wf + 1 + (8 if sp else 0), max_queries=S * T,
                         max_splits=64, special_tokens=sp)
    cache = kv.KVCache(cfg, device=dev)
    cache.set_tiling(TILINGS[args.tiling])
    if args.splits:
        cache.set_splits(args.splits)
    ar = synth.AR1Stream(1, 0, (T, H, D), device=dev)
    fill = S + Wf  # frames 0..71 fill the cache; from frame 71 on the cache holds 72 frames
    # warmup, then the timed steps (no per-step events), then as many steps again with events for the
    # per-call and kernel-only split
    total = fill + args.warmup + 2 * args.steps

    # generate every frame's inputs into HBM first
    frames = [ar.next() for _ in range(total)]
    torch.cuda.synchronize()

    out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    out_scale = torch.empty((S * T, H, D), dtype=torch.bfloat16, device=dev)
    scale_q = []
    for t in range(fill):
        q, k, v = frames[t]
        cache.append(0, t, k, v)
        cache.evict(0)
        if t < S:
            scale_q.append(q)
            if t == S - 1:
                cache.attend(0, torch.cat(scale_q), 1.0, out=out_scale)
        else:
            cache.attend(0, q, 1.0, out=out)
    assert cache.info(0)["persisted_frames"] == S + Wf

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(t, evp=None):
        q, k, v = frames[t]
        if args.fused:  # the events bracket the whole call: page write with the table upload, attention
            if evp is not None:
                evp[0].record(stream)
            cache.append_attend(0, t, k, v, q, 1.0, out=out)
            if evp is not None:
                evp[1].record(stream)
            return
        cache.append(0, t, k, v)
        cache.evict(0)
        if evp is not None:
            evp[0].record(stream)
        cache.attend(0, q, 1.0, out=out)
        if evp is not None:
            evp[1].record(stream)

    for i in range(args.warmup):
        step(fill + i)
    torch.cuda.synchronize()
    # timed steps: nothing recorded between the calls (an event record costs the GPU a few microseconds)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    sampler = ClockSampler() if args.sclk else None
    if sampler:
        sampler.start()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(fill + args.warmup + i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    sclk = sampler.stop(wall0, wall0 + wall) if sampler else None
    ms_total = t_start.elapsed_time(t_end)
    # the split: the same number of steps again, with events around each call and (recorded by the
    # library on the call's stream) around its attention kernel
    kv.kv_attend_timing(cache.handle, args.steps)
    s_start = torch.cuda.Event(enable_timing=True)
    s_end = torch.cuda.Event(enable_timing=True)
    s_start.record(stream)
    for i in range(args.steps):
        step(fill + args.warmup + args.steps + i, ev[i])
    s_end.record(stream)
    torch.cuda.synchronize()
    ms_instrumented = s_start.elapsed_time(s_end)
    info = cache.info(0)
    assert info["persisted_frames"] == S + Wf and info["tokens"] == (S + Wf) * T + info["special_tokens"]

    attend_ms = [a.elapsed_time(b) for a, b in ev]
    attend_avg_s = sum(attend_ms) / len(attend_ms) / 1e3
    attend_sorted = sorted(attend_ms)
    # every timed step evicts one frame (keyframe interval 1), so the special tokens attended grow by `sp`
    # per step: the mean over the timed steps is the last count less sp * (steps - 1) / 2
    n_keys = (S + Wf) * T + info["special_tokens"] - sp * (args.steps - 1) / 2.0
    flops = 4.0 * H * D * T * n_keys
    kern_ms, kern_n = kv.kv_attend_timing_read(cache.handle)
    kv.kv_attend_timing(cache.handle, 0)
    assert kern_n == args.steps
    kernel_avg_s = kern_ms / kern_n / 1e3
    achieved = flops / kernel_avg_s / 1e12
    achieved_call = flops / attend_avg_s / 1e12

    calib_copy(args.calib_copy_mib, dev)

    result = {
        "metric": "frames/sec per layer at 1004 tok/frame, 72-frame cache; % bf16 MFMA peak",
        "value": args.steps / (ms_total / 1e3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_total / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded AR(1) frame-correlated Q/K/V, bf16)",
        "config": {"workload": re.sub(r"_f\d+$", f"_f{total}", w["name"].replace("_h16_", f"_h{H}_"))
                               + (f"_sp{sp}" if sp else ""),
                   "tokens_per_frame": T, "heads": H, "head_dim": D, "special_tokens": sp,
                   "cache_frames": S + Wf, "cached_tokens": n_keys, "scale_frames": S, "sliding_window": Wf,
                   "keyframe_interval": 1,
                   "step": "append+evict+attend" + (" in one kv_append_attend call" if args.fused else ""),
                   "layers": 1,
                   "stream_frames": total},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": None,
                     "kernel": "attend_bf16_kernel (HIP events around the kernel alone, recorded by the library on "
                               "the call's stream)",
                     "kernel_avg_us": kernel_avg_s * 1e6,
                     "call": "kv_append_attend (page write with the table upload, attend_bf16_kernel, split-KV "
                             "combine)" if args.fused else "stream_attend (attend_bf16_kernel with the page table in its "
                                                           "arguments, split-KV combine)",
                     "achieved_call": achieved_call, "frac_call": achieved_call / PEAK_BF16_TFLOPS,
                     "avg_call_us": attend_avg_s * 1e6, "flop_per_call": flops,
                     "median_call_us": attend_sorted[len(attend_sorted) // 2] * 1e3,
                     "p90_call_us": attend_sorted[int(0.9 * (len(attend_sorted) - 1))] * 1e3},
        "wall_s_timed": wall,
        "ms_per_step_instrumented": ms_instrumented / args.steps,
    }
    rc = None if sp else recorded_counters(H, args.splits)
    if rc is not None:
        result["roofline"]["traffic"] = rc["traffic"]
        result["roofline"]["mfma_util_pct_counters"] = rc["mfma_util_pct"]
        result["roofline"]["rocprof_kernel_avg_us"] = rc["rocprof_kernel_avg_us"]
        result["roofline"]["counters"] = rc["summary"]
    if sclk is not None:
        result["sclk_mhz"] = sclk
        if sclk["median"]:
            # the same kernel against the bf16 peak at the clock it ran at
            clk_peak = PEAK_BF16_TFLOPS * sclk["median"] / PEAK_SCLK_MHZ
            result["roofline"]["peak_at_measured_sclk"] = clk_peak
            result["roofline"]["frac_at_measured_sclk"] = achieved / clk_peak
    if not args.no_cpu_baseline:
        last = fill + args.warmup + 2 * args.steps - 1
        attended = list(range(S)) + list(range(last - Wf + 1, last + 1))
        frames_kv = {f: (frames[f][1].float().cpu().numpy(), frames[f][2].float().cpu().numpy()) for f in attended}
        result["cpu_baseline"] = cpu_baseline(frames_kv, frames[last][0].float().cpu().numpy(), attended)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
