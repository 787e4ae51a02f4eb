"""Benchmark: indexed rANS64 encode + decode of the 1080p y latent on one MI355X.

One step is the whole coding path on one batch: table preparation + encode
and table preparation + decode (rans_prepare_tables followed by
rans_encode_prepared / rans_decode_prepared, exactly the launches that
rans_encode_with_indexes / rans_decode_with_indexes make, called separately
so that HIP events can bracket each coding kernel alone) of 1,566,720 int32 symbols (192x68x120) with 64
Gaussian 16-bit CDF rows at 4096 lanes -- the y latent of a 1920x1088 image
in a mean-scale hyperprior (kompressor README, "Getting Started").  Inputs are
synthetic, seeded, and resident in HBM before timing.  Before timing, the GPU
decode of the GPU container must give the input back; the CPU-baseline leg
runs the oracle on the same workload and checks the GPU container against
the oracle's byte for byte.

The line also reports:
- encode and decode calls of the interleaved-stream container
  (rans_encode_interleaved / rans_decode_interleaved: 64 states per stream;
  by default as many states as lanes, at most 4096 streams, else --streams),
  both as full calls and as *_prepared calls on tables prepared once;
- the decode call of the same lane container cut into 4 pieces per lane by
  split records (rans_decode_with_splits, the records written by
  rans_encode_with_splits beside the unchanged container);
- the device table builder on the workload's own table set (64 discretised
  Gaussians, scales log-spaced over 0.11..256, stride 3133), whose output
  must equal the workload's tables;
- "batch": the lane coding kernels on the batch workloads (16 1080p y
  latents at 65,536 lanes; 8 4K y latents at 1,024, 16,384 and 131,072
  lanes), the interleaved calls at 4096 streams, and the front end fused
  into the interleaved encoder, each container checked against the
  oracle's in the CPU-baseline leg (skip with --no-batch).

value = symbols per step / step time (a step encodes and decodes every
symbol once).  The roofline object reports the slower of the two coding
kernels: algorithmic bytes per launch (8 B per symbol of int32 symbols and
indexes plus the 4-byte container words) over its mean duration from HIP
events recorded around that kernel on the launch stream, on every 8th step
of the timed loop (every step when there are fewer than 128).
"""
from __future__ import annotations

import argparse
import concurrent.futures
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "rANS encode/decode Gsymbol/s on 1080p y-latent (1.57M syms); % of HBM roofline"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
SPLIT_PIECES = 4   # pieces per lane for the split-record decode figure
EVENT_EVERY = 8    # timed steps per sampled step with per-kernel HIP events (at most)
# The pages' own figure for this metric on the 1080p y latent: kompressor
# (CompressAI's rANS64 format, 24 CPU chunks) encodes the 1,566,720 symbols
# in 2.496 ms and decodes them in 2.114 ms (kompressor README, "Getting
# Started", the example run's output), i.e. 0.340 Gsym/s for encode plus
# decode.  Another machine and the real latent: context for vs_baseline,
# not a target.
PAGE_BASELINE = {"y1080": {"value": round(1_566_720 / (2.496e-3 + 2.114e-3) / 1e9, 4),
                           "source": "kompressor, 24 CPU chunks, encode 2.496 ms + decode "
                                     "2.114 ms on a real 1080p y latent of the same shape "
                                     "(kompressor README, \"Getting Started\")"}}

DEFAULT_LANES = {"tiny": 64, "z": 256, "y1080": 4096, "y1080x16": 65536, "y4kx8": 131072}
DESCRIPTION = {
    "tiny": "16,384 int32 symbols, 8 Gaussian CDF rows, 1% bypass",
    "z": "z latent 192x17x30, 192 logistic CDF rows",
    "y1080": "1080p y latent 192x68x120 = 1,566,720 int32 symbols, 64 Gaussian 16-bit CDF rows, "
             "0.1% bypass",
    "y1080x16": "16 x 1080p y latents = 25,067,520 symbols, 64 Gaussian CDF rows",
    "y4kx8": "8 x 4K y latents 192x136x240 = 50,135,040 symbols, skewed scales, 0.5% bypass",
}


def measured_traffic(kernel: str, config: str, lanes: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if current."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{config}_L{lanes}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    from learned_image_compression_amd.profiling import kernel_source_hash
    if t.get("source_hash") != kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


def table_set():
    """The workloads' Gaussian table set: 64 scales log-spaced over 0.11..256 and
    the standard-normal quantile of 1 - 5e-10 (two-sided tail mass 1e-9)."""
    import numpy as np
    from scipy.special import ndtri
    lo, hi, K = 0.11, 256.0, 64
    scales = np.exp(np.log(lo) + (np.log(hi) - np.log(lo)) * np.arange(K) / (K - 1))
    tail_z = float(ndtri(1.0 - 5e-10))
    return scales, tail_z, 2 * int(np.ceil(hi * tail_z)) + 3   # longest row: 3133


def cpu_model_name() -> str:
    """The host CPU's full model line: lscpu's "Model name", else /proc/cpuinfo's
    longest "model name" (some virtual machines shorten one of them)."""
    names = []
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        names += [l.split(":", 1)[1].strip() for l in out.splitlines()
                  if l.strip().lower().startswith("model name")]
    except (OSError, subprocess.SubprocessError):
        pass
    ids = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for l in fh:
                key, _, val = l.partition(":")
                key = key.strip()
                if key == "model name":
                    names.append(val.strip())
                elif key in ("cpu family", "model", "stepping") and key not in ids:
                    ids[key] = val.strip()
    except OSError:
        pass
    name = max(names, key=len) if names else ""
    # a shortened name ("AMD EPYC") still tells the part apart with its CPUID
    # family, model and stepping
    if ids:
        name += " (" + ", ".join(f"{k} {v}" for k, v in ids.items()) + ")"
    return name


def lane_groups(n: int, lanes: int, groups: int):
    """Split lanes 0 .. lanes-1 into `groups` contiguous groups; returns per group
    (first symbol, end symbol, lanes) with the lane partition's symbol bounds
    (lane j starts at floor(j * n / lanes))."""
    bounds = [(g * lanes // groups, (g + 1) * lanes // groups) for g in range(groups)]
    return [(j0 * n // lanes, j1 * n // lanes, j1 - j0) for j0, j1 in bounds]


def cpu_baseline(w, lanes, gpu_words, gpu_tables, min_seconds=10.0, max_reps=200, split=None,
                 interleaved=None):
    """The oracle as it stands on the full workload: one thread, repeated ~10 s,
    then fanned out over host threads by lane groups, repeated ~5 s.  Its
    container, split records, interleaved container and table set must equal
    the GPU's."""
    import numpy as np
    import oracle
    # single thread, pinned to one core of this process's affinity set (the
    # mask is set on the running process itself, and restored afterwards)
    affinity = sorted(os.sched_getaffinity(0))
    pinned = affinity[0]
    os.sched_setaffinity(0, {pinned})
    try:
        times = []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            rc, words = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes)
            rc2, out = oracle.decode(words, w.indexes, w.cdf, w.lengths, w.offsets, lanes)
            times.append(time.perf_counter() - t0)
            assert rc == 0 and rc2 == 0
            if (time.perf_counter() - t_start >= min_seconds and len(times) >= 3) or \
                    len(times) >= max_reps:
                break
    finally:
        os.sched_setaffinity(0, set(affinity))
    assert words.size == gpu_words.size and np.array_equal(words, gpu_words), \
        "GPU container differs from the oracle's"
    assert np.array_equal(out, w.symbols)
    scales, tail_z, tstride = table_set()
    t0 = time.perf_counter()
    rc, cdf, lengths, offsets = oracle.gaussian_tables(scales, tail_z, tstride)
    table_us = (time.perf_counter() - t0) * 1e6
    assert rc == 0 and all(np.array_equal(a, b) for a, b in zip((cdf, lengths, offsets), gpu_tables)), \
        "GPU table set differs from the oracle's"
    if split is not None:
        pieces, records = split
        rc, _, ometa = oracle.encode_split(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes,
                                           pieces)
        assert rc == 0 and np.array_equal(ometa.reshape(-1), records), \
            "GPU split records differ from the oracle's"
    if interleaved is not None:
        streams, words = interleaved
        rc, owords = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets,
                                               streams, 64)
        assert rc == 0 and np.array_equal(owords, words), \
            "GPU interleaved container differs from the oracle's"
    med = statistics.median(times)
    # The same oracle calls fanned out over host threads: thread g encodes and
    # decodes a contiguous group of lanes (their symbols, as a container of
    # its own).  The oracle is a C library called through ctypes, which
    # releases the interpreter lock for the call, so the threads run at once.
    # one thread per core of the affinity set, at most the 16 cores that one
    # GPU's share of the host holds
    nproc = len(affinity)
    threads = max(1, min(16, nproc, lanes))
    spans = lane_groups(w.n, lanes, threads)

    def group(span):
        b, e, lg = span
        rc, gw = oracle.encode(w.symbols[b:e], w.indexes[b:e], w.cdf, w.lengths, w.offsets, lg)
        rc2, go = oracle.decode(gw, w.indexes[b:e], w.cdf, w.lengths, w.offsets, lg)
        return rc == 0 and rc2 == 0 and np.array_equal(go, w.symbols[b:e])

    ttimes = []
    with concurrent.futures.ThreadPoolExecutor(threads) as pool:
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            assert all(pool.map(group, spans)), "threaded oracle round trip failed"
            ttimes.append(time.perf_counter() - t0)
            if (time.perf_counter() - t_start >= min_seconds / 2 and len(ttimes) >= 3) or \
                    len(ttimes) >= max_reps:
                break
    tmed = statistics.median(ttimes)
    model = cpu_model_name()
    return {
        "value": round(w.n / tmed / 1e9, 5),
        "unit": "Gsymbol/s",
        "cores": threads,
        "nproc": nproc,
        "kind": "oracle",
        "sample": f"whole {w.name} workload ({w.n} symbols, {lanes} lanes), encode+decode, "
                  f"the lanes split into {threads} contiguous groups run on {threads} threads "
                  f"(one oracle encode and decode per group), median of {len(ttimes)} "
                  f"repetitions ({sum(ttimes):.1f} s); {tmed / w.n * 1e9:.2f} ns/symbol",
        "cpu_model": model,
        "single_thread": {"value": round(w.n / med / 1e9, 5), "ns_per_symbol": round(med / w.n * 1e9, 2),
                          "pinned_cpu": pinned,
                          "sample": f"the whole workload in one oracle call each way on one "
                                    f"pinned core, median of {len(times)} repetitions "
                                    f"({sum(times):.1f} s)"},
        "table_build_us": round(table_us, 1),
        "parity": "GPU container, split records, interleaved container and table set equal "
                  "the oracle's",
    }


# Batch configurations reported beside the headline (the 16-latent batch at
# its lane count, the 4K batch at each of its three), and the interleaved
# stream count used for them.
BATCH_POINTS = (("y1080x16", 65536), ("y4kx8", 1024), ("y4kx8", 16384), ("y4kx8", 131072))
BATCH_STREAMS = 4096


def _median_us(fn, reps):
    """Median duration of fn() bracketed by HIP events on the current stream."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps + 2)]
    for a, b in ev:
        a.record()
        if fn():
            raise RuntimeError("launch failed")
        b.record()
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in ev[2:]) * 1e3


def batch_point(cfg: str, lanes: int, streams: int, check_oracle: bool, reps: int = 10):
    """One batch configuration: the lane coding kernels (the *_prepared calls, as
    in the timed step) and the interleaved calls on tables prepared once, plus
    the front end fused into the interleaved encoder, fed a latent built so
    that it yields exactly the workload's symbols and indexes (y = symbol,
    mean = 0, scale = the table's scale of the index, a strictly increasing
    table).  Every container is compared with the one before it and, with
    check_oracle, with the oracle's."""
    import ctypes
    import numpy as np
    import torch
    import oracle
    import workloads
    from learned_image_compression_amd import binding as B
    lib, vp, dev = B.load(), ctypes.c_void_p, torch.device("cuda:0")
    w = workloads.load(cfg)
    n = w.n
    tables = B.Tables.from_numpy(w.cdf, w.lengths, w.offsets, dev)
    K, stride = tables.num_tables, tables.stride
    sym = torch.from_numpy(w.symbols).to(dev)
    idx = torch.from_numpy(w.indexes).to(dev)
    hs = vp(torch.cuda.current_stream(dev).cuda_stream)
    cap = B.encode_bound_words(n, lanes)
    stream = torch.empty(cap, dtype=torch.int32, device=dev)
    nw = torch.zeros(1, dtype=torch.int64, device=dev)
    st = torch.zeros(2, dtype=torch.int32, device=dev)
    out = torch.empty(n, dtype=torch.int32, device=dev)
    ws = torch.zeros(B.workspace_bytes(n, lanes, K, stride), dtype=torch.uint8, device=dev)
    B.prepare_tables(tables, ws)
    enc = lambda: lib.rans_encode_prepared(vp(sym.data_ptr()), vp(idx.data_ptr()), n, K, stride,
                                           lanes, vp(stream.data_ptr()), cap, vp(nw.data_ptr()),
                                           vp(st.data_ptr()), vp(ws.data_ptr()), ws.numel(), hs)
    dec = lambda: lib.rans_decode_prepared(vp(stream.data_ptr()), cap, vp(idx.data_ptr()), n, K,
                                           stride, vp(out.data_ptr()), vp(st.data_ptr() + 4),
                                           vp(ws.data_ptr()), ws.numel(), hs)
    enc_us, dec_us = _median_us(enc, reps), _median_us(dec, reps)
    B.check(st[:1], f"{cfg} encode")
    B.check(st[1:], f"{cfg} decode")
    words = int(nw.item())
    assert torch.equal(out.cpu(), torch.from_numpy(w.symbols)), f"{cfg}: decode != input"
    lane_words = stream[:words].cpu().numpy().view(np.uint32).copy()
    del ws
    # interleaved container, plain and fused encode, on tables prepared once
    S = streams
    il_cap = int(lib.rans_interleaved_bound_words(n, S))
    il_ws = torch.zeros(int(lib.rans_interleaved_workspace_bytes(n, S, K, stride)),
                        dtype=torch.uint8, device=dev)
    B.prepare_tables(tables, il_ws)
    il_stream = torch.empty(il_cap, dtype=torch.int32, device=dev)
    il_enc = lambda: lib.rans_encode_interleaved_prepared(
        vp(sym.data_ptr()), vp(idx.data_ptr()), n, K, stride, S, vp(il_stream.data_ptr()), il_cap,
        vp(nw.data_ptr()), vp(st.data_ptr()), vp(il_ws.data_ptr()), il_ws.numel(), hs)
    il_dec = lambda: lib.rans_decode_interleaved_prepared(
        vp(il_stream.data_ptr()), il_cap, vp(idx.data_ptr()), n, K, stride, S,
        vp(out.data_ptr()), vp(st.data_ptr() + 4), vp(il_ws.data_ptr()), il_ws.numel(), hs)
    il_enc_us = _median_us(il_enc, reps)
    B.check(st[:1], f"{cfg} interleaved encode")
    il_words = int(nw.item())
    il_host = il_stream[:il_words].cpu().numpy().view(np.uint32).copy()
    out.zero_()
    il_dec_us = _median_us(il_dec, reps)
    B.check(st[1:], f"{cfg} interleaved decode")
    assert torch.equal(out.cpu(), torch.from_numpy(w.symbols)), f"{cfg}: interleaved decode != input"
    fused = None
    if int(np.abs(w.symbols).max(initial=0)) <= (1 << 24):
        table = (table_set()[0] if K == 64 else np.arange(1, K + 1)).astype(np.float32)
        assert np.all(np.diff(table) > 0)
        y = sym.to(torch.float32)
        mean = torch.zeros_like(y)
        scale = torch.from_numpy(table).to(dev)[idx.long()]
        d_table = torch.from_numpy(table).to(dev)
        il_stream.zero_()
        fz = lambda: lib.rans_encode_interleaved_latent_prepared(
            vp(y.data_ptr()), vp(mean.data_ptr()), vp(scale.data_ptr()), n, vp(d_table.data_ptr()),
            K, stride, S, vp(il_stream.data_ptr()), il_cap, vp(nw.data_ptr()), vp(st.data_ptr()),
            vp(il_ws.data_ptr()), il_ws.numel(), hs)
        fused = _median_us(fz, reps)
        B.check(st[:1], f"{cfg} fused encode")
        assert int(nw.item()) == il_words and np.array_equal(
            il_stream[:il_words].cpu().numpy().view(np.uint32), il_host), \
            f"{cfg}: fused container differs from the interleaved one"
    checked = "GPU round trips"
    if check_oracle:
        rc, owords = oracle.encode(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, lanes)
        assert rc == 0 and np.array_equal(owords, lane_words), \
            f"{cfg} L={lanes}: GPU container differs from the oracle's"
        rc, oil = oracle.encode_interleaved(w.symbols, w.indexes, w.cdf, w.lengths, w.offsets, S,
                                            64)
        assert rc == 0 and np.array_equal(oil, il_host), \
            f"{cfg} S={S}: GPU interleaved container differs from the oracle's"
        checked = "lane and interleaved containers equal the oracle's"
    bytes_lane = 8 * n + 4 * words
    bytes_il = 8 * n + 4 * il_words
    frac = lambda b, us: round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    r = {"config": cfg, "symbols": n, "lanes": lanes,
         "encode_us": round(enc_us, 2), "decode_us": round(dec_us, 2),
         "encode_gsym_s": round(n / enc_us / 1e3, 2), "decode_gsym_s": round(n / dec_us / 1e3, 2),
         "encode_frac": frac(bytes_lane, enc_us), "decode_frac": frac(bytes_lane, dec_us),
         "interleaved": {"streams": S, "encode_call_us": round(il_enc_us, 2),
                         "decode_call_us": round(il_dec_us, 2),
                         "encode_frac": frac(bytes_il, il_enc_us),
                         "decode_frac": frac(bytes_il, il_dec_us)},
         "parity": checked}
    if fused is not None:
        r["interleaved"]["fused_encode_call_us"] = round(fused, 2)
        # the fused call reads y, mean and scale (12 B/position) instead of
        # symbols and indexes (8 B)
        r["interleaved"]["fused_frac"] = frac(12 * n + 4 * il_words, fused)
    del il_ws, il_stream, stream, out, sym, idx
    torch.cuda.empty_cache()
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="y1080", choices=sorted(DEFAULT_LANES))
    ap.add_argument("--lanes", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--streams", type=int, default=None,
                    help="interleaved streams (default: lanes / 64, at most 4096)")
    ap.add_argument("--no-batch", action="store_true",
                    help="skip the batch configurations (profiling runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the lanes of one call are "
              "coded on one device (lanes are independent, so a contiguous lane range per GPU "
              "would shard the path, with one exclusive scan of per-GPU payload sizes).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from learned_image_compression_amd import binding as B

    lanes = args.lanes or DEFAULT_LANES[args.config]
    dev = torch.device("cuda:0")
    w = workloads.load(args.config)
    n = w.n
    tables = B.Tables.from_numpy(w.cdf, w.lengths, w.offsets, dev)
    sym = torch.from_numpy(w.symbols).to(dev)
    idx = torch.from_numpy(w.indexes).to(dev)
    cap = B.encode_bound_words(n, lanes)
    stream = torch.empty(cap, dtype=torch.int32, device=dev)
    nwords = torch.zeros(1, dtype=torch.int64, device=dev)
    st_enc = torch.zeros(1, dtype=torch.int32, device=dev)
    st_dec = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty(n, dtype=torch.int32, device=dev)
    ws = B.workspace_for(dev).get(B.workspace_bytes(n, lanes, tables.num_tables, tables.stride))

    # ---- before timing: the GPU round trip gives the input back -----------------
    B.encode_with_indexes(sym, idx, tables, lanes, stream_out=stream, stream_words=nwords,
                          status=st_enc, workspace=ws)
    B.check(st_enc, "encode")
    total_words = int(nwords.item())
    gpu_words = stream[:total_words].cpu().numpy().view(np.uint32).copy()
    assert gpu_words[0] == lanes and int(gpu_words[lanes]) == total_words - 1 - lanes
    B.decode_with_indexes(stream, idx, tables, symbols_out=out, status=st_dec,
                          workspace=ws, capacity_words=cap)
    B.check(st_dec, "decode")
    assert torch.equal(out.cpu(), torch.from_numpy(w.symbols)), "GPU decode != input"

    # ---- one step = prep + encode, prep + decode ---------------------------------
    # The entry points are called straight through ctypes with arguments
    # marshalled once, so the host adds as little as possible per launch.
    import ctypes
    lib = B.load()
    vp = ctypes.c_void_p
    hs = vp(torch.cuda.current_stream(dev).cuda_stream)
    prep_args = (vp(tables.cdf.data_ptr()), vp(tables.lengths.data_ptr()),
                 vp(tables.offsets.data_ptr()), tables.num_tables, tables.stride,
                 vp(ws.data_ptr()), ws.numel(), hs)
    enc_args = (vp(sym.data_ptr()), vp(idx.data_ptr()), n, tables.num_tables, tables.stride,
                lanes, vp(stream.data_ptr()), cap, vp(nwords.data_ptr()), vp(st_enc.data_ptr()),
                vp(ws.data_ptr()), ws.numel(), hs)
    dec_args = (vp(stream.data_ptr()), cap, vp(idx.data_ptr()), n, tables.num_tables,
                tables.stride, vp(out.data_ptr()), vp(st_dec.data_ptr()),
                vp(ws.data_ptr()), ws.numel(), hs)
    prep, enc, dec = lib.rans_prepare_tables, lib.rans_encode_prepared, lib.rans_decode_prepared

    # HIP events bracket each coding kernel on every EVENT_EVERY-th step of the
    # timed loop (events on every step would add about 5% to the step time)
    def step(ev):
        rc = prep(*prep_args)
        if ev:
            ev[0].record()
        rc |= enc(*enc_args)
        if ev:
            ev[1].record()
        rc |= prep(*prep_args)
        if ev:
            ev[2].record()
        rc |= dec(*dec_args)
        if ev:
            ev[3].record()
        if rc:
            raise RuntimeError(f"launch failed: {rc}")

    every = max(1, min(EVENT_EVERY, args.steps // 16))   # at least 16 sampled steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] if k % every == 0 else None
           for k in range(args.steps)]
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        step(evs[k])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    B.check(st_enc, "encode (timed)")
    B.check(st_dec, "decode (timed)")
    assert int(nwords.item()) == total_words
    assert torch.equal(out.cpu(), torch.from_numpy(w.symbols))

    gpu_ms = start.elapsed_time(stop) / args.steps
    ms_per_step = max(wall * 1e3 / args.steps, gpu_ms)
    sampled = [e for e in evs if e]
    enc_us = statistics.mean(e[0].elapsed_time(e[1]) for e in sampled) * 1e3
    dec_us = statistics.mean(e[2].elapsed_time(e[3]) for e in sampled) * 1e3
    value = n / (ms_per_step * 1e-3) / 1e9

    # ---- split records: the same container decoded as SPLIT_PIECES pieces/lane ----
    P = SPLIT_PIECES
    meta = torch.empty(3 * lanes * (P - 1), dtype=torch.int32, device=dev)
    sp_status = torch.zeros(1, dtype=torch.int32, device=dev)
    tab_full = (vp(tables.cdf.data_ptr()), vp(tables.lengths.data_ptr()),
                vp(tables.offsets.data_ptr()), tables.num_tables, tables.stride, lanes)
    if lib.rans_encode_with_splits(vp(sym.data_ptr()), vp(idx.data_ptr()), n, *tab_full, P,
                                   vp(stream.data_ptr()), cap, vp(nwords.data_ptr()),
                                   vp(meta.data_ptr()), vp(sp_status.data_ptr()),
                                   vp(ws.data_ptr()), ws.numel(), hs):
        raise RuntimeError("split encode launch failed")
    B.check(sp_status, "split encode")
    assert int(nwords.item()) == total_words and np.array_equal(
        stream[:total_words].cpu().numpy().view(np.uint32), gpu_words), "split container differs"
    gpu_records = meta.cpu().numpy().view(np.uint32).copy()

    def split_decode_us(pieces, reps=20):
        args = (vp(stream.data_ptr()), cap, vp(idx.data_ptr()), n, *tab_full[:5], pieces,
                vp(meta.data_ptr()), meta.numel(), vp(out.data_ptr()), vp(sp_status.data_ptr()),
                vp(ws.data_ptr()), ws.numel(), hs)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps + 3)]
        for e in sev:
            e[0].record()
            if lib.rans_decode_with_splits(*args):
                raise RuntimeError("split decode launch failed")
            e[1].record()
        torch.cuda.synchronize()
        B.check(sp_status, f"decode with {pieces} pieces")
        assert torch.equal(out.cpu(), torch.from_numpy(w.symbols)), "split decode != input"
        return statistics.median(a.elapsed_time(b) for a, b in sev[3:]) * 1e3

    split_us, plain_call_us = split_decode_us(P), split_decode_us(1)

    # ---- interleaved streams: 64 states per stream, as many states as lanes -------
    S_il = args.streams if args.streams else max(1, min(4096, lanes // 64))
    il_cap = int(lib.rans_interleaved_bound_words(n, S_il))
    il_ws = torch.zeros(int(lib.rans_interleaved_workspace_bytes(n, S_il, tables.num_tables,
                                                                 tables.stride)),
                        dtype=torch.uint8, device=dev)
    il_stream = torch.empty(il_cap, dtype=torch.int32, device=dev)
    il_nw = torch.zeros(1, dtype=torch.int64, device=dev)
    il_args = (vp(sym.data_ptr()), vp(idx.data_ptr()), n, *tab_full[:5], S_il)
    il_enc = lambda: lib.rans_encode_interleaved(*il_args, vp(il_stream.data_ptr()), il_cap,
                                                 vp(il_nw.data_ptr()), vp(sp_status.data_ptr()),
                                                 vp(il_ws.data_ptr()), il_ws.numel(), hs)
    il_dec = lambda: lib.rans_decode_interleaved(vp(il_stream.data_ptr()), il_cap,
                                                 vp(idx.data_ptr()), n, *tab_full[:5], S_il,
                                                 vp(out.data_ptr()), vp(st_dec.data_ptr()),
                                                 vp(il_ws.data_ptr()), il_ws.numel(), hs)
    iev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(23)]
    for e in iev:
        e[0].record()
        if il_enc():
            raise RuntimeError("interleaved encode launch failed")
        e[1].record()
        if il_dec():
            raise RuntimeError("interleaved decode launch failed")
        e[2].record()
    torch.cuda.synchronize()
    B.check(sp_status, "interleaved encode")
    B.check(st_dec, "interleaved decode")
    assert torch.equal(out.cpu(), torch.from_numpy(w.symbols)), "interleaved decode != input"
    il_words = int(il_nw.item())
    gpu_il = il_stream[:il_words].cpu().numpy().view(np.uint32).copy()
    il_enc_us = statistics.median(a.elapsed_time(b) for a, b, _ in iev[3:]) * 1e3
    il_dec_us = statistics.median(b.elapsed_time(c) for _, b, c in iev[3:]) * 1e3
    # the same calls on tables prepared once (the full calls above left them
    # prepared in il_ws)
    il_enc_p = lambda: lib.rans_encode_interleaved_prepared(
        vp(sym.data_ptr()), vp(idx.data_ptr()), n, tables.num_tables, tables.stride, S_il,
        vp(il_stream.data_ptr()), il_cap, vp(il_nw.data_ptr()), vp(sp_status.data_ptr()),
        vp(il_ws.data_ptr()), il_ws.numel(), hs)
    il_dec_p = lambda: lib.rans_decode_interleaved_prepared(
        vp(il_stream.data_ptr()), il_cap, vp(idx.data_ptr()), n, tables.num_tables, tables.stride,
        S_il,
        vp(out.data_ptr()), vp(st_dec.data_ptr()), vp(il_ws.data_ptr()), il_ws.numel(), hs)
    out.zero_()
    for e in iev:
        e[0].record()
        if il_enc_p():
            raise RuntimeError("prepared interleaved encode launch failed")
        e[1].record()
        if il_dec_p():
            raise RuntimeError("prepared interleaved decode launch failed")
        e[2].record()
    torch.cuda.synchronize()
    B.check(sp_status, "prepared interleaved encode")
    B.check(st_dec, "prepared interleaved decode")
    assert torch.equal(out.cpu(), torch.from_numpy(w.symbols)), "prepared interleaved decode != input"
    assert np.array_equal(il_stream[:il_words].cpu().numpy().view(np.uint32), gpu_il), \
        "prepared interleaved container differs"
    il_enc_p_us = statistics.median(a.elapsed_time(b) for a, b, _ in iev[3:]) * 1e3
    il_dec_p_us = statistics.median(b.elapsed_time(c) for _, b, c in iev[3:]) * 1e3

    # ---- device table builder on the workloads' table set ------------------------
    scales, tail_z, tstride = table_set()
    d_scales = torch.from_numpy(scales).to(dev)
    built, row_st = B.gaussian_tables(d_scales, tail_z, tstride)
    B.check_rows(row_st)
    gpu_tables = tuple(t.cpu().numpy() for t in (built.cdf, built.lengths, built.offsets))
    if w.num_tables == scales.size and w.stride == tstride:
        assert all(np.array_equal(a, b) for a, b in zip(gpu_tables, (w.cdf, w.lengths, w.offsets))), \
            "device-built tables differ from the workload's"
    # timed on preallocated outputs, straight through ctypes
    row_args = (vp(d_scales.data_ptr()), scales.size, tail_z, tstride, vp(built.cdf.data_ptr()),
                vp(built.lengths.data_ptr()), vp(built.offsets.data_ptr()),
                vp(row_st.data_ptr()), hs)
    tev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    tab_us = []
    for k in range(23):
        tev[0].record()
        if lib.rans_gaussian_tables(*row_args):
            raise RuntimeError("table build launch failed")
        tev[1].record()
        torch.cuda.synchronize()
        if k >= 3:
            tab_us.append(tev[0].elapsed_time(tev[1]) * 1e3)
    B.check_rows(row_st)

    bytes_per_launch = 8 * n + 4 * total_words   # same for encode and decode
    dominant, dom_us = ("decode", dec_us) if dec_us >= enc_us else ("encode", enc_us)
    achieved = bytes_per_launch / (dom_us * 1e-6) / 1e9
    traffic = measured_traffic(dominant, args.config, lanes)

    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "Gsymbol/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / PAGE_BASELINE[args.config]["value"], 2)
                        if args.config in PAGE_BASELINE else None),
        "baseline": PAGE_BASELINE.get(args.config),
        "dtype": "u64",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {DESCRIPTION[args.config]}", "lanes": lanes,
                   "symbols": n, "container_words": total_words,
                   "bits_per_symbol": round(32.0 * (total_words - 1 - lanes) / n, 4)},
        "encode_gsym_s": round(n / (enc_us * 1e-6) / 1e9, 3),
        "decode_gsym_s": round(n / (dec_us * 1e-6) / 1e9, 3),
        "kernel_us": {"encode": round(enc_us, 2), "decode": round(dec_us, 2),
                      "step_gpu": round(gpu_ms * 1e3, 2)},
        "roofline": {
            "bound": "hbm",
            "kernel": f"{dominant}_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 5),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bytes_per_launch,
        },
        "parity": "GPU decode of the GPU container equals the input",
        "split_decode": {"pieces": P, "records_bytes": 12 * lanes * (P - 1),
                         "call_us": round(split_us, 2), "one_piece_call_us": round(plain_call_us, 2),
                         "decode_gsym_s": round(n / (split_us * 1e-6) / 1e9, 3),
                         "note": "decode call incl. its table prep; same container, "
                                 "records beside it"},
        "interleaved": {"streams": S_il, "states": 64 * S_il, "container_words": il_words,
                        "encode_call_us": round(il_enc_us, 2), "decode_call_us": round(il_dec_us, 2),
                        "step_gsym_s": round(n / ((il_enc_us + il_dec_us) * 1e-6) / 1e9, 3),
                        "prepared_encode_call_us": round(il_enc_p_us, 2),
                        "prepared_decode_call_us": round(il_dec_p_us, 2),
                        "prepared_step_gsym_s": round(n / ((il_enc_p_us + il_dec_p_us) * 1e-6) / 1e9, 3),
                        "note": "*_call_us: the full calls, table prep included; prepared_*: the "
                                "*_prepared calls on tables prepared once; a different container: "
                                "64 interleaved states per stream, one shared word cursor"},
        "table_build": {"kernel": "table_rows_kernel",
                        "workload": f"{scales.size} Gaussian rows, scales log-spaced "
                                    f"{scales[0]:g}..{scales[-1]:g}, tail mass 1e-9, "
                                    f"stride {tstride}",
                        "us": round(statistics.median(tab_us), 2)},
    }
    if not args.no_batch:
        line["batch"] = [batch_point(c, L, BATCH_STREAMS, not args.no_cpu_baseline)
                         for c, L in BATCH_POINTS]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, lanes, gpu_words, gpu_tables, args.cpu_seconds,
                                            split=(P, gpu_records), interleaved=(S_il, gpu_il))
        line["parity"] = line["cpu_baseline"].pop("parity")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
