"""Helpers for the rocprofv3 summaries kept under profiles/.

Three commands, all meant to run under or after rocprofv3:

  python -m learned_image_compression_amd.profiling copy [--mib M]
      A plain device-to-device copy of M MiB (torch copy_, which runs the
      HIP runtime's copy kernel), repeated a few times.  Counter passes over it
      (FETCH_SIZE, WRITE_SIZE) give the scale between those counters and
      bytes actually moved: a copy of M MiB reads and writes M MiB.

  python -m learned_image_compression_amd.profiling latent [--n N] [--reps R]
      The latent front end and dequantisation on N seeded synthetic
      positions (a 64-scale table log-spaced over 0.11..256), R times each,
      for kernel-trace and counter passes; prints the bytes each call moves.

  python -m learned_image_compression_amd.profiling interleaved [--config C]
          [--streams S] [--reps R]
      Interleaved-stream encode and decode calls on a workload (workloads/),
      R times each, then the same encode with the front end fused in (fed a
      latent that yields the workload's symbols and indexes), for
      kernel-trace and counter passes; checks the round trip and the fused
      container and prints the container size and the bytes each call moves.

  python -m learned_image_compression_amd.profiling lanes [--config C]
          [--lanes L] [--reps R]
      Lane-container encode and decode on tables prepared once (the
      *_prepared calls, as bench.py times them), R times each, for
      kernel-trace and counter passes at any workload and lane count.

  python -m learned_image_compression_amd.profiling summarize ...
      Turns rocprofv3 CSV output (kernel trace statistics and the counter
      passes) into the short text and JSON summaries committed under
      profiles/.  Runs on the host only.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def _code_only(text: str) -> str:
    """A source file's code without its comments and blank lines (a string
    literal holding // or /* is not expected in these kernels)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.split("\n"))
    return "\n".join(ln for ln in lines if ln.strip())


def kernel_source_hash(name: str) -> str:
    """Hash of the code that makes up one coding kernel (rans_<name>.hip and
    the shared headers, comments left out): counter summaries recorded for
    other code are stale."""
    h = hashlib.sha256()
    extra = {"interleaved": ("rans_frontend.hpp", "rans_lookup.hpp"),
             "decode": ("rans_lookup.hpp",)}.get(name, ())
    for f in ("rans_internal.hpp", "rans_coding.hpp", *extra, f"rans_{name}.hip"):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]

KIB = 1024.0


def copy_main(mib: int, reps: int) -> None:
    import torch
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "reps": reps}), flush=True)


def latent_main(n: int, reps: int) -> None:
    import math
    import torch
    from learned_image_compression_amd import binding as B
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    y = torch.randn(n, device=dev, generator=g) * 3
    m = torch.randn(n, device=dev, generator=g)
    s = torch.exp(torch.rand(n, device=dev, generator=g) * 8 - 3)
    table = torch.exp(torch.linspace(math.log(0.11), math.log(256.0), 64)).float().to(dev)
    sym = torch.empty(n, dtype=torch.int32, device=dev)
    idx = torch.empty_like(sym)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    for _ in range(reps):
        B.latent_symbols(y, m, s, table, symbols_out=sym, indexes_out=idx)
        B.dequantize(sym, m, out=out)
    torch.cuda.synchronize()
    print(json.dumps({"positions": n, "reps": reps, "latent_bytes": 20 * n,
                      "dequantize_bytes": 12 * n}), flush=True)


def interleaved_main(config: str, streams: int, reps: int) -> None:
    import torch
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import workloads
    from learned_image_compression_amd import binding as B
    dev = torch.device("cuda:0")
    w = workloads.load(config)
    tables = B.Tables.from_numpy(w.cdf, w.lengths, w.offsets, dev)
    sym = torch.from_numpy(w.symbols).to(dev)
    idx = torch.from_numpy(w.indexes).to(dev)
    for _ in range(reps):
        stream, nwords, st = B.encode_interleaved(sym, idx, tables, streams)
        out, st2 = B.decode_interleaved(stream, idx, tables, streams)
    torch.cuda.synchronize()
    B.check(st, "interleaved encode")
    B.check(st2, "interleaved decode")
    if not torch.equal(out.cpu(), torch.from_numpy(w.symbols)):
        raise RuntimeError("interleaved round trip differs from the input")
    words = int(nwords.item())
    ref = stream[:words].clone()
    # the fused front end: y = symbol, mean = 0, scale = the index's entry of a
    # strictly increasing table, which give back exactly the workload's
    # symbols and indexes
    fused = None
    if int(sym.abs().max()) <= (1 << 24):
        K = tables.num_tables
        table = (torch.exp(torch.linspace(0.0, 1.0, K, dtype=torch.float64) * 7.6 - 2.2)
                 .float().to(dev))
        if bool((table[1:] > table[:-1]).all()):
            y = sym.float()
            mean = torch.zeros_like(y)
            scale = table[idx.long()]
            for _ in range(reps):
                fs, fnw, fst = B.encode_interleaved_latent(y, mean, scale, table, tables, streams)
            torch.cuda.synchronize()
            B.check(fst, "fused encode")
            if int(fnw.item()) != words or not torch.equal(fs[:words], ref):
                raise RuntimeError("fused container differs from the interleaved one")
            fused = 12 * w.n + 4 * words
    # a call reads symbols (or writes them) and indexes, and writes (or reads)
    # the container; the fused encode reads y, means and scales instead
    print(json.dumps({"config": config, "streams": streams, "reps": reps, "n": w.n,
                      "container_words": words,
                      "algorithmic_bytes_per_call": 8 * w.n + 4 * words,
                      "fused_algorithmic_bytes_per_call": fused}), flush=True)


def lanes_main(config: str, lanes: int, reps: int) -> None:
    import torch
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import workloads
    from learned_image_compression_amd import binding as B
    dev = torch.device("cuda:0")
    w = workloads.load(config)
    tables = B.Tables.from_numpy(w.cdf, w.lengths, w.offsets, dev)
    sym = torch.from_numpy(w.symbols).to(dev)
    idx = torch.from_numpy(w.indexes).to(dev)
    ws = torch.zeros(B.workspace_bytes(w.n, lanes, tables.num_tables, tables.stride),
                     dtype=torch.uint8, device=dev)
    B.prepare_tables(tables, ws)
    for _ in range(reps):
        stream, nwords, st = B.encode_with_indexes(sym, idx, tables, lanes, workspace=ws,
                                                   prepared=True)
        out, st2 = B.decode_with_indexes(stream, idx, tables, workspace=ws, prepared=True)
    torch.cuda.synchronize()
    B.check(st, "encode")
    B.check(st2, "decode")
    if not torch.equal(out.cpu(), torch.from_numpy(w.symbols)):
        raise RuntimeError("lane round trip differs from the input")
    words = int(nwords.item())
    print(json.dumps({"config": config, "lanes": lanes, "reps": reps, "n": w.n,
                      "container_words": words,
                      "algorithmic_bytes_per_call": 8 * w.n + 4 * words}), flush=True)


def _rows(path_glob: str):
    paths = sorted(glob.glob(path_glob, recursive=True))
    if not paths:
        raise FileNotFoundError(path_glob)
    with open(paths[0]) as fh:
        return list(csv.DictReader(fh))


def _kernel_key(name: str) -> str:
    # both forms of the lane encoder (one coding wave per CU up to 4096 lanes,
    # several beyond) are the encode kernel of their run
    if "encode_pc_kernel" in name:
        return "encode_kernel"
    if re.search(r"decode_kernel<[^>]*true>", name):
        return "decode_kernel_split"
    if re.search(r"il_encode_kernel<[^>]*true>", name):
        return "il_encode_kernel_fused"
    # the interleaved kernels first: their names contain the lane kernels'
    m = re.search(r"(il_encode_kernel|il_decode_kernel|il_scan_kernel|il_copy_kernel|"
                  r"encode_kernel|decode_kernel|prep_kernel|table_rows_kernel|"
                  r"latent_symbols_kernel|dequantize_kernel)", name)
    if m:
        return m.group(1)
    if "copyBuffer" in name:
        return "copy"
    return name.split("(")[0][-40:]


def counter_per_dispatch(path_glob: str, counter: str) -> dict:
    """Mean per-dispatch value of one counter, per kernel."""
    per = {}
    for r in _rows(path_glob):
        if r.get("Counter_Name") != counter:
            continue
        per.setdefault((_kernel_key(r["Kernel_Name"]), r["Dispatch_Id"]), 0.0)
        per[(_kernel_key(r["Kernel_Name"]), r["Dispatch_Id"])] += float(r["Counter_Value"])
    out = {}
    for (k, _), v in per.items():
        out.setdefault(k, []).append(v)
    return {k: statistics.mean(v) for k, v in out.items()}


def summarize_main(a) -> None:
    os.makedirs(a.out, exist_ok=True)
    if a.stats:
        # per kernel and launch shape (grid size): one kernel launched with
        # two shapes (the decoder with and without split pieces) is two rows
        rows = _rows(a.stats)
        groups = {}
        for r in rows:
            name = r["Kernel_Name"]
            if not re.search(r"rans|kernel", name):
                continue
            key = (name, int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
            groups.setdefault(key, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines = [f"# rocprofv3 kernel trace statistics: {a.label}", f"# command: {a.command}", "",
                 f"{'kernel':<52s} {'blocks':>7s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} "
                 f"{'max_us':>10s}"]
        for (name, blocks), d in sorted(groups.items(), key=lambda kv: -statistics.mean(kv[1])):
            short = re.sub(r"^void |\(anonymous namespace\)::|\(.*\)$", "", name)[:52]
            lines.append(f"{short:<52s} {blocks:7d} {len(d):6d} {statistics.mean(d):10.2f} "
                         f"{min(d):10.2f} {max(d):10.2f}")
        if a.bench_json:
            with open(a.bench_json) as fh:
                bench = [json.loads(l) for l in fh if l.strip().startswith("{")][-1]
            if "metric" in bench:
                lines += ["", "# bench.py line of the same run (kernel_us from HIP events):",
                          json.dumps({k: bench[k] for k in ("value", "unit", "ms_per_step",
                                                            "kernel_us", "split_decode",
                                                            "table_build") if k in bench})]
            else:
                lines += ["", "# line printed by the profiled command:", json.dumps(bench)]
        path = os.path.join(a.out, f"kernel_trace_{a.label}.txt")
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(path)
    if a.sq:
        # per kernel, the mean per dispatch of every counter in the given passes
        table = {}
        for g in a.sq:
            names = sorted({r["Counter_Name"] for r in _rows(g)})
            for c in names:
                for k, v in counter_per_dispatch(g, c).items():
                    table.setdefault(k, {})[c] = v
        lines = [f"# rocprofv3 counters (mean per dispatch): {a.label}", f"# command: {a.command}",
                 "# kernel sources: " + ", ".join(f"{k} {kernel_source_hash(k)}"
                                                  for k in ("encode", "decode", "interleaved")),
                 ""]
        for k in sorted(table):
            if not k.startswith(("il_", "encode", "decode", "prep", "table", "latent", "dequant")):
                continue
            lines.append(k)
            for c, v in sorted(table[k].items()):
                lines.append(f"  {c:<24s} {v:16.1f}")
        path = os.path.join(a.out, f"counters_{a.label}.txt")
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(path)
    if a.fetch and a.write:
        fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE")
        write = counter_per_dispatch(a.write, "WRITE_SIZE")
        cf = counter_per_dispatch(a.calib_fetch, "FETCH_SIZE")["copy"]
        cw = counter_per_dispatch(a.calib_write, "WRITE_SIZE")["copy"]
        copy_bytes = a.copy_mib * (1 << 20)
        f_scale = copy_bytes / (cf * KIB)
        w_scale = copy_bytes / (cw * KIB)
        if a.interleaved_streams:
            with open(a.bench_json) as fh:
                run = [json.loads(l) for l in fh if l.strip().startswith("{")][-1]
            t = {"workload": a.label, "config": a.config, "streams": a.interleaved_streams,
                 "n": run["n"], "container_words": run["container_words"],
                 "algorithmic_bytes_per_call": run["algorithmic_bytes_per_call"],
                 "commands": a.command,
                 "copy_calibration": {"copy_bytes": copy_bytes, "fetch_kib": round(cf, 1),
                                      "write_kib": round(cw, 1), "fetch_scale": round(f_scale, 4),
                                      "write_scale": round(w_scale, 4)}}
            t["source_hash"] = kernel_source_hash("interleaved")
            t["fused_algorithmic_bytes_per_call"] = run.get("fused_algorithmic_bytes_per_call")
            for key in ("il_encode_kernel", "il_encode_kernel_fused", "il_copy_kernel",
                        "il_decode_kernel"):
                if key not in fetch or key not in write:
                    continue
                rb = fetch[key] * KIB * f_scale
                wb = write[key] * KIB * w_scale
                t[key] = {"fetch_kib_per_dispatch": round(fetch[key], 1),
                          "write_kib_per_dispatch": round(write[key], 1),
                          "hbm_bytes_per_launch": round(rb + wb)}
            path = os.path.join(a.out, f"traffic_{a.label}.json")
            with open(path, "w") as fh:
                json.dump(t, fh, indent=1)
                fh.write("\n")
            print(path)
            return
        if a.latent_n:
            # the front end moves 20 bytes per position, dequantisation 12
            t = {"workload": a.label, "positions": a.latent_n, "commands": a.command,
                 "copy_calibration": {"copy_bytes": copy_bytes, "fetch_kib": round(cf, 1),
                                      "write_kib": round(cw, 1), "fetch_scale": round(f_scale, 4),
                                      "write_scale": round(w_scale, 4)}}
            for key, per in (("latent_symbols_kernel", 20), ("dequantize_kernel", 12)):
                rb = fetch[key] * KIB * f_scale
                wb = write[key] * KIB * w_scale
                t[key] = {"fetch_kib_per_dispatch": round(fetch[key], 1),
                          "write_kib_per_dispatch": round(write[key], 1),
                          "hbm_bytes_per_launch": round(rb + wb),
                          "algorithmic_bytes_per_launch": per * a.latent_n}
            path = os.path.join(a.out, f"traffic_{a.label}.json")
            with open(path, "w") as fh:
                json.dump(t, fh, indent=1)
                fh.write("\n")
            print(path)
            return
        for kernel in ("encode", "decode"):
            key = f"{kernel}_kernel"
            rb = fetch[key] * KIB * f_scale
            wb = write[key] * KIB * w_scale
            t = {
                "kernel": key, "workload": a.label, "config": a.config, "lanes": a.lanes,
                "fetch_kib_per_dispatch": round(fetch[key], 1),
                "write_kib_per_dispatch": round(write[key], 1),
                "copy_calibration": {"copy_bytes": copy_bytes, "fetch_kib": round(cf, 1),
                                     "write_kib": round(cw, 1), "fetch_scale": round(f_scale, 4),
                                     "write_scale": round(w_scale, 4)},
                "hbm_read_bytes_per_launch": round(rb),
                "hbm_write_bytes_per_launch": round(wb),
                "hbm_bytes_per_launch": round(rb + wb),
                "source_hash": kernel_source_hash(kernel),
                "commands": a.command,
            }
            path = os.path.join(a.out, f"traffic_{kernel}_{a.config}_L{a.lanes}.json")
            with open(path, "w") as fh:
                json.dump(t, fh, indent=1)
                fh.write("\n")
            print(path, t["hbm_bytes_per_launch"])


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(prog="python -m learned_image_compression_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=256)
    c.add_argument("--reps", type=int, default=3)
    lt = sub.add_parser("latent")
    lt.add_argument("--n", type=int, default=50135040)
    lt.add_argument("--reps", type=int, default=5)
    s = sub.add_parser("summarize")
    s.add_argument("--out", required=True)
    s.add_argument("--label", required=True)
    s.add_argument("--config", default="y1080")
    s.add_argument("--lanes", type=int, default=4096)
    s.add_argument("--command", default="")
    s.add_argument("--stats")
    s.add_argument("--bench-json")
    s.add_argument("--fetch")
    s.add_argument("--write")
    s.add_argument("--calib-fetch")
    s.add_argument("--calib-write")
    s.add_argument("--copy-mib", type=int, default=256)
    s.add_argument("--latent-n", type=int, default=0)
    s.add_argument("--interleaved-streams", type=int, default=0)
    s.add_argument("--sq", nargs="*", default=[], help="counter CSVs of SQ passes")
    il = sub.add_parser("interleaved")
    il.add_argument("--config", default="y1080x16")
    il.add_argument("--streams", type=int, default=4096)
    il.add_argument("--reps", type=int, default=5)
    ln = sub.add_parser("lanes")
    ln.add_argument("--config", default="y1080x16")
    ln.add_argument("--lanes", type=int, default=65536)
    ln.add_argument("--reps", type=int, default=5)
    a = ap.parse_args(argv)
    if a.cmd == "copy":
        copy_main(a.mib, a.reps)
    elif a.cmd == "latent":
        latent_main(a.n, a.reps)
    elif a.cmd == "interleaved":
        interleaved_main(a.config, a.streams, a.reps)
    elif a.cmd == "lanes":
        lanes_main(a.config, a.lanes, a.reps)
    else:
        summarize_main(a)


if __name__ == "__main__":
    main()
