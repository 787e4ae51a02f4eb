"""Host-side checks of the rocprofv3 summariser: kernel names map to the right
keys (counter passes over a bench run see the lane kernels, the split
decoder and the interleaved kernels side by side, and each must be averaged
on its own), and per-dispatch counters are summed over a dispatch's rows
before they are averaged over dispatches."""
from __future__ import annotations

import csv

from learned_image_compression_amd import profiling as P


def test_kernel_keys_keep_each_kernel_apart():
    names = {
        "void rans::(anonymous namespace)::encode_kernel<256, 1>(rans::EncodeArgs)": "encode_kernel",
        "rans::(anonymous namespace)::encode_pc_kernel(rans::EncodeArgs)": "encode_kernel",
        "void rans::(anonymous namespace)::decode_kernel<512, 8, false>(rans::DecodeArgs)":
            "decode_kernel",
        "void rans::(anonymous namespace)::decode_kernel<512, 8, true>(rans::DecodeArgs)":
            "decode_kernel_split",
        "void rans::(anonymous namespace)::il_encode_kernel<1024>(rans::IlArgs)": "il_encode_kernel",
        "void rans::(anonymous namespace)::il_decode_kernel<256>(rans::IlArgs)": "il_decode_kernel",
        "rans::(anonymous namespace)::il_scan_kernel(rans::IlArgs)": "il_scan_kernel",
        "rans::(anonymous namespace)::il_copy_kernel(rans::IlArgs)": "il_copy_kernel",
        "rans::(anonymous namespace)::prep_kernel(rans::PrepArgs)": "prep_kernel",
        "__amd_rocclr_copyBuffer": "copy",
    }
    for name, key in names.items():
        assert P._kernel_key(name) == key, name


def test_counter_per_dispatch_sums_rows_then_averages(tmp_path):
    path = tmp_path / "run_counter_collection.csv"
    rows = [
        # dispatch 1: the lane decoder, counter split over two rows (two XCDs)
        ("1", "void rans::(anonymous namespace)::decode_kernel<512, 8, false>(rans::DecodeArgs)", 10.0),
        ("1", "void rans::(anonymous namespace)::decode_kernel<512, 8, false>(rans::DecodeArgs)", 5.0),
        # dispatch 2: the lane decoder again
        ("2", "void rans::(anonymous namespace)::decode_kernel<512, 8, false>(rans::DecodeArgs)", 25.0),
        # dispatch 3: the interleaved decoder, which must not join the average above
        ("3", "void rans::(anonymous namespace)::il_decode_kernel<256>(rans::IlArgs)", 1000.0),
    ]
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, k, v in rows:
            w.writerow([d, k, "FETCH_SIZE", v])
        w.writerow(["1", rows[0][1], "WRITE_SIZE", 7.0])
    got = P.counter_per_dispatch(str(path), "FETCH_SIZE")
    assert got == {"decode_kernel": 20.0, "il_decode_kernel": 1000.0}


def test_kernel_source_hash_follows_code_not_comments(tmp_path, monkeypatch):
    import shutil
    src = tmp_path / "csrc"
    shutil.copytree(P.CSRC, src)
    monkeypatch.setattr(P, "CSRC", str(src))
    before = {k: P.kernel_source_hash(k) for k in ("encode", "decode", "interleaved")}
    path = src / "rans_coding.hpp"
    text = path.read_text()
    # comments, blank lines and trailing blanks do not change the hash
    path.write_text("// a note\n\n" + text.replace("namespace rans {", "namespace rans {   /* x */\n\n"))
    assert {k: P.kernel_source_hash(k) for k in before} == before
    # code does, for every kernel built from the file
    path.write_text(text + "\nstatic const int kProbe = 1;\n")
    after = {k: P.kernel_source_hash(k) for k in before}
    assert all(after[k] != before[k] for k in before)
