"""Plant plausible mistakes in copies of the oracle and check the pins catch each.

Every mutant below is a one-token slip someone could make while writing the
coder from its description (a wrong constant, a dropped term, a swapped
operand, an off-by-one, a wrong order).  Each mutated copy is compiled on the
CPU and run through the quick pins in a child process; a mutant that survives
means the pins are too weak.  Mistakes are planted only in these copies,
never in the oracle source itself.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
RUNNER = os.path.join(HERE, "mutant_runner.py")

MUTANTS = {
    "state_low": ("#define STATE_LOW (1ull << 31)", "#define STATE_LOW (1ull << 30)"),
    "reg_threshold": ("(uint64_t)p.freq << (63 - PREC)", "(uint64_t)p.freq << (62 - PREC)"),
    "bits_threshold": ("(1ull << (63 - BYPASS_BITS))", "(1ull << (62 - BYPASS_BITS))"),
    "flush_order": ("out[0] = (uint32_t)x;\n        out[1] = (uint32_t)(x >> 32);",
                    "out[1] = (uint32_t)x;\n        out[0] = (uint32_t)(x >> 32);"),
    "spill_order": ("out[2 + k] = emitted[ne - 1 - k];", "out[2 + k] = emitted[k];"),
    "zigzag_below": ("raw = -2 * v - 1;", "raw = -2 * v;"),
    "zigzag_above": ("raw = 2 * (v - mv);", "raw = 2 * (v - mv) + 2;"),
    "dropped_remainder": ("(*x / p.freq) * TOTAL_FREQ + (*x % p.freq) + p.start",
                          "(*x / p.freq) * TOTAL_FREQ + p.start"),
    "start_index": ("put_push(l, (uint32_t)row[v], (uint32_t)(row[v + 1] - row[v]))",
                    "put_push(l, (uint32_t)row[v] + (v > 0), (uint32_t)(row[v + 1] - row[v]))"),
    "scan_strict": ("(uint32_t)row[s + 1] <= cum", "(uint32_t)row[s + 1] < cum"),
    "partition_ceil": ("((uint64_t)j * b) / num_lanes;",
                       "((uint64_t)j * b + num_lanes - 1) / num_lanes;"),
    "refill_le": ("if (d->x < STATE_LOW) {", "if (d->x <= STATE_LOW) {"),
    "unzigzag_odd": ("value = -(int64_t)(raw >> 1) - 1;", "value = -(int64_t)(raw >> 1);"),
    "header_start": ("out[1 + j] = (uint32_t)used;", "out[1 + j] = (uint32_t)(used - w);"),
    "no_count": ("if ((rc = put_push(l, t, 0)))", "if (0 && (rc = put_push(l, t, 0)))"),
    "group_order": ("(((uint64_t)raw >> (BYPASS_BITS * k)) & BYPASS_MAX)",
                    "(((uint64_t)raw >> (BYPASS_BITS * (nb - 1 - k))) & BYPASS_MAX)"),
    "escape_slot": ("int64_t mv = (int64_t)lengths[index] - 2;  /* escape slot */",
                    "int64_t mv = (int64_t)lengths[index] - 1;  /* escape slot */"),
    "dec_state_shift": ("d.x = (uint64_t)freq * (d.x >> PREC) + cum - start;",
                        "d.x = (uint64_t)freq * (d.x >> (PREC - 1)) + cum - start;"),
    "end_check": ("if (d.x != want_x || d.pos != want_pos)", "if (d.x != want_x)"),
    # split records
    "split_cut_ceil": ("((unsigned __int128)(e - b) * s) / pieces)",
                       "((unsigned __int128)(e - b) * s + pieces - 1) / pieces)"),
    "split_left_count": ("cut_meta[3 * c + 2] = (uint32_t)ne;",
                         "cut_meta[3 * c + 2] = (uint32_t)(ne + (ne > 0));"),
    "split_start_pos": ("d.pos = W - m[2];", "d.pos = W - m[2] + (m[2] > 0);"),
    "split_state_half": ("cut_meta[3 * c + 1] = (uint32_t)(x >> 32);",
                         "cut_meta[3 * c + 1] = (uint32_t)(x >> 31);"),
    # table builder
    "q_round_half_up": ("f[k] = (int64_t)rint(p * TOTAL_FREQ);",
                        "f[k] = (int64_t)floor(p * TOTAL_FREQ + 0.5);"),
    "q_no_floor_one": ("if (f[k] < 1)\n            f[k] = 1;", "if (f[k] < 0)\n            f[k] = 0;"),
    "q_tie_highest": ("if (f[k] > f[top])", "if (f[k] >= f[top])"),
    "q_deficit_first_slot": ("f[top] += 1;", "f[0] += 1;"),
    "g_bin_edges": ("std_normal_cdf((v + 0.5) / scale) - std_normal_cdf((v - 0.5) / scale)",
                    "std_normal_cdf((v + 1.0) / scale) - std_normal_cdf(v / scale)"),
    "g_one_tail": ("pmf[m - 1] = 2.0 * std_normal_cdf(", "pmf[m - 1] = 1.0 * std_normal_cdf("),
    "g_half_width_floor": ("double cw = ceil(scale * tail_z);",
                           "double cw = floor(scale * tail_z);"),
    "g_offset_sign": ("*offset = -c;", "*offset = c;"),
    "g_padding": ("cdf_row[k] = (int32_t)TOTAL_FREQ;", "cdf_row[k] = 0;"),
    "g_root_two": ("-x * 0.70710678118654752440", "-x * 1.41421356237309504880"),
    # interleaved streams
    "il_state_order": ("for (uint32_t l = width; l-- > 0;) {", "for (uint32_t l = 0; l < width; ++l) {"),
    "il_slot_order": ("for (uint32_t s = max_slot; s-- > 0 && rc == ORACLE_OK;) {",
                      "for (uint32_t s = 0; s < max_slot && rc == ORACLE_OK; ++s) {"),
    "il_assignment": ("uint64_t k = g * width + l;\n                if (k >= m)\n                    continue;",
                      "uint64_t k = g * width + (width - 1 - l);\n                if (k >= m)\n                    continue;"),
    "il_flush_order": ("o[2 * l] = (uint32_t)x[l];\n                    o[2 * l + 1] = (uint32_t)(x[l] >> 32);",
                       "o[2 * l + 1] = (uint32_t)x[l];\n                    o[2 * l] = (uint32_t)(x[l] >> 32);"),
    # latent front end
    "l_round_half_up": ("float r = rintf(d);", "float r = floorf(d + 0.5f);"),
    "l_truncate": ("float r = rintf(d);", "float r = truncf(d);"),
    "l_index_strict": ("if (scales[i] <= scale_table[k])", "if (scales[i] < scale_table[k])"),
    "l_index_all_slots": ("for (int32_t k = 0; k < num_scales - 1; ++k)",
                          "for (int32_t k = 0; k < num_scales; ++k)"),
    "l_nan_symbol": ("if (d != d)\n        return INT32_MIN;", "if (d != d)\n        return 0;"),
    "l_saturate_high": ("if (r >= 2147483648.0f)\n        return INT32_MAX;",
                        "if (r > 2147483648.0f)\n        return INT32_MAX;"),
    "l_dequant_sign": ("y_hat[i] = (float)symbols[i] + means[i];",
                       "y_hat[i] = (float)symbols[i] - means[i];"),
}


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    # the header sits next to the original source
    inc = os.path.dirname(oracle.SOURCE)
    out = str(tmp_path / f"lib{name}.so")
    subprocess.run(["gcc", "-O1", "-std=c99", "-shared", "-fPIC", f"-I{inc}", str(src), "-o",
                    out, "-lm"], check=True)
    return out


def _run(lib_path):
    return subprocess.run([sys.executable, RUNNER, lib_path], capture_output=True, text=True,
                          timeout=300)


def test_unmutated_copy_passes(tmp_path):
    text = open(oracle.SOURCE).read()
    res = _run(_build(tmp_path, "control", text))
    assert res.returncode == 0, res.stdout + res.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(oracle.SOURCE).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    res = _run(_build(tmp_path, name, text.replace(old, new)))
    assert res.returncode != 0, f"mutant {name} survived the pins:\n{res.stdout}"
