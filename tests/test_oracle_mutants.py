"""Planted mistakes in copies of the oracle must each fail the pin suite.

Every mutant below is a plausible slip in one oracle function (a dropped
block, a sign, a bit position, a tie rule, a rounding rule, a reduction order,
a missing or mis-weighted term).  Each is compiled from a copy of
oracle/moe_oracle.c into a temporary directory and the pins in
tests/test_oracle_pins.py are run against it; the pins must fail.  Nothing
here touches a GPU.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "drop_last_q8_block": ("for (int32_t b = 0; b < cols / 32; ++b) {\n                double dw",
                           "for (int32_t b = 0; b < cols / 32 - 1; ++b) {\n                double dw"),
    "q2_min_sign": ("return d * s * q - dmin * m;", "return d * s * q + dmin * m;"),
    "q2_bit_order": ("int q = (sb[20 + i / 4] >> (2 * (i % 4))) & 3;",
                     "int q = (sb[20 + i / 4] >> (2 * (3 - i % 4))) & 3;"),
    "q2_sum_bit_order": ("{ return (sb[20 + i / 4] >> (2 * (i % 4))) & 3; }",
                         "{ return (sb[20 + i / 4] >> (2 * (3 - i % 4))) & 3; }"),
    "q2_scale_min_swap": ("int s = sb[4 + j] & 15, m = sb[4 + j] >> 4;", "int m = sb[4 + j] & 15, s = sb[4 + j] >> 4;"),
    "tie_to_larger_id": ("(best < 0 || key[e] > key[best])", "(best < 0 || key[e] >= key[best])"),
    "round_half_away": ("float v = rintf(x[b * 32 + j] * id);", "float v = roundf(x[b * 32 + j] * id);"),
    "weights_from_key": ("for (int32_t j = 0; j < k; ++j) S += s[ids[(int64_t)t * k + j]];",
                         "for (int32_t j = 0; j < k; ++j) S += key[ids[(int64_t)t * k + j]];"),
    "sequential_logit": ("for (int32_t len = H; len > 1; len /= 2)\n                for (int32_t i = 0; i < len / 2; ++i) "
                         "prod[i] = prod[2 * i] + prod[2 * i + 1];\n            logits[te] = (float)prod[0];",
                         "double acc = 0; for (int32_t i = 0; i < H; ++i) acc += prod[i];\n"
                         "            logits[te] = (float)acc;"),
    "no_shared": ("for (int32_t c = 0; c < H; ++c) acc[c] += y[c];\n            }", "}"),
    "unstable_sort": ("perm[offsets[e] + fill[e]++] = (int32_t)p;", "perm[offsets[e + 1] - 1 - fill[e]++] = (int32_t)p;"),
    "silu_sign": ("hf[r] = (float)(g[r] / (1.0 + exp(-g[r])) * u[r]);", "hf[r] = (float)(g[r] / (1.0 + exp(g[r])) * u[r]);"),
    "gate_up_swapped": ("hf[r] = (float)(g[r] / (1.0 + exp(-g[r])) * u[r]);",
                        "hf[r] = (float)(u[r] / (1.0 + exp(-u[r])) * g[r]);"),
    "quant_scale_128": ("float dd = amax / 127.0f;", "float dd = amax / 128.0f;"),
    "weight_wrong_slot": ("double we = slot >= 0 ? (double)w_[(int64_t)t * k + slot] : 0.0;",
                          "double we = slot >= 0 ? (double)w_[(int64_t)t * k + (k - 1 - slot)] : 0.0;"),
    "bias_ignored": ("key[e] = s[e] + (bias ? bias[e] : 0.0f);", "key[e] = s[e];"),
    "hash_reversed": ("ids[(int64_t)t * k + j] = e;", "ids[(int64_t)t * k + (k - 1 - j)] = e;"),
    "hash_row_stride": ("int32_t e = table[(int64_t)id * table_k + j];", "int32_t e = table[(int64_t)id * k + j];"),
    "hash_scored_unnormalised": ("ids[(int64_t)t * k + j]]) / S;", "ids[(int64_t)t * k + j]]);"),
    "hash_scored_term_dropped": ("for (int32_t j = 0; j < k; ++j) S += orc_sigmoid(",
                                 "for (int32_t j = 1; j < k; ++j) S += orc_sigmoid("),
    "hash_scored_equal_weights": ("            rc = orc_route_hash_scored(", "            rc = orc_route_hash(token_ids, wt->table, wt->vocab, table_k, T, E, k, ids_, w_); (void)("),
    "f16_exponent": ("else v = ldexp((double)(1024 + m), e - 25);", "else v = ldexp((double)(1024 + m), e - 24);"),
    "block_sum_index": ("acc += (int32_t)(int8_t)row[b * 34 + 2 + j] * (int32_t)aq[b * 32 + j];",
                        "acc += (int32_t)(int8_t)row[b * 34 + 2 + j] * (int32_t)aq[b * 32 + (j ^ 1)];"),
}


def _run(name, tmp):
    a, b = MUTANTS[name]
    src = open(SRC).read()
    assert a in src, f"mutant {name}: anchor not found in the oracle source"
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    with open(c, "w") as f:
        f.write(src.replace(a, b, 1))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                           "-I", os.path.join(ROOT, "oracle"), c, "-o", so, "-lm"], stderr=subprocess.DEVNULL)
    env = dict(os.environ, MOE_ORACLE_LIB=so, OMP_NUM_THREADS="1")
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, cwd=ROOT)
    return name, p.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
            results = dict(ex.map(lambda n: _run(n, tmp), MUTANTS))
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"
