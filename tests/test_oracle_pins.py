"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one oracle function against exact arithmetic (Python ints,
fractions, math.fsum), brute force on tiny inputs, or a closed form, chosen so
that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, a wrong tie rule, a wrong bit position) fails at least one of them.
The layer's definition follows the pages cited in oracle/moe_oracle.c.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import moe_synth as ms
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- formats ---

def f16_bits_to_fraction(bits: int) -> Fraction:
    """IEEE binary16 decoded from its definition (independent of the oracle)."""
    sign = -1 if bits >> 15 else 1
    e, m = (bits >> 10) & 31, bits & 1023
    assert e != 31
    if e == 0:
        return sign * Fraction(m, 2 ** 24)
    return sign * Fraction(1024 + m, 1) * Fraction(2) ** (e - 25)


def q8_row_values(row: bytes, cols: int):
    """Q8_32 row -> (fractions per weight, int codes); block = fp16 d + 32 int8."""
    vals, codes = [], []
    for b in range(cols // 32):
        blk = row[34 * b: 34 * b + 34]
        d = f16_bits_to_fraction(struct.unpack("<H", blk[:2])[0])
        qs = struct.unpack("<32b", blk[2:])
        codes += list(qs)
        vals += [d * q for q in qs]
    return vals, codes


def q2_row_values(row: bytes, cols: int):
    """Q2_256 row -> (fractions per weight, int codes, per-weight scale, per-weight min)."""
    vals, codes = [], []
    for sb in range(cols // 256):
        blk = row[84 * sb: 84 * sb + 84]
        d = f16_bits_to_fraction(struct.unpack("<H", blk[0:2])[0])
        dmin = f16_bits_to_fraction(struct.unpack("<H", blk[2:4])[0])
        sm, qs = blk[4:20], blk[20:84]
        for i in range(256):
            s, m = sm[i // 16] & 15, sm[i // 16] >> 4
            q = (qs[i // 4] >> (2 * (i % 4))) & 3
            codes.append(q)
            vals.append(d * s * q - dmin * m)
    return vals, codes


def test_f16_decode_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(bits.view(np.float16))
    ref = bits.view(np.float16).astype(np.float64)
    ours = np.array([oracle.f16_to_double(int(b)) for b in bits[finite]])
    assert np.array_equal(ours, ref[finite])


# --------------------------------------------------------- a1: router logits

def test_pairwise_sum_follows_the_tree():
    # sequential order gives 0, exact sum is 2; the pairwise tree
    # (1 + 2^53) + (1 - 2^53) rounds the first pair to 2^53 (ties to even)
    # and keeps the second exact, so it returns 1.
    v = np.array([1.0, 2.0 ** 53, 1.0, -(2.0 ** 53)])
    assert oracle.pairwise_sum(v) == 1.0
    # integers: exact whatever the tree
    ints = np.random.default_rng(3).integers(-2 ** 40, 2 ** 40, size=1024)
    assert oracle.pairwise_sum(ints.astype(np.float64)) == float(int(ints.sum()))


def test_router_logits_match_exactly_rounded_dot():
    rng = np.random.default_rng(11)
    T, E, H = 6, 20, 256
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (0.05 * rng.standard_normal((E, H))).astype(np.float32)
    got = oracle.router_logits(x, w)
    for t in range(T):
        for e in range(E):
            prods = [float(a) * float(b) for a, b in zip(x[t].tolist(), w[e].tolist())]  # exact in binary64
            exact = math.fsum(prods)                     # correctly rounded binary64 of the exact sum
            bound = H * 2.0 ** -52 * sum(abs(p) for p in prods)
            want = np.float32(exact)
            if got[t, e] != want:
                # only acceptable when the exact value sits within the fp64 error of an fp32 rounding boundary
                lo, hi = sorted((float(got[t, e]), float(want)))
                mid = (lo + hi) / 2
                assert abs(exact - mid) <= bound, (t, e)


def test_router_logit_reduction_order_worked_example():
    # products (1, 2^53, 1, -2^53): the adjacent-pair tree gives (2^53) + (1 - 2^53) = 1,
    # a half-split tree (p0+p2) + (p1+p3) gives 2, left-to-right gives 0 (exact sum: 2).
    x = np.array([[1.0, 2.0 ** 26, 1.0, -(2.0 ** 26)]], np.float32)
    w = np.array([[1.0, 2.0 ** 27, 1.0, 2.0 ** 27]], np.float32)
    assert oracle.router_logits(x, w)[0, 0] == 1.0


def test_router_logits_one_hot_input_selects_a_column():
    rng = np.random.default_rng(12)
    E, H = 16, 512
    w = rng.standard_normal((E, H)).astype(np.float32)
    x = np.zeros((3, H), np.float32)
    cols = [0, 77, 511]
    for t, c in enumerate(cols):
        x[t, c] = 1.0
    got = oracle.router_logits(x, w)
    for t, c in enumerate(cols):
        assert np.array_equal(got[t], w[:, c])


# --------------------------------------------------------- a2: selection ---

def ulp32(v):
    return float(np.spacing(np.float32(abs(v))))


def test_sigmoid_closed_forms():
    assert oracle.sigmoid(0.0) == 0.5
    l = float(np.float32(math.log(3.0)))          # sigmoid(ln 3) = 3/4
    assert abs(oracle.sigmoid(l) - 0.75) <= ulp32(0.75)
    for v in (-3.5, -0.75, 0.3, 2.0, 7.25):       # symmetry s(-l) = 1 - s(l)
        assert abs(oracle.sigmoid(-v) - (1.0 - oracle.sigmoid(v))) <= 2 * ulp32(0.5)
    assert oracle.sigmoid(100.0) == 1.0
    assert oracle.sigmoid(-200.0) == 0.0
    # monotone on a grid
    grid = np.linspace(-8, 8, 2001, dtype=np.float32)
    s = np.array([oracle.sigmoid(float(g)) for g in grid])
    assert np.all(np.diff(s) >= 0)


def brute_topk(key, k):
    return sorted(range(len(key)), key=lambda e: (-float(key[e]), e))[:k]


def test_route_learned_bruteforce_with_ties():
    rng = np.random.default_rng(21)
    T, E, k = 64, 16, 4
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[::3, 5] = logits[::3, 2]                # exact ties between experts 2 and 5
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    ids, w, s = oracle.route_learned(logits, bias, k)
    for t in range(T):
        key = [np.float32(s[t, e]) + np.float32(bias[e]) for e in range(E)]
        assert list(ids[t]) == brute_topk(key, k)
        assert abs(float(np.sum(w[t], dtype=np.float64)) - 1.0) <= k * 2.0 ** -24
        S = np.float64(sum(float(s[t, e]) for e in ids[t]))
        for j in range(k):
            assert abs(float(w[t, j]) * S - float(s[t, ids[t, j]])) <= 4 * ulp32(s[t, ids[t, j]])


def test_route_learned_all_equal_scores_and_zero_bias():
    E, k = 32, 6
    ids, w, _ = oracle.route_learned(np.zeros((2, E), np.float32), None, k)
    assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (2, 1)))
    assert np.all(w == np.float32(1.0 / k)) or np.allclose(w, 1.0 / k, atol=2 ** -24)
    # zero bias: sigmoid is monotone, so the selection is the top-k of the raw logits
    rng = np.random.default_rng(22)
    logits = rng.standard_normal((50, E)).astype(np.float32)
    ids, _, _ = oracle.route_learned(logits, np.zeros(E, np.float32), k)
    for t in range(50):
        assert list(ids[t]) == brute_topk(logits[t], k)


def test_route_hash_table_rows_and_rejects():
    table = ms.distinct_rows(1000, 6, 256, seed=5, tag=99)
    tok = np.array([0, 999, 17, 17, 512], np.int32)
    ids, w = oracle.route_hash(tok, table, 256)
    assert np.array_equal(ids, table[tok])
    assert np.all(w == np.float32(1) / np.float32(6))
    with pytest.raises(ValueError):
        oracle.route_hash(np.array([1000], np.int32), table, 256)
    bad = table.copy()
    bad[3, 1] = bad[3, 0]
    with pytest.raises(ValueError):
        oracle.route_hash(np.array([3], np.int32), bad, 256)
    bad = table.copy()
    bad[4, 2] = 256
    with pytest.raises(ValueError):
        oracle.route_hash(np.array([4], np.int32), bad, 256)


def test_route_hash_reduced_keeps_the_row_prefix():
    """Rows of 6 entries of which k are kept (reduced top-k): the ids are the
    first k table entries in table order, the weights 1/k."""
    table = ms.distinct_rows(1000, 6, 256, seed=6, tag=99)
    tok = np.array([0, 999, 17, 17, 512, 3], np.int32)
    for k in (1, 4, 6):
        ids, w = oracle.route_hash(tok, table, 256, k=k)
        assert np.array_equal(ids, table[tok, :k])
        assert np.all(w == np.float32(1) / np.float32(k))
    with pytest.raises(ValueError):
        oracle.route_hash(tok, table, 256, k=7)


def test_route_hash_scored_equal_scores_give_equal_weights():
    """Zero logits: every score is 1/2, the sum is k/2 exactly, so the
    renormalised weights are exactly 1/k (closed form)."""
    table = ms.distinct_rows(300, 6, 64, seed=7, tag=99)
    tok = np.arange(0, 300, 7, dtype=np.int32)
    for k in (3, 6):
        ids, w = oracle.route_hash_scored(tok, table, np.zeros((len(tok), 64), np.float32), k=k)
        assert np.array_equal(ids, table[tok, :k])
        assert np.all(w == np.float32(1) / np.float32(k))


def test_route_hash_scored_matches_learned_on_the_same_experts():
    """A table row holding the learned top-k (rank order) is weighted exactly
    as the learned router weights it: same scores, same summation order."""
    rng = np.random.default_rng(23)
    T, E, k = 40, 32, 6
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    ids_l, w_l, _ = oracle.route_learned(logits, bias, k)
    ids_h, w_h = oracle.route_hash_scored(np.arange(T, dtype=np.int32), np.ascontiguousarray(ids_l), logits)
    assert np.array_equal(ids_h, ids_l)
    assert np.array_equal(w_h.view(np.uint32), w_l.view(np.uint32))


def test_route_hash_scored_weights_are_renormalised_scores():
    """Weights sum to one, follow the ratios of the sigmoid scores and never
    decrease with the logit (384 experts, rows of 8, 4 or 8 kept)."""
    rng = np.random.default_rng(24)
    table = ms.distinct_rows(500, 8, 384, seed=8, tag=99)
    tok = rng.integers(0, 500, 64).astype(np.int32)
    logits = rng.standard_normal((64, 384)).astype(np.float32)
    for k in (4, 8):
        ids, w = oracle.route_hash_scored(tok, table, logits, k=k)
        assert np.array_equal(ids, table[tok, :k])
        for t in range(64):
            assert abs(float(np.sum(w[t], dtype=np.float64)) - 1.0) <= k * 2.0 ** -23
            lg = logits[t, ids[t]]
            order = np.argsort(lg, kind="stable")
            assert np.all(np.diff(w[t][order]) >= 0)
            sc = 1.0 / (1.0 + np.exp(-lg.astype(np.float64)))
            np.testing.assert_allclose(w[t] / w[t][0], sc / sc[0], rtol=1e-6)


def test_route_learned_reduced_top_k_is_a_prefix():
    """Keeping the N highest-ranked of the top 6 (reduced top-k) is the top-N:
    the same leading ids, weights renormalised over the kept experts."""
    rng = np.random.default_rng(25)
    T, E = 50, 256
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    ids6, w6, _ = oracle.route_learned(logits, bias, 6)
    for n in (1, 4):
        ids_n, w_n, _ = oracle.route_learned(logits, bias, n)
        assert np.array_equal(ids_n, ids6[:, :n])
        for t in range(T):
            assert abs(float(np.sum(w_n[t], dtype=np.float64)) - 1.0) <= n * 2.0 ** -23
            np.testing.assert_allclose(w_n[t] / w_n[t][0], w6[t, :n] / w6[t, 0], rtol=1e-6)


def test_route_learned_384_experts_top8_bruteforce():
    """The 384-expert sigmoid top-8 shape: the selection is a brute-force
    ranking of key = fp32 sigmoid + bias (larger first, ties to the smaller id)."""
    rng = np.random.default_rng(26)
    T, E, k = 24, 384, 8
    logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(E)).astype(np.float32)
    logits[:, 200], bias[200] = logits[:, 7], bias[7]     # exact ties between experts 7 and 200
    ids, _, _ = oracle.route_learned(logits, bias, k)
    for t in range(T):
        sig = (1.0 / (1.0 + np.exp(-logits[t].astype(np.float64)))).astype(np.float32)
        key = [np.float32(sig[e]) + np.float32(bias[e]) for e in range(E)]
        assert list(ids[t]) == brute_topk(key, k)


# -------------------------------------------------------- a3: quantizer ---

def test_quantizer_properties():
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.standard_normal(32 * 50), 1e-30 * rng.standard_normal(32 * 3),
                        np.zeros(32), -np.abs(rng.standard_normal(32)), 1e30 * rng.standard_normal(32)]
                       ).astype(np.float32)
    q, d = oracle.quantize(x)
    xb, qb = x.reshape(-1, 32).astype(np.float64), q.reshape(-1, 32).astype(np.int64)
    for b in range(xb.shape[0]):
        amax = np.max(np.abs(xb[b]))
        if amax == 0:
            assert d[b] == 0 and np.all(qb[b] == 0)
            continue
        assert np.max(np.abs(qb[b])) == 127
        assert np.all(np.abs(qb[b]) <= 127)
        err = np.abs(xb[b] - qb[b] * float(d[b]))
        assert np.all(err <= 0.5 * float(d[b]) * (1 + 2 ** -20) + 1e-300)
        assert abs(float(d[b]) - amax / 127) <= ulp32(amax / 127)


def test_quantizer_integer_blocks_are_exact_and_ties_go_to_even():
    rng = np.random.default_rng(32)
    x = rng.integers(-126, 127, size=(8, 32)).astype(np.float32)
    x[:, 5] = 127
    x[3, 5] = -127
    q, d = oracle.quantize(x.reshape(-1))
    assert np.all(d == 1.0) and np.array_equal(q.reshape(8, 32), x.astype(np.int8))
    blk = np.zeros(32, np.float32)
    blk[0] = 127.0
    blk[1:7] = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5]
    q, d = oracle.quantize(blk)
    assert d[0] == 1.0 and list(q[1:7]) == [2, 4, -2, -4, 0, 0]


# ----------------------------------------------- integer block dot sums ---

def test_block_sums_bruteforce_q8_and_q2():
    rows, cols = 5, 512
    rng = np.random.default_rng(41)
    aq = rng.integers(-127, 128, size=cols).astype(np.int8)
    m8 = ms.q8_bank(1, rows, cols, seed=7, tag=1)[0]
    got = oracle.block_sums(m8, "q8", rows, cols, aq)
    for r in range(rows):
        _, codes = q8_row_values(m8[r].tobytes(), cols)
        want = [sum(codes[b * 32 + j] * int(aq[b * 32 + j]) for j in range(32)) for b in range(cols // 32)]
        assert list(got[r]) == want
    m2 = ms.q2_bank(1, rows, cols, seed=7, tag=2)[0]
    got = oracle.block_sums(m2, "q2", rows, cols, aq)
    for r in range(rows):
        _, codes = q2_row_values(m2[r].tobytes(), cols)
        want = [sum(codes[g * 16 + i] * int(aq[g * 16 + i]) for i in range(16)) for g in range(cols // 16)]
        assert list(got[r]) == want


def test_matvec_matches_exact_rational_value():
    rows, cols = 3, 512
    rng = np.random.default_rng(42)
    x = rng.standard_normal(cols).astype(np.float32)
    aq, ad = oracle.quantize(x)
    xvals = [Fraction(float(ad[c // 32])) * int(aq[c]) for c in range(cols)]
    for fmt, bank, decode in (("q8", ms.q8_bank, q8_row_values), ("q2", ms.q2_bank, q2_row_values)):
        m = bank(1, rows, cols, seed=8, tag=3)[0]
        got = oracle.matvec(m, fmt, rows, cols, aq, ad)
        for r in range(rows):
            wv = decode(m[r].tobytes(), cols)[0]
            exact = sum(a * b for a, b in zip(wv, xvals))
            assert abs(got[r] - float(exact)) <= 1e-13 * float(sum(abs(a * b) for a, b in zip(wv, xvals)))


def test_q2_zero_codes_closed_form():
    # all codes 0: every weight equals -dmin*m_j, so row . x = -dmin * sum_j m_j * (sum of x over subblock j)
    cols = 256
    m = ms.q2_bank(1, 2, cols, seed=9, tag=4)[0].copy()
    m[:, 20:84] = 0
    x = np.random.default_rng(43).standard_normal(cols).astype(np.float32)
    aq, ad = oracle.quantize(x)
    got = oracle.matvec(m, "q2", 2, cols, aq, ad)
    for r in range(2):
        dmin = float(f16_bits_to_fraction(int(m[r, 2]) | int(m[r, 3]) << 8))
        want = 0.0
        for j in range(16):
            mj = int(m[r, 4 + j]) >> 4
            want += -dmin * mj * sum(float(ad[(16 * j + i) // 32]) * int(aq[16 * j + i]) for i in range(16))
        assert abs(got[r] - want) <= 1e-12 * (abs(want) + 1e-30)


# ----------------------------------------------------------- a4: sort ---

def test_sort_pairs_is_stable_counting_sort():
    rng = np.random.default_rng(51)
    T, k, E = 300, 6, 40
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm = oracle.sort_pairs(ids, E)
    flat = ids.reshape(-1)
    assert list(perm) == sorted(range(T * k), key=lambda p: (flat[p], p))
    assert list(counts) == [int(np.sum(flat == e)) for e in range(E)]
    assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) == counts)


# ------------------------------------------------------ whole-layer pins ---

@pytest.mark.parametrize("k,route", [(2, "learned"), (4, "learned"), (3, "hash_scored")])
def test_dense_masked_equals_routed_bitwise(k, route):
    cfg = ms.CONFIGS["tiny"].with_(top_k=k, route=route, vocab=97, table_k=5 if route != "learned" else 0)
    inp = ms.make_inputs(cfg)
    routed = oracle.forward(cfg, inp)
    dense = oracle.forward(cfg, inp, dense=True)
    assert np.array_equal(routed["out"].view(np.uint32), dense["out"].view(np.uint32))


def test_score_weighted_hash_layer_uses_its_table_and_router():
    """Layer wiring of the score-weighted variant with rows of 6, 4 kept: ids
    from the table prefix, weights from route_hash_scored on the router logits."""
    cfg = ms.CONFIGS["tiny"].with_(route="hash_scored", top_k=4, table_k=6, vocab=200, tokens=9)
    inp = ms.make_inputs(cfg)
    r = oracle.forward(cfg, inp)
    lg = oracle.router_logits(inp["x"], inp["router_w"])
    assert np.array_equal(r["logits"].view(np.uint32), lg.view(np.uint32))
    ids, w = oracle.route_hash_scored(inp["token_ids"], inp["hash_table"], lg, k=4)
    assert np.array_equal(r["ids"], inp["hash_table"][inp["token_ids"], :4]) and np.array_equal(r["ids"], ids)
    assert np.array_equal(r["w"].view(np.uint32), w.view(np.uint32))


def test_hash_layer_reproduces_its_table():
    cfg = ms.CONFIGS["hash_decode"].with_(hidden=256, n_experts=16, ffn=128, tokens=9, vocab=500)
    inp = ms.make_inputs(cfg)
    r = oracle.forward(cfg, inp)
    assert np.array_equal(r["ids"], inp["hash_table"][inp["token_ids"]])
    assert np.all(r["w"] == np.float32(1) / np.float32(cfg.top_k))


def _q8_matrix(codes: np.ndarray, scale_bits: int = 0x3C00) -> np.ndarray:
    """Q8_32 bytes of an integer matrix with every block scale = fp16 bits (default 1.0)."""
    rows, cols = codes.shape
    out = np.zeros((rows, cols // 32, 34), np.uint8)
    out[:, :, 0] = scale_bits & 0xFF
    out[:, :, 1] = scale_bits >> 8
    out[:, :, 2:] = codes.astype(np.int8).reshape(rows, cols // 32, 32).view(np.uint8)
    return out.reshape(rows, -1)


def _closed_form_case(rng, H, F):
    """Integer expert whose SwiGLU saturates: x has +-127 in every 32-block (scale 1),
    gate rows give g = 127 (sigmoid(127) == 1 in fp64), up rows give u in {-1,0,1} with
    a +-1 in every 32-block of h, so h = 127*u is quantized exactly with scale 1."""
    x = rng.integers(-3, 4, size=H)
    x[::32] = 127
    x[1::32] = 1
    wg = np.zeros((F, H), np.int64)
    wg[:, 0] = 1                                    # g_r = 127
    wu = np.zeros((F, H), np.int64)
    u_target = rng.integers(-1, 2, size=F)
    u_target[::32] = 1
    wu[:, 1] = u_target                             # x[1] == 1 -> u_r = u_target[r]
    wd = rng.integers(-127, 128, size=(H, F))
    h = 127 * u_target
    y = wd @ h
    return x, wg, wu, wd, y


def test_closed_form_integer_layer():
    """E=2, k=2, shared expert, all integer data: out = w0*y0 + w1*y1 + y_sh exactly."""
    H, F, E = 256, 64, 2
    rng = np.random.default_rng(61)
    cfg = ms.LayerConfig("closed", H, E, 2, F, 1, seed=0)
    cases = [_closed_form_case(rng, H, F) for _ in range(3)]
    x = cases[0][0]
    ys = []
    banks = {"gate": [], "up": [], "down": []}
    for i, (_, wg, wu, wd, _) in enumerate(cases):
        wd = cases[i][3]
        ys.append(wd @ (127 * (wu[:, 1])))
        # every expert sees the same x, so its g and u come from columns 0 and 1 of x = (127, 1)
        banks["gate"].append(_q8_matrix(wg))
        banks["up"].append(_q8_matrix(wu))
        banks["down"].append(_q8_matrix(wd))
    inp = {
        "x": x.astype(np.float32)[None, :],
        "router_w": (0.01 * rng.standard_normal((E, H))).astype(np.float32),
        "router_b": np.zeros(E, np.float32),
        "gate": np.stack(banks["gate"][:2]), "up": np.stack(banks["up"][:2]), "down": np.stack(banks["down"][:2]),
        "sh_gate": banks["gate"][2], "sh_up": banks["up"][2], "sh_down": banks["down"][2],
    }
    r = oracle.forward(cfg, inp)
    ids, w = r["ids"][0], r["w"][0]
    assert sorted(ids) == [0, 1]
    wmap = {int(ids[j]): float(w[j]) for j in range(2)}
    want = np.float32(wmap[0] * ys[0].astype(np.float64) + wmap[1] * ys[1].astype(np.float64) + ys[2])
    assert np.array_equal(r["out"][0], want)
    for slot in range(3):
        e = int(ids[slot]) if slot < 2 else 2
        assert np.array_equal(r["hq"][0, slot], (127 * cases[e][2][:, 1]).astype(np.int8))
        assert np.all(r["hd"][0, slot] == 1.0)


def test_saturated_negative_gate_gives_zero_not_nan():
    H, F = 256, 32
    cfg = ms.LayerConfig("neg", H, 1, 1, F, 1, seed=0, shared=False)
    x = np.full(H, 127.0, np.float32)
    wg = np.full((F, H), -127, np.int64)            # g = -127*127*256: exp(-g) overflows
    wu = np.ones((F, H), np.int64)
    wd = np.ones((H, F), np.int64)
    inp = {"x": x[None, :], "router_w": np.zeros((1, H), np.float32), "router_b": np.zeros(1, np.float32),
           "gate": _q8_matrix(wg)[None], "up": _q8_matrix(wu)[None], "down": _q8_matrix(wd)[None]}
    r = oracle.forward(cfg, inp)
    assert np.all(np.isfinite(r["out"])) and np.all(r["out"] == 0.0)
    assert np.all(r["hq"][0, 0] == 0) and np.all(r["hd"][0, 0] == 0.0)


def test_tiny_golden_fixture():
    """Regression against values written by tests/golden/make_golden.py (oracle only)."""
    path = os.path.join(GOLDEN, "tiny_oracle.json")
    g = json.load(open(path))
    cfg = ms.CONFIGS["tiny"]
    r = oracle.forward(cfg, ms.make_inputs(cfg))
    assert r["ids"].tolist() == g["ids"]
    assert [[float(v) for v in row] for row in r["w"]] == g["w"]
    assert r["out"][:, :8].tolist() == g["out_head"]
    assert float(np.sum(r["out"].astype(np.float64))) == g["out_sum"]
