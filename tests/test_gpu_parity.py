"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar (per the layer's contract): expert ids, combine weights, router logits,
quantized activations, the token sort and every sampled int32 block sum are
bit-exact; fp32 outputs agree within 2e-3 normwise (max |gpu - oracle| /
max |oracle|).  h is quantized from fp32 values whose accumulation order
differs between the GPU and the fp64 oracle, so its codes may differ by one
step where a value sits on a rounding boundary; the stage-2 (down) sums are
therefore checked with the GPU's own h codes fed to the oracle.
"""
import json
import os

import numpy as np
import pytest

import moe_synth as ms
import oracle

pytestmark = pytest.mark.gpu

TOL = 2e-3
# h block scales hd = amax|h| / 127 come from gate and up sums accumulated in
# fp32 over the K/32 = 128 block terms (one rounding per term's scale product
# and one per fma), where the oracle sums in fp64.  The worst-case forward
# error of such a sum is 129 * 2^-24 = 7.7e-6 times its condition C =
# sum |terms| / |sum|; for the largest |h| of a block of these sums of
# random-sign terms C is about 0.4 * sqrt(128) = 4.5 (the largest of 32 sits
# about two standard deviations out), so one sum's bound is ~3.5e-5, and h =
# SiLU(g) * u carries the errors of two sums.  Rounding errors add like a
# random walk in practice (sqrt(129) * 2^-24 * C = 3e-6 at one standard
# deviation).  The tolerance takes the single-sum worst case.
HD_RTOL = 3.5e-5
LOG = os.environ.get("MOE_PARITY_LOG")

torch = pytest.importorskip("torch")


def _qr():
    import quantized_routed_moe_amd as qr
    return qr


_cache = {}


def case(cfg):
    """(inputs, layer) for a config; one large case stays resident at a time."""
    if cfg not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        inp = ms.make_inputs(cfg)
        layer = _qr().MoELayer(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared, cfg.routed_fmt, cfg.route,
                               cfg.vocab if cfg.route != "learned" else 0, table_k=cfg.table_k).load(inp)
        _cache[cfg] = (inp, layer)
    return _cache[cfg]


def log(name, **kv):
    print(name, json.dumps(kv), flush=True)
    if LOG:
        with open(LOG, "a") as f:
            f.write(json.dumps({"case": name, **kv}) + "\n")


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def run_gpu(cfg, inp, layer, x=None, tok=None, stride=0):
    """The debug call (intermediates, and with stride > 0 the block-sum
    builds of the expert kernels) and the product call moe_layer_forward on
    the same inputs.  g["out"] is the product call's output; it must equal the
    debug call's bit for bit, and check() compares it with the oracle."""
    x = inp["x"] if x is None else x
    xt = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    tt = None
    if cfg.route != "learned":
        tok = inp["token_ids"] if tok is None else tok
        tt = torch.from_numpy(np.ascontiguousarray(tok)).cuda()
    r = layer.forward_debug(xt, tt, sum_row_stride=stride)
    plain = layer.forward(xt, tt)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in r.items()}
    g["out_debug"], g["out"] = g["out"], plain.cpu().numpy()
    assert np.array_equal(bits(g["out"]), bits(g["out_debug"])), "moe_layer_forward differs from the debug call"
    return g


def check(cfg, inp, g, x=None, tok=None, rows=None, stride=0, name=""):
    """Compare GPU results g with the oracle; rows = tokens to run the full oracle on."""
    x = inp["x"] if x is None else x
    T, H, E, k, F = x.shape[0], cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn
    if cfg.route != "learned":
        tok = inp["token_ids"] if tok is None else tok
    rows = np.arange(T) if rows is None else np.asarray(rows)
    # a1/a2: routing of every token, bit-exact
    if cfg.route != "hash":
        lo = oracle.router_logits(x, inp["router_w"])
        assert np.array_equal(bits(g["logits"]), bits(lo)), "router logits differ"
    if cfg.route == "learned":
        ids_o, w_o, _ = oracle.route_learned(lo, inp["router_b"], k)
    elif cfg.route == "hash":
        ids_o, w_o = oracle.route_hash(tok, inp["hash_table"], E, k=k)
    else:
        ids_o, w_o = oracle.route_hash_scored(tok, inp["hash_table"], lo, k=k)
    assert np.array_equal(g["ids"], ids_o), "expert selection differs"
    assert np.array_equal(bits(g["w"]), bits(w_o)), "combine weights differ"
    # a3: quantized x, bit-exact
    xq_o, xd_o = oracle.quantize(x)
    assert np.array_equal(g["xq"], xq_o) and np.array_equal(bits(g["xd"]), bits(xd_o)), "x quantization differs"
    # a4: sort, bit-exact
    c_o, off_o, perm_o = oracle.sort_pairs(ids_o, E)
    assert np.array_equal(g["counts"], c_o) and np.array_equal(g["offsets"], off_o)
    assert np.array_equal(g["perm"], perm_o), "token sort differs"
    # a5/a6: outputs of the sampled tokens
    o = oracle.forward(cfg, inp, x=x[rows], token_ids=tok[rows] if cfg.route != "learned" else None)
    out_g, out_o = g["out"][rows], o["out"]
    assert np.all(np.isfinite(out_g))
    scale = float(np.max(np.abs(out_o)))
    err = float(np.max(np.abs(out_g.astype(np.float64) - out_o)))
    # normwise; an all-zero reference (only zero tokens sampled) must be met exactly
    err = err / scale if scale > 0 else (0.0 if err == 0 else float("inf"))
    # h codes of the sampled pairs: equal except single steps at rounding boundaries
    S = k + 1 if cfg.shared else k
    n_h, n_bad, hd_rel = 0, 0, 0.0
    for i, t in enumerate(rows):
        for j in range(S):
            p = t * k + j if j < k else T * k + t
            hq_g, hq_o = g["hq"][p].astype(np.int32), o["hq"][i, j].astype(np.int32)
            diff = np.abs(hq_g - hq_o)
            assert diff.max() <= 1, "h codes differ by more than one step"
            n_h += diff.size
            n_bad += int(np.count_nonzero(diff))
            np.testing.assert_allclose(g["hd"][p], o["hd"][i, j], rtol=HD_RTOL, atol=0)
            nz = o["hd"][i, j] != 0
            if nz.any():
                rel = np.abs(g["hd"][p][nz].astype(np.float64) - o["hd"][i, j][nz]) / o["hd"][i, j][nz]
                hd_rel = max(hd_rel, float(rel.max()))
    assert n_bad <= max(2, n_h // 1000), f"{n_bad} of {n_h} h codes differ"
    # exact int32 block sums of sampled rows, for up to 12 of the checked
    # tokens (the first four, four from the middle, the last four)
    if stride:
        fmt = cfg.routed_fmt
        n = len(rows)
        pick = sorted(set(range(min(4, n))) | set(range(max(0, n // 2 - 2), min(n, n // 2 + 2))) |
                      set(range(max(0, n - 4), n)))
        for i in pick:
            t = rows[i]
            for j in range(S):
                p = t * k + j if j < k else T * k + t
                if j < k:
                    e = ids_o[t, j]
                    mats, f = (inp["gate"][e], inp["up"][e], inp["down"][e]), fmt
                else:
                    mats, f = (inp["sh_gate"], inp["sh_up"], inp["sh_down"]), "q8"
                nh = H // 32 if f == "q8" else H // 16
                nf = F // 32 if f == "q8" else F // 16
                for m, key in ((mats[0], "gate_sums"), (mats[1], "up_sums")):
                    want = oracle.block_sums(m, f, F, H, xq_o[t])[::stride]
                    assert np.array_equal(g[key][p][:, :nh], want), f"{key} differ (token {t}, slot {j})"
                want = oracle.block_sums(mats[2], f, H, F, np.ascontiguousarray(g["hq"][p]))[::stride]
                assert np.array_equal(g["down_sums"][p][:, :nf], want), f"down sums differ (token {t}, slot {j})"
    log(name or cfg.name, T=T, rows=len(rows), err=err, h_code_steps=n_bad, h_codes=n_h, hd_max_rel=hd_rel)
    assert err <= TOL, f"normwise output error {err:.3e} > {TOL}"


# ------------------------------------------------------------- small cases
SMALL = [
    ms.CONFIGS["tiny"],
    ms.LayerConfig("q8_learned_512", 512, 32, 4, 256, 7, seed=11),
    ms.LayerConfig("q8_learned_512_T32", 512, 32, 4, 256, 32, seed=12),
    ms.LayerConfig("q8_learned_512_T33", 512, 32, 4, 256, 33, seed=13),
    ms.LayerConfig("q8_learned_512_T100", 512, 32, 4, 256, 100, seed=14),
    ms.LayerConfig("q2_learned_512", 512, 32, 4, 512, 9, routed_fmt="q2", seed=15),
    ms.LayerConfig("q2_learned_1024_T40", 1024, 24, 3, 512, 40, routed_fmt="q2", seed=16),
    # 2-bit batches: the VALU kernels up to 63 tokens, the MFMA GEMMs from 64
    ms.LayerConfig("q2_learned_512_T33", 512, 32, 4, 512, 33, routed_fmt="q2", seed=68),
    ms.LayerConfig("q2_learned_512_T63", 512, 32, 4, 512, 63, routed_fmt="q2", seed=69),
    ms.LayerConfig("q2_mfma_512_T64", 512, 32, 4, 512, 64, routed_fmt="q2", seed=70),
    ms.LayerConfig("q8_hash_256", 256, 16, 2, 128, 3, route="hash", vocab=1000, seed=17),
    ms.LayerConfig("q8_hash_256_T50", 256, 16, 2, 128, 50, route="hash", vocab=1000, seed=18),
    ms.LayerConfig("q8_noshared_k1", 256, 8, 1, 256, 5, shared=False, seed=19),
    ms.LayerConfig("q8_all_experts", 256, 8, 8, 128, 6, seed=20),
    ms.LayerConfig("q8_nobias_T1", 1024, 64, 6, 512, 1, bias=False, seed=21),
    ms.LayerConfig("q8_hash_T1", 512, 32, 6, 256, 1, route="hash", vocab=300, seed=34),
    ms.LayerConfig("q2_learned_T1", 512, 32, 4, 512, 1, routed_fmt="q2", seed=35),
    ms.LayerConfig("q8_noshared_T1", 256, 16, 3, 128, 1, shared=False, seed=36),
    ms.LayerConfig("q2_hash_noshared_T1", 1024, 8, 2, 512, 1, routed_fmt="q2", route="hash", vocab=7, shared=False,
                   seed=37),
    ms.LayerConfig("q2_hash_T32", 512, 16, 6, 512, 32, routed_fmt="q2", route="hash", vocab=64, seed=22),
    ms.LayerConfig("q8_mfma_1024_T300", 1024, 16, 4, 512, 300, seed=26),
    ms.LayerConfig("q8_mfma_hash_T77", 512, 64, 6, 256, 77, route="hash", vocab=5000, seed=27),
    ms.LayerConfig("q8_mfma_noshared_T45", 256, 8, 3, 256, 45, shared=False, seed=28),
    # 2-bit routed experts on the MFMA GEMMs (the shared expert Q8 in the same launches)
    ms.LayerConfig("q2_mfma_512_T300", 512, 16, 4, 512, 300, routed_fmt="q2", seed=64),
    ms.LayerConfig("q2_mfma_hash_T77", 1024, 64, 6, 512, 77, routed_fmt="q2", route="hash", vocab=5000, seed=65),
    ms.LayerConfig("q2_mfma_noshared_T66", 512, 8, 3, 1024, 66, routed_fmt="q2", shared=False, seed=66),
    # routing variants: score-weighted hash, hash rows wider than top-k, 384 experts top-8
    ms.LayerConfig("q8_hashscored_T1", 512, 32, 6, 256, 1, route="hash_scored", vocab=300, seed=50),
    ms.LayerConfig("q8_hashscored_reduced_T9", 512, 32, 4, 256, 9, route="hash_scored", vocab=300, table_k=6,
                   seed=51),
    ms.LayerConfig("q8_hashscored_T70", 512, 64, 6, 256, 70, route="hash_scored", vocab=5000, seed=52),
    # the batched routing's two front ends: the decode front kernel up to 224 tokens, the tiled logits above
    ms.LayerConfig("q8_front_T224", 512, 64, 6, 256, 224, seed=71),
    ms.LayerConfig("q8_tiled_T225", 512, 64, 6, 256, 225, seed=72),
    ms.LayerConfig("q8_hashscored_T230", 512, 64, 6, 256, 230, route="hash_scored", vocab=5000, seed=73),
    ms.LayerConfig("q2_hash_reduced_T1", 512, 16, 4, 512, 1, routed_fmt="q2", route="hash", vocab=50, table_k=6,
                   seed=53),
    ms.LayerConfig("q8_hash_reduced_T40", 512, 32, 2, 256, 40, route="hash", vocab=400, table_k=6, seed=54),
    ms.LayerConfig("e384_top8_T1", 512, 384, 8, 256, 1, seed=55),
    ms.LayerConfig("e384_top8_T20", 512, 384, 8, 256, 20, seed=56),
    ms.LayerConfig("e384_top8_T100", 512, 384, 8, 256, 100, seed=57),
    # one token with more gate/up workgroups than CUs in the 64-row shape: the 32-row shape runs
    ms.LayerConfig("q8_narrow_T1", 512, 32, 4, 4096, 1, seed=58),
    ms.LayerConfig("q2_narrow_T1", 512, 16, 6, 4096, 1, routed_fmt="q2", seed=59),
    ms.LayerConfig("q8_hash_narrow_T1", 512, 16, 6, 4096, 1, route="hash", vocab=7, seed=62),
    # the remaining compiled widths: hidden 128 (one-lane router segments, Q8
    # only, VALU experts at every batch), hidden 2048 and ffn 1024 (every
    # expert kernel family at K = 2048 and 1024, Q8 and 2-bit), ffn 4096 on
    # the MFMA down GEMM
    ms.LayerConfig("q8_h128_T1", 128, 16, 2, 256, 1, seed=80),
    ms.LayerConfig("q8_h128_T6", 128, 16, 4, 128, 6, seed=81),
    ms.LayerConfig("q8_h128_T40", 128, 16, 2, 256, 40, seed=82),
    ms.LayerConfig("q8_h128_hash_T300", 128, 16, 2, 128, 300, route="hash", vocab=2000, seed=83),
    ms.LayerConfig("q8_h2048_f1024_T1", 2048, 32, 4, 1024, 1, seed=84),
    ms.LayerConfig("q8_h2048_f1024_T12", 2048, 32, 4, 1024, 12, seed=85),
    ms.LayerConfig("q8_h2048_f1024_T96", 2048, 32, 4, 1024, 96, seed=86),
    ms.LayerConfig("q2_h2048_f1024_T1", 2048, 16, 4, 1024, 1, routed_fmt="q2", seed=87),
    ms.LayerConfig("q2_h2048_f1024_T20", 2048, 16, 4, 1024, 20, routed_fmt="q2", seed=88),
    ms.LayerConfig("q2_h2048_f1024_T80", 2048, 16, 4, 1024, 80, routed_fmt="q2", seed=89),
    ms.LayerConfig("q8_f4096_T70", 512, 16, 2, 4096, 70, seed=90),
    ms.LayerConfig("q8_h4096_f1024_T1", 4096, 16, 2, 1024, 1, seed=91),
    # expert counts that fill no tile or wave evenly, and learned top-1
    ms.LayerConfig("e100_top5_T1", 512, 100, 5, 256, 1, seed=110),
    ms.LayerConfig("e100_top5_T7", 512, 100, 5, 256, 7, seed=111),
    ms.LayerConfig("e100_top5_T230", 512, 100, 5, 256, 230, seed=112),
    ms.LayerConfig("q2_e100_hash_T33", 512, 100, 5, 512, 33, routed_fmt="q2", route="hash", vocab=500, seed=113),
    ms.LayerConfig("top1_T1", 512, 16, 1, 256, 1, seed=114),
    ms.LayerConfig("top1_T70", 512, 16, 1, 256, 70, seed=115),
    # the one-token down kernel's widest instances: ffn 4096 with eight routed slots
    ms.LayerConfig("q8_top8_f4096_T1", 512, 32, 8, 4096, 1, seed=92),
    ms.LayerConfig("q2_top8_f4096_T1", 512, 32, 8, 4096, 1, routed_fmt="q2", seed=93),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_parity(cfg):
    inp, layer = case(cfg)
    g = run_gpu(cfg, inp, layer, stride=1)
    check(cfg, inp, g, stride=1)


@pytest.mark.parametrize("T,fmt", [(1, "q8"), (6, "q8"), (40, "q8"), (300, "q8"), (1, "q2"), (80, "q2")])
def test_degenerate_activations(T, fmt):
    """Blocks whose quantization scale is zero and saturated routing, on each
    path: a token of zeros (every x and h block has amax 0, so d = 0 and every
    code 0; its output is exactly zero), two zero 32-blocks inside another
    token, and tokens scaled by 1e3 (router sigmoids saturate to 0 or 1, gate
    values far below -89 give h = -0)."""
    cfg = ms.LayerConfig(f"degenerate_{fmt}_T{T}", 512, 16, 4, 512, T, routed_fmt=fmt, seed=95 + T)
    inp = ms.make_inputs(cfg)
    x = inp["x"].copy()
    x[0] = 0.0
    if T > 1:
        x[1, 32:96] = 0.0
    if T > 2:
        x[2:T:3] *= 1000.0
    layer = _qr().MoELayer(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared, cfg.routed_fmt, cfg.route,
                           0).load(inp)
    g = run_gpu(cfg, inp, layer, x=x, stride=1)
    check(cfg, inp, g, x=x, stride=1)
    assert not np.any(g["out"][0]), "a zero token's output is exactly zero"
    assert not np.any(g["xq"][0]) and not np.any(g["xd"][0])


def test_every_token_to_the_same_experts():
    """Hash table with one row: all tokens hit the same k experts (groups split per 8 tokens)."""
    cfg = ms.LayerConfig("hash_one_row", 512, 16, 6, 256, 32, route="hash", vocab=1, seed=23)
    inp, layer = case(cfg)
    g = run_gpu(cfg, inp, layer, stride=4)
    assert sorted(np.nonzero(g["counts"])[0].tolist()) == sorted(inp["hash_table"][0].tolist())
    check(cfg, inp, g, stride=4)


def test_skewed_bias_sends_all_tokens_to_one_expert():
    cfg = ms.LayerConfig("skew", 256, 16, 2, 128, 64, seed=24)
    inp = ms.make_inputs(cfg)
    inp["router_b"][5] = 10.0  # expert 5 wins every token
    layer = _qr().MoELayer(256, 16, 2, 128).load(inp)
    g = run_gpu(cfg, inp, layer, stride=2)
    assert g["counts"][5] == 64
    check(cfg, inp, g, stride=2, name="skew")


def test_skewed_bias_mfma_tiles():
    """One expert takes every token: 200 pairs cut into four 64-pair MFMA tiles (last one ragged)."""
    cfg = ms.LayerConfig("skew_mfma", 512, 16, 2, 256, 200, seed=29)
    inp = ms.make_inputs(cfg)
    inp["router_b"][3] = 10.0
    layer = _qr().MoELayer(512, 16, 2, 256).load(inp)
    g = run_gpu(cfg, inp, layer, stride=4)
    assert g["counts"][3] == 200
    check(cfg, inp, g, stride=4, name="skew_mfma")


@pytest.mark.parametrize("skew", [False, True])
def test_chunked_sort_ragged_and_skewed(skew):
    """4400 pairs: the sort runs as per-chunk histograms, one prefix workgroup and
    a per-chunk stable scatter (five 1024-pair chunks, the last one ragged);
    with a bias that gives one expert every token, that expert's pairs span
    every chunk."""
    cfg = ms.LayerConfig("sort_chunks_skew" if skew else "sort_chunks", 256, 64, 4, 256, 1100, seed=60 + skew)
    inp = ms.make_inputs(cfg)
    if skew:
        inp["router_b"][9] = 10.0
    layer = _qr().MoELayer(256, 64, 4, 256).load(inp)
    g = run_gpu(cfg, inp, layer, stride=8)
    if skew:
        assert g["counts"][9] == 1100
    check(cfg, inp, g, rows=np.r_[0:6, 500:506, 1094:1100], stride=8, name=cfg.name)


@pytest.mark.parametrize("T", [1, 7, 12, 40])
def test_tied_keys_take_the_smaller_expert_ids(T):
    """Experts share router rows and biases in groups of four, so every
    token's top-6 boundary falls inside a group of equal keys: the two
    smaller ids of that group are taken (decode select for T <= 32, the
    batched select above)."""
    cfg = ms.LayerConfig(f"ties_T{T}", 512, 64, 6, 256, T, seed=33)
    inp = ms.make_inputs(cfg)
    inp["router_w"] = np.ascontiguousarray(np.repeat(inp["router_w"][::4], 4, axis=0))
    inp["router_b"] = np.ascontiguousarray(np.repeat(inp["router_b"][::4], 4))
    layer = _qr().MoELayer(512, 64, 6, 256).load(inp)
    g = run_gpu(cfg, inp, layer, stride=4)
    groups = g["ids"].reshape(T, 6) // 4
    for row in groups:  # one whole group of four plus two of the next
        assert sorted(np.bincount(row).tolist())[-2:] == [2, 4], row
    check(cfg, inp, g, stride=4, name=f"ties_T{T}")


@pytest.mark.parametrize("fmt", ["q8", "q2"])
def test_max_tokens_small_shape(fmt):
    """The largest batch, 16,384 tokens: Q8 on the VALU kernels (F = 128),
    2-bit experts on the MFMA GEMMs (H = F = 512)."""
    cfg = (ms.LayerConfig("max_tokens", 256, 16, 2, 128, 16384, seed=25) if fmt == "q8" else
           ms.LayerConfig("max_tokens_q2", 512, 16, 2, 512, 16384, routed_fmt="q2", seed=67))
    inp, layer = case(cfg)
    g = run_gpu(cfg, inp, layer, stride=32)
    rows = np.r_[0:3, 8191:8194, 16381:16384]
    check(cfg, inp, g, rows=rows, stride=32)


def test_empty_batch_is_a_no_op():
    qr = _qr()
    cfg = ms.CONFIGS["tiny"]
    inp, layer = case(cfg)
    x = torch.empty((0, cfg.hidden), dtype=torch.float32, device="cuda")
    out = torch.empty((0, cfg.hidden), dtype=torch.float32, device="cuda")
    layer.ensure_workspace(1)
    qr.layer_forward(layer.shape, layer.weights(), x, None, out, layer.ws)


# ------------------------------------------------ determinism / batching
@pytest.mark.parametrize("cfg", [ms.LayerConfig("batch_learned", 512, 32, 4, 256, 12, seed=31),
                                 ms.LayerConfig("batch_learned_T3", 1024, 64, 6, 512, 3, seed=36),
                                 ms.LayerConfig("batch_hash", 512, 32, 4, 256, 12, route="hash", vocab=300,
                                                seed=32),
                                 ms.LayerConfig("batch_q2_T32", 512, 32, 4, 512, 32, routed_fmt="q2", seed=35),
                                 ms.LayerConfig("batch_q2_T40", 512, 32, 4, 512, 40, routed_fmt="q2", seed=35)],
                         ids=lambda c: c.name)
def test_batched_equals_single_token_calls_bitwise(cfg):
    """Batches the VALU expert kernels serve (up to 32 tokens; 2-bit experts up
    to 63, past 32 with the batched routing kernels) give every token the bits
    of a one-token call.  (Batches on the MFMA GEMMs accumulate in another
    order; they are held to the oracle tolerance.)"""
    inp, layer = case(cfg)
    x = torch.from_numpy(inp["x"]).cuda()
    tok = torch.from_numpy(inp["token_ids"]).cuda() if cfg.route != "learned" else None
    full = layer.forward(x, tok).clone()
    again = layer.forward(x, tok).clone()
    assert torch.equal(full.view(torch.int32), again.view(torch.int32)), "two identical calls differ"
    for t in range(cfg.tokens):
        one = layer.forward(x[t:t + 1].contiguous(), tok[t:t + 1].contiguous() if tok is not None else None)
        assert torch.equal(one.view(torch.int32), full[t:t + 1].view(torch.int32)), f"token {t} differs"


# --------------------------------------------------------- error paths
def test_out_of_range_token_id_is_flagged_not_faulted():
    cfg = ms.LayerConfig("bad_token", 256, 16, 2, 128, 4, route="hash", vocab=100, seed=33)
    inp, layer = case(cfg)
    x = torch.from_numpy(inp["x"]).cuda()
    tok = torch.tensor([1, 2, 100, -5], dtype=torch.int32, device="cuda")
    out = layer.forward(x, tok)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert layer.flags() & 1


def test_out_of_range_token_id_is_flagged_one_token():
    cfg = ms.LayerConfig("bad_token_T1", 256, 16, 2, 128, 1, route="hash", vocab=100, seed=38)
    inp, layer = case(cfg)
    x = torch.from_numpy(inp["x"]).cuda()
    layer.forward(x, torch.tensor([7], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert layer.flags() == 0
    out = layer.forward(x, torch.tensor([100], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert layer.flags() & 1


@pytest.mark.parametrize("fmt", ["q8", "q2"])
def test_mfma_tile_boundaries(fmt):
    """Hash routing, top-1, with a table that gives experts exactly 1, 31, 32,
    33, 63, 64, 65 and 129 tokens (the others none), in shuffled token order:
    every shape of the MFMA GEMMs' 64-pair tiles (one or both 32-pair halves
    live, ragged, several tiles per expert, empty experts between them) and the
    shared expert's ragged last tile, against the oracle with exact block sums
    (Q8 blocks, or 2-bit subblocks)."""
    qr = _qr()
    counts = [1, 31, 32, 33, 63, 64, 65, 129]
    T = sum(counts)
    F = 256 if fmt == "q8" else 512
    cfg = ms.LayerConfig(f"{fmt}_mfma_tile_edges", 512, 16, 1, F, T, routed_fmt=fmt, route="hash", vocab=T,
                         seed=63)
    inp = ms.make_inputs(cfg)
    order = np.random.default_rng(63).permutation(T).astype(np.int32)
    experts = np.repeat(2 * np.arange(len(counts)), counts).astype(np.int32)
    inp["hash_table"] = np.empty((T, 1), dtype=np.int32)
    inp["hash_table"][order, 0] = experts
    inp["token_ids"] = np.arange(T, dtype=np.int32)
    layer = qr.MoELayer(512, 16, 1, F, True, fmt, "hash", T).load(inp)
    g = run_gpu(cfg, inp, layer, stride=8)
    assert np.array_equal(g["counts"][::2][:len(counts)], counts)
    check(cfg, inp, g, rows=np.arange(0, T, 3), stride=8)


def test_repeated_expert_in_an_unchecked_hash_row():
    """A table row naming one expert twice (rejected by the table check, used
    anyway): one-token calls and a batched call agree bit for bit, the work
    list holds the repeated expert once with two pairs, and every call that
    routes a token through that row sets the repeated-expert flag."""
    qr = _qr()
    cfg = ms.LayerConfig("hash_dup", 512, 16, 4, 256, 6, route="hash", vocab=8, seed=39)
    inp = ms.make_inputs(cfg)
    inp["hash_table"][3] = np.array([5, 9, 5, 2], dtype=np.int32)
    layer = qr.MoELayer(512, 16, 4, 256, True, "q8", "hash", 8).load(inp)
    x = torch.from_numpy(inp["x"]).cuda()
    tok = torch.tensor([3, 1, 3, 0, 3, 7], dtype=torch.int32, device="cuda")
    batched = layer.forward(x, tok).clone()
    torch.cuda.synchronize()
    assert layer.flags() == qr.FLAG_REPEATED_EXPERT
    for t in range(cfg.tokens):
        layer.reset_flags()
        one = layer.forward(x[t:t + 1].contiguous(), tok[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(one.view(torch.int32), batched[t:t + 1].view(torch.int32)), f"token {t}"
        assert layer.flags() == (qr.FLAG_REPEATED_EXPERT if int(tok[t]) == 3 else 0), f"token {t}"
    r = layer.forward_debug(x[0:1].contiguous(), tok[0:1].contiguous())
    torch.cuda.synchronize()
    assert r["counts"].cpu().numpy()[5] == 2 and int((r["counts"] > 0).sum()) == 3
    assert torch.isfinite(batched).all()


@pytest.mark.parametrize("T", [1, 6, 40])
def test_repeated_expert_flag_each_selection_path(T):
    """The repeated-expert flag on each hash selection path: one token (in the
    gate/up kernel), a decode batch (the one-workgroup select) and a batch past
    the decode sizes (one wave per token); a table of distinct rows leaves the
    flags clear."""
    qr = _qr()
    cfg = ms.LayerConfig(f"hash_dup_T{T}", 512, 16, 4, 256, T, route="hash", vocab=64, seed=40 + T)
    inp = ms.make_inputs(cfg)
    layer = qr.MoELayer(512, 16, 4, 256, True, "q8", "hash", 64).load(inp)
    x = torch.from_numpy(inp["x"]).cuda()
    tok = torch.from_numpy(inp["token_ids"]).cuda()
    layer.forward(x, tok)
    torch.cuda.synchronize()
    assert layer.flags() == 0
    bad = inp["hash_table"].copy()
    row = int(inp["token_ids"][T - 1])
    bad[row, 3] = bad[row, 1]
    layer.hash_table = torch.from_numpy(bad).cuda()
    layer.forward(x, tok)
    torch.cuda.synchronize()
    assert layer.flags() == qr.FLAG_REPEATED_EXPERT


@pytest.mark.parametrize("T", [1, 5])
def test_score_weighted_hash_clamps_like_the_selection(T):
    """Score-weighted hash with an out-of-range token id and a table entry out
    of range (an unchecked table): the product call, whose router computes
    only the logits of the table's experts, clamps both as the selection does
    and equals the debug call (every logit computed) bit for bit; both
    conditions are flagged."""
    qr = _qr()
    cfg = ms.LayerConfig(f"hash_scored_clamp_T{T}", 512, 32, 4, 256, T, route="hash_scored", vocab=50,
                         seed=60 + T)
    inp = ms.make_inputs(cfg)
    inp["hash_table"][7] = np.array([3, 40, 9, 1], dtype=np.int32)  # expert 40 >= 32 experts
    layer = qr.MoELayer(512, 32, 4, 256, True, "q8", "hash_scored", 50).load(inp)
    tok = inp["token_ids"].copy()
    tok[0] = 7
    if T > 1:
        tok[T - 1] = 50  # token id >= vocab
    x = torch.from_numpy(inp["x"]).cuda()
    tt = torch.from_numpy(tok).cuda()
    r = layer.forward_debug(x, tt)
    plain = layer.forward(x, tt)
    torch.cuda.synchronize()
    assert torch.isfinite(plain).all()
    assert torch.equal(plain.view(torch.int32), r["out"].view(torch.int32))
    assert layer.flags() & qr.FLAG_BAD_TABLE_ENTRY
    if T > 1:
        assert layer.flags() & qr.FLAG_BAD_TOKEN


def test_check_hash_table():
    qr = _qr()
    cfg = ms.LayerConfig("table", 256, 16, 2, 128, 4, route="hash", vocab=1000, seed=34)
    inp, layer = case(cfg)
    assert layer.check_table() == -1
    bad = inp["hash_table"].copy()
    bad[777, 1] = bad[777, 0]
    layer.hash_table = torch.from_numpy(bad).cuda()
    with pytest.raises(qr.MoEError) as ei:
        layer.check_table()
    assert "777" in str(ei.value)
    layer.hash_table = torch.from_numpy(inp["hash_table"]).cuda()


# ------------------------------------------------------ full-size layers
@pytest.mark.slow
@pytest.mark.parametrize("name", ["decode_q8", "decode_q2", "hash_decode", "decode_topk4", "hash_scored_decode",
                                  "decode_motif3"])
def test_full_size_decode(name):
    cfg = ms.CONFIGS[name]
    inp, layer = case(cfg)
    g = run_gpu(cfg, inp, layer, stride=64)
    check(cfg, inp, g, stride=64)


@pytest.mark.slow
@pytest.mark.parametrize("T", [2048, 4096, 8192])
def test_full_size_prefill(T):
    """Prefill chunks of 2048, 4096 and 8192 tokens over the same layer (the
    larger ones take further rows of the same x stream): routing, x
    quantization and the sort of every token bit-exact; the outputs of every
    token at 2048 (the oracle's whole chunk) and of sampled tokens at 4096 and
    8192, with exact block sums of sampled rows."""
    cfg = ms.CONFIGS["prefill"]
    inp, layer = case(cfg)
    x = inp["x"] if T == cfg.tokens else ms.extra_tokens(cfg, T)
    g = run_gpu(cfg, inp, layer, x=x, stride=128)
    rows = None
    if T != cfg.tokens:
        rows = np.unique(np.r_[0, 1, 2, T // 4, T // 2, T - 2, T - 1, np.arange(37, T, T // 12)])
    check(cfg, inp, g, x=x, rows=rows, stride=128, name=f"prefill_T{T}")
    assert np.count_nonzero(g["counts"]) > 0


@pytest.mark.slow
def test_full_size_prefill_q2_sampled():
    """The 2048-token prefill chunk with 2-bit routed experts (Q8 shared expert)
    on the MFMA GEMMs: routing, x quantization and the sort bit-exact, outputs
    and exact 16-subblock sums of sampled tokens."""
    cfg = ms.CONFIGS["prefill_q2"]
    inp, layer = case(cfg)
    T = cfg.tokens
    g = run_gpu(cfg, inp, layer, stride=128)
    rows = np.r_[0, 1, 2, T // 4, T // 2, T - 2, T - 1, np.arange(37, T, T // 12)]
    check(cfg, inp, g, rows=np.unique(rows), stride=128)
    assert np.count_nonzero(g["counts"]) > 0


# ------------------------------------------------------- graph replay
@pytest.mark.parametrize("cfg", [ms.LayerConfig("graph_T1", 512, 32, 4, 256, 1, seed=41),
                                 ms.LayerConfig("graph_T7_hash", 512, 32, 4, 256, 7, route="hash", vocab=99, seed=42),
                                 ms.LayerConfig("graph_T40", 512, 32, 4, 256, 40, seed=43),
                                 ms.LayerConfig("graph_q2_T70", 512, 32, 4, 512, 70, routed_fmt="q2", seed=44)],
                         ids=lambda c: c.name)
def test_graph_replay_matches_eager(cfg):
    """The layer captured in a HIP graph replays to the eager result, replay after replay,
    with eager work and synchronisations in between (nothing in the path is a memset node)."""
    qr = _qr()
    inp, layer = case(cfg)
    x = torch.from_numpy(inp["x"]).cuda()
    tok = torch.from_numpy(inp["token_ids"]).cuda() if cfg.route != "learned" else None
    want = layer.forward(x, tok).clone()
    out = torch.empty_like(want)
    layer.ensure_workspace(cfg.tokens)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qr.layer_forward(layer.shape, layer.weights(), x, tok, out, layer.ws, torch.cuda.current_stream())
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), f"replay {i} differs"
        other = layer.forward(x, tok)          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int32), want.view(torch.int32))
