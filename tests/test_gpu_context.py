"""The library-owned layer (moe_ctx_create / moe_prepare / moe_ctx_forward /
moe_ctx_flags / moe_ctx_destroy) through the C ABI: the context packs the
canonical weights itself and then computes the same bits as the
caller-workspace call on weights packed by moe_pack_weights, within the
oracle's tolerance; a table that names an expert twice is refused at
prepare, and forward refuses to run until a prepare succeeded."""
import numpy as np
import pytest

import moe_synth as ms
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL = 2e-3


def _qr():
    import quantized_routed_moe_amd as qr
    return qr


def upload_canonical(inp, cfg):
    """Canonical weight bytes on the device, and the moe_weights struct of their pointers."""
    qr = _qr()
    keep = {}

    def dev(name):
        if name not in inp or inp[name] is None:
            return None
        keep[name] = torch.from_numpy(np.ascontiguousarray(inp[name])).cuda()
        return keep[name].data_ptr()

    w = qr.Weights(dev("router_w") if cfg.route != "hash" else None,
                   dev("router_b") if cfg.route == "learned" else None,
                   dev("hash_table") if cfg.route != "learned" else None,
                   dev("gate"), dev("up"), dev("down"),
                   dev("sh_gate") if cfg.shared else None, dev("sh_up") if cfg.shared else None,
                   dev("sh_down") if cfg.shared else None)
    return w, keep


def make_ctx(cfg, inp, max_tokens):
    qr = _qr()
    shape = qr.make_shape(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared, cfg.routed_fmt, cfg.route,
                          cfg.vocab if cfg.route != "learned" else 0, cfg.table_k)
    ctx = qr.Context(shape, max_tokens)
    w, keep = upload_canonical(inp, cfg)
    ctx.prepare(w)
    del keep
    return ctx


CASES = [
    ms.CONFIGS["tiny"],
    ms.LayerConfig("ctx_q8_T1", 512, 32, 4, 256, 1, seed=101),
    ms.LayerConfig("ctx_hash_T7", 512, 32, 4, 256, 7, route="hash", vocab=300, seed=102),
    ms.LayerConfig("ctx_q2_T70", 512, 32, 4, 512, 70, routed_fmt="q2", seed=103),
    ms.LayerConfig("ctx_hashscored_T1", 512, 32, 6, 256, 1, route="hash_scored", vocab=300, seed=104),
    ms.LayerConfig("ctx_nobias_noshared_T40", 256, 16, 2, 256, 40, bias=False, shared=False, seed=105),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_context_forward_equals_caller_workspace_forward(cfg):
    qr = _qr()
    inp = ms.make_inputs(cfg)
    layer = qr.MoELayer(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared, cfg.routed_fmt, cfg.route,
                        cfg.vocab if cfg.route != "learned" else 0, table_k=cfg.table_k).load(inp)
    ctx = make_ctx(cfg, inp, max_tokens=cfg.tokens + 5)
    x = torch.from_numpy(inp["x"]).cuda()
    tok = torch.from_numpy(inp["token_ids"]).cuda() if cfg.route != "learned" else None
    want = layer.forward(x, tok)
    got = torch.empty_like(want)
    ctx.forward(x, tok, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
    o = oracle.forward(cfg, inp)
    err = float(np.max(np.abs(got.cpu().numpy().astype(np.float64) - o["out"])) / np.max(np.abs(o["out"])))
    assert err <= TOL, err
    assert ctx.flags() == 0
    ctx.close()


def test_prepare_refuses_a_table_with_a_repeated_expert():
    qr = _qr()
    cfg = ms.LayerConfig("ctx_bad_table", 512, 16, 4, 256, 5, route="hash", vocab=50, seed=106)
    inp = ms.make_inputs(cfg)
    shape = qr.make_shape(512, 16, 4, 256, True, "q8", "hash", 50)
    ctx = qr.Context(shape, 8)
    x = torch.from_numpy(inp["x"]).cuda()
    tok = torch.from_numpy(inp["token_ids"]).cuda()
    out = torch.empty((5, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(qr.MoEError) as ei:
        ctx.forward(x, tok, out)          # nothing prepared yet
    assert ei.value.status == -8
    bad = dict(inp)
    bad["hash_table"] = inp["hash_table"].copy()
    bad["hash_table"][17, 2] = bad["hash_table"][17, 0]
    w, keep = upload_canonical(bad, cfg)
    with pytest.raises(qr.MoEError) as ei:
        ctx.prepare(w)
    assert ei.value.status == -6
    with pytest.raises(qr.MoEError) as ei:
        ctx.forward(x, tok, out)          # the refused prepare left the context unprepared
    assert ei.value.status == -8
    w, keep = upload_canonical(inp, cfg)
    ctx.prepare(w)
    ctx.forward(x, tok, out)
    torch.cuda.synchronize()
    o = oracle.forward(cfg, inp)
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - o["out"])) / np.max(np.abs(o["out"])))
    assert err <= TOL
    ctx.close()


def test_context_limits_flags_and_reprepare():
    """max_tokens is enforced; an out-of-range token id sets the context's flag
    and a reset clears it; a second prepare with other weights replaces the
    first in place."""
    qr = _qr()
    cfg = ms.LayerConfig("ctx_reprep", 512, 16, 2, 256, 6, route="hash", vocab=40, seed=107)
    inp = ms.make_inputs(cfg)
    ctx = make_ctx(cfg, inp, max_tokens=6)
    x = torch.from_numpy(ms.extra_tokens(cfg, 7)).cuda()
    tok = torch.from_numpy(inp["token_ids"]).cuda()
    out = torch.empty((7, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(qr.MoEError) as ei:
        ctx.forward(x, torch.cat([tok, tok[:1]]), out)
    assert ei.value.status == -3
    bad_tok = tok.clone()
    bad_tok[2] = 40
    ctx.forward(x[:6], bad_tok, out[:6])
    assert ctx.flags(reset=True) == qr.FLAG_BAD_TOKEN
    assert ctx.flags() == 0
    other = ms.make_inputs(cfg.with_(seed=108))
    other["token_ids"] = inp["token_ids"]
    w, keep = upload_canonical(other, cfg)
    ctx.prepare(w)
    ctx.forward(x[:6], tok, out[:6])
    layer = qr.MoELayer(512, 16, 2, 256, True, "q8", "hash", 40).load(other)
    want = layer.forward(x[:6], tok)
    torch.cuda.synchronize()
    assert torch.equal(out[:6].view(torch.int32), want.view(torch.int32))
    ctx.close()
