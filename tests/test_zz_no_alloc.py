"""moe_layer_forward_static, the entry point for callers that cannot
allocate, through the C ABI: its output equals moe_layer_forward's bit for
bit on the same inputs (both run the same kernels; only the workspace
differs), on two calls in a row whose second batch is the smaller one, and
stays within the oracle's tolerance.  Also replayed from a captured HIP graph."""
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


# (config, the two batch sizes in call order): a batch on the MFMA GEMMs then a
# decode batch, a hash-routed decode batch then one token, 2-bit experts on
# the GEMMs then on the VALU kernels, and the full-size decode layer
CASES = [
    (ms.LayerConfig("static_learned", 1024, 64, 6, 512, 40, seed=120), (40, 7)),
    (ms.LayerConfig("static_hash", 512, 32, 4, 256, 20, route="hash", vocab=300, seed=121), (20, 1)),
    (ms.LayerConfig("static_q2", 512, 32, 4, 512, 70, routed_fmt="q2", seed=122), (70, 33)),
    (ms.CONFIGS["decode_q8"].with_(tokens=8), (8, 1)),
]


@pytest.mark.parametrize("cfg,sizes", CASES, ids=[c.name for c, _ in CASES])
def test_static_forward_equals_workspace_forward(cfg, sizes):
    qr = _qr()
    inp = ms.make_inputs(cfg)
    layer = qr.MoELayer(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.shared, cfg.routed_fmt, cfg.route,
                        cfg.vocab if cfg.route != "learned" else 0, table_k=cfg.table_k).load(inp)
    x_all = torch.from_numpy(inp["x"]).cuda()
    tok_all = torch.from_numpy(inp["token_ids"]).cuda() if cfg.route != "learned" else None
    w = layer.weights()
    for T in sizes:
        print(f"{cfg.name}: static forward of {T} tokens", flush=True)
        x = x_all[:T].contiguous()
        tok = tok_all[:T].contiguous() if tok_all is not None else None
        got = torch.full((T, cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
        qr.layer_forward_static(layer.shape, w, x, tok, got)
        want = layer.forward(x, tok)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), f"{T} tokens differ"
        o = oracle.forward(cfg, inp, x=inp["x"][:T], token_ids=inp["token_ids"][:T] if tok is not None else None)
        err = float(np.max(np.abs(got.cpu().numpy().astype(np.float64) - o["out"])) / np.max(np.abs(o["out"])))
        assert err <= TOL, err


def test_static_forward_graph_replay():
    """Captured into a HIP graph, the static call replays to the eager bits,
    replay after replay, with eager calls of the same entry point between."""
    qr = _qr()
    cfg = ms.LayerConfig("static_graph", 512, 32, 4, 256, 5, seed=123)
    inp = ms.make_inputs(cfg)
    layer = qr.MoELayer(512, 32, 4, 256).load(inp)
    x = torch.from_numpy(inp["x"]).cuda()
    w = layer.weights()
    want = layer.forward(x).clone()
    out = torch.empty_like(want)
    qr.layer_forward_static(layer.shape, w, x, None, out)   # first call on the device: outside the capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qr.layer_forward_static(layer.shape, w, x, None, out, torch.cuda.current_stream())
    other = torch.empty_like(want)
    for i in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), f"replay {i}"
        qr.layer_forward_static(layer.shape, w, x[:2].contiguous(), None, other[:2])
        torch.cuda.synchronize()
        assert torch.equal(other[:2].view(torch.int32), layer.forward(x[:2].contiguous()).view(torch.int32))
