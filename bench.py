#!/usr/bin/env python3
"""Throughput of the routed-MoE layer on one MI355X.

A step is one call of the whole layer (routing, quantization, token sort,
expert gate/up + SwiGLU, down projection and weighted combine) on one batch
of synthetic tokens whose inputs are already resident in HBM.  The default
workload is the Q8 decode layer (1 token, hidden 4096, 256 experts top-6 +
1 shared, FFN 2048).  Prints ONE JSON line.

Timing: W eager warm-up steps, then the K timed steps are replayed from a
captured HIP graph (per-call host overhead excluded, as in a captured decode
loop); every step uses a different token and one of R address-distinct copies
of the weights every step re-reads (router, shared expert), so the 256 MB
Infinity Cache cannot serve them across steps.  A second, eager pass with
HIP events around each kernel gives the per-kernel durations used for the
roofline entry.  The CPU oracle is then timed on a bounded sample of the same
workload on the host cores.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (TOP/s)
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="decode_q8")
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--graph-steps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (for scaling rocprofv3 byte counters)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported by this build "
              "(multi-GPU expert parallelism is designed, not built)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import moe_synth as ms
    import quantized_routed_moe_amd as qr

    cfg = ms.CONFIGS[args.config]
    T, H, E, k, F = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn
    fmt = qr.FMT[cfg.routed_fmt]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    t_setup = time.time()
    inp = ms.make_inputs(cfg)
    layer = qr.MoELayer(H, E, k, F, cfg.shared, cfg.routed_fmt, cfg.route,
                        cfg.vocab if cfg.route == "hash" else 0).load(inp)
    R = max(1, args.replicas)
    reps = []
    for r in range(R):
        if r == 0:
            reps.append((layer.router_w, (layer.sh_gate, layer.sh_up, layer.sh_down)))
        else:
            rw = layer.router_w.clone() if layer.router_w is not None else None
            reps.append((rw, (layer.sh_gate.clone(), layer.sh_up.clone(), layer.sh_down.clone())))
    wlist = [layer.weights(router_w=rw, sh=sh) for rw, sh in reps]
    G = max(1, min(args.graph_steps, args.steps))
    n_steps = args.warmup + G
    xs = torch.from_numpy(ms.extra_tokens(cfg, n_steps * T)).to(dev).reshape(n_steps, T, H)
    toks = None
    if cfg.route == "hash":
        toks = torch.from_numpy(ms.uniform_i32(n_steps * T, 0, cfg.vocab - 1, cfg.seed,
                                               ms.TAG["token_ids"])).to(dev).reshape(n_steps, T)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = layer.ensure_workspace(T)

    def step(i, stream=None):
        qr.layer_forward(layer.shape, wlist[i % R], xs[i], toks[i] if toks is not None else None, out, ws, stream)

    # distinct experts each step touches (for the algorithmic byte counts)
    used = []
    for i in range(n_steps):
        r = layer.forward_debug(xs[i], toks[i] if toks is not None else None)
        used.append(int(torch.count_nonzero(r["counts"]).item()))
    torch.cuda.synchronize()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # capture G steps in one graph, check a replay against eager, then time K steps of replays
    gs = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        for i in range(G):
            step(args.warmup + i, torch.cuda.current_stream())
    graph.replay()
    torch.cuda.synchronize()
    replay_out = out.clone()
    step(args.warmup + G - 1)
    torch.cuda.synchronize()
    if not torch.equal(replay_out.view(torch.int32), out.view(torch.int32)):
        raise RuntimeError("graph replay differs from the eager call")
    replays = max(1, math.ceil(args.steps / G))
    K = replays * G
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    value = K * T / (t1 - t0)

    # eager region (host launch overhead included), then eager with per-kernel events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(args.warmup + i % G)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / K
    KP = min(K, 300)
    prof = qr.Profiler(max_events=8 * KP + 64)
    prof.attach()
    for i in range(KP):
        step(args.warmup + i % G)
    prof.detach()
    torch.cuda.synchronize()
    stages = prof.collect()
    prof.close()

    # algorithmic bytes per launch of each stage
    mq8 = qr.matrix_bytes(qr.FMT_Q8, F, H)
    mr_gu, mr_dn = qr.matrix_bytes(fmt, F, H), qr.matrix_bytes(fmt, H, F)
    sh = 1 if cfg.shared else 0
    P = T * k + sh * T
    u_avg = float(np.mean([used[args.warmup + i % G] for i in range(K)]))
    act_x = T * H + T * (H // 32) * 4
    act_h = P * F + P * (F // 32) * 4
    stage_bytes = {
        "route": (E * H * 4 if cfg.route == "learned" else T * k * 4) + T * H * 4 + act_x,
        "gateup": u_avg * 2 * mr_gu + sh * 2 * mq8 + act_x + act_h,
        "down": u_avg * mr_dn + sh * qr.matrix_bytes(qr.FMT_Q8, H, F) + act_h + T * H * 4,
    }
    layer_bytes = (u_avg * (2 * mr_gu + mr_dn) + sh * (2 * mq8 + qr.matrix_bytes(qr.FMT_Q8, H, F))
                   + (E * H * 4 if cfg.route == "learned" else 0) + 2 * T * H * 4)
    dom = max(stages, key=lambda s: stages[s][0])
    dom_us = stages[dom][0] / stages[dom][1] * 1e3
    dom_bytes = stage_bytes.get(dom)
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": round(dom_bytes / (dom_us * 1e-6) / 1e9, 1) if dom_bytes else None,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(dom_bytes / (dom_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) if dom_bytes else None,
        "traffic": None,
        "avg_launch_us": round(dom_us, 3),
        "algorithmic_bytes_per_launch": int(dom_bytes) if dom_bytes else None,
    }

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {T} token(s)/step, hidden {H}, {E} experts top-{k}"
                        f"{' + 1 shared' if cfg.shared else ''}, FFN {F}, routed {cfg.routed_fmt.upper()} "
                        f"(shared Q8), {cfg.route} routing",
            "tokens_per_step": T,
            "parallelism": "single GPU",
            "weight_replicas": R,
            "timing": f"HIP-graph replay of {G}-step graphs",
        },
        "layer_gbps": round(layer_bytes / (ms_step * 1e-3) / 1e9, 1),
        "layer_hbm_frac": round(layer_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "eager_ms_per_step": round(eager_ms, 5),
        "stages_us": {s: round(v[0] / v[1] * 1e3, 3) for s, v in stages.items()},
        "roofline": roofline,
        "cpu_baseline": None,
        "setup_s": round(time.time() - t_setup, 1),
    }

    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.set_threads(0)
        n_host = max(4096, 64 * T)
        xs_host = ms.extra_tokens(cfg, n_host)
        tk_host = (ms.uniform_i32(n_host, 0, cfg.vocab - 1, cfg.seed, ms.TAG["token_ids"])
                   if cfg.route == "hash" else None)
        n_tok, spent, batch = 0, 0.0, max(threads, 1)
        while spent < args.cpu_seconds and n_tok + batch <= xs_host.shape[0]:
            sel = slice(n_tok, n_tok + batch)
            t0 = time.perf_counter()
            oracle.forward(cfg, inp, x=xs_host[sel], token_ids=tk_host[sel] if tk_host is not None else None,
                           want=False)
            spent += time.perf_counter() - t0
            n_tok += batch
        res["cpu_baseline"] = {
            "value": round(n_tok / spent, 3) if spent > 0 else None,
            "unit": "tokens/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{n_tok} tokens of the same workload, {batch} per oracle call, {spent:.1f} s",
        }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
