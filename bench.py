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
Infinity Cache cannot serve them across steps.  A second, eager pass takes
each kernel's start and end from HIP events recorded by its own launch
(hipExtLaunchKernelGGL), the per-kernel durations used for the
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
# fp32 vector ALU issue rate without packed dual-issue: 256 CUs x 4 SIMDs x 16
# lanes x 2.4 GHz single-lane operations per second (the 157.3 TFLOP/s vector
# peak counts an FMA as 2 flops and packed fp32 as 2 lanes; this code issues
# neither packed fp32 nor anything wider)
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
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
    ap.add_argument("--traffic-from", nargs=4, metavar=("PMC_FETCH", "PMC_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write profiles/traffic.txt for --config from rocprofv3 --pmc CSVs and exit")
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


# --------------------------------------------------------------- accounting
# Kernel sources per stage kernel: a stored byte count applies only while
# these files (and the build flags) are unchanged.
CSRC = os.path.join(ROOT, "quantized_routed_moe_amd", "csrc")
KERNEL_SOURCES = {
    "decode_front_kernel": ["decode.hip", "dev_route.hpp", "dev_vec.hpp", "common.hpp"],
    "decode_select_kernel": ["decode.hip", "dev_route.hpp", "dev_vec.hpp", "common.hpp"],
    "decode_down1_kernel": ["decode.hip", "dev_route.hpp", "dev_vec.hpp", "common.hpp"],
    "decode_gateup1_kernel": ["decode.hip", "dev_route.hpp", "dev_vec.hpp", "common.hpp"],
    "gateup_vec_kernel": ["expert_vec.hip", "dev_vec.hpp", "common.hpp"],
    "down_vec_kernel": ["expert_vec.hip", "dev_vec.hpp", "common.hpp"],
    "combine_kernel": ["expert_vec.hip", "dev_vec.hpp", "common.hpp"],
    "gateup_mfma_kernel": ["expert_mfma.hip", "dev_vec.hpp", "common.hpp"],
    "down_mfma_kernel": ["expert_mfma.hip", "dev_vec.hpp", "common.hpp"],
    "quant_kernel": ["route.hip", "dev_route.hpp", "common.hpp"],
    "logits_tiled_kernel": ["route.hip", "dev_route.hpp", "common.hpp"],
    "select_kernel": ["route.hip", "dev_route.hpp", "common.hpp"],
    "sort_kernel": ["route.hip", "dev_route.hpp", "common.hpp"],
    "sort_hist_kernel": ["route.hip", "dev_route.hpp", "common.hpp"],
    "sort_scan_kernel": ["route.hip", "dev_route.hpp", "common.hpp"],
    "sort_scatter_kernel": ["route.hip", "dev_route.hpp", "common.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")


def kernel_base(name):
    """'void qrmoe::gateup_vec_kernel<4096, 1, false, true>(...)' -> 'gateup_vec_kernel'."""
    import re
    m = re.search(r"qrmoe::(\w+)", name)
    return m.group(1) if m else None


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "quantized_routed_moe_amd", "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def stage_kernel(cfg, stage):
    """Name of the one kernel a stage launches on this workload's path."""
    T = cfg.tokens
    # 2-bit batches take the MFMA GEMMs from 64 tokens (the library's kMfmaMinTokensQ2)
    mfma = cfg.hidden >= 256 and cfg.ffn >= 256 and (cfg.routed_fmt == "q8" or T >= 64)
    if T <= 32:
        # selection of 2..32 tokens: one workgroup up to 8 tokens (learned) or 20
        # (hash routes), else one wave per token and the sort kernel
        dsel = T <= (8 if cfg.route == "learned" else 20)
        if T > 1 and not dsel and stage in ("select", "sort"):
            return {"select": "select_kernel", "sort": "sort_kernel"}[stage]
        return {"route": "decode_front_kernel", "select": "decode_select_kernel",
                "gateup": "decode_gateup1_kernel" if T == 1 else "gateup_vec_kernel",
                "down": "decode_down1_kernel" if T == 1 else "down_vec_kernel",
                "combine": "combine_kernel"}.get(stage)
    if T <= 224:  # the library's kFrontMaxTokens: quantization and logits in the decode front kernel
        front = {"route": "decode_front_kernel", "quant": None, "logits": None}
        if stage in front:
            return front[stage]
    return {"quant": "quant_kernel", "logits": "logits_tiled_kernel", "select": "select_kernel",
            "sort": "sort_kernel" if T * cfg.top_k <= 4096 else "sort_scatter_kernel", "gateup": "gateup_mfma_kernel" if mfma else "gateup_vec_kernel",
            "down": "down_mfma_kernel" if mfma else "down_vec_kernel", "combine": "combine_kernel"}.get(stage)


def u_avg_of(used, warmup, G, K):
    return sum(used[warmup + i % G] for i in range(K)) / K


def stage_model(cfg, qr, u_avg):
    """Algorithmic bytes (and int8 MFMA operations) per launch of each stage.

    Bytes count what a stage must move at least once: the weights of every
    expert that receives a token, router weights, activations read and
    results written (x fp32, int8 codes + fp32 block scales, fp32 y, fp32
    out).  u_avg is the mean number of distinct routed experts per
    step.  Ops count 2 per int8 multiply-add of the expert GEMMs; valu counts
    the per-block dequantization the Q8_32 format requires of them, one
    int32 -> fp32 conversion and one fma per output and 32-block."""
    T, H, E, k, F = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn
    fmt = qr.FMT[cfg.routed_fmt]
    sh = 1 if cfg.shared else 0
    has_router = cfg.route != "hash"     # logits, scores and keys are computed (learned, hash_scored)
    table = T * k * 4 if cfg.route != "learned" else 0   # hash-table entries read
    mq8_gu, mq8_dn = qr.matrix_bytes(qr.FMT_Q8, F, H), qr.matrix_bytes(qr.FMT_Q8, H, F)
    mr_gu, mr_dn = qr.matrix_bytes(fmt, F, H), qr.matrix_bytes(fmt, H, F)
    Pr, P = T * k, T * k + sh * T
    x32 = T * H * 4
    xq = T * H + T * (H // 32) * 4
    hq = lambda n: n * F + n * (F // 32) * 4
    router = (E * H * 4 if has_router else 0) + table
    rout = 3 * T * E * 4 if has_router else 0
    st = {}
    if T <= 32:
        sel = (2 * T * E * 4 if has_router else T * 4) + T * k * 12
        st["route"] = router + x32 + xq + rout
        if T == 1:  # selection runs in the gate/up kernel
            st["gateup"] = u_avg * 2 * mr_gu + sh * 2 * mq8_gu + xq + hq(P) + sel
        else:
            st["select"] = sel
            if T > (8 if cfg.route == "learned" else 20):
                st["sort"] = T * k * 4 * 3
            st["gateup"] = u_avg * 2 * mr_gu + sh * 2 * mq8_gu + xq + hq(P)
        if T == 1:
            st["down"] = u_avg * mr_dn + sh * mq8_dn + hq(P) + x32
        else:
            st["down"] = u_avg * mr_dn + sh * mq8_dn + hq(P) + P * H * 4
            st["combine"] = P * H * 4 + x32
    else:
        if T <= 224:  # decode front kernel: quantization and logits in one launch
            st["route"] = router + x32 + xq + rout
        else:
            st["quant"] = x32 + xq
            if has_router:
                st["logits"] = router + x32 + rout
        st["select"] = (2 * T * E * 4 if has_router else T * 4) + T * k * 8
        st["sort"] = T * k * 4 * 3
        # 2-bit experts: the gate/up GEMM reads x's subblock sums and stores
        # h's, which the down GEMM reads
        xs16 = T * (H // 16) * 4 if cfg.routed_fmt == "q2" else 0
        hs16 = Pr * (F // 16) * 4 if cfg.routed_fmt == "q2" and T >= 64 else 0
        st["gateup"] = u_avg * 2 * mr_gu + sh * 2 * mq8_gu + xq + xs16 + hq(P) + hs16
        st["down"] = u_avg * mr_dn + sh * mq8_dn + hq(P) + hs16 + P * H * 4
        st["combine"] = P * H * 4 + x32
    ops = {"gateup": 2 * P * 2 * F * H, "down": 2 * P * H * F}
    valu = {"gateup": 2 * P * 2 * F * (H // 32), "down": 2 * P * H * (F // 32)}
    layer = (u_avg * (2 * mr_gu + mr_dn) + sh * (2 * mq8_gu + mq8_dn) + (E * H * 4 if has_router else 0) + 2 * x32)
    return {"stages": {s: {"bytes": b, "ops": ops.get(s), "valu": valu.get(s)} for s, b in st.items()},
            "layer_bytes": layer}


def stored_traffic(cfg, kernel):
    """HBM bytes per launch from profiles/traffic.txt, or None when absent or
    when the kernel's sources changed after the counters were taken."""
    if not kernel or not os.path.exists(TRAFFIC_FILE):
        return None
    want = source_hash(kernel)
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) < 3 or line.startswith("#") or f[0] != cfg.name or f[1] != kernel:
            continue
        kv = dict(x.split("=", 1) for x in f[2:])
        if kv.get("src") != want:
            return None
        return float(kv["bytes"])
    return None


def make_roofline(cfg, model, dom, dom_us):
    """Roofline entry of the dominant stage's kernel.  An MFMA GEMM is priced
    against the roof that binds it at this workload, the one its algorithmic
    work takes longest on at peak: weight bytes over HBM, int8 operations
    over the MFMA units, or the per-block dequantization (conversion + fma
    per output and block) over the vector ALUs; the other roofs' fractions
    are reported beside it."""
    kern = stage_kernel(cfg, dom)
    st = model["stages"].get(dom, {})
    traffic = stored_traffic(cfg, kern)
    b, ops, valu = st.get("bytes"), st.get("ops"), st.get("valu")
    base = {"traffic": traffic, "kernel": kern, "stage": dom, "avg_launch_us": round(dom_us, 3),
            "algorithmic_bytes_per_launch": int(b) if b else None}
    sec = dom_us * 1e-6
    hbm = {"bound": "hbm", "achieved": round(b / sec / 1e9, 1) if b else None, "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(b / sec / 1e9 / HBM_PEAK_GBS, 4) if b else None}
    if kern not in ("gateup_mfma_kernel", "down_mfma_kernel"):
        return {**hbm, **base}
    roofs = {
        "hbm": (b / (HBM_PEAK_GBS * 1e9), hbm),
        "mfma": (ops / (INT8_PEAK_TOPS * 1e12),
                 {"bound": "mfma", "achieved": round(ops / sec / 1e12, 1), "peak": INT8_PEAK_TOPS,
                  "unit": "TOP/s", "frac": round(ops / sec / 1e12 / INT8_PEAK_TOPS, 4)}),
        "alu": (valu / (VALU_PEAK_TOPS * 1e12),
                {"bound": "alu", "achieved": round(valu / sec / 1e12, 2), "peak": round(VALU_PEAK_TOPS, 2),
                 "unit": "T VALU lane-op/s", "frac": round(valu / sec / 1e12 / VALU_PEAK_TOPS, 4)}),
    }
    bind = max(roofs, key=lambda r: roofs[r][0])
    out = {**roofs[bind][1], **base, "algorithmic_ops_per_launch": int(ops), "algorithmic_valu_per_launch": int(valu)}
    for r, (_, e) in roofs.items():
        if r != bind:
            out[f"{r}_frac"] = e["frac"]
    return out


def traffic_from(args):
    """Writes profiles/traffic.txt lines for one workload from rocprofv3 --pmc
    CSVs: FETCH_SIZE and WRITE_SIZE of the layer kernels (KiB per dispatch)
    and of a plain 1 GiB device copy, which scales each counter to bytes."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        d = defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                d[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return d

    copy_bytes = 1 << 30

    def copy_factor(path, counter):
        v = [x for n, xs in per_kernel(path, counter).items() if "copyBuffer" in n or "copy" in n for x in xs]
        v = [x for x in v if x * 1024 > copy_bytes / 4]
        return copy_bytes / (sum(v) / len(v) * 1024)

    ff = copy_factor(args.copy_fetch, "FETCH_SIZE")
    wf = copy_factor(args.copy_write, "WRITE_SIZE")
    fetch = per_kernel(args.pmc_fetch, "FETCH_SIZE")
    write = per_kernel(args.pmc_write, "WRITE_SIZE")
    rows = {}
    for name, v in fetch.items():
        kb = kernel_base(name)
        if kb not in KERNEL_SOURCES:
            continue
        w = [x for n, xs in write.items() if kernel_base(n) == kb for x in xs]
        fk, wk = sum(v) / len(v), (sum(w) / len(w) if w else 0.0)
        rows[kb] = (fk, wk, fk * 1024 * ff + wk * 1024 * wf)
    cfg_name = args.config
    keep = []
    if os.path.exists(TRAFFIC_FILE):
        keep = [l for l in open(TRAFFIC_FILE) if not (l.split() and l.split()[0] == cfg_name)]
    with open(TRAFFIC_FILE, "w") as out:
        if not keep:
            out.write("# HBM traffic per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch),\n"
                      "# each scaled by the bytes a plain 1 GiB device copy moves per counted KiB.\n"
                      "# workload kernel fetch_kib= write_kib= fetch_factor= write_factor= bytes= src=<kernel sources sha256/16>\n")
        out.writelines(keep)
        for kb, (fk, wk, b) in sorted(rows.items()):
            out.write(f"{cfg_name} {kb} fetch_kib={fk:.1f} write_kib={wk:.1f} fetch_factor={ff:.4f} "
                      f"write_factor={wf:.4f} bytes={b:.0f} src={source_hash(kb)}\n")
    print(f"wrote {len(rows)} kernel(s) for {cfg_name} to {TRAFFIC_FILE}")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported by this build "
              "(multi-GPU expert parallelism is designed, not built)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.traffic_from:
        args.pmc_fetch, args.pmc_write, args.copy_fetch, args.copy_write = args.traffic_from
        traffic_from(args)
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
                        cfg.vocab if cfg.route != "learned" else 0, table_k=cfg.table_k).load(inp)
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
    if cfg.route != "learned":
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

    model = stage_model(cfg, qr, u_avg_of(used, args.warmup, G, K))
    dom = max(stages, key=lambda s: stages[s][0])
    dom_us = stages[dom][0] / stages[dom][1] * 1e3
    roofline = make_roofline(cfg, model, dom, dom_us)
    layer_bytes = model["layer_bytes"]
    stage_detail = {}
    for s_, (ms_tot, n_) in stages.items():
        us = ms_tot / n_ * 1e3
        b = model["stages"].get(s_, {}).get("bytes")
        stage_detail[s_] = {"us": round(us, 3), "bytes": int(b) if b else None,
                            "gbps": round(b / (us * 1e-6) / 1e9, 1) if b else None}

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
        "stages": stage_detail,
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
                   if cfg.route != "learned" else None)
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
