#!/usr/bin/env python3
"""Throughput of the routed-MoE layer on one MI355X.

A step is one call of the whole layer (routing, quantization, token sort,
expert gate/up + SwiGLU, down projection and weighted combine) on one batch
of synthetic tokens whose inputs are already resident in HBM.  The default
workload is the Q8 decode layer (1 token, hidden 4096, 256 experts top-6 +
1 shared, FFN 2048).  Prints ONE JSON line.

Timing: W eager warm-up steps, then the K timed steps are replayed from a
captured HIP graph (per-call host overhead excluded, as in a captured decode
loop).  Every step takes a fresh batch of tokens and the next of R
address-distinct copies of every weight tensor it reads (router, routed
gate/up/down banks, shared expert), so the 256 MB Infinity Cache cannot carry
weights from one step to the next.  The per-step spread (p10, median, p90)
comes from one-step graphs replayed back to back with an event between
replays.  An eager pass takes each kernel's start and end from HIP events
recorded by its own launch (hipExtLaunchKernelGGL): the per-kernel durations
used for the roofline entry.  A decode line also carries the prefill chunk's
record (the MFMA half of the metric), measured the same way.  The CPU oracle
is then timed on a bounded sample of the same workload on the host cores,
once with all of them and once single-threaded.
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
    ap.add_argument("--replicas", type=int, default=8,
                    help="address-distinct copies of every weight tensor, cycled step by step")
    ap.add_argument("--graph-steps", type=int, default=100)
    ap.add_argument("--spread-steps", type=int, default=0,
                    help="steps of the spread measurement (0: 200 for decode batches, 50 otherwise)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-seconds-single", type=float, default=6.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-config", default="prefill",
                    help="workload of the prefill sub-record carried by a decode line")
    ap.add_argument("--no-prefill", action="store_true", help="omit the prefill sub-record")
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


def host_info():
    """CPU model, visible cores and load average of the host running the bench."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        load = open("/proc/loadavg").read().split()[:3]
    except OSError:
        load = None
    return {"cpu_model": model, "cpus_visible": os.cpu_count(), "loadavg": load}


def gpu_clocks():
    """Current shader (sclk) and memory (mclk) clocks in MHz, from the driver's
    DPM tables in sysfs (the level marked '*'), else from rocm-smi; None when
    neither is readable."""
    import glob
    import re
    import subprocess
    out = {}
    for key in ("sclk", "mclk"):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{key}")):
            try:
                for line in open(path):
                    if "*" in line:
                        m = re.search(r"(\d+)\s*Mhz", line, re.I)
                        if m:
                            out[f"{key}_mhz"] = int(m.group(1))
            except OSError:
                continue
            if f"{key}_mhz" in out:
                break
    if len(out) < 2:
        try:
            r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
            for key in ("sclk", "mclk"):
                m = re.search(key + r"\s+clock level:\s*\d+:\s*\((\d+)\s*Mhz\)", r.stdout, re.I)
                if m and f"{key}_mhz" not in out:
                    out[f"{key}_mhz"] = int(m.group(1))
        except (OSError, subprocess.SubprocessError):
            pass
    return out or None


def pct(v, q):
    """q-th percentile (linear interpolation) of a list."""
    v = sorted(v)
    if not v:
        return None
    i = (len(v) - 1) * q / 100.0
    lo, hi = int(math.floor(i)), int(math.ceil(i))
    return v[lo] + (v[hi] - v[lo]) * (i - lo)


def replicate_weights(qr, layer, R):
    """R address-distinct copies of every weight tensor a step reads (router,
    routed gate/up/down banks, shared expert) as moe_weights structs; copy 0 is
    the layer's own.  Bias and hash table (a few KB per step) are shared."""
    names = ("router_w", "gate", "up", "down", "sh_gate", "sh_up", "sh_down")
    reps, keep = [], []
    for r in range(R):
        t = {n: getattr(layer, n) for n in names}
        if r:
            t = {n: (v.clone() if v is not None else None) for n, v in t.items()}
        keep.append(t)

        def p(v):
            return None if v is None else v.data_ptr()
        reps.append(qr.Weights(p(t["router_w"]), p(layer.router_b), p(layer.hash_table), p(t["gate"]), p(t["up"]),
                               p(t["down"]), p(t["sh_gate"]), p(t["sh_up"]), p(t["sh_down"])))
    return reps, keep


def measure(cfg, K, W, G, R, spread_n, prof_n):
    """Time one workload: W eager warm-up steps, K steps replayed from a graph
    of G steps (each step a fresh batch of tokens and the next of R weight
    copies), the per-step spread from about spread_n steps replayed as short
    graphs bracketed by events, and prof_n eager steps with per-kernel events."""
    import torch

    import moe_synth as ms
    import quantized_routed_moe_amd as qr

    T, H, E, k, F = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn
    dev = torch.device("cuda:0")
    inp = ms.make_inputs(cfg)
    layer = qr.MoELayer(H, E, k, F, cfg.shared, cfg.routed_fmt, cfg.route,
                        cfg.vocab if cfg.route != "learned" else 0, table_k=cfg.table_k).load(inp)
    wlist, keep = replicate_weights(qr, layer, R)
    n_steps = W + G
    xs = torch.from_numpy(ms.extra_tokens(cfg, n_steps * T)).to(dev).reshape(n_steps, T, H)
    toks = None
    if cfg.route != "learned":
        toks = torch.from_numpy(ms.uniform_i32(n_steps * T, 0, cfg.vocab - 1, cfg.seed,
                                               ms.TAG["token_ids"])).to(dev).reshape(n_steps, T)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = layer.ensure_workspace(T)

    def step(i, stream=None):
        qr.layer_forward(layer.shape, wlist[i % R], xs[i % n_steps], toks[i % n_steps] if toks is not None else None,
                         out, ws, stream)

    # distinct experts each step touches (for the algorithmic byte counts)
    used = []
    for i in range(n_steps):
        r = layer.forward_debug(xs[i], toks[i] if toks is not None else None)
        used.append(int(torch.count_nonzero(r["counts"]).item()))
        del r
    torch.cuda.synchronize()

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # G steps in one graph; a replay is checked bitwise against the eager call
    gs = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        for i in range(G):
            step(W + i, torch.cuda.current_stream())
    graph.replay()
    torch.cuda.synchronize()
    replay_out = out.clone()
    step(W + G - 1)
    torch.cuda.synchronize()
    if not torch.equal(replay_out.view(torch.int32), out.view(torch.int32)):
        raise RuntimeError("graph replay differs from the eager call")
    replays = max(1, math.ceil(K / G))
    K = replays * G
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K

    # spread: graphs of S steps replayed back to back with an event between
    # replays; a sample is one replay's time per step.  Decode batches take
    # S = 10 (a graph launch leaves a gap of several microseconds on the GPU,
    # which one-step graphs of a ~40 us step would count every time); longer
    # steps take S = 1.
    S = 10 if T <= 32 else 1
    n_rep = max(1, spread_n // S)
    sg = []
    for j in range(min(n_rep, max(1, G // S))):
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1, stream=gs):
            for i in range(S):
                step(W + j * S + i, torch.cuda.current_stream())
        sg.append(g1)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(n_rep):
        sg[i % len(sg)].replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) / S for i in range(n_rep)]

    # eager steps, host launch included; then eager steps with per-kernel events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i % G)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / K
    prof = qr.Profiler(max_events=24 * prof_n + 64)  # up to 12 launches per step, 2 events each
    prof.attach()
    for i in range(prof_n):
        step(W + i % G)
    prof.detach()
    torch.cuda.synchronize()
    stages = prof.collect()
    prof.close()
    del graph, sg, keep
    torch.cuda.empty_cache()
    return {"inp": inp, "T": T, "K": K, "G": G, "ms_step": ms_step, "eager_ms": eager_ms, "spread_ms": per,
            "spread_graph_steps": S,
            "stages": stages, "prof_n": prof_n, "u_avg": u_avg_of(used, W, G, K)}


def summarize(cfg, m):
    """Stage table, roofline entry and layer fractions of one measurement."""
    import quantized_routed_moe_amd as qr
    model = stage_model(cfg, qr, m["u_avg"])
    stages = m["stages"]
    # a stage's time per call (all its launches) decides the dominant stage; its
    # kernel's average launch duration prices the roofline entry
    dom = max(stages, key=lambda s: stages[s][0])
    dom_us = stages[dom][0] / stages[dom][1] * 1e3
    roofline = make_roofline(cfg, model, dom, dom_us)
    detail = {}
    for s_, (ms_tot, n_) in stages.items():
        us = ms_tot / m["prof_n"] * 1e3
        b = model["stages"].get(s_, {}).get("bytes")
        detail[s_] = {"us": round(us, 3), "launches": round(n_ / m["prof_n"], 2), "bytes": int(b) if b else None,
                      "gbps": round(b / (us * 1e-6) / 1e9, 1) if b else None}
    sec = m["ms_step"] * 1e-3
    P = cfg.tokens * cfg.top_k + (cfg.tokens if cfg.shared else 0)
    layer_ops = 2 * P * 3 * cfg.ffn * cfg.hidden
    per = m["spread_ms"]
    return {
        "ms_per_step": round(m["ms_step"], 5),
        "tokens_per_s": round(cfg.tokens / sec, 1),
        "step_ms_p10_median_p90": [round(pct(per, q), 5) for q in (10, 50, 90)],
        "spread": f"{len(per)} replays of {m['spread_graph_steps']}-step graphs, an event between replays; "
                  "a sample is one replay's time per step",
        "eager_ms_per_step": round(m["eager_ms"], 5),
        "layer_bytes": int(model["layer_bytes"]),
        "layer_gbps": round(model["layer_bytes"] / sec / 1e9, 1),
        "layer_hbm_frac": round(model["layer_bytes"] / sec / 1e9 / HBM_PEAK_GBS, 4),
        "layer_int8_ops": int(layer_ops),
        "layer_mfma_frac": round(layer_ops / sec / 1e12 / INT8_PEAK_TOPS, 4),
        "distinct_experts_per_step": round(m["u_avg"], 2),
        "stages": detail,
        "roofline": roofline,
        "model": model,
    }


def kernel_fracs(cfg, summ, stage):
    """HBM, int8-MFMA and vector-ALU fractions of one stage's kernel."""
    st = summ["model"]["stages"].get(stage)
    us = summ["stages"].get(stage, {}).get("us")
    if not st or not us:
        return None
    sec = us * 1e-6
    kern = stage_kernel(cfg, stage)
    e = {"kernel": kern, "us": us, "algorithmic_bytes": int(st["bytes"]),
         "hbm_frac": round(st["bytes"] / sec / 1e9 / HBM_PEAK_GBS, 4)}
    if st.get("ops"):
        e["int8_ops"] = int(st["ops"])
        e["mfma_frac"] = round(st["ops"] / sec / 1e12 / INT8_PEAK_TOPS, 4)
        e["alu_frac"] = round(st["valu"] / sec / 1e12 / VALU_PEAK_TOPS, 4)
    e["traffic"] = stored_traffic(cfg, kern)
    return e


def cpu_baseline(cfg, inp, seconds, threads):
    """The oracle as it stands, timed on the host on fresh tokens of the same
    workload: batches of `threads` tokens (OpenMP over tokens) until about
    `seconds` of compute."""
    import moe_synth as ms
    import oracle
    used = oracle.set_threads(threads)
    T = cfg.tokens
    n_host = max(4096, 64 * T)
    xs_host = ms.extra_tokens(cfg, n_host)
    tk_host = (ms.uniform_i32(n_host, 0, cfg.vocab - 1, cfg.seed, ms.TAG["token_ids"])
               if cfg.route != "learned" else None)
    n_tok, spent, batch = 0, 0.0, max(used, 1)
    while spent < seconds and n_tok + batch <= xs_host.shape[0]:
        sel = slice(n_tok, n_tok + batch)
        t0 = time.perf_counter()
        oracle.forward(cfg, inp, x=xs_host[sel], token_ids=tk_host[sel] if tk_host is not None else None, want=False)
        spent += time.perf_counter() - t0
        n_tok += batch
    return {"value": round(n_tok / spent, 3) if spent > 0 else None, "unit": "tokens/s", "cores": used,
            "sample": f"{n_tok} tokens of the same workload, {batch} per oracle call, {spent:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the layer's expert-parallel split over several GPUs is a design, not code)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.traffic_from:
        args.pmc_fetch, args.pmc_write, args.copy_fetch, args.copy_write = args.traffic_from
        traffic_from(args)
        return

    import torch

    import moe_synth as ms

    cfg = ms.CONFIGS[args.config]
    T, H, E, k, F = cfg.tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn
    torch.cuda.set_device(0)
    host = host_info()
    t_setup = time.time()
    R = max(1, args.replicas)
    G = max(1, min(args.graph_steps, args.steps))
    spread_n = args.spread_steps or (200 if T <= 32 else 50)
    m = measure(cfg, args.steps, args.warmup, G, R, spread_n, min(args.steps, 300))
    summ = summarize(cfg, m)
    K = m["K"]
    res = {
        "metric": METRIC,
        "value": summ["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": summ["ms_per_step"],
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
            "timing": f"HIP-graph replay of {G}-step graphs; every step a fresh batch and the next of {R} "
                      "address-distinct copies of all weights (router, routed banks, shared expert)",
        },
        "step_ms_p10_median_p90": summ["step_ms_p10_median_p90"],
        "spread": summ["spread"],
        "layer_gbps": summ["layer_gbps"],
        "layer_hbm_frac": summ["layer_hbm_frac"],
        "eager_ms_per_step": summ["eager_ms_per_step"],
        "distinct_experts_per_step": summ["distinct_experts_per_step"],
        "stages": summ["stages"],
        "roofline": summ["roofline"],
        "cpu_baseline": None,
        "host": host,
        "gpu_clocks": None,
    }
    inp = m.pop("inp")
    res["gpu_clocks"] = gpu_clocks()

    if not args.no_prefill and T <= 32:
        # the prefill half of the metric: MFMA utilisation of the chunk
        del inp
        pcfg = ms.CONFIGS[args.prefill_config]
        pm = measure(pcfg, 20, 3, 10, R, 50, 20)
        pm.pop("inp")
        ps = summarize(pcfg, pm)
        res["prefill"] = {
            "workload": f"{pcfg.name}: {pcfg.tokens} tokens/step, hidden {pcfg.hidden}, {pcfg.n_experts} experts "
                        f"top-{pcfg.top_k} + 1 shared, FFN {pcfg.ffn}, routed {pcfg.routed_fmt.upper()}, "
                        f"{pcfg.route} routing",
            "steps": pm["K"],
            **{key: ps[key] for key in ("ms_per_step", "tokens_per_s", "step_ms_p10_median_p90", "layer_bytes",
                                        "layer_gbps", "layer_hbm_frac", "layer_int8_ops", "layer_mfma_frac",
                                        "distinct_experts_per_step")},
            "gateup_mfma": kernel_fracs(pcfg, ps, "gateup"),
            "down_mfma": kernel_fracs(pcfg, ps, "down"),
            "stages": ps["stages"],
        }
        inp = None

    if not args.no_cpu_baseline:
        if inp is None:
            inp = ms.make_inputs(cfg)
        multi = cpu_baseline(cfg, inp, args.cpu_seconds, 0)
        single = cpu_baseline(cfg, inp, args.cpu_seconds_single, 1)
        res["cpu_baseline"] = {**multi, "kind": "oracle", "single_thread": single}
    res["host"]["loadavg_end"] = host_info()["loadavg"]
    res["setup_s"] = round(time.time() - t_setup, 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
