"""Seeded synthetic inputs for the quantized routed-MoE layer.

This package only draws random numbers and lays them out in the canonical
storage formats (see ``synth.c`` for the generator and format definitions).
It holds none of the layer's arithmetic and imports neither the oracle nor the
GPU package; both of those consume what it returns.

Workloads follow the DeepSeek V4 Flash MoE shape (page "DeepSeek V4 Flash —
DFlash Integration", section "Model Architecture": hidden 4096, 256 routed
experts top-6 plus one shared expert, expert FFN 2048, hash routing on the
first layers, learned router with optional bias elsewhere) with the value
distributions stated for each workload below.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libmoe_synth.so")

Q8_BLOCK_BYTES = 34     # fp16 d + 32 int8 codes
Q2_BLOCK_BYTES = 84     # fp16 d, fp16 dmin, 16 B scales/mins, 64 B codes
SCALE_LO, SCALE_HI = 0.001, 0.01

# Tensor tags: each tensor draws from its own substreams.
TAG = {
    "x": 1, "router_w": 2, "router_b": 3, "token_ids": 4, "hash_table": 5,
    "gate": 11, "up": 12, "down": 13, "sh_gate": 21, "sh_up": 22, "sh_down": 23,
}


def build(force: bool = False) -> str:
    """Compile the generator library in place (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fopenmp", "-fPIC",
                               "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P, I64, U64, D, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_int32
        lib.synth_normal_f32.argtypes = [P, I64, D, D, U64, U64]
        lib.synth_normal_f32.restype = None
        lib.synth_uniform_i32.argtypes = [P, I64, I32, I32, U64, U64]
        lib.synth_uniform_i32.restype = None
        lib.synth_distinct_rows.argtypes = [P, I64, I32, I32, U64, U64]
        lib.synth_distinct_rows.restype = ctypes.c_int
        lib.synth_q8_bank.argtypes = [P, I64, I64, I64, D, D, U64, U64]
        lib.synth_q8_bank.restype = ctypes.c_int
        lib.synth_q2_bank.argtypes = [P, I64, I64, I64, D, D, U64, U64]
        lib.synth_q2_bank.restype = ctypes.c_int
        lib.synth_f16_from_double.argtypes = [D]
        lib.synth_f16_from_double.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_f32(shape, mean: float, std: float, seed: int, tag: int) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(_ptr(out), out.size, mean, std, seed, tag)
    return out


def uniform_i32(n: int, lo: int, hi: int, seed: int, tag: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_i32(_ptr(out), n, lo, hi, seed, tag)
    return out


def distinct_rows(rows: int, k: int, n_values: int, seed: int, tag: int) -> np.ndarray:
    out = np.empty((rows, k), dtype=np.int32)
    if _load().synth_distinct_rows(_ptr(out), rows, k, n_values, seed, tag) != 0:
        raise ValueError("distinct_rows: need k <= n_values <= 4096")
    return out


def q8_bank(n_mats: int, rows: int, cols: int, seed: int, tag: int) -> np.ndarray:
    """Canonical Q8_32 bytes of n_mats matrices [rows][cols], shape (n_mats, rows, cols//32*34)."""
    if cols % 32:
        raise ValueError("Q8_32 needs cols % 32 == 0")
    out = np.empty((n_mats, rows, cols // 32 * Q8_BLOCK_BYTES), dtype=np.uint8)
    _load().synth_q8_bank(_ptr(out), n_mats, rows, cols, SCALE_LO, SCALE_HI, seed, tag)
    return out


def q2_bank(n_mats: int, rows: int, cols: int, seed: int, tag: int) -> np.ndarray:
    """Canonical Q2_256 bytes of n_mats matrices [rows][cols], shape (n_mats, rows, cols//256*84)."""
    if cols % 256:
        raise ValueError("Q2_256 needs cols % 256 == 0")
    out = np.empty((n_mats, rows, cols // 256 * Q2_BLOCK_BYTES), dtype=np.uint8)
    _load().synth_q2_bank(_ptr(out), n_mats, rows, cols, SCALE_LO, SCALE_HI, seed, tag)
    return out


def f16_from_double(v: float) -> int:
    return int(_load().synth_f16_from_double(float(v)))


@dataclass(frozen=True)
class LayerConfig:
    """One routed-MoE layer workload.

    hidden/n_experts/top_k/ffn follow the layer shape; ``tokens`` is the batch
    of one call.  ``routed_fmt`` is "q8" (Q8_32) or "q2" (Q2_256) for the routed
    experts; the shared expert is always Q8_32 with the same FFN width.
    ``route`` is "learned" (sigmoid router, bias-adjusted top-k), "hash"
    (token id -> fixed table of distinct experts, equal weights) or
    "hash_scored" (the table's experts weighted by their renormalised router
    scores).  Hash tables have ``table_k`` entries per row (0: top_k), of which
    the first top_k are used.
    """
    name: str
    hidden: int
    n_experts: int
    top_k: int
    ffn: int
    tokens: int
    routed_fmt: str = "q8"
    route: str = "learned"
    seed: int = 0
    vocab: int = 131072
    shared: bool = True
    bias: bool = True
    router_std: float = 0.05
    bias_std: float = 0.1
    table_k: int = 0

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


# The five workloads of the layer: a tiny parity case, Q8 decode, decode with
# 2-bit routed experts, hash-routed batched decode, and a prefill chunk; then
# the same prefill at larger chunks.
CONFIGS = {
    "tiny": LayerConfig("tiny", 256, 16, 2, 128, 4, seed=0),
    "decode_q8": LayerConfig("decode_q8", 4096, 256, 6, 2048, 1, seed=1),
    "decode_q2": LayerConfig("decode_q2", 4096, 256, 6, 2048, 1, routed_fmt="q2", seed=2),
    "hash_decode": LayerConfig("hash_decode", 4096, 256, 6, 2048, 32, route="hash", seed=3),
    "prefill": LayerConfig("prefill", 4096, 256, 6, 2048, 2048, seed=4),
    # Larger prefill chunks over the same layer (same seed: identical weights,
    # x rows prefix-stable): 4096 tokens, the default prefill chunk of page
    # "DwarfStar (ds4) — ROCm / gfx1151 fork", section "Benchmarking"; 8192,
    # the chunk of the qualified launch on page "DeepSeek V4 Flash — DFlash
    # Integration", section "DSpark".
    "prefill_4096": LayerConfig("prefill_4096", 4096, 256, 6, 2048, 4096, seed=4),
    "prefill_8192": LayerConfig("prefill_8192", 4096, 256, 6, 2048, 8192, seed=4),
    # Routing variants on the same layer: the reduced top-k of --ds4-expert-top-k
    # (4 of the decode layer's router, same seed), score-weighted hash routing
    # (the hash-routed batch, same seed), and the Motif-3 router shape of page
    # "ds4: dfm Edition", Motif-3 section (384 routed experts, sigmoid top-8,
    # one shared expert) at the DeepSeek widths, which that page does not give.
    "decode_topk4": LayerConfig("decode_topk4", 4096, 256, 4, 2048, 1, seed=1),
    "hash_scored_decode": LayerConfig("hash_scored_decode", 4096, 256, 6, 2048, 32, route="hash_scored", seed=3),
    "decode_motif3": LayerConfig("decode_motif3", 4096, 384, 8, 2048, 1, seed=5),
    # The prefill chunk with 2-bit routed experts (shared expert Q8), the
    # weight families the pages' model runs prefill with ("DwarfStar (ds4) —
    # ROCm / gfx1151 fork", Model Weights).
    "prefill_q2": LayerConfig("prefill_q2", 4096, 256, 6, 2048, 2048, routed_fmt="q2", seed=6),
}


def make_inputs(cfg: LayerConfig, tokens: int | None = None) -> dict:
    """All tensors of one call, as host numpy arrays (canonical weight bytes).

    x ~ N(0,1) fp32 [T][H]; router W ~ N(0, router_std) fp32 [E][H]; bias ~
    N(0, bias_std) fp32 [E] (zeros when cfg.bias is False); token ids uniform in
    [0, vocab); hash table [vocab][table_k or k] of distinct experts; Q8 codes uniform in
    [-127,127] with fp16 scales U(0.001, 0.01); Q2 codes, scales and mins
    uniform over their bit widths with fp16 d, dmin U(0.001, 0.01).
    Rows of x and token ids are prefix-stable in ``tokens``.
    """
    T = cfg.tokens if tokens is None else tokens
    H, E, k, F, s = cfg.hidden, cfg.n_experts, cfg.top_k, cfg.ffn, cfg.seed
    d = {"x": normal_f32((T, H), 0.0, 1.0, s, TAG["x"])}
    if cfg.route != "hash":
        d["router_w"] = normal_f32((E, H), 0.0, cfg.router_std, s, TAG["router_w"])
    if cfg.route == "learned":
        d["router_b"] = (normal_f32((E,), 0.0, cfg.bias_std, s, TAG["router_b"]) if cfg.bias
                         else np.zeros(E, dtype=np.float32))
    else:
        d["token_ids"] = uniform_i32(T, 0, cfg.vocab - 1, s, TAG["token_ids"])
        d["hash_table"] = distinct_rows(cfg.vocab, cfg.table_k or k, E, s, TAG["hash_table"])
    bank = q8_bank if cfg.routed_fmt == "q8" else q2_bank
    d["gate"] = bank(E, F, H, s, TAG["gate"])
    d["up"] = bank(E, F, H, s, TAG["up"])
    d["down"] = bank(E, H, F, s, TAG["down"])
    if cfg.shared:
        d["sh_gate"] = q8_bank(1, F, H, s, TAG["sh_gate"])[0]
        d["sh_up"] = q8_bank(1, F, H, s, TAG["sh_up"])[0]
        d["sh_down"] = q8_bank(1, H, F, s, TAG["sh_down"])[0]
    return d


def extra_tokens(cfg: LayerConfig, n: int) -> np.ndarray:
    """n activation rows drawn from the same stream as make_inputs' x (prefix-stable)."""
    return normal_f32((n, cfg.hidden), 0.0, 1.0, cfg.seed, TAG["x"])
