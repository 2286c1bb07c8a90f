"""CPU oracle of the quantized routed-MoE layer — TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``moe_oracle.c`` (plain C, fp64).  Only the test
suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package; the GPU library never does, and the two share no
code.  See ``moe_oracle.c`` for what each function computes and which passage
of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_HDR = os.path.join(_HERE, "moe_oracle.h")
_LIB = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "libmoe_oracle.so")

FMT = {"q8": 1, "q2": 2}
ROUTE = {"learned": 1, "hash": 2, "hash_scored": 3}

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "n_experts", "top_k", "ffn", "has_shared", "routed_fmt", "route", "table_k")]


class _Weights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p), ("table", ctypes.c_void_p),
                ("vocab", ctypes.c_int32), ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p),
                ("sh_down", ctypes.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sig = {
            "orc_f16_to_double": ([ctypes.c_uint16], ctypes.c_double),
            "orc_router_logits": ([P, P, I32, I32, I32, P], None),
            "orc_pairwise_sum": ([P, I32], ctypes.c_double),
            "orc_sigmoid": ([F], F),
            "orc_route_learned": ([P, P, I32, I32, I32, P, P, P], None),
            "orc_route_hash": ([P, P, I32, I32, I32, I32, I32, P, P], ctypes.c_int),
            "orc_route_hash_scored": ([P, P, I32, I32, P, I32, I32, I32, P, P], ctypes.c_int),
            "orc_quantize": ([P, I64, P, P], None),
            "orc_sort_pairs": ([P, I32, I32, I32, P, P, P], None),
            "orc_matvec": ([P, I32, I32, I32, P, P, P], None),
            "orc_block_sums": ([P, I32, I32, I32, P, P], None),
            "orc_expert": ([P, P, P, I32, I32, I32, P, P, P, P, P, P], None),
            "orc_forward": ([P, P, P, P, I32, I32, P, P, P, P, P, P, P, P, P], ctypes.c_int),
            "orc_set_threads": ([ctypes.c_int], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes, fn.restype = args, res
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous numpy arrays"
    return a.ctypes.data


def set_threads(n: int = 0) -> int:
    return _load().orc_set_threads(n)


def f16_to_double(h: int) -> float:
    return _load().orc_f16_to_double(h)


def pairwise_sum(v: np.ndarray) -> float:
    v = np.ascontiguousarray(v, dtype=np.float64)
    return _load().orc_pairwise_sum(_p(v), v.size)


def sigmoid(l: float) -> float:
    return _load().orc_sigmoid(l)


def router_logits(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    T, H = x.shape
    E = w.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    _load().orc_router_logits(_p(x), _p(w), T, E, H, _p(out))
    return out


def route_learned(logits: np.ndarray, bias: np.ndarray | None, k: int):
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    s = np.empty((T, E), dtype=np.float32)
    _load().orc_route_learned(_p(logits), _p(bias), T, E, k, _p(ids), _p(w), _p(s))
    return ids, w, s


def route_hash(token_ids: np.ndarray, table: np.ndarray, n_experts: int, k: int | None = None):
    """ids/weights from the first k (default: all) entries of each token's table row."""
    T = token_ids.shape[0]
    vocab, table_k = table.shape
    k = table_k if k is None else k
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = _load().orc_route_hash(_p(token_ids), _p(table), vocab, table_k, T, n_experts, k, _p(ids), _p(w))
    if rc != 0:
        raise ValueError("hash routing: token id or table entry out of range, or duplicate expert in a row")
    return ids, w


def route_hash_scored(token_ids: np.ndarray, table: np.ndarray, logits: np.ndarray, k: int | None = None):
    """Table-chosen experts weighted by their renormalised router scores."""
    T, E = logits.shape
    vocab, table_k = table.shape
    k = table_k if k is None else k
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = _load().orc_route_hash_scored(_p(token_ids), _p(table), vocab, table_k, _p(logits), T, E, k, _p(ids),
                                       _p(w))
    if rc != 0:
        raise ValueError("hash routing: token id or table entry out of range, or duplicate expert in a row")
    return ids, w


def quantize(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.size
    q = np.empty(x.shape, dtype=np.int8)
    d = np.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=np.float32)
    _load().orc_quantize(_p(x), n, _p(q), _p(d))
    return q, d


def sort_pairs(ids: np.ndarray, n_experts: int):
    T, k = ids.shape
    counts = np.empty(n_experts, dtype=np.int32)
    offsets = np.empty(n_experts + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    _load().orc_sort_pairs(_p(ids), T, k, n_experts, _p(counts), _p(offsets), _p(perm))
    return counts, offsets, perm


def matvec(mat: np.ndarray, fmt: str, rows: int, cols: int, aq: np.ndarray, ad: np.ndarray) -> np.ndarray:
    out = np.empty(rows, dtype=np.float64)
    _load().orc_matvec(_p(mat), FMT[fmt], rows, cols, _p(aq), _p(ad), _p(out))
    return out


def block_sums(mat: np.ndarray, fmt: str, rows: int, cols: int, aq: np.ndarray) -> np.ndarray:
    per = cols // 32 if fmt == "q8" else cols // 16
    out = np.empty((rows, per), dtype=np.int32)
    _load().orc_block_sums(_p(mat), FMT[fmt], rows, cols, _p(aq), _p(out))
    return out


def expert(gate, up, down, fmt: str, H: int, F: int, xq, xd):
    """One expert on one token -> (h fp32 [F], hq int8 [F], hd fp32 [F/32], y fp64 [H])."""
    h = np.empty(F, dtype=np.float32)
    hq = np.empty(F, dtype=np.int8)
    hd = np.empty(F // 32, dtype=np.float32)
    y = np.empty(H, dtype=np.float64)
    _load().orc_expert(_p(gate), _p(up), _p(down), FMT[fmt], H, F, _p(xq), _p(xd), _p(h), _p(hq), _p(hd), _p(y))
    return h, hq, hd, y


def forward(cfg, inp: dict, x: np.ndarray | None = None, token_ids: np.ndarray | None = None,
            dense: bool = False, want: bool = True) -> dict:
    """Whole layer for the rows of ``x`` (default: inp["x"]).

    cfg is a moe_synth.LayerConfig, inp the dict of make_inputs().  Returns out
    [T][H] fp32 and, when ``want``, ids/w/logits/xq/xd/h/hq/hd (slot k of h/hq/hd
    is the shared expert).
    """
    x = inp["x"] if x is None else np.ascontiguousarray(x, dtype=np.float32)
    if cfg.route != "learned":
        token_ids = inp["token_ids"] if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int32)
    T, H = x.shape
    E, k, F = cfg.n_experts, cfg.top_k, cfg.ffn
    S = k + 1
    table_k = inp["hash_table"].shape[1] if cfg.route != "learned" else 0
    shape = _Shape(H, E, k, F, 1 if cfg.shared else 0, FMT[cfg.routed_fmt], ROUTE[cfg.route], table_k)
    wt = _Weights(_p(inp.get("router_w")), _p(inp.get("router_b")), _p(inp.get("hash_table")),
                  cfg.vocab, _p(inp["gate"]), _p(inp["up"]), _p(inp["down"]),
                  _p(inp.get("sh_gate")), _p(inp.get("sh_up")), _p(inp.get("sh_down")))
    r = {"out": np.empty((T, H), dtype=np.float32)}
    if want:
        r.update(ids=np.empty((T, k), np.int32), w=np.empty((T, k), np.float32),
                 logits=np.zeros((T, E), np.float32), xq=np.empty((T, H), np.int8),
                 xd=np.empty((T, H // 32), np.float32), h=np.zeros((T, S, F), np.float32),
                 hq=np.zeros((T, S, F), np.int8), hd=np.zeros((T, S, F // 32), np.float32))
    g = r.get
    rc = _load().orc_forward(ctypes.byref(shape), ctypes.byref(wt), _p(x), _p(token_ids), T, 1 if dense else 0,
                             _p(r["out"]), _p(g("ids")), _p(g("w")),
                             _p(g("logits")) if cfg.route != "hash" else None,
                             _p(g("xq")), _p(g("xd")), _p(g("h")), _p(g("hq")), _p(g("hd")))
    if rc != 0:
        raise ValueError("oracle forward rejected its input")
    return r
