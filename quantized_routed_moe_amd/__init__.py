"""MI355X (gfx950) routed-MoE layer: Python binding of libqrmoe.so.

Argument marshalling only.  Every step of the layer runs in the HIP kernels
behind the C ABI in include/moe.h; PyTorch provides device memory and the
stream.  There is no CPU fallback: importing this package fails loudly when
the compiled library is missing.
"""
from __future__ import annotations

import ctypes
import os

# One HIP runtime per process: PyTorch ships its own libamdhip64, and once it
# is loaded the library's dependency of the same name resolves to it.  Loading
# the library first would map a second runtime next to PyTorch's, and calls
# through that one find no device.
import torch  # noqa: F401  (load order, see above)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqrmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                      "or `python quantized_routed_moe_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

FMT_Q8, FMT_Q2 = 1, 2
ROUTE_LEARNED, ROUTE_HASH, ROUTE_HASH_SCORED = 1, 2, 3
FMT = {"q8": FMT_Q8, "q2": FMT_Q2}
ROUTE = {"learned": ROUTE_LEARNED, "hash": ROUTE_HASH, "hash_scored": ROUTE_HASH_SCORED}
STAGES = ["route", "quant", "logits", "select", "sort", "gateup", "down", "combine"]
# sticky workspace flags (moe_workspace_flags)
FLAG_BAD_TOKEN, FLAG_BAD_TABLE_ENTRY, FLAG_REPEATED_EXPERT = 1, 2, 4
# bytes of the device array that serves moe_layer_forward_static as its workspace
STATIC_SCRATCH_BYTES = 16 << 20
ALIGN = 256


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {_lib.moe_status_string(status).decode()} (status {status})"
        if status == -5:  # MOE_ERR_HIP
            msg += f": {_lib.moe_last_hip_error().decode()}"
        super().__init__(msg)


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("hidden", "n_experts", "top_k", "ffn", "has_shared", "routed_fmt", "route", "vocab", "table_k")]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("router_w", "router_b", "hash_table", "gate", "up", "down", "sh_gate", "sh_up", "sh_down")]


class Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("ids", "w", "logits", "xq", "xd", "counts", "offsets", "perm", "hq", "hd",
                 "gate_sums", "up_sums", "down_sums")] + [("sum_row_stride", ctypes.c_int32)]


_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "moe_abi_version": ([], ctypes.c_int),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_last_hip_error": ([], ctypes.c_char_p),
    "moe_matrix_bytes": ([_I32, _I64, _I64], _I64),
    "moe_pack_weights": ([_I32, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "moe_check_hash_table": ([_P, _I32, _I32, _I32, _P, _SZ, ctypes.POINTER(_I32), _P], ctypes.c_int),
    "moe_workspace_bytes": ([ctypes.POINTER(Shape), _I32], _SZ),
    "moe_workspace_init": ([_P, _SZ, _P], ctypes.c_int),
    "moe_workspace_flags": ([_P, ctypes.POINTER(_I32), _P], ctypes.c_int),
    "moe_layer_forward": ([ctypes.POINTER(Shape), ctypes.POINTER(Weights), _P, _P, _I32, _P, _P, _SZ, _P],
                          ctypes.c_int),
    "moe_layer_forward_static": ([ctypes.POINTER(Shape), ctypes.POINTER(Weights), _P, _P, _I32, _P, _P],
                                 ctypes.c_int),
    "moe_layer_forward_debug": ([ctypes.POINTER(Shape), ctypes.POINTER(Weights), _P, _P, _I32, _P, _P, _SZ,
                                 ctypes.POINTER(Debug), _P], ctypes.c_int),
    "moe_ctx_create": ([ctypes.POINTER(Shape), _I32, ctypes.POINTER(_P), _P], ctypes.c_int),
    "moe_prepare": ([_P, ctypes.POINTER(Weights), _P], ctypes.c_int),
    "moe_ctx_forward": ([_P, _P, _P, _I32, _P, _P], ctypes.c_int),
    "moe_ctx_flags": ([_P, ctypes.POINTER(_I32), _I32, _P], ctypes.c_int),
    "moe_ctx_destroy": ([_P], None),
    "moe_stage_name": ([_I32], ctypes.c_char_p),
    "moe_prof_create": ([ctypes.POINTER(_P), _I32], ctypes.c_int),
    "moe_prof_destroy": ([_P], None),
    "moe_prof_attach": ([_P], ctypes.c_int),
    "moe_prof_collect": ([_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_I32), _I32], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes, _fn.restype = _args, _res

EXPORTED = tuple(_SIGS)


def _check(status: int, what: str):
    if status != 0:
        raise MoEError(status, what)


def _layout(t, name, dtype=None, shape=None):
    """The checks the C ABI cannot make on a plain pointer: the shape and
    dtype it assumes and a dense layout."""
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _on_gpu(t, name):
    """Device pointer of t; a host pointer handed to the kernels would fault."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: must be in GPU memory")
    return t.data_ptr()


def _dev(t, name, dtype=None, shape=None):
    _layout(t, name, dtype, shape)
    return _on_gpu(t, name)


def _batch(shape, x, token_ids, out):
    """Checked pointers of one forward call's x [T, H] fp32, token_ids [T]
    int32 (hash routes) and out [T, H] fp32; returns (T, x, tokens, out)."""
    import torch
    if x.dim() != 2:
        raise ValueError(f"x: expected [tokens, {shape.hidden}], got {tuple(x.shape)}")
    T = x.shape[0]
    _layout(x, "x", torch.float32, (T, shape.hidden))
    _layout(token_ids, "token_ids", torch.int32, (T,))
    _layout(out, "out", torch.float32, (T, shape.hidden))
    return T, _on_gpu(x, "x"), _on_gpu(token_ids, "token_ids"), _on_gpu(out, "out")


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def abi_version() -> int:
    return _lib.moe_abi_version()


def matrix_bytes(fmt: int, rows: int, cols: int) -> int:
    return _lib.moe_matrix_bytes(fmt, rows, cols)


def make_shape(hidden, n_experts, top_k, ffn, has_shared=True, routed_fmt="q8", route="learned", vocab=0,
               table_k=0) -> Shape:
    return Shape(hidden, n_experts, top_k, ffn, 1 if has_shared else 0, FMT[routed_fmt] if isinstance(routed_fmt, str)
                 else routed_fmt, ROUTE[route] if isinstance(route, str) else route, vocab, table_k)


def workspace_bytes(shape: Shape, tokens: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(shape), tokens)


def pack_weights(fmt: int, canonical, packed, n_mats: int, rows: int, cols: int, stream=None):
    _check(_lib.moe_pack_weights(fmt, _dev(canonical, "canonical"), _dev(packed, "packed"), n_mats, rows, cols,
                                 _stream(stream)), "moe_pack_weights")


def workspace_init(ws, stream=None):
    _check(_lib.moe_workspace_init(_dev(ws, "workspace"), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_workspace_init")


def workspace_flags(ws, stream=None) -> int:
    f = _I32(0)
    _check(_lib.moe_workspace_flags(_dev(ws, "workspace"), ctypes.byref(f), _stream(stream)), "moe_workspace_flags")
    return f.value


def check_hash_table(table, n_experts: int, ws, stream=None) -> int:
    """-1 when the table is valid; raises MoEError(BAD_TABLE) naming the first bad row otherwise."""
    bad = _I32(-1)
    vocab, k = table.shape
    import torch
    st = _lib.moe_check_hash_table(_dev(table, "table", torch.int32), vocab, k, n_experts, _dev(ws, "workspace"),
                                   ws.numel() * ws.element_size(), ctypes.byref(bad), _stream(stream))
    if st != 0:
        raise MoEError(st, f"moe_check_hash_table (first bad row {bad.value})")
    return bad.value


def layer_forward(shape: Shape, weights: Weights, x, token_ids, out, ws, stream=None, debug: Debug | None = None):
    T, px, pt, po = _batch(shape, x, token_ids, out)
    pw = _dev(ws, "workspace")
    nbytes = ws.numel() * ws.element_size()
    if debug is None:
        st = _lib.moe_layer_forward(ctypes.byref(shape), ctypes.byref(weights), px, pt, T, po, pw, nbytes,
                                    _stream(stream))
    else:
        st = _lib.moe_layer_forward_debug(ctypes.byref(shape), ctypes.byref(weights), px, pt, T, po, pw, nbytes,
                                          ctypes.byref(debug), _stream(stream))
    _check(st, "moe_layer_forward")
    return out


def layer_forward_static(shape: Shape, weights: Weights, x, token_ids, out, stream=None):
    """moe_layer_forward_static: the layer on the library's per-GPU scratch array (allocates nothing)."""
    T, px, pt, po = _batch(shape, x, token_ids, out)
    _check(_lib.moe_layer_forward_static(ctypes.byref(shape), ctypes.byref(weights), px, pt, T, po,
                                         _stream(stream)), "moe_layer_forward_static")
    return out


class Context:
    """A library-owned layer (moe_ctx_*): the library allocates the workspace
    and the packed weights, validates the hash table at prepare and refuses
    forward calls until a prepare succeeded."""

    def __init__(self, shape: Shape, max_tokens: int, stream=None):
        self.shape = shape
        self._h = _P()
        _check(_lib.moe_ctx_create(ctypes.byref(shape), max_tokens, ctypes.byref(self._h), _stream(stream)),
               "moe_ctx_create")

    def prepare(self, canonical: Weights, stream=None):
        """canonical: device pointers to the canonical weight bytes (see moe.h)."""
        _check(_lib.moe_prepare(self._h, ctypes.byref(canonical), _stream(stream)), "moe_prepare")

    def forward(self, x, token_ids, out, stream=None):
        T, px, pt, po = _batch(self.shape, x, token_ids, out)
        _check(_lib.moe_ctx_forward(self._h, px, pt, T, po, _stream(stream)), "moe_ctx_forward")
        return out

    def flags(self, reset: bool = False, stream=None) -> int:
        f = _I32(0)
        _check(_lib.moe_ctx_flags(self._h, ctypes.byref(f), 1 if reset else 0, _stream(stream)), "moe_ctx_flags")
        return f.value

    def close(self):
        if self._h:
            _lib.moe_ctx_destroy(self._h)
            self._h = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Profiler:
    """Per-stage HIP-event timing of the forward calls made while attached."""

    def __init__(self, max_events: int = 65536):
        self._h = _P()
        _check(_lib.moe_prof_create(ctypes.byref(self._h), max_events), "moe_prof_create")

    def attach(self):
        _lib.moe_prof_attach(self._h)

    def detach(self):
        _lib.moe_prof_attach(None)

    def collect(self) -> dict:
        ms = (ctypes.c_float * len(STAGES))()
        n = (_I32 * len(STAGES))()
        _check(_lib.moe_prof_collect(self._h, ms, n, len(STAGES)), "moe_prof_collect")
        return {STAGES[i]: (float(ms[i]), int(n[i])) for i in range(len(STAGES)) if n[i] > 0}

    def close(self):
        if self._h:
            _lib.moe_prof_destroy(self._h)
            self._h = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


from .layer import MoELayer  # noqa: E402

__all__ = ["MoELayer", "MoEError", "Context", "Shape", "Weights", "Debug", "Profiler", "make_shape", "workspace_bytes",
           "pack_weights", "layer_forward", "layer_forward_static", "STATIC_SCRATCH_BYTES", "workspace_init", "workspace_flags", "check_hash_table", "matrix_bytes",
           "abi_version", "FMT_Q8", "FMT_Q2", "FLAG_BAD_TOKEN", "FLAG_BAD_TABLE_ENTRY", "FLAG_REPEATED_EXPERT", "ROUTE_LEARNED", "ROUTE_HASH", "ROUTE_HASH_SCORED", "EXPORTED",
           "LIB_PATH"]
