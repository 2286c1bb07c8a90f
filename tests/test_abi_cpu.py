"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/moe.h, and rejects bad arguments on the host before it
enqueues anything (so no HIP call is made in these tests)."""
import ctypes
import os
import re

import pytest

import quantized_routed_moe_amd as qr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = qr._lib
OK, INVALID, UNSUPPORTED, TOO_MANY, WORKSPACE = 0, -1, -2, -3, -4


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), f"{n} declared in moe.h but not exported"
    assert set(names) == set(qr.EXPORTED)


def test_version_and_status_strings():
    assert qr.abi_version() == 3
    for st in range(-8, 1):
        assert L.moe_status_string(st) not in (None, b"unknown status")
    assert L.moe_status_string(-99) == b"unknown status"


def test_matrix_bytes():
    assert qr.matrix_bytes(qr.FMT_Q8, 2048, 4096) == 2048 * 4096 * 34 // 32
    assert qr.matrix_bytes(qr.FMT_Q2, 2048, 4096) == 2048 * 4096 * 84 // 256
    assert qr.matrix_bytes(qr.FMT_Q8, 4, 48) == -1
    assert qr.matrix_bytes(qr.FMT_Q2, 4, 128) == -1
    assert qr.matrix_bytes(7, 4, 256) == -1


def shape(**kw):
    base = dict(hidden=4096, n_experts=256, top_k=6, ffn=2048, has_shared=True, routed_fmt="q8", route="learned",
                vocab=0)
    base.update(kw)
    return qr.make_shape(**base)


def test_workspace_bytes_monotone_and_rejects_bad_shapes():
    s = shape()
    sizes = [qr.workspace_bytes(s, t) for t in (0, 1, 2, 31, 32, 33, 100, 2048, 16384)]
    assert all(b > 0 for b in sizes) and sizes == sorted(sizes)
    assert qr.workspace_bytes(s, 16385) == 0
    for bad in (dict(hidden=96), dict(hidden=8192), dict(ffn=64), dict(top_k=0), dict(top_k=9), dict(n_experts=4),
                dict(n_experts=2048), dict(routed_fmt=3), dict(route=0), dict(route=4), dict(route="hash", vocab=0),
                dict(route="hash_scored", vocab=0), dict(route="hash", vocab=10, table_k=5),
                dict(route="hash_scored", vocab=10, table_k=9), dict(routed_fmt="q2", hidden=256)):
        assert qr.workspace_bytes(shape(**bad), 4) == 0, bad
    for good in (dict(route="hash", vocab=10, table_k=6), dict(route="hash", vocab=10, top_k=4, table_k=8),
                 dict(route="hash_scored", vocab=10), dict(n_experts=384, top_k=8)):
        assert qr.workspace_bytes(shape(**good), 4) > 0, good


FAKE = 1 << 20  # 16- and 256-byte aligned host integers: never dereferenced by the host checks


def call_forward(s, w, x=FAKE, tok=None, T=4, out=FAKE * 3, ws=FAKE * 5, ws_bytes=1 << 40):
    return L.moe_layer_forward(ctypes.byref(s), ctypes.byref(w) if w is not None else None, x, tok, T, out, ws,
                               ws_bytes, None)


def good_weights(shared=True):
    p = [FAKE * (10 + i) for i in range(9)]
    w = qr.Weights(*p)
    if not shared:
        w.sh_gate = w.sh_up = w.sh_down = None
    return w


def test_forward_validation_codes():
    s, w = shape(), good_weights()
    assert call_forward(s, None) == INVALID
    assert L.moe_layer_forward(None, ctypes.byref(w), FAKE, None, 4, FAKE * 3, FAKE * 5, 1 << 40, None) == INVALID
    assert call_forward(shape(hidden=96), w) == UNSUPPORTED
    assert call_forward(shape(top_k=7, n_experts=6), w) == INVALID
    assert call_forward(s, w, T=-1) == INVALID
    assert call_forward(s, w, T=16385) == TOO_MANY
    assert call_forward(s, w, x=FAKE + 4) == INVALID                      # misaligned x
    assert call_forward(s, w, out=FAKE + 8) == INVALID                    # misaligned out
    assert call_forward(s, w, out=FAKE + 4096 * 4) == INVALID             # out overlaps x
    assert call_forward(s, w, ws=FAKE * 5 + 16) == WORKSPACE              # misaligned workspace
    assert call_forward(s, w, ws_bytes=1000) == WORKSPACE                 # too small
    w2 = good_weights()
    w2.router_w = None
    assert call_forward(s, w2) == INVALID                                 # learned router without weights
    assert call_forward(s, good_weights(shared=False)) == INVALID         # shared expert missing
    assert call_forward(shape(has_shared=False), good_weights()) == INVALID  # shared given but not declared
    hs = shape(route="hash", vocab=131072)
    assert call_forward(hs, w, tok=None) == INVALID                       # hash routing needs token ids
    w3 = good_weights()
    w3.hash_table = None
    assert call_forward(hs, w3, tok=FAKE * 7) == INVALID
    ss = shape(route="hash_scored", vocab=131072, top_k=4, table_k=6)
    assert call_forward(ss, w2, tok=FAKE * 7) == INVALID                  # score-weighted hash needs the router
    assert call_forward(ss, w3, tok=FAKE * 7) == INVALID                  # ... and the table
    assert call_forward(ss, w, tok=None) == INVALID                       # ... and token ids
    assert call_forward(s, w, T=0) == OK                                  # empty batch: nothing to do
    assert L.moe_layer_forward(ctypes.byref(s), None, None, None, 0, None, None, 0, None) == OK


def test_pack_and_table_validation_codes():
    assert L.moe_pack_weights(1, None, FAKE, 1, 8, 64, None) == INVALID
    assert L.moe_pack_weights(1, FAKE, FAKE + 4, 1, 8, 64, None) == INVALID
    assert L.moe_pack_weights(1, FAKE, FAKE, 1, 8, 64, None) == INVALID      # overlap
    assert L.moe_pack_weights(2, FAKE, FAKE * 9, 1, 8, 64, None) == INVALID  # cols not a multiple of 256
    assert L.moe_pack_weights(1, FAKE, FAKE * 9, 0, 8, 64, None) == OK       # nothing to pack
    bad = ctypes.c_int32(0)
    assert L.moe_check_hash_table(None, 10, 6, 256, FAKE, 4096, ctypes.byref(bad), None) == INVALID
    assert L.moe_check_hash_table(FAKE, 10, 6, 4, FAKE, 4096, ctypes.byref(bad), None) == INVALID
    assert L.moe_check_hash_table(FAKE, 10, 6, 256, FAKE, 16, ctypes.byref(bad), None) == WORKSPACE


def test_profiler_argument_checks():
    h = ctypes.c_void_p()
    assert L.moe_prof_create(ctypes.byref(h), 1) == INVALID
    assert L.moe_prof_create(None, 16) == INVALID
    assert L.moe_stage_name(5) == b"gateup" and L.moe_stage_name(99) == b"?"


def test_one_hip_runtime_per_process():
    """Importing the binding before torch must not map a second HIP runtime
    (the library has to use the runtime that owns torch's device memory)."""
    import subprocess
    import sys
    code = ("import quantized_routed_moe_amd, torch\n"
            "print('\\n'.join(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l})))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__)))).stdout.split()
    assert len(out) == 1, out


def test_context_calls_reject_bad_arguments_on_the_host():
    """The context calls refuse NULL handles, bad shapes and token limits
    before any HIP call (a valid shape would allocate, so none is used)."""
    h = ctypes.c_void_p()
    s = shape()
    assert L.moe_ctx_create(ctypes.byref(s), 4, None, None) == INVALID
    for bad in (dict(hidden=96), dict(top_k=9), dict(route=0), dict(routed_fmt="q2", hidden=256)):
        st = L.moe_ctx_create(ctypes.byref(shape(**bad)), 4, ctypes.byref(h), None)
        assert st in (INVALID, UNSUPPORTED), bad
        assert not h.value
    assert L.moe_ctx_create(ctypes.byref(s), 0, ctypes.byref(h), None) == INVALID
    assert L.moe_ctx_create(ctypes.byref(s), 16385, ctypes.byref(h), None) == TOO_MANY
    assert not h.value
    w = good_weights()
    assert L.moe_prepare(None, ctypes.byref(w), None) == INVALID
    assert L.moe_ctx_forward(None, FAKE, None, 4, FAKE * 3, None) == INVALID
    f = ctypes.c_int32(0)
    assert L.moe_ctx_flags(None, ctypes.byref(f), 0, None) == INVALID
    L.moe_ctx_destroy(None)
    assert L.moe_status_string(-8) == b"context has no prepared weights"


def test_static_forward_refuses_before_touching_the_device():
    """moe_layer_forward_static validates every argument, and refuses a batch
    whose workspace exceeds the static scratch, before it looks up the
    device array (there is no device here: a lookup would fail as a HIP
    error instead)."""
    s = shape()
    w = good_weights()
    assert qr.workspace_bytes(s, 120) <= qr.STATIC_SCRATCH_BYTES < qr.workspace_bytes(s, 121)
    assert L.moe_layer_forward_static(ctypes.byref(s), ctypes.byref(w), FAKE, None, 121, FAKE * 3, None) == WORKSPACE
    assert L.moe_layer_forward_static(ctypes.byref(s), ctypes.byref(w), FAKE, None, 16385, FAKE * 3,
                                      None) == TOO_MANY
    assert L.moe_layer_forward_static(ctypes.byref(s), ctypes.byref(w), None, None, 4, FAKE * 3, None) == INVALID
    assert L.moe_layer_forward_static(ctypes.byref(s), None, FAKE, None, 4, FAKE * 3, None) == INVALID
    assert L.moe_layer_forward_static(ctypes.byref(shape(hidden=96)), ctypes.byref(w), FAKE, None, 4, FAKE * 3,
                                      None) == UNSUPPORTED
    assert L.moe_layer_forward_static(ctypes.byref(s), ctypes.byref(w), FAKE, None, 0, FAKE * 3, None) == OK
    # out overlapping x
    assert L.moe_layer_forward_static(ctypes.byref(s), ctypes.byref(w), FAKE, None, 4, FAKE + 16, None) == INVALID


def test_binding_checks_caller_tensors_before_any_call():
    """The Python binding passes plain pointers, so it checks what the C ABI
    cannot: x and out [T, hidden] fp32, token_ids [T] int32, dense layout and
    GPU memory.  Each bad argument raises ValueError before the library is
    called (these tensors are on the CPU, the last check every case reaches
    when its shape and type are right)."""
    import torch

    s = shape()
    w = good_weights()
    H = s.hidden
    ws = torch.zeros(64, dtype=torch.uint8)
    x = torch.zeros(4, H)
    out = torch.zeros(4, H)
    tok = torch.zeros(4, dtype=torch.int32)
    cases = [
        (dict(x=torch.zeros(H)), "x: expected"),
        (dict(x=torch.zeros(4, H + 32)), "x: expected shape"),
        (dict(x=torch.zeros(4, H, dtype=torch.float64)), "x: expected torch.float32"),
        (dict(x=torch.zeros(H, 4).t()), "x: must be contiguous"),
        (dict(out=torch.zeros(3, H)), "out: expected shape"),
        (dict(token_ids=torch.zeros(5, dtype=torch.int32)), "token_ids: expected shape"),
        (dict(token_ids=torch.zeros(4, dtype=torch.int64)), "token_ids: expected torch.int32"),
        (dict(), "x: must be in GPU memory"),
    ]
    for change, msg in cases:
        a = dict(x=x, token_ids=tok, out=out)
        a.update(change)
        with pytest.raises(ValueError, match=msg):
            qr.layer_forward(s, w, a["x"], a["token_ids"], a["out"], ws)
        with pytest.raises(ValueError, match=msg):
            qr.layer_forward_static(s, w, a["x"], a["token_ids"], a["out"])
    with pytest.raises(ValueError, match="workspace: must be in GPU memory"):
        qr.workspace_init(ws)
    with pytest.raises(ValueError, match="table: must be in GPU memory"):
        qr.check_hash_table(torch.zeros(8, 4, dtype=torch.int32), 16, ws)
