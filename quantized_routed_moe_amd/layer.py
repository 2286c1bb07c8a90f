"""MoELayer: device-resident packed weights + workspace around the C ABI."""
from __future__ import annotations

import numpy as np
import torch

from . import (FMT, FMT_Q8, Debug, Weights, check_hash_table, layer_forward, make_shape, matrix_bytes, pack_weights,
               workspace_bytes, workspace_init, workspace_flags)

ALIGN = 256


def _device_bytes(n: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte (or better) aligned blocks
    t = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    assert t.data_ptr() % ALIGN == 0
    return t


def _upload(a, device) -> torch.Tensor:
    if isinstance(a, np.ndarray):
        a = torch.from_numpy(np.ascontiguousarray(a))
    return a.to(device, non_blocking=False).contiguous()


class MoELayer:
    """One routed-MoE layer: shape, packed weights on the GPU, a workspace.

    Weights are given in the canonical block formats (moe.h) and packed once
    on the device by the library's repack kernel.
    """

    def __init__(self, hidden, n_experts, top_k, ffn, has_shared=True, routed_fmt="q8", route="learned", vocab=0,
                 device="cuda", table_k=0):
        self.device = torch.device(device)
        self.H, self.E, self.k, self.F = hidden, n_experts, top_k, ffn
        self.routed_fmt, self.route, self.vocab, self.table_k = routed_fmt, route, vocab, table_k
        self.has_shared = has_shared
        self.shape = make_shape(hidden, n_experts, top_k, ffn, has_shared, routed_fmt, route, vocab, table_k)
        self.router_w = self.router_b = self.hash_table = None
        self.gate = self.up = self.down = None
        self.sh_gate = self.sh_up = self.sh_down = None
        self.ws = None
        self.ws_tokens = 0

    # -------------------------------------------------------------- weights
    def pack_bank(self, canonical, fmt: int, n_mats: int, rows: int, cols: int) -> torch.Tensor:
        mb = matrix_bytes(fmt, rows, cols)
        if mb < 0:
            raise ValueError("matrix shape does not fit the format")
        src = _upload(canonical, self.device).view(torch.uint8).reshape(-1)
        if src.numel() != n_mats * mb:
            raise ValueError(f"canonical bank has {src.numel()} bytes, expected {n_mats * mb}")
        dst = _device_bytes(n_mats * mb, self.device)
        pack_weights(fmt, src, dst, n_mats, rows, cols)
        torch.cuda.current_stream(self.device).synchronize()
        del src
        return dst

    def load(self, inp: dict) -> "MoELayer":
        """Upload canonical tensors (numpy or CPU torch): router_w (learned, hash_scored),
        router_b (learned), hash_table (hash routes), gate/up/down banks and
        sh_gate/sh_up/sh_down."""
        fmt = FMT[self.routed_fmt]
        if self.route != "hash":
            self.router_w = _upload(inp["router_w"], self.device)
        if self.route == "learned" and inp.get("router_b") is not None:
            self.router_b = _upload(inp["router_b"], self.device)
        if self.route != "learned":
            self.hash_table = _upload(inp["hash_table"], self.device)
        self.gate = self.pack_bank(inp["gate"], fmt, self.E, self.F, self.H)
        self.up = self.pack_bank(inp["up"], fmt, self.E, self.F, self.H)
        self.down = self.pack_bank(inp["down"], fmt, self.E, self.H, self.F)
        if self.has_shared:
            self.sh_gate = self.pack_bank(inp["sh_gate"], FMT_Q8, 1, self.F, self.H)
            self.sh_up = self.pack_bank(inp["sh_up"], FMT_Q8, 1, self.F, self.H)
            self.sh_down = self.pack_bank(inp["sh_down"], FMT_Q8, 1, self.H, self.F)
        return self

    def weights(self, router_w=None, sh=None) -> Weights:
        """ctypes weight struct; router_w / sh=(gate, up, down) override the stored ones."""
        rw = self.router_w if router_w is None else router_w
        g, u, d = (self.sh_gate, self.sh_up, self.sh_down) if sh is None else sh

        def p(t):
            return None if t is None else t.data_ptr()
        return Weights(p(rw), p(self.router_b), p(self.hash_table), p(self.gate), p(self.up), p(self.down),
                       p(g), p(u), p(d))

    def check_table(self) -> int:
        self.ensure_workspace(1)
        return check_hash_table(self.hash_table, self.E, self.ws)

    # ------------------------------------------------------------ workspace
    def ensure_workspace(self, tokens: int):
        if self.ws is None or tokens > self.ws_tokens:
            n = workspace_bytes(self.shape, tokens)
            if n == 0:
                raise ValueError("unsupported shape or token count")
            self.ws = _device_bytes(n, self.device)
            self.ws_tokens = tokens
            workspace_init(self.ws)
        return self.ws

    def flags(self) -> int:
        return workspace_flags(self.ws)

    def reset_flags(self):
        """Clear the workspace's sticky flags (and its other control words)."""
        workspace_init(self.ws)

    # -------------------------------------------------------------- forward
    def forward(self, x: torch.Tensor, token_ids: torch.Tensor | None = None, out: torch.Tensor | None = None,
                weights: Weights | None = None, stream=None) -> torch.Tensor:
        T = x.shape[0]
        self.ensure_workspace(T)
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.float32, device=self.device)
        layer_forward(self.shape, weights or self.weights(), x, token_ids, out, self.ws, stream)
        return out

    def forward_debug(self, x: torch.Tensor, token_ids: torch.Tensor | None = None, sum_row_stride: int = 0,
                      stream=None) -> dict:
        """Forward plus copies of the intermediates (see moe_debug in moe.h)."""
        T, H, E, k, F = x.shape[0], self.H, self.E, self.k, self.F
        P = T * k + (T if self.has_shared else 0)
        dev = self.device
        r = {
            "out": torch.empty((T, H), dtype=torch.float32, device=dev),
            "ids": torch.empty((T, k), dtype=torch.int32, device=dev),
            "w": torch.empty((T, k), dtype=torch.float32, device=dev),
            "logits": torch.zeros((T, E), dtype=torch.float32, device=dev),
            "xq": torch.empty((T, H), dtype=torch.int8, device=dev),
            "xd": torch.empty((T, H // 32), dtype=torch.float32, device=dev),
            "counts": torch.empty(E, dtype=torch.int32, device=dev),
            "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
            "perm": torch.empty(T * k, dtype=torch.int32, device=dev),
            "hq": torch.empty((P, F), dtype=torch.int8, device=dev),
            "hd": torch.empty((P, F // 32), dtype=torch.float32, device=dev),
        }
        dbg = Debug()
        for name in ("ids", "w", "logits", "xq", "xd", "counts", "offsets", "perm", "hq", "hd"):
            setattr(dbg, name, r[name].data_ptr())
        if sum_row_stride > 0:
            s = sum_row_stride
            per_h = H // 32 if self.routed_fmt == "q8" else H // 16
            per_f = F // 32 if self.routed_fmt == "q8" else F // 16
            # shared-expert pairs are Q8 (one sum per 32-block); routed 2-bit pairs have one per 16
            r["gate_sums"] = torch.full((P, F // s, per_h), -(2 ** 31), dtype=torch.int32, device=dev)
            r["up_sums"] = torch.full((P, F // s, per_h), -(2 ** 31), dtype=torch.int32, device=dev)
            r["down_sums"] = torch.full((P, H // s, per_f), -(2 ** 31), dtype=torch.int32, device=dev)
            dbg.gate_sums, dbg.up_sums, dbg.down_sums = (r[n].data_ptr() for n in ("gate_sums", "up_sums", "down_sums"))
            dbg.sum_row_stride = s
        self.ensure_workspace(T)
        layer_forward(self.shape, self.weights(), x, token_ids, r["out"], self.ws, stream, debug=dbg)
        return r
