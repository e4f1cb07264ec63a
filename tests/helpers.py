"""Glue between the seeded generators and the oracle's layer interface (tests only)."""
from functools import lru_cache

from speculative_decoding_moe_amd.workloads import gen


class GenLayer:
    """One generated MoE layer, exposing router() / expert(e) / shared() as raw encoded arrays."""

    def __init__(self, wl, layer=0):
        self.wl = wl
        self.layer = layer

    @lru_cache(maxsize=None)
    def router(self):
        return gen.router_weight(self.wl, self.layer)

    def expert(self, e):
        return gen.expert_tensors(self.wl, self.layer, int(e))

    def shared(self):
        return gen.shared_tensors(self.wl, self.layer)


class ArrayLayer:
    """A layer given directly as arrays (bf16 bits / fp32 router), for hand-built cases."""

    def __init__(self, router, experts, shared=None):
        self._router = router
        self._experts = experts
        self._shared = shared

    def router(self):
        return self._router

    def expert(self, e):
        return self._experts[int(e)]

    def shared(self):
        return self._shared


# Stale-workspace fill patterns: bytes, and word patterns that are -0 or NaN as bf16 or fp32 (a
# stale -0 or NaN reaching a matrix-core padding column would change results; "Speculating on a
# Strix Halo (part 2)", sections "Two bugs upstream" and "Whose bug is it?").
WS_FILLS = {
    "zero": 0x00, "ff": 0xFF, "80": 0x80, "7f": 0x7F,
    "neg_zero_bf16": ("int16", -32768),          # 0x8000 in every 16-bit word
    "neg_zero_f32": ("int32", -(1 << 31)),       # 0x80000000 in every 32-bit word
    "nan_bf16": ("int16", 0x7FC0),
    "nan_f32": ("int32", 0x7FC00000),
}


def fill_ws(ws, fill):
    """Fills a uint8 workspace tensor with a byte (int) or a (dtype name, word) pattern."""
    import torch
    if fill is None:
        return
    if isinstance(fill, tuple):
        dtype, v = fill
        n = ws.numel() - ws.numel() % 4
        ws[:n].view(getattr(torch, dtype)).fill_(v)
    else:
        ws.fill_(fill)
