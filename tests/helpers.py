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
