"""Parity at the largest layer the boundary accepts: hidden 2048, 512 experts, top-16, expert and
shared-expert intermediate 1024, bf16 and mxfp4. Each routed bf16 weight tensor is then 2 GiB, the
whole range the kernels' 32-bit buffer offsets address, and the last expert's rows sit at its top.
Both paths run: the single-block path at k = 16 (pre-norm and residual) and the gathered path at
64 tokens. Every token's routing is checked against the oracle's router; the outputs of sampled
tokens (the last, and the first token routed to the highest expert id) against the oracle, which
regenerates only the experts those tokens wake. Run on an MI355X: ``pytest -m gpu``.
"""
import numpy as np
import pytest
import torch

from test_gpu_gather import B, PRE, RES, check_outputs, check_routing, run  # noqa: F401
from speculative_decoding_moe_amd.workloads import gen

pytestmark = pytest.mark.gpu

MX_TOL = 3e-2
MAX_SHAPES = {
    "bf16": gen.LayerShape(hidden=2048, n_experts=512, top_k=16, inter=1024, shared_inter=1024),
    "mxfp4": gen.LayerShape(hidden=2048, n_experts=512, top_k=16, inter=1024, shared_inter=1024, wdtype="mxfp4"),
}


def sample_rows(ids):
    """The last token and the first token routed to the highest expert id in use."""
    top = int(np.argmax((ids == ids.max()).any(axis=1)))
    return sorted({ids.shape[0] - 1, top})


def check_outputs_mx(g, x, wl, rows, flags):
    import oracle
    from helpers import GenLayer
    rows = np.asarray(rows)
    ref = oracle.moe_block(x[rows], GenLayer(wl, 0), wl.shape.top_k, forced_ids=g["ids"][rows],
                           pre_norm=bool(flags & PRE), residual=bool(flags & RES), rms_eps=wl.rms_eps)
    gy, ry = g["y"][rows].astype(np.float64), ref["y"]
    if flags & RES:
        gy, ry = gy - x[rows], ry - x[rows]
    rms = float(np.sqrt(np.mean(ry ** 2)))
    err = float(np.abs(gy - ry).max())
    assert err <= MX_TOL * rms, f"max|dy| {err:.3e} > {MX_TOL} x RMS {rms:.3e}"
    return err / rms


@pytest.mark.parametrize("dtype", ["bf16", "mxfp4"])
def test_largest_layer(B, dtype):
    from speculative_decoding_moe_amd.workloads import device
    shape = MAX_SHAPES[dtype]
    wl = gen.Workload("maxsize", shape, k=16, seed=2468)
    print(f"[maxsize] building the {dtype} layer (E 512, H 2048, I 1024)", flush=True)
    layer = device.make_layer(wl, 0, "cuda")
    try:
        for k, flags in ((16, PRE | RES), (64, PRE | RES)):
            x = gen.hidden_states(wl, rep=k + flags, k=k)
            g = run(B, layer, x, flags)
            check_routing(g, x, wl, flags=flags & PRE)
            rows = sample_rows(g["ids"])
            if dtype == "bf16":
                r = check_outputs(g, x, wl, rows, flags, compare_delta=True)
            else:
                r = check_outputs_mx(g, x, wl, rows, flags)
            print(f"[maxsize] {dtype} k={k} flags={flags}: U={g['n_woken']} max id {int(g['ids'].max())} "
                  f"rows {rows} err/rms={r:.2e}", flush=True)
    finally:
        del layer
        torch.cuda.empty_cache()
