"""moe_verify_stack against chained moe_verify_block calls, through the C ABI: one call for the
whole stack must give the chained calls' outputs bit for bit, and the same woken counts per layer,
whatever the workspace held. The chained calls are themselves checked against the oracle in
test_gpu_parity.py (the teacher-forced and final-stream stack tests). Run on an MI355X:
``pytest -m gpu``.
"""
import numpy as np
import pytest
import torch

from helpers import WS_FILLS, fill_ws
from speculative_decoding_moe_amd.workloads import gen

pytestmark = pytest.mark.gpu

PRE, RES = 1, 2


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    from speculative_decoding_moe_amd import binding
    return binding


def _layers(wl, n):
    from speculative_decoding_moe_amd.workloads import device
    print(f"[stack] building {n} layers of {wl.shape}", flush=True)
    return [device.make_layer(wl, li, "cuda") for li in range(n)]


def chained(B, layers, x, flags):
    k, H = x.shape
    ws = torch.empty(layers[0].workspace_size(k), dtype=torch.uint8, device="cuda")
    bufs = [torch.empty((k, H), dtype=torch.float32, device="cuda") for _ in range(2)]
    nw = torch.zeros((len(layers), 4), dtype=torch.int32, device="cuda")
    cur = x
    for i, L in enumerate(layers):
        B.moe_verify_block(L, cur, flags, bufs[i % 2], None, None, nw[i], ws)
        cur = bufs[i % 2]
    torch.cuda.synchronize()
    return cur.cpu().numpy(), nw[:, 0].cpu().numpy()


def stacked(B, layers, x, flags, ws_fill=None):
    k, H = x.shape
    ws = torch.empty(B.moe_verify_stack_workspace_size(layers[0], k), dtype=torch.uint8, device="cuda")
    fill_ws(ws, None if ws_fill is None else WS_FILLS[ws_fill])
    y = torch.empty((k, H), dtype=torch.float32, device="cuda")
    nw = torch.full((len(layers),), -7, dtype=torch.int32, device="cuda")
    print(f"[stack] n={len(layers)} k={k} flags={flags} fill={ws_fill}", flush=True)
    B.moe_verify_stack(layers, x, flags, y, nw, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), nw.cpu().numpy()


SHAPES = {
    # the stack's own layer: mxfp4 routed experts, bf16 shared expert, four router column slices
    "mxfp4_h2048": (gen.WORKLOADS["stack40_mxfp4"].shape, 4),
    # bf16 at the verify layer's size
    "bf16_h2048": (gen.LayerShape(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512), 3),
    # one 768-column router slice (six 128-column windows, a ragged last pass of the combine), a
    # partial expert tile (40 experts), no shared expert
    "bf16_h768": (gen.LayerShape(hidden=768, n_experts=40, top_k=6, inter=256, shared_inter=0), 4),
    # two slices, mxfp4, I = 1024
    "mxfp4_h1024": (gen.LayerShape(hidden=1024, n_experts=64, top_k=4, inter=1024, shared_inter=1024,
                                   wdtype="mxfp4"), 3),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_stack_equals_chained_calls(B, name):
    shape, n = SHAPES[name]
    wl = gen.Workload("stack_" + name, shape, k=16, seed=8100, n_layers=n, pre_norm=True, residual=True)
    layers = _layers(wl, n)
    for k, flags in ((16, PRE | RES), (5, PRE | RES), (1, PRE | RES), (16, 0), (7, RES)):
        x = torch.from_numpy(gen.hidden_states(wl, rep=40 + k + flags, k=k)).cuda()
        yc, nc = chained(B, layers, x, flags)
        ys, ns = stacked(B, layers, x, flags, ws_fill="nan_f32" if k == 5 else None)
        assert np.array_equal(nc, ns), (k, flags, nc, ns)
        assert np.all(ns > 0)
        assert np.array_equal(yc.view(np.uint32), ys.view(np.uint32)), (
            k, flags, float(np.abs(yc.astype(np.float64) - ys).max()))
    del layers
    torch.cuda.empty_cache()


def test_stack_single_layer_and_replay(B):
    """One layer (no fused launch) equals moe_verify_block; a stack captured in a HIP graph and
    replayed on new inputs equals eager calls on each replay."""
    shape, _ = SHAPES["bf16_h768"]
    wl = gen.Workload("stack_replay", shape, k=16, seed=8200, n_layers=3, pre_norm=True, residual=True)
    layers = _layers(wl, 3)
    x = torch.from_numpy(gen.hidden_states(wl, rep=1, k=16)).cuda()
    yc, nc = chained(B, layers[:1], x, PRE | RES)
    ys, ns = stacked(B, layers[:1], x, PRE | RES)
    assert np.array_equal(yc.view(np.uint32), ys.view(np.uint32)) and np.array_equal(nc, ns)
    ws = torch.empty(B.moe_verify_stack_workspace_size(layers[0], 16), dtype=torch.uint8, device="cuda")
    xin = torch.empty((16, shape.hidden), dtype=torch.float32, device="cuda")
    y = torch.empty_like(xin)
    nw = torch.zeros(3, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    xin.copy_(x)
    with torch.cuda.stream(s):
        B.moe_verify_stack(layers, xin, PRE | RES, y, nw, ws)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.moe_verify_stack(layers, xin, PRE | RES, y, nw, ws)
    for rep in range(3):
        xr = torch.from_numpy(gen.hidden_states(wl, rep=100 + rep, k=16)).cuda()
        xin.copy_(xr)
        torch.cuda.synchronize()
        print(f"[stack] replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        got, gn = y.cpu().numpy(), nw.cpu().numpy()
        want, wn = chained(B, layers, xr, PRE | RES)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), rep
        assert np.array_equal(gn, wn), rep
    del layers
    torch.cuda.empty_cache()
