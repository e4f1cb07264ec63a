"""moe_verify_block_noalloc (the library's own device scratch, no allocation) against
moe_verify_block on a caller workspace: two calls in a row, the second on a smaller block, each
bit-identical to the caller-workspace call (same kernels, so the same bits)."""
import numpy as np
import pytest
import torch

from speculative_decoding_moe_amd.workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    from speculative_decoding_moe_amd import binding
    return binding


def _run(B, layer, x, flags, noalloc):
    k = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    y = torch.full_like(xd, float("nan"))
    ids = torch.full((k, layer.top_k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((k, layer.top_k), float("nan"), dtype=torch.float32, device="cuda")
    nw = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    if noalloc:
        B.moe_verify_block_noalloc(layer, xd, flags, y, ids, w, nw)
    else:
        ws = torch.empty(layer.workspace_size(k), dtype=torch.uint8, device="cuda")
        B.moe_verify_block(layer, xd, flags, y, ids, w, nw, ws)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (y, ids, w)] + [int(nw[0])]


@pytest.mark.parametrize("name,flags,ks", [("verify", 0, (16, 5)), ("stack40_mxfp4", 3, (16, 1)),
                                           ("tiny", 0, (4, 2))])
def test_noalloc_matches_workspace_call_twice(B, name, flags, ks):
    from speculative_decoding_moe_amd.workloads import device
    wl = gen.WORKLOADS[name]
    layer = device.make_layer(wl, 0, "cuda")
    for i, k in enumerate(ks):
        x = gen.hidden_states(wl, rep=600 + i, k=k)
        ref = _run(B, layer, x, flags, noalloc=False)
        got = _run(B, layer, x, flags, noalloc=True)
        for a, b, what in zip(got, ref, ("y", "ids", "w", "n_woken")):
            assert np.array_equal(np.asarray(a), np.asarray(b)), (name, k, what)
        assert np.all(np.isfinite(got[0])) and got[3] >= wl.shape.top_k


def test_noalloc_gathered_call_within_the_scratch(B):
    """A gathered call (MOE_GATHER) small enough for the scratch, after a larger single-block call."""
    from speculative_decoding_moe_amd.workloads import device
    wl = gen.WORKLOADS["verify"]
    layer = device.make_layer(wl, 0, "cuda")
    assert layer.workspace_size(40) <= B.NOALLOC_SCRATCH_BYTES
    for i, (k, flags) in enumerate(((16, 0), (40, B.MOE_GATHER), (3, B.MOE_GATHER))):
        x = gen.hidden_states(wl, rep=700 + i, k=k)
        ref = _run(B, layer, x, flags, noalloc=False)
        got = _run(B, layer, x, flags, noalloc=True)
        for a, b, what in zip(got, ref, ("y", "ids", "w", "n_woken")):
            assert np.array_equal(np.asarray(a), np.asarray(b)), (k, flags, what)
