"""Entry points captured in a HIP graph (torch.cuda.graph) and replayed. Every replay runs on new
inputs written by eager work between replays, and is compared bit for bit with an eager call on
the same inputs (its own outputs and workspace). Run on an MI355X: ``pytest -m gpu``."""
import numpy as np
import pytest
import torch

from speculative_decoding_moe_amd.workloads import gen

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    from speculative_decoding_moe_amd import binding
    return binding


def _capture(fn):
    """Captures fn() into a graph after two warm-up runs on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _same(a, b):
    return np.array_equal(a.contiguous().view(torch.int32).cpu().numpy(), b.contiguous().view(torch.int32).cpu().numpy())


@pytest.mark.parametrize("name,flags,k,noalloc", [("verify", 0, 16, False), ("stack40_mxfp4", 3, 5, False),
                                                  ("verify", 0, 16, True), ("batched", 0, 48, False)])
def test_verify_block_replays(B, name, flags, k, noalloc):
    from speculative_decoding_moe_amd.workloads import device
    wl = gen.WORKLOADS[name]
    layer = device.make_layer(wl, 0, "cuda")
    x = torch.from_numpy(gen.hidden_states(wl, rep=0, k=k)).cuda()
    y, ye = torch.empty_like(x), torch.empty_like(x)
    ids = torch.empty((k, layer.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((k, layer.top_k), dtype=torch.float32, device="cuda")
    nw = torch.zeros(4, dtype=torch.int32, device="cuda")
    ide, we, nwe = torch.empty_like(ids), torch.empty_like(w), torch.zeros_like(nw)
    ws = torch.empty(layer.workspace_size(k), dtype=torch.uint8, device="cuda")
    wse = torch.empty_like(ws)
    if noalloc:
        call = lambda: B.moe_verify_block_noalloc(layer, x, flags, y, ids, w, nw)  # noqa: E731
    else:
        call = lambda: B.moe_verify_block(layer, x, flags, y, ids, w, nw, ws)  # noqa: E731
    print(f"[graph] capture {name} k={k} flags={flags} noalloc={noalloc}", flush=True)
    g = _capture(call)
    for rep in range(1, REPLAYS + 1):
        x.copy_(torch.from_numpy(gen.hidden_states(wl, rep=rep, k=k)))
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        B.moe_verify_block(layer, x, flags, ye, ide, we, nwe, wse)
        torch.cuda.synchronize()
        assert _same(y, ye) and _same(ids, ide) and _same(w, we), rep
        assert int(nw[0]) == int(nwe[0]) > 0, rep


@pytest.mark.parametrize("n_seq", [1, 5])
def test_accept_prefix_replays(B, n_seq):
    """Greedy acceptance replayed on new logits: a record left by the previous replay must never
    be taken for this one's (the launch's epoch argument is frozen in the graph)."""
    NT, V = 17, 151936
    gnr = torch.Generator(device="cuda").manual_seed(11)
    shape = (n_seq, NT, V) if n_seq > 1 else (NT, V)
    lg = torch.randn(shape, device="cuda", generator=gnr)
    dr = torch.randint(0, V, (n_seq, NT - 1) if n_seq > 1 else (NT - 1,), dtype=torch.int32, device="cuda",
                       generator=gnr)
    tg = torch.empty((n_seq, NT) if n_seq > 1 else (NT,), dtype=torch.int32, device="cuda")
    acc = torch.empty(max(n_seq, 4), dtype=torch.int32, device="cuda")
    tge, acce = torch.empty_like(tg), torch.empty_like(acc)
    if n_seq > 1:
        ws = torch.empty(B.accept_prefix_batch_workspace_size(n_seq, NT, V), dtype=torch.uint8, device="cuda")
        call = lambda tg_, acc_, ws_: B.accept_prefix_batch(lg, dr, tg_, acc_[:n_seq], ws_)  # noqa: E731
    else:
        ws = torch.empty(B.accept_prefix_workspace_size(NT, V), dtype=torch.uint8, device="cuda")
        call = lambda tg_, acc_, ws_: B.accept_prefix(lg, dr, tg_, acc_, ws_)  # noqa: E731
    wse = torch.empty_like(ws)
    print(f"[graph] capture accept n_seq={n_seq}", flush=True)
    g = _capture(lambda: call(tg, acc, ws))
    for rep in range(1, REPLAYS + 1):
        lg.normal_(generator=gnr)
        # plant the drafts so that some are accepted: copy the new argmax into a prefix of them
        am = lg.argmax(dim=-1).to(torch.int32)
        cut = rep % (NT - 1)
        if n_seq > 1:
            dr[:, :cut] = am[:, :cut]
        else:
            dr[:cut] = am[:cut]
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        call(tge, acce, wse)
        torch.cuda.synchronize()
        assert torch.equal(tg, tge) and torch.equal(acc[:n_seq], acce[:n_seq]), rep
        assert torch.equal(tg, am), rep
        assert int(acc[:n_seq].min()) >= cut, rep


def test_lm_head_accept_replays(B):
    NT, H, V = 5, 2048, 4096 + 8
    gnr = torch.Generator(device="cuda").manual_seed(5)
    w = (torch.randn((V, H), device="cuda", generator=gnr) * 0.02).to(torch.bfloat16)
    wt = B.pack_head(w)
    h = torch.randn((NT, H), device="cuda", generator=gnr)
    dr = torch.zeros(NT - 1, dtype=torch.int32, device="cuda")
    tg, acc = torch.empty(NT, dtype=torch.int32, device="cuda"), torch.empty(4, dtype=torch.int32, device="cuda")
    tge, acce = torch.empty_like(tg), torch.empty_like(acc)
    ws = torch.empty(B.lm_head_accept_workspace_size(NT, H, V), dtype=torch.uint8, device="cuda")
    wse = torch.empty_like(ws)
    print("[graph] capture lm_head_accept", flush=True)
    g = _capture(lambda: B.lm_head_accept(h, wt, V, dr, tg, acc, ws))
    for rep in range(1, REPLAYS + 1):
        h.normal_(generator=gnr)
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        B.lm_head_accept(h, wt, V, dr, tge, acce, wse)
        torch.cuda.synchronize()
        assert torch.equal(tg, tge) and int(acc[0]) == int(acce[0]), rep
