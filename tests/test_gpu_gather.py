"""GPU parity of the gathered path of moe_verify_block (many sequences verified together: k > 16
tokens, or MOE_GATHER at any k), called through the C ABI, against the CPU oracle on the same
seeded inputs. Run on an MI355X: ``pytest -m gpu``.

Bars, as for the single-block path: expert ids bit-exact except where the oracle's logits are
within 1e-4 of a different valid selection; routing weights within 1e-6; woken counts exact;
outputs within 1e-2 x RMS (bf16 experts) in max-abs error. At hundreds of tokens the routing of
every token is checked against the oracle's router, and the outputs on sampled tokens (the
oracle computes each token on its own). Token independence is checked exactly: a token's row
does not depend on which other tokens share the call.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import WS_FILLS, GenLayer, fill_ws
from speculative_decoding_moe_amd.workloads import gen

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2
TIE = 1e-4
PRE, RES, GATHER = 1, 2, 4


@pytest.fixture(scope="session")
def B():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    from speculative_decoding_moe_amd import binding
    return binding


_LAYERS = {}


def dev_layer(wl, layer=0):
    from speculative_decoding_moe_amd.workloads import device
    key = (wl, layer)
    if key not in _LAYERS:
        if len(_LAYERS) > 4:
            _LAYERS.clear()
        _LAYERS[key] = device.make_layer(wl, layer, "cuda")
    return _LAYERS[key]


def run(B, layer, x, flags=0, ws_fill=None, ws=None):
    k = x.shape[0]
    print(f"[gather] k={k} flags={flags} E={layer.n_experts} H={layer.hidden}", flush=True)
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    y = torch.empty_like(xd)
    ids = torch.empty((k, layer.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((k, layer.top_k), dtype=torch.float32, device="cuda")
    nw = torch.empty(4, dtype=torch.int32, device="cuda")
    if ws is None:
        ws = torch.empty(layer.workspace_size(k), dtype=torch.uint8, device="cuda")
    fill_ws(ws, ws_fill)
    B.moe_verify_block(layer, xd, flags, y, ids, w, nw, ws)
    torch.cuda.synchronize()
    return {"y": y.cpu().numpy(), "ids": ids.cpu().numpy().astype(np.int64), "w": w.cpu().numpy(),
            "n_woken": int(nw[0].item())}


def _valid_topk_within(l, ids, tie):
    sel = set(int(e) for e in ids)
    rest = [e for e in range(l.size) if e not in sel]
    if rest and max(l[rest]) > min(l[list(sel)]) + tie:
        return False
    return all(l[ids[j]] >= l[ids[j + 1]] - tie for j in range(len(ids) - 1))


def check_routing(g, x, wl, flags=0):
    """Every token's ids and weights against the oracle's router; the woken count against the
    union of the GPU's own ids and the oracle's."""
    K = wl.shape.top_k
    L = GenLayer(wl, 0)
    xh = oracle.rms_norm(x.astype(np.float64), wl.rms_eps) if flags & PRE else x.astype(np.float64)
    logits = oracle.router_logits(xh, L.router())
    n_tie = 0
    for t in range(x.shape[0]):
        ref = oracle.select_topk(logits[t], K)
        if not np.array_equal(g["ids"][t], ref):
            assert _valid_topk_within(logits[t], g["ids"][t], TIE), (t, g["ids"][t], ref)
            n_tie += 1
        np.testing.assert_allclose(g["w"][t], oracle.routing_weights(logits[t], g["ids"][t]), rtol=0, atol=1e-6)
    assert g["n_woken"] == len(set(g["ids"].ravel().tolist()))
    if n_tie == 0:
        assert g["n_woken"] == oracle.woken_experts(g["ids"])[0].size
    return n_tie


def check_outputs(g, x, wl, tokens, flags=0, compare_delta=False):
    """Outputs of the sampled tokens against the oracle run on those tokens with the GPU's ids
    (already checked against the oracle's own selection)."""
    rows = np.asarray(tokens)
    kw = dict(pre_norm=bool(flags & PRE), residual=bool(flags & RES), rms_eps=wl.rms_eps)
    ref = oracle.moe_block(x[rows], GenLayer(wl, 0), wl.shape.top_k, forced_ids=g["ids"][rows], **kw)
    gy, ry = g["y"][rows].astype(np.float64), ref["y"]
    if compare_delta:
        gy, ry = gy - x[rows], ry - x[rows]
    rms = float(np.sqrt(np.mean(ry ** 2)))
    err = float(np.abs(gy - ry).max())
    assert err <= BF16_TOL * rms, f"max|dy| {err:.3e} > {BF16_TOL} x RMS {rms:.3e}"
    return err / rms


def test_gather_tiny_layer_all_tokens(B):
    """The tiny layer (H 256, 16 experts, top-2, I 128, no shared expert) through the gathered
    path at k = 4 (forced) and at k = 40 (every expert takes several column tiles' worth)."""
    wl = gen.WORKLOADS["tiny"]
    layer = dev_layer(wl)
    for k, flags in ((4, GATHER), (40, 0)):
        x = gen.hidden_states(wl, rep=200 + k, k=k)
        g = run(B, layer, x, flags)
        check_routing(g, x, wl)
        r = check_outputs(g, x, wl, np.arange(k))
        print(f"tiny gathered k={k}: U={g['n_woken']} err/rms={r:.2e}")


def test_gather_matches_single_block_path(B):
    """k = 16 through both paths: the same expert ids and weights, outputs both within the bar."""
    wl = gen.WORKLOADS["verify"]
    layer = dev_layer(wl)
    x = gen.hidden_states(wl, rep=21)
    a = run(B, layer, x, 0)
    b = run(B, layer, x, GATHER)
    assert np.array_equal(a["ids"], b["ids"]) and a["n_woken"] == b["n_woken"]
    np.testing.assert_allclose(a["w"], b["w"], rtol=0, atol=1e-6)
    check_routing(b, x, wl)
    r = check_outputs(b, x, wl, np.arange(16))
    rms = float(np.sqrt(np.mean(a["y"].astype(np.float64) ** 2)))
    assert float(np.abs(a["y"] - b["y"]).max()) <= 2 * BF16_TOL * rms
    print(f"gathered k=16: err/rms={r:.2e}")


@pytest.mark.parametrize("k", [17, 100, 512])
def test_gather_batched_parity(B, k):
    """The benchmark layer over k stacked tokens (32 sequences x 16 at k = 512): routing of
    every token, outputs on sampled tokens (first, last, and spread over the call)."""
    wl = gen.WORKLOADS["batched"]
    layer = dev_layer(wl)
    x = gen.hidden_states(wl, rep=k, k=k)
    g = run(B, layer, x)
    n_tie = check_routing(g, x, wl)
    rng = np.random.default_rng(k)
    sample = sorted(set([0, k - 1] + rng.choice(k, size=min(k, 10), replace=False).tolist()))
    r = check_outputs(g, x, wl, sample)
    print(f"batched k={k}: U={g['n_woken']} near-ties={n_tie} err/rms={r:.2e}")
    if k == 512:
        assert g["n_woken"] >= 250  # nearly every expert wakes


def test_gather_max_tokens_and_rows_independent_of_the_call(B):
    """k = 1024 (the largest call): each row equals the same token run in a smaller call and in
    a permuted call, bit for bit (a column's products never mix with other columns, and every
    reduction has a fixed order); sampled rows against the oracle."""
    wl = gen.WORKLOADS["batched"]
    layer = dev_layer(wl)
    x = gen.hidden_states(wl, rep=1024, k=1024)
    full = run(B, layer, x)
    check_routing(full, x, wl)
    # 40 rows spread over the call: tokens land in every position of their experts' 32-token
    # column groups (an expert with n tokens takes ceil(n / 32) groups)
    rows = sorted(set([0, 31, 32, 511, 1023] + np.random.default_rng(40).choice(1024, 40, replace=False).tolist()))
    r = check_outputs(full, x, wl, rows)
    print(f"gathered k=1024: {len(rows)} rows against the oracle, err/rms={r:.2e}")
    sub = np.array([3, 100, 511, 512, 700, 1023] + list(range(200, 231)))
    part = run(B, layer, x[sub])
    for key in ("y", "ids", "w"):
        assert np.array_equal(part[key], full[key][sub]), key
    p = np.random.default_rng(5).permutation(1024)[:300]
    perm = run(B, layer, x[p])
    for key in ("y", "ids", "w"):
        assert np.array_equal(perm[key], full[key][p]), key


def test_gather_identical_tokens_many_column_groups(B):
    """512 identical tokens: the K experts each take all 512 (16 column groups of 32 per weight
    pass), every other expert stays asleep, and every row is the same."""
    wl = gen.WORKLOADS["batched"]
    layer = dev_layer(wl)
    x = np.repeat(gen.hidden_states(wl, rep=77, k=1), 512, axis=0)
    g = run(B, layer, x)
    assert g["n_woken"] == wl.shape.top_k
    assert np.all(g["ids"] == g["ids"][0]) and np.all(g["y"] == g["y"][0])
    check_routing(g, x, wl)
    r = check_outputs(g, x, wl, [0, 255, 511])
    print(f"identical tokens: err/rms={r:.2e}")


@pytest.mark.parametrize("shape", [
    gen.LayerShape(hidden=128, n_experts=4, top_k=4, inter=128, shared_inter=128),     # K = E, H of one window
    gen.LayerShape(hidden=384, n_experts=512, top_k=16, inter=256, shared_inter=256),  # largest E and K, odd windows
    gen.LayerShape(hidden=1024, n_experts=64, top_k=6, inter=1024, shared_inter=0),    # I = 1024, no shared expert
    gen.LayerShape(hidden=256, n_experts=30, top_k=5, inter=128, shared_inter=128),    # E not a multiple of 4
    gen.LayerShape(hidden=256, n_experts=302, top_k=8, inter=128, shared_inter=0),     # E > 256, not a multiple of 4
])
def test_gather_edge_shapes(B, shape):
    wl = gen.Workload("edge", shape, k=16, seed=4321)
    from speculative_decoding_moe_amd.workloads import device
    layer = device.make_layer(wl, 0, "cuda")
    for k in (1, 33):
        x = gen.hidden_states(wl, rep=k, k=k)
        g = run(B, layer, x, GATHER)
        check_routing(g, x, wl)
        check_outputs(g, x, wl, np.arange(k) if k < 40 else [0, k - 1])


def test_gather_flags_prenorm_residual(B):
    wl = gen.WORKLOADS["batched"]
    layer = dev_layer(wl)
    x = gen.hidden_states(wl, rep=3, k=64) * 3.0
    g = run(B, layer, x, PRE | RES)
    check_routing(g, x, wl, flags=PRE)
    r = check_outputs(g, x, wl, [0, 17, 63], flags=PRE | RES, compare_delta=True)
    print(f"gathered pre-norm + residual: delta err/rms={r:.2e}")


def test_gather_determinism_and_stale_workspace(B):
    wl = gen.WORKLOADS["batched"]
    layer = dev_layer(wl)
    x = gen.hidden_states(wl, rep=9, k=300)
    base = run(B, layer, x, ws_fill=0)
    ws = torch.empty(layer.workspace_size(1024), dtype=torch.uint8, device="cuda")
    for fill in (0xFF, 0x80, 0x7F, None):
        g = run(B, layer, x, ws_fill=fill, ws=ws)
        for key in ("y", "ids", "w"):
            assert np.array_equal(g[key], base[key]), (fill, key)
        assert g["n_woken"] == base["n_woken"]
    # the workspace left by a larger call, then a smaller one
    run(B, layer, gen.hidden_states(wl, rep=10, k=1024), ws=ws)
    g = run(B, layer, x, ws=ws)
    assert np.array_equal(g["y"], base["y"])


@pytest.mark.parametrize("name,flags", [("batched", GATHER), ("stack40_mxfp4", GATHER | PRE | RES)])
@pytest.mark.parametrize("k", [1, 5])
def test_gather_stale_signed_zero_and_nan_workspace(B, name, flags, k):
    """Gathered calls with partial column groups: a workspace of -0 or NaN words (bf16 and fp32
    patterns) gives the same bits as a zeroed one."""
    wl = gen.WORKLOADS[name]
    layer = dev_layer(wl)
    x = gen.hidden_states(wl, rep=60 + k, k=k)
    base = run(B, layer, x, flags, ws_fill=0)
    ws = torch.empty(layer.workspace_size(64), dtype=torch.uint8, device="cuda")
    for fill in ("neg_zero_bf16", "neg_zero_f32", "nan_bf16", "nan_f32", "ff"):
        g = run(B, layer, x, flags, ws_fill=WS_FILLS[fill], ws=ws)
        for key in ("y", "ids", "w"):
            assert np.array_equal(g[key], base[key]), (fill, key)
        assert np.all(np.isfinite(g["y"]))
    check_routing(base, x, wl, flags=flags & PRE)


# ---- greedy acceptance for many sequences (accept_prefix_batch) -------------------------------
def run_accept_batch(B, logits, drafts, n_draft=None):
    S, NT, V = logits.shape
    print(f"[accept_batch] n_seq={S} n_target={NT} vocab={V}", flush=True)
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    dr = torch.from_numpy(np.ascontiguousarray(drafts, dtype=np.int32)).cuda() if drafts is not None else None
    nd = torch.from_numpy(np.asarray(n_draft, dtype=np.int32)).cuda() if n_draft is not None else None
    tg = torch.full((S, NT), -1, dtype=torch.int32, device="cuda")
    ac = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.accept_prefix_batch_workspace_size(S, NT, V), dtype=torch.uint8, device="cuda")
    B.accept_prefix_batch(lg, dr, tg, ac, ws, n_draft=nd)
    torch.cuda.synchronize()
    return tg.cpu().numpy().astype(np.int64), ac.cpu().numpy().astype(np.int64)


def test_accept_prefix_batch_32_sequences(B):
    """32 sequences x 17 rows x 151936: geometric drafts per sequence, each sequence with its own
    draft count; the drafts past a sequence's count are its targets (a kernel that read them
    would accept too much)."""
    wl = gen.WORKLOADS["verify"]
    S = 32
    logits = np.stack([gen.target_logits(wl, rep=500 + s)[0] for s in range(S)])
    t_ref = np.stack([oracle.argmax_first(logits[s]) for s in range(S)])
    rng = np.random.default_rng(12)
    n_d = rng.integers(0, 17, size=S)
    drafts = t_ref[:, :16].copy()
    for s in range(S):
        planted = gen.target_logits(wl, rep=500 + s)[1]
        d, _ = gen.draft_ids(wl, planted, rep=600 + s)
        drafts[s, :n_d[s]] = d[:n_d[s]]
    tg, ac = run_accept_batch(B, logits, drafts, n_d)
    assert np.array_equal(tg, t_ref)
    for s in range(S):
        assert ac[s] == oracle.accept_length(drafts[s, :n_d[s]], t_ref[s]), s
    # every sequence with the full count, and the same as accept_prefix one sequence at a time
    tg2, ac2 = run_accept_batch(B, logits, drafts)
    assert np.array_equal(tg2, t_ref)
    for s in (0, 7, 31):
        lg = torch.from_numpy(logits[s]).cuda()
        dr = torch.from_numpy(drafts[s].astype(np.int32)).cuda()
        one_t = torch.empty(17, dtype=torch.int32, device="cuda")
        one_a = torch.empty(4, dtype=torch.int32, device="cuda")
        ws = torch.empty(B.accept_prefix_workspace_size(17, wl.vocab), dtype=torch.uint8, device="cuda")
        B.accept_prefix(lg, dr, one_t, one_a, ws)
        torch.cuda.synchronize()
        assert np.array_equal(one_t.cpu().numpy(), t_ref[s]) and int(one_a[0].item()) == ac2[s]
        assert ac2[s] == oracle.accept_length(drafts[s], t_ref[s])


def test_accept_prefix_batch_counts_clamped_and_small_vocab(B):
    """Device draft counts outside [0, n_draft_max] are clamped; 1024 sequences over a tiny
    vocabulary (17408 rows) with exact ties; no drafts at all."""
    rng = np.random.default_rng(13)
    S, NT, V = 1024, 17, 7
    logits = rng.integers(0, 3, size=(S, NT, V)).astype(np.float32)  # many exact ties
    t_ref = np.stack([oracle.argmax_first(logits[s]) for s in range(S)])
    drafts = t_ref[:, :16].copy()
    drafts[:, 9] = (drafts[:, 9] + 1) % V
    n_d = rng.integers(-5, 30, size=S)
    tg, ac = run_accept_batch(B, logits, drafts, n_d)
    assert np.array_equal(tg, t_ref)
    for s in range(S):
        nd = min(max(int(n_d[s]), 0), 16)
        assert ac[s] == oracle.accept_length(drafts[s, :nd], t_ref[s]), (s, n_d[s])
    tg, ac = run_accept_batch(B, logits, None)
    assert np.array_equal(tg, t_ref) and np.all(ac == 0)


# ---- mxfp4 layers on the gathered path -----------------------------------------------------
MX_TOL = 3e-2


def check_outputs_tol(g, x, wl, tokens, flags, tol, compare_delta):
    rows = np.asarray(tokens)
    kw = dict(pre_norm=bool(flags & PRE), residual=bool(flags & RES), rms_eps=wl.rms_eps)
    ref = oracle.moe_block(x[rows], GenLayer(wl, 0), wl.shape.top_k, forced_ids=g["ids"][rows], **kw)
    gy, ry = g["y"][rows].astype(np.float64), ref["y"]
    if compare_delta:
        gy, ry = gy - x[rows], ry - x[rows]
    rms = float(np.sqrt(np.mean(ry ** 2)))
    err = float(np.abs(gy - ry).max())
    assert err <= tol * rms, f"max|dy| {err:.3e} > {tol} x RMS {rms:.3e}"
    return err / rms


@pytest.mark.parametrize("k", [17, 100, 512])
def test_gather_mxfp4_layer(B, k):
    """The 40-layer stack's mxfp4 layer (pre-norm, residual, bf16 shared expert) over k tokens:
    routing of every token, the MoE delta of sampled tokens within 3e-2 x RMS."""
    wl = gen.WORKLOADS["stack40_mxfp4"]
    layer = dev_layer(wl)
    x = gen.hidden_states(wl, rep=700 + k, k=k)
    g = run(B, layer, x, PRE | RES)
    check_routing(g, x, wl, flags=PRE)
    rng = np.random.default_rng(k + 1)
    sample = sorted(set([0, k - 1] + rng.choice(k, size=min(k, 8), replace=False).tolist()))
    r = check_outputs_tol(g, x, wl, sample, PRE | RES, MX_TOL, True)
    print(f"mxfp4 gathered k={k}: U={g['n_woken']} delta err/rms={r:.2e}")


def test_gather_mxfp4_matches_single_block_and_rows_independent(B):
    """k = 16 through both mxfp4 paths (the same ids; both deltas within the bar), and each row
    of a 300-token call bit-identical to the same tokens in a 37-token call."""
    wl = gen.WORKLOADS["stack40_mxfp4"]
    layer = dev_layer(wl)
    x = gen.hidden_states(wl, rep=31)
    a = run(B, layer, x, PRE | RES)
    b = run(B, layer, x, PRE | RES | GATHER)
    assert np.array_equal(a["ids"], b["ids"]) and a["n_woken"] == b["n_woken"]
    check_outputs_tol(b, x, wl, np.arange(16), PRE | RES, MX_TOL, True)
    xb = gen.hidden_states(wl, rep=32, k=300)
    full = run(B, layer, xb, PRE | RES)
    sub = np.array([0, 5, 150, 299] + list(range(40, 73)))
    part = run(B, layer, xb[sub], PRE | RES)
    for key in ("y", "ids", "w"):
        assert np.array_equal(part[key], full[key][sub]), key


@pytest.mark.parametrize("shape", [
    gen.LayerShape(hidden=512, n_experts=32, top_k=4, inter=256, shared_inter=256, wdtype="mxfp4"),
    gen.LayerShape(hidden=768, n_experts=64, top_k=6, inter=128, shared_inter=0, wdtype="mxfp4"),  # 3 windows per K half, one-window down
    gen.LayerShape(hidden=256, n_experts=512, top_k=16, inter=1024, shared_inter=1024, wdtype="mxfp4"),
])
def test_gather_mxfp4_edge_shapes(B, shape):
    wl = gen.Workload("edge", shape, k=16, seed=4321)
    from speculative_decoding_moe_amd.workloads import device
    layer = device.make_layer(wl, 0, "cuda")
    for k in (1, 33):
        x = gen.hidden_states(wl, rep=k, k=k)
        g = run(B, layer, x, GATHER)
        check_routing(g, x, wl)
        check_outputs_tol(g, x, wl, np.arange(k) if k < 40 else [0, k - 1], 0, MX_TOL, False)


@pytest.mark.parametrize("shape", [
    gen.LayerShape(hidden=512, n_experts=32, top_k=4, inter=384, shared_inter=384),   # I / 128 = 3 windows
    gen.LayerShape(hidden=512, n_experts=32, top_k=4, inter=512, shared_inter=256),   # shared expert smaller than I
    gen.LayerShape(hidden=384, n_experts=40, top_k=6, inter=640, shared_inter=128),   # 5 windows, 3 windows of H
    gen.LayerShape(hidden=256, n_experts=16, top_k=2, inter=256, shared_inter=768),   # shared expert larger than I
    gen.LayerShape(hidden=512, n_experts=32, top_k=4, inter=384, shared_inter=256, wdtype="mxfp4"),
    gen.LayerShape(hidden=256, n_experts=16, top_k=4, inter=768, shared_inter=1024, wdtype="mxfp4"),
])
def test_general_shapes(B, shape):
    """Layers outside the single-block shapes (I / 128 not dividing eight, or a shared expert of its
    own size) take the gathered path at every k: blocks of 1, 16 (without MOE_GATHER) and 70 tokens
    against the oracle, and the 16-token call equal, bit for bit, to the same call with MOE_GATHER."""
    from speculative_decoding_moe_amd.workloads import device
    wl = gen.Workload("general", shape, k=16, seed=5150)
    layer = device.make_layer(wl, 0, "cuda")
    mx = shape.wdtype == "mxfp4"
    for k, flags in ((1, 0), (16, 0), (70, PRE | RES)):
        x = gen.hidden_states(wl, rep=k, k=k)
        g = run(B, layer, x, flags)
        check_routing(g, x, wl, flags=flags & PRE)
        rows = np.arange(k) if k <= 16 else [0, 33, k - 1]
        if mx:
            check_outputs_tol(g, x, wl, rows, flags, MX_TOL, bool(flags & RES))
        else:
            check_outputs(g, x, wl, rows, flags, compare_delta=bool(flags & RES))
        if k == 16:
            h = run(B, layer, x, flags | GATHER)
            for key in ("y", "ids", "w"):
                assert np.array_equal(g[key], h[key]), key


def test_gather_largest_lists(B):
    """1024 tokens x top-16 of 512 experts (16384 routed pairs, every pair slot of the permutation
    kernel's threads in use), with and without the shared expert: routing of every token, sampled
    outputs against the oracle."""
    from speculative_decoding_moe_amd.workloads import device
    for Is in (256, 0):
        shape = gen.LayerShape(hidden=256, n_experts=512, top_k=16, inter=256, shared_inter=Is)
        wl = gen.Workload("edge", shape, k=16, seed=4322)
        layer = device.make_layer(wl, 0, "cuda")
        x = gen.hidden_states(wl, rep=9, k=1024)
        g = run(B, layer, x)
        check_routing(g, x, wl)
        check_outputs(g, x, wl, [0, 1, 511, 1022, 1023])


class _PeriodicRouterLayer(GenLayer):
    """A generated layer whose router rows repeat with period P, so logits tie exactly."""

    def __init__(self, wl, period):
        super().__init__(wl, 0)
        self.period = period

    def router(self):
        r = gen.router_weight(self.wl, 0)
        return np.ascontiguousarray(r[np.arange(r.shape[0]) % self.period])


@pytest.mark.parametrize("shape,period,k", [
    (gen.LayerShape(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512), 5, 300),
    (gen.LayerShape(hidden=256, n_experts=200, top_k=6, inter=256, shared_inter=0), 3, 77),   # E not a multiple of 16
    # many token groups with a last 64-expert group of the router that runs past E
    (gen.LayerShape(hidden=256, n_experts=200, top_k=6, inter=256, shared_inter=0), 3, 600),
    (gen.LayerShape(hidden=256, n_experts=200, top_k=6, inter=256, shared_inter=0), 3, 1024),
    (gen.LayerShape(hidden=256, n_experts=512, top_k=16, inter=256, shared_inter=256), 7, 40),
])
def test_gather_exact_router_ties_pick_lower_expert_ids(B, shape, period, k):
    """Identical router rows give bit-identical logits, so most picks are exact ties: the gathered
    path's top-K must take equal logits in ascending expert order, exactly as the oracle does."""
    from speculative_decoding_moe_amd.workloads import device
    wl = gen.Workload("ties", shape, k=16, seed=99)
    L = _PeriodicRouterLayer(wl, period)
    t = device.layer_tensors(wl, 0, "cuda")
    t["router_w"] = torch.from_numpy(L.router()).cuda()
    layer = device.make_layer(wl, 0, "cuda", tensors=t)
    x = gen.hidden_states(wl, rep=60, k=k)
    g = run(B, layer, x)
    xh = x.astype(np.float64)
    logits = oracle.router_logits(xh, L.router())
    for i in range(k):
        assert np.array_equal(g["ids"][i], oracle.select_topk(logits[i], shape.top_k)), i
        np.testing.assert_allclose(g["w"][i], oracle.routing_weights(logits[i], g["ids"][i]), rtol=0, atol=1e-6)
    assert g["n_woken"] == oracle.woken_experts(g["ids"])[0].size
    rows = [0, k // 2, k - 1]
    ref = oracle.moe_block(x[rows], L, shape.top_k)
    rms = float(np.sqrt(np.mean(ref["y"] ** 2)))
    assert float(np.abs(g["y"][rows] - ref["y"]).max()) <= BF16_TOL * rms
