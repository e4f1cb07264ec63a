"""GPU parity of the lossless acceptance at temperature (accept_sample) and of the acceptance
statistics (accept_histogram), through the C ABI, against the CPU oracle on the same seeded
inputs. Run on an MI355X: ``pytest -m gpu``.

Bars: the accepted length and the token equal the oracle's, except where a decision lies within
fp32 rounding of its boundary. The kernel computes p = 2^(z - max) / sum in fp32 with
z = logit log2(e) / T (sums in a fixed tree order over at most 8192-term chunks, then over the
chunks), so p and q carry a relative error far below MARGIN = 1e-4: a keep/reject decision may
differ only where |u q - p| <= MARGIN max(p, u q), and a sampled index only where the oracle's
running weight at the index boundary is within MARGIN of u times the total. Histograms: exact.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

MARGIN = 1e-4


@pytest.fixture(scope="session")
def B():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    from speculative_decoding_moe_amd import binding
    return binding


def run_sample(B, tl, dl, draft, T, ua, us, ws_fill=None):
    dev = "cuda"
    t = torch.from_numpy(np.ascontiguousarray(tl, dtype=np.float32)).to(dev)
    nd = len(draft)
    d = torch.from_numpy(np.ascontiguousarray(dl, dtype=np.float32)).to(dev) if nd else None
    di = torch.from_numpy(np.asarray(draft, dtype=np.int32)).to(dev) if nd else None
    uad = torch.from_numpy(np.asarray(ua, dtype=np.float32)).to(dev) if nd else None
    usd = torch.from_numpy(np.asarray(us, dtype=np.float32)).to(dev)
    ac = torch.full((4,), -7, dtype=torch.int32, device=dev)
    tk = torch.full((4,), -7, dtype=torch.int32, device=dev)
    ws = torch.empty(B.accept_sample_workspace_size(tl.shape[0], nd, tl.shape[1]), dtype=torch.uint8, device=dev)
    if ws_fill is not None:
        ws.fill_(ws_fill)
    B.accept_sample(t, d, di, T, uad, usd, ac, tk, ws)
    torch.cuda.synchronize()
    return int(ac[0].item()), int(tk[0].item())


def check_sample(tl, dl, draft, T, ua, us, got):
    """got = (a, token) equals the oracle's, or differs only at a boundary within MARGIN."""
    ua32 = np.asarray(ua, dtype=np.float32).astype(np.float64)
    us32 = np.asarray(us, dtype=np.float32).astype(np.float64)
    tl64 = np.asarray(tl, dtype=np.float32).astype(np.float64)
    dl64 = np.asarray(dl, dtype=np.float32).astype(np.float64) if len(draft) else dl
    ref = oracle.speculative_accept(tl64, dl64, draft, T, ua32, us32)
    if got == ref:
        return ref
    a_gpu, tok = got
    a_ref = ref[0]
    V = tl.shape[1]
    # the first position where the two decided differently must be a boundary case
    for i in range(min(a_gpu, a_ref) + 1):
        if i >= len(draft):
            break
        p = oracle.softmax_temp(tl64[i], T)
        q = oracle.softmax_temp(dl64[i], T)
        d = int(draft[i])
        if not 0 <= d < V:
            assert a_gpu == a_ref == i
            break
        keep_ref = ua32[i] * q[d] < p[d]
        keep_gpu = i < a_gpu
        if keep_ref != keep_gpu:
            gap = abs(ua32[i] * q[d] - p[d])
            assert gap <= MARGIN * max(p[d], ua32[i] * q[d]), f"position {i}: decision differs, gap {gap:.3e}"
            return ref  # the token then comes from a different row: nothing more to compare
    assert a_gpu == a_ref
    a = a_ref
    if a < len(draft):
        p = oracle.softmax_temp(tl64[a], T)
        w = np.maximum(p - oracle.softmax_temp(dl64[a], T), 0.0)
        if w.sum() <= 0:
            w = p
    elif a < tl.shape[0]:
        w = oracle.softmax_temp(tl64[a], T)
    else:
        assert tok == -1
        return ref
    assert 0 <= tok < V and w[tok] > 0, f"token {tok} has no weight"
    c = np.cumsum(w)
    target = us32[a] * c[-1]
    lo = c[tok - 1] if tok > 0 else 0.0
    assert lo <= target + MARGIN * c[-1] and c[tok] >= target - MARGIN * c[-1], (
        f"token {tok} vs oracle {ref[1]}: running weight [{lo:.6e}, {c[tok]:.6e}] misses {target:.6e}")
    return ref


def _case(seed, nt, nd, V, T, noise=0.5, scale=2.0):
    rng = np.random.default_rng(seed)
    tl = (rng.standard_normal((nt, V)) * scale).astype(np.float32)
    dl = (tl[:nd] + rng.standard_normal((nd, V)) * noise).astype(np.float32)
    draft = np.array([oracle.sample_inverse_cdf(oracle.softmax_temp(dl[i].astype(np.float64), T), rng.random())
                      for i in range(nd)], dtype=np.int32)
    ua = rng.random(nd).astype(np.float32)
    us = rng.random(nt).astype(np.float32)
    return tl, dl, draft, ua, us


@pytest.mark.parametrize("seed,nt,nd,V,T", [
    (1, 4, 4, 1000, 1.0),        # one ragged chunk, no bonus row
    (2, 17, 16, 151936, 1.0),    # the benchmark's shape: 19 chunks
    (3, 17, 16, 151936, 0.6),
    (4, 9, 8, 20001, 1.7),       # ragged vocabulary (not a multiple of 4)
    (5, 1, 0, 70000, 1.0),       # no drafts: the token is the target's own sample
    (6, 64, 64, 8192, 0.9),      # largest block, one exact chunk
])
def test_accept_sample_parity(B, seed, nt, nd, V, T):
    for rep in range(4):
        tl, dl, draft, ua, us = _case(seed * 100 + rep, nt, nd, V, T)
        got = run_sample(B, tl, dl, draft, T, ua, us)
        check_sample(tl, dl, draft, T, ua, us, got)


def test_accept_sample_special_cases(B):
    rng = np.random.default_rng(7)
    V, n, T = 5000, 6, 1.0
    tl = rng.standard_normal((n + 1, V)).astype(np.float32)
    draft = rng.integers(0, V, n).astype(np.int32)
    # a drafter equal to the target keeps every draft; the bonus token is the target's sample
    a, tok = run_sample(B, tl, tl[:n], draft, T, np.full(n, 0.999, np.float32), np.full(n + 1, 0.3, np.float32))
    assert a == n
    check_sample(tl, tl[:n], draft, T, np.full(n, 0.999, np.float32), np.full(n + 1, 0.3, np.float32), (a, tok))
    # no bonus row: no token
    assert run_sample(B, tl[:n], tl[:n], draft, T, np.zeros(n, np.float32), np.zeros(n, np.float32)) == (n, -1)
    # an id outside the vocabulary is rejected at its position
    bad = draft.copy()
    bad[3] = V + 2
    a, tok = run_sample(B, tl, tl[:n], bad, T, np.zeros(n, np.float32), np.full(n + 1, 0.5, np.float32))
    assert a == 3
    check_sample(tl, tl[:n], bad, T, np.zeros(n, np.float32), np.full(n + 1, 0.5, np.float32), (a, tok))
    # entries of probability zero (-inf logits) are never drawn
    tz = tl.copy()
    tz[n, : V // 2] = -np.inf
    for u in (0.0, 0.37, 0.999):
        a, tok = run_sample(B, tz, tz[:n], draft, T, np.zeros(n, np.float32), np.full(n + 1, u, np.float32))
        assert a == n and tok >= V // 2
        check_sample(tz, tz[:n], draft, T, np.zeros(n, np.float32), np.full(n + 1, u, np.float32), (a, tok))


def test_accept_sample_first_token_distribution(B):
    """Losslessness end to end: over many cycles with d_0 drawn from q_0, the first committed
    token's frequencies match the target's p_0 (chi-square, generous threshold)."""
    rng = np.random.default_rng(8)
    V, T, N = 6, 0.9, 4000
    tl = (rng.standard_normal((2, V)) * 1.5).astype(np.float32)
    dl = (tl[:1] + rng.standard_normal((1, V))).astype(np.float32)
    q0 = oracle.softmax_temp(dl[0].astype(np.float64), T)
    p0 = oracle.softmax_temp(tl[0].astype(np.float64), T)
    counts = np.zeros(V)
    for _ in range(N):
        d = np.array([oracle.sample_inverse_cdf(q0, rng.random())], dtype=np.int32)
        a, tok = run_sample(B, tl, dl, d, T, rng.random(1).astype(np.float32), rng.random(2).astype(np.float32))
        counts[int(d[0]) if a == 1 else tok] += 1
    chi2 = float(np.sum((counts - N * p0) ** 2 / (N * p0)))
    assert chi2 < 30.0, (chi2, counts, N * p0)   # 5 degrees of freedom: p ~ 1e-5 at 30


def test_accept_sample_stale_workspace(B):
    tl, dl, draft, ua, us = _case(9, 17, 16, 151936, 1.0)
    base = run_sample(B, tl, dl, draft, 1.0, ua, us, ws_fill=0)
    for fill in (0xFF, 0x7F, None):
        assert run_sample(B, tl, dl, draft, 1.0, ua, us, ws_fill=fill) == base


def test_accept_histogram_matches_oracle(B):
    rng = np.random.default_rng(10)
    for n_draft, n in ((16, 7000), (0, 5), (64, 100000)):
        a = rng.integers(-1, n_draft + 2, size=n).astype(np.int32)
        ad = torch.from_numpy(a).cuda()
        hist = torch.full((n_draft + 1,), -1, dtype=torch.int64, device="cuda")
        surv = torch.full((max(n_draft, 1),), -1, dtype=torch.int64, device="cuda")
        B.accept_histogram(ad, n_draft, hist, surv if n_draft else None)
        torch.cuda.synchronize()
        ref_h, ref_s = oracle.accept_histogram(a[(a >= 0) & (a <= n_draft)], n_draft)
        assert np.array_equal(hist.cpu().numpy(), ref_h)
        if n_draft:
            assert np.array_equal(surv.cpu().numpy(), ref_s)


@pytest.mark.parametrize("V", [1, 2, 5])
def test_accept_sample_tiny_vocabularies(B, V):
    """Vocabularies smaller than one float4 and than one chunk's first wave: with V = 1 every
    draft of id 0 is kept and the token is 0."""
    rng = np.random.default_rng(11 + V)
    n = 3
    tl = rng.standard_normal((n + 1, V)).astype(np.float32)
    dl = (tl[:n] + rng.standard_normal((n, V)) * 0.3).astype(np.float32)
    for rep in range(6):
        draft = rng.integers(0, V, n).astype(np.int32)
        ua = rng.random(n).astype(np.float32)
        us = rng.random(n + 1).astype(np.float32)
        got = run_sample(B, tl, dl, draft, 1.0, ua, us)
        check_sample(tl, dl, draft, 1.0, ua, us, got)
        if V == 1:
            assert got == (n, 0)


def run_sample_batch(B, tls, dls, drafts, T, uas, uss, ws_fill=None):
    """accept_sample_batch over stacked sequences; returns [(a, token)] per sequence."""
    S, nt, V = tls.shape
    nd = drafts.shape[1] if drafts is not None else 0
    print(f"[accept_sample_batch] n_seq={S} n_target={nt} n_draft={nd} vocab={V}", flush=True)
    t = torch.from_numpy(np.ascontiguousarray(tls, dtype=np.float32)).cuda()
    d = torch.from_numpy(np.ascontiguousarray(dls, dtype=np.float32)).cuda() if nd else None
    di = torch.from_numpy(np.ascontiguousarray(drafts, dtype=np.int32)).cuda() if nd else None
    ua = torch.from_numpy(np.ascontiguousarray(uas, dtype=np.float32)).cuda() if nd else None
    us = torch.from_numpy(np.ascontiguousarray(uss, dtype=np.float32)).cuda()
    ac = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    tk = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.accept_sample_batch_workspace_size(S, nt, nd, V), dtype=torch.uint8, device="cuda")
    if ws_fill is not None:
        ws.fill_(ws_fill)
    B.accept_sample_batch(t, d, di, T, ua, us, ac, tk, ws)
    torch.cuda.synchronize()
    return list(zip(ac.cpu().numpy().tolist(), tk.cpu().numpy().tolist()))


@pytest.mark.parametrize("S,nt,nd,V,T", [
    (16, 17, 16, 151936, 0.8),   # 16 sequences of the benchmark's shape
    (5, 9, 8, 20001, 1.3),       # ragged vocabulary
    (7, 3, 0, 1001, 1.0),        # no drafts: each token is the target's own sample
])
def test_accept_sample_batch_equals_single_calls(B, S, nt, nd, V, T):
    """Every sequence of one batched call gives exactly what accept_sample gives for it alone, and
    sampled sequences agree with the oracle (within fp32 rounding of a decision boundary)."""
    cases = [_case(1000 + 10 * S + s, nt, nd, V, T) for s in range(S)]
    tls = np.stack([c[0] for c in cases])
    dls = np.stack([c[1] for c in cases]) if nd else None
    drafts = np.stack([c[2] for c in cases]) if nd else None
    uas = np.stack([c[3] for c in cases]) if nd else None
    uss = np.stack([c[4] for c in cases])
    got = run_sample_batch(B, tls, dls, drafts, T, uas, uss)
    for s in range(S):
        tl, dl, draft, ua, us = cases[s]
        one = run_sample(B, tl, dl, draft, T, ua, us)
        assert got[s] == one, (s, got[s], one)
    for s in (0, S - 1):
        tl, dl, draft, ua, us = cases[s]
        check_sample(tl, dl, draft, T, ua, us, got[s])
    # the workspace left by another call does not matter
    assert run_sample_batch(B, tls, dls, drafts, T, uas, uss, ws_fill=0xFF) == got
