"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each oracle function is checked against something other than itself: closed forms, brute force
on tiny inputs, special cases that reduce to a library routine, and values the pages print.
"""
import itertools
import math
import os
import struct

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import softmax as sp_softmax

import oracle
from helpers import ArrayLayer, GenLayer
from speculative_decoding_moe_amd.workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- weight decoding
def _bf16_closed_form(bits: int) -> float:
    s = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        return s * math.inf if m == 0 else math.nan
    if e == 0:
        return s * m / 128.0 * 2.0 ** -126
    return s * (1.0 + m / 128.0) * 2.0 ** (e - 127)


def test_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bf16(bits)
    want = np.array([_bf16_closed_form(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # sign of zero survives
    assert math.copysign(1.0, got[0x8000]) == -1.0


def _e2m1_closed_form(code: int) -> float:
    """E2M1: sign bit 3, two exponent bits (bias 1), one mantissa bit; exponent 0 is subnormal."""
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * m * 0.5
    return s * 2.0 ** (e - 1) * (1.0 + m / 2.0)


def test_decode_mxfp4_exhaustive_codes_and_scales():
    # one row of 32 elements per (scale); every code appears in both nibble positions
    codes = np.arange(16, dtype=np.uint8)
    row = np.concatenate([codes, codes[::-1]])  # 32 element codes
    packed = (row[0::2] | (row[1::2] << 4)).astype(np.uint8)[None, :]  # [1][16]
    for s in range(255):
        got = oracle.decode_mxfp4(packed, np.array([[s]], dtype=np.uint8))[0]
        want = np.array([_e2m1_closed_form(int(c)) for c in row]) * 2.0 ** (s - 127)
        assert np.array_equal(got, want), s
    got = oracle.decode_mxfp4(packed, np.array([[255]], dtype=np.uint8))
    assert np.isnan(got).all()


def test_decode_mxfp4_nibble_order_and_block_scales():
    # byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0); second block scaled by 2^3
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 16] = 0x9F  # element 32 = code 15 (-6), element 33 = code 9 (-0.5)
    scales = np.array([[127, 130]], dtype=np.uint8)
    d = oracle.decode_mxfp4(codes, scales)[0]
    assert d[0] == 0.5 and d[1] == 1.0
    assert d[32] == -6.0 * 8 and d[33] == -0.5 * 8
    assert np.count_nonzero(d) == 4


# ---------------------------------------------------------------- router
def test_rms_norm_matches_library_and_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    got = oracle.rms_norm(x, 1e-6)
    want = F.rms_norm(torch.from_numpy(x), (64,), eps=1e-6).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=0)
    c = 3.0
    row = np.full((1, 8), c)
    assert oracle.rms_norm(row, 1e-6)[0, 0] == pytest.approx(c / math.sqrt(c * c + 1e-6), rel=1e-15)


def test_router_logits_brute_force():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 7))
    w = rng.standard_normal((5, 7)).astype(np.float32)
    got = oracle.router_logits(x, w)
    for t in range(3):
        for e in range(5):
            want = math.fsum(float(x[t, h]) * float(w[e, h]) for h in range(7))
            assert got[t, e] == pytest.approx(want, rel=1e-14, abs=1e-15)
    onehot = np.zeros((1, 7))
    onehot[0, 4] = 1.0
    assert np.array_equal(oracle.router_logits(onehot, w)[0], w[:, 4].astype(np.float64))


def _topk_brute(row, k):
    """The unique k-subset whose every member beats every non-member under (-logit, index)."""
    n = len(row)
    beats = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)  # noqa: E731
    winners = [s for s in itertools.combinations(range(n), k)
               if all(beats(a, b) for a in s for b in range(n) if b not in s)]
    assert len(winners) == 1
    s = list(winners[0])
    # descending order with the same tie rule
    return sorted(s, key=lambda a: (-row[a], a))


@pytest.mark.parametrize("seed", range(6))
def test_select_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    row = rng.integers(-3, 4, size=8).astype(np.float64)  # many exact ties
    for k in range(1, 9):
        assert list(oracle.select_topk(row, k)) == _topk_brute(row, k)


def test_select_topk_all_selected_and_order():
    row = np.array([0.5, 2.0, -1.0, 2.0, 0.0])
    assert list(oracle.select_topk(row, 5)) == [1, 3, 0, 4, 2]


def test_routing_weights_closed_forms():
    row = np.array([1.0, 5.0, 5.0 - math.log(3.0), -2.0])
    ids = oracle.select_topk(row, 2)
    assert list(ids) == [1, 2]
    np.testing.assert_allclose(oracle.routing_weights(row, ids), [0.75, 0.25], rtol=1e-15)
    assert oracle.routing_weights(row, oracle.select_topk(row, 1))[0] == 1.0
    eq = np.zeros(6)
    np.testing.assert_allclose(oracle.routing_weights(eq, oracle.select_topk(eq, 3)), [1 / 3] * 3, rtol=1e-15)


def test_routing_weights_equal_full_softmax_restricted_and_renormalised():
    rng = np.random.default_rng(2)
    for _ in range(20):
        row = rng.standard_normal(32) * 3
        ids = oracle.select_topk(row, 8)
        full = sp_softmax(row)
        want = full[ids] / full[ids].sum()
        got = oracle.routing_weights(row, ids)
        np.testing.assert_allclose(got, want, rtol=1e-13)
        assert abs(got.sum() - 1.0) < 1e-15
        assert np.all(np.diff(got) <= 0)  # descending logits give descending weights


def test_topk_gap_brute_force():
    row = np.array([0.3, 1.2, -0.4, 1.1, 0.9])
    assert oracle.topk_gap(row, 2) == pytest.approx(1.1 - 0.9)
    assert oracle.topk_gap(row, 5) == math.inf


# ---------------------------------------------------------------- union / permutation
def test_woken_experts_against_sets_and_bijection():
    rng = np.random.default_rng(3)
    for k in (1, 3, 16):
        ids = np.stack([rng.choice(40, size=4, replace=False) for _ in range(k)])
        woken, counts, offsets, perm = oracle.woken_experts(ids)
        assert list(woken) == sorted(set(ids.ravel().tolist()))
        assert counts.sum() == k * 4 and offsets[-1] == k * 4
        assert sorted(map(tuple, perm.tolist())) == [(t, j) for t in range(k) for j in range(4)]
        for u, e in enumerate(woken):
            seg = perm[offsets[u]:offsets[u + 1]]
            assert all(ids[t, j] == e for t, j in seg)
            assert list(seg[:, 0]) == sorted(seg[:, 0])
        if k == 1:
            assert woken.size == 4


def test_expected_union_size_closed_form():
    """Random independent tokens: E[U] = E (1 - (1 - K/E)^k) (each expert missed by all k)."""
    rng = np.random.default_rng(4)
    E, K, k = 16, 2, 4
    sizes = []
    for _ in range(4000):
        logits = rng.standard_normal((k, E))
        ids = np.stack([oracle.select_topk(r, K) for r in logits])
        sizes.append(oracle.woken_experts(ids)[0].size)
    want = E * (1 - (1 - K / E) ** k)
    assert want == pytest.approx(6.62, abs=0.005)
    assert np.mean(sizes) == pytest.approx(want, abs=0.06)
    assert 256 * (1 - (1 - 8 / 256) ** 16) == pytest.approx(101.96, abs=0.01)


# ---------------------------------------------------------------- experts
def test_silu_closed_forms_and_library():
    z = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-13, atol=1e-13)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_expert_ffn_hand_example():
    wg = np.array([[1.0, 0.0]])
    wu = np.array([[0.0, 2.0]])
    wd = np.array([[1.0], [-1.0]])
    x = np.array([1.0, 3.0])
    a = 1.0 / (1.0 + math.exp(-1.0)) * 6.0
    np.testing.assert_allclose(oracle.expert_ffn(x, wg, wu, wd), [a, -a], rtol=1e-15)


def test_expert_ffn_matches_library():
    rng = np.random.default_rng(5)
    wg, wu = rng.standard_normal((6, 10)), rng.standard_normal((6, 10))
    wd = rng.standard_normal((10, 6))
    x = rng.standard_normal(10)
    t = lambda a: torch.from_numpy(a)  # noqa: E731
    want = F.linear(F.silu(F.linear(t(x), t(wg))) * F.linear(t(x), t(wu)), t(wd)).numpy()
    np.testing.assert_allclose(oracle.expert_ffn(x, wg, wu, wd), want, rtol=1e-12)


def _dense_textbook_moe(x, layer, K, E, residual=False, pre_norm=False, eps=1e-6):
    """All E experts on every token, combined through a gate matrix that is zero off the top-K
    (full softmax, keep the top-K, renormalise). torch float64."""
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    xh = F.rms_norm(xt, (xt.shape[1],), eps=eps) if pre_norm else xt
    logits = xh @ torch.from_numpy(layer.router().astype(np.float64)).T
    probs = torch.softmax(logits, dim=-1)
    top = torch.topk(logits, K, dim=-1).indices
    G = torch.zeros_like(probs).scatter(1, top, probs.gather(1, top))
    G = G / G.sum(dim=1, keepdim=True)
    y = torch.zeros_like(xt)
    for e in range(E):
        raw = layer.expert(e)
        wg, wu, wd = (torch.from_numpy(oracle.decode_tensor(raw, n)) for n in ("gate", "up", "down"))
        ye = F.linear(F.silu(F.linear(xh, wg)) * F.linear(xh, wu), wd)
        y += G[:, e:e + 1] * ye
    sh = layer.shared()
    if sh is not None:
        wg, wu, wd = (torch.from_numpy(oracle.decode_tensor(sh, n)) for n in ("gate", "up", "down"))
        y += F.linear(F.silu(F.linear(xh, wg)) * F.linear(xh, wu), wd)
    if residual:
        y += xt
    return y.numpy()


def _tiny_with_shared():
    s = gen.LayerShape(hidden=64, n_experts=12, top_k=3, inter=32, shared_inter=32)
    return gen.Workload("tiny_shared", s, k=5, seed=77)


def test_moe_block_equals_dense_textbook_tiny():
    wl = gen.WORKLOADS["tiny"]
    layer = GenLayer(wl)
    x = gen.hidden_states(wl)
    r = oracle.moe_block(x, layer, wl.shape.top_k)
    want = _dense_textbook_moe(x, layer, wl.shape.top_k, wl.shape.n_experts)
    np.testing.assert_allclose(r["y"], want, rtol=1e-11, atol=1e-14)
    # a block wakes at most k*K experts and at least K
    assert wl.shape.top_k <= r["n_woken"] <= wl.k * wl.shape.top_k


def test_moe_block_with_shared_prenorm_residual_equals_dense():
    wl = _tiny_with_shared()
    layer = GenLayer(wl)
    x = gen.hidden_states(wl) * 3.0
    r = oracle.moe_block(x, layer, 3, pre_norm=True, residual=True)
    want = _dense_textbook_moe(x, layer, 3, 12, residual=True, pre_norm=True)
    np.testing.assert_allclose(r["y"], want, rtol=1e-11, atol=1e-13)


def test_moe_block_mxfp4_equals_dense():
    s = gen.LayerShape(hidden=64, n_experts=8, top_k=2, inter=64, shared_inter=32, wdtype="mxfp4")
    wl = gen.Workload("tiny_mx", s, k=3, seed=78)
    layer = GenLayer(wl)
    x = gen.hidden_states(wl)
    r = oracle.moe_block(x, layer, 2)
    np.testing.assert_allclose(r["y"], _dense_textbook_moe(x, layer, 2, 8), rtol=1e-11, atol=1e-14)


def test_block_rows_equal_single_token_decode_and_permutation_invariance():
    """Lossless verification: block row t equals the layer applied to token t alone
    ("Speculating on a Strix Halo", 'Speculative decoding'); permuting tokens permutes rows."""
    wl = _tiny_with_shared()
    layer = GenLayer(wl)
    x = gen.hidden_states(wl)
    blk = oracle.moe_block(x, layer, 3)
    for t in range(x.shape[0]):
        one = oracle.moe_block(x[t:t + 1], layer, 3)
        assert np.array_equal(one["y"][0], blk["y"][t])
        assert np.array_equal(one["ids"][0], blk["ids"][t])
    p = np.array([3, 0, 4, 1, 2])
    pb = oracle.moe_block(x[p], layer, 3)
    assert np.array_equal(pb["y"], blk["y"][p])
    assert np.array_equal(pb["ids"], blk["ids"][p])
    assert pb["n_woken"] == blk["n_woken"]


def test_forced_ids_reproduce_natural_selection_and_weights_follow_logits():
    wl = _tiny_with_shared()
    layer = GenLayer(wl)
    x = gen.hidden_states(wl)
    nat = oracle.moe_block(x, layer, 3)
    forced = oracle.moe_block(x, layer, 3, forced_ids=nat["ids"])
    assert np.array_equal(forced["y"], nat["y"])
    swapped = nat["ids"].copy()
    swapped[0, [1, 2]] = swapped[0, [2, 1]]
    f2 = oracle.moe_block(x, layer, 3, forced_ids=swapped)
    np.testing.assert_allclose(f2["w"][0], nat["w"][0][[0, 2, 1]], rtol=1e-15)
    np.testing.assert_allclose(f2["y"], nat["y"], rtol=1e-12, atol=1e-15)


def test_hand_built_layer_closed_form():
    """Two experts, K = 1, one token; the router picks expert 1; y = W_d1 (silu(g) u) exactly."""
    def bf(a):
        return gen.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    ex0 = {"format": "bf16", "gate": bf([[1, 0]]), "up": bf([[1, 0]]), "down": bf([[1], [1]])}
    ex1 = {"format": "bf16", "gate": bf([[0, 1]]), "up": bf([[2, 0]]), "down": bf([[1], [-2]])}
    router = np.array([[0.0, -1.0], [0.0, 1.0]], dtype=np.float32)
    layer = ArrayLayer(router, {0: ex0, 1: ex1})
    x = np.array([[0.5, 2.0]])
    r = oracle.moe_block(x, layer, 1)
    a = 2.0 / (1.0 + math.exp(-2.0)) * 1.0
    assert list(r["ids"][0]) == [1] and r["w"][0, 0] == 1.0
    np.testing.assert_allclose(r["y"][0], [a, -2 * a], rtol=1e-15)


def test_stack_of_one_layer_is_block_plus_residual():
    wl = _tiny_with_shared()
    layer = GenLayer(wl)
    x = gen.hidden_states(wl)
    st = oracle.moe_stack(x, [layer], 3)
    blk = oracle.moe_block(oracle.rms_norm(x, 1e-6), layer, 3)
    np.testing.assert_allclose(st[0]["y"], x + blk["y"], rtol=1e-14, atol=1e-15)


def test_stack_of_three_layers_equals_explicit_composition():
    """Chaining pin: x_{l+1} = x_l + MoE_l(RMSNorm(x_l)) composed by hand from the dense textbook
    MoE of each layer (torch fp64), for three different layers. Feeding a layer its own input
    instead of the previous output, normalising the residual, or reusing one layer's weights
    each fails this."""
    wl = _tiny_with_shared()
    layers = [GenLayer(wl, li) for li in range(3)]
    x0 = gen.hidden_states(wl) * 2.0
    st = oracle.moe_stack(x0, layers, 3)
    x = x0.astype(np.float64)
    for li, layer in enumerate(layers):
        x = _dense_textbook_moe(x, layer, 3, 12, residual=True, pre_norm=True)
        np.testing.assert_allclose(st[li]["y"], x, rtol=1e-10, atol=1e-12)
    # the layers differ, so the composition order matters
    swapped = oracle.moe_stack(x0, [layers[1], layers[0], layers[2]], 3)
    assert np.abs(swapped[1]["y"] - st[1]["y"]).max() > 1e-6


# ---------------------------------------------------------------- acceptance
def test_argmax_first_brute_force_and_ties():
    rng = np.random.default_rng(6)
    L = rng.integers(0, 5, size=(20, 30)).astype(np.float32)  # many exact ties
    got = oracle.argmax_first(L)
    for i in range(20):
        m = max(L[i])
        assert got[i] == min(j for j in range(30) if L[i, j] == m)


def test_accept_length_brute_force_and_edges():
    t = np.array([5, 9, 9, 2, 7])
    assert oracle.accept_length(np.array([], dtype=np.int64), t) == 0
    assert oracle.accept_length(np.array([5, 9, 9, 2]), t) == 4
    assert oracle.accept_length(np.array([4, 9, 9, 2]), t) == 0
    assert oracle.accept_length(np.array([5, 9, 1, 2]), t) == 2
    assert oracle.committed_tokens(np.array([5, 9, 1, 2]), t) == [5, 9, 9]
    assert oracle.committed_tokens(np.array([5, 9, 9, 2, 7]), t) == [5, 9, 9, 2, 7]
    rng = np.random.default_rng(7)
    for _ in range(500):
        n = int(rng.integers(0, 8))
        tg = rng.integers(0, 3, size=n + int(rng.integers(0, 2)))
        d = rng.integers(0, 3, size=n)
        brute = max(j for j in range(n + 1) if all(d[i] == tg[i] for i in range(j)))
        assert oracle.accept_length(d, tg) == brute


# ---------------------------------------------------------------- output head
def _bf16_bits(x):
    return gen.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_head_logits_brute_force_tiny():
    rng = np.random.default_rng(31)
    n, V, H = 3, 7, 5
    h = rng.standard_normal((n, H))
    w = _bf16_bits(rng.standard_normal((V, H)))
    got = oracle.head_logits(h, w)
    assert got.shape == (n, V)
    for i in range(n):
        for v in range(V):
            ref = sum(float(h[i, c]) * _bf16_closed_form(int(w[v, c])) for c in range(H))
            assert abs(got[i, v] - ref) <= 1e-12 * (1 + abs(ref))


def test_head_logits_one_hot_and_ones_rows():
    """A one-hot hidden state picks one weight column; an all-ones one sums every row (a
    transposed operand or a dropped term fails one of the two)."""
    rng = np.random.default_rng(32)
    V, H = 40, 24
    w = _bf16_bits(rng.standard_normal((V, H)) * 0.02)
    wf = np.array([[_bf16_closed_form(int(b)) for b in row] for row in w])
    h = np.zeros((3, H))
    h[0, 5] = 1.0
    h[1, 23] = -2.0
    h[2, :] = 1.0
    got = oracle.head_logits(h, w)
    assert np.array_equal(got[0], wf[:, 5])
    assert np.array_equal(got[1], -2.0 * wf[:, 23])
    np.testing.assert_allclose(got[2], wf.sum(axis=1), rtol=0, atol=1e-15)


def test_head_accept_planted_winners_ties_and_prefix():
    """Position i's hidden state points along coordinate c_i and row v_i is the unit vector of
    c_i, so v_i wins with logit ~10 against random rows of ~0.2; an identical later row loses the
    tie; the accepted length follows the drafts."""
    rng = np.random.default_rng(33)
    V, H = 300, 64
    planted, coords = [17, 250, 3, 17], [5, 40, 63, 5]
    w = _bf16_bits(rng.standard_normal((V, H)) * 0.02)
    h = 0.01 * np.abs(rng.standard_normal((4, H)))
    for i, (v, c) in enumerate(zip(planted, coords)):
        h[i, c] += 10.0
        w[v] = _bf16_bits(np.eye(H)[c])
    w[260] = w[250]                                        # exact tie: the lower index wins
    logits = oracle.head_logits(h, w)
    assert logits[1, 250] == logits[1, 260]
    t, a = oracle.head_accept(h, w, np.array([17, 250, 9, 17]))
    assert list(t) == planted
    assert a == 2
    assert oracle.head_accept(h, w, np.array(planted))[1] == 4
    assert oracle.head_accept(h, w, np.array([], dtype=np.int64))[1] == 0


# ---------------------------------------------------------------- stochastic acceptance
def test_softmax_temp_closed_forms_and_library():
    from scipy.special import softmax
    rng = np.random.default_rng(41)
    l = rng.standard_normal(50)
    for T in (0.3, 1.0, 2.5):
        np.testing.assert_allclose(oracle.softmax_temp(l, T), softmax(l / T), rtol=1e-13, atol=0)
    np.testing.assert_allclose(oracle.softmax_temp(np.full(8, 3.0), 0.7), np.full(8, 1 / 8), rtol=1e-15)
    p = oracle.softmax_temp(np.array([0.0, -np.inf, 1.0]), 1.0)
    assert p[1] == 0.0 and abs(p[2] / p[0] - math.e) < 1e-12


def test_sample_inverse_cdf_brute_force():
    rng = np.random.default_rng(42)
    for _ in range(300):
        w = rng.random(7) * (rng.random(7) < 0.7)
        if w.sum() == 0:
            continue
        u = float(rng.random())
        run, x = 0.0, None
        for i, wi in enumerate(w):
            run += wi
            if run > u * w.sum():
                x = i
                break
        got = oracle.sample_inverse_cdf(w, u)
        assert got == x and w[got] > 0
    # exact boundaries: u = 0 skips leading zero weights; a running sum equal to u * total is not
    # yet past it
    assert oracle.sample_inverse_cdf(np.array([0.0, 0.0, 2.0, 1.0]), 0.0) == 2
    assert oracle.sample_inverse_cdf(np.array([1.0, 1.0, 2.0]), 0.5) == 2
    assert oracle.sample_inverse_cdf(np.array([1.0, 0.0, 3.0]), 0.25) == 2


def _boundary(f, lo=0.0, hi=1.0, iters=60):
    """Smallest u in [lo, hi] with f(u) true, for f monotone (false then true); hi if never."""
    if not f(hi):
        return hi
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        lo, hi = (lo, mid) if f(mid) else (mid, hi)
    return hi


def test_speculative_accept_is_lossless():
    """The first committed token is distributed exactly as the target's p_0, and when every draft
    is kept the bonus token as p_n: the acceptance region and the sampled token's regions are
    measured by bisection on the oracle's own decisions, then combined over d_0 ~ q_0."""
    rng = np.random.default_rng(43)
    V, n, T = 6, 2, 0.8
    tl = rng.standard_normal((n + 1, V)) * 1.5
    dl = tl[:n] + rng.standard_normal((n, V))          # a drafter close to the target
    p0 = oracle.softmax_temp(tl[0], T)
    q0 = oracle.softmax_temp(dl[0], T)

    def run(d0, ua0, us0, us_bonus=0.5):
        return oracle.speculative_accept(tl, dl, np.array([d0, 0]), T, np.array([ua0, 0.0]),
                                         np.array([us0, 0.5, us_bonus]))

    dist = np.zeros(V)
    for d in range(V):
        alpha = _boundary(lambda u: run(d, u, 0.5)[0] == 0)   # accept while u < alpha
        dist[d] += q0[d] * alpha
        if alpha < 1.0:
            edges = [0.0] + [_boundary(lambda u, x=x: run(d, 1.0 - 1e-12, u)[1] >= x) for x in range(1, V)] + [1.0]
            dist += q0[d] * (1.0 - alpha) * np.diff(edges)
    np.testing.assert_allclose(dist, p0, rtol=0, atol=1e-12)
    pn = oracle.softmax_temp(tl[n], T)
    same = oracle.speculative_accept(tl, tl[:n], np.array([0, 1]), T, np.zeros(n), np.zeros(n + 1))
    assert same[0] == n
    edges = [0.0] + [_boundary(lambda u, x=x: oracle.speculative_accept(tl, tl[:n], np.array([0, 1]), T, np.zeros(n),
                                                                      np.array([0.0, 0.0, u]))[1] >= x)
                     for x in range(1, V)] + [1.0]
    np.testing.assert_allclose(np.diff(edges), pn, rtol=0, atol=1e-12)


def test_speculative_accept_special_cases():
    rng = np.random.default_rng(44)
    V, n = 30, 4
    tl = rng.standard_normal((n + 1, V))
    # a drafter equal to the target keeps every draft for any u < 1
    a, tok = oracle.speculative_accept(tl, tl[:n], rng.integers(0, V, n), 1.0, np.full(n, 0.999999), np.zeros(n + 1))
    assert a == n and tok == oracle.sample_inverse_cdf(oracle.softmax_temp(tl[n], 1.0), 0.0)
    # a draft the target gives probability zero is always rejected; the residual is then p itself
    # when the drafter is one-hot on it
    tz = tl.copy()
    tz[1, 7] = -np.inf
    dl = np.full((n, V), -np.inf)
    dl[:, 7] = 0.0
    dl[0] = tl[0]
    draft = np.array([3, 7, 7, 7])
    for u in (0.0, 0.5, 0.9):
        a, tok = oracle.speculative_accept(tz, dl, draft, 1.0, np.array([0.0, u, u, u]), np.full(n + 1, u))
        assert a == 1 and tok == oracle.sample_inverse_cdf(oracle.softmax_temp(tz[1], 1.0), u) and tok != 7
    # the low-temperature limit is greedy acceptance of the drafter's own argmax, and the token at
    # the first disagreement is the target's argmax
    sep = np.argsort(rng.random((n + 1, V)), axis=1).astype(np.float64)   # distinct integer logits
    tgt = oracle.argmax_first(sep)
    dsep = sep[:n].copy()
    dsep[2, (tgt[2] + 1) % V] = V + 5.0                                    # the drafter disagrees at 2
    draft = oracle.argmax_first(dsep)
    a, tok = oracle.speculative_accept(sep, dsep, draft, 1e-3, np.full(n, 0.5), np.full(n + 1, 0.5))
    assert a == oracle.accept_length(draft, tgt) == 2 and tok == tgt[2]
    # a rejection whose residual has no mass draws from the target itself
    a, tok = oracle.speculative_accept(sep, sep[:n] * 0.5, draft, 1e-3, np.full(n, 0.5), np.full(n + 1, 0.5))
    assert a == 2 and tok == tgt[2]
    # an id outside the vocabulary is rejected
    assert oracle.speculative_accept(tl, tl[:n], np.array([0, V, 1, 2]), 1.0, np.zeros(n), np.zeros(n + 1))[0] == 1
    # no bonus row: every draft kept gives no token
    assert oracle.speculative_accept(tl[:n], tl[:n], np.zeros(n, dtype=np.int64), 1.0, np.zeros(n),
                                     np.zeros(n)) == (n, -1)


def test_accept_histogram_brute_force():
    rng = np.random.default_rng(45)
    a = rng.integers(0, 17, size=500)
    hist, surv = oracle.accept_histogram(a, 16)
    assert hist.sum() == 500 and len(hist) == 17 and len(surv) == 16
    for j in range(17):
        assert hist[j] == sum(1 for v in a if v == j)
    for i in range(16):
        assert surv[i] == sum(1 for v in a if v >= i + 1)
    assert surv[0] == 500 - hist[0]


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


@pytest.mark.parametrize("row", _read_golden("geometric_acceptance.txt"), ids=lambda r: "-".join(r[:3]))
def test_geometric_acceptance_reproduces_printed_values(row):
    """Synthetic cycles with a geometric agreeing prefix, scored by the oracle's argmax and
    acceptance, reproduce the per-cycle values the part-2 page prints for that model."""
    p, gamma, what, printed, tol = float(row[0]), int(row[1]), row[2], float(row[3]), float(row[4])
    base = gen.Workload("mc", gen.LayerShape(8, 2, 1, 8, 0), k=1, seed=4242, vocab=64,
                        n_target=gamma + 1, n_draft=gamma, accept_p=p)
    n_cycles = 20000
    acc = np.empty(n_cycles, dtype=np.int64)
    for c in range(n_cycles):
        logits, planted = gen.target_logits(base, rep=c)
        draft, _ = gen.draft_ids(base, planted, rep=c)
        acc[c] = oracle.accept_length(draft, oracle.argmax_first(logits))
    closed_tau = (1 - p ** (gamma + 1)) / (1 - p)
    if what == "tau":
        got = acc.mean() + 1.0
        assert abs(got - closed_tau) < 4 * acc.std() / math.sqrt(n_cycles) + 1e-9
        assert abs(closed_tau - printed) <= tol
        assert abs(got - printed) <= tol + 4 * acc.std() / math.sqrt(n_cycles)
    elif what == "p_accept_none":
        got = np.mean(acc == 0)
        assert abs(got - (1 - p)) < 0.015
        assert abs((1 - p) - printed) <= tol
    elif what == "p_accept_exactly_one":
        got = np.mean(acc == 1)
        assert abs(got - p * (1 - p)) < 0.015
        assert abs(p * (1 - p) - printed) <= tol
    else:
        raise AssertionError(what)


def test_signed_zero_worked_example():
    """The part-2 page's 16x16 example, D = A B with D[i, j] = -(j+1)/16 whether B's zeros are +0
    or -0, run through the oracle's own product: the router logits of 16 tokens (B's columns,
    padded with signed zeros) against 16 experts (A's rows), l[t, e] = D[e, t]. A dropped term, a
    transposed operand or a sign slip in router_logits moves a printed value or its bits."""
    rows = _read_golden("signed_zero_mma.txt")
    A = np.zeros((16, 16), dtype=np.float32)
    A[:, 12] = -1.0
    for neg in (False, True):
        B = np.full((16, 16), -0.0 if neg else 0.0, dtype=np.float32)
        B[12, :] = (np.arange(16) + 1) / 16.0
        tokens = B.T.copy()  # token j is column j of B
        logits = oracle.router_logits(tokens, A).astype(np.float32)
        D = logits.T
        for i, j, v, bits in rows:
            assert D[int(i), int(j)] == float(v)
            assert struct.unpack("<I", struct.pack("<f", D[int(i), int(j)]))[0] == int(bits, 16)


# ---- tiled storage layout -------------------------------------------------------------------
def test_tile_bf16_hand_positions():
    """Positions read off the layout's definition by hand, for a 32 x 256 matrix whose entry is
    its own row-major index: slice l of tile (band, step) starts at chunk (band*8 + step)*64 + l."""
    from oracle import tile_bf16
    R, C = 32, 256
    w = np.arange(R * C, dtype=np.int64).reshape(R, C)
    t = tile_bf16(w).reshape(-1)
    assert t[0] == 0                     # band 0, step 0, slice 0: W[0][0]
    assert t[8] == 1 * C                 # slice 1 -> row 1, column 0
    assert t[15 * 8] == 15 * C           # slice 15 -> row 15
    assert t[16 * 8] == 8                # slice 16 -> row 0, columns 8..15
    assert t[16 * 8 + 7] == 15
    assert t[63 * 8] == 15 * C + 24      # slice 63 -> row 15, columns 24..31
    assert t[64 * 8] == 32               # next step: row 0, column 32
    assert t[8 * 64 * 8] == 16 * C       # band 1 starts after C/32 = 8 steps: row 16
    assert t[-1] == R * C - 1            # last element stays last


def test_tile_bf16_is_a_permutation_and_matches_position_formula():
    from oracle import tile_bf16, tiled_position_bf16
    rng = np.random.default_rng(5)
    w = rng.integers(0, 1 << 16, size=(3, 48, 384), dtype=np.uint16)
    t = tile_bf16(w)
    assert np.array_equal(np.sort(t.reshape(-1)), np.sort(w.reshape(-1)))
    for m, row, col in [(0, 0, 0), (1, 47, 383), (2, 17, 130), (0, 31, 95), (1, 5, 200)]:
        assert t[m].reshape(-1)[tiled_position_bf16(48, 384, row, col)] == w[m, row, col]


def test_tile_mxfp4_hand_positions():
    """Block b of row r occupies code bytes 16 b .. 16 b + 15; in the tiled order slice l of
    window w (band 0) is block 4 w + l // 16 of row l % 16."""
    from oracle import tile_mxfp4
    R, C = 16, 256                                    # 2 windows of 4 blocks per row
    blk = np.arange(R * C // 32, dtype=np.int64).reshape(R, C // 32)   # block id = row * 8 + block
    codes = np.repeat(blk[:, :, None], 16, axis=2).reshape(R, C // 2) % 256
    scales = (blk % 256).astype(np.int64)
    tc, ts = tile_mxfp4(codes, scales)
    tcb = tc.reshape(-1, 16)
    assert np.all(tcb == tcb[:, :1])                  # 16-byte slices stay whole
    ids = tcb[:, 0]
    assert ids[0] == 0                                # window 0, slice 0: row 0 block 0
    assert ids[1] == 8                                # slice 1: row 1 block 0
    assert ids[16] == 1                               # slice 16: row 0 block 1
    assert ids[63] == 15 * 8 + 3                      # slice 63: row 15 block 3
    assert ids[64] == 4                               # window 1, slice 0: row 0 block 4
    assert np.array_equal(ts.reshape(-1), ids)        # each scale travels with its block
