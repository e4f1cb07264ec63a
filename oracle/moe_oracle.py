"""CPU oracle for the MoE verify-block path. TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import or call
this package. The GPU library never imports, links or runs it, and this package imports nothing
from the GPU library. It is plain NumPy in float64, written from the definitions token by token:
grouping tokens by expert, the woken-expert union and the permutation are reorganisations of a
per-token sum, so the oracle computes the per-token sum directly and reports the union beside it.

Sources, cited by short name:
  [SH1] "Speculating on a Strix Halo" (natemacfadden.com/dflash)
  [SH2] "Speculating on a Strix Halo (part 2)" (natemacfadden.com/dflash-part2)
  [MI]  the DFlash-on-AMD-Instinct-MI355X article (allbreaknews.com/?p=4397)

Readings where the pages are silent (each listed with its reason in the design notes):
  * router: fp32 logits from fp32 normalised inputs; the K largest logits are selected, ties going
    to the lower expert index, output in descending-logit order; the routing weights are the
    softmax over the selected K (equal to a full softmax restricted to the K and renormalised);
  * expert FFN: SwiGLU, a = silu(W_g x) * (W_u x), y = W_d a, silu(z) = z / (1 + e^-z);
  * one always-on shared expert with weight 1 and no gate; no router bias, noise or capacity;
  * pre-norm RMSNorm with unit gain, eps inside the square root; residual on the raw stream;
  * argmax ties go to the lowest vocabulary index; draft i is compared with target i.

Every function has a pin in the CPU test suite (closed forms, brute force on tiny inputs,
special cases that reduce to a library routine, the pages' printed values). Parity unpinned:
nothing here; what stays unpinned is the GPU's exact fp32 rounding, checked by tolerance only.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes by the low three code bits (sign in bit 3): OCP MX v1.0 FP4 element format.
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# ----------------------------------------------------------------------------------------------
# weight decoding
# ----------------------------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64. bf16 is the upper half of an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns convert to quiet NaN
        return b.view(np.float32).astype(np.float64)


def decode_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """mxfp4 -> float64. codes uint8 [R][C/2] (element 2j in the low nibble of byte j), scales
    uint8 [R][C/32] (e8m0: 2^(s-127), 0xFF = NaN). Quantised target weights per [MI] 'Why
    Quantize the Target Model on Top?'; the E2M1 + e8m0 per-32 block format is OCP MX v1.0."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    r, half = codes.shape
    c = half * 2
    nib = np.empty((r, c), dtype=np.uint8)
    nib[:, 0::2] = codes & 0x0F
    nib[:, 1::2] = codes >> 4
    val = _E2M1[nib & 7]
    val = np.where(nib & 8, -val, val)
    s = scales.astype(np.float64)
    mult = np.where(scales == 0xFF, np.nan, np.exp2(s - 127.0))
    return val * np.repeat(mult, 32, axis=1)


def decode_tensor(raw: dict, name: str) -> np.ndarray:
    if raw["format"] == "bf16":
        return decode_bf16(raw[name])
    if raw["format"] == "mxfp4":
        return decode_mxfp4(raw[name], raw[name + "_scale"])
    raise ValueError(f"unknown weight format {raw['format']!r}")


# ----------------------------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------------------------
def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) per row, unit gain (pre-norm of each stacked MoE layer)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def router_logits(xh: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """l[t, e] = sum_h xh[t, h] * W_r[e, h]: every block token routes on its own
    ([SH1] 'What the pieces cost': each token routes to its own experts). One product per
    token, so a block row is computed exactly as that token alone would be."""
    w = np.asarray(w_router, dtype=np.float64)
    xh = np.asarray(xh, dtype=np.float64)
    return np.stack([w @ xh[t] for t in range(xh.shape[0])]) if xh.shape[0] else np.zeros((0, w.shape[0]))


def select_topk(logits_row: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits in descending order; equal logits go to the lower index.
    A full lexicographic sort on (-logit, index), not a heap ([SH1] ref. 1: 8 routed experts of
    256 per token)."""
    l = np.asarray(logits_row, dtype=np.float64)
    order = np.lexsort((np.arange(l.size), -l))
    return order[:k].astype(np.int64)


def routing_weights(logits_row: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits: exp(l_j - m) / sum_j' exp(l_j' - m), m their max."""
    sel = np.asarray(logits_row, dtype=np.float64)[ids]
    e = np.exp(sel - sel.max())
    return e / e.sum()


def topk_gap(logits_row: np.ndarray, k: int) -> float:
    """K-th minus (K+1)-th largest logit (inf when K = E): the near-tie margin of the selection."""
    v = np.sort(np.asarray(logits_row, dtype=np.float64))[::-1]
    return float(v[k - 1] - v[k]) if k < v.size else float("inf")


def woken_experts(ids: np.ndarray):
    """Union of the block's per-token expert sets and the token-by-expert permutation.

    Returns (woken ascending [U], counts [U], offsets [U+1], perm [k*K][2] of (token, slot)
    ordered by (expert, token)). The block wakes the union of its tokens' experts
    ([SH1] 'Spoilers' and 'What the pieces cost'); tokens are grouped by expert before one launch
    per projection ([SH1] 'The verify's own cost')."""
    ids = np.asarray(ids, dtype=np.int64)
    k, kk = ids.shape
    woken = sorted({int(e) for e in ids.ravel()})
    triples = sorted((int(ids[t, j]), t, j) for t in range(k) for j in range(kk))
    counts = [sum(1 for e, _, _ in triples if e == w) for w in woken]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    perm = np.array([(t, j) for _, t, j in triples], dtype=np.int64).reshape(-1, 2)
    return np.array(woken, dtype=np.int64), np.array(counts, dtype=np.int64), offsets, perm


# ----------------------------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """One expert on one token: W_d (silu(W_g x) * (W_u x)). Each expert is a [2048 x 512]-class
    weight applied to the tokens routed to it ([SH1] 'The verify's own cost')."""
    g = w_gate @ x
    u = w_up @ x
    return w_down @ (silu(g) * u)


class _DecodedLayer:
    """Decodes and memoises the experts one layer call touches."""

    def __init__(self, layer):
        self.layer = layer
        self.cache = {}

    def expert(self, e: int):
        if e not in self.cache:
            raw = self.layer.expert(e)
            self.cache[e] = tuple(decode_tensor(raw, n) for n in ("gate", "up", "down"))
        return self.cache[e]

    def shared(self):
        if "shared" not in self.cache:
            raw = self.layer.shared()
            self.cache["shared"] = None if raw is None else tuple(
                decode_tensor(raw, n) for n in ("gate", "up", "down"))
        return self.cache["shared"]


def moe_block(x: np.ndarray, layer, top_k: int, *, pre_norm: bool = False, rms_eps: float = 1e-6,
              residual: bool = False, forced_ids: np.ndarray | None = None) -> dict:
    """The MoE layer over a verify block of k tokens, computed token by token.

    ``layer`` provides router() -> fp32 [E][H], expert(e) / shared() -> raw encoded tensors.
    The target checks the whole block in one pass ([SH1] 'Speculative decoding'); the block's
    expert work is the union of its tokens' experts plus the always-on shared expert ([SH1]
    'What the pieces cost'). y_t = sum_j w_tj * FFN_{e_tj}(xh_t) + FFN_shared(xh_t) [+ x_t].
    ``forced_ids`` [k][K] replaces the selection (for tokens whose GPU ids differ at a near-tie);
    weights are then the softmax over the forced logits.
    """
    x = np.asarray(x, dtype=np.float64)
    k, _ = x.shape
    xh = rms_norm(x, rms_eps) if pre_norm else x
    logits = router_logits(xh, layer.router())
    dec = _DecodedLayer(layer)
    ids = np.zeros((k, top_k), dtype=np.int64)
    w = np.zeros((k, top_k), dtype=np.float64)
    gaps = np.zeros(k, dtype=np.float64)
    y = np.zeros_like(x)
    for t in range(k):
        ids[t] = select_topk(logits[t], top_k) if forced_ids is None else np.asarray(forced_ids[t])
        w[t] = routing_weights(logits[t], ids[t])
        gaps[t] = topk_gap(logits[t], top_k)
        acc = np.zeros(x.shape[1], dtype=np.float64)
        for j in range(top_k):
            acc += w[t, j] * expert_ffn(xh[t], *dec.expert(int(ids[t, j])))
        sh = dec.shared()
        if sh is not None:
            acc += expert_ffn(xh[t], *sh)
        y[t] = acc + x[t] if residual else acc
    woken, counts, offsets, perm = woken_experts(ids)
    return {"y": y, "ids": ids, "w": w, "logits": logits, "gap": gaps, "woken": woken,
            "counts": counts, "offsets": offsets, "perm": perm, "n_woken": int(woken.size)}


def moe_stack(x0: np.ndarray, layers, top_k: int, *, rms_eps: float = 1e-6) -> list:
    """Stacked pre-norm MoE layers with a residual add: x_{l+1} = x_l + MoE_l(RMSNorm(x_l))."""
    outs = []
    x = np.asarray(x0, dtype=np.float64)
    for layer in layers:
        r = moe_block(x, layer, top_k, pre_norm=True, rms_eps=rms_eps, residual=True)
        outs.append(r)
        x = r["y"]
    return outs


# ----------------------------------------------------------------------------------------------
# acceptance
# ----------------------------------------------------------------------------------------------
def head_logits(h: np.ndarray, w_head_bits: np.ndarray) -> np.ndarray:
    """Target logits of the block positions, l[i, v] = sum_c h[i, c] * W[v, c], with the output
    head W [V][H] in bf16 and the positions' final hidden states h [n][H] taken as given (no
    final normalisation). The head is one matrix read once for the whole block ([SH1] 'What the
    pieces cost'); it is the [hidden x V] matrix whose streaming cost grows with V ([SH1] 'Should
    we shrink the vocab?')."""
    return np.asarray(h, dtype=np.float64) @ decode_bf16(w_head_bits).T


def head_accept(h: np.ndarray, w_head_bits: np.ndarray, draft: np.ndarray):
    """The output head followed by greedy acceptance: (target ids, accepted length)."""
    t = argmax_first(head_logits(h, w_head_bits))
    return t, accept_length(np.asarray(draft), t)


def argmax_first(logits: np.ndarray) -> np.ndarray:
    """Greedy target token per block position: the lowest index attaining the row maximum."""
    return np.argmax(np.asarray(logits), axis=1).astype(np.int64)


def accept_length(draft: np.ndarray, target_ids: np.ndarray) -> int:
    """Longest prefix on which the draft equals what the target would itself produce: draft n
    counts only if drafts 0..n-1 did ([SH1] 'Speculative decoding'; [SH2] 'Why drafter
    performance doesn't really matter')."""
    a = 0
    n = min(len(draft), len(target_ids))
    while a < n and int(draft[a]) == int(target_ids[a]):
        a += 1
    return a


def softmax_temp(logits_row: np.ndarray, temperature: float) -> np.ndarray:
    """p = softmax(l / T) in float64 (the maximum subtracted first; -inf logits give 0)."""
    z = np.asarray(logits_row, dtype=np.float64) / float(temperature)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def sample_inverse_cdf(weights: np.ndarray, u: float) -> int:
    """The smallest index x whose running sum of the non-negative weights exceeds u times their
    total (u in [0, 1)); an index of zero weight is never returned."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    return int(np.searchsorted(c, float(u) * c[-1], side="right"))


def speculative_accept(target_logits: np.ndarray, draft_logits: np.ndarray, draft: np.ndarray,
                       temperature: float, u_accept: np.ndarray, u_sample: np.ndarray):
    """Lossless acceptance of a draft block at temperature T: the committed tokens are
    distributed exactly as the target's own samples ([SH1] 'Speculative decoding', which relies
    on its reference 2, Leviathan et al., for the rule restated here).

    With p_i = softmax(target_logits[i] / T) and q_i = softmax(draft_logits[i] / T), draft d_i is
    kept while u_accept[i] * q_i(d_i) < p_i(d_i) (probability min(1, p_i(d_i) / q_i(d_i))). At the
    first rejection a, the target's own token is drawn from the residual max(0, p_a - q_a)
    (renormalised) with u_sample[a]; if every draft is kept, from p_n (n = len(draft)) with
    u_sample[n] when that row exists. Returns (a, token), token -1 when there is no row to draw
    from. A residual with no mass (p_a = q_a, reachable only through rounding or a draft that q_a
    gives probability zero) is read as its limit, p_a itself. A draft id outside [0, V) has
    target probability zero and is rejected."""
    n = len(draft)
    for i in range(n):
        p = softmax_temp(target_logits[i], temperature)
        q = softmax_temp(draft_logits[i], temperature)
        d = int(draft[i])
        if not (0 <= d < len(p)) or not (float(u_accept[i]) * q[d] < p[d]):
            r = np.maximum(p - q, 0.0)
            return i, sample_inverse_cdf(r if r.sum() > 0 else p, u_sample[i])
    if len(target_logits) > n:
        return n, sample_inverse_cdf(softmax_temp(target_logits[n], temperature), u_sample[n])
    return n, -1


def accept_histogram(accepted: np.ndarray, n_draft: int):
    """Cycle statistics of accepted lengths ([SH2] 'Why drafter performance doesn't really
    matter' counts cycles by accepted length; [MI] plots the per-position marginal): hist[j] = the
    number of cycles that accepted exactly j drafts (0 <= j <= n_draft), and survival[i] = the
    number that accepted at least i + 1 (the marginal P(accept >= i + 1) times the cycle count)."""
    a = np.asarray(accepted, dtype=np.int64)
    hist = np.array([int(np.sum(a == j)) for j in range(n_draft + 1)], dtype=np.int64)
    survival = np.array([int(np.sum(a >= i + 1)) for i in range(n_draft)], dtype=np.int64)
    return hist, survival


def committed_tokens(draft: np.ndarray, target_ids: np.ndarray) -> list:
    """The accepted draft prefix plus the target's own token after it, when there is one:
    tau = a + 1 tokens per cycle ([SH1] 'Speculative decoding')."""
    a = accept_length(draft, target_ids)
    out = [int(d) for d in draft[:a]]
    if a < len(target_ids):
        out.append(int(target_ids[a]))
    return out
