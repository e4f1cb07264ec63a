"""Seeded synthetic inputs for the MoE verify-block path.

This module only *draws* inputs. It holds none of the method's arithmetic (no routing, top-k,
expert products, combine, argmax or acceptance). The CPU oracle (through the tests) and the
GPU library consume exactly the arrays made here.

The pages measure real prompts (MATH-500, HumanEval, ...) on a real Qwen3.6-35B-A3B target;
neither is available, so seeded synthetic inputs with the workload shapes stand in for them:

* expert and output-head weights: bf16 ~N(0, 0.02^2), or (experts) mxfp4 (E2M1 codes, one e8m0 scale per 32 values along
  the reduction dimension) quantised from the same fp32 draws;
* router weights: fp32 ~N(0, 0.02^2); block hidden states: fp32 ~N(0, 1);
* target logits: fp32 ~N(0, 1); draft ids: uniform, or agreeing with a planted target id for a
  geometric prefix (per-position acceptance p) and uniform afterwards.

Expert weight streams are counter based so that the host can regenerate any single expert and a
GPU kernel can fill whole layers in place with identical bits:

* element n of tensor (seed, layer, kind, expert) is 16-bit word n of the numpy
  ``Philox(key=[seed, tensor_id])`` raw stream (Philox4x64-10, Salmon et al., "Parallel random
  numbers: as easy as 1, 2, 3", SC 2011), with tensor_id = layer<<32 | kind<<16 | expert;
* the 16-bit word indexes a 65536-entry table of standard-normal quantiles
  Phi^-1((i + 1/2)/65536) stored as float32 and multiplied by 0.02 in float32;
* bf16 weights are that float32 rounded to nearest-even; mxfp4 weights quantise it (below).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from functools import lru_cache

import numpy as np

KIND_GATE, KIND_UP, KIND_DOWN = 0, 1, 2
KIND_HEAD = 3  # the target's output head [V][H] (layer 0, expert 0)
SHARED_EXPERT_ID = 0xFFFF
WEIGHT_STD = 0.02
PLANTED_LOGIT = 8.0  # exceeds every N(0,1) draw of a 151936-wide row with probability ~1e-10


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    wdtype: str = "bf16"  # "bf16" | "mxfp4" (routed experts; shared expert stays bf16)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    k: int
    seed: int
    n_layers: int = 1
    vocab: int = 0
    n_target: int = 0
    n_draft: int = 0
    accept_p: float | None = None      # geometric agreeing prefix; None = uniform drafts
    sigma: float | None = None          # correlated block: x_t = b + sigma * n_t
    sigmas: tuple = field(default_factory=tuple)
    pre_norm: bool = False
    residual: bool = False
    rms_eps: float = 1e-6


_L1 = LayerShape(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512)

WORKLOADS = {
    "tiny": Workload("tiny", LayerShape(256, 16, 2, 128, 0), k=4, seed=1000,
                     vocab=1000, n_target=4, n_draft=4),
    "decode": Workload("decode", _L1, k=1, seed=1001),
    "verify": Workload("verify", _L1, k=16, seed=1002, vocab=151936, n_target=17, n_draft=16,
                       accept_p=0.7),
    "correlated": Workload("correlated", _L1, k=16, seed=1003, sigma=0.1,
                           sigmas=(0.0, 0.05, 0.1, 0.3, 1.0)),
    "stack40_mxfp4": Workload("stack40_mxfp4",
                              LayerShape(2048, 256, 8, 512, 512, wdtype="mxfp4"), k=16,
                              seed=1004, n_layers=40, vocab=151936, n_target=17, n_draft=16,
                              accept_p=0.7, pre_norm=True, residual=True),
    # 32 sequences verified together, 16 independent block tokens each
    "batched": Workload("batched", _L1, k=512, seed=1005),
}


# ----------------------------------------------------------------------------------------------
# counter-based weight streams
# ----------------------------------------------------------------------------------------------
def tensor_id(layer: int, kind: int, expert: int) -> int:
    return (int(layer) << 32) | (int(kind) << 16) | int(expert)


@lru_cache(maxsize=1)
def normal_quantile_table() -> np.ndarray:
    """float32 [65536]: WEIGHT_STD * Phi^-1((i + 1/2) / 65536), the multiply done in float32."""
    from scipy.special import ndtri
    q = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0).astype(np.float32)
    return (q * np.float32(WEIGHT_STD)).astype(np.float32)


@lru_cache(maxsize=1)
def bf16_table() -> np.ndarray:
    """uint16 [65536]: the quantile table rounded to bf16 (nearest, ties to even)."""
    return f32_to_bf16_bits(normal_quantile_table())


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns, nearest-even (inputs are finite)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def stream_words(seed: int, tid: int, n: int) -> np.ndarray:
    """The first n 16-bit words of the Philox(key=[seed, tid]) raw stream (little-endian)."""
    g = np.random.Philox(key=np.array([seed, tid], dtype=np.uint64))
    raw = g.random_raw((n + 3) // 4)
    return raw.view(np.uint16)[:n]


def weight_f32(seed: int, layer: int, kind: int, expert: int, rows: int, cols: int) -> np.ndarray:
    idx = stream_words(seed, tensor_id(layer, kind, expert), rows * cols)
    return normal_quantile_table()[idx].reshape(rows, cols)


def weight_bf16(seed: int, layer: int, kind: int, expert: int, rows: int, cols: int) -> np.ndarray:
    idx = stream_words(seed, tensor_id(layer, kind, expert), rows * cols)
    return bf16_table()[idx].reshape(rows, cols)


# mxfp4 quantiser (input preparation only: both sides consume the codes it writes).
# Per block of 32 consecutive values: shared exponent s = floor(log2(max|w|)) - 2 (the E2M1 largest
# normal is 1.5 * 2^2), scale byte = s + 127, and each w / 2^s is rounded to the nearest E2M1
# magnitude {0, .5, 1, 1.5, 2, 3, 4, 6} with ties to the even code, saturating at 6. The low nibble
# of byte j holds element 2j.
_E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
_TIE_ROUNDS_UP = np.array([False, True, False, True, False, True, False])


def quantize_mxfp4_rows(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    blk = w.reshape(rows, cols // 32, 32)
    amax = np.abs(blk).max(axis=2)
    e = ((amax.view(np.uint32) >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32) - 127
    s = e - 2
    s[amax == 0] = -127
    scale = (s + 127).astype(np.uint8)
    q = np.abs(np.ldexp(blk, (-s)[..., None]).astype(np.float32))
    mag = np.zeros(q.shape, dtype=np.uint8)
    for t, up in zip(_E2M1_MIDPOINTS, _TIE_ROUNDS_UP):
        mag += (q > t) | ((q == t) & up)
    code = mag | np.where(blk < 0, np.uint8(8), np.uint8(0))
    code = code.reshape(rows, cols)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale.reshape(rows, cols // 32)


def weight_mxfp4(seed, layer, kind, expert, rows, cols):
    return quantize_mxfp4_rows(weight_f32(seed, layer, kind, expert, rows, cols))


def expert_tensors(wl: Workload, layer: int, expert: int) -> dict:
    """Raw encoded tensors of one routed expert: gate/up [I][H], down [H][I]."""
    s = wl.shape
    dims = {KIND_GATE: (s.inter, s.hidden), KIND_UP: (s.inter, s.hidden), KIND_DOWN: (s.hidden, s.inter)}
    out = {"format": s.wdtype}
    for kind, name in ((KIND_GATE, "gate"), (KIND_UP, "up"), (KIND_DOWN, "down")):
        r, c = dims[kind]
        if s.wdtype == "bf16":
            out[name] = weight_bf16(wl.seed, layer, kind, expert, r, c)
        else:
            out[name], out[name + "_scale"] = weight_mxfp4(wl.seed, layer, kind, expert, r, c)
    return out


def shared_tensors(wl: Workload, layer: int) -> dict | None:
    s = wl.shape
    if s.shared_inter == 0:
        return None
    i = s.shared_inter
    return {"format": "bf16",
            "gate": weight_bf16(wl.seed, layer, KIND_GATE, SHARED_EXPERT_ID, i, s.hidden),
            "up": weight_bf16(wl.seed, layer, KIND_UP, SHARED_EXPERT_ID, i, s.hidden),
            "down": weight_bf16(wl.seed, layer, KIND_DOWN, SHARED_EXPERT_ID, s.hidden, i)}


def head_weight(wl: Workload) -> np.ndarray:
    """bf16 bits [V][H] of the target's output head (the same counter-based stream as the
    experts' weights, tensor kind KIND_HEAD)."""
    return weight_bf16(wl.seed, 0, KIND_HEAD, 0, wl.vocab, wl.shape.hidden)


# ----------------------------------------------------------------------------------------------
# small host-drawn inputs
# ----------------------------------------------------------------------------------------------
def router_weight(wl: Workload, layer: int) -> np.ndarray:
    rng = np.random.default_rng([wl.seed, 7, layer])
    s = wl.shape
    return (rng.standard_normal((s.n_experts, s.hidden), dtype=np.float32) * np.float32(WEIGHT_STD)).astype(np.float32)


def hidden_states(wl: Workload, rep: int = 0, k: int | None = None, sigma: float | None = None) -> np.ndarray:
    """fp32 [k][H]. Independent rows ~N(0,1), or b + sigma*n_t for the correlated block."""
    k = wl.k if k is None else k
    sigma = wl.sigma if sigma is None else sigma
    rng = np.random.default_rng([wl.seed, 1, rep])
    h = wl.shape.hidden
    if sigma is None:
        return rng.standard_normal((k, h), dtype=np.float32)
    base = rng.standard_normal((1, h), dtype=np.float32)
    noise = rng.standard_normal((k, h), dtype=np.float32)
    return (base + np.float32(sigma) * noise).astype(np.float32)


def target_logits(wl: Workload, rep: int = 0, n_target: int | None = None):
    """fp32 [n_target][V] ~N(0,1). With a geometric acceptance model, one entry per row is
    planted at PLANTED_LOGIT so the intended target id is known without any argmax; returns
    (logits, planted_ids or None)."""
    n = wl.n_target if n_target is None else n_target
    rng = np.random.default_rng([wl.seed, 2, rep])
    logits = rng.standard_normal((n, wl.vocab), dtype=np.float32)
    if wl.accept_p is None:
        return logits, None
    planted = rng.integers(0, wl.vocab, size=n, dtype=np.int64).astype(np.int32)
    logits[np.arange(n), planted] = np.float32(PLANTED_LOGIT)
    return logits, planted


def draft_ids(wl: Workload, planted: np.ndarray | None, rep: int = 0, n_draft: int | None = None):
    """int32 [n_draft]. Uniform on [0, V) without a planted target; otherwise an agreeing prefix
    of length L with P(L >= i) = p^i (truncated at n_draft), then one id drawn uniformly from
    V minus the target id, then uniform ids. Returns (draft, L or None)."""
    n = wl.n_draft if n_draft is None else n_draft
    rng = np.random.default_rng([wl.seed, 3, rep])
    if planted is None:
        return rng.integers(0, wl.vocab, size=n, dtype=np.int64).astype(np.int32), None
    L = 0
    while L < n and rng.random() < wl.accept_p:
        L += 1
    d = rng.integers(0, wl.vocab, size=n, dtype=np.int64)
    d[:L] = planted[:L]
    if L < n:
        other = rng.integers(0, wl.vocab - 1)
        d[L] = other + (other >= planted[L])
    return d.astype(np.int32), L
