#!/usr/bin/env python3
"""Benchmark of the MoE verify-block hot path on one MI355X.

One step = one MoE layer over a verify block of k = 16 tokens (H 2048, 256 experts, top-8, SwiGLU
I 512, one shared expert I 512, bf16 weights, fp32 router) followed by greedy acceptance over
17 x 151936 fp32 target logits: every kernel of the path, through the C ABI.

Inputs are resident in HBM before timing. The 256 MB last-level cache would hold a decode step's
experts, so steps rotate over several byte-identical copies of the layer weights and over a pool
of distinct blocks (distinct routings); every step streams its woken experts from HBM.

Reported (one JSON line): achieved HBM GB/s of the whole step from algorithmic bytes
(woken experts once each + shared expert + router + block in/out + logits), ms per step, the
gate/up kernel's roofline (per-kernel HIP events recorded by the library on the launch stream),
k and sigma sweeps, and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE verify-block latency (ms) and achieved HBM GB/s vs k=1..16, 1 GPU"
HBM_PEAK_GBPS = 8000.0
GATEUP_SRC = os.path.join(ROOT, "speculative_decoding_moe_amd", "csrc", "moe_verify.hip")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "k_layer_verify_k16_bf16_traffic.txt")
HEAD_PMC_SUMMARY = os.path.join(ROOT, "profiles", "k_head_v151936_h2048_traffic.txt")


class HipEvents:
    """hipEvent_t handles through the HIP runtime (events land on the library's launch stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def record(self, e, stream):
        if self.hip.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        self.hip.hipEventSynchronize(b)
        v = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(v), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(v.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def layer_bytes(shape, U, k):
    """Algorithmic HBM bytes of one MoE layer call: woken experts once, shared expert, router,
    block in and out."""
    H, I, Is, E = shape.hidden, shape.inter, shape.shared_inter, shape.n_experts
    per_expert = 3 * H * I * 2 if shape.wdtype == "bf16" else 3 * H * I * (0.5 + 1.0 / 32.0)
    return U * per_expert + 3 * H * Is * 2 + E * H * 4 + 2 * k * H * 4


def gateup_bytes(shape, U):
    """Algorithmic bytes of the gate/up kernel: gate and up rows of the woken experts and the
    shared expert (bf16)."""
    H, I, Is = shape.hidden, shape.inter, shape.shared_inter
    if shape.wdtype == "bf16":
        return (U * 2 * H * I + 2 * H * Is) * 2
    return U * 2 * H * I * (0.5 + 1.0 / 32.0) + 2 * H * Is * 2


def down_bytes(shape, U):
    """Algorithmic bytes of the down kernel: down rows of the woken experts and the shared expert
    (bf16)."""
    H, I, Is = shape.hidden, shape.inter, shape.shared_inter
    per_expert = H * I * 2 if shape.wdtype == "bf16" else H * I * (0.5 + 1.0 / 32.0)
    return U * per_expert + H * Is * 2


def expert_bytes(shape, U):
    """Algorithmic bytes of the one-launch layer kernel (gate/up, down and combine phases): every
    woken expert's gate, up and down weights once, and the shared expert's."""
    return gateup_bytes(shape, U) + down_bytes(shape, U)


def traffic_from_profile(summary=None):
    """HBM bytes per launch from a committed rocprofv3 counter summary (the gate/up one by default),
    or None when the summary is missing or was taken on different kernel source."""
    summary = PMC_SUMMARY if summary is None else summary
    if not os.path.exists(summary):
        return None
    src_hash = hashlib.sha256(open(GATEUP_SRC, "rb").read()).hexdigest()
    fields = {}
    for line in open(summary):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != src_hash:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, n_samples, one_core_samples=3):
    """The oracle as it stands, timed on the host for a bounded sample of the same steps (median of
    the steps' rates), with the BLAS thread pool as configured and with one thread."""
    import numpy as np

    import oracle
    from speculative_decoding_moe_amd.workloads import gen

    class CachedLayer:  # raw encoded weights pre-generated, so timing covers only the oracle
        def __init__(self):
            self.cache = {}

        def router(self):
            if "r" not in self.cache:
                self.cache["r"] = gen.router_weight(wl, 0)
            return self.cache["r"]

        def expert(self, e):
            if e not in self.cache:
                self.cache[e] = gen.expert_tensors(wl, 0, int(e))
            return self.cache[e]

        def shared(self):
            if "s" not in self.cache:
                self.cache["s"] = gen.shared_tensors(wl, 0)
            return self.cache["s"]

    layer = CachedLayer()

    def run(n):
        times, rates = [], []
        for p in range(n):
            x = gen.hidden_states(wl, rep=p)
            logits, planted = gen.target_logits(wl, rep=p)
            draft, _ = gen.draft_ids(wl, planted, rep=p)
            oracle.moe_block(x, layer, wl.shape.top_k)  # untimed pass: generates the woken experts
            t0 = time.perf_counter()
            r = oracle.moe_block(x, layer, wl.shape.top_k)
            tg = oracle.argmax_first(logits)
            oracle.accept_length(draft, tg)
            t = time.perf_counter() - t0
            times.append(t)
            rates.append((layer_bytes(wl.shape, r["n_woken"], wl.k) + logits.nbytes) / t / 1e9)
        return float(np.median(times)), float(np.median(rates))

    t_all, v_all = run(n_samples)
    threads = 1
    t_one = v_one = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        with threadpool_limits(limits=1):
            t_one, v_one = run(one_core_samples)
    except Exception:
        pass
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(v_all, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"median of {n_samples} verify steps (k=16 MoE layer + acceptance over 17x151936 logits), "
                      f"{t_all:.3f} s per step on the host, {threads} BLAS threads; host has {os.cpu_count()} CPUs "
                      f"({cpu_model})",
            "value_1core": round(v_one, 4) if v_one else None,
            "sample_1core": f"median of {one_core_samples} steps with one BLAS thread, "
                            f"{t_one:.3f} s per step" if t_one else None}


def cpu_stack_sample(n_layers_timed, NT, V):
    """The oracle on the 40-layer mxfp4 stack + acceptance: a bounded sample of its first layers
    (each timed call decodes its woken experts' fp4 codes itself), scaled to the stack's 40 layers,
    plus the acceptance over NT x V logits."""
    import numpy as np

    import oracle
    from speculative_decoding_moe_amd.workloads import gen
    sw = gen.WORKLOADS["stack40_mxfp4"]

    class RawLayer:  # the layer's raw encoded weights, generated before the timed call
        def __init__(self, li, woken):
            self.r = gen.router_weight(sw, li)
            self.sh = gen.shared_tensors(sw, li)
            self.ex = {int(e): gen.expert_tensors(sw, li, int(e)) for e in woken}

        def router(self):
            return self.r

        def expert(self, e):
            return self.ex[int(e)]

        def shared(self):
            return self.sh

    x = gen.hidden_states(sw).astype(np.float64)
    per_layer = []
    for li in range(n_layers_timed):
        logits = oracle.router_logits(oracle.rms_norm(x, sw.rms_eps), gen.router_weight(sw, li))
        woken = {int(e) for t in range(x.shape[0]) for e in oracle.select_topk(logits[t], sw.shape.top_k)}
        layer = RawLayer(li, woken)
        t0 = time.perf_counter()
        r = oracle.moe_block(x, layer, sw.shape.top_k, pre_norm=True, residual=True, rms_eps=sw.rms_eps)
        per_layer.append(time.perf_counter() - t0)
        x = r["y"]
    alog, _ = gen.target_logits(gen.WORKLOADS["verify"], rep=0)
    t0 = time.perf_counter()
    oracle.argmax_first(alog)
    t_acc = time.perf_counter() - t0
    med = float(np.median(per_layer))
    return {"ms_stack_plus_accept": round((med * sw.n_layers + t_acc) * 1e3, 1), "cores": os.cpu_count(),
            "sample": f"first {n_layers_timed} of the {sw.n_layers} mxfp4 layers timed (median {med * 1e3:.0f} ms "
                      f"per layer, woken experts' codes decoded inside), scaled to {sw.n_layers} layers, plus the "
                      f"acceptance over {NT}x{V} logits ({t_acc * 1e3:.1f} ms)"}


def context(sweep_k, value):
    """The pages' own numbers for this path (other hardware and real prompts: context, not
    targets), beside the same quantities measured here."""
    out = {"note": "pages' figures were measured on a Strix Halo APU with real prompts; ours on MI355X, "
                   "synthetic random routing; context only"}
    if sweep_k:
        k1, k16 = sweep_k[0], sweep_k[-1]
        out["verify16_over_decode"] = {"ours": round(k16["ms"] / k1["ms"], 2),
                                       "pages_pytorch_bf16": 1.6, "pages_llamacpp_q8": [4.2, 4.7]}
        out["woken_experts_k16"] = {"ours": k16["U_mean"], "pages_real_text": [47, 52],
                                    "pages_repeated_token": 31, "decode": 8}
    out["effective_GBps"] = {"ours_step": value, "pages_pytorch_bf16_decode": 47, "pages_llamacpp_q8_decode": 147}
    return out


def fit_line(points):
    """Least squares t = t0 + B / BW over (bytes, seconds) points: t0 in us, BW in GB/s, and the
    residuals in us."""
    import numpy as np
    B = np.array([p[0] for p in points], dtype=np.float64)
    t = np.array([p[1] for p in points], dtype=np.float64)
    A = np.stack([np.ones_like(B), B], axis=1)
    (t0, inv_bw), *_ = np.linalg.lstsq(A, t, rcond=None)
    res = t - (t0 + inv_bw * B)
    return {"t0_us": round(t0 * 1e6, 2), "bw_GBps": round(1.0 / inv_bw / 1e9, 1) if inv_bw > 0 else None,
            "residual_us": [round(r * 1e6, 2) for r in res]}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated to defeat the LLC")
    ap.add_argument("--pool", type=int, default=16, help="distinct blocks cycled through")
    ap.add_argument("--cpu-samples", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the 40-layer mxfp4 stack measurement")
    ap.add_argument("--no-head", action="store_true", help="skip the output-head (lm_head_accept) measurement")
    ap.add_argument("--no-sample", action="store_true", help="skip the accept_sample / statistics measurement")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the many-sequence (gathered path) measurement")
    ap.add_argument("--batched-tokens", type=int, default=0,
                    help="measure the gathered path at this token count only (for profiling)")
    ap.add_argument("--profile-run", nargs="?", const="k16", default=None,
                    choices=["k16", "k1", "k4", "k8", "sigma0", "sigma0.3"],
                    help="counter-collection run of one layer configuration (k16: the benchmark step, plus "
                         "the output head, the gathered path and the stack's mxfp4 layer; k1/k4/k8: the k "
                         "sweep's blocks; sigma0/sigma0.3: correlated k = 16 blocks): warmup + steps without "
                         "events, then a plain copy of known size for calibrating HBM traffic counters; "
                         "prints one JSON line")
    ap.add_argument("--cpu-stack-layers", type=int, default=1,
                    help="layers of the 40-layer mxfp4 stack the CPU oracle times (scaled to 40)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the verify block is a single-GPU path here; "
              "run with --gpus 1 (sharding is described, not built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from speculative_decoding_moe_amd import binding
    from speculative_decoding_moe_amd.workloads import device, gen

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    wl = gen.WORKLOADS["verify"]
    s = wl.shape
    k, K, V, NT = wl.k, s.top_k, wl.vocab, wl.n_target
    R, P = max(1, args.copies), max(1, args.pool)

    print(f"[bench] filling {R} weight copies of the layer", file=sys.stderr, flush=True)
    base = device.layer_tensors(wl, 0, dev)
    copies = [base] + [{n: (t.clone() if t is not None else None) for n, t in base.items()} for _ in range(R - 1)]
    layers = [device.make_layer(wl, 0, dev, tensors=c) for c in copies]
    del copies, base

    print(f"[bench] preparing {P} blocks and logits", file=sys.stderr, flush=True)
    xs, lgs, drs = [], [], []
    for p in range(P):
        xs.append(torch.from_numpy(gen.hidden_states(wl, rep=p)).to(dev))
        logits, planted = gen.target_logits(wl, rep=p)
        draft, _ = gen.draft_ids(wl, planted, rep=p)
        lgs.append(torch.from_numpy(logits).to(dev))
        drs.append(torch.from_numpy(draft).to(dev))
    y = torch.empty((k, s.hidden), dtype=torch.float32, device=dev)
    ids = torch.empty((k, K), dtype=torch.int32, device=dev)
    w = torch.empty((k, K), dtype=torch.float32, device=dev)
    nsteps = args.steps
    nw_all = torch.zeros((max(nsteps, args.warmup) + 1, 4), dtype=torch.int32, device=dev)
    ws = torch.empty(layers[0].workspace_size(16), dtype=torch.uint8, device=dev)
    tgt = torch.empty((NT,), dtype=torch.int32, device=dev)
    acc = torch.empty((4,), dtype=torch.int32, device=dev)
    aws = torch.empty(binding.accept_prefix_workspace_size(NT, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    ev = HipEvents()

    def step(i, timed_events=None):
        L = layers[i % R]
        p = i % P
        if timed_events is None:
            binding.moe_verify_block(L, xs[p], 0, y, ids, w, nw_all[i], ws)
        else:
            binding.moe_verify_block_timed(L, xs[p], 0, y, timed_events[:5], ids, w, nw_all[i], ws)
        binding.accept_prefix(lgs[p], drs[p], tgt, acc, aws)
        if timed_events is not None:
            ev.record(timed_events[5], stream)

    if args.profile_run in (None, "k16"):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()

    if args.profile_run:
        cfg = args.profile_run
        if cfg != "k16":  # one configuration of the sweeps, layer calls only (warm-up included)
            if cfg.startswith("sigma"):
                cw = gen.WORKLOADS["correlated"]
                blocks = [torch.from_numpy(gen.hidden_states(cw, rep=300 + p, sigma=float(cfg[5:]))).to(dev)
                          for p in range(4)]
            else:
                blocks = [torch.from_numpy(gen.hidden_states(wl, rep=200 + p, k=int(cfg[1:]))).to(dev)
                          for p in range(4)]
            kk = blocks[0].shape[0]
            pnw = torch.zeros((nsteps + args.warmup + 1, 4), dtype=torch.int32, device=dev)
            for i in range(nsteps + args.warmup):
                binding.moe_verify_block(layers[i % R], blocks[i % 4], 0, y[:kk], ids[:kk], w[:kk], pnw[i], ws)
            torch.cuda.synchronize()
            pU = pnw[:nsteps + args.warmup, 0].cpu().numpy().astype(np.int64)
            layer_b = {"layer_bytes_mean": float(np.mean([expert_bytes(s, u) for u in pU]))}
        else:
            for i in range(nsteps):
                step(i)
            torch.cuda.synchronize()
            Uall = nw_all[:max(nsteps, args.warmup), 0].cpu().numpy().astype(np.int64)
        if cfg == "k16":
            # the output head: 4 calls on 2 packed copies
            hw = gen.Workload("head", s, k=16, seed=wl.seed, vocab=V, n_target=16)
            w_rm = device.head_tensor(hw, dev)
            heads = [binding.pack_head(w_rm) for _ in range(2)]
            del w_rm
            hh = torch.from_numpy(gen.hidden_states(hw, rep=0, k=16)).to(dev)
            htg = torch.empty((16,), dtype=torch.int32, device=dev)
            hac = torch.empty((4,), dtype=torch.int32, device=dev)
            hws = torch.empty(binding.lm_head_accept_workspace_size(16, s.hidden, V), dtype=torch.uint8, device=dev)
            for r in range(4):
                binding.lm_head_accept(hh, heads[r % 2], V, drs[0][:15].contiguous(), htg, hac, hws)
            torch.cuda.synchronize()
            del heads
            # the gathered path: 4 calls of 512 tokens (32 sequences x 16) on the rotating copies
            bt = 512
            bx = torch.from_numpy(gen.hidden_states(gen.WORKLOADS["batched"], rep=400, k=bt)).to(dev)
            bws = torch.empty(layers[0].workspace_size(bt), dtype=torch.uint8, device=dev)
            by = torch.empty((bt, s.hidden), dtype=torch.float32, device=dev)
            bnw = torch.zeros((4, 4), dtype=torch.int32, device=dev)
            for r in range(4):
                binding.moe_verify_block(layers[r % R], bx, 0, by, None, None, bnw[r], bws)
            torch.cuda.synchronize()
            bU = bnw[:, 0].cpu().numpy().astype(np.int64)
            del bws, by
            # the 40-layer stack's mxfp4 layer: 4 generated layers, each called twice
            mw = gen.WORKLOADS["stack40_mxfp4"]
            mlayers = [device.make_layer(mw, li, dev) for li in range(4)]
            mws = torch.empty(mlayers[0].workspace_size(mw.k), dtype=torch.uint8, device=dev)
            mbuf = [torch.empty((mw.k, s.hidden), dtype=torch.float32, device=dev) for _ in range(2)]
            mnw = torch.zeros((8, 4), dtype=torch.int32, device=dev)
            for r in range(8):
                mx_in = torch.from_numpy(gen.hidden_states(mw, rep=r)).to(dev)
                binding.moe_verify_block(mlayers[r % 4], mx_in, binding.MOE_PRE_RMSNORM | binding.MOE_RESIDUAL,
                                         mbuf[r % 2], None, None, mnw[r], mws)
            torch.cuda.synchronize()
            mU = mnw[:, 0].cpu().numpy().astype(np.int64)
            del mws, mbuf
            # the gathered path on that mxfp4 layer: 4 calls of 512 tokens
            mbws = torch.empty(mlayers[0].workspace_size(bt), dtype=torch.uint8, device=dev)
            mby = torch.empty((bt, s.hidden), dtype=torch.float32, device=dev)
            mbnw = torch.zeros((4, 4), dtype=torch.int32, device=dev)
            for r in range(4):
                binding.moe_verify_block(mlayers[r % 4], bx, binding.MOE_PRE_RMSNORM | binding.MOE_RESIDUAL, mby,
                                         None, None, mbnw[r], mbws)
            torch.cuda.synchronize()
            mbU = mbnw[:, 0].cpu().numpy().astype(np.int64)
            del mlayers, mbws, mby
            layer_b = {"layer_bytes_mean": float(np.mean([expert_bytes(s, u) for u in Uall])),
                       "step_bytes_mean": float(np.mean([layer_bytes(s, u, k) for u in Uall])),
                       "head_bytes": (V + 15) // 16 * 16 * s.hidden * 2 + 16 * s.hidden * 4,
                       "bexp_gateup_bytes": float(np.mean([gateup_bytes(s, u) for u in bU])),
                       "bexp_down_bytes": float(np.mean([gateup_bytes(s, u) / 2 for u in bU])),
                       "mx_layer_bytes_mean": float(np.mean([expert_bytes(mw.shape, u) for u in mU])),
                       "mx_bexp_gateup_bytes": float(np.mean([gateup_bytes(mw.shape, u) for u in mbU])),
                       "mx_bexp_down_bytes": float(np.mean([down_bytes(mw.shape, u) for u in mbU])),
                       "accept_bytes": NT * V * 4}
        copy_mib = 512
        src = torch.empty(copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            device.copy_bytes(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": cfg, "launches": int(nsteps), **layer_b, "copy_bytes": copy_mib << 20,
                          "copy_launches": 3}), flush=True)
        return

    # ---- headline: K whole steps bracketed by synchronisations ----
    t_start, t_stop = ev.create(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev.record(t_start, stream)
    for i in range(nsteps):
        step(i)
    ev.record(t_stop, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev.ms(t_start, t_stop)
    ev.destroy([t_start, t_stop])
    U = nw_all[:nsteps, 0].cpu().numpy().astype(np.int64)
    step_bytes = np.array([layer_bytes(s, u, k) + NT * V * 4 for u in U], dtype=np.float64)
    ms_per_step = total_ms / nsteps
    value = float(step_bytes.sum() / (total_ms * 1e-3) / 1e9)

    # ---- step-time distribution: one event between consecutive steps ----
    marks = ev.create(nsteps + 1)
    torch.cuda.synchronize()
    for i in range(nsteps):
        ev.record(marks[i], stream)
        step(i)
    ev.record(marks[nsteps], stream)
    torch.cuda.synchronize()
    per_step_us = np.array([ev.ms(marks[i], marks[i + 1]) * 1e3 for i in range(nsteps)])
    ev.destroy(marks)
    dist = {"p10_us": round(float(np.percentile(per_step_us, 10)), 2),
            "p50_us": round(float(np.median(per_step_us)), 2),
            "p90_us": round(float(np.percentile(per_step_us, 90)), 2)}

    # ---- per-kernel pass: the library records events at its kernel boundaries ----
    evs = [ev.create(6) for _ in range(nsteps)]
    for i in range(nsteps):
        step(i, evs[i])
    torch.cuda.synchronize()
    U2 = nw_all[:nsteps, 0].cpu().numpy().astype(np.int64)
    # events: [0] before the router kernel, [1] after it, [2] = [3] = [4] after the one-launch
    # layer kernel (gate/up, down, combine), [5] after the acceptance; the layer kernel is timed
    # to the first event after it (each further record adds its own time)
    spans = {"router": (0, 1), "experts": (1, 2), "accept": (4, 5)}
    dur = {n: [] for n in spans}
    for i in range(nsteps):
        e = evs[i]
        for n, (j0, j1) in spans.items():
            dur[n].append(ev.ms(e[j0], e[j1]))
        ev.destroy(e)
    lay_ms = float(np.mean(dur["experts"]))
    lay_bytes = float(np.mean([expert_bytes(s, u) for u in U2]))
    achieved = lay_bytes / (lay_ms * 1e-3) / 1e9
    kernels_us = {n: round(float(np.mean(v)) * 1e3, 2) for n, v in dur.items()}

    # ---- achievable streaming read (reference kernel, 2 GiB so the LLC cannot hold it) ----
    rd = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(2):
        device.stream_read(rd, sink)
    a_, b_ = ev.create(2)
    rd_times = []
    for _ in range(5):
        ev.record(a_, stream)
        device.stream_read(rd, sink)
        ev.record(b_, stream)
        torch.cuda.synchronize()
        rd_times.append(ev.ms(a_, b_))
    ev.destroy([a_, b_])
    read_ceiling = float(rd.numel() / (np.median(rd_times) * 1e-3) / 1e9)
    del rd

    roofline = {"bound": "hbm", "kernel": "k_layer (gate/up, down and combine phases of the layer)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_from_profile(),
                "bytes_per_launch": round(lay_bytes), "avg_launch_us": round(lay_ms * 1e3, 2),
                "achievable_read_GBps": round(read_ceiling, 1),
                "frac_of_achievable": round(achieved / read_ceiling, 4),
                "expert_kernels_GBps": round(achieved, 1)}

    # ---- sweeps (same layer; k = 1..16 and correlated blocks at k = 16) ----
    sweep_k, sweep_sigma, fit = [], [], None
    if not args.no_sweep:
        reps = 20

        def time_blocks(blocks):
            nw = torch.zeros((len(blocks) * reps + 1, 4), dtype=torch.int32, device=dev)
            kb = blocks[0].shape[0]
            for i in range(5):
                binding.moe_verify_block(layers[i % R], blocks[i % len(blocks)], 0, y[:kb], ids[:kb], w[:kb], nw[0],
                                         ws)
            a, b = ev.create(2)
            torch.cuda.synchronize()
            ev.record(a, stream)
            n = len(blocks) * reps
            for i in range(n):
                xb = blocks[i % len(blocks)]
                binding.moe_verify_block(layers[i % R], xb, 0, y[:xb.shape[0]], ids[:xb.shape[0]],
                                         w[:xb.shape[0]], nw[i], ws)
            ev.record(b, stream)
            torch.cuda.synchronize()
            t = ev.ms(a, b) / n
            ev.destroy([a, b])
            Us = nw[:n, 0].cpu().numpy()
            byt = float(np.mean([layer_bytes(s, u, blocks[0].shape[0]) for u in Us]))
            return t, float(Us.mean()), byt

        points = []
        for kk in range(1, 17):
            blocks = [torch.from_numpy(gen.hidden_states(wl, rep=200 + p, k=kk)).to(dev) for p in range(4)]
            t, Um, byt = time_blocks(blocks)
            points.append((byt, t * 1e-3))
            sweep_k.append({"k": kk, "U_mean": round(Um, 2), "ms": round(t, 4),
                            "GBps": round(byt / (t * 1e-3) / 1e9, 1)})
        cw = gen.WORKLOADS["correlated"]
        for sg in cw.sigmas:
            blocks = [torch.from_numpy(gen.hidden_states(cw, rep=300 + p, sigma=sg)).to(dev) for p in range(4)]
            t, Um, byt = time_blocks(blocks)
            points.append((byt, t * 1e-3))
            sweep_sigma.append({"sigma": sg, "U_mean": round(Um, 2), "ms": round(t, 4),
                                "GBps": round(byt / (t * 1e-3) / 1e9, 1)})
        fit = fit_line(points)
        fit["points"] = "16 k-sweep points then 5 sigma points (k = 16), layer calls only"
        fit["same_U_check_ms"] = {"k1_U8": sweep_k[0]["ms"], "k16_sigma0_U8": sweep_sigma[0]["ms"]}
        print("[bench] sweeps done", file=sys.stderr, flush=True)

    # ---- many sequences verified together: the gathered path at 4..64 sequences x 16 tokens ----
    batched = None
    if not args.no_batched:
        print("[bench] timing the gathered path", file=sys.stderr, flush=True)
        bw_ = gen.WORKLOADS["batched"]
        tmax = 1024
        bws = torch.empty(layers[0].workspace_size(tmax), dtype=torch.uint8, device=dev)
        by = torch.empty((tmax, s.hidden), dtype=torch.float32, device=dev)
        bids = torch.empty((tmax, K), dtype=torch.int32, device=dev)
        bwt = torch.empty((tmax, K), dtype=torch.float32, device=dev)
        rows = []
        for T in ((args.batched_tokens,) if args.batched_tokens else (64, 128, 256, 512, 1024)):
            blocks = [torch.from_numpy(gen.hidden_states(bw_, rep=400 + p, k=T)).to(dev) for p in range(2)]
            reps = 8
            nw = torch.zeros((reps + 1, 4), dtype=torch.int32, device=dev)
            evs = ev.create(5 * reps)
            for i in range(3):
                binding.moe_verify_block(layers[i % R], blocks[i % 2], 0, by[:T], bids[:T], bwt[:T], nw[reps], bws)
            torch.cuda.synchronize()
            for i in range(reps):
                binding.moe_verify_block_timed(layers[i % R], blocks[i % 2], 0, by[:T], evs[5 * i:5 * i + 5],
                                               bids[:T], bwt[:T], nw[i], bws)
            torch.cuda.synchronize()
            seg = np.array([[ev.ms(evs[5 * i + j], evs[5 * i + j + 1]) for j in range(4)] for i in range(reps)])
            tot = np.array([ev.ms(evs[5 * i], evs[5 * i + 4]) for i in range(reps)])
            ev.destroy(evs)
            Us = nw[:reps, 0].cpu().numpy().astype(np.float64)
            Um = float(Us.mean())
            t_ms = float(tot.mean())
            byt = float(np.mean([layer_bytes(s, u, T) for u in Us]))
            gub = float(np.mean([gateup_bytes(s, u) for u in Us]))
            dnb = gub / 2
            flops = 2.0 * 3 * s.hidden * s.inter * T * K + 2.0 * 3 * s.hidden * s.shared_inter * T
            sm = seg.mean(axis=0)
            rows.append({"tokens": T, "sequences": T // 16, "U_mean": round(Um, 2), "ms": round(t_ms, 4),
                         "tokens_per_s": round(T / (t_ms * 1e-3)), "GBps": round(byt / (t_ms * 1e-3) / 1e9, 1),
                         "expert_TFLOPs": round(flops / (t_ms * 1e-3) / 1e12, 1),
                         "kernels_us": {"route": round(sm[0] * 1e3, 2), "gateup": round(sm[1] * 1e3, 2),
                                        "down": round(sm[2] * 1e3, 2), "combine": round(sm[3] * 1e3, 2)},
                         "gateup_GBps": round(gub / (sm[1] * 1e-3) / 1e9, 1),
                         "down_GBps": round(dnb / (sm[2] * 1e-3) / 1e9, 1)})
            del blocks
        # the same over the 40-layer stack's mxfp4 layer (pre-norm, residual): 4 rotating copies
        mw = gen.WORKLOADS["stack40_mxfp4"]
        mbase = device.layer_tensors(mw, 0, dev)
        mlayers = [device.make_layer(mw, 0, dev, tensors=mbase)] + [
            device.make_layer(mw, 0, dev, tensors={n: (t.clone() if t is not None else None) for n, t in mbase.items()})
            for _ in range(3)]
        del mbase
        mws = torch.empty(mlayers[0].workspace_size(tmax), dtype=torch.uint8, device=dev)
        mrows = []
        for T in ((args.batched_tokens,) if args.batched_tokens else (64, 256, 512, 1024)):
            blocks = [torch.from_numpy(gen.hidden_states(mw, rep=400 + p, k=T)).to(dev) for p in range(2)]
            reps = 8
            nw = torch.zeros((reps + 1, 4), dtype=torch.int32, device=dev)
            evs = ev.create(5 * reps)
            for i in range(3):
                binding.moe_verify_block(mlayers[i % 4], blocks[i % 2], 3, by[:T], bids[:T], bwt[:T], nw[reps], mws)
            torch.cuda.synchronize()
            for i in range(reps):
                binding.moe_verify_block_timed(mlayers[i % 4], blocks[i % 2], 3, by[:T], evs[5 * i:5 * i + 5],
                                               bids[:T], bwt[:T], nw[i], mws)
            torch.cuda.synchronize()
            seg = np.array([[ev.ms(evs[5 * i + j], evs[5 * i + j + 1]) for j in range(4)] for i in range(reps)])
            tot = np.array([ev.ms(evs[5 * i], evs[5 * i + 4]) for i in range(reps)])
            ev.destroy(evs)
            Us = nw[:reps, 0].cpu().numpy().astype(np.float64)
            t_ms = float(tot.mean())
            byt = float(np.mean([layer_bytes(mw.shape, u, T) for u in Us]))
            sm = seg.mean(axis=0)
            mrows.append({"tokens": T, "sequences": T // 16, "U_mean": round(float(Us.mean()), 2), "ms": round(t_ms, 4),
                          "tokens_per_s": round(T / (t_ms * 1e-3)), "GBps": round(byt / (t_ms * 1e-3) / 1e9, 1),
                          "kernels_us": {"route": round(sm[0] * 1e3, 2), "gateup": round(sm[1] * 1e3, 2),
                                         "down": round(sm[2] * 1e3, 2), "combine": round(sm[3] * 1e3, 2)}})
            del blocks
        del mlayers, mws
        # greedy acceptance of 32 sequences at once: 32 x 17 rows x V logits
        ns = 32
        blg = torch.randn((ns, NT, V), device=dev, generator=torch.Generator(device=dev).manual_seed(wl.seed))
        bdr = torch.randint(0, V, (ns, NT - 1), dtype=torch.int32, device=dev)
        btg = torch.empty((ns, NT), dtype=torch.int32, device=dev)
        bac = torch.empty((ns,), dtype=torch.int32, device=dev)
        baws = torch.empty(binding.accept_prefix_batch_workspace_size(ns, NT, V), dtype=torch.uint8, device=dev)
        for _ in range(3):
            binding.accept_prefix_batch(blg, bdr, btg, bac, baws)
        a_, b_ = ev.create(2)
        torch.cuda.synchronize()
        ev.record(a_, stream)
        for _ in range(20):
            binding.accept_prefix_batch(blg, bdr, btg, bac, baws)
        ev.record(b_, stream)
        torch.cuda.synchronize()
        acc_us = ev.ms(a_, b_) * 1e3 / 20
        ev.destroy([a_, b_])
        accept_batch = {"workload": f"accept_prefix_batch: {ns} sequences x {NT} rows x {V} fp32 logits",
                        "us_per_call": round(acc_us, 2),
                        "GBps": round(ns * NT * V * 4 / (acc_us * 1e-6) / 1e9, 1)}
        # acceptance at temperature of the same 32 sequences (a drafter 0.5 N(0,1) away, T = 1)
        gq = torch.Generator(device=dev).manual_seed(wl.seed + 1)
        bdl = (blg[:, :NT - 1] + 0.5 * torch.randn((ns, NT - 1, V), device=dev, generator=gq)).contiguous()
        bua = torch.rand((ns, NT - 1), device=dev, generator=gq)
        bus = torch.rand((ns, NT), device=dev, generator=gq)
        btk = torch.empty((ns,), dtype=torch.int32, device=dev)
        bsws = torch.empty(binding.accept_sample_batch_workspace_size(ns, NT, NT - 1, V), dtype=torch.uint8,
                           device=dev)
        for _ in range(3):
            binding.accept_sample_batch(blg, bdl, bdr, 1.0, bua, bus, bac, btk, bsws)
        a_, b_ = ev.create(2)
        torch.cuda.synchronize()
        ev.record(a_, stream)
        for _ in range(20):
            binding.accept_sample_batch(blg, bdl, bdr, 1.0, bua, bus, bac, btk, bsws)
        ev.record(b_, stream)
        torch.cuda.synchronize()
        smp_us = ev.ms(a_, b_) * 1e3 / 20
        ev.destroy([a_, b_])
        accept_batch_sample = {"workload": f"accept_sample_batch: {ns} sequences x ({NT} target + {NT - 1} draft) "
                                           f"rows x {V} fp32 logits, T = 1",
                               "us_per_call": round(smp_us, 2),
                               "GBps": round(ns * (2 * NT - 1) * V * 4 / (smp_us * 1e-6) / 1e9, 1)}
        del blg, bdl
        batched = {"workload": "gathered path: 4..64 sequences x 16 independent N(0,1) tokens through the k = 16 "
                               "layer (bf16); event times per call, route = router + top-K + permutation",
                   "accept_32_sequences": accept_batch,
                   "accept_sample_32_sequences": accept_batch_sample,
                   "points": rows,
                   "points_mxfp4": {"workload": "the 40-layer stack's mxfp4 layer (pre-norm, residual, bf16 shared "
                                                "expert) over 4..64 sequences x 16 tokens", "points": mrows},
                   "single_block_k16_ms": sweep_k[-1]["ms"] if sweep_k else None}
        del bws, by
        print("[bench] gathered path done", file=sys.stderr, flush=True)

    # ---- 40-layer mxfp4 stack: one verify pass (pre-norm, residual) + acceptance ----
    stack = None
    if not args.no_stack:
        del layers
        torch.cuda.empty_cache()
        sw = gen.WORKLOADS["stack40_mxfp4"]
        print(f"[bench] filling the {sw.n_layers}-layer mxfp4 stack", file=sys.stderr, flush=True)
        slayers = [device.make_layer(sw, li, dev) for li in range(sw.n_layers)]
        sws = torch.empty(slayers[0].workspace_size(sw.k), dtype=torch.uint8, device=dev)
        bufs = [torch.empty((sw.k, sw.shape.hidden), dtype=torch.float32, device=dev) for _ in range(2)]
        snw = torch.zeros((sw.n_layers * 8, 4), dtype=torch.int32, device=dev)
        sxs = [torch.from_numpy(gen.hidden_states(sw, rep=p)).to(dev) for p in range(4)]
        flags = binding.MOE_PRE_RMSNORM | binding.MOE_RESIDUAL

        def stack_pass(rep, record=None):
            cur = sxs[rep % len(sxs)]
            for li, L in enumerate(slayers):
                out = bufs[li % 2]
                binding.moe_verify_block(L, cur, flags, out, None, None,
                                         snw[(rep % 8) * sw.n_layers + li], sws)
                cur = out
            binding.accept_prefix(lgs[rep % P], drs[rep % P], tgt, acc, aws)

        for r in range(2):
            stack_pass(r)
        a_, b_ = ev.create(2)
        torch.cuda.synchronize()
        sreps = 8
        ev.record(a_, stream)
        for r in range(sreps):
            stack_pass(r)
        ev.record(b_, stream)
        torch.cuda.synchronize()
        st_ms = ev.ms(a_, b_) / sreps
        ev.destroy([a_, b_])
        SU = snw[:sreps * sw.n_layers, 0].cpu().numpy().astype(np.int64)
        sbytes = float(np.sum([layer_bytes(sw.shape, u, sw.k) for u in SU]) / sreps) + NT * V * 4
        stack = {"workload": f"{sw.n_layers} x MoE layer (H {sw.shape.hidden}, 256 experts, top-8, I 512, "
                             "mxfp4 routed experts, bf16 shared, pre-norm + residual), k = 16, then acceptance",
                 "ms": round(st_ms, 4), "GBps": round(sbytes / (st_ms * 1e-3) / 1e9, 1),
                 "U_mean": round(float(SU.mean()), 2), "bytes_per_pass": round(sbytes),
                 "ms_per_layer": round(st_ms / sw.n_layers, 5)}
        print("[bench] stack done", file=sys.stderr, flush=True)

    # ---- output head with fused argmax + greedy acceptance (16 positions, 15 drafts) ----
    head = None
    if not args.no_head:
        print("[bench] filling the output head", file=sys.stderr, flush=True)
        hw = gen.Workload("head", s, k=16, seed=wl.seed, vocab=V, n_target=16)
        w_rm = device.head_tensor(hw, dev)
        heads = [binding.pack_head(w_rm) for _ in range(2)]  # 2 x 622 MB: no call finds it in the LLC
        del w_rm
        hhs = [torch.from_numpy(gen.hidden_states(hw, rep=p, k=16)).to(dev) for p in range(4)]
        hdr = drs[0][:15].contiguous()
        htg = torch.empty((16,), dtype=torch.int32, device=dev)
        hac = torch.empty((4,), dtype=torch.int32, device=dev)
        hws = torch.empty(binding.lm_head_accept_workspace_size(16, s.hidden, V), dtype=torch.uint8, device=dev)
        for r in range(5):
            binding.lm_head_accept(hhs[r % 4], heads[r % 2], V, hdr, htg, hac, hws)
        a_, b_ = ev.create(2)
        torch.cuda.synchronize()
        hreps = 40
        ev.record(a_, stream)
        for r in range(hreps):
            binding.lm_head_accept(hhs[r % 4], heads[r % 2], V, hdr, htg, hac, hws)
        ev.record(b_, stream)
        torch.cuda.synchronize()
        h_us = ev.ms(a_, b_) * 1e3 / hreps
        ev.destroy([a_, b_])
        hbytes = (V + 15) // 16 * 16 * s.hidden * 2 + 16 * s.hidden * 4
        head = {"workload": f"output head bf16 {V} x {s.hidden}, 16 positions, fused argmax + greedy acceptance "
                            "(lm_head_accept: head kernel + final reduction)",
                "us_per_call": round(h_us, 2), "bytes_per_call": hbytes,
                "GBps": round(hbytes / (h_us * 1e-6) / 1e9, 1),
                "frac_of_peak": round(hbytes / (h_us * 1e-6) / 1e9 / 8000.0, 4),
                "frac_of_achievable": (round(hbytes / (h_us * 1e-6) / 1e9 / roofline["achievable_read_GBps"], 4)
                                       if roofline.get("achievable_read_GBps") else None),
                "traffic": traffic_from_profile(HEAD_PMC_SUMMARY)}
        del heads
        print("[bench] head done", file=sys.stderr, flush=True)

    # ---- lossless acceptance at temperature + acceptance statistics (17 target, 16 draft rows) ----
    samp = None
    if not args.no_sample:
        print("[bench] timing accept_sample", file=sys.stderr, flush=True)
        g = torch.Generator(device=dev)
        g.manual_seed(wl.seed)
        nt_, nd_, temp = NT, NT - 1, 1.0
        # synthetic cycles: target logits 2 N(0,1), a drafter 0.5 N(0,1) away, drafts drawn from it
        tls = [torch.randn((nt_, V), generator=g, device=dev) * 2.0 for _ in range(4)]
        dls = [(t[:nd_] + 0.5 * torch.randn((nd_, V), generator=g, device=dev)).contiguous() for t in tls]
        dds = [torch.multinomial(torch.softmax(d / temp, dim=1), 1, generator=g).view(-1).to(torch.int32).contiguous()
               for d in dls]
        ncyc = 512
        uas = torch.rand((ncyc, nd_), generator=g, device=dev)
        uss = torch.rand((ncyc, nt_), generator=g, device=dev)
        sacc = torch.zeros((ncyc,), dtype=torch.int32, device=dev)
        stok = torch.zeros((ncyc,), dtype=torch.int32, device=dev)
        sws = torch.empty(binding.accept_sample_workspace_size(nt_, nd_, V), dtype=torch.uint8, device=dev)

        def scall(c):
            i = c % 4
            binding.accept_sample(tls[i], dls[i], dds[i], temp, uas[c], uss[c], sacc[c:c + 1], stok[c:c + 1], sws)

        for c in range(5):
            scall(c)
        a_, b_ = ev.create(2)
        torch.cuda.synchronize()
        ev.record(a_, stream)
        for c in range(ncyc):
            scall(c)
        ev.record(b_, stream)
        torch.cuda.synchronize()
        s_us = ev.ms(a_, b_) * 1e3 / ncyc
        ev.destroy([a_, b_])
        hist = torch.empty((nd_ + 1,), dtype=torch.int64, device=dev)
        surv = torch.empty((nd_,), dtype=torch.int64, device=dev)
        binding.accept_histogram(sacc, nd_, hist, surv)
        torch.cuda.synchronize()
        sbytes = (nt_ + nd_) * V * 4
        hh, sv = hist.cpu().numpy(), surv.cpu().numpy()
        samp = {"workload": f"accept_sample: {nt_} target + {nd_} draft rows x {V} fp32 logits, T = {temp}, "
                            f"synthetic drafter (target + 0.5 N(0,1) logits, drafts drawn from it), {ncyc} cycles",
                "us_per_call": round(s_us, 2), "bytes_per_call": sbytes,
                "GBps": round(sbytes / (s_us * 1e-6) / 1e9, 1),
                "tau_mean": round(float((np.arange(nd_ + 1) * hh).sum() / ncyc + 1.0), 3),
                "hist_accepted": [int(v) for v in hh],
                "marginal_accept": [round(float(v) / ncyc, 4) for v in sv]}
        print("[bench] sample done", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on {args.cpu_samples} steps", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_samples)
        if not args.no_stack and args.cpu_stack_layers > 0:
            print(f"[bench] timing the CPU oracle on {args.cpu_stack_layers} stack layers", file=sys.stderr, flush=True)
            cpu["stack40_mxfp4"] = cpu_stack_sample(args.cpu_stack_layers, NT, V)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": nsteps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "MoE verify block k=16 (H 2048, 256 experts, top-8, SwiGLU I 512 + shared "
                               "I 512, bf16 experts, fp32 router) + greedy acceptance over 17x151936 fp32 logits",
                   "k": k, "hidden": s.hidden, "n_experts": s.n_experts, "top_k": K, "inter": s.inter,
                   "shared_inter": s.shared_inter, "vocab": V, "n_target": NT, "weight_copies": R,
                   "block_pool": P, "U_mean": round(float(U.mean()), 2),
                   "bytes_per_step_mean": round(float(step_bytes.mean())), "wall_s": round(wall, 4)},
        "roofline": roofline,
        "step_time": dist,
        "kernels_us": kernels_us,
        "sweep_k": sweep_k,
        "sweep_sigma": sweep_sigma,
        "sweep_fit": fit,
        "batched": batched,
        "stack40_mxfp4": stack,
        "lm_head": head,
        "accept_sample": samp,
        "cpu_baseline": cpu,
        "context": context(sweep_k, value),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
