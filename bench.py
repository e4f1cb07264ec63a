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
PMC_SUMMARY = os.path.join(ROOT, "profiles", "k_gateup_verify_k16_bf16_traffic.txt")


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
    return (U * 2 * H * I + 2 * H * Is) * 2


def traffic_from_profile():
    """HBM bytes per gate/up launch from the committed rocprofv3 counter summary, or None when the
    summary is missing or was taken on different kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    src_hash = hashlib.sha256(open(GATEUP_SRC, "rb").read()).hexdigest()
    fields = {}
    for line in open(PMC_SUMMARY):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != src_hash:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, n_samples):
    """The oracle as it stands, timed on the host for a bounded sample of the same steps."""
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
    total_t, total_bytes = 0.0, 0.0
    for p in range(n_samples):
        x = gen.hidden_states(wl, rep=p)
        logits, planted = gen.target_logits(wl, rep=p)
        draft, _ = gen.draft_ids(wl, planted, rep=p)
        oracle.moe_block(x, layer, wl.shape.top_k)  # untimed pass: generates the woken experts
        t0 = time.perf_counter()
        r = oracle.moe_block(x, layer, wl.shape.top_k)
        tg = oracle.argmax_first(logits)
        oracle.accept_length(draft, tg)
        total_t += time.perf_counter() - t0
        total_bytes += layer_bytes(wl.shape, r["n_woken"], wl.k) + logits.nbytes
    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        pass
    return {"value": round(total_bytes / total_t / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_samples} verify steps (k=16 MoE layer + acceptance over 17x151936 logits), "
                      f"{total_t / n_samples:.2f} s per step on the host, host has {os.cpu_count()} CPUs"}


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
    ap.add_argument("--profile-run", action="store_true",
                    help="counter-collection run: warmup + steps without events, then a plain copy of "
                         "known size for calibrating HBM traffic counters; prints one JSON line")
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

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    if args.profile_run:
        for i in range(nsteps):
            step(i)
        torch.cuda.synchronize()
        Un = nw_all[:nsteps, 0].cpu().numpy().astype(np.int64)
        Uw = nw_all[:args.warmup, 0].cpu().numpy().astype(np.int64)
        Uall = np.concatenate([Uw, Un])
        copy_mib = 512
        src = torch.empty(copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            device.copy_bytes(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": True, "launches": int(len(Uall)),
                          "gateup_bytes_mean": float(np.mean([gateup_bytes(s, u) for u in Uall])),
                          "layer_bytes_mean": float(np.mean([layer_bytes(s, u, k) for u in Uall])),
                          "copy_bytes": copy_mib << 20, "copy_launches": 3}), flush=True)
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
    U = nw_all[:nsteps, 0].cpu().numpy().astype(np.int64)
    step_bytes = np.array([layer_bytes(s, u, k) + NT * V * 4 for u in U])
    ms_per_step = total_ms / nsteps
    value = float(step_bytes.sum() / (total_ms * 1e-3) / 1e9)

    # ---- per-kernel pass: the library records events at its kernel boundaries ----
    evs = [ev.create(6) for _ in range(nsteps)]
    for i in range(nsteps):
        step(i, evs[i])
    torch.cuda.synchronize()
    U2 = nw_all[:nsteps, 0].cpu().numpy().astype(np.int64)
    names = ["router", "gateup", "down", "combine", "accept"]
    dur = {n: [] for n in names}
    for i in range(nsteps):
        e = evs[i]
        for j, n in enumerate(names):
            dur[n].append(ev.ms(e[j], e[j + 1]))
        ev.destroy(e)
    gu_ms = float(np.mean(dur["gateup"]))
    gu_bytes = float(np.mean([gateup_bytes(s, u) for u in U2]))
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": "k_gateup", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic_from_profile(),
                "bytes_per_launch": round(gu_bytes), "avg_launch_us": round(gu_ms * 1e3, 2)}
    kernels_us = {n: round(float(np.mean(v)) * 1e3, 2) for n, v in dur.items()}

    # ---- sweeps (same layer; k = 1..16 and correlated blocks at k = 16) ----
    sweep_k, sweep_sigma = [], []
    if not args.no_sweep:
        reps = 20

        def time_blocks(blocks):
            nw = torch.zeros((len(blocks) * reps + 1, 4), dtype=torch.int32, device=dev)
            for i in range(5):
                binding.moe_verify_block(layers[i % R], blocks[i % len(blocks)], 0, y, ids, w, nw[0], ws)
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

        for kk in range(1, 17):
            blocks = [torch.from_numpy(gen.hidden_states(wl, rep=200 + p, k=kk)).to(dev) for p in range(4)]
            t, Um, byt = time_blocks(blocks)
            sweep_k.append({"k": kk, "U_mean": round(Um, 2), "ms": round(t, 4),
                            "GBps": round(byt / (t * 1e-3) / 1e9, 1)})
        cw = gen.WORKLOADS["correlated"]
        for sg in cw.sigmas:
            blocks = [torch.from_numpy(gen.hidden_states(cw, rep=300 + p, sigma=sg)).to(dev) for p in range(4)]
            t, Um, byt = time_blocks(blocks)
            sweep_sigma.append({"sigma": sg, "U_mean": round(Um, 2), "ms": round(t, 4),
                                "GBps": round(byt / (t * 1e-3) / 1e9, 1)})
        print(f"[bench] sweeps done", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on {args.cpu_samples} steps", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_samples)

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
        "kernels_us": kernels_us,
        "sweep_k": sweep_k,
        "sweep_sigma": sweep_sigma,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
