"""Calls from two host threads on two streams at once, through the C ABI. Each caller brings its
own workspace and outputs. The gathered layer path (bf16 and mxfp4), the batched greedy
acceptance and the output head with acceptance must then give, on every call, the bits the same
call gives alone on one stream. So the library keeps no hidden state between such calls, and its
host side may be entered from several threads. The single-block layer path is left out: its phases
need every workgroup of the launch resident, so the header asks callers to order those calls on
one stream. Run on an MI355X: ``pytest -m gpu``.
"""
import threading

import numpy as np
import pytest
import torch

from speculative_decoding_moe_amd.workloads import gen

pytestmark = pytest.mark.gpu

REPS = 6  # calls per thread, alternating two input sets


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    from speculative_decoding_moe_amd import binding
    return binding


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32).copy() if t.dtype == torch.float32 else t.cpu().numpy().copy()


class Caller:
    """One caller's inputs (two sets), workspaces and per-call outputs."""

    def __init__(self, B, layers, head, tag, k):
        self.B, self.layers, self.head = B, layers, head
        g = torch.Generator(device="cuda").manual_seed(9100 + tag)
        self.k = k
        H = layers[0].hidden
        self.x = []
        for v in range(2):
            wl = gen.Workload("streams", gen.LayerShape(H, 64, 4, 256, 256), k=k, seed=9200 + 10 * tag + v)
            self.x.append(torch.from_numpy(gen.hidden_states(wl, rep=v, k=k)).cuda())
        self.ws = [torch.empty(L.workspace_size(k), dtype=torch.uint8, device="cuda") for L in layers]
        self.S, self.NT, self.V = 4, 17, 20000
        self.lg = [torch.randn((self.S, self.NT, self.V), device="cuda", generator=g) for _ in range(2)]
        self.dr = torch.randint(0, self.V, (self.S, 16), device="cuda", generator=g, dtype=torch.int32)
        self.dr[:, :3] = self.lg[0][:, :3].argmax(dim=2).to(torch.int32)  # a few accepted drafts
        self.aws = torch.empty(self.B.accept_prefix_batch_workspace_size(self.S, self.NT, self.V), dtype=torch.uint8,
                               device="cuda")
        self.hV, self.hn = head[1], 9
        self.hh = [torch.randn((self.hn, H), device="cuda", generator=g) for _ in range(2)]
        self.hws = torch.empty(self.B.lm_head_accept_workspace_size(self.hn, H, self.hV), dtype=torch.uint8,
                               device="cuda")
        self.hdr = torch.randint(0, self.hV, (self.hn - 1,), device="cuda", generator=g, dtype=torch.int32)

    def outputs(self):
        """Zeroed outputs, so elements a call leaves alone compare equal too."""
        H, K = self.layers[0].hidden, self.layers[0].top_k
        o = {}
        for i in range(len(self.layers)):
            o[f"y{i}"] = torch.zeros((self.k, H), dtype=torch.float32, device="cuda")
            o[f"ids{i}"] = torch.zeros((self.k, K), dtype=torch.int32, device="cuda")
            o[f"w{i}"] = torch.zeros((self.k, K), dtype=torch.float32, device="cuda")
            o[f"nw{i}"] = torch.zeros(4, dtype=torch.int32, device="cuda")
        o["tg"] = torch.zeros((self.S, self.NT), dtype=torch.int32, device="cuda")
        o["ac"] = torch.zeros(self.S, dtype=torch.int32, device="cuda")
        o["htg"] = torch.zeros(self.hn, dtype=torch.int32, device="cuda")
        o["hac"] = torch.zeros(4, dtype=torch.int32, device="cuda")
        return o

    def call(self, v, o):
        B = self.B
        for i, L in enumerate(self.layers):
            B.moe_verify_block(L, self.x[v], 0, o[f"y{i}"], o[f"ids{i}"], o[f"w{i}"], o[f"nw{i}"], self.ws[i])
        B.accept_prefix_batch(self.lg[v], self.dr, o["tg"], o["ac"], self.aws)
        B.lm_head_accept(self.hh[v], self.head[0], self.hV, self.hdr, o["htg"], o["hac"], self.hws)


def test_two_streams_two_threads(B):
    from speculative_decoding_moe_amd.workloads import device
    H = 1024
    layers = []
    for wd in ("bf16", "mxfp4"):
        wl = gen.Workload("streams_" + wd, gen.LayerShape(H, 64, 4, 256, 256, wdtype=wd), k=16, seed=9000)
        layers.append(device.make_layer(wl, 0, "cuda"))
    hw = gen.Workload("streams_head", gen.LayerShape(H, 16, 2, 128, 0), k=9, seed=9050, vocab=12000, n_target=9)
    head = (B.pack_head(device.head_tensor(hw, "cuda")), hw.vocab)
    callers = [Caller(B, layers, head, 0, 48), Caller(B, layers, head, 1, 100)]

    # each caller alone on the default stream: the expected bits of each input set
    want = []
    for c in callers:
        per = []
        for v in range(2):
            o = c.outputs()
            print(f"[streams] alone k={c.k} set {v}", flush=True)
            c.call(v, o)
            torch.cuda.synchronize()
            per.append({n: _bits(t) for n, t in o.items()})
        want.append(per)

    outs = [[c.outputs() for _ in range(REPS)] for c in callers]
    streams = [torch.cuda.Stream() for _ in callers]
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(len(callers))

    def work(j):
        try:
            torch.cuda.set_device(0)
            start.wait(timeout=60)
            with torch.cuda.stream(streams[j]):
                for r in range(REPS):
                    callers[j].call(r % 2, outs[j][r])
        except Exception as e:  # reported by the main thread
            errors.append((j, repr(e)))

    print(f"[streams] two threads x {REPS} calls", flush=True)
    threads = [threading.Thread(target=work, args=(j,), daemon=True) for j in range(len(callers))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a caller thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for j, c in enumerate(callers):
        for r in range(REPS):
            got = {n: _bits(t) for n, t in outs[j][r].items()}
            ref = want[j][r % 2]
            for n in ref:
                assert np.array_equal(got[n], ref[n]), (j, r, n)
        assert np.all(want[j][0]["nw0"][:1] > 0) and np.all(want[j][0]["ac"] >= 0) and want[j][0]["hac"][0] >= 0
    del layers, head
    torch.cuda.empty_cache()
