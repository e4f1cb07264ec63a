"""The Python binding rejects tensors the C ABI cannot check (element type, shape, layout, device)
before any library call, so nothing here needs a GPU: every case raises ValueError on the host."""
from types import SimpleNamespace

import pytest
import torch

from speculative_decoding_moe_amd import binding as B

H, K = 256, 2
LAYER = SimpleNamespace(hidden=H, top_k=K)


def f32(*s):
    return torch.zeros(s, dtype=torch.float32)


def i32(*s):
    return torch.zeros(s, dtype=torch.int32)


def ws():
    return torch.zeros(64, dtype=torch.uint8)


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_moe_verify_block_rejects_bad_tensors():
    k = 4
    ok = dict(topk_ids=i32(k, K), topk_w=f32(k, K), n_woken=i32(4), workspace=ws())
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H).double(), 0, f32(k, H), **ok), "x must have dtype")
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H).half(), 0, f32(k, H), **ok), "x must have dtype")
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H + 128), 0, f32(k, H + 128), **ok), "x must have shape")
    _raises(lambda: B.moe_verify_block(LAYER, f32(H, k).t(), 0, f32(k, H), **ok), "x must be contiguous")
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H), 0, f32(k + 1, H), **ok), "y must have shape")
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H), 0, f32(k, H), topk_ids=i32(k, K + 1)), "topk_ids")
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H), 0, f32(k, H), topk_ids=f32(k, K)), "topk_ids")
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H), 0, f32(k, H), topk_w=f32(k - 1, K)), "topk_w")
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H), 0, f32(k, H), n_woken=i32(0)), "n_woken")
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H), 0, f32(k, H), n_woken=f32(1)), "n_woken")
    # a well-formed call on host tensors: only the device is wrong
    _raises(lambda: B.moe_verify_block(LAYER, f32(k, H), 0, f32(k, H), **ok), "must be on a GPU device")


def test_moe_verify_block_timed_needs_five_events():
    _raises(lambda: B.moe_verify_block_timed(LAYER, f32(2, H), 0, f32(2, H), [0, 0, 0], workspace=ws()),
            "must be on a GPU device|events")


def test_accept_prefix_rejects_bad_tensors():
    lg, tg, acc = f32(5, 100), i32(5), i32(1)
    _raises(lambda: B.accept_prefix(lg.double(), i32(4), tg, acc, ws()), "logits must have dtype")
    _raises(lambda: B.accept_prefix(f32(5, 100, 1), i32(4), tg, acc, ws()), "logits must have shape")
    _raises(lambda: B.accept_prefix(f32(100, 5).t(), i32(4), tg, acc, ws()), "logits must be contiguous")
    _raises(lambda: B.accept_prefix(lg, i32(4), tg, acc, ws(), n_draft=5), "n_draft 5 outside")
    _raises(lambda: B.accept_prefix(lg, None, tg, acc, ws(), n_draft=1), "n_draft 1 outside")
    _raises(lambda: B.accept_prefix(lg, i32(4).long(), tg, acc, ws()), "draft_ids must have dtype")
    _raises(lambda: B.accept_prefix(lg, i32(4), i32(4), acc, ws()), "target_ids must hold")
    _raises(lambda: B.accept_prefix(lg, i32(4), tg, i32(0), ws()), "accepted must hold")
    _raises(lambda: B.accept_prefix(lg, i32(4), tg, acc, ws()), "must be on a GPU device")


def test_accept_prefix_batch_rejects_bad_tensors():
    lg = f32(3, 5, 100)
    _raises(lambda: B.accept_prefix_batch(f32(5, 100), i32(3, 4), i32(3, 5), i32(3), ws()), "logits must have shape")
    _raises(lambda: B.accept_prefix_batch(lg, i32(2, 4), i32(3, 5), i32(3), ws()), "draft_ids must have shape")
    _raises(lambda: B.accept_prefix_batch(lg, i32(3, 4), i32(3, 4), i32(3), ws()), "target_ids must have shape")
    _raises(lambda: B.accept_prefix_batch(lg, i32(3, 4), i32(3, 5), i32(2), ws()), "accepted must have shape")
    _raises(lambda: B.accept_prefix_batch(lg, i32(3, 4), i32(3, 5), i32(3), ws(), n_draft=i32(4)), "n_draft")
    _raises(lambda: B.accept_prefix_batch(lg, i32(3, 4), i32(3, 5), i32(3), ws()), "must be on a GPU device")


def test_lm_head_accept_rejects_bad_tensors():
    h = f32(4, 128)
    wt = torch.zeros(112 * 128, dtype=torch.int16)  # 100 rows padded to 112
    _raises(lambda: B.lm_head_accept(h.double(), wt, 100, i32(3), i32(4), i32(1), ws()), "h must have dtype")
    _raises(lambda: B.lm_head_accept(h, wt[:-1], 100, i32(3), i32(4), i32(1), ws()), "w_head_tiled must hold")
    _raises(lambda: B.lm_head_accept(h, wt.float(), 100, i32(3), i32(4), i32(1), ws()), "w_head_tiled must have")
    _raises(lambda: B.lm_head_accept(h, wt, 100, i32(3), i32(3), i32(1), ws()), "target_ids must hold")
    _raises(lambda: B.lm_head_accept(h, wt, 100, i32(3), i32(4), i32(1), ws(), n_draft=4), "n_draft 4 outside")
    _raises(lambda: B.lm_head_accept(h, wt, 100, i32(3), i32(4), i32(1), ws()), "must be on a GPU device")


def test_accept_sample_rejects_bad_tensors():
    tl, dl, d = f32(5, 50), f32(4, 50), i32(4)
    ua, us = f32(4), f32(5)
    _raises(lambda: B.accept_sample(tl, f32(3, 50), d, 1.0, ua, us, i32(1), i32(1), ws()), "draft_logits must have")
    _raises(lambda: B.accept_sample(tl, dl, d, 1.0, f32(3), us, i32(1), i32(1), ws()), "u_accept must hold")
    _raises(lambda: B.accept_sample(tl, dl, d, 1.0, ua, f32(4), i32(1), i32(1), ws()), "u_sample must hold")
    _raises(lambda: B.accept_sample(tl, dl, d, 1.0, ua, us, i32(1), i32(0), ws()), "token must hold")
    _raises(lambda: B.accept_sample(tl, dl, d, 1.0, ua, us, i32(1), i32(1), ws()), "must be on a GPU device")


def test_accept_sample_batch_rejects_bad_tensors():
    tl, dl, d = f32(2, 5, 50), f32(2, 4, 50), i32(2, 4)
    ua, us = f32(2, 4), f32(2, 5)
    _raises(lambda: B.accept_sample_batch(tl, dl, d, 1.0, ua, f32(2, 4), i32(2), i32(2), ws()), "u_sample must have")
    _raises(lambda: B.accept_sample_batch(tl, f32(2, 4, 49), d, 1.0, ua, us, i32(2), i32(2), ws()), "draft_logits")
    _raises(lambda: B.accept_sample_batch(tl, dl, d, 1.0, ua, us, i32(3), i32(2), ws()), "accepted must have")
    _raises(lambda: B.accept_sample_batch(tl, dl, d, 1.0, ua, us, i32(2), i32(2), ws()), "must be on a GPU device")


def test_accept_histogram_rejects_bad_tensors():
    acc = i32(10)
    hist, surv = torch.zeros(5, dtype=torch.int64), torch.zeros(4, dtype=torch.int64)
    _raises(lambda: B.accept_histogram(acc, 4, hist.int(), surv), "hist must have dtype")
    _raises(lambda: B.accept_histogram(acc, 4, hist[:4], surv), "hist must hold")
    _raises(lambda: B.accept_histogram(acc, 4, hist, surv[:3]), "survival must hold")
    _raises(lambda: B.accept_histogram(acc, 4, hist, surv), "must be on a GPU device")


def test_layer_and_pack_reject_bad_tensors():
    E, I = 4, 128
    t = dict(router_w=f32(E, H), w_gate=torch.zeros(E, I, H, dtype=torch.int16),
             w_up=torch.zeros(E, I, H, dtype=torch.int16), w_down=torch.zeros(E, H, I, dtype=torch.int16))
    mk = lambda **o: B.MoeLayer(hidden=H, n_experts=E, top_k=2, inter=I, shared_inter=0, **{**t, **o})  # noqa: E731
    _raises(lambda: mk(router_w=f32(E, H).double()), "router_w must have dtype")
    _raises(lambda: mk(w_up=torch.zeros(E - 1, I, H, dtype=torch.int16)), "w_up must hold")
    _raises(lambda: mk(w_down=f32(E, H, I)), "w_down must have dtype")
    _raises(lambda: mk(), "must be on a GPU device")
    _raises(lambda: B.pack_weights(f32(16, 128)), "src must have dtype")
    _raises(lambda: B.pack_weights(torch.zeros(16, 64, dtype=torch.uint8), torch.zeros(16, 3, dtype=torch.uint8)),
            "src_scales must have shape")
    _raises(lambda: B.pack_weights(torch.zeros(16, 128, dtype=torch.int16)), "must be on a GPU device")
