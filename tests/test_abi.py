"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments on the host
before any HIP call (no GPU needed: nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_verify.h")
LIB = os.path.join(ROOT, "speculative_decoding_moe_amd", "libmoeverify.so")


@pytest.fixture(scope="module")
def b():
    if not os.path.exists(LIB):
        from speculative_decoding_moe_amd import _build
        _build.build()
    from speculative_decoding_moe_amd import binding
    return binding


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points(b):
    assert _declared_functions() == sorted(b.EXPORTS)


def test_library_exports_every_declared_symbol(b):
    lib = ctypes.CDLL(LIB)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(b):
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = b.status_string(st)
        assert s and s != "unknown status"
    assert b.status_string(12345) == "unknown status"


FAKE = 0x7F0000000000  # 16-byte aligned stand-in address; never dereferenced by host validation


def _layer(b, **over):
    d = dict(hidden=2048, n_experts=256, top_k=8, inter=512, shared_inter=512, wdtype=0, layout=1, rms_eps=1e-6,
             router_w=FAKE, w_gate=FAKE + 0x1000, w_up=FAKE + 0x2000, w_down=FAKE + 0x3000, s_gate=None,
             s_up=None, s_down=None, sh_gate=FAKE + 0x4000, sh_up=FAKE + 0x5000, sh_down=FAKE + 0x6000)
    d.update(over)
    return b.MoeLayerStruct(*(d[f] for f, _ in b.MoeLayerStruct._fields_))


def _call(b, L, k=16, flags=0, x=FAKE + 0x10000000, y=FAKE + 0x20000000, ids=None, w=None, n=None,
          ws=FAKE + 0x40000000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = b.lib.moe_verify_workspace_size(ctypes.byref(L), k) if 1 <= k <= 1024 else 1 << 30
    return b.lib.moe_verify_block(ctypes.byref(L), x, k, flags, y, ids, w, n, ws, ws_bytes, None)


def test_workspace_size(b):
    L = _layer(b)
    n1 = b.lib.moe_verify_workspace_size(ctypes.byref(L), 1)
    n16 = b.lib.moe_verify_workspace_size(ctypes.byref(L), 16)
    assert 0 < n1 < n16
    assert n16 % 256 == 0
    assert b.lib.moe_verify_workspace_size(ctypes.byref(L), 0) == 0
    # the gathered path (k > 16) grows with k, up to 1024 tokens
    n17 = b.lib.moe_verify_workspace_size(ctypes.byref(L), 17)
    n1024 = b.lib.moe_verify_workspace_size(ctypes.byref(L), 1024)
    assert n16 <= n17 < n1024 and n1024 % 256 == 0
    assert b.lib.moe_verify_workspace_size(ctypes.byref(L), 1025) == 0
    mx = _layer(b, wdtype=1, s_gate=FAKE + 0x7000, s_up=FAKE + 0x8000, s_down=FAKE + 0x9000)
    m16 = b.lib.moe_verify_workspace_size(ctypes.byref(mx), 16)
    m1024 = b.lib.moe_verify_workspace_size(ctypes.byref(mx), 1024)
    assert 0 < m16 and m1024 > n1024  # the MX-fp8 windows of the gathered path on top
    assert b.lib.moe_verify_workspace_size(None, 4) == 0
    assert b.lib.moe_verify_workspace_size(ctypes.byref(_layer(b, hidden=100)), 4) == 0


@pytest.mark.parametrize("over,status", [
    (dict(hidden=100), -2), (dict(hidden=64), -2), (dict(hidden=4096), -2), (dict(hidden=1152), -2),
    (dict(n_experts=0), -2), (dict(n_experts=513), -2), (dict(top_k=0), -2), (dict(top_k=17), -2),
    (dict(n_experts=4, top_k=5), -2), (dict(inter=192), -2), (dict(inter=1152), -2), (dict(inter=2048), -2),
    (dict(inter=0), -2), (dict(shared_inter=64), -2), (dict(shared_inter=1280), -2), (dict(shared_inter=-128), -2),
    (dict(wdtype=2), -3), (dict(wdtype=1), -3), (dict(layout=0), -3),
    (dict(router_w=None), -1), (dict(w_down=None), -1), (dict(sh_up=None), -1),
    (dict(w_gate=FAKE + 8), -4), (dict(rms_eps=-1.0), -8), (dict(rms_eps=float("nan")), -8),
])
def test_bad_layer_rejected(b, over, status):
    assert _call(b, _layer(b, **over), ws_bytes=1 << 30) == status


@pytest.mark.parametrize("over", [dict(inter=384), dict(inter=640, shared_inter=128), dict(shared_inter=256),
                                  dict(inter=256, shared_inter=1024), dict(inter=768, shared_inter=0)])
def test_general_sizes_take_the_gathered_workspace(b, over):
    """Layers outside the single-block shapes (I / 128 not dividing eight, or a shared expert of
    another size) are accepted and take the gathered path at every k: their workspace for a
    16-token block is the gathered path's, which grows with the token count, and one byte less
    is refused before anything is launched."""
    L = _layer(b, **over)
    n1 = b.lib.moe_verify_workspace_size(ctypes.byref(L), 1)
    n16 = b.lib.moe_verify_workspace_size(ctypes.byref(L), 16)
    n17 = b.lib.moe_verify_workspace_size(ctypes.byref(L), 17)
    assert 0 < n1 < n16 < n17
    for k in (1, 16):
        need = b.lib.moe_verify_workspace_size(ctypes.byref(L), k)
        assert _call(b, L, k=k, ws_bytes=need - 1) == b.MOE_ERR_WORKSPACE
        assert _call(b, L, k=k, flags=4, ws_bytes=need - 1) == b.MOE_ERR_WORKSPACE


def test_bad_call_arguments_rejected(b):
    L = _layer(b)
    assert b.lib.moe_verify_block(None, FAKE, 4, 0, FAKE, None, None, None, FAKE, 1 << 30, None) == -1
    assert _call(b, L, x=None) == -1
    assert _call(b, L, y=None) == -1
    assert _call(b, L, ws=None) == -1
    assert _call(b, L, k=0) == -2
    assert _call(b, L, k=1025) == -2
    assert _call(b, L, flags=8) == -8
    assert _call(b, L, x=FAKE + 0x10000004) == -4
    assert _call(b, L, ids=FAKE + 0x30000002) == -4
    need = b.lib.moe_verify_workspace_size(ctypes.byref(L), 16)
    assert _call(b, L, ws_bytes=need - 1) == -5
    # y overlapping x, or the workspace
    assert _call(b, L, y=FAKE + 0x10000000) == -6
    assert _call(b, L, y=FAKE + 0x40000000 + 256) == -6
    assert _call(b, L, x=FAKE + 0x40000000 + 4096) == -6
    assert _call(b, L, ids=FAKE + 0x40000000 + 512) == -6


def test_gathered_path_validation(b):
    """Calls of more than 16 tokens (or MOE_GATHER) take the gathered path; every case here is
    rejected before any HIP call."""
    L = _layer(b)
    need = b.lib.moe_verify_workspace_size(ctypes.byref(L), 100)
    assert need > b.lib.moe_verify_workspace_size(ctypes.byref(L), 16)
    assert _call(b, L, k=100, ws_bytes=1024) == -5
    assert _call(b, L, k=1024, ws_bytes=b.lib.moe_verify_workspace_size(ctypes.byref(L), 1024) - 1) == -5
    assert _call(b, L, k=8, flags=4, ws_bytes=0) == -5
    assert _call(b, L, k=100, x=FAKE + 0x10000004) == -4
    assert _call(b, L, k=100, ids=FAKE + 0x30000002) == -4
    assert _call(b, L, k=100, y=FAKE + 0x10000000 + 4096) == -6          # y overlaps x
    assert _call(b, L, k=100, y=FAKE + 0x40000000 + 256) == -6           # y overlaps the workspace
    assert _call(b, L, k=100, ids=FAKE + 0x40000000 + need - 64) == -6   # ids overlap the workspace
    assert _call(b, L, k=100, flags=1 | 2 | 8) == -8
    # mxfp4 layers: the gathered path needs its larger workspace (MX-fp8 windows)
    mx = _layer(b, wdtype=1, s_gate=FAKE + 0x7000, s_up=FAKE + 0x8000, s_down=FAKE + 0x9000)
    assert _call(b, mx, k=17, ws_bytes=1024) == -5
    assert _call(b, mx, k=1024, ws_bytes=b.lib.moe_verify_workspace_size(ctypes.byref(mx), 1024) - 1) == -5
    assert _call(b, mx, k=16, flags=4, ws_bytes=1024) == -5


def test_mxfp4_layer_needs_h_multiple_of_256(b):
    L = _layer(b, hidden=384, wdtype=1, s_gate=FAKE + 0x7000, s_up=FAKE + 0x8000, s_down=FAKE + 0x9000)
    assert _call(b, L, ws_bytes=1 << 30) == -2


def test_mxfp4_layer_needs_scales(b):
    L = _layer(b, wdtype=1, s_gate=FAKE + 0x7000, s_up=FAKE + 0x8000, s_down=None)
    assert _call(b, L, ws_bytes=1 << 30) == -3


def test_accept_prefix_validation(b):
    f = b.lib.accept_prefix
    ws = FAKE + 0x50000000
    need = b.lib.accept_prefix_workspace_size(17, 151936)
    assert need > 0
    assert b.lib.accept_prefix_workspace_size(0, 10) == 0
    assert b.lib.accept_prefix_workspace_size(65, 10) == 0
    assert b.lib.accept_prefix_workspace_size(4, 0) == 0
    lg, dr, tg, ac = FAKE, FAKE + 0x10000000, FAKE + 0x20000000, FAKE + 0x30000000
    assert f(None, 17, 151936, dr, 16, tg, ac, ws, need, None) == -1
    assert f(lg, 17, 151936, None, 16, tg, ac, ws, need, None) == -1
    assert f(lg, 0, 151936, dr, 0, tg, ac, ws, need, None) == -2
    assert f(lg, 17, 151936, dr, 18, tg, ac, ws, need, None) == -2
    assert f(lg, 17, 151936, dr, -1, tg, ac, ws, need, None) == -2
    assert f(lg, 17, 0, dr, 16, tg, ac, ws, need, None) == -2
    assert f(lg, 17, 151936, dr, 16, tg + 4, ac, ws, need, None) == -4
    assert f(lg, 17, 151936, dr, 16, tg, ac, ws, need - 1, None) == -5
    assert f(lg, 17, 151936, dr, 16, lg + 64, ac, ws, need, None) == -6
    assert f(lg, 17, 151936, dr, 16, tg, tg, ws, need, None) == -6


def test_accept_prefix_batch_validation(b):
    f = b.lib.accept_prefix_batch
    ws = FAKE + 0x50000000
    need = b.lib.accept_prefix_batch_workspace_size(32, 17, 151936)
    assert need >= 32 * b.lib.accept_prefix_workspace_size(17, 151936) - 32 * 512
    assert b.lib.accept_prefix_batch_workspace_size(0, 17, 10) == 0
    assert b.lib.accept_prefix_batch_workspace_size(1025, 17, 10) == 0
    assert b.lib.accept_prefix_batch_workspace_size(1024, 64, 10) == 0   # more than 65535 rows
    assert b.lib.accept_prefix_batch_workspace_size(4, 65, 10) == 0
    assert b.lib.accept_prefix_batch_workspace_size(4, 17, 0) == 0
    lg, dr, nd, tg, ac = FAKE, FAKE + 0x20000000, FAKE + 0x21000000, FAKE + 0x22000000, FAKE + 0x23000000
    assert f(None, 32, 17, 151936, dr, 16, nd, tg, ac, ws, need, None) == -1
    assert f(lg, 32, 17, 151936, None, 16, nd, tg, ac, ws, need, None) == -1
    assert f(lg, 32, 17, 151936, dr, 16, nd, None, ac, ws, need, None) == -1
    assert f(lg, 0, 17, 151936, dr, 16, nd, tg, ac, ws, need, None) == -2
    assert f(lg, 32, 17, 151936, dr, 18, nd, tg, ac, ws, need, None) == -2
    assert f(lg, 32, 17, 151936, dr, -1, nd, tg, ac, ws, need, None) == -2
    assert f(lg, 1024, 64, 151936, dr, 16, nd, tg, ac, ws, need, None) == -2
    assert f(lg, 32, 17, 151936, dr, 16, nd + 4, tg, ac, ws, need, None) == -4
    assert f(lg, 32, 17, 151936, dr, 16, nd, tg, ac, ws, need - 1, None) == -5
    assert f(lg, 32, 17, 151936, dr, 16, nd, lg + 4096, ac, ws, need, None) == -6   # targets inside the logits
    assert f(lg, 32, 17, 151936, dr, 16, nd, tg, tg + 64, ws, need, None) == -6     # accepted inside the targets
    assert f(lg, 32, 17, 151936, dr, 16, nd, tg, ws + 256, ws, need, None) == -6    # accepted inside the workspace


def test_lm_head_accept_validation(b):
    f = b.lib.lm_head_accept
    V, H = 151936, 2048
    need = b.lib.lm_head_accept_workspace_size(16, H, V)
    assert need > 0
    assert b.lib.lm_head_accept_workspace_size(0, H, V) == 0
    assert b.lib.lm_head_accept_workspace_size(17, H, V) == 0
    assert b.lib.lm_head_accept_workspace_size(4, H, 0) == 0
    h, w, dr, tg, ac, ws = (FAKE, FAKE + 0x10000000, FAKE + 0x60000000, FAKE + 0x61000000, FAKE + 0x62000000,
                            FAKE + 0x63000000)
    ok = (h, 16, H, w, V, 1, dr, 15, tg, ac, ws, need, None)

    def call(**kw):
        names = ("h", "n", "H", "w", "V", "layout", "dr", "nd", "tg", "ac", "ws", "wsb", "s")
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[k] for k in names])

    # every call below fails a host-side check: none reaches a launch
    assert call(h=None) == -1
    assert call(dr=None) == -1
    assert call(n=0) == -2
    assert call(n=17) == -2
    assert call(nd=17) == -2
    assert call(H=2000) == -2       # not a multiple of 128
    assert call(H=4096) == -2       # above the largest supported hidden size
    assert call(V=0) == -2
    assert call(V=1 << 21, H=2048) == -2  # 32-bit offsets into the head
    assert call(layout=0) == -3
    assert call(h=h + 4) == -4
    assert call(wsb=need - 1) == -5
    assert call(tg=h + 64) == -6
    assert call(ac=tg) == -6
    assert call(ws=w + 4096) == -6


def test_accept_sample_validation(b):
    f = b.lib.accept_sample
    V, nt, nd = 151936, 17, 16
    need = b.lib.accept_sample_workspace_size(nt, nd, V)
    assert need > 0
    assert b.lib.accept_sample_workspace_size(0, 0, V) == 0
    assert b.lib.accept_sample_workspace_size(65, 0, V) == 0
    assert b.lib.accept_sample_workspace_size(4, 5, V) == 0
    assert b.lib.accept_sample_workspace_size(4, 4, (1 << 24) + 1) == 0
    tl, dl, di, ua, us, ac, tk, ws = (FAKE, FAKE + 0x10000000, FAKE + 0x20000000, FAKE + 0x21000000,
                                      FAKE + 0x22000000, FAKE + 0x23000000, FAKE + 0x24000000, FAKE + 0x30000000)
    ok = dict(tl=tl, nt=nt, V=V, dl=dl, di=di, nd=nd, T=1.0, ua=ua, us=us, ac=ac, tk=tk, ws=ws, wsb=need, s=None)
    names = ("tl", "nt", "V", "dl", "di", "nd", "T", "ua", "us", "ac", "tk", "ws", "wsb", "s")

    def call(**kw):
        args = dict(ok)
        args.update(kw)
        return f(*[args[k] for k in names])

    # every call below fails a host-side check: none reaches a launch
    assert call(tl=None) == -1
    assert call(us=None) == -1
    assert call(dl=None) == -1
    assert call(di=None) == -1
    assert call(ua=None) == -1
    assert call(tk=None) == -1
    assert call(nt=0) == -2
    assert call(nt=65) == -2
    assert call(nd=18) == -2
    assert call(V=0) == -2
    assert call(T=0.0) == -2
    assert call(T=-1.0) == -2
    assert call(T=float("inf")) == -2
    assert call(T=float("nan")) == -2
    assert call(tl=tl + 4) == -4
    assert call(ac=ac + 2) == -4
    assert call(wsb=need - 1) == -5
    assert call(tk=tl + 64) == -6
    assert call(tk=ac) == -6
    assert call(ac=ws + 64) == -6


def test_accept_sample_batch_validation(b):
    f = b.lib.accept_sample_batch
    need = b.lib.accept_sample_batch_workspace_size(32, 17, 16, 151936)
    assert need >= 32 * 17 * 10 * 8
    assert b.lib.accept_sample_batch_workspace_size(0, 17, 16, 100) == 0
    assert b.lib.accept_sample_batch_workspace_size(1025, 17, 16, 100) == 0
    assert b.lib.accept_sample_batch_workspace_size(4, 17, 18, 100) == 0
    tl, dl, di, ua, us, ac, tk, ws = (FAKE, FAKE + 0x40000000, FAKE + 0x80000000, FAKE + 0x81000000,
                                      FAKE + 0x82000000, FAKE + 0x83000000, FAKE + 0x84000000, FAKE + 0x90000000)
    assert f(None, 32, 17, 151936, dl, di, 16, 1.0, ua, us, ac, tk, ws, need, None) == -1
    assert f(tl, 32, 17, 151936, None, di, 16, 1.0, ua, us, ac, tk, ws, need, None) == -1
    assert f(tl, 0, 17, 151936, dl, di, 16, 1.0, ua, us, ac, tk, ws, need, None) == -2
    assert f(tl, 1025, 17, 151936, dl, di, 16, 1.0, ua, us, ac, tk, ws, need, None) == -2
    assert f(tl, 32, 17, 151936, dl, di, 16, 0.0, ua, us, ac, tk, ws, need, None) == -2
    assert f(tl, 32, 17, 151936, dl, di, 16, float("inf"), ua, us, ac, tk, ws, need, None) == -2
    assert f(tl + 4, 32, 17, 151936, dl, di, 16, 1.0, ua, us, ac, tk, ws, need, None) == -4
    assert f(tl, 32, 17, 151936, dl, di, 16, 1.0, ua, us, ac, tk, ws, need - 1, None) == -5
    assert f(tl, 32, 17, 151936, dl, di, 16, 1.0, ua, us, tl + 4096, tk, ws, need, None) == -6  # accepted inside the logits
    assert f(tl, 32, 17, 151936, dl, di, 16, 1.0, ua, us, ac, ac + 64, ws, need, None) == -6    # token overlaps accepted


def test_accept_histogram_validation(b):
    f = b.lib.accept_histogram
    a, h, sv = FAKE, FAKE + 0x1000, FAKE + 0x2000
    assert f(None, 10, 4, h, sv, None) == -1
    assert f(a, 10, 4, None, sv, None) == -1
    assert f(a, 10, 4, h, None, None) == -1
    assert f(a, -1, 4, h, sv, None) == -2
    assert f(a, 10, 65, h, sv, None) == -2
    assert f(a, 10, 4, h + 4, sv, None) == -4
    assert f(a, 10, 4, a + 8, sv, None) == -6
    assert f(a, 10, 4, h, h + 8, None) == -6


def test_pack_weights_validation(b):
    f = b.lib.moe_pack_weights
    src, dst, ss, ds = FAKE, FAKE + 0x10000000, FAKE + 0x20000000, FAKE + 0x30000000
    assert f(0, 4, 512, 2048, None, None, dst, None, None) == -1
    assert f(0, 4, 512, 2048, src, None, None, None, None) == -1
    assert f(1, 4, 512, 2048, src, None, dst, ds, None) == -1   # mxfp4 without source scales
    assert f(1, 4, 512, 2048, src, ss, dst, None, None) == -1
    assert f(2, 4, 512, 2048, src, None, dst, None, None) == -3
    assert f(0, 0, 512, 2048, src, None, dst, None, None) == -2
    assert f(0, 4, 520, 2048, src, None, dst, None, None) == -2  # rows not a multiple of 16
    assert f(0, 4, 512, 2000, src, None, dst, None, None) == -2  # cols not a multiple of 128
    assert f(0, 4, 512, 64, src, None, dst, None, None) == -2
    assert f(0, 4, 512, 2048, src + 8, None, dst, None, None) == -4
    assert f(0, 4, 512, 2048, src, None, src + 4096, None, None) == -6   # dst overlaps src
    assert f(1, 1, 512, 2048, src, ss, dst, ss + 16, None) == -6          # scales overlap


def test_noalloc_rejects_calls_beyond_its_scratch_and_bad_arguments(b):
    """Host-side checks of moe_verify_block_noalloc, all before any HIP call."""
    L = _layer(b)
    x, y = FAKE + 0x10000000, FAKE + 0x20000000
    call = lambda L, k, flags=0, x=x, y=y: b.lib.moe_verify_block_noalloc(ctypes.byref(L), x, k, flags, y, None,  # noqa: E731
                                                                          None, None, None)
    assert b.lib.moe_verify_workspace_size(ctypes.byref(L), 1024) > b.NOALLOC_SCRATCH_BYTES
    assert call(L, 1024) == b.MOE_ERR_WORKSPACE          # gathered 1024 tokens: about 104 MB
    assert call(L, 17) == b.MOE_ERR_WORKSPACE or b.lib.moe_verify_workspace_size(ctypes.byref(L), 17) <= \
        b.NOALLOC_SCRATCH_BYTES
    assert call(L, 0) == b.MOE_ERR_SHAPE
    assert call(L, 1025) == b.MOE_ERR_SHAPE
    assert call(L, 16, flags=8) == b.MOE_ERR_ARG
    assert call(L, 16, x=None) == b.MOE_ERR_NULL
    assert call(L, 16, y=None) == b.MOE_ERR_NULL
    assert call(_layer(b, inter=192), 16) == b.MOE_ERR_SHAPE
    # the largest layer's 16-token block fits: its workspace is below the scratch size
    big = _layer(b, n_experts=512, top_k=16, inter=1024, shared_inter=1024)
    assert 0 < b.lib.moe_verify_workspace_size(ctypes.byref(big), 16) <= b.NOALLOC_SCRATCH_BYTES


def _stack(b, layers, k=16, flags=3, x=FAKE + 0x10000000, y=FAKE + 0x20000000, n=None, ws=FAKE + 0x40000000,
           ws_bytes=None):
    arr = (b.MoeLayerStruct * max(1, len(layers)))(*layers)
    if ws_bytes is None:
        ws_bytes = 1 << 30
    return b.lib.moe_verify_stack(arr if layers else None, len(layers), x, k, flags, y, n, ws, ws_bytes, None)


def test_stack_workspace_size(b):
    """A stack's workspace is one layer's single-block workspace plus a second counter set and two
    activation buffers; 0 for blocks or layer sizes that take the gathered path."""
    L = _layer(b)
    s1 = b.lib.moe_verify_stack_workspace_size(ctypes.byref(L), 1)
    s16 = b.lib.moe_verify_stack_workspace_size(ctypes.byref(L), 16)
    assert 0 < s1 < s16 and s16 % 256 == 0
    assert s16 >= 16 * 2048 * 4 * 2  # the two activation buffers
    assert b.lib.moe_verify_stack_workspace_size(ctypes.byref(L), 0) == 0
    assert b.lib.moe_verify_stack_workspace_size(ctypes.byref(L), 17) == 0
    assert b.lib.moe_verify_stack_workspace_size(ctypes.byref(_layer(b, inter=384)), 16) == 0
    assert b.lib.moe_verify_stack_workspace_size(None, 16) == 0


def test_stack_arguments_rejected(b):
    """moe_verify_stack validates everything on the host before any launch."""
    L = _layer(b)
    need = b.lib.moe_verify_stack_workspace_size(ctypes.byref(L), 16)
    assert _stack(b, []) == b.MOE_ERR_NULL
    assert _stack(b, [L], x=None) == b.MOE_ERR_NULL
    assert _stack(b, [L], y=None) == b.MOE_ERR_NULL
    assert _stack(b, [L], ws=None) == b.MOE_ERR_NULL
    assert _stack(b, [L, _layer(b, hidden=100)]) == b.MOE_ERR_SHAPE           # an invalid layer
    assert _stack(b, [L, _layer(b, n_experts=128)]) == b.MOE_ERR_SHAPE         # shapes differ
    mx = _layer(b, wdtype=1, s_gate=FAKE + 0x7000, s_up=FAKE + 0x8000, s_down=FAKE + 0x9000)
    assert _stack(b, [L, mx]) == b.MOE_ERR_SHAPE                                # formats differ
    assert _stack(b, [L], k=0) == b.MOE_ERR_SHAPE
    assert _stack(b, [L], k=17) == b.MOE_ERR_SHAPE
    assert _stack(b, [_layer(b, inter=384)]) == b.MOE_ERR_SHAPE                # a gathered-path layer
    assert _stack(b, [L], flags=4) == b.MOE_ERR_ARG                             # MOE_GATHER
    assert _stack(b, [L], flags=8) == b.MOE_ERR_ARG
    assert _stack(b, [L], x=FAKE + 8) == b.MOE_ERR_ALIGN
    assert _stack(b, [L], n=FAKE + 0x30000004) == b.MOE_ERR_ALIGN
    assert _stack(b, [L], ws_bytes=need - 1) == b.MOE_ERR_WORKSPACE
    assert _stack(b, [L], y=FAKE + 0x10000000 + 256) == b.MOE_ERR_ALIAS         # y overlaps x
    assert _stack(b, [L], y=FAKE + 0x40000000 + 4096) == b.MOE_ERR_ALIAS        # y inside the workspace
    assert _stack(b, [L, L], n=FAKE + 0x40000000) == b.MOE_ERR_ALIAS            # n_woken inside the workspace
    many = [L] * (b.STACK_MAX_LAYERS + 1)
    assert b.lib.moe_verify_stack((b.MoeLayerStruct * len(many))(*many), len(many), FAKE + 0x10000000, 16, 3,
                                  FAKE + 0x20000000, None, FAKE + 0x40000000, 1 << 30, None) == b.MOE_ERR_SHAPE
