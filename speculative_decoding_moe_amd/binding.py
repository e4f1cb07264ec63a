"""Thin Python binding of libmoeverify.so (include/moe_verify.h): argument marshalling only.

Every step of the MoE verify pass runs in the library's HIP kernels. Tensors are torch tensors
on a ROCm device; the call is enqueued on torch's current stream. If the library cannot be
loaded, import fails loudly: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoeverify.so")

MOE_OK = 0
MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN = -1, -2, -3, -4
MOE_ERR_WORKSPACE, MOE_ERR_ALIAS, MOE_ERR_HIP, MOE_ERR_ARG = -5, -6, -7, -8
MOE_W_BF16, MOE_W_MXFP4 = 0, 1
MOE_LAYOUT_TILED = 1
MOE_PRE_RMSNORM, MOE_RESIDUAL, MOE_GATHER = 1, 2, 4

NOALLOC_SCRATCH_BYTES = 24 << 20  # MOE_NOALLOC_SCRATCH_BYTES
STACK_MAX_LAYERS = 4096  # MOE_STACK_MAX_LAYERS

EXPORTS = ("moe_verify_workspace_size", "moe_verify_block", "moe_verify_block_timed", "moe_verify_block_noalloc",
           "moe_verify_stack_workspace_size", "moe_verify_stack", "moe_pack_weights", "accept_prefix_workspace_size", "accept_prefix",
           "accept_prefix_batch_workspace_size", "accept_prefix_batch",
           "lm_head_accept_workspace_size", "lm_head_accept", "accept_sample_workspace_size",
           "accept_sample", "accept_sample_batch_workspace_size", "accept_sample_batch",
           "accept_histogram", "moe_status_string")


class MoeLayerStruct(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("wdtype", ctypes.c_int32),
        ("layout", ctypes.c_int32), ("rms_eps", ctypes.c_float),
        ("router_w", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
        ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p),
    ]


class MoeVerifyError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m speculative_decoding_moe_amd._build`")
    lib = ctypes.CDLL(path)
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    lib.moe_verify_workspace_size.argtypes = [ctypes.POINTER(MoeLayerStruct), i32]
    lib.moe_verify_workspace_size.restype = sz
    lib.moe_verify_block.argtypes = [ctypes.POINTER(MoeLayerStruct), vp, i32, u32, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_verify_block.restype = ctypes.c_int
    lib.moe_verify_block_timed.argtypes = [ctypes.POINTER(MoeLayerStruct), vp, i32, u32, vp, vp, vp, vp, vp, sz,
                                           vp, ctypes.POINTER(vp)]
    lib.moe_verify_block_timed.restype = ctypes.c_int
    lib.moe_verify_block_noalloc.argtypes = [ctypes.POINTER(MoeLayerStruct), vp, i32, u32, vp, vp, vp, vp, vp]
    lib.moe_verify_block_noalloc.restype = ctypes.c_int
    lib.moe_verify_stack_workspace_size.argtypes = [ctypes.POINTER(MoeLayerStruct), i32]
    lib.moe_verify_stack_workspace_size.restype = sz
    lib.moe_verify_stack.argtypes = [ctypes.POINTER(MoeLayerStruct), i32, vp, i32, u32, vp, vp, vp, sz, vp]
    lib.moe_verify_stack.restype = ctypes.c_int
    lib.moe_pack_weights.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.moe_pack_weights.restype = ctypes.c_int
    lib.accept_prefix_workspace_size.argtypes = [i32, i32]
    lib.accept_prefix_workspace_size.restype = sz
    lib.accept_prefix.argtypes = [vp, i32, i32, vp, i32, vp, vp, vp, sz, vp]
    lib.accept_prefix.restype = ctypes.c_int
    lib.accept_prefix_batch_workspace_size.argtypes = [i32, i32, i32]
    lib.accept_prefix_batch_workspace_size.restype = sz
    lib.accept_prefix_batch.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.accept_prefix_batch.restype = ctypes.c_int
    lib.lm_head_accept_workspace_size.argtypes = [i32, i32, i32]
    lib.lm_head_accept_workspace_size.restype = sz
    lib.lm_head_accept.argtypes = [vp, i32, i32, vp, i32, i32, vp, i32, vp, vp, vp, sz, vp]
    lib.lm_head_accept.restype = ctypes.c_int
    lib.accept_sample_workspace_size.argtypes = [i32, i32, i32]
    lib.accept_sample_workspace_size.restype = sz
    lib.accept_sample.argtypes = [vp, i32, i32, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
    lib.accept_sample.restype = ctypes.c_int
    lib.accept_sample_batch_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.accept_sample_batch_workspace_size.restype = sz
    lib.accept_sample_batch.argtypes = [vp, i32, i32, i32, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
    lib.accept_sample_batch.restype = ctypes.c_int
    lib.accept_histogram.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.accept_histogram.restype = ctypes.c_int
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.moe_status_string(int(status)).decode()


def _check(status: int):
    if status != MOE_OK:
        raise MoeVerifyError(status, status_string(status))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


import torch as _torch  # noqa: E402  (device tensors are torch tensors)

F32, I32, I64, U8 = (_torch.float32,), (_torch.int32,), (_torch.int64,), (_torch.uint8,)
_BITS16 = (_torch.bfloat16, _torch.int16, _torch.uint16, _torch.float16)


def _req(name, t, dtypes, shape=None, min_numel=None, optional=False):
    """Checks one tensor argument before the library sees its pointer: the C ABI gets no sizes
    or element types, so a wrong tensor would be read or written past its end on the device.
    dtypes: a tuple of torch dtypes (None: any); shape: a tuple whose None entries match any
    size; min_numel: a lower bound on the element count. Raises ValueError. (Kept to plain
    comparisons: it runs on every call of the hot path.)"""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, _torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if shape is not None:
        got = t.shape
        ok = len(got) == len(shape)
        if ok:
            for g, w in zip(got, shape):
                if w is not None and g != w:
                    ok = False
                    break
        if not ok:
            want = "(" + ", ".join("*" if d is None else str(int(d)) for d in shape) + ")"
            raise ValueError(f"{name} must have shape {want}, got {tuple(got)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors):
    """Every given tensor (None skipped) lives on a GPU device; checked after the element types and
    shapes of all arguments, so a host-side test reaches each of those checks."""
    for name in tensors:
        t = tensors[name]
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")


def _req_ws(workspace):
    _req("workspace", workspace, None)


def _stream_handle():
    import torch
    return torch.cuda.current_stream().cuda_stream


def pack_weights(src, src_scales=None, stream=None):
    """Tiled copy (MOE_LAYOUT_TILED) of stacked row-major matrices: bf16 src [n][rows][cols] (any
    16-bit dtype), or mxfp4 codes [n][rows][cols/2] uint8 with scales [n][rows][cols/32]. A 2-D
    input is one matrix. Returns (dst, dst_scales); library call."""
    import torch
    mx = src_scales is not None
    if src is None or src.dim() not in (2, 3):
        raise ValueError("src must be a 2-D or 3-D tensor")
    _req("src", src.contiguous(), U8 if mx else _BITS16)
    shp = tuple(src.shape) if src.dim() == 3 else (1,) + tuple(src.shape)
    if mx:
        _req("src_scales", src_scales.contiguous(), U8,
             shape=(shp[0], shp[1], shp[2] // 16) if src.dim() == 3 else (shp[1], shp[2] // 16))
    _on_gpu(src=src, src_scales=src_scales)
    n, rows = shp[0], shp[1]
    cols = shp[2] * 2 if mx else shp[2]
    src = src.contiguous()
    dst = torch.empty_like(src)
    dst_s = None
    if mx:
        src_scales = src_scales.contiguous()
        dst_s = torch.empty_like(src_scales)
    st = lib.moe_pack_weights(MOE_W_MXFP4 if mx else MOE_W_BF16, n, rows, cols, _ptr(src), _ptr(src_scales),
                              _ptr(dst), _ptr(dst_s), _stream_handle() if stream is None else stream)
    _check(st)
    return dst, dst_s


class MoeLayer:
    """Holds the device tensors of one MoE layer and the C descriptor that points at them.

    Expert matrices are in MOE_LAYOUT_TILED (see pack_weights / from_rowmajor): bf16 as 16-bit
    tensors, mxfp4 as uint8 code tensors plus uint8 scale tensors, with the documented shapes."""

    @classmethod
    def from_rowmajor(cls, **kw):
        """Packs row-major expert weights (pack_weights) and builds the layer from the copies."""
        t = dict(kw)
        mx = t.get("s_gate") is not None
        for n in ("gate", "up", "down"):
            if mx:
                t["w_" + n], t["s_" + n] = pack_weights(t["w_" + n], t["s_" + n])
            else:
                t["w_" + n], _ = pack_weights(t["w_" + n])
        for n in ("sh_gate", "sh_up", "sh_down"):
            if t.get(n) is not None:
                t[n], _ = pack_weights(t[n])
        return cls(**t)

    def __init__(self, *, hidden, n_experts, top_k, inter, shared_inter, router_w, w_gate, w_up,
                 w_down, s_gate=None, s_up=None, s_down=None, sh_gate=None, sh_up=None,
                 sh_down=None, rms_eps=1e-6, layout=MOE_LAYOUT_TILED):
        mx = s_gate is not None
        H, E, I, Is = int(hidden), int(n_experts), int(inter), int(shared_inter)
        wt = U8 if mx else _BITS16
        per = (lambda r, c: r * c // 2) if mx else (lambda r, c: r * c)
        _req("router_w", router_w, F32, min_numel=E * H)
        for n, t, (r, c) in (("w_gate", w_gate, (I, H)), ("w_up", w_up, (I, H)), ("w_down", w_down, (H, I))):
            _req(n, t, wt, min_numel=E * per(r, c))
        for n, t, (r, c) in (("s_gate", s_gate, (I, H)), ("s_up", s_up, (I, H)), ("s_down", s_down, (H, I))):
            _req(n, t, U8, min_numel=E * r * c // 32, optional=not mx)
        for n, t in (("sh_gate", sh_gate), ("sh_up", sh_up), ("sh_down", sh_down)):
            _req(n, t, _BITS16, min_numel=Is * H, optional=Is == 0)
        _on_gpu(router_w=router_w, w_gate=w_gate, w_up=w_up, w_down=w_down, s_gate=s_gate, s_up=s_up,
                s_down=s_down, sh_gate=sh_gate, sh_up=sh_up, sh_down=sh_down)
        self.tensors = dict(router_w=router_w, w_gate=w_gate, w_up=w_up, w_down=w_down,
                            s_gate=s_gate, s_up=s_up, s_down=s_down, sh_gate=sh_gate,
                            sh_up=sh_up, sh_down=sh_down)
        self.hidden, self.n_experts, self.top_k = hidden, n_experts, top_k
        self.inter, self.shared_inter = inter, shared_inter
        self.wdtype = MOE_W_MXFP4 if s_gate is not None else MOE_W_BF16
        self.struct = MoeLayerStruct(
            hidden, n_experts, top_k, inter, shared_inter, self.wdtype, layout, rms_eps,
            *(_ptr(self.tensors[n]) for n in ("router_w", "w_gate", "w_up", "w_down", "s_gate",
                                              "s_up", "s_down", "sh_gate", "sh_up", "sh_down")))

    def workspace_size(self, k_max: int) -> int:
        return int(lib.moe_verify_workspace_size(ctypes.byref(self.struct), int(k_max)))


def moe_verify_workspace_size(layer: MoeLayer, k_max: int) -> int:
    return layer.workspace_size(k_max)


def _check_block_args(layer, x, y, topk_ids, topk_w, n_woken, workspace):
    _req("x", x, F32, shape=(None, layer.hidden))
    k = int(x.shape[0])
    _req("y", y, F32, shape=(k, layer.hidden))
    _req("topk_ids", topk_ids, I32, shape=(k, layer.top_k), optional=True)
    _req("topk_w", topk_w, F32, shape=(k, layer.top_k), optional=True)
    _req("n_woken", n_woken, I32, min_numel=1, optional=True)
    _req("workspace", workspace, None, optional=True)
    _on_gpu(x=x, y=y, topk_ids=topk_ids, topk_w=topk_w, n_woken=n_woken, workspace=workspace)
    return k


def moe_verify_block(layer: MoeLayer, x, flags: int, y, topk_ids=None, topk_w=None, n_woken=None,
                     workspace=None, stream=None) -> None:
    """y = [x +] MoE([RMSNorm](x)) over a block of k = x.shape[0] tokens (library call)."""
    k = _check_block_args(layer, x, y, topk_ids, topk_w, n_woken, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.moe_verify_block(ctypes.byref(layer.struct), _ptr(x), k, int(flags), _ptr(y),
                              _ptr(topk_ids), _ptr(topk_w), _ptr(n_woken), _ptr(workspace),
                              ws_bytes, _stream_handle() if stream is None else stream)
    _check(st)


def moe_verify_block_noalloc(layer: MoeLayer, x, flags: int, y, topk_ids=None, topk_w=None, n_woken=None,
                             stream=None) -> None:
    """moe_verify_block on the library's own device scratch: allocates nothing (library call)."""
    k = _check_block_args(layer, x, y, topk_ids, topk_w, n_woken, None)
    st = lib.moe_verify_block_noalloc(ctypes.byref(layer.struct), _ptr(x), k, int(flags), _ptr(y), _ptr(topk_ids),
                                      _ptr(topk_w), _ptr(n_woken), _stream_handle() if stream is None else stream)
    _check(st)


def moe_verify_stack_workspace_size(layer: MoeLayer, k_max: int) -> int:
    return int(lib.moe_verify_stack_workspace_size(ctypes.byref(layer.struct), int(k_max)))


def moe_verify_stack(layers, x, flags: int, y, n_woken=None, workspace=None, stream=None) -> None:
    """y = L_{n-1}(... L_0(x)) over a block of k = x.shape[0] tokens, layers of one shape, in
    one library call: equal to chained moe_verify_block calls."""
    layers = list(layers)
    if not layers or len(layers) > STACK_MAX_LAYERS:
        raise ValueError(f"layers must hold 1..{STACK_MAX_LAYERS} MoeLayer objects")
    for i, L in enumerate(layers):
        if not isinstance(L, MoeLayer):
            raise ValueError(f"layers[{i}] must be a MoeLayer")
    k = _check_block_args(layers[0], x, y, None, None, None, workspace)
    _req("n_woken", n_woken, I32, min_numel=len(layers), optional=True)
    _on_gpu(n_woken=n_woken)
    arr = (MoeLayerStruct * len(layers))(*[L.struct for L in layers])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.moe_verify_stack(arr, len(layers), _ptr(x), k, int(flags), _ptr(y), _ptr(n_woken), _ptr(workspace),
                              ws_bytes, _stream_handle() if stream is None else stream)
    _check(st)


def moe_verify_block_timed(layer: MoeLayer, x, flags: int, y, events, topk_ids=None, topk_w=None,
                           n_woken=None, workspace=None, stream=None) -> None:
    """moe_verify_block that also records 5 caller-owned hipEvent_t handles at kernel boundaries."""
    if len(events) != 5:
        raise ValueError("events must hold 5 hipEvent_t handles")
    k = _check_block_args(layer, x, y, topk_ids, topk_w, n_woken, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ev = (ctypes.c_void_p * 5)(*[e for e in events])
    st = lib.moe_verify_block_timed(ctypes.byref(layer.struct), _ptr(x), k, int(flags), _ptr(y),
                                    _ptr(topk_ids), _ptr(topk_w), _ptr(n_woken), _ptr(workspace),
                                    ws_bytes, _stream_handle() if stream is None else stream, ev)
    _check(st)


def accept_prefix_workspace_size(n_target: int, vocab: int) -> int:
    return int(lib.accept_prefix_workspace_size(int(n_target), int(vocab)))


def accept_prefix_batch_workspace_size(n_seq: int, n_target: int, vocab: int) -> int:
    return int(lib.accept_prefix_batch_workspace_size(int(n_seq), int(n_target), int(vocab)))


def accept_prefix_batch(logits, draft_ids, target_ids, accepted, workspace, n_draft=None, stream=None) -> None:
    """accept_prefix for n_seq sequences at once (library call): logits [n_seq][n_target][V],
    draft_ids [n_seq][n_draft_max] or None, n_draft: optional int32 device tensor [n_seq] of
    per-sequence draft counts; target_ids [n_seq][n_target] and accepted [n_seq] are outputs."""
    _req("logits", logits, F32, shape=(None, None, None))
    n_seq, n_target, vocab = (int(v) for v in logits.shape)
    _req("draft_ids", draft_ids, I32, shape=(n_seq, None), optional=True)
    nd_max = int(draft_ids.shape[1]) if draft_ids is not None else 0
    _req("n_draft", n_draft, I32, shape=(n_seq,), optional=True)
    _req("target_ids", target_ids, I32, shape=(n_seq, n_target))
    _req("accepted", accepted, I32, shape=(n_seq,))
    _req_ws(workspace)
    _on_gpu(logits=logits, draft_ids=draft_ids, n_draft=n_draft, target_ids=target_ids, accepted=accepted,
            workspace=workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.accept_prefix_batch(_ptr(logits), n_seq, n_target, vocab, _ptr(draft_ids), nd_max, _ptr(n_draft),
                                 _ptr(target_ids), _ptr(accepted), _ptr(workspace), ws_bytes,
                                 _stream_handle() if stream is None else stream)
    _check(st)


def accept_prefix(logits, draft_ids, target_ids, accepted, workspace, n_draft=None, stream=None) -> None:
    """Per-row argmax of logits [n_target][V] and the greedy accepted length (library call)."""
    _req("logits", logits, F32, shape=(None, None))
    n_target, vocab = int(logits.shape[0]), int(logits.shape[1])
    nd = _draft_count(draft_ids, n_draft)
    _req("target_ids", target_ids, I32, min_numel=n_target)
    _req("accepted", accepted, I32, min_numel=1)
    _req_ws(workspace)
    _on_gpu(logits=logits, draft_ids=draft_ids, target_ids=target_ids, accepted=accepted, workspace=workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.accept_prefix(_ptr(logits), n_target, vocab, _ptr(draft_ids), nd, _ptr(target_ids),
                           _ptr(accepted), _ptr(workspace), ws_bytes,
                           _stream_handle() if stream is None else stream)
    _check(st)


def _draft_count(draft_ids, n_draft):
    """The number of drafts compared: all of draft_ids (int32, 1-D), or the first n_draft."""
    _req("draft_ids", draft_ids, I32, shape=(None,), optional=True)
    have = 0 if draft_ids is None else int(draft_ids.numel())
    nd = have if n_draft is None else int(n_draft)
    if nd < 0 or nd > have:
        raise ValueError(f"n_draft {nd} outside [0, {have}] (the drafts given)")
    return nd


def pack_head(w_rowmajor, stream=None):
    """Tiled copy of a bf16 output head [V][H] (any 16-bit dtype) for lm_head_accept: the rows
    are zero-padded to a multiple of 16, then packed (library call). Returns the packed tensor."""
    import torch
    V, H = int(w_rowmajor.shape[0]), int(w_rowmajor.shape[1])
    v16 = (V + 15) // 16 * 16
    src = w_rowmajor.contiguous()
    if v16 != V:
        src = torch.cat([src, torch.zeros((v16 - V, H), dtype=src.dtype, device=src.device)])
    dst, _ = pack_weights(src, stream=stream)
    return dst


def lm_head_accept_workspace_size(n_target: int, hidden: int, vocab: int) -> int:
    return int(lib.lm_head_accept_workspace_size(int(n_target), int(hidden), int(vocab)))


def lm_head_accept(h, w_head_tiled, vocab, draft_ids, target_ids, accepted, workspace, n_draft=None,
                   stream=None) -> None:
    """Output head h [n][H] . W[v] over v < vocab with the argmax fused, then the greedy accepted
    length (library call); w_head_tiled comes from pack_head."""
    _req("h", h, F32, shape=(None, None))
    n_target, hidden = int(h.shape[0]), int(h.shape[1])
    _req("w_head_tiled", w_head_tiled, _BITS16, min_numel=(int(vocab) + 15) // 16 * 16 * hidden)
    nd = _draft_count(draft_ids, n_draft)
    _req("target_ids", target_ids, I32, min_numel=n_target)
    _req("accepted", accepted, I32, min_numel=1)
    _req_ws(workspace)
    _on_gpu(h=h, w_head_tiled=w_head_tiled, draft_ids=draft_ids, target_ids=target_ids, accepted=accepted,
            workspace=workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.lm_head_accept(_ptr(h), n_target, hidden, _ptr(w_head_tiled), int(vocab), MOE_LAYOUT_TILED,
                            _ptr(draft_ids), nd, _ptr(target_ids), _ptr(accepted), _ptr(workspace), ws_bytes,
                            _stream_handle() if stream is None else stream)
    _check(st)


def accept_sample_workspace_size(n_target: int, n_draft: int, vocab: int) -> int:
    return int(lib.accept_sample_workspace_size(int(n_target), int(n_draft), int(vocab)))


def accept_sample_batch_workspace_size(n_seq: int, n_target: int, n_draft: int, vocab: int) -> int:
    return int(lib.accept_sample_batch_workspace_size(int(n_seq), int(n_target), int(n_draft), int(vocab)))


def accept_sample_batch(target_logits, draft_logits, draft_ids, temperature, u_accept, u_sample, accepted, token,
                        workspace, stream=None) -> None:
    """accept_sample for n_seq sequences at once (library call): target_logits [n_seq][n_target][V],
    draft_logits [n_seq][n_draft][V], draft_ids / u_accept [n_seq][n_draft], u_sample [n_seq][n_target];
    accepted and token [n_seq] are outputs. The draft arguments may be None with no drafts."""
    _req("target_logits", target_logits, F32, shape=(None, None, None))
    n_seq, n_target, vocab = (int(v) for v in target_logits.shape)
    _req("draft_ids", draft_ids, I32, shape=(n_seq, None), optional=True)
    n_draft = 0 if draft_ids is None else int(draft_ids.shape[1])
    _req("draft_logits", draft_logits, F32, shape=(n_seq, n_draft, vocab), optional=n_draft == 0)
    _req("u_accept", u_accept, F32, shape=(n_seq, n_draft), optional=n_draft == 0)
    _req("u_sample", u_sample, F32, shape=(n_seq, n_target))
    _req("accepted", accepted, I32, shape=(n_seq,))
    _req("token", token, I32, shape=(n_seq,))
    _req_ws(workspace)
    _on_gpu(target_logits=target_logits, draft_logits=draft_logits, draft_ids=draft_ids, u_accept=u_accept,
            u_sample=u_sample, accepted=accepted, token=token, workspace=workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.accept_sample_batch(_ptr(target_logits), n_seq, n_target, vocab, _ptr(draft_logits), _ptr(draft_ids),
                                 n_draft, float(temperature), _ptr(u_accept), _ptr(u_sample), _ptr(accepted),
                                 _ptr(token), _ptr(workspace), ws_bytes, _stream_handle() if stream is None else stream)
    _check(st)


def accept_sample(target_logits, draft_logits, draft_ids, temperature, u_accept, u_sample, accepted, token,
                  workspace, stream=None) -> None:
    """Lossless acceptance at temperature T (library call): accepted[0] = a, token[0] = the
    target's own token (or -1). draft_logits / draft_ids / u_accept may be None with no drafts."""
    _req("target_logits", target_logits, F32, shape=(None, None))
    n_target, vocab = int(target_logits.shape[0]), int(target_logits.shape[1])
    _req("draft_ids", draft_ids, I32, shape=(None,), optional=True)
    n_draft = 0 if draft_ids is None else int(draft_ids.shape[0])
    _req("draft_logits", draft_logits, F32, shape=(n_draft, vocab), optional=n_draft == 0)
    _req("u_accept", u_accept, F32, min_numel=n_draft, optional=n_draft == 0)
    _req("u_sample", u_sample, F32, min_numel=n_target)
    _req("accepted", accepted, I32, min_numel=1)
    _req("token", token, I32, min_numel=1)
    _req_ws(workspace)
    _on_gpu(target_logits=target_logits, draft_logits=draft_logits, draft_ids=draft_ids, u_accept=u_accept,
            u_sample=u_sample, accepted=accepted, token=token, workspace=workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.accept_sample(_ptr(target_logits), n_target, vocab, _ptr(draft_logits), _ptr(draft_ids), n_draft,
                           float(temperature), _ptr(u_accept), _ptr(u_sample), _ptr(accepted), _ptr(token),
                           _ptr(workspace), ws_bytes, _stream_handle() if stream is None else stream)
    _check(st)


def accept_histogram(accepted, n_draft, hist, survival, stream=None) -> None:
    """Histogram of accepted lengths and the per-position survival counts (library call)."""
    nd = int(n_draft)
    _req("accepted", accepted, I32, shape=(None,))
    _req("hist", hist, I64, min_numel=max(nd + 1, 1))
    _req("survival", survival, I64, min_numel=max(nd, 0), optional=nd == 0)
    _on_gpu(accepted=accepted, hist=hist, survival=survival)
    st = lib.accept_histogram(_ptr(accepted), int(accepted.numel()), int(n_draft), _ptr(hist), _ptr(survival),
                              _stream_handle() if stream is None else stream)
    _check(st)
