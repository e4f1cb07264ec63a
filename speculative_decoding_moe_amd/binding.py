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

EXPORTS = ("moe_verify_workspace_size", "moe_verify_block", "moe_verify_block_timed",
           "moe_pack_weights", "accept_prefix_workspace_size", "accept_prefix",
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


def _stream_handle():
    import torch
    return torch.cuda.current_stream().cuda_stream


def pack_weights(src, src_scales=None, stream=None):
    """Tiled copy (MOE_LAYOUT_TILED) of stacked row-major matrices: bf16 src [n][rows][cols] (any
    16-bit dtype), or mxfp4 codes [n][rows][cols/2] uint8 with scales [n][rows][cols/32]. A 2-D
    input is one matrix. Returns (dst, dst_scales); library call."""
    import torch
    mx = src_scales is not None
    shp = tuple(src.shape) if src.dim() == 3 else (1,) + tuple(src.shape)
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


def moe_verify_block(layer: MoeLayer, x, flags: int, y, topk_ids=None, topk_w=None, n_woken=None,
                     workspace=None, stream=None) -> None:
    """y = [x +] MoE([RMSNorm](x)) over a block of k = x.shape[0] tokens (library call)."""
    k = int(x.shape[0])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.moe_verify_block(ctypes.byref(layer.struct), _ptr(x), k, int(flags), _ptr(y),
                              _ptr(topk_ids), _ptr(topk_w), _ptr(n_woken), _ptr(workspace),
                              ws_bytes, _stream_handle() if stream is None else stream)
    _check(st)


def moe_verify_block_timed(layer: MoeLayer, x, flags: int, y, events, topk_ids=None, topk_w=None,
                           n_woken=None, workspace=None, stream=None) -> None:
    """moe_verify_block that also records 5 caller-owned hipEvent_t handles at kernel boundaries."""
    k = int(x.shape[0])
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
    n_seq, n_target, vocab = (int(v) for v in logits.shape)
    nd_max = int(draft_ids.shape[1]) if draft_ids is not None else 0
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.accept_prefix_batch(_ptr(logits), n_seq, n_target, vocab, _ptr(draft_ids), nd_max, _ptr(n_draft),
                                 _ptr(target_ids), _ptr(accepted), _ptr(workspace), ws_bytes,
                                 _stream_handle() if stream is None else stream)
    _check(st)


def accept_prefix(logits, draft_ids, target_ids, accepted, workspace, n_draft=None, stream=None) -> None:
    """Per-row argmax of logits [n_target][V] and the greedy accepted length (library call)."""
    n_target, vocab = int(logits.shape[0]), int(logits.shape[1])
    nd = int(draft_ids.shape[0]) if (n_draft is None and draft_ids is not None) else int(n_draft or 0)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.accept_prefix(_ptr(logits), n_target, vocab, _ptr(draft_ids), nd, _ptr(target_ids),
                           _ptr(accepted), _ptr(workspace), ws_bytes,
                           _stream_handle() if stream is None else stream)
    _check(st)


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
    n_target, hidden = int(h.shape[0]), int(h.shape[1])
    nd = int(draft_ids.shape[0]) if (n_draft is None and draft_ids is not None) else int(n_draft or 0)
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
    n_seq, n_target, vocab = (int(v) for v in target_logits.shape)
    n_draft = 0 if draft_ids is None else int(draft_ids.shape[1])
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.accept_sample_batch(_ptr(target_logits), n_seq, n_target, vocab, _ptr(draft_logits), _ptr(draft_ids),
                                 n_draft, float(temperature), _ptr(u_accept), _ptr(u_sample), _ptr(accepted),
                                 _ptr(token), _ptr(workspace), ws_bytes, _stream_handle() if stream is None else stream)
    _check(st)


def accept_sample(target_logits, draft_logits, draft_ids, temperature, u_accept, u_sample, accepted, token,
                  workspace, stream=None) -> None:
    """Lossless acceptance at temperature T (library call): accepted[0] = a, token[0] = the
    target's own token (or -1). draft_logits / draft_ids / u_accept may be None with no drafts."""
    n_target, vocab = int(target_logits.shape[0]), int(target_logits.shape[1])
    n_draft = 0 if draft_ids is None else int(draft_ids.shape[0])
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.accept_sample(_ptr(target_logits), n_target, vocab, _ptr(draft_logits), _ptr(draft_ids), n_draft,
                           float(temperature), _ptr(u_accept), _ptr(u_sample), _ptr(accepted), _ptr(token),
                           _ptr(workspace), ws_bytes, _stream_handle() if stream is None else stream)
    _check(st)


def accept_histogram(accepted, n_draft, hist, survival, stream=None) -> None:
    """Histogram of accepted lengths and the per-position survival counts (library call)."""
    st = lib.accept_histogram(_ptr(accepted), int(accepted.numel()), int(n_draft), _ptr(hist), _ptr(survival),
                              _stream_handle() if stream is None else stream)
    _check(st)
