"""MI355X (gfx950) scaled dot-product attention forward and multi-head layer.

Thin ctypes binding over the C ABI of ``libtsd_attn.so`` (declared in
``include/tsd_attn.h``). This module only marshals arguments: PyTorch
supplies device memory and the current HIP stream, every arithmetic step runs
in the library's HIP kernels. There is no CPU fallback: if the library is not
built, or a tensor is not on the GPU, the call raises.

    attn_fwd(q, k, v, mask="none"|"causal"|"padding"|"causal_padding",
             valid_lens=None, scale=None, out_dtype=None, return_lse=False)
             -> o  (or (o, lse))
    attn_weights(q, k, mask=..., valid_lens=None, scale=None) -> A  (Nk <= 1024)
    attn_bwd(q, k, v, o, do, lse, mask=..., valid_lens=None, scale=None) -> (dq, dk, dv)
    mha_fwd(x, w_qkv, w_o, h) -> y
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["attn_fwd", "attn_weights", "attn_bwd", "mha_fwd", "mha_cross_fwd", "mha_workspace_bytes", "library_path", "load_library", "AttnError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtsd_attn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP = 0, 1, 2, 3
MASK_KINDS = {"none": 0, "causal": 1, "padding": 2, "causal_padding": 3}
DTYPE_F32, DTYPE_BF16 = 0, 1

EXPORTS = ("attn_fwd", "attn_fwd_ex", "attn_weights", "attn_bwd", "attn_bwd_workspace_bytes", "attn_bwd_noalloc",
           "attn_bwd_noalloc_max_scratch_bytes", "mha_workspace_bytes", "mha_fwd", "mha_cross_workspace_bytes",
           "mha_cross_fwd", "attn_status_string",
           "attn_last_error")

_lib = None


class AttnError(RuntimeError):
    """A HIP-side failure reported by the library (ATTN_EHIP)."""


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libtsd_attn.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libtsd_attn.so is not built; run `python -m transformer_scaled_dot_amd.build` "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.attn_fwd.argtypes = [P, P, P, I32, P, ctypes.c_float, P, I32, I32, I32, I32, I32, I32, I32, P]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_ex.argtypes = [P, P, P, I32, P, ctypes.c_float, P, P, I32, I32, I32, I32, I32, I32, I32, I32, P]
    lib.attn_fwd_ex.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, I32, P, ctypes.c_float, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                             P, ctypes.c_size_t, P]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_weights.argtypes = [P, P, I32, P, ctypes.c_float, P, I32, I32, I32, I32, I32, I32, I32, P]
    lib.attn_weights.restype = ctypes.c_int
    lib.attn_bwd_workspace_bytes.argtypes = [I32, I32, I32]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, I32, P, ctypes.c_float, P, P, P, I32, I32, I32, I32, I32, I32,
                                     I32, P]
    lib.attn_bwd_noalloc.restype = ctypes.c_int
    lib.attn_bwd_noalloc_max_scratch_bytes.argtypes = []
    lib.attn_bwd_noalloc_max_scratch_bytes.restype = ctypes.c_size_t
    lib.mha_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.mha_workspace_bytes.restype = ctypes.c_size_t
    lib.mha_fwd.argtypes = [P, P, P, I32, P, I32, I32, I32, I32, P, ctypes.c_size_t, P]
    lib.mha_fwd.restype = ctypes.c_int
    lib.mha_cross_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.mha_cross_workspace_bytes.restype = ctypes.c_size_t
    lib.mha_cross_fwd.argtypes = [P, P, P, P, I32, I32, P, P, I32, I32, I32, I32, I32, P, ctypes.c_size_t, P]
    lib.mha_cross_fwd.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [I32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _raise_for(lib, status: int, what: str):
    if status == ATTN_OK:
        return
    msg = "%s: %s (%s)" % (what, lib.attn_status_string(status).decode(), lib.attn_last_error().decode())
    if status == ATTN_EHIP:
        raise AttnError(msg)
    raise ValueError(msg)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise ValueError("unsupported dtype %s (bfloat16 or float32)" % t.dtype)


def _check_gpu(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU (got %s)" % t.device)
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream_ptr(device):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def attn_fwd(q, k, v, mask: str = "none", valid_lens=None, scale: float | None = None, out_dtype=None, out=None,
             return_lse: bool = False, lse=None):
    """O = softmax(q k^T * scale + M) v for q [B,H,Nq,d], k, v [B,H_kv,Nk,d].

    ``mask``: "none", "causal" (key j > query i hidden), "padding" (key j
    >= valid_lens[b] hidden; ``valid_lens`` an int32 GPU tensor [B]) or
    "causal_padding" (hidden by either rule). k and v may have H_kv heads,
    H_kv dividing H: query head h reads K/V head h // (H // H_kv).
    ``scale`` defaults to 1/sqrt(d). ``out_dtype`` defaults to q's dtype;
    bf16 inputs may request a float32 output. With ``return_lse`` (or an
    ``lse`` tensor given) the call also returns the float32 [B,H,Nq]
    log-sum-exp of each row's visible scaled scores. Enqueued on the
    current stream.
    """
    import torch

    lib = load_library()
    if mask not in MASK_KINDS:
        raise ValueError("mask must be one of %s" % sorted(MASK_KINDS))
    _check_gpu(q, k, v, valid_lens, lse)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != (B, Hkv, Nk, d):
        raise ValueError("k and v must be [B, H_kv, Nk, d] matching q")
    if Hkv < 1 or H % Hkv:
        raise ValueError("the K/V head count must divide the query head count")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if mask in ("padding", "causal_padding"):
        if valid_lens is None or valid_lens.dtype != torch.int32 or tuple(valid_lens.shape) != (B,):
            raise ValueError("%s mask needs valid_lens: int32 GPU tensor of shape [B]" % mask)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    else:
        _check_gpu(out)
        if tuple(out.shape) != (B, H, Nq, d) or out.dtype != out_dtype:
            raise ValueError("out has the wrong shape or dtype")
    if lse is not None:
        if tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
            raise ValueError("lse must be a float32 [B, H, Nq] tensor")
    elif return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    uses_lens = mask in ("padding", "causal_padding")
    st = lib.attn_fwd_ex(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                         ctypes.c_void_p(v.data_ptr()), MASK_KINDS[mask],
                         ctypes.c_void_p(valid_lens.data_ptr() if uses_lens else 0), ctypes.c_float(scale),
                         ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr() if lse is not None else 0),
                         B, H, Hkv, Nq, Nk, d, _dtype_code(q), _dtype_code(out), _stream_ptr(q.device))
    _raise_for(lib, st, "attn_fwd")
    return (out, lse) if lse is not None else out


def attn_weights(q, k, mask: str = "none", valid_lens=None, scale: float | None = None):
    """The attention weights A = softmax(q k^T * scale + M), float32 [B, H, Nq, Nk], for short key
    sequences (Nk <= 1024): the pages' second result of attention. q [B,H,Nq,d], k [B,H_kv,Nk,d] (bf16 or
    float32); masks, valid_lens and scale as for attn_fwd. Enqueued on the current stream."""
    import torch

    lib = load_library()
    if mask not in MASK_KINDS:
        raise ValueError("mask must be one of %s" % sorted(MASK_KINDS))
    _check_gpu(q, k, valid_lens)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k must be 4-D [B, H, N, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d or k.dtype != q.dtype:
        raise ValueError("k must be [B, H_kv, Nk, d] with q's dtype")
    uses_lens = mask in ("padding", "causal_padding")
    if uses_lens and (valid_lens is None or valid_lens.dtype != torch.int32 or tuple(valid_lens.shape) != (B,)):
        raise ValueError("%s mask needs valid_lens: int32 GPU tensor of shape [B]" % mask)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    a = torch.empty((B, H, Nq, Nk), dtype=torch.float32, device=q.device)
    P = ctypes.c_void_p
    st = lib.attn_weights(P(q.data_ptr()), P(k.data_ptr()), MASK_KINDS[mask],
                          P(valid_lens.data_ptr() if uses_lens else 0), ctypes.c_float(scale), P(a.data_ptr()), B, H,
                          Hkv, Nq, Nk, d, _dtype_code(q), _stream_ptr(q.device))
    _raise_for(lib, st, "attn_weights")
    return a


def attn_bwd(q, k, v, o, do, lse, mask: str = "none", valid_lens=None, scale: float | None = None, workspace=None):
    """Gradients (dq, dk, dv) of attn_fwd's output with respect to q, k and v, given the output gradient
    ``do``, the forward's output ``o`` and its log-sum-exp ``lse`` (from attn_fwd(..., return_lse=True)
    with the same inputs, mask and scale). bf16, head_dim 64 or 128; k and v may have H_kv heads.
    Enqueued on the current stream."""
    import torch

    lib = load_library()
    if mask not in MASK_KINDS:
        raise ValueError("mask must be one of %s" % sorted(MASK_KINDS))
    _check_gpu(q, k, v, o, do, lse, valid_lens, workspace)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != (B, Hkv, Nk, d):
        raise ValueError("k and v must be [B, H_kv, Nk, d] matching q")
    if tuple(o.shape) != tuple(q.shape) or tuple(do.shape) != tuple(q.shape):
        raise ValueError("o and do must have q's shape")
    if tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, Nq] tensor")
    if Hkv < 1 or H % Hkv:
        raise ValueError("the K/V head count must divide the query head count")
    uses_lens = mask in ("padding", "causal_padding")
    if uses_lens and (valid_lens is None or valid_lens.dtype != torch.int32 or tuple(valid_lens.shape) != (B,)):
        raise ValueError("%s mask needs valid_lens: int32 GPU tensor of shape [B]" % mask)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = int(lib.attn_bwd_workspace_bytes(B, H, Nq))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    P = ctypes.c_void_p
    st = lib.attn_bwd(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), P(do.data_ptr()),
                      P(lse.data_ptr()), MASK_KINDS[mask], P(valid_lens.data_ptr() if uses_lens else 0),
                      ctypes.c_float(scale), P(dq.data_ptr()), P(dk.data_ptr()), P(dv.data_ptr()), B, H, Hkv, Nq,
                      Nk, d, _dtype_code(q), P(workspace.data_ptr()),
                      ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream_ptr(q.device))
    _raise_for(lib, st, "attn_bwd")
    return dq, dk, dv


def mha_workspace_bytes(batch: int, seq: int, d_model: int, h: int, dtype=None) -> int:
    import torch

    code = DTYPE_BF16 if dtype in (None, torch.bfloat16) else DTYPE_F32
    return int(load_library().mha_workspace_bytes(batch, seq, d_model, h, code))


def mha_fwd(x, w_qkv, w_o, h: int, out=None, workspace=None):
    """Multi-head self-attention layer without bias or mask:
    y = concat_i softmax(Q_i K_i^T / sqrt(d_k)) V_i . w_o with
    [Q | K | V] = x w_qkv; x [B, N, d_model], w_qkv [d_model, 3 d_model],
    w_o [d_model, d_model], all bf16 on the GPU."""
    import torch

    lib = load_library()
    _check_gpu(x, w_qkv, w_o)
    if x.dim() != 3:
        raise ValueError("x must be [B, N, d_model]")
    B, N, dm = x.shape
    if tuple(w_qkv.shape) != (dm, 3 * dm) or tuple(w_o.shape) != (dm, dm):
        raise ValueError("w_qkv must be [d_model, 3 d_model] and w_o [d_model, d_model]")
    if w_qkv.dtype != x.dtype or w_o.dtype != x.dtype:
        raise ValueError("x, w_qkv, w_o must share a dtype")
    need = int(lib.mha_workspace_bytes(B, N, dm, int(h), _dtype_code(x)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    else:
        _check_gpu(workspace)
    if out is None:
        out = torch.empty((B, N, dm), dtype=x.dtype, device=x.device)
    else:
        _check_gpu(out)
        if tuple(out.shape) != (B, N, dm) or out.dtype != x.dtype:
            raise ValueError("out has the wrong shape or dtype")
    st = lib.mha_fwd(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w_qkv.data_ptr()),
                     ctypes.c_void_p(w_o.data_ptr()), int(h), ctypes.c_void_p(out.data_ptr()), B, N, dm,
                     _dtype_code(x), ctypes.c_void_p(workspace.data_ptr()),
                     ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream_ptr(x.device))
    _raise_for(lib, st, "mha_fwd")
    return out


def mha_cross_fwd(xq, xkv, w_qkv, w_o, h: int, mask: str = "none", valid_lens=None, out=None, workspace=None):
    """Multi-head cross-attention layer: queries from xq [B, Nq, d_model], keys and values from xkv
    [B, Nkv, d_model], the weights of mha_fwd (W_qkv [d_model, 3 d_model] = [W_Q | W_K | W_V], W_o);
    mask "none" or "padding" (keys j >= valid_lens[b] of xkv hidden). Returns [B, Nq, d_model]."""
    import torch

    lib = load_library()
    if mask not in ("none", "padding"):
        raise ValueError("cross-attention masks: none or padding")
    _check_gpu(xq, xkv, w_qkv, w_o, valid_lens, out, workspace)
    if xq.dim() != 3 or xkv.dim() != 3 or xkv.shape[0] != xq.shape[0] or xkv.shape[2] != xq.shape[2]:
        raise ValueError("xq [B, Nq, d_model] and xkv [B, Nkv, d_model] expected")
    B, Nq, dm = xq.shape
    Nkv = xkv.shape[1]
    if tuple(w_qkv.shape) != (dm, 3 * dm) or tuple(w_o.shape) != (dm, dm):
        raise ValueError("w_qkv must be [d_model, 3 d_model] and w_o [d_model, d_model]")
    if mask == "padding" and (valid_lens is None or valid_lens.dtype != torch.int32 or tuple(valid_lens.shape) != (B,)):
        raise ValueError("padding mask needs valid_lens: int32 GPU tensor of shape [B]")
    need = int(lib.mha_cross_workspace_bytes(B, Nq, Nkv, dm, int(h), _dtype_code(xq)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=xq.device)
    if out is None:
        out = torch.empty((B, Nq, dm), dtype=xq.dtype, device=xq.device)
    P = ctypes.c_void_p
    st = lib.mha_cross_fwd(P(xq.data_ptr()), P(xkv.data_ptr()), P(w_qkv.data_ptr()), P(w_o.data_ptr()), int(h),
                           MASK_KINDS[mask], P(valid_lens.data_ptr() if mask == "padding" else 0), P(out.data_ptr()),
                           B, Nq, Nkv, dm, _dtype_code(xq), P(workspace.data_ptr()),
                           ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream_ptr(xq.device))
    _raise_for(lib, st, "mha_cross_fwd")
    return out
