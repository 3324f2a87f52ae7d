"""CPU oracle for scaled dot-product attention and the multi-head layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product package. It
shares no code with the HIP library (it is plain C, float64, in
``attn_oracle.c``, built with gcc).

Every function takes float64 numpy arrays holding the exact input values
(bfloat16 or float32 inputs widened to float64) and returns float64.

Masks: none, causal (key j hidden when j > i), padding (keys j >= valid_len[b])
and causal_padding (hidden by either rule). K/V may have fewer heads than Q:
query head h reads K/V head h // (H // H_kv) ("Self-Attention 机制", section
MHA -> MQA -> GQA -> MLA). The per-row log-sum-exp of the visible scaled
scores can be returned alongside the output, and attention_backward gives
the gradients with respect to Q, K and V by the chain rule.

Pins (tests/test_oracle_pins.py) tie it to what the pages fix: the
3-token hand-worked example of "04. Self-Attention: Transformer 的核心计算"
(section 六) and of "Transformer 详解" (section 手算一遍), row sums of 1,
exact zeros at masked positions, permutation equivariance, closed forms, and
torch's float64 CPU routines (attention, with grouped K/V heads, and
logsumexp) on tiny shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MASK = {"none": 0, "causal": 1, "padding": 2, "causal_padding": 3}
_USES_VALID_LENS = ("padding", "causal_padding")

_libs = {}


def compile_source(src: str, out: str) -> str:
    """gcc -O2 -fopenmp (IEEE float64, no fast-math) into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-Wall", src, "-o", tmp,
                           "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile attn_oracle.c unless an up-to-date library is present."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def _load(path: str | None = None):
    """The oracle library at ``path`` (default: the one built from
    attn_oracle.c). Other paths serve the planted-mistake tests, which
    compile altered copies of the source on the CPU."""
    if path is None:
        path = build()
    if path not in _libs:
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_attn.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, I64, ctypes.c_int, P, ctypes.c_double, P,
                                    P, P, ctypes.c_int]
        lib.oracle_attn.restype = ctypes.c_int
        lib.oracle_attn_rows.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, I64, ctypes.c_int, P,
                                         ctypes.c_double, P, I64, P, P, ctypes.c_int]
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, I64, ctypes.c_int, P,
                                        ctypes.c_double, P, P, P, ctypes.c_int]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_mha.argtypes = [P, P, P, I64, I64, I64, I64, P, ctypes.c_int]
        lib.oracle_mha.restype = ctypes.c_int
        lib.oracle_mha_cross.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, ctypes.c_int, P, P, ctypes.c_int]
        lib.oracle_mha_cross.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _libs[path] = lib
    return _libs[path]


def max_threads(lib=None) -> int:
    """Number of host threads an oracle call uses."""
    return int(_load(lib).oracle_max_threads())


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data) if a is not None else ctypes.c_void_p(0)


def _check_attn(q, k, v, mask, valid_lens):
    """q [B,H,Nq,d]; k, v [B,H_kv,Nk,d(v)] with H_kv dividing H (query head h reads K/V head
    h // (H // H_kv))."""
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if mask not in MASK:
        raise ValueError("unknown mask %r" % (mask,))
    B, H, Nq, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or Hkv < 1 or H % Hkv or v.shape[:3] != k.shape[:3] or k.shape[3] != d:
        raise ValueError("shape mismatch")
    vl = None
    if mask in _USES_VALID_LENS:
        if valid_lens is None:
            raise ValueError("padding mask needs valid_lens")
        vl = np.ascontiguousarray(valid_lens, dtype=np.int32)
        if vl.shape != (B,):
            raise ValueError("valid_lens must be [B]")
    return B, H, k.shape[1], Nq, k.shape[2], d, v.shape[3], vl


def attention(q, k, v, mask="none", valid_lens=None, scale=None, return_weights=False, threads=0, lib=None,
              return_lse=False):
    """O = softmax(q k^T * scale + M) v per (batch, head); optionally the
    weights A [B,H,Nq,Nk] and the per-row log-sum-exp of the visible scaled
    scores [B,H,Nq] (returned in that order after O). ``scale`` defaults to
    1/sqrt(d). k and v may have fewer heads than q (grouped K/V heads)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Hkv, Nq, Nk, d, dv, vl = _check_attn(q, k, v, mask, valid_lens)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    O = np.zeros((B, H, Nq, dv), dtype=np.float64)
    A = np.zeros((B, H, Nq, Nk), dtype=np.float64) if return_weights else None
    L = np.zeros((B, H, Nq), dtype=np.float64) if return_lse else None
    rc = _load(lib).oracle_attn(_ptr(q), _ptr(k), _ptr(v), B, H, Hkv, Nq, Nk, d, dv, MASK[mask], _ptr(vl), scale,
                             _ptr(O), _ptr(A), _ptr(L), int(threads))
    if rc < 0:
        raise ValueError("oracle_attn rejected its arguments")
    out = [O] + ([A] if return_weights else []) + ([L] if return_lse else [])
    return tuple(out) if len(out) > 1 else O


def attention_backward(q, k, v, do, mask="none", valid_lens=None, scale=None, threads=0, lib=None):
    """Gradients (dq, dk, dv) of sum(O * do) for O = attention(q, k, v, ...):
    the chain rule through the forward stages (softmax Jacobian included);
    dk, dv have k's and v's shapes (grouped K/V heads sum their query
    heads' contributions)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, Hkv, Nq, Nk, d, dv, vl = _check_attn(q, k, v, mask, valid_lens)
    if do.shape != (B, H, Nq, dv):
        raise ValueError("do must have the output's shape")
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    dq, dk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    rc = _load(lib).oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(do), B, H, Hkv, Nq, Nk, d, dv, MASK[mask],
                                 _ptr(vl), scale, _ptr(dq), _ptr(dk), _ptr(dvv), int(threads))
    if rc < 0:
        raise ValueError("oracle_attn_bwd rejected its arguments")
    return dq, dk, dvv


def attention_rows(q, k, v, rows, mask="none", valid_lens=None, scale=None, threads=0, lib=None, return_lse=False):
    """Output rows for flat indices r = (b*H + h)*Nq + i; returns [len(rows), dv]
    (and the rows' log-sum-exp [len(rows)] with ``return_lse``)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Hkv, Nq, Nk, d, dv, vl = _check_attn(q, k, v, mask, valid_lens)
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, dv), dtype=np.float64)
    L = np.zeros(rows.size, dtype=np.float64) if return_lse else None
    rc = _load(lib).oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v), B, H, Hkv, Nq, Nk, d, dv, MASK[mask], _ptr(vl),
                                  scale, _ptr(rows), rows.size, _ptr(O), _ptr(L), int(threads))
    if rc < 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return (O, L) if return_lse else O


def attention_rows_per_head(q, k, v, rows, mask="none", valid_lens=None, scale=None, threads=0, return_lse=False,
                            lib=None):
    """Like :func:`attention_rows`, but ``q, k, v`` may be any arrays that
    index as [b, h] -> [N, d] (e.g. float32 views of huge inputs): only the
    heads that the rows touch are widened to float64, one head at a time.
    Flat row r belongs to batch b, query head h = divmod(r // Nq, H) and
    query i = r % Nq; it reads K/V head h // (H // H_kv) of batch b and, for
    the padding masks, valid_lens[b]."""
    rows = np.asarray(rows, dtype=np.int64)
    H, Nq = q.shape[1], q.shape[2]
    grp = H // k.shape[1]
    out = np.zeros((rows.size, v.shape[3]), dtype=np.float64)
    lse = np.zeros(rows.size, dtype=np.float64)
    bh_of = rows // Nq
    for bh in np.unique(bh_of):
        b, h = divmod(int(bh), H)
        sel = np.nonzero(bh_of == bh)[0]
        vl = None if mask not in _USES_VALID_LENS else np.asarray([valid_lens[b]], dtype=np.int32)
        out[sel], lse[sel] = attention_rows(_f64(q[b, h])[None, None], _f64(k[b, h // grp])[None, None],
                                            _f64(v[b, h // grp])[None, None], rows[sel] % Nq, mask=mask,
                                            valid_lens=vl, scale=scale, threads=threads, return_lse=True, lib=lib)
    return (out, lse) if return_lse else out


def mha(x, w_qkv, w_o, h, threads=0, lib=None):
    """Multi-head layer: Y = concat_i softmax(Q_i K_i^T / sqrt(d_k)) V_i . W_o
    with [Q | K | V] = x W_qkv, no bias, no mask. x [B,N,d_model]."""
    x, w_qkv, w_o = _f64(x), _f64(w_qkv), _f64(w_o)
    B, N, dm = x.shape
    if w_qkv.shape != (dm, 3 * dm) or w_o.shape != (dm, dm) or dm % h:
        raise ValueError("bad mha shapes")
    Y = np.zeros((B, N, dm), dtype=np.float64)
    rc = _load(lib).oracle_mha(_ptr(x), _ptr(w_qkv), _ptr(w_o), B, N, dm, int(h), _ptr(Y), int(threads))
    if rc < 0:
        raise ValueError("oracle_mha rejected its arguments")
    return Y


def mha_cross(xq, xkv, w_qkv, w_o, h, mask="none", valid_lens=None, threads=0, lib=None):
    """Multi-head cross-attention layer: queries from xq [B,Nq,d_model], keys and values from xkv
    [B,Nkv,d_model], Q = xq W_Q and [K | V] = xkv [W_K | W_V] with W_qkv = [W_Q | W_K | W_V], heads split
    as in :func:`mha`, mask "none" or "padding" (keys j >= valid_lens[b] hidden), Y = concat . W_o."""
    xq, xkv, w_qkv, w_o = _f64(xq), _f64(xkv), _f64(w_qkv), _f64(w_o)
    B, Nq, dm = xq.shape
    if xkv.ndim != 3 or xkv.shape[0] != B or xkv.shape[2] != dm:
        raise ValueError("xkv must be [B, Nkv, d_model]")
    if w_qkv.shape != (dm, 3 * dm) or w_o.shape != (dm, dm) or dm % h:
        raise ValueError("bad mha shapes")
    if mask not in ("none", "padding"):
        raise ValueError("cross-attention masks: none or padding")
    vl = None
    if mask == "padding":
        vl = np.ascontiguousarray(valid_lens, dtype=np.int32)
        if vl.shape != (B,):
            raise ValueError("valid_lens must be [B]")
    Y = np.zeros((B, Nq, dm), dtype=np.float64)
    rc = _load(lib).oracle_mha_cross(_ptr(xq), _ptr(xkv), _ptr(w_qkv), _ptr(w_o), B, Nq, xkv.shape[1], dm, int(h),
                                     MASK[mask], _ptr(vl), _ptr(Y), int(threads))
    if rc < 0:
        raise ValueError("oracle_mha_cross rejected its arguments")
    return Y
