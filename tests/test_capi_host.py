"""The C ABI library on the host (no GPU): it loads, exports every function
include/tsd_attn.h declares, and rejects bad arguments with the documented
status codes before making any HIP call."""
import ctypes
import os
import re

import pytest

import transformer_scaled_dot_amd as tsd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsd_attn.h")

EINVAL, EUNSUP = 1, 2
BF16, F32 = 1, 0


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    return re.findall(r"TSD_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tsd.library_path()):
        import __graft_entry__

        __graft_entry__.build()
    return tsd.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert sorted(names) == sorted(tsd.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.attn_status_string(0) == b"ok"
    assert lib.attn_status_string(1) == b"invalid argument"
    assert lib.attn_status_string(2) == b"unsupported configuration"
    assert lib.attn_status_string(3) == b"HIP error"
    assert lib.attn_status_string(99) == b"unknown status"


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced: every call below fails validation


def call_attn(lib, Q=FAKE, K=FAKE + (1 << 28), V=FAKE + (2 << 28), mask=0, vl=0, scale=0.125, O=FAKE + (3 << 28),
              B=1, H=1, Nq=8, Nk=8, d=64, ind=BF16, outd=BF16):
    P = ctypes.c_void_p
    return lib.attn_fwd(P(Q), P(K), P(V), mask, P(vl), ctypes.c_float(scale), P(O), B, H, Nq, Nk, d, ind, outd,
                        P(0))


@pytest.mark.parametrize("kw,status", [
    (dict(Q=0), EINVAL),
    (dict(O=0), EINVAL),
    (dict(K=0), EINVAL),
    (dict(B=-1), EINVAL),
    (dict(d=0), EINVAL),
    (dict(mask=7), EINVAL),
    (dict(ind=5), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(scale=float("inf")), EINVAL),
    (dict(mask=2, vl=0), EINVAL),
    (dict(Q=FAKE + 2), EINVAL),
    (dict(O=FAKE), EINVAL),                       # O aliases Q
    (dict(scale=-1.0), EUNSUP),
    (dict(d=32), EUNSUP),                         # bf16 needs 64 or 128
    (dict(d=48, ind=F32, outd=F32), EUNSUP),
    (dict(ind=F32, outd=BF16, d=64), EUNSUP),
    (dict(mask=1, Nq=8, Nk=9), EUNSUP),
])
def test_attn_fwd_rejects(lib, kw, status):
    assert call_attn(lib, **kw) == status
    assert lib.attn_last_error() != b""


def call_attn_ex(lib, Q=FAKE, K=FAKE + (1 << 28), V=FAKE + (2 << 28), mask=0, vl=0, scale=0.125, O=FAKE + (3 << 28),
                 lse=0, B=1, H=4, Hkv=2, Nq=8, Nk=8, d=64, ind=BF16, outd=BF16):
    P = ctypes.c_void_p
    return lib.attn_fwd_ex(P(Q), P(K), P(V), mask, P(vl), ctypes.c_float(scale), P(O), P(lse), B, H, Hkv, Nq, Nk, d,
                           ind, outd, P(0))


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=0), EINVAL),
    (dict(Hkv=3), EINVAL),                        # does not divide H = 4
    (dict(Hkv=-2), EINVAL),
    (dict(mask=3, vl=0), EINVAL),                 # causal and padding need valid_lens
    (dict(mask=4), EINVAL),
    (dict(lse=FAKE + (4 << 28) + 2), EINVAL),     # lse misaligned
    (dict(lse=FAKE + (3 << 28)), EINVAL),         # lse overlaps O
    (dict(lse=FAKE), EINVAL),                     # lse overlaps Q
    (dict(mask=3, vl=FAKE + (5 << 28), Nq=8, Nk=9), EUNSUP),
    (dict(d=32), EUNSUP),
])
def test_attn_fwd_ex_rejects(lib, kw, status):
    assert call_attn_ex(lib, **kw) == status
    assert lib.attn_last_error() != b""


def test_attn_fwd_ex_empty_is_ok_without_gpu(lib):
    assert call_attn_ex(lib, Nq=0, lse=FAKE + (4 << 28)) == 0
    assert call_attn_ex(lib, B=0, mask=3, vl=FAKE + (5 << 28)) == 0


def test_attn_fwd_empty_is_ok_without_gpu(lib):
    # no output element: nothing is launched
    assert call_attn(lib, Nq=0) == 0
    assert call_attn(lib, B=0) == 0


def call_weights(lib, Q=FAKE, K=FAKE + (1 << 28), mask=0, vl=0, scale=0.125, A=FAKE + (2 << 28), B=1, H=2, Hkv=2,
                 Nq=8, Nk=8, d=64, dt=BF16):
    P = ctypes.c_void_p
    return lib.attn_weights(P(Q), P(K), mask, P(vl), ctypes.c_float(scale), P(A), B, H, Hkv, Nq, Nk, d, dt, P(0))


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), EINVAL),
    (dict(d=0), EINVAL),
    (dict(Hkv=3), EINVAL),
    (dict(mask=5), EINVAL),
    (dict(dt=9), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(Q=0), EINVAL),
    (dict(A=0), EINVAL),
    (dict(mask=2, vl=0), EINVAL),
    (dict(A=FAKE + (2 << 28) + 2), EINVAL),       # A not 4-byte aligned
    (dict(A=FAKE), EINVAL),                       # A overlaps Q
    (dict(Q=FAKE + 1), EINVAL),                   # bf16 Q not 2-byte aligned
    (dict(scale=-1.0), EUNSUP),
    (dict(Nk=1025, Nq=8), EUNSUP),                # only short key sequences
    (dict(d=257), EUNSUP),
    (dict(mask=1, Nq=8, Nk=9), EUNSUP),
])
def test_attn_weights_rejects(lib, kw, status):
    assert call_weights(lib, **kw) == status
    assert lib.attn_last_error() != b""


def test_attn_weights_empty_is_ok_without_gpu(lib):
    assert call_weights(lib, Nq=0) == 0
    assert call_weights(lib, Nk=0, Q=0, K=0, A=0) == 0


GB = 1 << 28  # spacing of the fake buffers below: no two overlap at the sizes used


def call_bwd(lib, Q=FAKE, K=FAKE + GB, V=FAKE + 2 * GB, O=FAKE + 3 * GB, dO=FAKE + 4 * GB, lse=FAKE + 5 * GB, mask=0,
             vl=0, scale=0.125, dQ=FAKE + 6 * GB, dK=FAKE + 7 * GB, dV=FAKE + 8 * GB, B=1, H=4, Hkv=2, Nq=8, Nk=8,
             d=64, dt=BF16, ws=FAKE + 9 * GB, wsb=1 << 20):
    P = ctypes.c_void_p
    return lib.attn_bwd(P(Q), P(K), P(V), P(O), P(dO), P(lse), mask, P(vl), ctypes.c_float(scale), P(dQ), P(dK),
                        P(dV), B, H, Hkv, Nq, Nk, d, dt, P(ws), ctypes.c_size_t(wsb), P(0))


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), EINVAL),                           # negative size
    (dict(Nk=-3), EINVAL),
    (dict(d=0), EINVAL),                            # head_dim <= 0
    (dict(Hkv=0), EINVAL),                          # kv_heads not positive
    (dict(Hkv=3), EINVAL),                          # does not divide H = 4
    (dict(mask=-1), EINVAL),                        # unknown mask kind
    (dict(mask=4), EINVAL),
    (dict(dt=7), EINVAL),                           # unknown dtype
    (dict(scale=float("nan")), EINVAL),             # scale not finite
    (dict(scale=float("-inf")), EINVAL),
    (dict(scale=-0.5), EUNSUP),                     # negative scale
    (dict(dt=F32), EUNSUP),                         # only bf16
    (dict(d=32), EUNSUP),                           # head_dim 64 or 128
    (dict(mask=1, Nq=8, Nk=9), EUNSUP),             # causal needs seq_q == seq_k
    (dict(mask=3, vl=FAKE + 10 * GB, Nq=9, Nk=8), EUNSUP),
    (dict(Q=0), EINVAL),                            # null pointers on the query side
    (dict(O=0), EINVAL),
    (dict(dO=0), EINVAL),
    (dict(lse=0), EINVAL),
    (dict(dQ=0), EINVAL),
    (dict(K=0), EINVAL),                            # and on the key side
    (dict(V=0), EINVAL),
    (dict(dK=0), EINVAL),
    (dict(dV=0), EINVAL),
    (dict(mask=2, vl=0), EINVAL),                   # padding needs valid_lens
    (dict(mask=3, vl=0), EINVAL),
    (dict(ws=0), EINVAL),                           # workspace missing
    (dict(wsb=255), EINVAL),                        # workspace too small (needs 2 * 4 * 64 * 4 bytes)
    (dict(Q=FAKE + 8), EINVAL),                     # tensors 16-byte aligned
    (dict(dV=FAKE + 8 * GB + 4), EINVAL),
    (dict(lse=FAKE + 5 * GB + 2), EINVAL),          # lse 4-byte aligned
    (dict(mask=2, vl=FAKE + 10 * GB + 1), EINVAL),  # valid_lens 4-byte aligned
    (dict(ws=FAKE + 9 * GB + 16), EINVAL),          # workspace 256-byte aligned
    (dict(dQ=FAKE), EINVAL),                        # an output overlaps an input
    (dict(dK=FAKE + 5 * GB), EINVAL),               # dK over lse
    (dict(ws=FAKE + 3 * GB), EINVAL),               # the workspace over O
    (dict(dK=FAKE + 6 * GB), EINVAL),               # outputs overlap each other
    (dict(ws=FAKE + 8 * GB), EINVAL),               # the workspace over dV
])
def test_attn_bwd_rejects(lib, kw, status):
    assert call_bwd(lib, **kw) == status
    assert lib.attn_last_error() != b""


def test_attn_bwd_empty_is_ok_without_gpu(lib):
    assert call_bwd(lib, Nq=0, Nk=0) == 0
    assert call_bwd(lib, B=0, Q=0, K=0, V=0, O=0, dO=0, lse=0, dQ=0, dK=0, dV=0, ws=0, wsb=0) == 0


def test_attn_bwd_workspace_bytes(lib):
    # lse * log2(e) and D per query row, float32, rows padded to whole 64-row tiles, rounded up to 256 bytes
    assert lib.attn_bwd_workspace_bytes(4, 16, 4096) == 2 * 4 * 16 * 4096 * 4
    assert lib.attn_bwd_workspace_bytes(1, 3, 65) == 2 * 3 * 128 * 4
    assert lib.attn_bwd_workspace_bytes(1, 1, 1) == 512
    assert lib.attn_bwd_workspace_bytes(-1, 1, 1) == 0


def call_mha(lib, X=FAKE, W=FAKE + (1 << 28), Wo=FAKE + (2 << 28), h=8, O=FAKE + (3 << 28), B=1, N=16, dm=512,
             dt=BF16, ws=FAKE + (4 << 28), wsb=1 << 27):
    P = ctypes.c_void_p
    return lib.mha_fwd(P(X), P(W), P(Wo), h, P(O), B, N, dm, dt, P(ws), ctypes.c_size_t(wsb), P(0))


@pytest.mark.parametrize("kw,status", [
    (dict(X=0), EINVAL),
    (dict(ws=0), EINVAL),
    (dict(h=0), EINVAL),
    (dict(h=7), EINVAL),               # 512 % 7 != 0
    (dict(wsb=10), EINVAL),
    (dict(ws=FAKE + (4 << 28) + 16), EINVAL),  # workspace not 256-byte aligned
    (dict(O=FAKE), EINVAL),             # output aliases X
    (dict(dt=F32), EUNSUP),
    (dict(h=16), EUNSUP),               # d_k = 32
    (dict(dm=96, h=1), EUNSUP),         # d_k = 96
])
def test_mha_fwd_rejects(lib, kw, status):
    assert call_mha(lib, **kw) == status


def call_cross(lib, Xq=FAKE, Xkv=FAKE + (1 << 28), W=FAKE + (2 << 28), Wo=FAKE + (3 << 28), h=8, mask=0, vl=0,
               O=FAKE + (4 << 28), B=2, Nq=16, Nkv=24, dm=512, dt=BF16, ws=FAKE + (5 << 28), wsb=1 << 27):
    P = ctypes.c_void_p
    return lib.mha_cross_fwd(P(Xq), P(Xkv), P(W), P(Wo), h, mask, P(vl), P(O), B, Nq, Nkv, dm, dt, P(ws),
                             ctypes.c_size_t(wsb), P(0))


@pytest.mark.parametrize("kw,status", [
    (dict(Xq=0), EINVAL),
    (dict(Xkv=0), EINVAL),
    (dict(ws=0), EINVAL),
    (dict(h=7), EINVAL),
    (dict(Nkv=-1), EINVAL),
    (dict(mask=2, vl=0), EINVAL),                  # padding needs valid_lens
    (dict(mask=5), EINVAL),
    (dict(wsb=100), EINVAL),
    (dict(O=FAKE), EINVAL),                        # output aliases Xq
    (dict(ws=FAKE + (1 << 28)), EINVAL),           # workspace over Xkv
    (dict(mask=1), EUNSUP),                        # causal is for self-attention only
    (dict(mask=3, vl=FAKE + (6 << 28)), EUNSUP),
    (dict(dt=F32), EUNSUP),
    (dict(h=16), EUNSUP),                          # d_k = 32
])
def test_mha_cross_fwd_rejects(lib, kw, status):
    assert call_cross(lib, **kw) == status
    assert lib.attn_last_error() != b""


def test_mha_cross_workspace_bytes(lib):
    assert lib.mha_cross_workspace_bytes(4, 2048, 512, 512, 8, BF16) == (2 * 4 * 2048 + 2 * 4 * 512) * 512 * 2
    assert lib.mha_cross_workspace_bytes(1, 4, 4, 512, 7, BF16) == 0
    assert lib.mha_cross_workspace_bytes(1, 4, -1, 512, 8, BF16) == 0
    assert call_cross(lib, Nq=0) == 0  # no output row: nothing to do


def test_mha_workspace_bytes(lib):
    assert lib.mha_workspace_bytes(4, 2048, 512, 8, BF16) == 4 * 4 * 2048 * 512 * 2
    assert lib.mha_workspace_bytes(4, 2048, 512, 7, BF16) == 0
    assert lib.mha_workspace_bytes(4, 2048, 512, 8, F32) == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tsd.attn_fwd(q, q, q)
    x = torch.zeros(1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tsd.mha_fwd(x, torch.zeros(128, 384, dtype=torch.bfloat16), torch.zeros(128, 128, dtype=torch.bfloat16), 2)


@pytest.mark.parametrize("args", [(0, 256, 1000), (8, 0, 1000), (8, 65537, 1000), (8, 256, 0), (8, 256, 100001)])
def test_clock_probe_rejects(args):
    """The benchmark's clock probe lives in its own library, not in the attention library's exports."""
    from transformer_scaled_dot_amd import probe

    ptr, blocks, spin = args
    assert probe._load().tsd_probe_clock(ctypes.c_void_p(ptr), blocks, spin, None) == 1
    assert not hasattr(tsd.load_library(), "attn_clock_probe")
