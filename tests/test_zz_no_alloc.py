"""attn_bwd_noalloc: the backward pass without a workspace argument, its per-row terms in the library's
static scratch array. On the host: sizes past the array are rejected before any HIP call. On an MI355X
(through the C ABI): two calls in a row, the second smaller, each equal bit for bit to attn_bwd with a
caller workspace on the same inputs (the same kernels run on the same values; attn_bwd's own parity with
the oracle is test_gpu_backward.py's)."""
import ctypes

import numpy as np
import pytest

import synth
import transformer_scaled_dot_amd as tsd

torch = pytest.importorskip("torch")

MASKS = {"none": 0, "causal": 1, "padding": 2, "causal_padding": 3}
FAKE = 1 << 20
GB = 1 << 28


def noalloc(lib, q, k, v, o, do, lse, dq, dk, dv, mask, vl, scale, dims, stream):
    B, H, Hkv, Nq, Nk, d = dims
    P = ctypes.c_void_p
    return lib.attn_bwd_noalloc(P(q), P(k), P(v), P(o), P(do), P(lse), MASKS[mask], P(vl), ctypes.c_float(scale),
                                P(dq), P(dk), P(dv), B, H, Hkv, Nq, Nk, d, 1, P(stream))


def test_noalloc_rejects_sizes_past_its_scratch():
    lib = tsd.load_library()
    cap = lib.attn_bwd_noalloc_max_scratch_bytes()
    assert cap == 8 << 20
    # 2^20 padded query rows fit exactly; one more 64-row tile does not
    assert lib.attn_bwd_workspace_bytes(1, 32, 32768) == cap
    args = [FAKE + i * GB for i in range(9)]
    st = noalloc(lib, *args[:6], *args[6:9], "none", 0, 0.125, (1, 32, 32, 32769, 8, 64), None)
    assert st == 1 and b"scratch" in lib.attn_last_error()
    # the ordinary argument checks come first
    st = noalloc(lib, 0, *args[1:6], *args[6:9], "none", 0, 0.125, (1, 2, 2, 8, 8, 64), None)
    assert st == 1


def _case(dev, seed, B, H, Hkv, N, d, mask, vl):
    q = synth.normal_tensor(seed, (B, H, N, d)).torch(dev)
    k = synth.normal_tensor(seed + 1, (B, Hkv, N, d)).torch(dev)
    v = synth.normal_tensor(seed + 2, (B, Hkv, N, d)).torch(dev)
    g = synth.normal_tensor(seed + 3, (B, H, N, d)).torch(dev)
    vl_t = torch.tensor(vl, dtype=torch.int32, device=dev) if vl is not None else None
    o, lse = tsd.attn_fwd(q, k, v, mask=mask, valid_lens=vl_t, return_lse=True)
    return q, k, v, g, o, lse, vl_t


@pytest.mark.gpu
def test_noalloc_matches_attn_bwd_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = tsd.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    # first a larger call (2 x 8 x 1000 rows), then a smaller one: the second reads only what it wrote
    for seed, (B, H, Hkv, N, d, mask, vl) in ((7100, (2, 8, 4, 1000, 128, "causal_padding", [1000, 613])),
                                               (7200, (1, 2, 1, 333, 64, "causal", None))):
        q, k, v, g, o, lse, vl_t = _case(dev, seed, B, H, Hkv, N, d, mask, vl)
        ref = tsd.attn_bwd(q, k, v, o, g, lse, mask=mask, valid_lens=vl_t)
        out = [torch.full_like(t, float("nan")) for t in (q, k, v)]
        scale = 1.0 / np.sqrt(d)
        st = noalloc(lib, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), g.data_ptr(), lse.data_ptr(),
                     out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(), mask,
                     vl_t.data_ptr() if vl_t is not None else 0, scale, (B, H, Hkv, N, N, d), stream)
        torch.cuda.synchronize()
        assert st == 0, lib.attn_last_error()
        for name, a, b in zip(("dQ", "dK", "dV"), out, ref):
            assert torch.equal(a, b), "%s differs from attn_bwd (seed %d)" % (name, seed)
        print("noalloc call seed %d [%d,%d/%d,%d,%d] %s: bit-identical to attn_bwd" % (seed, B, H, Hkv, N, d, mask),
              flush=True)
