"""Parity of the HIP backward pass (attn_bwd, through the C ABI) with the CPU oracle's gradients, on an
MI355X. The GPU forward supplies O and the log-sum-exp, as in a training step.

Tolerance, per element, from the arithmetic of the bf16 path (u = 2^-8, the bf16 unit roundoff):
  * the weights P_ij are recomputed from the forward's log-sum-exp, which is within u of the exact one
    (test_gpu_features.py), and rounded to bf16 for the products: |dP| relative error <= 2u;
  * D_i = dO_i . O_i uses the forward's bf16 output: error <= u * sum_c |dO_ic O_ic|;
  * dS_ij = P_ij (dP_ij - D_i) is rounded to bf16 (u) on top of P's 2u;
so, with A the exact weights, dP_ij = dO_i . v_j and E_ij = A_ij (3u |dP_ij - D_i| + u sum_c |dO_ic O_ic|):
  |err dV_jc| <= 2u sum_i A_ij |dO_ic|,
  |err dQ_ic| <= scale sum_j E_ij |k_jc|,   |err dK_jc| <= scale sum_i E_ij |q_ic|,
each plus 1e-4 for the float32 accumulation and the final bf16 rounding of the gradient (u |grad|).
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U = 2.0 ** -8


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_scaled_dot_amd as tsd

    tsd.load_library()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def bounds(q, k, v, g, A, mask, vl, scale):
    """Per-element error bounds of the bf16 path for dQ, dK, dV (see the module docstring)."""
    B, H, Nq, d = q.shape
    Hkv = k.shape[1]
    grp = H // Hkv
    kh = np.repeat(k, grp, axis=1)
    vh = np.repeat(v, grp, axis=1)
    O = np.einsum("bhij,bhjc->bhic", A, vh)
    dP = np.einsum("bhic,bhjc->bhij", g, vh)
    Dl = np.sum(g * O, axis=-1)
    DO = np.sum(np.abs(g * O), axis=-1)
    E = A * (3 * U * np.abs(dP - Dl[..., None]) + U * DO[..., None])
    tq = scale * np.einsum("bhij,bhjc->bhic", E, np.abs(kh)) + 1e-4
    tk = scale * np.einsum("bhij,bhic->bhjc", E, np.abs(q))
    tv = 2 * U * np.einsum("bhij,bhic->bhjc", A, np.abs(g))
    tk = tk.reshape(B, Hkv, grp, -1, d).sum(axis=2) + 1e-4
    tv = tv.reshape(B, Hkv, grp, -1, d).sum(axis=2) + 1e-4
    return tq, tk, tv


def check(name, got, ref, tol):
    err = np.abs(got - ref)
    ratio = float((err / tol).max()) if err.size else 0.0
    say("%s: max abs err %.3e, max|ref| %.3e, worst err/bound %.3f" % (name, float(err.max()) if err.size else 0,
                                                                   float(np.abs(ref).max()) if ref.size else 0,
                                                                   ratio))
    assert np.all(np.isfinite(got)), name + ": non-finite gradient"
    assert ratio <= 1.0, name


def run_case(dev, seed, B, H, Hkv, Nq, Nk, d, mask, vl=None, scale=None):
    import transformer_scaled_dot_amd as tsd

    q = synth.normal_tensor(seed, (B, H, Nq, d))
    k = synth.normal_tensor(seed + 1, (B, Hkv, Nk, d))
    v = synth.normal_tensor(seed + 2, (B, Hkv, Nk, d))
    g = synth.normal_tensor(seed + 3, (B, H, Nq, d))
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    vl_t = torch.from_numpy(np.asarray(vl, dtype=np.int32)).to(dev) if vl is not None else None
    Q, K, V, G = q.torch(dev), k.torch(dev), v.torch(dev), g.torch(dev)
    o, lse = tsd.attn_fwd(Q, K, V, mask=mask, valid_lens=vl_t, scale=scale, return_lse=True)
    dq, dk, dv = tsd.attn_bwd(Q, K, V, o, G, lse, mask=mask, valid_lens=vl_t, scale=scale)
    torch.cuda.synchronize()
    got = [x.float().cpu().numpy().astype(np.float64) for x in (dq, dk, dv)]
    vlc = None if vl is None else np.minimum(np.asarray(vl, dtype=np.int32), Nk)
    ref = oracle.attention_backward(q.f64, k.f64, v.f64, g.f64, mask=mask, valid_lens=vlc, scale=scale)
    _, A = oracle.attention(q.f64, k.f64, v.f64, mask=mask, valid_lens=vlc, scale=scale, return_weights=True)
    tols = bounds(q.f64, k.f64, v.f64, g.f64, A, mask, vlc, scale)
    name = "bwd [%d,%d/%d,%d,%d] d%d %s" % (B, H, Hkv, Nq, Nk, d, mask)
    for what, x, r, t in zip(("dQ", "dK", "dV"), got, ref, tols):
        check("%s %s" % (name, what), x, r, t)


@pytest.mark.parametrize("mask", ["none", "causal", "padding", "causal_padding"])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_self_attention(dev, d, mask):
    run_case(dev, 4000 + d, 2, 2, 2, 300, 300, d, mask, vl=[130, 300])


@pytest.mark.parametrize("mask", ["none", "padding"])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_cross_attention(dev, d, mask):
    run_case(dev, 4100 + d, 2, 2, 2, 150, 270, d, mask, vl=[1, 200])


@pytest.mark.parametrize("hkv", [1, 2])
@pytest.mark.parametrize("mask", ["causal", "causal_padding"])
def test_backward_grouped_heads(dev, mask, hkv):
    run_case(dev, 4200 + hkv, 2, 4, hkv, 200, 200, 128, mask, vl=[0, 77])


def test_backward_ragged_and_tiny(dev):
    for (nq, nk) in [(1, 1), (5, 5), (64, 64), (129, 129)]:
        run_case(dev, 4300 + nq, 1, 2, 1, nq, nk, 64, "causal")
    run_case(dev, 4310, 1, 2, 2, 70, 33, 128, "none", scale=0.3)
    # scale 0: uniform weights over the visible keys, dQ = dK = 0; masked scores must still get weight 0
    for d in (64, 128):
        run_case(dev, 4320 + d, 2, 2, 1, 100, 100, d, "causal", scale=0.0)
        run_case(dev, 4330 + d, 2, 2, 2, 90, 150, d, "padding", vl=[17, 150], scale=0.0)
        run_case(dev, 4340 + d, 2, 2, 2, 130, 130, d, "causal_padding", vl=[0, 77], scale=0.0)


def test_backward_longer(dev):
    """1024 keys: many query tiles per key block and key tiles per query block."""
    run_case(dev, 4400, 1, 2, 1, 1024, 1024, 128, "causal")


@pytest.mark.timeout(600)
def test_backward_full_size_eight_heads(dev):
    """The causal 4K launch shape (B4 H16 N4096 d128): the backward runs on the whole workload and eight of
    its 64 (batch, head) slices, spread over the batches and heads, are compared element by element with the
    oracle (a head's gradients depend only on that head's Q, K, V and dO), within the same per-element
    bounds."""
    import transformer_scaled_dot_amd as tsd

    B, H, N, d = 4, 16, 4096, 128
    q, k, v, g = (synth.normal_tensor(4500 + i, (B, H, N, d)) for i in range(4))
    Q, K, V, G = q.torch(dev), k.torch(dev), v.torch(dev), g.torch(dev)
    o, lse = tsd.attn_fwd(Q, K, V, mask="causal", return_lse=True)
    dq, dk, dv = tsd.attn_bwd(Q, K, V, o, G, lse, mask="causal")
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(d)
    for b, h in ((0, 0), (0, 9), (1, 3), (1, 14), (2, 6), (2, 11), (3, 1), (3, 15)):
        sl = lambda t: t.f32[b:b + 1, h:h + 1].astype(np.float64)
        got = [x[b:b + 1, h:h + 1].float().cpu().numpy().astype(np.float64) for x in (dq, dk, dv)]
        ref = oracle.attention_backward(sl(q), sl(k), sl(v), sl(g), mask="causal", scale=scale)
        _, A = oracle.attention(sl(q), sl(k), sl(v), mask="causal", scale=scale, return_weights=True)
        tols = bounds(sl(q), sl(k), sl(v), sl(g), A, "causal", None, scale)
        for what, x, r, t in zip(("dQ", "dK", "dV"), got, ref, tols):
            check("bwd [4,16,4096,128] causal, head (%d,%d) %s" % (b, h, what), x, r, t)
