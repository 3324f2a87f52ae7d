"""Parity of attn_weights (the weight matrix A = softmax(Q K^T * scale + M) for short key sequences, the
pages' second result of attention) with the oracle's weights, through the C ABI, on an MI355X.

The scores and the softmax run in float32 for both input types (bf16 inputs are widened exactly), so A is
held to the float32 tolerance, max |A - A_ref| <= 1e-5, for both. Masked weights must be exactly 0 and
rows without a visible key all zero, as in the oracle."""
import json
import math

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_scaled_dot_amd as tsd

    tsd.load_library()
    return torch.device("cuda:0")


def weights(dev, q, k, mask, vl=None, scale=None):
    import transformer_scaled_dot_amd as tsd

    vl_t = torch.from_numpy(np.asarray(vl, dtype=np.int32)).to(dev) if vl is not None else None
    a = tsd.attn_weights(q.torch(dev), k.torch(dev), mask=mask, valid_lens=vl_t, scale=scale)
    torch.cuda.synchronize()
    return a.cpu().numpy().astype(np.float64)


def check(name, got, ref):
    err = np.abs(got - ref)
    print("%s: max abs err %.3e" % (name, float(err.max()) if err.size else 0.0), flush=True)
    assert np.all(np.isfinite(got))
    assert np.all(got[ref == 0.0] == 0.0), name + ": a masked weight is not exactly 0"
    assert float(err.max()) <= TOL, name


def test_hand_example_weights(dev, golden_dir):
    """The pages' 3-token example (d_k = 2, Q = K = X): page 4's printed weight matrix and page 1's row 3."""
    g = json.load(open(golden_dir + "/hand_example.json", encoding="utf-8"))
    X = np.asarray(g["X"], dtype=np.float32)[None, None]
    t = synth.Tensor(X.copy(), "f32", X.shape)
    got = weights(dev, t, t, "none")
    _, ref = oracle.attention(X, X, X, return_weights=True)
    check("hand example A", got, ref)
    W = np.asarray(g["page4"]["weights_as_printed_flat"]).reshape(3, 3).T
    np.testing.assert_allclose(got[0, 0], W, atol=g["page4"]["tol"])
    np.testing.assert_allclose(got[0, 0, 2], g["page1"]["row3_weights"], atol=g["page1"]["tol"])
    np.testing.assert_allclose(got.sum(axis=-1), 1.0, atol=1e-6)


# the causal masks are defined for seq_q == seq_k (the entry point rejects the rest): only those pairs take them
WEIGHT_CASES = [(nq, nk, d, mask) for nq, nk, d in [(5, 5, 16), (70, 70, 64), (130, 130, 128), (64, 1024, 128),
                                                    (33, 1000, 64)]
                for mask in ["none", "causal", "padding", "causal_padding"] if nq == nk or not mask.startswith("causal")]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nq,nk,d,mask", WEIGHT_CASES)
def test_weights_match_oracle(dev, dtype, mask, nq, nk, d):
    B, H = 2, 2
    q = synth.normal_tensor(8100 + nq + d, (B, H, nq, d), dtype)
    k = synth.normal_tensor(8200 + nk + d, (B, H, nk, d), dtype)
    vl = [max(1, nk // 3), nk]
    got = weights(dev, q, k, mask, vl)
    zeros_v = np.zeros((B, H, nk, 1))
    _, ref = oracle.attention(q.f64, k.f64, zeros_v, mask=mask, valid_lens=vl, return_weights=True)
    check("A %s [%d,%d,%d,%d] d%d %s" % (dtype, B, H, nq, nk, d, mask), got, ref)


def test_weights_grouped_heads_empty_rows_and_scale(dev):
    """Grouped K/V heads (6 query heads over 2), a batch with valid_len 0 (all-zero rows) and a scale
    far from 1/sqrt(d)."""
    B, H, Hkv, nq, nk, d = 2, 6, 2, 40, 300, 32
    q = synth.normal_tensor(8300, (B, H, nq, d))
    k = synth.normal_tensor(8301, (B, Hkv, nk, d))
    vl = [0, 211]
    got = weights(dev, q, k, "padding", vl, scale=0.6)
    _, ref = oracle.attention(q.f64, k.f64, np.zeros((B, Hkv, nk, 1)), mask="padding", valid_lens=vl, scale=0.6,
                              return_weights=True)
    check("A grouped [2,6/2,40,300] d32 padding scale 0.6", got, ref)
    assert np.all(got[0] == 0.0)
    np.testing.assert_allclose(got[1].sum(axis=-1), 1.0, atol=1e-5)
