"""Pins that tie the CPU oracle to facts fixed by the pages and by
mathematics, independent of the oracle's own code.

Each pin is a function ``pin_xxx(lib)`` that raises AssertionError when the
oracle library at path ``lib`` (None = the real oracle) disagrees. They are
collected by ``test_oracle_pins.py`` and, against deliberately altered
copies of the oracle source, by ``test_oracle_mutants.py`` (every planted
mistake must trip at least one pin).

Pages cited:
  p1 = "04. Self-Attention：Transformer 的核心计算"
  p2 = the "attention-mechanism" page (zjrzb.cn)
  p3 = "多模态大模型学习笔记（十四）——Transformer学习之Self-Attention"
  p4 = "Transformer 详解：自注意力、多头与位置编码"
  p5 = "Self-Attention 机制"
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "hand_example.json"), encoding="utf-8") as f:
        return json.load(f)


def _randn(seed, shape, std=1.0):
    return synth.normal_f64(seed, int(np.prod(shape))).reshape(shape) * std


def _hand():
    g = _golden()
    X = np.asarray(g["X"], dtype=np.float64)
    return g, X


# --- hand-worked example ----------------------------------------------------

def pin_hand_example_page1(lib):
    """p1 section 六: scaled scores, e^s, their sum, row-3 weights and output."""
    g, X = _hand()
    p = g["page1"]
    tol = p["tol"]
    O, A = oracle.attention(X[None, None], X[None, None], X[None, None], return_weights=True, lib=lib)
    A, O = A[0, 0], O[0, 0]
    np.testing.assert_allclose(A[2], p["row3_weights"], atol=tol)
    np.testing.assert_allclose(O[2], p["row3_output"], atol=tol)
    # e^{s_3j} = A_3j * sum_j e^{s_3j}
    np.testing.assert_allclose(A[2] * p["row3_exp_sum"], p["row3_exp"], atol=3 * tol)
    # score differences are log-weight ratios: s_ij - s_ik = log(A_ij / A_ik)
    S = np.asarray(p["scaled_scores"])
    for i in range(3):
        np.testing.assert_allclose(np.log(A[i] / A[i, 0]), S[i] - S[i, 0], atol=2 * tol)


def _page4_weights(p):
    flat = np.asarray(p["weights_as_printed_flat"])
    return flat.reshape(3, 3).T  # column-major reading, see the fixture


def pin_hand_example_page4(lib):
    """p4 section 手算一遍: the full 3x3 weight matrix and all three outputs."""
    g, X = _hand()
    p = g["page4"]
    tol = p["tol"]
    O, A = oracle.attention(X[None, None], X[None, None], X[None, None], return_weights=True, lib=lib)
    W = _page4_weights(p)
    np.testing.assert_allclose(W[2], p["row3_weights"], atol=1e-12)  # the reading is consistent
    np.testing.assert_allclose(A[0, 0], W, atol=tol)
    np.testing.assert_allclose(O[0, 0], p["outputs"], atol=tol)
    np.testing.assert_allclose(A[0, 0, 2] * p["row3_exp_sum"], p["row3_exp"], atol=3 * tol)


def pin_hand_example_mha(lib):
    """The same example through the multi-head layer: d_model = 2, one head,
    W_QKV = [I | I | I] (p5 五步计算: the three projections concatenated),
    W_O = I, so Y equals p4's three outputs."""
    g, X = _hand()
    I2 = np.eye(2)
    Y = oracle.mha(X[None], np.concatenate([I2, I2, I2], axis=1), I2, 1, lib=lib)
    np.testing.assert_allclose(Y[0], g["page4"]["outputs"], atol=g["page4"]["tol"])


def pin_hand_example_zero_padded(lib):
    """Zero columns appended to q, k and v change no dot product and no
    weighted sum: padding d_k = 2 to 16 with the scale held at 1/sqrt(2)
    reproduces the example (this is how a width-16 kernel runs it)."""
    g, X = _hand()
    Xp = np.zeros((3, 16))
    Xp[:, :2] = X
    O = oracle.attention(Xp[None, None], Xp[None, None], Xp[None, None], scale=1 / np.sqrt(2), lib=lib)[0, 0]
    np.testing.assert_allclose(O[:, :2], g["page4"]["outputs"], atol=g["page4"]["tol"])
    assert np.all(O[:, 2:] == 0.0)


# --- invariants -------------------------------------------------------------

_SHAPES = [(2, 3, 7, 5, 4), (1, 2, 9, 9, 8), (3, 1, 4, 11, 6)]  # B, H, Nq, Nk, d


def _inputs(seed, B, H, Nq, Nk, d, std=1.0):
    return (_randn(seed, (B, H, Nq, d), std), _randn(seed + 1, (B, H, Nk, d), std),
            _randn(seed + 2, (B, H, Nk, d), std))


def _visible(mask, Nq, Nk, L=None):
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    if mask == "causal":
        return j <= i
    if mask == "padding":
        return np.broadcast_to(j < L, (Nq, Nk))
    if mask == "causal_padding":
        return (j <= i) & (j < L)
    return np.ones((Nq, Nk), dtype=bool)


_ALL_MASKS = ("none", "causal", "padding", "causal_padding")


def pin_rows_sum_to_one(lib):
    """Every softmax row sums to 1 (p1 section 四 stage 3; p2 listing prints
    A.sum(-1); p4 section 手算一遍)."""
    for t, (B, H, Nq, Nk, d) in enumerate(_SHAPES):
        q, k, v = _inputs(100 + 10 * t, B, H, Nq, Nk, d)
        for mask in _ALL_MASKS:
            vl = np.arange(B, dtype=np.int32) % Nk + 1
            _, A = oracle.attention(q, k, v, mask=mask, valid_lens=vl, return_weights=True, lib=lib)
            np.testing.assert_allclose(A.sum(-1), 1.0, atol=1e-13)


def pin_masked_weights_exactly_zero(lib):
    """Masked positions get weight exactly 0 (e^{-inf} = 0: p1 section 七,
    p2 section 掩码), visible ones a positive weight."""
    for t, (B, H, Nq, Nk, d) in enumerate(_SHAPES):
        q, k, v = _inputs(200 + 10 * t, B, H, Nq, Nk, d)
        vl = (np.arange(B, dtype=np.int32) * 3) % Nk + 1
        for mask in ("causal", "padding", "causal_padding"):
            _, A = oracle.attention(q, k, v, mask=mask, valid_lens=vl, return_weights=True, lib=lib)
            for b in range(B):
                vis = _visible(mask, Nq, Nk, vl[b])
                assert np.all(A[b][:, ~vis] == 0.0)
                assert np.all(A[b][:, vis] > 0.0)


def pin_masked_keys_do_not_matter(lib):
    """Changing K and V at masked positions leaves the output bit-for-bit
    unchanged."""
    B, H, Nq, Nk, d = 2, 2, 8, 8, 6
    q, k, v = _inputs(300, B, H, Nq, Nk, d)
    vl = np.asarray([3, 6], dtype=np.int32)
    O = oracle.attention(q, k, v, mask="padding", valid_lens=vl, lib=lib)
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, :, vl[b]:] = 1e4 * _randn(301 + b, k2[b, :, vl[b]:].shape)
        v2[b, :, vl[b]:] = -1e4
    O2 = oracle.attention(q, k2, v2, mask="padding", valid_lens=vl, lib=lib)
    assert np.array_equal(O, O2)
    # causal: keys after the last query row's position can hold anything
    Oc = oracle.attention(q, k, v, mask="causal", lib=lib)
    for i in range(Nq):
        k3, v3 = k.copy(), v.copy()
        k3[:, :, i + 1:] = 1e4
        v3[:, :, i + 1:] = -1e4
        O3 = oracle.attention(q, k3, v3, mask="causal", lib=lib)
        assert np.array_equal(O3[:, :, i], Oc[:, :, i])


def pin_causal_first_row_is_first_value(lib):
    """Under the causal mask query 0 sees only key 0: weight exactly 1."""
    q, k, v = _inputs(400, 2, 3, 6, 6, 5)
    O = oracle.attention(q, k, v, mask="causal", lib=lib)
    assert np.array_equal(O[:, :, 0], v[:, :, 0])


def pin_query_permutation_equivariance(lib):
    """Permuting the query rows permutes the output rows the same way
    (p2 section 工程权衡与边界; p4 section 位置编码提供顺序信息)."""
    B, H, Nq, Nk, d = 2, 2, 9, 7, 5
    q, k, v = _inputs(500, B, H, Nq, Nk, d)
    perm = np.argsort(_randn(509, (Nq,)))
    vl = np.asarray([4, 7], dtype=np.int32)
    for mask in ("none", "padding"):
        O = oracle.attention(q, k, v, mask=mask, valid_lens=vl, lib=lib)
        Op = oracle.attention(q[:, :, perm], k, v, mask=mask, valid_lens=vl, lib=lib)
        np.testing.assert_allclose(Op, O[:, :, perm], atol=1e-14, rtol=0)


def pin_joint_kv_permutation_invariance(lib):
    """Permuting key and value rows together leaves every output unchanged
    (the weighted sum runs over a set)."""
    B, H, Nq, Nk, d = 2, 2, 6, 10, 4
    q, k, v = _inputs(600, B, H, Nq, Nk, d)
    perm = np.argsort(_randn(609, (Nk,)))
    O = oracle.attention(q, k, v, lib=lib)
    Op = oracle.attention(q, k[:, :, perm], v[:, :, perm], lib=lib)
    np.testing.assert_allclose(Op, O, atol=1e-13, rtol=0)


# --- closed forms -----------------------------------------------------------

def pin_zero_scale_gives_mean_of_visible_values(lib):
    """scale = 0 makes every visible score equal, so the weights are uniform:
    the mean of all V rows (no mask), of V[0..i] (causal), of V[0..L-1]
    (padding)."""
    B, H, N, d = 2, 2, 7, 3
    q, k, v = _inputs(700, B, H, N, N, d)
    O = oracle.attention(q, k, v, scale=0.0, lib=lib)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=1e-14)
    Oc = oracle.attention(q, k, v, mask="causal", scale=0.0, lib=lib)
    pref = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(Oc, pref, atol=1e-14)
    vl = np.asarray([2, 5], dtype=np.int32)
    Op = oracle.attention(q, k, v, mask="padding", valid_lens=vl, scale=0.0, lib=lib)
    for b in range(B):
        np.testing.assert_allclose(Op[b], np.broadcast_to(v[b, :, : vl[b]].mean(axis=1, keepdims=True),
                                                          Op[b].shape), atol=1e-14)
    # both: row i averages V[0 .. min(i, L-1)] (the prefix means stop growing at the padding boundary)
    Ocp = oracle.attention(q, k, v, mask="causal_padding", valid_lens=vl, scale=0.0, lib=lib)
    for b in range(B):
        for i in range(N):
            np.testing.assert_allclose(Ocp[b, :, i], pref[b, :, min(i, vl[b] - 1)], atol=1e-14)


def pin_single_key_returns_its_value(lib):
    """With one key its weight is 1, so every output row is that value row."""
    q, k, v = _inputs(800, 2, 3, 5, 1, 4)
    O = oracle.attention(q, k, v, lib=lib)
    assert np.array_equal(O, np.broadcast_to(v, O.shape))


def pin_one_hot_limit(lib):
    """A very large scale with distinct scores puts all weight on the
    highest-scoring key (the saturation p1 section 四 stage 2 warns about);
    the stable softmax must not overflow on the way."""
    B, H, Nq, Nk, d = 1, 2, 5, 8, 4
    q, k, v = _inputs(900, B, H, Nq, Nk, d)
    O = oracle.attention(q, k, v, scale=1e4, lib=lib)
    s = np.einsum("bhid,bhjd->bhij", q, k)
    j = s.argmax(-1)
    expect = np.take_along_axis(v, j[..., None], axis=2)
    np.testing.assert_allclose(O, expect, atol=1e-12)


def pin_row_without_visible_key_is_zero(lib):
    """valid_len = 0: no key is visible; output and weights are 0 (the
    convention chosen where the pages are silent)."""
    q, k, v = _inputs(1000, 2, 1, 3, 4, 2)
    vl = np.asarray([0, 4], dtype=np.int32)
    O, A = oracle.attention(q, k, v, mask="padding", valid_lens=vl, return_weights=True, lib=lib)
    assert np.all(O[0] == 0.0) and np.all(A[0] == 0.0)
    assert np.all(np.isfinite(O[1]))


# --- library routine --------------------------------------------------------

def pin_matches_torch_float64_attention(lib):
    """torch.nn.functional.scaled_dot_product_attention on CPU in float64
    with an explicit boolean keep-mask computes the same definition."""
    import torch
    import torch.nn.functional as F

    for t, (B, H, Nq, Nk, d) in enumerate(_SHAPES + [(2, 2, 33, 17, 16)]):
        q, k, v = _inputs(1100 + 10 * t, B, H, Nq, Nk, d, std=1.5)
        vl = (np.arange(B, dtype=np.int32) * 5) % Nk + 1
        for mask in _ALL_MASKS:
            if mask.startswith("causal") and Nq > Nk:
                continue
            keep = np.stack([_visible(mask, Nq, Nk, vl[b]) for b in range(B)])[:, None]
            ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                                 attn_mask=torch.from_numpy(keep)).numpy()
            O = oracle.attention(q, k, v, mask=mask, valid_lens=vl, lib=lib)
            np.testing.assert_allclose(O, ref, atol=1e-12, rtol=0)


def pin_mha_matches_torch_float64(lib):
    """The multi-head layer against torch float64 ops: one GEMM with
    [W_Q|W_K|W_V], view(B,N,h,d_k).transpose(1,2) per p5 维度全程跟踪,
    per-head attention, inverse transpose, W_O."""
    import torch
    import torch.nn.functional as F

    for (B, N, dm, h) in [(2, 6, 16, 4), (1, 5, 12, 3), (2, 7, 8, 1)]:
        x = _randn(1200 + dm, (B, N, dm))
        wqkv = _randn(1201 + dm, (dm, 3 * dm), np.sqrt(1.0 / dm))
        wo = _randn(1202 + dm, (dm, dm), np.sqrt(1.0 / dm))
        X, Wqkv, Wo = map(torch.from_numpy, (x, wqkv, wo))
        P = X @ Wqkv
        dk = dm // h
        qh, kh, vh = (P[..., i * dm:(i + 1) * dm].reshape(B, N, h, dk).transpose(1, 2) for i in range(3))
        ctx = F.scaled_dot_product_attention(qh, kh, vh).transpose(1, 2).reshape(B, N, dm)
        ref = (ctx @ Wo).numpy()
        Y = oracle.mha(x, wqkv, wo, h, lib=lib)
        np.testing.assert_allclose(Y, ref, atol=1e-12, rtol=0)


def pin_mha_identity_projections_split_heads(lib):
    """With W_QKV = [I | I | I] and W_O = I the layer is concat_i of
    attention on the i-th block of d_k columns of X (head i <-> columns
    [i d_k, (i+1) d_k), p5 维度全程跟踪)."""
    B, N, h, dk = 2, 5, 3, 4
    dm = h * dk
    x = _randn(1300, (B, N, dm))
    I = np.eye(dm)
    Y = oracle.mha(x, np.concatenate([I, I, I], axis=1), I, h, lib=lib)
    for i in range(h):
        xi = x[:, :, i * dk:(i + 1) * dk][:, None]
        Oi = oracle.attention(xi, xi, xi, lib=lib)[:, 0]
        np.testing.assert_allclose(Y[:, :, i * dk:(i + 1) * dk], Oi, atol=1e-14, rtol=0)


def pin_mha_cross_matches_torch_float64(lib):
    """The cross-attention layer against torch float64 ops: Q from the query sequence through W_Q, K and V
    from the other sequence through W_K and W_V ("多模态大模型学习笔记（十四）" section 4), heads split and
    concatenated as in the self-attention layer, keys past each batch's valid length hidden."""
    import torch
    import torch.nn.functional as F

    for (B, Nq, Nkv, dm, h) in [(2, 5, 9, 16, 4), (1, 7, 3, 12, 3), (2, 4, 4, 8, 1)]:
        xq = _randn(1500 + dm, (B, Nq, dm))
        xkv = _randn(1501 + dm, (B, Nkv, dm))
        wqkv = _randn(1502 + dm, (dm, 3 * dm), np.sqrt(1.0 / dm))
        wo = _randn(1503 + dm, (dm, dm), np.sqrt(1.0 / dm))
        vl = np.asarray([Nkv, max(1, Nkv // 2)][:B], dtype=np.int32)
        Xq, Xkv, Wqkv, Wo = map(torch.from_numpy, (xq, xkv, wqkv, wo))
        dk = dm // h
        qh = (Xq @ Wqkv[:, :dm]).reshape(B, Nq, h, dk).transpose(1, 2)
        kh = (Xkv @ Wqkv[:, dm:2 * dm]).reshape(B, Nkv, h, dk).transpose(1, 2)
        vh = (Xkv @ Wqkv[:, 2 * dm:]).reshape(B, Nkv, h, dk).transpose(1, 2)
        for mask in ("none", "padding"):
            keep = None
            if mask == "padding":
                keep = torch.from_numpy(np.arange(Nkv)[None, :] < vl[:, None])[:, None, None, :]
            ctx = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=keep).transpose(1, 2).reshape(B, Nq, dm)
            Y = oracle.mha_cross(xq, xkv, wqkv, wo, h, mask=mask, valid_lens=vl, lib=lib)
            np.testing.assert_allclose(Y, (ctx @ Wo).numpy(), atol=1e-12, rtol=0)


def pin_mha_cross_reduces_to_self_attention(lib):
    """With the query and key sequences the same and no mask, the cross-attention layer is the multi-head
    self-attention layer; with W_QKV = [I | I | I] and W_O = I, head i is attention of the i-th column
    block of the queries over the i-th block of the other sequence."""
    B, N, dm, h = 2, 6, 12, 3
    x = _randn(1510, (B, N, dm))
    wqkv = _randn(1511, (dm, 3 * dm), np.sqrt(1.0 / dm))
    wo = _randn(1512, (dm, dm), np.sqrt(1.0 / dm))
    np.testing.assert_allclose(oracle.mha_cross(x, x, wqkv, wo, h, lib=lib), oracle.mha(x, wqkv, wo, h, lib=lib),
                               atol=1e-13, rtol=0)
    xkv = _randn(1513, (B, 4, dm))
    I = np.eye(dm)
    Y = oracle.mha_cross(x, xkv, np.concatenate([I, I, I], axis=1), I, h, lib=lib)
    dk = dm // h
    for i in range(h):
        qi, ki = x[:, :, i * dk:(i + 1) * dk][:, None], xkv[:, :, i * dk:(i + 1) * dk][:, None]
        np.testing.assert_allclose(Y[:, :, i * dk:(i + 1) * dk], oracle.attention(qi, ki, ki, lib=lib)[:, 0],
                                   atol=1e-14, rtol=0)


def pin_row_subset_equals_full(lib):
    """Output rows computed one by one equal the same rows of the full call
    (the full-size GPU checks rely on this)."""
    B, H, Nq, Nk, d = 2, 3, 11, 11, 8
    q, k, v = _inputs(1400, B, H, Nq, Nk, d)
    vl = np.asarray([5, 11], dtype=np.int32)
    rows = np.asarray([0, 1, 10, 17, 33, 44, 65], dtype=np.int64)
    for mask in _ALL_MASKS:
        O, L = oracle.attention(q, k, v, mask=mask, valid_lens=vl, lib=lib, return_lse=True)
        Or, Lr = oracle.attention_rows(q, k, v, rows, mask=mask, valid_lens=vl, lib=lib, return_lse=True)
        assert np.array_equal(Or, O.reshape(-1, d)[rows]) and np.array_equal(Lr, L.reshape(-1)[rows])
    # grouped K/V heads: the same on three query heads sharing one K/V head
    kg, vg = k[:, :1], v[:, :1]
    O = oracle.attention(q, kg, vg, mask="causal", lib=lib).reshape(-1, d)
    Or = oracle.attention_rows(q, kg, vg, rows, mask="causal", lib=lib)
    assert np.array_equal(Or, O[rows])


def pin_rows_per_head_equals_full(lib, mod=None):
    """The per-head row helper (flat row -> batch, query head, query index; K/V head h // (H / H_kv); the
    batch's own valid length) gives the same rows, bit for bit, as the full call, for every mask, grouped
    and plain K/V heads, per-batch valid lengths and float32 views of the inputs. ``mod`` is the module
    whose helper is checked (the oracle itself by default; altered copies in the planted-mistake test)."""
    mod = oracle if mod is None else mod
    B, H, Nq, Nk, d = 2, 4, 9, 11, 8
    vl = np.asarray([3, 11], dtype=np.int32)
    q32 = _randn(1450, (B, H, Nq, d)).astype(np.float32)
    for hkv in (1, 2, 4):
        k32 = _randn(1451 + hkv, (B, hkv, Nk, d)).astype(np.float32)
        v32 = _randn(1461 + hkv, (B, hkv, Nk, d)).astype(np.float32)
        q, k, v = (t.astype(np.float64) for t in (q32, k32, v32))
        # every row, in an order that visits the heads and batches out of sequence
        rows = np.asarray([(r * 37) % (B * H * Nq) for r in range(B * H * Nq)], dtype=np.int64)
        for mask in _ALL_MASKS:
            O, L = oracle.attention(q, k, v, mask=mask, valid_lens=vl, lib=lib, return_lse=True)
            Or, Lr = mod.attention_rows_per_head(q32, k32, v32, rows, mask=mask, valid_lens=vl, return_lse=True,
                                                 lib=lib)
            assert np.array_equal(Or, O.reshape(-1, d)[rows]), (hkv, mask)
            assert np.array_equal(Lr, L.reshape(-1)[rows]), (hkv, mask)


# --- log-sum-exp of the scores ----------------------------------------------

def pin_lse_hand_example_page1(lib):
    """p1 section 六 prints e^{s_3j} and their sum for row 3: the log-sum-exp is the log of that sum;
    rows 1 and 2 share their sum of raw exponentials."""
    g, X = _hand()
    p = g["page1"]
    _, L = oracle.attention(X[None, None], X[None, None], X[None, None], return_lse=True, lib=lib)
    L = L[0, 0]
    np.testing.assert_allclose(np.exp(L[2]), p["row3_exp_sum"], atol=3 * p["tol"])
    np.testing.assert_allclose(np.exp(L[2]), np.sum(p["row3_exp"]), atol=3 * p["tol"])
    assert L[0] == L[1]


def pin_lse_zero_scale_counts_visible_keys(lib):
    """scale = 0: every visible score is 0, so the log-sum-exp is ln(number of visible keys) and -inf for a
    row with none."""
    B, H, N, d = 2, 2, 6, 3
    q, k, v = _inputs(1500, B, H, N, N, d)
    vl = np.asarray([0, 4], dtype=np.int32)
    for mask in _ALL_MASKS:
        _, L = oracle.attention(q, k, v, mask=mask, valid_lens=vl, scale=0.0, return_lse=True, lib=lib)
        for b in range(B):
            n = _visible(mask, N, N, vl[b]).sum(axis=1)
            with np.errstate(divide="ignore"):
                want = np.log(n.astype(np.float64))
            np.testing.assert_array_equal(np.isneginf(L[b]), np.broadcast_to(n == 0, L[b].shape))
            np.testing.assert_allclose(L[b][:, n > 0], np.broadcast_to(want[n > 0], (H, int((n > 0).sum()))),
                                       atol=1e-14)


def pin_lse_matches_torch_logsumexp(lib):
    """torch.logsumexp over the masked scaled scores (float64 CPU), and the weights are exp(s - lse)."""
    import torch

    for t, (B, H, Nq, Nk, d) in enumerate(_SHAPES):
        q, k, v = _inputs(1600 + 10 * t, B, H, Nq, Nk, d, std=2.0)
        vl = (np.arange(B, dtype=np.int32) * 3) % Nk + 1
        scale = 0.7
        s = torch.from_numpy(np.einsum("bhid,bhjd->bhij", q, k) * scale)
        for mask in _ALL_MASKS:
            if mask.startswith("causal") and Nq > Nk:
                continue
            keep = torch.from_numpy(np.stack([_visible(mask, Nq, Nk, vl[b]) for b in range(B)])[:, None])
            ref = torch.logsumexp(s.masked_fill(~keep, float("-inf")), dim=-1).numpy()
            _, A, L = oracle.attention(q, k, v, mask=mask, valid_lens=vl, scale=scale, return_weights=True,
                                       return_lse=True, lib=lib)
            np.testing.assert_allclose(L, ref, atol=1e-12, rtol=0)
            w = np.where(keep.numpy(), np.exp(s.numpy() - L[..., None]), 0.0)
            np.testing.assert_allclose(A, w, atol=1e-12, rtol=0)


# --- grouped K/V heads --------------------------------------------------------

def pin_grouped_kv_heads_match_torch(lib):
    """p5 section MHA -> MQA -> GQA -> MLA: every H / H_kv query heads share one K/V head. torch's float64
    attention with enable_gqa (consecutive query heads per K/V head) computes the same."""
    import torch
    import torch.nn.functional as F

    for t, (B, H, Hkv, Nq, Nk, d) in enumerate([(2, 4, 2, 5, 7, 4), (1, 6, 3, 9, 9, 8), (2, 3, 1, 4, 6, 5)]):
        q = _randn(1700 + 10 * t, (B, H, Nq, d))
        k = _randn(1701 + 10 * t, (B, Hkv, Nk, d))
        v = _randn(1702 + 10 * t, (B, Hkv, Nk, d))
        vl = (np.arange(B, dtype=np.int32) * 2) % Nk + 1
        for mask in _ALL_MASKS:
            if mask.startswith("causal") and Nq > Nk:
                continue
            keep = torch.from_numpy(np.stack([_visible(mask, Nq, Nk, vl[b]) for b in range(B)])[:, None])
            ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                                 attn_mask=keep, enable_gqa=True).numpy()
            O = oracle.attention(q, k, v, mask=mask, valid_lens=vl, lib=lib)
            np.testing.assert_allclose(O, ref, atol=1e-12, rtol=0)


def pin_group_sizes_degenerate(lib):
    """H_kv = H is the plain multi-head case; H_kv = 1 (one K/V head for all query heads) gives, for each
    query head, what a single-head call on that head's queries gives."""
    B, H, N, d = 2, 4, 6, 5
    q, k, v = _inputs(1800, B, H, N, N, d)
    O = oracle.attention(q, k, v, mask="causal", lib=lib)
    assert np.array_equal(O, oracle.attention(q, k, v, mask="causal", lib=lib))
    Om = oracle.attention(q, k[:, :1], v[:, :1], mask="causal", lib=lib)
    for h in range(H):
        Oh = oracle.attention(q[:, h:h + 1], k[:, :1], v[:, :1], mask="causal", lib=lib)
        assert np.array_equal(Om[:, h:h + 1], Oh)
    # and each group of two query heads reads its own K/V head
    Og = oracle.attention(q, k[:, :2], v[:, :2], mask="causal", lib=lib)
    for h in range(H):
        Oh = oracle.attention(q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1], mask="causal", lib=lib)
        assert np.array_equal(Og[:, h:h + 1], Oh)


# --- gradients ------------------------------------------------------------------

def _fwd_loss(q, k, v, g, mask, vl, scale, lib):
    return float(np.sum(oracle.attention(q, k, v, mask=mask, valid_lens=vl, scale=scale, lib=lib) * g))


def pin_backward_matches_torch_autograd(lib):
    """torch autograd through float64 attention on the CPU (with enable_gqa and a boolean keep mask)."""
    import torch
    import torch.nn.functional as F

    for t, (B, H, Hkv, Nq, Nk, d) in enumerate([(2, 2, 2, 6, 6, 4), (1, 4, 2, 7, 9, 5), (2, 3, 1, 5, 5, 3)]):
        q = _randn(1900 + 10 * t, (B, H, Nq, d))
        k = _randn(1901 + 10 * t, (B, Hkv, Nk, d))
        v = _randn(1902 + 10 * t, (B, Hkv, Nk, d))
        g = _randn(1903 + 10 * t, (B, H, Nq, d))
        vl = (np.arange(B, dtype=np.int32) * 3) % Nk + 2
        for mask in _ALL_MASKS:
            if mask.startswith("causal") and Nq > Nk:
                continue
            keep = torch.from_numpy(np.stack([_visible(mask, Nq, Nk, vl[b]) for b in range(B)])[:, None])
            Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
            O = F.scaled_dot_product_attention(Q, K, V, attn_mask=keep, enable_gqa=True, scale=0.8)
            (O * torch.from_numpy(g)).sum().backward()
            dq, dk, dv = oracle.attention_backward(q, k, v, g, mask=mask, valid_lens=vl, scale=0.8, lib=lib)
            np.testing.assert_allclose(dq, Q.grad.numpy(), atol=1e-12, rtol=0)
            np.testing.assert_allclose(dk, K.grad.numpy(), atol=1e-12, rtol=0)
            np.testing.assert_allclose(dv, V.grad.numpy(), atol=1e-12, rtol=0)


def pin_backward_finite_differences(lib):
    """Central differences of sum(O * g) on a tiny shape, for a few entries of each of Q, K and V."""
    B, H, Hkv, N, d = 1, 2, 1, 5, 3
    q, k, v = _randn(2000, (B, H, N, d)), _randn(2001, (B, Hkv, N, d)), _randn(2002, (B, Hkv, N, d))
    g = _randn(2003, (B, H, N, d))
    vl = np.asarray([4], dtype=np.int32)
    eps = 1e-5
    for mask in ("causal", "causal_padding"):
        grads = oracle.attention_backward(q, k, v, g, mask=mask, valid_lens=vl, scale=0.7, lib=lib)
        for which, (x, gx) in enumerate(zip((q, k, v), grads)):
            for e in range(0, x.size, 3):
                xp, xm = x.copy(), x.copy()
                xp.flat[e] += eps
                xm.flat[e] -= eps
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                fd = (_fwd_loss(*args_p, g, mask, vl, 0.7, lib) - _fwd_loss(*args_m, g, mask, vl, 0.7, lib)) / (2 * eps)
                assert abs(fd - gx.flat[e]) <= 1e-8, (mask, which, e, fd, gx.flat[e])


def pin_backward_translation_invariances(lib):
    """Adding one vector to every key shifts each row's scores by a constant (softmax unchanged): the key
    gradients of a head sum to 0. Adding one vector to every value row shifts every output row that sees a
    key by it: the value gradients of a head sum to the output gradients of those rows."""
    B, H, N, d = 2, 3, 8, 4
    q, k, v = _inputs(2100, B, H, N, N, d)
    g = _randn(2104, (B, H, N, d))
    vl = np.asarray([0, 5], dtype=np.int32)
    for mask in _ALL_MASKS:
        _, dk, dv = oracle.attention_backward(q, k, v, g, mask=mask, valid_lens=vl, lib=lib)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-13)
        for b in range(B):
            sees = _visible(mask, N, N, vl[b]).any(axis=1)
            np.testing.assert_allclose(dv[b].sum(axis=1), g[b][:, sees].sum(axis=1), atol=1e-13)


def pin_backward_zero_scale_and_masked_keys(lib):
    """scale = 0: scores do not depend on Q or K, so dQ = dK = 0 exactly, and each row spreads its output
    gradient uniformly over its visible keys. Keys no row can see (j >= valid_len) get zero gradients."""
    B, H, N, d = 2, 2, 6, 3
    q, k, v = _inputs(2200, B, H, N, N, d)
    g = _randn(2203, (B, H, N, d))
    vl = np.asarray([2, 6], dtype=np.int32)
    for mask in _ALL_MASKS:
        dq, dk, dv = oracle.attention_backward(q, k, v, g, mask=mask, valid_lens=vl, scale=0.0, lib=lib)
        assert np.all(dq == 0.0) and np.all(dk == 0.0)
        for b in range(B):
            vis = _visible(mask, N, N, vl[b]).astype(np.float64)
            w = vis / np.maximum(vis.sum(axis=1, keepdims=True), 1)
            np.testing.assert_allclose(dv[b], np.einsum("ij,hic->hjc", w, g[b]), atol=1e-14)
    _, dk, dv = oracle.attention_backward(q, k, v, g, mask="padding", valid_lens=vl, lib=lib)
    assert np.all(dk[0, :, 2:] == 0.0) and np.all(dv[0, :, 2:] == 0.0)


PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]
