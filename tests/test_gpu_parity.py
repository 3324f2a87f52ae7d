"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the
same seeded inputs, on an MI355X.

Tolerances (max / mean absolute error against the float64 oracle):
  float32 inputs:                       max <= 1e-5
  bfloat16 inputs, f32 accumulation:    max <= 2e-2 and mean <= 2e-3
Every shape, the full-size workloads included, is compared element by
element with the oracle on the whole output; the long-context workload's
oracle runs one head at a time (heads are independent). Properties that hold
for every row at any size (weights summing to one, masked keys never reaching
the output) are checked besides.
"""
import math

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16_MAX, TOL_BF16_MEAN = 2e-2, 2e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_scaled_dot_amd as tsd

    tsd.load_library()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def gpu_attn(dev, q, k, v, mask="none", vl=None, scale=None, out_dtype=None):
    import transformer_scaled_dot_amd as tsd

    vl_t = torch.from_numpy(np.asarray(vl, dtype=np.int32)).to(dev) if vl is not None else None
    od = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    o = tsd.attn_fwd(q.torch(dev), k.torch(dev), v.torch(dev), mask=mask, valid_lens=vl_t, scale=scale,
                     out_dtype=od)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64)


def check(name, got, ref, dtype):
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    say("%s: max abs err %.3e, mean %.3e, max|ref| %.3f" % (name, mx, mean, float(np.abs(ref).max()) if ref.size else 0))
    assert np.all(np.isfinite(got)), "non-finite output"
    if dtype == "f32":
        assert mx <= TOL_F32, name
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, name


# ---------------------------------------------------------------- float32 path

def test_config1_f32_full(dev):
    q, k, v, _ = synth.attn_inputs(1)
    got = gpu_attn(dev, q, k, v)
    check("C1 f32 [2,1,5,16]", got, oracle.attention(q.f64, k.f64, v.f64), "f32")


def test_hand_example_f32(dev, golden_dir):
    """The pages' 3-token example, zero-padded from d_k = 2 to 16 with the
    scale held at 1/sqrt(2) (zeros add nothing to any product)."""
    import json

    g = json.load(open(golden_dir + "/hand_example.json", encoding="utf-8"))
    X = np.zeros((1, 1, 3, 16), dtype=np.float32)
    X[0, 0, :, :2] = np.asarray(g["X"], dtype=np.float32)
    t = synth.Tensor(X.copy(), "f32", X.shape)
    got = gpu_attn(dev, t, t, t, scale=1 / math.sqrt(2))
    check("hand example f32", got, oracle.attention(X, X, X, scale=1 / math.sqrt(2)), "f32")
    np.testing.assert_allclose(got[0, 0, :, :2], g["page4"]["outputs"], atol=g["page4"]["tol"])
    np.testing.assert_allclose(got[0, 0, 2, :2], g["page1"]["row3_output"], atol=g["page1"]["tol"])
    assert np.all(got[0, 0, :, 2:] == 0.0)


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "padding"])
def test_f32_ragged(dev, d, mask):
    N = 37 if d >= 64 else 70
    q, k, v, _ = synth.attn_inputs(1, B=2, H=2, N=N, d=d)
    vl = np.asarray([N // 3, N], dtype=np.int32)
    got = gpu_attn(dev, q, k, v, mask=mask, vl=vl)
    check("f32 d%d %s N%d" % (d, mask, N), got, oracle.attention(q.f64, k.f64, v.f64, mask=mask, valid_lens=vl), "f32")


# ---------------------------------------------------------------- bf16 path

# up to three 256-row query tiles and ten 64-key tiles, with ragged tails on both
SMALL = [(1, 1), (5, 5), (64, 64), (200, 200), (333, 333), (130, 77), (77, 300), (600, 600), (530, 620)]


# causal is defined for seq_q == seq_k only (the C ABI rejects the rest; test_capi_host.py checks that)
RAGGED_CASES = [(nq, nk, mask) for (nq, nk) in SMALL for mask in ("none", "causal", "padding")
                if mask != "causal" or nq == nk]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk,mask", RAGGED_CASES)
def test_bf16_ragged(dev, nq, nk, mask, d, out):
    q, k, v, _ = synth.attn_inputs(2, B=2, H=3, N=nq, Nk=nk, d=d)
    vl = np.asarray([max(1, nk // 2), nk + 5], dtype=np.int32)  # second one past the end: clamped
    got = gpu_attn(dev, q, k, v, mask=mask, vl=vl, out_dtype=out)
    ref = oracle.attention(q.f64, k.f64, v.f64, mask=mask, valid_lens=np.minimum(vl, nk))
    check("bf16 [2,3,%d,%d] d%d %s out %s" % (nq, nk, d, mask, out), got, ref, "bf16")


def test_config2_padding_full(dev):
    q, k, v, vl = synth.attn_inputs(2)
    say("C2 valid_lens", vl.tolist())
    got = gpu_attn(dev, q, k, v, mask="padding", vl=vl)
    check("C2 bf16 [8,8,512,64] padding", got, oracle.attention(q.f64, k.f64, v.f64, mask="padding", valid_lens=vl),
          "bf16")


def test_padding_masked_keys_never_reach_output(dev):
    """Keys at or past valid_len may hold anything: the output is
    bit-for-bit the same (weight exactly 0; the pages' e^{-inf} = 0)."""
    q, k, v, vl = synth.attn_inputs(2, B=8, H=2, N=512)
    o1 = gpu_attn(dev, q, k, v, mask="padding", vl=vl)
    kr, vr = k.raw.copy(), v.raw.copy()
    for b in range(8):
        kr[b, :, vl[b]:] = synth.f32_to_bf16_bits(np.full(kr[b, :, vl[b]:].shape, 1e4, np.float32))
        vr[b, :, vl[b]:] = synth.f32_to_bf16_bits(np.full(vr[b, :, vl[b]:].shape, -3e4, np.float32))
    o2 = gpu_attn(dev, q, synth.Tensor(kr, "bf16", k.shape), synth.Tensor(vr, "bf16", v.shape), mask="padding", vl=vl)
    assert np.array_equal(o1, o2)


def test_causal_future_keys_never_reach_output(dev):
    N = 700
    q, k, v, _ = synth.attn_inputs(3, B=1, H=2, N=N, d=128)
    o1 = gpu_attn(dev, q, k, v, mask="causal")
    cut = 333
    kr, vr = k.raw.copy(), v.raw.copy()
    kr[:, :, cut:] = synth.f32_to_bf16_bits(np.full(kr[:, :, cut:].shape, 1e4, np.float32))
    vr[:, :, cut:] = synth.f32_to_bf16_bits(np.full(vr[:, :, cut:].shape, -3e4, np.float32))
    o2 = gpu_attn(dev, q, synth.Tensor(kr, "bf16", k.shape), synth.Tensor(vr, "bf16", v.shape), mask="causal")
    assert np.array_equal(o1[:, :, :cut], o2[:, :, :cut])
    # query 0 sees only key 0: its output is V[0] exactly
    assert np.array_equal(o1[:, :, 0], v.f64[:, :, 0])


@pytest.mark.parametrize("d", [128, 64])
def test_item_transitions_padding(dev, d):
    """More (256-row query block, head) items than CUs, so that every workgroup of the persistent kernel (both
    head widths) runs several items back to back, with key counts of 0, 1, under one tile, exactly one tile
    and several tiles (the next item's first tiles are fetched by the previous item's tile loop, or separately
    after items of fewer than two tiles). Keys at or past valid_len hold NaN: they are never fetched, so they
    never reach an output."""
    B, H, N = 8, 40, 260
    q, k, v, _ = synth.attn_inputs(2, B=B, H=H, N=N, d=d)
    vl = np.asarray([0, 1, 63, 64, 65, 128, 260, 17], dtype=np.int32)
    kr, vr = k.raw.copy(), v.raw.copy()
    for b in range(B):
        kr[b, :, vl[b]:] = 0x7FC0
        vr[b, :, vl[b]:] = 0x7FC0
    got = gpu_attn(dev, q, synth.Tensor(kr, "bf16", k.shape), synth.Tensor(vr, "bf16", v.shape), mask="padding",
                   vl=vl)
    assert np.all(got[0] == 0.0)
    heads = [1, 7, 20, 39]  # the oracle on a few heads of every batch (all heads are independent)
    ref = oracle.attention(q.f64[:, heads], k.f64[:, heads], v.f64[:, heads], mask="padding", valid_lens=vl)
    check("bf16 [8,40,260,%d] padding, valid_lens %s, heads %s" % (d, vl.tolist(), heads), got[:, heads], ref, "bf16")


@pytest.mark.parametrize("d,N,out", [(128, 40, "bf16"), (128, 70, "bf16"), (128, 300, "bf16"), (64, 40, "bf16"),
                                     (64, 70, "bf16"), (64, 300, "bf16"), (64, 300, "f32"), (64, 1100, "bf16")])
def test_item_transitions_causal(dev, d, N, out):
    """Causal, B*H = 320 heads (several items per workgroup of the persistent kernel): at N = 40 every item
    has one key tile (all next-item tiles fetched after the item), at 70 two, at 300 a mix of 4 and 5; at
    1100 items of up to 17 tiles (the next item's Q rows fetched block by block in the last steps)."""
    B, H = 4, 80
    q, k, v, _ = synth.attn_inputs(3, B=B, H=H, N=N, d=d)
    got = gpu_attn(dev, q, k, v, mask="causal", out_dtype=out)
    heads = [0, 33, 79]
    ref = oracle.attention(q.f64[:, heads], k.f64[:, heads], v.f64[:, heads], mask="causal")
    # bf16 inputs and products: the bf16 bound also for a float32 output
    check("%s out [4,80,%d,%d] causal, heads %s" % (out, N, d, heads), got[:, heads], ref, "bf16")


def test_empty_and_degenerate(dev):
    import transformer_scaled_dot_amd as tsd

    # valid_len 0: no visible key, output exactly 0
    q, k, v, _ = synth.attn_inputs(2, B=2, H=1, N=70, d=64)
    got = gpu_attn(dev, q, k, v, mask="padding", vl=[0, 70])
    assert np.all(got[0] == 0.0)
    check("bf16 valid_len 0/70 other batch", got[1:], oracle.attention(q.f64[1:], k.f64[1:], v.f64[1:]), "bf16")
    # scale 0: uniform weights over visible keys -> mean of those V rows
    got = gpu_attn(dev, q, k, v, mask="causal", scale=0.0)
    ref = np.cumsum(v.f64, axis=2) / np.arange(1, 71)[None, None, :, None]
    check("bf16 causal scale 0 (prefix means)", got, ref, "bf16")
    # seq_q = 0: nothing to do
    z = torch.zeros(1, 1, 0, 64, dtype=torch.bfloat16, device=dev)
    kk = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16, device=dev)
    assert tsd.attn_fwd(z, kk, kk).shape == (1, 1, 0, 64)


def oracle_by_heads(q, k, v, mask, vl=None, label="", heads_per_call=None):
    """The oracle's whole output, computed over groups of (query head, K/V head) pairs of all batches so
    that only one group's inputs are widened to float64 at a time; prints its progress."""
    B, H = q.shape[:2]
    grp = H // k.shape[1]
    step = heads_per_call or H
    out = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    for h0 in range(0, H, step):
        hs = list(range(h0, min(H, h0 + step)))
        kv = sorted({h // grp for h in hs})
        # every query head of the group reads its own K/V head: pass one K/V head per query head
        kk = np.stack([k[:, h // grp] for h in hs], axis=1)
        vv = np.stack([v[:, h // grp] for h in hs], axis=1)
        out[:, hs] = oracle.attention(q[:, hs], kk, vv, mask=mask, valid_lens=vl)
        if step < H:
            say("%s: oracle heads %d..%d of %d done (K/V heads %s)" % (label, hs[0], hs[-1], H, kv))
    return out


def test_config3_causal_full_size(dev):
    """B4 H16 N4096 d128 causal, the launch the bench times: every output element against the oracle, and
    every row's weights summing to one (V = 1)."""
    q, k, v, _ = synth.attn_inputs(3)
    got = gpu_attn(dev, q, k, v, mask="causal")
    ref = oracle_by_heads(q.f32, k.f32, v.f32, "causal")
    check("C3 bf16 [4,16,4096,128] causal (every element)", got, ref, "bf16")
    del got, ref
    ones = synth.Tensor(synth.f32_to_bf16_bits(np.ones(v.shape, np.float32)), "bf16", v.shape)
    o1 = gpu_attn(dev, q, k, ones, mask="causal", out_dtype="f32")
    err = np.abs(o1 - 1.0)
    say("C3 V=1: max |O-1| %.3e" % err.max())
    assert err.max() <= 4e-3


def test_reference_max_moves_d128(dev):
    """The 128-wide-head kernel keeps a per-row reference maximum that it moves (rescaling the partial
    output and sum) only when a tile's maximum exceeds it by more than 2^8 in the exponent. Keys whose
    scores rise from tile to tile (each 64-key tile's keys carry a growing component along the queries'
    common direction) and a large scale make that move happen on most rows and tiles; the count is taken on
    the CPU from the scores, and every element is compared with the oracle."""
    B, H, N, d = 1, 4, 1024, 128
    scale = 0.3
    z = [synth.normal_f64(6100 + i, B * H * N * d).reshape(B, H, N, d) for i in range(3)]
    u = np.ones(d) / np.sqrt(d)
    tile = (np.arange(N) // 64).astype(np.float64)
    qf = z[0] + 1.5 * u
    kf = z[1] + (4.0 * tile)[None, None, :, None] * u
    mk = lambda a: synth.Tensor(synth.f32_to_bf16_bits(a.astype(np.float32)), "bf16", a.shape)
    q, k, v = mk(qf), mk(kf), mk(z[2])
    # how often a tile's maximum (log2 units) exceeds the row's last reference by more than 8
    moves = 0
    for h in range(H):
        S = q.f64[0, h] @ k.f64[0, h].T * scale * np.log2(np.e)
        for mask in ("none", "causal"):
            Sm = np.where(np.tril(np.ones((N, N), bool)), S, -np.inf) if mask == "causal" else S
            tmax = Sm.reshape(N, N // 64, 64).max(axis=2)
            ref = tmax[:, 0].copy()
            for t in range(1, N // 64):
                up = tmax[:, t] > ref + 8
                moves += int(up.sum())
                ref[up] = tmax[up, t]
    say("reference moves in the inputs (rows x tiles, both masks): %d" % moves)
    assert moves > 15000
    for mask in ("none", "causal"):
        for out in ("bf16", "f32"):
            got = gpu_attn(dev, q, k, v, mask=mask, scale=scale, out_dtype=out)
            ref = oracle.attention(q.f64, k.f64, v.f64, mask=mask, scale=scale)
            check("bf16 [1,4,1024,128] %s scale %.2f rising tile maxima, out %s" % (mask, scale, out), got, ref,
                  "bf16")


def test_config4_mha_full(dev):
    import transformer_scaled_dot_amd as tsd

    x, wqkv, wo = synth.mha_inputs(4)
    y = tsd.mha_fwd(x.torch(dev), wqkv.torch(dev), wo.torch(dev), 8)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    check("C4 mha bf16 [4,2048,512] h8", got, oracle.mha(x.f64, wqkv.f64, wo.f64, 8), "bf16")


@pytest.mark.parametrize("B,N,dm,h", [(1, 96, 128, 2), (2, 77, 256, 2), (1, 130, 512, 8), (3, 33, 256, 4),
                                      (1, 300, 768, 6), (8, 1100, 512, 8)])
def test_mha_shapes(dev, B, N, dm, h):
    """The multi-head layer against the oracle, every element; [8,1100,512] h8 has 320 items of 256 rows (more
    than CUs: the persistent attention kernel, several items per workgroup, concat layout, a ragged last
    block)."""
    import transformer_scaled_dot_amd as tsd

    x, wqkv, wo = synth.mha_inputs(4, B=B, N=N, d_model=dm)
    y = tsd.mha_fwd(x.torch(dev), wqkv.torch(dev), wo.torch(dev), h)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    check("mha bf16 [%d,%d,%d] h%d" % (B, N, dm, h), got, oracle.mha(x.f64, wqkv.f64, wo.f64, h), "bf16")


def test_mha_identity_projection_hand_example(dev, golden_dir):
    """W_QKV = [I | I | I], W_O = I: every head is attention on its own
    64-column block of X (the split/concat order of the layer)."""
    import transformer_scaled_dot_amd as tsd

    B, N, h, dk = 1, 40, 2, 64
    dm = h * dk
    x = synth.normal_tensor(77, (B, N, dm), "bf16")
    I = np.eye(dm, dtype=np.float32)
    wqkv = synth.Tensor(synth.f32_to_bf16_bits(np.concatenate([I, I, I], axis=1)), "bf16", (dm, 3 * dm))
    wo = synth.Tensor(synth.f32_to_bf16_bits(I), "bf16", (dm, dm))
    y = tsd.mha_fwd(x.torch(dev), wqkv.torch(dev), wo.torch(dev), h)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    check("mha identity projections", got, oracle.mha(x.f64, wqkv.f64, wo.f64, h), "bf16")


def bf16_half_ulp(x):
    """Half a unit in the last place of bfloat16 (8 significant bits) at |x|: the most that rounding a
    value of that size to the bf16 output can change it."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 8)


@pytest.mark.timeout(900)
def test_config5_long_context(dev):
    """B1 H32 N32768 d128 causal, inputs x2: every output element against the oracle (run one head at a
    time). The float32 output carries no output rounding: every element is held to the tolerance. A bf16
    output adds its own representation error on top of the arithmetic's, up to half a unit in the last
    place of |O| (2^-7 for 2 <= |O| < 4, 2^-6 for 4 <= |O| < 8, values these x2 inputs reach), so each
    bf16-output element is held to the tolerance plus that half unit, and the mean to the mean tolerance."""
    q, k, v, _ = synth.attn_inputs(5)
    got = gpu_attn(dev, q, k, v, mask="causal", out_dtype="f32")
    gotb = gpu_attn(dev, q, k, v, mask="causal")
    ref = oracle_by_heads(q.f32, k.f32, v.f32, "causal", label="C5", heads_per_call=2)
    check("C5 bf16 [1,32,32768,128] x2 causal, f32 out (every element)", got, ref, "bf16")
    del got
    err = np.abs(gotb - ref)
    tol = TOL_BF16_MAX + bf16_half_ulp(ref)
    say("C5 bf16 out: max abs err %.3e, mean %.3e, worst err / (tolerance + half unit) %.3f"
        % (float(err.max()), float(err.mean()), float((err / tol).max())))
    assert np.all(np.isfinite(gotb))
    assert np.all(err <= tol) and float(err.mean()) <= TOL_BF16_MEAN


def test_clock_probe_reports_plausible_rate(dev):
    """The measurement probe (not part of the attention path): a clock between 0.3 and 3 GHz and a matrix
    rate between 50 TFLOP/s and the published 2.5 PFLOP/s dense bf16 peak scaled to that clock (4 SIMDs per
    compute unit, 1024 bf16 flops per SIMD cycle)."""
    from transformer_scaled_dot_amd.probe import clock_probe

    p = clock_probe(dev, spin_us=1000)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ceiling = cus * 4 * 1024 * p["clock_mhz"] * 1e6 / 1e12
    say("clock probe: %.0f MHz, %.1f TFLOP/s (clock-scaled ceiling %.1f)" % (p["clock_mhz"], p["tflops"], ceiling))
    assert 300 < p["clock_mhz"] < 3000
    assert 50 < p["tflops"] <= ceiling * 1.02


@pytest.mark.parametrize("mask", ["none", "causal", "padding", "causal_padding"])
def test_d64_eight_wave_launch(dev, mask):
    """Head_dim 64 on a grid of 256-row items that covers every CU (the persistent kernel, one item per
    workgroup): B2 H16 N2000 (8 query tiles of 256 rows per head, the last tile ragged), every element against
    the oracle."""
    B, H, N, d = 2, 16, 2000, 64
    q, k, v = (synth.normal_tensor(5100 + i, (B, H, N, d)) for i in range(3))
    vl = np.asarray([1999, 777], dtype=np.int32)
    pad = mask in ("padding", "causal_padding")
    got = gpu_attn(dev, q, k, v, mask=mask, vl=vl if pad else None)
    ref = oracle.attention(q.f64, k.f64, v.f64, mask=mask, valid_lens=vl if pad else None)
    check("bf16 [2,16,2000,64] %s, persistent launch" % mask, got, ref, "bf16")


def test_d64_eight_wave_grouped_lse(dev):
    """The persistent d64 launch with grouped K/V heads (16 query heads over 4) and the log-sum-exp."""
    import transformer_scaled_dot_amd as tsd

    B, H, Hkv, N, d = 2, 16, 4, 2000, 64
    q = synth.normal_tensor(5200, (B, H, N, d))
    k, v = (synth.normal_tensor(5201 + i, (B, Hkv, N, d)) for i in range(2))
    vl = np.asarray([2000, 1234], dtype=np.int32)
    o, lse = tsd.attn_fwd(q.torch(dev), k.torch(dev), v.torch(dev), mask="causal_padding",
                          valid_lens=torch.from_numpy(vl).to(dev), return_lse=True)
    torch.cuda.synchronize()
    ref, rl = oracle.attention(q.f64, k.f64, v.f64, mask="causal_padding", valid_lens=vl, return_lse=True)
    check("bf16 [2,16/4,2000,64] causal_padding, persistent launch", o.float().cpu().numpy().astype(np.float64), ref,
          "bf16")
    err = np.abs(lse.cpu().numpy().astype(np.float64) - rl)
    say("  lse max abs err %.3e" % err.max())
    assert err.max() <= 2.0 ** -8 + 1e-4


@pytest.mark.parametrize("B,Nq,Nkv,dm,h,mask", [(2, 77, 130, 256, 4, "none"), (2, 200, 64, 512, 8, "padding"),
                                                 (1, 33, 300, 768, 6, "padding"), (3, 130, 130, 128, 1, "none"),
                                                 (2, 64, 1, 256, 2, "none")])
def test_mha_cross_layer(dev, B, Nq, Nkv, dm, h, mask):
    """The cross-attention layer (queries from one sequence, keys and values from another) against the
    oracle, every element: head widths 64 and 128, ragged lengths on both sides, a single key, and the
    key padding mask with one batch's keys cut to a third."""
    import transformer_scaled_dot_amd as tsd

    xq = synth.normal_tensor(5300 + Nq, (B, Nq, dm))
    xkv = synth.normal_tensor(5301 + Nkv, (B, Nkv, dm))
    _, wqkv, wo = synth.mha_inputs(4, B=1, N=1, d_model=dm)
    vl = np.asarray([Nkv, max(1, Nkv // 3), Nkv][:B], dtype=np.int32)
    vl_t = torch.from_numpy(vl).to(dev) if mask == "padding" else None
    y = tsd.mha_cross_fwd(xq.torch(dev), xkv.torch(dev), wqkv.torch(dev), wo.torch(dev), h, mask=mask,
                          valid_lens=vl_t)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    ref = oracle.mha_cross(xq.f64, xkv.f64, wqkv.f64, wo.f64, h, mask=mask, valid_lens=vl)
    check("mha cross [%d,%d<-%d,%d] h%d %s" % (B, Nq, Nkv, dm, h, mask), got, ref, "bf16")


def test_mha_cross_equals_self_layer(dev):
    """With the same sequence on both sides and no mask, the cross layer computes the self-attention
    layer (the same kernels: bit for bit)."""
    import transformer_scaled_dot_amd as tsd

    x, wqkv, wo = synth.mha_inputs(4, B=2, N=300, d_model=512)
    X, W, Wo = x.torch(dev), wqkv.torch(dev), wo.torch(dev)
    y1 = tsd.mha_fwd(X, W, Wo, 8)
    y2 = tsd.mha_cross_fwd(X, X, W, Wo, 8)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
