"""Parity of the HIP path with the CPU oracle for the causal-and-padding mask,
grouped K/V heads and the per-row log-sum-exp (through the C ABI entry
point attn_fwd_ex), on an MI355X.

Output tolerances are those of test_gpu_parity.py. Log-sum-exp tolerances:
  bfloat16 inputs: the kernel sums the bf16-rounded weights it applies to V;
    bf16 keeps 8 significant bits, so each is within a relative 2^-8 (its
    unit roundoff) of the exact weight, the sum too, and ln l is within
    2^-8 of the exact value; float32 scores, logs and the final multiply add
    well under 1e-4 for |lse| < 100: 2^-8 + 1e-4.
  float32 inputs: the row state is updated once per key with float32
    exponentials and products (unit roundoff 2^-24 each), so for up to 800
    keys the sum is within a relative ~800 * 2^-24 ~ 5e-5 at worst: 1e-4.
Rows without a visible key must give -inf on both sides.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16_MAX, TOL_BF16_MEAN = 2e-2, 2e-3
TOL_LSE_BF16 = 2.0 ** -8 + 1e-4
TOL_LSE_F32 = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_scaled_dot_amd as tsd

    tsd.load_library()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def inputs(seed, B, H, Hkv, Nq, Nk, d, dtype="bf16"):
    return (synth.normal_tensor(seed, (B, H, Nq, d), dtype), synth.normal_tensor(seed + 1, (B, Hkv, Nk, d), dtype),
            synth.normal_tensor(seed + 2, (B, Hkv, Nk, d), dtype))


def run(dev, q, k, v, mask, vl=None, out_dtype=None):
    import transformer_scaled_dot_amd as tsd

    vl_t = torch.from_numpy(np.asarray(vl, dtype=np.int32)).to(dev) if vl is not None else None
    od = {None: None, "f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    o, lse = tsd.attn_fwd(q.torch(dev), k.torch(dev), v.torch(dev), mask=mask, valid_lens=vl_t, out_dtype=od,
                          return_lse=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_out(name, got, ref, dtype):
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    say("%s: max abs err %.3e, mean %.3e" % (name, mx, mean))
    assert np.all(np.isfinite(got)), "non-finite output"
    if dtype == "f32":
        assert mx <= TOL_F32, name
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, name


def check_lse(name, got, ref, dtype):
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), name + ": -inf rows differ"
    err = np.abs(got[~empty] - ref[~empty])
    mx = float(err.max()) if err.size else 0.0
    say("%s lse: max abs err %.3e (%d rows without a visible key)" % (name, mx, int(empty.sum())))
    assert np.all(np.isfinite(got[~empty]))
    assert mx <= (TOL_LSE_F32 if dtype == "f32" else TOL_LSE_BF16), name


# valid lengths at and around the 64-key tiles, the 64-row waves and the 256-row work items, one of them 0 and
# one past the end (clamped)
LENS = [0, 1, 64, 130, 255, 257, 450, 700]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [600, 333])
def test_causal_padding_bf16(dev, n, d, out):
    B, H = len(LENS), 2
    q, k, v = inputs(3100 + n + d, B, H, H, n, n, d)
    vl = np.asarray(LENS, dtype=np.int32)
    got, lse = run(dev, q, k, v, "causal_padding", vl, out)
    ref, rl = oracle.attention(q.f64, k.f64, v.f64, mask="causal_padding", valid_lens=np.minimum(vl, n),
                               return_lse=True)
    name = "bf16 [%d,%d,%d] d%d causal_padding out %s" % (B, H, n, d, out)
    check_out(name, got, ref, "bf16")
    check_lse(name, lse, rl, "bf16")


@pytest.mark.parametrize("d", [16, 64, 128])
def test_causal_padding_f32(dev, d):
    B, H, n = 4, 2, 77
    q, k, v = inputs(3200 + d, B, H, H, n, n, d, "f32")
    vl = np.asarray([0, 5, 33, 90], dtype=np.int32)
    got, lse = run(dev, q, k, v, "causal_padding", vl)
    ref, rl = oracle.attention(q.f64, k.f64, v.f64, mask="causal_padding", valid_lens=np.minimum(vl, n),
                               return_lse=True)
    check_out("f32 d%d causal_padding" % d, got, ref, "f32")
    check_lse("f32 d%d causal_padding" % d, lse, rl, "f32")


@pytest.mark.parametrize("mask", ["none", "causal", "padding", "causal_padding"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hkv", [1, 2, 4])
def test_grouped_kv_heads_bf16(dev, hkv, d, mask):
    B, H = 2, 4
    nq, nk = (300, 300) if mask.startswith("causal") else (200, 270)
    q, k, v = inputs(3300 + 10 * hkv + d, B, H, hkv, nq, nk, d)
    vl = np.asarray([nk // 3, nk], dtype=np.int32)
    got, lse = run(dev, q, k, v, mask, vl)
    ref, rl = oracle.attention(q.f64, k.f64, v.f64, mask=mask, valid_lens=vl, return_lse=True)
    name = "bf16 H%d H_kv%d [%d,%d] d%d %s" % (H, hkv, nq, nk, d, mask)
    check_out(name, got, ref, "bf16")
    check_lse(name, lse, rl, "bf16")


@pytest.mark.parametrize("hkv", [1, 3])
def test_grouped_kv_heads_f32(dev, hkv):
    B, H, nq, nk, d = 2, 6, 20, 45, 32
    q, k, v = inputs(3400 + hkv, B, H, hkv, nq, nk, d, "f32")
    vl = np.asarray([7, 45], dtype=np.int32)
    for mask in ("none", "padding"):
        got, lse = run(dev, q, k, v, mask, vl)
        ref, rl = oracle.attention(q.f64, k.f64, v.f64, mask=mask, valid_lens=vl, return_lse=True)
        check_out("f32 H_kv%d %s" % (hkv, mask), got, ref, "f32")
        check_lse("f32 H_kv%d %s" % (hkv, mask), lse, rl, "f32")


@pytest.mark.parametrize("mask", ["none", "causal", "padding"])
@pytest.mark.parametrize("d", [64, 128])
def test_lse_plain_heads(dev, d, mask):
    """The log-sum-exp of the three original masks, with ragged sizes and a scale far from 1/sqrt(d)."""
    import transformer_scaled_dot_amd as tsd

    B, H, n = 2, 3, 333
    q, k, v = inputs(3500 + d, B, H, H, n, n, d)
    vl = np.asarray([0, 200], dtype=np.int32)
    vl_t = torch.from_numpy(vl).to(dev)
    o, lse = tsd.attn_fwd(q.torch(dev), k.torch(dev), v.torch(dev), mask=mask, valid_lens=vl_t, scale=0.3,
                          return_lse=True)
    torch.cuda.synchronize()
    ref, rl = oracle.attention(q.f64, k.f64, v.f64, mask=mask, valid_lens=vl, scale=0.3, return_lse=True)
    check_out("bf16 d%d %s scale 0.3" % (d, mask), o.float().cpu().numpy().astype(np.float64), ref, "bf16")
    check_lse("bf16 d%d %s scale 0.3" % (d, mask), lse.cpu().numpy().astype(np.float64), rl, "bf16")


def test_lse_output_equals_plain_call(dev):
    """Asking for the log-sum-exp does not change O (bit for bit), and H_kv = H is the plain call."""
    import transformer_scaled_dot_amd as tsd

    q, k, v = inputs(3600, 2, 4, 4, 520, 520, 128)
    Q, K, V = q.torch(dev), k.torch(dev), v.torch(dev)
    o1 = tsd.attn_fwd(Q, K, V, mask="causal")
    o2, _ = tsd.attn_fwd(Q, K, V, mask="causal", return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_causal_grouped_full_size(dev):
    """The causal 4K launch shape (B4 H16 N4096 d128) with 4 K/V heads, the causal-and-padding mask and the
    log-sum-exp: every output element and every row's log-sum-exp against the oracle."""
    B, H, Hkv, N, d = 4, 16, 4, 4096, 128
    q, k, v = inputs(3700, B, H, Hkv, N, N, d)
    vl = np.asarray([4096, 3000, 1111, 64], dtype=np.int32)
    got, lse = run(dev, q, k, v, "causal_padding", vl)
    ref, rl = oracle.attention(q.f64, k.f64, v.f64, mask="causal_padding", valid_lens=vl, return_lse=True)
    check_out("bf16 [4,16/4,4096,128] causal_padding (every element)", got, ref, "bf16")
    check_lse("bf16 [4,16/4,4096,128] causal_padding (every row)", lse, rl, "bf16")


@pytest.mark.parametrize("case", ["padding_d64", "causal_d128", "mha"])
def test_graph_replay_matches_eager(dev, case):
    """The attention and multi-head calls captured into a HIP graph (torch.cuda.CUDAGraph, as bench.py times
    its launch-bound workloads): three replays, each preceded by clearing the outputs and an eager launch of
    another shape and followed by a synchronisation, each give bitwise the outputs of the same calls run
    eagerly."""
    import transformer_scaled_dot_amd as tsd

    sets = []
    if case == "mha":
        B, N, dm, h = 2, 256, 256, 4
        for s in range(2):
            x = synth.normal_tensor(700 + s, (B, N, dm), "bf16").torch(dev)
            wq = (synth.normal_tensor(710 + s, (dm, 3 * dm), "bf16").torch(dev).float() / dm ** 0.5).to(torch.bfloat16)
            wo = (synth.normal_tensor(720 + s, (dm, dm), "bf16").torch(dev).float() / dm ** 0.5).to(torch.bfloat16)
            ws = torch.empty(int(tsd.load_library().mha_workspace_bytes(B, N, dm, h, 1)), dtype=torch.uint8, device=dev)
            sets.append((x, wq, wo, ws, torch.empty((B, N, dm), dtype=torch.bfloat16, device=dev)))

        def call(i):
            x, wq, wo, ws, o = sets[i]
            tsd.mha_fwd(x, wq, wo, h, out=o, workspace=ws)
    else:
        if case == "padding_d64":
            B, H, N, d, mask, vl = 2, 4, 300, 64, "padding", [200, 300]
        else:
            B, H, N, d, mask, vl = 1, 2, 500, 128, "causal", None
        vl_t = torch.tensor(vl, dtype=torch.int32, device=dev) if vl else None
        for s in range(2):
            q, k, v = inputs(730 + 3 * s, B, H, H, N, N, d)
            sets.append((q.torch(dev), k.torch(dev), v.torch(dev),
                         torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)))

        def call(i):
            q, k, v, o = sets[i]
            tsd.attn_fwd(q, k, v, mask=mask, valid_lens=vl_t, out=o)

    outs = [st[-1] for st in sets]
    for i in range(len(sets)):
        call(i)
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(len(sets)):
            call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(len(sets)):
            call(i)
    oq, ok_, ov = inputs(760, 1, 2, 2, 130, 130, 64)
    for rep in range(3):
        say("graph replay", case, rep)
        for o in outs:
            o.zero_()
        tsd.attn_fwd(oq.torch(dev), ok_.torch(dev), ov.torch(dev), mask="causal")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(o, w), "replay %d, set %d differs from the eager result" % (rep, j)
