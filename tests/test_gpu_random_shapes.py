"""Seeded random shapes against the oracle, on an MI355X: batch, heads, grouped K/V heads, ragged sequence lengths
(including empty and single-row sequences), every mask with valid lengths anywhere in [0, N_k], both head widths of
the bf16 path with both output types and the log-sum-exp, the fp32 path at every head width, and the backward pass
on a few of them. The shapes are drawn once from fixed seeds, so every run checks the same cases; each case prints
its shape before it runs. Tolerances are those of test_gpu_parity.py and test_gpu_features.py; the backward pass
uses test_gpu_backward.py's per-element bounds."""
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
MASKS = ["none", "causal", "padding", "causal_padding"]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import transformer_scaled_dot_amd as tsd

    tsd.load_library()
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def draw(n, seed, dims, max_n, outs=("f32", "bf16", "bf16")):
    """n cases (index, B, H, H_kv, N_q, N_k, d, mask, valid_lens, out): masks in turn, the causal ones with
    N_q = N_k (the only shapes they are defined for here), valid lengths uniform in [0, N_k], output types in
    turn from outs."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        mask = MASKS[i % len(MASKS)]
        d = int(rng.choice(dims))
        B = int(rng.integers(1, 4))
        hkv = int(rng.integers(1, 4))
        H = hkv * int(rng.integers(1, 4))
        nq = int(rng.integers(1, max_n + 1))
        nk = nq if mask.startswith("causal") else int(rng.integers(1, max_n + 1))
        vl = [int(x) for x in rng.integers(0, nk + 1, size=B)] if mask in ("padding", "causal_padding") else None
        cases.append((i, B, H, hkv, nq, nk, d, mask, vl, outs[i % len(outs)]))
    return cases


def case_id(c):
    i, B, H, hkv, nq, nk, d, mask, vl, out = c
    return "%d-B%dH%dkv%d-%dx%d-d%d-%s-%s" % (i, B, H, hkv, nq, nk, d, mask, out)


def check_out(name, got, ref, dtype):
    err = np.abs(got - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    say("%s: max abs err %.3e, mean %.3e" % (name, mx, mean))
    assert np.all(np.isfinite(got)), name + ": non-finite output"
    if dtype == "f32":
        assert mx <= TOL_F32, name
    else:
        assert mx <= TOL_BF16_MAX and mean <= TOL_BF16_MEAN, name


def check_lse(name, got, ref, dtype):
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), name + ": rows without a visible key differ"
    err = np.abs(got[~empty] - ref[~empty])
    mx = float(err.max()) if err.size else 0.0
    say("%s lse: max abs err %.3e (%d rows without a visible key)" % (name, mx, int(empty.sum())))
    assert np.all(np.isfinite(got[~empty])), name
    assert mx <= (TOL_LSE_F32 if dtype == "f32" else TOL_LSE_BF16), name


def run_forward(dev, c, dtype):
    import transformer_scaled_dot_amd as tsd

    i, B, H, hkv, nq, nk, d, mask, vl, out = c
    name = "%s %s" % (dtype, case_id(c))
    say("case", name, "valid_lens", vl)
    seed = 9000 + 10 * i + (0 if dtype == "bf16" else 5)
    q = synth.normal_tensor(seed, (B, H, nq, d), dtype)
    k = synth.normal_tensor(seed + 1, (B, hkv, nk, d), dtype)
    v = synth.normal_tensor(seed + 2, (B, hkv, nk, d), dtype)
    vl_t = torch.tensor(vl, dtype=torch.int32, device=dev) if vl is not None else None
    od = torch.float32 if (dtype == "f32" or out == "f32") else torch.bfloat16
    o, lse = tsd.attn_fwd(q.torch(dev), k.torch(dev), v.torch(dev), mask=mask, valid_lens=vl_t, out_dtype=od,
                          return_lse=True)
    torch.cuda.synchronize()
    ref, rl = oracle.attention(q.f64, k.f64, v.f64, mask=mask, valid_lens=vl, return_lse=True)
    check_out(name, o.float().cpu().numpy().astype(np.float64), ref, dtype)
    check_lse(name, lse.cpu().numpy().astype(np.float64), rl, dtype)


@pytest.mark.parametrize("c", draw(24, 20261202, (64, 128), 700), ids=case_id)
def test_random_shapes_bf16(dev, c):
    run_forward(dev, c, "bf16")


@pytest.mark.parametrize("c", draw(12, 20261203, (16, 32, 64, 128), 300, outs=("f32",)), ids=case_id)
def test_random_shapes_f32(dev, c):
    run_forward(dev, c, "f32")


@pytest.mark.parametrize("c", draw(8, 20261204, (64, 128), 260, outs=("bf16",)), ids=case_id)
def test_random_shapes_backward(dev, c):
    from test_gpu_backward import run_case

    i, B, H, hkv, nq, nk, d, mask, vl, _ = c
    say("case bwd", case_id(c), "valid_lens", vl)
    run_case(dev, 9500 + 10 * i, B, H, hkv, nq, nk, d, mask, vl=vl)
