"""The seeded input generator (no GPU)."""
import numpy as np

import synth


def test_splitmix64_reference_outputs():
    # first outputs of Vigna's splitmix64 reference code from state 1234567
    assert synth.splitmix64(1234567, 0, 3).tolist() == [6457827717110365317, 3203168211198807973,
                                                        9817491932198370423]
    # counter-based access is the same stream
    assert synth.splitmix64(1234567, 2, 1).tolist() == [9817491932198370423]


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 3.0e38],
                 dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(f))
    # tie at 1 + 2^-8 goes to the even neighbour 1.0; 1 + 3*2^-8 ties up to 1 + 2^-6
    expect = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, np.float32(3.0e38)], dtype=np.float32)
    assert np.array_equal(got[:5], expect[:5])
    assert abs(got[5] - 3.0e38) / 3.0e38 < 2 ** -8


def test_normals_moments_and_determinism():
    z = synth.normal_f64(7, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.var() - 1) < 5e-3
    assert np.array_equal(z[:1000], synth.normal_f64(7, 1000))
    assert not np.array_equal(z[:1000], synth.normal_f64(8, 1000))


def test_scaled_score_variance():
    """With unit-variance q, k the scaled score q.k/sqrt(d_k) has variance 1
    (p1 section 四 stage 2; p5 为什么要除以 sqrt(d_k)); the long-context
    workload doubles q and k, so its scaled scores have variance 16."""
    for config, target in ((3, 1.0), (5, 16.0)):
        q, k, _, _ = synth.attn_inputs(config, B=1, H=1, N=2048)
        s = (q.f64[0, 0] @ k.f64[0, 0].T) / np.sqrt(q.shape[-1])
        assert abs(s.var() / target - 1) < 0.03


def test_valid_lens_range():
    _, _, _, vl = synth.attn_inputs(2, N=8, d=64)
    assert vl.dtype == np.int32 and vl.shape == (8,)
    assert np.all((vl >= 256) & (vl <= 512))
    many = synth.uniform_ints(99, 100000, 256, 512)
    assert many.min() == 256 and many.max() == 512


def test_config_shapes():
    x, wqkv, wo = synth.mha_inputs(4, B=1, N=4)
    assert x.shape == (1, 4, 512) and wqkv.shape == (512, 1536) and wo.shape == (512, 512)
    assert abs(wqkv.f64.var() * 512 - 1) < 0.02
