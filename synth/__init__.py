"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no attention arithmetic: it only draws numbers. Both the
HIP path and the CPU oracle receive exactly the values produced here (the
oracle widens them to float64), so neither side ever generates its own
inputs.

Generator: SplitMix64 (S. Vigna, public-domain reference implementation of
``splitmix64``) used as a counter-based stream: draw k of stream ``seed`` is
``mix(seed + (k + 1) * GAMMA)``, which equals the k-th output of the
sequential generator started at state ``seed``. Uniforms take the top 53
bits; normals come from the Box-Muller transform on pairs of uniforms in
float64, then are rounded to float32 and, for bfloat16 tensors, to bfloat16
with round-to-nearest-even.

Sub-seeds: ``1000 * config + tensor_id`` with tensor ids Q=0, K=1, V=2,
valid_lens=3, X=4, W_qkv=5, W_o=6.
"""
from __future__ import annotations

import os

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_ID = {"Q": 0, "K": 1, "V": 2, "valid_lens": 3, "X": 4, "W_qkv": 5, "W_o": 6}

_CHUNK = 1 << 22


def sub_seed(config: int, tensor: str) -> int:
    return 1000 * int(config) + TENSOR_ID[tensor]


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws ``start .. start+count-1`` of the SplitMix64 stream ``seed``."""
    k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * GAMMA)


def uniform01(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Uniform doubles in (0, 1]: ((x >> 11) + 1) * 2^-53."""
    x = splitmix64(seed, start, count)
    return ((x >> np.uint64(11)).astype(np.float64) + 1.0) * (1.0 / 9007199254740992.0)


def _normal_pairs(seed: int, p0: int, n: int) -> np.ndarray:
    u = uniform01(seed, 2 * n, start=2 * p0)
    r = np.sqrt(-2.0 * np.log(u[0::2]))
    t = (2.0 * np.pi) * u[1::2]
    z = np.empty(2 * n, dtype=np.float64)
    z[0::2] = r * np.cos(t)
    z[1::2] = r * np.sin(t)
    return z


def normal_f64(seed: int, count: int) -> np.ndarray:
    """``count`` standard normals (Box-Muller on consecutive uniform pairs).
    Chunks are independent slices of the stream, so they are filled by a
    few threads (numpy releases the GIL) without changing any value."""
    out = np.empty(count, dtype=np.float64)
    pairs = (count + 1) // 2

    def fill(p0):
        n = min(_CHUNK, pairs - p0)
        z = _normal_pairs(seed, p0, n)
        lo = 2 * p0
        hi = min(count, lo + 2 * n)
        out[lo:hi] = z[: hi - lo]

    starts = list(range(0, pairs, _CHUNK))
    if len(starts) <= 1:
        for p0 in starts:
            fill(p0)
    else:
        import concurrent.futures as cf

        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1, len(starts))) as ex:
            list(ex.map(fill, starts))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (b & 0x7FFFFFFF) > 0x7F800000
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    rounded = np.where(nan, (b >> np.uint32(16)) | np.uint32(0x40), rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Tensor:
    """A synthetic tensor: ``f64`` holds the exact values (after rounding to
    the storage dtype), ``raw`` the storage (float32 array or uint16
    bfloat16 bits) with ``shape``."""

    def __init__(self, raw: np.ndarray, dtype: str, shape):
        self.raw = raw.reshape(shape)
        self.dtype = dtype
        self.shape = tuple(shape)

    @property
    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.raw).reshape(self.shape)
        return self.raw

    @property
    def f64(self) -> np.ndarray:
        return self.f32.astype(np.float64)

    def torch(self, device="cpu"):
        import torch

        if self.dtype == "bf16":
            t = torch.from_numpy(self.raw.view(np.int16).copy()).view(torch.bfloat16)
        else:
            t = torch.from_numpy(self.raw.copy())
        return t.reshape(self.shape).to(device)


def normal_tensor(seed: int, shape, dtype: str = "bf16", std: float = 1.0) -> Tensor:
    """N(0, std^2) values, rounded to float32 and then to ``dtype``."""
    n = int(np.prod(shape))
    x = (normal_f64(seed, n) * std).astype(np.float32)
    if dtype == "bf16":
        return Tensor(f32_to_bf16_bits(x), "bf16", shape)
    if dtype == "f32":
        return Tensor(x, "f32", shape)
    raise ValueError(dtype)


def uniform_ints(seed: int, count: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on [lo, hi] inclusive, as int32."""
    u = uniform01(seed, count)  # (0, 1]
    v = lo + np.floor((1.0 - u) * (hi - lo + 1)).astype(np.int64)
    return np.clip(v, lo, hi).astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads. Sizes follow the shapes the pages use: the 3-token
# worked example and a [b=2, n=5, d=16] float test, the base model's
# d_model=512 / 8 heads of 64, a 4096-token causal layer with 128-wide heads
# and a 32768-token, 32-head long-context case.
# ---------------------------------------------------------------------------
CONFIGS = {
    1: dict(name="sdpa_f32_b2_n5_d16", kind="attn", B=2, H=1, N=5, d=16, dtype="f32", mask="none", std=1.0),
    2: dict(name="sdpa_bf16_b8_h8_n512_d64_padding", kind="attn", B=8, H=8, N=512, d=64, dtype="bf16",
            mask="padding", std=1.0, lens=(256, 512)),
    3: dict(name="sdpa_bf16_b4_h16_n4096_d128_causal", kind="attn", B=4, H=16, N=4096, d=128, dtype="bf16",
            mask="causal", std=1.0),
    4: dict(name="mha_bf16_b4_n2048_dmodel512_h8", kind="mha", B=4, N=2048, d_model=512, h=8, dtype="bf16"),
    5: dict(name="sdpa_bf16_b1_h32_n32768_d128_causal_x2", kind="attn", B=1, H=32, N=32768, d=128, dtype="bf16",
            mask="causal", std=2.0),
}


def attn_inputs(config: int, B=None, H=None, N=None, d=None, dtype=None, std=None, lens=None, Nk=None):
    """Q, K, V (and valid_lens for padding) for an attention workload.
    Any size argument overrides the config's value (same seeds)."""
    c = CONFIGS[config]
    B = c["B"] if B is None else B
    H = c["H"] if H is None else H
    N = c["N"] if N is None else N
    Nk = N if Nk is None else Nk
    d = c["d"] if d is None else d
    dtype = c["dtype"] if dtype is None else dtype
    std = c["std"] if std is None else std
    q = normal_tensor(sub_seed(config, "Q"), (B, H, N, d), dtype, std)
    k = normal_tensor(sub_seed(config, "K"), (B, H, Nk, d), dtype, std)
    v = normal_tensor(sub_seed(config, "V"), (B, H, Nk, d), dtype, std)
    vl = None
    lens = c.get("lens") if lens is None else lens
    if lens is not None:
        lo, hi = lens
        vl = uniform_ints(sub_seed(config, "valid_lens"), B, lo, hi)
    return q, k, v, vl


def mha_inputs(config: int = 4, B=None, N=None, d_model=None, dtype=None):
    c = CONFIGS[config]
    B = c["B"] if B is None else B
    N = c["N"] if N is None else N
    d_model = c["d_model"] if d_model is None else d_model
    dtype = c["dtype"] if dtype is None else dtype
    x = normal_tensor(sub_seed(config, "X"), (B, N, d_model), dtype, 1.0)
    w_std = float(np.sqrt(1.0 / d_model))
    w_qkv = normal_tensor(sub_seed(config, "W_qkv"), (d_model, 3 * d_model), dtype, w_std)
    w_o = normal_tensor(sub_seed(config, "W_o"), (d_model, d_model), dtype, w_std)
    return x, w_qkv, w_o
