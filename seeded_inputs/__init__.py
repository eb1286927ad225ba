"""Seeded synthetic inputs for the H-BitLinear forward pass.

This module is shared by the oracle side and the HIP side of every test and benchmark.  It
holds random-number generation and workload recipes only -- none of the layer's arithmetic
(no ternarisation, transform, quantisation or product).

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014) used counter-style -- draw i of stream ``seed`` is
``mix64(seed + (i + 1) * 0x9E3779B97F4A7C15)`` -- so any slice of a stream can be produced
on its own.  Uniforms take the top 53 bits; normals use Box-Muller (both outputs of a pair);
Laplace uses the inverse CDF.  Everything is computed in float64 and rounded once to
float32, so a stream is the same wherever numpy's libm is the same.

Workload recipes mirror the activation statistics the pages describe for H-BitLinear inputs
(Gaussian-like inputs to the first linears; outlier channels and mass near zero at the
inputs of the attention output and FFN down projections).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
SEED_BASE = 0xB17E7000


def seed_for(config: int, role: int) -> int:
    """Per-config, per-tensor seed: 0xB17E7000 + 16 * config + role."""
    return SEED_BASE + 16 * int(config) + int(role)


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of the SplitMix64 stream ``seed`` (uint64)."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform(seed: int, count: int, start: int = 0) -> np.ndarray:
    """float64 uniforms in [0, 1) from the top 53 bits."""
    z = splitmix64(seed, start, count)
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def _chunks(count: int, chunk: int = 1 << 24):
    for s in range(0, count, chunk):
        yield s, min(chunk, count - s)


def normal(seed: int, count: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """float32 normals by Box-Muller over consecutive uniform pairs."""
    out = np.empty(count, np.float32)
    npairs = (count + 1) // 2
    for s, c in _chunks(npairs):
        u = uniform(seed, 2 * c, 2 * s)
        u1 = 1.0 - u[0::2]            # (0, 1]
        u2 = u[1::2]
        r = np.sqrt(-2.0 * np.log(u1))
        th = 2.0 * math.pi * u2
        z = np.empty(2 * c, np.float64)
        z[0::2] = r * np.cos(th)
        z[1::2] = r * np.sin(th)
        lo = 2 * s
        hi = min(count, 2 * (s + c))
        out[lo:hi] = (mean + std * z[: hi - lo]).astype(np.float32)
    return out


def laplace(seed: int, count: int, b: float) -> np.ndarray:
    """float32 Laplace(0, b) by the inverse CDF."""
    out = np.empty(count, np.float32)
    for s, c in _chunks(count):
        u = uniform(seed, c, s) - 0.5          # [-0.5, 0.5)
        a = np.abs(u)
        z = -b * np.sign(u) * np.log(np.maximum(1.0 - 2.0 * a, 1e-300))
        out[s:s + c] = z.astype(np.float32)
    return out


def choose_columns(seed: int, K: int, k: int) -> np.ndarray:
    """k distinct indices in [0, K) by a partial Fisher-Yates shuffle driven by ``seed``."""
    perm = np.arange(K, dtype=np.int64)
    u = uniform(seed, k)
    for i in range(k):
        j = i + int(u[i] * (K - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:k])


def with_outlier_columns(x: np.ndarray, seed: int, fraction_or_count, factor: float):
    """Multiply k chosen columns (channels) of every token row by ``factor``."""
    K = x.shape[1]
    k = fraction_or_count if isinstance(fraction_or_count, int) else int(round(fraction_or_count * K))
    cols = choose_columns(seed, K, k)
    x[:, cols] *= np.float32(factor)
    return cols


# ---- recipes -----------------------------------------------------------------------------

ROLE_X, ROLE_X_B, ROLE_OUTLIERS, ROLE_W0 = 0, 1, 2, 3


def gaussian_activations(config: int, M: int, K: int, role: int = ROLE_X) -> np.ndarray:
    return normal(seed_for(config, role), M * K).reshape(M, K)


def gaussian_weights(config: int, N: int, K: int, layer: int = 0, std: float = 0.02):
    """fp32 N(0, std) weights for one linear (std = 0.02 taken as the standard deviation)."""
    return normal(seed_for(config, ROLE_W0 + layer), N * K, 0.0, std).reshape(N, K)


def tiny_activations(M: int = 16, K: int = 256) -> np.ndarray:
    """N(0,1) with 4 outlier channels x20 (the CPU-sized H-BitLinear case)."""
    x = gaussian_activations(1, M, K)
    with_outlier_columns(x, seed_for(1, ROLE_OUTLIERS), 4, 20.0)
    return x


def wo_activations(M: int, K: int, config: int = 3) -> np.ndarray:
    """Heavy-tailed input of the attention output projection: Laplace(0, 0.05) with 1% of
    channels x50."""
    x = laplace(seed_for(config, ROLE_X), M * K, 0.05).reshape(M, K)
    with_outlier_columns(x, seed_for(config, ROLE_OUTLIERS), 0.01, 50.0)
    return x


def wdown_activations(M: int, K: int, config: int = 4, outliers=0.005) -> np.ndarray:
    """Input of the FFN down projection: SiLU(a) * b with a, b ~ N(0,1) (mostly near zero),
    plus outlier channels x30 (0.5% of K, or a given count)."""
    a = normal(seed_for(config, ROLE_X), M * K).reshape(M, K)
    b = normal(seed_for(config, ROLE_X_B), M * K).reshape(M, K)
    a64 = a.astype(np.float64)
    x = (a64 / (1.0 + np.exp(-a64)) * b).astype(np.float32)
    with_outlier_columns(x, seed_for(config, ROLE_OUTLIERS), outliers, 30.0)
    return x


@dataclass
class Linear:
    name: str
    M: int
    K: int
    N: int
    act_bits: int
    use_hadamard: bool
    x_kind: str            # "gauss", "wo", "wdown", "tiny"
    layer: int = 0


@dataclass
class Workload:
    config: int
    name: str
    linears: list = field(default_factory=list)


def workload(config: int, M: int | None = None) -> Workload:
    """The five synthetic workloads (config numbers 1..5)."""
    if config == 1:
        M = 16 if M is None else M
        return Workload(1, "hbitlinear_tiny_M16_K256_N256_int8_hadamard",
                        [Linear("tiny", M, 256, 256, 8, True, "tiny")])
    if config == 2:
        M = 16 if M is None else M
        return Workload(2, f"bitlinear_w158a8_decode_M{M}_K4096_N4096",
                        [Linear("decode", M, 4096, 4096, 8, False, "gauss")])
    if config == 3:
        M = 4096 if M is None else M
        return Workload(3, f"hbitlinear_wo_int4_M{M}_K4096_N4096",
                        [Linear("wo", M, 4096, 4096, 4, True, "wo")])
    if config == 4:
        M = 8192 if M is None else M
        return Workload(4, f"hbitlinear_wdown_int4_M{M}_K16384_N4096",
                        [Linear("wdown", M, 16384, 4096, 4, True, "wdown")])
    if config == 5:
        M = 16384 if M is None else M
        return Workload(5, f"bitnet_v2_7b_block_int4_M{M}", [
            Linear("q", M, 4096, 4096, 4, False, "gauss", 0),
            Linear("k", M, 4096, 4096, 4, False, "gauss", 1),
            Linear("v", M, 4096, 4096, 4, False, "gauss", 2),
            Linear("wo", M, 4096, 4096, 4, True, "wo", 3),
            Linear("gate", M, 4096, 8192, 4, False, "gauss_ffn", 4),
            Linear("up", M, 4096, 8192, 4, False, "gauss_ffn", 5),
            Linear("wdown", M, 8192, 4096, 4, True, "wdown41", 6),
        ])
    raise ValueError(f"unknown config {config}")


def activations(config: int, lin: Linear) -> np.ndarray:
    """Synthetic fp32 activations for one linear of a workload."""
    if lin.x_kind == "tiny":
        return tiny_activations(lin.M, lin.K)
    if lin.x_kind == "gauss":
        return gaussian_activations(config, lin.M, lin.K, ROLE_X)
    if lin.x_kind == "gauss_ffn":
        return gaussian_activations(config, lin.M, lin.K, ROLE_X_B)
    if lin.x_kind == "wo":
        return wo_activations(lin.M, lin.K, config)
    if lin.x_kind == "wdown":
        return wdown_activations(lin.M, lin.K, config)
    if lin.x_kind == "wdown41":
        # separate seeds from the Wo input of the same block
        return wdown_activations(lin.M, lin.K, config + 8, outliers=41)
    raise ValueError(lin.x_kind)


def weights(config: int, lin: Linear) -> np.ndarray:
    return gaussian_weights(config, lin.N, lin.K, lin.layer)
