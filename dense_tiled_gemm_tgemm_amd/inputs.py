"""Seeded synthetic inputs and the workload registry.

This module holds no arithmetic of the matrix product: it only draws the
operands. Both the GPU tests and the oracle receive the arrays it returns.

Generator (same recipe for every workload): ``rng =
numpy.random.default_rng(seed)`` (PCG64); draw A as an (M, K) float64 array,
then B in its stored shape ((K, N) for the KxN layout, (N, K) for NxK); scale;
round to binary16 with numpy's ``astype(float16)`` (round to nearest even).
Uniform draws use ``rng.uniform(-1, 1, shape)``, normal draws
``rng.standard_normal(shape) * sigma``.

The five workloads are the square fp16 sizes the pages benchmark (page 1's
sweep of square fp16 sizes; page 5's 8192^3 problem with its right operand
stored N x K), a ragged shape whose sizes are multiples of no tile size, and a
transformer-projection shape (8192 tokens, hidden 4096, fused QKV width 12288).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    b_layout: str          # "KxN" (B[k*ldb + j]) or "NxK" (B[j*ldb + k])
    a_dist: tuple          # ("uniform", lo, hi) or ("normal", sigma)
    b_dist: tuple
    seed: int
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def b_shape(self):
        return (self.K, self.N) if self.b_layout == "KxN" else (self.N, self.K)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("sq256", 256, 256, 256, "KxN", ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), 0,
                 "256^3, B K x N, U[-1,1]"),
        Workload("sq4096", 4096, 4096, 4096, "KxN", ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), 1,
                 "4096^3, B K x N, U[-1,1]"),
        Workload("sq8192_nt", 8192, 8192, 8192, "NxK", ("normal", 0.1), ("normal", 0.1), 2,
                 "8192^3, B stored N x K, N(0,1)*0.1"),
        Workload("ragged", 3001, 5003, 4099, "KxN", ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), 3,
                 "3001 x 5003 x 4099, B K x N, U[-1,1]"),
        Workload("qkv_proj", 8192, 12288, 4096, "NxK", ("normal", 1.0), ("normal", 0.02), 4,
                 "M=8192 tokens, K=4096 hidden, N=12288 fused QKV, B stored N x K"),
    ]
}

# The workload the headline throughput is quoted on.
HEADLINE = "sq8192_nt"


def _draw64(rng: np.random.Generator, dist: tuple, shape) -> np.ndarray:
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], shape)
    if kind == "normal":
        return rng.standard_normal(shape) * dist[1]
    raise ValueError(f"unknown distribution {dist!r}")


def _draw(rng: np.random.Generator, dist: tuple, shape) -> np.ndarray:
    return _draw64(rng, dist, shape).astype(np.float16)


def to_bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of finite values: round to binary32 with
    numpy, then keep the upper 16 bits rounded to nearest even (add 0x7fff plus
    the lowest kept bit, then shift). Used to draw inputs only."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def make_inputs(w: Workload, ab_type: str = "f16"):
    """(A, B) as C-contiguous arrays: A is (M, K), B is ``w.b_shape``.
    ab_type "f16": float16 arrays; "bf16": uint16 bfloat16 bit patterns drawn
    from the same seeded values; "f32": float32 arrays of the same values."""
    rng = np.random.default_rng(w.seed)
    if ab_type == "f16":
        A = _draw(rng, w.a_dist, (w.M, w.K))
        B = _draw(rng, w.b_dist, w.b_shape)
    elif ab_type == "bf16":
        A = to_bf16_bits(_draw64(rng, w.a_dist, (w.M, w.K)))
        B = to_bf16_bits(_draw64(rng, w.b_dist, w.b_shape))
    elif ab_type == "f32":
        A = _draw64(rng, w.a_dist, (w.M, w.K)).astype(np.float32)
        B = _draw64(rng, w.b_dist, w.b_shape).astype(np.float32)
    else:
        raise ValueError(f"unknown input type {ab_type!r}")
    return A, B


def random_bf16(shape, seed: int, dist=("uniform", -1.0, 1.0)) -> np.ndarray:
    """Seeded bfloat16 bit patterns (uint16) for small ad-hoc shapes."""
    return to_bf16_bits(_draw64(np.random.default_rng(seed), dist, shape))


def random_f32(shape, seed: int, dist=("uniform", -1.0, 1.0)) -> np.ndarray:
    """Seeded binary32 array for small ad-hoc shapes."""
    return _draw64(np.random.default_rng(seed), dist, shape).astype(np.float32)


def random_bias(n: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """Seeded float32 bias vector, uniform in [-scale, scale]."""
    return (np.random.default_rng(seed).uniform(-scale, scale, n)).astype(np.float32)


def random_f16(shape, seed: int, dist=("uniform", -1.0, 1.0)) -> np.ndarray:
    """Seeded binary16 array for small ad-hoc shapes."""
    return _draw(np.random.default_rng(seed), dist, shape)


def ternary_f16(shape, seed: int) -> np.ndarray:
    """Seeded array with entries in {-1, 0, +1} (exactly representable)."""
    rng = np.random.default_rng(seed)
    return rng.integers(-1, 2, size=shape).astype(np.float16)


def sha256(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()


def sample_points(M: int, N: int, n_random: int, seed: int, tile_m: int = 256, tile_n: int = 256):
    """Output elements to check on workloads too large for a full check.

    Every row of the last tile-row and every column of the last tile-column
    (when M or N is not a multiple of the tile), the four corners of every
    8th tile, and ``n_random`` uniformly random elements from
    ``default_rng(seed)``. Duplicates are removed; order is row-major.
    """
    pts = set()
    rng = np.random.default_rng(seed)
    gm, gn = -(-M // tile_m), -(-N // tile_n)
    if M % tile_m:
        r0 = (gm - 1) * tile_m
        for i in range(r0, M):
            for j in rng.integers(0, N, size=4):
                pts.add((i, int(j)))
            pts.add((i, N - 1))
    if N % tile_n:
        c0 = (gn - 1) * tile_n
        for j in range(c0, N):
            for i in rng.integers(0, M, size=4):
                pts.add((int(i), j))
            pts.add((M - 1, j))
    t = 0
    for ti in range(gm):
        for tj in range(gn):
            if t % 8 == 0:
                i0, j0 = ti * tile_m, tj * tile_n
                i1, j1 = min(i0 + tile_m, M) - 1, min(j0 + tile_n, N) - 1
                pts.update({(i0, j0), (i0, j1), (i1, j0), (i1, j1)})
            t += 1
    I = rng.integers(0, M, size=n_random)
    J = rng.integers(0, N, size=n_random)
    pts.update(zip(I.tolist(), J.tolist()))
    arr = np.array(sorted(pts), dtype=np.int64).reshape(-1, 2)
    return arr[:, 0].copy(), arr[:, 1].copy()
