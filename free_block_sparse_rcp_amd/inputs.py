"""Seeded synthetic inputs for the SparsePR attention operator.

This module is shared by the HIP path, the oracle's tests and the bench. It
only draws numbers: it holds none of the operator's arithmetic (no responses,
clustering, routing, attention or fitting). Every array it returns is a
function of the seed alone.

The pages evaluate SparsePR on four real video models (skillfed article
"Partition the Support, Reconstruct the Residual", results paragraph); their
weights and activations are not available, so these generators stand in for
them with token grids, head counts, head dims and temperatures of the same
shape (see ``configs.py``).

Generators
----------
G1 (tiny, single head): 3-D sinusoidal position code plus one of 32 Gaussian
    cluster centres, small Gaussian noise on Q and K, V ~ N(0, 1).
G2 (multi-head): 64 smooth spatiotemporal feature channels (Gaussian-blurred
    white noise, standardised) projected per head, plus per-head cluster
    centres and noise; optional neighbourhood smoothing of the keys.

Tokens are ordered ``i = (t * H_g + h) * W_g + w`` on a ``(T_g, H_g, W_g)`` grid.
Half-precision workloads are drawn in fp32 and rounded to bfloat16 with
round-to-nearest-even (through torch); the returned fp32 arrays then hold the
exact bf16 values, which is what both the GPU path and the oracle consume.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
from scipy import ndimage


@dataclass
class Inputs:
    """One call's inputs. Arrays are numpy, ``Q, K, V`` are ``[H, N, d]`` fp32
    holding exactly representable values of ``dtype``."""

    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    scale: np.ndarray            # [H] fp32 softmax temperature tau per head
    sample_idx: np.ndarray       # [S] int32, distinct token indices
    init_idx: np.ndarray         # [G] int32, distinct token indices
    rand_key_perm: np.ndarray    # [N] int32, permutation (random-block variant)
    rand_query_perm: np.ndarray  # [N] int32, permutation (random-block variant)
    dtype: str                   # "f32" or "bf16"
    heads: Sequence[int]         # which heads of the workload these are


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to ``dtype`` (RNE) and return them as fp32."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return t.to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(f"unknown dtype {dtype}")


def grid_coords(grid):
    """Integer (t, h, w) coordinates of each token in token order."""
    tg, hg, wg = grid
    t, h, w = np.meshgrid(np.arange(tg), np.arange(hg), np.arange(wg), indexing="ij")
    return t.reshape(-1), h.reshape(-1), w.reshape(-1)


def sinusoid_code(grid, d: int) -> np.ndarray:
    """3-D sinusoidal position code [N, d] with axis widths (d/4, 3d/8, 3d/8).

    Per axis of width ``wa`` and integer coordinate ``p``: pairs
    (sin p*w_j, cos p*w_j) with w_j = 10000 ** (-2 j / wa), j < wa / 2.
    """
    widths = (d // 4, 3 * d // 8, 3 * d // 8)
    assert sum(widths) == d and all(w % 2 == 0 for w in widths)
    coords = grid_coords(grid)
    parts = []
    for p, wa in zip(coords, widths):
        j = np.arange(wa // 2)
        omega = 10000.0 ** (-2.0 * j / wa)
        ang = p[:, None].astype(np.float64) * omega[None, :]
        pair = np.empty((p.size, wa), dtype=np.float64)
        pair[:, 0::2] = np.sin(ang)
        pair[:, 1::2] = np.cos(ang)
        parts.append(pair)
    return np.concatenate(parts, axis=1)


def random_block_perms(seed: int, n: int):
    """Seeded key and query permutations for the random-block variant."""
    rng = np.random.default_rng(np.random.SeedSequence(seed + 100))
    return (rng.permutation(n).astype(np.int32), rng.permutation(n).astype(np.int32))


def gen_g1(grid, d: int, n_samples: int, n_groups: int, seed: int, scale: float,
           dtype: str = "f32") -> Inputs:
    """G1: single head. Draw order: centres, labels, eps_Q, eps_K, V, sample, init."""
    n = int(np.prod(grid))
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal((32, d))
    lab = rng.integers(0, 32, n)
    eps_q = rng.standard_normal((n, d))
    eps_k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    sample_idx = rng.choice(n, n_samples, replace=False).astype(np.int32)
    init_idx = rng.choice(n, n_groups, replace=False).astype(np.int32)
    phi = sinusoid_code(grid, d)
    q = phi + mu[lab] + 0.5 * eps_q
    k = phi + mu[lab] + 0.5 * eps_k
    kp, qp = random_block_perms(seed, n)
    return Inputs(
        Q=round_to_dtype(q[None], dtype), K=round_to_dtype(k[None], dtype),
        V=round_to_dtype(v[None], dtype),
        scale=np.array([scale], dtype=np.float32), sample_idx=sample_idx,
        init_idx=init_idx, rand_key_perm=kp, rand_query_perm=qp, dtype=dtype, heads=[0])


def _smooth_features(rng, grid, blur, channels: int = 64) -> np.ndarray:
    f = rng.standard_normal(tuple(grid) + (channels,))
    for axis, s in enumerate(blur):
        f = ndimage.gaussian_filter1d(f, sigma=s, axis=axis, mode="reflect", truncate=3.0)
    f = f.reshape(-1, channels)
    f = (f - f.mean(axis=0)) / f.std(axis=0)
    return f


def gen_g2(grid, d: int, n_heads: int, n_samples: int, n_groups: int, seed: int,
           scales: Sequence[float], blur, key_smoothing: bool = False,
           dtype: str = "bf16", heads: Optional[Sequence[int]] = None) -> Inputs:
    """G2: multi-head smooth features + clustered noise.

    ``SeedSequence(seed)`` spawns ``n_heads + 1`` streams; stream ``n_heads`` is
    shared (features, cluster labels, sample and init indices), stream ``h``
    belongs to head ``h``. ``heads`` selects a subset without changing any
    head's values.
    """
    n = int(np.prod(grid))
    heads = list(range(n_heads)) if heads is None else list(heads)
    streams = np.random.SeedSequence(seed).spawn(n_heads + 1)
    shared = np.random.default_rng(streams[n_heads])
    feats = _smooth_features(shared, grid, blur)
    lab = shared.integers(0, 64, n)
    sample_idx = shared.choice(n, n_samples, replace=False).astype(np.int32)
    init_idx = shared.choice(n, n_groups, replace=False).astype(np.int32)
    Q = np.empty((len(heads), n, d), dtype=np.float32)
    K = np.empty_like(Q)
    V = np.empty_like(Q)

    def one_head(i, h):
        rng = np.random.default_rng(streams[h])
        a = rng.standard_normal((64, d)) / 8.0
        a2 = a + 0.25 * rng.standard_normal((64, d)) / 8.0
        mu = rng.standard_normal((64, d))
        eps_q = rng.standard_normal((n, d))
        eps_k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, d))
        q = (feats @ a + mu[lab] + 0.5 * eps_q) / 1.5
        k = (feats @ a2 + mu[lab] + 0.5 * eps_k) / 1.5
        if key_smoothing:
            kg = k.reshape(tuple(grid) + (d,))
            box = ndimage.uniform_filter(kg, size=(3, 3, 3, 1), mode="reflect")
            k = ((kg + box) / 2.0).reshape(n, d)
            k = k / k.std(axis=0)
        Q[i] = round_to_dtype(q, dtype)
        K[i] = round_to_dtype(k, dtype)
        V[i] = round_to_dtype(v, dtype)

    # heads draw from independent streams, so they can be generated concurrently
    workers = max(1, min(len(heads), 8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda ih: one_head(*ih), enumerate(heads)))
    kp, qp = random_block_perms(seed, n)
    sc = np.asarray([scales[h] for h in heads], dtype=np.float32)
    return Inputs(Q=Q, K=K, V=V, scale=sc, sample_idx=sample_idx, init_idx=init_idx,
                  rand_key_perm=kp, rand_query_perm=qp, dtype=dtype, heads=heads)
