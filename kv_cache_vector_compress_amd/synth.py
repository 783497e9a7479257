"""Seeded synthetic inputs for the TurboQuant KV-cache hot path.

This module draws random numbers and nothing else: it holds none of the
compression method's arithmetic (no codebook, no bucketing, no projection,
no score).  Both the HIP path and the fp64 oracle take its outputs as plain
input arrays, so the two sides never share a computation.

What it produces, and the passages each recipe follows:

* ``haar_rotation(d, seed)`` -- the random orthogonal matrix R.  The pages
  (atskills.one "turboquant-pytorch", *Why Random Rotation?*; nav.superapi.store
  "turboquant-pytorch", 算法细节 / 随机旋转) only ask for a random orthogonal
  matrix that needs no data; the recipe here is the textbook Haar draw: QR of a
  seeded standard-normal d x d matrix, with the signs of R's diagonal fixed so
  the draw is Haar distributed.  R is fixed per (d, seed).
* ``gaussian_projection(m, d, seed)`` -- the QJL matrix S, i.i.d. N(0, 1),
  fixed per (m, d, seed).  The QJL sign projection is named on the same pages
  (第二阶段 / Stage 2); its matrix is a standard Gaussian sketch.
* KV-like tensors: Gaussian vectors with a few outlier channels scaled x8 and
  per-token norms drawn from LogNormal(0, 0.3), rounded to fp16 -- the stand-in
  for the Qwen2.5-3B KV activations the pages validate on (nav.superapi.store
  "turboquant-pytorch", 比特宽度选择指南), which are not available here.
* Unit-norm Gaussian rows (fp32) for the tiny parity case, and the
  Gaussian-plus-cluster-mixture database for the vector-search workload
  (ai-manual.ru article, *Где TurboQuant выстреливает*; jansverre.net post,
  *Hvem er dette nyttig for?*).

Every tensor is generated per "slot" (one KV head of one layer / batch item)
from ``numpy.random.SeedSequence([seed, slot])``, so any slice of a large
workload can be regenerated on its own, bit for bit, without generating the
rest.
"""
from __future__ import annotations

import dataclasses
from typing import Sequence

import numpy as np

# Seeds used by the standard workloads.  Data seeds: K, V, Q; matrix seeds.
SEED_K = 0
SEED_V = 1
SEED_Q = 2
SEED_R = 42
SEED_S = 43
SEED_OUTLIER = 7


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def haar_rotation(d: int, seed: int = SEED_R) -> np.ndarray:
    """Haar-random orthogonal d x d matrix (float64, row-major)."""
    g = np.random.Generator(np.random.PCG64(seed)).standard_normal((d, d))
    q, u = np.linalg.qr(g)
    q = q * np.sign(np.diag(u))[None, :]
    return np.ascontiguousarray(q)


def gaussian_projection(m: int, d: int, seed: int = SEED_S) -> np.ndarray:
    """i.i.d. N(0, 1) matrix of shape (m, d), float64."""
    return np.random.Generator(np.random.PCG64(seed)).standard_normal((m, d))


def unit_gaussian(n: int, d: int, seed: int, dtype=np.float32) -> np.ndarray:
    """n rows of i.i.d. N(0, 1) entries, each row scaled to unit L2 norm."""
    x = np.random.Generator(np.random.PCG64(seed)).standard_normal((n, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    return x.astype(dtype)


def outlier_channels(head: int, d: int, frac: float = 0.04, seed: int = SEED_OUTLIER) -> np.ndarray:
    """The fixed set of outlier channels of one KV head (about frac * d of them)."""
    n_out = max(1, int(round(frac * d)))
    return np.sort(_rng(seed, head).choice(d, size=n_out, replace=False))


def kv_slot(seed: int, slot: int, head: int, n_tok: int, d: int,
            outlier_scale: float = 8.0, lognorm_sigma: float = 0.3,
            dtype=np.float16) -> np.ndarray:
    """One slot's (n_tok, d) KV-like vectors.

    Each vector is normalise(g * w) * rho with g ~ N(0, I), w = outlier_scale
    on the head's outlier channels and 1 elsewhere, rho ~ LogNormal(0, sigma).
    """
    rng = _rng(seed, slot)
    g = rng.standard_normal((n_tok, d), dtype=np.float32)
    w = np.ones(d, dtype=np.float32)
    w[outlier_channels(head, d)] = outlier_scale
    g *= w[None, :]
    g /= np.linalg.norm(g, axis=1, keepdims=True)
    rho = rng.lognormal(0.0, lognorm_sigma, size=(n_tok, 1)).astype(np.float32)
    return (g * rho).astype(dtype)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one standard workload."""
    name: str
    n_seq: int           # number of KV slots (layers x KV heads x batch)
    n_tok: int           # tokens per slot
    d: int               # head_dim
    m: int               # QJL proj_dim
    key_bits: int
    value_bits: int
    G: int               # query heads per KV head
    dtype: str           # "f16" or "f32"
    heads_per_slot_cycle: int  # slot -> head mapping period (outlier set per head)

    def head_of_slot(self, slot: int) -> int:
        return slot % self.heads_per_slot_cycle


# Standard workload shapes (the per-slot recipes are in kv_slot and unit_gaussian).
TINY = Workload("tiny_d128_b3_T1024", 1, 1024, 128, 64, 3, 3, 4, "f32", 1)
QWEN_DECODE = Workload("qwen2.5-3b_decode_36x2x8192", 72, 8192, 128, 64, 3, 3, 8, "f16", 72)
LONG_CONTEXT = Workload("long_context_8x8x131072", 64, 131072, 128, 64, 3, 3, 4, "f16", 8)


def workload_keys(w: Workload, slots: Sequence[int] | None = None, n_tok: int | None = None) -> np.ndarray:
    """Keys of the given slots, shape (len(slots), n_tok, d)."""
    return _kv(w, SEED_K, slots, n_tok)


def workload_values(w: Workload, slots: Sequence[int] | None = None, n_tok: int | None = None) -> np.ndarray:
    return _kv(w, SEED_V, slots, n_tok)


def _kv(w: Workload, seed: int, slots, n_tok) -> np.ndarray:
    slots = range(w.n_seq) if slots is None else slots
    n_tok = w.n_tok if n_tok is None else n_tok
    if w.dtype == "f32":
        # tiny case: unit-norm i.i.d. Gaussian rows in fp32
        return np.stack([unit_gaussian(n_tok, w.d, seed=seed * 1000003 + s) for s in slots])
    return np.stack([kv_slot(seed, s, w.head_of_slot(s), n_tok, w.d) for s in slots])


def workload_queries(w: Workload, slots: Sequence[int] | None = None) -> np.ndarray:
    """Queries (len(slots), G, d): same recipe as the keys, one row per query head."""
    slots = range(w.n_seq) if slots is None else slots
    if w.dtype == "f32":
        return np.stack([unit_gaussian(w.G, w.d, seed=SEED_Q * 1000003 + s) for s in slots])
    return np.stack([kv_slot(SEED_Q, s, w.head_of_slot(s), w.G, w.d) for s in slots])


def vector_database(n: int, d: int, seed: int, n_clusters: int = 64, spread: float = 0.3,
                    start: int = 0) -> np.ndarray:
    """Rows [start, start+n) of a unit-norm fp32 database: even rows isotropic
    Gaussian, odd rows from a mixture normalise(mu_c + spread * g / sqrt(d))."""
    centres = _rng(seed, 1 << 30).standard_normal((n_clusters, d))
    centres /= np.linalg.norm(centres, axis=1, keepdims=True)
    out = np.empty((n, d), dtype=np.float32)
    block = 4096
    for b0 in range((start // block) * block, start + n, block):
        rng = _rng(seed, b0 // block)
        g = rng.standard_normal((block, d))
        cl = rng.integers(0, n_clusters, size=block)
        rows = np.arange(b0, b0 + block)
        mix = centres[cl] + spread * g / np.sqrt(d)
        x = np.where((rows % 2 == 1)[:, None], mix, g)
        x /= np.linalg.norm(x, axis=1, keepdims=True)
        lo, hi = max(b0, start), min(b0 + block, start + n)
        if lo < hi:
            out[lo - start:hi - start] = x[lo - b0:hi - b0]
    return out


def vector_search_device(torch, n: int, d: int, n_queries: int, dev, seed: int = 4, n_clusters: int = 64,
                         spread: float = 0.3):
    """The vector-search workload generated on the device with a seeded torch
    generator (the host generator above would take minutes at 2M rows):
    database (1, n, d) fp32, unit-norm rows, odd rows from the mixture
    normalise(mu_c + spread g / sqrt(d)), even rows isotropic Gaussian; and
    (1, n_queries, d) unit-norm Gaussian queries."""
    g = torch.Generator(device=dev).manual_seed(seed)
    cent = torch.randn((n_clusters, d), device=dev, generator=g)
    cent /= cent.norm(dim=1, keepdim=True)
    X = torch.randn((1, n, d), device=dev, generator=g)
    odd = torch.arange(n, device=dev) % 2 == 1
    cl = torch.randint(0, n_clusters, (n,), device=dev, generator=g)
    X[0, odd] = cent[cl[odd]] + spread * X[0, odd] / d ** 0.5
    X /= X.norm(dim=-1, keepdim=True)
    Q = torch.randn((1, n_queries, d), device=dev, generator=g)
    Q /= Q.norm(dim=-1, keepdim=True)
    return X, Q
