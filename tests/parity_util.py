"""Comparison helpers for the GPU-vs-oracle parity tests.

The acceptance rules (stated once here, used by every parity test):
  * codes: bit-exact, except an index may differ by one cell where the
    oracle's rotated coordinate lies within FLIP_EPS = 1e-5 of a boundary,
    and a sign bit may differ where |S r| < FLIP_EPS; allowed flips must stay
    under 0.01% of the compared coordinates (indices and signs counted
    separately).  A token with an allowed index flip has a legitimately
    different residual: its signs and gamma are judged against the oracle's
    stage 2 re-run on the GPU's cells (oracle.qjl_stage), the same way its
    scores are judged on the GPU's codes;
  * ||k||, ||v||, gamma: 1e-6 relative;
  * scores: |est_gpu - est_oracle| <= 2e-3 ||q|| ||k||;
  * attention output: ||out_gpu - out_oracle|| / ||out_oracle|| <= 5e-3 per
    (slot, query head), against the oracle on the GPU's own codes always, and
    end to end wherever the slot's attended prefix holds no flipped token
    (check_attend_two_level);
  * reconstruction ||x|| R^T c[idx] (tq_get_keys / tq_get_values): every
    element within 1e-5 ||x|| of the oracle's.  The kernel sums d fp32
    products of R and the fp32 centroid times the norm: each carries a
    rounding of 2^-24, so the error is near sqrt(d) 2^-24 ||x|| <= 2e-6 ||x||
    at d = 1024 (the centroids in fp32 add 2^-24 relative).
"""
from __future__ import annotations

import numpy as np

from oracle import turboquant as O

FLIP_EPS = 1e-5
FLIP_FRAC = 1e-4
NORM_RTOL = 1e-6
SCORE_TOL = 2e-3
ATTEND_TOL = 5e-3
DEQ_TOL = 1e-5


def near_boundary(y: np.ndarray, beta: np.ndarray) -> np.ndarray:
    if beta.size == 0:
        return np.zeros(y.shape, dtype=bool)
    return np.min(np.abs(y[..., None] - beta), axis=-1) < FLIP_EPS


def check_codes(gpu_idx, ref_idx, ref_y, beta, what="idx"):
    """Returns (n_allowed_flips, per-token bool mask of flipped tokens)."""
    diff = gpu_idx != ref_idx
    if not diff.any():
        return 0, np.zeros(gpu_idx.shape[:-1], dtype=bool)
    ok = near_boundary(ref_y, beta) & (np.abs(gpu_idx.astype(np.int64) - ref_idx) == 1)
    bad = diff & ~ok
    assert not bad.any(), (f"{what}: {int(bad.sum())} code mismatches away from a boundary, "
                           f"first at {np.argwhere(bad)[:5].tolist()}")
    n = int(diff.sum())
    assert n <= max(1, FLIP_FRAC * diff.size), f"{what}: {n} boundary flips > 0.01% of {diff.size}"
    return n, diff.any(axis=-1)


def check_keys(gpu: dict, ref: dict, beta: np.ndarray, S: np.ndarray, centroids: np.ndarray) -> dict:
    n_idx, tok_flip = check_codes(gpu["idx"], ref["idx"], ref["y"], beta, "key idx")
    z, signs, gamma = ref["z"].copy(), ref["signs"].copy(), ref["gamma"].copy()
    if tok_flip.any():
        alt = O.qjl_stage(ref["y"][tok_flip], gpu["idx"][tok_flip], S, centroids)
        z[tok_flip], signs[tok_flip], gamma[tok_flip] = alt["z"], alt["signs"], alt["gamma"]
    sdiff = gpu["signs"] != signs
    bad = sdiff & ~(np.abs(z) < FLIP_EPS)
    assert not bad.any(), f"sign mismatches away from 0: {int(bad.sum())}, first {np.argwhere(bad)[:5].tolist()}"
    n_sign = int(sdiff.sum())
    assert n_sign <= max(1, FLIP_FRAC * sdiff.size), f"{n_sign} sign flips > 0.01%"
    np.testing.assert_allclose(gpu["norm"], ref["norm"], rtol=NORM_RTOL, atol=1e-30)
    np.testing.assert_allclose(gpu["gamma"], gamma, rtol=NORM_RTOL, atol=1e-7)
    return dict(idx_flips=n_idx, sign_flips=n_sign, flip_tokens=tok_flip | sdiff.any(axis=-1))


def check_values(gpu: dict, ref: dict, beta: np.ndarray) -> dict:
    n_idx, tok_flip = check_codes(gpu["idx"], ref["idx"], ref["y"], beta, "value idx")
    np.testing.assert_allclose(gpu["norm"], ref["norm"], rtol=NORM_RTOL, atol=1e-30)
    return dict(idx_flips=n_idx, flip_tokens=tok_flip)


def check_scores(gpu_scores, ref_scores, qnorm, knorm, tol=SCORE_TOL, skip_tokens=None):
    """qnorm (n_seq, G), knorm (n_seq, T).  skip_tokens (n_seq, T): tokens
    with an allowed code flip, judged instead against the oracle evaluated on
    the GPU's own codes."""
    bound = tol * qnorm[:, :, None] * knorm[:, None, :] + 1e-30
    err = np.abs(gpu_scores - ref_scores)
    if skip_tokens is not None:
        err = np.where(skip_tokens[:, None, :], 0.0, err)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"score error {worst:.3f} x tolerance (max abs {float(err.max()):.3e})"
    return worst


def check_attend(gpu_out, ref_out, tol=ATTEND_TOL):
    num = np.linalg.norm(gpu_out - ref_out, axis=-1)
    den = np.linalg.norm(ref_out, axis=-1) + 1e-30
    rel = num / den
    assert float(rel.max()) <= tol, f"attend rel-L2 {float(rel.max()):.3e} > {tol}"
    return float(rel.max())


def check_attend_two_level(gpu_out, ref_on_gpu_codes, ref_end_to_end, flip_tokens, tol=ATTEND_TOL):
    """Attention output judged at two levels, both to the same tolerance:
      (1) every (slot, query head) against the oracle's attention evaluated
          on the GPU's own codes -- this isolates the attention kernels from
          code flips;
      (2) end to end, against the oracle's attention on its own codes, for
          every slot whose attended prefix holds no token with an allowed
          flip (key index, key sign or value index).  A slot with such a
          token is judged by (1) alone: one allowed flip of a heavily
          weighted value in a short cache moves the output by several 1e-3.
    flip_tokens: (n_seq, n_tokens) bool over the attended prefix.  Returns
    (worst rel-L2 on the GPU's codes, worst end-to-end rel-L2 over the clean
    slots or None, number of slots left out of the end-to-end check)."""
    rel_gpu = check_attend(gpu_out, ref_on_gpu_codes, tol)
    clean = ~np.asarray(flip_tokens, dtype=bool).any(axis=-1)
    rel_e2e = check_attend(gpu_out[clean], ref_end_to_end[clean], tol) if clean.any() else None
    return rel_gpu, rel_e2e, int((~clean).sum())


def unpack_gpu_keys(cache, d, m, bits, n_tok):
    return O.unpack_keys(cache.key_words()[:, :n_tok], d, m, bits)


def unpack_gpu_values(cache, d, bits, n_tok):
    return O.unpack_values(cache.value_words(), d, bits, n_tokens=n_tok)


def check_dequant(gpu_out, ref_out, norms, tol=DEQ_TOL, skip_tokens=None):
    """Max over elements of |x^_gpu - x^_oracle| / ||x|| (rows of zero norm
    must be exactly 0); asserts it is <= tol.  skip_tokens: (n_seq, T) mask
    of tokens left out (index flips when comparing against the oracle's
    own codes)."""
    err = np.abs(gpu_out.astype(np.float64) - ref_out)
    n = norms.astype(np.float64)[..., None]
    zero = (n == 0)[..., 0]
    assert not err[zero].any(), "a zero-norm row did not reconstruct to 0"
    rel = np.where(n > 0, err / np.where(n > 0, n, 1.0), 0.0).max(axis=-1)
    if skip_tokens is not None:
        rel = np.where(skip_tokens, 0.0, rel)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= tol, f"reconstruction error {worst:.3g} ||x|| > {tol}"
    return worst
