"""fp64 CPU oracle of TurboQuant's KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package.  The
product path (the HIP library and its Python binding) never imports it and
shares no code with it: not a kernel, a helper, a table or a constant
generator.  Inputs come from the seeded generators, and R and S are passed in
as plain arrays.

Sources, cited by page and section throughout this file:
  [affpapa]   affpapa.org, "turboquant-pytorch -- скилл для Claude Code"
  [atskills]  atskills.one, "turboquant-pytorch" (aradotso agent skill),
              section "What this skill does" (Stage 1 / Stage 2, Core API,
              Algorithm Details: Why Random Rotation?, Why QJL for Keys but
              Not Values?)
  [superapi]  nav.superapi.store, "turboquant-pytorch": 主要能力, 核心 API,
              常见使用模式, 算法细节, 比特宽度选择指南, 限制与注意事项
  [aimanual]  ai-manual.ru, TurboQuant article (online quantisation without
              calibration; its per-vector Cholesky rotation is NOT what is
              built here: every other page uses one fixed random rotation)
  [jansverre] jansverre.net, "TurboQuant er nå tilgjengelig som
              Python-bibliotek": Hva er TurboQuant, kort fortalt?; Hva gjør
              Python-implementasjonen?; Kjente begrensninger

Notation: d = head_dim, b = bits, L = 2**b levels, m = proj_dim,
c[0..L-1] ascending centroids, beta[0..L-2] ascending boundaries,
R (d x d) the rotation, S (m x d) the QJL matrix.

Readings taken where the pages are silent:
  * rotation is y = R x with R row-major;
  * the QJL matrix acts on the rotated residual r = R x - c[idx];
  * idx_j = #{i : beta_i < y_j}, so a value equal to a boundary goes to the
    lower cell; sign bit s_i = 1 iff (S r)_i >= 0;
  * norms ||k|| and gamma = ||r|| are kept in fp32;
  * scores are unscaled <q, k> estimates; attention applies scale (1/sqrt(d)
    by default) before the softmax;
  * a zero vector has x = 0 (it is still encoded, and contributes nothing);
  * keys at 0 bits (the (b-1) + QJL bit budget at b = 1) use the single cell
    0: no code words, r = y, and the score is the plain QJL estimate.

Parity pins for every function are in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from functools import lru_cache

import numpy as np
from scipy import integrate

SQRT_HALF_PI = math.sqrt(math.pi / 2.0)


# ---------------------------------------------------------------------------
# Lloyd-Max codebook
# ---------------------------------------------------------------------------

def _phi(x: float) -> float:
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi) if math.isfinite(x) else 0.0


def _cell_mass_and_moment(a: float, b: float) -> tuple[float, float]:
    """P = int_a^b phi, M = int_a^b x phi, by numerical integration (quad)."""
    kw = dict(epsabs=0.0, epsrel=2e-14, limit=200)
    p = integrate.quad(_phi, a, b, **kw)[0]
    mo = integrate.quad(lambda x: x * _phi(x), a, b, **kw)[0]
    return p, mo


def _lloyd_step(c: np.ndarray):
    """One Lloyd-Max update for N(0, 1): boundaries at centroid midpoints,
    centroids at the conditional means of their cells.  Returns the new
    centroids and the Jacobian d(new)/d(old) used to accelerate the iteration
    (the Jacobian changes only the speed, not the fixed point)."""
    L = len(c)
    beta = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate([[-np.inf], beta, [np.inf]])
    new = np.empty(L)
    dmu_da = np.zeros(L)
    dmu_db = np.zeros(L)
    for i in range(L):
        a, b = edges[i], edges[i + 1]
        p, mo = _cell_mass_and_moment(a, b)
        mu = mo / p
        new[i] = mu
        if np.isfinite(a):
            dmu_da[i] = _phi(a) * (mu - a) / p
        if np.isfinite(b):
            dmu_db[i] = _phi(b) * (b - mu) / p
    jac = np.zeros((L, L))
    for i in range(L):
        if i > 0:          # a_i = (c_{i-1} + c_i) / 2
            jac[i, i - 1] += 0.5 * dmu_da[i]
            jac[i, i] += 0.5 * dmu_da[i]
        if i < L - 1:      # b_i = (c_i + c_{i+1}) / 2
            jac[i, i] += 0.5 * dmu_db[i]
            jac[i, i + 1] += 0.5 * dmu_db[i]
    return new, jac


@lru_cache(maxsize=None)
def _lloyd_max_standard(bits: int) -> tuple[tuple[float, ...], tuple[float, ...]]:
    """Lloyd-Max quantiser of N(0, 1) with 2**bits levels, by numerical
    integration ([superapi] 核心 API: build_lloyd_max_codebook(dim, bits)
    returns (boundaries, centroids); 限制与注意事项: built by numerical
    integration, cached per (dim, bits)).

    Start: cell means of 2**bits equal-probability cells.  Then plain Lloyd
    iterations, polished by Newton steps on c = T(c) until the update is
    below 1e-15.  The result is made exactly symmetric."""
    from scipy.stats import norm
    L = 1 << bits
    edges = norm.ppf(np.linspace(0.0, 1.0, L + 1))
    c = np.array([_cell_mass_and_moment(edges[i], edges[i + 1])[1] /
                  _cell_mass_and_moment(edges[i], edges[i + 1])[0] for i in range(L)])
    for _ in range(20):
        c, _j = _lloyd_step(c)
    for _ in range(60):
        t, jac = _lloyd_step(c)
        step = np.linalg.solve(jac - np.eye(L), -(t - c))
        c = c + step
        if np.max(np.abs(step)) < 1e-15:
            break
    c = 0.5 * (c - c[::-1])           # c_i = -c_{L-1-i} exactly
    beta = 0.5 * (c[:-1] + c[1:])
    if L % 2 == 0:
        beta[L // 2 - 1] = 0.0
    return tuple(beta.tolist()), tuple(c.tolist())


def lloyd_max_codebook(dim: int, bits: int) -> tuple[np.ndarray, np.ndarray]:
    """(boundaries, centroids) for coordinates ~ N(0, 1/dim), fp64 ascending.

    The rotated coordinates of a unit vector are modelled as N(0, 1/d)
    ([atskills] Why Random Rotation?; [superapi] 算法细节 / 随机旋转), so the
    codebook is the standard-normal one scaled by 1/sqrt(d)."""
    if not (0 <= bits <= 8):
        raise ValueError("bits must be in 0..8")
    if bits == 0:
        # One cell covering the whole line: no boundary, and the Lloyd-Max
        # centroid of that cell is the mean of N(0, 1/d), 0.  Keys at 0 bits
        # are then pure QJL signs of the rotated direction ([atskills] Stage 2
        # applied to r = y).
        return np.zeros(0), np.zeros(1)
    beta, c = _lloyd_max_standard(bits)
    s = 1.0 / math.sqrt(dim)
    return np.asarray(beta) * s, np.asarray(c) * s


# ---------------------------------------------------------------------------
# Stage 1 (rotation + Lloyd-Max bucketing) and stage 2 (QJL)
# ---------------------------------------------------------------------------

def _as64(x) -> np.ndarray:
    x = np.asarray(x)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    return x.astype(np.float64)


def normalise(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Split rows into norm and direction ([superapi] 限制与注意事项: the
    inner-product quantiser expects unit vectors; the compressors normalise
    internally).  A zero row has direction 0."""
    n = np.linalg.norm(x, axis=-1)
    safe = np.where(n > 0, n, 1.0)
    return n, x / safe[..., None] * (n > 0)[..., None]


def rotate(x: np.ndarray, R: np.ndarray) -> np.ndarray:
    """y = R x for every row x ([superapi] 主要能力, stage 1: random orthogonal
    rotation)."""
    return x @ R.T


def bucketize(y: np.ndarray, boundaries: np.ndarray) -> np.ndarray:
    """idx = #{i : beta_i < y}: the Lloyd-Max cell of each coordinate
    ([superapi] 主要能力: Lloyd-Max scalar quantisation of each coordinate)."""
    return np.searchsorted(boundaries, y, side="left").astype(np.int64)


def compress_keys(K, R, S, boundaries, centroids) -> dict:
    """Both stages for keys ([atskills] Stage 1 + Stage 2; [superapi] 核心 API
    TurboQuantProd.compress and TurboQuantCompressorV2; 算法细节: keys take
    QJL because bias in <q, k> corrupts the attention weights).

    K: (..., T, d) array of any float type.  Returns idx (..., T, d) int,
    signs (..., T, m) uint8, norm and gamma (..., T) fp32, and the fp64 y, z
    used to judge near-boundary flips."""
    K = _as64(K)
    n, x = normalise(K)
    y = rotate(x, R)
    idx = bucketize(y, boundaries)
    q = qjl_stage(y, idx, S, centroids)
    return dict(idx=idx, signs=q["signs"], norm=n.astype(np.float32), gamma=q["gamma"], y=y, z=q["z"])


def qjl_stage(y, idx, S, centroids) -> dict:
    """Stage 2 of the key compressor on given cells ([atskills] Stage 2;
    [superapi] 主要能力): residual r = y - c[idx], gamma = ||r||, projection
    z = S r and its sign bits [z >= 0].  Used by compress_keys, and to
    re-evaluate a token whose cell index legitimately differs (a coordinate
    within floating-point error of a boundary) on those other cells."""
    r = _as64(y) - np.asarray(centroids, dtype=np.float64)[idx]
    z = r @ _as64(S).T
    return dict(z=z, signs=(z >= 0).astype(np.uint8), gamma=np.linalg.norm(r, axis=-1).astype(np.float32))


def compress_values(V, R, boundaries, centroids) -> dict:
    """Stage 1 only for values ([atskills] Why QJL for Keys but Not Values?;
    [superapi] 核心 API TurboQuantCompressorMSE)."""
    V = _as64(V)
    n, x = normalise(V)
    y = rotate(x, R)
    idx = bucketize(y, boundaries)
    return dict(idx=idx, norm=n.astype(np.float32), y=y)


def prepare_queries(Q, R, S) -> tuple[np.ndarray, np.ndarray]:
    """q~ = R q and p = S q~ for every query head."""
    Q = _as64(Q)
    qt = rotate(Q, R)
    return qt, qt @ S.T


def key_scores(Q, R, S, centroids, keys: dict) -> np.ndarray:
    """Asymmetric score estimates <q, k> from compressed keys, unscaled
    ([superapi] 常见使用模式: asymmetric_attention_scores computes attention
    scores straight from compressed keys; [atskills] Stage 2 makes the
    inner-product estimate unbiased):

        est = ||k|| * ( <q~, c[idx]> + gamma * sqrt(pi/2) / m * <p, 2 s - 1> )

    Q: (n_seq, G, d); keys from compress_keys over (n_seq, T, d).
    Returns (n_seq, G, T) fp64."""
    qt, p = prepare_queries(Q, R, S)
    m = S.shape[0]
    khat = centroids[keys["idx"]]                              # (n_seq, T, d)
    sgn = 2.0 * keys["signs"].astype(np.float64) - 1.0          # (n_seq, T, m)
    mse = np.einsum("sgd,std->sgt", qt, khat)
    qjl = np.einsum("sgm,stm->sgt", p, sgn)
    n = keys["norm"].astype(np.float64)[:, None, :]
    g = keys["gamma"].astype(np.float64)[:, None, :]
    return n * (mse + g * (SQRT_HALF_PI / m) * qjl)


def dequantize_values(R, centroids, values: dict) -> np.ndarray:
    """v^ = ||v|| R^T c[idx] ([superapi] 核心 API TurboQuantMSE.dequantize;
    常见使用模式: weighted sum over the decompressed values)."""
    rot = centroids[values["idx"]] * values["norm"].astype(np.float64)[..., None]
    return rot @ R


def attend(Q, R, S, centroids, keys: dict, values: dict, scale: float | None = None,
           n_tokens: int | None = None, value_centroids=None) -> np.ndarray:
    """softmax(scale * est) . V^ over the compressed cache ([superapi]
    常见使用模式: scores from the compressed keys, softmax, then the weighted
    sum of the decompressed values).  The weighted sum is taken in the rotated
    domain and rotated back once: out = R^T sum_t a_t ||v_t|| c[idx_t].
    No causal mask: a decode query sees the whole cache.

    ``centroids`` is the key codebook; ``value_centroids`` the value
    codebook (defaults to the key codebook: same bit width).

    Returns (n_seq, G, d) fp64."""
    d = R.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    vc = centroids if value_centroids is None else value_centroids
    est = key_scores(Q, R, S, centroids, keys)
    T = est.shape[-1] if n_tokens is None else n_tokens
    logits = scale * est[..., :T]
    logits -= logits.max(axis=-1, keepdims=True)
    a = np.exp(logits)
    a /= a.sum(axis=-1, keepdims=True)
    vrot = vc[values["idx"][:, :T]] * values["norm"][:, :T].astype(np.float64)[..., None]
    acc = np.einsum("sgt,std->sgd", a, vrot)
    return acc @ R


def attend_online(Q, R, S, centroids, keys: dict, values: dict, scale: float | None = None,
                  chunk: int = 64, value_centroids=None) -> np.ndarray:
    """The same attention as ``attend`` computed chunk by chunk with a running
    (max, sum, acc) per query head and a final log-sum-exp merge -- the
    streaming form a split-token decode uses.  Equal to ``attend`` up to
    rounding."""
    d = R.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    vc = centroids if value_centroids is None else value_centroids
    est = scale * key_scores(Q, R, S, centroids, keys)
    n_seq, G, T = est.shape
    vrot = vc[values["idx"]] * values["norm"].astype(np.float64)[..., None]
    mx = np.full((n_seq, G), -np.inf)
    sm = np.zeros((n_seq, G))
    acc = np.zeros((n_seq, G, d))
    for t0 in range(0, T, chunk):
        e = est[..., t0:t0 + chunk]
        m_new = np.maximum(mx, e.max(axis=-1))
        alpha = np.exp(mx - m_new)
        p = np.exp(e - m_new[..., None])
        sm = sm * alpha + p.sum(axis=-1)
        acc = acc * alpha[..., None] + np.einsum("sgt,std->sgd", p, vrot[:, t0:t0 + chunk])
        mx = m_new
    return (acc / sm[..., None]) @ R


# ---------------------------------------------------------------------------
# Record layout (packing).  The layout is this build's own: the pages give no
# storage format.  Tokens are encoded as little-endian 32-bit words.
# ---------------------------------------------------------------------------
#
# Coordinate groups.  A "quad" is 4 consecutive coordinates 16 t + 4 q + i
# (i = 0..3) for tile t = 0..d/16-1 and lane group q = 0..3.  Lane group q's
# quads are taken 8 at a time ("octets", g = t // 8, slot s = t % 8); the b
# code words of (q, g) hold the codes of its 8 quads as follows, byte lane i
# of every word belonging to coordinate 16 t + 4 q + i:
#   b = 1: word 0 bit s;   b = 2: word s//4, bits 2(s%4)..+1;
#   b = 4: word s//2, bits 4(s%2)..+3;
#   b = 3: s in {0,1}: word 0 bits 3s..+2;  s in {2,3}: word 1 bits 3(s-2)..+2;
#          s in {4,5}: word 2 bits 3(s-4)..+2;
#          s = 6: bits 0,1 in word 0 bits 6,7 and bit 2 in word 2 bit 6;
#          s = 7: bits 0,1 in word 1 bits 6,7 and bit 2 in word 2 bit 7
#   (bit positions are within byte lane i, i.e. add 8 i).
#
# Key record (one per token), words, with n = d // 128 full octet columns
# and n' = m // 64 full sign pairs:
#   [codes: for q in 0..3, for g in 0..n-1, b words of (q, g)]
#   [if d % 128 == 64, the half column g = n (tiles t = 8 n .. 8 n + 3):
#    b words for p = 0, then b words for p = 1; group p holds lane group p
#    at slots 0..3 and lane group p + 2 at slots 4..7, slot s <-> tile
#    8 n + s % 4 of lane group p + 2 (s // 4)]
#   [signs: proj coordinate 16 t + 4 q + i with t < 4 n' sits in word
#           2 (t // 4) + q // 2 at bit 16 (q % 2) + 4 (t % 4) + i; if
#           m % 64 == 32, projection 64 n' + j (j < 32) sits in word 2 n'
#           at bit j]
#   [fp32 ||k||] [fp32 gamma]
#
# Value block (128 tokens of one slot), words:
#   [codes: for w in 0..b-1, for q in 0..3, for coordinate c in 0..d-1: one
#    word; token tau of the block (tile s = tau // 16, lane group
#    q = (tau % 16) // 4, byte lane i = tau % 4) has its code of coordinate c
#    in the b words (w = 0..b-1) of (q, c) at slot s, byte lane i]
#   [128 fp32 norms ||v||, token order]

def _slot_fields(bits: int):
    """For slot s: list of (word, bit offset within byte, width, code bit)."""
    f = {}
    for s in range(8):
        if bits == 1:
            f[s] = [(0, s, 1, 0)]
        elif bits == 2:
            f[s] = [(s // 4, 2 * (s % 4), 2, 0)]
        elif bits == 4:
            f[s] = [(s // 2, 4 * (s % 2), 4, 0)]
        elif bits == 3:
            if s < 6:
                f[s] = [(s // 2, 3 * (s % 2), 3, 0)]
            elif s == 6:
                f[s] = [(0, 6, 2, 0), (2, 6, 1, 2)]
            else:
                f[s] = [(1, 6, 2, 0), (2, 7, 1, 2)]
        else:
            raise ValueError("bits must be 1..4")
    return f


def _put_codes(words: np.ndarray, codes: np.ndarray, bits: int) -> None:
    """words: (..., b) uint32 for one (q, group); codes: (..., 8, 4) ints
    (slot s, byte lane i).  ORs the codes in."""
    fields = _slot_fields(bits)
    for s in range(8):
        for (w, off, width, cbit) in fields[s]:
            part = (codes[..., s, :] >> cbit) & ((1 << width) - 1)
            for i in range(4):
                words[..., w] |= (part[..., i].astype(np.uint32) << np.uint32(8 * i + off))


def _get_codes(words: np.ndarray, bits: int) -> np.ndarray:
    fields = _slot_fields(bits)
    out = np.zeros(words.shape[:-1] + (8, 4), dtype=np.int64)
    for s in range(8):
        for (w, off, width, cbit) in fields[s]:
            for i in range(4):
                part = (words[..., w].astype(np.int64) >> (8 * i + off)) & ((1 << width) - 1)
                out[..., s, i] |= part << cbit
    return out


def key_record_words(d: int, m: int, bits: int) -> int:
    return bits * d // 32 + m // 32 + 2


def value_block_words(d: int, bits: int) -> int:
    return 4 * bits * d + 128


def pack_keys(idx, signs, norm, gamma, bits: int) -> np.ndarray:
    """Encode compressed keys (..., T, d) into records (..., T, words) uint32
    (d a multiple of 64, m a multiple of 32)."""
    idx = np.asarray(idx)
    lead, d = idx.shape[:-1], idx.shape[-1]
    m = signs.shape[-1]
    if d % 64 or m % 32:
        raise ValueError("head_dim must be a multiple of 64 and proj_dim of 32")
    n_full, half = d // 128, d % 128 == 64
    rec = np.zeros(lead + (key_record_words(d, m, bits),), dtype=np.uint32)
    if bits == 0 and np.any(idx != 0):
        raise ValueError("0-bit keys have the single cell 0")
    if bits:
        # coordinate 16 t + 4 q + i  ->  (q, g = t // 8, s = t % 8, i)
        cq = idx[..., :128 * n_full].reshape(lead + (n_full, 8, 4, 4))          # (..., g, s, q, i)
        for q in range(4):
            for g in range(n_full):
                words = np.zeros(lead + (bits,), dtype=np.uint32)
                _put_codes(words, cq[..., g, :, q, :], bits)
                base = (q * n_full + g) * bits
                rec[..., base:base + bits] = words
        if half:
            hq = idx[..., 128 * n_full:].reshape(lead + (4, 4, 4))             # (..., t, q, i)
            for p in range(2):
                slots = np.concatenate([hq[..., :, p, :], hq[..., :, p + 2, :]], axis=-2)  # (..., 8, 4)
                words = np.zeros(lead + (bits,), dtype=np.uint32)
                _put_codes(words, slots, bits)
                base = (4 * n_full + p) * bits
                rec[..., base:base + bits] = words
    sw0 = bits * d // 32
    nf = m // 64
    sg = np.asarray(signs).astype(np.uint32)
    sgf = sg[..., :64 * nf].reshape(lead + (4 * nf, 4, 4))                      # (..., t, q, i)
    for t in range(4 * nf):
        for q in range(4):
            for i in range(4):
                w = sw0 + 2 * (t // 4) + q // 2
                rec[..., w] |= sgf[..., t, q, i] << np.uint32(16 * (q % 2) + 4 * (t % 4) + i)
    for j in range(m - 64 * nf):
        rec[..., sw0 + 2 * nf] |= sg[..., 64 * nf + j] << np.uint32(j)
    rec[..., -2] = np.asarray(norm, dtype=np.float32).view(np.uint32)
    rec[..., -1] = np.asarray(gamma, dtype=np.float32).view(np.uint32)
    return rec


def unpack_keys(rec, d: int, m: int, bits: int) -> dict:
    rec = np.asarray(rec, dtype=np.uint32)
    lead = rec.shape[:-1]
    n_full, half = d // 128, d % 128 == 64
    idx = np.zeros(lead + (d,), dtype=np.int64)
    if bits:   # 0-bit records carry no codes
        full = np.zeros(lead + (n_full, 8, 4, 4), dtype=np.int64)
        for q in range(4):
            for g in range(n_full):
                base = (q * n_full + g) * bits
                full[..., g, :, q, :] = _get_codes(rec[..., base:base + bits], bits)
        idx[..., :128 * n_full] = full.reshape(lead + (128 * n_full,))
        if half:
            hq = np.zeros(lead + (4, 4, 4), dtype=np.int64)                       # (..., t, q, i)
            for p in range(2):
                base = (4 * n_full + p) * bits
                slots = _get_codes(rec[..., base:base + bits], bits)               # (..., 8, 4)
                hq[..., :, p, :] = slots[..., :4, :]
                hq[..., :, p + 2, :] = slots[..., 4:, :]
            idx[..., 128 * n_full:] = hq.reshape(lead + (64,))
    sw0 = bits * d // 32
    nf = m // 64
    signs = np.zeros(lead + (m,), dtype=np.uint8)
    sgf = np.zeros(lead + (4 * nf, 4, 4), dtype=np.uint8)
    for t in range(4 * nf):
        for q in range(4):
            for i in range(4):
                w = sw0 + 2 * (t // 4) + q // 2
                sgf[..., t, q, i] = (rec[..., w] >> np.uint32(16 * (q % 2) + 4 * (t % 4) + i)) & 1
    signs[..., :64 * nf] = sgf.reshape(lead + (64 * nf,))
    for j in range(m - 64 * nf):
        signs[..., 64 * nf + j] = (rec[..., sw0 + 2 * nf] >> np.uint32(j)) & 1
    return dict(idx=idx, signs=signs,
                norm=rec[..., -2].view(np.float32), gamma=rec[..., -1].view(np.float32))


def pack_values(idx, norm, bits: int, capacity: int | None = None) -> np.ndarray:
    """Encode compressed values (n_seq, T, d) into 128-token blocks
    (n_seq, ceil(T/128), block words) uint32.  Slots past T stay zero."""
    idx = np.asarray(idx)
    n_seq, T, d = idx.shape
    cap = capacity if capacity is not None else -(-T // 128) * 128
    nb = cap // 128
    full = np.zeros((n_seq, cap, d), dtype=np.int64)
    full[:, :T] = idx
    nrm = np.zeros((n_seq, cap), dtype=np.float32)
    nrm[:, :T] = norm
    blocks = np.zeros((n_seq, nb, value_block_words(d, bits)), dtype=np.uint32)
    # token tau -> (s = tau // 16, q = (tau % 16) // 4, i = tau % 4)
    tq = full.reshape(n_seq, nb, 8, 4, 4, d)              # (n, blk, s, q, i, c)
    for q in range(4):
        codes = np.moveaxis(tq[:, :, :, q, :, :], -1, 2)   # (n, blk, c, s, i)
        words = np.zeros((n_seq, nb, d, bits), dtype=np.uint32)
        _put_codes(words, codes, bits)
        for w in range(bits):
            off = (w * 4 + q) * d
            blocks[:, :, off:off + d] = words[..., w]
    blocks[:, :, 4 * bits * d:] = nrm.reshape(n_seq, nb, 128).view(np.uint32)
    return blocks


def unpack_values(blocks, d: int, bits: int, n_tokens: int | None = None) -> dict:
    blocks = np.asarray(blocks, dtype=np.uint32)
    n_seq, nb, _ = blocks.shape
    idx = np.zeros((n_seq, nb, 8, 4, 4, d), dtype=np.int64)
    for q in range(4):
        words = np.stack([blocks[:, :, (w * 4 + q) * d:(w * 4 + q + 1) * d] for w in range(bits)], axis=-1)
        codes = _get_codes(words, bits)                    # (n, blk, c, s, i)
        idx[:, :, :, q, :, :] = np.moveaxis(codes, 2, -1)
    idx = idx.reshape(n_seq, nb * 128, d)
    nrm = blocks[:, :, 4 * bits * d:].copy().view(np.float32).reshape(n_seq, nb * 128)
    T = nb * 128 if n_tokens is None else n_tokens
    return dict(idx=idx[:, :T], norm=nrm[:, :T])


# ---------------------------------------------------------------------------
# Metrics ([superapi] 常见使用模式: attention cosine and top-1 match against
# the true attention; memory-savings estimate from layers, KV heads, length,
# head_dim and bits)
# ---------------------------------------------------------------------------

def attention_fidelity(Q, K, est, scale: float | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Per (seq, head): cosine between softmax(scale q.K^T) and
    softmax(scale est), and whether their argmax agree."""
    Q = _as64(Q)
    K = _as64(K)
    d = Q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    true = np.einsum("sgd,std->sgt", Q, K) * scale
    estl = est * scale

    def sm(z):
        z = z - z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=-1, keepdims=True)

    a, b = sm(true), sm(estl)
    cos = (a * b).sum(-1) / np.linalg.norm(a, axis=-1) / np.linalg.norm(b, axis=-1)
    top1 = a.argmax(-1) == b.argmax(-1)
    return cos, top1


def memory_bytes_page_formula(layers: int, kv_heads: int, seq_len: int, head_dim: int, bits: int) -> float:
    """Compressed K+V bytes under the accounting that reproduces the pages'
    figures ([superapi] 主要能力 and 比特宽度选择指南: 289 MB fp16 -> 76 / 58 /
    40 MB at 4 / 3 / 2 bits): b bits per coordinate for K and for V plus three
    16-bit scalars (||k||, ||v||, gamma) per token and KV head, i.e.
    2 b d + 48 bits.  The QJL sign bits are not counted by that accounting."""
    return layers * kv_heads * seq_len * (2 * bits * head_dim + 48) / 8.0


def memory_bytes_fp16(layers: int, kv_heads: int, seq_len: int, head_dim: int) -> float:
    return layers * kv_heads * seq_len * 2 * head_dim * 2.0
