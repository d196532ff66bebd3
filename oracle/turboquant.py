"""CPU oracle for the TurboQuant hot path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library neither imports nor links it, and this
package imports nothing from the library: the two share no code. The only
shared inputs are the seeded arrays produced by the ``synth`` package.

Everything here is plain, slow numpy/scipy in float64. It follows the steps in
the pages' order; where the pages leave a step open, the reading taken is
stated at the function (and listed in the design notes).

Pages cited (title, section):
  [ebisuda] "TurboQuant: Google's 6x KV Cache Compression Algorithm Gains
            Open-Source Momentum" (ebisuda.net), sections
            "第1段階：PolarQuant（MSE最適圧縮）", "第2段階：QJL残差補正（1ビット）",
            "性能サマリー".
  [hakusoku] "TurboQuant: 極限圧縮によるAI効率の再定義" (hakusoku.com), sections
            "QJL：ゼロオーバーヘッド・1ビット圧縮", "TurboQuantの実験結果".
  [gemilab] "TurboQuant PolarQuant/QJL technical deep dive" (gemilab.net),
            sections "Transformerの Attention 機構", "QJLの応用".

Parity status: every public function below is pinned by a ``-m "not gpu"``
test in tests/test_oracle_pins.py (closed forms, textbook special cases,
brute force, invariants or library routines); the packed bit layout is a
format choice, pinned by hand-written fixtures in tests/golden/.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy import special

__all__ = [
    "splitmix64_mix", "seeded_gaussian", "rotation_from_gaussian", "sketch_from_gaussian", "coord_density", "coord_cdf",
    "lloyd_max", "Codebook", "codebook", "encode", "qjl_stage", "Encoded", "query_prep", "qjl_constant",
    "scores", "scores_from_parts", "dequantize_keys", "attention_decode", "attention_prefill", "topk", "stored_norms",
    "recall_at_k", "pack_keys", "unpack_keys", "pack_values", "unpack_values",
    "key_record_bytes", "value_record_bytes",
]


# ---------------------------------------------------------------------------
# Setup: random rotation and sketch matrix
# ---------------------------------------------------------------------------

def rotation_from_gaussian(G: np.ndarray, return_fp64: bool = False):
    """Random orthogonal rotation from the QR factorization of a Gaussian matrix.

    [ebisuda, 第1段階] rotates every input vector by a random orthogonal
    matrix obtained from the QR decomposition of a Gaussian matrix. QR is
    unique once diag(R) is made positive, so Q is multiplied by
    diag(sign(diag R)) with sign(0) = +1 (reading: this makes Q unique and
    Haar-distributed). The stored table is the fp32 rounding of that Q.
    Convention: the rotated vector is y = Pi @ u.
    """
    G = np.asarray(G, dtype=np.float64)
    Q, R = np.linalg.qr(G)
    s = np.where(np.diag(R) >= 0.0, 1.0, -1.0)
    Q = Q * s[None, :]
    Pi = Q.astype(np.float32)
    return (Pi, Q, R * s[:, None]) if return_fp64 else Pi


# Seeded Gaussian draws. The pages say only that the rotation is the QR factor
# of a Gaussian matrix and the sketch a Gaussian matrix; the seed-to-matrix map
# is a reading: a counter-based generator (the SplitMix64 output function,
# Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
# OOPSLA 2014) turned into normal pairs by the Box-Muller transform (Box &
# Muller, 1958). Stream 1 draws the rotation's Gaussian matrix, stream 2 the
# sketch's; entries are filled row-major.
SPLITMIX_GAMMA = 0x9E3779B97F4A7C15
STREAM_ROTATION = 1
STREAM_SKETCH = 2


def splitmix64_mix(z):
    """The SplitMix64 output function on uint64 values (numpy arrays wrap mod 2^64):
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
    z ^= z >> 31."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def seeded_gaussian(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """rows x cols float64 N(0,1) draws for (seed, stream): word i =
    mix(seed XOR stream * GAMMA XOR i) (mod 2^64), u_i = (word_i >> 11) / 2^53 in
    [0, 1); entries 2k and 2k + 1 are r cos(2 pi u_{2k+1}) and r sin(2 pi u_{2k+1})
    with r = sqrt(-2 ln(1 - u_{2k})), filled row-major (rows * cols even)."""
    n = rows * cols
    assert n % 2 == 0
    key = np.uint64((int(seed) ^ ((int(stream) * SPLITMIX_GAMMA) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF)
    words = splitmix64_mix(key ^ np.arange(n, dtype=np.uint64))
    u = (words >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(1.0 - u1))  # 1 - u is exact in fp64
    out = np.empty(n, dtype=np.float64)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out.reshape(rows, cols)


def sketch_from_gaussian(G: np.ndarray) -> np.ndarray:
    """JL sketch matrix S (m x d) with i.i.d. N(0,1) entries, stored in fp32.

    [gemilab, QJLの応用] projects the quantization error with a random
    Gaussian matrix before keeping one bit per projected coordinate.
    """
    return np.asarray(G, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------------------
# Setup: Lloyd-Max codebook for one rotated coordinate
# ---------------------------------------------------------------------------

def _log_beta_norm(d: int) -> float:
    # log B(1/2, (d-1)/2): normalizer of (1-x^2)^((d-3)/2) on [-1, 1]
    return float(special.betaln(0.5, (d - 1) / 2.0))


def coord_density(d: int, x):
    """Density of one coordinate of a uniformly random unit vector in R^d.

    [ebisuda, 第1段階]: after the random rotation each coordinate follows a
    Beta law (close to N(0, 1/d) in high dimension). Exactly,
    f_d(x) = (1 - x^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1], i.e.
    (1 + x)/2 ~ Beta((d-1)/2, (d-1)/2). Reading: the exact law is used,
    the Gaussian is only its limit.
    """
    x = np.asarray(x, dtype=np.float64)
    inside = np.abs(x) < 1.0
    out = np.zeros_like(x)
    xi = x[inside]
    out[inside] = np.exp((d - 3) / 2.0 * np.log1p(-xi * xi) - _log_beta_norm(d))
    return out


def coord_cdf(d: int, x):
    """CDF of f_d: the regularized incomplete beta I_{(1+x)/2}((d-1)/2, (d-1)/2)."""
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    a = (d - 1) / 2.0
    return special.betainc(a, a, (1.0 + x) / 2.0)


def _first_moment(d: int, a, b):
    """Integral of x f_d(x) over [a, b] in closed form:
    [(1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)] / ((d-1) B(1/2, (d-1)/2))."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    lb = _log_beta_norm(d)

    def g(x):
        x = np.clip(x, -1.0, 1.0)
        with np.errstate(divide="ignore"):
            return np.exp((d - 1) / 2.0 * np.log1p(-x * x) - math.log(d - 1) - lb)

    return g(a) - g(b)


def _second_moment(d: int, a, b):
    """Integral of x^2 f_d(x) over [a, b], by parts:
    [a w(a) - b w(b)]/(d-1) + B(1/2,(d+1)/2)/((d-1) B(1/2,(d-1)/2)) (F_{d+2}(b) - F_{d+2}(a)),
    with w(x) = (1-x^2)^((d-1)/2) / B(1/2,(d-1)/2)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    lb = _log_beta_norm(d)

    def w(x):
        x = np.clip(x, -1.0, 1.0)
        with np.errstate(divide="ignore"):
            return np.exp((d - 1) / 2.0 * np.log1p(-x * x) - lb)

    boundary = (a * w(a) - b * w(b)) / (d - 1)
    ratio = math.exp(float(special.betaln(0.5, (d + 1) / 2.0)) - lb) / (d - 1)
    return boundary + ratio * (coord_cdf(d + 2, b) - coord_cdf(d + 2, a))


def lloyd_max(d: int, bits: int, tol: float = 1e-14, max_iter: int = 200000):
    """Lloyd-Max quantizer of f_d at `bits` bits: 2^bits centroids (ascending), fp64.

    [ebisuda, 第1段階]: Lloyd-Max solves the continuous 1-D k-means problem
    and finds the bucket boundaries and centroids that minimize MSE at the
    given bit width (3 bits = 8 levels); the codebook is precomputed per bit
    width and does not depend on data.

    Steps: start from the centroids of the equal-mass cells; then alternate
    (boundaries = midpoints of neighbouring centroids) and (centroid = mean of
    f_d over its cell) until no centroid moves by more than `tol`; finally
    make the table exactly antisymmetric (f_d is even). The cell mass uses
    the regularized incomplete beta, the first moment its closed form.
    f_d is log-concave for d >= 3, so the fixed point is unique.
    """
    if d < 3:
        raise ValueError("d >= 3 required (f_d is not log-concave for d < 3)")
    L = 1 << bits
    a = (d - 1) / 2.0
    q = special.betaincinv(a, a, np.arange(L + 1) / L)
    edges = 2.0 * q - 1.0
    edges[0], edges[-1] = -1.0, 1.0
    c = _first_moment(d, edges[:-1], edges[1:]) / (coord_cdf(d, edges[1:]) - coord_cdf(d, edges[:-1]))
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        mass = coord_cdf(d, edges[1:]) - coord_cdf(d, edges[:-1])
        c_new = _first_moment(d, edges[:-1], edges[1:]) / mass
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol:
            break
    c = 0.5 * (c - c[::-1])
    return c


@dataclass
class Codebook:
    d: int
    bits: int
    centroids64: np.ndarray   # fp64 Lloyd-Max centroids (ascending)
    centroids: np.ndarray     # stored table: fp32 centroids
    boundaries: np.ndarray    # stored table: fp32 of the fp64 midpoints
    distortion: float         # per-coordinate MSE of the stored tables under f_d

    @property
    def levels(self) -> int:
        return 1 << self.bits


def codebook(d: int, bits: int) -> Codebook:
    """Stored codebook: fp32 centroids, fp32 boundaries (fp32 of the fp64
    midpoints) and the analytic per-coordinate distortion of those tables,
    D = sum_i int_{cell_i} (x - c_i)^2 f_d(x) dx. Reading: tables are fp32."""
    c64 = lloyd_max(d, bits)
    t64 = 0.5 * (c64[:-1] + c64[1:])
    cen = c64.astype(np.float32)
    bnd = t64.astype(np.float32)
    e = np.concatenate(([-1.0], bnd.astype(np.float64), [1.0]))
    cc = cen.astype(np.float64)
    m0 = coord_cdf(d, e[1:]) - coord_cdf(d, e[:-1])
    m1 = _first_moment(d, e[:-1], e[1:])
    m2 = _second_moment(d, e[:-1], e[1:])
    D = float(np.sum(m2 - 2.0 * cc * m1 + cc * cc * m0))
    return Codebook(d, bits, c64, cen, bnd, D)


# ---------------------------------------------------------------------------
# Encode (quantize) keys and values
# ---------------------------------------------------------------------------

@dataclass
class Encoded:
    idx: np.ndarray          # (n, d) int64 codebook indices
    sigma: np.ndarray | None  # (n, m) bool QJL sign bits (keys only)
    norm: np.ndarray         # (n,) fp64 ||x||
    rho: np.ndarray | None   # (n,) fp64 ||r|| (keys only)
    y: np.ndarray            # (n, d) fp64 rotated unit vector (for boundary distances)
    z: np.ndarray | None     # (n, m) fp64 sketch of the residual (for sign distances)
    S: np.ndarray | None = None  # the sketch matrix used (keys), for re-deriving stage 2


def encode(X: np.ndarray, Pi: np.ndarray, cb: Codebook | None, S: np.ndarray | None = None) -> Encoded:
    """Quantize rows of X (fp32 or bf16 values).

    Stage 1 [ebisuda, 第1段階]: n = ||x||, u = x / n, y = Pi u; each rotated
    coordinate is mapped independently to the codebook: idx_j = number of
    boundaries t_i with t_i <= y_j (reading: a tie goes to the upper cell).
    Only per-vector scalars are kept, no per-block scale or zero point.
    Stage 2 [ebisuda, 第2段階; hakusoku, QJL] (keys, S given): residual
    r = y - c[idx] in the rotated domain (reading), rho = ||r||, z = S r,
    sigma_i = [z_i >= 0] (reading: sign(0) = +1).
    A zero vector gives an all-zero record (reading).
    Key variants: S omitted gives MSE-only keys (stage 1 alone); cb None (no
    codebook bits) gives pure QJL keys: the residual is the whole rotated unit
    vector, r = y, so rho = ||y|| = 1 up to rounding [hakusoku, QJL].
    """
    X = np.asarray(X, dtype=np.float64)
    Pi64 = np.asarray(Pi, dtype=np.float64)
    n = np.sqrt(np.sum(X * X, axis=1))
    nz = n > 0
    U = np.zeros_like(X)
    U[nz] = X[nz] / n[nz, None]
    Y = U @ Pi64.T
    if cb is None:
        idx = np.zeros(Y.shape, dtype=np.int64)
    else:
        idx = np.searchsorted(cb.boundaries.astype(np.float64), Y, side="right").astype(np.int64)
    idx[~nz] = 0
    sigma = rho = Z = None
    if S is not None:
        rho, Z, sigma = qjl_stage(Y, idx, cb, S, nz)
    return Encoded(idx, sigma, n, rho, Y, Z, None if S is None else np.asarray(S))


def qjl_stage(Y: np.ndarray, idx: np.ndarray, cb: Codebook | None, S: np.ndarray, live: np.ndarray):
    """Stage 2 of the key encoder for given stage-1 codes [ebisuda, 第2段階;
    hakusoku, QJL]: residual r = y - c[idx] in the rotated domain (pure QJL
    keys, cb None: r = y), rho = ||r||, z = S r, sigma = [z >= 0]; rows with
    live False (zero vectors) give r = 0, rho = 0 and sigma all False.
    `encode` applies it to its own codes; the parity checks apply it to another
    encoder's codes (a code decided on the other side of a boundary changes r)."""
    Y = np.asarray(Y, dtype=np.float64)
    R = Y - cb.centroids.astype(np.float64)[idx] if cb is not None else Y.copy()
    R[~live] = 0.0
    rho = np.sqrt(np.sum(R * R, axis=1))
    Z = R @ np.asarray(S, dtype=np.float64).T
    sigma = Z >= 0.0
    sigma[~live] = False
    return rho, Z, sigma


# ---------------------------------------------------------------------------
# Estimator: scores and attention over packed records
# ---------------------------------------------------------------------------

def qjl_constant(m: int) -> float:
    """sqrt(pi/2)/m. For g ~ N(0, I): E[<g,q> sign<g,r>] = sqrt(2/pi) <q, r/||r||>,
    so sqrt(pi/2)/m * ||r|| * sum_i <s_i,q> sign<s_i,r> is unbiased for <q, r>
    (reading of the 1-bit bias correction in [ebisuda, 第2段階])."""
    return math.sqrt(math.pi / 2.0) / m


def query_prep(Qv: np.ndarray, Pi: np.ndarray, S: np.ndarray):
    """Full-precision query side of the asymmetric estimator [hakusoku, QJL]:
    q_rot = Pi q and q_s = S q_rot, in fp64."""
    Q = np.asarray(Qv, dtype=np.float64)
    q_rot = Q @ np.asarray(Pi, dtype=np.float64).T
    q_s = q_rot @ np.asarray(S, dtype=np.float64).T
    return q_rot, q_s


def scores_from_parts(q_rot, q_s, idx, sigma, norm, rho, cb: Codebook | None, m: int):
    """s = n (<q_rot, c[idx]> + sqrt(pi/2)/m * rho * <q_s, 2 sigma - 1>) for all
    (query, key) pairs: the stage-1 inner product plus the QJL correction
    [ebisuda, 第2段階; hakusoku, QJL]. norm, rho are the stored values (fp32 or
    compact fp16).
    MSE-only keys (sigma None) keep the first term, pure QJL keys (cb None) the
    second."""
    nn = np.asarray(norm, dtype=np.float64)[None, :]
    out = np.zeros((np.asarray(q_rot).shape[0], nn.shape[1]))
    if cb is not None:
        C = cb.centroids.astype(np.float64)[idx]               # (n, d)
        out += np.asarray(q_rot) @ C.T                         # (nq, n)
    if sigma is not None:
        pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0   # (n, m)
        rr = np.asarray(rho, dtype=np.float64)[None, :]
        out += qjl_constant(m) * rr * (np.asarray(q_s) @ pm.T)
    return nn * out


def scores(Qv, Pi, S, cb: Codebook | None, keys: dict, qjl: bool = True):
    """Scores of queries against a packed key array (see pack_keys)."""
    d = Pi.shape[0]
    bits = cb.bits if cb is not None else 0
    idx, sigma = unpack_keys(keys["bits"], d, bits, qjl)
    q_rot, q_s = query_prep(Qv, Pi, S)
    norms = np.asarray(keys["norms"]).reshape(idx.shape[0], 1 + int(qjl))
    rho = norms[:, 1] if qjl else None
    return scores_from_parts(q_rot, q_s, idx, sigma, norms[:, 0], rho, cb, S.shape[0])


def dequantize_keys(Pi, S, cb: Codebook, idx, sigma, norm, rho):
    """k_hat = n Pi^T (c[idx] + sqrt(pi/2)/m rho S^T (2 sigma - 1)): the key whose
    inner product with any q equals the score (linearity); [gemilab, QJLの応用]
    describes decoding as an approximate reconstruction of the error."""
    m = S.shape[0]
    C = cb.centroids.astype(np.float64)[idx]
    pm = 2.0 * np.asarray(sigma, dtype=np.float64) - 1.0
    corr = qjl_constant(m) * np.asarray(rho, np.float64)[:, None] * (pm @ np.asarray(S, np.float64))
    return np.asarray(norm, np.float64)[:, None] * ((C + corr) @ np.asarray(Pi, np.float64))


def attention_decode(Qh, Pi, S, cbk: Codebook | None, cbv: Codebook, keys: dict, values: dict, seq_len: int,
                     scale: float, qjl: bool = True):
    """One decode step for one (sequence, KV head): softmax(q K^T * scale) V for
    each query head that shares this KV head [gemilab, Attention機構], with the
    keys' scores from the estimator and V dequantized with its own codebook:
    v_hat_t = ||v_t|| Pi^T c_v[idx_t] (stage 1 only for values, reading).
    Qh: (g, d) queries. Returns (g, d) fp64 outputs."""
    d = Pi.shape[0]
    s = scores(Qh, Pi, S, cbk, keys, qjl)[:, :seq_len]         # (g, L)
    logits = s * scale
    mx = np.max(logits, axis=1, keepdims=True)
    p = np.exp(logits - mx)
    p /= np.sum(p, axis=1, keepdims=True)
    vidx = unpack_values(values["bits"], d, cbv.bits, seq_len)
    Vrot = values["norms"][:seq_len].astype(np.float64)[:, None] * cbv.centroids.astype(np.float64)[vidx]
    o_rot = p @ Vrot
    return o_rot @ np.asarray(Pi, dtype=np.float64)


def attention_prefill(Qpos, Pi, S, cbk: Codebook | None, cbv: Codebook, keys: dict, values: dict, seq_len: int,
                      scale: float, causal: bool, qjl: bool = True):
    """Many query positions of one (sequence, KV head) over its packed cache:
    position i (of n_q) sees tokens t < seq_len, and with `causal` only
    t < seq_len - n_q + i + 1 (reading: the chunk's own tokens are already in the
    cache). Qpos: (n_q, g, d). A position that sees no token gets zeros.
    Returns (n_q, g, d) fp64."""
    Qpos = np.asarray(Qpos)
    nq = Qpos.shape[0]
    out = np.zeros(Qpos.shape, dtype=np.float64)
    for i in range(nq):
        lim = min(seq_len - nq + i + 1, seq_len) if causal else seq_len
        if lim > 0:
            out[i] = attention_decode(Qpos[i], Pi, S, cbk, cbv, keys, values, lim, scale, qjl)
    return out


def topk(score_row: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, ordered by (-score, index): ties go to
    the lower index (reading)."""
    s = np.asarray(score_row)
    order = np.lexsort((np.arange(s.shape[0]), -s))
    return order[:k]


def recall_at_k(found: np.ndarray, exact: np.ndarray) -> float:
    """Mean over queries of |found_q intersect exact_q| / k."""
    k = exact.shape[1]
    return float(np.mean([len(set(f.tolist()) & set(e.tolist())) / k for f, e in zip(found, exact)]))


# ---------------------------------------------------------------------------
# Packed record format (a format choice; the pages fix none)
# ---------------------------------------------------------------------------
# Keys, one record per vector (m == d), W = d/32 coordinate groups, Q = 1 with
# the QJL stage (0 for MSE-only keys; B = 0 with Q = 1 for pure QJL keys):
#   bits  : uint32 [n][W][B+Q]; for group w, word p < B holds bit p of idx_j
#           at bit position (j - 32w) for j in [32w, 32w+32); word B (when Q)
#           holds sigma_i at bit position (i - 32w).
#   norms : float32 [n][1+Q] = (||x||) or (||x||, ||r||).
# Values, token-major blocks of 32 tokens, W_t = ceil(n/32) blocks:
#   bits  : uint32 [W_t][d][B]; word [t//32][j][p] holds bit p of idx[t][j]
#           at bit position t % 32. Unused tail bits are 0.
#   norms : float32 [n] = ||v||.
# Compact norms (norm_f16): every norm stored as float16 instead, rounded to
# nearest even from the exact value and saturated at the largest finite
# float16, 65504 (reading: the pages fix no norm precision).

F16_MAX = 65504.0


def stored_norms(x, norm_f16: bool = False) -> np.ndarray:
    """Norms as a record stores them: float32, or float16 (nearest even,
    saturated at F16_MAX) with compact norms."""
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, F16_MAX).astype(np.float16) if norm_f16 else x.astype(np.float32)


def key_record_bytes(d: int, bits: int, qjl: bool = True, norm_f16: bool = False) -> int:
    return (d // 32) * (bits + int(qjl)) * 4 + (2 if norm_f16 else 4) * (1 + int(qjl))


def value_record_bytes(d: int, bits: int, norm_f16: bool = False) -> int:
    return d * bits // 8 + (2 if norm_f16 else 4)


def pack_keys(enc: Encoded, bits: int, qjl: bool = True, norm_f16: bool = False) -> dict:
    idx, sig = enc.idx, enc.sigma
    n, d = idx.shape
    assert d % 32 == 0 and (not qjl or sig.shape == (n, d))
    W = d // 32
    out = np.zeros((n, W, bits + int(qjl)), dtype=np.uint64)
    pos = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    for w in range(W):
        blk = idx[:, 32 * w:32 * w + 32].astype(np.uint64)
        for p in range(bits):
            out[:, w, p] = np.sum(((blk >> np.uint64(p)) & np.uint64(1)) * pos, axis=1)
        if qjl:
            out[:, w, bits] = np.sum(sig[:, 32 * w:32 * w + 32].astype(np.uint64) * pos, axis=1)
    if qjl:
        norms = np.stack([stored_norms(enc.norm, norm_f16), stored_norms(enc.rho, norm_f16)], axis=1)
    else:
        norms = stored_norms(enc.norm, norm_f16)[:, None]
    return {"bits": out.astype(np.uint32), "norms": norms}


def unpack_keys(words: np.ndarray, d: int, bits: int, qjl: bool = True):
    """(idx, sigma); sigma is None for MSE-only keys."""
    n = words.shape[0]
    w = words.reshape(n, d // 32, bits + int(qjl)).astype(np.uint64)
    sh = np.arange(32, dtype=np.uint64)
    idx = np.zeros((n, d), dtype=np.int64)
    for p in range(bits):
        b = (w[:, :, p, None] >> sh) & np.uint64(1)
        idx |= (b.reshape(n, d).astype(np.int64) << p)
    sig = ((w[:, :, bits, None] >> sh) & np.uint64(1)).reshape(n, d).astype(bool) if qjl else None
    return idx, sig


def pack_values(enc: Encoded, bits: int, norm_f16: bool = False) -> dict:
    idx = enc.idx
    n, d = idx.shape
    nb = (n + 31) // 32
    pad = np.zeros((nb * 32, d), dtype=np.uint64)
    pad[:n] = idx
    blk = pad.reshape(nb, 32, d)                                # [blk][t][j]
    pos = (np.uint64(1) << np.arange(32, dtype=np.uint64))[None, :, None]
    out = np.zeros((nb, d, bits), dtype=np.uint64)
    for p in range(bits):
        out[:, :, p] = np.sum(((blk >> np.uint64(p)) & np.uint64(1)) * pos, axis=1)
    return {"bits": out.astype(np.uint32), "norms": stored_norms(enc.norm, norm_f16)}


def unpack_values(words: np.ndarray, d: int, bits: int, n: int):
    nb = words.shape[0]
    w = words.reshape(nb, d, bits).astype(np.uint64)
    sh = np.arange(32, dtype=np.uint64)
    idx = np.zeros((nb, 32, d), dtype=np.int64)
    for p in range(bits):
        b = (w[:, None, :, p] >> sh[None, :, None]) & np.uint64(1)   # [blk][t][j]
        idx |= b.astype(np.int64) << p
    return idx.reshape(nb * 32, d)[:n]
