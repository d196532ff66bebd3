"""CPU oracle for PolarQuant keys -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. The GPU library neither imports nor links it and this
module imports nothing from the library: the two share no code.

Plain numpy/scipy in float64, following the steps the pages give for
PolarQuant: random preconditioning, a recursive polar transformation, angle
codebooks designed from the angles' distribution, the radius kept apart.

Pages cited (title, section):
  [arxiv-summary] PolarQuant summary page (ai-summary of the PolarQuant paper),
            sections "3.中核となる技術的要素" (random preconditioning, polar
            transformation, codebooks from the angle distribution, recursive
            transform) and "4.有効性の検証方法と成果" (about 4.2x compression).
  [gemilab] "TurboQuant PolarQuant/QJL technical deep dive", section
            "PolarQuant：極座標変換による根本的削減" (v = r u, the inner product is
            governed by the direction).

Readings where the pages are silent (the pages give no recursion order, bit
allocation, angle range convention or record layout):
  P1 preconditioning: y = Pi x with the random rotation of the TurboQuant path
     (QR of a seeded Gaussian matrix); d a power of two, d = 2^L.
  P2 recursion: level 1 pairs coordinates (y[2i], y[2i+1]) into radius
     hypot and angle atan2(y[2i+1], y[2i]) in [-pi, pi]; level l >= 2 pairs
     the radii of level l-1 the same way, angle in [0, pi/2]; the last radius
     is ||x||. d - 1 angles in all.
  P3 angle laws for a uniformly random direction (what a random rotation
     produces; exact for Gaussian vectors): level 1 uniform on the circle;
     level l >= 2 with m = 2^(l-1): sin^2(psi) ~ Beta(m/2, m/2), density
     2^(2-m) sin^(m-1)(2 psi) / B(m/2, m/2) on [0, pi/2]; angles independent.
  P4 codebooks: level 1 the uniform quantizer with cells starting at -pi
     (the Lloyd-Max fixed point for a uniform law on the circle); levels >= 2
     Lloyd-Max for their law, made exactly symmetric about pi/4. Stored tables
     are fp32: boundaries (fp32 of the fp64 midpoints), cos and sin of the
     fp64 centroids rounded to fp32. Code = #{boundaries <= psi}.
  P5 bit allocation: b1 bits per level-1 angle, b2 per higher angle; default
     (4, 3): 477 bits per d = 128 vector with the fp32 radius, 4.29x against
     fp16, the pages' "about 4.2x".
  P6 record: level-1 codes little-endian in a bit stream of ceil(b1 d/2 / 32)
     words, then the higher codes (level 2 first, each level in node order)
     in a stream of ceil(b2 (d/2 - 1) / 32) words; the radius ||x|| as fp32.
  P7 scores: s = <Pi q, y_hat>, y_hat rebuilt from the stored tables top-down.

Parity status: transform, inverse, angle laws, level-1 and level-2 1-bit
codebooks, the Lloyd fixed point and the packing are pinned by tests; the
reading choices P1-P6 themselves have no reference on the pages to pin
against: "parity unpinned" for the bit allocation and record layout.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass

import numpy as np
from scipy import integrate, special


# ---------------------------------------------------------------------------
# Recursive polar transformation ([arxiv-summary] 3; readings P2)
# ---------------------------------------------------------------------------

def polar_transform(Y: np.ndarray):
    """(radius (n,), [level-1 angles (n, d/2), level-2 (n, d/4), ...]) of the
    rows of Y (d a power of two)."""
    Y = np.asarray(Y, dtype=np.float64)
    d = Y.shape[1]
    assert d >= 2 and d & (d - 1) == 0
    a, b = Y[:, 0::2], Y[:, 1::2]
    levels = [np.arctan2(b, a)]
    r = np.hypot(a, b)
    while r.shape[1] > 1:
        a, b = r[:, 0::2], r[:, 1::2]
        levels.append(np.arctan2(b, a))
        r = np.hypot(a, b)
    return r[:, 0], levels


def polar_inverse(radius, levels):
    """Rows rebuilt from the radius and the angles: node i of level l splits
    its radius into (r cos psi, r sin psi) for children 2i, 2i + 1."""
    r = np.asarray(radius, dtype=np.float64)[:, None]
    for ang in reversed(levels[1:]):
        r = np.stack([r * np.cos(ang), r * np.sin(ang)], axis=2).reshape(r.shape[0], -1)
    ang = levels[0]
    return np.stack([r * np.cos(ang), r * np.sin(ang)], axis=2).reshape(r.shape[0], -1)


# ---------------------------------------------------------------------------
# Angle laws (reading P3)
# ---------------------------------------------------------------------------

def angle_density(level: int, psi):
    """Density of a level-`level` angle of a uniformly random direction."""
    psi = np.asarray(psi, dtype=np.float64)
    if level == 1:
        return np.where((psi >= -math.pi) & (psi <= math.pi), 1.0 / (2 * math.pi), 0.0)
    m = 2 ** (level - 1)
    inside = (psi >= 0) & (psi <= math.pi / 2)
    logc = (2 - m) * math.log(2.0) - special.betaln(m / 2, m / 2)
    s = np.clip(np.sin(2 * np.clip(psi, 0, math.pi / 2)), 0, None)
    with np.errstate(divide="ignore"):
        val = np.exp(logc + (m - 1) * np.log(s)) if m > 1 else np.full_like(s, math.exp(logc))
    return np.where(inside, val, 0.0)


def angle_cdf(level: int, psi):
    psi = np.asarray(psi, dtype=np.float64)
    if level == 1:
        return np.clip((psi + math.pi) / (2 * math.pi), 0.0, 1.0)
    m = 2 ** (level - 1)
    p = np.clip(psi, 0.0, math.pi / 2)
    return special.betainc(m / 2, m / 2, np.sin(p) ** 2)


def _moment(level: int, a: float, b: float, k: int) -> float:
    v, _ = integrate.quad(lambda t: t ** k * float(angle_density(level, t)), a, b, epsabs=1e-15, epsrel=1e-13,
                          limit=200)
    return v


# ---------------------------------------------------------------------------
# Angle codebooks (reading P4)
# ---------------------------------------------------------------------------

def lloyd_max_angle(level: int, bits: int, tol: float = 1e-12, max_iter: int = 10000) -> np.ndarray:
    """fp64 centroids (ascending) of the MSE-optimal 2^bits-level quantizer of
    the level's angle law. Level 1: the uniform grid of cells starting at
    -pi. Levels >= 2: Lloyd iterations from the equal-mass cells (midpoint
    boundaries, conditional-mean centroids) until no centroid moves by `tol`,
    then symmetrized about pi/4 (the law is symmetric there)."""
    L = 1 << bits
    if level == 1:
        w = 2 * math.pi / L
        return -math.pi + (np.arange(L) + 0.5) * w
    m = 2 ** (level - 1)
    q = special.betaincinv(m / 2, m / 2, np.arange(L + 1) / L)
    edges = np.arcsin(np.sqrt(q))
    edges[0], edges[-1] = 0.0, math.pi / 2
    c = np.array([_moment(level, edges[i], edges[i + 1], 1) / _moment(level, edges[i], edges[i + 1], 0)
                  for i in range(L)])
    for _ in range(max_iter):
        e = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [math.pi / 2]))
        cn = np.array([_moment(level, e[i], e[i + 1], 1) / _moment(level, e[i], e[i + 1], 0) for i in range(L)])
        delta = np.max(np.abs(cn - c))
        c = cn
        if delta < tol:
            break
    return 0.5 * (c + (math.pi / 2 - c[::-1]))


@dataclass
class AngleCodebook:
    level: int
    bits: int
    centroids64: np.ndarray
    boundaries: np.ndarray   # fp32, 2^bits - 1 entries
    cos: np.ndarray          # fp32 cos of the fp64 centroids
    sin: np.ndarray          # fp32 sin of the fp64 centroids


def angle_codebook(level: int, bits: int) -> AngleCodebook:
    c = lloyd_max_angle(level, bits)
    if level == 1:
        t = -math.pi + np.arange(1, 1 << bits) * (2 * math.pi / (1 << bits))
    else:
        t = 0.5 * (c[:-1] + c[1:])
    return AngleCodebook(level, bits, c, t.astype(np.float32), np.cos(c).astype(np.float32),
                         np.sin(c).astype(np.float32))


@dataclass
class PolarCodebooks:
    d: int
    b1: int
    b2: int
    levels: list             # AngleCodebook per level 1..L

    @property
    def L(self) -> int:
        return int(round(math.log2(self.d)))


@functools.lru_cache(maxsize=None)
def polar_codebooks(d: int, b1: int = 4, b2: int = 3) -> PolarCodebooks:
    L = int(round(math.log2(d)))
    assert 1 << L == d and 1 <= b1 <= 4 and 1 <= b2 <= 4
    return PolarCodebooks(d, b1, b2, [angle_codebook(1, b1)] + [angle_codebook(l, b2) for l in range(2, L + 1)])


def angle_codes(psi, cb: AngleCodebook) -> np.ndarray:
    """#{stored boundaries <= psi} (fp64 comparison against the fp32 table)."""
    psi = np.asarray(psi, dtype=np.float64)
    return np.sum(psi[..., None] >= cb.boundaries.astype(np.float64), axis=-1).astype(np.int64)


# ---------------------------------------------------------------------------
# Encode, decode, score (readings P1, P6, P7)
# ---------------------------------------------------------------------------

@dataclass
class PolarEncoded:
    codes: list              # per level, (n, d / 2^l) int64
    norm: np.ndarray         # (n,) fp64 ||x||
    angles: list             # per level, fp64 angles (for boundary distances)


def polar_encode(X, Pi, pcb: PolarCodebooks) -> PolarEncoded:
    X = np.asarray(X, dtype=np.float64)
    Y = X @ np.asarray(Pi, dtype=np.float64).T                 # y = Pi x per row
    radius, levels = polar_transform(Y)
    codes = [angle_codes(a, cb) for a, cb in zip(levels, pcb.levels)]
    return PolarEncoded(codes, radius, levels)


def polar_rebuild(codes, norm, pcb: PolarCodebooks) -> np.ndarray:
    """y_hat (n, d) fp64 from the codes and the stored fp32 tables, top-down."""
    r = np.asarray(norm, dtype=np.float64)[:, None]
    for lv in range(pcb.L, 1, -1):
        cb = pcb.levels[lv - 1]
        k = codes[lv - 1]
        c, s = cb.cos.astype(np.float64)[k], cb.sin.astype(np.float64)[k]
        r = np.stack([r * c, r * s], axis=2).reshape(r.shape[0], -1)
    cb = pcb.levels[0]
    k = codes[0]
    c, s = cb.cos.astype(np.float64)[k], cb.sin.astype(np.float64)[k]
    return np.stack([r * c, r * s], axis=2).reshape(r.shape[0], -1)


def record_words(d: int, b1: int, b2: int):
    """(level-1 words, higher-level words) of a record."""
    return -(-(b1 * d // 2) // 32), -(-(b2 * (d // 2 - 1)) // 32)


def polar_record_bytes(d: int, b1: int = 4, b2: int = 3) -> int:
    w1, w2 = record_words(d, b1, b2)
    return 4 * (w1 + w2) + 4


def _pack_stream(codes: np.ndarray, bits: int, nwords: int) -> np.ndarray:
    n, k = codes.shape
    out = np.zeros((n, nwords), dtype=np.uint64)
    for j in range(k):
        off = j * bits
        w, sh = off // 32, off % 32
        v = codes[:, j].astype(np.uint64)
        out[:, w] |= (v << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:
            out[:, w + 1] |= v >> np.uint64(32 - sh)
    return out.astype(np.uint32)


def _unpack_stream(words: np.ndarray, bits: int, k: int) -> np.ndarray:
    w64 = words.astype(np.uint64)
    n = words.shape[0]
    out = np.zeros((n, k), dtype=np.int64)
    mask = np.uint64((1 << bits) - 1)
    for j in range(k):
        off = j * bits
        w, sh = off // 32, off % 32
        v = w64[:, w] >> np.uint64(sh)
        if sh + bits > 32:
            v |= w64[:, w + 1] << np.uint64(32 - sh)
        out[:, j] = (v & mask).astype(np.int64)
    return out


def pack_polar(enc: PolarEncoded, pcb: PolarCodebooks) -> dict:
    d = pcb.d
    w1, w2 = record_words(d, pcb.b1, pcb.b2)
    s1 = _pack_stream(enc.codes[0], pcb.b1, w1)
    s2 = _pack_stream(np.concatenate(enc.codes[1:], axis=1), pcb.b2, w2)
    return {"bits": np.concatenate([s1, s2], axis=1), "norms": enc.norm.astype(np.float32)}


def unpack_polar(words: np.ndarray, pcb: PolarCodebooks) -> list:
    d = pcb.d
    w1, w2 = record_words(d, pcb.b1, pcb.b2)
    c1 = _unpack_stream(words[:, :w1], pcb.b1, d // 2)
    hi = _unpack_stream(words[:, w1:w1 + w2], pcb.b2, d // 2 - 1)
    codes, o = [c1], 0
    for lv in range(2, pcb.L + 1):
        k = d >> lv
        codes.append(hi[:, o:o + k])
        o += k
    return codes


def polar_scores(Qv, Pi, pcb: PolarCodebooks, keys: dict) -> np.ndarray:
    """s = <Pi q, y_hat> for every (query, key) pair (reading P7)."""
    codes = unpack_polar(keys["bits"], pcb)
    Yh = polar_rebuild(codes, np.asarray(keys["norms"], dtype=np.float64), pcb)
    q_rot = np.asarray(Qv, dtype=np.float64) @ np.asarray(Pi, dtype=np.float64).T
    return q_rot @ Yh.T


def polar_attention_decode(Qh, Pi, pcb: PolarCodebooks, cbv, keys: dict, values: dict, seq_len: int,
                           scale: float, unpack_values):
    """softmax(scale * s) V_hat for the query heads of one KV stream, s from
    PolarQuant keys, V_hat = ||v|| Pi^T c_v[idx] from stage-1 value records
    ([gemilab] Attention機構). unpack_values: the value-record reader."""
    d = Pi.shape[0]
    s = polar_scores(Qh, Pi, pcb, {"bits": keys["bits"][:seq_len], "norms": keys["norms"][:seq_len]})
    lg = s * scale
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    vidx = unpack_values(values["bits"], d, cbv.bits, seq_len)
    Vrot = np.asarray(values["norms"][:seq_len], dtype=np.float64)[:, None] * cbv.centroids.astype(np.float64)[vidx]
    return (p @ Vrot) @ np.asarray(Pi, dtype=np.float64)


__all__ = [
    "polar_transform", "polar_inverse", "angle_density", "angle_cdf", "lloyd_max_angle", "AngleCodebook",
    "angle_codebook", "PolarCodebooks", "polar_codebooks", "angle_codes", "PolarEncoded", "polar_encode",
    "polar_rebuild", "record_words", "polar_record_bytes", "pack_polar", "unpack_polar", "polar_scores",
    "polar_attention_decode",
]
