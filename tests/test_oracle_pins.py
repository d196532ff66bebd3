"""Pins of the CPU oracle against what the pages and mathematics fix.

Every check compares the oracle with something other than itself: closed
forms, a textbook table, brute force on tiny inputs, independent quadrature,
library routines, or statistical laws with known moments.
"""
import math
import os

import numpy as np
import pytest
from scipy import integrate, special

import synth
from oracle import turboquant as T

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ctx(d, seed=0, m=None):
    m = d if m is None else m
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_ROTATION, d, d))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_SKETCH, m, d))
    return Pi, S


# --- seeded Gaussian draws ----------------------------------------------------

def test_splitmix64_output_function_published_values():
    """The SplitMix64 generator (state += 0x9E3779B97F4A7C15, then the output
    function) seeded with 1234567 gives the reference implementation's first
    five outputs (the published test vector of splitmix64.c)."""
    M = (1 << 64) - 1
    got = [int(T.splitmix64_mix(np.uint64((1234567 + k * T.SPLITMIX_GAMMA) & M))) for k in range(1, 6)]
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423, 4593380528125082431,
                   16408922859458223821]


def test_seeded_gaussian_is_standard_normal():
    """10^6 draws: mean 0 and variance 1 within 3 standard errors; the
    Kolmogorov-Smirnov distance to N(0,1) is small; the Box-Muller pairs are
    uncorrelated and their squared radius has mean 2 (r^2 / 2 ~ Exp(1));
    different streams and seeds give different draws."""
    from scipy import stats
    n = 10 ** 6
    g = T.seeded_gaussian(3, 1, 1000, 1000).ravel()
    se = 1 / math.sqrt(n)
    assert abs(g.mean()) < 3 * se
    assert abs(g.var() - 1) < 3 * math.sqrt(2 / n)
    assert stats.kstest(g, "norm").statistic < 2e-3
    a, b = g[0::2], g[1::2]
    assert abs(np.mean(a * b)) < 3 / math.sqrt(n / 2)
    r2 = a * a + b * b
    assert abs(r2.mean() - 2) < 3 * 2 / math.sqrt(n / 2)
    assert not np.array_equal(T.seeded_gaussian(3, 2, 10, 10), T.seeded_gaussian(3, 1, 10, 10))
    assert not np.array_equal(T.seeded_gaussian(4, 1, 10, 10), T.seeded_gaussian(3, 1, 10, 10))


# --- rotation ---------------------------------------------------------------

@pytest.mark.parametrize("d", [8, 128, 1536])
def test_rotation_is_orthogonal(d):
    G = synth.gaussian_matrix(3, synth.TAG_ROTATION, d, d)
    Pi, Q, R = T.rotation_from_gaussian(G, return_fp64=True)
    assert np.max(np.abs(Pi.astype(np.float64).T @ Pi.astype(np.float64) - np.eye(d))) <= 1e-5
    assert np.max(np.abs(Q @ R - G)) <= 1e-12 * max(1.0, np.max(np.abs(G))) * d
    assert np.all(np.diag(R) > 0)
    assert np.allclose(np.triu(R), R)


def test_rotation_matches_gram_schmidt():
    """Classical Gram-Schmidt on the columns of G, written with plain loops,
    yields the unique Q with positive diag(R): it must equal the oracle's Q."""
    d = 6
    G = synth.gaussian_matrix(11, synth.TAG_ROTATION, d, d)
    cols = []
    for j in range(d):
        v = [G[i][j] for i in range(d)]
        for q in cols:
            dot = sum(q[i] * G[i][j] for i in range(d))
            v = [v[i] - dot * q[i] for i in range(d)]
        nv = math.sqrt(sum(x * x for x in v))
        cols.append([x / nv for x in v])
    Qgs = np.array(cols).T
    _, Q, _ = T.rotation_from_gaussian(G, return_fp64=True)
    assert np.max(np.abs(Q - Qgs)) < 1e-10


def test_sketch_is_rounded_gaussian():
    G = synth.gaussian_matrix(5, synth.TAG_SKETCH, 16, 32)
    S = T.sketch_from_gaussian(G)
    assert S.dtype == np.float32 and S.shape == (16, 32)
    assert np.array_equal(S, G.astype(np.float32))


# --- coordinate density and moments ------------------------------------------

@pytest.mark.parametrize("d", [3, 5, 128, 1536])
def test_density_normalized_and_second_moment(d):
    f = lambda x: float(T.coord_density(d, np.array([x]))[0])
    s = 1.0 / math.sqrt(d)
    lim = min(1.0, 40 * s)
    mass = integrate.quad(f, -lim, lim, points=[0.0], limit=200)[0]
    m2 = integrate.quad(lambda x: x * x * f(x), -lim, lim, points=[0.0], limit=200)[0]
    assert abs(mass - 1.0) < 1e-9
    assert abs(m2 - 1.0 / d) < 1e-9 / d  # E[x_j^2] = 1/d for a uniform unit vector


def test_density_matches_unit_vector_sampling():
    # empirical check: coordinates of normalized Gaussian vectors in d=8
    d = 8
    x = synth.unit_gaussian(1, (99,), (200000, d)).astype(np.float64)[:, 0]
    for a in (-0.5, 0.0, 0.3):
        emp = np.mean(x <= a)
        se = math.sqrt(emp * (1 - emp) / x.size)
        assert abs(emp - float(T.coord_cdf(d, a))) < 4 * se


@pytest.mark.parametrize("d", [4, 128])
def test_cell_moments_vs_quadrature(d):
    f = lambda x: float(T.coord_density(d, np.array([x]))[0])
    a, b = -0.05, 0.12
    assert abs((T.coord_cdf(d, b) - T.coord_cdf(d, a)) - integrate.quad(f, a, b)[0]) < 1e-12
    assert abs(T._first_moment(d, a, b) - integrate.quad(lambda x: x * f(x), a, b)[0]) < 1e-12
    assert abs(T._second_moment(d, a, b) - integrate.quad(lambda x: x * x * f(x), a, b)[0]) < 1e-12


# --- codebook -----------------------------------------------------------------

@pytest.mark.parametrize("d,bits", [(4, 2), (128, 1), (128, 2), (128, 3), (128, 4), (1536, 3)])
def test_codebook_fixed_point(d, bits):
    """Centroid condition c_i = E[X | cell_i] and midpoint condition, by
    independent quadrature; antisymmetric table."""
    c = T.lloyd_max(d, bits)
    f = lambda x: float(T.coord_density(d, np.array([x]))[0])
    t = 0.5 * (c[:-1] + c[1:])
    e = np.concatenate(([-1.0], t, [1.0]))
    lim = min(1.0, 40 / math.sqrt(d))
    for i in range(len(c)):
        a, b = max(e[i], -lim), min(e[i + 1], lim)
        m0 = integrate.quad(f, a, b, limit=200, epsabs=1e-15, epsrel=1e-13)[0]
        m1 = integrate.quad(lambda x: x * f(x), a, b, limit=200, epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(m1 / m0 - c[i]) < 1e-10 * max(1.0, abs(c[i])) + 1e-12
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(c, -c[::-1])


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_codebook_d3_is_uniform(bits):
    """d = 3: f_3 is uniform on [-1, 1], so c_i = -1 + (2i+1)/L and D = 1/(3 L^2)."""
    L = 1 << bits
    cb = T.codebook(3, bits)
    exact = -1.0 + (2.0 * np.arange(L) + 1.0) / L
    assert np.max(np.abs(cb.centroids64 - exact)) < 1e-13
    assert abs(cb.distortion - 1.0 / (3 * L * L)) < 1e-9


@pytest.mark.parametrize("d", [4, 128, 1536])
def test_codebook_one_bit_closed_form(d):
    """B = 1: c = +-E|X| = +-Gamma(d/2)/(sqrt(pi) Gamma((d+1)/2)), D = 1/d - E|X|^2."""
    e_abs = math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    cb = T.codebook(d, 1)
    # gammaln/betaln at large arguments carry ~1e-12 relative rounding
    assert abs(cb.centroids64[1] - e_abs) < 1e-11 * e_abs
    assert abs(cb.centroids64[0] + e_abs) < 1e-11 * e_abs
    # stored table: fp32 centroid; analytic D of the stored table differs from the
    # fp64 optimum only by (c32 - c64)^2
    assert abs(cb.distortion - (1.0 / d - e_abs ** 2)) < 1e-12
    if d == 128:
        assert abs(e_abs - 0.0706616) < 1e-7


def _max_table():
    rows = {}
    with open(os.path.join(GOLDEN, "gaussian_lloyd_max.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            rows[int(parts[0])] = (float(parts[1]), [float(v) for v in parts[2:]])
    return rows


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_codebook_gaussian_limit(bits):
    """Large d: sqrt(d) c -> the textbook Gaussian Lloyd-Max levels (Max 1960)."""
    mse, levels = _max_table()[bits]
    d = 200000
    cb = T.codebook(d, bits)
    pos = math.sqrt(d) * cb.centroids64[len(levels):]
    assert np.max(np.abs(pos - np.array(levels))) < 2e-4
    assert abs(d * cb.distortion - mse) < 2e-4


@pytest.mark.parametrize("d", [128, 1536])
def test_distortion_within_page_bound(d):
    """[ebisuda, 性能サマリー]: within about 2.7x of the information-theoretic
    limit 4^-B (per unit-variance coordinate); the stored table's D*d*4^B lies
    in [1, 2.7]."""
    for bits in (1, 2, 3, 4):
        ratio = d * T.codebook(d, bits).distortion * 4 ** bits
        assert 1.0 <= ratio <= 2.7


def test_distortion_vs_quadrature():
    d, bits = 128, 3
    cb = T.codebook(d, bits)
    f = lambda x: float(T.coord_density(d, np.array([x]))[0])
    e = np.concatenate(([-1.0], cb.boundaries.astype(np.float64), [1.0]))
    D = 0.0
    for i in range(cb.levels):
        ci = float(cb.centroids[i])
        a, b = max(e[i], -0.6), min(e[i + 1], 0.6)
        D += integrate.quad(lambda x: (x - ci) ** 2 * f(x), a, b, limit=200, epsabs=1e-16, epsrel=1e-12)[0]
    assert abs(D - cb.distortion) < 1e-12


def test_stored_tables_are_rounded_midpoints():
    cb = T.codebook(128, 3)
    assert cb.centroids.dtype == np.float32 and cb.boundaries.dtype == np.float32
    mid = 0.5 * (cb.centroids64[:-1] + cb.centroids64[1:])
    assert np.array_equal(cb.boundaries, mid.astype(np.float32))
    assert cb.boundaries[3] == 0.0


# --- quantization -------------------------------------------------------------

@pytest.mark.parametrize("d,bits", [(3, 2), (4, 2), (4, 1)])
def test_quantize_bruteforce_nearest_codeword(d, bits):
    """Per-coordinate thresholding = nearest product codeword (exhaustive over
    all L^d codewords) for the stored centroid table."""
    cb = T.codebook(d, bits)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(2, synth.TAG_ROTATION, d, d))
    X = synth.gaussian(7, (1,), (300, d))
    enc = T.encode(X, Pi, cb)
    L = cb.levels
    grid = np.array(np.meshgrid(*[np.arange(L)] * d, indexing="ij")).reshape(d, -1).T
    words = cb.centroids.astype(np.float64)[grid]
    for i in range(X.shape[0]):
        dist = np.sum((words - enc.y[i]) ** 2, axis=1)
        best = grid[np.argmin(dist)]
        # skip exact ties (measure zero)
        assert np.array_equal(best, enc.idx[i])


@pytest.mark.parametrize("d", [3, 4])
def test_lloyd_threshold_by_grid_search(d):
    """L = 4: one free positive threshold t; with centroids the conditional means,
    a 1-D grid search of the MSE over t finds Lloyd's t_1."""
    cb = T.codebook(d, 2)

    def mse(t):
        e = np.array([-1.0, -t, 0.0, t, 1.0])
        m0 = T.coord_cdf(d, e[1:]) - T.coord_cdf(d, e[:-1])
        m1 = T._first_moment(d, e[:-1], e[1:])
        m2 = T._second_moment(d, e[:-1], e[1:])
        return float(np.sum(m2 - m1 * m1 / m0))

    ts = np.linspace(0.05, 0.95, 9001)
    vals = np.array([mse(t) for t in ts])
    t_best = ts[np.argmin(vals)]
    assert abs(t_best - 0.5 * (cb.centroids64[2] + cb.centroids64[3])) < 2e-4


@pytest.mark.parametrize("bits", [2, 3])
def test_mse_matches_analytic_distortion(bits):
    """Gaussian data: mean over vectors and coordinates of (y - c[idx])^2
    equals the stored table's D within 3 standard errors."""
    d = 128
    Pi, _ = _ctx(d)
    cb = T.codebook(d, bits)
    X = synth.gaussian(0, (0, synth.TAG_KEYS), (4096, d))
    enc = T.encode(X, Pi, cb)
    err = (enc.y - cb.centroids.astype(np.float64)[enc.idx]) ** 2
    per_vec = err.mean(axis=1)
    se = per_vec.std(ddof=1) / math.sqrt(per_vec.size)
    assert abs(per_vec.mean() - cb.distortion) < 3 * se


def test_zero_vector_record_is_zero():
    d = 32
    Pi, S = _ctx(d)
    cb = T.codebook(d, 3)
    X = np.zeros((2, d), np.float32)
    X[1, 3] = 1.0
    enc = T.encode(X, Pi, cb, S)
    assert enc.norm[0] == 0 and enc.rho[0] == 0 and not enc.sigma[0].any() and not enc.idx[0].any()
    packed = T.pack_keys(enc, 3)
    assert not packed["bits"][0].any() and not packed["norms"][0].any()


# --- QJL estimator --------------------------------------------------------------

def _score_one(q, x, Pi, S, cb):
    enc = T.encode(x[None, :], Pi, cb, S)
    q_rot, q_s = T.query_prep(q[None, :], Pi, S)
    return T.scores_from_parts(q_rot, q_s, enc.idx, enc.sigma, enc.norm, enc.rho, cb, S.shape[0])[0, 0], enc


def test_qjl_unbiased_over_sketch_and_rotation():
    """Fixed (q, x); 1000 independent draws of S (rotation fixed), and separately
    of (rotation, S): mean(s - <q,x>) within 3 standard errors of 0."""
    d = 64
    cb = T.codebook(d, 2)
    q = synth.gaussian(1, (21,), (d,)).astype(np.float64)
    x = synth.gaussian(1, (22,), (d,)).astype(np.float64)
    exact = float(q @ x)
    Pi0 = T.rotation_from_gaussian(synth.gaussian_matrix(100, synth.TAG_ROTATION, d, d))
    for vary_rot in (False, True):
        errs = []
        for seed in range(1000):
            Pi = T.rotation_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_ROTATION, d, d)) if vary_rot else Pi0
            S = T.sketch_from_gaussian(synth.gaussian_matrix(5000 + seed, synth.TAG_SKETCH, d, d))
            s, _ = _score_one(q, x, Pi, S, cb)
            errs.append(s - exact)
        errs = np.array(errs)
        se = errs.std(ddof=1) / math.sqrt(errs.size)
        assert abs(errs.mean()) < 3 * se


def test_qjl_variance_closed_form():
    """Rotation fixed, S varies: Var(s) = (n^2 rho^2 / m) ((pi/2)||q||^2 - <q_rot, r_hat>^2)."""
    d = 64
    cb = T.codebook(d, 2)
    q = synth.gaussian(2, (21,), (d,)).astype(np.float64)
    x = synth.gaussian(2, (22,), (d,)).astype(np.float64)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(7, synth.TAG_ROTATION, d, d))
    vals = []
    for seed in range(1000):
        S = T.sketch_from_gaussian(synth.gaussian_matrix(9000 + seed, synth.TAG_SKETCH, d, d))
        s, enc = _score_one(q, x, Pi, S, cb)
        vals.append(s)
    vals = np.array(vals)
    q_rot = Pi.astype(np.float64) @ q
    r = enc.y[0] - cb.centroids.astype(np.float64)[enc.idx[0]]
    rhat = r / np.linalg.norm(r)
    n = np.linalg.norm(x)
    var = (n * n * (r @ r) / d) * (math.pi / 2 * (q_rot @ q_rot) - (q_rot @ rhat) ** 2)
    emp = vals.var(ddof=1)
    assert abs(emp - var) < 3 * math.sqrt(2.0 / (vals.size - 1)) * var


def test_mse_only_keys_bias_is_one_minus_total_distortion():
    """MSE-only keys (stage 1 alone): over random rotations the score's mean is
    (1 - d D) <q, x>, D the codebook's per-coordinate distortion. Closed form:
    the centroid condition gives E[y_j c(y_j)] = E[c(y_j)^2], so
    sum_j E[y_j c_j] = 1 - d D, and the part of Pi q orthogonal to y averages
    out by symmetry. 1000 rotations, within 3 standard errors; the bias itself
    is many standard errors away from 0 (the estimator is not unbiased)."""
    d, bits = 64, 1
    cb = T.codebook(d, bits)
    x = synth.gaussian(3, (22,), (d,)).astype(np.float64)
    q = x + 0.5 * synth.gaussian(3, (21,), (d,)).astype(np.float64)  # correlated: a large <q, x>
    exact = float(q @ x)
    vals = []
    for seed in range(1000):
        Pi = T.rotation_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_ROTATION, d, d))
        enc = T.encode(x[None, :], Pi, cb)
        q_rot = Pi.astype(np.float64) @ q
        vals.append(T.scores_from_parts(q_rot[None, :], None, enc.idx, None, enc.norm, None, cb, d)[0, 0])
    vals = np.array(vals)
    se = vals.std(ddof=1) / math.sqrt(vals.size)
    want = (1.0 - d * cb.distortion) * exact
    assert abs(vals.mean() - want) < 3 * se
    assert abs(vals.mean() - exact) > 10 * se


def test_pure_qjl_keys_unbiased():
    """Pure QJL keys (no codebook bits, residual = the rotated unit vector): the
    score is unbiased over the sketch, mean error within 3 standard errors, and
    rho = ||y|| = 1 (to the fp32 rounding of Pi)."""
    d = 64
    q = synth.gaussian(4, (21,), (d,)).astype(np.float64)
    x = synth.gaussian(4, (22,), (d,)).astype(np.float64)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(11, synth.TAG_ROTATION, d, d))
    errs = []
    for seed in range(1000):
        S = T.sketch_from_gaussian(synth.gaussian_matrix(7000 + seed, synth.TAG_SKETCH, d, d))
        enc = T.encode(x[None, :], Pi, None, S)
        assert abs(enc.rho[0] - 1.0) < 1e-6 and not enc.idx.any()  # Pi is fp32: orthogonal to ~1e-7
        q_rot, q_s = T.query_prep(q[None, :], Pi, S)
        errs.append(T.scores_from_parts(q_rot, q_s, enc.idx, enc.sigma, enc.norm, enc.rho, None, d)[0, 0] - q @ x)
    errs = np.array(errs)
    assert abs(errs.mean()) < 3 * errs.std(ddof=1) / math.sqrt(errs.size)


def test_key_variant_scores_split_the_full_score():
    """The TurboQuant score is the MSE-only score of the same codes plus the QJL
    term of the residual: scores of the three packed formats add up."""
    d = 64
    Pi, S = _ctx(d, seed=5)
    cb = T.codebook(d, 2)
    X = synth.gaussian(5, (1,), (40, d))
    Qv = synth.gaussian(5, (2,), (3, d))
    enc = T.encode(X, Pi, cb, S)
    full = T.scores(Qv, Pi, S, cb, T.pack_keys(enc, 2))
    mse = T.scores(Qv, Pi, S, cb, T.pack_keys(T.encode(X, Pi, cb), 2, qjl=False), qjl=False)
    q_rot, q_s = T.query_prep(Qv, Pi, S)
    corr = T.scores_from_parts(q_rot, q_s, enc.idx, enc.sigma, enc.norm.astype(np.float32),
                               enc.rho.astype(np.float32), None, d)
    assert np.max(np.abs(full - (mse + corr))) < 1e-9 * np.max(np.abs(full))


def test_score_is_inner_product_with_dequantized_key():
    d = 128
    Pi, S = _ctx(d)
    cb = T.codebook(d, 3)
    X = synth.gaussian(0, (1,), (50, d))
    Qv = synth.gaussian(0, (2,), (7, d))
    enc = T.encode(X, Pi, cb, S)
    q_rot, q_s = T.query_prep(Qv, Pi, S)
    s = T.scores_from_parts(q_rot, q_s, enc.idx, enc.sigma, enc.norm, enc.rho, cb, d)
    khat = T.dequantize_keys(Pi, S, cb, enc.idx, enc.sigma, enc.norm, enc.rho)
    assert np.max(np.abs(s - Qv.astype(np.float64) @ khat.T)) < 1e-12 * np.max(np.abs(s)) * d


def test_large_bit_width_limit():
    """With many MSE bits the residual is tiny and s -> <q,x>: |s - <q,x>| stays
    within 4 standard deviations of the closed-form QJL spread for >= 99.9%."""
    d = 64
    cb = T.codebook(d, 7)
    Pi, S = _ctx(d, seed=4)
    X = synth.gaussian(4, (1,), (2000, d)).astype(np.float64)
    Qv = synth.gaussian(4, (2,), (1, d)).astype(np.float64)
    enc = T.encode(X, Pi, cb, S)
    q_rot, q_s = T.query_prep(Qv, Pi, S)
    s = T.scores_from_parts(q_rot, q_s, enc.idx, enc.sigma, enc.norm, enc.rho, cb, d)[0]
    exact = X @ Qv[0]
    R = enc.y - cb.centroids.astype(np.float64)[enc.idx]
    rhat = R / np.linalg.norm(R, axis=1, keepdims=True)
    var = (enc.norm ** 2 * enc.rho ** 2 / d) * (math.pi / 2 * (q_rot[0] @ q_rot[0]) - (rhat @ q_rot[0]) ** 2)
    frac = np.mean(np.abs(s - exact) <= 4 * np.sqrt(var) + 1e-6)
    assert frac >= 0.999
    # a few coordinates fall in the overload region beyond the outer level, so
    # the bound is on the typical error, not the maximum
    assert np.median(np.abs(s - exact)) < 0.05 * np.median(np.abs(exact))


# --- attention ----------------------------------------------------------------

def test_attention_matches_textbook_softmax_and_torch():
    """Oracle decode = softmax(q K_hat^T * scale) V_hat on dense fp64 K_hat,
    V_hat, and = torch's scaled_dot_product_attention (fp64, CPU)."""
    import torch
    d, L, g = 128, 77, 4
    Pi, S = _ctx(d)
    cbk, cbv = T.codebook(d, 3), T.codebook(d, 3)
    K = synth.outlier_kv(0, (1,), synth.TAG_SCALES_K, (L, d))
    V = synth.outlier_kv(0, (2,), synth.TAG_SCALES_V, (L, d))
    Qh = synth.gaussian(0, (3,), (g, d), "bf16")
    ek, ev = T.encode(K, Pi, cbk, S), T.encode(V, Pi, cbv)
    keys, vals = T.pack_keys(ek, 3), T.pack_values(ev, 3)
    scale = 1 / math.sqrt(d)
    o = T.attention_decode(Qh, Pi, S, cbk, cbv, keys, vals, L, scale)
    idx, sig = T.unpack_keys(keys["bits"], d, 3)
    Khat = T.dequantize_keys(Pi, S, cbk, idx, sig, keys["norms"][:, 0], keys["norms"][:, 1])
    Vhat = vals["norms"].astype(np.float64)[:, None] * (cbv.centroids.astype(np.float64)[ev.idx] @ Pi.astype(np.float64))
    lg = Qh.astype(np.float64) @ Khat.T * scale
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ref = p @ Vhat
    assert np.max(np.abs(o - ref)) < 1e-10
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qh.astype(np.float64))[None], torch.from_numpy(Khat)[None].expand(1, L, d).contiguous(),
        torch.from_numpy(Vhat)[None], scale=scale)[0].numpy()
    assert np.max(np.abs(o - t)) < 1e-10


def test_prefill_matches_masked_sdpa():
    """Oracle prefill = torch's scaled_dot_product_attention (fp64, CPU) over the
    dense K_hat, V_hat with a boolean mask that lets query i of n_q see the keys
    t <= L - n_q + i (a lower triangle shifted to the cache's end); without
    causality every query sees all L keys. The last causal query is the decode."""
    import torch
    d, L, g, nq = 128, 53, 2, 9
    Pi, S = _ctx(d)
    cbk, cbv = T.codebook(d, 2), T.codebook(d, 3)
    K = synth.outlier_kv(1, (1,), synth.TAG_SCALES_K, (L, d))
    V = synth.outlier_kv(1, (2,), synth.TAG_SCALES_V, (L, d))
    Q = synth.gaussian(1, (3,), (nq, g, d), "bf16")
    ek, ev = T.encode(K, Pi, cbk, S), T.encode(V, Pi, cbv)
    keys, vals = T.pack_keys(ek, 2), T.pack_values(ev, 3)
    scale = 0.1
    idx, sig = T.unpack_keys(keys["bits"], d, 2)
    Khat = T.dequantize_keys(Pi, S, cbk, idx, sig, keys["norms"][:, 0], keys["norms"][:, 1])
    Vhat = vals["norms"].astype(np.float64)[:, None] * (cbv.centroids.astype(np.float64)[ev.idx] @ Pi.astype(np.float64))
    qt = torch.from_numpy(Q.astype(np.float64)).permute(1, 0, 2).contiguous()      # (g, nq, d)
    kt = torch.from_numpy(Khat)[None].expand(g, L, d).contiguous()
    vt = torch.from_numpy(Vhat)[None].expand(g, L, d).contiguous()
    mask = torch.from_numpy(np.tril(np.ones((nq, L), dtype=bool), k=L - nq))
    for causal in (True, False):
        o = T.attention_prefill(Q, Pi, S, cbk, cbv, keys, vals, L, scale, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask if causal else None,
                                                               scale=scale).permute(1, 0, 2).numpy()
        assert np.max(np.abs(o - ref)) < 1e-10
    o = T.attention_prefill(Q, Pi, S, cbk, cbv, keys, vals, L, scale, True)
    assert np.array_equal(o[-1], T.attention_decode(Q[-1], Pi, S, cbk, cbv, keys, vals, L, scale))
    # a chunk longer than the cache: the first n_q - L positions see nothing
    o = T.attention_prefill(synth.gaussian(1, (4,), (L + 3, g, d), "bf16"), Pi, S, cbk, cbv, keys, vals, L, scale,
                            True)
    assert np.all(o[:3] == 0) and np.all(np.any(o[3:] != 0, axis=2))


def test_split_softmax_merge_equals_single_pass():
    rng = np.random.default_rng(0)
    lg = rng.normal(size=1000) * 4
    v = rng.normal(size=(1000, 8))
    p = np.exp(lg - lg.max())
    ref = (p @ v) / p.sum()
    parts = []
    for c in range(0, 1000, 128):
        x = lg[c:c + 128]
        m = x.max()
        e = np.exp(x - m)
        parts.append((m, e.sum(), e @ v[c:c + 128]))
    M = max(pm for pm, _, _ in parts)
    num = sum(np.exp(pm - M) * a for pm, _, a in parts)
    den = sum(np.exp(pm - M) * l for pm, l, _ in parts)
    assert np.max(np.abs(num / den - ref)) < 1e-12


# --- top-k and records ------------------------------------------------------------

def test_topk_order_and_ties():
    s = np.array([0.5, 2.0, 2.0, -1.0, 3.0, 2.0])
    assert T.topk(s, 4).tolist() == [4, 1, 2, 5]
    rng = np.random.default_rng(1)
    x = rng.normal(size=5000)
    assert np.array_equal(T.topk(x, 10), np.argsort(-x, kind="stable")[:10])


def test_recall_at_k():
    found = np.array([[1, 2, 3], [4, 5, 6]])
    exact = np.array([[3, 2, 9], [7, 8, 9]])
    assert T.recall_at_k(found, exact) == pytest.approx((2 / 3 + 0) / 2)


def test_record_bytes():
    assert T.key_record_bytes(128, 2) == 56      # b = 3 keys
    assert T.key_record_bytes(128, 3) == 72      # b = 4 keys
    assert T.key_record_bytes(1536, 3) == 776    # b = 4 keys at d = 1536
    assert T.value_record_bytes(128, 3) == 52    # 3-bit values
    d = 128
    Pi, S = _ctx(d)
    enc = T.encode(synth.gaussian(0, (1,), (64, d)), Pi, T.codebook(d, 3), S)
    pk = T.pack_keys(enc, 3)
    assert (pk["bits"].nbytes + pk["norms"].nbytes) // 64 == 72
    pv = T.pack_values(enc, 3)
    assert (pv["bits"].nbytes + pv["norms"].nbytes) // 64 == 52
    # key variants: MSE-only (codes and |k|) and pure QJL (signs and both norms)
    assert T.key_record_bytes(128, 3, qjl=False) == 52
    assert T.key_record_bytes(128, 0) == 24
    pm = T.pack_keys(T.encode(synth.gaussian(0, (1,), (64, d)), Pi, T.codebook(d, 3)), 3, qjl=False)
    assert (pm["bits"].nbytes + pm["norms"].nbytes) // 64 == 52
    pq = T.pack_keys(T.encode(synth.gaussian(0, (1,), (64, d)), Pi, None, S), 0)
    assert (pq["bits"].nbytes + pq["norms"].nbytes) // 64 == 24


def test_compact_norms_rounding_and_saturation():
    """Compact norms follow IEEE half precision: exactly representable values
    keep their bit patterns (1.0 = 0x3C00, 0.5 = 0x3800, 2.5 = 0x4100, the
    largest finite 65504 = 0x7BFF), ties go to the even neighbour (1 + 2^-11
    -> 1.0, 1 + 3*2^-11 -> 1 + 2^-9), larger values saturate at 65504, and the
    relative error is at most 2^-11 over the normal range."""
    x = np.array([1.0, 0.5, 2.5, 65504.0, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 65519.0, 7e4, 1e9, 0.0])
    h = T.stored_norms(x, True)
    assert h.dtype == np.float16
    assert h[:4].view(np.uint16).tolist() == [0x3C00, 0x3800, 0x4100, 0x7BFF]
    assert float(h[4]) == 1.0 and float(h[5]) == 1 + 2 ** -9
    assert np.all(h[6:9].view(np.uint16) == 0x7BFF) and float(h[9]) == 0.0
    v = np.exp(np.random.default_rng(5).uniform(np.log(2.0 ** -14), np.log(65504.0), 100000))
    assert np.max(np.abs(T.stored_norms(v, True).astype(np.float64) / v - 1)) <= 2.0 ** -11
    assert T.stored_norms(x, False).dtype == np.float32


def test_compact_norm_scores_stay_within_the_rounding_bound():
    """With compact norms every score moves by at most the fp16 rounding of
    ||k|| and ||r|| acting on its two terms: |s16 - s32| <= 2^-11 n |a| +
    (2^-10 + 2^-22) n |b| for s = n (a + b) (a the stage-1 term, b the QJL term);
    record bytes shrink by 2 per norm."""
    d = 128
    Pi, S = _ctx(d)
    cb = T.codebook(d, 3)
    K = synth.outlier_kv(6, (1,), synth.TAG_SCALES_K, (500, d))
    Q = synth.gaussian(6, (2,), (8, d))
    enc = T.encode(K, Pi, cb, S)
    k32, k16 = T.pack_keys(enc, 3), T.pack_keys(enc, 3, norm_f16=True)
    assert k16["norms"].dtype == np.float16
    s32, s16 = T.scores(Q, Pi, S, cb, k32), T.scores(Q, Pi, S, cb, k16)
    idx, sig = T.unpack_keys(k32["bits"], d, 3)
    q_rot, q_s = T.query_prep(Q, Pi, S)
    ones = np.ones(500)
    a = T.scores_from_parts(q_rot, q_s, idx, None, ones, None, cb, d)
    b = T.scores_from_parts(q_rot, q_s, idx, sig, ones, k32["norms"][:, 1], None, d)
    n = k32["norms"][:, 0].astype(np.float64)[None, :]
    assert np.all(np.abs(s16 - s32) <= 2.0 ** -11 * n * np.abs(a) + (2.0 ** -10 + 2.0 ** -22) * n * np.abs(b) + 1e-12)
    assert T.key_record_bytes(d, 3, norm_f16=True) == 68 and T.value_record_bytes(d, 3, norm_f16=True) == 50
    assert T.key_record_bytes(d, 3, qjl=False, norm_f16=True) == 50 and T.key_record_bytes(d, 0, norm_f16=True) == 20
    pv = T.pack_values(T.encode(K, Pi, cb), 3, norm_f16=True)
    assert pv["norms"].nbytes == 2 * 500 and (k16["bits"].nbytes + k16["norms"].nbytes) == 68 * 500


# --- packing format ---------------------------------------------------------------

def _golden_words(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            rows.append(line.split())
    return rows


def test_pack_keys_golden():
    d = 32
    idx = (np.arange(d) % 8)[None, :]
    sig = (np.arange(d) % 3 == 0)[None, :]
    enc = T.Encoded(idx, sig, np.ones(1), np.ones(1), None, None)
    words = T.pack_keys(enc, 3)["bits"].reshape(-1)
    exp = [int(w, 16) for w in _golden_words("packing_keys.txt")[0][1:]]
    assert words.tolist() == exp
    i2, s2 = T.unpack_keys(T.pack_keys(enc, 3)["bits"], d, 3)
    assert np.array_equal(i2, idx) and np.array_equal(s2, sig)


def test_pack_key_variants_golden():
    """MSE-only and pure QJL key records are the TurboQuant record with the sign
    word, or the code words, left out (same golden words)."""
    d = 32
    idx = (np.arange(d) % 8)[None, :]
    sig = (np.arange(d) % 3 == 0)[None, :]
    exp = [int(w, 16) for w in _golden_words("packing_keys.txt")[0][1:]]
    mse = T.pack_keys(T.Encoded(idx, None, np.ones(1), None, None, None), 3, qjl=False)
    assert mse["bits"].reshape(-1).tolist() == exp[:3] and mse["norms"].shape == (1, 1)
    qjl = T.pack_keys(T.Encoded(np.zeros_like(idx), sig, np.ones(1), np.ones(1), None, None), 0)
    assert qjl["bits"].reshape(-1).tolist() == exp[3:] and qjl["norms"].shape == (1, 2)
    i2, s2 = T.unpack_keys(mse["bits"], d, 3, qjl=False)
    assert np.array_equal(i2, idx) and s2 is None
    i3, s3 = T.unpack_keys(qjl["bits"], d, 0)
    assert not i3.any() and np.array_equal(s3, sig)


def test_pack_values_golden():
    d, n = 32, 34
    idx = (np.arange(n)[:, None] + np.arange(d)[None, :]) % 8
    enc = T.Encoded(idx, None, np.ones(n), None, None, None)
    words = T.pack_values(enc, 3)["bits"]
    assert words.shape == (2, d, 3)
    for row in _golden_words("packing_values.txt"):
        blk, j = int(row[0]), int(row[1])
        assert words[blk, j].tolist() == [int(w, 16) for w in row[2:]]
    assert np.array_equal(T.unpack_values(words, d, 3, n), idx)
