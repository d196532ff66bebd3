"""Pins of the PolarQuant oracle (oracle/polarquant.py) against what the
mathematics fixes: the polar transform is invertible and keeps the norm, the
angle laws integrate to one and match Monte-Carlo angles of random
directions, the 1-bit level-2 codebook has a closed form, the level-1
codebook is the uniform grid, Lloyd's fixed point holds, codes are the
nearest stored centroid, rebuilt vectors converge to the input as bits grow,
and the packed layout matches a hand-built fixture."""
import math

import numpy as np
import pytest
from scipy import integrate, stats

import synth
from oracle import polarquant as PQ
from oracle import turboquant as T


def test_polar_transform_inverts_and_keeps_the_norm():
    Y = synth.gaussian(61, (1,), (50, 128)).astype(np.float64)
    r, levels = PQ.polar_transform(Y)
    assert len(levels) == 7 and [a.shape[1] for a in levels] == [64, 32, 16, 8, 4, 2, 1]
    assert np.allclose(r, np.linalg.norm(Y, axis=1), rtol=1e-13)
    assert np.max(np.abs(PQ.polar_inverse(r, levels) - Y)) < 1e-12
    assert np.all(levels[0] >= -math.pi) and np.all(levels[0] <= math.pi)
    for a in levels[1:]:
        assert np.all(a >= 0) and np.all(a <= math.pi / 2)
    # a 2-d vector: the textbook polar coordinates
    r2, l2 = PQ.polar_transform(np.array([[3.0, 4.0]]))
    assert r2[0] == 5.0 and abs(l2[0][0, 0] - math.atan2(4, 3)) < 1e-15


@pytest.mark.parametrize("level", [1, 2, 3, 5, 7])
def test_angle_laws_normalized_and_match_random_directions(level):
    lo, hi = (-math.pi, math.pi) if level == 1 else (0.0, math.pi / 2)
    mass, _ = integrate.quad(lambda t: float(PQ.angle_density(level, t)), lo, hi, limit=200)
    assert abs(mass - 1) < 1e-10
    # angles of Gaussian vectors (any rotation-invariant law): KS against the CDF
    Y = synth.gaussian(62, (level,), (4000, 128)).astype(np.float64)
    _, levels = PQ.polar_transform(Y)
    sample = levels[level - 1].ravel()[:20000]
    ks = stats.kstest(sample, lambda x: PQ.angle_cdf(level, x))
    assert ks.pvalue > 1e-3
    if level == 2:  # closed form: f = sin(2 psi), F = sin^2(psi)
        t = np.linspace(0, math.pi / 2, 9)
        assert np.allclose(PQ.angle_density(2, t), np.sin(2 * t), atol=1e-14)
        assert np.allclose(PQ.angle_cdf(2, t), np.sin(t) ** 2, atol=1e-14)


def test_angle_codebook_closed_forms():
    # level 2, 1 bit: split at pi/4, centroids E[psi | psi < pi/4] = 1/2 and pi/2 - 1/2
    c = PQ.lloyd_max_angle(2, 1)
    assert np.allclose(c, [0.5, math.pi / 2 - 0.5], atol=1e-11)
    # level 1: the uniform grid, cells from -pi
    cb = PQ.angle_codebook(1, 3)
    assert np.allclose(cb.centroids64, -math.pi + (np.arange(8) + 0.5) * math.pi / 4)
    assert np.allclose(cb.boundaries, -math.pi + np.arange(1, 8) * math.pi / 4, atol=1e-6)


@pytest.mark.parametrize("level,bits", [(2, 3), (4, 2), (7, 3)])
def test_lloyd_fixed_point_and_symmetry(level, bits):
    c = PQ.lloyd_max_angle(level, bits)
    assert np.all(np.diff(c) > 0)
    assert np.allclose(c + c[::-1], math.pi / 2, atol=1e-12)
    e = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [math.pi / 2]))
    for i in range(len(c)):
        m0, _ = integrate.quad(lambda t: float(PQ.angle_density(level, t)), e[i], e[i + 1], limit=200)
        m1, _ = integrate.quad(lambda t: t * float(PQ.angle_density(level, t)), e[i], e[i + 1], limit=200)
        assert abs(m1 / m0 - c[i]) < 1e-9


def test_codes_are_the_nearest_stored_centroid():
    pcb = PQ.polar_codebooks(128, 4, 3)
    rng = np.random.default_rng(63)
    for lv in (2, 5):
        cb = pcb.levels[lv - 1]
        psi = rng.uniform(0, math.pi / 2, 5000)
        k = PQ.angle_codes(psi, cb)
        brute = np.argmin(np.abs(psi[:, None] - cb.centroids64[None, :]), axis=1)
        near = np.min(np.abs(psi[:, None] - cb.boundaries.astype(np.float64)[None, :]), axis=1) < 1e-6
        assert np.all((k == brute) | near)


def test_rebuild_converges_and_scores_equal_dequantized_dot():
    """Reconstruction error falls with the bit widths (a monotone invariant);
    the rotated-domain score equals <q, Pi^T y_hat> computed in the original
    domain."""
    d = 128
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, d, d))
    X = synth.gaussian(64, (1,), (200, d)).astype(np.float64)
    errs = []
    for b1, b2 in ((2, 1), (3, 2), (4, 3), (4, 4)):
        pcb = PQ.polar_codebooks(d, b1, b2)
        enc = PQ.polar_encode(X, Pi, pcb)
        Yh = PQ.polar_rebuild(enc.codes, enc.norm, pcb)
        Y = X @ Pi.astype(np.float64).T
        errs.append(np.mean(np.sum((Yh - Y) ** 2, axis=1) / np.sum(Y ** 2, axis=1)))
    assert all(errs[i + 1] < errs[i] for i in range(3)) and errs[-1] < 0.05
    pcb = PQ.polar_codebooks(d, 4, 3)
    keys = PQ.pack_polar(PQ.polar_encode(X, Pi, pcb), pcb)
    Q = synth.gaussian(64, (2,), (5, d)).astype(np.float64)
    s = PQ.polar_scores(Q, Pi, pcb, keys)
    Kh = PQ.polar_rebuild(PQ.unpack_polar(keys["bits"], pcb), keys["norms"], pcb) @ Pi.astype(np.float64)
    assert np.max(np.abs(s - Q @ Kh.T)) < 1e-9 * np.max(np.abs(s))


def test_record_layout_and_bytes():
    """d = 8, b1 = 4, b2 = 3: four level-1 codes in one word (4 bits each),
    three higher codes (level 2 nodes 0, 1, then level 3) in one word at bits
    0, 3, 6; 60 bytes per d = 128 record at (4, 3): 4.27x against fp16."""
    pcb = PQ.polar_codebooks(8, 4, 3)
    enc = PQ.PolarEncoded([np.array([[1, 15, 0, 9]]), np.array([[5, 2]]), np.array([[7]])], np.array([2.0]), [])
    rec = PQ.pack_polar(enc, pcb)
    assert rec["bits"].tolist() == [[0x90F1, 5 | (2 << 3) | (7 << 6)]]
    back = PQ.unpack_polar(rec["bits"], pcb)
    assert [c.tolist() for c in back] == [[[1, 15, 0, 9]], [[5, 2]], [[7]]]
    assert PQ.polar_record_bytes(128, 4, 3) == 60 and abs(256 / 60 - 4.27) < 0.01
    # codes crossing a word boundary (b2 = 3: code 10 spans bits 30..32)
    pcb = PQ.polar_codebooks(32, 4, 3)
    codes = [np.arange(16)[None, :] % 16, (np.arange(8)[None, :] * 3) % 8, np.array([[1, 6, 3, 5]]),
             np.array([[2, 7]]), np.array([[4]])]
    rec = PQ.pack_polar(PQ.PolarEncoded(codes, np.array([1.0]), []), pcb)
    assert [c.tolist() for c in PQ.unpack_polar(rec["bits"], pcb)] == [c.tolist() for c in codes]


def _polar_setup(d, L, seed):
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_ROTATION, d, d))
    pcb = PQ.polar_codebooks(d, 4, 3)
    cbv = T.codebook(d, 3)
    K = synth.outlier_kv(seed, (1,), synth.TAG_SCALES_K, (L, d))
    V = synth.outlier_kv(seed, (2,), synth.TAG_SCALES_V, (L, d))
    keys = PQ.pack_polar(PQ.polar_encode(K, Pi, pcb), pcb)
    ev = T.encode(V, Pi, cbv)
    return Pi, pcb, cbv, keys, T.pack_values(ev, 3), ev


def test_polar_attention_matches_sdpa_on_rebuilt_keys():
    """Oracle PolarQuant decode = softmax(q K_hat^T * scale) V_hat on the dense
    fp64 rebuilt keys K_hat = Pi^T y_hat (rows: y_hat @ Pi) and values
    V_hat = ||v|| Pi^T c_v[idx], by numpy and by torch's
    scaled_dot_product_attention (fp64, CPU); records past seq_len (here
    garbage) are not read ([gemilab] Attention機構)."""
    import torch
    d, L, n, g = 128, 96, 70, 4
    Pi, pcb, cbv, keys, vals, ev = _polar_setup(d, L, 0)
    # records past the sequence hold garbage that must not matter
    keys["bits"][n:] = np.uint32(0xDEADBEEF)
    keys["norms"][n:] = np.float32(1e30)
    Qh = synth.gaussian(0, (3,), (g, d), "bf16").astype(np.float64)
    scale = 1 / math.sqrt(d)
    o = PQ.polar_attention_decode(Qh, Pi, pcb, cbv, keys, vals, n, scale, T.unpack_values)
    P64 = Pi.astype(np.float64)
    Yh = PQ.polar_rebuild(PQ.unpack_polar(keys["bits"][:n], pcb), keys["norms"][:n], pcb)
    Khat = Yh @ P64
    Vhat = vals["norms"][:n].astype(np.float64)[:, None] * (cbv.centroids.astype(np.float64)[ev.idx[:n]] @ P64)
    lg = Qh @ Khat.T * scale
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.max(np.abs(o - p @ Vhat)) < 1e-10
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qh)[None], torch.from_numpy(Khat)[None], torch.from_numpy(Vhat)[None], scale=scale)[0].numpy()
    assert np.max(np.abs(o - t)) < 1e-10
    # a swapped rotation (Pi in place of Pi^T on the way back) changes the output
    wrong = (p @ (vals["norms"][:n].astype(np.float64)[:, None] * cbv.centroids.astype(np.float64)[ev.idx[:n]])) @ P64.T
    assert np.max(np.abs(o - wrong)) > 1e-3


def test_polar_attention_bruteforce_tiny_d():
    """d = 4 by hand: level-1 angles t0, t1 of the pairs, level-2 angle f of
    the two radii; y_hat = ||x|| (cos f cos t0, cos f sin t0, sin f cos t1,
    sin f sin t1) from the stored cos/sin tables, k_hat = Pi^T y_hat, and a
    per-token softmax loop in plain Python."""
    d, L, n = 4, 9, 7
    Pi, pcb, cbv, keys, vals, ev = _polar_setup(d, L, 5)
    Qh = synth.gaussian(5, (3,), (2, d)).astype(np.float64)
    scale = 0.5
    o = PQ.polar_attention_decode(Qh, Pi, pcb, cbv, keys, vals, n, scale, T.unpack_values)
    c1, c2 = PQ.unpack_polar(keys["bits"], pcb)
    l1, l2 = pcb.levels[0], pcb.levels[1]
    P64 = Pi.astype(np.float64)
    for h in range(Qh.shape[0]):
        logits, vrows = [], []
        for t in range(n):
            r = float(keys["norms"][t])
            f = int(c2[t, 0])
            r0, r1 = r * float(l2.cos[f]), r * float(l2.sin[f])
            a0, a1 = int(c1[t, 0]), int(c1[t, 1])
            y = [r0 * float(l1.cos[a0]), r0 * float(l1.sin[a0]), r1 * float(l1.cos[a1]), r1 * float(l1.sin[a1])]
            k = [sum(P64[i][j] * y[i] for i in range(d)) for j in range(d)]
            logits.append(scale * sum(Qh[h][j] * k[j] for j in range(d)))
            cv = [float(vals["norms"][t]) * float(cbv.centroids[ev.idx[t][i]]) for i in range(d)]
            vrows.append([sum(P64[i][j] * cv[i] for i in range(d)) for j in range(d)])
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        z = sum(w)
        ref = [sum(w[t] * vrows[t][j] for t in range(n)) / z for j in range(d)]
        assert np.max(np.abs(o[h] - np.array(ref))) < 1e-12
