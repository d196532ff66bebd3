"""Comparison rules between GPU results and the oracle (test helpers).

Packed codes and sign bits: bit-exact, except at most 1e-4 of coordinates
whose oracle value lies within 1e-5 of a decision boundary (codes: the fp64
rotated coordinate y against the stored boundaries; signs: the fp64 sketch
value z against 0). A vector with an excused code flip has a different
residual (the cascade): its sign bits and ||r|| are compared against the
oracle's stage 2 re-derived from the GPU's own codes (fp64 r = y - c[idx_gpu],
z = S r), under the same band and norm tolerance.
Scores: |ds| <= 1e-3 |s| or |ds| <= 1e-6 ||q|| ||x||. Attention: 2e-3 max-abs.
"""
import numpy as np

from oracle import turboquant as T

BAND = 1e-5
MAX_FRAC = 1e-4


def boundary_distance(y: np.ndarray, cb) -> np.ndarray:
    b = cb.boundaries.astype(np.float64)
    return np.min(np.abs(y[..., None] - b), axis=-1)


def check_codes(g_idx, enc, cb, what="codes"):
    """Returns the boolean (n,) mask of vectors with an excused code flip."""
    flips = g_idx != enc.idx
    nflip = int(flips.sum())
    if nflip:
        dist = boundary_distance(enc.y, cb)
        bad = flips & ~(dist < BAND)
        assert not bad.any(), f"{what}: {int(bad.sum())} code mismatches outside the boundary band"
        assert np.all(np.abs(g_idx[flips] - enc.idx[flips]) == 1), f"{what}: non-adjacent code flip"
    assert nflip <= MAX_FRAC * g_idx.size, f"{what}: {nflip} excused flips > {MAX_FRAC} of {g_idx.size}"
    return flips.any(axis=1)


def norms_match(g, ref, rel, absol, f16=False):
    """Stored norms against the oracle's exact ones: within rel * ref + absol
    (fp32), or (compact fp16 norms) the nearest-even fp16 of a value within
    that band: between the roundings of its two ends (rounding is monotonic)."""
    g = np.asarray(g).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not f16:
        return bool(np.all(np.abs(g - ref) <= rel * ref + absol))
    lo = T.stored_norms(np.maximum(ref * (1 - rel) - absol, 0.0), True).astype(np.float64)
    hi = T.stored_norms(ref * (1 + rel) + absol, True).astype(np.float64)
    return bool(np.all((g >= lo) & (g <= hi)))


def check_key_records(words, norms, enc, cb, bits, d, qjl=True, norm_f16=False):
    """Key records of any variant: MSE-only (qjl False: codes and ||k||) and
    pure QJL (bits 0, cb None: signs and both norms) included; norm_f16:
    compact records with fp16 norms."""
    norms = np.asarray(norms).reshape(words.shape[0], 1 + int(qjl))
    g_idx, g_sig = T.unpack_keys(words, d, bits, qjl)
    if bits > 0:
        cascade = check_codes(g_idx, enc, cb, "key codes")
    else:
        assert not g_idx.any()
        cascade = np.zeros(words.shape[0], dtype=bool)
    nsflip = 0
    if qjl:
        # the oracle's stage 2; for cascade vectors, re-derived from the GPU's codes
        ref_sig, ref_z, ref_rho = enc.sigma.copy(), enc.z.copy(), enc.rho.copy()
        if cascade.any():
            assert enc.S is not None, "cascade vectors need the sketch matrix (encode with S)"
            rows = np.nonzero(cascade)[0]
            rho_c, z_c, sig_c = T.qjl_stage(enc.y[rows], g_idx[rows], cb, enc.S, enc.norm[rows] > 0)
            ref_sig[rows], ref_z[rows], ref_rho[rows] = sig_c, z_c, rho_c
        sflip = g_sig != ref_sig
        if sflip.any():
            bad = sflip & ~(np.abs(ref_z) < BAND)
            assert not bad.any(), f"sign mismatches outside the band: {int(bad.sum())}"
        assert sflip.sum() <= MAX_FRAC * g_sig.size
        nsflip = int(sflip.sum())
    assert norms_match(norms[:, 0], enc.norm, 2e-6, 1e-30, norm_f16), "||k|| mismatch"
    if qjl:
        assert norms_match(norms[:, 1], ref_rho, 2e-5, 1e-7, norm_f16), "||r|| mismatch"
    return int(cascade.sum()), nsflip


def check_value_records(words, norms, enc, cb, bits, d, n, norm_f16=False):
    g_idx = T.unpack_values(words, d, bits, n)
    check_codes(g_idx, enc, cb, "value codes")
    assert norms_match(norms[:n], enc.norm, 2e-6, 1e-30, norm_f16), "||v|| mismatch"


def check_scores(s_gpu, s_ref, qnorm, xnorm):
    tol = np.maximum(1e-3 * np.abs(s_ref), 1e-6 * np.outer(qnorm, xnorm))
    err = np.abs(s_gpu - s_ref)
    assert np.all(err <= tol), f"score mismatch: worst excess {np.max(err - tol)}"


def check_topk(idx_gpu, val_gpu, s_ref, k, qnorm, xnorm):
    """Top-k sets equal up to near-ties; reported values match the oracle's."""
    for q in range(s_ref.shape[0]):
        ref = T.topk(s_ref[q], k)
        got = idx_gpu[q][:k]
        tol = 1e-6 * qnorm[q] * np.max(xnorm) + 1e-3 * abs(s_ref[q][ref[-1]])
        kth = s_ref[q][ref[-1]]
        for t in set(got.tolist()) ^ set(ref.tolist()):
            assert abs(s_ref[q][t] - kth) <= tol, f"query {q}: top-k differs beyond a near-tie"
        assert np.all(np.abs(val_gpu[q][:k] - s_ref[q][got]) <= np.maximum(1e-3 * np.abs(s_ref[q][got]), tol))
        assert np.all(np.diff(val_gpu[q][:k]) <= 0)
