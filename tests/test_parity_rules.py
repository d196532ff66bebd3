"""CPU tests of the GPU-vs-oracle comparison rules in tests/parity.py.

The rules excuse a code decided on the other side of a decision boundary only
within 1e-5 of it; such a flip changes the residual, so that vector's sign bits
and ||r|| are compared against the oracle's stage 2 re-derived from the other
side's codes. Simulated "GPU" records are built on the CPU from the oracle's
own functions, with one planted deviation at a time, and the rules must accept
the faithful records and reject each planted mistake."""
import numpy as np
import pytest

import synth
from oracle import turboquant as T
from tests import parity as P

D, B = 128, 3


def _setup():
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(0, synth.TAG_ROTATION, D, D))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(0, synth.TAG_SKETCH, D, D))
    cb = T.codebook(D, B)
    # vector 0: rotated coordinate 5 placed 3e-7 above boundary 4 (x = Pi^T y)
    rng = synth.rng(7, 1)
    y = rng.standard_normal(D)
    y /= np.linalg.norm(y)
    y[5] = float(cb.boundaries[4]) + 3e-7
    rest = np.delete(np.arange(D), 5)
    y[rest] *= np.sqrt(1.0 - y[5] ** 2) / np.linalg.norm(y[rest])
    X = np.vstack([y @ Pi.astype(np.float64), rng.standard_normal((100, D))])  # one flip <= 1e-4 of the codes
    enc = T.encode(X, Pi, cb, S)
    assert abs(enc.y[0, 5] - cb.boundaries[4]) < 1e-5 and enc.idx[0, 5] == 5
    return Pi, S, cb, X, enc


def _gpu_like(enc, cb, S, flip_code=True):
    """Records as a faithful encoder that decided coordinate (0, 5) in the
    lower cell would write them: its codes, then stage 2 from those codes."""
    idx = enc.idx.copy()
    if flip_code:
        idx[0, 5] -= 1
    rho, z, sig = T.qjl_stage(enc.y, idx, cb, S, enc.norm > 0)
    rec = T.pack_keys(T.Encoded(idx, sig, enc.norm, rho, enc.y, z), B)
    return rec["bits"].reshape(len(idx), -1), rec["norms"], sig, z


def test_faithful_records_pass_with_and_without_a_flip():
    Pi, S, cb, X, enc = _setup()
    for flip in (False, True):
        words, norms, _, _ = _gpu_like(enc, cb, S, flip)
        ncas, _ = P.check_key_records(words, norms, enc, cb, B, D)
        assert ncas == int(flip)


def test_cascade_vector_signs_are_checked():
    """A sign bit wrong beyond the band on the vector with the excused flip is
    caught (before the re-derivation such vectors' signs went unchecked)."""
    Pi, S, cb, X, enc = _setup()
    words, norms, sig, z = _gpu_like(enc, cb, S)
    i = int(np.argmax(np.abs(z[0])))  # the sign farthest from the band
    sig2 = sig.copy()
    sig2[0, i] = ~sig2[0, i]
    idx = T.unpack_keys(words, D, B)[0]
    bad = T.pack_keys(T.Encoded(idx, sig2, enc.norm, norms[:, 1].astype(np.float64), None, None), B)
    with pytest.raises(AssertionError, match="sign"):
        P.check_key_records(bad["bits"].reshape(len(idx), -1), norms, enc, cb, B, D)


def test_cascade_vector_with_the_oracles_signs_fails():
    """An encoder that flipped the code but kept the residual of the other cell
    (the oracle's signs and ||r||) does not match the re-derived stage 2."""
    Pi, S, cb, X, enc = _setup()
    idx = enc.idx.copy()
    idx[0, 5] -= 1
    words = T.pack_keys(T.Encoded(idx, enc.sigma, enc.norm, enc.rho, None, None), B)["bits"].reshape(len(idx), -1)
    norms = np.stack([enc.norm, enc.rho], axis=1).astype(np.float32)
    with pytest.raises(AssertionError):
        P.check_key_records(words, norms, enc, cb, B, D)


def test_cascade_vector_residual_norm_is_checked():
    Pi, S, cb, X, enc = _setup()
    words, norms, _, _ = _gpu_like(enc, cb, S)
    norms = norms.copy()
    norms[0, 1] *= 1.001
    with pytest.raises(AssertionError, match=r"\|\|r\|\|"):
        P.check_key_records(words, norms, enc, cb, B, D)


def test_flip_outside_the_band_fails():
    Pi, S, cb, X, enc = _setup()
    idx = enc.idx.copy()
    far = int(np.argmax(P.boundary_distance(enc.y[1], cb)))
    idx[1, far] = idx[1, far] + (1 if idx[1, far] < 7 else -1)
    rho, z, sig = T.qjl_stage(enc.y, idx, cb, S, enc.norm > 0)
    rec = T.pack_keys(T.Encoded(idx, sig, enc.norm, rho, None, None), B)
    with pytest.raises(AssertionError, match="outside the boundary band"):
        P.check_key_records(rec["bits"].reshape(len(idx), -1), rec["norms"], enc, cb, B, D)
