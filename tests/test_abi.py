"""CPU tests of the C-ABI library: it loads, exports every symbol include/tq.h
declares, its host-only setup matches the oracle, and argument validation
returns status codes before touching a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import turboquant as T

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

tq = pytest.importorskip("kv_cache_vector_turboquant_amd", reason="libtq.so not built")


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert "tq_quantize_kv" in names and "tq_attention_decode" in names
    lib = tq.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(tq.EXPORTED_SYMBOLS) == names


@pytest.mark.parametrize("d,bits", [(3, 1), (3, 2), (64, 3), (128, 1), (128, 2), (128, 3), (128, 4), (1536, 3),
                                    (1536, 4)])
def test_codebook_matches_oracle(d, bits):
    lib_cb = tq.codebook_build(d, bits)
    o = T.codebook(d, bits)
    # independent implementations of the same fixed point agree after fp32 rounding
    assert np.array_equal(lib_cb.centroids, o.centroids)
    assert np.array_equal(lib_cb.boundaries, o.boundaries)
    assert abs(lib_cb.distortion - o.distortion) <= 1e-9 * o.distortion


@pytest.mark.parametrize("d,bits", [(128, 1), (128, 2), (128, 3), (128, 4)])
def test_walsh_coefficients_reproduce_table(d, bits):
    """The odd Walsh expansion the kernels use: c[idx] = sum_S w_S prod_{p in S}(2 b_p - 1)."""
    cb = tq.codebook_build(d, bits)
    L = 1 << bits
    subsets = sorted([s for s in range(1, L) if bin(s).count("1") % 2 == 1], key=lambda s: (bin(s).count("1"), s))
    for idx in range(L):
        val = 0.0
        for w, S in zip(cb.walsh.astype(np.float64), subsets):
            chi = 1.0
            for p in range(bits):
                if S >> p & 1:
                    chi *= 1.0 if (idx >> p) & 1 else -1.0
            val += w * chi
        assert abs(val - cb.centroids[idx]) <= 2e-7 * abs(cb.centroids[idx])


@pytest.mark.parametrize("d", [32, 128, 1536])
def test_rotation_matches_oracle(d):
    G = synth.gaussian_matrix(0, synth.TAG_ROTATION, d, d)
    lib_pi = tq.rotation_build(G)
    o_pi = T.rotation_from_gaussian(G)
    ulp = np.abs(lib_pi.view(np.int32).astype(np.int64) - o_pi.view(np.int32))
    assert ulp.max() <= 1
    assert np.count_nonzero(ulp) <= 1e-5 * d * d + 1
    assert np.max(np.abs(lib_pi.astype(np.float64).T @ lib_pi.astype(np.float64) - np.eye(d))) <= 1e-5


@pytest.mark.parametrize("seed,stream,rows,cols", [(0, 1, 128, 128), (0, 2, 128, 128), (12345, 1, 64, 96),
                                                    (2 ** 63 + 5, 2, 1536, 1536)])
def test_seeded_gaussian_matches_oracle(seed, stream, rows, cols):
    """The library's counter-based Gaussian draws and the oracle's, two
    independent implementations of one published definition, agree bitwise in
    fp64 or (libm ulp differences) within 1 fp32 ulp after rounding."""
    lib_g = tq.gaussian_matrix(seed, stream, rows, cols)
    o_g = T.seeded_gaussian(seed, stream, rows, cols)
    same = lib_g == o_g
    ulp = np.abs(lib_g.astype(np.float32).view(np.int32).astype(np.int64) - o_g.astype(np.float32).view(np.int32))
    assert ulp.max() <= 1
    assert np.mean(same) > 0.99, f"bitwise fp64 agreement {np.mean(same):.4f}"


@pytest.mark.parametrize("d", [128, 1536])
def test_seeded_rotation_matches_oracle(d):
    """Pi and S of a context built from a seed alone (host part of
    tq_ctx_create_seeded) against the oracle's rotation and sketch of its own
    draws for the same seed. The two QRs (Householder here, LAPACK there) of
    draws that differ in the last fp64 bit of a few entries agree within 1 fp32
    ulp except a few entries in 10^5, which stay within 2^-24 absolute (a few
    ulp of a small entry); Pi is orthogonal to 1e-5."""
    for seed in (0, 7):
        g = tq.gaussian_matrix(seed, tq.TQ_STREAM_ROTATION, d, d)
        lib_pi = tq.rotation_build(g)
        o_pi = T.rotation_from_gaussian(T.seeded_gaussian(seed, T.STREAM_ROTATION, d, d))
        ulp = np.abs(lib_pi.view(np.int32).astype(np.int64) - o_pi.view(np.int32))
        assert np.count_nonzero(ulp > 1) <= 1e-5 * d * d
        assert np.max(np.abs(lib_pi.astype(np.float64) - o_pi)) <= 2.0 ** -24
        lib_s = tq.gaussian_matrix(seed, tq.TQ_STREAM_SKETCH, d, d).astype(np.float32)
        o_s = T.sketch_from_gaussian(T.seeded_gaussian(seed, T.STREAM_SKETCH, d, d))
        assert np.abs(lib_s.view(np.int32).astype(np.int64) - o_s.view(np.int32)).max() <= 1
    assert np.max(np.abs(lib_pi.astype(np.float64).T @ lib_pi.astype(np.float64) - np.eye(d))) <= 1e-5


def test_format_version():
    assert tq.format_version() == tq.FORMAT_VERSION == 1
    assert "#define TQ_FORMAT_VERSION 1" in open(os.path.join(ROOT, "include", "tq.h")).read()


def test_host_errors():
    lib = tq.lib()
    cb = tq.CCodebook()
    assert lib.tq_codebook_build(2, 3, ctypes.byref(cb)) == tq.TQ_ERR_UNSUPPORTED
    assert "d must be" in tq.last_error()
    assert lib.tq_codebook_build(128, 5, ctypes.byref(cb)) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_codebook_build(128, 0, ctypes.byref(cb)) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_codebook_build(128, 3, None) == tq.TQ_ERR_ARG
    out = np.zeros(4, np.float32)
    assert lib.tq_rotation_build(2, None, out.ctypes.data) == tq.TQ_ERR_ARG
    g = np.zeros((8, 8))
    assert lib.tq_rotation_build(1, g.ctypes.data, out.ctypes.data) == tq.TQ_ERR_UNSUPPORTED
    with pytest.raises(tq.TQError):
        tq.codebook_build(128, 9)


def test_hot_entry_points_reject_null_context():
    lib = tq.lib()
    p = tq.CPacked(None, None, 0, 3, 1)
    assert lib.tq_quantize_kv(None, None, 0, 1, 1, 128, 128, ctypes.byref(p), 0, 0, None, 0, None) == tq.TQ_ERR_ARG
    c = tq.CCache()
    assert lib.tq_append_token(None, ctypes.byref(c), None, None, 0, None) == tq.TQ_ERR_ARG
    assert lib.tq_cache_write(None, ctypes.byref(c), None, None, 0, 1, 128, 128, 0, None, 0, None) == tq.TQ_ERR_ARG
    assert lib.tq_attention_decode(None, ctypes.byref(c), None, 0, 4, 1.0, None, None, 0, None) == tq.TQ_ERR_ARG
    assert lib.tq_attention_prefill(None, ctypes.byref(c), None, 0, 8, 4, 1, 1.0, None, None, 0, None) == tq.TQ_ERR_ARG
    assert lib.tq_attention_prefill_ws_bytes(None, ctypes.byref(c), 8, 4) == 0
    assert lib.tq_scores(None, None, 0, 1, ctypes.byref(p), None, 10, None, None, None, 0, None) == tq.TQ_ERR_ARG
    assert lib.tq_ctx_destroy(None) == tq.TQ_ERR_ARG
    assert lib.tq_quantize_ws_bytes(None, 1, 1, 1) == 0
    assert tq.last_error() != ""


def test_time_next_decode_arguments():
    lib = tq.lib()
    assert lib.tq_time_next_decode(ctypes.c_void_p(16), None) == tq.TQ_ERR_ARG
    assert "both events" in tq.last_error()
    assert lib.tq_time_next_decode(None, ctypes.c_void_p(16)) == tq.TQ_ERR_ARG
    assert lib.tq_time_next_decode(None, None) == tq.TQ_OK


def test_read_probe_arguments():
    lib = tq.lib()
    sink = ctypes.c_void_p(256)
    assert lib.tq_read_probe(None, 16, 1, sink, None) == tq.TQ_ERR_ARG
    assert lib.tq_read_probe(ctypes.c_void_p(256), 15, 1, sink, None) == tq.TQ_ERR_ARG      # size
    assert lib.tq_read_probe(ctypes.c_void_p(264), 16, 1, sink, None) == tq.TQ_ERR_ARG      # alignment
    assert lib.tq_read_probe(ctypes.c_void_p(256), 16, 0, sink, None) == tq.TQ_ERR_ARG      # grid
    assert lib.tq_read_probe(ctypes.c_void_p(256), 16, 65537, sink, None) == tq.TQ_ERR_ARG
    assert "tq_read_probe" in tq.last_error()


def test_ctx_create_argument_errors():
    lib = tq.lib()
    h = ctypes.c_void_p()
    g = np.zeros((128, 128))
    assert lib.tq_ctx_create(128, None, g.ctypes.data, ctypes.byref(h)) == tq.TQ_ERR_ARG
    assert lib.tq_ctx_create(100, g.ctypes.data, g.ctypes.data, ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_ctx_create(128, g.ctypes.data, g.ctypes.data, None) == tq.TQ_ERR_ARG


@pytest.mark.parametrize("level,bits", [(1, 4), (2, 1), (2, 3), (3, 3), (5, 2), (7, 3), (7, 4)])
def test_angle_codebooks_equal_the_oracle(level, bits):
    """The library's PolarQuant angle tables (its own Lloyd iteration, incomplete
    beta and Gauss-Legendre quadrature) equal the oracle's (scipy) fp32 tables
    bit for bit; the fp64 centroids agree to 1e-11."""
    from oracle import polarquant as PQ
    h = tq.angle_codebook_build(level, bits)
    o = PQ.angle_codebook(level, bits)
    assert np.max(np.abs(h["centroids"] - o.centroids64)) < 1e-11
    assert np.array_equal(h["boundaries"], o.boundaries)
    assert np.array_equal(h["cos"], o.cos) and np.array_equal(h["sin"], o.sin)


def test_angle_codebook_arguments():
    lib = tq.lib()
    c = tq.CAngleCodebook()
    assert lib.tq_angle_codebook_build(0, 3, ctypes.byref(c)) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_angle_codebook_build(2, 5, ctypes.byref(c)) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_angle_codebook_build(2, 3, None) == tq.TQ_ERR_ARG
