"""The library's host code (tq_host.cpp: Lloyd-Max codebooks with their own
incomplete beta, the Householder QR with its worker threads, the seeded
Gaussian draws, PolarQuant angle codebooks, argument validation) built for the
CPU with AddressSanitizer and UndefinedBehaviorSanitizer (g++, errors fatal)
and exercised in a child process; the kernel launchers are stand-ins
(tests/asan/kernel_stubs.cpp), so nothing touches a GPU."""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_vector_turboquant_amd", "csrc")

CHILD = textwrap.dedent(r"""
    import ctypes, sys
    import numpy as np
    lib = ctypes.CDLL(sys.argv[1])
    i32, vp = ctypes.c_int32, ctypes.c_void_p
    class CB(ctypes.Structure):
        _fields_ = [("d", i32), ("bits", i32), ("centroid", ctypes.c_float * 16), ("boundary", ctypes.c_float * 15),
                    ("walsh", ctypes.c_float * 8), ("distortion", ctypes.c_double)]
    class ACB(ctypes.Structure):
        _fields_ = [("level", i32), ("bits", i32), ("centroid", ctypes.c_double * 16), ("boundary", ctypes.c_float * 15),
                    ("cos_c", ctypes.c_float * 16), ("sin_c", ctypes.c_float * 16)]
    lib.tq_last_error.restype = ctypes.c_char_p
    assert lib.tq_format_version() == 1
    for d in (3, 4, 64, 128, 1536, 4096):
        for b in (1, 2, 3, 4):
            c = CB()
            assert lib.tq_codebook_build(d, b, ctypes.byref(c)) == 0
            assert c.distortion > 0
    assert lib.tq_codebook_build(2, 3, ctypes.byref(CB())) != 0 and lib.tq_last_error()
    assert lib.tq_codebook_build(128, 5, ctypes.byref(CB())) != 0
    assert lib.tq_codebook_build(128, 3, None) != 0
    for lv in (1, 2, 5, 12):
        for b in (1, 4):
            assert lib.tq_angle_codebook_build(lv, b, ctypes.byref(ACB())) == 0
    lib.tq_gaussian_matrix.argtypes = [ctypes.c_uint64, ctypes.c_uint32, i32, i32, vp]
    lib.tq_rotation_build.argtypes = [i32, vp, vp]
    for d in (2, 33, 128, 300):
        g = np.empty((d, d))
        assert lib.tq_gaussian_matrix(7, 1, d, d, g.ctypes.data) == (0 if (d * d) % 2 == 0 else 1)
        if (d * d) % 2:
            continue
        pi = np.empty((d, d), np.float32)
        assert lib.tq_rotation_build(d, g.ctypes.data, pi.ctypes.data) == 0
        assert np.max(np.abs(pi.astype(np.float64).T @ pi - np.eye(d))) < 1e-5
    assert lib.tq_gaussian_matrix(1, 1, 0, 4, None) != 0
    # argument validation of the context and hot calls (no GPU call is reached)
    assert lib.tq_ctx_create(128, None, None, None) != 0
    assert lib.tq_ctx_create_seeded(100, 0, ctypes.byref(vp())) != 0
    for fn in ("tq_attention_decode", "tq_decode_step", "tq_quantize_kv", "tq_scores", "tq_append_token",
               "tq_attention_decode_noalloc", "tq_attention_prefill", "tq_cache_write", "tq_polar_quantize",
               "tq_polar_scores", "tq_polar_attention_decode", "tq_decode_logits"):
        f = getattr(lib, fn)
        f.restype = i32
        assert f(*([None] * 14)) != 0, fn
    assert lib.tq_time_next_decode(vp(1), None) != 0
    print("host code clean under ASan/UBSan")
""")


def _build(tmp):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("g++ or the HIP headers are missing")
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    objs = []
    for src in (os.path.join(CSRC, "tq_host.cpp"), os.path.join(ROOT, "tests", "asan", "kernel_stubs.cpp")):
        o = os.path.join(tmp, os.path.basename(src) + ".o")
        subprocess.run([gxx, *flags, "-c", src, "-o", o], check=True)
        objs.append(o)
    so = os.path.join(tmp, "libtq_host_asan.so")
    subprocess.run([gxx, "-shared", "-fsanitize=address,undefined", *objs, "-o", so, "-L/opt/rocm/lib", "-lamdhip64",
                    "-lpthread"], check=True)
    return so, gxx


def test_host_code_under_address_and_undefined_sanitizers(tmp_path):
    so, gxx = _build(str(tmp_path))
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run([gxx, "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=" ".join(p for p in (asan, ubsan) if os.path.isabs(p)),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", CHILD, so], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-6000:])
    assert "host code clean" in r.stdout
