"""A context built by the library from a seed alone (tq_ctx_create_seeded)
against the oracle's own seeded draws: the exported Pi and S agree, and keys
quantized with that context match the oracle's encoding under the usual code
rule (the oracle encodes with the exported tables, so that both sides use
identical fp32 Pi and S)."""
import numpy as np
import pytest

import synth
from oracle import turboquant as T
from tests import parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tq = pytest.importorskip("kv_cache_vector_turboquant_amd")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("d,seed", [(128, 0), (128, 99), (1536, 3)])
def test_seeded_context_tables_and_quantize(d, seed):
    ctx = tq.Context.from_seed(d, seed)
    rot, sk = ctx.export()
    o_pi = T.rotation_from_gaussian(T.seeded_gaussian(seed, T.STREAM_ROTATION, d, d))
    o_s = T.sketch_from_gaussian(T.seeded_gaussian(seed, T.STREAM_SKETCH, d, d))
    assert np.max(np.abs(rot.astype(np.float64) - o_pi)) <= 2.0 ** -24
    assert np.abs(sk.view(np.int32).astype(np.int64) - o_s.view(np.int32)).max() <= 1
    assert np.max(np.abs(rot.astype(np.float64).T @ rot.astype(np.float64) - np.eye(d))) <= 1e-5
    n = 4096 if d == 128 else 1024
    X = synth.outlier_kv(seed, (1,), synth.TAG_SCALES_K, (n, d)) if d == 128 else synth.gaussian(seed, (1,), (n, d))
    xt = torch.from_numpy(X).cuda()
    if d == 128:
        xt = xt.to(torch.bfloat16)
    keys = tq.Packed(n, d, 3, True)
    tq.quantize_kv(ctx, xt, keys)
    torch.cuda.synchronize()
    kw, kn = keys.host()
    cb = T.codebook(d, 3)
    P.check_key_records(kw, kn, T.encode(X, rot, cb, sk), cb, 3, d)
