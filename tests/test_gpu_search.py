"""GPU parity of the fused search path of tq_scores (d a multiple of 128):
fixed-point query digits on the fp6 x fp4 MFMA over 128-coordinate blocks and a
fused top-k, against the oracle on identical packed bytes. Covers several
block counts, ragged key and query counts, every key format, k up to 64,
bf16 queries, compact fp16 norms and exact ties (duplicated keys: equal scores
go to the lower index)."""
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

DEV = "cuda"


def _ctx(d, seed=0):
    ctx = tq.Context(d, seed)
    Pi = T.rotation_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_ROTATION, d, d))
    S = T.sketch_from_gaussian(synth.gaussian_matrix(seed, synth.TAG_SKETCH, d, d))
    return ctx, Pi, S


def _keys(X, Pi, S, bits, qjl, norm_f16=False):
    d = Pi.shape[0]
    cb = T.codebook(d, bits) if bits > 0 else None
    enc = T.encode(X, Pi, cb, S if qjl else None)
    pk = T.pack_keys(enc, bits, qjl, norm_f16)
    kp = tq.Packed(X.shape[0], d, bits, True, qjl=qjl, norm_f16=norm_f16)
    kp.words.copy_(torch.from_numpy(pk["bits"].reshape(X.shape[0], -1).view(np.int32)).to(DEV).view_as(kp.words))
    kp.norms.copy_(torch.from_numpy(np.ascontiguousarray(pk["norms"])).to(DEV).view_as(kp.norms))
    return cb, enc, pk, kp


@pytest.mark.parametrize("d,n,nq,k,bits,qjl,qdt,f16", [
    (256, 3001, 5, 64, 3, True, "bf16", False),
    (512, 1000, 9, 7, 2, True, "f32", True),
    (128, 777, 3, 1, 4, True, "f32", False),
    (128, 2050, 6, 12, 1, True, "bf16", False),
    (384, 1500, 4, 20, 3, False, "f32", False),
    (128, 999, 7, 5, 0, True, "f32", False),
])
def test_search_scores_and_topk(d, n, nq, k, bits, qjl, qdt, f16):
    ctx, Pi, S = _ctx(d, 3)
    X = synth.unit_gaussian(d + n, (1,), (n, d))
    Qv = synth.gaussian(d + n, (2,), (nq, d), qdt)
    cb, enc, pk, kp = _keys(X, Pi, S, bits, qjl, f16)
    q = torch.from_numpy(Qv).to(DEV)
    if qdt == "bf16":
        q = q.to(torch.bfloat16)
    sc, ti, tv = tq.scores(ctx, q.contiguous(), kp, want_scores=True, topk=k)
    torch.cuda.synchronize()
    ref = T.scores(Qv, Pi, S, cb, pk, qjl)
    qn = np.linalg.norm(Qv.astype(np.float64), axis=1)
    xn = np.asarray(pk["norms"]).reshape(n, -1)[:, 0].astype(np.float64)
    P.check_scores(sc.cpu().numpy(), ref, qn, xn)
    P.check_topk(ti.cpu().numpy(), tv.cpu().numpy(), ref, k, qn, xn)
    # the top-k alone (no score matrix) gives the same result
    sc2, ti2, tv2 = tq.scores(ctx, q.contiguous(), kp, want_scores=False, topk=k)
    torch.cuda.synchronize()
    assert sc2 is None
    assert np.array_equal(ti2.cpu().numpy(), ti.cpu().numpy()) and np.array_equal(tv2.cpu().numpy(), tv.cpu().numpy())


def test_search_ties_go_to_the_lower_index():
    """Every key appears three times (records copied): equal scores, so the
    top-k must list the copies in increasing index order."""
    d, base = 128, 300
    ctx, Pi, S = _ctx(d, 4)
    X0 = synth.unit_gaussian(44, (1,), (base, d))
    X = np.concatenate([X0, X0, X0])
    Qv = synth.gaussian(44, (2,), (6, d))
    cb, enc, pk, kp = _keys(X, Pi, S, 3, True)
    k = 30
    _, ti, tv = tq.scores(ctx, torch.from_numpy(Qv).to(DEV), kp, want_scores=False, topk=k)
    torch.cuda.synchronize()
    ti, tv = ti.cpu().numpy(), tv.cpu().numpy()
    ref = T.scores(Qv, Pi, S, cb, pk)
    for qi in range(Qv.shape[0]):
        want = T.topk(ref[qi], k)
        # GPU and oracle scores of the copies are identical bytes, so the order of
        # equal scores is fixed: a copy's three indices appear in increasing order
        for j in range(0, k, 3):
            tri = ti[qi][j:j + 3]
            if len(tri) == 3 and len({int(t) % base for t in tri}) == 1:
                assert list(tri) == sorted(tri)
        assert np.all(np.diff(tv[qi]) <= 0)
        assert set((ti[qi] % base).tolist()) == set((want % base).tolist()) or \
            abs(ref[qi][want[-1]] - tv[qi][-1]) <= 1e-3 * abs(ref[qi][want[-1]])
