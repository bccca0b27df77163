"""tq_score_topk through the C ABI: identical to tq_score followed by tq_topk (same estimates,
same order (-value, index)), and within the score tolerance of the oracle's top-k.

The fused form (one sub-plan, D > 128 and a multiple of 128, at least 8 queries per group)
keeps per-query candidate lists on chip; the other shapes select from a temporary score
matrix.  Both are covered, with ragged key counts and query tiles, ties, and keys whose
scores rise with their index (every key block then refills the lists)."""
import numpy as np
import pytest

from oracle import layout
from oracle import turboquant as otq
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _oracle_codes(sp, xs):
    ref = otq.encode_split(sp, xs.astype(np.float64))
    st = [parity.stored(c) for c in ref]
    return st, torch.from_numpy(layout.pack_split(sp, st)).to(DEV)


def _unfused(plan, y, rec, n, k, nqg, groups):
    est = tq.tq_score(plan, y, rec, n=n, nq_per_group=nqg, n_groups=groups)
    ids, vals = tq.tq_topk(est, k)
    return est, ids, vals


@pytest.mark.parametrize("d,bits,n,nqg,groups,k,mask", [
    (1536, 4, 20077, 40, 1, 10, False),     # the retrieval shape, scaled down; ragged tail
    (2048, 3, 5000, 8, 2, 64, False),       # two groups, largest k
    (256, 2, 1000, 16, 1, 17, False),       # k above 16 on the fused path
    (512, 5, 300, 9, 1, 1, False),          # ragged query tile (9 = 8 + 1), k = 1
    (1024, 3, 129, 13, 1, 64, False),       # two key blocks, the second holding one key
    (1024, 2, 64, 8, 1, 64, False),         # k = n, one partial key block
    (128, 3, 4096, 4, 8, 10, False),        # D = 128: scores to a temporary, then top-k
    (200, 3, 777, 4, 1, 10, False),         # fewer than 8 queries per group: not fused
    (128, 4, 1500, 4, 2, 10, True),         # outlier split: two sub-plans, not fused
    (1536, 4, 5077, 256, 1, 10, False),     # 256 queries: decoded fp16 key tiles, then top-k
    (2048, 3, 3000, 130, 2, 64, False),     # two groups, a ragged query block
])
def test_score_topk_equals_score_then_topk_and_oracle(d, bits, n, nqg, groups, k, mask):
    rng = np.random.default_rng(d * 7 + n)
    xs = rng.standard_normal((groups * n, d)).astype(np.float32)
    xs[2] = 0.0
    ys = rng.standard_normal((groups * nqg, d)).astype(np.float32)
    if mask:
        m = np.zeros(d, dtype=np.uint8)
        m[rng.choice(d, d // 4, replace=False)] = 1
        sp = otq.make_split_plan(d, bits, 9, m, bits + 1)
        plan = tq.tq_plan_create(d, bits, 9, m, bits + 1)
    else:
        sp = otq.make_split_plan(d, bits, 9)
        plan = tq.tq_plan_create(d, bits, 9)
    st, rec = _oracle_codes(sp, xs)
    y = torch.from_numpy(ys).to(DEV)
    est, ids0, vals0 = _unfused(plan, y, rec, n, k, nqg, groups)
    ids, vals = tq.tq_score_topk(plan, y, rec, n, k, nq_per_group=nqg, n_groups=groups)
    torch.cuda.synchronize()
    ids, vals, est = ids.cpu().numpy(), vals.cpu().numpy(), est.cpu().numpy()
    assert np.array_equal(ids, ids0.cpu().numpy())
    assert np.array_equal(vals, vals0.cpu().numpy())
    assert np.array_equal(vals, np.take_along_axis(est, ids, 1))
    for g in range(groups):
        sub = [{kk: v[g * n:(g + 1) * n] for kk, v in s.items()} for s in st]
        yg = ys[g * nqg:(g + 1) * nqg].astype(np.float64)
        est_ref = otq.score_split(sp, sub, yg)
        qn = np.linalg.norm(yg, axis=1)
        xn = np.linalg.norm(xs[g * n:(g + 1) * n].astype(np.float64), axis=1)
        rows = slice(g * nqg, (g + 1) * nqg)
        parity.check_topk(ids[rows], vals[rows], est_ref, k, qn, xn, "d=%d group %d" % (d, g))
        # each returned value within the score tolerance of the oracle's estimate of that key
        err = np.abs(vals[rows] - np.take_along_axis(est_ref, ids[rows], 1))
        assert np.all(err <= parity.SCORE_TOL * qn[:, None] * xn[ids[rows]]), "d=%d values" % d


def _single_record_plan(d, bits, seed):
    sp = otq.make_split_plan(d, bits, seed)
    plan = tq.tq_plan_create(d, bits, seed)
    rng = np.random.default_rng(seed)
    x0 = rng.standard_normal((1, d))
    st, _ = _oracle_codes(sp, x0)
    return sp, plan, st, x0


def test_score_topk_ties_go_to_the_smaller_index():
    """Every key holds the same record, so each query's scores are all equal: the top-k is
    the first k indices, on the fused path and on the temporary-matrix path alike."""
    for d, nqg in ((1536, 16), (128, 4)):
        sp, plan, st, _ = _single_record_plan(d, 3, 21)
        n, k = 3000, 12
        rec1 = layout.pack_split(sp, st)
        rec = torch.from_numpy(np.repeat(rec1, n, axis=0)).to(DEV)
        y = torch.from_numpy(np.random.default_rng(1).standard_normal((nqg, d)).astype(np.float32)).to(DEV)
        ids, vals = tq.tq_score_topk(plan, y, rec, n, k)
        est = tq.tq_score(plan, y, rec, n=n)
        torch.cuda.synchronize()
        ids, vals, est = ids.cpu().numpy(), vals.cpu().numpy(), est.cpu().numpy()
        assert np.all(est == est[:, :1])
        assert np.array_equal(ids, np.tile(np.arange(k), (nqg, 1)))
        assert np.array_equal(vals, est[:, :k])


def test_score_topk_rising_and_falling_scores():
    """Keys share one direction and differ in norm, rising with the index: a query along the
    key direction ranks the last keys first and every key block refills its lists; the
    opposite query ranks the first keys first."""
    d, bits, n, k = 1536, 4, 40000, 10
    sp, plan, st, x0 = _single_record_plan(d, bits, 5)
    norms = np.linspace(1.0, 3.0, n).astype(np.float32)
    st_n = [{kk: np.repeat(v, n, axis=0) for kk, v in s.items()} for s in st]
    st_n[0]["norm"] = norms.astype(np.float64)
    rec = torch.from_numpy(layout.pack_split(sp, st_n)).to(DEV)
    u = x0[0] / np.linalg.norm(x0[0])
    rng = np.random.default_rng(2)
    ys = np.concatenate([u[None], -u[None], rng.standard_normal((6, d))]).astype(np.float32)
    y = torch.from_numpy(ys).to(DEV)
    ids, vals = tq.tq_score_topk(plan, y, rec, n, k)
    est, ids0, vals0 = _unfused(plan, y, rec, n, k, 8, 1)
    torch.cuda.synchronize()
    ids, vals = ids.cpu().numpy(), vals.cpu().numpy()
    assert np.array_equal(ids, ids0.cpu().numpy())
    assert np.array_equal(vals, vals0.cpu().numpy())
    est = est.cpu().numpy()
    assert np.all(np.diff(est[0]) >= 0) and np.all(np.diff(est[1]) <= 0)
    # ties in the rising row keep the smaller index first
    order0 = sorted(range(n), key=lambda i: (-est[0, i], i))[:k]
    assert ids[0].tolist() == order0
    assert ids[1].tolist() == list(range(k))
    est_ref = otq.score_split(sp, st_n, ys[:2].astype(np.float64))
    parity.check_topk(ids[:2], vals[:2], est_ref, k, np.linalg.norm(ys[:2], axis=1),
                      norms.astype(np.float64), "rising/falling")


def test_score_topk_invalid_calls_raise():
    plan = tq.tq_plan_create(256, 3, 0)
    rec = torch.zeros((10, plan.record_bytes), dtype=torch.uint8, device=DEV)
    y = torch.zeros((8, 256), device=DEV)
    for k in (0, 11, 65):
        with pytest.raises(tq.TqError):
            tq.tq_score_topk(plan, y, rec, 10, k)
