"""Second stage of two-stage retrieval (tq_rerank) through the C ABI: exact inner products
on the candidates against the fp64 oracle, and the recall the two stages reach together
against an exact fp32 search."""
import numpy as np
import pytest

import workloads
from oracle import turboquant as otq

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"
TOL = 1e-5     # fp32 accumulation of d products, relative to |q| |x|


def _check_rerank(ids, vals, ref_ids, ref_vals, exact, qn, xn, k, what):
    """ids equal the oracle's except where values tie within the tolerance; every returned
    value is the exact inner product of its id within the tolerance."""
    for q in range(ids.shape[0]):
        valid = ids[q] >= 0
        assert np.array_equal(valid, ref_ids[q] >= 0), what
        assert np.all(vals[q][~valid] == -np.inf)
        g = ids[q][valid]
        tol = TOL * qn[q] * (xn[g].max() if g.size else 1.0)
        assert np.all(np.abs(vals[q][valid] - exact[q, g]) <= tol), what
        assert np.all(np.diff(vals[q][valid]) <= 0), what
        if set(g.tolist()) != set(ref_ids[q][valid].tolist()):
            kth = ref_vals[q][valid][-1]
            for i in set(g.tolist()) - set(ref_ids[q][valid].tolist()):
                assert exact[q, i] >= kth - 2 * tol, "%s: query %d id %d" % (what, q, i)


@pytest.mark.parametrize("n,d,nq,kc,k,dtype", [
    (5000, 200, 37, 64, 10, "float32"), (3000, 1536, 16, 64, 10, "bfloat16"),
    (800, 96, 9, 256, 64, "float32"), (100, 33, 5, 100, 1, "float32"), (40, 128, 3, 64, 64, "bfloat16")])
def test_rerank_matches_oracle(n, d, nq, kc, k, dtype):
    rng = np.random.default_rng(n + d)
    X = rng.standard_normal((n, d)).astype(np.float32)
    Y = rng.standard_normal((nq, d)).astype(np.float32)
    cand = rng.integers(0, n, (nq, kc)).astype(np.int64)
    cand[:, :3] = cand[:, 3:6]                      # repeated ids
    cand[0, -2:] = [-1, n + 5]                      # ids out of range
    x = torch.from_numpy(X).to(DEV).to(getattr(torch, dtype))
    y = torch.from_numpy(Y).to(DEV).to(getattr(torch, dtype))
    ids, vals = tq.tq_rerank(y, x, torch.from_numpy(cand).to(DEV), k)
    torch.cuda.synchronize()
    X64 = x.float().cpu().numpy().astype(np.float64)
    Y64 = y.float().cpu().numpy().astype(np.float64)
    ref_ids, ref_vals = otq.rerank(Y64, X64, cand, k)
    _check_rerank(ids.cpu().numpy(), vals.cpu().numpy(), ref_ids, ref_vals, Y64 @ X64.T,
                  np.linalg.norm(Y64, axis=1), np.linalg.norm(X64, axis=1), k, "rerank n=%d" % n)


def test_two_stage_retrieval_recall():
    """Quantized top-64 (tq_score_topk on 4-bit codes of d = 1536 keys), then the exact
    top-10 of those 64: recall@10 against an exact fp32 search rises above the first stage's."""
    n, nq, d, k = 100000, 64, 1536, 10
    keys, queries = workloads.retrieval_inputs(DEV, n_keys=n, n_queries=nq, d=d, seed=3)
    plan = tq.tq_plan_create(d, 4, 0)
    codes = tq.tq_encode(plan, keys)
    ids1, _ = tq.tq_score_topk(plan, queries, codes, n, k)
    cand, _ = tq.tq_score_topk(plan, queries, codes, n, 64)
    ids2, _ = tq.tq_rerank(queries, keys, cand, k)
    exact = torch.topk(queries @ keys.T, k, dim=1).indices.cpu().numpy()
    r1 = np.mean([len(set(exact[q]) & set(ids1[q].tolist())) / k for q in range(nq)])
    r2 = np.mean([len(set(exact[q]) & set(ids2[q].tolist())) / k for q in range(nq)])
    print("recall@10: quantized %.3f, two-stage %.3f" % (r1, r2))
    assert r2 > r1 and r2 > 0.9


def test_rerank_invalid_arguments():
    x = torch.zeros((10, 8), device=DEV)
    y = torch.zeros((2, 8), device=DEV)
    cand = torch.zeros((2, 4), dtype=torch.int64, device=DEV)
    for k in (0, 5):
        with pytest.raises(tq.TqError):
            tq.tq_rerank(y, x, cand, k)
