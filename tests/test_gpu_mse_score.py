"""Scores from TurboQuant-MSE records through the C ABI against the fp64 oracle:
est = n <Pi pad(y), c[idx]>, the overview's quantized distance (§4.2.2) with the norm kept
apart (§4.2.1), as used for the MSE-quantized heads of §4.1.1 and the MSE index of §4.2.1.

The records are compared with the oracle's encode; every (query, key) pair with the oracle
evaluated on the library's own records (its cells and fp32 norms), and, for keys whose cells
match the oracle's, on the oracle's own codes, within 1e-3 ||q|| ||x||; grouped queries,
ragged key counts, zero keys, bf16 and fp32 on both sides, the bit-sliced scorer (D <= 128)
and the decoded fp16 key tiles (D >= 256) with one query, padded query tiles and several query
blocks.  tq_score_noalloc gives the same scores bit for bit and tq_score_topk the oracle's
top-k of them."""
import numpy as np
import pytest

from oracle import layout
from oracle import turboquant as otq
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("d,bits,n,nqg,groups,kdt,qdt", [
    (128, 3, 5000, 4, 2, "bfloat16", "float32"), (128, 4, 3001, 1, 1, "float32", "bfloat16"),
    (128, 2, 2049, 7, 3, "bfloat16", "bfloat16"), (128, 1, 1000, 4, 1, "float32", "float32"),
    (100, 3, 777, 5, 2, "float32", "float32"), (64, 2, 1500, 12, 1, "bfloat16", "float32"),
    (32, 4, 700, 4, 2, "float32", "bfloat16"), (1, 2, 65, 3, 1, "float32", "float32"),
    (128, 3, 17, 4, 5, "bfloat16", "float32"), (128, 3, 32768, 4, 8, "bfloat16", "bfloat16"),
    (200, 3, 1500, 4, 2, "float32", "float32"), (256, 2, 700, 300, 1, "bfloat16", "float32"),
    (512, 1, 401, 1, 3, "float32", "bfloat16"), (1536, 4, 3000, 130, 1, "float32", "float32"),
    (2048, 3, 129, 33, 2, "bfloat16", "bfloat16"), (300, 2, 1, 5, 2, "float32", "float32"),
    (128, 4, 1, 4, 3, "bfloat16", "float32")])
def test_mse_scores_match_oracle(d, bits, n, nqg, groups, kdt, qdt):
    rng = np.random.default_rng(d * 13 + bits * 5 + n)
    X = rng.standard_normal((groups * n, d)).astype(np.float32)
    if d == 1:
        X = np.rint(4 * X).astype(np.float32)      # rotated values exact on both sides
    X[0] = 0.0
    X[1] *= 1e4
    Y = rng.standard_normal((groups * nqg, d)).astype(np.float32)
    plan, op = tq.tq_plan_create_mse(d, bits, 11), otq.make_mse_plan(d, bits, 11)
    x = torch.from_numpy(X).to(DEV).to(getattr(torch, kdt))
    y = torch.from_numpy(Y).to(DEV).to(getattr(torch, qdt))
    codes = tq.tq_encode(plan, x)
    est = tq.tq_score(plan, y, codes, n, nq_per_group=nqg, n_groups=groups)
    again = torch.full_like(est, 7.0)
    tq.tq_score_noalloc(plan, y, codes, n, again, nq_per_group=nqg, n_groups=groups)
    k = min(10, n)
    ids, vals = tq.tq_score_topk(plan, y, codes, n, k, nq_per_group=nqg, n_groups=groups)
    torch.cuda.synchronize()
    assert torch.equal(est, again), "tq_score_noalloc differs from tq_score"
    Xd, Yd, E = _np(x), _np(y), _np(est)
    got = layout.unpack_mse(codes.cpu().numpy(), op.D, bits)
    own = otq.encode_mse(op, Xd)
    parity.compare_codes_mse(op, own, got, "mse score d=%d b=%d" % (d, bits))
    same = np.all(own["idx"] == got["idx"], axis=1)
    own_norm = own["norm"].astype(np.float32).astype(np.float64)
    xn, qn = np.linalg.norm(Xd, axis=1), np.linalg.norm(Yd, axis=1)
    ids, vals = ids.cpu().numpy(), _np(vals)
    for g in range(groups):
        ks, qs = slice(g * n, (g + 1) * n), slice(g * nqg, (g + 1) * nqg)
        ref = otq.score_mse(op, dict(idx=got["idx"][ks], norm=got["norm"][ks]), Yd[qs])
        parity.check_scores(E[qs], ref, qn[qs], xn[ks], "group %d, library records" % g)
        sg = same[ks]
        ref_own = otq.score_mse(op, dict(idx=own["idx"][ks][sg], norm=own_norm[ks][sg]), Yd[qs])
        parity.check_scores(E[qs][:, sg], ref_own, qn[qs], xn[ks][sg],
                            "group %d, oracle codes" % g)
        parity.check_topk(ids[qs], vals[qs], ref, k, qn[qs], xn[ks], "group %d top-k" % g)


@pytest.mark.parametrize("d", [128, 300])
def test_mse_scores_of_zero_queries(d):
    """A zero query scores exactly 0 against every key, on both scorers."""
    rng = np.random.default_rng(5)
    plan = tq.tq_plan_create_mse(d, 3, 2)
    x = torch.from_numpy(rng.standard_normal((300, d)).astype(np.float32)).to(DEV)
    codes = tq.tq_encode(plan, x)
    y = torch.zeros((4, d), dtype=torch.float32, device=DEV)
    est = tq.tq_score(plan, y, codes, 300, nq_per_group=4)
    torch.cuda.synchronize()
    assert torch.count_nonzero(est).item() == 0
