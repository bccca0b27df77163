"""tq_score_noalloc through the C ABI: the entry point that allocates nothing (its query
workspace is the library's fixed per-device array) gives exactly tq_score's scores, on
consecutive calls whose second input is smaller, on every scorer path; a request whose
workspace exceeds the array is refused before any launch, and the array serves later calls."""
import numpy as np
import pytest

from oracle import layout
from oracle import turboquant as otq
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _case(d, bits, n, nqg, groups, seed, dtype=torch.bfloat16, mask=None, obits=0):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((groups * n, d)).astype(np.float32)).to(DEV).to(dtype)
    q = torch.from_numpy(rng.standard_normal((groups * nqg, d)).astype(np.float32)).to(DEV).to(dtype)
    plan = tq.tq_plan_create(d, bits, seed, mask, obits) if mask is not None else \
        tq.tq_plan_create(d, bits, seed)
    codes = tq.tq_encode(plan, x)
    return plan, x, q, codes


def _same_as_tq_score(plan, q, codes, n, nqg, groups):
    ref = tq.tq_score(plan, q, codes, n=n, nq_per_group=nqg, n_groups=groups)
    out = torch.full_like(ref, float("nan"))
    tq.tq_score_noalloc(plan, q, codes, n, out, nq_per_group=nqg, n_groups=groups)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    return out


def test_two_calls_in_a_row_the_second_smaller():
    """A large call then a smaller one (fewer groups, queries, keys and a shorter D): each
    equals tq_score exactly; the smaller one is also checked against the oracle."""
    plan, x, q, codes = _case(128, 3, 5000, 4, 8, 1)
    _same_as_tq_score(plan, q, codes, 5000, 4, 8)
    plan2, x2, q2, codes2 = _case(64, 4, 333, 3, 2, 2, dtype=torch.float32)
    out = _same_as_tq_score(plan2, q2, codes2, 333, 3, 2)
    sp = otq.make_split_plan(64, 4, 2)
    xs, ys = x2.cpu().numpy().astype(np.float64), q2.cpu().numpy().astype(np.float64)
    got = parity.unpack_gpu(sp, codes2.cpu().numpy())
    for g in range(2):
        sub = [{k: v[g * 333:(g + 1) * 333] for k, v in got[0].items()}]
        est = parity.oracle_scores_on_gpu_codes(sp, sub, ys[g * 3:(g + 1) * 3])
        parity.check_scores(out[g * 3:(g + 1) * 3].cpu().numpy(), est,
                            np.linalg.norm(ys[g * 3:(g + 1) * 3], axis=1),
                            np.linalg.norm(xs[g * 333:(g + 1) * 333], axis=1), "noalloc group %d" % g)


def test_every_scorer_path():
    """Outlier split (two sub-plans on the bit-sliced scorer), D = 256 with 8 queries per group
    (the wide scorer) and D = 512 with 2 queries per group (the vector-unit scorer), in
    decreasing workspace order."""
    d = 128
    mask = np.zeros(d, dtype=np.uint8)
    mask[np.random.default_rng(3).choice(d, 32, replace=False)] = 1
    plan, x, q, codes = _case(d, 3, 1000, 4, 4, 3, mask=mask, obits=5)
    _same_as_tq_score(plan, q, codes, 1000, 4, 4)
    plan, x, q, codes = _case(256, 4, 700, 8, 2, 4, dtype=torch.float32)
    _same_as_tq_score(plan, q, codes, 700, 8, 2)
    plan, x, q, codes = _case(512, 3, 300, 2, 3, 5, dtype=torch.float32)
    _same_as_tq_score(plan, q, codes, 300, 2, 3)


def test_request_beyond_the_array_is_refused():
    """1024 groups of 4 queries at 5 bits need 18 KiB of images per group (18 MiB in all):
    refused with TQ_EINVAL and nothing written; the next call in range still matches."""
    plan, x, q, codes = _case(128, 5, 16, 4, 1024, 6)
    out = torch.full((4096, 16), 7.0, device=DEV)
    with pytest.raises(tq.TqError):
        tq.tq_score_noalloc(plan, q, codes, 16, out, nq_per_group=4, n_groups=1024)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    _same_as_tq_score(plan, q[:4 * 512], codes, 16, 4, 512)
