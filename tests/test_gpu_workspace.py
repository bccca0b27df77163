"""The per-stream workspace of tq_score, tq_score_topk and tq_attend: calls whose workspace
grows, shrinks and grows again on one stream, and calls interleaved on two streams, give
exactly the results of the entry point that uses its own fixed array (tq_score_noalloc) or of
the same call made alone."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _case(d, bits, n, nqg, groups, seed):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((groups * n, d)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((groups * nqg, d)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    plan = tq.tq_plan_create(d, bits, seed)
    return plan, q, tq.tq_encode(plan, x)


def _noalloc(plan, q, codes, n, nqg, groups):
    out = torch.full((groups * nqg, n), float("nan"), device=DEV)
    tq.tq_score_noalloc(plan, q, codes, n, out, nq_per_group=nqg, n_groups=groups)
    return out


def test_one_stream_growing_and_shrinking():
    cases = [(128, 3, 700, 4, 2, 1), (128, 3, 3000, 8, 64, 2), (64, 4, 100, 1, 1, 3),
             (128, 2, 2000, 16, 96, 4), (128, 3, 700, 4, 2, 1)]
    for d, bits, n, nqg, groups, seed in cases:
        plan, q, codes = _case(d, bits, n, nqg, groups, seed)
        got = tq.tq_score(plan, q, codes, n=n, nq_per_group=nqg, n_groups=groups)
        ref = _noalloc(plan, q, codes, n, nqg, groups)
        ids, vals = tq.tq_score_topk(plan, q, codes, n, 8, nq_per_group=nqg, n_groups=groups)
        ids2, vals2 = tq.tq_topk(ref, 8)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (d, bits, n, nqg, groups)
        assert torch.equal(ids, ids2) and torch.equal(vals, vals2)


def test_attend_after_a_larger_score_workspace():
    """tq_attend's partial results reuse the buffer a larger score call grew; the output
    equals that of the same call on a fresh stream."""
    d, n, nqg, groups = 128, 5000, 4, 6
    kplan, q, kc = _case(d, 3, n, nqg, groups, 5)
    vplan = tq.tq_plan_create_mse(d, 3, 6)
    rng = np.random.default_rng(7)
    v = torch.from_numpy(rng.standard_normal((groups * n, d)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    vc = tq.tq_encode(vplan, v)
    logits = tq.tq_score(kplan, q, kc, n=n, nq_per_group=nqg, n_groups=groups)
    big_plan, bq, bc = _case(128, 3, 4000, 32, 64, 8)
    tq.tq_score(big_plan, bq, bc, n=4000, nq_per_group=32, n_groups=64)
    out = tq.tq_attend(vplan, logits, vc, n, 0.125, nq_per_group=nqg, n_groups=groups)
    torch.cuda.synchronize()
    fresh = torch.cuda.Stream()
    fresh.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(fresh):
        out2 = tq.tq_attend(vplan, logits, vc, n, 0.125, nq_per_group=nqg, n_groups=groups)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_two_streams_interleaved():
    """Two streams, each with its own buffer, issue calls of different sizes in turn; every
    result equals the same call made alone."""
    a = _case(128, 3, 3000, 4, 16, 11)
    b = _case(128, 4, 1500, 8, 40, 12)
    ref_a = _noalloc(*a, 3000, 4, 16)
    ref_b = _noalloc(*b, 1500, 8, 40)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for i in range(6):
        plan, q, codes = a if i % 2 == 0 else b
        n, nqg, groups = (3000, 4, 16) if i % 2 == 0 else (1500, 8, 40)
        # streams s0 s1 s1 s0 s0 s1: each stream's buffer serves both sizes in turn
        st = streams[(i + i // 2) % 2]
        out = torch.empty((groups * nqg, n), device=DEV)
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            tq.tq_score(plan, q, codes, n=n, nq_per_group=nqg, n_groups=groups, scores=out)
        outs.append((out, ref_a if i % 2 == 0 else ref_b))
    torch.cuda.synchronize()
    for i, (out, ref) in enumerate(outs):
        assert torch.equal(out, ref), i
