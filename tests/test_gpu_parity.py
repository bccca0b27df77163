"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest

import workloads
from oracle import layout
from oracle import turboquant as otq
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _encode_and_compare(sp, plan, x_t, what):
    codes = tq.tq_encode(plan, x_t)
    torch.cuda.synchronize()
    got = parity.unpack_gpu(sp, codes.cpu().numpy())
    xs = _np(x_t).reshape(-1, sp.d)
    ref = otq.encode_split(sp, xs)
    stats = [parity.compare_codes(p, r, g, "%s/sub%d" % (what, i))
             for i, (p, r, g) in enumerate(zip(sp.plans, ref, got))]
    return codes, ref, got, stats


# ----------------------------------------------------------------------------- small config

@pytest.fixture(scope="module")
def small():
    keys, queries = workloads.small_inputs()
    sp = otq.make_split_plan(128, 4, 0)
    plan = tq.tq_plan_create(128, 4, 0)
    return keys, queries, sp, plan


def test_plan_layout(small):
    _, _, sp, plan = small
    assert plan.record_bytes == layout.record_bytes(128, 3) == 72
    assert plan.desc["sub"][0]["D"] == 128 and plan.desc["sub"][0]["R"] == 3


def test_encode_small_matches_oracle(small):
    keys, _, sp, plan = small
    x = torch.from_numpy(keys).to(DEV)
    _, _, _, stats = _encode_and_compare(sp, plan, x, "small")
    print(stats)


def test_encode_is_deterministic(small):
    keys, _, _, plan = small
    x = torch.from_numpy(keys).to(DEV)
    a = tq.tq_encode(plan, x)
    b = tq.tq_encode(plan, x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_qjl_stage_matches_oracle(small):
    _, _, sp, plan = small
    p = sp.plans[0]
    rng = np.random.default_rng(3)
    r = (rng.standard_normal((1000, 128)) * 0.03).astype(np.float32)
    beta = tq.tq_qjl(plan, 0, torch.from_numpy(r).to(DEV)).cpu().numpy().view(np.uint32)
    got = ((beta[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(1000, 128)
    ref, proj = otq.qjl_signs(p.S, r.astype(np.float64))
    mis = got != ref
    band = parity.sign_band(p, r.astype(np.float64), proj)
    assert not (mis & ~band).any()
    assert mis.sum() <= parity.MISMATCH_FRACTION * mis.size


def test_score_small_matches_oracle_on_oracle_codes(small):
    keys, queries, sp, plan = small
    ref = parity.stored(otq.encode(sp.plans[0], keys.astype(np.float64)))
    rec = layout.pack(ref, 128, 3)
    codes = torch.from_numpy(rec).to(DEV)
    q = torch.from_numpy(queries).to(DEV)
    est = tq.tq_score(plan, q, codes, n=4096).cpu().numpy()
    est_ref = otq.score(sp.plans[0], ref, queries.astype(np.float64))
    r = parity.check_scores(est, est_ref, np.linalg.norm(queries, axis=1),
                            np.linalg.norm(keys, axis=1), "small")
    print("max err / tol:", r)


def test_end_to_end_small_and_topk(small):
    keys, queries, sp, plan = small
    x = torch.from_numpy(keys).to(DEV)
    codes = tq.tq_encode(plan, x)
    q = torch.from_numpy(queries).to(DEV)
    est = tq.tq_score(plan, q, codes, n=4096)
    ids, vals = tq.tq_topk(est, 10)
    torch.cuda.synchronize()
    est = est.cpu().numpy()
    got = parity.unpack_gpu(sp, codes.cpu().numpy())
    ref = [otq.encode(sp.plans[0], keys.astype(np.float64))]
    parity.compare_codes(sp.plans[0], ref[0], got[0], "small e2e")
    parity.check_scores_end_to_end(sp, ref, got, est, queries, keys, "small e2e")
    # selection: against the oracle's top-k of its estimates for the codes the GPU scored
    est_g = parity.oracle_scores_on_gpu_codes(sp, got, queries)
    qn, xn = np.linalg.norm(queries, axis=1), np.linalg.norm(keys, axis=1)
    parity.check_topk(ids.cpu().numpy(), vals.cpu().numpy(), est_g, 10, qn, xn, "small top-10")
    # values returned are the GPU scores of the returned ids
    assert np.array_equal(vals.cpu().numpy(), np.take_along_axis(est, ids.cpu().numpy(), 1))


# ----------------------------------------------------------------------------- top-k

@pytest.mark.parametrize("nq,n,k", [(5, 1000, 10), (3, 4096, 1), (2, 300000, 64), (4, 37, 37),
                                    (1, 1, 1), (7, 70000, 16)])
def test_topk_matches_oracle_exactly_with_ties(nq, n, k):
    rng = np.random.default_rng(nq * 1000 + k)
    s = np.round(rng.standard_normal((nq, n)), 2).astype(np.float32)   # many ties
    ids, vals = tq.tq_topk(torch.from_numpy(s).to(DEV), k)
    ids_ref, vals_ref = otq.topk(s.astype(np.float64), k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.array_equal(vals.cpu().numpy().astype(np.float64), vals_ref)


@pytest.mark.parametrize("pattern,nq,n,k", [
    ("rising", 3, 50001, 64),      # every element beats the threshold: a compaction per round
    ("falling", 2, 40000, 64),     # the first round holds the answer
    ("signed_zero", 2, 9001, 64),  # -0 and +0 tie, decided by index
    ("half_neg_inf", 2, 10000, 33),
    ("rising", 2, 4099, 7),        # one full round of loads and three elements
    ("normal", 4, 1000003, 64),    # odd length: element loads
])
def test_topk_streaming_patterns(pattern, nq, n, k):
    """Row patterns that drive the selection's candidate buffer to its limits, against the
    oracle's top-k (ordered by (-value, index))."""
    rng = np.random.default_rng(n + k)
    if pattern == "rising":
        s = np.tile(np.arange(n, dtype=np.float32) / n, (nq, 1))
    elif pattern == "falling":
        s = np.tile(-np.arange(n, dtype=np.float32), (nq, 1))
    elif pattern == "signed_zero":
        s = np.zeros((nq, n), dtype=np.float32)
        s[:, ::3] = -0.0
        s[:, 5::7] = -1.0
    elif pattern == "half_neg_inf":
        s = rng.standard_normal((nq, n)).astype(np.float32)
        s[rng.random((nq, n)) < 0.5] = -np.inf
    else:
        s = rng.standard_normal((nq, n)).astype(np.float32)
    ids, vals = tq.tq_topk(torch.from_numpy(s).to(DEV), k)
    ids_ref, vals_ref = otq.topk(s.astype(np.float64), k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref), pattern
    assert np.array_equal(vals.cpu().numpy().astype(np.float64), vals_ref), pattern


# ----------------------------------------------------------------------------- shapes and edges

@pytest.mark.parametrize("d,bits,n,dtype", [
    (128, 3, 1, "float32"), (128, 3, 1001, "bfloat16"), (100, 3, 517, "float32"),
    (33, 5, 300, "bfloat16"), (1, 2, 65, "float32"), (64, 2, 200, "float32"),
    (256, 4, 130, "bfloat16"), (512, 3, 70, "float32"), (1024, 2, 40, "float32"),
    (1536, 4, 40, "float32"), (2048, 5, 20, "bfloat16"), (32, 4, 129, "float32"),
    # D >= 1024: the sign GEMM's workgroups cover key tiles in groups of 8 per XCD; 12 and
    # 10 tiles of 128 keys leave a partial group and a ragged last tile
    (1024, 3, 128 * 11 + 5, "float32"), (2048, 4, 128 * 9 + 1, "bfloat16")])
def test_encode_and_score_shapes(d, bits, n, dtype):
    rng = np.random.default_rng(d + n)
    xs = rng.standard_normal((n, d)).astype(np.float32)
    if d == 1:
        # one channel: every vector is a multiple of e_1, so the rotated coordinates that
        # are exactly zero recur in every row; small integers keep both sides exact there
        xs = np.rint(4 * xs).astype(np.float32)
    xs[0] *= 0.0                                             # zero vector
    ys = rng.standard_normal((6, d)).astype(np.float32)
    x = torch.from_numpy(xs).to(DEV).to(getattr(torch, dtype))
    y = torch.from_numpy(ys).to(DEV).to(getattr(torch, dtype))
    sp = otq.make_split_plan(d, bits, 11)
    plan = tq.tq_plan_create(d, bits, 11)
    codes, ref, got, _ = _encode_and_compare(sp, plan, x, "d=%d" % d)
    xs64, ys64 = _np(x), _np(y)
    # score kernel on oracle codes, 2 groups of 3 queries (second group reuses the codes)
    rec = layout.pack_split(sp, [parity.stored(c) for c in ref])
    rec2 = torch.from_numpy(np.concatenate([rec, rec])).to(DEV)
    est = tq.tq_score(plan, y, rec2, n=n, nq_per_group=3, n_groups=2).cpu().numpy()
    est_ref = otq.score_split(sp, [parity.stored(c) for c in ref], ys64)
    parity.check_scores(est, est_ref, np.linalg.norm(ys64, axis=1), np.linalg.norm(xs64, axis=1),
                        "d=%d" % d)
    assert np.all(est[:, 0] == 0.0)


@pytest.mark.parametrize("d,dtype,lo,hi", [(128, "bfloat16", -12, 12), (128, "bfloat16", -2, 4),
                                           (64, "bfloat16", -12, 12), (100, "bfloat16", -9, 9),
                                           (32, "float32", -12, 12), (128, "float32", -12, 12)])
def test_encode_over_a_wide_range_of_norms(d, dtype, lo, hi):
    """Codes depend on x / ||x|| only; rows scaled by 10^u, u uniform in [lo, hi], cover the
    kernels' per-vector scaling (and, for moderate norms, its unscaled shortcut)."""
    rng = np.random.default_rng(d + hi)
    n = 333
    xs = rng.standard_normal((n, d)) * 10.0 ** rng.uniform(lo, hi, (n, 1))
    xs[5] = 0.0
    x = torch.from_numpy(xs.astype(np.float32)).to(DEV).to(getattr(torch, dtype))
    for bits in (3, 4):
        sp = otq.make_split_plan(d, bits, 3)
        plan = tq.tq_plan_create(d, bits, 3)
        _encode_and_compare(sp, plan, x, "norms 1e%d..1e%d d=%d b=%d" % (lo, hi, d, bits))


@pytest.mark.parametrize("d,bits,n,nqg,groups", [
    (256, 4, 1000, 8, 1), (2048, 4, 300, 13, 1), (1536, 3, 517, 40, 1), (512, 2, 260, 16, 2),
    (1024, 5, 129, 9, 2), (200, 3, 777, 64, 1),
    # at least 128 queries per group: the decoded fp16 key tiles (blocks of 256 queries and
    # 128 keys), with ragged query blocks, ragged key blocks and every index width
    (256, 4, 1000, 128, 1), (2048, 3, 333, 300, 1), (1536, 5, 517, 256, 2), (512, 2, 129, 200, 1),
    (300, 3, 700, 513, 1), (1024, 4, 2000, 1000, 1)])
def test_score_many_queries_long_vectors(d, bits, n, nqg, groups):
    """The scorers for D > 128 with many queries per group, on oracle codes: the chunked
    bit-sliced scorer (8 to 127 queries per group) and the decoded fp16 key tiles (128 or
    more); ragged key counts, ragged query tiles."""
    rng = np.random.default_rng(d + nqg)
    xs = rng.standard_normal((groups * n, d)).astype(np.float32)
    xs[3] = 0.0
    ys = rng.standard_normal((groups * nqg, d)).astype(np.float32)
    sp = otq.make_split_plan(d, bits, 5)
    plan = tq.tq_plan_create(d, bits, 5)
    ref = otq.encode_split(sp, xs.astype(np.float64))
    rec = torch.from_numpy(layout.pack_split(sp, [parity.stored(c) for c in ref])).to(DEV)
    y = torch.from_numpy(ys).to(DEV)
    est = tq.tq_score(plan, y, rec, n=n, nq_per_group=nqg, n_groups=groups).cpu().numpy()
    st = parity.stored(ref[0])
    for g in range(groups):
        sub = {k: v[g * n:(g + 1) * n] for k, v in st.items()}
        est_ref = otq.score(sp.plans[0], sub, ys[g * nqg:(g + 1) * nqg].astype(np.float64))
        parity.check_scores(est[g * nqg:(g + 1) * nqg], est_ref,
                            np.linalg.norm(ys[g * nqg:(g + 1) * nqg], axis=1),
                            np.linalg.norm(xs[g * n:(g + 1) * n], axis=1), "d=%d group %d" % (d, g))


@pytest.mark.parametrize("d,bits,dtype", [(1024, 3, "float32"), (2048, 4, "bfloat16")])
def test_long_vector_encode_across_batches(d, bits, dtype):
    """D >= 1024 encodes in batches of 32768 vectors (signs from a second launch): rows on
    both sides of the batch boundary and in the ragged last batch match the oracle."""
    n = 32768 + 77
    g = torch.Generator(device=DEV)
    g.manual_seed(d)
    x = torch.randn((n, d), generator=g, device=DEV, dtype=torch.float32).to(getattr(torch, dtype))
    sp = otq.make_split_plan(d, bits, 7)
    plan = tq.tq_plan_create(d, bits, 7)
    codes = tq.tq_encode(plan, x)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(0, 40), np.arange(32768 - 40, 32768 + 40), np.arange(n - 37, n)])
    ri = torch.as_tensor(rows, device=DEV)
    got = parity.unpack_gpu(sp, codes[ri].cpu().numpy())
    ref = otq.encode_split(sp, _np(x[ri]))
    for i, (p, r, gg) in enumerate(zip(sp.plans, ref, got)):
        parity.compare_codes(p, r, gg, "d=%d batches/sub%d" % (d, i))


def test_strided_rows_and_query_groups():
    d, n = 128, 300
    rng = np.random.default_rng(5)
    big = torch.from_numpy(rng.standard_normal((n, 160)).astype(np.float32)).to(DEV)
    x = big[:, 16:144]                                       # row stride 160, offset 16
    sp = otq.make_split_plan(d, 3, 2)
    plan = tq.tq_plan_create(d, 3, 2)
    _encode_and_compare(sp, plan, x, "strided")
    ref = [otq.encode(sp.plans[0], _np(x))]
    for g in (1, 2, 3, 5, 8):
        y = torch.from_numpy(rng.standard_normal((2 * g, d)).astype(np.float32)).to(DEV)
        codes = tq.tq_encode(plan, torch.cat([x, x]).contiguous())
        est = tq.tq_score(plan, y, codes, n=n, nq_per_group=g, n_groups=2).cpu().numpy()
        c = codes.cpu().numpy()
        assert np.array_equal(c[:n], c[n:])                 # both groups hold the same records
        got = parity.unpack_gpu(sp, c[:n])
        parity.compare_codes(sp.plans[0], ref[0], got[0], "strided, group %d" % g)
        for h in range(2):
            parity.check_scores_end_to_end(sp, ref, got, est[h * g:(h + 1) * g],
                                           _np(y)[h * g:(h + 1) * g], _np(x),
                                           "group size %d, group %d" % (g, h))


def test_outlier_split_plan_small():
    d = 128
    rng = np.random.default_rng(9)
    mask = np.zeros(d, dtype=np.uint8)
    mask[np.sort(rng.choice(d, 32, replace=False))] = 1
    xs = rng.standard_normal((700, d)).astype(np.float32)
    xs[:, mask == 1] *= 10
    ys = rng.standard_normal((4, d)).astype(np.float32)
    for bits, obits in ((3, 5), (2, 4)):
        sp = otq.make_split_plan(d, bits, 0, mask, obits)
        plan = tq.tq_plan_create(d, bits, 0, mask, obits)
        assert plan.record_bytes == sum(layout.record_bytes(p.D, p.R) for p in sp.plans)
        x = torch.from_numpy(xs).to(DEV).to(torch.bfloat16)
        codes, ref, got, _ = _encode_and_compare(sp, plan, x, "split %d/%d" % (bits, obits))
        rec = torch.from_numpy(layout.pack_split(sp, [parity.stored(c) for c in ref])).to(DEV)
        y = torch.from_numpy(ys).to(DEV).to(torch.bfloat16)
        est = tq.tq_score(plan, y, rec, n=700).cpu().numpy()
        est_ref = otq.score_split(sp, [parity.stored(c) for c in ref], _np(y))
        parity.check_scores(est, est_ref, np.linalg.norm(_np(y), axis=1),
                            np.linalg.norm(_np(x), axis=1), "split score")


@pytest.mark.parametrize("nq", [5, 70])
def test_outlier_split_plan_long_vectors(nq):
    """A split plan whose sub-plans are D = 256 (240 regular channels) and D = 64 (60 outlier
    channels): the long-vector query path for both (the projection w = S y' with fewer rows of
    S than one workgroup covers for the short one), against the oracle's split estimate; two
    calls give the same scores bit for bit (the sums of w are added in a fixed order)."""
    d, n = 300, 900
    rng = np.random.default_rng(nq)
    mask = np.zeros(d, dtype=np.uint8)
    mask[np.sort(rng.choice(d, 60, replace=False))] = 1
    xs = rng.standard_normal((n, d)).astype(np.float32)
    xs[:, mask == 1] *= 8
    ys = rng.standard_normal((nq, d)).astype(np.float32)
    sp = otq.make_split_plan(d, 3, 4, mask, 4)
    plan = tq.tq_plan_create(d, 3, 4, mask, 4)
    assert [p.D for p in sp.plans] == [256, 64]
    st = [parity.stored(c) for c in otq.encode_split(sp, xs.astype(np.float64))]
    rec = torch.from_numpy(layout.pack_split(sp, st)).to(DEV)
    y = torch.from_numpy(ys).to(DEV)
    est = tq.tq_score(plan, y, rec, n=n)
    est2 = tq.tq_score(plan, y, rec, n=n)
    torch.cuda.synchronize()
    assert torch.equal(est, est2)
    est_ref = otq.score_split(sp, st, ys.astype(np.float64))
    parity.check_scores(est.cpu().numpy(), est_ref, np.linalg.norm(ys.astype(np.float64), axis=1),
                        np.linalg.norm(xs.astype(np.float64), axis=1), "split d=300 nq=%d" % nq)


def test_invalid_calls_raise():
    plan = tq.tq_plan_create(128, 3, 0)
    x = torch.zeros((4, 64), device=DEV)
    with pytest.raises(ValueError):
        tq.tq_encode(plan, x)
    with pytest.raises(tq.TqError):
        tq.tq_topk(torch.zeros((2, 5), device=DEV), 6)


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_encode_d128_bf16_every_index_width(bits):
    """bf16 keys at d = 128 (the 32-vector matrix-core encoder): every index width, a ragged
    count (not a multiple of 32 or of a workgroup's 256), zero vectors, strided rows, and
    norms from 1e-8 to 1e8 in one batch (so waves take both the unscaled and the scaled fp16
    conversion)."""
    d = 128
    rng = np.random.default_rng(100 + bits)
    n = 4096 + 77
    xs = rng.standard_normal((n, d))
    xs[:, :6] = rng.standard_t(3, (n, 6))
    xs[2048:] *= 10.0 ** rng.uniform(-8, 8, (n - 2048, 1))
    xs[[0, 31, 32, 4100]] = 0.0
    big = torch.zeros((n, 192), dtype=torch.bfloat16, device=DEV)
    big[:, 40:168] = torch.from_numpy(xs.astype(np.float32)).to(DEV).to(torch.bfloat16)
    x = big[:, 40:168]                                        # row stride 192, offset 40
    sp = otq.make_split_plan(d, bits, 21)
    plan = tq.tq_plan_create(d, bits, 21)
    codes, ref, got, stats = _encode_and_compare(sp, plan, x, "d=128 b=%d" % bits)
    # the same vectors as a contiguous tensor give the same records
    again = tq.tq_encode(plan, x.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(codes, again)
    ys = rng.standard_normal((8, d)).astype(np.float32)
    est = tq.tq_score(plan, torch.from_numpy(ys).to(DEV), codes, n=n).cpu().numpy()
    parity.check_scores_end_to_end(sp, ref, got, est, ys, _np(x), "d=128 b=%d" % bits)
