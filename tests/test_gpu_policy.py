"""The KV-cache policy layer through the C ABI against the fp64 oracle: outlier channels by
variance (tq_calibrate_outliers) and the streaming append (tq_encode_scatter)."""
import numpy as np
import pytest

from oracle import layout, policy
from oracle import turboquant as otq
from tests import parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import rotation_online_vector_amd as tq  # noqa: E402

DEV = "cuda:0"


def _np64(t):
    return t.detach().cpu().double().numpy()


def _check_mask(mask, var_ref, n_out, what):
    """The chosen set is unique except among channels whose variances tie with the n_out-th
    within fp64 summation-order rounding; check what is unique."""
    mask = np.asarray(mask).astype(bool)
    assert mask.sum() == n_out, what
    if n_out == 0 or n_out == len(var_ref):
        return
    kth = np.sort(var_ref)[::-1][n_out - 1]
    tol = 1e-9 * abs(kth) + 1e-300
    assert np.all(var_ref[mask] >= kth - tol), what
    assert np.all(mask[var_ref > kth + tol]), what


@pytest.mark.parametrize("n,d,n_out,dtype", [(5000, 128, 32, "bfloat16"), (777, 100, 25, "float32"),
                                             (1, 64, 16, "float32"), (300, 1000, 250, "bfloat16"),
                                             (4096, 8, 8, "bfloat16"), (50, 33, 0, "float32")])
def test_calibrate_outliers_matches_oracle(n, d, n_out, dtype):
    rng = np.random.default_rng(n + d)
    X = rng.standard_normal((n, d)) * rng.uniform(0.2, 3.0, d) + rng.uniform(-50, 50, d)
    planted = np.sort(rng.choice(d, min(n_out, d) // 2, replace=False))
    X[:, planted] *= 20
    xt = torch.from_numpy(X.astype(np.float32)).to(DEV).to(getattr(torch, dtype))
    var, mask = tq.tq_calibrate_outliers(xt, n_out)
    torch.cuda.synchronize()
    Xe = _np64(xt)                          # the values the library read
    ref = policy.channel_variance(Xe)
    assert np.allclose(var.cpu().numpy(), ref, rtol=1e-9, atol=1e-300)
    _check_mask(mask.cpu().numpy(), ref, n_out, "n=%d d=%d" % (n, d))
    if n > 1:
        assert np.all(mask.cpu().numpy()[planted] == 1)


def test_calibrate_outliers_many_partials_sampled_channels():
    """300000 rows x 4096 channels: more row blocks than the partial buffer holds, so rows per
    partial grow; variances of sampled channels against the oracle."""
    n, d = 300_000, 4096
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    xt = (torch.randn((n, d), generator=g, device=DEV) * 2 + 3).to(torch.bfloat16)
    xt[:, 77] *= 30
    var, mask = tq.tq_calibrate_outliers(xt, 1024)
    torch.cuda.synchronize()
    cols = np.sort(np.concatenate([np.random.default_rng(1).choice(d, 24, replace=False), [0, 77, d - 1]]))
    ref = policy.channel_variance(_np64(xt[:, torch.as_tensor(cols, device=DEV)]))
    assert np.allclose(var.cpu().numpy()[cols], ref, rtol=1e-9)
    assert int(mask.sum()) == 1024 and int(mask[77]) == 1


def test_calibrated_mask_drives_a_split_plan():
    """Policy: a head's keys calibrate its outlier channels (a quarter of them), the mask makes
    the split plan, and its codes and scores match the oracle's split plan on the same mask."""
    d, n = 128, 3000
    rng = np.random.default_rng(3)
    X = rng.standard_normal((n, d))
    hot = np.sort(rng.choice(d, 32, replace=False))
    X[:, hot] *= 8
    xt = torch.from_numpy(X.astype(np.float32)).to(DEV)
    _, mask = tq.tq_calibrate_outliers(xt, 32)
    m = mask.cpu().numpy()
    assert np.array_equal(np.nonzero(m)[0], hot)
    plan = tq.tq_plan_create(d, 3, 5, m, 5)
    sp = otq.make_split_plan(d, 3, 5, m, 5)
    codes = tq.tq_encode(plan, xt)
    Q = rng.standard_normal((4, d))
    sc = tq.tq_score(plan, torch.from_numpy(Q.astype(np.float32)).to(DEV), codes, n=n)
    torch.cuda.synchronize()
    got = parity.unpack_gpu(sp, codes.cpu().numpy())
    ref = otq.encode_split(sp, X)
    for i, (p, r, gg) in enumerate(zip(sp.plans, ref, got)):
        parity.compare_codes(p, r, gg, "policy sub%d" % i)
    est = otq.score_split(sp, [parity.stored(c) for c in got], Q)
    parity.check_scores(sc.cpu().numpy(), est, np.linalg.norm(Q, axis=1), np.linalg.norm(X, axis=1), "policy")


@pytest.mark.parametrize("mode,d,bits,dtype", [("ip", 128, 3, "bfloat16"), ("mse", 128, 3, "bfloat16"),
                                               ("split", 128, 3, "float32"), ("ip", 1536, 4, "float32"),
                                               ("mse", 40, 2, "float32")])
def test_encode_scatter_appends_one_token_per_group(mode, d, bits, dtype):
    """A decode step: token t of each of G groups goes to row g * cap + t of the cache; rows are
    byte-identical to tq_encode of the same vectors and within the oracle's bands; the rest of
    the cache is untouched; rows outside the cache are skipped."""
    G, cap, t = 64, 40, 17
    rng = np.random.default_rng(d + bits)
    if mode == "mse":
        plan, op = tq.tq_plan_create_mse(d, bits, 2), otq.make_mse_plan(d, bits, 2)
    elif mode == "split":
        m = np.zeros(d, dtype=np.uint8)
        m[rng.choice(d, 32, replace=False)] = 1
        plan, op = tq.tq_plan_create(d, bits, 2, m, 5), otq.make_split_plan(d, bits, 2, m, 5)
    else:
        plan, op = tq.tq_plan_create(d, bits, 2), otq.make_split_plan(d, bits, 2)
    rb = plan.record_bytes
    before = torch.from_numpy(rng.integers(0, 256, (G * cap, rb), dtype=np.uint8)).to(DEV)
    cache = before.clone()
    X = torch.from_numpy(rng.standard_normal((G + 2, d)).astype(np.float32)).to(DEV).to(getattr(torch, dtype))
    idx = np.concatenate([np.arange(G) * cap + t, [-1, G * cap]]).astype(np.int64)
    tq.tq_encode_scatter(plan, X, cache, torch.from_numpy(idx).to(DEV))
    direct = tq.tq_encode(plan, X[:G])
    torch.cuda.synchronize()
    c, b = cache.cpu().numpy(), before.cpu().numpy()
    rows = idx[:G]
    assert np.array_equal(c[rows], direct.cpu().numpy())
    expect = policy.place(b, direct.cpu().numpy(), idx[:G])
    assert np.array_equal(c, expect)                    # nothing else moved; out-of-range skipped
    Xh = _np64(X[:G])
    if mode == "mse":
        parity.compare_codes_mse(op, otq.encode_mse(op, Xh), layout.unpack_mse(c[rows], op.D, op.R), "append mse")
    else:
        got = parity.unpack_gpu(op, c[rows])
        for i, (p, r, gg) in enumerate(zip(op.plans, otq.encode_split(op, Xh), got)):
            parity.compare_codes(p, r, gg, "append %s sub%d" % (mode, i))


def test_policy_entry_points_reject_bad_arguments():
    x = torch.zeros((10, 16), device=DEV)
    with pytest.raises(tq.TqError):
        tq.tq_calibrate_outliers(x, 17)
    plan = tq.tq_plan_create(16, 3, 0)
    cache = torch.zeros((4, plan.record_bytes), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        tq.tq_encode_scatter(plan, x, cache, torch.zeros(3, dtype=torch.int64, device=DEV))
