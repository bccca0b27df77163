"""The GPU-vs-oracle comparison rules on the CPU: codes taken from the oracle itself, stored
and unpacked as the library stores them, pass; planted mistakes of the kinds the rules exist
to catch fail."""
import numpy as np
import pytest

from oracle import layout, rotation
from oracle import turboquant as otq
from tests import parity


@pytest.fixture(scope="module")
def case():
    d, n = 128, 1000
    rng = np.random.default_rng(41)
    sp = otq.make_split_plan(d, 3, 4)
    plan = sp.plans[0]
    # vector 0 has coordinate 7 just inside the band of the positive threshold
    z = rng.standard_normal((n, d))
    z /= np.linalg.norm(z, axis=1, keepdims=True)
    t = plan.thresholds[-1]
    others = np.arange(d) != 7
    z[0, others] *= np.sqrt(1 - (t * (1 - 3e-6)) ** 2) / np.linalg.norm(z[0, others])
    z[0, 7] = t * (1 - 3e-6)
    X = rotation.unrotate(z, plan.signs) * 3.0
    ref = otq.encode(plan, X)
    assert parity.code_band(plan, ref["z"])[0, 7]
    got = layout.unpack(layout.pack(parity.stored(ref), plan.D, plan.R), plan.D, plan.R)
    return sp, plan, X, ref, got


def _copy(g):
    return {k: np.array(v) for k, v in g.items()}


def test_oracle_codes_as_stored_pass(case):
    sp, plan, X, ref, got = case
    st = parity.compare_codes(plan, ref, got, "self")
    assert st["idx_mismatch"] == 0 and st["sign_mismatch"] == 0


def test_index_change_outside_the_band_fails(case):
    sp, plan, X, ref, got = case
    g = _copy(got)
    g["idx"][3, 11] = (g["idx"][3, 11] + 1) % (1 << plan.R)
    with pytest.raises(AssertionError, match="outside the band"):
        parity.compare_codes(plan, ref, g, "planted")


def test_in_band_cell_change_checks_signs_from_the_moved_cell(case):
    sp, plan, X, ref, got = case
    g = _copy(got)
    g["idx"][0, 7] += 1                                   # the in-band neighbour cell
    q = otq.qjl_given_idx(plan, ref["z"][:1], g["idx"][:1])
    g["beta"][0] = q["beta"][0]
    g["gamma"][0] = np.float32(q["gamma"][0])
    # 1 of 128000 coordinates: within the 1e-5 budget
    parity.compare_codes(plan, ref, g, "moved cell")
    # the same cell change with the signs of the unmoved residual fails
    g2 = _copy(g)
    g2["beta"][0] = ref["beta"][0]
    g2["gamma"][0] = got["gamma"][0]
    if np.array_equal(q["beta"][0], ref["beta"][0]):
        pytest.skip("moving the cell flipped no sign for this vector")
    with pytest.raises(AssertionError):
        parity.compare_codes(plan, ref, g2, "stale signs")


def test_too_many_in_band_mismatches_fail():
    plan = otq.make_plan(32, 3, 0)
    t = plan.thresholds[-1] * (1 + 1e-7)                  # in band in all three vectors
    z = np.full((3, 32), np.sqrt((1 - t * t) / 31))
    z[:, 0] = t
    ref = otq.encode(plan, rotation.unrotate(z, plan.signs))
    g = {k: np.array(v) for k, v in ref.items()}
    g["idx"][0, 0] -= 1                                    # 1 of 96 coordinates > 1e-5
    q = otq.qjl_given_idx(plan, ref["z"][:1], g["idx"][:1])
    g["beta"][0], g["gamma"][0] = q["beta"][0], q["gamma"][0]
    with pytest.raises(AssertionError, match="in-band index mismatches"):
        parity.compare_codes(plan, ref, g, "budget")


def test_sign_flip_outside_the_band_fails(case):
    sp, plan, X, ref, got = case
    g = _copy(got)
    j = int(np.argmax(np.abs(ref["p"][5])))
    g["beta"][5, j] ^= 1
    with pytest.raises(AssertionError, match="sign mismatches outside the band"):
        parity.compare_codes(plan, ref, g, "planted")


def test_norm_beyond_1e6_fails(case):
    sp, plan, X, ref, got = case
    g = _copy(got)
    g["norm"] = np.asarray(ref["norm"]) * (1 + 2e-6)
    with pytest.raises(AssertionError, match="rel err"):
        parity.compare_codes(plan, ref, g, "planted")


def test_gamma_beyond_its_bound_fails(case):
    """gamma may differ by 1e-6 of itself plus 4 ulps (2^-22) of ||z|| = 1: 1.1 times that
    bound fails (the next test: 0.9 times it passes)."""
    sp, plan, X, ref, got = case
    g = _copy(got)
    gam = np.asarray(ref["gamma"])
    g["gamma"] = gam + 1.1 * (1e-6 * gam + 2.0 ** -22)
    with pytest.raises(AssertionError, match="gamma err"):
        parity.compare_codes(plan, ref, g, "planted")


def test_gamma_within_its_bound_passes(case):
    sp, plan, X, ref, got = case
    g = _copy(got)
    gam = np.asarray(ref["gamma"])
    g["gamma"] = gam + 0.9 * (1e-6 * gam + 2.0 ** -22)
    parity.compare_codes(plan, ref, g, "at the bound")


def test_scores_end_to_end_use_gpu_codes_where_codes_differ(case):
    sp, plan, X, ref, got = case
    rng = np.random.default_rng(42)
    Y = rng.standard_normal((4, 128))
    g = _copy(got)
    g["idx"][0, 7] += 1
    q = otq.qjl_given_idx(plan, ref["z"][:1], g["idx"][:1])
    g["beta"][0], g["gamma"][0] = q["beta"][0], np.float32(q["gamma"][0])
    est = otq.score(plan, g, Y)                          # what a correct scorer gives on g
    assert parity.check_scores_end_to_end(sp, [ref], [g], est, Y, X, "moved") < 1.0
    bad = est.copy()
    bad[:, 0] = otq.score(plan, parity.stored(ref), Y)[:, 0] + 0.05 * np.abs(est[:, 0]).max()
    with pytest.raises(AssertionError):
        parity.check_scores_end_to_end(sp, [ref], [g], bad, Y, X, "planted")


def test_topk_rules():
    rng = np.random.default_rng(43)
    est = rng.standard_normal((3, 500))
    qn, xn = np.ones(3), np.ones(500)
    ids, vals = otq.topk(est, 10)
    parity.check_topk(ids, vals, est, 10, qn, xn, "self")
    dup = ids.copy()
    dup[1, 3] = dup[1, 2]
    with pytest.raises(AssertionError, match="repeats"):
        parity.check_topk(dup, np.take_along_axis(est, dup, 1), est, 10, qn, xn, "dup")
    rev = ids[:, ::-1].copy()
    with pytest.raises(AssertionError, match="order"):
        parity.check_topk(rev, np.take_along_axis(est, rev, 1), est, 10, qn, xn, "order")
    far = ids.copy()
    far[0, -1] = int(np.argmin(est[0]))
    v = np.take_along_axis(est, far, 1)
    o = np.lexsort((far, -v), axis=1)
    far, v = np.take_along_axis(far, o, 1), np.take_along_axis(v, o, 1)
    with pytest.raises(AssertionError):
        parity.check_topk(far, v, est, 10, qn, xn, "far")
