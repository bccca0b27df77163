"""Comparison rules between the HIP path and the fp64 oracle.

Codes: quantizer indices must be identical except at coordinates whose rotated value lies
within 1e-5 (relative) of a decision threshold; such in-band mismatches may make up at most
1e-5 of all coordinates (no floor: one mismatch among fewer than 1e5 coordinates fails).
QJL bits: identical except where the projection lies within 1e-5 (relative) of zero, with the
same 1e-5 budget.  For a vector whose cells match the oracle's, the bits are compared with
the oracle's own encode; for a vector with an in-band cell change, with the oracle's residual,
projection and signs recomputed from the GPU's cells (a moved cell moves the residual, and
with it many signs legitimately).  Norms: 1e-6 relative (fp32 vs fp64).  Residual norms:
1e-6 of gamma plus 2^-22 (four fp32 ulps of ||z|| = 1): gamma = ||z - c[idx]|| is formed from
the rotated coordinates, whose fp32 rounding is a few ulps of ||z|| however small gamma is.
Scores: |est_gpu - est_oracle| <= 1e-3 ||q|| ||x|| for every pair, against the oracle's own
codes where the codes are identical and against the oracle evaluated on the GPU's codes
elsewhere.  Top-k: distinct ids in (-value, id) order, every value within tolerance of the
oracle's estimate of its id, ranks within tolerance of the oracle's ranks, and ids outside the
oracle's top-k only where the oracle's k-th value is within tolerance.
"""
import numpy as np

from oracle import layout
from oracle import turboquant as otq

BAND = 1e-5
MISMATCH_FRACTION = 1e-5
NORM_REL = 1e-6
GAMMA_REL = 1e-6
GAMMA_ABS = 2.0 ** -22     # in the unit domain of the oracle's z (||z|| = 1)
SCORE_TOL = 1e-3

# largest deviations seen in this process (reported at the end of a test session)
STATS = dict(norm_rel=0.0, gamma_rel=0.0, gamma_ratio=0.0, idx_mismatch=0, idx_compared=0, sign_mismatch=0,
             sign_compared=0, vectors_recomputed=0, score_ratio=0.0)


def _note(key, value, op=max):
    STATS[key] = op(STATS[key], value)


def code_band(plan, z):
    """True where a coordinate of z lies within the relative band of a threshold."""
    t = plan.thresholds
    scale = np.maximum(np.abs(t), 1.0 / np.sqrt(plan.D))
    return np.any(np.abs(z[..., None] - t) <= BAND * scale, axis=-1)


def sign_band(plan, r, p):
    """True where a projection lies within the relative band of zero."""
    row_norm = np.linalg.norm(plan.S, axis=1)
    return np.abs(p) <= BAND * row_norm[None, :] * np.linalg.norm(r, axis=1)[:, None]


def _check_norms(ocodes, gcodes, what):
    on, gn = np.asarray(ocodes["norm"]), np.asarray(gcodes["norm"])
    nrm_rel = np.abs(gn - on) / np.maximum(on, 1e-300)
    nrm_rel = np.where(on > 0, nrm_rel, 0.0)
    assert np.all(nrm_rel <= NORM_REL), "%s: norm rel err %g" % (what, nrm_rel.max())
    assert np.all(gn[on == 0] == 0), "%s: zero vector with a nonzero norm" % what
    _note("norm_rel", float(nrm_rel.max()) if nrm_rel.size else 0.0)
    return float(nrm_rel.max()) if nrm_rel.size else 0.0


def _check_indices(plan, ocodes, gcodes, what):
    idx_mis = ocodes["idx"] != gcodes["idx"]
    out_of_band = idx_mis & ~code_band(plan, ocodes["z"])
    assert not out_of_band.any(), "%s: %d index mismatches outside the band (first at %s)" % (
        what, int(out_of_band.sum()), np.argwhere(out_of_band)[:3].tolist())
    n_idx = int(idx_mis.sum())
    assert n_idx <= MISMATCH_FRACTION * idx_mis.size, \
        "%s: %d in-band index mismatches of %d" % (what, n_idx, idx_mis.size)
    _note("idx_mismatch", n_idx, lambda a, b: a + b)
    _note("idx_compared", int(idx_mis.size), lambda a, b: a + b)
    return idx_mis


def compare_codes(plan, ocodes, gcodes, what=""):
    """ocodes: oracle encode dict; gcodes: unpacked GPU codes.  Returns a stats dict."""
    idx_mis = _check_indices(plan, ocodes, gcodes, what)
    same = ~idx_mis.any(axis=1)
    beta = np.array(ocodes["beta"])
    r, p, gamma = np.array(ocodes["r"]), np.array(ocodes["p"]), np.array(ocodes["gamma"])
    moved = np.flatnonzero(~same)
    if moved.size:
        q = otq.qjl_given_idx(plan, ocodes["z"][moved], gcodes["idx"][moved])
        beta[moved], r[moved], p[moved], gamma[moved] = q["beta"], q["r"], q["p"], q["gamma"]
        _note("vectors_recomputed", int(moved.size), lambda a, b: a + b)
    b_mis = beta != gcodes["beta"]
    b_out = b_mis & ~sign_band(plan, r, p)
    assert not b_out.any(), "%s: %d sign mismatches outside the band (first at %s)" % (
        what, int(b_out.sum()), np.argwhere(b_out)[:3].tolist())
    assert b_mis.sum() <= MISMATCH_FRACTION * b_mis.size, \
        "%s: %d in-band sign mismatches of %d" % (what, int(b_mis.sum()), b_mis.size)
    _note("sign_mismatch", int(b_mis.sum()), lambda a, b: a + b)
    _note("sign_compared", int(b_mis.size), lambda a, b: a + b)
    nrm_rel = _check_norms(ocodes, gcodes, what)
    g_err = np.abs(gcodes["gamma"] - gamma)
    g_rel = g_err / np.maximum(gamma, 1e-300)
    g_ratio = g_err / (GAMMA_REL * gamma + GAMMA_ABS)
    assert np.all(g_ratio <= 1.0), "%s: gamma err %g (rel err %g, vector %d)" % (
        what, g_err.max(), g_rel[np.argmax(g_ratio)], int(np.argmax(g_ratio)))
    _note("gamma_rel", float(g_rel.max()) if g_rel.size else 0.0)
    _note("gamma_ratio", float(g_ratio.max()) if g_ratio.size else 0.0)
    return dict(idx_mismatch=int(idx_mis.sum()), sign_mismatch=int(b_mis.sum()),
                vectors_same_idx=int(same.sum()), norm_rel=nrm_rel,
                gamma_rel=float(g_rel.max()) if g_rel.size else 0.0)


def stored(codes):
    """The oracle codes as they are stored (fp32 norm and gamma)."""
    c = dict(codes)
    c["norm"] = np.asarray(codes["norm"], dtype=np.float32).astype(np.float64)
    c["gamma"] = np.asarray(codes["gamma"], dtype=np.float32).astype(np.float64)
    return c


def check_scores(est_gpu, est_ref, qnorm, xnorm, what=""):
    bound = SCORE_TOL * qnorm[:, None] * xnorm[None, :]
    err = np.abs(est_gpu - est_ref)
    bad = err > bound
    assert not bad.any(), "%s: %d score errors above 1e-3|q||x| (max ratio %g)" % (
        what, int(bad.sum()), float(np.max(err / np.maximum(bound, 1e-30))))
    ratio = float(np.max(err / np.maximum(bound, 1e-30))) if err.size else 0.0
    _note("score_ratio", ratio)
    return ratio


def identical_vectors(ocodes_list, gcodes_list):
    """Vectors whose cells and sign bits are identical in every sub-plan."""
    same = np.ones(len(ocodes_list[0]["idx"]), dtype=bool)
    for o, g in zip(ocodes_list, gcodes_list):
        same &= np.all(o["idx"] == g["idx"], 1)
        if "beta" in o:
            same &= np.all(o["beta"] == g["beta"], 1)
    return same


def oracle_scores_on_gpu_codes(sp, gcodes_list, Y):
    """The oracle's estimate evaluated on the GPU's codes (its cells, signs, fp32 norms)."""
    return otq.score_split(sp, gcodes_list, np.asarray(Y, dtype=np.float64))


def check_scores_end_to_end(sp, ocodes_list, gcodes_list, est_gpu, Y, X, what=""):
    """Every pair: vectors with identical codes against the oracle's own codes (stored in
    fp32), the others against the oracle evaluated on the GPU's codes.  Returns the fraction
    of identical vectors."""
    same = identical_vectors(ocodes_list, gcodes_list)
    qn = np.linalg.norm(np.asarray(Y, dtype=np.float64), axis=1)
    xn = np.linalg.norm(np.asarray(X, dtype=np.float64), axis=1)
    est_own = otq.score_split(sp, [stored(c) for c in ocodes_list], np.asarray(Y, np.float64))
    check_scores(est_gpu[:, same], est_own[:, same], qn, xn[same], what + " (identical codes)")
    if (~same).any():
        est_g = oracle_scores_on_gpu_codes(sp, [{k: v[~same] for k, v in g.items()}
                                                for g in gcodes_list], Y)
        check_scores(est_gpu[:, ~same], est_g, qn, xn[~same], what + " (GPU codes)")
    return float(same.mean())


def check_topk(ids_gpu, vals_gpu, est_ref, k, qnorm, xnorm, what=""):
    """GPU top-k against the oracle's top-k of est_ref, the oracle's estimates for the codes
    the GPU scored.  Per row: k distinct valid ids in (-value, id) order; each value within
    the score tolerance of the oracle's estimate of its id; the i-th value within tolerance
    of the oracle's i-th; an id outside the oracle's top-k only if the oracle rates it within
    tolerance of its k-th value."""
    ids_ref, vals_ref = otq.topk(est_ref, k)
    n = est_ref.shape[1]
    for q in range(est_ref.shape[0]):
        ids, vals = np.asarray(ids_gpu[q], dtype=np.int64), np.asarray(vals_gpu[q], np.float64)
        assert len(ids) == k and np.all((ids >= 0) & (ids < n)), "%s: query %d bad ids" % (what, q)
        assert len(np.unique(ids)) == k, "%s: query %d repeats an id" % (what, q)
        ordered = (vals[:-1] > vals[1:]) | ((vals[:-1] == vals[1:]) & (ids[:-1] < ids[1:]))
        assert ordered.all(), "%s: query %d not in (-value, id) order" % (what, q)
        tol_id = SCORE_TOL * qnorm[q] * xnorm[ids]
        assert np.all(np.abs(vals - est_ref[q, ids]) <= tol_id), \
            "%s: query %d value off the oracle's estimate of its id" % (what, q)
        tol_rank = SCORE_TOL * qnorm[q] * max(float(xnorm[ids].max()), float(xnorm[ids_ref[q]].max()))
        assert np.all(np.abs(vals - vals_ref[q]) <= tol_rank), \
            "%s: query %d ranks differ beyond tolerance" % (what, q)
        kth = vals_ref[q, -1]
        for i in set(ids.tolist()) - set(ids_ref[q].tolist()):
            tol = SCORE_TOL * qnorm[q] * max(xnorm[i], xnorm[ids_ref[q, -1]])
            assert est_ref[q, i] >= kth - tol, "%s: query %d id %d not near the k-th" % (what, q, i)


def unpack_gpu(sp, codes_u8):
    return layout.unpack_split(sp, codes_u8)


def compare_codes_mse(plan, ocodes, gcodes, what=""):
    """TurboQuant-MSE codes: indices as in compare_codes (exact outside the band, at most
    1e-5 in-band mismatches), norms to 1e-6 relative, zero norms exact."""
    idx_mis = _check_indices(plan, ocodes, gcodes, what)
    nrm_rel = _check_norms(ocodes, gcodes, what)
    return dict(idx_mismatch=int(idx_mis.sum()), norm_rel=nrm_rel)


def check_dequantized(x_gpu, x_ref, norms, bf16, what=""):
    """Reconstruction vs the oracle's on the same codes: within 2e-6 of the vector norm per
    element (fp32 transform rounding), plus half a bf16 step of the value for bf16 output."""
    tol = 2e-6 * norms[:, None] + (2.0 ** -8 * np.abs(x_ref) if bf16 else 0.0)
    err = np.abs(x_gpu - x_ref)
    bad = err > tol
    assert not bad.any(), "%s: %d elements off (max err/tol %g)" % (
        what, int(bad.sum()), float(np.max(err / np.maximum(tol, 1e-30))))
    return float(np.max(err / np.maximum(tol, 1e-30)))
