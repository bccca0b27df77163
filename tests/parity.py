"""Comparison rules between the HIP path and the fp64 oracle.

Codes: quantizer indices must be identical except at coordinates whose rotated
value lies within 1e-5 (relative) of a decision threshold; QJL bits identical
except where the projection lies within 1e-5 (relative) of zero; such in-band
mismatches may make up at most 1e-5 of all coordinates / bits.  Bits of a
vector whose indices differ (an in-band cell change moves the residual) are
not compared.  Norms and residual norms: fp32 vs fp64.  Scores:
|est_gpu - est_oracle| <= 1e-3 ||q|| ||x|| for every pair.
"""
import numpy as np

from oracle import layout
from oracle import turboquant as otq

BAND = 1e-5
MISMATCH_FRACTION = 1e-5
SCORE_TOL = 1e-3


def code_band(plan, z):
    """True where a coordinate of z lies within the relative band of a threshold."""
    t = plan.thresholds
    scale = np.maximum(np.abs(t), 1.0 / np.sqrt(plan.D))
    return np.any(np.abs(z[..., None] - t) <= BAND * scale, axis=-1)


def sign_band(plan, r, p):
    """True where a projection lies within the relative band of zero."""
    row_norm = np.linalg.norm(plan.S, axis=1)
    return np.abs(p) <= BAND * row_norm[None, :] * np.linalg.norm(r, axis=1)[:, None]


def compare_codes(plan, ocodes, gcodes, what=""):
    """ocodes: oracle encode dict; gcodes: unpacked GPU codes.  Returns a stats dict."""
    idx_mis = ocodes["idx"] != gcodes["idx"]
    band = code_band(plan, ocodes["z"])
    out_of_band = idx_mis & ~band
    assert not out_of_band.any(), "%s: %d index mismatches outside the band (first at %s)" % (
        what, int(out_of_band.sum()), np.argwhere(out_of_band)[:3].tolist())
    n_idx = idx_mis.sum()
    assert n_idx <= max(1, MISMATCH_FRACTION * idx_mis.size) or n_idx == 0, \
        "%s: %d in-band index mismatches of %d" % (what, n_idx, idx_mis.size)
    same = ~idx_mis.any(axis=1)
    b_mis = (ocodes["beta"] != gcodes["beta"]) & same[:, None]
    sband = sign_band(plan, ocodes["r"], ocodes["p"])
    b_out = b_mis & ~sband
    assert not b_out.any(), "%s: %d sign mismatches outside the band (first at %s)" % (
        what, int(b_out.sum()), np.argwhere(b_out)[:3].tolist())
    assert b_mis.sum() <= max(1, MISMATCH_FRACTION * b_mis.size), \
        "%s: %d in-band sign mismatches" % (what, b_mis.sum())
    nrm_rel = np.abs(gcodes["norm"] - ocodes["norm"]) / np.maximum(ocodes["norm"], 1e-30)
    assert np.all(nrm_rel[ocodes["norm"] > 0] <= 1e-6), "%s: norm rel err %g" % (what, nrm_rel.max())
    assert np.all(gcodes["norm"][ocodes["norm"] == 0] == 0)
    g_rel = np.abs(gcodes["gamma"] - ocodes["gamma"]) / np.maximum(ocodes["gamma"], 1e-30)
    g_rel = g_rel[same]
    assert np.all(g_rel <= 1e-5), "%s: gamma rel err %g" % (what, g_rel.max())
    return dict(idx_mismatch=int(n_idx), sign_mismatch=int(b_mis.sum()),
                vectors_same_idx=int(same.sum()), norm_rel=float(nrm_rel.max()),
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
    return float(np.max(err / np.maximum(bound, 1e-30)))


def check_topk(ids_gpu, vals_gpu, est_ref, k, qnorm, xnorm, what=""):
    """ids identical to the oracle's top-k except for ties within the score tolerance."""
    ids_ref, vals_ref = otq.topk(est_ref, k)
    for q in range(est_ref.shape[0]):
        a, b = set(ids_gpu[q].tolist()), set(ids_ref[q].tolist())
        if a == b:
            continue
        kth = vals_ref[q, -1]
        for i in a - b:
            tol = SCORE_TOL * qnorm[q] * max(xnorm[i], xnorm[ids_ref[q, -1]])
            assert est_ref[q, i] >= kth - tol, "%s: query %d id %d not near the k-th" % (what, q, i)


def unpack_gpu(sp, codes_u8):
    return layout.unpack_split(sp, codes_u8)


def compare_codes_mse(plan, ocodes, gcodes, what=""):
    """TurboQuant-MSE codes: indices as in compare_codes (exact outside the band), norms to
    1e-6 relative, zero norms exact."""
    idx_mis = ocodes["idx"] != gcodes["idx"]
    out_of_band = idx_mis & ~code_band(plan, ocodes["z"])
    assert not out_of_band.any(), "%s: %d index mismatches outside the band (first at %s)" % (
        what, int(out_of_band.sum()), np.argwhere(out_of_band)[:3].tolist())
    n_idx = idx_mis.sum()
    assert n_idx <= max(1, MISMATCH_FRACTION * idx_mis.size), \
        "%s: %d in-band index mismatches of %d" % (what, n_idx, idx_mis.size)
    nrm_rel = np.abs(gcodes["norm"] - ocodes["norm"]) / np.maximum(ocodes["norm"], 1e-30)
    assert np.all(nrm_rel[ocodes["norm"] > 0] <= 1e-6), "%s: norm rel err %g" % (what, nrm_rel.max())
    assert np.all(gcodes["norm"][ocodes["norm"] == 0] == 0)
    return dict(idx_mismatch=int(n_idx), norm_rel=float(nrm_rel.max()))


def check_dequantized(x_gpu, x_ref, norms, bf16, what=""):
    """Reconstruction vs the oracle's on the same codes: within 2e-6 of the vector norm per
    element (fp32 transform rounding), plus half a bf16 step of the value for bf16 output."""
    tol = 2e-6 * norms[:, None] + (2.0 ** -8 * np.abs(x_ref) if bf16 else 0.0)
    err = np.abs(x_gpu - x_ref)
    bad = err > tol
    assert not bad.any(), "%s: %d elements off (max err/tol %g)" % (
        what, int(bad.sum()), float(np.max(err / np.maximum(tol, 1e-30))))
    return float(np.max(err / np.maximum(tol, 1e-30)))
