"""The TurboQuant-style quantizer and estimator, step by step in fp64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Steps (TurboQuant technical overview, intelliparadigm.com; TurboQuant deep
dive, blog.hotdry.top):
  1. norm split: x is zero-padded to D, n = ||x||, u = x / n (u = 0 if n = 0);
     the norm is stored on its own (overview §4.2.1).
  2. rotation z = Pi u (overview §2.1; oracle/rotation.py).
  3. (b-1)-bit Lloyd-Max scalar quantizer on every coordinate (overview
     §1.2.2, §1.2.3 first stage): idx_i = #{j : t_j <= z_i}, zhat_i = c[idx_i].
  4. residual r = z - zhat (overview §2.3.1), gamma = ||r||.
  5. 1-bit QJL: p = S r with S a k x D Gaussian matrix, beta_j = [p_j >= 0]
     (overview §2.3.2; deep dive §3: one sign bit per dimension, so k = D).
  6. asymmetric estimate against a full-precision query y (deep dive §3:
     high-precision query, low-precision data; overview §4.2.2: the query takes
     the same rotation):
        y' = Pi pad(y),  w = S y',
        est = n * ( <y', zhat> + gamma * sqrt(pi/2) / k * sum_j w_j (2 beta_j - 1) ).
     The constant sqrt(pi/2)/k is not printed on the pages; it is the one that
     makes the estimate unbiased (overview §1.2.3): for a Gaussian row s,
     E[sign(<s, r>) <s, y'>] = sqrt(2/pi) <r, y'> / ||r||.
  7. top-k by estimate, ties broken by the smaller key index (overview §4.2.2,
     first retrieval stage); the second stage re-scores the candidates exactly.

With an outlier mask (overview §4.1.1: a share of outlier channels kept at a
higher bit-width) the channels split into two independent sub-plans, each
padded to its own power of two with its own rotation, codebook and QJL
matrix; the estimate is the sum of the two sub-estimates.

TurboQuant-MSE (overview §1.2.1-1.2.2; §4.1.1 recommends it at 3 bits for most
attention heads, §4.2.1 for the vectors of an index): steps 1-3 with all b bits
on the Lloyd-Max quantizer and no residual stage; the norm is kept.
Dequantization (overview §4.1.2: dequantize in one batch before attention)
inverts the rotation, which is orthogonal: xhat = n * (Pi^T c[idx])[:d].  For
an inner-product plan the same reconstruction uses the (b-1)-bit first stage.
"""
import math
from dataclasses import dataclass

import numpy as np

from . import codebook, philox, rotation

MIN_D = 32
MAX_D = 2048


def padded_length(d):
    """D = smallest power of two >= d, and at least 32 (one 32-bit code word)."""
    D = MIN_D
    while D < d:
        D *= 2
    return D


@dataclass
class Plan:
    d: int                 # channels this (sub-)plan quantizes
    bits: int              # b: total bits per coordinate (b-1 MSE + 1 QJL)
    seed: int
    subset: int            # 0 regular channels, 1 outlier channels
    D: int
    R: int
    k: int
    levels: np.ndarray     # 2^R ascending, fp64
    thresholds: np.ndarray  # 2^R - 1 ascending, fp64
    signs: np.ndarray      # (3, D) +-1
    S: np.ndarray          # (k, D), bf16-valued fp64 (None for an MSE plan)
    mse: bool = False      # TurboQuant-MSE: R = b, no QJL stage


def make_plan(d, bits, seed, subset=0):
    D = padded_length(d)
    R = bits - 1
    levels, thresholds = codebook.solve_codebook(D, R)
    signs = philox.rotation_signs(seed, subset, D)
    S = philox.qjl_matrix(seed, subset, D, D)
    return Plan(d=d, bits=bits, seed=seed, subset=subset, D=D, R=R, k=D,
                levels=levels, thresholds=thresholds, signs=signs, S=S)


def make_mse_plan(d, bits, seed):
    """TurboQuant-MSE plan: a b-bit Lloyd-Max codebook for the rotated-coordinate law and
    the same rotation a plan with this seed uses; no QJL matrix."""
    D = padded_length(d)
    levels, thresholds = codebook.solve_codebook(D, bits)
    signs = philox.rotation_signs(seed, 0, D)
    return Plan(d=d, bits=bits, seed=seed, subset=0, D=D, R=bits, k=0,
                levels=levels, thresholds=thresholds, signs=signs, S=None, mse=True)


@dataclass
class SplitPlan:
    """Sub-plans over channel subsets (one subset when there is no mask)."""
    d: int
    channels: list          # per sub-plan: int array of channel indices
    plans: list


def make_split_plan(d, bits, seed, mask=None, outlier_bits=0):
    if mask is None:
        return SplitPlan(d=d, channels=[np.arange(d)], plans=[make_plan(d, bits, seed, 0)])
    mask = np.asarray(mask).astype(bool)
    reg = np.nonzero(~mask)[0]
    out = np.nonzero(mask)[0]
    return SplitPlan(d=d, channels=[reg, out],
                     plans=[make_plan(len(reg), bits, seed, 0),
                            make_plan(len(out), outlier_bits, seed, 1)])


def pad(X, D):
    X = np.asarray(X, dtype=np.float64)
    out = np.zeros(X.shape[:-1] + (D,))
    out[..., :X.shape[-1]] = X
    return out


def bucketize(z, thresholds):
    """idx = number of thresholds t_j with t_j <= z."""
    return np.sum(z[..., None] >= thresholds, axis=-1)


def qjl_signs(S, r):
    """beta_j = 1 if (S r)_j >= 0 else 0, for each row r."""
    p = r @ S.T
    return (p >= 0).astype(np.uint8), p


def unit_rotated(Xp, signs):
    """(norm, z) with z = Pi (x / ||x||) for each row x of Xp (z = 0 for a zero row).  Pi is
    linear, so the row is rotated first and divided by its norm afterwards: the Hadamard
    rounds then act on the stored values themselves, exactly when these carry few significant
    bits, and a rotated coordinate that is exactly zero stays zero instead of picking up a
    rounding residue of either sign (which would move it across a threshold at 0)."""
    norm = np.sqrt(np.sum(Xp * Xp, axis=-1))
    safe = np.where(norm > 0, norm, 1.0)
    z = np.where(norm[:, None] > 0, rotation.rotate(Xp, signs) / safe[:, None], 0.0)
    return norm, z


def encode(plan, X):
    """Codes of the rows of X (n x d): dict with idx (n, D), beta (n, k),
    norm (n,), gamma (n,), and the intermediates z, r, p."""
    Xp = pad(X, plan.D)
    norm, z = unit_rotated(Xp, plan.signs)
    idx = bucketize(z, plan.thresholds)
    zhat = plan.levels[idx]
    r = z - zhat
    gamma = np.sqrt(np.sum(r * r, axis=-1))
    beta, p = qjl_signs(plan.S, r)
    return dict(idx=idx, beta=beta, norm=norm, gamma=gamma, z=z, r=r, p=p)


def qjl_given_idx(plan, z, idx):
    """Steps 4-5 of `encode` for rotated directions z whose cells were chosen elsewhere:
    r = z - c[idx], gamma = ||r||, p = S r, beta = [p >= 0].  A coordinate within rounding of
    a threshold may be placed in either neighbouring cell; the residual, and with it the sign
    bits, then follow the cell actually chosen (overview §2.3.1-2.3.2: the residual is the
    error of the first stage as quantized).  Returns dict(r, gamma, p, beta)."""
    r = np.asarray(z, dtype=np.float64) - plan.levels[np.asarray(idx)]
    gamma = np.sqrt(np.sum(r * r, axis=-1))
    beta, p = qjl_signs(plan.S, r)
    return dict(r=r, gamma=gamma, p=p, beta=beta)


def encode_mse(plan, X):
    """TurboQuant-MSE codes of the rows of X (n x d): dict with idx (n, D), norm (n,) and
    the rotated direction z."""
    Xp = pad(X, plan.D)
    norm, z = unit_rotated(Xp, plan.signs)
    return dict(idx=bucketize(z, plan.thresholds), norm=norm, z=z)


def dequantize(plan, codes):
    """xhat = n * (Pi^T c[idx])[:d] for each stored vector: the centroids of its cells taken
    back through the inverse rotation and scaled by its norm (uses idx and norm only)."""
    zhat = plan.levels[np.asarray(codes["idx"])]
    return np.asarray(codes["norm"])[:, None] * rotation.unrotate(zhat, plan.signs)[:, :plan.d]


def score_mse(plan, codes, Y):
    """est[q, n] from TurboQuant-MSE codes (uses idx and norm only).  The overview's quantized
    distance (§4.2.2) rotates the query with the key rotation and sums, coordinate by
    coordinate, the query value against the centroid of the key's cell; the index keeps the
    norm apart (§4.2.1), so the sum is scaled by it:
        est = n * <Pi pad(y), c[idx]>.
    The query stays at full precision, as for the inner-product estimate (the page's sketch
    also quantizes it; the asymmetric reading is the deep dive's, §三).  This is the plain
    inner product of y with the reconstruction of `dequantize`, since Pi is orthogonal.  For an
    inner-product plan the same sum over the (b-1)-bit first stage is the first term of
    `score`.  The estimate is biased: the cell centroids shrink it, and over random rotations
    its mean is <x, y> (1 - D E[(Z - c(Z))^2]) with Z a rotated coordinate."""
    yr = rotation.rotate(pad(Y, plan.D), plan.signs)
    zhat = plan.levels[np.asarray(codes["idx"])]
    return np.asarray(codes["norm"])[None, :] * (yr @ zhat.T)


def dequantize_split(sp, codes_list):
    """Per sub-plan reconstruction, each written back to its own channels."""
    n = len(codes_list[0]["norm"])
    out = np.zeros((n, sp.d))
    for p, c, ch in zip(sp.plans, codes_list, sp.channels):
        out[:, ch] = dequantize(p, c)
    return out


def prepare_query(plan, Y):
    """y' = Pi pad(y) and w = S y' for each row y of Y."""
    yr = rotation.rotate(pad(Y, plan.D), plan.signs)
    return yr, yr @ plan.S.T


def qjl_constant(k):
    return math.sqrt(math.pi / 2.0) / k


def score(plan, codes, Y):
    """est[q, n] for every query row of Y against every encoded key (per-key
    centroid lookup summed with the query coordinates, plus the QJL term)."""
    yr, w = prepare_query(plan, Y)
    zhat = plan.levels[codes["idx"]]                      # (n, D)
    mse_term = yr @ zhat.T                                # (nq, n)
    s = 2.0 * codes["beta"].astype(np.float64) - 1.0      # (n, k)
    qjl_term = (w @ s.T) * (codes["gamma"][None, :] * qjl_constant(plan.k))
    return codes["norm"][None, :] * (mse_term + qjl_term)


def score_by_reconstruction(plan, codes, Y):
    """The same estimate computed another way: reconstruct the key's rotated
    direction zhat + gamma sqrt(pi/2)/k S^T (2 beta - 1), scale by n, and take
    the plain inner product with the rotated query."""
    yr = rotation.rotate(pad(Y, plan.D), plan.signs)
    s = 2.0 * codes["beta"].astype(np.float64) - 1.0
    recon = plan.levels[codes["idx"]] + \
        (codes["gamma"] * qjl_constant(plan.k))[:, None] * (s @ plan.S)
    return yr @ (recon * codes["norm"][:, None]).T


def encode_split(sp, X):
    return [encode(p, np.asarray(X)[..., ch]) for p, ch in zip(sp.plans, sp.channels)]


def score_split(sp, codes_list, Y):
    Y = np.asarray(Y)
    return sum(score(p, c, Y[..., ch]) for p, c, ch in zip(sp.plans, codes_list, sp.channels))


def attend(vplan, logits, vcodes, scale, nq_per_group):
    """Decode attention over quantized values (overview §4.1.2: the cache is dequantized in
    one batch for the attention step; the attention arithmetic itself is the model's, taken
    here in its plain form): for query row r of group g = r // nq_per_group,
        p = softmax(scale * logits[r]) over the group's n tokens,
        out[r] = sum_j p_j vhat_j,
    with vhat the dequantized value vectors of group g (vcodes holds n_groups * n records,
    group after group).  Returns (rows, d) fp64."""
    logits = np.asarray(logits, dtype=np.float64)
    rows, n = logits.shape
    V = dequantize(vplan, vcodes)
    out = np.zeros((rows, V.shape[1]))
    for r in range(rows):
        g = r // nq_per_group
        l = scale * logits[r]
        e = np.exp(l - l.max())
        out[r] = (e / e.sum()) @ V[g * n:(g + 1) * n]
    return out


def rerank(Y, X, cand, k):
    """Second stage of two-stage retrieval (overview §4.2.2: the quantized first stage screens
    a top-K, the second refines on the candidate set): for each query row y of Y, the exact
    inner products <y, x_j> with the full-precision rows x_j of X for j in cand[q] (ids
    outside [0, n) are ignored), and the k best of them ordered by (-value, id).  Returns
    (ids, values); slots past the valid candidates hold id -1 and value -inf."""
    Y = np.asarray(Y, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    cand = np.asarray(cand)
    n = X.shape[0]
    ids = np.full((Y.shape[0], k), -1, dtype=np.int64)
    vals = np.full((Y.shape[0], k), -np.inf)
    for q in range(Y.shape[0]):
        c = np.unique(cand[q][(cand[q] >= 0) & (cand[q] < n)])
        v = X[c] @ Y[q]
        order = np.lexsort((c, -v))[:k]
        ids[q, :len(order)] = c[order]
        vals[q, :len(order)] = v[order]
    return ids, vals


def topk(est, k):
    """Per row: the k largest estimates, ordered by (-estimate, key index)."""
    est = np.asarray(est)
    n = est.shape[-1]
    ids = np.empty(est.shape[:-1] + (k,), dtype=np.int64)
    vals = np.empty(est.shape[:-1] + (k,), dtype=est.dtype)
    for q in np.ndindex(est.shape[:-1]):
        order = np.lexsort((np.arange(n), -est[q]))[:k]
        ids[q] = order
        vals[q] = est[q][order]
    return ids, vals
