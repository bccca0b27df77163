"""Lloyd-Max scalar quantizer for the coordinate law of a randomly rotated unit vector.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Law: after a random rotation, one coordinate T of a unit vector in D dimensions
follows a symmetric Beta law, T = 2B - 1 with B ~ Beta((D-1)/2, (D-1)/2), i.e.
density f(t) proportional to (1 - t^2)^((D-3)/2) on [-1, 1], which tends to
N(0, 1/D) (TurboQuant technical overview, intelliparadigm.com, §1.2.1 and
§2.2.1).  D is the rotated (zero-padded, power-of-two) length.

Quantizer: per-coordinate Lloyd-Max, alternating "centroids from boundaries"
and "boundaries from centroids" until the boundaries stop moving (same page,
§1.2.2 pseudo-code and §2.2.2 precompute flow).  Boundaries are midpoints of
adjacent levels; a level is the conditional mean of its cell.

The page's initializer is "uniform"; read here as uniform boundaries over
[-4/sqrt(D), 4/sqrt(D)] (the bulk of the law) rather than over [-1, 1], which
would leave cells with no mass at large D.  The law is log-concave for
D >= 3, so the fixed point is unique and the initializer only affects the
iteration count.
"""
import numpy as np
from scipy import special, stats


def _beta_alpha(D):
    return (D - 1) / 2.0


def beta_cell_mass(D, lo, hi):
    """P(lo < T < hi) via the regularized incomplete Beta function."""
    a = _beta_alpha(D)
    return special.betainc(a, a, (1.0 + np.asarray(hi)) / 2.0) - \
        special.betainc(a, a, (1.0 + np.asarray(lo)) / 2.0)


def beta_cell_first_moment(D, lo, hi):
    """E[T ; lo < T < hi] = [(1-lo^2)^a - (1-hi^2)^a] / (2 a Z), Z = 2^(2a-1) B(a, a).

    Uses d/dt (1-t^2)^a = -2 a t (1-t^2)^(a-1); evaluated in log space."""
    a = _beta_alpha(D)
    log_z = (2 * a - 1) * np.log(2.0) + special.betaln(a, a)

    def term(t):
        t = np.asarray(t, dtype=np.float64)
        one_minus = 1.0 - t * t
        with np.errstate(divide="ignore"):
            lg = a * np.log(np.maximum(one_minus, 0.0))
        return np.exp(lg - np.log(2 * a) - log_z)

    return term(lo) - term(hi)


def gaussian_cell_mass(lo, hi):
    return stats.norm.cdf(hi) - stats.norm.cdf(lo)


def gaussian_cell_first_moment(lo, hi):
    """E[Z ; lo < Z < hi] = phi(lo) - phi(hi) for Z ~ N(0, 1)."""
    return stats.norm.pdf(lo) - stats.norm.pdf(hi)


def lloyd_max(mass, first_moment, support, init_thresholds, tol, max_iter):
    """Plain Lloyd iteration: centroids <- cell means; thresholds <- midpoints.

    Returns (levels, thresholds, iterations)."""
    t = np.array(init_thresholds, dtype=np.float64)
    lo_end, hi_end = support
    it = 0
    while True:
        edges = np.concatenate([[lo_end], t, [hi_end]])
        levels = first_moment(edges[:-1], edges[1:]) / mass(edges[:-1], edges[1:])
        t_new = 0.5 * (levels[:-1] + levels[1:])
        it += 1
        moved = np.max(np.abs(t_new - t)) if t.size else 0.0
        t = t_new
        if moved <= tol or it >= max_iter:
            break
    edges = np.concatenate([[lo_end], t, [hi_end]])
    levels = first_moment(edges[:-1], edges[1:]) / mass(edges[:-1], edges[1:])
    return levels, t, it


def solve_codebook(D, R, tol_rel=1e-13, max_iter=400000):
    """Lloyd-Max levels (2^R, ascending) and thresholds (2^R - 1) for the law of
    one rotated coordinate in D dimensions.

    The law is symmetric about 0 (a Beta law with equal parameters), so the
    optimal quantizer is odd-symmetric: the levels returned are mirrored
    exactly (c_l = -c_{L-1-l}) and the thresholds are their midpoints, which
    puts the middle threshold exactly at 0 (a zero coordinate counts as >= it)."""
    L = 2 ** R
    s = 1.0 / np.sqrt(D)
    span = min(4.0 * s, 0.999)
    init = -span + 2.0 * span * np.arange(1, L) / L
    levels, t, _ = lloyd_max(lambda lo, hi: beta_cell_mass(D, lo, hi),
                             lambda lo, hi: beta_cell_first_moment(D, lo, hi),
                             (-1.0, 1.0), init, tol_rel * s, max_iter)
    levels = 0.5 * (levels - levels[::-1])
    return levels, 0.5 * (levels[:-1] + levels[1:])


def solve_gaussian_codebook(R, tol=1e-13, max_iter=400000):
    """Lloyd-Max levels and thresholds for N(0, 1) (the large-D limit)."""
    L = 2 ** R
    init = -4.0 + 8.0 * np.arange(1, L) / L
    levels, t, _ = lloyd_max(gaussian_cell_mass, gaussian_cell_first_moment,
                             (-np.inf, np.inf), init, tol, max_iter)
    return levels, t


def codebook_mse(D, levels, thresholds):
    """E(T - Q(T))^2 = E T^2 - sum_l P_l c_l^2 (levels are cell means; E T^2 = 1/D)."""
    edges = np.concatenate([[-1.0], thresholds, [1.0]])
    p = beta_cell_mass(D, edges[:-1], edges[1:])
    return 1.0 / D - float(np.sum(p * levels ** 2))
