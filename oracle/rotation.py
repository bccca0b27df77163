"""Randomized Hadamard rotation, written out as dense fp64 matrix algebra.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages replace a dense random orthogonal matrix (QR of a Gaussian matrix,
TurboQuant technical overview, intelliparadigm.com, §1.2.1) by a structured
product of Hadamard matrices and random +-1 diagonals with three mixing rounds
(same page, §2.1.1 "structured random matrix" and §2.1.2 OnlineRotation).  The
pages disagree on the order inside a round; this build takes "+-1 diagonal,
then Walsh-Hadamard transform", three times:

    Pi = Ht S3 Ht S2 Ht S1,   Ht = H_D / sqrt(D),

with H_D the Sylvester Hadamard matrix, (H_D)_ij = (-1)^popcount(i & j), and
S_r the fixed diagonals of the plan (drawn once from the seed, not per call,
since queries must see the same rotation as keys: same page, §4.2.2).
Each Ht is orthonormal, so Pi is orthogonal.
"""
import numpy as np


def popcount(a):
    a = np.asarray(a, dtype=np.int64)
    c = np.zeros_like(a)
    while np.any(a):
        c += a & 1
        a = a >> 1
    return c


def sylvester_hadamard(D):
    """H_D with entries (-1)^popcount(i & j)."""
    i = np.arange(D)
    return np.where(popcount(i[:, None] & i[None, :]) % 2 == 0, 1.0, -1.0)


def rotate(U, signs):
    """Rows of U (n x D) mapped through Pi: for each round r, multiply by the
    diagonal S_r, then by the Hadamard matrix; the three 1/sqrt(D) factors of
    Ht = H_D / sqrt(D) are applied together as one final D^(-3/2).  With the
    integer matrix H_D the transform is exact for inputs with few significant
    bits, so coordinates that are exactly zero stay exactly zero."""
    D = U.shape[-1]
    H = sylvester_hadamard(D)
    Z = np.asarray(U, dtype=np.float64)
    for r in range(3):
        Z = (Z * signs[r][None, :]) @ H.T
    return Z * float(D) ** -1.5


def unrotate(Z, signs):
    """Rows of Z mapped through Pi^T = S1 Ht S2 Ht S3 Ht, the inverse of `rotate` since Pi is
    orthogonal: for each round from the last, multiply by the Hadamard matrix, then by that
    round's diagonal; the three 1/sqrt(D) factors are applied together at the end."""
    D = Z.shape[-1]
    H = sylvester_hadamard(D)
    U = np.asarray(Z, dtype=np.float64)
    for r in (2, 1, 0):
        U = (U @ H.T) * signs[r][None, :]
    return U * float(D) ** -1.5


def rotation_matrix(signs):
    """Pi as a dense D x D matrix (column j = Pi e_j)."""
    D = signs.shape[1]
    return rotate(np.eye(D), signs).T


def haar_rotation(D, rng):
    """Dense Haar-random orthogonal matrix (QR of a Gaussian matrix with the
    sign fix that makes the law exactly Haar), used only as a cross-check of
    the coordinate law."""
    G = rng.standard_normal((D, D))
    Q, Rm = np.linalg.qr(G)
    return Q * np.sign(np.diag(Rm))[None, :]
