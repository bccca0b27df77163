"""Counter-based randomness for the plan: Philox4x32-10 and fp64 Box-Muller.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages ask for the rotation signs and the QJL projection to be produced by
a pseudo-random generator from a seed instead of being stored (TurboQuant
technical overview, intelliparadigm.com, §2.1.2 "online computation avoids
storage" and §2.3.2 "QJL transform", engineering note).  They name no
generator.  This build fixes Philox4x32-10, written here from its published
definition (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
1, 2, 3", SC'11): a 4-word counter and 2-word key, ten rounds, each round two
32x32->64 multiplications whose high halves are XOR-ed with the key and the
other counter words, the key advanced by the two Weyl constants between
rounds.  Gaussians use the Box-Muller transform (Box & Muller, 1958) in fp64.

Counter layout (shared definition, implemented independently by the library):
  key  = (seed mod 2^32, seed >> 32)
  ctr  = (block mod 2^32, block >> 32, domain, 0)
  domain = purpose << 24 | subset << 16 | round << 8
  purpose 1 = rotation signs (round 0, 1, 2), purpose 2 = QJL Gaussian (round 0)
  subset 0 = regular channels, 1 = outlier channels.
Each block yields four 32-bit words w0..w3.
"""
import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85

PURPOSE_SIGNS = 1
PURPOSE_GAUSS = 2


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox4x32 rounds on arrays of counters and keys (32-bit values, broadcast).

    Returns four uint64 arrays holding the 32-bit output words."""
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    k0 = np.asarray(k0, dtype=np.uint64) & MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & MASK32
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(c0, c1, c2, c3, k0, k1)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & MASK32
        p0 = PHILOX_M0 * c0          # < 2^64, exact in uint64
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def domain_word(purpose, subset, rnd):
    return (purpose << 24) | (subset << 16) | (rnd << 8)


def stream_words(seed, purpose, subset, rnd, n_blocks):
    """The 4*n_blocks words of one stream, in block order (w0, w1, w2, w3 per block)."""
    b = np.arange(n_blocks, dtype=np.uint64)
    w = philox4x32_10(b & MASK32, b >> np.uint64(32), domain_word(purpose, subset, rnd), 0,
                      seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    return np.stack(w, axis=1).reshape(-1)


def rotation_signs(seed, subset, D):
    """The three +-1 diagonals Sigma_1..Sigma_3 of the randomized Hadamard rotation.

    Coordinate i of round r takes bit (i mod 32) of word i // 32 of stream
    (signs, subset, r); a set bit means -1."""
    n_words = (D + 31) // 32
    out = np.empty((3, D), dtype=np.float64)
    for r in range(3):
        words = stream_words(seed, PURPOSE_SIGNS, subset, r, (n_words + 3) // 4)[:n_words]
        i = np.arange(D)
        bit = (words[i // 32] >> (i % 32).astype(np.uint64)) & np.uint64(1)
        out[r] = np.where(bit == 1, -1.0, 1.0)
    return out


def uniforms_from_words(words):
    """u = (w + 1/2) / 2^32, strictly inside (0, 1)."""
    return (words.astype(np.float64) + 0.5) * (2.0 ** -32)


def box_muller(u1, u2):
    """Box-Muller pair: sqrt(-2 ln u1) * (cos 2 pi u2, sin 2 pi u2), fp64."""
    rho = np.sqrt(-2.0 * np.log(u1))
    theta = 2.0 * np.pi * u2
    return rho * np.cos(theta), rho * np.sin(theta)


def gaussian_stream(seed, subset, count):
    """`count` fp64 normals of the QJL stream: block b gives elements 4b..4b+3 as
    the two Box-Muller pairs (w0, w1) and (w2, w3)."""
    n_blocks = (count + 3) // 4
    w = stream_words(seed, PURPOSE_GAUSS, subset, 0, n_blocks).reshape(n_blocks, 4)
    u = uniforms_from_words(w)
    a0, a1 = box_muller(u[:, 0], u[:, 1])
    a2, a3 = box_muller(u[:, 2], u[:, 3])
    return np.stack([a0, a1, a2, a3], axis=1).reshape(-1)[:count]


def round_to_bf16(x):
    """Round fp64 values to the nearest bfloat16 (8 significant bits), ties to even.

    Values are returned as fp64 (every bf16 value is exactly representable)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                   # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # rint: half to even


def bf16_bits(x_bf16_valued):
    """The 16-bit patterns of values that are exactly bf16 (upper half of the fp32 pattern)."""
    f = np.asarray(x_bf16_valued, dtype=np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def qjl_matrix(seed, subset, k, D):
    """The QJL projection S (k x D): S[j, i] = bf16_RNE(element j*D + i of the Gaussian stream)."""
    return round_to_bf16(gaussian_stream(seed, subset, k * D)).reshape(k, D)
