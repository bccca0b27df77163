"""Byte layout of stored codes, packed and unpacked with plain integer loops.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is stored per vector follows the pages: the quantizer indices and the QJL
sign bits (TurboQuant technical overview, intelliparadigm.com, §1.2.3 and
§2.3.2) and the vector's L2 norm kept separately (same page, §4.2.1); the
residual norm gamma is stored too because the unbiased estimate needs it.

Layout of one vector's record for a (sub-)plan with length D and R index bits
(little-endian; D/32 chunks of 32 coordinates):
  for chunk g = 0 .. D/32 - 1:
      R words:  word m has bit t = bit m of idx[32 g + t]      (t = 0..31)
      1 word:   bit t = beta[32 g + t]                          (k = D)
  float32 norm, float32 gamma
Record bytes = 4 (R + 1) D / 32 + 8.  A vector split by an outlier mask stores
the regular sub-plan's record followed by the outlier sub-plan's record.

A TurboQuant-MSE record (R = b index bits, no QJL stage) drops the sign word and
the residual norm:
  for chunk g: R words as above;  then float32 norm.
Record bytes = 4 R D / 32 + 4.
"""
import numpy as np


def record_bytes(D, R):
    return 4 * (R + 1) * (D // 32) + 8


def pack(codes, D, R):
    """codes: dict with idx (n, D), beta (n, D), norm (n,), gamma (n,) -> uint8 (n, record_bytes)."""
    idx = np.asarray(codes["idx"], dtype=np.int64)
    beta = np.asarray(codes["beta"], dtype=np.int64)
    n = idx.shape[0]
    G = D // 32
    words = np.zeros((n, G, R + 1), dtype=np.uint64)
    for g in range(G):
        for t in range(32):
            i = 32 * g + t
            for m in range(R):
                words[:, g, m] |= ((idx[:, i] >> m) & 1).astype(np.uint64) << np.uint64(t)
            words[:, g, R] |= (beta[:, i] & 1).astype(np.uint64) << np.uint64(t)
    body = words.astype("<u4").reshape(n, -1).view(np.uint8)
    tail = np.stack([np.asarray(codes["norm"], dtype="<f4"),
                     np.asarray(codes["gamma"], dtype="<f4")], axis=1).view(np.uint8)
    return np.concatenate([body, tail], axis=1)


def unpack(records, D, R):
    """Inverse of pack: uint8 (n, record_bytes) -> dict idx, beta, norm, gamma."""
    records = np.ascontiguousarray(records, dtype=np.uint8)
    n = records.shape[0]
    G = D // 32
    words = records[:, :4 * G * (R + 1)].copy().view("<u4").reshape(n, G, R + 1).astype(np.int64)
    idx = np.zeros((n, D), dtype=np.int64)
    beta = np.zeros((n, D), dtype=np.uint8)
    for g in range(G):
        for t in range(32):
            i = 32 * g + t
            for m in range(R):
                idx[:, i] |= ((words[:, g, m] >> t) & 1) << m
            beta[:, i] = (words[:, g, R] >> t) & 1
    tail = records[:, 4 * G * (R + 1):4 * G * (R + 1) + 8].copy().view("<f4")
    return dict(idx=idx, beta=beta, norm=tail[:, 0].astype(np.float64),
                gamma=tail[:, 1].astype(np.float64))


def pack_split(sp, codes_list):
    return np.concatenate([pack(c, p.D, p.R) for p, c in zip(sp.plans, codes_list)], axis=1)


def unpack_split(sp, records):
    out, off = [], 0
    for p in sp.plans:
        nb = record_bytes(p.D, p.R)
        out.append(unpack(records[:, off:off + nb], p.D, p.R))
        off += nb
    return out


def record_bytes_mse(D, R):
    return 4 * R * (D // 32) + 4


def pack_mse(codes, D, R):
    """codes: dict with idx (n, D), norm (n,) -> uint8 (n, record_bytes_mse)."""
    idx = np.asarray(codes["idx"], dtype=np.int64)
    n = idx.shape[0]
    G = D // 32
    words = np.zeros((n, G, R), dtype=np.uint64)
    for g in range(G):
        for t in range(32):
            for m in range(R):
                words[:, g, m] |= ((idx[:, 32 * g + t] >> m) & 1).astype(np.uint64) << np.uint64(t)
    body = words.astype("<u4").reshape(n, -1).view(np.uint8)
    tail = np.asarray(codes["norm"], dtype="<f4").reshape(n, 1).view(np.uint8)
    return np.concatenate([body, tail], axis=1)


def unpack_mse(records, D, R):
    """Inverse of pack_mse: uint8 (n, record_bytes_mse) -> dict idx, norm."""
    records = np.ascontiguousarray(records, dtype=np.uint8)
    n = records.shape[0]
    G = D // 32
    words = records[:, :4 * G * R].copy().view("<u4").reshape(n, G, R).astype(np.int64)
    idx = np.zeros((n, D), dtype=np.int64)
    for g in range(G):
        for t in range(32):
            for m in range(R):
                idx[:, 32 * g + t] |= ((words[:, g, m] >> t) & 1) << m
    norm = records[:, 4 * G * R:4 * G * R + 4].copy().view("<f4")[:, 0]
    return dict(idx=idx, norm=norm.astype(np.float64))
