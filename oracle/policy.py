"""The KV-cache policy layer in fp64: outlier channels by variance, and appending tokens.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

TurboQuant technical overview (intelliparadigm.com), §4.1.1: analyse the per-head
distributions, keep about a quarter of the channels as outliers at a higher bit width (here:
the channels of largest variance over a calibration sample, the plainest reading of "outlier
channel"), 3-bit TurboQuant-MSE for most heads and the inner-product variant for key heads;
§4.1.2: the cache is written as tokens arrive (one record per head and decode step).

Pins (tests/test_oracle_pins.py): the variance against the pairwise-difference identity;
planted channels, shift and permutation invariance and ties for the choice; placement by hand.
"""
import numpy as np


def channel_variance(X):
    """Population variance of every channel (column) of X over its rows: mean((x - mean)^2)."""
    X = np.asarray(X, dtype=np.float64)
    if X.shape[0] == 0:
        return np.zeros(X.shape[1])
    mu = X.mean(axis=0)
    return ((X - mu) ** 2).mean(axis=0)


def outlier_channels(X, n_out):
    """The n_out channels of largest variance, ordered by (-variance, channel); returns
    (sorted channel list, uint8 mask of length d)."""
    v = channel_variance(X)
    order = np.lexsort((np.arange(v.shape[0]), -v))
    ch = np.sort(order[:n_out])
    mask = np.zeros(v.shape[0], dtype=np.uint8)
    mask[ch] = 1
    return ch, mask


def place(cache, records, index):
    """Append: record i goes to row index[i] of the cache (rows outside [0, len(cache))
    are dropped).  cache, records: uint8 (rows, record_bytes).  Returns the new cache."""
    out = np.array(cache, dtype=np.uint8, copy=True)
    for i, j in enumerate(np.asarray(index, dtype=np.int64)):
        if 0 <= j < out.shape[0]:
            out[j] = records[i]
    return out
