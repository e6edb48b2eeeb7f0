"""Independent dense references used to pin the oracle (test helpers only).

These build an explicit boolean visibility matrix and use scipy's logsumexp,
a different route from the oracle's per-row key lists, so that a mistake in
either shows up as a disagreement.
"""
import numpy as np
from scipy.special import logsumexp


def bf16_bits(x):
    """Round float32 -> bf16 (round-to-nearest-even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dense(q, k, v, visible, scale=None):
    """q [Hq,R,d], k/v [Hkv,T,d] float64; visible [R,T] bool. Returns (O [Hq,R,d], LSE [Hq,R])."""
    hq, R, d = q.shape
    hkv, T, _ = k.shape
    G = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    kk = np.repeat(k, G, axis=0)
    vv = np.repeat(v, G, axis=0)
    s = np.matmul(q, np.transpose(kk, (0, 2, 1))) * scale
    s = np.where(visible[None, :, :], s, -np.inf)
    lse = logsumexp(s, axis=-1)
    p = np.exp(s - lse[..., None])
    return np.matmul(p, vv), lse


def causal_mask(R, T, offset=0):
    """Row i sees key j iff j <= i + offset."""
    return np.arange(T)[None, :] <= (np.arange(R)[:, None] + offset)
