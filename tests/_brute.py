"""Brute-force checks of the oracle: an explicit n x n mask and a dense softmax.

Deliberately shaped unlike the oracle: everything is dense numpy over the whole
sequence, the mask is built token pair by token pair, and the softmax is the
textbook exp / sum over a masked row.  Tiny inputs only.
"""
import numpy as np


def token_mask(n, length, bsize, radius, causal, window=None):
    """bool [n, n]: entry (t, s) kept.  With ``window`` the band is the token
    window |t - s| <= window instead of the block band."""
    t = np.arange(n)[:, None]
    s = np.arange(n)[None, :]
    if window is None:
        near = np.abs(t // bsize - s // bsize) <= radius
    else:
        near = np.abs(t - s) <= window
    keep = (t < length) & (s < length) & near
    if causal:
        keep &= s <= t
    return keep


def dense_reference(q, k, v, seqlens, bsize, radius, causal, scale=None, window=None):
    """float64 (o, lse) from a dense masked softmax."""
    q = q.astype(np.float64)
    k = k.astype(np.float64)
    v = v.astype(np.float64)
    batch, heads, n, d = q.shape
    sc = 1.0 / np.sqrt(d) if not scale else scale
    o = np.zeros((batch, heads, n, d))
    lse = np.full((batch, heads, n), -np.inf)
    for b in range(batch):
        L = int(seqlens[b]) if seqlens is not None else n
        keep = token_mask(n, L, bsize, radius, causal, window)
        for h in range(heads):
            qq = np.nan_to_num(q[b, h], nan=0.0)
            kk = np.nan_to_num(k[b, h], nan=0.0)
            vv = np.nan_to_num(v[b, h], nan=0.0)
            s = sc * (qq @ kk.T)
            s = np.where(keep, s, -np.inf)
            for t in range(L):
                row = s[t]
                mx = row.max()
                w = np.exp(row - mx)
                o[b, h, t] = (w @ vv) / w.sum()
                lse[b, h, t] = mx + np.log(w.sum())
    return o, lse
