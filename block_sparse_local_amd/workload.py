"""Work and traffic accounting for a banded block-sparse attention forward.

Used for reporting only (bench.py); nothing here runs on the compute path.

useful pairs   kept (query t, key s) pairs summed over sequences and heads: for
               row t of block i = t // 32 the keys run from max(0, (i-R)*32) to
               min(len, (i+R+1)*32) (exclusive), or to t + 1 when causal.
               With a token window W the keys run from max(0, t-W) to
               min(len, t+W+1) (or t + 1 when causal), and the kernel's band
               is R = ceil(W/32).
useful FLOP    4 * d per useful pair (2d for Q.K, 2d for P.V); exp and the
               final division are not counted.
block pairs    (query block, key block) pairs the kernel computes, each a
               32 x 32 x d score product and a 32 x 32 x d value product.
alg. bytes     Q, K, V read once and O written once over the real rows only:
               4 * sum(len) * heads * d * element size.  Halo re-reads, the
               zero rows written for padding and lse are implementation costs.

Backward pass (account_backward): useful FLOP = 10 * d per useful pair (the
four products dV, dP, dQ, dK, 2d each, plus the scores recomputed once: the
usual 2.5 times the forward); algorithmic bytes = Q, K, V, O, dO and lse read
once, dQ, dK, dV written once, over the real rows.
"""
import numpy as np

BLOCK = 32
MI355X_BF16_DENSE_FLOPS = 2.5e15   # dense bf16 MFMA peak (no sparsity)
MI355X_FP32_VECTOR_FLOPS = 157.3e12
MI355X_HBM_BYTES = 8.0e12


def band_radius(radius, window=0):
    """The block radius swept: R, or ceil(W/32) for a token window W >= 1."""
    return -(-int(window) // BLOCK) if window > 0 else radius


def key_range(t, L, radius, causal, window=0):
    """Kept keys [lo, hi) of query rows t (int64 array) of a length-L sequence."""
    if window > 0:
        lo = np.maximum(0, t - window)
        hi = np.minimum(int(L), t + window + 1)
    else:
        i = t // BLOCK
        lo = np.maximum(0, (i - radius) * BLOCK)
        hi = np.minimum(int(L), (i + radius + 1) * BLOCK)
    if causal:
        hi = np.minimum(hi, t + 1)
    return lo, hi


def useful_pairs_per_head(lens, radius, causal, window=0):
    total = 0
    for L in np.asarray(lens, dtype=np.int64):
        t = np.arange(int(L), dtype=np.int64)
        lo, hi = key_range(t, L, radius, causal, window)
        total += int((hi - lo).sum())
    return total


def block_pairs_per_head(lens, radius, causal, window=0):
    radius = band_radius(radius, window)
    total = 0
    for L in lens:
        nb = -(-int(L) // BLOCK)
        i = np.arange(nb)
        lo = np.maximum(0, i - radius)
        hi = np.minimum(nb - 1, i + radius)
        if causal:
            hi = np.minimum(hi, i)
        total += int((hi - lo + 1).sum())
    return total


def account(lens, heads, d, radius, causal, dtype="bf16", window=0):
    esz = 2 if dtype == "bf16" else 4
    up = useful_pairs_per_head(lens, radius, causal, window) * heads
    bp = block_pairs_per_head(lens, radius, causal, window) * heads
    tokens = int(np.sum(lens))
    flops = 4.0 * d * up
    computed = 4.0 * d * BLOCK * BLOCK * bp
    nbytes = 4.0 * tokens * heads * d * esz
    peak = MI355X_BF16_DENSE_FLOPS if dtype == "bf16" else MI355X_FP32_VECTOR_FLOPS
    t_mfma = flops / peak
    t_hbm = nbytes / MI355X_HBM_BYTES
    # the bf16 path computes on MFMA; the fp32 path on the vector ALUs
    compute_unit = "mfma" if dtype == "bf16" else "alu"
    return dict(useful_pairs=up, block_pairs=bp, tokens=tokens, useful_flops=flops,
                computed_flops=computed, alg_bytes=nbytes, t_mfma=t_mfma, t_hbm=t_hbm,
                bound="hbm" if t_hbm >= t_mfma else compute_unit, flops_peak=peak)


def account_backward(lens, heads, d, radius, causal, dtype="bf16", window=0):
    esz = 2 if dtype == "bf16" else 4
    up = useful_pairs_per_head(lens, radius, causal, window) * heads
    bp = block_pairs_per_head(lens, radius, causal, window) * heads
    tokens = int(np.sum(lens))
    flops = 10.0 * d * up
    # the kernels recompute S and dP in both the dQ and the dK/dV kernel
    computed = 14.0 * d * BLOCK * BLOCK * bp
    nbytes = (8.0 * d * esz + 4.0) * tokens * heads
    peak = MI355X_BF16_DENSE_FLOPS if dtype == "bf16" else MI355X_FP32_VECTOR_FLOPS
    t_mfma = flops / peak
    t_hbm = nbytes / MI355X_HBM_BYTES
    compute_unit = "mfma" if dtype == "bf16" else "alu"
    return dict(useful_pairs=up, block_pairs=bp, tokens=tokens, useful_flops=flops,
                computed_flops=computed, alg_bytes=nbytes, t_mfma=t_mfma, t_hbm=t_hbm,
                bound="hbm" if t_hbm >= t_mfma else compute_unit, flops_peak=peak)
