"""Seeded synthetic inputs, shared by the HIP path's tests and the oracle.

This module draws numbers and nothing else: it holds none of the attention
arithmetic (no band, no scores, no softmax).  The workloads stand in for the
nucleotide corpora the pages train on (GENCODE transcripts), which are not
needed to exercise the attention forward: Q, K, V are activations, replaced here
by normal draws of the shapes and scales below.

Recipe:
  * every [n, d] slice (tensor t in {Q=0, K=1, V=2, dO=3}, sequence b, head h; dO
    is the output gradient the backward pass takes) has its
    own PCG64 stream ``numpy.random.default_rng([seed, cfg, t, b, h])``, so the
    values do not depend on the order of generation or on the batch order;
  * values are ``standard_normal(float32) * sigma``, then rounded to bf16
    (round to nearest even) for the bf16 workloads; kept fp32 otherwise;
  * the mRNA workload draws its lengths from ``default_rng([seed, 2, 3])``
    uniformly in [500, 2048] and pads the buffer up to a multiple of 32;
  * the million-token workload samples 64 query blocks with
    ``default_rng([seed, 5, 4]).choice(nblk, 64, replace=False)``, sorted;
  * with ``poison=True`` every padded row (t >= len_b) of Q, K, V (and dO) is
    NaN, so a kernel that reads padding shows it.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np

BLOCK = 32


@dataclass(frozen=True)
class Workload:
    key: str            # short id: c1 .. c5
    cfg: int            # index mixed into every seed
    name: str
    batch: int
    heads: int
    d: int
    radius: int
    causal: bool
    dtype: str          # "bf16" or "f32"
    sigma: float
    n: int = 0          # buffer length; 0 = derived from the drawn lengths
    last_len: int = 0   # length of the last sequence when it differs from n
    ragged: bool = False

    def describe(self):
        return (f"{self.name}: batch {self.batch} x heads {self.heads} x N {self.n or 'ragged'}"
                f" x d {self.d}, R {self.radius}, {'causal' if self.causal else 'non-causal'},"
                f" {self.dtype}")


WORKLOADS = {
    "c1": Workload("c1", 1, "tiny-fp32", 1, 1, 32, 1, False, "f32", 1.0, n=256),
    "c2": Workload("c2", 2, "mrna-gpt125m", 8, 12, 64, 1, False, "bf16", 1.0, ragged=True),
    "c3": Workload("c3", 3, "gpt350m-causal", 4, 16, 64, 4, True, "bf16", 0.5, n=8192),
    "c4": Workload("c4", 4, "gpt1.3b-long-131k", 1, 16, 128, 8, False, "bf16", 1.0,
                   n=131072, last_len=130000),
    "c5": Workload("c5", 5, "million-token", 1, 8, 64, 2, False, "bf16", 1.0, n=1048576),
}


def lengths(w: Workload, seed: int = 42):
    """(seqlens int32[batch], n): per-sequence lengths and the padded buffer length."""
    if w.ragged:
        lens = np.random.default_rng([seed, w.cfg, 3]).integers(500, 2049, size=w.batch)
        n = int(-(-int(lens.max()) // BLOCK) * BLOCK)
        return lens.astype(np.int32), n
    lens = np.full(w.batch, w.n, dtype=np.int32)
    if w.last_len:
        lens[-1] = w.last_len
    return lens, w.n


def sample_blocks(w: Workload, n: int, seed: int = 42, count: int = 64):
    nblk = n // BLOCK
    return np.sort(np.random.default_rng([seed, w.cfg, 4]).choice(nblk, count, replace=False))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (ties to even).  Finite
    inputs only (normal draws are always finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 arrays that already hold bf16 values (or NaN) -> uint16 bit patterns."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _slice(seed, cfg, t, b, h, n, d, sigma, bf16):
    x = np.random.default_rng([seed, cfg, t, b, h]).standard_normal((n, d), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return round_bf16(x) if bf16 else x


def draw(seed, cfg, batch, heads, n, d, sigma=1.0, bf16=True, seqlens=None, poison=False,
         threads=None, tensors=3):
    """(q, k, v) float32 [batch, heads, n, d] from the per-slice streams above;
    with tensors=4 also the output gradient dO (tensor index 3)."""
    out = [np.empty((batch, heads, n, d), dtype=np.float32) for _ in range(tensors)]

    def fill(job):
        t, b, h = job
        out[t][b, h] = _slice(seed, cfg, t, b, h, n, d, sigma, bf16)
        if poison and seqlens is not None and seqlens[b] < n:
            out[t][b, h, seqlens[b]:, :] = np.nan

    jobs = [(t, b, h) for t in range(tensors) for b in range(batch) for h in range(heads)]
    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    if len(jobs) == 1 or nthr == 1:
        for j in jobs:
            fill(j)
    else:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(fill, jobs))
    return tuple(out)


def make(key: str, seed: int = 42, poison: bool = False, heads=None, n=None, grad=False):
    """Inputs of a named workload: dict(q, k, v, seqlens, n, workload), plus
    ``dout`` with grad=True.  ``heads`` and ``n`` shrink a workload for quick
    runs (lengths are clipped to n)."""
    w = WORKLOADS[key]
    lens, nbuf = lengths(w, seed)
    if n is not None:
        nbuf = n
        lens = np.minimum(lens, n).astype(np.int32)
    hh = heads or w.heads
    t = draw(seed, w.cfg, w.batch, hh, nbuf, w.d, w.sigma, w.dtype == "bf16", lens, poison,
             tensors=4 if grad else 3)
    out = dict(q=t[0], k=t[1], v=t[2], seqlens=lens, n=nbuf, workload=w, heads=hh)
    if grad:
        out["dout"] = t[3]
    return out


# ------------------------------------------------------------ nucleotide text
# Stand-in for the transcript corpus the NucleoByte page trains on (GENCODE
# transcripts, FASTA): ASCII bases back to back with byte offsets per sequence.
# Draws only: bases uniform over A, C, G, T; about one base in a thousand an
# 'N' (an unknown base, as FASTA files carry); runs of soft-masked (lowercase)
# bases covering about a tenth of the text.  One PCG64 stream per slab,
# ``default_rng([seed, cfg, 6])``; lengths from ``default_rng([seed, cfg, 3])``.

@dataclass(frozen=True)
class DnaWorkload:
    key: str
    cfg: int
    name: str
    batch: int
    lo: int          # shortest sequence, bases
    hi: int          # longest sequence, bases
    k: int = 6

    def describe(self):
        return (f"{self.name}: {self.batch} sequences of {self.lo}..{self.hi} bases, "
                f"{self.k}-mers")


DNA_WORKLOADS = {
    # transcript-length slab: the mRNA workload's length range, 65,536 sequences
    "k1": DnaWorkload("k1", 11, "gencode-slab-6mer", 65536, 500, 2048),
    # a handful of long sequences (chromosome-scale runs)
    "k2": DnaWorkload("k2", 12, "long-6mer", 8, 1 << 20, 1 << 22),
}


def dna(seed, cfg, batch, lo, hi, n_rate=1e-3, soft_rate=0.1):
    """Returns (bases uint8, starts int64 [batch + 1])."""
    lens = np.random.default_rng([seed, cfg, 3]).integers(lo, hi + 1, size=batch)
    starts = np.zeros(batch + 1, dtype=np.int64)
    np.cumsum(lens, out=starts[1:])
    total = int(starts[-1])
    rng = np.random.default_rng([seed, cfg, 6])
    alphabet = np.frombuffer(b"ACGT", dtype=np.uint8)
    bases = alphabet[rng.integers(0, 4, size=total, dtype=np.uint8)]
    if total:
        unknown = rng.random(total) < n_rate
        bases[unknown] = ord("N")
        # soft-masked runs: run starts at rate soft_rate / 50, each 50 bases long
        run_starts = np.flatnonzero(rng.random(total) < soft_rate / 50.0)
        if run_starts.size:
            mark = np.zeros(total + 51, dtype=np.int32)
            np.add.at(mark, run_starts, 1)
            np.add.at(mark, run_starts + 50, -1)
            lower = np.cumsum(mark)[:total] > 0
            bases[lower] = bases[lower] | 0x20
    return bases, starts


def make_dna(key, seed=42):
    w = DNA_WORKLOADS[key]
    bases, starts = dna(seed, w.cfg, w.batch, w.lo, w.hi)
    lens = np.diff(starts)
    windows = int(max(0, lens.max() - w.k + 1))
    n_out = (windows + BLOCK - 1) // BLOCK * BLOCK
    return dict(workload=w, bases=bases, starts=starts, n_out=n_out)
