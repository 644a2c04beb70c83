"""ctypes wrapper over the fp64 CPU oracle (oracle/orc.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the HIP library ``block_sparse_local_amd``
and never imports it.

Every function takes numpy arrays on the host.  Q, K, V are float32 arrays of
shape [batch, heads, n, d] holding the exact (bf16- or fp32-rounded) values a
GPU consumes; results are float64.  The computation follows the NucleoByte
project page, section 3 ("Localized Block-Sparse Attention Matrix" for the
band rule, "Softmax Normalization & Online Numerical Stability" for the scores
and the softmax, "Custom Backpropagation" for the gradients); see orc.c for
the definitions.  ``kmer_tokenize`` follows the same page's section 2, item 1
("Fused 2-Bit Tokenization"), with the 6-mer vocabulary of section 5.

Parity pins (what ties each routine to something other than itself) live in
``tests/test_oracle_*.py``.  No oracle routine is "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


class OracleError(RuntimeError):
    pass


def _declare(lib):
    i = ctypes.c_int
    lib.orc_version.restype = i
    lib.orc_active_blocks.argtypes = [i, i, i, i, i, _i32p, _i32p]
    lib.orc_masks.argtypes = [i, i, i, i, i, _i32p, _i32p, _u32p]
    lib.orc_forward_f64.argtypes = [i, i, i, i, i, i, i, ctypes.c_double, _i32p, _f32p, _f32p,
                                    _f32p, _f64p, _f64p, _f64p, i]
    lib.orc_forward_blocks_f64.argtypes = [i, i, i, i, i, i, i, ctypes.c_double, _i32p, _f32p,
                                           _f32p, _f32p, ctypes.c_int64, _i32p, _f64p, _f64p,
                                           _f64p, i]
    lib.orc_forward_recurrence_f64.argtypes = [i, i, i, i, i, i, i, ctypes.c_double, _i32p,
                                               _f32p, _f32p, _f32p, _f64p]
    lib.orc_backward_f64.argtypes = [i, i, i, i, i, i, i, ctypes.c_double, _i32p, _f32p, _f32p,
                                     _f32p, _f32p, _f64p, _f64p, _f64p, i]
    lib.orc_backward_blocks_f64.argtypes = [i, i, i, i, i, i, i, ctypes.c_double, _i32p, _f32p,
                                            _f32p, _f32p, _f32p, ctypes.c_int64, _i32p, _f64p,
                                            _f64p, _f64p, i]
    lib.orc_masks_w.argtypes = [i, i, i, i, i, i, _i32p, _i32p, _u32p]
    lib.orc_forward_w_f64.argtypes = [i, i, i, i, i, i, i, i, ctypes.c_double, _i32p, _f32p,
                                      _f32p, _f32p, _f64p, _f64p, _f64p, i]
    lib.orc_forward_blocks_w_f64.argtypes = [i, i, i, i, i, i, i, i, ctypes.c_double, _i32p,
                                             _f32p, _f32p, _f32p, ctypes.c_int64, _i32p, _f64p,
                                             _f64p, _f64p, i]
    lib.orc_forward_recurrence_w_f64.argtypes = [i, i, i, i, i, i, i, i, ctypes.c_double, _i32p,
                                                 _f32p, _f32p, _f32p, _f64p]
    lib.orc_backward_w_f64.argtypes = [i, i, i, i, i, i, i, i, ctypes.c_double, _i32p, _f32p,
                                       _f32p, _f32p, _f32p, _f64p, _f64p, _f64p, i]
    lib.orc_backward_blocks_w_f64.argtypes = [i, i, i, i, i, i, i, i, ctypes.c_double, _i32p,
                                              _f32p, _f32p, _f32p, _f32p, ctypes.c_int64, _i32p,
                                              _f64p, _f64p, _f64p, i]
    lib.orc_kmer_tokenize.argtypes = [i, ctypes.POINTER(ctypes.c_uint8),
                                      ctypes.POINTER(ctypes.c_int64), i, i, _i32p, _i32p]
    for name in ("orc_masks_w", "orc_forward_w_f64", "orc_forward_blocks_w_f64",
                 "orc_forward_recurrence_w_f64", "orc_kmer_tokenize", "orc_active_blocks", "orc_masks", "orc_forward_f64", "orc_forward_blocks_f64",
                 "orc_forward_recurrence_f64", "orc_backward_f64", "orc_backward_blocks_f64",
                 "orc_backward_w_f64", "orc_backward_blocks_w_f64"):
        getattr(lib, name).restype = i
    return lib


def load(path=None):
    """Load liborc.so (compiling it with gcc if it is missing); ``path`` loads
    another build, e.g. a mutant compiled by the mutation tests."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        # ORC_LIBRARY selects another build of the same source (the sanitizer
        # build of tests/test_host_sanitize.py); unset, the in-tree build
        lib_path = os.environ.get("ORC_LIBRARY") or os.path.join(_HERE, "liborc.so")
        if not os.path.exists(lib_path):
            if os.environ.get("ORC_LIBRARY"):
                raise OracleError(f"ORC_LIBRARY={lib_path} does not exist")
            _build.build()
        _lib = _declare(ctypes.CDLL(lib_path))
    return _lib


def default_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a, typ):
    return None if a is None else a.ctypes.data_as(typ)


def _lens(batch, n, seqlens):
    if seqlens is None:
        return None
    s = np.ascontiguousarray(seqlens, dtype=np.int32)
    if s.shape != (batch,):
        raise ValueError("seqlens must have shape [batch]")
    return s


def _check(rc, name):
    if rc != 0:
        raise OracleError(f"{name} failed with code {rc}")


def window_radius(window, bsize=32):
    """The block radius a token window of ``window`` tokens reaches: ceil(W/B)."""
    return -(-int(window) // int(bsize))


def _radius(radius, window, bsize):
    return radius if window is None else window_radius(window, bsize)


def active_blocks(batch, n, bsize, radius, causal, seqlens=None, lib=None, window=None):
    """int32 [batch, n/bsize, 2R+1]: ascending visited key blocks, -1 padded.
    With a token window W, R = ceil(W/B) (every block of that band holds a
    pair within W)."""
    lib = lib or load()
    radius = _radius(radius, window, bsize)
    s = _lens(batch, n, seqlens)
    nblk = n // bsize if bsize > 0 else 0
    out = np.full((batch, nblk, max(2 * radius + 1, 1)), -7, dtype=np.int32)
    _check(lib.orc_active_blocks(batch, n, bsize, radius, int(causal), _ptr(s, _i32p),
                                 _ptr(out, _i32p)), "orc_active_blocks")
    return out


def masks(batch, n, bsize, radius, causal, seqlens=None, active=None, lib=None, window=None):
    """uint32 [batch, n/bsize, 2R+1, bsize]: word r bit c set iff key c of the
    slot's key block is kept for query row r of the query block."""
    lib = lib or load()
    radius = _radius(radius, window, bsize)
    s = _lens(batch, n, seqlens)
    if active is None:
        active = active_blocks(batch, n, bsize, radius, causal, seqlens, lib=lib)
    active = np.ascontiguousarray(active, dtype=np.int32)
    out = np.zeros(active.shape + (bsize,), dtype=np.uint32)
    if window is None:
        _check(lib.orc_masks(batch, n, bsize, radius, int(causal), _ptr(s, _i32p),
                             _ptr(active, _i32p), _ptr(out, _u32p)), "orc_masks")
    else:
        _check(lib.orc_masks_w(batch, n, bsize, radius, int(causal), int(window), _ptr(s, _i32p),
                               _ptr(active, _i32p), _ptr(out, _u32p)), "orc_masks_w")
    return out


def _f32(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError("oracle inputs are float32 arrays holding the exact input values")
    return a


def forward(q, k, v, seqlens=None, bsize=32, radius=1, causal=False, scale=0.0, nthreads=None,
            lib=None, window=None):
    """Two-pass definition.  Returns (o [b,h,n,d], lse [b,h,n], psum [b,h,n])
    in float64; psum is the sum of each row's normalised probabilities.
    ``window`` (>= 0) selects the token window |t - s| <= W instead of the
    block band."""
    lib = lib or load()
    radius = _radius(radius, window, bsize)
    q, k, v = _f32(q), _f32(k), _f32(v)
    batch, heads, n, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v shapes differ")
    s = _lens(batch, n, seqlens)
    o = np.empty((batch, heads, n, d), dtype=np.float64)
    lse = np.empty((batch, heads, n), dtype=np.float64)
    psum = np.empty((batch, heads, n), dtype=np.float64)
    if window is None:
        _check(lib.orc_forward_f64(batch, heads, n, d, bsize, radius, int(causal), float(scale),
                                   _ptr(s, _i32p), _ptr(q, _f32p), _ptr(k, _f32p),
                                   _ptr(v, _f32p), _ptr(o, _f64p), _ptr(lse, _f64p),
                                   _ptr(psum, _f64p), nthreads or default_threads()),
               "orc_forward_f64")
    else:
        _check(lib.orc_forward_w_f64(batch, heads, n, d, bsize, radius, int(causal), int(window),
                                     float(scale), _ptr(s, _i32p), _ptr(q, _f32p),
                                     _ptr(k, _f32p), _ptr(v, _f32p), _ptr(o, _f64p),
                                     _ptr(lse, _f64p), _ptr(psum, _f64p),
                                     nthreads or default_threads()), "orc_forward_w_f64")
    return o, lse, psum


def forward_blocks(q, k, v, sel, seqlens=None, bsize=32, radius=1, causal=False, scale=0.0,
                   nthreads=None, lib=None, window=None):
    """Only the query blocks listed in ``sel`` (int array [m, 3] of (b, h, i)).
    Returns (o [m, bsize, d], lse [m, bsize], psum [m, bsize])."""
    lib = lib or load()
    radius = _radius(radius, window, bsize)
    q, k, v = _f32(q), _f32(k), _f32(v)
    batch, heads, n, d = q.shape
    s = _lens(batch, n, seqlens)
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 3)
    m = sel.shape[0]
    o = np.empty((m, bsize, d), dtype=np.float64)
    lse = np.empty((m, bsize), dtype=np.float64)
    psum = np.empty((m, bsize), dtype=np.float64)
    _check(lib.orc_forward_blocks_w_f64(batch, heads, n, d, bsize, radius, int(causal),
                                        -1 if window is None else int(window), float(scale),
                                        _ptr(s, _i32p), _ptr(q, _f32p), _ptr(k, _f32p),
                                        _ptr(v, _f32p), m, _ptr(sel, _i32p), _ptr(o, _f64p),
                                        _ptr(lse, _f64p), _ptr(psum, _f64p),
                                        nthreads or default_threads()), "orc_forward_blocks_w_f64")
    return o, lse, psum


def forward_recurrence(q, k, v, seqlens=None, bsize=32, radius=1, causal=False, scale=0.0,
                       lib=None, window=None):
    """The page's running (m, d, O) recurrence, block by block, divided by d at
    the end.  Single threaded; meant for small inputs."""
    lib = lib or load()
    radius = _radius(radius, window, bsize)
    q, k, v = _f32(q), _f32(k), _f32(v)
    batch, heads, n, d = q.shape
    s = _lens(batch, n, seqlens)
    o = np.empty((batch, heads, n, d), dtype=np.float64)
    _check(lib.orc_forward_recurrence_w_f64(batch, heads, n, d, bsize, radius, int(causal),
                                            -1 if window is None else int(window), float(scale),
                                            _ptr(s, _i32p), _ptr(q, _f32p), _ptr(k, _f32p),
                                            _ptr(v, _f32p), _ptr(o, _f64p)),
           "orc_forward_recurrence_w_f64")
    return o


def backward(q, k, v, dout, seqlens=None, bsize=32, radius=1, causal=False, scale=0.0,
             nthreads=None, lib=None, window=None):
    """Gradients of the forward with respect to q, k, v for the output gradient
    ``dout`` (float32 [b,h,n,d]).  Returns (dq, dk, dv), float64 [b,h,n,d].
    ``window`` (>= 0): the gradients of the token-window forward."""
    lib = lib or load()
    radius = _radius(radius, window, bsize)
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    batch, heads, n, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, dout shapes differ")
    s = _lens(batch, n, seqlens)
    dq = np.empty((batch, heads, n, d), dtype=np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    _check(lib.orc_backward_w_f64(batch, heads, n, d, bsize, radius, int(causal),
                                  -1 if window is None else int(window), float(scale),
                                  _ptr(s, _i32p), _ptr(q, _f32p), _ptr(k, _f32p), _ptr(v, _f32p),
                                  _ptr(dout, _f32p), _ptr(dq, _f64p), _ptr(dk, _f64p),
                                  _ptr(dv, _f64p), nthreads or default_threads()),
           "orc_backward_w_f64")
    return dq, dk, dv


def backward_blocks(q, k, v, dout, sel, seqlens=None, bsize=32, radius=1, causal=False,
                    scale=0.0, nthreads=None, lib=None, window=None):
    """For each (b, h, i) in ``sel``: dq of query block i and dk, dv of key
    block i.  Returns (dq, dk, dv), each float64 [m, bsize, d]."""
    lib = lib or load()
    radius = _radius(radius, window, bsize)
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    batch, heads, n, d = q.shape
    s = _lens(batch, n, seqlens)
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 3)
    m = sel.shape[0]
    dq = np.empty((m, bsize, d), dtype=np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    _check(lib.orc_backward_blocks_w_f64(batch, heads, n, d, bsize, radius, int(causal),
                                         -1 if window is None else int(window), float(scale),
                                         _ptr(s, _i32p), _ptr(q, _f32p), _ptr(k, _f32p),
                                         _ptr(v, _f32p), _ptr(dout, _f32p), m, _ptr(sel, _i32p),
                                         _ptr(dq, _f64p), _ptr(dk, _f64p), _ptr(dv, _f64p),
                                         nthreads or default_threads()),
           "orc_backward_blocks_w_f64")
    return dq, dk, dv


def kmer_specials(k=6):
    """Special IDs after the 4^k k-mer IDs: PAD, MASK, UNK (4^k + 3 is reserved)."""
    four_k = 4 ** k
    return dict(pad=four_k, mask=four_k + 1, unk=four_k + 2, vocab=four_k + 4)


def kmer_tokenize(bases, starts, k=6, n_out=None, lib=None):
    """Sliding-window k-mer IDs.  ``bases`` uint8 (the sequences' ASCII bytes
    back to back), ``starts`` int64 [batch + 1] byte offsets.  Returns (ids
    int32 [batch, n_out], ntok int32 [batch]); ``n_out`` defaults to the longest
    sequence's window count."""
    lib = lib or load()
    bases = np.ascontiguousarray(bases, dtype=np.uint8)
    starts = np.ascontiguousarray(starts, dtype=np.int64)
    batch = starts.shape[0] - 1
    if n_out is None:
        n_out = int(max(0, (np.diff(starts) - k + 1).max(initial=0)))
    ids = np.full((batch, n_out), -7, dtype=np.int32)
    ntok = np.full(batch, -7, dtype=np.int32)
    bp = bases.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)) if bases.size else None
    _check(lib.orc_kmer_tokenize(batch, bp, starts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 k, n_out, _ptr(ids, _i32p), _ptr(ntok, _i32p)),
           "orc_kmer_tokenize")
    return ids, ntok
