"""ctypes binding of libbsl.so (include/bsl.h), same names as the C ABI.

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, statuses become exceptions.  Every step of the
computation runs in the library's HIP kernels; there is no fallback, and using
the binding without the built library raises ``BslError``.

    plan = bsl_create(BslDesc(head_dim=64, heads=8, radius=2))
    bsl_forward(plan, batch, n, q, k, v, o, seqlens, None)
    bsl_destroy(plan)

or, with shape checks on torch tensors, ``Plan(...).forward(q, k, v, seqlens)``.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# BSL_LIBRARY selects another build of the same library (a design variant made
# by `build.py --variant ... --out ...`); unset, the in-tree build is used
LIB_PATH = os.environ.get("BSL_LIBRARY") or os.path.join(HERE, "libbsl.so")

BSL_OK, BSL_E_INVALID, BSL_E_UNSUPPORTED, BSL_E_DEVICE, BSL_E_NOMEM = range(5)
BSL_BF16, BSL_F32 = 0, 1

# every function include/bsl.h declares
EXPORTS = ("bsl_create", "bsl_forward", "bsl_forward_traced", "bsl_forward_varlen",
           "bsl_varlen_offsets", "bsl_backward", "bsl_backward_noalloc", "bsl_backward_varlen",
           "bsl_kmer_tokenize",
           "bsl_kmer_ceiling", "bsl_check_seqlens", "bsl_check_cu_seqlens", "bsl_destroy", "bsl_status_string",
           "bsl_last_error", "bsl_version")


class BslError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


class BslDesc(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("radius", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("window", ctypes.c_int32)]

    def __init__(self, head_dim=64, heads=1, radius=1, causal=False, dtype=BSL_BF16, scale=0.0,
                 block_size=32, window=0):
        super().__init__(head_dim, heads, block_size, radius, int(causal), dtype, scale, window)


_lib = None


def load(path=LIB_PATH):
    """The loaded library (loads it on first use)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise BslError(BSL_E_UNSUPPORTED,
                       f"{path} is not built; run `python -m block_sparse_local_amd.build`")
    # torch's wheel carries its own HIP runtime, which it asks for by file name;
    # loading torch first lets libbsl's libamdhip64.so.7 dependency resolve to
    # that same copy, so the process has one HIP runtime, not two.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.bsl_create.argtypes = [ctypes.POINTER(BslDesc), ctypes.POINTER(vp)]
    lib.bsl_forward.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.bsl_forward_traced.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bsl_forward_varlen.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    i32p = ctypes.POINTER(i32)
    lib.bsl_varlen_offsets.argtypes = [i32, i32p, i32p, i32p, i32p]
    lib.bsl_backward.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.bsl_backward_noalloc.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp]
    lib.bsl_backward_varlen.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp]
    lib.bsl_kmer_tokenize.argtypes = [i32, vp, ctypes.c_int64, vp, i32, i32, vp, vp, vp]
    lib.bsl_kmer_ceiling.argtypes = [i32, ctypes.POINTER(ctypes.c_int64), i32, ctypes.POINTER(i32)]
    lib.bsl_check_seqlens.argtypes = [i32, i32, vp, vp, vp]
    lib.bsl_check_cu_seqlens.argtypes = [i32, i32, vp, vp, vp]
    lib.bsl_destroy.argtypes = [vp]
    lib.bsl_status_string.argtypes = [ctypes.c_int]
    lib.bsl_status_string.restype = ctypes.c_char_p
    lib.bsl_last_error.argtypes = []
    lib.bsl_last_error.restype = ctypes.c_char_p
    lib.bsl_version.argtypes = []
    lib.bsl_version.restype = i32
    for name in ("bsl_create", "bsl_forward", "bsl_forward_traced", "bsl_forward_varlen",
                 "bsl_varlen_offsets", "bsl_backward", "bsl_backward_noalloc",
                 "bsl_backward_varlen", "bsl_kmer_tokenize", "bsl_kmer_ceiling",
                 "bsl_check_seqlens", "bsl_check_cu_seqlens", "bsl_destroy"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status):
    if status != BSL_OK:
        lib = load()
        raise BslError(status, f"{lib.bsl_status_string(status).decode()}: "
                               f"{lib.bsl_last_error().decode()}")


def _ptr(x):
    """torch tensor -> device address; int -> itself; None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


# ------------------------------------------------------------- raw C names

def bsl_create(desc):
    plan = ctypes.c_void_p()
    _check(load().bsl_create(ctypes.byref(desc), ctypes.byref(plan)))
    return plan


def bsl_forward(plan, batch, n, q, k, v, o, seqlens=None, lse=None, stream=None):
    _check(load().bsl_forward(plan, batch, n, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(seqlens),
                              _ptr(lse), _stream(stream)))


def bsl_forward_traced(plan, batch, n, q, k, v, o, seqlens, lse, active, masks, stream=None):
    _check(load().bsl_forward_traced(plan, batch, n, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(seqlens), _ptr(lse), _ptr(active), _ptr(masks),
                                     _stream(stream)))


def bsl_forward_varlen(plan, batch, tokens, max_seqlen, q, k, v, o, cu_seqlens, lse=None,
                       stream=None):
    _check(load().bsl_forward_varlen(plan, batch, tokens, max_seqlen, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(o), _ptr(cu_seqlens), _ptr(lse), _stream(stream)))


def bsl_varlen_offsets(lengths):
    """Host lengths -> (cu_seqlens int32[batch + 1], max_seqlen, ceiling)."""
    import numpy as np
    lens = np.ascontiguousarray(lengths, dtype=np.int32)
    if lens.ndim != 1:
        raise ValueError("lengths must be one-dimensional")
    cu = np.zeros(lens.shape[0] + 1, dtype=np.int32)
    mx, ceil = ctypes.c_int32(), ctypes.c_int32()
    i32p = ctypes.POINTER(ctypes.c_int32)
    _check(load().bsl_varlen_offsets(lens.shape[0], lens.ctypes.data_as(i32p),
                                     cu.ctypes.data_as(i32p), ctypes.byref(mx), ctypes.byref(ceil)))
    return cu, mx.value, ceil.value


def bsl_backward(plan, batch, n, q, k, v, o, dout, lse, seqlens, dq, dk, dv, delta, stream=None):
    _check(load().bsl_backward(plan, batch, n, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                               _ptr(lse), _ptr(seqlens), _ptr(dq), _ptr(dk), _ptr(dv),
                               _ptr(delta), _stream(stream)))


def bsl_backward_noalloc(plan, batch, n, q, k, v, o, dout, lse, seqlens, dq, dk, dv,
                         stream=None):
    _check(load().bsl_backward_noalloc(plan, batch, n, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                       _ptr(dout), _ptr(lse), _ptr(seqlens), _ptr(dq), _ptr(dk),
                                       _ptr(dv), _stream(stream)))


def bsl_backward_varlen(plan, batch, tokens, max_seqlen, q, k, v, o, dout, lse, cu_seqlens, dq,
                        dk, dv, delta, stream=None):
    _check(load().bsl_backward_varlen(plan, batch, tokens, max_seqlen, _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(o), _ptr(dout), _ptr(lse), _ptr(cu_seqlens), _ptr(dq),
                                      _ptr(dk), _ptr(dv), _ptr(delta), _stream(stream)))


def bsl_kmer_tokenize(batch, bases, nbytes, starts, k, n_out, ids, ntok=None, stream=None):
    _check(load().bsl_kmer_tokenize(batch, _ptr(bases), nbytes, _ptr(starts), k, n_out, _ptr(ids),
                                    _ptr(ntok), _stream(stream)))


def bsl_check_seqlens(batch, n, seqlens, result, stream=None):
    _check(load().bsl_check_seqlens(batch, n, _ptr(seqlens), _ptr(result), _stream(stream)))


def bsl_check_cu_seqlens(batch, tokens, cu_seqlens, result, stream=None):
    _check(load().bsl_check_cu_seqlens(batch, tokens, _ptr(cu_seqlens), _ptr(result),
                                       _stream(stream)))


def check_seqlens(seqlens, n):
    """Device int32 lengths -> (bad entries, first bad index or -1); waits for the result."""
    import torch
    res = torch.empty(2, dtype=torch.int32, device=seqlens.device)
    bsl_check_seqlens(seqlens.numel(), n, seqlens, res)
    bad, first = res.tolist()
    return bad, first


def check_cu_seqlens(cu_seqlens, tokens):
    """Device int32 offsets [batch + 1] -> (bad entries, first bad index or -1)."""
    import torch
    res = torch.empty(2, dtype=torch.int32, device=cu_seqlens.device)
    bsl_check_cu_seqlens(cu_seqlens.numel() - 1, tokens, cu_seqlens, res)
    bad, first = res.tolist()
    return bad, first


def bsl_kmer_ceiling(starts, k=6):
    """Host int64 starts [batch + 1] -> the padded row width (a multiple of 32)."""
    import numpy as np
    st = np.ascontiguousarray(starts, dtype=np.int64)
    if st.ndim != 1 or st.shape[0] < 1:
        raise ValueError("starts must be one-dimensional with batch + 1 entries")
    out = ctypes.c_int32()
    _check(load().bsl_kmer_ceiling(st.shape[0] - 1, st.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                   k, ctypes.byref(out)))
    return out.value


def kmer_specials(k=6):
    """The special IDs after the 4^k k-mer IDs (BSL_KMER_* in include/bsl.h)."""
    pad = 1 << (2 * k)
    return dict(pad=pad, mask=pad + 1, unk=pad + 2, vocab=pad + 4)


def kmer_tokenize(bases, starts, k=6, n_out=None, ids=None, ntok=None, stream=None):
    """bases: uint8 CUDA tensor (the text); starts: int64 CUDA tensor [batch + 1].
    Returns (ids int32 [batch, n_out], ntok int32 [batch]); ``n_out`` is
    required (bsl_kmer_ceiling computes it from host offsets)."""
    import torch
    if bases.dtype != torch.uint8 or not bases.is_cuda or bases.dim() != 1:
        raise ValueError("bases must be a one-dimensional uint8 CUDA tensor")
    if starts.dtype != torch.int64 or not starts.is_cuda or starts.dim() != 1 or starts.shape[0] < 1:
        raise ValueError("starts must be an int64 CUDA tensor of shape [batch + 1]")
    if not bases.is_contiguous() or not starts.is_contiguous():
        raise ValueError("bases and starts must be contiguous")
    if n_out is None:
        raise ValueError("n_out is required (bsl_kmer_ceiling gives it from host offsets)")
    batch = starts.shape[0] - 1
    if ids is None:
        ids = torch.empty((batch, n_out), dtype=torch.int32, device=bases.device)
    if ntok is None:
        ntok = torch.empty(batch, dtype=torch.int32, device=bases.device)
    if ids.dtype != torch.int32 or ids.shape != (batch, n_out) or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 tensor of shape [batch, n_out]")
    if ntok.dtype != torch.int32 or ntok.shape != (batch,) or not ntok.is_contiguous():
        raise ValueError("ntok must be a contiguous int32 tensor of shape [batch]")
    bsl_kmer_tokenize(batch, bases, bases.numel(), starts, k, n_out, ids, ntok, stream)
    return ids, ntok


def bsl_destroy(plan):
    _check(load().bsl_destroy(plan))


def bsl_status_string(status):
    return load().bsl_status_string(status).decode()


def bsl_last_error():
    return load().bsl_last_error().decode()


def bsl_version():
    return load().bsl_version()


# ------------------------------------------------------ torch convenience

def require(name, t, dtype, shape, device):
    """Raise ValueError unless ``t`` is a contiguous CUDA tensor of this dtype
    and shape on ``device`` (the device of q: every pointer a call takes must
    be memory that GPU can read or write; a host tensor's address handed to a
    kernel would fault it)."""
    if t.device != device:
        raise ValueError(f"{name} must be a tensor on {device} (the device of q)")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def check_padded(q, k, v, o, seqlens, lse, dtype):
    """Tensors of a padded-layout call: q, k, v, o [batch, heads, n, d] of the
    plan's dtype, seqlens int32 [batch] (or None), lse float32 [batch, heads, n]
    (or None), all contiguous on q's device."""
    import torch
    if not getattr(q, "is_cuda", False):
        raise ValueError("q must be a CUDA tensor")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        require(name, t, dtype, tuple(q.shape), q.device)
    if seqlens is not None:
        require("seqlens", seqlens, torch.int32, (q.shape[0],), q.device)
    if lse is not None:
        require("lse", lse, torch.float32, tuple(q.shape[:3]), q.device)


def check_packed(q, k, v, o, cu_seqlens, lse, dtype):
    """Tensors of a packed-layout call: q, k, v, o [tokens, heads, d] of the
    plan's dtype, cu_seqlens int32 [batch + 1], lse float32 [heads, tokens]
    (or None), all contiguous on q's device."""
    import torch
    if not getattr(q, "is_cuda", False):
        raise ValueError("q must be a CUDA tensor")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        require(name, t, dtype, tuple(q.shape), q.device)
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must be an int32 CUDA tensor of shape [batch + 1]")
    require("cu_seqlens", cu_seqlens, torch.int32, tuple(cu_seqlens.shape), q.device)
    if lse is not None:
        require("lse", lse, torch.float32, (q.shape[1], q.shape[0]), q.device)


class Plan:
    """A plan plus shape/dtype checks for torch tensors on the current GPU."""

    def __init__(self, head_dim, heads, radius, causal=False, dtype="bf16", scale=0.0, window=0):
        self.head_dim, self.heads, self.radius, self.causal = head_dim, heads, radius, causal
        self.dtype, self.window = dtype, window
        code = {"bf16": BSL_BF16, "f32": BSL_F32}[dtype]
        self.handle = bsl_create(BslDesc(head_dim, heads, radius, causal, code, scale,
                                         window=window))

    @property
    def band_radius(self):
        """The block radius the kernels sweep: R, or ceil(W / 32) with a token window."""
        return -(-self.window // 32) if self.window > 0 else self.radius

    def close(self):
        if self.handle is not None:
            bsl_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _tdt(self):
        import torch
        return {"bf16": torch.bfloat16, "f32": torch.float32}[self.dtype]

    def _check_tensors(self, q, k, v, o, seqlens, lse):
        if q.dim() != 4 or q.shape[1] != self.heads or q.shape[3] != self.head_dim:
            raise ValueError(f"q must be [batch, {self.heads}, n, {self.head_dim}]")
        check_padded(q, k, v, o, seqlens, lse, self._tdt())

    def forward(self, q, k, v, seqlens=None, o=None, lse=None, stream=None):
        import torch
        if o is None:
            o = torch.empty_like(q)
        self._check_tensors(q, k, v, o, seqlens, lse)
        bsl_forward(self.handle, q.shape[0], q.shape[2], q, k, v, o, seqlens, lse, stream)
        return o

    def forward_traced(self, q, k, v, seqlens=None, o=None, lse=None, stream=None):
        """Returns (o, active, masks); see bsl_forward_traced in include/bsl.h."""
        import torch
        if o is None:
            o = torch.empty_like(q)
        self._check_tensors(q, k, v, o, seqlens, lse)
        batch, n = q.shape[0], q.shape[2]
        w = 2 * self.band_radius + 1
        active = torch.empty((batch, n // 32, w), dtype=torch.int32, device=q.device)
        masks = torch.empty((batch, n // 32, w, 32), dtype=torch.int32, device=q.device)
        bsl_forward_traced(self.handle, batch, n, q, k, v, o, seqlens, lse, active, masks, stream)
        return o, active, masks

    def forward_varlen(self, q, k, v, cu_seqlens, max_seqlen, o=None, lse=None, stream=None):
        """Packed layout: q, k, v [tokens, heads, head_dim]; cu_seqlens int32
        [batch + 1] on the device; lse float32 [heads, tokens].  See
        bsl_forward_varlen in include/bsl.h."""
        import torch
        if o is None:
            o = torch.empty_like(q)
        if q.dim() != 3 or q.shape[1] != self.heads or q.shape[2] != self.head_dim:
            raise ValueError(f"q must be [tokens, {self.heads}, {self.head_dim}]")
        check_packed(q, k, v, o, cu_seqlens, lse, self._tdt())
        bsl_forward_varlen(self.handle, cu_seqlens.shape[0] - 1, q.shape[0], max_seqlen, q, k, v,
                           o, cu_seqlens, lse, stream)
        return o

    def backward_varlen(self, q, k, v, o, dout, lse, cu_seqlens, max_seqlen, dq=None, dk=None,
                        dv=None, delta=None, stream=None):
        """Packed layout: q, k, v, o, dout, dq, dk, dv [tokens, heads, head_dim];
        lse and delta float32 [heads, tokens].  Returns (dq, dk, dv); rows outside
        every sequence keep what dq, dk, dv held.  See bsl_backward_varlen in
        include/bsl.h."""
        import torch
        dq = torch.zeros_like(q) if dq is None else dq
        dk = torch.zeros_like(q) if dk is None else dk
        dv = torch.zeros_like(q) if dv is None else dv
        if delta is None:
            delta = torch.empty((self.heads, q.shape[0]), dtype=torch.float32, device=q.device)
        if q.dim() != 3 or q.shape[1] != self.heads or q.shape[2] != self.head_dim:
            raise ValueError(f"q must be [tokens, {self.heads}, {self.head_dim}]")
        if lse is None:
            raise ValueError("the backward pass needs the lse the forward wrote")
        check_packed(q, k, v, o, cu_seqlens, lse, self._tdt())
        for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
            require(name, t, q.dtype, tuple(q.shape), q.device)
        require("delta", delta, torch.float32, (self.heads, q.shape[0]), q.device)
        bsl_backward_varlen(self.handle, cu_seqlens.shape[0] - 1, q.shape[0], max_seqlen, q, k, v,
                            o, dout, lse, cu_seqlens, dq, dk, dv, delta, stream)
        return dq, dk, dv

    def backward(self, q, k, v, o, dout, lse, seqlens=None, dq=None, dk=None, dv=None,
                 delta=None, stream=None):
        """Returns (dq, dk, dv); see bsl_backward in include/bsl.h.  ``lse`` is the
        one the forward wrote; ``delta`` (float32 [batch, heads, n]) is made here
        when not given."""
        import torch
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
        if delta is None:
            delta = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        if lse is None:
            raise ValueError("the backward pass needs the lse the forward wrote")
        self._check_tensors(q, k, v, o, seqlens, lse)
        for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
            require(name, t, q.dtype, tuple(q.shape), q.device)
        require("delta", delta, torch.float32, tuple(q.shape[:3]), q.device)
        bsl_backward(self.handle, q.shape[0], q.shape[2], q, k, v, o, dout, lse, seqlens, dq, dk,
                     dv, delta, stream)
        return dq, dk, dv
