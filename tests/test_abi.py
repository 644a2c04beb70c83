"""The C-ABI library on the CPU: it loads, exports what include/bsl.h declares,
and rejects bad arguments before touching a device.  No compute call here."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

from block_sparse_local_amd import bsl, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsl.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsl.LIB_PATH):
        from block_sparse_local_amd import build
        build.build()
    return bsl.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsl_[a-z_]+)\s*\(", text)))


def test_desc_layout_matches_header():
    """bsl_desc is seven int32/float fields then window: 32 bytes, window last."""
    assert ctypes.sizeof(bsl.BslDesc) == 32
    assert bsl.BslDesc.window.offset == 28
    assert bsl.BslDesc().window == 0


def test_header_and_binding_agree():
    assert _declared() == sorted(bsl.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bsl.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_matches_header(lib):
    m = re.search(r"#define BSL_VERSION (\d+)", open(HEADER).read())
    assert bsl.bsl_version() == int(m.group(1))


def test_status_strings(lib):
    for code in range(5):
        assert bsl.bsl_status_string(code).startswith("BSL_")
    assert "unknown" in bsl.bsl_status_string(99)


def _create_status(lib, **kw):
    desc = bsl.BslDesc(**kw)
    plan = ctypes.c_void_p()
    return lib.bsl_create(ctypes.byref(desc), ctypes.byref(plan)), plan


@pytest.mark.parametrize("kw,status", [
    (dict(heads=0), bsl.BSL_E_INVALID),
    (dict(radius=-1), bsl.BSL_E_INVALID),
    (dict(causal=2), bsl.BSL_E_INVALID),
    (dict(scale=float("nan")), bsl.BSL_E_INVALID),
    (dict(block_size=16), bsl.BSL_E_UNSUPPORTED),
    (dict(head_dim=48), bsl.BSL_E_UNSUPPORTED),
    (dict(head_dim=256), bsl.BSL_E_UNSUPPORTED),
    (dict(dtype=7), bsl.BSL_E_UNSUPPORTED),
    (dict(window=-1), bsl.BSL_E_INVALID),
    (dict(window=(1 << 29) + 1), bsl.BSL_E_UNSUPPORTED),
])
def test_create_rejects_bad_descriptors_before_device_use(lib, kw, status):
    st, plan = _create_status(lib, **kw)
    assert st == status
    assert plan.value is None
    assert bsl.bsl_last_error() != ""


def test_null_arguments(lib):
    assert lib.bsl_create(None, None) == bsl.BSL_E_INVALID
    assert lib.bsl_forward(None, 1, 32, 16, 16, 16, 16, None, None, None) == bsl.BSL_E_INVALID
    assert "plan" in bsl.bsl_last_error()
    assert lib.bsl_forward_traced(None, 1, 32, 16, 16, 16, 16, None, None, 16, 16,
                                  None) == bsl.BSL_E_INVALID
    assert lib.bsl_forward_varlen(None, 1, 64, 64, 16, 16, 16, 16, 16, None,
                                  None) == bsl.BSL_E_INVALID
    assert "plan" in bsl.bsl_last_error()
    assert lib.bsl_backward(None, 1, 32, 16, 16, 16, 16, 16, 16, None, 16, 16, 16, 16,
                            None) == bsl.BSL_E_INVALID
    assert lib.bsl_backward_varlen(None, 1, 64, 64, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16,
                                   None) == bsl.BSL_E_INVALID
    assert "plan" in bsl.bsl_last_error()
    assert lib.bsl_destroy(None) == bsl.BSL_OK


def test_varlen_offsets_collate_lengths(lib):
    """The host collator: exclusive prefix sums, the longest length and the
    dynamic ceiling (the longest length rounded up to a multiple of 32)."""
    rng = np.random.default_rng(4)
    for lens in ([], [0], [1], [32], [33, 0, 5], list(rng.integers(0, 3000, 64))):
        cu, mx, ceil = bsl.bsl_varlen_offsets(lens)
        assert cu.tolist() == [0] + np.cumsum(np.asarray(lens, np.int64)).tolist()
        assert mx == (max(lens) if len(lens) else 0)
        assert ceil % 32 == 0 and ceil - 32 < mx <= ceil if mx else ceil == 0
    # the ragged mRNA batch: the ceiling is the padded buffer length it is drawn with
    w = inputs.WORKLOADS["c2"]
    lens, n = inputs.lengths(w, 42)
    cu, mx, ceil = bsl.bsl_varlen_offsets(lens)
    assert ceil == n and mx == int(lens.max()) and cu[-1] == int(lens.sum())


@pytest.mark.parametrize("lens", [[3, -1, 4], [2 ** 31 - 1, 1], [2 ** 31 - 20]])
def test_varlen_offsets_reject_bad_lengths_and_write_nothing(lib, lens):
    i32p = ctypes.POINTER(ctypes.c_int32)
    a = np.asarray(lens, np.int32)
    cu = np.full(len(lens) + 1, -7, np.int32)
    mx, ceil = ctypes.c_int32(-7), ctypes.c_int32(-7)
    st = lib.bsl_varlen_offsets(len(lens), a.ctypes.data_as(i32p), cu.ctypes.data_as(i32p),
                                ctypes.byref(mx), ctypes.byref(ceil))
    assert st == bsl.BSL_E_INVALID and bsl.bsl_last_error() != ""
    assert np.all(cu == -7) and mx.value == -7 and ceil.value == -7


def test_varlen_offsets_null_pointers(lib):
    i32p = ctypes.POINTER(ctypes.c_int32)
    cu = np.zeros(2, np.int32)
    a = np.ones(1, np.int32)
    mx, ceil = ctypes.c_int32(), ctypes.c_int32()
    assert lib.bsl_varlen_offsets(1, None, cu.ctypes.data_as(i32p), ctypes.byref(mx),
                                  ctypes.byref(ceil)) == bsl.BSL_E_INVALID
    assert lib.bsl_varlen_offsets(1, a.ctypes.data_as(i32p), None, ctypes.byref(mx),
                                  ctypes.byref(ceil)) == bsl.BSL_E_INVALID
    assert lib.bsl_varlen_offsets(-1, a.ctypes.data_as(i32p), cu.ctypes.data_as(i32p),
                                  ctypes.byref(mx), ctypes.byref(ceil)) == bsl.BSL_E_INVALID
    assert lib.bsl_varlen_offsets(0, None, cu.ctypes.data_as(i32p), ctypes.byref(mx),
                                  ctypes.byref(ceil)) == bsl.BSL_OK


def test_binding_raises_on_error(lib):
    with pytest.raises(bsl.BslError) as e:
        bsl.bsl_create(bsl.BslDesc(head_dim=48))
    assert e.value.status == bsl.BSL_E_UNSUPPORTED


def test_library_override_is_loud_when_missing(tmp_path):
    """BSL_LIBRARY points the binding at another build; a missing one is an error,
    never a silent fall back to anything else."""
    missing = tmp_path / "not_built.so"
    code = ("import sys\n"
            "from block_sparse_local_amd import bsl\n"
            "try:\n"
            "    bsl.load()\n"
            "except bsl.BslError as e:\n"
            "    print('BslError', e)\n"
            "    sys.exit(3)\n")
    env = dict(os.environ, BSL_LIBRARY=str(missing))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 3, r.stdout + r.stderr
    assert str(missing) in r.stdout


def test_kmer_ceiling_host():
    import numpy as np
    assert bsl.bsl_kmer_ceiling(np.array([0, 100, 2100]), 6) == 2016
    assert bsl.bsl_kmer_ceiling(np.array([0, 3]), 6) == 0
    assert bsl.bsl_kmer_ceiling(np.array([0, 38]), 6) == 64
    assert bsl.bsl_kmer_ceiling(np.array([7]), 6) == 0
    for starts, k in (([5, 3], 6), ([-1, 3], 6), ([0, 8], 0), ([0, 8], 13)):
        with pytest.raises(bsl.BslError):
            bsl.bsl_kmer_ceiling(np.array(starts), k)


def test_kmer_argument_errors_before_any_launch(lib):
    """Rejected before anything touches a device (these run without a GPU)."""
    bad = [(-1, 1, 8, 6, 8), (2, -1, 8, 6, 8), (2, 8, 8, 0, 8), (2, 8, 8, 13, 8),
           (2, 8, 8, 6, -1)]
    for batch, nbytes, st, k, n_out in bad:
        assert lib.bsl_kmer_tokenize(batch, 4096, nbytes, 8192, k, n_out, 16384, None, None) == 1
    # NULL starts or ids
    assert lib.bsl_kmer_tokenize(2, 4096, 8, None, 6, 8, 16384, None, None) == 1
    assert lib.bsl_kmer_tokenize(2, 4096, 8, 8192, 6, 8, None, None, None) == 1
    # ids overlapping the text
    assert lib.bsl_kmer_tokenize(2, 4096, 100, 8192, 6, 8, 4100, None, None) == 1
    # batch 0 is a no-op
    assert lib.bsl_kmer_tokenize(0, None, 0, None, 6, 8, None, None, None) == 0


def test_check_validators_reject_bad_arguments_before_any_launch(lib):
    """The length/offset validators validate their arguments on the host, so
    these errors need no GPU; nothing is launched."""
    fake = ctypes.c_void_p(0x10000)
    other = ctypes.c_void_p(0x20000)
    assert lib.bsl_check_seqlens(-1, 32, fake, other, None) == bsl.BSL_E_INVALID
    assert lib.bsl_check_seqlens(2, -1, fake, other, None) == bsl.BSL_E_INVALID
    assert lib.bsl_check_seqlens(2, 32, None, other, None) == bsl.BSL_E_INVALID
    assert lib.bsl_check_seqlens(2, 32, fake, None, None) == bsl.BSL_E_INVALID
    # the result may not overlap the checked array
    assert lib.bsl_check_seqlens(4, 32, fake, ctypes.c_void_p(0x10008), None) == bsl.BSL_E_INVALID
    assert lib.bsl_check_cu_seqlens(-1, 10, fake, other, None) == bsl.BSL_E_INVALID
    assert lib.bsl_check_cu_seqlens(1, -5, fake, other, None) == bsl.BSL_E_INVALID
    # offsets always hold batch + 1 entries, so NULL is an error even for batch 0
    assert lib.bsl_check_cu_seqlens(0, 10, None, other, None) == bsl.BSL_E_INVALID
    assert lib.bsl_check_cu_seqlens(2, 10, fake, ctypes.c_void_p(0x10004), None) == bsl.BSL_E_INVALID
    assert "overlaps" in bsl.bsl_last_error()
