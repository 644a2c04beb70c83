"""GPU parity of the token-window variant (bsl_desc.window = W >= 1): key s is
scored for query t when |t - s| <= W, the plain reading of the local
neighbourhood W of the NucleoByte project page (section 2, "The Architectural
Goal", item 3); the kernels sweep the blocks within ceil(W/32) of the query block
and mask per token.  The oracle's window mode is pinned in
test_oracle_window.py.

Checked here, through the C ABI:
  * small ragged batches (lengths 0, 1, 31, 32, 33, ...) in both dtypes and
    every head size against the oracle, with the kernel's own active lists and
    masks bit-exact against the oracle's;
  * the packed layout against the oracle and bit for bit against the padded
    layout;
  * a window as wide as the buffer gives the same bits as the block band that
    covers the buffer (no token mask is then needed anywhere);
  * the 131072-token, 16-head, d 128 shape with W = 256 (the same eight-block
    band), sampled query blocks on every head against the oracle;
  * (the backward of a window plan: test_gpu_backward.py).
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_local_amd import bsl, inputs
from tests._gpu import LSE_TOL, check_rows, run, say
from tests.test_gpu_varlen import _check as check_packed
from tests.test_gpu_varlen import run_varlen

pytestmark = pytest.mark.gpu


def _case(seed, dtype, dd, nblk, lens, heads=2):
    n = nblk * 32
    q, k, v = inputs.draw(seed, 91, len(lens), heads, n, dd, 1.0, dtype == "bf16",
                          np.array(lens, np.int32), poison=True, threads=1)
    return dict(q=q, k=k, v=v, seqlens=np.array(lens, np.int32), n=n)


def _check_against_oracle(res, d, kw, window, what):
    lens = d["seqlens"]
    o, lse, _ = oracle.forward(d["q"], d["k"], d["v"], lens, 32, 0, kw["causal"], window=window)
    check_rows(res["o"], o, lens, kw["dtype"], what)
    for b, L in enumerate(lens):
        assert np.all(np.isneginf(res["lse"][b, :, L:]))
        if L:
            assert np.max(np.abs(res["lse"][b, :, :L] - lse[b, :, :L])) <= LSE_TOL[kw["dtype"]]
    batch = len(lens)
    act = oracle.active_blocks(batch, d["n"], 32, 0, kw["causal"], lens, window=window)
    msk = oracle.masks(batch, d["n"], 32, 0, kw["causal"], lens, act, window=window)
    assert res["active"].shape == act.shape
    assert np.array_equal(res["active"], act), f"{what}: active lists differ from the oracle"
    assert np.array_equal(res["masks"], msk), f"{what}: masks differ from the oracle"


CASES = []
for _dt in ("bf16", "f32"):
    for _w in (1, 7, 31, 32, 33, 100):
        for _c in (False, True):
            CASES.append((_dt, 64, _w, _c))
    for _dd in (32, 128):
        for _w in (9, 40):
            for _c in (False, True):
                CASES.append((_dt, _dd, _w, _c))


@pytest.mark.parametrize("dtype,dd,window,causal", CASES)
def test_window_small_ragged(dtype, dd, window, causal):
    nblk = 13
    lens = [nblk * 32, 0, 1, 31, 32, 33, 250, 385]
    d = _case(dd * 1000 + window * 2 + int(causal), dtype, dd, nblk, lens)
    # radius deliberately unrelated to the window: a window plan does not use it
    kw = dict(head_dim=dd, heads=2, radius=5, causal=causal, dtype=dtype, window=window)
    say(f"[window] small {kw}")
    res = run(kw, d, traced=True, with_lse=True)
    _check_against_oracle(res, d, kw, window, f"window {dtype} d{dd} W{window} c{int(causal)}")
    # the untraced launch computes the same bits
    plain = run(kw, d, with_lse=True)
    assert np.array_equal(plain["o"].view(np.uint32), res["o"].view(np.uint32))
    assert np.array_equal(plain["lse"].view(np.uint32), res["lse"].view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("window,causal", [(5, False), (64, True), (200, False)])
def test_window_packed_layout(dtype, window, causal):
    lens = [300, 0, 1, 31, 32, 33, 250, 416]
    n = 416
    d = _case(window * 3 + int(causal), dtype, 64, n // 32, lens)
    kw = dict(head_dim=64, heads=2, radius=0, causal=causal, dtype=dtype, window=window)
    say(f"[window] packed {kw}")
    res = run_varlen(kw, d, lens)
    o, lse, _ = oracle.forward(d["q"], d["k"], d["v"], d["seqlens"], 32, 0, causal,
                               window=window)
    padded = run(kw, d, with_lse=True)
    check_packed(res, d, lens, kw, ref=(o, lse), padded=padded)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_as_wide_as_the_buffer_is_the_covering_band(dtype):
    nblk = 9
    lens = [nblk * 32, 200, 33]
    d = _case(17, dtype, 128, nblk, lens)
    n = nblk * 32
    say(f"[window] W = n = {n} against R = {nblk} ({dtype})")
    win = run(dict(head_dim=128, heads=2, radius=0, causal=False, dtype=dtype, window=n),
              d, traced=True, with_lse=True)
    band = run(dict(head_dim=128, heads=2, radius=nblk, causal=False, dtype=dtype),
               d, traced=True, with_lse=True)
    assert np.array_equal(win["o"].view(np.uint32), band["o"].view(np.uint32))
    assert np.array_equal(win["lse"].view(np.uint32), band["lse"].view(np.uint32))
    assert np.array_equal(win["masks"], band["masks"])
    # the window's lists are ceil(n/32) = nblk blocks wide on either side
    assert win["active"].shape[2] == 2 * nblk + 1


def test_window_full_size_sampled():
    """131072 tokens, 16 heads, d 128, bf16, W = 256 (the eight-block band of
    the long-context workload, cut per token), one sequence of 120000 tokens
    (a ragged tail); sampled query blocks on every head against the oracle."""
    heads, n, dd, window = 16, 131072, 128, 256
    L = 120000
    say(f"[window] full size: 1 x {heads} x {n} x {dd}, W {window}, length {L}")
    lens = np.array([L], np.int32)
    q, k, v = inputs.draw(2024, 92, 1, heads, n, dd, 1.0, True, lens, poison=True)
    nblk, nb = n // 32, (L + 31) // 32
    rng = np.random.default_rng([2024, 92])
    blocks = sorted({0, 1, 2, nb - 3, nb - 2, nb - 1, nb, nblk - 1}
                    | set(int(x) for x in rng.choice(nblk, 40, replace=False)))
    sel = np.array([(0, h, i) for h in range(heads) for i in blocks], dtype=np.int32)
    ob, lb, _ = oracle.forward_blocks(q, k, v, sel, lens, 32, 0, False, window=window)
    rows = np.array([i * 32 + r for _, _, i in sel for r in range(32)]).reshape(len(sel), 32)
    valid = rows < L
    d = dict(q=q, k=k, v=v, seqlens=lens, n=n)
    kw = dict(head_dim=dd, heads=heads, radius=0, causal=False, dtype="bf16", window=window)
    res = run(kw, d, with_lse=True)
    got = np.stack([res["o"][b, h, i * 32:(i + 1) * 32] for b, h, i in sel])
    assert np.all(got[~valid] == 0.0)
    e = np.abs(got[valid].astype(np.float64) - ob[valid])
    say(f"  sampled {len(sel)} blocks: max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    assert e.max() <= 2e-2 and e.mean() <= 2e-3
    gl = np.stack([res["lse"][b, h, i * 32:(i + 1) * 32] for b, h, i in sel])
    assert np.all(np.isneginf(gl[~valid]))
    assert np.max(np.abs(gl[valid] - lb[valid])) <= LSE_TOL["bf16"]
    check_rows(res["o"], None, lens, "bf16", "window full size")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_extreme_window_and_radius(dtype):
    """The largest window (2^29, band 2^24 blocks) and the largest radius (2^24)
    are accepted and reduce to the band that covers the buffer: same bits."""
    nblk = 6
    lens = [nblk * 32, 77]
    d = _case(5, dtype, 64, nblk, lens)
    kw = dict(head_dim=64, heads=2, causal=False, dtype=dtype)
    say(f"[window] extreme window / radius ({dtype})")
    ref = run(dict(kw, radius=nblk), d, with_lse=True)
    for extra in (dict(radius=0, window=1 << 29), dict(radius=1 << 24)):
        got = run(dict(kw, **extra), d, with_lse=True)
        assert np.array_equal(got["o"].view(np.uint32), ref["o"].view(np.uint32)), extra
        assert np.array_equal(got["lse"].view(np.uint32), ref["lse"].view(np.uint32)), extra
