"""Pins for the oracle's token-window variant (CPU only).

The NucleoByte page bounds attention to a local neighbourhood W (section 2,
item 3) but gives no rule for it beyond the block band; read plainly, key s is in
reach of query t when |t - s| <= W.  The oracle's window mode is pinned by:
  * W = 0: every row attends to itself alone, so O = V row by row and lse is
    the row's own score (closed form);
  * W at least the sequence length: plain dense attention, against torch's
    scaled_dot_product_attention in fp64 with an explicit padding/causal mask
    (an independent library routine);
  * brute force with an explicit n x n token mask and a dense softmax;
  * the page's block recurrence run in window mode against the two-pass
    definition;
  * the block lists: exactly the blocks holding a kept pair, and the masks bit
    for bit against the token mask.
"""
import numpy as np
import pytest
import torch

import oracle
from tests._brute import dense_reference, token_mask


def _draw(rng, batch, heads, n, d):
    return [rng.standard_normal((batch, heads, n, d)).astype(np.float32) for _ in range(3)]


@pytest.mark.parametrize("causal", [False, True])
def test_window_zero_is_identity(causal):
    rng = np.random.default_rng(11)
    q, k, v = _draw(rng, 2, 2, 64, 8)
    lens = np.array([64, 37], dtype=np.int32)
    o, lse, psum = oracle.forward(q, k, v, lens, 32, 0, causal, window=0)
    for b, L in enumerate(lens):
        assert np.array_equal(o[b, :, :L], v[b, :, :L].astype(np.float64))
        own = np.einsum("hnd,hnd->hn", q[b].astype(np.float64), k[b].astype(np.float64)) / np.sqrt(8)
        assert np.allclose(lse[b, :, :L], own[:, :L], atol=1e-12, rtol=0)
        assert np.all(o[b, :, L:] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_window_covering_everything_is_dense_sdpa(causal):
    rng = np.random.default_rng(12)
    n, d = 96, 16
    q, k, v = _draw(rng, 2, 3, n, d)
    lens = np.array([96, 61], dtype=np.int32)
    o, _, _ = oracle.forward(q, k, v, lens, 32, 0, causal, window=n)
    for b, L in enumerate(lens):
        qt, kt, vt = (torch.from_numpy(x[b, :, :L].astype(np.float64)) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
        assert np.max(np.abs(o[b, :, :L] - ref.numpy())) <= 1e-12


@pytest.mark.parametrize("bsize", [4, 8, 32])
@pytest.mark.parametrize("window", [1, 3, 7, 8, 9, 31, 32, 33, 50])
@pytest.mark.parametrize("causal", [False, True])
def test_window_brute_force_and_recurrence(bsize, window, causal):
    rng = np.random.default_rng(bsize * 100 + window)
    n = 4 * 32
    q, k, v = _draw(rng, 2, 2, n, 8)
    lens = np.array([n, 77], dtype=np.int32)
    o, lse, psum = oracle.forward(q, k, v, lens, bsize, 0, causal, window=window)
    ro, rl = dense_reference(q, k, v, lens, bsize, 0, causal, window=window)
    assert np.max(np.abs(o - ro)) <= 1e-12
    for b, L in enumerate(lens):
        assert np.allclose(lse[b, :, :L], rl[b, :, :L], atol=1e-12, rtol=0)
        assert np.allclose(psum[b, :, :L], 1.0, atol=1e-13)
    r = oracle.forward_recurrence(q, k, v, lens, bsize, 0, causal, window=window)
    assert np.max(np.abs(r - ro)) <= 1e-12


@pytest.mark.parametrize("window", [0, 1, 31, 32, 33, 64, 100])
@pytest.mark.parametrize("causal", [False, True])
def test_window_lists_and_masks_brute_force(window, causal):
    bsize, nblk = 32, 9
    n = nblk * bsize
    lens = np.array([n, 200, 33, 0], dtype=np.int32)
    act = oracle.active_blocks(len(lens), n, bsize, 0, causal, lens, window=window)
    msk = oracle.masks(len(lens), n, bsize, 0, causal, lens, act, window=window)
    assert act.shape[2] == 2 * oracle.window_radius(window, bsize) + 1
    for b, L in enumerate(lens):
        keep = token_mask(n, int(L), bsize, 0, causal, window)
        for i in range(nblk):
            rows = keep[i * bsize:(i + 1) * bsize]
            ref = [j for j in range(nblk) if rows[:, j * bsize:(j + 1) * bsize].any()]
            assert [int(j) for j in act[b, i] if j >= 0] == ref, (b, i)
            for slot, j in enumerate(act[b, i]):
                if j < 0:
                    assert np.all(msk[b, i, slot] == 0)
                    continue
                blk = rows[:, j * bsize:(j + 1) * bsize]
                words = [sum(1 << c for c in range(bsize) if blk[r, c]) for r in range(bsize)]
                assert list(msk[b, i, slot]) == words


def test_window_constant_values_and_shift_invariance():
    rng = np.random.default_rng(13)
    q, k, v = _draw(rng, 1, 2, 96, 8)
    lens = np.array([90], dtype=np.int32)
    c = np.full_like(v, 0.625)
    o, _, _ = oracle.forward(q, k, c, lens, 32, 0, False, window=20)
    assert np.allclose(o[0, :, :90], 0.625, atol=1e-14, rtol=0)
    # a vector added to every key shifts each row's scores by one constant
    o1, _, _ = oracle.forward(q, k, v, lens, 32, 0, False, window=20)
    u = rng.standard_normal(8).astype(np.float32)
    o2, _, _ = oracle.forward(q, (k + u).astype(np.float32), v, lens, 32, 0, False, window=20)
    assert np.max(np.abs(o1 - o2)) <= 1e-5


def test_window_rejects_a_band_too_narrow():
    rng = np.random.default_rng(14)
    q, k, v = _draw(rng, 1, 1, 64, 8)
    lib = oracle.load()
    import ctypes
    out = np.zeros((1, 1, 64, 8))
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    rc = lib.orc_forward_w_f64(1, 1, 64, 8, 32, 0, 0, 40, 0.0, None, q.ctypes.data_as(f32p),
                               k.ctypes.data_as(f32p), v.ctypes.data_as(f32p),
                               out.ctypes.data_as(f64p), None, None, 1)
    assert rc == -1   # W = 40 needs a block radius of 2
    rc = lib.orc_forward_w_f64(1, 1, 64, 8, 32, 2, 0, -2, 0.0, None, q.ctypes.data_as(f32p),
                               k.ctypes.data_as(f32p), v.ctypes.data_as(f32p),
                               out.ctypes.data_as(f64p), None, None, 1)
    assert rc == -1


# ------------------------------------------------------------ backward pins

DYADIC = 2.0 ** -7  # inputs are multiples of this; the perturbations stay exact


def _dyadic(rng, shape, lim=1.0):
    return (np.round(rng.uniform(-lim, lim, shape) / DYADIC) * DYADIC).astype(np.float32)


def _fd_window(q, k, v, g, lens, bsize, window, causal, which, idx):
    """Richardson-extrapolated central difference of sum(O * g) in one input
    element, through the window forward."""
    args = [q, k, v]

    def at(delta):
        a = [x.copy() for x in args]
        a[which][idx] = np.float32(float(args[which][idx]) + delta)
        assert float(a[which][idx]) == float(args[which][idx]) + delta
        o, _, _ = oracle.forward(*a, lens, bsize, 0, causal, window=window, nthreads=1)
        return float(np.sum(o * g.astype(np.float64)))

    def central(h):
        return (at(h) - at(-h)) / (2 * h)

    h = 2.0 ** -10
    return (4 * central(h / 2) - central(h)) / 3


@pytest.mark.parametrize("bsize,nblk,window,causal,lens,d", [
    (8, 5, 3, False, [40, 29], 8),
    (8, 5, 9, True, [40, 19], 8),
    (4, 8, 6, False, [32, 13], 4),
    (16, 3, 20, True, [48, 48], 8),
])
def test_window_backward_matches_finite_differences(bsize, nblk, window, causal, lens, d):
    rng = np.random.default_rng(window * 7 + nblk)
    n = nblk * bsize
    lens = np.array(lens, np.int32)
    q, k, v, g = (_dyadic(rng, (len(lens), 2, n, d)) for _ in range(4))
    dq, dk, dv = oracle.backward(q, k, v, g, lens, bsize, 0, causal, window=window, nthreads=1)
    grads = (dq, dk, dv)
    for which in range(3):
        for _ in range(6):
            b = int(rng.integers(len(lens)))
            t = int(rng.integers(max(1, int(lens[b]))))
            idx = (b, int(rng.integers(2)), t, int(rng.integers(d)))
            fd = _fd_window(q, k, v, g, lens, bsize, window, causal, which, idx)
            assert abs(grads[which][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (which, idx)


@pytest.mark.parametrize("causal", [False, True])
def test_window_zero_backward_closed_form(causal):
    """W = 0: every row attends to itself alone, so O = V, dV = dO and the
    query and key gradients vanish, exactly."""
    rng = np.random.default_rng(11)
    lens = np.array([64, 37], np.int32)
    q, k, v, g = _draw(rng, 2, 3, 64, 8) + _draw(rng, 2, 3, 64, 8)[:1]
    dq, dk, dv = oracle.backward(q, k, v, g, lens, 32, 0, causal, window=0)
    for b, L in enumerate(lens):
        assert np.array_equal(dv[b, :, :L], g[b, :, :L].astype(np.float64))
        assert np.all(dq[b] == 0.0) and np.all(dk[b] == 0.0)
        assert np.all(dv[b, :, L:] == 0.0)


def test_window_covering_everything_backward_is_the_covering_band():
    rng = np.random.default_rng(12)
    lens = np.array([96, 50], np.int32)
    q, k, v, g = _draw(rng, 2, 2, 96, 8) + _draw(rng, 2, 2, 96, 8)[:1]
    a = oracle.backward(q, k, v, g, lens, 32, 0, False, window=96)
    b = oracle.backward(q, k, v, g, lens, 32, 3, False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_window_backward_blocks_match_full():
    rng = np.random.default_rng(13)
    lens = np.array([160, 75], np.int32)
    q, k, v, g = _draw(rng, 2, 2, 160, 8) + _draw(rng, 2, 2, 160, 8)[:1]
    for causal in (False, True):
        full = oracle.backward(q, k, v, g, lens, 32, 0, causal, window=40)
        sel = np.array([(b, h, i) for b in range(2) for h in range(2) for i in range(5)], np.int32)
        blk = oracle.backward_blocks(q, k, v, g, sel, lens, 32, 0, causal, window=40)
        for x, y in zip(full, blk):
            got = np.stack([x[b, h, i * 32:(i + 1) * 32] for b, h, i in sel])
            assert np.allclose(got, y, rtol=0, atol=1e-12)
