"""Pins of the oracle's backward pass (CPU only).

The oracle's gradients (NucleoByte project page, section 3, "Custom
Backpropagation": D_t and dS_ts as written there, dQ, dK, dV by the chain
rule) are tied to things other than themselves:
  * central finite differences of the forward oracle (itself pinned by
    test_oracle_forward.py), Richardson-extrapolated, on inputs for which every
    perturbed value is exact in float32;
  * torch's fp64 autograd through an explicit masked softmax attention, when
    the radius covers the whole sequence (a library routine, written unlike
    the oracle);
  * invariants: the value gradients sum to the summed output gradients, the key
    gradients sum to zero, a constant shift of every key changes nothing,
    scaling V scales dQ and dK, causal row 0 has zero query gradient, padding
    gets zero gradient.
"""
import numpy as np
import pytest

import oracle

DYADIC = 2.0 ** -7  # inputs are multiples of this; perturbations below stay exact


def _dyadic(rng, shape, lim=1.0):
    return (np.round(rng.uniform(-lim, lim, shape) / DYADIC) * DYADIC).astype(np.float32)


def _loss(q, k, v, g, lens, bsize, radius, causal, scale=0.0):
    o, _, _ = oracle.forward(q, k, v, lens, bsize, radius, causal, scale, nthreads=1)
    return float(np.sum(o * g.astype(np.float64)))


def _fd(q, k, v, g, lens, bsize, radius, causal, which, idx, scale=0.0):
    """Richardson-extrapolated central difference of the loss in one element."""
    args = [q, k, v]
    x = args[which]

    def at(delta):
        y = x.copy()
        y[idx] = np.float32(float(x[idx]) + delta)
        assert float(y[idx]) == float(x[idx]) + delta  # exact in float32
        a = list(args)
        a[which] = y
        return _loss(*a, g, lens, bsize, radius, causal, scale)

    def central(h):
        return (at(h) - at(-h)) / (2 * h)

    h = 2.0 ** -10
    return (4 * central(h / 2) - central(h)) / 3


CASES = [
    # bsize, nblk, radius, causal, lens, d
    (8, 5, 1, False, [40, 29], 8),
    (8, 5, 2, True, [40, 19], 8),
    (4, 8, 0, False, [32, 13], 4),
    (16, 3, 1, True, [48, 48], 8),
]


@pytest.mark.parametrize("case", CASES)
def test_gradients_match_finite_differences(case):
    bsize, nblk, radius, causal, lens, d = case
    n = nblk * bsize
    rng = np.random.default_rng(7 + nblk + radius)
    q, k, v, g = [_dyadic(rng, (2, 1, n, d)) for _ in range(4)]
    lens = np.array(lens, dtype=np.int32)
    grads = oracle.backward(q, k, v, g, lens, bsize, radius, causal, nthreads=1)
    for which in range(3):
        # elements in valid rows of both sequences, plus one padded row
        picks = [(0, 0, int(rng.integers(0, lens[0])), int(rng.integers(0, d))) for _ in range(6)]
        picks += [(1, 0, int(rng.integers(0, lens[1])), int(rng.integers(0, d))) for _ in range(6)]
        if lens[1] < n:
            picks.append((1, 0, int(lens[1]), 0))
        for idx in picks:
            fd = _fd(q, k, v, g, lens, bsize, radius, causal, which, idx)
            an = grads[which][idx]
            assert abs(fd - an) <= 1e-8 + 1e-7 * abs(an), (which, idx, fd, an)


def test_custom_scale_matches_finite_differences():
    rng = np.random.default_rng(11)
    n, d = 24, 8
    q, k, v, g = [_dyadic(rng, (1, 1, n, d)) for _ in range(4)]
    lens = np.array([21], dtype=np.int32)
    scale = 0.75
    dq, dk, dv = oracle.backward(q, k, v, g, lens, 8, 1, False, scale, nthreads=1)
    for which, grad in enumerate((dq, dk, dv)):
        for idx in [(0, 0, 3, 1), (0, 0, 17, 6), (0, 0, 20, 0)]:
            fd = _fd(q, k, v, g, lens, 8, 1, False, which, idx, scale)
            assert abs(fd - grad[idx]) <= 1e-8 + 1e-7 * abs(grad[idx])


def _torch_dense(q, k, v, g, lens, causal, scale):
    torch = pytest.importorskip("torch")
    qt, kt, vt = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    gt = torch.tensor(g, dtype=torch.float64)
    batch, heads, n, d = q.shape
    loss = 0.0
    for b in range(batch):
        L = int(lens[b])
        if L == 0:
            continue
        s = torch.matmul(qt[b, :, :L], kt[b, :, :L].transpose(-1, -2)) * scale
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), vt[b, :, :L])
        loss = loss + (o * gt[b, :, :L]).sum()
    loss.backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_dense_case_matches_torch_autograd(causal):
    rng = np.random.default_rng(3)
    bsize, nblk, d = 16, 4, 16
    n = nblk * bsize
    q, k, v, g = [rng.standard_normal((3, 2, n, d)).astype(np.float32) for _ in range(4)]
    lens = np.array([64, 37, 1], dtype=np.int32)
    radius = nblk - 1  # every block in every band: dense attention
    ours = oracle.backward(q, k, v, g, lens, bsize, radius, causal)
    ref = _torch_dense(q, k, v, g, lens, causal, 1.0 / np.sqrt(d))
    for a, r in zip(ours, ref):
        assert np.max(np.abs(a - r)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    rng = np.random.default_rng(5)
    bsize, nblk, radius, d = 8, 6, 1, 8
    n = nblk * bsize
    q, k, v, g = [_dyadic(rng, (2, 2, n, d)) for _ in range(4)]
    lens = np.array([48, 27], dtype=np.int32)
    dq, dk, dv = oracle.backward(q, k, v, g, lens, bsize, radius, causal)
    for b in range(2):
        L = lens[b]
        # sum over keys of dV = sum over valid rows of dO (each row's P sums to 1)
        assert np.allclose(dv[b].sum(axis=1), g[b, :, :L].astype(np.float64).sum(axis=1),
                           atol=1e-12)
        # sum over keys of dK = 0 (each row's dS sums to zero)
        assert np.max(np.abs(dk[b].sum(axis=1))) <= 1e-12
        # padding: no gradient
        for x in (dq, dk, dv):
            assert not np.any(x[b, :, L:])
    if causal:
        # row 0 attends to key 0 alone: its softmax is constant
        assert np.max(np.abs(dq[:, :, 0])) <= 1e-13
    # a constant shift of every key changes no row's softmax: same gradients
    u = _dyadic(rng, (1, 1, 1, d), lim=0.5)
    dq2, dk2, dv2 = oracle.backward(q, (k + u).astype(np.float32), v, g, lens, bsize, radius,
                                    causal)
    for a, b_ in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert np.max(np.abs(a - b_)) <= 1e-12
    # V -> 2V scales dQ and dK by 2 and leaves dV alone
    dq3, dk3, dv3 = oracle.backward(q, k, (2 * v).astype(np.float32), g, lens, bsize, radius,
                                    causal)
    assert np.max(np.abs(dq3 - 2 * dq)) <= 1e-12
    assert np.max(np.abs(dk3 - 2 * dk)) <= 1e-12
    assert np.max(np.abs(dv3 - dv)) <= 1e-12


def test_blocks_match_full_backward():
    rng = np.random.default_rng(9)
    bsize, nblk, radius, d = 8, 7, 2, 8
    n = nblk * bsize
    q, k, v, g = [rng.standard_normal((2, 2, n, d)).astype(np.float32) for _ in range(4)]
    lens = np.array([56, 30], dtype=np.int32)
    for causal in (False, True):
        dq, dk, dv = oracle.backward(q, k, v, g, lens, bsize, radius, causal)
        sel = np.array([[0, 0, 0], [0, 1, 3], [1, 0, 3], [1, 1, 6], [0, 1, 6]], dtype=np.int32)
        bq, bk, bv = oracle.backward_blocks(q, k, v, g, sel, lens, bsize, radius, causal)
        for w, (b, h, i) in enumerate(sel):
            rows = slice(i * bsize, (i + 1) * bsize)
            assert np.max(np.abs(bq[w] - dq[b, h, rows])) <= 1e-13
            assert np.max(np.abs(bk[w] - dk[b, h, rows])) <= 1e-13
            assert np.max(np.abs(bv[w] - dv[b, h, rows])) <= 1e-13


def test_backward_rejects_bad_arguments():
    q = np.zeros((1, 1, 64, 8), dtype=np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.backward(q, q, q, q, [65], 32, 1, False)   # length past the buffer
    with pytest.raises(oracle.OracleError):
        oracle.backward(q, q, q, q, None, 32, -1, False)  # negative radius
    with pytest.raises(oracle.OracleError):
        oracle.backward_blocks(q, q, q, q, [[0, 0, 2]], None, 32, 1, False)  # block 2 of 2
    with pytest.raises(TypeError):
        oracle.backward(q, q, q, q.astype(np.float64), None, 32, 1, False)
