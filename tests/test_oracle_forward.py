"""Pins for the oracle's attention outputs (CPU only).

No page prints an attention output, so the values are tied down by mathematics:
a dense brute force with an explicit token mask, a library routine (torch's
scaled_dot_product_attention in fp64) where the band covers everything,
closed-form special cases, invariants of softmax attention, and the page's own
running recurrence (NucleoByte page, section 3, "Softmax Normalization & Online
Numerical Stability") taken block by block.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from tests._brute import dense_reference, token_mask


def _rand(rng, batch, heads, n, d, scale=1.0):
    return [(rng.standard_normal((batch, heads, n, d)) * scale).astype(np.float32)
            for _ in range(3)]


@st.composite
def _case(draw):
    bsize = draw(st.sampled_from([1, 2, 4, 8, 16, 32]))
    nblk = draw(st.integers(1, 6 if bsize >= 16 else 10))
    n = nblk * bsize
    radius = draw(st.integers(0, 10))
    d = draw(st.sampled_from([1, 2, 3, 5, 8, 16, 32, 64]))
    batch = draw(st.integers(1, 3))
    heads = draw(st.integers(1, 2))
    causal = draw(st.booleans())
    lens = [draw(st.integers(0, n)) for _ in range(batch)]
    seed = draw(st.integers(0, 2**31 - 1))
    return bsize, n, radius, d, batch, heads, causal, np.array(lens, dtype=np.int32), seed


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_case())
def test_matches_dense_brute_force(case):
    bsize, n, radius, d, batch, heads, causal, lens, seed = case
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, batch, heads, n, d)
    o, lse, psum = oracle.forward(q, k, v, lens, bsize, radius, causal, nthreads=2)
    ro, rl = dense_reference(q, k, v, lens, bsize, radius, causal)
    assert np.max(np.abs(o - ro)) <= 1e-12
    for b in range(batch):
        L = lens[b]
        assert np.all(o[b, :, L:] == 0.0)
        assert np.all(np.isneginf(lse[b, :, L:]))
        assert np.allclose(lse[b, :, :L], rl[b, :, :L], rtol=0, atol=1e-12)
        assert np.allclose(psum[b, :, :L], 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", range(4))
def test_full_band_is_library_attention(seed, causal):
    """R >= nb - 1: every block pair is in the band, so the result is ordinary
    attention with a key-padding (and causal) mask; torch's fp64 SDPA on the CPU
    is an independent routine for that."""
    rng = np.random.default_rng([11, seed])
    batch, heads, nblk, d = 2, 3, 5, 16
    n = nblk * 32
    lens = np.array([n, int(rng.integers(1, n))], dtype=np.int32)
    q, k, v = _rand(rng, batch, heads, n, d)
    o, _, _ = oracle.forward(q, k, v, lens, 32, nblk - 1 + seed, causal)
    for b in range(batch):
        L = int(lens[b])
        qt = torch.from_numpy(q[b:b + 1, :, :L].astype(np.float64))
        kt = torch.from_numpy(k[b:b + 1, :, :L].astype(np.float64))
        vt = torch.from_numpy(v[b:b + 1, :, :L].astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
        assert np.max(np.abs(o[b, :, :L] - ref[0].numpy())) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_recurrence_equals_definition(causal):
    """The page's block-by-block running max / denominator / output, divided by the
    denominator once at the end, equals the two-pass definition."""
    rng = np.random.default_rng(5)
    n, d = 9 * 32, 24
    lens = np.array([n, 200, 33, 1], dtype=np.int32)
    q, k, v = _rand(rng, 4, 2, n, d, scale=2.0)
    for radius in (0, 1, 3):
        o, _, _ = oracle.forward(q, k, v, lens, 32, radius, causal)
        r = oracle.forward_recurrence(q, k, v, lens, 32, radius, causal)
        assert np.max(np.abs(o - r)) <= 1e-12


def test_explicit_scale():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 1, 2, 128, 8)
    o, _, _ = oracle.forward(q, k, v, None, 32, 1, False, scale=0.3)
    ro, _ = dense_reference(q, k, v, None, 32, 1, False, scale=0.3)
    assert np.max(np.abs(o - ro)) <= 1e-12
    o2, _, _ = oracle.forward(q, k, v, None, 32, 1, False)
    assert np.max(np.abs(o - o2)) > 1e-3    # the scale matters


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(7)
    q, k, _ = _rand(rng, 2, 2, 160, 16)
    v = np.full_like(q, 0.75)
    lens = np.array([160, 77], dtype=np.int32)
    o, _, _ = oracle.forward(q, k, v, lens, 32, 1, False)
    for b, L in enumerate(lens):
        assert np.max(np.abs(o[b, :, :L] - 0.75)) <= 1e-15
        assert np.all(o[b, :, L:] == 0.0)


def test_batch_permutation_is_exact():
    rng = np.random.default_rng(8)
    q, k, v = _rand(rng, 4, 2, 128, 8)
    lens = np.array([128, 5, 99, 64], dtype=np.int32)
    perm = np.array([2, 0, 3, 1])
    o, lse, _ = oracle.forward(q, k, v, lens, 32, 1, True)
    op, lp, _ = oracle.forward(q[perm], k[perm], v[perm], lens[perm], 32, 1, True)
    assert np.array_equal(op, o[perm])
    assert np.array_equal(lp, lse[perm])


def test_key_shift_and_value_affine_invariance():
    """Adding one vector u to every key adds q.u to a whole score row (softmax
    unchanged); a V + b maps O to a O + b.  The inputs are small dyadic numbers
    so that the shifted and scaled inputs are exact in float32."""
    rng = np.random.default_rng(9)
    shape = (2, 2, 128, 8)
    q = (rng.integers(-64, 64, shape) / 32).astype(np.float32)
    k = (rng.integers(-64, 64, shape) / 32).astype(np.float32)
    v = (rng.integers(-64, 64, shape) / 32).astype(np.float32)
    lens = np.array([128, 70], dtype=np.int32)
    o, _, _ = oracle.forward(q, k, v, lens, 32, 1, False)
    u = (rng.integers(-8, 8, 8) / 4).astype(np.float32)
    o_k, _, _ = oracle.forward(q, k + u, v, lens, 32, 1, False)
    o_v, _, _ = oracle.forward(q, k, 2.0 * v + 0.5, lens, 32, 1, False)
    for b, L in enumerate(lens):
        assert np.max(np.abs(o_k[b, :, :L] - o[b, :, :L])) <= 1e-12
        assert np.max(np.abs(o_v[b, :, :L] - (2.0 * o[b, :, :L] + 0.5))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_average_the_attended_values(causal):
    """Q = 0 makes every kept score 0, so each row is the plain mean of V over
    its kept keys."""
    rng = np.random.default_rng(10)
    n, d, radius = 7 * 32, 4, 2
    _, k, v = _rand(rng, 1, 1, n, d)
    q = np.zeros_like(k)
    L = 200
    o, _, _ = oracle.forward(q, k, v, np.array([L], np.int32), 32, radius, causal)
    keep = token_mask(n, L, 32, radius, causal)
    for t in range(L):
        ref = v[0, 0][keep[t]].astype(np.float64).mean(axis=0)
        assert np.max(np.abs(o[0, 0, t] - ref)) <= 1e-14


def test_single_key_rows_copy_the_value_exactly():
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 3, 2, 64, 8)
    # causal row 0 attends only to key 0
    o, _, _ = oracle.forward(q, k, v, None, 32, 1, True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0].astype(np.float64))
    # a length-1 sequence attends only to its one key
    o1, _, _ = oracle.forward(q, k, v, np.array([1, 1, 1], np.int32), 32, 1, False)
    assert np.array_equal(o1[:, :, 0], v[:, :, 0].astype(np.float64))
    assert np.all(o1[:, :, 1:] == 0.0)
    # block size 1 with radius 0: each token attends to itself only
    o2, _, _ = oracle.forward(q, k, v, None, 1, 0, False)
    assert np.array_equal(o2, v.astype(np.float64))


def test_padding_is_never_read():
    """NaN in every padded row of Q, K and V leaves the result unchanged."""
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 2, 2, 96, 8)
    lens = np.array([96, 50], dtype=np.int32)
    o, lse, _ = oracle.forward(q, k, v, lens, 32, 1, False)
    for a in (q, k, v):
        a[1, :, 50:] = np.nan
    o2, lse2, _ = oracle.forward(q, k, v, lens, 32, 1, False)
    assert np.array_equal(o, o2)
    assert np.array_equal(lse, lse2)


def test_selected_blocks_match_full_run():
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 2, 3, 8 * 32, 16)
    lens = np.array([256, 150], dtype=np.int32)
    o, lse, psum = oracle.forward(q, k, v, lens, 32, 2, False)
    sel = np.array([[0, 0, 0], [1, 2, 4], [1, 1, 7], [0, 2, 5]], dtype=np.int32)
    ob, lb, pb = oracle.forward_blocks(q, k, v, sel, lens, 32, 2, False)
    for w, (b, h, i) in enumerate(sel):
        assert np.array_equal(ob[w], o[b, h, i * 32:(i + 1) * 32])
        assert np.array_equal(lb[w], lse[b, h, i * 32:(i + 1) * 32])
        assert np.array_equal(pb[w], psum[b, h, i * 32:(i + 1) * 32])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 2, 2, 256, 16)
    a, _, _ = oracle.forward(q, k, v, None, 32, 2, True, nthreads=1)
    b, _, _ = oracle.forward(q, k, v, None, 32, 2, True, nthreads=7)
    assert np.array_equal(a, b)


def test_empty_and_bad_inputs():
    z = np.zeros((0, 1, 32, 4), np.float32)
    o, _, _ = oracle.forward(z, z, z, np.zeros(0, np.int32))
    assert o.shape == (0, 1, 32, 4)
    x = np.zeros((1, 1, 40, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.forward(x, x, x)                      # 40 is not a multiple of 32
    y = np.zeros((1, 1, 64, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.forward(y, y, y, np.array([65], np.int32))
    with pytest.raises(oracle.OracleError):
        oracle.forward_blocks(y, y, y, np.array([[0, 0, 2]]))
