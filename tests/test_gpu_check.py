"""GPU tests of the length and offset validators (bsl_check_seqlens,
bsl_check_cu_seqlens) against their definitions written out in numpy: a
length is valid in [0, n]; offsets start at 0, never decrease and stay within
tokens.  The result buffer starts as garbage and must be written in full."""
import numpy as np
import pytest
import torch

from block_sparse_local_amd import bsl
from tests._gpu import say

pytestmark = pytest.mark.gpu


def _expect_lengths(x, n):
    bad = np.flatnonzero((x < 0) | (x > n))
    return len(bad), int(bad[0]) if len(bad) else -1


def _expect_offsets(cu, tokens):
    wrong = np.zeros(len(cu), bool)
    wrong[0] = cu[0] != 0
    wrong[1:] = (cu[1:] < cu[:-1]) | (cu[1:] > tokens)
    bad = np.flatnonzero(wrong)
    return len(bad), int(bad[0]) if len(bad) else -1


def _run(fn, batch, limit, arr):
    dev_arr = torch.from_numpy(np.ascontiguousarray(arr, np.int32)).cuda() if arr is not None else None
    res = torch.full((2,), 12345, dtype=torch.int32, device="cuda")
    fn(batch, limit, dev_arr, res)
    torch.cuda.synchronize()
    return tuple(res.cpu().tolist())


@pytest.mark.parametrize("batch", [1, 7, 256, 257, 100000])
def test_check_seqlens_matches_definition(batch):
    rng = np.random.default_rng(batch)
    n = 4096
    x = rng.integers(0, n + 1, size=batch).astype(np.int32)
    say(f"[check] seqlens batch {batch}")
    assert _run(bsl.bsl_check_seqlens, batch, n, x) == (0, -1)
    # plant bad values: negative, one past n, and the extremes
    k = min(batch, 5)
    pos = rng.choice(batch, k, replace=False)
    vals = np.array([-1, n + 1, np.iinfo(np.int32).min, np.iinfo(np.int32).max, -7])[:k]
    x[pos] = vals
    assert _run(bsl.bsl_check_seqlens, batch, n, x) == _expect_lengths(x, n)
    # boundary values are valid
    x[:] = 0
    x[-1] = n
    assert _run(bsl.bsl_check_seqlens, batch, n, x) == (0, -1)


def test_check_seqlens_empty_batch():
    assert _run(bsl.bsl_check_seqlens, 0, 32, None) == (0, -1)


@pytest.mark.parametrize("batch", [1, 8, 300, 65536])
def test_check_cu_seqlens_matches_definition(batch):
    rng = np.random.default_rng(batch + 1)
    lens = rng.integers(0, 2049, size=batch)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    tokens = int(cu[-1]) + 3
    cu = cu.astype(np.int32)
    say(f"[check] cu_seqlens batch {batch}")
    assert _run(bsl.bsl_check_cu_seqlens, batch, tokens, cu) == (0, -1)
    for case in range(4):
        c = cu.copy()
        if case == 0:
            c[0] = 5                           # does not start at 0
        elif case == 1 and batch > 1:
            c[batch // 2 + 1] = c[batch // 2] - 1  # a decreasing pair
        elif case == 2:
            c[-1] = tokens + 1                 # past the buffer
        else:
            c[1:] = c[1:][::-1].copy()         # reversed: decreasing almost everywhere
        assert _run(bsl.bsl_check_cu_seqlens, batch, tokens, c) == _expect_offsets(c, tokens)


def test_check_cu_seqlens_empty_batch():
    assert _run(bsl.bsl_check_cu_seqlens, 0, 10, np.zeros(1, np.int32)) == (0, -1)
    assert _run(bsl.bsl_check_cu_seqlens, 0, 10, np.ones(1, np.int32)) == (1, 0)


def test_convenience_wrappers():
    x = torch.tensor([3, 40, -2, 32], dtype=torch.int32, device="cuda")
    assert bsl.check_seqlens(x, 32) == (2, 1)
    cu = torch.tensor([0, 10, 9, 30], dtype=torch.int32, device="cuda")
    assert bsl.check_cu_seqlens(cu, 25) == (2, 2)
