"""GPU parity: libbsl.so (through its C ABI) against the fp64 oracle.

Every input is seeded and synthetic (block_sparse_local_amd.inputs).  Padded
rows of Q, K and V hold NaN in these runs and O starts as NaN, so a kernel that
reads padding or skips a row fails.  Active-block lists and masks recorded by
the kernel itself must equal the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_local_amd import bsl, inputs
from tests._gpu import LSE_TOL, check_rows, dev, lens_dev, run, say

pytestmark = pytest.mark.gpu


def _plan_kw(w, dtype=None):
    return dict(head_dim=w.d, heads=w.heads, radius=w.radius, causal=w.causal,
                dtype=dtype or w.dtype)


def _check_trace(res, w, d):
    act = oracle.active_blocks(w.batch, d["n"], 32, w.radius, w.causal, d["seqlens"])
    msk = oracle.masks(w.batch, d["n"], 32, w.radius, w.causal, d["seqlens"], act)
    assert np.array_equal(res["active"], act), "active-block lists differ from the oracle"
    assert np.array_equal(res["masks"], msk), "masks differ from the oracle"
    say(f"  trace: {int((act >= 0).sum())} block pairs, lists and masks bit-exact")


def _check_lse(got, want, lens, dtype):
    for b, L in enumerate(lens):
        assert np.all(np.isneginf(got[b, :, L:]))
        if L:
            assert np.max(np.abs(got[b, :, :L] - want[b, :, :L])) <= LSE_TOL[dtype]


def _check_all_launches(plan_kw, d, what, radius, causal, dtype, window=None):
    """The three launches a caller can make, each against the oracle element
    by element: the benchmark's own (untraced, no lse), untraced with lse (what
    a training step runs before its backward) and traced with lse (whose visited
    blocks and masks must also equal the oracle's bit for bit).  The traced
    instantiation drains its K/V ring on every step, so it does not stand in for
    the pipelined one."""
    lens = d["seqlens"]
    o, lse, _ = oracle.forward(d["q"], d["k"], d["v"], lens, 32, radius, causal, window=window)
    bench = run(plan_kw, d)
    check_rows(bench["o"], o, lens, dtype, f"{what} (untraced, no lse)")
    plain = run(plan_kw, d, with_lse=True)
    check_rows(plain["o"], o, lens, dtype, f"{what} (untraced, lse)")
    _check_lse(plain["lse"], lse, lens, dtype)
    # with or without lse the untraced kernel computes O the same way
    assert np.array_equal(bench["o"], plain["o"])
    traced = run(plan_kw, d, traced=True, with_lse=True)
    check_rows(traced["o"], o, lens, dtype, f"{what} (traced, lse)")
    _check_lse(traced["lse"], lse, lens, dtype)
    return traced


@pytest.mark.parametrize("key", ["c1", "c2", "c3"])
def test_workload_full_oracle(key):
    say(f"[parity] {key}")
    d = inputs.make(key, 42, poison=True)
    w = d["workload"]
    res = _check_all_launches(_plan_kw(w), d, key, w.radius, w.causal, w.dtype)
    _check_trace(res, w, d)


@pytest.mark.parametrize("seed", [43, 44, 45, 46])
@pytest.mark.parametrize("key", ["c1", "c2", "c3"])
def test_workload_seed_sweep(key, seed):
    """The correctness sweep over further seeds (new values and, for the mRNA
    batch, new ragged lengths), whole outputs against the oracle and the
    trace bit-exact."""
    say(f"[parity] {key} seed {seed}")
    d = inputs.make(key, seed, poison=True)
    w = d["workload"]
    res = _check_all_launches(_plan_kw(w), d, f"{key} seed {seed}", w.radius, w.causal, w.dtype)
    _check_trace(res, w, d)


def _sample_c4(nblk, nb, rng):
    pick = {0, 1, 2, nb - 3, nb - 2, nb - 1, nb, nblk - 1}
    pick |= set(int(x) for x in rng.choice(nblk, 56, replace=False))
    return sorted(pick)


@pytest.mark.parametrize("key", ["c4", "c5"])
def test_workload_full_size(key):
    """Full-size run in the benchmark's launch configuration (untraced, no lse),
    every valid output element of every head against the oracle (head by head on
    the host); then the traced launch with lse on sampled query blocks of every
    head, and its visited blocks and masks everywhere.  The million-token
    workload asks only for its 64 seeded query blocks: those are among the
    sampled ones, and the whole output is checked as well."""
    say(f"[parity] {key} full size")
    d = inputs.make(key, 42, poison=True)
    w = d["workload"]
    n = d["n"]
    nblk = n // 32
    L = int(d["seqlens"][0])
    plain = run(_plan_kw(w), d)
    check_rows(plain["o"], None, d["seqlens"], "bf16", key)   # every padded row is zero
    worst, total, count = 0.0, 0.0, 0
    for h in range(w.heads):
        sl = lambda x: np.ascontiguousarray(x[:, h:h + 1])
        ref, _, _ = oracle.forward(sl(d["q"]), sl(d["k"]), sl(d["v"]), d["seqlens"], 32,
                                   w.radius, w.causal)
        e = np.abs(plain["o"][0, h, :L].astype(np.float64) - ref[0, 0, :L])
        assert np.all(np.isfinite(e)), f"{key} head {h}: non-finite output"
        worst = max(worst, float(e.max()))
        total += float(e.sum())
        count += e.size
        say(f"  {key} head {h}: max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
        del ref, e
    say(f"  {key} bench launch, all {w.heads * ((L + 31) // 32)} block-heads: max-abs "
        f"{worst:.3e} mean-abs {total / count:.3e} over {count} values")
    assert worst <= 2e-2 and total / count <= 2e-3
    del plain

    if key == "c5":
        blocks = [int(x) for x in inputs.sample_blocks(w, n, 42)]
    else:
        nb = (L + 31) // 32
        blocks = _sample_c4(nblk, nb, np.random.default_rng([42, 4, 5]))
    sel = np.array([(0, h, i) for h in range(w.heads) for i in blocks], dtype=np.int32)
    ob, lb, _ = oracle.forward_blocks(d["q"], d["k"], d["v"], sel, d["seqlens"], 32, w.radius,
                                      w.causal)
    rows = np.array([i * 32 + r for _, _, i in sel for r in range(32)]).reshape(len(sel), 32)
    valid = rows < L
    res = run(_plan_kw(w), d, traced=True, with_lse=True)
    got = np.stack([res["o"][b, h, i * 32:(i + 1) * 32] for b, h, i in sel])
    assert np.all(got[~valid] == 0.0)
    e = np.abs(got[valid].astype(np.float64) - ob[valid])
    say(f"  {key} traced, sampled {len(sel)} blocks: max-abs {e.max():.3e} "
        f"mean-abs {e.mean():.3e}")
    assert e.max() <= 2e-2 and e.mean() <= 2e-3
    gl = np.stack([res["lse"][b, h, i * 32:(i + 1) * 32] for b, h, i in sel])
    assert np.all(np.isneginf(gl[~valid]))
    assert np.max(np.abs(gl[valid] - lb[valid])) <= LSE_TOL["bf16"]
    check_rows(res["o"], None, d["seqlens"], "bf16", key)   # every padded row is zero
    _check_trace(res, w, d)


def _rand_case(seed, dtype, dd, radius, causal, nblk, lens, heads=2):
    n = nblk * 32
    batch = len(lens)
    q, k, v = inputs.draw(seed, 77, batch, heads, n, dd, 1.0, dtype == "bf16",
                          np.array(lens, np.int32), poison=True, threads=1)
    return dict(q=q, k=k, v=v, seqlens=np.array(lens, np.int32), n=n)


SMALL = []
for _dt in ("bf16", "f32"):
    for _dd in (32, 64, 128):
        for _r, _c in ((0, False), (1, False), (2, False), (3, True), (8, False), (2, True)):
            SMALL.append((_dt, _dd, _r, _c))


@pytest.mark.parametrize("dtype,dd,radius,causal", SMALL)
def test_small_shapes_ragged(dtype, dd, radius, causal):
    """Several tiles, ragged tails (0, 1, 31, 32, 33 and a full buffer), a block
    count that is not a multiple of the workgroup's 4 query blocks."""
    nblk = 13
    lens = [nblk * 32, 0, 1, 31, 32, 33, 250, 385]
    d = _rand_case(dd * 10 + radius, dtype, dd, radius, causal, nblk, lens)
    kw = dict(head_dim=dd, heads=2, radius=radius, causal=causal, dtype=dtype)
    say(f"[parity] small {kw}")
    res = _check_all_launches(kw, d, f"small {dtype} d{dd} R{radius} c{int(causal)}", radius,
                              causal, dtype)
    act = oracle.active_blocks(len(lens), d["n"], 32, radius, causal, d["seqlens"])
    msk = oracle.masks(len(lens), d["n"], 32, radius, causal, d["seqlens"], act)
    assert np.array_equal(res["active"], act)
    assert np.array_equal(res["masks"], msk)


def test_page_usage_shape():
    """The shape the NucleoByte page's usage example runs (section 6): batch 2,
    2 heads, 4096 tokens, head dim 64 (embed 128 over 2 heads), radius 1."""
    say("[parity] usage shape 2x2x4096x64 R1")
    q, k, v = inputs.draw(42, 6, 2, 2, 4096, 64)
    d = dict(q=q, k=k, v=v, seqlens=np.array([4096, 4096], np.int32), n=4096)
    res = run(dict(head_dim=64, heads=2, radius=1), d)
    o, _, _ = oracle.forward(q, k, v, d["seqlens"], 32, 1, False)
    check_rows(res["o"], o, d["seqlens"], "bf16", "usage shape")


def test_scale_override():
    q, k, v = inputs.draw(3, 8, 1, 2, 256, 64)
    d = dict(q=q, k=k, v=v, seqlens=np.array([200], np.int32), n=256)
    res = run(dict(head_dim=64, heads=2, radius=2, scale=0.05), d)
    o, _, _ = oracle.forward(q, k, v, d["seqlens"], 32, 2, False, scale=0.05)
    check_rows(res["o"], o, d["seqlens"], "bf16", "scale 0.05")


# ----------------------------------------------------------------- invariants

def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def test_poison_sentinel_determinism_and_permutation():
    say("[invariants] poison / sentinel / repeat / permutation")
    lens = np.array([300, 1000, 17, 640], np.int32)
    n = 1024
    clean = inputs.draw(5, 9, 4, 3, n, 64, 1.0, True, lens, poison=False)
    dirty = inputs.draw(5, 9, 4, 3, n, 64, 1.0, True, lens, poison=True)
    plan = bsl.Plan(64, 3, 2, False)
    sl = lens_dev(lens)
    outs = []
    for src, fill in ((clean, 0.0), (dirty, 12345.0), (dirty, float("nan"))):
        q, k, v = (dev(x, "bf16") for x in src)
        o = torch.full_like(q, fill)
        plan.forward(q, k, v, sl, o=o)
        outs.append(_bits(o))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    perm = np.array([2, 0, 3, 1])
    q, k, v = (dev(x[perm], "bf16") for x in dirty)
    o = torch.empty_like(q)
    plan.forward(q, k, v, lens_dev(lens[perm]), o=o)
    assert np.array_equal(_bits(o), outs[0][perm])
    plan.close()


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_exact(causal):
    """V = 0.75 everywhere: the probabilities sum to one, so O is 0.75 exactly
    after bf16 rounding."""
    lens = np.array([512, 77], np.int32)
    q, k, _ = inputs.draw(6, 10, 2, 2, 512, 128, 1.0, True, lens, poison=True)
    v = np.full_like(q, 0.75)
    d = dict(q=q, k=k, v=v, seqlens=lens, n=512)
    res = run(dict(head_dim=128, heads=2, radius=3, causal=causal), d)
    for b, L in enumerate(lens):
        assert np.all(res["o"][b, :, :L] == 0.75)
        assert np.all(res["o"][b, :, L:] == 0.0)


def test_single_key_rows_exact():
    """Causal row 0 and a length-1 sequence attend to one key: O = V there."""
    lens = np.array([1, 256], np.int32)
    q, k, v = inputs.draw(7, 11, 2, 2, 256, 64, 1.0, True, lens, poison=True)
    d = dict(q=q, k=k, v=v, seqlens=lens, n=256)
    res = run(dict(head_dim=64, heads=2, radius=1, causal=True), d)
    assert np.array_equal(res["o"][:, :, 0], v[:, :, 0])
    assert np.all(res["o"][0, :, 1:] == 0.0)


def test_errors_write_nothing():
    plan = bsl.Plan(64, 1, 1, False)
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    with pytest.raises(bsl.BslError) as e:          # n not a multiple of 32
        bsl.bsl_forward(plan.handle, 1, 40, q, q, q, o)
    assert e.value.status == bsl.BSL_E_INVALID
    with pytest.raises(bsl.BslError) as e:          # misaligned pointer
        bsl.bsl_forward(plan.handle, 1, 32, q.data_ptr() + 2, q, q, o)
    assert e.value.status == bsl.BSL_E_INVALID
    with pytest.raises(bsl.BslError) as e:          # trace buffers missing
        bsl.bsl_forward_traced(plan.handle, 1, 64, q, q, q, o, None, None, None, None)
    assert e.value.status == bsl.BSL_E_INVALID
    with pytest.raises(bsl.BslError) as e:          # output overlapping an input
        bsl.bsl_forward(plan.handle, 1, 64, q, q, q, q)
    assert e.value.status == bsl.BSL_E_INVALID
    bsl.bsl_forward(plan.handle, 0, 64, q, q, q, o)  # empty batch: no-op
    bsl.bsl_forward(plan.handle, 1, 0, q, q, q, o)   # empty buffer: no-op
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
    plan.close()


def test_large_tensors_64bit_offsets():
    """2^31 elements per tensor (batch 1, 16 heads, 2^20 rows, head dim 128: 4 GiB
    each in bf16), so row offsets past 2^31 bytes are exercised.  Inputs are
    seeded normal draws made on the device (torch's generator); sampled query
    blocks, the last ones of the last head among them, are checked against the
    oracle on the slice of rows their band covers (the band of a query block
    lies inside its own 2R + 1 blocks, so the slice gives the same keys)."""
    heads, n, dd, R = 16, 1 << 20, 128, 8
    say(f"[parity] large tensors 1 x {heads} x {n} x {dd} R{R}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    shape = (1, heads, n, dd)
    q, k, v = (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
               .to(torch.bfloat16) for _ in range(3))
    o = torch.full_like(q, float("nan"))
    plan = bsl.Plan(head_dim=dd, heads=heads, radius=R, causal=False)
    plan.forward(q, k, v, None, o=o)
    torch.cuda.synchronize()
    nblk = n // 32
    picks = [(heads - 1, nblk - 1), (heads - 1, nblk - 2), (heads - 1, nblk - 9),
             (heads - 1, 20000), (12, nblk - 1), (0, 0), (7, 5)]
    worst = 0.0
    for h, i in picks:
        lo = max(0, i - R)
        hi = min(nblk, i + R + 1)
        rows = slice(lo * 32, hi * 32)
        sub = [t[:, h:h + 1, rows].float().cpu().numpy() for t in (q, k, v)]
        ln = np.array([(hi - lo) * 32], dtype=np.int32)
        ref, _, _ = oracle.forward(sub[0], sub[1], sub[2], ln, 32, R, False)
        r0 = (i - lo) * 32
        want = ref[0, 0, r0:r0 + 32]
        got = o[0, h, i * 32:(i + 1) * 32].float().cpu().numpy()
        e = np.abs(got.astype(np.float64) - want)
        worst = max(worst, float(e.max()))
        assert np.all(np.isfinite(got)) and e.max() <= 2e-2 and e.mean() <= 2e-3, (h, i, e.max())
    say(f"  {len(picks)} sampled blocks: max-abs {worst:.3e}")
    plan.close()
    del q, k, v, o
    torch.cuda.empty_cache()


def test_binding_refuses_host_or_strided_side_tensors():
    """lse, delta, seqlens and cu_seqlens must live on q's GPU (a host address
    handed to a kernel would fault it) and be contiguous; the binding raises
    before anything is launched, and O is left untouched."""
    plan = bsl.Plan(64, 2, 1, False)
    q = torch.zeros((2, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    lens = torch.tensor([64, 40], dtype=torch.int32)
    with pytest.raises(ValueError, match="seqlens"):
        plan.forward(q, q, q, lens, o=o)                                   # host lengths
    with pytest.raises(ValueError, match="seqlens"):
        plan.forward(q, q, q, torch.tensor([64, 0, 40, 0], dtype=torch.int32,
                                           device="cuda")[::2], o=o)       # strided
    with pytest.raises(ValueError, match="lse"):
        plan.forward(q, q, q, None, o=o, lse=torch.zeros((2, 2, 64)))     # host lse
    lse = torch.zeros((2, 2, 64), device="cuda")
    with pytest.raises(ValueError, match="delta"):
        plan.backward(q, q, q, o, q, lse, None, delta=torch.zeros((2, 2, 64)))
    qp = torch.zeros((100, 2, 64), dtype=torch.bfloat16, device="cuda")
    op = torch.full_like(qp, 3.0)
    with pytest.raises(ValueError, match="cu_seqlens"):
        plan.forward_varlen(qp, qp, qp, torch.tensor([0, 60, 100], dtype=torch.int32), 60, o=op)
    with pytest.raises(ValueError, match="lse"):
        plan.forward_varlen(qp, qp, qp, torch.tensor([0, 60, 100], dtype=torch.int32,
                                                     device="cuda"), 60, o=op,
                            lse=torch.zeros((2, 100)))
    torch.cuda.synchronize()
    assert torch.all(o == 3.0) and torch.all(op == 3.0)
    plan.close()
