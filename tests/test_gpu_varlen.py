"""GPU parity of the packed layout: bsl_forward_varlen (through the C ABI)
against the fp64 oracle and against bsl_forward on the same data.

The packed layout drops the padding between sequences (NucleoByte project page,
section 1, "Padding Waste"): sequences lie back to back in [tokens][heads][d]
arrays, located by offsets.  The operation per sequence is the padded one, so
  * the oracle (pinned in test_oracle_forward.py) is run on the same sequences
    in its own padded layout, and the packed output, unpacked, must match it
    within the usual tolerances;
  * the padded GPU path on the same data must give the same bits on every row:
    same band, same masks, same arithmetic, only the addressing differs.
A packed sequence's neighbours are the next sequence's real rows (not NaN
padding), so bit equality with the padded run also shows that nothing past a
sequence's end leaks into it.  Rows of the buffer outside every sequence start
as NaN and must come back untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_local_amd import bsl, inputs
from tests._gpu import LSE_TOL, TOL, dev, host, lens_dev, run, say

pytestmark = pytest.mark.gpu


def pack(x, lens, slack=0):
    """[batch, heads, n, d] (valid rows t < lens[b]) -> [tokens + slack, heads, d];
    the slack rows hold NaN."""
    parts = [x[b, :, :int(L)].transpose(1, 0, 2) for b, L in enumerate(lens)]
    heads, d = x.shape[1], x.shape[3]
    parts.append(np.full((slack, heads, d), np.nan, dtype=x.dtype))
    return np.ascontiguousarray(np.concatenate(parts, axis=0))


def offsets(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def unpack_rows(packed, cu, b, L):
    """Sequence b's rows of a packed [tokens, heads, d] array as [heads, L, d]."""
    return packed[cu[b]:cu[b] + L].transpose(1, 0, 2)


def run_varlen(kw, d, lens, slack=5, max_seqlen=None, cu=None):
    dtype = kw.get("dtype", "bf16")
    q, k, v = (dev(pack(d[x], lens, slack), dtype) for x in ("q", "k", "v"))
    cu = offsets(lens) if cu is None else np.asarray(cu, np.int32)
    tokens = q.shape[0]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((kw["heads"], tokens), float("nan"), dtype=torch.float32, device="cuda")
    plan = bsl.Plan(**kw)
    plan.forward_varlen(q, k, v, lens_dev(cu), int(max(lens, default=0))
                        if max_seqlen is None else max_seqlen, o=o, lse=lse)
    torch.cuda.synchronize()
    plan.close()
    return dict(o=host(o), lse=lse.cpu().numpy(), cu=cu, tokens=tokens)


def _bits(a, dtype):
    """float32 host values that came from a device tensor -> comparable bit patterns."""
    return a.view(np.uint32) >> 16 if dtype == "bf16" else a.view(np.uint32)


def _check(res, d, lens, kw, ref=None, padded=None):
    """Sequences' rows against the oracle (ref = (o, lse)) and against the
    padded GPU run bit for bit; rows outside every sequence untouched."""
    dtype = kw.get("dtype", "bf16")
    cu = res["cu"]
    mx_tol, mean_tol = TOL[dtype]
    errs = []
    for b, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        got = unpack_rows(res["o"], cu, b, L)
        g_lse = res["lse"][:, cu[b]:cu[b] + L]
        if ref is not None:
            errs.append(np.abs(got.astype(np.float64) - ref[0][b, :, :L]).ravel())
            assert np.max(np.abs(g_lse - ref[1][b, :, :L])) <= LSE_TOL[dtype]
        if padded is not None:
            assert np.array_equal(_bits(got, dtype), _bits(padded["o"][b, :, :L], dtype)), \
                f"sequence {b}: packed and padded outputs differ"
            assert np.array_equal(g_lse.view(np.uint32),
                                  padded["lse"][b, :, :L].view(np.uint32)), \
                f"sequence {b}: packed and padded lse differ"
    if errs:
        e = np.concatenate(errs)
        assert np.all(np.isfinite(e))
        say(f"  packed: max-abs {e.max():.3e} mean-abs {e.mean():.3e} over {e.size} values")
        assert e.max() <= mx_tol and e.mean() <= mean_tol
    # rows that belong to no sequence: untouched (still NaN)
    covered = np.zeros(res["tokens"], bool)
    for b, L in enumerate(lens):
        covered[cu[b]:cu[b] + int(L)] = True
    assert np.all(np.isnan(res["o"][~covered])), "rows outside every sequence were written"
    assert np.all(np.isnan(res["lse"][:, ~covered]))


SMALL = []
for _dt in ("bf16", "f32"):
    for _dd in (32, 64, 128):
        for _r, _c in ((0, False), (1, False), (3, True), (8, False)):
            SMALL.append((_dt, _dd, _r, _c))


@pytest.mark.parametrize("dtype,dd,radius,causal", SMALL)
def test_varlen_small(dtype, dd, radius, causal):
    """Ragged lengths (0, 1, 31, 32, 33 and longer ones), several tiles, slack
    rows after the last sequence."""
    lens = [300, 0, 1, 31, 32, 33, 250, 416]
    n = 416
    q, k, v = inputs.draw(dd * 10 + radius + 5, 78, len(lens), 2, n, dd, 1.0, dtype == "bf16",
                          np.array(lens, np.int32), poison=True, threads=1)
    d = dict(q=q, k=k, v=v, seqlens=np.array(lens, np.int32), n=n)
    kw = dict(head_dim=dd, heads=2, radius=radius, causal=causal, dtype=dtype)
    say(f"[varlen] small {kw}")
    res = run_varlen(kw, d, lens)
    o, lse, _ = oracle.forward(q, k, v, d["seqlens"], 32, radius, causal)
    padded = run(kw, d, with_lse=True)
    _check(res, d, lens, kw, ref=(o, lse), padded=padded)


@pytest.mark.parametrize("key", ["c2", "c3"])
def test_varlen_workload_full_oracle(key):
    """The ragged mRNA batch (its natural packed form) and the causal 8k batch,
    whole, against the oracle and the padded path."""
    say(f"[varlen] {key}")
    d = inputs.make(key, 42, poison=True)
    w = d["workload"]
    kw = dict(head_dim=w.d, heads=w.heads, radius=w.radius, causal=w.causal, dtype=w.dtype)
    lens = [int(x) for x in d["seqlens"]]
    res = run_varlen(kw, d, lens, slack=0)
    o, lse, _ = oracle.forward(d["q"], d["k"], d["v"], d["seqlens"], 32, w.radius, w.causal)
    padded = run(kw, d, with_lse=True)
    _check(res, d, lens, kw, ref=(o, lse), padded=padded)


@pytest.mark.parametrize("key", ["c4", "c5"])
def test_varlen_workload_full_size(key):
    """Full size, packed ([tokens][heads][d]) against padded, bit for bit on every
    row, on the device; the padded path is itself checked against the oracle on
    sampled blocks in test_gpu_parity.py, and here the oracle checks a few
    sampled blocks of the packed output directly."""
    say(f"[varlen] {key} full size")
    d = inputs.make(key, 42, poison=True)
    w = d["workload"]
    L = int(d["seqlens"][0])
    kw = dict(head_dim=w.d, heads=w.heads, radius=w.radius, causal=w.causal, dtype=w.dtype)
    plan = bsl.Plan(**kw)
    qp, kp, vp = (dev(d[x], "bf16") for x in ("q", "k", "v"))
    op = torch.full_like(qp, float("nan"))
    lp = torch.full(qp.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(qp, kp, vp, lens_dev(d["seqlens"]), o=op, lse=lp)
    # batch 1: the packed form is the first L rows, token-major
    qv, kv, vv = (x[0, :, :L].transpose(0, 1).contiguous() for x in (qp, kp, vp))
    slack = 3
    pad_rows = torch.full((slack, w.heads, w.d), float("nan"), dtype=qv.dtype, device="cuda")
    qv, kv, vv = (torch.cat([x, pad_rows]) for x in (qv, kv, vv))
    ov = torch.full_like(qv, float("nan"))
    lv = torch.full((w.heads, L + slack), float("nan"), dtype=torch.float32, device="cuda")
    cu = lens_dev([0, L])
    plan.forward_varlen(qv, kv, vv, cu, L, o=ov, lse=lv)
    torch.cuda.synchronize()
    same_o = torch.equal(ov[:L].transpose(0, 1).view(torch.int16),
                         op[0, :, :L].view(torch.int16))
    same_lse = torch.equal(lv[:, :L].view(torch.int32), lp[0, :, :L].view(torch.int32))
    untouched = bool(torch.isnan(ov[L:].float()).all()) and bool(torch.isnan(lv[:, L:]).all())
    say(f"  {key}: packed == padded bitwise: o {same_o}, lse {same_lse}; slack untouched "
        f"{untouched}")
    assert same_o and same_lse and untouched
    # a few sampled blocks of the packed output against the oracle
    nb = (L + 31) // 32
    blocks = sorted({0, nb // 2, nb - 1})
    sel = np.array([(0, h, i) for h in range(0, w.heads, 3) for i in blocks], dtype=np.int32)
    ob, lb, _ = oracle.forward_blocks(d["q"], d["k"], d["v"], sel, d["seqlens"], 32, w.radius,
                                      w.causal)
    ovh = ov[:L].float().cpu().numpy()
    for x, (_, h, i) in enumerate(sel):
        r1 = min(L, (i + 1) * 32)
        got = ovh[i * 32:r1, h]
        e = np.abs(got.astype(np.float64) - ob[x][:r1 - i * 32])
        assert e.max() <= 2e-2 and e.mean() <= 2e-3
    plan.close()


def test_varlen_offsets_are_clamped_and_length_bounded():
    """Offsets are clamped into [0, tokens] on the device and max_seqlen bounds
    each sequence (its first max_seqlen rows are the sequence); a decreasing
    pair is an empty sequence; rows of no sequence stay untouched.  The reference applies the same rules on the
    host, then runs the oracle."""
    dd, heads, tokens = 64, 2, 300
    rng = np.random.default_rng(12)
    x = [inputs.round_bf16(rng.standard_normal((tokens, heads, dd), dtype=np.float32))
         for _ in range(3)]
    # sequence 1 is longer than max_seqlen; 3 runs past the buffer; 4 is a
    # decreasing pair (placed last: out-of-order offsets make sequences overlap)
    cu = np.array([0, 70, 200, 290, 400, 380], dtype=np.int32)
    max_seqlen = 96
    kw = dict(head_dim=dd, heads=heads, radius=1, causal=False, dtype="bf16")
    q, k, v = (dev(a, "bf16") for a in x)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((heads, tokens), float("nan"), dtype=torch.float32, device="cuda")
    plan = bsl.Plan(**kw)
    plan.forward_varlen(q, k, v, lens_dev(cu), max_seqlen, o=o, lse=lse)
    torch.cuda.synchronize()
    plan.close()
    oh, lh = host(o), lse.cpu().numpy()
    covered = np.zeros(tokens, bool)
    for b in range(len(cu) - 1):
        s0 = min(max(int(cu[b]), 0), tokens)
        s1 = min(max(int(cu[b + 1]), s0), tokens)
        L = min(s1 - s0, max_seqlen)
        say(f"  sequence {b}: rows [{s0}, {s0 + L})")
        if L == 0:
            continue
        covered[s0:s0 + L] = True
        nbuf = -(-L // 32) * 32   # the oracle's padded buffer; its padding is never read
        seq = [np.full((1, heads, nbuf, dd), np.nan, np.float32) for _ in range(3)]
        for a, t in zip(x, seq):
            t[0, :, :L] = a[s0:s0 + L].transpose(1, 0, 2)
        ro, rl, _ = oracle.forward(*seq, np.array([L], np.int32), 32, 1, False)
        got = oh[s0:s0 + L].transpose(1, 0, 2)
        assert np.max(np.abs(got - ro[0, :, :L])) <= 2e-2
        assert np.max(np.abs(lh[:, s0:s0 + L] - rl[0, :, :L])) <= LSE_TOL["bf16"]
    assert np.all(np.isnan(oh[~covered])) and np.all(np.isnan(lh[:, ~covered]))


def test_varlen_rejects_bad_arguments():
    plan = bsl.Plan(head_dim=64, heads=2, radius=1)
    t = torch.zeros((64, 2, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(t, 7.0)
    spare = torch.zeros(64 * 2 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    cu = lens_dev([0, 64])
    h = plan.handle
    for args in [
        (1, 64, 64, t, t, t, o, None),          # no offsets
        (-1, 64, 64, t, t, t, o, cu),           # negative batch
        (1, 64, -1, t, t, t, o, cu),            # negative max_seqlen
        (1, 64, 64, t, t, t, t, cu),            # o is q
        (1, 64, 64, t, None, t, o, cu),         # NULL k
        (1, 64, 64, t, t, t, t[1:], cu),        # o overlaps q, k and v
        (1, 64, 64, t, t, t, spare.data_ptr() + 2, cu),   # o not 16-byte aligned
    ]:
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_forward_varlen(h, *args)
        assert e.value.status == bsl.BSL_E_INVALID, args[:3]
    # zero sizes are no-ops
    bsl.bsl_forward_varlen(h, 0, 64, 64, t, t, t, o, cu)
    bsl.bsl_forward_varlen(h, 1, 0, 64, t, t, t, o, cu)
    bsl.bsl_forward_varlen(h, 1, 64, 0, t, t, t, o, cu)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
    plan.close()
