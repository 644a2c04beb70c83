"""GPU parity of the backward pass: bsl_backward (through the C ABI) against the
fp64 oracle's gradients (NucleoByte project page, section 3, "Custom
Backpropagation"; oracle pinned in test_oracle_backward.py).

The GPU forward runs first and its bf16 O and lse feed the backward, as in
training.  Padded rows of Q, K, V and dO hold NaN and every output starts as
NaN, so a kernel that reads padding or skips an element fails.

Tolerance: the kernels round P and dS to bf16
(relative 2^-9) before the products and take D from the bf16 O, so each
gradient element carries a relative error of a few 2^-9 of the terms it sums.
The bar is max-abs <= 2e-2 * s and mean-abs <= 2e-3 * s, with s the root mean
square of the reference gradient over valid rows (at least 1): the forward's
bars, measured in units of the gradient's own size.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_local_amd import bsl, inputs
from tests._gpu import dev, host, lens_dev, say

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL = 2e-2, 2e-3


def _gpu_backward(d, heads, dd, radius, causal, window=0, dtype="bf16"):
    q, k, v, g = (dev(d[x], dtype) for x in ("q", "k", "v", "dout"))
    sl = lens_dev(d["seqlens"])
    plan = bsl.Plan(head_dim=dd, heads=heads, radius=radius, causal=causal, window=window,
                    dtype=dtype)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(q, k, v, sl, o=o, lse=lse)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    delta = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    plan.backward(q, k, v, o, g, lse, sl, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    out = dict(dq=host(dq), dk=host(dk), dv=host(dv), delta=delta.cpu().numpy(), o=host(o))
    plan.close()
    return out


def _compare(name, got, ref, lens, max_tol=None, mean_tol=None):
    """Valid rows within the bar, padded rows exactly zero."""
    max_tol = MAX_TOL if max_tol is None else max_tol
    mean_tol = MEAN_TOL if mean_tol is None else mean_tol
    errs, refs = [], []
    for b, L in enumerate(lens):
        L = int(L)
        assert np.all(got[b, :, L:] == 0.0), f"{name}: padded rows of sequence {b} are not zero"
        if L:
            errs.append(np.abs(got[b, :, :L].astype(np.float64) - ref[b, :, :L]).ravel())
            refs.append(ref[b, :, :L].ravel())
    if not errs:
        return
    e, r = np.concatenate(errs), np.concatenate(refs)
    assert np.all(np.isfinite(e)), f"{name}: non-finite values"
    s = max(1.0, float(np.sqrt(np.mean(r * r))))
    say(f"  {name}: max-abs {e.max():.3e} mean-abs {e.mean():.3e} (ref rms {s:.3g}, "
        f"max |ref| {np.abs(r).max():.3g})")
    assert e.max() <= max_tol * s, f"{name}: max-abs {e.max()} > {max_tol * s}"
    assert e.mean() <= mean_tol * s, f"{name}: mean-abs {e.mean()} > {mean_tol * s}"


def _case(batch, heads, n, dd, radius, causal, lens, seed, sigma=1.0):
    lens = np.array(lens, dtype=np.int32)
    q, k, v, g = inputs.draw(seed, 90, batch, heads, n, dd, sigma, True, lens, poison=True,
                             tensors=4)
    return dict(q=q, k=k, v=v, dout=g, seqlens=lens, n=n)


CASES = [
    # batch, heads, n, d, radius, causal, lens
    (2, 2, 256, 64, 1, False, [256, 150]),
    (2, 2, 256, 128, 2, True, [256, 61]),
    (2, 2, 256, 64, 0, False, [256, 33]),
    (1, 2, 96, 128, 3, False, [96]),          # radius past the last block: dense
    (3, 1, 224, 64, 1, True, [0, 1, 200]),    # empty and one-token sequences
    (2, 2, 320, 128, 1, False, [320, 289]),
    (1, 3, 512, 64, 4, True, [512]),
    (2, 2, 192, 128, 0, False, [192, 37]),    # d 128: diagonal block only, ragged
    (3, 2, 160, 128, 2, False, [0, 1, 159]),  # d 128: empty and one-token sequences
]


@pytest.mark.parametrize("case", CASES)
def test_backward_small(case):
    batch, heads, n, dd, radius, causal, lens = case
    say(f"[backward] b{batch} h{heads} n{n} d{dd} R{radius} causal{int(causal)} lens {lens}")
    d = _case(batch, heads, n, dd, radius, causal, lens, seed=len(lens) * 7 + dd + radius)
    res = _gpu_backward(d, heads, dd, radius, causal)
    dq, dk, dv = oracle.backward(d["q"], d["k"], d["v"], d["dout"], d["seqlens"], 32, radius,
                                 causal)
    _compare("dq", res["dq"], dq, d["seqlens"])
    _compare("dk", res["dk"], dk, d["seqlens"])
    _compare("dv", res["dv"], dv, d["seqlens"])
    # D = dO . O on valid rows (O the GPU's bf16 output), 0 on padded rows
    for b, L in enumerate(d["seqlens"]):
        assert np.all(res["delta"][b, :, L:] == 0.0)
        ref = np.einsum("hnd,hnd->hn", d["dout"][b, :, :L].astype(np.float64),
                        res["o"][b, :, :L].astype(np.float64))
        assert np.max(np.abs(res["delta"][b, :, :L] - ref), initial=0.0) <= 1e-3 * max(
            1.0, np.abs(ref).max(initial=0.0))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_bf16_head_dim_32(causal):
    """bf16 plans at head_dim 32 take the vector-ALU backward (fp32 arithmetic
    on the bf16 inputs, gradients rounded once to bf16)."""
    say(f"[backward] bf16 d32 causal{int(causal)}")
    d = _case(2, 2, 256, 32, 2, causal, [256, 77], seed=32 + int(causal))
    res = _gpu_backward(d, 2, 32, 2, causal)
    dq, dk, dv = oracle.backward(d["q"], d["k"], d["v"], d["dout"], d["seqlens"], 32, 2, causal)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        _compare(name, res[name], ref, d["seqlens"])


WINDOW_CASES = [
    # batch, heads, n, d, window, causal, lens
    (2, 2, 256, 64, 1, False, [256, 150]),
    (2, 2, 256, 128, 20, True, [256, 61]),
    (2, 2, 256, 64, 33, False, [256, 33]),
    (3, 1, 224, 64, 64, True, [0, 1, 200]),
    (2, 2, 320, 128, 100, False, [320, 289]),
    (1, 2, 96, 128, 96, False, [96]),          # the window covers the sequence: dense
]


@pytest.mark.parametrize("case", WINDOW_CASES)
def test_backward_token_window(case):
    """The backward of a token-window plan against the oracle's window
    backward (pinned by finite differences of the window forward)."""
    batch, heads, n, dd, window, causal, lens = case
    say(f"[backward] window {window} b{batch} h{heads} n{n} d{dd} causal{int(causal)} lens {lens}")
    d = _case(batch, heads, n, dd, 0, causal, lens, seed=window * 3 + dd)
    res = _gpu_backward(d, heads, dd, 5, causal, window=window)
    dq, dk, dv = oracle.backward(d["q"], d["k"], d["v"], d["dout"], d["seqlens"], 32, 0, causal,
                                 window=window)
    _compare("dq", res["dq"], dq, d["seqlens"])
    _compare("dk", res["dk"], dk, d["seqlens"])
    _compare("dv", res["dv"], dv, d["seqlens"])


def test_backward_token_window_full_size_sampled():
    """The long-context shape (16 heads, d 128, 131072 rows, a 120000-token
    sequence) with W = 256: sampled blocks of dQ, dK, dV against the oracle."""
    heads, n, dd, window, L = 16, 131072, 128, 256, 120000
    say(f"[backward] window {window} full size 1 x {heads} x {n} x {dd}, length {L}")
    lens = np.array([L], np.int32)
    q, k, v, g = inputs.draw(2025, 93, 1, heads, n, dd, 1.0, True, lens, poison=True, tensors=4)
    d = dict(q=q, k=k, v=v, dout=g, seqlens=lens, n=n)
    res = _gpu_backward(d, heads, dd, 0, False, window=window)
    nb = (L + 31) // 32
    rng = np.random.default_rng([2025, 93])
    blocks = sorted({0, 1, nb - 2, nb - 1} | set(int(x) for x in rng.choice(nb, 12, replace=False)))
    sel = np.array([(0, h, i) for h in range(heads) for i in blocks], np.int32)
    rq, rk, rv = oracle.backward_blocks(q, k, v, g, sel, lens, 32, 0, False, window=window)
    for name, ref in (("dq", rq), ("dk", rk), ("dv", rv)):
        got = np.stack([res[name][b, h, i * 32:(i + 1) * 32] for b, h, i in sel])
        rows = np.array([[i * 32 + r for r in range(32)] for _, _, i in sel])
        valid = rows < L
        assert np.all(got[~valid] == 0.0)
        e = np.abs(got[valid].astype(np.float64) - ref[valid])
        s = max(1.0, float(np.sqrt(np.mean(ref[valid] ** 2))))
        say(f"  {name}: max-abs {e.max():.3e} mean-abs {e.mean():.3e} (ref rms {s:.3g})")
        assert e.max() <= MAX_TOL * s and e.mean() <= MEAN_TOL * s


def test_backward_c3_reduced():
    """The causal long-context workload's shape per head (R 4, d 64, sigma 0.5)."""
    say("[backward] c3 reduced to 4 heads")
    d = inputs.make("c3", 42, poison=True, heads=4, grad=True)
    w = d["workload"]
    d = dict(q=d["q"][:1], k=d["k"][:1], v=d["v"][:1], dout=d["dout"][:1],
             seqlens=d["seqlens"][:1], n=d["n"])
    res = _gpu_backward(d, 4, w.d, w.radius, w.causal)
    dq, dk, dv = oracle.backward(d["q"], d["k"], d["v"], d["dout"], d["seqlens"], 32, w.radius,
                                 w.causal)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        _compare(name, res[name], ref, d["seqlens"])


@pytest.mark.parametrize("key", ["c4", "c5"])
def test_backward_full_size_sampled(key):
    """Full-size backward; the oracle checks sampled blocks (dQ of query block i,
    dK and dV of key block i) on every head."""
    say(f"[backward] {key} full size")
    d = inputs.make(key, 42, poison=True, grad=True)
    w = d["workload"]
    n = d["n"]
    nblk = n // 32
    L = int(d["seqlens"][0])
    nb = (L + 31) // 32
    rng = np.random.default_rng([42, w.cfg, 6])
    blocks = sorted({0, 1, nb - 2, nb - 1, nb, nblk - 1} & set(range(nblk))
                    | set(int(x) for x in rng.choice(nblk, 10, replace=False)))
    res = _gpu_backward(d, w.heads, w.d, w.radius, w.causal)
    sel = np.array([(0, h, i) for h in range(w.heads) for i in blocks], dtype=np.int32)
    bq, bk, bv = oracle.backward_blocks(d["q"], d["k"], d["v"], d["dout"], sel, d["seqlens"], 32,
                                        w.radius, w.causal)
    rows = np.array([[i * 32 + r for r in range(32)] for _, _, i in sel])
    valid = rows < L
    for name, ref in (("dq", bq), ("dk", bk), ("dv", bv)):
        got = np.stack([res[name][b, h, i * 32:(i + 1) * 32] for b, h, i in sel])
        assert np.all(got[~valid] == 0.0), f"{name}: padded rows not zero"
        e = np.abs(got[valid].astype(np.float64) - ref[valid])
        r = ref[valid]
        s = max(1.0, float(np.sqrt(np.mean(r * r))))
        say(f"  {key} {name} sampled {len(sel)} blocks: max-abs {e.max():.3e} "
            f"mean-abs {e.mean():.3e} (ref rms {s:.3g})")
        assert np.all(np.isfinite(e))
        assert e.max() <= MAX_TOL * s and e.mean() <= MEAN_TOL * s


def test_backward_rejects_bad_arguments():
    plan = bsl.Plan(head_dim=64, heads=1, radius=1)
    t = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    outs = [torch.zeros_like(t) for _ in range(3)]
    delta = torch.zeros_like(lse)
    with pytest.raises(bsl.BslError) as e:   # dq aliases q
        bsl.bsl_backward(plan.handle, 1, 64, t, t, t, t, t, lse, None, t, outs[1], outs[2], delta)
    assert e.value.status == bsl.BSL_E_INVALID
    with pytest.raises(bsl.BslError) as e:   # n not a multiple of 32
        bsl.bsl_backward(plan.handle, 1, 48, t, t, t, t, t, lse, None, *outs, delta)
    assert e.value.status == bsl.BSL_E_INVALID
    with pytest.raises(bsl.BslError) as e:   # missing workspace
        bsl.bsl_backward(plan.handle, 1, 64, t, t, t, t, t, lse, None, *outs, None)
    assert e.value.status == bsl.BSL_E_INVALID
    plan.close()
    pf = bsl.Plan(head_dim=64, heads=1, radius=1, dtype="f32")
    tf = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(bsl.BslError) as e:   # fp32 plan: dq aliases q
        bsl.bsl_backward(pf.handle, 1, 64, tf, tf, tf, tf, tf, lse, None, tf,
                         torch.zeros_like(tf), torch.zeros_like(tf), delta)
    assert e.value.status == bsl.BSL_E_INVALID
    pf.close()


# ------------------------------------------------------- packed layout backward

def _pack(x, lens, slack):
    """[batch, heads, n, d] (rows t < lens[b]) -> [tokens + slack, heads, d], NaN slack rows."""
    parts = [x[b, :, :int(L)].transpose(1, 0, 2) for b, L in enumerate(lens)]
    parts.append(np.full((slack, x.shape[1], x.shape[3]), np.nan, dtype=x.dtype))
    return np.ascontiguousarray(np.concatenate(parts, axis=0))


PACKED_CASES = [
    # heads, n, d, radius, causal, window, lens
    (2, 256, 64, 1, False, 0, [256, 0, 1, 31, 33, 150]),
    (2, 256, 128, 2, True, 0, [200, 256, 61]),
    (3, 224, 64, 0, False, 40, [224, 100, 7]),
    (2, 320, 128, 1, False, 0, [320, 289]),
]


@pytest.mark.parametrize("case", PACKED_CASES)
def test_backward_packed_layout(case):
    """bsl_backward_varlen: per sequence the same bits as bsl_backward on the
    padded layout, within the bar of the oracle, and rows outside every
    sequence (NaN slack at the end) left untouched."""
    heads, n, dd, radius, causal, window, lens = case
    say(f"[backward] packed h{heads} n{n} d{dd} R{radius} causal{int(causal)} W{window} {lens}")
    lens = np.array(lens, np.int32)
    d = _case(len(lens), heads, n, dd, radius, causal, lens, seed=dd + radius + 3 * window + 1)
    padded = _gpu_backward(d, heads, dd, radius, causal, window=window)
    slack = 5
    q, k, v, g = (dev(_pack(d[x], lens, slack), "bf16") for x in ("q", "k", "v", "dout"))
    tokens = q.shape[0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_d = lens_dev(cu)
    plan = bsl.Plan(head_dim=dd, heads=heads, radius=radius, causal=causal, window=window)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((heads, tokens), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward_varlen(q, k, v, cu_d, int(lens.max()), o=o, lse=lse)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    delta = torch.full((heads, tokens), float("nan"), dtype=torch.float32, device="cuda")
    plan.backward_varlen(q, k, v, o, g, lse, cu_d, int(lens.max()), dq=dq, dk=dk, dv=dv,
                         delta=delta)
    torch.cuda.synchronize()
    plan.close()
    got = dict(dq=host(dq), dk=host(dk), dv=host(dv))
    ref = oracle.backward(d["q"], d["k"], d["v"], d["dout"], lens, 32, radius, causal,
                          window=window if window else None)
    covered = np.zeros(tokens, bool)
    for name, r in zip(("dq", "dk", "dv"), ref):
        unpacked = np.zeros_like(padded[name])
        for b, L in enumerate(lens):
            L = int(L)
            rows = got[name][cu[b]:cu[b] + L].transpose(1, 0, 2)
            unpacked[b, :, :L] = rows
            covered[cu[b]:cu[b] + L] = True
            assert np.array_equal(rows.view(np.uint32) >> 16,
                                  padded[name][b, :, :L].view(np.uint32) >> 16), \
                f"{name}: sequence {b} differs from the padded layout"
        _compare(name, unpacked, r, lens)
        assert np.all(np.isnan(got[name][~covered])), f"{name}: rows outside the sequences written"
    dl = delta.cpu().numpy()
    assert np.all(np.isnan(dl[:, ~covered]))
    for b, L in enumerate(lens):
        L = int(L)
        assert np.array_equal(dl[:, cu[b]:cu[b] + L].view(np.uint32),
                              padded["delta"][b, :, :L].view(np.uint32))


# ------------------------------------------------------------ fp32 backward

# fp32 throughout: unit roundoff 2^-24, sums of at most (2R+1) 32 terms and
# the hardware 2^x (about 1 ulp), so errors stay near 1e-6 of the gradient's
# size (measured: max-abs 1.4e-6, mean-abs 5e-8); the bar is the fp32 forward's
# 1e-5, in units of the gradient's size.
F32_MAX, F32_MEAN = 1e-5, 1e-6

F32_CASES = [
    # heads, n, d, radius, causal, window, lens
    (2, 256, 32, 1, False, 0, [256, 150]),
    (2, 256, 64, 2, True, 0, [256, 61]),
    (1, 192, 128, 1, False, 0, [192, 0, 33]),
    (2, 224, 64, 0, False, 40, [224, 1, 100]),
    (1, 96, 32, 3, True, 0, [96]),
]


@pytest.mark.parametrize("case", F32_CASES)
def test_backward_f32(case):
    heads, n, dd, radius, causal, window, lens = case
    say(f"[backward] fp32 h{heads} n{n} d{dd} R{radius} causal{int(causal)} W{window} {lens}")
    lens_a = np.array(lens, np.int32)
    q, k, v, g = inputs.draw(dd + radius + window, 94, len(lens), heads, n, dd, 1.0, False,
                             lens_a, poison=True, tensors=4)
    d = dict(q=q, k=k, v=v, dout=g, seqlens=lens_a, n=n)
    res = _gpu_backward(d, heads, dd, radius, causal, window=window, dtype="f32")
    ref = oracle.backward(q, k, v, g, lens_a, 32, radius, causal,
                          window=window if window else None)
    for name, r in zip(("dq", "dk", "dv"), ref):
        _compare(name, res[name], r, lens_a, F32_MAX, F32_MEAN)
    for b, L in enumerate(lens_a):
        assert np.all(res["delta"][b, :, L:] == 0.0)


def test_backward_f32_packed_layout():
    heads, n, dd = 2, 160, 64
    lens = np.array([160, 0, 1, 90], np.int32)
    q, k, v, g = inputs.draw(7, 95, len(lens), heads, n, dd, 1.0, False, lens, poison=True,
                             tensors=4)
    d = dict(q=q, k=k, v=v, dout=g, seqlens=lens, n=n)
    padded = _gpu_backward(d, heads, dd, 1, False, dtype="f32")
    qp, kp, vp, gp = (dev(_pack(d[x], lens, 3), "f32") for x in ("q", "k", "v", "dout"))
    tokens = qp.shape[0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_d = lens_dev(cu)
    plan = bsl.Plan(head_dim=dd, heads=heads, radius=1, dtype="f32")
    o = torch.full_like(qp, float("nan"))
    lse = torch.full((heads, tokens), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward_varlen(qp, kp, vp, cu_d, int(lens.max()), o=o, lse=lse)
    dq, dk, dv = (torch.full_like(qp, float("nan")) for _ in range(3))
    delta = torch.full((heads, tokens), float("nan"), dtype=torch.float32, device="cuda")
    plan.backward_varlen(qp, kp, vp, o, gp, lse, cu_d, int(lens.max()), dq=dq, dk=dk, dv=dv,
                         delta=delta)
    torch.cuda.synchronize()
    plan.close()
    got = dict(dq=host(dq), dk=host(dk), dv=host(dv))
    covered = np.zeros(tokens, bool)
    for name in ("dq", "dk", "dv"):
        for b, L in enumerate(lens):
            L = int(L)
            covered[cu[b]:cu[b] + L] = True
            rows = got[name][cu[b]:cu[b] + L].transpose(1, 0, 2)
            assert np.array_equal(rows.view(np.uint32), padded[name][b, :, :L].view(np.uint32))
        assert np.all(np.isnan(got[name][~covered]))


def test_backward_packed_offsets_are_clamped():
    """Offsets out of order or past the buffer are clamped on the device, as in
    the forward: with offsets [0, 60, 40, 1000, 2000] over 100 rows the
    sequences become [0, 60), an empty one, [40, 100) and an empty one, so the
    call succeeds and every row it writes (here all 100) is finite."""
    heads, dd, tokens = 2, 64, 100
    rng = np.random.default_rng(5)
    q, k, v, g = (torch.from_numpy(inputs.bf16_bits(
        rng.standard_normal((tokens, heads, dd)).astype(np.float32)).view(np.int16))
        .view(torch.bfloat16).cuda() for _ in range(4))
    cu = lens_dev(np.array([0, 60, 40, 1000, 2000], np.int32))
    plan = bsl.Plan(head_dim=dd, heads=heads, radius=1)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((heads, tokens), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward_varlen(q, k, v, cu, 64, o=o, lse=lse)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    delta = torch.full((heads, tokens), float("nan"), dtype=torch.float32, device="cuda")
    plan.backward_varlen(q, k, v, o, g, lse, cu, 64, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    plan.close()
    for t in (dq, dk, dv):
        assert np.all(np.isfinite(host(t))), "every row lies in a clamped sequence"
    assert np.all(np.isfinite(delta.cpu().numpy()))
