"""bsl_backward_noalloc (the backward for callers that cannot allocate) through
the C ABI against bsl_backward on the same inputs: the same kernels with the
row vector D in the library's fixed workspace instead of the caller's delta,
so the gradients must be equal bit for bit.  Two calls in a row, the second
smaller than the first, so a workspace that still holds the first call's rows
cannot leak into the second; both also within the oracle's bar.  A call past
the workspace's limit is refused before any launch and writes nothing."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_local_amd import bsl, inputs
from tests._gpu import dev, host, lens_dev, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def _run_both(batch, heads, n, dd, radius, causal, lens, seed):
    lens = np.array(lens, dtype=np.int32)
    q, k, v, g = inputs.draw(seed, 91, batch, heads, n, dd, 1.0, True, lens, poison=True,
                             tensors=4)
    qd, kd, vd, gd = (dev(x, "bf16") for x in (q, k, v, g))
    sl = lens_dev(lens)
    plan = bsl.Plan(head_dim=dd, heads=heads, radius=radius, causal=causal)
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(qd, kd, vd, sl, o=o, lse=lse)
    ref = [torch.full_like(qd, float("nan")) for _ in range(3)]
    delta = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    bsl.bsl_backward(plan.handle, batch, n, qd, kd, vd, o, gd, lse, sl, *ref, delta)
    got = [torch.full_like(qd, float("nan")) for _ in range(3)]
    bsl.bsl_backward_noalloc(plan.handle, batch, n, qd, kd, vd, o, gd, lse, sl, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert np.array_equal(_bits(a), _bits(b)), f"{name} differs from bsl_backward"
    # and both against the oracle's gradients, within the backward's bar
    refs = oracle.backward(q, k, v, g, lens, 32, radius, causal)
    for name, a, r in zip(("dq", "dk", "dv"), got, refs):
        a = host(a)
        e = np.concatenate([np.abs(a[b, :, :L] - r[b, :, :L]).ravel()
                            for b, L in enumerate(lens) if L])
        s = max(1.0, float(np.sqrt(np.mean(np.concatenate(
            [r[b, :, :L].ravel() for b, L in enumerate(lens) if L]) ** 2))))
        say(f"  noalloc {name}: max-abs {e.max():.3e} mean-abs {e.mean():.3e} (ref rms {s:.3g})")
        assert np.all(np.isfinite(e)) and e.max() <= 2e-2 * s and e.mean() <= 2e-3 * s
        for b, L in enumerate(lens):
            assert np.all(a[b, :, L:] == 0.0)
    plan.close()


def test_noalloc_backward_equals_backward_twice():
    say("[noalloc] 2 x 4 heads x 1024 x d128 R2, then 1 x 2 heads x 256 x d64 R1 causal")
    _run_both(2, 4, 1024, 128, 2, False, [1000, 700], 5)
    _run_both(1, 2, 256, 64, 1, True, [200], 6)


def test_noalloc_refuses_past_its_limit():
    plan = bsl.Plan(head_dim=64, heads=8, radius=1)
    q = torch.zeros((1, 8, 32, 64), dtype=torch.bfloat16, device="cuda")
    dq = torch.full_like(q, 3.0)
    lse = torch.zeros((1, 8, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(bsl.BslError) as e:
        # 8 heads x (2^20 + 32) rows: one block past the 8 Mi-row workspace
        bsl.bsl_backward_noalloc(plan.handle, 1, (1 << 20) + 32, q, q, q, q, q, lse, None, dq,
                                 dq.clone(), dq.clone())
    assert e.value.status == bsl.BSL_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(dq == 3.0)
    plan.close()
