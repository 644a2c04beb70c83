"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its C ABI, compare with the oracle."""
import sys

import numpy as np
import torch

from block_sparse_local_amd import bsl, inputs

# Tolerances on valid output elements versus the fp64 oracle: bf16 inputs
# max-abs <= 2e-2 and mean-abs <= 2e-3; the fp32 path max-abs <= 1e-5.
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-5, 1e-5)}
LSE_TOL = {"bf16": 1e-2, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    """float32 numpy holding exact input values -> contiguous CUDA tensor."""
    if dtype == "bf16":
        bits = inputs.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t):
    return t.float().cpu().numpy()


def lens_dev(lens):
    return torch.from_numpy(np.ascontiguousarray(lens, dtype=np.int32)).cuda()


def check_rows(o_gpu, o_ref, lens, dtype, what=""):
    """o_gpu float32 [b,h,n,d] (host), o_ref float64 same shape or None for
    padded-rows-only.  Valid rows within tolerance, padded rows exactly 0."""
    mx_tol, mean_tol = TOL[dtype]
    errs = []
    for b, L in enumerate(lens):
        L = int(L)
        pad = o_gpu[b, :, L:]
        assert np.all(pad == 0.0), f"{what}: padded rows of sequence {b} are not zero"
        if o_ref is not None and L > 0:
            errs.append(np.abs(o_gpu[b, :, :L].astype(np.float64) - o_ref[b, :, :L]).ravel())
    if errs:
        e = np.concatenate(errs)
        assert np.all(np.isfinite(e)), f"{what}: non-finite output"
        say(f"  {what}: max-abs {e.max():.3e} mean-abs {e.mean():.3e} over {e.size} values")
        assert e.max() <= mx_tol, f"{what}: max-abs {e.max()} > {mx_tol}"
        assert e.mean() <= mean_tol, f"{what}: mean-abs {e.mean()} > {mean_tol}"
        return float(e.max()), float(e.mean())
    return 0.0, 0.0


def run(plan_kw, d, traced=False, with_lse=False, o_fill=None):
    """Run the library on inputs dict ``d`` (from inputs.make or hand-built).
    Returns dict(o=float32 host, lse=..., active=..., masks=...)."""
    dtype = plan_kw.get("dtype", "bf16")
    q, k, v = dev(d["q"], dtype), dev(d["k"], dtype), dev(d["v"], dtype)
    sl = lens_dev(d["seqlens"])
    o = torch.empty_like(q)
    o.fill_(o_fill if o_fill is not None else float("nan"))
    lse = None
    if with_lse:
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    plan = bsl.Plan(**plan_kw)
    out = {}
    if traced:
        o, act, msk = plan.forward_traced(q, k, v, sl, o=o, lse=lse)
        torch.cuda.synchronize()
        out["active"] = act.cpu().numpy()
        out["masks"] = msk.cpu().numpy().view(np.uint32)
    else:
        plan.forward(q, k, v, sl, o=o, lse=lse)
        torch.cuda.synchronize()
    out["o"] = host(o)
    if with_lse:
        out["lse"] = lse.cpu().numpy()
    plan.close()
    return out
