"""The forward and the no-alloc backward captured in one HIP graph and replayed.

bsl_forward and bsl_backward_noalloc allocate nothing and only enqueue on the
stream they are given, so a caller can capture them (here with torch's graph
capture around the C ABI calls) and replay the graph.  Every replay must give
the eager results bit for bit: the kernels are deterministic (no atomics, a
fixed reduction order).  Between replays the outputs are overwritten with NaN
by eager fill kernels and the host synchronises, so a replay that skipped or
repeated a node, or read a stale workspace, would show."""
import numpy as np
import pytest
import torch

from block_sparse_local_amd import bsl, inputs
from tests._gpu import dev, lens_dev, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


@pytest.mark.parametrize("dd,radius,causal", [(64, 1, False), (128, 2, True)])
def test_graph_forward_and_noalloc_backward(dd, radius, causal):
    batch, heads, n, lens = 2, 2, 512, np.array([500, 300], dtype=np.int32)
    say(f"[graph] b{batch} h{heads} n{n} d{dd} R{radius} causal{int(causal)} "
        f"lens {[int(x) for x in lens]}")
    q, k, v, g = inputs.draw(17 + dd, 92, batch, heads, n, dd, 1.0, True, lens, poison=True,
                             tensors=4)
    qd, kd, vd, gd = (dev(x, "bf16") for x in (q, k, v, g))
    sl = lens_dev(lens)
    plan = bsl.Plan(head_dim=dd, heads=heads, radius=radius, causal=causal)
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    outs = (o, lse, dq, dk, dv)

    def step(stream):
        bsl.bsl_forward(plan.handle, batch, n, qd, kd, vd, o, sl, lse, stream)
        bsl.bsl_backward_noalloc(plan.handle, batch, n, qd, kd, vd, o, gd, lse, sl, dq, dk, dv,
                                 stream)

    # eager reference on the current stream
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [_bits(t) for t in outs]

    # one eager run on a side stream first, as torch asks before a capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("o", "lse", "dq", "dk", "dv"), outs, ref):
            assert np.array_equal(_bits(t), r), f"replay {rep}: {name} differs from the eager run"
        say(f"  replay {rep}: o, lse, dq, dk, dv equal to the eager run bit for bit")
    del graph
    plan.close()
