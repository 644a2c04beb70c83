"""The seeded input generator (CPU only): check values, rounding, independence."""
import numpy as np
import torch

from block_sparse_local_amd import inputs


def test_check_values_seed_42():
    d = inputs.make("c1", 42)
    assert np.array_equal(d["q"][0, 0, 0, :4],
                          np.array([-0.19986728, -2.0394027, 0.80581766, 0.24691227], np.float32))
    lens, n = inputs.lengths(inputs.WORKLOADS["c2"], 42)
    assert list(lens) == [895, 538, 1299, 1817, 1987, 1386, 1722, 1236]
    assert n == 2016
    s = inputs.sample_blocks(inputs.WORKLOADS["c5"], 1048576, 42)
    assert list(s[:4]) == [176, 1180, 1243, 1407] and s[-1] == 31569 and len(set(s)) == 64
    lens4, n4 = inputs.lengths(inputs.WORKLOADS["c4"], 42)
    assert n4 == 131072 and list(lens4) == [130000]


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]      # exact ties and an exact value
    ours = inputs.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)
    bits = inputs.bf16_bits(ours)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(back, ours)


def test_slices_are_order_free_and_poison_only_padding():
    a = inputs.make("c2", 42, poison=True, heads=2)
    b = inputs.draw(42, 2, 8, 2, a["n"], 64, 1.0, True, a["seqlens"], poison=False, threads=1)
    for t, name in enumerate("qkv"):
        x = a[name]
        for bi, L in enumerate(a["seqlens"]):
            assert np.array_equal(x[bi, :, :L], b[t][bi, :, :L])
            assert np.isnan(x[bi, :, L:]).all()
    # heads drawn alone equal heads drawn with the others
    one = inputs.draw(42, 2, 8, 1, a["n"], 64, 1.0, True)
    assert np.array_equal(one[0][:, 0], b[0][:, 0])
