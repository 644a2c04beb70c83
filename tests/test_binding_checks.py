"""The Python binding's tensor checks (CPU only): every tensor a call hands to
the library must be a contiguous tensor of the right dtype and shape on q's
CUDA device.  A host tensor's address given to a kernel would fault the GPU,
and a strided lengths vector would be read as if it were dense, so both are
refused before any call reaches the library."""
import pytest
import torch

from block_sparse_local_amd import bsl

CUDA0 = torch.device("cuda", 0)


def test_require_refuses_a_tensor_on_another_device():
    for name in ("lse", "delta", "seqlens", "cu_seqlens"):
        t = torch.zeros(4, dtype=torch.float32)
        with pytest.raises(ValueError, match=f"{name} must be a tensor on cuda:0"):
            bsl.require(name, t, torch.float32, (4,), CUDA0)


def test_require_refuses_strided_wrong_dtype_or_shape():
    cpu = torch.device("cpu")
    lens = torch.arange(8, dtype=torch.int32)[::2]           # a strided view of 4 lengths
    with pytest.raises(ValueError, match="seqlens must be a contiguous"):
        bsl.require("seqlens", lens, torch.int32, (4,), cpu)
    with pytest.raises(ValueError, match="cu_seqlens must be a contiguous"):
        bsl.require("cu_seqlens", torch.zeros(5, dtype=torch.int64), torch.int32, (5,), cpu)
    with pytest.raises(ValueError, match="lse must be a contiguous"):
        bsl.require("lse", torch.zeros(2, 3), torch.float32, (3, 2), cpu)
    bsl.require("seqlens", lens.contiguous(), torch.int32, (4,), cpu)   # accepted


def test_layout_checks_refuse_host_q():
    q = torch.zeros(1, 2, 32, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q must be a CUDA tensor"):
        bsl.check_padded(q, q, q, q, None, None, torch.bfloat16)
    qp = torch.zeros(32, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q must be a CUDA tensor"):
        bsl.check_packed(qp, qp, qp, qp, torch.zeros(2, dtype=torch.int32), None, torch.bfloat16)
