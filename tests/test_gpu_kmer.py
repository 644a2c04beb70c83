"""GPU parity of the fused k-mer tokenizer (bsl_kmer_tokenize, through the C
ABI) against the oracle, bit for bit: IDs, UNK and PAD entries, window counts.

Inputs are seeded synthetic nucleotide text (block_sparse_local_amd.inputs.dna:
uniform bases, about one 'N' per thousand, soft-masked lowercase runs), plus
hand-made edge cases.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_local_amd import bsl, inputs
from tests._gpu import say

pytestmark = pytest.mark.gpu


def _run(bases, starts, k, n_out, base_offset=0, ids_offset=0):
    """Device run; ``base_offset`` / ``ids_offset`` place the text / the output
    that many elements into a larger allocation (unaligned pointers)."""
    bd_full = torch.zeros(len(bases) + base_offset + 64, dtype=torch.uint8, device="cuda")
    bd = bd_full[base_offset:base_offset + len(bases)]
    if len(bases):
        bd.copy_(torch.from_numpy(np.ascontiguousarray(bases)))
    sd = torch.from_numpy(np.ascontiguousarray(starts, dtype=np.int64)).cuda()
    batch = len(starts) - 1
    ids_full = torch.full((batch * n_out + ids_offset + 8,), -5, dtype=torch.int32, device="cuda")
    ids = ids_full[ids_offset:ids_offset + batch * n_out].view(batch, n_out)
    ntok = torch.full((batch,), -5, dtype=torch.int32, device="cuda")
    bsl.kmer_tokenize(bd, sd, k, n_out, ids=ids, ntok=ntok)
    torch.cuda.synchronize()
    tail = ids_full[ids_offset + batch * n_out:].cpu().numpy()
    assert np.all(tail == -5), "wrote past the output row block"
    if ids_offset:
        assert np.all(ids_full[:ids_offset].cpu().numpy() == -5), "wrote before the output"
    return ids.cpu().numpy(), ntok.cpu().numpy()


def _compare(bases, starts, k, n_out, what, **kw):
    got, gnt = _run(bases, starts, k, n_out, **kw)
    ref, rnt = oracle.kmer_tokenize(bases, starts, k, n_out)
    assert np.array_equal(gnt, rnt), f"{what}: window counts differ"
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} IDs differ, first at {bad[0]}"
    say(f"  {what}: {int(rnt.sum())} windows bit-exact")


@pytest.mark.parametrize("k", [1, 2, 5, 6, 7, 12])
def test_random_batches(k):
    say(f"[kmer] random k={k}")
    bases, starts = inputs.dna(42, 70 + k, 37, 0, 5000)
    n_out = bsl.bsl_kmer_ceiling(starts, k)
    _compare(bases, starts, k, n_out, f"k={k} n_out={n_out}")


def test_edges_lengths_alignment_truncation():
    say("[kmer] edges")
    seqs = [b"", b"A", b"ACGTA", b"ACGTAC", b"acgtacg", b"NNNNNNNNNN", b"ACGTNACGTACGTACGTACGTT",
            b"T" * 2047, b"G" * 2048, b"C" * 2053, b"ACGT" * 1200 + b"n" + b"acgt" * 300]
    bases = np.frombuffer(b"".join(seqs), dtype=np.uint8)
    starts = np.zeros(len(seqs) + 1, dtype=np.int64)
    starts[1:] = np.cumsum([len(s) for s in seqs])
    for n_out in (0, 1, 7, 33, 2048, 2049, 6400):
        for bo, io in ((0, 0), (3, 0), (0, 1), (13, 5)):
            _compare(bases, starts, 6, n_out, f"n_out={n_out} text+{bo} ids+{io}",
                     base_offset=bo, ids_offset=io)


def test_offsets_are_clamped():
    """Offsets outside the buffer or decreasing: clamped on the device, never an
    access outside the text."""
    say("[kmer] clamped offsets")
    bases, _ = inputs.dna(1, 80, 1, 3000, 3000)
    raw = np.array([-50, 100, 90, 1500, 2990, 2999, 10 ** 9], dtype=np.int64)
    got, gnt = _run(bases, raw, 6, 1600)
    n = len(bases)
    for b in range(len(raw) - 1):
        s0 = min(max(raw[b], 0), n)
        s1 = min(max(raw[b + 1], s0), n)
        ref, rnt = oracle.kmer_tokenize(bases[s0:s1], np.array([0, s1 - s0]), 6, 1600)
        assert gnt[b] == rnt[0] and np.array_equal(got[b], ref[0]), b


def test_counts_only_and_errors():
    bases = torch.from_numpy(np.frombuffer(b"ACGTACGTAC", np.uint8).copy()).cuda()
    starts = torch.tensor([0, 4, 10], dtype=torch.int64, device="cuda")
    ids = torch.empty((2, 0), dtype=torch.int32, device="cuda")
    ntok = torch.full((2,), -5, dtype=torch.int32, device="cuda")
    bsl.kmer_tokenize(bases, starts, 6, 0, ids=ids, ntok=ntok)
    torch.cuda.synchronize()
    assert ntok.cpu().tolist() == [0, 0]
    ids = torch.full((2, 8), -5, dtype=torch.int32, device="cuda")
    for k in (0, 13):
        with pytest.raises(bsl.BslError):
            bsl.kmer_tokenize(bases, starts, k, 8, ids=ids)
    with pytest.raises(bsl.BslError):   # output overlapping the offsets
        bsl.bsl_kmer_tokenize(2, bases, 10, starts.data_ptr(), 6, 8, starts.data_ptr() + 8)
    torch.cuda.synchronize()
    assert np.all(ids.cpu().numpy() == -5), "a rejected call wrote"


@pytest.mark.parametrize("key", ["k1", "k2"])
def test_workload_full(key):
    """The benchmark's workloads in its launch configuration, every window
    compared."""
    say(f"[kmer] workload {key}")
    d = inputs.make_dna(key, 42)
    _compare(d["bases"], d["starts"], d["workload"].k, d["n_out"], key)
