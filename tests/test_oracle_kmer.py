"""Pins for the oracle's k-mer tokenizer (CPU only).

The tokenizer follows the NucleoByte project page, section 2 item 1 ("Fused
2-Bit Tokenization") and section 5 (6-mers, 4096 IDs plus padding and mask
entries).  What ties the oracle to something other than itself:
  * the page's own printed 6-mer IDs (tests/golden/kmer_page_ids.txt);
  * the lexicographic rank of every k-mer over A < C < G < T, enumerated with
    itertools (an independent formulation of the base-4 code);
  * the sliding-window relation between neighbouring windows, which the oracle
    never uses (it computes each window from scratch);
  * unknown bases, case, short sequences and padding, by construction.
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from block_sparse_local_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def _tok(text, k=6, n_out=None):
    if isinstance(text, str):
        text = text.encode()
    b = np.frombuffer(text, dtype=np.uint8)
    return oracle.kmer_tokenize(b, np.array([0, len(b)]), k, n_out)


def test_page_printed_ids():
    rows = []
    with open(os.path.join(HERE, "golden", "kmer_page_ids.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                kmer, ident = line.split()
                rows.append((kmer, int(ident)))
    assert len(rows) == 3
    for kmer, ident in rows:
        ids, nt = _tok(kmer)
        assert nt[0] == 1 and ids[0, 0] == ident, (kmer, ids, ident)


def test_page_vocabulary_size():
    """Section 5: 6-mers give 4096 IDs plus padding/mask entries; the usage
    example in section 6 builds the model with vocab_size 4100."""
    sp = oracle.kmer_specials(6)
    assert sp["vocab"] == 4100 and sp["pad"] == 4096 and sp["unk"] == 4098


@pytest.mark.parametrize("k", [1, 2, 3, 4, 6])
def test_lexicographic_rank(k):
    kmers = ["".join(t) for t in itertools.product("ACGT", repeat=k)]
    text = "".join(kmers)
    starts = np.arange(len(kmers) + 1, dtype=np.int64) * k
    ids, nt = oracle.kmer_tokenize(np.frombuffer(text.encode(), np.uint8), starts, k)
    assert np.all(nt == 1)
    assert np.array_equal(ids[:, 0], np.arange(4 ** k))


@pytest.mark.parametrize("k", [1, 3, 6, 12])
def test_sliding_relation_and_decode(k):
    rng = np.random.default_rng(7)
    text = rng.choice(list(b"ACGT"), 500).astype(np.uint8).tobytes()
    ids, nt = _tok(text, k)
    assert nt[0] == 500 - k + 1
    code = {ord("A"): 0, ord("C"): 1, ord("G"): 2, ord("T"): 3}
    row = ids[0].astype(np.int64)
    for t in range(nt[0] - 1):
        assert row[t + 1] == (row[t] % 4 ** (k - 1)) * 4 + code[text[t + k]]
    for t in (0, 17, nt[0] - 1):
        digits = np.base_repr(int(row[t]), 4).rjust(k, "0")
        assert "".join("ACGT"[int(c)] for c in digits) == text[t:t + k].decode()


def test_unknown_bases_case_and_padding():
    k = 6
    sp = oracle.kmer_specials(k)
    text = "ACGTACGTACGTNACGTACGTAC"   # N at position 12
    ids, nt = _tok(text, k, n_out=32)
    assert nt[0] == len(text) - k + 1
    for t in range(nt[0]):
        expect_unk = t <= 12 < t + k
        assert (ids[0, t] == sp["unk"]) == expect_unk, t
    assert np.all(ids[0, nt[0]:] == sp["pad"])
    low, _ = _tok(text.lower(), k, n_out=32)
    assert np.array_equal(low, ids)
    mixed, _ = _tok("acgtACGTacgtNacgtACGTAC", k, n_out=32)
    assert np.array_equal(mixed, ids)
    # other non-bases (IUPAC codes, RNA's U, separators) are unknown too
    for ch in "RYUX-*\n":
        w, _ = _tok("ACGTA" + ch, k)
        assert w[0, 0] == sp["unk"], ch


def test_short_sequences_counts_and_truncation():
    sp = oracle.kmer_specials(6)
    seqs = [b"", b"ACGTA", b"ACGTAC", b"ACGTACG", b"A" * 100]
    starts = np.zeros(len(seqs) + 1, dtype=np.int64)
    starts[1:] = np.cumsum([len(s) for s in seqs])
    ids, nt = oracle.kmer_tokenize(np.frombuffer(b"".join(seqs), np.uint8), starts, 6, 64)
    assert list(nt) == [0, 0, 1, 2, 64]      # 95 windows truncated to the 64-wide row
    assert np.all(ids[0] == sp["pad"]) and np.all(ids[1] == sp["pad"])
    assert ids[2, 0] == 0b00_01_10_11_00_01 and np.all(ids[2, 1:] == sp["pad"])
    assert np.all(ids[4] == 0)                # AAAAAA


def test_batch_order_and_offsets():
    """Each row depends only on its own bytes: permuting the sequences permutes
    the rows; a sequence stored at another offset gives the same row."""
    d = inputs.dna(5, 99, 12, 10, 300)
    bases, starts = d
    ids, nt = oracle.kmer_tokenize(bases, starts, 6, 320)
    perm = np.random.default_rng(1).permutation(12)
    chunks = [bases[starts[b]:starts[b + 1]] for b in perm]
    pst = np.zeros(13, dtype=np.int64)
    pst[1:] = np.cumsum([len(c) for c in chunks])
    pids, pnt = oracle.kmer_tokenize(np.concatenate(chunks), pst, 6, 320)
    assert np.array_equal(pids, ids[perm]) and np.array_equal(pnt, nt[perm])


def test_rejects_bad_arguments():
    b = np.frombuffer(b"ACGTACGT", np.uint8)
    for starts, k in ((np.array([0, 8]), 0), (np.array([0, 8]), 13), (np.array([4, 2]), 6),
                      (np.array([-1, 8]), 6)):
        with pytest.raises(oracle.OracleError):
            oracle.kmer_tokenize(b, starts, k, 8)


def test_generator_recipe():
    bases, starts = inputs.dna(42, 11, 64, 500, 2048)
    assert starts[0] == 0 and np.all(np.diff(starts) >= 500) and np.all(np.diff(starts) <= 2048)
    up = bases & 0xDF
    assert set(np.unique(up)) <= set(b"ACGTN")
    assert 0.0 < np.mean(bases == ord("N")) + np.mean(bases == ord("n")) < 0.01
    assert 0.03 < np.mean(bases >= ord("a")) < 0.2
