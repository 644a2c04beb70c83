"""Are the oracle's pins strong enough?  (CPU only.)

Each case below copies oracle/orc.c into a temporary directory, plants one
plausible mistake (a dropped term, a wrong sign or bound, a swapped operand),
compiles it and runs a small battery of the same pins the other oracle tests
use.  Every mutant must fail at least one pin; the unmodified source must pass
them all.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from tests._brute import dense_reference, token_mask

MUTANTS = {
    "drop_scale": ("const double sc = p->scale * dot;", "const double sc = dot;"),
    "exp_sign": ("const double w = exp(sbuf[e] - m);", "const double w = exp(m - sbuf[e]);"),
    "band_off_by_one": ("if (abs(t / bsize - s / bsize) > radius)",
                        "if (abs(t / bsize - s / bsize) >= radius)"),
    "causal_strict": ("if (causal && s > t)\n        return 0;\n    return 1;",
                      "if (causal && s >= t)\n        return 0;\n    return 1;"),
    "key_length": ("if (t < 0 || t >= len || s < 0 || s >= len)",
                   "if (t < 0 || t >= len || s < 0 || s > len)"),
    "values_from_keys": ("const float *vs = p->v + (base + sidx[e]) * d;",
                         "const float *vs = p->k + (base + sidx[e]) * d;"),
    "query_from_key": ("const float *qt = p->q + (base + t) * d;",
                       "const float *qt = p->k + (base + t) * d;"),
    "no_normalise": ("        o_row[c] /= l;\n", "        o_row[c] /= 1.0;\n"),
    "lse_drops_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "floor_blocks": ("return (len + bsize - 1) / bsize;", "return len / bsize;"),
    "causal_blocks": ("if (causal && j > i)", "if (causal && j >= i)"),
    "list_drops_last": ("j <= i + radius; ++j)\n                if (block_in_band",
                        "j < i + radius; ++j)\n                if (block_in_band"),
    "recurrence_no_correction": ("acc[e] *= corr;", "acc[e] *= 1.0;"),
    "recurrence_den": ("den = den * corr + add;", "den = den + add;"),
    "window_hi": ("int s_hi = (ib + p->radius + 1) * p->bsize; /* exclusive */",
                  "int s_hi = (ib + p->radius) * p->bsize; /* exclusive */"),
}


def _battery(lib):
    """Run the pins; return the names of those that fail."""
    failed = []
    rng = np.random.default_rng(2024)
    cases = [(32, 6, 1, False, [192, 150]), (32, 6, 2, True, [192, 70]),
             (4, 10, 3, False, [40, 17]), (8, 5, 0, True, [40, 33])]
    for bsize, nblk, radius, causal, lens in cases:
        n = nblk * bsize
        lens = np.array(lens, dtype=np.int32)
        q, k, v = [(rng.standard_normal((2, 2, n, 8))).astype(np.float32) for _ in range(3)]
        try:
            o, lse, psum = oracle.forward(q, k, v, lens, bsize, radius, causal, lib=lib)
            ro, rl = dense_reference(q, k, v, lens, bsize, radius, causal)
            if not np.max(np.abs(o - ro)) <= 1e-12:
                failed.append("brute_force_o")
            for b in range(2):
                L = lens[b]
                if not np.allclose(lse[b, :, :L], rl[b, :, :L], rtol=0, atol=1e-12):
                    failed.append("brute_force_lse")
                if not np.allclose(psum[b, :, :L], 1.0, atol=1e-13):
                    failed.append("psum")
            r = oracle.forward_recurrence(q, k, v, lens, bsize, radius, causal, lib=lib)
            if not np.max(np.abs(r - ro)) <= 1e-12:
                failed.append("recurrence")
            act = oracle.active_blocks(2, n, bsize, radius, causal, lens, lib=lib)
            msk = oracle.masks(2, n, bsize, radius, causal, lens, act, lib=lib)
            for b in range(2):
                keep = token_mask(n, int(lens[b]), bsize, radius, causal)
                for i in range(nblk):
                    rows = keep[i * bsize:(i + 1) * bsize]
                    ref = [j for j in range(nblk) if rows[:, j * bsize:(j + 1) * bsize].any()]
                    if [int(j) for j in act[b, i] if j >= 0] != ref:
                        failed.append("lists")
                    for slot, j in enumerate(act[b, i]):
                        if j < 0:
                            continue
                        blk = rows[:, j * bsize:(j + 1) * bsize]
                        words = [sum(1 << c for c in range(bsize) if blk[rr, c])
                                 for rr in range(bsize)]
                        if list(msk[b, i, slot]) != words:
                            failed.append("masks")
        except oracle.OracleError:
            failed.append("error")
    return sorted(set(failed))


def test_unmodified_oracle_passes_battery():
    assert _battery(oracle.load()) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with open(obuild.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "orc_mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib_path = obuild.build(out=os.path.join(tmp, "liborc_mutant.so"), src=path)
        lib = oracle.load(lib_path)
        assert _battery(lib) != [], f"mutant {name} slipped through every pin"


# ------------------------------------------------------------ backward pass

BWD_MUTANTS = {
    "bwd_drop_D": ("const double dS = P * (dP - Dt);", "const double dS = P * dP;"),
    "bwd_dq_no_scale": ("dq_row[c] += p->scale * dS * (double)ks[c];",
                        "dq_row[c] += dS * (double)ks[c];"),
    "bwd_dk_wrong_operand": ("dks[c] += p->scale * dS * (double)q_row[c];",
                             "dks[c] += p->scale * dS * ((double)ks[c] + 0.0 * q_row[c]);"),
    "bwd_dv_uses_dS": ("dvs[c] += P * (double)dot_[c];", "dvs[c] += dS * (double)dot_[c];"),
    "bwd_unnormalised_P": ("            sbuf[e] /= l;\n", "            sbuf[e] /= 1.0;\n"),
    "bwd_D_from_query": ("Dt += (double)dot_[c] * orow[c];",
                         "Dt += (double)dot_[c] * (double)q_row[c];"),
    "bwd_dP_from_keys": ("const float *vs = p->v + (base + s) * d;",
                         "const float *vs = p->k + (base + s) * d;"),
    "bwd_blocks_drop_last_row_block": ("qi <= i + p->radius; ++qi)", "qi < i + p->radius; ++qi)"),
}


def _fd_grad(lib, q, k, v, g, lens, bsize, radius, causal, which, idx):
    def loss(x):
        a = [q, k, v]
        a[which] = x
        o, _, _ = oracle.forward(*a, lens, bsize, radius, causal, nthreads=1, lib=lib)
        return float(np.sum(o * g))
    h = 2.0 ** -10
    x = [q, k, v][which]

    def central(hh):
        up, dn = x.copy(), x.copy()
        up[idx] += np.float32(hh)
        dn[idx] -= np.float32(hh)
        return (loss(up) - loss(dn)) / (2 * hh)
    return (4 * central(h / 2) - central(h)) / 3


def _bwd_battery(lib):
    """Backward pins against a (possibly mutated) oracle; the forward used for
    the finite differences is the unmodified one."""
    failed = []
    ref_lib = oracle.load()
    rng = np.random.default_rng(99)
    for bsize, nblk, radius, causal, lens in [(8, 5, 1, False, [40, 27]), (8, 5, 2, True, [40, 21])]:
        n = nblk * bsize
        lens = np.array(lens, dtype=np.int32)
        q, k, v, g = [(np.round(rng.uniform(-1, 1, (2, 1, n, 8)) * 128) / 128).astype(np.float32)
                      for _ in range(4)]
        try:
            dq, dk, dv = oracle.backward(q, k, v, g, lens, bsize, radius, causal, lib=lib)
            for which, grad in enumerate((dq, dk, dv)):
                for idx in [(0, 0, 5, 1), (0, 0, 33, 7), (1, 0, 20, 3)]:
                    fd = _fd_grad(ref_lib, q, k, v, g, lens, bsize, radius, causal, which, idx)
                    if not abs(fd - grad[idx]) <= 1e-8 + 1e-7 * abs(grad[idx]):
                        failed.append("finite_differences")
            for b in range(2):
                if not np.allclose(dv[b].sum(axis=1), g[b, :, :lens[b]].sum(axis=1), atol=1e-12):
                    failed.append("dv_sum")
                if not np.max(np.abs(dk[b].sum(axis=1))) <= 1e-12:
                    failed.append("dk_sum")
            sel = np.array([[0, 0, i] for i in range(nblk)] + [[1, 0, i] for i in range(nblk)],
                           dtype=np.int32)
            bq, bk, bv = oracle.backward_blocks(q, k, v, g, sel, lens, bsize, radius, causal,
                                                lib=lib)
            for w, (b, h, i) in enumerate(sel):
                rows = slice(i * bsize, (i + 1) * bsize)
                if not (np.allclose(bq[w], dq[b, h, rows], atol=1e-13)
                        and np.allclose(bk[w], dk[b, h, rows], atol=1e-13)
                        and np.allclose(bv[w], dv[b, h, rows], atol=1e-13)):
                    failed.append("blocks_vs_full")
        except oracle.OracleError:
            failed.append("error")
    return sorted(set(failed))


def test_unmodified_oracle_passes_backward_battery():
    assert _bwd_battery(oracle.load()) == []


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name):
    old, new = BWD_MUTANTS[name]
    with open(obuild.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "orc_mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib_path = obuild.build(out=os.path.join(tmp, "liborc_mutant.so"), src=path)
        lib = oracle.load(lib_path)
        assert _bwd_battery(lib) != [], f"mutant {name} slipped through every pin"


# ------------------------------------------------------------ k-mer tokenizer

KMER_MUTANTS = {
    "kmer_lsb_first": ("for (int p = k - 1; p >= 0; --p) {", "for (int p = 0; p < k; ++p) {"),
    "kmer_swap_c_g": ("case 'C': case 'c': return 1;\n    case 'G': case 'g': return 2;",
                      "case 'C': case 'c': return 2;\n    case 'G': case 'g': return 1;"),
    "kmer_unknown_ignored": ("id = bad ? unk : (int32_t)value;",
                             "id = (bad && 0) ? unk : (int32_t)value;"),
    "kmer_count_off_by_one": ("int64_t nt = len - k + 1;", "int64_t nt = len - k;"),
    "kmer_case_sensitive": ("case 'A': case 'a': return 0;", "case 'A': return 0;"),
    "kmer_pad_zero": ("int32_t id = pad;", "int32_t id = 0 * pad;"),
    "kmer_window_shift": ("const int c = base_code(seq[t + p]);",
                          "const int c = base_code(seq[t + p + (t > 0)]);"),
}


def _kmer_battery(lib):
    failed = []
    here = os.path.dirname(os.path.abspath(__file__))

    def tok(text, k=6, n_out=None):
        b = np.frombuffer(text, dtype=np.uint8)
        return oracle.kmer_tokenize(b, np.array([0, len(b)]), k, n_out, lib=lib)
    try:
        with open(os.path.join(here, "golden", "kmer_page_ids.txt")) as f:
            for line in f:
                if line.strip() and not line.startswith("#"):
                    kmer, ident = line.split()
                    if tok(kmer.encode())[0][0, 0] != int(ident):
                        failed.append("page_ids")
        import itertools
        kmers = "".join("".join(t) for t in itertools.product("ACGT", repeat=3)).encode()
        ids, _ = oracle.kmer_tokenize(np.frombuffer(kmers, np.uint8),
                                      np.arange(65, dtype=np.int64) * 3, 3, lib=lib)
        if not np.array_equal(ids[:, 0], np.arange(64)):
            failed.append("lexicographic")
        rng = np.random.default_rng(3)
        text = rng.choice(list(b"ACGT"), 200).astype(np.uint8).tobytes()
        ids, nt = tok(text)
        code = {65: 0, 67: 1, 71: 2, 84: 3}
        if nt[0] != 195:
            failed.append("count")
        row = ids[0].astype(np.int64)
        if any(row[t + 1] != (row[t] % 1024) * 4 + code[text[t + 6]] for t in range(min(nt[0], 195) - 1)):
            failed.append("sliding")
        ids, nt = tok(b"ACGTACGTACGTNACGTACGTAC", 6, 32)
        unk = [t for t in range(nt[0]) if ids[0, t] == 4098]
        if unk != list(range(7, 13)):
            failed.append("unknown")
        if not np.all(ids[0, nt[0]:] == 4096):
            failed.append("pad")
        if not np.array_equal(tok(b"acgtacgtacgtnacgtacgtac", 6, 32)[0], ids):
            failed.append("case")
    except oracle.OracleError:
        failed.append("error")
    return sorted(set(failed))


def test_unmodified_oracle_passes_kmer_battery():
    assert _kmer_battery(oracle.load()) == []


@pytest.mark.parametrize("name", sorted(KMER_MUTANTS))
def test_kmer_mutant_is_caught(name):
    old, new = KMER_MUTANTS[name]
    with open(obuild.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "orc_mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib_path = obuild.build(out=os.path.join(tmp, "liborc_mutant.so"), src=path)
        lib = oracle.load(lib_path)
        assert _kmer_battery(lib) != [], f"mutant {name} slipped through every pin"


# ------------------------------------------------------------ token window

WINDOW_MUTANTS = {
    "window_off_by_one": ("if (window >= 0 && abs(t - s) > window)",
                          "if (window >= 0 && abs(t - s) >= window)"),
    "window_ignored": ("if (window >= 0 && abs(t - s) > window)",
                       "if (window >= 1 << 30 && abs(t - s) > window)"),
    "window_one_sided": ("if (window >= 0 && abs(t - s) > window)",
                         "if (window >= 0 && t - s > window)"),
}


def _window_battery(lib):
    failed = []
    rng = np.random.default_rng(7)
    for bsize, window, causal, lens in [(32, 5, False, [96, 70]), (8, 12, True, [96, 41]),
                                        (4, 0, False, [32, 17])]:
        n = 96 if bsize != 4 else 32
        lens = np.array(lens, dtype=np.int32)
        q, k, v = [(rng.standard_normal((2, 1, n, 8))).astype(np.float32) for _ in range(3)]
        try:
            o, _, _ = oracle.forward(q, k, v, lens, bsize, 0, causal, lib=lib, window=window)
            ro, _ = dense_reference(q, k, v, lens, bsize, 0, causal, window=window)
            if not np.max(np.abs(o - ro)) <= 1e-12:
                failed.append("brute_force")
            act = oracle.active_blocks(2, n, bsize, 0, causal, lens, lib=lib, window=window)
            msk = oracle.masks(2, n, bsize, 0, causal, lens, act, lib=lib, window=window)
            for b in range(2):
                keep = token_mask(n, int(lens[b]), bsize, 0, causal, window)
                for i in range(n // bsize):
                    for slot, j in enumerate(act[b, i]):
                        if j < 0:
                            continue
                        blk = keep[i * bsize:(i + 1) * bsize, j * bsize:(j + 1) * bsize]
                        words = [sum(1 << c for c in range(bsize) if blk[r, c])
                                 for r in range(bsize)]
                        if list(msk[b, i, slot]) != words:
                            failed.append("masks")
        except oracle.OracleError:
            failed.append("error")
    return sorted(set(failed))


def test_unmodified_oracle_passes_window_battery():
    assert _window_battery(oracle.load()) == []


@pytest.mark.parametrize("name", sorted(WINDOW_MUTANTS))
def test_window_mutant_is_caught(name):
    old, new = WINDOW_MUTANTS[name]
    with open(obuild.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "orc_mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib_path = obuild.build(out=os.path.join(tmp, "liborc_mutant.so"), src=path)
        lib = oracle.load(lib_path)
        assert _window_battery(lib) != [], f"mutant {name} slipped through every pin"
