"""Host-side logic of bench.py and of the work accounting it reports (CPU only).

The accounting is pinned to the oracle: the useful (query, key) pairs of a
workload are the set bits of the oracle's masks, and the block pairs are the
oracle's active-block entries (NucleoByte project page, section 3, "Localized
Block-Sparse Attention Matrix")."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from block_sparse_local_amd import inputs, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SRC = '''// header comment
#include "launch.h"   // trailing comment
/* block
   comment */
#define SLACK 8.0f
__device__ int f(int x) { return x + 1; } // done
const char *s = "a // not a comment";
'''


def test_code_text_ignores_comments_and_layout():
    base = bench.code_text(SRC)
    edited = SRC.replace("// header comment", "// a different header\n// and one more line")
    edited = edited.replace("/* block\n   comment */", "/* shorter */")
    edited = edited.replace("{ return x + 1; }", "{   return   x + 1;  }")
    assert bench.code_text(edited) == base
    assert "//" in base  # the one inside the string literal survives
    assert "comment" not in base.replace("not a comment", "")


def test_code_text_sees_code_and_literal_changes():
    base = bench.code_text(SRC)
    assert bench.code_text(SRC.replace("8.0f", "4.0f")) != base
    assert bench.code_text(SRC.replace("x + 1", "x + 2")) != base
    assert bench.code_text(SRC.replace('"a // not', '"b // not')) != base
    # line breaks are kept (the preprocessor needs them): a reflow counts as a change
    assert bench.code_text(SRC.replace("{ return x + 1; }", "{\n return x + 1;\n}")) != base
    # a preprocessor line stays a line of its own
    assert "#define SLACK 8.0f\n" in base


def test_stored_traffic_needs_the_current_kernel_code(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    (csrc / "k.hip").write_text(SRC)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["csrc/k.hip"])
    sha = bench.kernel_sha()
    prof = tmp_path / "profiles" / "pmc_traffic_fwd_bf16_cx.txt"
    prof.write_text(f"traffic_bytes_per_launch: 1.5e+09\nkernel_code_sha256_16: {sha}\n")
    assert bench.stored_traffic("cx") == 1.5e9
    assert bench.stored_traffic("missing") is None
    # a comment edit keeps the summary valid, a code edit voids it
    (csrc / "k.hip").write_text("// new note\n" + SRC)
    assert bench.stored_traffic("cx") == 1.5e9
    (csrc / "k.hip").write_text(SRC.replace("x + 1", "x - 1"))
    assert bench.stored_traffic("cx") is None
    # another build of the library (a design variant) never borrows the summary
    (csrc / "k.hip").write_text(SRC)
    monkeypatch.setenv("BSL_LIBRARY", str(tmp_path / "variant.so"))
    assert bench.stored_traffic("cx") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("key", ["c1", "c2", "c3"])
def test_account_matches_the_oracle(key):
    w = inputs.WORKLOADS[key]
    lens, n = inputs.lengths(w, 42)
    act = oracle.active_blocks(w.batch, n, 32, w.radius, w.causal, lens)
    msk = oracle.masks(w.batch, n, 32, w.radius, w.causal, lens, act)
    bits = int(np.unpackbits(msk.astype("<u4").view(np.uint8)).sum())
    acc = workload.account(lens, w.heads, w.d, w.radius, w.causal, w.dtype)
    esz = 2 if w.dtype == "bf16" else 4
    assert acc["useful_pairs"] == bits * w.heads
    assert acc["block_pairs"] == int((act >= 0).sum()) * w.heads
    assert acc["useful_flops"] == 4.0 * w.d * bits * w.heads
    assert acc["computed_flops"] == 4.0 * w.d * 32 * 32 * int((act >= 0).sum()) * w.heads
    assert acc["alg_bytes"] == 4.0 * int(np.sum(lens)) * w.heads * w.d * esz
    assert acc["tokens"] == int(np.sum(lens))


@pytest.mark.parametrize("window,causal", [(1, False), (33, True), (100, False), (256, True)])
def test_account_window_matches_the_oracle(window, causal):
    lens = np.array([1000, 0, 33, 517], np.int32)
    n = 1024
    act = oracle.active_blocks(len(lens), n, 32, 0, causal, lens, window=window)
    msk = oracle.masks(len(lens), n, 32, 0, causal, lens, act, window=window)
    bits = int(np.unpackbits(msk.astype("<u4").view(np.uint8)).sum())
    acc = workload.account(lens, 3, 64, 0, causal, "bf16", window=window)
    assert acc["useful_pairs"] == bits * 3
    assert acc["block_pairs"] == int((act >= 0).sum()) * 3
    assert acc["alg_bytes"] == 4.0 * int(lens.sum()) * 3 * 64 * 2


def test_account_bound_and_peaks():
    # bf16 at this shape is memory bound; fp32 is priced against the vector ALUs
    a = workload.account([4096], 16, 128, 8, False, "bf16")
    assert a["bound"] == "hbm" and a["flops_peak"] == 2.5e15
    assert a["t_hbm"] == a["alg_bytes"] / 8.0e12
    f = workload.account([256], 1, 32, 1, False, "f32")
    assert f["flops_peak"] == 157.3e12
    assert f["bound"] in ("hbm", "alu")
    # a radius covering the whole sequence makes every pair useful
    full = workload.account([96], 1, 64, 5, False, "bf16")
    assert full["useful_pairs"] == 96 * 96
    causal = workload.account([96], 1, 64, 5, True, "bf16")
    assert causal["useful_pairs"] == 96 * 97 // 2


def test_summarize_roofline_fields():
    w = inputs.WORKLOADS["c4"]
    lens, n = inputs.lengths(w, 42)
    acc = workload.account(lens, w.heads, w.d, w.radius, w.causal, w.dtype)
    per_launch = np.full(10, 1.0e-3)
    r = {"acc": acc, "w": w, "per_launch": per_launch, "wall": 0.0105, "steps": 10}
    t_step, roof, extra = bench.summarize(r, traffic=2.2e9)
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] == pytest.approx(acc["alg_bytes"] / 1.0e-3 / 1e9)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 8000.0)
    assert roof["traffic"] == 2.2e9
    assert t_step == pytest.approx(1.05e-3)
    assert extra["useful_tflops"] == pytest.approx(acc["useful_flops"] / 1.05e-3 / 1e12)
    assert extra["tokens_per_s"] == pytest.approx(acc["tokens"] / 1.05e-3)
    assert extra["median_launch_us"] == pytest.approx(1.0e3)
    assert extra["p90_launch_us"] == pytest.approx(1.0e3)


def test_account_backward():
    w = inputs.WORKLOADS["c2"]
    lens, n = inputs.lengths(w, 42)
    fwd = workload.account(lens, w.heads, w.d, w.radius, w.causal, w.dtype)
    bwd = workload.account_backward(lens, w.heads, w.d, w.radius, w.causal, w.dtype)
    assert bwd["useful_pairs"] == fwd["useful_pairs"]
    assert bwd["useful_flops"] == 2.5 * fwd["useful_flops"]
    assert bwd["alg_bytes"] == (8 * w.d * 2 + 4) * int(np.sum(lens)) * w.heads
    assert bwd["computed_flops"] == 14.0 * w.d * 32 * 32 * fwd["block_pairs"]
    # the long-context shape is bound by the matrix cores, unlike its forward
    c4 = inputs.WORKLOADS["c4"]
    l4, _ = inputs.lengths(c4, 42)
    b4 = workload.account_backward(l4, c4.heads, c4.d, c4.radius, c4.causal, c4.dtype)
    assert b4["bound"] == "mfma" and b4["t_mfma"] > b4["t_hbm"]



@pytest.mark.parametrize("window,causal", [(40, False), (256, True)])
def test_account_backward_window_matches_the_oracle(window, causal):
    lens = np.array([700, 129], np.int32)
    n = 704
    act = oracle.active_blocks(len(lens), n, 32, 0, causal, lens, window=window)
    msk = oracle.masks(len(lens), n, 32, 0, causal, lens, act, window=window)
    bits = int(np.unpackbits(msk.astype("<u4").view(np.uint8)).sum())
    acc = workload.account_backward(lens, 4, 128, 0, causal, "bf16", window=window)
    assert acc["useful_pairs"] == bits * 4
    assert acc["useful_flops"] == 10.0 * 128 * bits * 4
    assert acc["block_pairs"] == int((act >= 0).sum()) * 4
