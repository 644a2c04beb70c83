#!/usr/bin/env python3
"""Benchmark: banded block-sparse attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c4|c5|c3|c2|c1]

One step is one forward call of the whole hot path (block plan, Q/K/V loads,
scores, masks, online softmax, P V, normalisation and store) over one batch of
seeded synthetic inputs already resident in HBM.  W untimed steps, then K timed
steps between two device synchronisations.  Prints one JSON line:

  value        useful TFLOP/s (4 * d per kept query/key pair) over the timed
               region's wall clock
  roofline     the kernel's algorithmic bytes (or FLOP) per launch over its
               mean launch time from HIP events on the launch stream, against
               the MI355X peak; traffic = HBM bytes per launch measured with
               rocprofv3 counters (profiles/), null when the kernel source has
               changed since
  cpu_baseline the fp64 oracle, as written, timed on this host's cores over a
               bounded sample of query blocks of the same workload

The default workload is the 1.3B-shape long-context case: batch 1, 16 heads,
131072-row buffer holding a 130000-token sequence, head dim 128, radius 8.
The million-token case (c5, the other workload with a roofline target) is
timed in the same run, beside the headline (``--no-secondary`` skips it);
every timed workload also gets a cold-cache pass (1 GiB written between
launches, outside the events), reported under ``detail.cold``;
``--window W`` also times the chosen workload with a token window of W tokens
(|t - s| <= W) in place of the block band.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# the headline metric, verbatim as the benchmark definition states it
METRIC = "block-sparse attn fwd useful TFLOP/s + tokens/s; % of bf16 MFMA/HBM roofline"

KERNEL_SOURCES = ["block_sparse_local_amd/csrc/fwd_bf16.hip", "block_sparse_local_amd/csrc/cdna4.h",
                  "block_sparse_local_amd/csrc/launch.h"]


def _scan(src, on_comment, on_space):
    """Walk C/C++ source; string and character literals are copied verbatim,
    comments and whitespace runs are replaced by what the callbacks return."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i) and on_comment:
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i) and on_comment:
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif c.isspace() and on_space:
            j = i
            while j < n and src[j].isspace():
                j += 1
            out.append(on_space(src[i:j]))
            i = j
        else:
            out.append(c)
            i += 1
    return "".join(out)


def code_text(src):
    """C/C++ source with comments removed and every whitespace run outside
    string and character literals reduced to one newline (if it held one, for
    the preprocessor) or one space: two sources with the same code_text compile
    to the same kernel, so a comment edit does not void the stored counter
    summaries."""
    bare = _scan(src, True, None)
    return _scan(bare, False, lambda ws: "\n" if "\n" in ws else " ").strip()


BWD_SOURCES = ["block_sparse_local_amd/csrc/bwd_bf16.hip", "block_sparse_local_amd/csrc/cdna4.h",
               "block_sparse_local_amd/csrc/bwd_launch.h"]
KMER_SOURCES = ["block_sparse_local_amd/csrc/kmer.hip", "block_sparse_local_amd/csrc/kmer_launch.h"]


def kernel_sha():
    """Hash of the bf16 kernel's code (comments and layout excluded)."""
    return code_sha(KERNEL_SOURCES)


def code_sha(sources):
    """Hash of the code of the given sources (comments and layout excluded)."""
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode("utf-8"))
    return h.hexdigest()[:16]


def stored_traffic(workload_key, kernel="fwd_bf16", sources=None):
    """Bytes per launch from the committed counter summary, if it was taken on
    the current kernel code."""
    if os.environ.get("BSL_LIBRARY"):
        return None  # the stored counters describe the in-tree build only
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{kernel}_{workload_key}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^kernel_code_sha256_16:\s*(\w+)", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not sha or not val or sha.group(1) != code_sha(sources or KERNEL_SOURCES):
        return None
    return float(val.group(1))


def to_device(x, dtype):
    import torch
    from block_sparse_local_amd import inputs
    if dtype == "bf16":
        return torch.from_numpy(inputs.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def pack_device(x, lens):
    """[batch, heads, n, d] device tensor -> the packed [tokens, heads, d] layout
    (each sequence's real rows, token-major, back to back)."""
    import torch
    return torch.cat([x[b, :, :int(L)].transpose(0, 1) for b, L in enumerate(lens)]).contiguous()


def time_workload(key, steps, warmup, cold=False, log=print, layout="padded", window=0):
    """Times bsl_forward on the workload (layout "padded": [batch][heads][n][d])
    or bsl_forward_varlen on the same sequences packed ("packed":
    [tokens][heads][d], no padding between sequences); window >= 1 replaces the
    block band with a token window of that many tokens."""
    import torch
    from block_sparse_local_amd import bsl, inputs, workload

    t0 = time.time()
    d = inputs.make(key, 42)
    w = d["workload"]
    lens = d["seqlens"]
    log(f"[bench] {key} inputs drawn in {time.time() - t0:.1f}s: {w.describe()} ({layout}"
        f"{f', token window {window}' if window else ''})")
    q, k, v = (to_device(d[x], w.dtype) for x in ("q", "k", "v"))
    plan = bsl.Plan(w.d, w.heads, w.radius, w.causal, w.dtype, window=window)
    if layout == "packed":
        q, k, v = (pack_device(x, lens) for x in (q, k, v))
        cu_host, max_len, _ = bsl.bsl_varlen_offsets(lens)
        cu = torch.from_numpy(cu_host).cuda()

        def call():
            plan.forward_varlen(q, k, v, cu, max_len, o=o, stream=stream)
    else:
        sl = torch.from_numpy(lens).cuda()

        def call():
            plan.forward(q, k, v, sl, o=o, stream=stream)
    o = torch.empty_like(q)
    buffer_bytes = 4 * q.numel() * q.element_size()
    acc = workload.account(lens, w.heads, w.d, w.radius, w.causal, w.dtype, window)
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if cold else None

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()

    def timed(flush):
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        t_begin = time.perf_counter()
        for s in range(steps):
            if flush is not None:
                flush.fill_(float(s))
            starts[s].record(stream)
            call()
            ends[s].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_begin
        return wall, np.array([a.elapsed_time(b) * 1e-3 for a, b in zip(starts, ends)])

    wall, per_launch = timed(flush)
    # caches made cold before every launch: 1 GiB written between launches
    # (outside the events), more than the L2s and the 256 MB Infinity Cache hold
    if flush is None:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        _, cold_launch = timed(flush)
    else:
        cold_launch = per_launch
    plan.close()
    del q, k, v, o, flush
    torch.cuda.empty_cache()
    return dict(key=key, w=w, d=d, acc=acc, wall=wall, per_launch=per_launch, steps=steps,
                layout=layout, buffer_bytes=buffer_bytes, window=window, cold_launch=cold_launch)


def copy_bandwidth(reps=10):
    """Achievable HBM rate on this GPU, for context beside the 8 TB/s peak: a
    1 GiB device-to-device copy, bytes read + written over its mean time."""
    import torch
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        b.copy_(a)
    ev[1].record()
    torch.cuda.synchronize()
    sec = ev[0].elapsed_time(ev[1]) * 1e-3 / reps
    nbytes = 2 * a.numel() * a.element_size()
    del a, b
    torch.cuda.empty_cache()
    return {"value": nbytes / sec / 1e9, "unit": "GB/s",
            "what": "1 GiB device-to-device copy (torch), read + written bytes over time"}


def time_backward(key, steps, warmup, log=print, window=0, layout="padded"):
    """The backward pass (bsl_backward) on the workload's inputs and a seeded
    output gradient, after one forward that supplies O and lse; window >= 1
    differentiates the token-window forward instead of the block band, and
    layout "packed" times bsl_backward_varlen on the same sequences packed."""
    import torch
    from block_sparse_local_amd import bsl, inputs, workload

    d = inputs.make(key, 42, grad=True)
    w = d["workload"]
    lens = d["seqlens"]
    q, k, v, g = (to_device(d[x], w.dtype) for x in ("q", "k", "v", "dout"))
    sl = torch.from_numpy(lens).cuda()
    plan = bsl.Plan(w.d, w.heads, w.radius, w.causal, w.dtype, window=window)
    stream = torch.cuda.current_stream()
    if layout == "packed":
        q, k, v, g = (pack_device(x, lens) for x in (q, k, v, g))
        cu_host, max_len, _ = bsl.bsl_varlen_offsets(lens)
        cu = torch.from_numpy(cu_host).cuda()
        o = torch.empty_like(q)
        lse = torch.empty((w.heads, q.shape[0]), dtype=torch.float32, device="cuda")
        plan.forward_varlen(q, k, v, cu, max_len, o=o, lse=lse, stream=stream)
        delta = torch.empty((w.heads, q.shape[0]), dtype=torch.float32, device="cuda")
    else:
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        plan.forward(q, k, v, sl, o=o, lse=lse, stream=stream)
        delta = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def call():
        if layout == "packed":
            plan.backward_varlen(q, k, v, o, g, lse, cu, max_len, dq=dq, dk=dk, dv=dv,
                                 delta=delta, stream=stream)
        else:
            plan.backward(q, k, v, o, g, lse, sl, dq=dq, dk=dk, dv=dv, delta=delta,
                          stream=stream)
    acc = workload.account_backward(lens, w.heads, w.d, w.radius, w.causal, w.dtype, window)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t_begin = time.perf_counter()
    for s in range(steps):
        starts[s].record(stream)
        call()
        ends[s].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_begin
    per_launch = np.array([a.elapsed_time(b) * 1e-3 for a, b in zip(starts, ends)])
    plan.close()
    del q, k, v, g, o, lse, dq, dk, dv, delta
    torch.cuda.empty_cache()
    log(f"[bench] {key} backward{f' (token window {window})' if window else ''}"
        f"{' (packed)' if layout == 'packed' else ''}: {wall / steps * 1e3:.3f} ms/step")
    return dict(key=key, w=w, d=d, acc=acc, wall=wall, per_launch=per_launch, steps=steps,
                window=window, layout=layout)


def cpu_baseline_backward(r, target_flops=6.0e11, log=print):
    """The fp64 oracle's backward on every head of the first tokens of the
    workload's first sequence (a bounded sample of the same shape, about
    ``target_flops`` useful FLOP)."""
    import oracle
    from block_sparse_local_amd import workload
    d, w = r["d"], r["w"]
    window = r.get("window", 0)
    per_token = 10.0 * w.d * (2 * workload.band_radius(w.radius, window) + 1) * 32 * w.heads
    rows = max(32, int(target_flops / per_token) // 32 * 32)
    L = min(rows, int(d["seqlens"][0]))
    n = -(-L // 32) * 32
    sl = lambda x: np.ascontiguousarray(x[:1, :, :n])
    lens = np.array([L], dtype=np.int32)
    threads = min(16, oracle.default_threads())
    t0 = time.perf_counter()
    oracle.backward(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["dout"]), lens, 32, w.radius,
                    w.causal, nthreads=threads, window=window if window > 0 else None)
    dt = time.perf_counter() - t0
    acc = workload.account_backward(lens, w.heads, w.d, w.radius, w.causal, w.dtype, window)
    log(f"[bench] oracle backward: {w.heads} heads x {L} tokens in {dt:.1f}s")
    return {"value": acc["useful_flops"] / dt / 1e12, "unit": "TFLOP/s",
            "cores": min(threads, w.heads), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"backward of all {w.heads} heads over the first {L} tokens of sequence 0 "
                      f"(one thread per head); {acc['useful_flops'] / 1e9:.1f} useful GFLOP in "
                      f"{dt:.2f}s",
            "seconds": dt}


def cpu_model():
    """The host processor's model name from /proc/cpuinfo, with its family,
    model and stepping numbers and the logical CPU count (a virtual machine
    may report only a generic name), or the platform's description."""
    try:
        info, count = {}, 0
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "processor":
                    count += 1
                elif key in ("model name", "cpu family", "model", "stepping") and key not in info:
                    info[key] = val.strip()
        if "model name" in info:
            ids = ", ".join(f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info)
            return f"{info['model name']} ({ids}; {count} logical CPUs)" if ids else info["model name"]
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(r, target_flops=1.0e12, log=print):
    """Time the fp64 oracle on a bounded, evenly spread sample of query blocks
    (every head) of the same workload, on this host's cores."""
    import oracle
    from block_sparse_local_amd import workload
    d, w = r["d"], r["w"]
    lens = d["seqlens"]
    n = d["n"]
    nblk = n // 32
    per_block = r["acc"]["useful_flops"] / max(1, sum(-(-int(L) // 32) for L in lens) * w.heads)
    want = int(max(1, min(nblk * w.batch, target_flops / max(per_block, 1.0) / w.heads)))
    sel = []
    for b in range(w.batch):
        nb = -(-int(lens[b]) // 32)
        if nb == 0:
            continue
        share = max(1, int(round(want * nb / max(1, sum(-(-int(L) // 32) for L in lens)))))
        for i in np.unique(np.linspace(0, nb - 1, min(share, nb)).astype(int)):
            for h in range(w.heads):
                sel.append((b, h, int(i)))
    sel = np.array(sel, dtype=np.int32)
    threads = min(16, oracle.default_threads())
    window = r.get("window", 0)
    t0 = time.perf_counter()
    oracle.forward_blocks(d["q"], d["k"], d["v"], sel, lens, 32, w.radius, w.causal,
                          nthreads=threads, window=window if window > 0 else None)
    dt = time.perf_counter() - t0
    # useful work of exactly the sampled query rows
    flops = 0.0
    tokens = 0
    for b in range(w.batch):
        rows = sel[sel[:, 0] == b]
        if len(rows) == 0:
            continue
        L = int(lens[b])
        for i in np.unique(rows[:, 2]):
            hcount = int((rows[:, 2] == i).sum())
            t = np.arange(i * 32, min(L, i * 32 + 32))
            lo, hi = workload.key_range(t, L, w.radius, w.causal, window)
            flops += 4.0 * w.d * float((hi - lo).sum()) * hcount
            tokens += len(t) * hcount
    log(f"[bench] oracle: {len(sel)} (sequence, head, query block) units in {dt:.1f}s "
        f"on {threads} threads")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{len(sel)} query blocks (of {w.batch * nblk * w.heads} block-heads): "
                      f"{len(sel) // w.heads} evenly spaced blocks x all {w.heads} heads; "
                      f"{flops / 1e9:.1f} useful GFLOP in {dt:.2f}s",
            "tokens_per_s": tokens / w.heads / dt,
            "seconds": dt}


def time_kmer(key, steps, warmup, log=print):
    """The fused k-mer tokenizer (bsl_kmer_tokenize) on a seeded nucleotide
    workload resident in HBM: text, offsets, padded int32 ID rows, counts."""
    import torch
    from block_sparse_local_amd import bsl, inputs

    t0 = time.time()
    d = inputs.make_dna(key, 42)
    w = d["workload"]
    log(f"[bench] {key} text drawn in {time.time() - t0:.1f}s: {w.describe()}, "
        f"{len(d['bases'])} bytes, rows of {d['n_out']}")
    bases = torch.from_numpy(d["bases"]).cuda()
    starts = torch.from_numpy(d["starts"]).cuda()
    batch, n_out = w.batch, d["n_out"]
    ids = torch.empty((batch, n_out), dtype=torch.int32, device="cuda")
    ntok = torch.empty(batch, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        bsl.kmer_tokenize(bases, starts, w.k, n_out, ids=ids, ntok=ntok, stream=stream)
    torch.cuda.synchronize()
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t_begin = time.perf_counter()
    for s in range(steps):
        ev0[s].record(stream)
        bsl.kmer_tokenize(bases, starts, w.k, n_out, ids=ids, ntok=ntok, stream=stream)
        ev1[s].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_begin
    per_launch = np.array([a.elapsed_time(b) * 1e-3 for a, b in zip(ev0, ev1)])
    windows = int(ntok.sum().item())
    del bases, starts, ids, ntok
    torch.cuda.empty_cache()
    # algorithmic bytes: the text read once, the offsets, every ID row element
    # and every count written once
    alg = len(d["bases"]) + 8 * (batch + 1) + 4 * batch * n_out + 4 * batch
    mean = float(per_launch.mean())
    t_step = wall / steps
    roof = {"bound": "hbm", "achieved": alg / mean / 1e9, "peak": 8000.0, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(key, "kmer", KMER_SOURCES)
    out = {"config": {"workload": f"{key} {w.describe()}", "sequences": batch,
                      "bases": int(len(d["bases"])), "k": w.k, "n_out": n_out,
                      "windows": windows},
           "metric": "k-mer tokens/s", "value": windows / t_step, "unit": "tokens/s",
           "ms_per_step": t_step * 1e3, "roofline": roof,
           "detail": {"mean_launch_us": mean * 1e6,
                      "median_launch_us": float(np.median(per_launch)) * 1e6,
                      "alg_bytes": alg, "windows": windows}}
    log(f"[bench] {key} tokenizer: {t_step * 1e3:.3f} ms/step, {windows / t_step / 1e9:.2f} G "
        f"windows/s, {roof['achieved']:.0f} GB/s ({roof['frac'] * 100:.1f}% of hbm peak)")
    return out, d


def cpu_baseline_kmer(d, log=print, target_bytes=2.0e9):
    """The oracle tokenizer (one thread: it is a single loop) on the first
    sequences of the same workload, about ``target_bytes`` of text."""
    import oracle
    w = d["workload"]
    starts = d["starts"]
    nseq = int(np.searchsorted(starts, target_bytes)) or 1
    nseq = min(nseq, w.batch)
    sub = starts[:nseq + 1]
    text = d["bases"][:int(sub[-1])]
    t0 = time.perf_counter()
    _, nt = oracle.kmer_tokenize(text, sub, w.k, d["n_out"])
    dt = time.perf_counter() - t0
    windows = int(nt.sum())
    log(f"[bench] oracle tokenizer: {nseq} sequences, {windows} windows in {dt:.1f}s")
    return {"value": windows / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"the first {nseq} of {w.batch} sequences ({len(text)} bases, "
                      f"{windows} windows), one thread", "seconds": dt}


def summarize(r, traffic=None):
    acc, w = r["acc"], r["w"]
    t_step = r["wall"] / r["steps"]
    mean_launch = float(r["per_launch"].mean())
    alg_bytes, flops = acc["alg_bytes"], acc["useful_flops"]
    bound = acc["bound"]
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": alg_bytes / mean_launch / 1e9, "peak": 8000.0,
                "unit": "GB/s"}
    else:
        roof = {"bound": bound, "achieved": flops / mean_launch / 1e12,
                "peak": acc["flops_peak"] / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    cold = r.get("cold_launch")
    extra = {
        "useful_tflops": flops / t_step / 1e12,
        "tokens_per_s": acc["tokens"] / t_step,
        "mean_launch_us": mean_launch * 1e6,
        "median_launch_us": float(np.median(r["per_launch"])) * 1e6,
        "min_launch_us": float(r["per_launch"].min()) * 1e6,
        "p90_launch_us": float(np.percentile(r["per_launch"], 90)) * 1e6,
        "alg_bytes": alg_bytes,
        "useful_flops": flops,
        "computed_flops": acc["computed_flops"],
        "useful_pairs": acc["useful_pairs"],
        "block_pairs": acc["block_pairs"],
        "hbm_frac": alg_bytes / mean_launch / 8.0e12,
        "mfma_frac": flops / mean_launch / acc["flops_peak"],
        "roofline_frac": max(acc["t_hbm"], acc["t_mfma"]) / mean_launch,
    }
    if cold is not None:
        med = float(np.median(cold))
        extra["cold"] = {
            "what": "1 GiB written between launches (outside the events): every launch starts "
                    "with cold L2s and Infinity Cache",
            "median_launch_us": med * 1e6, "min_launch_us": float(cold.min()) * 1e6,
            "p90_launch_us": float(np.percentile(cold, 90)) * 1e6,
            "useful_tflops": flops / med / 1e12, "tokens_per_s": acc["tokens"] / med,
            "roofline_frac": max(acc["t_hbm"], acc["t_mfma"]) / med,
        }
    return t_step, roof, extra


def config_of(r):
    w, d = r["w"], r["d"]
    return {"workload": f"{w.key} {w.describe()}", "batch": w.batch, "heads": w.heads,
            "n": int(d["n"]), "head_dim": w.d, "radius": w.radius, "causal": w.causal,
            "block_size": 32, "tokens": int(np.sum(d["seqlens"])),
            "seqlens": [int(x) for x in d["seqlens"]] if w.batch <= 8 else "ragged"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-secondary", dest="secondary", action="store_false",
                    help="do not also time the million-token workload (c5), which the default "
                         "run times beside the headline workload")
    ap.add_argument("--cold", action="store_true",
                    help="overwrite 1 GiB between steps (outside the events)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward pass (bsl_backward) on the same workload")
    ap.add_argument("--varlen", action="store_true",
                    help="also time the same workload in the packed layout (bsl_forward_varlen)")
    ap.add_argument("--kmer", action="store_true",
                    help="also time the fused k-mer tokenizer (bsl_kmer_tokenize)")
    ap.add_argument("--kmer-workload", default="k1", choices=["k1", "k2"])
    ap.add_argument("--window", type=int, default=0,
                    help="also time the workload with a token window of this many tokens "
                         "(bsl_desc.window) in place of the block band")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 1 GiB device copies (for counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the banded attention forward is not sharded across "
              "GPUs in this library (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    import torch
    torch.cuda.set_device(0)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(max(1, args.steps)):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copied {a.numel() * 4} bytes x {max(1, args.steps)}")
        return

    r = time_workload(args.workload, args.steps, args.warmup, args.cold, log)
    traffic = stored_traffic(args.workload) if r["w"].dtype == "bf16" else None
    t_step, roof, extra = summarize(r, traffic)
    log(f"[bench] {args.workload}: {t_step * 1e3:.3f} ms/step, {extra['useful_tflops']:.1f} "
        f"useful TFLOP/s, {roof['achieved']:.0f} {roof['unit']} ({roof['frac'] * 100:.1f}% of "
        f"{roof['bound']} peak)")

    line = {
        "metric": METRIC,
        "value": extra["useful_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["w"].dtype,
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16 (no dataset)",
        "config": config_of(r),
        "tokens_per_s": extra["tokens_per_s"],
        "roofline": roof,
        "detail": extra,
        "copy_bandwidth": copy_bandwidth(),
    }
    if args.cold:
        line["timing"] = "cold: 1 GiB overwritten between steps"
    if os.environ.get("BSL_LIBRARY"):
        line["library"] = os.environ["BSL_LIBRARY"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(r, log=log)
    r_w_dtype = r["w"].dtype
    padded_bytes = r["buffer_bytes"]
    del r
    if args.varlen:
        rv = time_workload(args.workload, args.steps, args.warmup, args.cold, log, "packed")
        tv, roofv, extrav = summarize(rv, stored_traffic(args.workload, "fwd_bf16_packed"))
        line["varlen"] = {"layout": "packed [tokens][heads][head_dim], offsets cu_seqlens",
                          "ms_per_step": tv * 1e3, "value": extrav["useful_tflops"],
                          "unit": "TFLOP/s", "tokens_per_s": extrav["tokens_per_s"],
                          "roofline": roofv, "detail": extrav,
                          "buffer_bytes": rv["buffer_bytes"],
                          "padded_buffer_bytes": padded_bytes,
                          "padded_ms_per_step": t_step * 1e3}
        if not args.no_cpu_baseline:
            # the oracle has one layout: the same sequences, the same operation
            line["varlen"]["cpu_baseline"] = cpu_baseline(rv, log=log)
        if args.backward and r_w_dtype == "bf16":
            rbv = time_backward(args.workload, args.steps, args.warmup, log, layout="packed")
            tbv, roofbv, extrabv = summarize(rbv, None)
            line["varlen"]["backward"] = {"ms_per_step": tbv * 1e3,
                                          "value": extrabv["useful_tflops"], "unit": "TFLOP/s",
                                          "tokens_per_s": extrabv["tokens_per_s"],
                                          "roofline": roofbv, "detail": extrabv}
            del rbv
        log(f"[bench] {args.workload} packed: {tv * 1e3:.3f} ms/step "
            f"({roofv['frac'] * 100:.1f}% of {roofv['bound']} peak); buffers "
            f"{rv['buffer_bytes'] / 2**20:.1f} MiB vs {padded_bytes / 2**20:.1f} MiB padded")
        del rv
    if args.window > 0:
        rw = time_workload(args.workload, args.steps, args.warmup, args.cold, log,
                           window=args.window)
        tw, roofw, extraw = summarize(rw, stored_traffic(f"{args.workload}_window{args.window}"))
        line["window"] = {"window": args.window, "band_radius": -(-args.window // 32),
                          "ms_per_step": tw * 1e3, "value": extraw["useful_tflops"],
                          "unit": "TFLOP/s", "tokens_per_s": extraw["tokens_per_s"],
                          "roofline": roofw, "detail": extraw}
        if not args.no_cpu_baseline:
            line["window"]["cpu_baseline"] = cpu_baseline(rw, log=log)
        if args.backward and r_w_dtype == "bf16":
            rbw = time_backward(args.workload, args.steps, args.warmup, log, window=args.window)
            tbw, roofbw, extrabw = summarize(rbw, None)
            line["window"]["backward"] = {"ms_per_step": tbw * 1e3,
                                          "value": extrabw["useful_tflops"], "unit": "TFLOP/s",
                                          "tokens_per_s": extrabw["tokens_per_s"],
                                          "roofline": roofbw, "detail": extrabw}
            if not args.no_cpu_baseline:
                line["window"]["backward"]["cpu_baseline"] = cpu_baseline_backward(rbw, log=log)
            del rbw
        log(f"[bench] {args.workload} token window {args.window}: {tw * 1e3:.3f} ms/step, "
            f"{extraw['useful_tflops']:.1f} useful TFLOP/s ({roofw['frac'] * 100:.1f}% of "
            f"{roofw['bound']} peak)")
        del rw
    if args.secondary and args.workload != "c5":
        r5 = time_workload("c5", args.steps, args.warmup, args.cold, log)
        t5, roof5, extra5 = summarize(r5, stored_traffic("c5"))
        line["secondary"] = {"config": config_of(r5), "ms_per_step": t5 * 1e3,
                             "value": extra5["useful_tflops"], "unit": "TFLOP/s",
                             "tokens_per_s": extra5["tokens_per_s"], "roofline": roof5,
                             "detail": extra5}
        log(f"[bench] c5: {t5 * 1e3:.3f} ms/step, {roof5['achieved']:.0f} {roof5['unit']} "
            f"({roof5['frac'] * 100:.1f}%)")
    if args.backward and r_w_dtype == "bf16":
        rb = time_backward(args.workload, args.steps, args.warmup, log)
        tb, roofb, extrab = summarize(rb, stored_traffic(args.workload, "bwd_bf16", BWD_SOURCES))
        line["backward"] = {"ms_per_step": tb * 1e3, "value": extrab["useful_tflops"],
                            "unit": "TFLOP/s", "tokens_per_s": extrab["tokens_per_s"],
                            "roofline": roofb, "detail": extrab}
        if not args.no_cpu_baseline:
            line["backward"]["cpu_baseline"] = cpu_baseline_backward(rb, log=log)
        log(f"[bench] {args.workload} backward: {tb * 1e3:.3f} ms/step, "
            f"{extrab['useful_tflops']:.1f} useful TFLOP/s ({roofb['frac'] * 100:.1f}% of "
            f"{roofb['bound']} peak)")
    if args.kmer:
        kout, kd = time_kmer(args.kmer_workload, args.steps, args.warmup, log)
        if not args.no_cpu_baseline:
            kout["cpu_baseline"] = cpu_baseline_kmer(kd, log=log)
        line["kmer"] = kout
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
