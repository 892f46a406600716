#!/usr/bin/env python3
"""Throughput of exact attention (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-sweep] [--no-cpu-baseline]

A step is one forward and one backward pass (fa_fwd, then fa_bwd on its O, m,
l) over one batch of the workload, inputs resident in HBM.  The default
workload is the GPT-2-medium-shaped causal layer at N=4096 (B=2, H=16, d=64,
bf16).  The printed JSON line reports:

  value        (fwd + bwd algorithmic FLOPs) / time per step, in TFLOP/s;
               forward FLOPs are 4*B*H*N^2*d (halved when causal), backward
               2.5x that.
  roofline     the dominant call of the step (the one with the larger mean
               duration), timed with HIP events on the stream it runs on,
               against MI355X's dense bf16 MFMA peak (2500 TFLOP/s); traffic
               is the HBM bytes read + written per call from rocprofv3
               counters (scaled by a plain copy's counter reading), or null
               when the kernels changed after the counters were taken.
  cpu_baseline the fp64 oracle on a bounded sample of the same workload, on
               this host's cores (a reported baseline, not a target).
  fwd, bwd     mean, p10, p50 and p90 of each call's duration (hot cache:
               back-to-back steps).
  cold_cache   the same calls each timed after a 512 MiB buffer has been
               read, so neither L2 nor the 256 MB MALL holds their inputs (a
               read, not a write: written lines would be dirty, and their
               write-back would land inside the timed call).
  limiter      matrix-core busy, VALU busy and co-issue fractions of the
               step's kernels from rocprofv3 SQ counters (committed summary,
               null when the kernels changed after it was taken).
  sweep        the other workloads: forward / backward TFLOP/s and the paged
               decode's bandwidth against 8 TB/s (calls rotate over three
               copies of the 311 MB cache so that none finds its K/V in
               MALL; the rate on one copy is reported beside it).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
BUSY_FILE = os.path.join(ROOT, "profiles", "busy_counters.json")
FLUSH_BYTES = 512 << 20     # > L2 (8 x 4 MB) + MALL (256 MB)
DECODE_COPIES = 3           # 3 x 311 MB of paged cache > 2 x MALL


# ---------------------------------------------------------------- IO model --
# FA notes §3.5: standard attention needs Theta(N d + N^2) HBM accesses,
# FlashAttention Theta(N^2 d^2 / M) for on-chip memory of M elements.  The
# bench reports both beside the measured bytes (constants dropped, per head).

def standard_accesses(N, d):
    """Theta(N d + N^2) accesses of standard attention (one head)."""
    return N * d + N * N


def flash_accesses(N, d, M):
    """Theta(N^2 d^2 / M) accesses of the tiled method (one head)."""
    return N * N * d * d / M


def score_matrix_bytes(N, bytes_per_element, matrices=1, heads=1):
    """Size of materialising `matrices` N x N matrices for `heads` heads."""
    return N * N * bytes_per_element * matrices * heads


def compulsory_bytes(w, backward):
    """Bytes every implementation must move: inputs read once, outputs
    written once (fwd: Q,K,V in, O out, m,l out; bwd: Q,K,V,O,dO in,
    dQ,dK,dV out, m,l in)."""
    s = 2 if w.dtype == "bf16" else (1 if w.dtype == "fp8" else 4)
    nd = w.B * w.H * w.N * w.d
    rows = w.B * w.H * w.N
    if backward:
        return s * 8 * nd + 8 * rows
    return s * 4 * nd + 8 * rows


LDS_BYTES_PER_CU = 160 * 1024
THETA_M_ELEMENTS = LDS_BYTES_PER_CU // 2   # on-chip memory M in bf16 elements
QUERY_TILE = 128                           # queries per forward workgroup


def io_block(w, measured):
    """Bytes per forward call: measured (rocprofv3 counters, or None),
    compulsory (every input read once, every output written once), the
    Theta(N^2 d^2 / M) bound of FA notes §3.5 (constants dropped, M = one
    CU's LDS in elements), and the tile-reload model: Q read and O written
    once, all of K and V read once per 128-query tile (half of them under
    the causal mask), i.e. what HBM would see with no cache reuse across
    query tiles.  Halving follows the causal mask's half of the score
    matrix."""
    s = 2 if w.dtype == "bf16" else (1 if w.dtype == "fp8" else 4)
    bh, nd = w.B * w.H, w.N * w.d
    half = 0.5 if w.causal else 1.0
    tiles = -(-w.N // QUERY_TILE)
    return {"unit": "bytes per call", "measured": measured,
            "compulsory": compulsory_bytes(w, False),
            "theta_bound": s * bh * flash_accesses(w.N, w.d,
                                                   THETA_M_ELEMENTS) * half,
            "tile_reload_model": s * bh * (2 * nd + 2 * nd * tiles * half)}


def strip_c_comments(text):
    """C/C++ source without its comments (// and /* */ outside string and
    character literals), each comment replaced by one space, and every run
    of whitespace collapsed to one space: what the compiler sees as tokens."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                       # literal: copy through its end
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash():
    """Hash of what the kernels are built from: the comment-stripped,
    whitespace-normalised sources under csrc/ and the compiler flags.  The
    committed counter summaries are valid only for this hash (a comment edit
    leaves it unchanged; any code or flag change does not)."""
    from exact_io_aware_15_amd import build as fa_build
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_io_aware_15_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(strip_c_comments(f.read()).encode())
    flags = [f for f in fa_build.FLAGS + fa_build.KERNEL_FLAGS
             if not os.path.isabs(f)]       # include paths vary by checkout
    h.update(" ".join(flags).encode())
    for name in sorted(fa_build.SOURCE_FLAGS):
        h.update((name + " " + " ".join(fa_build.SOURCE_FLAGS[name])).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2_medium_causal_4k")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the paged decode (paged_gqa_decode)")
    ap.add_argument("--sweep-only", default=None, metavar="WORKLOAD",
                    help="time only this sweep workload (or "
                         "paged_chunked_prefill) and print its entry")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the comparison timings (cold-cache step, "
                         "single-copy decode): for profiling runs, so that "
                         "every traced dispatch is one the reported rates "
                         "count")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the machine probes (matrix-core loop rate, "
                         "clock under load, streaming read rate)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many "
                         "bytes --steps times (the reference reading that "
                         "scales the HBM byte counters)")
    return ap.parse_args()


class Attn:
    """Device-resident inputs of one attention workload, and its step."""

    def __init__(self, w):
        import torch
        import exact_io_aware_15_amd as fa
        from workloads import to_device
        self.w, self.fa, self.torch = w, fa, torch
        self.varlen = w.kind == "varlen"
        self.fp8 = w.kind == "fp8"
        self.mask = None
        if w.kind == "sparse":
            from workloads import block_sparse_mask
            self.mask = torch.from_numpy(block_sparse_mask(w.H, w.N)).cuda()
        if self.fp8:      # E4M3 codes, V transposed, per-head descales
            q, k, v, qd, kd, vd = w.fp8_inputs()
            self.descales = [torch.from_numpy(x).cuda() for x in (qd, kd, vd)]
            self.do = None
            self.kv_len = None
            nbytes = 1
        elif self.varlen:   # packed ragged batch, [H, total, d]
            cu, q, k, v = w.varlen_inputs()
            self.cu = torch.from_numpy(cu).cuda()
            self.do = to_device(w.varlen_dout())
            nbytes = fa.bwd_varlen_workspace_bytes(w.H, int(cu[-1]), w.d)
            self.kv_len = None
        else:
            q, k, v = w.qkv()
            self.do = to_device(w.dout())
            kl = w.kv_len()
            self.kv_len = None if kl is None else torch.from_numpy(kl).cuda()
            nbytes = (fa.bwd_block_sparse_workspace_bytes(w.B, w.H, w.N, w.d)
                      if self.mask is not None else
                      fa.bwd_workspace_bytes(w.B, w.H, w.N, w.d))
        self.q, self.k, self.v = (to_device(t) for t in (q, k, v))
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8,
                              device="cuda")

    def fwd(self):
        if self.fp8:
            return self.fa.fwd_fp8(self.q, self.k, self.v, *self.descales,
                                   causal=self.w.causal)
        if self.mask is not None:
            return self.fa.fwd_block_sparse(self.q, self.k, self.v, self.mask,
                                            causal=self.w.causal)
        if self.varlen:
            return self.fa.fwd_varlen(self.q, self.k, self.v, self.cu,
                                      self.w.N, causal=self.w.causal)
        if self.w.p_drop > 0:
            return self.fa.fwd_dropout(self.q, self.k, self.v, self.w.p_drop,
                                       self.w.seed, 0, causal=self.w.causal,
                                       kv_len=self.kv_len)
        return self.fa.fwd(self.q, self.k, self.v, causal=self.w.causal,
                           kv_len=self.kv_len)

    def bwd(self, o, m, l):
        if self.mask is not None:
            return self.fa.bwd_block_sparse(self.q, self.k, self.v, o, self.do,
                                            m, l, self.mask,
                                            causal=self.w.causal,
                                            workspace=self.ws)
        if self.varlen:
            return self.fa.bwd_varlen(self.q, self.k, self.v, o, self.do, m,
                                      l, self.cu, self.w.N,
                                      causal=self.w.causal, workspace=self.ws)
        if self.w.p_drop > 0:
            return self.fa.bwd_dropout(self.q, self.k, self.v, o, self.do, m,
                                       l, self.w.p_drop, self.w.seed, 0,
                                       causal=self.w.causal,
                                       kv_len=self.kv_len, workspace=self.ws)
        return self.fa.bwd(self.q, self.k, self.v, o, self.do, m, l,
                           causal=self.w.causal, kv_len=self.kv_len,
                           workspace=self.ws)


def percentiles(ms):
    """p10 / p50 / p90 of a list of durations (nearest rank)."""
    xs = sorted(ms)
    pick = lambda q: xs[min(len(xs) - 1, int(q * len(xs)))]  # noqa: E731
    return {"p10": round(pick(0.1), 4), "p50": round(pick(0.5), 4),
            "p90": round(pick(0.9), 4)}


# Untimed warm-up runs at least W calls and at least this long: the first
# ~15 ms of steady GPU work measure up to 10% slower (clocks and caches
# settle), which five steps of the 4K workload do not cover.
MIN_WARM_S = 0.2


def warm(fn, warmup):
    """Calls fn(i) at least `warmup` times and until MIN_WARM_S of GPU work
    has passed (synchronising every few calls so wall time tracks the GPU);
    returns the number of calls."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < MIN_WARM_S:
        fn(n)
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_step(attn, steps, warmup, backward=True, per_call=None):
    """Run warmup steps, then `steps` timed steps bracketed by one event
    and a synchronisation on each side (the step time), then `steps` more
    with events around each forward and backward call (the split between
    the two and each call's percentiles, filled into per_call if it is a
    dict; those events cost a few microseconds per step, so they stay out
    of the step time).  Returns mean ms of step, fwd and bwd, and the host
    wall time per step of the first loop."""
    torch = attn.torch

    def one(_):
        o, m, l = attn.fwd()
        if backward:
            attn.bwd(o, m, l)
    warm(one, warmup)
    s0, s1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s0.record()
    for _ in range(steps):
        one(None)
    s1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    step_ms = s0.elapsed_time(s1) / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        o, m, l = attn.fwd()
        ev[i][1].record()
        if backward:
            attn.bwd(o, m, l)
        ev[i][2].record()
    torch.cuda.synchronize()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps if backward \
        else 0.0
    if per_call is not None:
        per_call["fwd"] = percentiles([e[0].elapsed_time(e[1]) for e in ev])
        if backward:
            per_call["bwd"] = percentiles([e[1].elapsed_time(e[2])
                                           for e in ev])
    return step_ms, fwd_ms, bwd_ms, wall


def time_cold(torch, calls, reps):
    """Each of `calls` (functions run in order, each given the previous
    one's result) timed `reps` times right after FLUSH_BYTES have been
    read on the same stream; returns the median ms of each."""
    scratch = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)]
           for _ in calls] for _ in range(reps)]
    for i in range(reps):
        prev = None
        for j, fn in enumerate(calls):
            scratch.sum()
            ev[i][j][0].record()
            prev = fn(prev)
            ev[i][j][1].record()
    torch.cuda.synchronize()
    del scratch
    return [percentiles([ev[i][j][0].elapsed_time(ev[i][j][1])
                         for i in range(reps)])["p50"]
            for j in range(len(calls))]


def decode_bench(steps, warmup, splits=None, compare=True):
    """Back-to-back decode calls, rotating over DECODE_COPIES copies of the
    paged cache (a serving step reads each layer's cache once, so no call
    should find its K/V in cache); the same on a single copy is reported
    beside it."""
    import numpy as np
    import torch
    import exact_io_aware_15_amd as fa
    from workloads import to_device
    from workloads import WORKLOADS
    w = WORKLOADS["paged_gqa_decode"]
    q, cache = w.decode_inputs(poison_tails=False)
    qd = to_device(q)
    kcs = [to_device(cache.k_cache) for _ in range(DECODE_COPIES)]
    vcs = [to_device(cache.v_cache) for _ in range(DECODE_COPIES)]
    table = torch.from_numpy(cache.block_table).cuda()
    lens = torch.from_numpy(cache.seq_lens).cuda()
    splits = w.splits if splits is None else splits
    ws = torch.empty(fa.decode_workspace_bytes(w.B, w.H, w.d, splits),
                     dtype=torch.uint8, device="cuda")

    def run(copies):
        warm(lambda i: fa.decode_paged(qd, kcs[i % copies], vcs[i % copies],
                                       table, lens, splits, workspace=ws),
             warmup)
        e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        e0.record()
        for i in range(steps):
            c = i % copies
            fa.decode_paged(qd, kcs[c], vcs[c], table, lens, splits,
                            workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    ms = run(DECODE_COPIES)
    same_ms = run(1) if compare else None
    total_len = int(np.sum(cache.seq_lens))
    # K and V rows read: len * Hkv * d * 2 bytes each
    kv_bytes = total_len * w.Hkv * w.d * 2 * 2
    gbs = kv_bytes / ms / 1e6
    return {"workload": w.name, "num_splits": splits, "ms": round(ms, 4),
            "kv_bytes": kv_bytes,
            "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "cache_copies": DECODE_COPIES,
            "same_copy": None if same_ms is None else {
                "ms": round(same_ms, 4),
                "GB/s": round(kv_bytes / same_ms / 1e6, 1),
                "note": "back-to-back on one copy: part of the K/V is "
                        "still in MALL"},
            "roofline": {"kernel": "fa_decode_paged (decode_split_kernel + "
                                   "decode_merge_kernel launches)",
                         "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic_for("fa_decode_paged")},
            "limiter": busy_counters(w.name)}


def prefill_bench(steps, warmup):
    """fa_prefill_paged on the chunked-prefill workload: TFLOP/s at
    4*Hq*d per (new token, visible cached key)."""
    import torch
    import exact_io_aware_15_amd as fa
    from workloads import WORKLOADS, to_device
    w = WORKLOADS["paged_chunked_prefill"]
    cu, q, cache = w.prefill_inputs(poison_tails=False)
    qd = to_device(q)
    kc, vc = to_device(cache.k_cache), to_device(cache.v_cache)
    table = torch.from_numpy(cache.block_table).cuda()
    lens = torch.from_numpy(cache.seq_lens).cuda()
    cud = torch.from_numpy(cu).cuda()

    def call():
        return fa.prefill_paged(qd, kc, vc, table, lens, cud,
                                w.seq_range[1], causal=True)
    warm(lambda _: call(), warmup)
    e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tf = w.prefill_flops() / ms / 1e9
    return {"workload": w.name, "ms": round(ms, 4), "tflops": round(tf, 1),
            "frac": round(tf / PEAK_BF16_TFLOPS, 4)}


SWEEP = ["bert_large_padded", "gpt2_medium_causal_1k", "long_causal_16k_d128",
         "long_causal_64k_d64", "varlen_causal_prefill", "block_sparse_16k",
         "gpt2_medium_causal_4k_dropout", "long_causal_16k_d128_fp8"]


def sweep_one(name, steps, warmup, out):
    """Times one sweep workload (forward, and backward where it has one);
    comparisons refer to entries already in `out`."""
    import dataclasses
    from workloads import WORKLOADS
    w = WORKLOADS[name]
    attn = Attn(w)
    step_ms, fwd_ms, bwd_ms, _ = time_step(attn, steps, warmup,
                                           backward=w.backward)
    r = {"fwd_ms": round(fwd_ms, 4),
         "fwd_tflops": round(w.fwd_flops() / fwd_ms / 1e9, 1)}
    r["fwd_frac"] = round(r["fwd_tflops"] / PEAK_BF16_TFLOPS, 4)
    if w.backward:
        r["bwd_ms"] = round(bwd_ms, 4)
        r["bwd_tflops"] = round(w.bwd_flops() / bwd_ms / 1e9, 1)
        r["bwd_frac"] = round(r["bwd_tflops"] / PEAK_BF16_TFLOPS, 4)
    eff = effective_fraction(w)
    if eff is not None:   # key padding: FLOPs of the valid (query, key) pairs
        r["valid_pair_fraction"] = round(eff, 4)
        r["fwd_tflops_effective"] = round(r["fwd_tflops"] * eff, 1)
        if w.backward:
            r["bwd_tflops_effective"] = round(r["bwd_tflops"] * eff, 1)
    if w.kind == "attn":
        r["io"] = io_block(w, traffic_for(f"fa_fwd:{name}"))
    if w.kind == "fp8":   # against the bf16 forward of the same shape
        r["fwd_frac_of_fp8_peak"] = round(r["fwd_tflops"] / PEAK_FP8_TFLOPS,
                                          4)
        bf = out.get("long_causal_16k_d128")
        if bf is not None:
            r["speedup_vs_bf16_fwd"] = round(bf["fwd_ms"] / fwd_ms, 2)
    if w.p_drop > 0:   # the same inputs without dropout
        plain = Attn(dataclasses.replace(w, p_drop=0.0))
        _, pfwd, pbwd, _ = time_step(plain, steps, warmup, backward=True)
        r["no_dropout_fwd_ms"] = round(pfwd, 4)
        r["no_dropout_bwd_ms"] = round(pbwd, 4)
        r["dropout_cost_fwd"] = round(fwd_ms / pfwd, 3)
        r["dropout_cost_bwd"] = round(bwd_ms / pbwd, 3)
        del plain
    if w.kind == "sparse":   # the same shape without the mask
        dense = Attn(dataclasses.replace(w, kind="attn"))
        _, dfwd, dbwd, _ = time_step(dense, steps, warmup, backward=True)
        r["dense_fwd_ms"] = round(dfwd, 4)
        r["dense_bwd_ms"] = round(dbwd, 4)
        r["speedup_fwd"] = round(dfwd / fwd_ms, 2)
        r["speedup_bwd"] = round(dbwd / bwd_ms, 2)
        del dense
    r["limiter"] = busy_counters(name)
    out[name] = r
    del attn
    return r


def effective_fraction(w):
    """Share of the nominal N x N (query, key) pairs that key padding leaves
    valid (None without padding): sum_b N * kv_len_b / (B * N^2)."""
    import numpy as np
    kl = w.kv_len() if w.kind == "attn" else None
    if kl is None:
        return None
    return float(np.sum(np.asarray(kl, np.float64))) / (w.B * w.N)


def sweep(steps, warmup):
    out = {}
    for name in SWEEP:
        sweep_one(name, steps, warmup, out)
    out["paged_gqa_decode"] = decode_bench(max(steps, 20), warmup)
    out["paged_chunked_prefill"] = prefill_bench(max(steps, 20), warmup)
    return out


def cpu_baseline(w, budget_s):
    """fp64 oracle forward + backward on whole heads of the workload until
    about budget_s seconds have been spent; TFLOP/s at the workload's
    algorithmic FLOP count per head."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    q, k, v = w.qkv()
    do = w.dout()
    kl = w.kv_len()
    per_head = (w.fwd_flops() + w.bwd_flops()) / (w.B * w.H)
    t0 = time.perf_counter()
    heads = 0
    while True:
        b, h = divmod(heads % (w.B * w.H), w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        klb = None if kl is None else kl[b:b + 1]
        oracle.attention_fwd(q.exact[sl], k.exact[sl], v.exact[sl], None,
                             w.causal, klb)
        oracle.attention_bwd(q.exact[sl], k.exact[sl], v.exact[sl],
                             do.exact[sl], None, w.causal, klb)
        heads += 1
        el = time.perf_counter() - t0
        if el >= budget_s or heads >= w.B * w.H:
            break
    blas, _ = _blas_info()
    return {"value": round(per_head * heads / el / 1e12, 6),
            "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd on {heads} of {w.B * w.H} heads "
                      f"of {w.name} ({el:.1f} s)",
            "os_cpu_count": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas": blas}


def _blas_info():
    """Name and thread count of the BLAS numpy uses."""
    import numpy as np
    name = None
    try:
        cfg = np.show_config(mode="dicts")
        name = cfg.get("Build Dependencies", {}).get("blas", {}).get("name")
    except Exception:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        pass
    return name, threads


def _visible_pairs(rows, n_keys, causal, kv):
    """(query, key) pairs the rows see: keys < kv, and <= the row if causal."""
    import numpy as np
    rows = np.asarray(rows, np.int64)
    vis = np.full(rows.shape, min(kv, n_keys), np.int64)
    if causal:
        vis = np.minimum(vis, rows + 1)
    return int(vis.sum())


def cpu_baseline_configs(budget_s):
    """The fp64 oracle on a bounded sample of every configuration, each for
    about budget_s / 8 seconds: the forward of each attention workload on
    chunks of 256 rows of its heads in turn (causal rows see their prefix),
    the backward of the three fwd+bwd workloads on whole heads in turn, and
    the paged decode on its sequences in turn (a sample shorter than the
    budget is repeated).  Rates use the algorithmic counts of the sample
    (4 d FLOP per visible pair forward, 10 d backward; K and V bytes read
    for the decode)."""
    import numpy as np
    import oracle
    from workloads import WORKLOADS
    per = budget_s / 8
    out = {}
    for name in ("tiny_f32", "bert_large_padded", "gpt2_medium_causal_1k",
                 "gpt2_medium_causal_4k", "long_causal_16k_d128",
                 "long_causal_64k_d64"):
        w = WORKLOADS[name]
        q, k, v = w.qkv()
        kl = w.kv_len()
        heads = w.B * w.H
        step = min(w.N, 256)
        chunks = -(-w.N // step)
        t0, it, pairs = time.perf_counter(), 0, 0
        while True:   # chunk `it % chunks` of head `it // chunks % heads`
            b, h = divmod(it // chunks % heads, w.H)
            kv = w.N if kl is None else int(kl[b])
            r0 = (it % chunks) * step
            rows = np.arange(r0, min(w.N, r0 + step))
            sl = (slice(b, b + 1), slice(h, h + 1))
            oracle.attention_fwd(q.exact[sl], k.exact[sl], v.exact[sl], None,
                                 w.causal, None if kl is None else kl[b:b + 1],
                                 rows=rows)
            pairs += _visible_pairs(rows, w.N, w.causal, kv)
            it += 1
            if time.perf_counter() - t0 >= per:
                break
        el = time.perf_counter() - t0
        e = {"fwd_tflops": round(4 * w.d * pairs / el / 1e12, 6),
             "fwd_sample": f"{it} chunks of up to {step} rows over "
                           f"{min(heads, -(-it // chunks))} of {heads} heads "
                           f"({el:.2f} s)"}
        if w.backward:
            do = w.dout()
            t0, nh, pairs = time.perf_counter(), 0, 0
            while True:
                b, h = divmod(nh % heads, w.H)
                kv = w.N if kl is None else int(kl[b])
                sl = (slice(b, b + 1), slice(h, h + 1))
                oracle.attention_bwd(q.exact[sl], k.exact[sl], v.exact[sl],
                                     do.exact[sl], None, w.causal,
                                     None if kl is None else kl[b:b + 1])
                pairs += _visible_pairs(np.arange(w.N), w.N, w.causal, kv)
                nh += 1
                if time.perf_counter() - t0 >= per:
                    break
            el = time.perf_counter() - t0
            e["bwd_tflops"] = round(10 * w.d * pairs / el / 1e12, 6)
            e["bwd_sample"] = f"{nh} whole heads ({el:.2f} s)"
        out[name] = e
    w = WORKLOADS["paged_gqa_decode"]
    q, cache = w.decode_inputs(poison_tails=False)
    t0, it = time.perf_counter(), 0
    kv_bytes = 0
    while True:
        nb = it % w.B
        oracle.decode_paged(q.exact[nb:nb + 1], cache.k_cache.exact,
                            cache.v_cache.exact, cache.block_table[nb:nb + 1],
                            cache.seq_lens[nb:nb + 1])
        kv_bytes += int(cache.seq_lens[nb]) * w.Hkv * w.d * 2 * 2
        it += 1
        if time.perf_counter() - t0 >= per:
            break
    el = time.perf_counter() - t0
    out["paged_gqa_decode"] = {"GB/s": round(kv_bytes / el / 1e9, 4),
                               "sample": f"{it} sequence decodes over "
                                         f"{min(it, w.B)} of {w.B} sequences "
                                         f"({el:.2f} s)"}
    return out


def machine_probe():
    """Measured context for the roofline fractions: a pure bf16 MFMA loop on
    every SIMD (attainable matrix-core rate, and the engine clock while it
    runs) and a streaming read of 1 GiB (practical HBM read rate)."""
    from exact_io_aware_15_amd import probe
    tf, ghz, sec = probe.mfma_bf16(iters=120000, waves_per_simd=4)
    gbs = probe.read_bw(1 << 30, 5)
    return {"mfma_bf16_tflops": round(tf, 1), "clock_ghz_under_mfma":
            round(ghz, 3), "mfma_loop_s": round(sec, 4),
            "read_gbs": round(gbs, 1),
            "note": "mfma: 4 independent v_mfma_f32_32x32x16_bf16 chains "
                    "per wave, 4 waves per SIMD, ~30 ms; read: grid-stride "
                    "16-byte non-temporal loads over 1 GiB, best of 5 launch "
                    "shapes"}


def busy_counters(workload):
    """Per-kernel fractions of the cycles in which the matrix cores were
    busy, the VALU was issuing, and both at once, from the committed SQ
    counter summary of `workload`, if it was taken on the current kernel
    sources (else None)."""
    try:
        with open(BUSY_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("workloads", {}).get(workload)


def traffic_for(call):
    """HBM bytes per call from the committed counter summary, if it was
    taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("calls", {}).get(call)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the attention kernels would shard over independent "
              "(batch, head) units, but multi-GPU runs are not supported.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_bytes > 0:
        x = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(args.steps):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "steps": args.steps}))
        return
    if args.decode_only:
        print(json.dumps(decode_bench(args.steps, args.warmup,
                                      compare=not args.no_compare)),
              flush=True)
        return
    if args.sweep_only:
        if args.sweep_only == "paged_chunked_prefill":
            r = prefill_bench(args.steps, args.warmup)
        else:
            r = sweep_one(args.sweep_only, args.steps, args.warmup, {})
        print(json.dumps({args.sweep_only: r}), flush=True)
        return
    machine = None if args.no_probe else machine_probe()
    w = WORKLOADS[args.workload]
    attn = Attn(w)
    per_call = {}
    step_ms, fwd_ms, bwd_ms, wall_ms = time_step(attn, args.steps,
                                                 args.warmup,
                                                 per_call=per_call)
    cold = None
    if not args.no_compare:
        cf, cb = time_cold(
            torch, [lambda _: attn.fwd(), lambda oml: attn.bwd(*oml)],
            max(10, args.steps // 2))
        cold = {"fwd_ms_p50": round(cf, 4), "bwd_ms_p50": round(cb, 4),
                "fwd_tflops": round(w.fwd_flops() / cf / 1e9, 1),
                "bwd_tflops": round(w.bwd_flops() / cb / 1e9, 1),
                "note": f"{FLUSH_BYTES >> 20} MiB read before each call"}
    flops = w.fwd_flops() + w.bwd_flops()
    value = flops / step_ms / 1e9
    if bwd_ms >= fwd_ms:
        call, dur, cflops = "fa_bwd", bwd_ms, w.bwd_flops()
        kern = ("fa_bwd (bwd_pre_kernel, then bwd_fused_kernel: the dK/dV "
                "and dQ workgroups in one launch)")
    else:
        call, dur, cflops = "fa_fwd", fwd_ms, w.fwd_flops()
        kern = "fa_fwd (fwd_bf16_kernel)"
    achieved = cflops / dur / 1e9
    line = {
        # value: TFLOP/s of the fwd+bwd step at the headline shape; the
        # fraction of the bf16 peak is frac_of_bf16_peak, and the other
        # lengths from 1K to 16K are in "sweep".
        "metric": ("attention fwd+bwd TFLOP/s and % of bf16 MFMA peak at "
                   "N=1K\u201316K (1 GPU)"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": MIN_WARM_S,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, no datasets or weights)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N,
                   "d": w.d, "causal": w.causal, "dtype": w.dtype,
                   "fwd_flops": w.fwd_flops(), "bwd_flops": w.bwd_flops()},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd": {"ms": round(fwd_ms, 4), **per_call["fwd"],
                "tflops": round(w.fwd_flops() / fwd_ms / 1e9, 1)},
        "bwd": {"ms": round(bwd_ms, 4), **per_call["bwd"],
                "tflops": round(w.bwd_flops() / bwd_ms / 1e9, 1)},
        "cold_cache": cold,
        "limiter": busy_counters(w.name),
        "host_wall_ms_per_step": round(wall_ms, 4),
        "roofline": {"kernel": kern, "bound": "mfma",
                     "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for(call),
                     "measured_mfma_peak": None if machine is None else
                     machine["mfma_bf16_tflops"],
                     "frac_of_measured_mfma_peak": None if machine is None
                     else round(achieved / machine["mfma_bf16_tflops"], 4),
                     "clock_ghz_measured": None if machine is None else
                     machine["clock_ghz_under_mfma"]},
        "machine": machine,
        "kernel_source_hash": source_hash(),
        "io": {
            "unit": "bytes per call",
            "fa_bwd_measured": traffic_for("fa_bwd"),
            "fa_bwd_compulsory": compulsory_bytes(w, True),
            "fa_fwd_measured": traffic_for("fa_fwd"),
            "fa_fwd_compulsory": compulsory_bytes(w, False),
            # Theta(N^2 d^2 / M) per head x B*H heads (halved when causal),
            # M = one CU's LDS in bf16 elements; constants dropped
            "fwd_theta_bound": (w.B * w.H * 2 * flash_accesses(
                w.N, w.d, LDS_BYTES_PER_CU // 2) * (0.5 if w.causal else 1)),
            "standard_theta": w.B * w.H * 2 * standard_accesses(w.N, w.d),
            "materialised_scores_fp32": score_matrix_bytes(
                w.N, 4, 1, w.B * w.H),
        },
    }
    del attn
    if not args.no_sweep:
        line["sweep"] = sweep(max(10, args.steps // 2), args.warmup)
        dec = line["sweep"]["paged_gqa_decode"]["roofline"]
        if machine is not None:
            dec["measured_read_ceiling"] = machine["read_gbs"]
            dec["frac_of_measured_read_ceiling"] = round(
                dec["achieved"] / machine["read_gbs"], 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        line["cpu_baseline"]["configs"] = cpu_baseline_configs(
            args.cpu_seconds * 1.5)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
