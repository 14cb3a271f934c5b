"""Benchmark: fp8 paged decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one call of the library (decode kernel, plus the log-sum-exp merge
kernel when the plan splits) over one batch already resident in HBM.  The
default workload is 40 query / 8 kv heads, head_dim 128, 256 sequences of
4096 tokens, fp8-e4m3fn K/V in 16-token blocks with a shuffled block table
(2.15 GB of K/V per call, far beyond the 256 MB Infinity Cache, so every call
streams from HBM).

Prints one JSON line: achieved algorithmic HBM GB/s (value: the bytes of one
call over the timed region's time per call, i.e. whole-job throughput; the
region's calls run back to back between two HIP events on the stream the
kernels run on), the per-call median and mean (a second, untimed loop with an
event pair around each call), the median of graph replays (five runs of ten
replays of ten calls back to back, after six untimed runs: the pages' timing
method), the roofline object for the decode kernel (its average launch
duration: the region's time per call, one launch a call; counter traffic from
the committed rocprofv3 summary when it matches the current kernel source),
and the fp64 CPU oracle timed on bounded samples (median of three, all host
cores and one core).  Before the warm-up calls, untimed calls run for
--settle-ms (100 ms): the first calls after the inputs are generated run
slower (the kernel trace shows the first at ~400 µs and the next twenty ~2%
above the rest).

Other modes:
    --workload all          also print one line per workload of the suite to stderr
                            (decode workloads, and the fp8 cache write for a decode step
                            and for a prefill-sized batch)
    --copy-calibration      time a plain 1 GiB device copy (for scaling PMC counters)
    --read-ceiling          the bandwidth plain reads reach: a streaming read of 2 GiB
                            (several grid sizes, with and without the streaming hint)
                            and the decode's page-gather reads alone on the target
                            workload (libpa_probe.so)
    --valu-compare          the decode (MFMA for qKᵀ and PV) against the same decode with
                            its dot products on the vector ALUs (libpa_probe.so), per call,
                            on the target and on 32/8, 32/4 and 8/1 heads at ctx 4096 x 256
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention µs/call and achieved HBM GB/s (% of MI355X peak)"
PEAK_GBS = 8000.0          # MI355X HBM3E, AMD's published peak
PAGES_ASM_US = 363.04      # pa_fwd_asm, 40/8 ctx 4096 256 seqs, MI355X (the pages' table)
PAGES_HIP_US = 448.27      # ROCM_ATTN HIP paged attention, same row
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pa_decode_kernel_40x8_ctx4096_s256_pmc.md")
KERNEL_SRC = os.path.join(ROOT, "paged_attention_decode_03_amd", "csrc", "pa_decode_kernels.hip")


def kernel_source_hash() -> str:
    """sha256 (16 hex digits) of the decode kernel's source with // comments
    and blank lines removed, so that comment edits keep counter data valid."""
    code = []
    with open(KERNEL_SRC, encoding="utf-8") as f:
        for line in f:
            line = line.split("//", 1)[0].rstrip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def counter_traffic():
    """HBM bytes per launch from the committed PMC summary, or None when the
    summary is missing or was taken on a different kernel source."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    h = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def make_workload(name, device):
    import workloads
    if name.endswith("_lpt") and not name.startswith("ragged_"):
        # any workload of the suite with longest-first dispatch
        case = make_workload(name[:-4], device)
        case.longest_first = True
        case.name = name
        return case
    if name == "target":
        hq, hkv, s, ctx = workloads.TARGET
        return workloads.dense(hq, hkv, s, ctx, seed=0, device=device)
    m = re.fullmatch(r"dense_(\d+)x(\d+)_ctx(\d+)_s(\d+)", name)
    if m:
        hq, hkv, ctx, s = map(int, m.groups())
        return workloads.dense(hq, hkv, s, ctx, seed=0, device=device)
    m = re.fullmatch(r"slotscales_(\d+)x(\d+)_ctx(\d+)_s(\d+)", name)
    if m:
        hq, hkv, ctx, s = map(int, m.groups())
        return workloads.make_case(hq, hkv, [ctx] * s, seed=0, device=device, scale_mode="per_slot",
                                   name=name)
    m = re.fullmatch(r"tokenrows_(nhd|combined|packed)_(\d+)x(\d+)_ctx(\d+)_s(\d+)", name)
    if m:
        layout = m.group(1)
        hq, hkv, ctx, s = map(int, m.groups()[1:])
        case = workloads.dense(hq, hkv, s, ctx, seed=0, device=device)
        case.token_rows = workloads.token_row_views(case, layout)
        return case
    m = re.fullmatch(r"specdec_(\d+)x(\d+)_ctx(\d+)_s(\d+)_q(\d+)", name)
    if m:
        hq, hkv, ctx, s, ql = map(int, m.groups())
        return workloads.make_multi_case(hq, hkv, [ctx] * s, [ql] * s, seed=0, device=device,
                                         name=name)
    m = re.fullmatch(r"mixed_(\d+)x(\d+)_s(\d+)(?:_qmax(\d+))?", name)
    if m:
        # decode rows next to short prefill chunks and drafts: contexts uniform in
        # [1, 4000]; 60% of the sequences have one query, the rest 2..5, 8 or 16
        # (with _qmaxN: those up to N)
        import numpy as np
        hq, hkv, s = map(int, m.groups()[:3])
        qmax = int(m.group(4) or 16)
        lens = workloads.ragged_lens(s, seed=3)
        g = np.random.default_rng(81)
        ql = np.where(g.random(s) < 0.6, 1, g.choice([c for c in (2, 3, 4, 5, 8, 16) if c <= qmax], size=s))
        ql = np.minimum(ql, lens).tolist()
        return workloads.make_multi_case(hq, hkv, lens, ql, seed=81, max_blocks=250, device=device,
                                         name=name)
    m = re.fullmatch(r"unified_(\d+)x(\d+)_ctx(\d+)_s(\d+)(?:_q(\d+))?_([a-z0-9+]+)", name)
    if m:
        # the unified call's options: window<N>, softcap<C>, alibi, sinks, joined by '+'
        hq, hkv, ctx, s = map(int, m.groups()[:4])
        ql = int(m.group(5) or 0)
        if ql:
            case = workloads.make_multi_case(hq, hkv, [ctx] * s, [ql] * s, seed=0, device=device,
                                             name=name)
        else:
            case = workloads.dense(hq, hkv, s, ctx, seed=0, device=device)
        import torch
        opts = {}
        for part in m.group(6).split("+"):
            if part.startswith("window"):
                opts["sliding_window"] = int(part[6:])
            elif part.startswith("softcap"):
                opts["softcap"] = float(part[7:])
            elif part == "alibi":
                opts["alibi_slopes"] = (2.0 ** (-8.0 * (torch.arange(hq, device=device) + 1) / hq)).float()
            elif part == "sinks":
                opts["sinks"] = torch.linspace(-1.0, 2.0, hq, device=device)
            else:
                raise SystemExit(f"unknown option {part} in {name}")
        case.meta["options"] = opts
        case.name = name
        return case
    m = re.fullmatch(r"ragged_(\d+)x(\d+)_seed(\d+)(_lpt)?", name)
    if m:
        hq, hkv, seed = map(int, m.groups()[:3])
        case = workloads.ragged(hq, hkv, seed, device=device)
        case.longest_first = m.group(4) is not None
        case.name = name
        return case
    raise SystemExit(f"unknown workload {name}")


def suite_names():
    import workloads
    names = [f"dense_{a}x{b}_ctx{c}_s{s}"
             for (a, b, s, c) in workloads.DENSE_1K + workloads.DENSE_4K + workloads.PAGES_TABLE_EXTRA]
    names += ["target", "dense_20x4_ctx4096_s256"]
    names += ["slotscales_40x8_ctx4096_s256"]
    names += [f"specdec_40x8_ctx4096_s256_q{q}" for q in (2, 3, 4, 8)]
    names += ["mixed_40x8_s256", "mixed_40x8_s256_lpt", "mixed_40x8_s256_qmax8", "mixed_40x8_s256_qmax8_lpt"]
    names += [f"tokenrows_{lay}_40x8_ctx4096_s256" for lay in ("nhd", "combined", "packed")]
    names += ["tokenrows_nhd_40x8_ctx4096_s64", "tokenrows_nhd_40x8_ctx1024_s16"]
    names += ["unified_40x8_ctx4096_s256_" + o for o in ("window1024", "softcap30", "alibi", "sinks")]
    names += ["unified_40x8_ctx4096_s256_q4_window128+sinks"]
    names += [f"ragged_{a}x{b}_seed0" for (a, b) in workloads.RAGGED_LAYOUTS]
    names += [f"ragged_{a}x{b}_seed0_lpt" for (a, b) in workloads.RAGGED_LAYOUTS]
    names += [f"dense_{a}x{b}_ctx{c}_s{s}" for (a, b, s, c) in workloads.LOW_BATCH]
    return names


def workload_bytes(case):
    """Algorithmic bytes of one call; with a sliding window, only the K/V of
    the tokens some query's window holds (and their table entries), plus the
    option arrays."""
    b = case.algorithmic_bytes()
    opts = case.meta.get("options")
    if not opts:
        return b
    import torch
    lens = case.seq_lens.to(torch.int64).cpu()
    win = opts.get("sliding_window", 0)
    if win > 0:
        cu = case.cu_seqlens_q
        ql = torch.ones_like(lens) if cu is None else (cu[1:] - cu[:-1]).to(torch.int64).cpu()
        seen = torch.minimum(lens, win + ql - 1)           # tokens the union of the windows covers
        b -= case.kv_bytes()
        b += int(seen.sum().item()) * case.num_kv_heads * 128 * 2
        pages_all = (lens + 15) // 16
        pages_seen = pages_all - (lens - seen) // 16
        b -= int((pages_all - pages_seen).sum().item()) * 4
    b += 4 * case.num_heads * sum(1 for k in ("alibi_slopes", "sinks") if opts.get(k) is not None)
    return b


def make_call(case, out, stream=None):
    """One call of the entry point that serves `case` (per-tensor scales, per-slot
    scales, token rows, longest-first dispatch, or several queries per
    sequence), writing `out`."""
    import torch
    import paged_attention_decode_03_amd as pa
    dev = case.q.device
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device=dev)
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device=dev)
    if case.k_slot_scales is not None:
        return lambda: pa.paged_decode_attention_slot_scales(
            case.q, case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.scale,
            case.k_slot_scales, case.v_slot_scales, out=out, stream=stream)
    if getattr(case, "token_rows", None) is not None:
        kv, vv = case.token_rows
        return lambda: pa.paged_decode_attention_nhd(case.q, kv, vv, case.block_tables,
                                                     case.seq_lens, case.scale, ks, vs, out=out,
                                                     stream=stream)
    opts = case.meta.get("options")
    if opts is not None:
        cu = case.cu_seqlens_q
        max_q = 1 if cu is None else int((cu[1:] - cu[:-1]).max().item())
        return lambda: pa.paged_attention_unified(case.q, cu, max_q, case.k_cache, case.v_cache,
                                                  case.block_tables, case.seq_lens, case.scale, ks,
                                                  vs, out=out, stream=stream, **opts)
    if getattr(case, "longest_first", False):
        cu = case.cu_seqlens_q
        max_q = 1 if cu is None else int((cu[1:] - cu[:-1]).max().item())
        return lambda: pa.paged_attention_unified(case.q, cu, max_q, case.k_cache, case.v_cache,
                                                  case.block_tables, case.seq_lens, case.scale, ks,
                                                  vs, longest_first=True, out=out, stream=stream)
    if case.cu_seqlens_q is not None:
        max_q = int((case.cu_seqlens_q[1:] - case.cu_seqlens_q[:-1]).max().item())
        return lambda: pa.paged_multi_query_attention(
            case.q, case.cu_seqlens_q, max_q, case.k_cache, case.v_cache, case.block_tables,
            case.seq_lens, case.scale, ks, vs, out=out, stream=stream)
    return lambda: pa.paged_decode_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                                             case.seq_lens, case.scale, ks, vs, out=out,
                                             stream=stream)


def time_calls(case, steps, warmup, per_call=False, settle_ms=0.0):
    """µs per call over the timed region: `steps` calls back to back between
    two HIP events recorded on the stream the kernels run on, after
    `warmup` untimed calls (and, with settle_ms, untimed calls for at least
    that long before them: the first calls after the inputs are generated run
    slower).  With per_call, also a second, untimed loop of `steps` calls,
    each between its own event pair (events between calls delay the next
    launch, so they stay out of the timed region); returns (region µs,
    per-call µs list, settle calls)."""
    import torch
    dev = case.q.device
    out = torch.empty_like(case.q)
    stream = torch.cuda.Stream(dev)
    call = make_call(case, out, stream)
    settled = 0
    if settle_ms > 0:
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < settle_ms:
            for _ in range(8):
                call()
            settled += 8
            torch.cuda.synchronize(dev)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize(dev)
    region = start.elapsed_time(end) * 1e3 / steps
    if not per_call:
        return region
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for a, b in pairs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize(dev)
    return region, [a.elapsed_time(b) * 1e3 for a, b in pairs], settled


COLD_MIN_BYTES = 512 << 20   # twice the 256 MB Infinity Cache
COLD_MAX_RESIDENT = 16 << 30


def cold_copies(case):
    """Copies of `case` in distinct device buffers, enough that the calls of one
    round over them touch at least COLD_MIN_BYTES, so a call finds none of its
    inputs left in the Infinity Cache by the previous ones.  [case] when the
    workload already touches that much (or its layout is a view of a larger
    tensor: token rows)."""
    import copy
    import torch
    touched = workload_bytes(case)
    if touched >= COLD_MIN_BYTES or getattr(case, "token_rows", None) is not None:
        return [case]
    resident = sum(t.numel() * t.element_size() for t in vars(case).values()
                   if isinstance(t, torch.Tensor))
    k = -(-COLD_MIN_BYTES // touched)
    k = max(2, min(k, COLD_MAX_RESIDENT // max(resident, 1)))
    out = [case]
    for _ in range(k - 1):
        c = copy.copy(case)
        for name, t in vars(case).items():
            if isinstance(t, torch.Tensor):
                setattr(c, name, t.clone())
        out.append(c)
    return out


def time_calls_cold(case, steps, warmup):
    """Average µs per call over calls that rotate through cold_copies(case)
    (each with its own output), HIP events on the launch stream: the
    cold-cache figure of a workload smaller than twice the Infinity Cache."""
    import torch
    dev = case.q.device
    cases = cold_copies(case)
    stream = torch.cuda.Stream(dev)
    calls = [make_call(c, torch.empty_like(c.q), stream) for c in cases]
    for i in range(max(warmup, len(calls))):
        calls[i % len(calls)]()
    torch.cuda.synchronize(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        calls[i % len(calls)]()
    end.record(stream)
    torch.cuda.synchronize(dev)
    us = start.elapsed_time(end) * 1e3 / steps
    del calls, cases
    return us


def time_graph(case, replays=50, calls_per_graph=10, per_replay=False):
    """Average µs per call when `calls_per_graph` calls are captured in one HIP
    graph and the graph is replayed (the way the pages time impl.forward);
    with per_replay, also the µs per call of each replay (events around it)."""
    import torch
    dev = case.q.device
    out = torch.empty_like(case.q)
    call = make_call(case, out)
    stream = torch.cuda.Stream(dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        for _ in range(3):
            call()          # sizes the capture stream's split-KV scratch
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(calls_per_graph):
            call()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(replays if per_replay else 0)]
    start.record()
    for i in range(replays):
        if per_replay:
            pairs[i][0].record()
        g.replay()
        if per_replay:
            pairs[i][1].record()
    end.record()
    torch.cuda.synchronize(dev)
    mean = start.elapsed_time(end) * 1e3 / (replays * calls_per_graph)
    if not per_replay:
        return mean
    return mean, [a.elapsed_time(b) * 1e3 / calls_per_graph for a, b in pairs]


def cache_write_case(num_tokens, num_kv_heads=8, seed=0, pattern="prefill"):
    """New keys/values (bf16 N(0,1), per-tensor scale amax/448) for `num_tokens`
    tokens.  pattern "prefill": sequences of 2048 new tokens, each filling its
    own shuffled blocks in order; "chunks": prefill chunks of 1..4095 tokens
    (about 2048 on average) that each continue a sequence at a random slot of
    its last block (chunked prefill, prefix caching); "decode": one token per
    sequence at a random slot (a decode step).  The cache has 25% spare
    blocks."""
    import numpy as np
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    nb = (num_tokens + 15) // 16 * 5 // 4 + 1
    key = torch.randn(num_tokens, num_kv_heads, 128, generator=g, device="cuda").to(torch.bfloat16)
    value = torch.randn(num_tokens, num_kv_heads, 128, generator=g, device="cuda").to(torch.bfloat16)
    if pattern == "prefill":
        blocks = torch.randperm(nb, generator=g, device="cuda")[:(num_tokens + 15) // 16]
        t = torch.arange(num_tokens, device="cuda")
        slots = blocks[t // 16] * 16 + t % 16
    elif pattern == "chunks":
        rng = np.random.default_rng(seed + 17)
        lens, starts = [], []
        while sum(lens) < num_tokens:
            lens.append(int(min(rng.integers(1, 4096), num_tokens - sum(lens))))
            starts.append(int(rng.integers(0, 16)))
        nb = sum((a + n + 15) // 16 for a, n in zip(starts, lens)) * 5 // 4 + 1
        perm = torch.randperm(nb, generator=g, device="cuda")
        parts, b = [], 0
        for a, n in zip(starts, lens):
            k = (a + n + 15) // 16
            t = torch.arange(n, device="cuda") + a
            parts.append(perm[b:b + k][t // 16] * 16 + t % 16)
            b += k
        slots = torch.cat(parts)
    else:
        slots = torch.randperm(nb * 16, generator=g, device="cuda")[:num_tokens]
    slots = slots.to(torch.int64)
    k_cache = torch.zeros(nb, num_kv_heads, 8, 16, 16, dtype=torch.uint8, device="cuda")
    v_cache = torch.zeros(nb, num_kv_heads, 128, 16, dtype=torch.uint8, device="cuda")
    ks = (key.float().abs().max() / 448).reshape(1)
    vs = (value.float().abs().max() / 448).reshape(1)
    return key, value, k_cache, v_cache, slots, ks, vs


def cache_write_bytes(num_tokens, num_kv_heads=8):
    """Algorithmic bytes of one cache write: bf16 key and value in, fp8 key and
    value out, the int64 slots and the two scales."""
    return num_tokens * num_kv_heads * 128 * (2 + 2 + 1 + 1) + 8 * num_tokens + 8


def time_cache_write(num_tokens, steps, warmup, num_kv_heads=8, pattern="prefill"):
    import torch
    import paged_attention_decode_03_amd as pa
    key, value, kc, vc, slots, ks, vs = cache_write_case(num_tokens, num_kv_heads, pattern=pattern)
    stream = torch.cuda.Stream()
    for _ in range(warmup):
        pa.paged_kv_cache_write(key, value, kc, vc, slots, ks, vs, stream=stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        pa.paged_kv_cache_write(key, value, kc, vc, slots, ks, vs, stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / steps


def cpu_baseline(target_seconds=4.0, max_seqs=256):
    """The fp64 oracle as it stands, on bounded samples of the same workload:
    on every host core (os.cpu_count() threads), the median of three runs of
    as many sequences as about target_seconds of work allow (a multiple of 4
    up to the workload's 256, sized by a first run of 4); and the same on one
    core, on a sample sized the same way.  Reported in the metric's unit
    (algorithmic GB/s of the sample)."""
    import statistics
    import oracle
    import workloads
    hq, hkv, _, ctx = workloads.TARGET
    cores = os.cpu_count() or 1

    def run(n, threads):
        case = workloads.dense(hq, hkv, n, ctx, seed=1, device="cpu")
        args = (case.q_bits(), case.k_cache.numpy(), case.v_cache.numpy(), case.block_tables.numpy(),
                case.seq_lens.numpy(), case.scale, case.k_scale, case.v_scale)
        t0 = time.perf_counter()
        oracle.decode(*args, num_threads=threads)
        return case.algorithmic_bytes(), time.perf_counter() - t0

    def median_of_three(threads):
        n = 4
        _, dt = run(n, threads)
        n = max(4, int(min(max_seqs, n * target_seconds / max(dt, 1e-3))) // 4 * 4)
        runs = [run(n, threads) for _ in range(3)]
        b = runs[0][0]
        dt = statistics.median(r[1] for r in runs)
        return n, b, dt, [round(r[1], 2) for r in runs]

    n, b, dt, all_dt = median_of_three(cores)
    n1, b1, dt1, all_dt1 = median_of_three(1)
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of 256 sequences of the same shape (40/8 heads, ctx {ctx}), all heads; "
                      f"median of 3 runs {all_dt} s on {cores} threads",
            "one_core": {"value": round(b1 / dt1 / 1e9, 5), "unit": "GB/s", "cores": 1,
                         "sample": f"{n1} sequences of the same shape; median of 3 runs {all_dt1} s"}}


def read_ceiling(steps):
    """JSON lines: GB/s of a plain streaming read over 2 GiB for several grid
    sizes and both cache policies, and of the decode's page-gather reads
    alone on the target workload (K+V pages, table and lengths)."""
    import torch
    lib = probe_library()
    stream = torch.cuda.Stream()

    def timed(fn):
        for _ in range(3):
            assert fn() == 0
        torch.cuda.synchronize()
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(steps)]
        for a, b in pairs:
            a.record(stream)
            assert fn() == 0
            b.record(stream)
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
        return per[len(per) // 2], sum(per) / len(per)

    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    best = 0.0
    for nt in (1, 0):
        for blocks in (1024, 2048, 4096, 8192, 16384):
            chunk = nbytes // blocks
            med, mean = timed(lambda: lib.pa_probe_read_stream(buf.data_ptr(), chunk, blocks, nt,
                                                               sink.data_ptr(), stream.cuda_stream))
            gbs = nbytes / med / 1e3
            best = max(best, gbs)
            print(json.dumps({"probe": "read_stream", "bytes": nbytes, "workgroups": blocks,
                              "threads": 256, "nontemporal": nt, "us_median": round(med, 2),
                              "us_mean": round(mean, 2), "GBps": round(gbs, 1),
                              "frac_of_peak": round(gbs / PEAK_GBS, 4)}), flush=True)
    del buf
    case = make_workload("target", "cuda")
    S, Hkv, W = case.num_seqs, case.num_kv_heads, case.max_blocks
    sink = torch.empty(S * Hkv, dtype=torch.int32, device="cuda")
    b = case.kv_bytes() + S * W * 4 + 4 * S
    for pps, depth in ((2, 2), (1, 2), (1, 3), (1, 4), (2, 3), (2, 4), (4, 2), (4, 3), (4, 4)):
        med, mean = timed(lambda: lib.pa_probe_page_gather(
            case.k_cache.data_ptr(), case.v_cache.data_ptr(), case.block_tables.data_ptr(),
            case.seq_lens.data_ptr(), S, Hkv, W, pps, depth, sink.data_ptr(), stream.cuda_stream))
        print(json.dumps({"probe": "page_gather", "workload": "40/8 heads, 256 seqs x ctx 4096",
                          "pages_per_stage": pps, "ring_depth": depth, "bytes": b,
                          "us_median": round(med, 2), "us_mean": round(mean, 2),
                          "GBps": round(b / med / 1e3, 1),
                          "frac_of_peak": round(b / med / 1e3 / PEAK_GBS, 4)}), flush=True)
    print(json.dumps({"read_stream_best_GBps": round(best, 1),
                      "read_stream_best_frac": round(best / PEAK_GBS, 4)}), flush=True)


def probe_library():
    """libpa_probe.so (built with the library; the benchmark's probes only),
    with its entry points' argument types set."""
    import ctypes
    from paged_attention_decode_03_amd import build as pa_build
    lib = ctypes.CDLL(pa_build.PROBE_LIB)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.pa_probe_read_stream.argtypes = [vp, ctypes.c_uint64, i32, i32, vp, vp]
    lib.pa_probe_page_gather.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.pa_probe_decode_valu.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int64,
                                         ctypes.c_float, vp, vp, vp, vp]
    return lib


def valu_decode(lib, case, k_scale, v_scale, out, stream):
    """The decode with its dot products on the vector ALUs (the probe), into
    `out`; returns the probe's status."""
    return lib.pa_probe_decode_valu(case.q.data_ptr(), case.k_cache.data_ptr(), case.v_cache.data_ptr(),
                                    case.block_tables.data_ptr(), case.seq_lens.data_ptr(), case.num_seqs,
                                    case.num_heads, case.num_kv_heads, case.max_blocks,
                                    case.k_cache.shape[0], case.scale, k_scale.data_ptr(),
                                    v_scale.data_ptr(), out.data_ptr(), stream.cuda_stream)


VALU_COMPARE_WORKLOADS = ("target", "dense_32x8_ctx4096_s256", "dense_32x4_ctx4096_s256",
                          "dense_8x1_ctx4096_s256")


def valu_compare(steps, warmup):
    """JSON lines: the decode (MFMA for qKᵀ and PV, in plain order) against the
    same decode with its dot products on the vector ALUs (probe), on the same inputs and
    stream: per-call median and mean (HIP events around each call on the
    launch stream) and GB/s, and the largest difference between the two
    outputs."""
    import torch
    import paged_attention_decode_03_amd as pa
    pa.load_library()
    lib = probe_library()
    stream = torch.cuda.Stream()
    for name in VALU_COMPARE_WORKLOADS:
        case = make_workload(name, "cuda")
        ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
        vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
        out_m, out_v = torch.empty_like(case.q), torch.empty_like(case.q)
        def mfma():
            # the plain order, one wave per (sequence, kv head), like the probe
            pa.paged_attention_unified(case.q, None, 1, case.k_cache, case.v_cache, case.block_tables,
                                       case.seq_lens, case.scale, ks, vs, longest_first=-1, out=out_m,
                                       stream=stream)
            return 0

        calls = {"mfma": mfma, "valu": lambda: valu_decode(lib, case, ks, vs, out_v, stream)}
        res = {"workload": name, "group": case.num_heads // case.num_kv_heads,
               "bytes": case.algorithmic_bytes()}
        for kind, fn in calls.items():
            for _ in range(warmup):
                assert fn() == 0
            torch.cuda.synchronize()
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(steps)]
            for a, b in pairs:
                a.record(stream)
                assert fn() == 0
                b.record(stream)
            torch.cuda.synchronize()
            per = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
            med = per[len(per) // 2]
            res[kind] = {"us_median": round(med, 2), "us_mean": round(sum(per) / len(per), 2),
                         "GBps": round(res["bytes"] / med / 1e3, 1),
                         "frac_of_peak": round(res["bytes"] / med / 1e3 / PEAK_GBS, 4)}
        res["valu_over_mfma"] = round(res["valu"]["us_median"] / res["mfma"]["us_median"], 3)
        res["max_abs_diff"] = float((out_m.float() - out_v.float()).abs().max())
        print(json.dumps(res), flush=True)
        del case, out_m, out_v
        torch.cuda.empty_cache()


def P_one_launch(case):
    """Whether one call of `case` is a single launch of the decode kernel (one
    partition, no order kernel, one query per sequence)."""
    import paged_attention_decode_03_amd as pa
    if case.cu_seqlens_q is not None or getattr(case, "longest_first", False) or case.meta.get("options"):
        return False
    P, _, _ = pa.pa_decode_plan(case.num_seqs, case.num_heads, case.num_kv_heads, case.max_blocks, 256)
    return P == 1


def copy_calibration(steps):
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "us_per_copy": dt * 1e6,
                      "GBps_read_plus_write": 2 * n / dt / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="target")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--read-ceiling", action="store_true")
    ap.add_argument("--valu-compare", action="store_true",
                    help="the decode against the same decode on the vector ALUs (probe)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay timing (profiler runs: only the timed calls)")
    ap.add_argument("--after-suite-workloads", type=int, default=0,
                    help="first allocate, run and free the suite's first N workloads in this "
                         "process (the condition the target meets inside --workload all)")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed calls for at least this long before the warm-up calls "
                         "(the first calls after input generation run slower)")
    ap.add_argument("--cold", action="store_true",
                    help="rotate the calls over copies of the inputs in distinct buffers "
                         "(at least 512 MiB touched per round), so a small workload is "
                         "timed from HBM rather than from the Infinity Cache")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only: the kernel works on one GPU's share of "
              "heads/sequences (tensor or data parallel shards need no exchange inside attention) "
              "and there is no cross-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.read_ceiling:
        read_ceiling(args.steps)
        return
    if args.valu_compare:
        valu_compare(args.steps, args.warmup)
        return

    import paged_attention_decode_03_amd as pa
    pa.load_library()

    if args.workload == "all":
        # graph replay warms up over the first graphs of a process (see the
        # target's graph timing below): six untimed graphs of the default
        # workload first
        warm = make_workload("target", "cuda")
        for _ in range(6):
            time_graph(warm, replays=10, calls_per_graph=10)
        del warm
        torch.cuda.empty_cache()
        for name in suite_names():
            case = make_workload(name, "cuda")
            us = time_calls(case, args.steps, args.warmup)
            us_graph = time_graph(case)
            us_cold = time_calls_cold(case, args.steps, args.warmup) \
                if workload_bytes(case) < COLD_MIN_BYTES else None
            P, ppp, _ = pa.pa_decode_plan(case.num_seqs, case.num_heads, case.num_kv_heads,
                                          case.max_blocks, 256)
            b = workload_bytes(case)
            if case.k_slot_scales is not None:
                b += case.kv_bytes() // 128 * 4   # one fp32 K or V scale per cached token and kv head
            row = {"workload": name, "us_per_call": round(us, 2),
                   "us_per_call_graph": round(us_graph, 2),
                   "us_per_call_cold": None if us_cold is None else round(us_cold, 2),
                   "GBps": round(b / us / 1e3, 1), "frac_of_peak": round(b / us / 1e3 / PEAK_GBS, 4),
                   "bytes": b}
            if case.cu_seqlens_q is None:   # the exported planner covers one query per sequence
                row.update({"partitions": P, "pages_per_partition": ppp})
            print(json.dumps(row), file=sys.stderr, flush=True)
            del case
            torch.cuda.empty_cache()
        for name, T, pattern in (("cache_write_decode_256x8", 256, "decode"),
                                 ("cache_write_prefill_32768x8", 32768, "prefill"),
                                 ("cache_write_chunks_32768x8", 32768, "chunks")):
            us = time_cache_write(T, args.steps, args.warmup, pattern=pattern)
            b = cache_write_bytes(T)
            print(json.dumps({"workload": name, "us_per_call": round(us, 2),
                              "GBps": round(b / us / 1e3, 1),
                              "frac_of_peak": round(b / us / 1e3 / PEAK_GBS, 4), "bytes": b}),
                  file=sys.stderr, flush=True)
        args.workload = "target"

    m = re.fullmatch(r"cache_write_(prefill|chunks|decode)_(\d+)x(\d+)", args.workload)
    if m:   # one workload of the cache write, for profiling runs
        T, hkv = int(m.group(2)), int(m.group(3))
        us = time_cache_write(T, args.steps, args.warmup, num_kv_heads=hkv, pattern=m.group(1))
        b = cache_write_bytes(T, hkv)
        print(json.dumps({"workload": args.workload, "us_per_call": round(us, 2),
                          "GBps": round(b / us / 1e3, 1), "frac_of_peak": round(b / us / 1e3 / PEAK_GBS, 4),
                          "bytes": b}), flush=True)
        return

    for name in suite_names()[:max(0, args.after_suite_workloads)]:
        w = make_workload(name, "cuda")
        time_calls(w, 20, 5)
        del w
        torch.cuda.empty_cache()
    case = make_workload(args.workload, "cuda")
    if args.cold:
        us = time_calls_cold(case, args.steps, args.warmup)
        per = None
    else:
        us, per, settled = time_calls(case, args.steps, args.warmup, per_call=True,
                                      settle_ms=args.settle_ms)
    B = workload_bytes(case)
    gbs = B / us / 1e3
    import statistics
    us_med = statistics.median(per) if per else None
    us_evmean = sum(per) / len(per) if per else None
    # graph replay, the pages' timing method (not in the timed region): five
    # runs of 10 replays back to back (an event pair around each replay would
    # leave the GPU idle between replays), their per-call averages.  The
    # the first graphs a process replays run slower than later ones (measured
    # on MI355X, graphs of 10 calls replayed 10 times: the first five
    # 336.3-337.5 us a call, the sixth 330.3, then 324.8-325.3, with the timed
    # region at 326.2), so six are replayed untimed first.
    g_per = None
    if not (args.cold or args.no_graph):
        g_per = [time_graph(case, replays=10, calls_per_graph=10) for _ in range(11)][6:]
    g_med = statistics.median(g_per) if g_per else None
    g_mean = sum(g_per) / len(g_per) if g_per else None
    # the decode kernel's average launch duration: the timed region's calls run
    # back to back, so where a call is one launch (one partition) the region's
    # average per call is that kernel's average duration
    kernel_us = us
    k_gbs = B / kernel_us / 1e3
    one_launch = P_one_launch(case)
    P, ppp, _ = pa.pa_decode_plan(case.num_seqs, case.num_heads, case.num_kv_heads, case.max_blocks, 256)
    traffic = counter_traffic() if args.workload == "target" else None
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "us_per_call": round(us, 3),
        "value_basis": "algorithmic bytes per call / (timed region / steps): whole-job throughput",
        "settle_calls": None if args.cold else settled,
        "us_per_call_median": None if us_med is None else round(us_med, 3),
        "us_per_call_mean_of_calls": None if us_evmean is None else round(us_evmean, 3),
        "per_call_basis": "a second, untimed loop of the same calls, an event pair around each",
        "us_per_call_graph_median": None if g_med is None else round(g_med, 3),
        "us_per_call_graph_mean": None if g_mean is None else round(g_mean, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(PAGES_ASM_US / us, 4) if args.workload == "target" else None,
        "vs_baseline_ref": "pages' MI355X pa_fwd_asm 363.04 us/call at this workload (ratio of call times)",
        "vs_pages_hip": round(PAGES_HIP_US / us, 4) if args.workload == "target" else None,
        "dtype": "fp8_e4m3fn KV, bf16 q/out, bf16/fp16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) q, K, V; per-tensor fp8 scales; shuffled block table)",
        "config": {"workload": args.workload if args.workload != "target" else
                   "40q/8kv heads, head_dim 128, 256 seqs x ctx 4096, fp8 e4m3fn KV, 16-token blocks",
                   "num_seqs": case.num_seqs, "num_heads": case.num_heads,
                   "num_kv_heads": case.num_kv_heads, "max_blocks_per_seq": case.max_blocks,
                   "partitions": P, "pages_per_partition": ppp, "algorithmic_bytes": B,
                   "inputs": "rotated over copies (cold cache)" if args.cold else "one set"},
        "roofline": {"bound": "hbm", "achieved": round(k_gbs, 2), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(k_gbs / PEAK_GBS, 4), "traffic": traffic,
                     "kernel_us_mean": round(kernel_us, 3), "one_launch_per_call": one_launch},
    }
    del case
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
