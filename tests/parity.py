"""Helpers shared by the GPU parity tests: run the HIP library through its
binding, run the fp64 oracle on the same bytes, compare."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

import oracle

# Bound for bf16 output against the fp64 oracle: max abs 1e-2, mean abs 5e-4
# (how it is applied where bf16 rounding alone exceeds it: see compare).
MAX_ABS = 1e-2
MEAN_ABS = 5e-4


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(case, pages_per_partition=None, out=None, stream=None):
    import paged_attention_decode_03_amd as pa
    c = case if case.q.is_cuda else case.to("cuda")
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
    if pages_per_partition is None:
        o = pa.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                                      c.scale, ks, vs, out=out, stream=stream)
    else:
        o = pa.paged_decode_attention_split(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                                            c.scale, ks, vs, pages_per_partition, out=out,
                                            stream=stream)
    torch.cuda.synchronize()
    return o


def run_oracle(case, seqs=None):
    """fp64 oracle output for the sequences `seqs` (all when None): [len(seqs), Hq, 128]."""
    h = case.host() if case.q.is_cuda else case
    idx = np.arange(h.num_seqs) if seqs is None else np.asarray(seqs)
    q_bits = h.q_bits()[idx]
    return oracle.decode(q_bits, h.k_cache.numpy(), h.v_cache.numpy(),
                         h.block_tables.numpy()[idx], h.seq_lens.numpy()[idx],
                         h.scale, h.k_scale, h.v_scale)


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (8 significant bits; subnormals at 2^-133)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def compare(gpu_out, ref, label, seqs=None, max_abs=MAX_ABS, mean_abs=MEAN_ABS, relative=False,
            term_scale=None):
    """Check bf16 GPU output against the fp64 oracle.

    Max bound, element by element: |gpu - oracle| <= 1e-2 wherever a bf16
    value can meet it at all (wherever the correctly rounded oracle does);
    where none can (|out| >= 4, half a bf16 step is above 1e-2) the output
    must be one of the two bf16 neighbours of the exact value, i.e. less than
    one bf16 step away from it.
    Mean bound: mean |gpu - bf16(oracle)| <= 5e-4 always (error beyond the
    correctly rounded answer), and mean |gpu - oracle| <= 5e-4 where bf16
    rounding itself takes at most half of that budget (short contexts with
    |out| near 1, such as one-token sequences or the first queries of a new
    sequence, have a rounding floor near or above 5e-4 mean).

    relative=True (workloads whose outputs are far larger than N(0,1) data's,
    e.g. per-token magnitudes spread over 2^8): every error is divided by
    max(1, |oracle|) before the same bounds are applied.

    term_scale (same shape as ref: the magnitude of the terms each output
    sums, sum_t p_t |V_t|, from the oracle): every error is divided by
    max(1, term_scale) instead, for data whose terms spread so far that an
    output can be a near cancellation of much larger terms.
    """
    g = gpu_out.float().cpu().double().numpy()
    if seqs is not None:
        g = g[np.asarray(seqs)]
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{label}: non-finite output"
    err = np.abs(g - ref)
    rne = oracle.bf16_bits_to_f64(oracle.bf16_rne(ref))
    floor = np.abs(rne - ref)
    err_rne = np.abs(g - rne)
    ulp = bf16_ulp(ref)
    if term_scale is not None:
        ts = np.asarray(term_scale, dtype=np.float64)
        if seqs is not None and ts.shape != ref.shape:
            ts = ts[np.asarray(seqs)]
        assert ts.shape == ref.shape and (ts >= np.abs(ref) * (1 - 1e-12)).all(), "term_scale below |out|"
        denom = np.maximum(1.0, ts)
    else:
        denom = np.maximum(1.0, np.abs(ref)) if relative else np.ones_like(ref)
    err_s, floor_s, err_rne_s = err / denom, floor / denom, err_rne / denom
    reach = floor_s <= max_abs
    mode = " (relative to the terms)" if term_scale is not None else (" (relative)" if relative else "")
    record = {"label": label, "mode": mode.strip(" ()") or "absolute", "n": int(err.size),
              "max_vs_fp64": float(err_s.max()), "mean_vs_fp64": float(err_s.mean()),
              "max_vs_bf16_oracle": float(err_rne_s.max()), "mean_vs_bf16_oracle": float(err_rne_s.mean()),
              "bf16_floor_mean": float(floor_s.mean()), "beyond_reach": int((~reach).sum())}
    if os.environ.get("PA_PARITY_LOG"):
        # one JSON line per comparison (the whole-workload error table)
        with open(os.environ["PA_PARITY_LOG"], "a") as f:
            f.write(json.dumps(record) + "\n")
    log(f"[{label}]{mode} vs fp64: max={err_s.max():.3e} mean={err_s.mean():.3e} | "
        f"vs bf16(oracle): max={err_rne_s.max():.3e} mean={err_rne_s.mean():.3e} | "
        f"bf16 floor: max={floor_s.max():.3e} mean={floor_s.mean():.3e} | "
        f"beyond reach of 1e-2: {int((~reach).sum())} | n={err.size}")
    over = reach & (err_s > max_abs)
    assert not over.any(), \
        f"{label}: {int(over.sum())} errors above {max_abs} (worst {err_s[reach].max():.3e})"
    far = ~reach & (err >= ulp)
    assert not far.any(), f"{label}: {int(far.sum())} outputs not a bf16 neighbour of the exact value"
    assert err_rne_s.mean() <= mean_abs, \
        f"{label}: mean error vs bf16(oracle) {err_rne_s.mean():.3e} > {mean_abs}"
    if floor_s.mean() <= mean_abs / 2:
        assert err_s.mean() <= mean_abs, f"{label}: mean abs error {err_s.mean():.3e} > {mean_abs}"
    return err
