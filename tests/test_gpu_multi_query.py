"""Parity of the multi-token (causal) attention entry point with the fp64 oracle
on MI355X (gfx950).

Sequence s has seq_lens[s] cached tokens, the last q_len[s] of which are its
new queries; query i sees cache tokens 0 .. seq_lens[s] - q_len[s] + i.
Small cases are compared element by element in full, across group sizes 1..16
(so 16 .. 1 query tokens per work item), query counts that fill one or
several tiles with a ragged tail, sequences without queries, queries that see
a single token, and split contexts where a query sees none of a later
partition.  The full-size speculative-decode and mixed workloads are compared
on sampled sequences.  Bound: max abs 1e-2, mean abs 5e-4 against the fp64
oracle for bf16 output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare, log, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_attention_decode_03_amd as pa
    pa.load_library()   # raises if the library is missing: no fallback


def q_lens_of(case):
    cu = case.cu_seqlens_q.cpu().numpy()
    return np.diff(cu)


def run_multi_gpu(case, max_seqlen_q=None, out=None, stream=None):
    import paged_attention_decode_03_amd as pa
    c = case if case.q.is_cuda else case.to("cuda")
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
    if max_seqlen_q is None:
        max_seqlen_q = max(1, int(q_lens_of(case).max(initial=0)))
    o = pa.paged_multi_query_attention(c.q, c.cu_seqlens_q, max_seqlen_q, c.k_cache, c.v_cache,
                                       c.block_tables, c.seq_lens, c.scale, ks, vs, out=out,
                                       stream=stream)
    torch.cuda.synchronize()
    return o


def run_multi_oracle(case, seqs=None):
    """(oracle rows, their row indices in the full output) for sequences `seqs`."""
    h = case.host() if case.q.is_cuda else case
    cu = h.cu_seqlens_q.numpy().astype(np.int64)
    S = h.num_seqs
    idx = np.arange(S) if seqs is None else np.asarray(seqs)
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in idx]).astype(np.int64)
    sub_cu = np.zeros(len(idx) + 1, np.int32)
    sub_cu[1:] = np.cumsum(cu[idx + 1] - cu[idx])
    ref = oracle.attend_multi(h.q_bits()[rows], sub_cu, h.k_cache.numpy(), h.v_cache.numpy(),
                              h.block_tables.numpy()[idx], h.seq_lens.numpy()[idx], h.scale,
                              h.k_scale, h.v_scale)
    return ref, rows


def check(case, label, seqs=None, relative=False, **kw):
    out = run_multi_gpu(case, **kw)
    ref, rows = run_multi_oracle(case, seqs)
    compare(out, ref, label, seqs=rows, relative=relative)
    return out


# ---------------------------------------------------------------- small, full

SMALL = [
    # (hq, hkv, seq_lens, q_lens)
    (8, 8, [1, 16, 17, 40, 300], [1, 16, 5, 33, 17]),          # G=1: 16 queries per tile
    (16, 8, [9, 64, 65, 200], [9, 8, 9, 20]),                  # G=2: 8 per tile
    (12, 4, [3, 50, 129], [3, 7, 11]),                         # G=3: 5 per tile, one idle column
    (20, 4, [31, 32, 33, 100], [4, 6, 1, 13]),                 # G=5: 3 per tile
    (40, 8, [1, 100, 1000, 17, 4], [1, 4, 4, 17, 2]),          # G=5, the target layout
    (40, 8, [100, 64, 1000, 9], [9, 8, 1, 9]),                 # G=5, three tiles an item, one query alone
    (32, 4, [64, 65, 256, 257], [2, 3, 4, 5]),                 # G=8: 2 per tile
    (16, 1, [48, 333, 7], [3, 2, 7]),                          # G=16: 1 per tile
    (8, 2, [40, 70, 90, 5], [0, 12, 0, 5]),                    # sequences without queries
]


@pytest.mark.parametrize("hq,hkv,lens,qlens", SMALL, ids=lambda x: str(x))
def test_small_layouts(hq, hkv, lens, qlens):
    case = workloads.make_multi_case(hq, hkv, lens, qlens, seed=hq * 11 + hkv)
    log(f"multi {hq}/{hkv} lens={lens} q_lens={qlens}")
    check(case, f"multi {hq}/{hkv}")


def test_one_query_per_sequence_equals_decode_bitwise():
    """With one query per sequence the multi-token entry point computes what
    decode computes, in the same order: the outputs are bit-identical.  (The
    shape splits into 16 partitions, so both merge with the merge kernel; the
    decode merges up to 4 partitions in its own last work item instead.)"""
    lens = [1, 15, 16, 17, 100, 1000, 4000, 333]
    case = workloads.make_multi_case(40, 8, lens, [1] * len(lens), seed=21)
    dec = workloads.make_case(40, 8, lens, seed=21)
    dec.q = case.q.clone()
    a = run_multi_gpu(case)
    b = run_gpu(dec)
    log("multi q_len=1 vs decode: bitwise")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fresh_sequences_first_query_sees_one_token():
    """q_len = seq_len: query 0 attends to token 0 only, so its output is
    V_0 * v_scale.  With power-of-two scales that product is a bf16 value, so
    the row must equal it exactly.  Every query is also checked against the
    oracle."""
    case = workloads.make_multi_case(8, 2, [16, 23, 5], [16, 23, 5], seed=31, scale_mode="pow2")
    out = check(case, "fresh prefill chunks")
    h = case.host()
    cu = h.cu_seqlens_q.numpy()
    table = oracle.fp8_table()
    for s in range(h.num_seqs):
        blk = int(h.block_tables[s, 0])
        for kvh in range(2):
            v0 = table[h.v_cache[blk, kvh, :, 0].numpy()] * h.v_scale
            for g in range(4):
                got = out[cu[s], kvh * 4 + g].float().cpu().double().numpy()
                assert np.array_equal(got, v0), (s, kvh, g)


def test_split_contexts_with_queries_that_miss_partitions():
    """Few sequences and long contexts make the planner split; a tile whose
    queries straddle a partition boundary has queries that see none of the
    later partition (their partial carries no weight in the merge)."""
    case = workloads.make_multi_case(8, 8, [300, 2100, 4000], [200, 37, 16], seed=41,
                                     max_blocks=250)
    check(case, "split, queries across partition ends")
    case = workloads.make_multi_case(32, 2, [129, 1500], [129, 3], seed=42, max_blocks=100)
    check(case, "split, G=16, fresh 129")


def test_max_seqlen_q_larger_than_needed():
    case = workloads.make_multi_case(16, 4, [70, 20], [6, 3], seed=51)
    ref, rows = run_multi_oracle(case)
    compare(run_multi_gpu(case, max_seqlen_q=40), ref, "max_seqlen_q=40", seqs=rows)


def test_graph_capture_replays_match_eager():
    import paged_attention_decode_03_amd as pa
    case = workloads.make_multi_case(40, 8, [900, 40, 2000, 1], [4, 4, 3, 1], seed=61).to("cuda")
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
    out = torch.empty_like(case.q)

    def step():
        pa.paged_multi_query_attention(case.q, case.cu_seqlens_q, 4, case.k_cache, case.v_cache,
                                       case.block_tables, case.seq_lens, case.scale, ks, vs,
                                       out=out)

    step()   # eager: also sizes the split-KV scratch before capture
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()   # eager on the capture stream: sizes that stream's split-KV scratch
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        step()   # eager work between replays
        torch.cuda.synchronize()
    ref, rows = run_multi_oracle(case)
    compare(out, ref, "multi graph replay", seqs=rows)


def test_binding_rejects_bad_cu_seqlens():
    import paged_attention_decode_03_amd as pa
    case = workloads.make_multi_case(8, 2, [10, 20], [2, 3], seed=62).to("cuda")
    ks = torch.tensor([case.k_scale], device="cuda")
    vs = torch.tensor([case.v_scale], device="cuda")
    with pytest.raises(TypeError, match="cu_seqlens_q"):
        pa.paged_multi_query_attention(case.q, case.cu_seqlens_q[:-1], 3, case.k_cache,
                                       case.v_cache, case.block_tables, case.seq_lens,
                                       case.scale, ks, vs)
    with pytest.raises(TypeError, match="cu_seqlens_q"):
        pa.paged_multi_query_attention(case.q, case.cu_seqlens_q.to(torch.int64), 3, case.k_cache,
                                       case.v_cache, case.block_tables, case.seq_lens,
                                       case.scale, ks, vs)
    # host floats as scales are refused (a per-call copy a graph cannot replay)
    with pytest.raises(TypeError, match="host float"):
        pa.paged_multi_query_attention(case.q, case.cu_seqlens_q, 3, case.k_cache,
                                       case.v_cache, case.block_tables, case.seq_lens,
                                       case.scale, case.k_scale, case.v_scale)


# ---------------------------------------------------------------- full size, every query row

def test_speculative_decode_target_layout():
    """40/8 heads, 256 sequences of 4096 tokens, 4 new tokens each (one
    accepted token plus three drafts)."""
    S, ctx = 256, 4096
    case = workloads.make_multi_case(40, 8, [ctx] * S, [4] * S, seed=71, device="cuda")
    log(f"spec decode 40/8 x{S} ctx {ctx} q_len 4")
    check(case, "spec decode q_len 4")


def test_speculative_decode_eight_queries():
    """40/8 heads, 64 sequences of 4096 tokens, 8 new tokens each: three query
    tiles a sequence, which a batch of 512 (sequence, kv head) units spreads
    over two items (of two tiles and of one) reading the same pages."""
    S, ctx = 64, 4096
    case = workloads.make_multi_case(40, 8, [ctx] * S, [8] * S, seed=72, device="cuda")
    log(f"spec decode 40/8 x{S} ctx {ctx} q_len 8")
    check(case, "spec decode q_len 8")


def test_three_tiles_an_item():
    """256 sequences at 40/8 (2048 (sequence, kv head) units: eight per CU),
    ragged contexts in [1, 1000], 8 queries (three tiles) in 40% of them and
    one in the rest: one item of three tiles per (sequence, kv head), and
    sequences shorter than their queries' span."""
    S = 256
    lens = workloads.ragged_lens(S, hi=1000, seed=5)
    g = np.random.default_rng(85)
    ql = np.minimum(np.where(g.random(S) < 0.6, 1, 8), lens).tolist()
    case = workloads.make_multi_case(40, 8, lens, ql, seed=85, max_blocks=64, device="cuda")
    log("three tiles an item, 256 ragged sequences")
    check(case, "three tiles an item")


def test_mixed_batch():
    """Decode rows (q_len 1) next to short prefill chunks and drafts: ragged
    contexts in [1, 4000], q_len in {1, 2..8, 16}."""
    S = 256
    lens = workloads.ragged_lens(S, seed=3)
    g = np.random.default_rng(81)
    ql = np.where(g.random(S) < 0.6, 1, g.choice([2, 3, 4, 5, 8, 16], size=S))
    ql = np.minimum(ql, lens).tolist()
    case = workloads.make_multi_case(40, 8, lens, ql, seed=81, max_blocks=250, device="cuda")
    log("mixed batch")
    check(case, "mixed batch")
