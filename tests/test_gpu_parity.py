"""Parity of the HIP library with the fp64 oracle on MI355X (gfx950).

Small cases are compared element by element in full; the full-size workloads
(dense 1K/4K, the 256-sequence ragged mix over four head layouts and three
seeds, the low-batch long-context grid, and 40/8 heads x 4096 tokens x 256
sequences in the benchmark's launch configuration) are compared on sampled
sequences.  Bound: max abs error <= 1e-2 and mean abs error <= 5e-4 against
the fp64 oracle, for bf16 output.
"""
import numpy as np
import pytest
import torch

import workloads
from parity import compare, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_attention_decode_03_amd as pa
    pa.load_library()   # raises if the library is missing: no fallback


# ---------------------------------------------------------------- small, full

def test_tiny():
    case = workloads.tiny(0)
    log("tiny: 4 seqs ctx {1,17,33,64}, 8/2 heads, 32 blocks")
    compare(run_gpu(case), run_oracle(case), "tiny")


SMALL = [
    (8, 2, [1, 15, 16, 17, 63, 64, 65, 200]),
    (5, 1, [1, 2, 31, 32, 33, 500]),
    (40, 8, [1, 100, 1000, 17]),
    (32, 4, [64, 65, 129, 255, 256, 257]),
    (16, 1, [1, 333, 48]),
    (8, 8, [7, 90, 16]),
    (16, 16, [40, 3]),
    (2, 1, [1024, 5]),
]


@pytest.mark.parametrize("hq,hkv,lens", SMALL, ids=lambda x: str(x))
def test_small_layouts(hq, hkv, lens):
    case = workloads.make_case(hq, hkv, lens, seed=hq * 7 + hkv)
    log(f"small {hq}/{hkv} lens={lens}")
    compare(run_gpu(case), run_oracle(case), f"small {hq}/{hkv}")


@pytest.mark.parametrize("ppp", [1, 2, 3, 5, 7, 64, 256])
def test_forced_partition_sizes(ppp):
    case = workloads.make_case(16, 2, [1, 15, 16, 17, 100, 1000, 0, 333, 4000], seed=3,
                               max_blocks=250)
    log(f"split ppp={ppp}")
    compare(run_gpu(case, pages_per_partition=ppp), run_oracle(case), f"split ppp={ppp}")


def test_empty_sequences_give_zero_rows():
    case = workloads.make_case(8, 2, [0, 37, 0, 1], seed=5, max_blocks=4)
    out = run_gpu(case)
    assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[2]) == 0
    compare(out, run_oracle(case), "with empty sequences")
    out_split = run_gpu(case, pages_per_partition=1)
    assert torch.count_nonzero(out_split[0]) == 0
    compare(out_split, run_oracle(case), "with empty sequences, split")


def test_all_fp8_codes_through_v_are_exact():
    """One-token contexts return V_0 * v_scale; with v_scale = 1 every finite
    fp8 value is a bf16 value, so the output must equal it exactly (the sum
    that forms the output starts from +0, so the code for -0 gives +0, as in
    the oracle)."""
    case = workloads.make_case(4, 1, [1, 1], seed=9, max_blocks=1, extra_blocks=2)
    codes = np.arange(256, dtype=np.uint8)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    v = case.v_cache.clone()
    for s in range(2):
        blk = int(case.block_tables[s, 0])
        v[blk, 0, :, 0] = torch.from_numpy(codes[s * 128:(s + 1) * 128].copy())
    case.v_cache = v
    case.v_scale = 1.0
    out = run_gpu(case).cpu()
    expect = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().to(torch.bfloat16).view(2, 128)
    for s in range(2):
        for h in range(4):
            assert torch.equal(out[s, h].float(), expect[s].float()), (s, h)


# ---------------------------------------------------------------- invariants

def test_run_to_run_bitwise_determinism():
    case = workloads.ragged(40, 8, seed=0, num_seqs=64, device="cuda")
    a = run_gpu(case).clone()
    b = run_gpu(case)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_block_placement_invariance_bitwise():
    case = workloads.make_case(8, 2, [33, 90, 16, 1, 700], seed=31)
    base = run_gpu(case).cpu()
    NB = case.k_cache.shape[0]
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(99))
    k2 = torch.empty_like(case.k_cache)
    v2 = torch.empty_like(case.v_cache)
    k2[perm] = case.k_cache
    v2[perm] = case.v_cache
    moved = workloads.Case("moved", case.q, k2, v2, perm[case.block_tables.long()].to(torch.int32),
                           case.seq_lens, case.scale, case.k_scale, case.v_scale)
    assert torch.equal(run_gpu(moved).cpu().view(torch.int16), base.view(torch.int16))


def test_sequence_order_permutes_outputs_bitwise():
    case = workloads.make_case(8, 2, [33, 90, 16, 1, 0, 250], seed=32, max_blocks=16)
    base = run_gpu(case).cpu()
    order = torch.tensor([3, 0, 5, 4, 2, 1])
    pc = workloads.Case("perm", case.q[order], case.k_cache, case.v_cache, case.block_tables[order],
                        case.seq_lens[order], case.scale, case.k_scale, case.v_scale)
    assert torch.equal(run_gpu(pc).cpu().view(torch.int16), base[order].view(torch.int16))


def test_nan_poison_outside_context_is_never_read():
    lens = [1, 17, 33, 64, 5, 250]
    a = workloads.make_case(8, 2, lens, 33, max_blocks=20, poison=True)
    b = workloads.make_case(8, 2, lens, 33, max_blocks=20, poison=False)
    for ppp in (None, 1, 3):
        oa, ob = run_gpu(a, ppp).cpu(), run_gpu(b, ppp).cpu()
        assert torch.isfinite(oa.float()).all()
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_split_and_unsplit_agree():
    case = workloads.make_case(40, 8, [4096, 1, 2000, 3001], seed=12)
    ref = run_oracle(case)
    outs = {ppp: run_gpu(case, ppp).cpu() for ppp in (0, 1, 8, 64, 256)}
    for ppp, o in outs.items():
        compare(o, ref, f"ppp={ppp}")
    d = (outs[1].float() - outs[256].float()).abs().max().item()
    assert d <= 2e-2


def test_non_default_stream():
    case = workloads.make_case(8, 2, [300, 20], seed=13).to("cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = run_gpu(case, stream=s)
    compare(out, run_oracle(case), "side stream")


def test_graph_capture_replays_match_eager():
    import paged_attention_decode_03_amd as pa
    cases = [workloads.make_case(40, 8, [4096, 33], seed=14).to("cuda"),       # split path
             workloads.make_case(8, 2, [1, 17, 200], seed=15).to("cuda")]
    ks = [torch.tensor([c.k_scale], device="cuda") for c in cases]
    vs = [torch.tensor([c.v_scale], device="cuda") for c in cases]
    outs = [torch.empty_like(c.q) for c in cases]

    def step():
        for c, k, v, o in zip(cases, ks, vs, outs):
            pa.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                                      c.scale, k, v, out=o)

    step()   # eager: also sizes the split-KV scratch before capture
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
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
        for o in outs:
            o.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {r}"
        step()   # eager work between replays
        torch.cuda.synchronize()
    compare(outs[1], run_oracle(cases[1]), "graph replay")


# ---------------------------------------------------------------- full sizes, every sequence

@pytest.mark.parametrize("hq,hkv,s,ctx", workloads.DENSE_1K + workloads.DENSE_4K,
                         ids=lambda x: str(x))
def test_dense_full_size(hq, hkv, s, ctx):
    log(f"dense {hq}/{hkv} seqs={s} ctx={ctx}")
    case = workloads.dense(hq, hkv, s, ctx, seed=0, device="cuda")
    out = run_gpu(case)
    compare(out, run_oracle(case), f"dense {hq}/{hkv} s{s} ctx{ctx}")


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("hq,hkv", workloads.RAGGED_LAYOUTS, ids=lambda x: str(x))
def test_ragged_full_size(hq, hkv, seed):
    log(f"ragged {hq}/{hkv} seed={seed}")
    case = workloads.ragged(hq, hkv, seed=seed, device="cuda")
    out = run_gpu(case)
    compare(out, run_oracle(case), f"ragged {hq}/{hkv} seed {seed}")


@pytest.mark.parametrize("hq,hkv,s,ctx", workloads.LOW_BATCH, ids=lambda x: str(x))
def test_low_batch_long_context(hq, hkv, s, ctx):
    log(f"low batch {hq}/{hkv} seqs={s} ctx={ctx}")
    case = workloads.dense(hq, hkv, s, ctx, seed=s, device="cuda")
    out = run_gpu(case)
    compare(out, run_oracle(case), f"low-batch s{s} ctx{ctx}")


def test_target_40x8_ctx4096_256seqs():
    """The benchmark's workload and launch configuration."""
    hq, hkv, s, ctx = workloads.TARGET
    case = workloads.dense(hq, hkv, s, ctx, seed=0, device="cuda")
    out = run_gpu(case)
    compare(out, run_oracle(case), "target 40/8 ctx4096 s256")
    again = run_gpu(case)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))


def test_tp2_share_20x4_ctx4096_256seqs():
    case = workloads.dense(20, 4, 256, 4096, seed=0, device="cuda")
    out = run_gpu(case)
    compare(out, run_oracle(case), "20/4 ctx4096 s256")


# ---------------------------------------------------------------- per-slot scales

def run_gpu_slot(case):
    import paged_attention_decode_03_amd as pa
    c = case if case.q.is_cuda else case.to("cuda")
    out = pa.paged_decode_attention_slot_scales(c.q, c.k_cache, c.v_cache, c.block_tables,
                                                c.seq_lens, c.scale, c.k_slot_scales,
                                                c.v_slot_scales)
    torch.cuda.synchronize()
    return out


def oracle_slot(case, seqs=None, abs_values=False):
    """fp64 oracle with per-slot scales; abs_values: on |V| (every V code's
    sign bit cleared), i.e. sum_t p_t |V_t|, the magnitude of the terms."""
    import oracle
    h = case.host()
    idx = np.arange(h.num_seqs) if seqs is None else np.asarray(seqs)
    v = h.v_cache.numpy() & 0x7F if abs_values else h.v_cache.numpy()
    return oracle.decode_slot_scales(h.q_bits()[idx], h.k_cache.numpy(), v,
                                     h.block_tables.numpy()[idx], h.seq_lens.numpy()[idx],
                                     h.scale, h.k_slot_scales.numpy(), h.v_slot_scales.numpy())


@pytest.mark.parametrize("hq,hkv,lens", [(8, 2, [1, 17, 33, 64]), (40, 8, [1, 100, 1000, 17]),
                                         (16, 1, [1, 333, 48]), (5, 1, [2, 31, 500])],
                         ids=lambda x: str(x))
def test_slot_scales_small(hq, hkv, lens):
    case = workloads.make_case(hq, hkv, lens, seed=hq + 3 * hkv, scale_mode="per_slot")
    compare(run_gpu_slot(case), oracle_slot(case), f"slot scales {hq}/{hkv}", relative=True)


def test_slot_scales_equal_to_tensor_scales_match_per_tensor_path():
    case = workloads.make_case(40, 8, [4096, 77, 1], seed=61)
    NB = case.k_cache.shape[0]
    case.k_slot_scales = torch.full((NB, 8, 16), case.k_scale, dtype=torch.float32)
    case.v_slot_scales = torch.full((NB, 8, 16), case.v_scale, dtype=torch.float32)
    ref = run_oracle(case)
    compare(run_gpu_slot(case), ref, "slot scales = tensor scales")


@pytest.mark.parametrize("hq,hkv,s,ctx", [(40, 8, 256, 4096), (40, 8, 1, 32768), (40, 8, 4, 4096)],
                         ids=lambda x: str(x))
def test_slot_scales_full_size(hq, hkv, s, ctx):
    case = workloads.make_case(hq, hkv, [ctx] * s, seed=62, device="cuda", scale_mode="per_slot")
    out = run_gpu_slot(case)
    compare(out, oracle_slot(case), f"slot scales {hq}/{hkv} s{s} ctx{ctx}", relative=True)


def test_slot_scales_ragged_with_poison():
    case = workloads.make_case(32, 8, workloads.ragged_lens(64, seed=5), seed=63, device="cuda",
                               max_blocks=250, scale_mode="per_slot")
    out = run_gpu_slot(case)
    compare(out, oracle_slot(case), "slot scales ragged", relative=True)


@pytest.mark.parametrize("num_seqs", [8, 32, 64], ids=lambda n: f"S{n}")
def test_slot_scales_spread_far_beyond_fp16(num_seqs):
    """Per-slot V scales spread over 2^40 within every partition, and each
    sequence's first token's V scale a further 2^-40 below (its V values are
    tiny): the fp16 weights must neither saturate nor lose the small terms.
    8, 32 and 64 sequences at 40/8 take the merge kernel (8 partitions), the
    merge in the decode (4) and no split.

    With terms this far apart, an output can be a near cancellation of terms
    hundreds of times larger than itself, so the bound is applied relative to
    the magnitude of the sum's terms, sum_t p_t |V_t|, which the oracle
    computes on the same case with every V code's sign cleared."""
    lens = [(1, 5, 16, 17, 300, 1000, 2048, 4096)[i % 8] for i in range(num_seqs)]
    case = workloads.make_case(40, 8, lens, seed=64 + num_seqs, scale_mode="per_slot",
                               slot_log2_span=8, v_slot_log2_span=40, tiny_first_v=True,
                               max_blocks=256)
    terms = oracle_slot(case, abs_values=True)
    compare(run_gpu_slot(case), oracle_slot(case), f"slot scales spread 2^40, S={num_seqs}",
            term_scale=terms)


# ---------------------------------------------------------------- caller errors on the device

def test_block_ids_outside_the_caches_read_as_zero_pages():
    """A block id outside [0, num_blocks) in a used table entry is a caller
    error the host cannot see: every entry point must read such a page as
    zeros (no memory access), i.e. give bit for bit the result of the same
    table pointing at an all-zero block."""
    import paged_attention_decode_03_amd as pa
    case = workloads.make_case(8, 2, [40, 70, 33], seed=97, extra_blocks=4, scale_mode="per_slot")
    NB = case.k_cache.shape[0]
    used = set(case.block_tables.flatten().tolist())
    zero_blk = next(b for b in range(NB) if b not in used)
    case.k_cache[zero_blk] = 0
    case.v_cache[zero_blk] = 0
    # an id outside the caches reads as an all-zero page: zero K, V and slot scales
    case.k_slot_scales[zero_blk] = 0.0
    case.v_slot_scales[zero_blk] = 0.0
    bad_ids = [NB, NB + 7, -1, 2**31 - 1]
    spots = [(0, 1), (1, 0), (1, 3), (2, 2)]    # (sequence, table entry) inside each context
    zero_tab = case.block_tables.clone()
    bad_tab = case.block_tables.clone()
    for (s, j), b in zip(spots, bad_ids):
        zero_tab[s, j] = zero_blk
        bad_tab[s, j] = b
    c = case.to("cuda")
    ks = torch.tensor([case.k_scale], device="cuda")
    vs = torch.tensor([case.v_scale], device="cuda")
    cu = torch.tensor([0, 2, 5, 6], dtype=torch.int32, device="cuda")
    q_multi = torch.randn(6, 8, 128, device="cuda").to(torch.bfloat16)
    kv, vv = workloads.token_row_views(c, "nhd")

    def calls(tab):
        tab = tab.to("cuda")
        outs = [pa.paged_decode_attention(c.q, c.k_cache, c.v_cache, tab, c.seq_lens, c.scale, ks, vs),
                pa.paged_decode_attention_split(c.q, c.k_cache, c.v_cache, tab, c.seq_lens, c.scale,
                                                ks, vs, 1),
                pa.paged_decode_attention_slot_scales(c.q, c.k_cache, c.v_cache, tab, c.seq_lens,
                                                      c.scale, c.k_slot_scales, c.v_slot_scales),
                pa.paged_multi_query_attention(q_multi, cu, 3, c.k_cache, c.v_cache, tab, c.seq_lens,
                                               c.scale, ks, vs),
                pa.paged_decode_attention_nhd(c.q, kv, vv, tab, c.seq_lens, c.scale, ks, vs)]
        torch.cuda.synchronize()
        return outs

    for name, a, b in zip(("decode", "split", "slot scales", "multi-query", "token rows"),
                          calls(zero_tab), calls(bad_tab)):
        log(f"invalid block ids, {name}")
        assert torch.isfinite(b.float()).all(), name
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    # the zero-block table is ordinary input: the decode meets the bound on it
    # (per-tensor scales of 1 over codes up to 448: errors relative to |out|)
    case.block_tables = zero_tab
    compare(calls(zero_tab)[0], run_oracle(case), "zero-block table", relative=True)


def test_two_waves_per_item():
    """Two waves per work item (each computing every other stage of 4 pages,
    combined in LDS) run where one partition leaves two work items per CU
    (64 sequences x 8 kv heads = 512 items on 256 CUs) and the contexts stay
    whole: an explicit partition of the whole table, or longest-first
    dispatch.  Ragged contexts with empty, one-token, one-stage and
    one-token-past-a-stage sequences, in both cache-policy instantiations (an
    80-block table: cached loads; 256 blocks: streamed, V through LDS), with
    NaN poison outside the contexts (must equal the clean case bit for bit),
    must meet the bound; longest-first must equal the whole-table call bit
    for bit.  The library's own plan splits such launches in two (merged in
    the decode), which must meet the bound as well."""
    import paged_attention_decode_03_amd as pa
    for W, top in ((80, 1280), (256, 4096)):
        assert pa.pa_decode_plan(64, 40, 8, W, 256)[:2] == (2, W // 2)
        lens = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, top, top - 1, 700, 333, 1000] * 4
        cases = [workloads.make_case(40, 8, lens, seed=51 + W, max_blocks=W, poison=p) for p in (True, False)]
        log(f"two waves per item, {W}-block table, poison vs clean")
        a, b = run_gpu(cases[0], W).cpu(), run_gpu(cases[1], W).cpu()
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        for s in range(64):
            if lens[s] == 0:
                assert torch.count_nonzero(a[s]) == 0
        ref = run_oracle(cases[1])
        compare(a, ref, f"two waves per item, W={W}")
        c = cases[0].to("cuda")
        ks = torch.tensor([c.k_scale], device="cuda")
        vs = torch.tensor([c.v_scale], device="cuda")
        lpt = pa.paged_attention_unified(c.q, None, 1, c.k_cache, c.v_cache, c.block_tables,
                                         c.seq_lens, c.scale, ks, vs, longest_first=True)
        torch.cuda.synchronize()
        log(f"two waves per item, {W}-block table, longest first")
        assert torch.equal(lpt.cpu().view(torch.int16), a.view(torch.int16))
        log(f"two partitions, {W}-block table")
        compare(run_gpu(cases[0]).cpu(), ref, f"two partitions, W={W}")


def test_fused_merge_counters_stay_consistent():
    """Split contexts with few partitions (here 4 at 32/8 heads and 2 at 16/1)
    are merged by the last work item of each (sequence, kv head) to finish,
    counted by arrival counters in the scratch that every call leaves at zero;
    more partitions (8 at 40/8) go to the merge kernel.  Calls of these shapes
    in turn, a repeat (bit for bit), and a captured graph replayed three times
    with eager calls of the other shapes in between must all meet the bound."""
    import paged_attention_decode_03_amd as pa
    lens_a = [0, 1, 15, 16, 17, 127, 128, 129, 1024, 1023, 513, 700, 64, 65, 900, 1000] + \
             [1024 - 37 * i for i in range(8)]
    a = workloads.make_case(32, 8, lens_a, seed=61, max_blocks=64)
    b = workloads.make_case(40, 8, lens_a[:16], seed=62, max_blocks=64)
    d = workloads.make_case(16, 1, [2048, 0, 1, 1025, 1024, 2047] * 50, seed=64, max_blocks=128)
    assert pa.pa_decode_plan(24, 32, 8, 64, 256)[:2] == (4, 16)
    assert pa.pa_decode_plan(16, 40, 8, 64, 256)[:2] == (8, 8)
    assert pa.pa_decode_plan(300, 16, 1, 128, 256)[:2] == (2, 64)
    first = run_gpu(a).cpu()
    log("fused merge: shapes A (4 partitions), B (8: merge kernel), D (2), A")
    compare(first, run_oracle(a), "fused merge A")
    compare(run_gpu(b).cpu(), run_oracle(b), "merge kernel B")
    compare(run_gpu(d).cpu(), run_oracle(d), "fused merge D")
    big = workloads.make_case(40, 8, [300] * 64, seed=63)   # one partition: no counters
    run_gpu(big)
    again = run_gpu(a).cpu()
    assert torch.equal(again.view(torch.int16), first.view(torch.int16))
    c = a.to("cuda")
    ks = torch.tensor([c.k_scale], device="cuda")
    vs = torch.tensor([c.v_scale], device="cuda")
    out = torch.empty_like(c.q)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    # the capture stream's split-KV scratch, reserved before capture
    pa.pa_workspace_reserve(pa.pa_workspace_bytes(c.num_seqs, c.num_heads, c.num_kv_heads,
                                                  c.max_blocks, device=0), stream=s)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(2):
                pa.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                                          c.scale, ks, vs, out=out)
    for r in range(3):
        out.fill_(7.0)
        run_gpu(b)                      # eager work of other shapes between replays
        run_gpu(d)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"fused merge: graph replay {r}")
        assert torch.equal(out.cpu().view(torch.int16), first.view(torch.int16)), f"replay {r}"


def test_longest_first_order_covers_every_sequence():
    """Longest-first dispatch (an order computed on the device) must compute
    every sequence exactly once with the same arithmetic: the unified call with
    no row offsets and longest_first must equal the plain decode bit for bit,
    for ragged contexts that split and for ones that do not, with the order
    sorted inside each work item (up to 512 sequences) and by the order kernel
    (more), for several queries per sequence, and in a graph replay."""
    import paged_attention_decode_03_amd as pa
    for S, seed in ((48, 5), (300, 6), (3, 7), (512, 8), (700, 9)):
        lens = workloads.ragged_lens(S, seed=seed)
        case = workloads.make_case(40, 8, lens, seed=98 + S, max_blocks=250).to("cuda")
        ks = torch.tensor([case.k_scale], device="cuda")
        vs = torch.tensor([case.v_scale], device="cuda")
        args = (case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.scale, ks, vs)
        plain = pa.paged_decode_attention(case.q, *args)
        ordered = pa.paged_attention_unified(case.q, None, 1, *args, longest_first=True)
        torch.cuda.synchronize()
        log(f"longest first S={S}")
        assert torch.equal(ordered.view(torch.int16), plain.view(torch.int16)), f"S={S}"
    # several queries per sequence (one to six at 8 heads a group: one to three
    # 16-row query tiles)
    lens = workloads.ragged_lens(96, lo=8, hi=3000, seed=10)
    ql = [1 + (i * 7) % 6 for i in range(96)]
    mcase = workloads.make_multi_case(32, 4, lens, ql, seed=99).to("cuda")
    margs = (mcase.k_cache, mcase.v_cache, mcase.block_tables, mcase.seq_lens, mcase.scale,
             torch.tensor([mcase.k_scale], device="cuda"), torch.tensor([mcase.v_scale], device="cuda"))
    a = pa.paged_attention_unified(mcase.q, mcase.cu_seqlens_q, 6, *margs)
    b = pa.paged_attention_unified(mcase.q, mcase.cu_seqlens_q, 6, *margs, longest_first=True)
    torch.cuda.synchronize()
    log("longest first, several queries")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    out = torch.empty_like(case.q)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    pa.pa_workspace_reserve(pa.pa_workspace_bytes(case.num_seqs, case.num_heads, case.num_kv_heads,
                                                  case.max_blocks, longest_first=True, device=0),
                            stream=s)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pa.paged_attention_unified(case.q, None, 1, *args, longest_first=True, out=out)
    for r in range(3):
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), plain.view(torch.int16)), f"replay {r}"


@pytest.mark.parametrize("kind", ["ragged", "one_bin", "two_bins", "several_queries", "options",
                                  "several_queries_options"])
def test_default_longest_first_matches_plain_order(kind):
    """256 sequences at 40/8 heads with 250-block tables are ordered longest
    first by default (each work item sorts the lengths; where they all fall in
    one bin it keeps the plain order without sorting), and 257 sequences are
    not (more than the default order's 256).  The per-sequence arithmetic is
    the same either way, so the 256-sequence call must equal the first 256
    sequences of the 257-sequence call bit for bit: ragged lengths, lengths of
    one bin (250 pages: 3985..4000 tokens), two bins, several queries per
    sequence, and the unified call's softcap, ALiBi and sinks with one query
    and with several."""
    import paged_attention_decode_03_amd as pa
    S = 257
    opts = {}
    if kind.endswith("options"):
        opts = dict(softcap=25.0, alibi_slopes=torch.linspace(-0.05, 0.02, 40, device="cuda"),
                    sinks=torch.linspace(-1.0, 2.0, 40, device="cuda"))
    if kind == "one_bin":
        lens = [3985 + (i * 7) % 16 for i in range(S)]
    elif kind == "two_bins":
        lens = [4000 if i % 3 else 1990 + i % 11 for i in range(S)]
    else:
        lens = workloads.ragged_lens(S, seed=23)
    ql = [min(1 + (i * 5) % 6, lens[i]) for i in range(S)] if kind.startswith("several") else None
    if ql is None:
        case = workloads.make_case(40, 8, lens, seed=123, max_blocks=250, device="cuda")
    else:
        case = workloads.make_multi_case(40, 8, lens, ql, seed=124, max_blocks=250, device="cuda")
    ks = torch.tensor([case.k_scale], device="cuda")
    vs = torch.tensor([case.v_scale], device="cuda")
    tail = (case.scale, ks, vs)
    if ql is None and opts:
        full = pa.paged_attention_unified(case.q, None, 1, case.k_cache, case.v_cache,
                                          case.block_tables, case.seq_lens, *tail, **opts)
        part = pa.paged_attention_unified(case.q[:256].contiguous(), None, 1, case.k_cache,
                                          case.v_cache, case.block_tables[:256].contiguous(),
                                          case.seq_lens[:256].contiguous(), *tail, **opts)
        rows = 256
    elif ql is None:
        full = pa.paged_decode_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                                         case.seq_lens, *tail)
        part = pa.paged_decode_attention(case.q[:256].contiguous(), case.k_cache, case.v_cache,
                                         case.block_tables[:256].contiguous(),
                                         case.seq_lens[:256].contiguous(), *tail)
        rows = 256
    else:
        cu = case.cu_seqlens_q
        rows = int(cu[256])
        full = pa.paged_attention_unified(case.q, cu, 6, case.k_cache, case.v_cache,
                                          case.block_tables, case.seq_lens, *tail, **opts)
        part = pa.paged_attention_unified(case.q[:rows].contiguous(), cu[:257].contiguous(), 6,
                                          case.k_cache, case.v_cache,
                                          case.block_tables[:256].contiguous(),
                                          case.seq_lens[:256].contiguous(), *tail, **opts)
    torch.cuda.synchronize()
    log(f"default order {kind}")
    assert torch.equal(part.view(torch.int16), full[:rows].view(torch.int16))


def test_default_longest_first_with_two_waves_per_item():
    """256 sequences at 32/4 heads (1024 (sequence, kv head) units: four per
    CU) with 250-block tables are ordered longest first by default and run
    two waves per item, whose partial sums combine in another order: the
    256-sequence call agrees with the first 256 sequences of the 257-sequence
    call (plain order, one wave per item) to rounding, and repeats itself bit
    for bit; asked for the plain order (longest_first -1), the 256-sequence
    call equals the 257-sequence one bit for bit."""
    import paged_attention_decode_03_amd as pa
    S = 257
    lens = workloads.ragged_lens(S, seed=24)
    case = workloads.make_case(32, 4, lens, seed=125, max_blocks=250, device="cuda")
    tail = (case.scale, torch.tensor([case.k_scale], device="cuda"), torch.tensor([case.v_scale], device="cuda"))
    full = pa.paged_decode_attention(case.q, case.k_cache, case.v_cache, case.block_tables,
                                     case.seq_lens, *tail)
    sub = (case.q[:256].contiguous(), case.k_cache, case.v_cache, case.block_tables[:256].contiguous(),
           case.seq_lens[:256].contiguous())
    part = pa.paged_decode_attention(*sub, *tail)
    again = pa.paged_decode_attention(*sub, *tail)
    # longest_first = -1: the plain order, one wave per item, as with 257 sequences
    plain = pa.paged_attention_unified(sub[0], None, 1, *sub[1:], *tail, longest_first=-1)
    torch.cuda.synchronize()
    log("default order, two waves per item, 32/4 x 256")
    assert torch.equal(part.view(torch.int16), again.view(torch.int16))
    assert torch.equal(plain.view(torch.int16), full[:256].view(torch.int16))
    d = (part.float() - full[:256].float()).abs()
    ref = full[:256].float().abs()
    # one bf16 rounding apart at most: 2^-8 relative, or absolute near zero
    assert bool((d <= torch.clamp(ref, min=2.0 ** -6) * 2.0 ** -7).all()), float(d.max())
    assert float(d.mean()) < 1e-4


@pytest.mark.parametrize("name", ["ragged_32x4_seed0", "ragged_32x4_seed1", "ragged_8x1_600seqs"])
def test_longest_first_with_two_waves_per_item(name):
    """Longest-first launches of 2 to 4 items per CU run two waves per item
    (ragged 32/4 x 256 sequences: 1024 items; 600 ragged sequences at 8/1:
    600 items, ordered by the order kernel): every sequence meets the bound
    against the oracle, the plain order's result too, and a repeat gives the
    same bits."""
    import paged_attention_decode_03_amd as pa
    if name.startswith("ragged_32x4"):
        case = workloads.ragged(32, 4, seed=int(name[-1]), device="cuda")
    else:
        case = workloads.make_case(8, 1, workloads.ragged_lens(600, seed=11), seed=111, device="cuda",
                                   max_blocks=250)
    ks = torch.tensor([case.k_scale], device="cuda")
    vs = torch.tensor([case.v_scale], device="cuda")
    args = (case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.scale, ks, vs)
    lpt = pa.paged_attention_unified(case.q, None, 1, *args, longest_first=True)
    again = pa.paged_attention_unified(case.q, None, 1, *args, longest_first=True)
    plain = pa.paged_decode_attention(case.q, *args)
    torch.cuda.synchronize()
    log(f"longest first, two waves per item: {name}")
    assert torch.equal(lpt.view(torch.int16), again.view(torch.int16))
    ref = run_oracle(case)
    compare(lpt, ref, f"longest first two waves {name}")
    compare(plain, ref, f"plain order {name}")


def test_cache_policy_does_not_change_results():
    """Working sets within the Infinity Cache are read with the default cache
    policy, larger ones with the streaming hint: two instantiations of the
    same arithmetic.  The same sequences with a table padded to 2048 blocks
    (K/V bound 8 x 2048 x 8 x 4 KiB = 512 MiB: streaming) and with a 256-block
    table (64 MiB: cached), at one explicit partition size, must agree bit for
    bit, and meet the bound against the oracle."""
    lens = [4096, 1, 3000, 17, 2048, 4095, 100, 777]
    case = workloads.make_case(40, 8, lens, seed=41, max_blocks=256).to("cuda")
    wide = torch.zeros(len(lens), 2048, dtype=torch.int32, device="cuda")
    wide[:, :256] = case.block_tables
    padded = workloads.Case("padded", case.q, case.k_cache, case.v_cache, wide, case.seq_lens,
                            case.scale, case.k_scale, case.v_scale)
    log("cache policy: 256- vs 2048-block tables, 32 blocks per partition")
    a = run_gpu(case, 32)
    b = run_gpu(padded, 32)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    compare(a, run_oracle(case), "cache policy")


def test_streamed_path_poison_empty_and_splits():
    """The streamed-set instantiation (V pages through LDS) at its edges: tail
    slots and unused blocks poisoned with NaN, empty and one-token sequences,
    partial last pages, with and without split contexts.  A 2048-block table
    (K/V bound 512 MiB) selects it; the poisoned case must equal the clean
    one bit for bit and meet the bound."""
    lens = [0, 1, 17, 4095, 33, 2000, 0, 256, 3001, 15]
    cases = [workloads.make_case(40, 8, lens, seed=43, max_blocks=2048, poison=p) for p in (True, False)]
    for ppp in (None, 64, 24):
        log(f"streamed path, poison vs clean, pages per partition {ppp}")
        a, b = run_gpu(cases[0], ppp).cpu(), run_gpu(cases[1], ppp).cpu()
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        compare(a, run_oracle(cases[1]), f"streamed path ppp={ppp}")
