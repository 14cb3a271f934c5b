"""Parity of the unified call's options on MI355X: sliding window, logit
softcap, ALiBi slopes and attention sinks, on top of several queries per
sequence, against the fp64 oracle's attend_ext.  Without options the call must
return the multi-query entry point's output bit for bit; a window of one token
returns the query's own V exactly; split contexts check that a sink is counted
once and that partitions wholly before a window carry no weight.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import compare, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_attention_decode_03_amd as pa
    pa.load_library()   # raises if the library is missing: no fallback


def max_q(case):
    cu = case.cu_seqlens_q.cpu().numpy()
    return max(1, int(np.diff(cu).max(initial=0)))


def run_unified(case, out=None, stream=None, **opt):
    import paged_attention_decode_03_amd as pa
    c = case if case.q.is_cuda else case.to("cuda")
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
    dev_opt = {k: (torch.as_tensor(v, dtype=torch.float32, device="cuda")
                   if k in ("alibi_slopes", "sinks") and v is not None else v)
               for k, v in opt.items()}
    o = pa.paged_attention_unified(c.q, c.cu_seqlens_q, max_q(case), c.k_cache, c.v_cache,
                                   c.block_tables, c.seq_lens, c.scale, ks, vs, out=out,
                                   stream=stream, **dev_opt)
    torch.cuda.synchronize()
    return o


def run_ext_oracle(case, seqs=None, **opt):
    h = case.host() if case.q.is_cuda else case
    cu = h.cu_seqlens_q.numpy().astype(np.int64)
    idx = np.arange(h.num_seqs) if seqs is None else np.asarray(seqs)
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in idx]).astype(np.int64)
    sub_cu = np.zeros(len(idx) + 1, np.int32)
    sub_cu[1:] = np.cumsum(cu[idx + 1] - cu[idx])
    ref = oracle.attend_ext(h.q_bits()[rows], sub_cu, h.k_cache.numpy(), h.v_cache.numpy(),
                            h.block_tables.numpy()[idx], h.seq_lens.numpy()[idx], h.scale,
                            h.k_scale, h.v_scale, **opt)
    return ref, rows


def check(case, label, seqs=None, **opt):
    out = run_unified(case, **opt)
    ref, rows = run_ext_oracle(case, seqs, **opt)
    compare(out, ref, label, seqs=rows)
    return out


def slopes_for(hq):
    """ALiBi slopes of the usual geometric form 2^(-8 (h + 1) / Hq)."""
    return (2.0 ** (-8.0 * (np.arange(hq) + 1) / hq)).astype(np.float32)


CASES = [
    (8, 2, [40, 70, 5, 129, 300], [3, 8, 5, 1, 17]),
    (40, 8, [1, 100, 1000, 17, 4], [1, 4, 4, 17, 2]),
    (16, 1, [48, 333, 7], [3, 2, 7]),
]


@pytest.mark.parametrize("hq,hkv,lens,qlens", CASES, ids=lambda x: str(x))
def test_no_options_is_multi_query_bitwise(hq, hkv, lens, qlens):
    import paged_attention_decode_03_amd as pa
    case = workloads.make_multi_case(hq, hkv, lens, qlens, seed=hq + 1).to("cuda")
    a = run_unified(case)
    ks = torch.tensor([case.k_scale], device="cuda")
    vs = torch.tensor([case.v_scale], device="cuda")
    b = pa.paged_multi_query_attention(case.q, case.cu_seqlens_q, max_q(case), case.k_cache,
                                       case.v_cache, case.block_tables, case.seq_lens, case.scale,
                                       ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("window", [1, 2, 7, 16, 40, 100, 5000])
@pytest.mark.parametrize("hq,hkv,lens,qlens", CASES, ids=lambda x: str(x))
def test_sliding_window(hq, hkv, lens, qlens, window):
    case = workloads.make_multi_case(hq, hkv, lens, qlens, seed=hq + window)
    log(f"window {window} {hq}/{hkv} lens={lens} q_lens={qlens}")
    check(case, f"window {window} {hq}/{hkv}", sliding_window=window)


def test_window_of_one_returns_own_value_exactly():
    case = workloads.make_multi_case(8, 2, [40, 70, 5], [3, 8, 5], seed=91, scale_mode="pow2")
    out = run_unified(case, sliding_window=1).float().cpu().double().numpy()
    ref, rows = run_ext_oracle(case, sliding_window=1)
    assert np.array_equal(out[rows], ref)      # V of the own position, a bf16 value


@pytest.mark.parametrize("cap", [0.5, 5.0, 30.0])
@pytest.mark.parametrize("hq,hkv,lens,qlens", CASES, ids=lambda x: str(x))
def test_softcap(hq, hkv, lens, qlens, cap):
    case = workloads.make_multi_case(hq, hkv, lens, qlens, seed=hq + int(cap * 10))
    check(case, f"softcap {cap} {hq}/{hkv}", softcap=cap)


@pytest.mark.parametrize("hq,hkv,lens,qlens", CASES, ids=lambda x: str(x))
def test_alibi(hq, hkv, lens, qlens):
    case = workloads.make_multi_case(hq, hkv, lens, qlens, seed=hq + 5)
    check(case, f"alibi {hq}/{hkv}", alibi_slopes=slopes_for(hq))


@pytest.mark.parametrize("hq,hkv,lens,qlens", CASES, ids=lambda x: str(x))
def test_sinks(hq, hkv, lens, qlens):
    case = workloads.make_multi_case(hq, hkv, lens, qlens, seed=hq + 6)
    sinks = np.linspace(-2.0, 4.0, hq).astype(np.float32)
    check(case, f"sinks {hq}/{hkv}", sinks=sinks)


def test_split_contexts_with_sinks_and_windows():
    """Few sequences and long contexts: the planner splits, so the sink must be
    counted in one partition only and partitions before a window carry no
    weight."""
    case = workloads.make_multi_case(8, 8, [300, 2100, 4000], [200, 37, 16], seed=93,
                                     max_blocks=250)
    sinks = np.linspace(-1.0, 3.0, 8).astype(np.float32)
    check(case, "split, sinks", sinks=sinks)
    check(case, "split, window 128 + sinks", sliding_window=128, sinks=sinks)
    check(case, "split, window 1000", sliding_window=1000)


def test_all_options_together():
    case = workloads.make_multi_case(40, 8, [1, 100, 1000, 17, 4, 2500], [1, 4, 4, 17, 2, 3],
                                     seed=94)
    check(case, "window + softcap + alibi + sinks", sliding_window=64, softcap=20.0,
          alibi_slopes=slopes_for(40), sinks=np.linspace(-1, 1, 40).astype(np.float32))


def test_options_with_three_tiles_an_item():
    """256 sequences at 40/8 with up to 8 queries each (three tiles, one item
    of three tiles per (sequence, kv head)): softcap and ALiBi compiled into
    that item's logit loop, and window with sinks."""
    S = 256
    lens = workloads.ragged_lens(S, hi=300, seed=6)
    g = np.random.default_rng(86)
    ql = np.minimum(np.where(g.random(S) < 0.5, 1, g.choice([2, 5, 7, 8], size=S)), lens).tolist()
    case = workloads.make_multi_case(40, 8, lens, ql, seed=86, max_blocks=32, device="cuda")
    log("options, three tiles an item")
    check(case, "three tiles: softcap + alibi", softcap=5.0, alibi_slopes=slopes_for(40))
    check(case, "three tiles: window + sinks", sliding_window=40,
          sinks=np.linspace(-1.0, 3.0, 40).astype(np.float32))


def test_graph_capture_replays_match_eager():
    import paged_attention_decode_03_amd as pa
    case = workloads.make_multi_case(40, 8, [900, 40, 2000, 1], [4, 4, 3, 1], seed=95).to("cuda")
    ks = torch.tensor([case.k_scale], device="cuda")
    vs = torch.tensor([case.v_scale], device="cuda")
    sinks = torch.linspace(-1, 2, 40, device="cuda")
    out = torch.empty_like(case.q)

    def step():
        pa.paged_attention_unified(case.q, case.cu_seqlens_q, 4, case.k_cache, case.v_cache,
                                   case.block_tables, case.seq_lens, case.scale, ks, vs,
                                   sliding_window=256, softcap=30.0, sinks=sinks, out=out)

    step()
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
        step()
        torch.cuda.synchronize()
    ref, rows = run_ext_oracle(case, sliding_window=256, softcap=30.0, sinks=sinks.cpu().numpy())
    compare(out, ref, "options graph replay", seqs=rows)


def test_one_query_per_sequence_without_row_offsets():
    """cu_seqlens_q=None means one query per sequence: with options it must
    equal the call with row offsets 0, 1, .., S bit for bit, and with
    longest-first dispatch too."""
    import paged_attention_decode_03_amd as pa
    lens = [1, 100, 1000, 17, 4, 2500, 33, 2]
    case = workloads.make_multi_case(40, 8, lens, [1] * len(lens), seed=97).to("cuda")
    ks = torch.tensor([case.k_scale], device="cuda")
    vs = torch.tensor([case.v_scale], device="cuda")
    sinks = torch.linspace(-1, 2, 40, device="cuda")
    args = (case.k_cache, case.v_cache, case.block_tables, case.seq_lens, case.scale, ks, vs)
    opt = dict(sliding_window=64, softcap=20.0, sinks=sinks)
    a = pa.paged_attention_unified(case.q, case.cu_seqlens_q, 1, *args, **opt)
    b = pa.paged_attention_unified(case.q, None, 1, *args, **opt)
    c = pa.paged_attention_unified(case.q, None, 1, *args, longest_first=True, **opt)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    ref, rows = run_ext_oracle(case, sliding_window=64, softcap=20.0, sinks=sinks.cpu().numpy())
    compare(b, ref, "one query per sequence, options", seqs=rows)


def test_options_on_a_ragged_batch_ordered_longest_first():
    """40/8 heads, 256 sequences of 1..4000 tokens with 250-block tables: the
    shape on which calls order longest first by themselves (the work items
    sort the lengths).  Softcap, ALiBi and sinks, one query per sequence and
    two to four, every row against the oracle."""
    S = 256
    lens = workloads.ragged_lens(S, seed=12)
    one = workloads.make_multi_case(40, 8, lens, [1] * S, seed=97, max_blocks=250, device="cuda")
    opts = dict(softcap=30.0, alibi_slopes=slopes_for(40), sinks=np.linspace(-1.0, 2.0, 40).astype(np.float32))
    log("options, ragged 256, one query")
    check(one, "ragged ordered: softcap + alibi + sinks", **opts)
    ql = [min(2 + i % 3, lens[i]) for i in range(S)]
    several = workloads.make_multi_case(40, 8, lens, ql, seed=98, max_blocks=250, device="cuda")
    log("options, ragged 256, 2..4 queries")
    check(several, "ragged ordered, 2..4 queries: softcap + sinks", softcap=30.0, sinks=opts["sinks"])


def test_speculative_decode_with_window_and_sinks():
    """40/8 heads, 256 sequences of 4096 tokens, 4 queries each, a 128-token
    window and per-head sinks: only the last pages of each sequence are read."""
    S, ctx = 256, 4096
    case = workloads.make_multi_case(40, 8, [ctx] * S, [4] * S, seed=96, device="cuda")
    sinks = np.linspace(-1.0, 2.0, 40).astype(np.float32)
    log("spec decode with window 128 + sinks")
    check(case, "spec decode window + sinks", sliding_window=128, sinks=sinks)
