"""The split-KV scratch on the GPU: one buffer per (device, stream), reserved
before capture, never freed while a captured graph may use it, and safe for
calls that run concurrently on two streams."""
import pytest
import torch

import workloads
from parity import compare, log, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_attention_decode_03_amd as pa
    pa.load_library()


def scales(c):
    return (torch.tensor([c.k_scale], device="cuda"), torch.tensor([c.v_scale], device="cuda"))


def decode(c, out, stream=None):
    """One decode call; the case's device scales are made once (outside any capture)."""
    import paged_attention_decode_03_amd as pa
    if "dev_scales" not in c.meta:
        c.meta["dev_scales"] = scales(c)
    ks, vs = c.meta["dev_scales"]
    return pa.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.scale,
                                     ks, vs, out=out, stream=stream)


def test_capture_without_reserved_scratch_is_refused_then_works_after_reserve():
    import paged_attention_decode_03_amd as pa
    c = workloads.make_case(40, 8, [4096, 2000], seed=201, max_blocks=256).to("cuda")
    need = pa.pa_workspace_bytes(2, 40, 8, 256, device=0)
    assert need > 0
    ks, vs = scales(c)
    out = torch.empty_like(c.q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            try:
                pa.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                                          c.scale, ks, vs, out=out)
            except pa.PagedAttentionError as e:
                err = e
    torch.cuda.synchronize()
    assert err is not None and err.code == -5, err
    log(f"refused in capture: {err}")
    pa.pa_workspace_reserve(need, stream=s)
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g2, stream=s):
            pa.paged_decode_attention(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                                      c.scale, ks, vs, out=out)
    out.fill_(3.0)
    g2.replay()
    torch.cuda.synchronize()
    compare(out, run_oracle(c), "capture after reserve")


def test_growing_the_scratch_after_capture_keeps_the_graph_valid():
    """Capture a split call, then grow the same stream's scratch with an eager
    call that needs more, then replay: the graph still uses its own (retired,
    never freed) buffer, and gives the eager result bit for bit every time,
    with eager calls of the larger shape in between."""
    small = workloads.make_case(40, 8, [4096, 1500], seed=202, max_blocks=256).to("cuda")
    big = workloads.make_case(40, 8, [32768, 30000, 9000, 32768], seed=203).to("cuda")
    import paged_attention_decode_03_amd as pa
    assert pa.pa_workspace_bytes(4, 40, 8, big.max_blocks, device=0) > \
        pa.pa_workspace_bytes(2, 40, 8, 256, device=0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out_s = torch.empty_like(small.q)
    out_b = torch.empty_like(big.q)
    with torch.cuda.stream(s):
        decode(small, out_s, s)          # sizes this stream's scratch for the small shape only
        torch.cuda.synchronize()
        eager = out_s.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            decode(small, out_s, s)
    torch.cuda.synchronize()
    for r in range(3):
        with torch.cuda.stream(s):
            decode(big, out_b, s)        # grows the scratch (first time), then reuses it
        torch.cuda.synchronize()
        out_s.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        log(f"replay {r} after growth")
        assert torch.equal(out_s.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
    compare(out_s, run_oracle(small), "graph after scratch growth")
    compare(out_b, run_oracle(big), "the larger shape")


def test_split_calls_on_two_streams_run_concurrently():
    """Two split workloads (one merged in the decode, one by the merge kernel)
    enqueued alternately on two streams with no synchronisation between them:
    each stream has its own partials and arrival counters, so every result
    equals the same call run alone, bit for bit."""
    a = workloads.make_case(32, 8, [1024] * 24, seed=204, max_blocks=64).to("cuda")    # 4 partitions
    b = workloads.make_case(40, 8, [1024] * 16, seed=205, max_blocks=64).to("cuda")    # 8 partitions
    ref_a = decode(a, torch.empty_like(a.q)).clone()
    ref_b = decode(b, torch.empty_like(b.q)).clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a = [torch.empty_like(a.q) for _ in range(8)]
    outs_b = [torch.empty_like(b.q) for _ in range(8)]
    for oa, ob in zip(outs_a, outs_b):
        decode(a, oa, s1)
        decode(b, ob, s2)
    torch.cuda.synchronize()
    for i, (oa, ob) in enumerate(zip(outs_a, outs_b)):
        assert torch.equal(oa.view(torch.int16), ref_a.view(torch.int16)), f"stream 1 call {i}"
        assert torch.equal(ob.view(torch.int16), ref_b.view(torch.int16)), f"stream 2 call {i}"
    compare(ref_a, run_oracle(a), "stream 1 (merge in the decode)")
    compare(ref_b, run_oracle(b), "stream 2 (merge kernel)")
