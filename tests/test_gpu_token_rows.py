"""Parity of the token-row (NHD / flash-style) cache entry point on MI355X.

The same cache bytes are re-laid into the three token-row layouts (separate
[blocks, 16, kv_heads, 128] tensors; one [blocks, 2, 16, kv_heads, 128]
tensor; a packed [blocks, kv_heads, 16, 256] tensor seen through
transpose(1, 2)).  The kernel must return the page-layout kernel's output bit
for bit (same arithmetic, same order) and meet the bound against the fp64
oracle run on the token-row bytes themselves.
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


def run_nhd(case, kview, vview, out=None, stream=None):
    import paged_attention_decode_03_amd as pa
    c = case if case.q.is_cuda else case.to("cuda")
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
    o = pa.paged_decode_attention_nhd(c.q, kview, vview, c.block_tables, c.seq_lens, c.scale, ks,
                                      vs, out=out, stream=stream)
    torch.cuda.synchronize()
    return o


def gpu_views(case, layout):
    """Token-row views built on the GPU (views of one allocation where the
    layout keeps K and V together)."""
    c = case if case.q.is_cuda else case.to("cuda")
    return workloads.token_row_views(c, layout)


def oracle_rows(case, layout, seqs=None):
    h = case.host() if case.q.is_cuda else case
    kv, vv = workloads.token_row_views(h, layout)
    kb, st = workloads.strided_buffer(kv)
    vb, st2 = workloads.strided_buffer(vv)
    assert st == st2
    idx = np.arange(h.num_seqs) if seqs is None else np.asarray(seqs)
    return oracle.decode_strided(h.q_bits()[idx], kb, vb, *st, h.num_kv_heads,
                                 h.block_tables.numpy()[idx], h.seq_lens.numpy()[idx], h.scale,
                                 h.k_scale, h.v_scale)


SMALL = [
    (8, 2, [1, 17, 33, 64]),
    (40, 8, [1, 100, 1000, 17]),
    (32, 4, [64, 65, 129, 255, 256, 257]),
    (16, 1, [1, 333, 48]),
    (8, 8, [7, 90, 16]),
    (40, 8, [4096, 33]),          # few work items: split contexts and the merge
    (8, 2, [0, 37, 0, 1]),        # empty sequences
]


@pytest.mark.parametrize("layout", workloads.TOKEN_ROW_LAYOUTS)
@pytest.mark.parametrize("hq,hkv,lens", SMALL, ids=lambda x: str(x))
def test_small_layouts_match_page_kernel_and_oracle(hq, hkv, lens, layout):
    case = workloads.make_case(hq, hkv, lens, seed=hq * 5 + hkv, max_blocks=max(4, (max(lens) + 15) // 16))
    kv, vv = gpu_views(case, layout)
    log(f"token rows {layout} {hq}/{hkv} lens={lens} strides={kv.stride()[:3]}")
    got = run_nhd(case, kv, vv)
    ref_page = run_gpu(case)
    assert torch.equal(got.view(torch.int16), ref_page.view(torch.int16)), "differs from page layout"
    compare(got, oracle_rows(case, layout), f"token rows {layout} {hq}/{hkv}")


def test_graph_capture_replays_match_eager():
    import paged_attention_decode_03_amd as pa
    case = workloads.make_case(40, 8, [4096, 33, 1000], seed=71).to("cuda")
    kv, vv = gpu_views(case, "combined")
    ks = torch.tensor([case.k_scale], device="cuda")
    vs = torch.tensor([case.v_scale], device="cuda")
    out = torch.empty_like(case.q)

    def step():
        pa.paged_decode_attention_nhd(case.q, kv, vv, case.block_tables, case.seq_lens, case.scale,
                                      ks, vs, out=out)

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
    compare(out, oracle_rows(case, "combined"), "token rows graph replay")


def test_binding_rejects_mismatched_views():
    import paged_attention_decode_03_amd as pa
    case = workloads.make_case(8, 2, [20], seed=72).to("cuda")
    kv, vv = gpu_views(case, "nhd")
    with pytest.raises(ValueError):
        pa.paged_decode_attention_nhd(case.q, kv, vv[:, :, :1], case.block_tables, case.seq_lens,
                                      case.scale, case.k_scale, case.v_scale)
    with pytest.raises(TypeError):
        pa.paged_decode_attention_nhd(case.q, kv.transpose(2, 3), vv.transpose(2, 3),
                                      case.block_tables, case.seq_lens, case.scale, case.k_scale,
                                      case.v_scale)


@pytest.mark.parametrize("layout", workloads.TOKEN_ROW_LAYOUTS)
def test_mid_batch_splits_into_eight_items_per_cu(layout):
    """64 sequences x 1024 tokens at 40/8: one partition would leave two work
    items per CU; the page layout splits in two, token rows into four (eight
    items per CU, still eight kv heads a workgroup: 256 workgroups).  Bit for
    bit the page layout's split entry point with the same partitions, and the
    oracle's result on every sequence."""
    import paged_attention_decode_03_amd as pa
    case = workloads.dense(40, 8, 64, 1024, seed=9, device="cuda")
    assert pa.pa_decode_plan(64, 40, 8, 64, 256)[:2] == (2, 32)
    kv, vv = gpu_views(case, layout)
    got = run_nhd(case, kv, vv)
    del kv, vv
    ref_split = run_gpu(case, 16)
    log(f"token rows {layout} 64 x 1024")
    assert torch.equal(got.view(torch.int16), ref_split.view(torch.int16)), "differs from 4-partition page layout"
    compare(got, oracle_rows(case, layout), f"token rows {layout} 64 x 1024")


def test_small_batch_groups_fewer_kv_heads():
    """16 sequences x 1024 tokens at 40/8 (8 partitions, 1024 work items): four
    kv heads a workgroup keep a workgroup per CU; the result is the page
    layout's bit for bit."""
    case = workloads.dense(40, 8, 16, 1024, seed=10, device="cuda")
    kv, vv = gpu_views(case, "nhd")
    got = run_nhd(case, kv, vv)
    ref_page = run_gpu(case)
    log("token rows nhd 16 x 1024")
    assert torch.equal(got.view(torch.int16), ref_page.view(torch.int16))
    compare(got, oracle_rows(case, "nhd"), "token rows nhd 16 x 1024")


def test_target_shape_every_layout():
    """40/8 heads, 256 sequences x 4096 tokens (the benchmark's shape) in all
    three token-row layouts: each equals the page-layout kernel bit for bit
    and meets the bound against the token-row oracle on every sequence (the
    oracle's layouts agree bit for bit, so it runs once, on NHD)."""
    hq, hkv, S, ctx = workloads.TARGET
    case = workloads.dense(hq, hkv, S, ctx, seed=3, device="cuda")
    ref_page = run_gpu(case)
    ref = oracle_rows(case, "nhd")
    for layout in workloads.TOKEN_ROW_LAYOUTS:
        kv, vv = gpu_views(case, layout)
        got = run_nhd(case, kv, vv)
        del kv, vv
        log(f"token rows {layout} target")
        assert torch.equal(got.view(torch.int16), ref_page.view(torch.int16)), f"{layout}: differs from page layout"
        compare(got, ref, f"token rows {layout} target")
