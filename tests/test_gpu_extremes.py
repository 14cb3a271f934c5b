"""Sizes at the ends of the ranges: a context of 131072 tokens, 4096 short
sequences, and caches past 4 GiB whose used pages lie at the far end (64-bit
page offsets), each against the fp64 oracle or, for the large caches, bit for
bit against the same pages placed at the front of a small cache."""
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
    pa.load_library()


def test_one_sequence_of_131072_tokens():
    """8192 blocks in one table row: 128 partitions of 64 blocks, merged by the
    merge kernel."""
    import paged_attention_decode_03_amd as pa
    assert pa.pa_decode_plan(1, 40, 8, 8192, 256)[:2] == (128, 64)
    case = workloads.make_case(40, 8, [131072], seed=501, device="cuda")
    log("one sequence of 131072 tokens")
    compare(run_gpu(case), run_oracle(case), "ctx 131072")


def test_4096_short_ragged_sequences():
    """32768 work items of at most 8 blocks (contexts 1..128, a 16-block
    table), and the same with longest-first dispatch (beyond what a work item
    sorts itself: the order kernel)."""
    import paged_attention_decode_03_amd as pa
    lens = workloads.ragged_lens(4096, lo=1, hi=128, seed=17)
    case = workloads.make_case(32, 8, lens, seed=502, device="cuda", max_blocks=16)
    out = run_gpu(case)
    ks = torch.tensor([case.k_scale], device="cuda")
    vs = torch.tensor([case.v_scale], device="cuda")
    lpt = pa.paged_attention_unified(case.q, None, 1, case.k_cache, case.v_cache, case.block_tables,
                                     case.seq_lens, case.scale, ks, vs, longest_first=True)
    torch.cuda.synchronize()
    log("4096 short sequences")
    assert torch.equal(out.view(torch.int16), lpt.view(torch.int16))
    compare(out, run_oracle(case), "4096 sequences x 1..128 tokens")


@pytest.mark.parametrize("entry", ["page", "split", "token_rows"])
def test_pages_past_4_gib_of_cache(entry):
    """Caches of 2^19 blocks x 8 kv heads (8 GiB each): the used pages are
    copied to the last blocks, the table is rewritten to point there, and the
    result must equal the compact case's bit for bit (byte offsets past 2^32
    in the page address)."""
    import paged_attention_decode_03_amd as pa
    small = workloads.make_case(40, 8, [4096, 1000, 17, 2500], seed=503, device="cuda", max_blocks=256)
    NB = 1 << 19
    used = small.block_tables.flatten().unique()
    far = NB - 1 - torch.arange(used.numel(), device="cuda")          # the last blocks
    remap = torch.full((small.k_cache.shape[0],), -1, dtype=torch.int64, device="cuda")
    remap[used.long()] = far
    big_k = torch.empty((NB,) + tuple(small.k_cache.shape[1:]), dtype=torch.uint8, device="cuda")
    big_v = torch.empty((NB,) + tuple(small.v_cache.shape[1:]), dtype=torch.uint8, device="cuda")
    big_k[far] = small.k_cache[used.long()]
    big_v[far] = small.v_cache[used.long()]
    big_bt = remap[small.block_tables.long()].to(torch.int32)
    assert int(big_bt.max()) * 8 * 2048 > (1 << 32)
    big = workloads.Case("far pages", small.q, big_k, big_v, big_bt, small.seq_lens, small.scale,
                         small.k_scale, small.v_scale)
    ks = torch.tensor([small.k_scale], device="cuda")
    vs = torch.tensor([small.v_scale], device="cuda")
    if entry == "page":
        a, b = run_gpu(small), run_gpu(big)
    elif entry == "split":
        a, b = run_gpu(small, 8), run_gpu(big, 8)
    else:
        ka, va = workloads.token_row_views(small, "nhd")
        kb, vb = workloads.token_row_views(big, "nhd")
        a = pa.paged_decode_attention_nhd(small.q, ka, va, small.block_tables, small.seq_lens,
                                          small.scale, ks, vs)
        b = pa.paged_decode_attention_nhd(big.q, kb, vb, big.block_tables, big.seq_lens, big.scale,
                                          ks, vs)
        torch.cuda.synchronize()
        del ka, va, kb, vb
    log(f"pages past 4 GiB ({entry})")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    if entry == "page":
        compare(a, run_oracle(small), "compact pages")
    del big_k, big_v
    torch.cuda.empty_cache()
