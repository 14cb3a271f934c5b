"""paged_decode_attention_noalloc (split-KV scratch in the library's fixed
per-GPU array) against paged_decode_attention_split (scratch the library
allocates), through the C ABI: the same kernels and plan, so the same bits,
and the bound against the oracle."""
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


def both(case, ppp=0):
    """(noalloc output, allocating split output) for one case."""
    import paged_attention_decode_03_amd as pa
    c = case.to("cuda")
    ks = torch.tensor([c.k_scale], device="cuda")
    vs = torch.tensor([c.v_scale], device="cuda")
    args = (c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens, c.scale, ks, vs)
    out_fixed = torch.full_like(c.q, 7.0)
    pa.paged_decode_attention_noalloc(*args, ppp, out=out_fixed)
    out_alloc = pa.paged_decode_attention_split(*args, ppp)
    torch.cuda.synchronize()
    return out_fixed, out_alloc


# (label, case, pages per partition): two in a row, the second smaller, for
# each way the scratch is used
PAIRS = [
    ("merge kernel (8 partitions), then a smaller batch merged in the decode (4)",
     lambda: workloads.make_case(40, 8, [4096] * 16, seed=401, max_blocks=256), 0,
     lambda: workloads.make_case(32, 8, [1024] * 24, seed=402, max_blocks=64), 0),
    ("merge in the decode, then a smaller one",
     lambda: workloads.make_case(32, 8, [1024, 0, 17, 1000] * 6, seed=403, max_blocks=64), 0,
     lambda: workloads.make_case(8, 2, [33, 64, 1, 50], seed=404, max_blocks=4), 1),
    ("forced small partitions (64 of 4 blocks), then a smaller batch",
     lambda: workloads.make_case(40, 8, [4096, 4000, 100, 1], seed=405, max_blocks=256), 4,
     lambda: workloads.make_case(40, 8, [2048, 5], seed=406, max_blocks=128), 8),
]


@pytest.mark.parametrize("idx", range(len(PAIRS)), ids=[p[0][:40] for p in PAIRS])
def test_noalloc_matches_the_allocating_entry_point(idx):
    label, first, ppp1, second, ppp2 = PAIRS[idx]
    for n, (make, ppp) in enumerate(((first, ppp1), (second, ppp2))):
        case = make()
        fixed, alloc = both(case, ppp)
        log(f"noalloc call {n + 1} ({label}): {case.num_seqs} sequences, ppp={ppp}")
        assert torch.equal(fixed.view(torch.int16), alloc.view(torch.int16)), f"call {n + 1}"
        compare(fixed, run_oracle(case), f"noalloc call {n + 1}")


def test_noalloc_unsplit_batch_needs_no_scratch():
    case = workloads.make_case(40, 8, [300] * 64, seed=407)
    fixed, alloc = both(case)
    assert torch.equal(fixed.view(torch.int16), alloc.view(torch.int16))


def test_noalloc_rejects_a_plan_beyond_its_array():
    """256 sequences in partitions of one block need 1.36 GB of partials:
    PA_ERR_WORKSPACE, and nothing is launched (out keeps its contents)."""
    import paged_attention_decode_03_amd as pa
    c = workloads.make_case(40, 8, [64] * 256, seed=408, max_blocks=256).to("cuda")
    ks = torch.tensor([c.k_scale], device="cuda")
    vs = torch.tensor([c.v_scale], device="cuda")
    out = torch.full_like(c.q, 3.0)
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.paged_decode_attention_noalloc(c.q, c.k_cache, c.v_cache, c.block_tables, c.seq_lens,
                                          c.scale, ks, vs, 1, out=out)
    torch.cuda.synchronize()
    assert e.value.code == -5 and "fixed array" in str(e.value)
    assert bool((out == 3.0).all())
