"""paged_decode_attention_desc on the GPU: strided views of q, the block table
and the caches give the flat entry point's result on dense copies, bit for bit
(the same kernels and arithmetic), and meet the bound against the oracle."""
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


def strided_views(c, pad_heads=3, pad_blocks=5):
    """q as a slice of [S, Hq + pad, 128]; the block table as the first W
    columns of a wider one; K and V as the halves of one [NB, 2, Hkv, 2048]
    tensor (block stride 2 * Hkv * 2048 bytes), V seen through its 5-D view."""
    S, Hq, _ = c.q.shape
    NB, Hkv = c.k_cache.shape[:2]
    qb = torch.zeros(S, Hq + pad_heads, 128, dtype=torch.bfloat16, device="cuda")
    qb[:, :Hq] = c.q
    bt = torch.full((S, c.max_blocks + pad_blocks), -7, dtype=torch.int32, device="cuda")
    bt[:, :c.max_blocks] = c.block_tables
    kv = torch.empty(NB, 2, Hkv, 2048, dtype=torch.uint8, device="cuda")
    kv[:, 0] = c.k_cache.reshape(NB, Hkv, 2048)
    kv[:, 1] = c.v_cache.reshape(NB, Hkv, 2048)
    k = kv[:, 0].view(torch.float8_e4m3fn).unflatten(2, (8, 16, 16))
    v = kv[:, 1].view(torch.float8_e4m3fn).unflatten(2, (1, 128, 16))
    return qb[:, :Hq], k, v, bt[:, :c.max_blocks]


@pytest.mark.parametrize("lens", [[1, 17, 33, 64], [4096, 100, 1, 2000], [1024] * 64],
                         ids=["tiny", "split", "unsplit"])
def test_strided_views_match_the_dense_call_bitwise(lens):
    import paged_attention_decode_03_amd as pa
    c = workloads.make_case(40, 8, lens, seed=300 + len(lens), max_blocks=256).to("cuda")
    q, k, v, bt = strided_views(c)
    assert q.stride(0) == 43 * 128 and bt.stride(0) == 261 and k.stride(0) == 2 * 8 * 2048
    ks = torch.tensor([c.k_scale], device="cuda")
    vs = torch.tensor([c.v_scale], device="cuda").reshape(())   # a 0-dim scale
    out = pa.paged_decode_attention_desc(q, k, v, bt, c.seq_lens, c.scale, ks, vs)
    dense = run_gpu(c)
    torch.cuda.synchronize()
    log(f"descriptor form, {len(lens)} sequences")
    assert torch.equal(out.view(torch.int16), dense.view(torch.int16))
    compare(out, run_oracle(c), f"descriptor form {len(lens)} seqs")


def test_dtype_and_layout_errors_come_from_the_library():
    import paged_attention_decode_03_amd as pa
    c = workloads.make_case(8, 2, [20, 5], seed=310).to("cuda")
    ks = torch.tensor([c.k_scale], device="cuda")
    vs = torch.tensor([c.v_scale], device="cuda")
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.paged_decode_attention_desc(c.q.float(), c.k_cache, c.v_cache, c.block_tables,
                                       c.seq_lens, c.scale, ks, vs,
                                       out=torch.empty_like(c.q))
    assert e.value.code == -7
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.paged_decode_attention_desc(c.q.transpose(1, 2).contiguous().transpose(1, 2), c.k_cache,
                                       c.v_cache, c.block_tables, c.seq_lens, c.scale, ks, vs)
    assert e.value.code == -8
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.paged_decode_attention_desc(c.q, c.k_cache, c.v_cache, c.block_tables.to(torch.int64),
                                       c.seq_lens, c.scale, ks, vs)
    assert e.value.code == -7
