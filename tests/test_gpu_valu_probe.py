"""The benchmark's VALU decode probe (dot products on the vector ALUs, timed
beside the MFMA decode by `bench.py --valu-compare`) computes the same
attention: checked against the fp64 oracle for every group size it takes,
ragged and empty contexts, and on the full target workload."""
import pytest
import torch

import workloads
from parity import compare, log, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    return bench.probe_library()


def run_probe(lib, case):
    import bench
    ks = torch.tensor([case.k_scale], dtype=torch.float32, device="cuda")
    vs = torch.tensor([case.v_scale], dtype=torch.float32, device="cuda")
    out = torch.full_like(case.q, float("nan"))
    stream = torch.cuda.current_stream()
    assert bench.valu_decode(lib, case, ks, vs, out, stream) == 0
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("group", range(1, 9))
def test_valu_probe_each_group_size(probe, group):
    """Contexts 0 (an all-zero row), 1, 15, 16, 17, 100 and 333 tokens: the
    last page's masked tokens and V bytes, several ring rounds."""
    lens = [0, 1, 15, 16, 17, 100, 333]
    case = workloads.make_case(2 * group, 2, lens, seed=700 + group, device="cuda")
    out = run_probe(probe, case)
    log(f"VALU probe, group {group}")
    compare(out, run_oracle(case), f"valu probe G={group}")
    assert (out[0] == 0).all()


def test_valu_probe_bad_block_id_reads_zero_page(probe):
    """A block id outside the caches reads as an all-zero page (as in the
    decode): the same output as the case with that entry pointing at a zero
    block."""
    case = workloads.make_case(40, 8, [40, 64], seed=710, device="cuda", extra_blocks=2)
    nb = case.k_cache.shape[0]
    used = {int(b) for s, n in ((0, 3), (1, 4)) for b in case.block_tables[s, :n].tolist()}
    zero_id = next(b for b in range(nb) if b not in used)
    case.k_cache[zero_id].zero_()
    case.v_cache[zero_id].zero_()
    a_bt = case.block_tables.clone()
    a_bt[1, 2] = zero_id
    b_bt = case.block_tables.clone()
    b_bt[1, 2] = nb + 12345
    case.block_tables = a_bt
    a = run_probe(probe, case)
    case.block_tables = b_bt
    b = run_probe(probe, case)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_valu_probe_target_workload(probe):
    """40/8 heads, 256 sequences x 4096 tokens: every sequence against the
    oracle (what the comparison times)."""
    hq, hkv, s, ctx = workloads.TARGET
    case = workloads.dense(hq, hkv, s, ctx, seed=0, device="cuda")
    out = run_probe(probe, case)
    log("VALU probe, target workload")
    compare(out, run_oracle(case), "valu probe target")
