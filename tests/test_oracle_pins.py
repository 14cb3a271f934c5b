"""Pins of the fp64 oracle against things other than itself (CPU only).

* fp8 decoding: torch's own float8_e4m3fn conversion on all 256 codes, and
  values worked out by hand from the OCP e4m3fn definition.
* Attention: two independent dense routes on K/V gathered by array indexing
  (torch's scaled_dot_product_attention in fp64, and a numpy softmax), closed
  forms (one token, constant V, zero query, a hand-worked two-token fixture),
  and invariants (physical block placement, sequence order, NaN poison in
  memory the method must not read, exact power-of-two scalings).
* The split-KV log-sum-exp merge against the unsplit definition.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# fp8 / bf16 decoding

def test_fp8_table_matches_torch_all_codes(oracle_lib):
    ours = oracle.fp8_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # signed zero survives
    assert math.copysign(1.0, ours[0x80]) == -1.0


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x30, 0.5), (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x77, 240.0),
    (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0), (0x81, -(2.0 ** -9)),
])
def test_fp8_values_from_format_definition(oracle_lib, code, value):
    assert oracle.fp8_e4m3fn_value(code) == value


def test_fp8_nan_codes(oracle_lib):
    t = oracle.fp8_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2


def test_bf16_value_and_rounding(oracle_lib):
    assert oracle.bf16_value(0x3F80) == 1.0
    assert oracle.bf16_value(0xC000) == -2.0
    assert oracle.bf16_value(0x0001) == 2.0 ** -133
    # ties go to even, both directions
    bits = oracle.bf16_rne(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -30]))
    assert list(bits) == [0x3F80, 0x3F82, 0xBF80, 0x3F81]
    # subnormal step, zero, overflow, NaN
    assert list(oracle.bf16_rne(np.array([2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -133, 0.0]))) == [1, 0, 2, 0]
    assert list(oracle.bf16_rne(np.array([3.5e38, -3.5e38]))) == [0x7F80, 0xFF80]
    assert oracle.bf16_rne(np.array([float("nan")]))[0] == 0x7FC0


def test_bf16_rne_matches_torch_on_float32_exact_values(oracle_lib):
    g = torch.Generator().manual_seed(1)
    x = (torch.randn(4096, generator=g) * torch.exp2(torch.randint(-20, 20, (4096,), generator=g).float()))
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.bf16_rne(x.double().numpy())
    assert np.array_equal(ours, ref)


# --------------------------------------------------------------------------
# independent dense routes (gather by array indexing, dequantise with torch)

def gather_dense(case, s):
    """K, V of sequence s as float64 [L, Hkv, 128] via numpy fancy indexing."""
    L = int(case.seq_lens[s])
    t = np.arange(L)
    blocks = case.block_tables.numpy()[s, t // 16]
    slots = t % 16
    kb = case.k_cache.numpy()[blocks, :, :, slots, :]      # [L, Hkv, 8, 16]
    vb = case.v_cache.numpy()[blocks, :, :, slots]         # [L, Hkv, 128]
    kb = kb.reshape(L, case.num_kv_heads, 128)
    K = torch.from_numpy(np.ascontiguousarray(kb)).view(torch.float8_e4m3fn).to(torch.float64) * case.k_scale
    V = torch.from_numpy(np.ascontiguousarray(vb)).view(torch.float8_e4m3fn).to(torch.float64) * case.v_scale
    return K, V


def sdpa_reference(case):
    S, Hq, Hkv = case.num_seqs, case.num_heads, case.num_kv_heads
    G = Hq // Hkv
    out = np.zeros((S, Hq, 128))
    q = case.q.to(torch.float64)
    for s in range(S):
        if int(case.seq_lens[s]) == 0:
            continue
        K, V = gather_dense(case, s)
        Kr = K.permute(1, 0, 2).repeat_interleave(G, dim=0)   # [Hq, L, 128]
        Vr = V.permute(1, 0, 2).repeat_interleave(G, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(
            q[s][:, None, :].contiguous(), Kr.contiguous(), Vr.contiguous(), scale=case.scale)
        out[s] = o[:, 0, :].numpy()
    return out


def numpy_reference(case):
    S, Hq, Hkv = case.num_seqs, case.num_heads, case.num_kv_heads
    G = Hq // Hkv
    out = np.zeros((S, Hq, 128))
    q = case.q.to(torch.float64).numpy()
    for s in range(S):
        if int(case.seq_lens[s]) == 0:
            continue
        K, V = gather_dense(case, s)
        K, V = K.numpy(), V.numpy()
        for h in range(Hq):
            z = case.scale * (K[:, h // G, :] @ q[s, h])
            w = np.exp(z - z.max())
            out[s, h] = (w[:, None] * V[:, h // G, :]).sum(0) / w.sum()
    return out


def run_oracle(case, **kw):
    return oracle.decode(case.q_bits(), case.k_cache.numpy(), case.v_cache.numpy(),
                         case.block_tables.numpy(), case.seq_lens.numpy(), case.scale,
                         case.k_scale, case.v_scale, **kw)


def small_cases():
    yield workloads.tiny(0)
    yield workloads.tiny(5)
    yield workloads.make_case(16, 2, [3, 16, 31, 100, 257], 3, name="g8")
    yield workloads.make_case(5, 1, [1, 2, 15, 16, 17, 48], 4, name="g5")
    yield workloads.make_case(16, 1, [70, 1], 7, name="g16")
    yield workloads.make_case(4, 4, [40, 0, 9], 8, max_blocks=5, name="mha_with_empty")
    for (hq, hkv) in workloads.RAGGED_LAYOUTS:
        lens = workloads.ragged_lens(6, seed=hq + hkv)
        yield workloads.make_case(hq, hkv, [min(x, 600) for x in lens], 11,
                                  name=f"ragged_sub_{hq}x{hkv}")


@pytest.mark.parametrize("case", list(small_cases()), ids=lambda c: c.name)
def test_oracle_matches_sdpa_fp64(oracle_lib, case):
    ours = run_oracle(case)
    ref = sdpa_reference(case)
    assert np.isfinite(ours).all()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", list(small_cases())[:4], ids=lambda c: c.name)
def test_oracle_matches_numpy_softmax(oracle_lib, case):
    np.testing.assert_allclose(run_oracle(case), numpy_reference(case), rtol=0, atol=1e-12)


def test_oracle_threads_do_not_change_result(oracle_lib):
    case = workloads.make_case(16, 2, [33, 500, 7], 2)
    assert np.array_equal(run_oracle(case, num_threads=1), run_oracle(case, num_threads=4))


# --------------------------------------------------------------------------
# closed forms

def _two_token_fixture():
    kv = {}
    with open(os.path.join(GOLDEN, "two_token_case.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                kv[k] = v
    return kv


def test_golden_two_token_hand_worked(oracle_lib):
    kv = _two_token_fixture()
    nb = int(kv["num_blocks"])
    p = int(kv["physical_block"])
    q = np.zeros((1, 1, 128), np.uint16)
    q[0, 0, 0] = int(kv["q_dim0_bits"], 16)
    k = np.zeros((nb, 1, 8, 16, 16), np.uint8)
    v = np.zeros((nb, 1, 128, 16), np.uint8)
    k[p, 0, 0, 0, 0] = int(kv["k_tok0_dim0"], 16)
    k[p, 0, 0, 1, 0] = int(kv["k_tok1_dim0"], 16)
    v[p, 0, :, 0] = int(kv["v_tok0"], 16)
    v[p, 0, :, 1] = int(kv["v_tok1"], 16)
    k[p, 0, :, 2:, :] = 0x7F   # slots past seq_len hold NaN and must not be read
    v[p, 0, :, 2:] = 0x7F
    bt = np.array([[p]], np.int32)
    sl = np.array([int(kv["seq_len"])], np.int32)
    out = oracle.decode(q, k, v, bt, sl, float(kv["scale"]), float(kv["k_scale"]), float(kv["v_scale"]))
    expected = float(kv["expected_every_dim"])
    np.testing.assert_allclose(out[0, 0], expected, rtol=1e-15, atol=0)
    # the same number from the closed form sigma(z0 - z1) V0 + (1 - sigma) V1
    sig = 1.0 / (1.0 + math.exp(-(2.0 - 1.0)))
    assert abs(expected - (sig * 1.0 + (1 - sig) * 2.0)) < 1e-15


def test_one_token_context_returns_v0(oracle_lib):
    case = workloads.make_case(8, 2, [1, 1, 17], 21)
    out = run_oracle(case)
    for s in range(3):
        L = int(case.seq_lens[s])
        _, V = gather_dense(case, s)
        if L == 1:
            for h in range(8):
                assert np.array_equal(out[s, h], V[0, h // 4].numpy())


def test_constant_v_gives_that_v(oracle_lib):
    case = workloads.make_case(8, 2, [5, 64, 200], 22)
    v = case.v_cache.clone()
    code = 0x3B   # 1.375
    for s in range(3):
        L = int(case.seq_lens[s])
        for b in range((L + 15) // 16):
            v[int(case.block_tables[s, b])] = code
    case.v_cache = v
    out = run_oracle(case)
    np.testing.assert_allclose(out, 1.375 * case.v_scale, rtol=1e-13, atol=0)  # n-term summation rounding


def test_zero_query_gives_mean_of_v(oracle_lib):
    case = workloads.make_case(8, 2, [3, 50, 129], 23)
    case.q = torch.zeros_like(case.q)
    out = run_oracle(case)
    for s in range(3):
        _, V = gather_dense(case, s)
        mean = V.mean(0).numpy()               # [Hkv, 128]
        for h in range(8):
            np.testing.assert_allclose(out[s, h], mean[h // 4], rtol=0, atol=1e-13)


def test_identical_heads_give_identical_outputs(oracle_lib):
    case = workloads.make_case(8, 2, [77], 24)
    q = case.q.clone()
    q[0, 1:4] = q[0, 0]
    case.q = q
    out = run_oracle(case)
    for h in range(1, 4):
        assert np.array_equal(out[0, h], out[0, 0])
    assert not np.array_equal(out[0, 4], out[0, 0])


# --------------------------------------------------------------------------
# invariants

def test_block_placement_invariance(oracle_lib):
    case = workloads.make_case(8, 2, [33, 90, 16, 1], 31)
    base = run_oracle(case)
    NB = case.k_cache.shape[0]
    g = torch.Generator().manual_seed(99)
    perm = torch.randperm(NB, generator=g)          # block b moves to perm[b]
    k2 = torch.empty_like(case.k_cache)
    v2 = torch.empty_like(case.v_cache)
    k2[perm] = case.k_cache
    v2[perm] = case.v_cache
    bt2 = perm[case.block_tables.long()].to(torch.int32)
    moved = workloads.Case("moved", case.q, k2, v2, bt2, case.seq_lens, case.scale,
                           case.k_scale, case.v_scale)
    assert np.array_equal(run_oracle(moved), base)


def test_sequence_order_permutes_outputs(oracle_lib):
    case = workloads.make_case(8, 2, [33, 90, 16, 1, 0], 32, max_blocks=8)
    base = run_oracle(case)
    order = torch.tensor([3, 0, 4, 2, 1])
    perm_case = workloads.Case("perm", case.q[order], case.k_cache, case.v_cache,
                               case.block_tables[order], case.seq_lens[order],
                               case.scale, case.k_scale, case.v_scale)
    assert np.array_equal(run_oracle(perm_case), base[order.numpy()])


def test_nan_poison_outside_context_is_never_read(oracle_lib):
    lens = [1, 17, 33, 64, 5]
    a = workloads.make_case(8, 2, lens, 33, max_blocks=6, poison=True)
    b = workloads.make_case(8, 2, lens, 33, max_blocks=6, poison=False)
    assert (a.k_cache == 0x7F).sum() > 0
    ra, rb = run_oracle(a), run_oracle(b)
    assert np.isfinite(ra).all()
    assert np.array_equal(ra, rb)


def test_nan_inside_context_propagates_to_its_head_only(oracle_lib):
    case = workloads.make_case(8, 2, [20, 20], 34)
    q = case.q.clone()
    q[1, 5, 7] = float("nan")
    case.q = q
    out = run_oracle(case)
    assert np.isnan(out[1, 5]).all()
    mask = np.ones((2, 8), bool)
    mask[1, 5] = False
    assert np.isfinite(out[mask]).all()


def test_power_of_two_scalings_are_exact(oracle_lib):
    case = workloads.make_case(8, 2, [40, 3], 35)
    base = run_oracle(case)
    v2 = run_oracle(workloads.Case("v2", case.q, case.k_cache, case.v_cache, case.block_tables,
                                   case.seq_lens, case.scale, case.k_scale, 2 * case.v_scale))
    assert np.array_equal(v2, 2 * base)
    k2 = run_oracle(workloads.Case("k2", case.q, case.k_cache, case.v_cache, case.block_tables,
                                   case.seq_lens, case.scale, 2 * case.k_scale, case.v_scale))
    s2 = run_oracle(workloads.Case("s2", case.q, case.k_cache, case.v_cache, case.block_tables,
                                   case.seq_lens, 2 * case.scale, case.k_scale, case.v_scale))
    assert np.array_equal(k2, s2)
    assert not np.array_equal(k2, base)


def test_empty_sequence_gives_zeros_and_overlong_is_rejected(oracle_lib):
    case = workloads.make_case(4, 1, [0, 9], 36, max_blocks=2)
    out = run_oracle(case)
    assert np.array_equal(out[0], np.zeros((4, 128)))
    bad = case.seq_lens.clone()
    bad[1] = 33            # 2 blocks hold at most 32 tokens
    with pytest.raises(ValueError):
        oracle.decode(case.q_bits(), case.k_cache.numpy(), case.v_cache.numpy(),
                      case.block_tables.numpy(), bad.numpy(), case.scale, case.k_scale, case.v_scale)


# --------------------------------------------------------------------------
# split-KV merge

@pytest.mark.parametrize("tpp", [16, 48, 64, 1000])
def test_partition_merge_equals_unsplit(oracle_lib, tpp):
    """Partitions cut the 64-block table row (1024 tokens), so every context
    shorter than the row leaves empty partitions; the merge must skip them
    and still equal the unsplit definition."""
    case = workloads.make_case(10, 2, [1, 15, 16, 17, 100, 1024, 0, 333], 41, max_blocks=64)
    whole = run_oracle(case)
    split, empty = oracle.decode_partitioned(case.q_bits(), case.k_cache.numpy(),
                                             case.v_cache.numpy(), case.block_tables.numpy(),
                                             case.seq_lens.numpy(), case.scale, case.k_scale,
                                             case.v_scale, tpp, return_empty=True)
    np.testing.assert_allclose(split, whole, rtol=0, atol=1e-12)
    # empty partitions per head row: ceil(1024 / tpp) minus those holding a token
    nparts = -(-1024 // tpp)
    expect = sum(nparts - (-(-int(n) // tpp)) for n in case.seq_lens) * case.num_heads
    assert empty == expect
    if tpp < 1024:
        assert empty > 0


def test_partition_merge_of_an_empty_context_is_zero(oracle_lib):
    """A row whose every partition is empty gives an all-zero output (no
    -inf - (-inf) in the merge)."""
    case = workloads.make_case(4, 1, [0, 0, 5], 42, max_blocks=8)
    split = oracle.decode_partitioned(case.q_bits(), case.k_cache.numpy(), case.v_cache.numpy(),
                                      case.block_tables.numpy(), case.seq_lens.numpy(),
                                      case.scale, case.k_scale, case.v_scale, 16)
    assert np.isfinite(split).all()
    assert not split[:2].any()
    np.testing.assert_allclose(split, run_oracle(case), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# per-slot scale tables

def test_slot_scales_equal_to_tensor_scales_reproduce_per_tensor_decode(oracle_lib):
    case = workloads.make_case(8, 2, [1, 17, 90, 33], 51)
    NB = case.k_cache.shape[0]
    ks = np.full((NB, 2, 16), case.k_scale, np.float32)
    vs = np.full((NB, 2, 16), case.v_scale, np.float32)
    a = oracle.decode_slot_scales(case.q_bits(), case.k_cache.numpy(), case.v_cache.numpy(),
                                  case.block_tables.numpy(), case.seq_lens.numpy(), case.scale, ks, vs)
    assert np.array_equal(a, run_oracle(case))


@pytest.mark.parametrize("hq,hkv,lens", [(8, 2, [1, 17, 33, 64]), (40, 8, [100, 3, 257]),
                                         (16, 1, [48, 1])])
def test_slot_scales_match_sdpa(oracle_lib, hq, hkv, lens):
    case = workloads.make_case(hq, hkv, lens, 52, scale_mode="per_slot")
    ks, vs = case.k_slot_scales.numpy(), case.v_slot_scales.numpy()
    assert np.isnan(ks).any()            # unused slots carry NaN scales
    ours = oracle.decode_slot_scales(case.q_bits(), case.k_cache.numpy(), case.v_cache.numpy(),
                                     case.block_tables.numpy(), case.seq_lens.numpy(), case.scale,
                                     ks, vs)
    assert np.isfinite(ours).all()
    G = hq // hkv
    q = case.q.to(torch.float64)
    for s, L in enumerate(lens):
        t = np.arange(L)
        blocks = case.block_tables.numpy()[s, t // 16]
        slots = t % 16
        kb = case.k_cache.numpy()[blocks, :, :, slots, :].reshape(L, hkv, 128)
        vb = case.v_cache.numpy()[blocks, :, :, slots]
        K = torch.from_numpy(np.ascontiguousarray(kb)).view(torch.float8_e4m3fn).double() * \
            torch.from_numpy(ks[blocks, :, slots]).double()[:, :, None]
        V = torch.from_numpy(np.ascontiguousarray(vb)).view(torch.float8_e4m3fn).double() * \
            torch.from_numpy(vs[blocks, :, slots]).double()[:, :, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[s][:, None, :].contiguous(), K.permute(1, 0, 2).repeat_interleave(G, 0).contiguous(),
            V.permute(1, 0, 2).repeat_interleave(G, 0).contiguous(), scale=case.scale)[:, 0]
        np.testing.assert_allclose(ours[s], ref.numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# several query tokens per sequence (causal)

def run_multi(case):
    return oracle.attend_multi(case.q_bits(), case.cu_seqlens_q.numpy(), case.k_cache.numpy(),
                               case.v_cache.numpy(), case.block_tables.numpy(),
                               case.seq_lens.numpy(), case.scale, case.k_scale, case.v_scale)


def test_multi_with_one_query_per_sequence_is_decode(oracle_lib):
    lens = [1, 17, 90, 33, 0]
    case = workloads.make_multi_case(8, 2, lens, [1, 1, 1, 1, 0], 71, max_blocks=8)
    dec = workloads.Case("d", case.q[[0, 1, 2, 3]], case.k_cache, case.v_cache,
                         case.block_tables[:4], case.seq_lens[:4], case.scale, case.k_scale,
                         case.v_scale)
    assert np.array_equal(run_multi(case), run_oracle(dec))


@pytest.mark.parametrize("hq,hkv,lens,qlens", [
    (8, 2, [5, 40, 17], [5, 3, 16]), (40, 8, [100, 33], [4, 1]), (16, 1, [64, 2], [7, 2]),
    (5, 1, [300, 16, 1], [2, 16, 1]),
])
def test_multi_matches_causal_sdpa(oracle_lib, hq, hkv, lens, qlens):
    case = workloads.make_multi_case(hq, hkv, lens, qlens, 72)
    ours = run_multi(case)
    G = hq // hkv
    cu = case.cu_seqlens_q.numpy()
    q = case.q.to(torch.float64)
    for s, (L, ql) in enumerate(zip(lens, qlens)):
        K, V = gather_dense(case, s)
        Q = q[cu[s]:cu[s + 1]].permute(1, 0, 2).contiguous()             # [Hq, ql, 128]
        i = torch.arange(ql)[:, None]
        t = torch.arange(L)[None, :]
        mask = t <= (L - ql + i)                                          # bottom-right causal
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, K.permute(1, 0, 2).repeat_interleave(G, 0).contiguous(),
            V.permute(1, 0, 2).repeat_interleave(G, 0).contiguous(), attn_mask=mask,
            scale=case.scale)                                             # [Hq, ql, 128]
        np.testing.assert_allclose(ours[cu[s]:cu[s + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_multi_first_query_of_a_fresh_sequence_sees_token_zero(oracle_lib):
    case = workloads.make_multi_case(4, 1, [9], [9], 73)
    out = run_multi(case)
    _, V = gather_dense(case, 0)
    for h in range(4):
        assert np.array_equal(out[0, h], V[0, 0].numpy())


def test_multi_rejects_more_queries_than_context(oracle_lib):
    case = workloads.make_multi_case(4, 1, [9], [9], 74)
    bad = case.seq_lens.clone()
    bad[0] = 8
    with pytest.raises(ValueError):
        oracle.attend_multi(case.q_bits(), case.cu_seqlens_q.numpy(), case.k_cache.numpy(),
                            case.v_cache.numpy(), case.block_tables.numpy(), bad.numpy(),
                            case.scale, case.k_scale, case.v_scale)


# --------------------------------------------------------------------------
# Token-row cache layouts (each token's 128 dims contiguous, byte strides for
# block, token and kv head): the flash-style caches of the unified backend.

def run_strided(case, layout):
    kv, vv = workloads.token_row_views(case, layout)
    kb, ks = workloads.strided_buffer(kv)
    vb, vs = workloads.strided_buffer(vv)
    assert ks == vs
    return oracle.decode_strided(case.q_bits(), kb, vb, *ks, case.num_kv_heads,
                                 case.block_tables.numpy(), case.seq_lens.numpy(), case.scale,
                                 case.k_scale, case.v_scale)


@pytest.mark.parametrize("layout", workloads.TOKEN_ROW_LAYOUTS)
@pytest.mark.parametrize("case", list(small_cases())[:5], ids=lambda c: c.name)
def test_token_row_layouts_reproduce_page_layout(oracle_lib, case, layout):
    """The same cache bytes re-laid by torch permutes give the page-layout
    oracle's result bit for bit (same loads, same order of operations)."""
    assert np.array_equal(run_strided(case, layout), run_oracle(case))


@pytest.mark.parametrize("hq,hkv,lens", [(8, 2, [1, 17, 33, 64]), (12, 4, [100, 3, 257, 0])])
def test_token_row_layout_matches_sdpa_on_nhd_gather(oracle_lib, hq, hkv, lens):
    """K/V gathered straight from the [blocks, 16, kv_heads, 128] tensor by
    numpy indexing, decoded by torch, fp64 SDPA: an independent route."""
    case = workloads.make_case(hq, hkv, lens, seed=hq + hkv, extra_blocks=3)
    kv, vv = workloads.token_row_views(case, "nhd")
    ours = run_strided(case, "nhd")
    G = hq // hkv
    q = case.q.to(torch.float64)
    for s, L in enumerate(lens):
        if L == 0:
            assert not ours[s].any()
            continue
        t = np.arange(L)
        blocks = case.block_tables.numpy()[s, t // 16]
        kb = kv.numpy()[blocks, t % 16]          # [L, Hkv, 128]
        vb = vv.numpy()[blocks, t % 16]
        K = torch.from_numpy(np.ascontiguousarray(kb)).view(torch.float8_e4m3fn).double() * case.k_scale
        V = torch.from_numpy(np.ascontiguousarray(vb)).view(torch.float8_e4m3fn).double() * case.v_scale
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[s][:, None, :].contiguous(), K.permute(1, 0, 2).repeat_interleave(G, 0).contiguous(),
            V.permute(1, 0, 2).repeat_interleave(G, 0).contiguous(), scale=case.scale)[:, 0]
        np.testing.assert_allclose(ours[s], ref.numpy(), rtol=0, atol=1e-12)


def test_token_row_strides_select_the_right_bytes(oracle_lib):
    """Exchanging the token and kv-head strides of an NHD view reads other
    tokens' bytes: the result must change (the strides are really used)."""
    case = workloads.make_case(8, 2, [40, 33], seed=91)
    kv, vv = workloads.token_row_views(case, "nhd")
    kb, (bs, ts, hs) = workloads.strided_buffer(kv)
    vb, _ = workloads.strided_buffer(vv)
    assert (ts, hs) == (256, 128)
    args = (case.block_tables.numpy(), case.seq_lens.numpy(), case.scale, case.k_scale, case.v_scale)
    good = oracle.decode_strided(case.q_bits(), kb, vb, bs, ts, hs, 2, *args)
    assert np.array_equal(good, run_oracle(case))
    wrong = oracle.decode_strided(case.q_bits(), kb, vb, bs, hs, ts, 2, *args)
    assert not np.allclose(wrong, good)


def test_token_row_buffer_too_small_is_rejected(oracle_lib):
    case = workloads.make_case(8, 2, [40], seed=92)
    kv, vv = workloads.token_row_views(case, "nhd")
    kb, st = workloads.strided_buffer(kv)
    vb, _ = workloads.strided_buffer(vv)
    with pytest.raises(ValueError):
        oracle.decode_strided(case.q_bits(), kb[:100], vb, *st, 2, case.block_tables.numpy(),
                              case.seq_lens.numpy(), case.scale, case.k_scale, case.v_scale)


# --------------------------------------------------------------------------
# The unified backend's options on top of several queries per sequence:
# sliding window, logit softcap, ALiBi slopes, attention sinks.

def run_ext(case, **kw):
    return oracle.attend_ext(case.q_bits(), case.cu_seqlens_q.numpy(), case.k_cache.numpy(),
                             case.v_cache.numpy(), case.block_tables.numpy(), case.seq_lens.numpy(),
                             case.scale, case.k_scale, case.v_scale, **kw)


def ext_case(seed=81, hq=8, hkv=2, lens=(40, 70, 5, 129), qlens=(3, 8, 5, 1)):
    return workloads.make_multi_case(hq, hkv, list(lens), list(qlens), seed)


def equal_keys(case):
    """Every cached token of every kv head gets the same K codes (those of
    physical block 0, slot 0), so all logits of a query are equal."""
    k = case.k_cache.clone()
    codes = k[0, :, :, 0:1, :].clone()            # [Hkv, 8, 1, 16]
    k[:] = codes.unsqueeze(0)
    case.k_cache = k
    return case


def positions(case):
    """(row, sequence, position) of every query row."""
    cu = case.cu_seqlens_q.numpy()
    out = []
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s]); ql = int(cu[s + 1] - cu[s])
        for i in range(ql):
            out.append((int(cu[s]) + i, s, L - ql + i))
    return out


def v_rows(case, s, kvh, ts):
    """fp64 V rows (dequantised by torch) of tokens ts of sequence s."""
    bt = case.block_tables.numpy()[s]
    vb = np.stack([case.v_cache.numpy()[bt[t // 16], kvh, :, t % 16] for t in ts])
    return torch.from_numpy(vb).view(torch.float8_e4m3fn).double().numpy() * case.v_scale


def test_ext_defaults_reproduce_multi_query(oracle_lib):
    case = ext_case()
    assert np.array_equal(run_ext(case), run_multi(case))
    big = run_ext(case, sliding_window=10_000, alibi_slopes=np.zeros(8, np.float32),
                  sinks=np.full(8, -1e30, np.float32))
    assert np.array_equal(big, run_multi(case))


def test_window_of_one_returns_own_value(oracle_lib):
    case = ext_case(seed=82)
    out = run_ext(case, sliding_window=1)
    G = case.num_heads // case.num_kv_heads
    for row, s, p in positions(case):
        for h in range(case.num_heads):
            assert np.array_equal(out[row, h], v_rows(case, s, h // G, [p])[0])


@pytest.mark.parametrize("window", [2, 7, 16, 33])
def test_window_matches_masked_sdpa(oracle_lib, window):
    case = ext_case(seed=83)
    ours = run_ext(case, sliding_window=window)
    G = case.num_heads // case.num_kv_heads
    q = case.q.double()
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        K, V = gather_dense(case, s)                       # [L, Hkv, 128]
        rows = [(r, p) for r, s2, p in positions(case) if s2 == s]
        if not rows:
            continue
        pos = torch.tensor([p for _, p in rows])
        t = torch.arange(L)
        allowed = (t[None, :] <= pos[:, None]) & (t[None, :] > pos[:, None] - window)
        for h in range(case.num_heads):
            qh = q[[r for r, _ in rows], h]                # [n_q, 128]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qh[None], K[:, h // G][None].contiguous(), V[:, h // G][None].contiguous(),
                attn_mask=allowed[None], scale=case.scale)[0]
            np.testing.assert_allclose(ours[[r for r, _ in rows], h], ref.numpy(), rtol=0, atol=1e-12)


def test_softcap_limits(oracle_lib):
    case = ext_case(seed=84)
    plain = run_multi(case)
    np.testing.assert_allclose(run_ext(case, softcap=1e12), plain, rtol=0, atol=1e-12)
    # a vanishing cap flattens every logit to ~0: uniform weights, the mean of the visible V
    flat = run_ext(case, softcap=1e-12)
    G = case.num_heads // case.num_kv_heads
    for row, s, p in positions(case):
        for h in range(case.num_heads):
            mean = v_rows(case, s, h // G, range(p + 1)).mean(axis=0)
            np.testing.assert_allclose(flat[row, h], mean, rtol=0, atol=1e-9)


def test_softcap_bounds_the_logit_spread(oracle_lib):
    """With cap c every logit lies in (-c, c), so no weight ratio exceeds
    e^(2c): with c = 0.5 and one dominant key the output stays near the mean."""
    case = ext_case(seed=85)
    capped = run_ext(case, softcap=0.5)
    G = case.num_heads // case.num_kv_heads
    for row, s, p in positions(case):
        for h in range(case.num_heads):
            Vv = v_rows(case, s, h // G, range(p + 1))
            # a convex combination with weights within a factor e of each other
            lo = Vv.min(axis=0); hi = Vv.max(axis=0)
            assert np.all(capped[row, h] >= lo - 1e-12) and np.all(capped[row, h] <= hi + 1e-12)
            w_min = 1.0 / (1 + (p) * np.e)                  # smallest possible weight
            assert np.all(np.abs(capped[row, h] - Vv.mean(axis=0)) <= (1 - (p + 1) * w_min) * (hi - lo) + 1e-12)


def test_alibi_on_equal_keys_gives_geometric_weights(oracle_lib):
    case = equal_keys(ext_case(seed=86))
    slopes = np.array([0.5, 0.25, 0.125, 0.0625, 1.0, 2.0, 0.03125, 0.0], np.float32)
    out = run_ext(case, alibi_slopes=slopes)
    G = case.num_heads // case.num_kv_heads
    for row, s, p in positions(case):
        for h in range(case.num_heads):
            ts = np.arange(p + 1)
            w = np.exp(np.float64(slopes[h]) * (ts - p))
            ref = (w[:, None] * v_rows(case, s, h // G, ts)).sum(0) / w.sum()
            np.testing.assert_allclose(out[row, h], ref, rtol=0, atol=1e-12)


def test_sink_on_equal_keys_scales_the_mean(oracle_lib):
    case = equal_keys(ext_case(seed=87))
    sinks = np.linspace(-3, 3, 8).astype(np.float32)
    out = run_ext(case, sinks=sinks)
    G = case.num_heads // case.num_kv_heads
    q = case.q.double().numpy()
    for row, s, p in positions(case):
        for h in range(case.num_heads):
            kvh = h // G
            K0 = torch.from_numpy(np.ascontiguousarray(case.k_cache.numpy()[0, kvh, :, 0, :].reshape(128))) \
                .view(torch.float8_e4m3fn).double().numpy() * case.k_scale
            z = case.scale * float(q[row, h] @ K0)
            n = p + 1
            frac = n * np.exp(z) / (n * np.exp(z) + np.exp(np.float64(sinks[h])))
            ref = v_rows(case, s, kvh, range(n)).mean(axis=0) * frac
            np.testing.assert_allclose(out[row, h], ref, rtol=1e-12, atol=1e-12)


def dense_ext_reference(case, window=0, cap=0.0, slopes=None, sinks=None, cap_after_bias=False):
    """The options composed on an independent route: K/V gathered by numpy
    indexing and decoded by torch, logits in torch fp64, then (in this order)
    the softcap c*tanh(z/c), the ALiBi bias slope*(t - p), the window mask, a
    sink column with a zero value row, and torch's softmax.
    cap_after_bias=True applies the bias before the cap instead (a plausible
    mistake the pins must tell apart)."""
    G = case.num_heads // case.num_kv_heads
    q = case.q.double()
    out = np.zeros((case.q.shape[0], case.num_heads, 128))
    for s in range(case.num_seqs):
        L = int(case.seq_lens[s])
        rows = [(r, p) for r, s2, p in positions(case) if s2 == s]
        if not rows:
            continue
        K, V = gather_dense(case, s)                                  # [L, Hkv, 128]
        t = torch.arange(L, dtype=torch.float64)
        for r, p in rows:
            for h in range(case.num_heads):
                kvh = h // G
                z = case.scale * (K[:, kvh] @ q[r, h])                  # [L]
                bias = (float(slopes[h]) * (t - p)) if slopes is not None else torch.zeros(L, dtype=torch.float64)
                if cap_after_bias:
                    z = z + bias
                    if cap > 0:
                        z = cap * torch.tanh(z / cap)
                else:
                    if cap > 0:
                        z = cap * torch.tanh(z / cap)
                    z = z + bias
                seen = t <= p
                if window > 0:
                    seen &= t > p - window
                zz = z[seen]
                vv = V[:, kvh][seen]
                if sinks is not None:
                    zz = torch.cat([zz, torch.tensor([float(sinks[h])], dtype=torch.float64)])
                    vv = torch.cat([vv, torch.zeros(1, 128, dtype=torch.float64)])
                w = torch.softmax(zz, dim=0)
                out[r, h] = (w @ vv).numpy()
    return out


COMPOSED = {
    "cap+alibi": dict(cap=2.0),
    "cap5+alibi": dict(cap=5.0),
    "cap30+alibi": dict(cap=30.0),
    "window+sinks": dict(window=9),
    "all four": dict(window=13, cap=5.0),
}


@pytest.mark.parametrize("combo", list(COMPOSED))
def test_options_composed_match_a_dense_torch_route(oracle_lib, combo):
    """Finite softcaps with ALiBi, a window with sinks, and all four options
    together, against the independent dense route (within 1e-12)."""
    cfg = COMPOSED[combo]
    case = ext_case(seed=89, lens=(40, 70, 5, 129, 200), qlens=(3, 8, 5, 1, 4))
    slopes = np.array([0.5, 0.25, 0.125, 0.0625, 1.0, 2.0, 0.03125, 0.0], np.float32) \
        if "alibi" in combo or combo == "all four" else None
    sinks = np.linspace(-2, 4, 8).astype(np.float32) if "sinks" in combo or combo == "all four" else None
    # scale the queries up so the softcap bites (logits of several units)
    case.q = (case.q.float() * 4).to(torch.bfloat16)
    ours = run_ext(case, sliding_window=cfg.get("window", 0), softcap=cfg.get("cap", 0.0),
                   alibi_slopes=slopes, sinks=sinks)
    ref = dense_ext_reference(case, window=cfg.get("window", 0), cap=cfg.get("cap", 0.0),
                              slopes=slopes, sinks=sinks)
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def test_cap_is_applied_before_the_bias(oracle_lib):
    """Applying the ALiBi bias before the softcap gives a measurably different
    result on this case, so the order is pinned by the composition test."""
    case = ext_case(seed=90, lens=(40, 70, 129), qlens=(3, 8, 4))
    case.q = (case.q.float() * 4).to(torch.bfloat16)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625, 1.0, 2.0, 0.03125, 0.0], np.float32)
    ours = run_ext(case, softcap=2.0, alibi_slopes=slopes)
    right = dense_ext_reference(case, cap=2.0, slopes=slopes)
    swapped = dense_ext_reference(case, cap=2.0, slopes=slopes, cap_after_bias=True)
    np.testing.assert_allclose(ours, right, rtol=0, atol=1e-12)
    assert np.abs(ours - swapped).max() > 1e-6


def test_sink_counts_once_with_a_window(oracle_lib):
    """A window with a sink: the sink enlarges the denominator once per query
    (not per window position); dropping it changes the result."""
    case = ext_case(seed=91, lens=(40, 70, 129), qlens=(3, 8, 4))
    sinks = np.linspace(-1, 3, 8).astype(np.float32)
    with_sink = run_ext(case, sliding_window=7, sinks=sinks)
    ref = dense_ext_reference(case, window=7, sinks=sinks)
    np.testing.assert_allclose(with_sink, ref, rtol=0, atol=1e-12)
    assert np.abs(with_sink - run_ext(case, sliding_window=7)).max() > 1e-3


def test_ext_rejects_bad_options(oracle_lib):
    case = ext_case(seed=88)
    with pytest.raises(ValueError):
        run_ext(case, sliding_window=-1)
    with pytest.raises(ValueError):
        run_ext(case, softcap=-1.0)
    with pytest.raises(ValueError):
        run_ext(case, sinks=np.zeros(3, np.float32))
