"""Parity of the fp8 KV-cache write kernel with the oracle on MI355X: the
cache bytes must match bit for bit (rounding, saturation, NaN, layout, skipped
slots, untouched bytes), and decoding a cache written by the kernel must match
the oracle decoding the cache the oracle writes from the same keys/values."""
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
    pa.load_library()


def bits(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def run_both(key, value, slots, NB, ks, vs, seed=0):
    """Kernel and oracle from the same pre-filled caches; returns both results.
    Slots past the caches are skipped by the kernel (it cannot report them);
    the oracle, which rejects them, gets -1 there."""
    import paged_attention_decode_03_amd as pa
    T, Hkv, _ = key.shape
    g = torch.Generator().manual_seed(seed)
    k0 = torch.randint(0, 256, (NB, Hkv, 8, 16, 16), generator=g, dtype=torch.int32).to(torch.uint8)
    v0 = torch.randint(0, 256, (NB, Hkv, 128, 16), generator=g, dtype=torch.int32).to(torch.uint8)
    kc, vc = k0.cuda(), v0.cuda()
    pa.paged_kv_cache_write(key.cuda() if not key.is_cuda else key, value.cuda() if not value.is_cuda else value,
                            kc, vc, slots.cuda(), torch.tensor([ks], device="cuda"),
                            torch.tensor([vs], device="cuda"))
    torch.cuda.synchronize()
    ok, ov = oracle.cache_write(bits(key).reshape(T, Hkv, 128), bits(value).reshape(T, Hkv, 128),
                                k0.numpy(), v0.numpy(),
                                np.where(slots.cpu().numpy() >= NB * 16, -1, slots.cpu().numpy()), ks, vs)
    return kc.cpu().numpy(), vc.cpu().numpy(), ok, ov


def assert_same(a, b, what):
    diff = np.flatnonzero(a.ravel() != b.ravel())
    assert diff.size == 0, f"{what}: {diff.size} bytes differ, first at {diff[:5]}: " \
                           f"{a.ravel()[diff[:5]]} vs {b.ravel()[diff[:5]]}"


@pytest.mark.parametrize("T,Hkv,NB", [(1, 1, 1), (37, 2, 9), (300, 8, 40), (4096, 8, 300)])
def test_random_tokens_bit_exact(T, Hkv, NB):
    g = torch.Generator().manual_seed(T)
    key = (torch.randn(T, Hkv, 128, generator=g) * torch.exp2(torch.randint(-12, 4, (T, Hkv, 128), generator=g).float())).to(torch.bfloat16)
    value = (3 * torch.randn(T, Hkv, 128, generator=g)).to(torch.bfloat16)
    slots = torch.randperm(NB * 16, generator=g)[:T].to(torch.int64)
    if T > 2:
        slots[1] = -1
    ks, vs = float(np.float32(0.0173)), float(np.float32(0.0291))
    kc, vc, ok, ov = run_both(key, value, slots, NB, ks, vs)
    log(f"cache write T={T} Hkv={Hkv}: comparing {kc.size + vc.size} bytes")
    assert_same(kc, ok, "k_cache")
    assert_same(vc, ov, "v_cache")


def test_every_tie_and_special_value():
    """With scale 1 the division is exact: every fp8 midpoint (a bf16 value)
    must round to even; specials saturate / stay NaN with their sign."""
    table = oracle.fp8_table()
    pos = np.sort(table[:0x7F])
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([mids, -mids, pos, -pos,
                           [448.0, 464.0, 480.0, 2.0 ** 20, -(2.0 ** 20), np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0]])
    vals = torch.tensor(vals, dtype=torch.float32)
    assert torch.equal(vals.to(torch.bfloat16).float().nan_to_num(0), vals.nan_to_num(0))  # exact in bf16
    n = vals.numel()
    T = (n + 127) // 128
    flat = torch.zeros(T * 128, dtype=torch.float32)
    flat[:n] = vals
    key = flat.view(T, 1, 128).to(torch.bfloat16)
    value = (-flat).view(T, 1, 128).to(torch.bfloat16)
    slots = torch.arange(T, dtype=torch.int64) * 3
    kc, vc, ok, ov = run_both(key, value, slots, (3 * T + 15) // 16 + 1, 1.0, 1.0)
    assert_same(kc, ok, "k_cache")
    assert_same(vc, ov, "v_cache")


def test_skipped_slots_leave_the_cache_untouched():
    T, Hkv, NB = 64, 2, 4
    g = torch.Generator().manual_seed(7)
    key = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    value = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    slots = torch.full((T,), -1, dtype=torch.int64)
    slots[::4] = torch.arange(16, dtype=torch.int64) * 2          # 16 tokens written
    slots[3] = NB * 16 + 5                                        # past the caches: skipped
    kc, vc, ok, ov = run_both(key, value, slots, NB, 0.02, 0.03)
    assert_same(kc, ok, "k_cache")
    assert_same(vc, ov, "v_cache")


def test_strided_key_value_from_a_fused_projection():
    import paged_attention_decode_03_amd as pa
    T, Hq, Hkv, NB = 50, 8, 2, 8
    g = torch.Generator().manual_seed(11)
    qkv = torch.randn(T, (Hq + 2 * Hkv) * 128, generator=g).to(torch.bfloat16).cuda()
    key = qkv[:, Hq * 128:(Hq + Hkv) * 128].view(T, Hkv, 128)
    value = qkv[:, (Hq + Hkv) * 128:].view(T, Hkv, 128)
    assert key.stride(0) == (Hq + 2 * Hkv) * 128
    slots = torch.randperm(NB * 16, generator=g)[:T].to(torch.int64)
    kc, vc, ok, ov = run_both(key, value, slots, NB, 0.011, 0.013)
    assert_same(kc, ok, "k_cache")
    assert_same(vc, ov, "v_cache")


def test_write_then_decode_matches_oracle_write_then_decode():
    """The kernel writes a whole cache from bf16 K/V; decoding it must match the
    oracle decoding the cache the oracle wrote from the same K/V."""
    import paged_attention_decode_03_amd as pa
    lens = [1, 17, 100, 513, 2000]
    Hq, Hkv = 40, 8
    base = workloads.make_case(Hq, Hkv, lens, seed=21, poison=False)
    T = sum(lens)
    g = torch.Generator().manual_seed(22)
    key = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    value = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    slots = []
    for s, L in enumerate(lens):
        for t in range(L):
            slots.append(int(base.block_tables[s, t // 16]) * 16 + t % 16)
    slots = torch.tensor(slots, dtype=torch.int64)
    NB = base.k_cache.shape[0]
    ks, vs = float(np.float32(6.0 / 448)), float(np.float32(6.0 / 448))
    kc, vc, ok, ov = run_both(key, value, slots, NB, ks, vs, seed=23)
    assert_same(kc, ok, "k_cache")
    assert_same(vc, ov, "v_cache")
    q = base.q.cuda()
    out = pa.paged_decode_attention(q, torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(),
                                    base.block_tables.cuda(), base.seq_lens.cuda(), base.scale,
                                    torch.tensor([ks], device="cuda"), torch.tensor([vs], device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.decode(base.q_bits(), ok, ov, base.block_tables.numpy(), base.seq_lens.numpy(),
                        base.scale, ks, vs)
    compare(out, ref, "write then decode")


@pytest.mark.parametrize("pattern", ["aligned", "offset", "mixed"])
def test_whole_block_runs(pattern):
    """Prefill-like slot patterns: runs of 16 consecutive tokens filling one block
    in order (written a whole page at a time), runs starting mid-block, and runs
    broken by skipped or reordered tokens."""
    T, Hkv, NB = 16 * 24 + 7, 4, 64
    g = torch.Generator().manual_seed(31)
    key = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    value = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    blocks = torch.randperm(NB, generator=g)[:(T + 40) // 16 + 2]
    if pattern == "aligned":
        slots = torch.tensor([int(blocks[t // 16]) * 16 + t % 16 for t in range(T)], dtype=torch.int64)
    elif pattern == "offset":
        slots = torch.tensor([int(blocks[(t + 5) // 16]) * 16 + (t + 5) % 16 for t in range(T)], dtype=torch.int64)
    else:
        slots = torch.tensor([int(blocks[t // 16]) * 16 + t % 16 for t in range(T)], dtype=torch.int64)
        slots[20] = -1
        slots[40], slots[41] = slots[41].clone(), slots[40].clone()
        slots[64 + 3] = NB * 16 + 3
    kc, vc, ok, ov = run_both(key, value, slots, NB, 0.015, 0.021)
    assert_same(kc, ok, "k_cache")
    assert_same(vc, ov, "v_cache")


def test_sequences_of_every_length_and_start():
    """A batch of prefill chunks of 1..40 tokens, each continuing its
    sequence at every slot 0..15 of a block (its earlier tokens already
    cached): runs of every start slot and length, sequence boundaries inside
    the groups of 16 tokens, runs that cross a group boundary and blocks
    written from two groups."""
    Hkv, NB = 2, 400
    g = torch.Generator().manual_seed(41)
    perm = torch.randperm(NB, generator=g).tolist()
    slots, b = [], 0
    for i, (length, start) in enumerate((l, s) for l in range(1, 41) for s in (0, 1, 5, 8, 15) if (l + s) % 3 != 1):
        nblk = (start + length + 15) // 16
        blocks = perm[b:b + nblk]
        b += nblk
        slots += [blocks[(start + t) // 16] * 16 + (start + t) % 16 for t in range(length)]
    slots = torch.tensor(slots, dtype=torch.int64)
    T = slots.numel()
    key = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    value = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    log(f"prefill chunks: {T} tokens, {b} blocks")
    kc, vc, ok, ov = run_both(key, value, slots, NB, 0.013, 0.017, seed=5)
    assert_same(kc, ok, "k_cache")
    assert_same(vc, ov, "v_cache")


# scales taking the short correctly rounded quotient, and ones outside its
# range (tiny, huge, subnormal, negative) that take the division
QUOTIENT_SCALES = [0.0173, 1.0 / 3.0, 3.0, 0.99999994, 7.3e-3, 1.1e2, 2.0 ** -60, 2.0 ** 60,
                   -0.021, 1.0e-20, 3.0e19, 1.0e-39]


@pytest.mark.parametrize("scale", QUOTIENT_SCALES)
def test_every_bf16_value_bit_exact(scale):
    """All 65536 bf16 bit patterns (zeros, subnormals, infinities and NaNs of
    both signs included) through both write paths, in-order whole blocks and
    scattered tokens, against the oracle's fp32 division and rounding."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    key = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).view(512, 1, 128)
    value = torch.from_numpy(pats[::-1].view(np.int16).copy()).view(torch.bfloat16).view(512, 1, 128)
    ks = float(np.float32(scale))
    vs = float(np.float32(scale * 1.37))
    in_order = torch.arange(512, dtype=torch.int64)
    scattered = torch.randperm(512, generator=torch.Generator().manual_seed(7)).to(torch.int64)
    for name, slots in (("whole blocks", in_order), ("scattered", scattered)):
        log(f"every bf16 value, scale {ks:g} / {vs:g}, {name}")
        kc, vc, ok, ov = run_both(key, value, slots, 32, ks, vs)
        assert_same(kc, ok, f"k_cache ({name})")
        assert_same(vc, ov, f"v_cache ({name})")
