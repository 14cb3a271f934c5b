"""Pins of the oracle's fp8 encoder and cache write (CPU only).

The encoder is checked against torch's float32 -> float8_e4m3fn cast (round to
nearest even; torch does not saturate, so inputs are clamped to +-448 first,
which is what saturation means), on every tie between neighbouring codes, the
values one float32 ulp either side of every tie, a wide random sample, and the
round trip through decoding.  The cache write is checked against an independent
route: torch's cast of key / k_scale and numpy indexing into the page layout.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads


def torch_codes(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_round_trips_every_finite_code(oracle_lib):
    table = oracle.fp8_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = oracle.fp8_encode(table[codes].astype(np.float32))
    assert np.array_equal(back, codes)


def test_encode_matches_torch_on_ties_and_neighbours(oracle_lib):
    table = oracle.fp8_table()
    pos = np.sort(table[[c for c in range(0x00, 0x7F)]])            # 0 .. 448
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)            # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    x = np.concatenate([mids, up, dn, -mids, -up, -dn])
    assert np.array_equal(oracle.fp8_encode(x), torch_codes(x))


def test_encode_matches_torch_on_random_values(oracle_lib):
    g = np.random.default_rng(0)
    x = (g.standard_normal(200_000) * np.exp2(g.integers(-14, 10, 200_000))).astype(np.float32)
    assert np.array_equal(oracle.fp8_encode(x), torch_codes(x))


@pytest.mark.parametrize("value,code", [
    (1.0625, 0x38), (1.1875, 0x3A), (1.5 * 2.0 ** -9, 0x02), (0.5 * 2.0 ** -9, 0x00),
    (448.0, 0x7E), (464.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE), (float("inf"), 0x7E),
    (float("-inf"), 0xFE), (float("nan"), 0x7F), (-0.0, 0x80), (0.0, 0x00),
    (2.0 ** -6, 0x08), (15 * 2.0 ** -10, 0x08), (240.0, 0x77),
])
def test_encode_hand_values(oracle_lib, value, code):
    assert int(oracle.fp8_encode(np.array([value], np.float32))[0]) == code


def test_cache_write_matches_torch_cast_and_layout(oracle_lib):
    g = torch.Generator().manual_seed(3)
    T, Hkv, NB = 37, 2, 9
    key = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    value = (3 * torch.randn(T, Hkv, 128, generator=g)).to(torch.bfloat16)
    slots = torch.randperm(NB * 16, generator=g)[:T].to(torch.int64)
    slots[5] = -1                      # padding token: not cached
    ks, vs = 0.0125, 0.03125
    k0 = torch.randint(0, 256, (NB, Hkv, 8, 16, 16), generator=g, dtype=torch.int32).to(torch.uint8)
    v0 = torch.randint(0, 256, (NB, Hkv, 128, 16), generator=g, dtype=torch.int32).to(torch.uint8)
    kc, vc = oracle.cache_write(key.view(torch.int16).numpy().view(np.uint16),
                                value.view(torch.int16).numpy().view(np.uint16),
                                k0.numpy(), v0.numpy(), slots.numpy(), ks, vs)
    ek = torch_codes((key.float() / ks).numpy())                    # [T, Hkv, 128]
    ev = torch_codes((value.float() / vs).numpy())
    kc_exp = k0.numpy().copy()
    vc_exp = v0.numpy().copy()
    for t in range(T):
        s = int(slots[t])
        if s < 0:
            continue
        b, j = divmod(s, 16)
        kc_exp[b, :, :, j, :] = ek[t].reshape(Hkv, 8, 16)
        vc_exp[b, :, :, j] = ev[t]
    assert np.array_equal(kc, kc_exp)
    assert np.array_equal(vc, vc_exp)


def test_cache_write_then_decode_matches_dense_attention(oracle_lib):
    """Tokens written by the cache writer decode to the quantised keys/values."""
    g = torch.Generator().manual_seed(4)
    T, Hkv, Hq = 40, 2, 8
    NB = 6
    key = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    value = torch.randn(T, Hkv, 128, generator=g).to(torch.bfloat16)
    perm = torch.randperm(NB, generator=g)[:3].to(torch.int32)
    slots = torch.tensor([int(perm[t // 16]) * 16 + t % 16 for t in range(T)], dtype=torch.int64)
    ks, vs = float(np.float32(0.01)), float(np.float32(0.02))   # the fp32 values a caller passes
    kc, vc = oracle.cache_write(key.view(torch.int16).numpy().view(np.uint16),
                                value.view(torch.int16).numpy().view(np.uint16),
                                np.zeros((NB, Hkv, 8, 16, 16), np.uint8),
                                np.zeros((NB, Hkv, 128, 16), np.uint8), slots.numpy(), ks, vs)
    q = torch.randn(1, Hq, 128, generator=g).to(torch.bfloat16)
    bt = np.array([perm.numpy()], np.int32)
    out = oracle.decode(q.view(torch.int16).numpy().view(np.uint16), kc, vc, bt,
                        np.array([T], np.int32), 0.0883883461356163, ks, vs)
    Kq = torch.from_numpy(torch_codes((key.float() / ks).numpy())).view(torch.float8_e4m3fn).double() * ks
    Vq = torch.from_numpy(torch_codes((value.float() / vs).numpy())).view(torch.float8_e4m3fn).double() * vs
    G = Hq // Hkv
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double()[0][:, None, :], Kq.permute(1, 0, 2).repeat_interleave(G, 0).contiguous(),
        Vq.permute(1, 0, 2).repeat_interleave(G, 0).contiguous(), scale=0.0883883461356163)[:, 0]
    np.testing.assert_allclose(out[0], ref.numpy(), rtol=0, atol=1e-12)


def test_cache_write_rejects_slots_past_the_cache(oracle_lib):
    key = np.zeros((2, 1, 128), np.uint16)
    with pytest.raises(ValueError):
        oracle.cache_write(key, key, np.zeros((1, 1, 8, 16, 16), np.uint8),
                           np.zeros((1, 1, 128, 16), np.uint8), np.array([3, 16]), 1.0, 1.0)
