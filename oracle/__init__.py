"""fp64 CPU oracle for single-token paged decode attention over an fp8 KV cache.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use it; the product library never imports, links or calls it.
It shares no code with the HIP path.  The arithmetic lives in ``pa_oracle.c``
(plain loops in double precision, written from the definition), built by
:func:`build` with gcc into ``liboracle.so`` and called through ctypes.

Every function is pinned in ``tests/test_oracle_pins.py`` against things
other than itself: torch's own fp8 decoding, a dense attention computed by
``torch.nn.functional.scaled_dot_product_attention`` in fp64 on K/V gathered
by array indexing, closed forms, hand-worked fixtures and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile pa_oracle.c into liboracle.so (gcc, -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    f32 = ctypes.c_float
    lib.pa_oracle_fp8_e4m3fn.argtypes = [ctypes.c_uint8]
    lib.pa_oracle_fp8_e4m3fn.restype = ctypes.c_double
    lib.pa_oracle_bf16.argtypes = [ctypes.c_uint16]
    lib.pa_oracle_bf16.restype = ctypes.c_double
    lib.pa_oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.pa_oracle_bf16_rne.restype = ctypes.c_uint16
    lib.pa_oracle_decode.argtypes = [P, P, P, P, P, i32, i32, i32, i32,
                                     f32, f32, f32, P, i32]
    lib.pa_oracle_decode.restype = i32
    lib.pa_oracle_decode_partitioned.argtypes = [P, P, P, P, P, i32, i32, i32, i32,
                                                 f32, f32, f32, i32, P, P]
    lib.pa_oracle_decode_partitioned.restype = i32
    lib.pa_oracle_decode_slot_scales.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f32, P, P, P, i32]
    lib.pa_oracle_decode_slot_scales.restype = i32
    lib.pa_oracle_decode_strided.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, P, P, i32, i32, i32, i32, f32, f32,
                                             f32, P, i32]
    lib.pa_oracle_decode_strided.restype = i32
    lib.pa_oracle_attend_ext.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f32, f32, f32,
                                         i32, f32, P, P, P, i32]
    lib.pa_oracle_attend_ext.restype = i32
    lib.pa_oracle_attend_multi.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f32, f32, f32, P, i32]
    lib.pa_oracle_attend_multi.restype = i32
    lib.pa_oracle_fp8_e4m3fn_encode.argtypes = [ctypes.c_float]
    lib.pa_oracle_fp8_e4m3fn_encode.restype = ctypes.c_uint8
    lib.pa_oracle_cache_write.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, P, P, P, i32, i32,
                                          ctypes.c_int64, f32, f32]
    lib.pa_oracle_cache_write.restype = i32
    _lib = lib
    return lib


def fp8_e4m3fn_value(byte: int) -> float:
    """Value of one fp8 e4m3fn byte (OCP format, from its definition)."""
    return _load().pa_oracle_fp8_e4m3fn(byte & 0xFF)


def fp8_table() -> np.ndarray:
    """Values of all 256 fp8 e4m3fn codes, float64."""
    lib = _load()
    return np.array([lib.pa_oracle_fp8_e4m3fn(b) for b in range(256)], dtype=np.float64)


def bf16_value(bits: int) -> float:
    return _load().pa_oracle_bf16(bits & 0xFFFF)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Correctly rounded bfloat16 bit patterns (uint16) of float64 values."""
    lib = _load()
    flat = np.ascontiguousarray(x, dtype=np.float64).ravel()
    out = np.fromiter((lib.pa_oracle_bf16_rne(float(v)) for v in flat),
                      dtype=np.uint16, count=flat.size)
    return out.reshape(np.shape(x))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (plain bit placement)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _check(q_bits, k_cache, v_cache, block_tables, seq_lens):
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k_cache = np.ascontiguousarray(k_cache, dtype=np.uint8)
    v_cache = np.ascontiguousarray(v_cache, dtype=np.uint8)
    block_tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if q_bits.ndim != 3 or q_bits.shape[2] != 128:
        raise ValueError("q must be [S, Hq, 128] bf16 bits")
    S, Hq, _ = q_bits.shape
    if k_cache.ndim != 5 or k_cache.shape[2:] != (8, 16, 16):
        raise ValueError("k_cache must be [NB, Hkv, 8, 16, 16] bytes")
    NB, Hkv = k_cache.shape[:2]
    if v_cache.reshape(-1).size != NB * Hkv * 128 * 16:
        raise ValueError("v_cache must hold [NB, Hkv, 128, 16] bytes")
    if block_tables.ndim != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must be [S, W]")
    if seq_lens.shape != (S,):
        raise ValueError("seq_lens must be [S]")
    W = block_tables.shape[1]
    for s in range(S):
        used = block_tables[s, : (int(seq_lens[s]) + 15) // 16]
        if used.size and (used.min() < 0 or used.max() >= NB):
            raise ValueError(f"sequence {s}: block id out of range")
    return q_bits, k_cache, v_cache, block_tables, seq_lens, S, Hq, Hkv, W


def decode(q_bits, k_cache, v_cache, block_tables, seq_lens, scale, k_scale,
           v_scale, num_threads: int | None = None) -> np.ndarray:
    """fp64 paged decode attention.  Returns float64 [S, Hq, 128].

    q_bits: uint16 bf16 patterns [S, Hq, 128]; k_cache: uint8 [NB, Hkv, 8, 16, 16];
    v_cache: uint8 [NB, Hkv, 128, 16] (or the same bytes with an extra unit dim);
    block_tables: int32 [S, W]; seq_lens: int32 [S]; scale, k_scale, v_scale: the
    fp32 values the caller passes.
    """
    q_bits, k_cache, v_cache, bt, sl, S, Hq, Hkv, W = _check(
        q_bits, k_cache, v_cache, block_tables, seq_lens)
    out = np.zeros((S, Hq, 128), dtype=np.float64)
    nt = num_threads if num_threads else (os.cpu_count() or 1)
    rc = _load().pa_oracle_decode(
        q_bits.ctypes.data, k_cache.ctypes.data, v_cache.ctypes.data, bt.ctypes.data,
        sl.ctypes.data, S, Hq, Hkv, W, float(scale), float(k_scale), float(v_scale),
        out.ctypes.data, int(nt))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out


def decode_strided(q_bits, k_buf, v_buf, block_stride, token_stride, head_stride, num_kv_heads,
                   block_tables, seq_lens, scale, k_scale, v_scale,
                   num_threads: int | None = None) -> np.ndarray:
    """fp64 paged decode attention over a token-row cache layout.

    k_buf / v_buf: uint8 buffers starting at the K / V base; token t of kv head
    k in physical block p has its 128 fp8 dims at byte
    p * block_stride + (t % 16) * token_stride + k * head_stride.
    Returns float64 [S, Hq, 128]."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k_buf = np.ascontiguousarray(np.asarray(k_buf).reshape(-1), dtype=np.uint8)
    v_buf = np.ascontiguousarray(np.asarray(v_buf).reshape(-1), dtype=np.uint8)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if q_bits.ndim != 3 or q_bits.shape[2] != 128 or bt.ndim != 2 or sl.shape != (q_bits.shape[0],):
        raise ValueError("q [S, Hq, 128], block_tables [S, W], seq_lens [S] expected")
    S, Hq, _ = q_bits.shape
    W = bt.shape[1]
    Hkv = int(num_kv_heads)
    need = 0
    for s in range(S):
        n = int(sl[s])
        if n < 0 or n > 16 * W:
            raise ValueError("seq_lens out of range")
        if n:
            pmax = int(bt[s, :(n + 15) // 16].max())
            if int(bt[s, :(n + 15) // 16].min()) < 0:
                raise ValueError("negative block id in use")
            need = max(need, pmax * block_stride + 15 * token_stride + (Hkv - 1) * head_stride + 128)
    if need > min(k_buf.size, v_buf.size):
        raise ValueError("a block in use lies past the end of a cache buffer")
    out = np.zeros((S, Hq, 128), dtype=np.float64)
    nt = num_threads if num_threads else (os.cpu_count() or 1)
    rc = _load().pa_oracle_decode_strided(
        q_bits.ctypes.data, k_buf.ctypes.data, v_buf.ctypes.data, int(block_stride),
        int(token_stride), int(head_stride), bt.ctypes.data, sl.ctypes.data, S, Hq, Hkv, W,
        float(scale), float(k_scale), float(v_scale), out.ctypes.data, int(nt))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out


def decode_slot_scales(q_bits, k_cache, v_cache, block_tables, seq_lens, scale, k_scales,
                       v_scales, num_threads: int | None = None) -> np.ndarray:
    """fp64 paged decode with per-slot scale tables k_scales / v_scales
    (float32 [NB, Hkv, 16]) instead of per-tensor scales."""
    q_bits, k_cache, v_cache, bt, sl, S, Hq, Hkv, W = _check(
        q_bits, k_cache, v_cache, block_tables, seq_lens)
    ks = np.ascontiguousarray(k_scales, dtype=np.float32)
    vs = np.ascontiguousarray(v_scales, dtype=np.float32)
    if ks.shape != (k_cache.shape[0], Hkv, 16) or vs.shape != ks.shape:
        raise ValueError("scale tables must be float32 [NB, Hkv, 16]")
    out = np.zeros((S, Hq, 128), dtype=np.float64)
    rc = _load().pa_oracle_decode_slot_scales(
        q_bits.ctypes.data, k_cache.ctypes.data, v_cache.ctypes.data, bt.ctypes.data,
        sl.ctypes.data, S, Hq, Hkv, W, float(scale), ks.ctypes.data, vs.ctypes.data,
        out.ctypes.data, int(num_threads if num_threads else (os.cpu_count() or 1)))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out


def attend_multi(q_bits, cu_seqlens_q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale,
                 v_scale, num_threads: int | None = None) -> np.ndarray:
    """Causal attention of several new tokens per sequence over the cache.

    q_bits: uint16 bf16 [T, Hq, 128]; cu_seqlens_q: int32 [S + 1] query row
    offsets (cu[0] = 0, cu[S] = T).  Query i of sequence s sees cache tokens
    0 .. seq_lens[s] - q_len + i.  Returns float64 [T, Hq, 128]."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    S = sl.shape[0]
    if cu.shape != (S + 1,) or q_bits.ndim != 3 or q_bits.shape[0] != int(cu[-1]):
        raise ValueError("cu_seqlens_q must be [S+1] with cu[S] = number of query rows")
    _, Hq, _ = q_bits.shape
    fake_q = np.zeros((S, Hq, 128), np.uint16)
    _, k_cache, v_cache, bt, sl, S, Hq, Hkv, W = _check(fake_q, k_cache, v_cache, block_tables, sl)
    out = np.zeros((q_bits.shape[0], Hq, 128), dtype=np.float64)
    rc = _load().pa_oracle_attend_multi(
        q_bits.ctypes.data, cu.ctypes.data, k_cache.ctypes.data, v_cache.ctypes.data,
        bt.ctypes.data, sl.ctypes.data, S, Hq, Hkv, W, float(scale), float(k_scale),
        float(v_scale), out.ctypes.data, int(num_threads if num_threads else (os.cpu_count() or 1)))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out


def attend_ext(q_bits, cu_seqlens_q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale,
               v_scale, sliding_window: int = 0, softcap: float = 0.0, alibi_slopes=None,
               sinks=None, num_threads: int | None = None) -> np.ndarray:
    """attend_multi with the unified backend's options: a sliding window of
    `sliding_window` tokens ending at each query (0 = none), logit softcap
    (0 = none), per-head ALiBi slopes and per-head sink logits (float32 [Hq],
    or None).  Returns float64 [T, Hq, 128]."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    S = sl.shape[0]
    if cu.shape != (S + 1,) or q_bits.ndim != 3 or q_bits.shape[0] != int(cu[-1]):
        raise ValueError("cu_seqlens_q must be [S+1] with cu[S] = number of query rows")
    _, Hq, _ = q_bits.shape
    fake_q = np.zeros((S, Hq, 128), np.uint16)
    _, k_cache, v_cache, bt, sl, S, Hq, Hkv, W = _check(fake_q, k_cache, v_cache, block_tables, sl)
    def vec(x):
        if x is None:
            return None
        a = np.ascontiguousarray(x, dtype=np.float32)
        if a.shape != (Hq,):
            raise ValueError("per-head options must have num_heads entries")
        return a
    sl_a, sk_a = vec(alibi_slopes), vec(sinks)
    out = np.zeros((q_bits.shape[0], Hq, 128), dtype=np.float64)
    rc = _load().pa_oracle_attend_ext(
        q_bits.ctypes.data, cu.ctypes.data, k_cache.ctypes.data, v_cache.ctypes.data,
        bt.ctypes.data, sl.ctypes.data, S, Hq, Hkv, W, float(scale), float(k_scale),
        float(v_scale), int(sliding_window), float(softcap),
        None if sl_a is None else sl_a.ctypes.data, None if sk_a is None else sk_a.ctypes.data,
        out.ctypes.data, int(num_threads if num_threads else (os.cpu_count() or 1)))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return out


def decode_partitioned(q_bits, k_cache, v_cache, block_tables, seq_lens, scale,
                       k_scale, v_scale, tokens_per_part: int, return_empty: bool = False):
    """The same quantity via per-partition partials and a log-sum-exp merge.

    Partitions of `tokens_per_part` tokens cut the whole table row (16 * W
    tokens), so contexts shorter than the row leave empty partitions, which
    the merge skips.  Returns float64 [S, Hq, 128], and with return_empty also
    the number of empty partitions formed over all (sequence, head) rows."""
    q_bits, k_cache, v_cache, bt, sl, S, Hq, Hkv, W = _check(
        q_bits, k_cache, v_cache, block_tables, seq_lens)
    out = np.zeros((S, Hq, 128), dtype=np.float64)
    empty = ctypes.c_int64(0)
    rc = _load().pa_oracle_decode_partitioned(
        q_bits.ctypes.data, k_cache.ctypes.data, v_cache.ctypes.data, bt.ctypes.data,
        sl.ctypes.data, S, Hq, Hkv, W, float(scale), float(k_scale), float(v_scale),
        int(tokens_per_part), out.ctypes.data, ctypes.byref(empty))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return (out, int(empty.value)) if return_empty else out


def fp8_encode(values) -> np.ndarray:
    """fp8 e4m3fn codes (uint8) of float32 values: nearest-even, saturating at 448."""
    lib = _load()
    flat = np.ascontiguousarray(values, dtype=np.float32).ravel()
    out = np.fromiter((lib.pa_oracle_fp8_e4m3fn_encode(float(v)) for v in flat),
                      dtype=np.uint8, count=flat.size)
    return out.reshape(np.shape(values))


def cache_write(key_bits, value_bits, k_cache, v_cache, slot_mapping, k_scale, v_scale):
    """Quantise and scatter new tokens into (copies of) the caches.

    key_bits / value_bits: uint16 bf16 patterns [T, Hkv, 128] (any token stride);
    k_cache uint8 [NB, Hkv, 8, 16, 16]; v_cache uint8 [NB, Hkv, 128, 16];
    slot_mapping int64 [T] (negative: skip).  Returns the new (k_cache, v_cache).
    """
    key_bits = np.asarray(key_bits, dtype=np.uint16)
    value_bits = np.asarray(value_bits, dtype=np.uint16)
    T, Hkv, D = key_bits.shape
    if D != 128 or value_bits.shape != key_bits.shape:
        raise ValueError("key/value must be [T, Hkv, 128]")
    kb = np.ascontiguousarray(key_bits)
    vb = np.ascontiguousarray(value_bits)
    kc = np.array(k_cache, dtype=np.uint8, copy=True, order="C")
    vc = np.array(v_cache, dtype=np.uint8, copy=True, order="C")
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    NB = kc.shape[0]
    if kc.shape[1] != Hkv or vc.size != kc.size:
        raise ValueError("cache shapes disagree with key/value")
    rc = _load().pa_oracle_cache_write(kb.ctypes.data, vb.ctypes.data, Hkv * 128, Hkv * 128,
                                       kc.ctypes.data, vc.ctypes.data, sm.ctypes.data, T, Hkv, NB,
                                       float(k_scale), float(v_scale))
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return kc, vc
