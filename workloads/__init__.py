"""Seeded synthetic inputs for fp8 paged decode attention.

This module only *makes inputs*: it holds none of the attention arithmetic and
is shared by the tests, the benchmark and the smoke check, which feed the same
bytes to the HIP library and to the CPU oracle.

Recipe (the shapes and distributions of the workloads the vLLM pull request
lishuoshuo-amd/vllm #3 measures in "Kernel latency, accuracy runs and kernel
error": fp8 cache, 16-token blocks, head_dim 128, 40/8 and 32/8 heads,
16-256 sequences at one context length, and a ragged 1-4000 token mix over
four head layouts and three seeds):

* q: N(0, 1) drawn in fp32, rounded to bf16.
* K and V: N(0, 1) in fp32 over the whole cache tensor; each tensor gets its
  own per-tensor scale ``amax(|x|) / 448`` (or the next power of two above it,
  ``scale_mode="pow2"``) and is stored as ``fp8_e4m3fn(clamp(x / scale, +-448))``
  with torch's round-to-nearest-even cast.
* Block table: a seeded random permutation of physical block ids, handed to
  the sequences' logical blocks in order ("shuffled").  Physical blocks that
  no sequence uses, table entries past a sequence's last block, and the slots
  past ``seq_len`` in a sequence's last block are filled with fp8 NaN (0x7F),
  so any read of them would show in the output.
* ``torch.Generator`` seeded with ``seed`` on ``device``.  The same seed gives
  the same bytes on the same device type; CPU and GPU streams differ.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

HEAD_DIM = 128
BLOCK = 16
FP8_MAX = 448.0
FP8_NAN = 0x7F


@dataclass
class Case:
    name: str
    q: torch.Tensor              # bf16 [S, Hq, 128]
    k_cache: torch.Tensor        # uint8 [NB, Hkv, 8, 16, 16]
    v_cache: torch.Tensor        # uint8 [NB, Hkv, 128, 16]
    block_tables: torch.Tensor   # int32 [S, W]
    seq_lens: torch.Tensor       # int32 [S]
    scale: float                 # softmax scale (an fp32 value)
    k_scale: float               # fp32 value (1.0 when per-slot tables are used)
    v_scale: float               # fp32 value
    meta: dict = field(default_factory=dict)
    k_slot_scales: torch.Tensor | None = None   # float32 [NB, Hkv, 16], per-slot mode only
    v_slot_scales: torch.Tensor | None = None
    cu_seqlens_q: torch.Tensor | None = None    # int32 [S + 1]: several query rows per sequence

    @property
    def num_seqs(self) -> int:
        return self.seq_lens.shape[0]

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    @property
    def num_kv_heads(self) -> int:
        return self.k_cache.shape[1]

    @property
    def max_blocks(self) -> int:
        return self.block_tables.shape[1]

    def host(self) -> "Case":
        """A copy with every tensor on the CPU."""
        return self.to("cpu")

    def to(self, device) -> "Case":
        opt = (lambda t: None if t is None else t.to(device))
        return Case(self.name, self.q.to(device), self.k_cache.to(device),
                    self.v_cache.to(device), self.block_tables.to(device),
                    self.seq_lens.to(device), self.scale, self.k_scale,
                    self.v_scale, dict(self.meta), opt(self.k_slot_scales),
                    opt(self.v_slot_scales), opt(self.cu_seqlens_q))

    def q_bits(self):
        """q as uint16 bf16 bit patterns (numpy), for the oracle."""
        return self.q.cpu().contiguous().view(torch.int16).numpy().view("uint16")

    def kv_bytes(self) -> int:
        """fp8 K+V bytes one call must read (every cached token, both caches)."""
        return int(self.seq_lens.to(torch.int64).sum().item()) * self.num_kv_heads * HEAD_DIM * 2

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move: K+V fp8 of every cached token (once), q in
        and out as bf16 for every query row, the block-table entries in use,
        seq_lens, the query row offsets when there are several queries per
        sequence, and the scales."""
        lens = self.seq_lens.to(torch.int64)
        table = int(((lens + BLOCK - 1) // BLOCK).sum().item()) * 4
        rows = self.q.shape[0]
        qo = 2 * rows * self.num_heads * HEAD_DIM * 2
        cu = 0 if self.cu_seqlens_q is None else 4 * (self.num_seqs + 1)
        return self.kv_bytes() + qo + table + 4 * self.num_seqs + cu + 8


def _quantise(x: torch.Tensor, scale_mode: str):
    """Per-tensor fp8 e4m3fn quantisation of an fp32 tensor -> (uint8 codes, scale)."""
    amax = float(x.abs().max().item())
    if amax == 0.0:
        amax = 1.0
    if scale_mode == "amax":
        s = float(torch.tensor(amax / FP8_MAX, dtype=torch.float32).item())
    elif scale_mode == "pow2":
        s = 2.0 ** math.ceil(math.log2(amax / FP8_MAX))
    else:
        raise ValueError(scale_mode)
    codes = (x / s).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, s


def _quantise_per_slot(x: torch.Tensor, layout: str):
    """Per-(block, kv head, slot) fp8 quantisation of one cache's fp32 values,
    given as [NB, Hkv, 2048] in page order -> (uint8 codes, float32 [NB, Hkv, 16])."""
    NB, Hkv = x.shape[:2]
    if layout == "k":          # page = [8 chunks][16 slots][16 dims]
        v = x.view(NB, Hkv, 8, BLOCK, 16)
        amax = v.abs().amax(dim=(2, 4))
        s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
        q = (v / s[:, :, None, :, None]).clamp_(-FP8_MAX, FP8_MAX)
    else:                      # page = [128 dims][16 slots]
        v = x.view(NB, Hkv, HEAD_DIM, BLOCK)
        amax = v.abs().amax(dim=2)
        s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
        q = (v / s[:, :, None, :]).clamp_(-FP8_MAX, FP8_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(NB * Hkv * 2048)
    return codes, s.to(torch.float32).contiguous()


def make_case(num_heads: int, num_kv_heads: int, seq_lens, seed: int = 0, *,
              device="cpu", max_blocks: int | None = None, extra_blocks: int | None = None,
              scale_mode: str = "amax", poison: bool = True, name: str = "case",
              softmax_scale: float | None = None, slot_log2_span: float = 8.0,
              v_slot_log2_span: float | None = None, tiny_first_v: bool = False) -> Case:
    """Build one seeded case.  ``seq_lens`` is a list/tensor of per-sequence token counts.

    scale_mode: "amax" / "pow2" (per-tensor scales), or "per_slot": each token's
    K and V get a random magnitude 2^U(-span/2, span/2) (span = slot_log2_span,
    default 8; V's v_slot_log2_span when given) and their own scale amax/448 per
    (block, kv head, slot), returned
    as k_slot_scales / v_slot_scales (slots outside every context get NaN
    scales); tiny_first_v also shrinks every sequence's first token's V by
    2^-40, so its slot scale sits far below the others."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    lens = torch.as_tensor(seq_lens, dtype=torch.int64).cpu()
    S = int(lens.numel())
    pages = (lens + BLOCK - 1) // BLOCK
    W = int(max_blocks) if max_blocks is not None else max(1, int(pages.max().item()) if S else 1)
    if S and int(pages.max().item()) > W:
        raise ValueError("max_blocks smaller than the longest sequence")
    used = int(pages.sum().item())
    if extra_blocks is None:
        extra_blocks = max(1, used // 256)
    NB = used + max(1, int(extra_blocks))

    q = torch.randn(S, num_heads, HEAD_DIM, generator=g, device=device).to(torch.bfloat16)

    perm = torch.randperm(NB, generator=g, device=device).to(torch.int32).cpu()
    bt = torch.empty(S, W, dtype=torch.int32)
    poison_ids = perm[used:]
    cursor = 0
    for s in range(S):
        n = int(pages[s])
        bt[s, :n] = perm[cursor:cursor + n]
        cursor += n
        if W > n:
            # entries past the last block point at (NaN-filled) blocks no sequence owns
            bt[s, n:] = poison_ids[torch.arange(W - n) % poison_ids.numel()]

    ks_tab = vs_tab = None
    if scale_mode == "per_slot":
        n = NB * num_kv_heads * HEAD_DIM * BLOCK
        kx = torch.randn(n, generator=g, device=device).view(NB, num_kv_heads, 8, BLOCK, 16)
        span = float(slot_log2_span)
        kx *= torch.exp2(torch.rand(NB, num_kv_heads, 1, BLOCK, 1, generator=g, device=device) * span - span / 2)
        k_codes, ks_tab = _quantise_per_slot(kx.reshape(NB, num_kv_heads, 2048), "k")
        del kx
        vx = torch.randn(n, generator=g, device=device).view(NB, num_kv_heads, HEAD_DIM, BLOCK)
        vspan = span if v_slot_log2_span is None else float(v_slot_log2_span)
        vx *= torch.exp2(torch.rand(NB, num_kv_heads, 1, BLOCK, generator=g, device=device) * vspan - vspan / 2)
        if tiny_first_v:
            first = bt[:, 0][lens > 0].to(device=device, dtype=torch.int64)
            vx[first, :, :, 0] *= 2.0 ** -40
        v_codes, vs_tab = _quantise_per_slot(vx.reshape(NB, num_kv_heads, 2048), "v")
        del vx
        k_scale = v_scale = 1.0
    else:
        kx = torch.randn(NB * num_kv_heads * HEAD_DIM * BLOCK, generator=g, device=device)
        k_codes, k_scale = _quantise(kx, scale_mode)
        del kx
        vx = torch.randn(NB * num_kv_heads * HEAD_DIM * BLOCK, generator=g, device=device)
        v_codes, v_scale = _quantise(vx, scale_mode)
        del vx
    k_cache = k_codes.view(NB, num_kv_heads, HEAD_DIM // 16, BLOCK, 16)
    v_cache = v_codes.view(NB, num_kv_heads, HEAD_DIM, BLOCK)

    if poison:
        pid = poison_ids.to(device=device, dtype=torch.int64)
        k_cache[pid] = FP8_NAN
        v_cache[pid] = FP8_NAN
        if ks_tab is not None:
            ks_tab[pid] = float("nan")
            vs_tab[pid] = float("nan")
        for s in range(S):
            L = int(lens[s])
            if L % BLOCK:
                last = int(bt[s, L // BLOCK])
                k_cache[last, :, :, L % BLOCK:, :] = FP8_NAN
                v_cache[last, :, :, L % BLOCK:] = FP8_NAN
                if ks_tab is not None:
                    ks_tab[last, :, L % BLOCK:] = float("nan")
                    vs_tab[last, :, L % BLOCK:] = float("nan")

    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(HEAD_DIM)
    scale = float(torch.tensor(scale, dtype=torch.float32).item())
    return Case(name=name, q=q, k_cache=k_cache, v_cache=v_cache,
                block_tables=bt.to(device), seq_lens=lens.to(torch.int32).to(device),
                scale=scale, k_scale=float(k_scale), v_scale=float(v_scale),
                meta=dict(seed=seed, num_blocks=NB, used_blocks=used, scale_mode=scale_mode),
                k_slot_scales=ks_tab, v_slot_scales=vs_tab)


def make_multi_case(num_heads: int, num_kv_heads: int, seq_lens, q_lens, seed: int = 0,
                    **kw) -> Case:
    """Several new query tokens per sequence: sequence s has seq_lens[s] cached
    tokens, the last q_lens[s] of which are its queries (q rows
    cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1, N(0,1) rounded to bf16)."""
    base = make_case(num_heads, num_kv_heads, seq_lens, seed, **kw)
    ql = torch.as_tensor(q_lens, dtype=torch.int64)
    if ql.numel() != base.num_seqs or bool((ql < 0).any()) or \
            bool((ql > torch.as_tensor(seq_lens, dtype=torch.int64)).any()):
        raise ValueError("need 0 <= q_lens[s] <= seq_lens[s] for every sequence")
    cu = torch.zeros(base.num_seqs + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(ql, 0).to(torch.int32)
    g = torch.Generator(device=base.q.device)
    g.manual_seed(int(seed) + 7919)
    base.q = torch.randn(int(cu[-1]), num_heads, HEAD_DIM, generator=g,
                         device=base.q.device).to(torch.bfloat16)
    base.cu_seqlens_q = cu.to(base.q.device)
    return base


# ----------------------------------------------------------------------------
# The same cache bytes in token-row layouts (each token's 128 dims contiguous),
# as the flash-style caches of the unified backend keep them.

TOKEN_ROW_LAYOUTS = ("nhd", "combined", "packed")


def token_row_views(case, layout: str = "nhd"):
    """(k_view, v_view), each [num_blocks, 16, num_kv_heads, 128] uint8 with a
    contiguous last dim, holding exactly the bytes of case.k_cache / v_cache:
      nhd       two tensors [NB, 16, Hkv, 128];
      combined  one tensor [NB, 2, 16, Hkv, 128], K at [:, 0], V at [:, 1];
      packed    one tensor [NB, Hkv, 16, 256] (K then V per token), viewed
                through transpose(1, 2) and a split of the last dim."""
    NB, Hkv = case.k_cache.shape[:2]
    k_nhd = case.k_cache.permute(0, 3, 1, 2, 4).reshape(NB, BLOCK, Hkv, HEAD_DIM).contiguous()
    v_nhd = case.v_cache.reshape(NB, Hkv, HEAD_DIM, BLOCK).permute(0, 3, 1, 2).contiguous()
    if layout == "nhd":
        return k_nhd, v_nhd
    if layout == "combined":
        kv = torch.stack([k_nhd, v_nhd], dim=1).contiguous()
        return kv[:, 0], kv[:, 1]
    if layout == "packed":
        kv = torch.cat([k_nhd.permute(0, 2, 1, 3), v_nhd.permute(0, 2, 1, 3)], dim=-1).contiguous()
        t = kv.transpose(1, 2)
        return t[..., :HEAD_DIM], t[..., HEAD_DIM:]
    raise ValueError(layout)


def strided_buffer(view: torch.Tensor):
    """(uint8 numpy array of the storage from the view's first byte,
    (block_stride, token_stride, head_stride) in bytes) of a CPU token-row view."""
    flat = torch.empty(0, dtype=torch.uint8).set_(view.untyped_storage())
    return flat[view.storage_offset():].numpy(), tuple(int(x) for x in view.stride()[:3])


# ----------------------------------------------------------------------------
# The named workloads (token counts, head layouts, batch sizes).

def tiny(seed: int = 0, device="cpu") -> Case:
    """4 sequences of 1/17/33/64 tokens, 8 q / 2 kv heads, 32 physical blocks."""
    return make_case(8, 2, [1, 17, 33, 64], seed, device=device, max_blocks=4,
                     extra_blocks=22, name="tiny")


def dense(num_heads: int, num_kv_heads: int, num_seqs: int, ctx: int, seed: int = 0,
          device="cpu") -> Case:
    """Every sequence at the same context length."""
    return make_case(num_heads, num_kv_heads, [ctx] * num_seqs, seed, device=device,
                     name=f"dense_{num_heads}x{num_kv_heads}_ctx{ctx}_s{num_seqs}")


def ragged_lens(num_seqs: int = 256, lo: int = 1, hi: int = 4000, seed: int = 0):
    g = torch.Generator().manual_seed(10_000 + int(seed))
    return torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist()


def ragged(num_heads: int, num_kv_heads: int, seed: int, num_seqs: int = 256,
           device="cpu") -> Case:
    """Context lengths uniform in [1, 4000]; the table is 250 blocks wide."""
    return make_case(num_heads, num_kv_heads, ragged_lens(num_seqs, seed=seed), seed,
                     device=device, max_blocks=250,
                     name=f"ragged_{num_heads}x{num_kv_heads}_seed{seed}")


RAGGED_LAYOUTS = [(32, 8), (40, 8), (32, 4), (8, 1)]
DENSE_1K = [(40, 8, s, 1024) for s in (16, 64, 256)]
DENSE_4K = [(32, 8, s, 4096) for s in (24, 64, 256)]
# the other rows of the pages' latency table (40/8 at ctx 4096, 32/8 at ctx 1024)
PAGES_TABLE_EXTRA = [(40, 8, s, 4096) for s in (16, 64)] + [(32, 8, s, 1024) for s in (24, 64, 256)]
LOW_BATCH = [(40, 8, s, L) for s in (1, 2, 3, 4) for L in (4096, 8192, 16384, 32768)]
TARGET = (40, 8, 256, 4096)
