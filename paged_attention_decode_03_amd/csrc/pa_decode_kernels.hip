// gfx950 kernels for single-token paged decode attention over an fp8-e4m3fn
// KV cache (16-token blocks, head_dim 128, GQA groups of up to 16 query heads).
//
// The operation follows the vLLM pull request lishuoshuo-amd/vllm #3
// (Overview; Details > Layout: K pages [head_size/16][16][16], V pages
// [head_size][16], addressed by a dense page stride) and the API page
// vllm.v1.attention.backends.rocm_aiter_unified_attn
// (RocmAiterUnifiedAttentionImpl.forward: block_table, seqused_k,
// softmax_scale, k_descale / v_descale).
//
// One wavefront owns one work item (sequence, kv head, partition) and keeps
// every query head of the kv head's group in the 16 columns of its MFMA tiles,
// so each fp8 K/V byte is fetched from HBM once and used by the whole group.
//
//   QK^T  v_mfma_f32_16x16x32_bf16: A = K page (16 tokens x 32 dims, fp8 -> bf16
//         exactly), B = q^T (32 dims x 16 heads).  Four per page.
//   PV    v_mfma_f32_16x16x16_f16:  A = V^T (16 dims x 16 tokens, fp8 -> fp16
//         exactly), B = P^T (16 tokens x 16 heads, fp16).  Eight per page,
//         plus one with A = ones that accumulates the softmax denominator from
//         the same rounded P.
//
// The D layout of both MFMAs puts head (lane & 15) and rows 4*(lane >> 4)+i in
// lane `lane`, so the QK^T result is already the B operand of PV and every
// per-head softmax quantity (running max, rescale factor) is lane-local; the
// only cross-lane step is a max over the four 16-lane rows (permlane swaps).
//
// Loads go from HBM into VGPRs:
//   K: two fully coalesced 1 KiB dwordx4 loads per page, in the layout the
//      MFMA wants (lane l: token l & 15, 16-dim chunks l >> 4 and 4 + (l >> 4)),
//   V: two 1 KiB dwordx4 loads per page (lane l: dims l and 64 + l, all 16
//      slots), the page copied to LDS and read back one operand dword at a
//      time: two load instructions a page where the operand layout would take
//      eight dword loads, which measured faster (most where a wave is alone
//      on its SIMD).
// Token-row caches (TR: each token's 128 dims contiguous, the flash-style
// layouts of the API page's unified backend) load K the same way (lane l:
// 16 B chunks of token l & 15's row) and V as whole 128 B token rows (eight
// per load); a V page then passes through LDS, transposed into the dims x
// tokens operand.
// Several queries per sequence (MQ): the 16 columns hold (query token, head)
// pairs, and an item holds one or two such tiles against the same K/V.
// Pages are software-pipelined PPS at a time, one stage ahead.
#include <float.h>
#include <limits.h>
#include <math.h>

#include "pa_decode_kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef _Float16 f16x4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));

// Tuning (compile time): pages per pipeline stage, depth of the register ring
// of stages (depth - 1 stages are in flight while one is computed), waves per
// SIMD the register budget is sized for, and the cache-policy bits of the K/V
// loads (gfx950 buffer-load aux: 2 = nt, i.e. streamed once, not kept).
// When a sequence's query tiles are spread over several items, those items
// read the same pages: their loads use the default policy instead, so the
// pages stay in L2 for the other items.
// Stages of two pages (one wave per item): on small batches an item's pages
// land nearly at once, and smaller stages leave less compute after the last
// one (measured on MI355X against four pages: 40/8 ctx 1024 x 16 12.5 -> 11.4
// us, 32/8 ctx 1024 x 24 14.6 -> 13.4 us, 40/8 ctx 4096 x 16 26.7 -> 25.3 us;
// the target, ragged, token-row and several-queries rows the same or up to 3%
// faster).  Two waves per item use two-page stages too, in a deeper ring.
#ifndef PA_PAGES_PER_STAGE
#define PA_PAGES_PER_STAGE 2
#endif
#ifndef PA_RING_DEPTH
#define PA_RING_DEPTH 2
#endif
#ifndef PA_WAVES_PER_EU
#define PA_WAVES_PER_EU 2
#endif
#ifndef PA_LOAD_AUX
#define PA_LOAD_AUX 2
#endif
constexpr int kPagesPerStage = PA_PAGES_PER_STAGE;
constexpr int kRingDepth = PA_RING_DEPTH;
// The per-slot-scale variant keeps 8 more VGPRs per page in flight; 2 pages per
// stage keep it at 2 waves per SIMD.
#ifndef PA_SLOT_SCALE_PAGES_PER_STAGE
#define PA_SLOT_SCALE_PAGES_PER_STAGE 2
#endif
constexpr int kSlotScalePagesPerStage = PA_SLOT_SCALE_PAGES_PER_STAGE;
// Two query tiles per item hold a second set of accumulators: 2 pages per stage
// keep that variant at 2 waves per SIMD too.
constexpr int kTwoTilePagesPerStage = 2;
// Three tiles per item: a third set of accumulators; one page per stage keeps
// it within 256 VGPRs (2 waves per SIMD).
constexpr int kThreeTilePagesPerStage = 1;
// Two waves per item run where a launch holds two items per CU, i.e. one wave
// per SIMD: their register budget is a whole SIMD's, spent on a ring of four
// two-page stages (three in flight while one is computed).  Measured on
// MI355X, 40/8 x 64 sequences against a ring of two four-page stages: ctx 1024
// 26.5 -> 24.4 us, 2048 47.2 -> 42.3 us, 4096 91.8 -> 87.9 us (three four-page
// stages: 25.7, 43.2, 88.8 us; four of them: slower).
constexpr int kTwoWaveRingDepth = 4;
constexpr int kTwoWaveWavesPerEU = 1;
constexpr int kTwoWavePagesPerStage = 2;

// Word 3 of a raw buffer resource (no format conversion, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;
constexpr float kLog2e = 1.4426950408889634f;
// Token rows: kv heads per workgroup (waves walking a sequence's blocks together),
// and each wave's LDS for one stage of V pages (16 rows of 128 + 8 bytes per page).
constexpr int kMaxKvPerGroup = 8;



constexpr int kVRow = kHeadDim + 8;
template <int PPS>
constexpr int kVtBytes = PPS * kBlockTokens * kVRow;

// Wave-uniform load through the scalar data cache (read-only data).
template <typename T>
__device__ __forceinline__ T scalar_load(const T* ptr) {
  return *(const __attribute__((address_space(4))) T*)(ptr);
}

// Eight fp8 e4m3fn codes (two dwords, byte order) -> eight bf16, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// Four fp8 e4m3fn codes (one dword, byte order) -> four fp16, exactly.
__device__ __forceinline__ f16x4 fp8x4_to_f16(uint32_t v) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, true);
  f16x4 r = {a[0], a[1], b[0], b[1]};
  return r;
}

// max(a, b) for values that are never NaN: the one instruction.  (fmaxf on
// values that came through a lane permute first quiets each operand, two
// more instructions.)
__device__ __forceinline__ float max_nonnan(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Max of x over lanes l, l^16, l^32, l^48 (the four 16-lane rows); x is
// never NaN (logits, or -inf where masked).
__device__ __forceinline__ float max_over_rows(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nonnan(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

// The value lane I of this lane's quad (lanes 4k .. 4k + 3) holds (DPP quad
// broadcast).  Every lane of a quad is a valid source, so with all rows and
// banks enabled no lane keeps `old`; it is still given (0), so that no lane
// can ever read an undefined register.
template <int I>
__device__ __forceinline__ uint32_t quad_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x55 * I, 0xF, 0xF, false);
}

// The four values lanes 0..3 of this lane's quad hold.
__device__ __forceinline__ u32x4 quad_gather(uint32_t v) {
  return u32x4{quad_lane<0>(v), quad_lane<1>(v), quad_lane<2>(v), quad_lane<3>(v)};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a;
  const __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Byte mask of the first n of a dword's four slots (n <= 0: none, n >= 4: all).
__device__ __forceinline__ uint32_t slot_bytes(int n) {
  return n >= 4 ? 0xFFFFFFFFu : (n <= 0 ? 0u : ((1u << (8 * n)) - 1u));
}

__device__ __forceinline__ int clamp_len(int len, int max_blocks) {
  return min(max(len, 0), max_blocks * kBlockTokens);
}

// Longest-first order: sequences bucketed by context pages into kOrderBins
// bins (bin 0 longest).  The order kernel takes up to kOrderThreads *
// kOrderPer sequences; a one-wave work item computes its own sequence for up
// to 64 * kInKernelOrderPer.
constexpr int kOrderThreads = 256;
constexpr int kOrderPer = 32;
constexpr int kOrderBins = 256;
constexpr int kInKernelOrderPer = 8;

// The sequence of longest-first slot `slot`, computed by one wave alone: the
// sequences in bin order and, within a bin, in index order (a stable counting
// sort, so every wave of the grid computes the same permutation).  The bin
// histogram lives in this wave's LDS; a wave's LDS operations run in order.
__device__ __forceinline__ int lpt_sequence(const DecodeParams& p, int slot, int plain, int lane) {
  __shared__ int cnt[kOrderBins];
  const int S = p.num_seqs;
  const int wmax = p.max_blocks > 0 ? p.max_blocks : 1;
  int bin[kInKernelOrderPer];
#pragma unroll
  for (int k = 0; k < kInKernelOrderPer; ++k) {
    const int s = lane + 64 * k;
    int b = -1;
    if (s < S) {
      const int len = min(max(p.seq_lens[s], 0), p.max_blocks * kBlockTokens);
      const int pages = (len + kBlockTokens - 1) / kBlockTokens;
      b = kOrderBins - 1 - (int)((int64_t)pages * (kOrderBins - 1) / wmax);
    }
    bin[k] = b;
  }
  // every length in one bin (a batch of equal lengths): no order to make, the
  // item keeps its sequence of the plain order (`plain`)
  const int b0 = __builtin_amdgcn_readfirstlane(bin[0]);
  uint64_t other = 0;
#pragma unroll
  for (int k = 0; k < kInKernelOrderPer; ++k) other |= __builtin_amdgcn_ballot_w64(bin[k] >= 0 && bin[k] != b0);
  if (other == 0) return plain;
#pragma unroll
  for (int b = 0; b < kOrderBins / 64; ++b) cnt[b * 64 + lane] = 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int k = 0; k < kInKernelOrderPer; ++k)
    if (bin[k] >= 0) atomicAdd(&cnt[bin[k]], 1);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  // exclusive scan over the bins: lane l owns bins 4 l .. 4 l + 3
  int c[4], st[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) c[k] = cnt[4 * lane + k];
  const int own = c[0] + c[1] + c[2] + c[3];
  int incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  st[0] = incl - own;
#pragma unroll
  for (int k = 1; k < 4; ++k) st[k] = st[k - 1] + c[k - 1];
  // the bin holding the slot, and the slot's rank within it
  int code = -1, rank = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (slot >= st[k] && slot < st[k] + c[k]) {
      code = 4 * lane + k;
      rank = slot - st[k];
    }
  const uint64_t hitm = __builtin_amdgcn_ballot_w64(code >= 0);
  if (hitm == 0) return slot;  // (not reached: every slot < S lies in some bin)
  const int hl = __builtin_ctzll(hitm);
  const int B = __builtin_amdgcn_readlane(code, hl);
  int j = __builtin_amdgcn_readlane(rank, hl);
  // the j-th sequence of bin B in index order
#pragma unroll
  for (int k = 0; k < kInKernelOrderPer; ++k) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(bin[k] == B);
    const int cntk = __builtin_popcountll(m);
    if (j < cntk) {
      const int r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      const uint64_t pick = __builtin_amdgcn_ballot_w64(((m >> lane) & 1) && r == j);
      return 64 * k + __builtin_ctzll(pick);
    }
    j -= cntk;
  }
  return slot;  // (not reached)
}

// Longest-first slots are dealt to the CUs in rounds of one work item per CU.
// Taken in plain order, every round would give the same CUs its longest
// sequences, and those CUs would get more than their share of the bytes; so
// every other round runs in reverse (a CU that takes a round's longest
// sequence takes the next round's shortest).  A bijection on [0, S).
__device__ __forceinline__ int snake_slot(int slot, int per_round, int S) {
  const int r = slot / per_round;
  if (!(r & 1)) return slot;
  const int end = min((r + 1) * per_round, S);
  return r * per_round + (end - 1 - slot);
}

template <int PPS>
struct Stage {
  u32x4 k[PPS][2];     // per page: 16 bytes of chunk (l >> 4) and of chunk 4 + (l >> 4)
  uint32_t v[PPS][8];  // per page: slots 4 e .. 4 e + 3 of dims lane (e < 4) and 64 + lane (token rows: row bytes)
  uint32_t ks[PPS];    // per-slot scale of slot 4 rq + (lane & 3) (per-slot variant only)
  uint32_t vs[PPS];
};

// SS: per-slot scale tables instead of per-tensor scales.  K scales multiply
// the logits token by token.  A V scale v_t = f_t 2^E_t (f_t in [0.5, 1))
// enters the numerator's weights: token t's numerator weight is
// 2^(z_t + E_t - mv) f_t, where mv is a running max of z_t + E_t (kept next to
// the denominator's running max m of z_t, with its own rescale of the
// accumulator), so every fp16 weight lies in [0, 1) and the largest term of
// the numerator has a weight of at least 1/2, whatever the spread of the
// scales.  The epilogue multiplies by 2^(mv - m).
// MQ: several query tokens per sequence (rows cu_seqlens_q[s] ..), causal.  The
// 16 MFMA columns then hold (query token, head) pairs: q_tile tokens of the
// tile times the group's heads.  Query i of a sequence with L tokens and q_len
// queries sees tokens 0 .. L - q_len + i, so a tile's context ends at its last
// query's position and the tokens past each column's own position are masked.
//
// NT (several queries): query tiles per item.  With NT = 2 or 3 one wave holds
// that many tiles' columns (sets of accumulators against the same K/V
// registers), so up to NT * q_tile queries of a sequence cost one read of its
// pages.
//
// WPI (page layout, one query per sequence): waves per work item.  With 2,
// wave w computes stages w, w + 2, ... of the item and wave 1 hands its
// (max, denominator, accumulator) to wave 0 through LDS at the end, which
// combines them by the log-sum-exp rule: twice the waves on a CU for the same
// work items, no second kernel.
//
// OPT (several queries): the per-logit options, softcap and ALiBi, compiled
// in.  Without them the logit loop holds no branch for them (a wave-uniform
// branch there measured 2.7% on 8 queries per sequence); window and sinks
// need no per-logit work and run in every several-queries kernel.
template <int PPS, int NB, bool SS, bool MQ, int AUX = PA_LOAD_AUX, bool TR = false, int NT = 1,
          int WPI = 1, bool OPT = false>
__global__ __launch_bounds__(TR ? 64 * kMaxKvPerGroup : 64 * WPI)
__attribute__((amdgpu_waves_per_eu(WPI == 2 ? kTwoWaveWavesPerEU : PA_WAVES_PER_EU))) void pa_decode_kernel(const DecodeParams p) {
  const int lane = threadIdx.x & 63;
  // Token rows: a workgroup holds kv_group kv heads of one sequence (one wave
  // each); on one CU at the same time, they walk the sequence's blocks at
  // about the same pace, so the token rows they share are read close together.
  // (wave-uniform, and known to be: buffer descriptors built from it stay scalar)
  // (two waves per item: the wave's share of the item's stages)
  const int wave = (TR || WPI > 1) ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
  static_assert(WPI == 1 || (WPI == 2 && !TR && !MQ && !SS && NT == 1), "two waves: plain page-layout decode");
  const int col = lane & 15;  // MFMA column (query head in group); K load row (token)
  const int rq = lane >> 4;   // row quad: rows 4*rq .. 4*rq+3 of the 16x16 tiles

  int item = blockIdx.x;
  int qt0 = 0;  // first query tile of the item (it holds NT)
  if constexpr (MQ) {
    // The items of one (sequence, kv head, partition) read the same pages:
    // place them 8 blocks apart, which puts them on one XCD (blocks go to the
    // 8 XCDs round robin) at about the same time, so one item's page reads are
    // served by that XCD's L2 for the others.
    const int ngroups = (p.num_q_tiles + NT - 1) / NT;
    const int xcd = item & 7;
    const int r = item >> 3;
    qt0 = (r % ngroups) * NT;
    item = (r / ngroups) * 8 + xcd;
    if (item >= p.num_seqs * p.num_kv_heads * p.num_parts) return;  // grid padding
  }
  int rest = item / p.num_parts;
  // partition: rotated across units, so that the first partition of every
  // unit (the one each context has) does not always land on the same XCDs.
  // Blocks go to the 8 XCDs round robin, so with P partitions a block's XCD
  // depends on the unit only through rest mod 8 / gcd(P, 8): rotating by
  // rest / (8 / gcd(P, 8)) gives every XCD every partition index in turn.
  int part = item % p.num_parts;
  if (p.num_parts > 1) {
    const int g = min(p.num_parts & -p.num_parts, 8);  // gcd(P, 8)
    part += (rest >> (3 - __builtin_ctz(g))) % p.num_parts;
    if (part >= p.num_parts) part -= p.num_parts;
  }
  const int kv_units = TR ? p.num_kv_heads / p.kv_group : p.num_kv_heads;  // work items per (sequence, partition)
  const int kvh = TR ? (rest % kv_units) * p.kv_group + wave : rest % kv_units;
  // longest-first: the sequence of this slot, from the order kernel or computed
  // here (one-wave workgroups only)
  const int plain = rest / kv_units;
  const int slot = p.lpt_round_slots > 0 ? snake_slot(plain, p.lpt_round_slots, p.num_seqs) : plain;
  const int ppp = p.pages_per_part;
  const int pbeg = part * ppp;  // < max_blocks: the planner never makes an empty partition range
  const int span = min(ppp, p.max_blocks - pbeg);
  // The sequence.  With the order computed here, the prologue's reads start
  // with the plain order's sequence (what a batch whose lengths all share one
  // bin keeps, found without a histogram) while the order is computed, and
  // are made again where it picks another sequence.
  int s = (!TR && p.order_in_kernel) ? plain : p.seq_order ? scalar_load(p.seq_order + slot) : slot;

  // column -> (query token of the tile, head of the group)
  int qi = 0, g = col, q0 = s, q_len = 1;
  int qrow[NT];      // row of q and out
  bool hvalid[NT];   // the column holds a query of this sequence
  size_t orow[NT];    // element offset of the row in out (dense)
  int32_t idv[kMaxPagesPerPart / 64];
  // B operand of QK^T: q^T, 8 dims per MFMA.  Element e of qop[h2][c] is dim
  // 16 * (4 * h2 + rq) + 8 * c + e, matching the K bytes this lane loads.
  bf16x8 qop[NT][2][2];
  int len_raw = 0;
  // Start the independent reads of the prologue together: this partition's
  // slice of the block-table row (its length is not known yet, so entries
  // past the context are read too and discarded below), the sequence length,
  // and q.
  // (false: the item's tiles hold no query of the sequence, nothing is read)
  auto prologue = [&](int sq) -> bool {
    q0 = sq;
    q_len = 1;
    if constexpr (MQ) {
      qi = col / p.group;
      g = col - qi * p.group;
      // no row offsets: one query per sequence (the options without several queries)
      q0 = p.cu_seqlens_q ? scalar_load(p.cu_seqlens_q + sq) : sq;
      q_len = p.cu_seqlens_q ? scalar_load(p.cu_seqlens_q + sq + 1) - q0 : 1;
      if (qt0 * p.q_tile >= q_len) return false;
    }
    const int hh = kvh * p.group + g;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int qt = qt0 + u;
      qrow[u] = q0 + qt * p.q_tile + qi;
      hvalid[u] = MQ ? (col < p.q_tile * p.group && qt < p.num_q_tiles && qt * p.q_tile + qi < q_len &&
                        qrow[u] >= 0 && qrow[u] < p.num_q_rows)
                     : col < p.group;
      orow[u] = ((size_t)qrow[u] * p.num_heads + hh) * kHeadDim;
    }
    const int32_t* bt = p.block_tables + (size_t)sq * p.bt_row_stride;
#pragma unroll
    for (int k = 0; k < kMaxPagesPerPart / 64; ++k)
      idv[k] = (k * 64 < span) ? bt[pbeg + min(k * 64 + lane, span - 1)] : 0;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if (hvalid[u]) {
        const uint16_t* qp = p.q + (size_t)qrow[u] * p.q_row_stride + (size_t)hh * kHeadDim;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            qop[u][h2][c] = *(const bf16x8*)(qp + 16 * (4 * h2 + rq) + 8 * c);
      } else {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            qop[u][h2][c] = bf16x8{};
      }
    }
    len_raw = scalar_load(p.seq_lens + sq);
    return true;
  };
  bool has_work = prologue(s);
  if (!TR && p.order_in_kernel) {
    int s_pick;
    if constexpr (WPI == 1) {
      s_pick = __builtin_amdgcn_readfirstlane(lpt_sequence(p, slot, plain, lane));
    } else {
      // one wave sorts (the histogram in LDS is its own); the other reads its pick
      __shared__ int lpt_pick;
      if (wave == 0) {
        const int v = lpt_sequence(p, slot, plain, lane);
        if (lane == 0) lpt_pick = v;
      }
      __syncthreads();
      s_pick = __builtin_amdgcn_readfirstlane(lpt_pick);
    }
    if (s_pick != s) {
      s = s_pick;
      has_work = prologue(s);
    }
  }
  if (!has_work) return;  // no query of this sequence in the item's tiles
  const int h = kvh * p.group + g;

  const int Lseq = clamp_len(len_raw, p.max_blocks);
  // tokens this item's queries can see: all of them for one query per sequence;
  // up to the tile's last query's position otherwise
  int L = Lseq, pos_first = Lseq - 1;
  int pos_col[NT];  // the column's query position (its causal end)
#pragma unroll
  for (int u = 0; u < NT; ++u) pos_col[u] = Lseq - 1;
  if constexpr (MQ) {
    const int base = Lseq - q_len;  // position of query 0
    L = max(0, min(Lseq, base + min((qt0 + NT) * p.q_tile, q_len)));
    pos_first = base + qt0 * p.q_tile;
#pragma unroll
    for (int u = 0; u < NT; ++u) pos_col[u] = hvalid[u] ? base + (qt0 + u) * p.q_tile + qi : L - 1;
  }
  const int npages = (L + kBlockTokens - 1) / kBlockTokens;
  const int nused = (npages + ppp - 1) / ppp;  // partitions holding tokens
  if (part > 0 && part >= nused) return;
  const bool direct = nused <= 1;  // one partition: write the final output here

  if (L == 0) {  // empty context: an all-zero row
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if (hvalid[u] && (WPI == 1 || wave == 0)) {
#pragma unroll
        for (int jd = 0; jd < 8; ++jd)
          *(uint2*)(p.out + orow[u] + jd * 16 + rq * 4) = make_uint2(0u, 0u);
      }
    }
    return;
  }

  const int pend = min(pbeg + ppp, npages);
  const int tend = min(L, pend * kBlockTokens);  // first token this item must not use
  // several queries: first token this column must not use (its own causal end)
  int tlim[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) tlim[u] = MQ ? min(tend, pos_col[u] + 1) : tend;

  // Options of the several-queries form (window, softcap, ALiBi, sinks).
  // Window: this column uses tokens tlo .. pos_col; the item starts at the
  // first whole stage holding a token any of its columns can see (pstart).
  int tlo[NT], tlo_max = INT_MIN, pstart = pbeg;
#pragma unroll
  for (int u = 0; u < NT; ++u) tlo[u] = 0;
  float slope_l2 = 0.0f, sink_l2 = -INFINITY;
  if constexpr (MQ) {
    if (p.window > 0) {
#pragma unroll
      for (int u = 0; u < NT; ++u) tlo[u] = pos_col[u] - p.window + 1;
      tlo_max = L - p.window;  // the latest window start among the item's columns
      const int lo_pg = max(0, pos_first - p.window + 1) / kBlockTokens;
      if (lo_pg > pbeg) pstart = pbeg + min(lo_pg - pbeg, ppp) / PPS * PPS;  // whole stages
    }
    if (p.alibi_slopes) slope_l2 = p.alibi_slopes[h] * kLog2e;  // h < num_heads in every lane
    if (p.sinks) sink_l2 = p.sinks[h] * kLog2e;
  }
  const int ioff = MQ ? pstart - pbeg : 0;  // first staged page this item loads

  // logits in log2 units: z * scale * k_scale * log2(e) (k_scale per slot when SS)
  const float c_log2 = SS ? p.scale_log2e : p.scale_log2e * scalar_load(p.k_scale);
  // Per-tensor scales without per-logit options: the scale enters the
  // exponent instead, each weight 2^(z |c| - m) by one fma, and the running
  // max is |c| times the max of the raw products z.  A negative scale is
  // folded into q beforehand (an exact bf16 negation), so that the raw
  // products' max is the scaled logits' max.  (|c| = 0: every weight 1.)
  constexpr bool kFold = !SS && !(MQ && OPT);
  const float c_abs = kFold ? fmaxf(fabsf(c_log2), FLT_MIN) : 0.0f;
  if (kFold && c_log2 < 0.0f) {
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          qop[u][h2][c] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qop[u][h2][c]) ^ 0x80008000u);
  }
  // softcap: the natural-unit logit z * scale * k_scale, capped, then in log2 units
  const bool capped = MQ && OPT && p.softcap > 0.0f;
  const float c_nat = MQ ? p.scale * scalar_load(p.k_scale) : 0.0f;
  const float cap_k = MQ && capped ? 2.0f * kLog2e / p.softcap : 0.0f;
  const float cap_l2 = MQ ? p.softcap * kLog2e : 0.0f;
  const bool biased = MQ && OPT && p.alibi_slopes != nullptr;

  const size_t page_stride = (size_t)p.block_stride;
  const size_t head_off = (size_t)kvh * p.head_stride;
  const uint8_t* kpage0 = p.k_cache + head_off;
  const uint8_t* vpage0 = p.v_cache + head_off;
  // K: token lane & 15, chunks lane >> 4 (koff) and 4 + (lane >> 4) (koff + khi)
  const int tstride = TR ? (int)p.token_stride : 0;
  const int koff = TR ? col * tstride + rq * 16 : lane * 16;
  constexpr int khi = TR ? 64 : 1024;
  // V (token rows): bytes 16 (lane & 7) .. +15 of tokens lane >> 3 and
  // 8 + (lane >> 3) (each load reads eight whole 128-byte rows); the page
  // layout's V loads take dims lane and 64 + lane
  const int voff = TR ? (lane >> 3) * tstride + (lane & 7) * 16 : 0;
  // bytes a page's descriptor covers
  const int page_bytes = TR ? (kBlockTokens - 1) * tstride + kHeadDim : kPageBytes;

  f32x4 acc[NT][8];  // O^T tiles: dims 16*jd + 4*rq + i for column `col`
  f32x4 accl[NT];    // softmax denominator (same value in every element)
  float m_run[NT];
  // the max the weights are taken against: m_run, except 0 for a column that
  // has seen no token yet (several queries: a causal end before this item's
  // tokens), whose every z is -inf and whose weights 2^-inf are then 0;
  // updated with m_run
  float m_ref[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
#pragma unroll
    for (int jd = 0; jd < 8; ++jd) acc[u][jd] = f32x4{0.f, 0.f, 0.f, 0.f};
    accl[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[u] = -INFINITY;
    if constexpr (MQ) {
      // the sink: one more softmax term 2^sink with no value, counted once (partition 0)
      if (part == 0 && hvalid[u] && sink_l2 > -INFINITY) {
        m_run[u] = sink_l2;
        accl[u] = f32x4{1.f, 1.f, 1.f, 1.f};
      }
    }
    m_ref[u] = (MQ && m_run[u] == -INFINITY) ? 0.0f : m_run[u];
  }
  const f16x4 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
  float mv_run = -INFINITY;  // per-slot variant: running max of z + E(v_scale), the numerator's

  // The partition's physical block ids, staged in LDS.  A load of a page past
  // the partition gets a buffer descriptor of zero bytes: it is still issued
  // (so the pipeline's wait counts do not depend on the data) but it returns
  // zeros without touching memory.  Those ids are therefore never used.
  const int npg = MQ ? max(0, pend - pstart) : pend - pbeg;
  const int nsteps = (npg + PPS - 1) / PPS;
  constexpr int kIdsCap = kMaxPagesPerPart + (WPI * NB + 1) * PPS;
  __shared__ __attribute__((aligned(16))) int32_t ids[kIdsCap];
  const int ids_fill = ioff + (nsteps + WPI * NB) * PPS;  // every index a load can reach
#pragma unroll
  for (int k = 0; k < (kIdsCap + 63) / 64; ++k) {
    const int i = k * 64 + lane;
    const int32_t v = (k < kMaxPagesPerPart / 64) ? idv[k < kMaxPagesPerPart / 64 ? k : 0] : 0;
    if (wave == 0 && k * 64 < ids_fill && i < ids_fill) ids[i] = (i < ioff + npg) ? v : 0;
  }
  __syncthreads();

  constexpr int kAux = AUX;
  // Token rows: the stage's V pages pass through LDS, row j of page pp at
  // vtb + (pp * 16 + j) * kVRow, in one of two buffers per wave (stage parity).
  // Each wave owns its buffers and a wave's LDS operations execute in order,
  // so the wave's own program order puts the writes before the gathers and
  // the gathers before the next writes into the same buffer.  Rows are
  // 128 + 8 bytes apart so that the 4-byte column gathers below (4 rows x 16
  // columns x 4 row groups) hit distinct banks.
  // (dynamic LDS, kv_group * 2 * kVtBytes<PPS> bytes, sized at launch)
  extern __shared__ __attribute__((aligned(16))) uint8_t pa_dyn_lds[];
  // (page layout: one stage of V pages per wave, PPS * kPageBytes bytes)
  uint8_t* const vt = pa_dyn_lds + (TR ? wave * 2 * kVtBytes<PPS> : wave * PPS * kPageBytes);
  auto load = [&](Stage<PPS>& st, int stage) {
    const int i0 = stage * PPS;           // page of the item (pages past npg are empty)
    const int32_t* idp = ids + ioff + i0;  // their staged block ids
    int32_t pid[PPS];
    if constexpr (PPS % 4 == 0) {
#pragma unroll
      for (int c = 0; c < PPS / 4; ++c) {
        const int4 v = *(const int4*)(idp + 4 * c);
        pid[4 * c] = v.x;
        pid[4 * c + 1] = v.y;
        pid[4 * c + 2] = v.z;
        pid[4 * c + 3] = v.w;
      }
    } else if constexpr (PPS % 2 == 0) {
#pragma unroll
      for (int c = 0; c < PPS / 2; ++c) {
        const int2 v = *(const int2*)(idp + 2 * c);
        pid[2 * c] = v.x;
        pid[2 * c + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int pp = 0; pp < PPS; ++pp) pid[pp] = idp[pp];
    }
#pragma unroll
    for (int pp = 0; pp < PPS; ++pp) {
      // a block id outside the caches (a caller error the host cannot see) reads
      // as an all-zero page instead of touching memory
      // (the same in every lane; read as such, so that the descriptors stay scalar)
      const int32_t pu = __builtin_amdgcn_readfirstlane(pid[pp]);
      const bool used = i0 + pp < npg && (uint32_t)pu < p.num_blocks_u32;
      const int bytes = used ? page_bytes : 0;
      const size_t off = (size_t)pu * page_stride;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kpage0 + off), (short)0, bytes, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)(vpage0 + off), (short)0, bytes, kRsrcWord3);
      if constexpr (SS) {
        const size_t srow = ((size_t)__builtin_amdgcn_readfirstlane(pid[pp]) * p.num_kv_heads + kvh) * kBlockTokens;
        const int sbytes = used ? kBlockTokens * 4 : 0;
        const __amdgpu_buffer_rsrc_t rks =
            __builtin_amdgcn_make_buffer_rsrc((void*)(p.k_slot_scales + srow), (short)0, sbytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rvs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(p.v_slot_scales + srow), (short)0, sbytes, kRsrcWord3);
        // one dword a lane: the scale of slot 4 rq + (lane & 3); the lane's
        // four slots 4 rq .. 4 rq + 3 are gathered from its quad at use
        st.ks[pp] = __builtin_amdgcn_raw_buffer_load_b32(rks, (rq * 4 + (lane & 3)) * 4, 0, 0);
        st.vs[pp] = __builtin_amdgcn_raw_buffer_load_b32(rvs, (rq * 4 + (lane & 3)) * 4, 0, 0);
      }
      st.k[pp][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, 0, kAux));
      st.k[pp][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff + khi, 0, kAux));
      if constexpr (TR) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w =
              __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff + 8 * h * tstride, 0, kAux));
#pragma unroll
          for (int e = 0; e < 4; ++e) st.v[pp][4 * h + e] = w[e];
        }
      } else {
        // dims lane and 64 + lane, all 16 slots
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w =
              __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane * 16 + 1024 * h, 0, kAux));
#pragma unroll
          for (int e = 0; e < 4; ++e) st.v[pp][4 * h + e] = w[e];
        }
      }
    }
    // keep the scheduler from hoisting compute above these loads
    __builtin_amdgcn_sched_barrier(0);
  };

  // PV operand: dims 16 jd + col, tokens 4 rq .. 4 rq + 3 of page pp (byte i = token 4 rq + i)
  auto vword = [&](const Stage<PPS>& st, const uint8_t* vtb, int pp, int jd) -> uint32_t {
    if constexpr (TR) {
      const uint8_t* b = vtb + (pp * kBlockTokens + 4 * rq) * kVRow + 16 * jd + col;
      return (uint32_t)b[0] | ((uint32_t)b[kVRow] << 8) | ((uint32_t)b[2 * kVRow] << 16) |
             ((uint32_t)b[3 * kVRow] << 24);
    } else {
      return *(const uint32_t*)(vtb + pp * kPageBytes + (col + 16 * jd) * 16 + 4 * rq);
    }
  };

  auto compute = [&](Stage<PPS>& st, int stage, bool last) {
    const int j0 = pstart + stage * PPS;
    if (last) {
      // Slots past the context may hold anything (even NaN): their V bytes are
      // zeroed here, once, so that no PV operand needs a mask.
#pragma unroll
      for (int pp = 0; pp < PPS; ++pp) {
        const int nv = tend - (j0 + pp) * kBlockTokens;  // tokens of the page to keep
        if constexpr (TR) {
          // dwords 4 h .. 4 h + 3: 16 bytes of token 8 h + (lane >> 3)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              st.v[pp][4 * h + e] = 8 * h + (lane >> 3) < nv ? st.v[pp][4 * h + e] : 0u;
        } else {
          // dword 4 h + e: slots 4 e .. 4 e + 3 of one dim
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) st.v[pp][4 * h + e] &= slot_bytes(nv - 4 * e);
        }
      }
    }
    uint8_t* const vtb = vt + (TR ? (stage & 1) * kVtBytes<PPS> : 0);
    if constexpr (!TR) {
      // the stage's V pages, copied as they are (one buffer: the wave's LDS
      // operations run in order, so these writes follow the last stage's reads)
#pragma unroll
      for (int pp = 0; pp < PPS; ++pp) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          *(u32x4*)(vtb + pp * kPageBytes + 1024 * h + lane * 16) =
              u32x4{st.v[pp][4 * h], st.v[pp][4 * h + 1], st.v[pp][4 * h + 2], st.v[pp][4 * h + 3]};
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
    if constexpr (TR) {
#pragma unroll
      for (int pp = 0; pp < PPS; ++pp) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint8_t* dst = vtb + (pp * kBlockTokens + 8 * h + (lane >> 3)) * kVRow + (lane & 7) * 16;
          *(uint2*)dst = make_uint2(st.v[pp][4 * h], st.v[pp][4 * h + 1]);
          *(uint2*)(dst + 8) = make_uint2(st.v[pp][4 * h + 2], st.v[pp][4 * h + 3]);
        }
      }
      // the wave's own buffer: its LDS writes and the gathers below are
      // ordered by the wave alone (no barrier: measured, holding the
      // workgroup's waves in step cost 10% on NHD caches)
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    }
    // columns with their own causal end: the stages reaching past the tile's first
    // position; with a window, also the stages before the latest window start
    const bool causal = MQ && ((j0 + PPS) * kBlockTokens > pos_first + 1 || j0 * kBlockTokens < tlo_max);
    f32x4 z[NT][PPS];
#pragma unroll
    for (int pp = 0; pp < PPS; ++pp) {
      bf16x8 kb[2][2];  // the page's K operand, shared by the item's tiles
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x4 kk = st.k[pp][h2];
        kb[h2][0] = fp8x8_to_bf16(kk[0], kk[1]);
        kb[h2][1] = fp8x8_to_bf16(kk[2], kk[3]);
      }
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[h2][0], qop[u][h2][0], t, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[h2][1], qop[u][h2][1], t, 0, 0, 0);
        }
        z[u][pp] = t;
      }
    }
    // per-slot K scales of the lane's four slots of each page
    u32x4 ksq[PPS];
    if constexpr (SS) {
#pragma unroll
      for (int pp = 0; pp < PPS; ++pp) ksq[pp] = quad_gather(st.ks[pp]);
    }
    // scale (and the options: softcap, ALiBi), mask, running max.  The mask,
    // which only stages at a causal end or window start need, sits under one
    // wave-uniform branch for all tiles.
    const bool masked = last || causal;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if constexpr (MQ && OPT) {
#pragma unroll
        for (int pp = 0; pp < PPS; ++pp) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = z[u][pp][i] * c_log2;
            if (capped) {
              // c tanh(z / c) = c (1 - 2 / (e^(2 z / c) + 1)), then in log2 units
              const float e2 = __builtin_amdgcn_exp2f(z[u][pp][i] * c_nat * cap_k);
              v = cap_l2 * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e2 + 1.0f));
            }
            if (biased) v += slope_l2 * (float)((j0 + pp) * kBlockTokens + rq * 4 + i - pos_col[u]);
            z[u][pp][i] = v;
          }
        }
      } else if constexpr (!kFold) {
#pragma unroll
        for (int pp = 0; pp < PPS; ++pp) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = z[u][pp][i] * c_log2;
            if constexpr (SS) v *= __uint_as_float(ksq[pp][i]);
            z[u][pp][i] = v;
          }
        }
      }
    }
    if (masked) {
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int pp = 0; pp < PPS; ++pp)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = (j0 + pp) * kBlockTokens + rq * 4 + i;
            const bool keep = MQ ? (t < tlim[u] && t >= tlo[u]) : t < tlim[u];
            z[u][pp][i] = keep ? z[u][pp][i] : -INFINITY;
          }
    }
    // Each lane's max over its own rows of the stage first: where no lane's
    // exceeds the tile's running max, no column max can (the running max is
    // then unchanged), so the max across the four row groups and the rescale
    // run only where some lane's does.
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      float mx = -INFINITY;
#pragma unroll
      for (int pp = 0; pp < PPS; ++pp)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[u][pp][i]);
      if (__builtin_amdgcn_ballot_w64((kFold ? mx * c_abs : mx) > m_run[u])) {
        const float mr = max_over_rows(mx);
        const float m_new = fmaxf(m_run[u], kFold ? mr * c_abs : mr);
        const float alpha = (m_new == m_run[u]) ? 1.0f : __builtin_amdgcn_exp2f(m_run[u] - m_new);
        if constexpr (!SS) {  // (per-slot: the numerator has a running max of its own)
#pragma unroll
          for (int jd = 0; jd < 8; ++jd) acc[u][jd] *= alpha;
        }
        accl[u] *= alpha;
        m_run[u] = m_new;
        m_ref[u] = (MQ && m_new == -INFINITY) ? 0.0f : m_new;
      }
    }
    // P = 2^(z - m) in fp16, then PV
    // per-slot V scales v = f 2^E: the numerator's logits z + E, their running
    // max, and the accumulator rescaled when it grows
    float zv[SS ? PPS : 1][4], vf[SS ? PPS : 1][4];
    if constexpr (SS) {
      float mxv = -INFINITY;
#pragma unroll
      for (int pp = 0; pp < PPS; ++pp) {
        const u32x4 vsq = quad_gather(st.vs[pp]);  // the lane's four slots' V scales
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float vsc = __uint_as_float(vsq[i]);
          vf[pp][i] = __builtin_amdgcn_frexp_mantf(vsc);
          // a zero scale adds exactly nothing: it must not set the numerator's max
          zv[pp][i] = vf[pp][i] == 0.0f ? -INFINITY : z[0][pp][i] + (float)__builtin_amdgcn_frexp_expf(vsc);
          mxv = fmaxf(mxv, zv[pp][i]);
        }
      }
      if (__builtin_amdgcn_ballot_w64(mxv > mv_run)) {  // (as for m above)
        const float mv_new = fmaxf(mv_run, max_over_rows(mxv));
        const float beta = (mv_new == mv_run) ? 1.0f : __builtin_amdgcn_exp2f(mv_run - mv_new);
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) acc[0][jd] *= beta;
        mv_run = mv_new;
      }
    }
#pragma unroll
    for (int pp = 0; pp < PPS; ++pp) {
      if constexpr (SS) {
        f16x4 pb, pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(z[0][pp][i] - m_run[0]);
          pb[i] = (_Float16)e;
          // 2^(z + E - mv) f in [0, 1); tokens past the context (z = -inf; their
          // scale may be NaN) and zero scales give 0 (mv may still be -inf)
          const float w = zv[pp][i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(zv[pp][i] - mv_run) * vf[pp][i];
          pv[i] = (_Float16)w;
        }
#pragma unroll
        for (int jd = 0; jd < 8; ++jd)
          acc[0][jd] = __builtin_amdgcn_mfma_f32_16x16x16f16(fp8x4_to_f16(vword(st, vtb, pp, jd)), pv, acc[0][jd], 0, 0, 0);
        accl[0] = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, pb, accl[0], 0, 0, 0);
      } else {
        f16x4 pb[NT];
#pragma unroll
        for (int u = 0; u < NT; ++u) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pb[u][i] = (_Float16)__builtin_amdgcn_exp2f(kFold ? __builtin_fmaf(z[u][pp][i], c_abs, -m_ref[u])
                                                              : z[u][pp][i] - m_ref[u]);
        }
#pragma unroll
        for (int jd = 0; jd < 8; ++jd) {
          const f16x4 va = fp8x4_to_f16(vword(st, vtb, pp, jd));  // shared by the tiles
#pragma unroll
          for (int u = 0; u < NT; ++u) acc[u][jd] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pb[u], acc[u][jd], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < NT; ++u) accl[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, pb[u], accl[u], 0, 0, 0);
      }
    }
  };

  // Register ring of NB stages: NB - 1 stages are in flight while one is
  // computed.  Loads past the last stage are empty (see above).  With two
  // waves per item, the wave's i-th stage is stage 2 i + wave of the item.
  Stage<PPS> ring[NB];
  // (token rows: the waves of a workgroup are kv heads, each with every stage)
  const int wsub = WPI > 1 ? wave : 0;
  const int nloc = WPI == 1 ? nsteps : max(0, (nsteps - wsub + WPI - 1) / WPI);
#pragma unroll
  for (int k = 0; k < NB - 1; ++k) load(ring[k], WPI * k + wsub);
  for (int st = 0; st < nloc; st += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (st + k >= nloc) break;
      load(ring[(k + NB - 1) % NB], WPI * (st + k + NB - 1) + wsub);
      const int g = WPI * (st + k) + wsub;
      compute(ring[k], g, g == nsteps - 1);
    }
  }
  if constexpr (WPI == 2) {
    // Wave 1's (max, denominator, accumulator) to wave 0, lane by lane (both
    // waves hold the same (head, dims) in a lane), combined as
    // m = max(m0, m1), acc = acc0 2^(m0 - m) + acc1 2^(m1 - m), likewise l.
    __shared__ f32x4 x_acc[8][64];
    __shared__ float x_m[64], x_l[64];
    if (wave == 1) {
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) x_acc[jd][lane] = acc[0][jd];
      x_m[lane] = m_run[0];
      x_l[lane] = accl[0][0];
    }
    __syncthreads();
    if (wave == 1) return;
    const float m1 = x_m[lane];
    const float m = fmaxf(m_run[0], m1);
    if (m > -INFINITY) {  // (-inf in both: a column that holds no head)
      const float f0 = __builtin_amdgcn_exp2f(m_run[0] - m);
      const float f1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) acc[0][jd] = acc[0][jd] * f0 + x_acc[jd][lane] * f1;
      const float l = accl[0][0] * f0 + x_l[lane] * f1;
      accl[0] = f32x4{l, l, l, l};
      m_run[0] = m;
    }
  }

  // Partials go through buffer descriptors based at the item's first row
  // (offsets stay small), stored agent-coherent (sc1: written through the
  // XCD's L2).  The merge in the decode's last item needs that; for the merge
  // kernel it leaves fewer dirty lines for the kernel's end to write back
  // (measured on MI355X: 40/8 ctx 1024 x 16 13.1 -> 12.8 us, 2 x 8192 13.5 ->
  // 13.1 us; nontemporal stores instead: 1-1.7 us slower).
  constexpr int kAuxSc1 = 16;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    if (!hvalid[u]) continue;
    const float lsum = accl[u][0];
    if (direct) {
      // several queries: lsum is 0 for a query that sees no token (more queries than context)
      const float inv = (!MQ || lsum > 0.0f)
                            ? (SS ? __builtin_amdgcn_exp2f(mv_run - m_run[u]) : scalar_load(p.v_scale)) / lsum
                            : 0.0f;
      uint16_t* o = p.out + orow[u] + rq * 4;
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) {
        const f32x4 a = acc[u][jd];
        *(uint2*)(o + jd * 16) = make_uint2(pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv));
      }
    } else if constexpr (MQ) {
      // (several queries: a lane's row depends on its query, so the partials
      // take plain stores with 64-bit addresses)
      const size_t prow = ((size_t)qrow[u] * p.num_heads + h) * p.num_parts + part;
      float* a = p.part_acc + prow * kHeadDim + rq * 4;
#pragma unroll
      for (int jd = 0; jd < 8; ++jd) *(f32x4*)(a + jd * 16) = acc[u][jd];
      if (rq == 0) *(float2*)(p.part_ml + prow * 2) = make_float2(m_run[u], lsum);
    } else {
      // row (sequence, head) = rbase + lrow: rbase the kv head's first head
      // (wave-uniform), lrow the lane's head; offsets below 16 x P x 512 bytes
      const size_t rbase = ((size_t)s * p.num_heads + (size_t)kvh * p.group) * p.num_parts;
      const int lrow = g * p.num_parts + part;
      // per-slot scales: the numerator relative to the denominator's max m
      const float vfold = SS ? __builtin_amdgcn_exp2f(mv_run - m_run[u]) : 1.0f;
      const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)(p.part_acc + rbase * kHeadDim), (short)0, 0x7FFFFFF0,
                                                        kRsrcWord3);
      const auto rm = __builtin_amdgcn_make_buffer_rsrc((void*)(p.part_ml + rbase * 2), (short)0, 0x7FFFFFF0,
                                                        kRsrcWord3);
#pragma unroll
      for (int jd = 0; jd < 8; ++jd)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[u][jd] * vfold), ra,
                                               (lrow * kHeadDim + rq * 4 + jd * 16) * 4, 0, kAuxSc1);
      if (rq == 0)
        __builtin_amdgcn_raw_buffer_store_b64(
            __builtin_bit_cast(__attribute__((__vector_size__(8))) uint32_t, make_float2(m_run[u], lsum)), rm,
            lrow * 8, 0, kAuxSc1);
    }
  }
  if constexpr (!MQ) {
    if (!direct && p.fused_merge) {
      // Arrival: once this item's partial stores are performed, count it; the
      // unit's last item (count nused - 1 before its own) merges, and leaves
      // the counter at zero for the next call.
      // (the signal fences keep the compiler from moving memory accesses
      // across the wait and the count)
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      const int unit = s * p.num_kv_heads + kvh;
      int before = 0;
      if (lane == 0) before = __hip_atomic_fetch_add(p.unit_count + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      before = __builtin_amdgcn_readlane(before, 0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (before != nused - 1) return;
      if (lane == 0) __hip_atomic_store(p.unit_count + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // The unit's G heads x nused partitions (nused <= 4, G * nused <= 40): lane (hs, d4)
      // takes dims 4 d4 .. 4 d4 + 3 of heads 2 k + hs, three head pairs (all
      // their partitions' loads in flight together) at a time.
      const int hs = lane >> 5, d4 = lane & 31;
      const float vsc = SS ? 1.0f : scalar_load(p.v_scale);
      const size_t row0 = (size_t)s * p.num_heads + (size_t)kvh * p.group;  // (s, first head of the group)
      const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)(p.part_acc + row0 * p.num_parts * kHeadDim), (short)0,
                                                        0x7FFFFFF0, kRsrcWord3);
      const auto rm = __builtin_amdgcn_make_buffer_rsrc((void*)(p.part_ml + row0 * p.num_parts * 2), (short)0,
                                                        0x7FFFFFF0, kRsrcWord3);
      constexpr int kPairs = 3;
      for (int k0 = 0; 2 * k0 < p.group; k0 += kPairs) {
        f32x4 av[kPairs][kFusedMergeMaxParts];
        float2 mv[kPairs][kFusedMergeMaxParts];
#pragma unroll
        for (int kk = 0; kk < kPairs; ++kk) {
          const int g2 = 2 * (k0 + kk) + hs;
#pragma unroll
          for (int j = 0; j < kFusedMergeMaxParts; ++j) {
            av[kk][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            mv[kk][j] = make_float2(-INFINITY, 0.f);
            if (g2 < p.group && j < nused) {
              const int pr = g2 * p.num_parts + j;
              av[kk][j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        ra, (pr * kHeadDim + 4 * d4) * 4, 0, kAuxSc1));
              mv[kk][j] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rm, pr * 8, 0, kAuxSc1));
            }
          }
        }
#pragma unroll
        for (int kk = 0; kk < kPairs; ++kk) {
          const int g2 = 2 * (k0 + kk) + hs;
          float M = -INFINITY;
#pragma unroll
          for (int j = 0; j < kFusedMergeMaxParts; ++j) M = fmaxf(M, mv[kk][j].x);
          f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
          float den = 0.f;
#pragma unroll
          for (int j = 0; j < kFusedMergeMaxParts; ++j) {
            const float w = mv[kk][j].x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv[kk][j].x - M);
            num += av[kk][j] * w;
            den += mv[kk][j].y * w;
          }
          if (g2 < p.group) {
            const float inv = den > 0.0f ? vsc / den : 0.0f;
            *(uint2*)(p.out + (row0 + g2) * kHeadDim + 4 * d4) =
                make_uint2(pack_bf16x2(num[0] * inv, num[1] * inv), pack_bf16x2(num[2] * inv, num[3] * inv));
          }
        }
      }
    }
  }
}

// Log-sum-exp merge of the partitions of one (sequence, query head):
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = v_scale * sum_p w_p a_p / sum_p w_p l_p.
// Sequences whose context fits one partition were finished by the decode kernel.
// 256 threads: thread t owns dims 4*(t & 31) .. +3 of partitions p = t >> 5 (mod 8),
// merged on the fly against a running max; the eight partial results are then
// combined in LDS with the same formula.
constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void pa_merge_kernel(const DecodeParams p) {
  const int t = threadIdx.x;
  const int sh = blockIdx.x;  // (query row, head)
  const int r = sh / p.num_heads;
  int s = r, L = 0;
  if (p.multi_query && p.cu_seqlens_q) {
    // the row's sequence: last s with cu_seqlens_q[s] <= r
    int lo = 0, hi = p.num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (scalar_load(p.cu_seqlens_q + mid) <= r) lo = mid; else hi = mid;
    }
    s = lo;
    const int q0 = scalar_load(p.cu_seqlens_q + s);
    const int q_len = scalar_load(p.cu_seqlens_q + s + 1) - q0;
    const int Lseq = clamp_len(scalar_load(p.seq_lens + s), p.max_blocks);
    const int qt = (r - q0) / p.q_tile;
    if (qt >= p.num_q_tiles) return;  // past max_seqlen_q: not computed
    // the decode item holding this row covered tiles up to the end of its group
    const int tiles_end = (qt / p.tiles_per_item + 1) * p.tiles_per_item;
    L = max(0, min(Lseq, Lseq - q_len + min(tiles_end * p.q_tile, q_len)));
  } else {
    L = clamp_len(scalar_load(p.seq_lens + s), p.max_blocks);
  }
  const int npages = (L + kBlockTokens - 1) / kBlockTokens;
  const int nused = (npages + p.pages_per_part - 1) / p.pages_per_part;
  if (nused <= 1) return;  // uniform over the block

  __shared__ float red_max[8];
  __shared__ float4 red_acc[8][32];
  __shared__ float red_den[8];

  // Thread (pl, d4) folds partitions pl, pl + 8, ... into a running
  // (max, numerator, denominator) as it goes, so all of its loads are
  // independent of any reduction and issue together (one memory round trip).
  const int d4 = t & 31;
  const int pl = t >> 5;
  const float2* ml = (const float2*)(p.part_ml + (size_t)sh * p.num_parts * 2);
  const float4* acc = (const float4*)(p.part_acc + (size_t)sh * p.num_parts * kHeadDim) + d4;
  float m = -INFINITY;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  constexpr int kChunk = 8;  // partitions per thread loaded before any is folded
  for (int i0 = pl; i0 < nused; i0 += 8 * kChunk) {
    float2 mlv[kChunk];
    float4 av[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int i = i0 + 8 * u;
      mlv[u] = i < nused ? ml[i] : make_float2(-INFINITY, 0.f);
      av[u] = i < nused ? acc[(size_t)i * (kHeadDim / 4)] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      // m = -inf (l = 0): a partition a causal query saw none of, or past nused
      if (mlv[u].x == -INFINITY) continue;
      const float mn = fmaxf(m, mlv[u].x);
      const float so = __builtin_amdgcn_exp2f(m - mn);  // 0 while m = -inf
      const float sn = __builtin_amdgcn_exp2f(mlv[u].x - mn);
      den = den * so + mlv[u].y * sn;
      num.x = num.x * so + av[u].x * sn;
      num.y = num.y * so + av[u].y * sn;
      num.z = num.z * so + av[u].z * sn;
      num.w = num.w * so + av[u].w * sn;
      m = mn;
    }
  }
  red_acc[pl][d4] = num;
  if (d4 == 0) {
    red_max[pl] = m;
    red_den[pl] = den;
  }
  __syncthreads();
  if (t < 32) {
    float M = red_max[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) M = fmaxf(M, red_max[k]);
    float4 n = make_float4(0.f, 0.f, 0.f, 0.f);
    float dsum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = red_max[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(red_max[k] - M);
      const float4 a = red_acc[k][t];
      n.x += w * a.x;
      n.y += w * a.y;
      n.z += w * a.z;
      n.w += w * a.w;
      dsum += w * red_den[k];
    }
    const float inv = dsum > 0.0f ? (p.v_slot_scales ? 1.0f : scalar_load(p.v_scale)) / dsum : 0.0f;
    *(uint2*)(p.out + (size_t)sh * kHeadDim + 4 * t) =
        make_uint2(pack_bf16x2(n.x * inv, n.y * inv), pack_bf16x2(n.z * inv, n.w * inv));
  }
}

}  // namespace

// Sequences ordered by length, longest first (by context pages, in kOrderBins
// buckets; order within a bucket is arbitrary, which no result depends on:
// every work item computes the same thing in any order).  One workgroup: each
// thread reads the lengths of up to kOrderPer sequences once and keeps their
// buckets, a bucket histogram in LDS, an exclusive scan from the longest bucket
// down, then each sequence takes the next slot of its bucket.  More sequences
// than the workgroup holds keep the plain order (the host does not order them).

__global__ __launch_bounds__(kOrderThreads) void pa_order_kernel(const DecodeParams p) {
  __shared__ int cnt[kOrderBins];
  __shared__ int wave_sum[kOrderThreads / 64];
  const int t = threadIdx.x;
  const int S = p.num_seqs;
  const int wmax = p.max_blocks > 0 ? p.max_blocks : 1;  // pages of the longest possible context
  int bin[kOrderPer];
#pragma unroll
  for (int k = 0; k < kOrderPer; ++k) {
    const int s = t + k * kOrderThreads;
    int b = -1;
    if (s < S) {
      const int pages = (clamp_len(p.seq_lens[s], p.max_blocks) + kBlockTokens - 1) / kBlockTokens;
      b = kOrderBins - 1 - (int)((int64_t)pages * (kOrderBins - 1) / wmax);  // 0 = longest
    }
    bin[k] = b;
  }
  if (t < kOrderBins) cnt[t] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kOrderPer; ++k)
    if (bin[k] >= 0) atomicAdd(&cnt[bin[k]], 1);
  __syncthreads();
  // exclusive scan of the bins (one bin per thread)
  static_assert(kOrderBins == kOrderThreads, "one bin per thread");
  const int own = t < kOrderBins ? cnt[t] : 0;
  const int lane = t & 63;
  int incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_sum[t >> 6] = incl;
  __syncthreads();
  int base = incl - own;
  for (int w = 0; w < (t >> 6); ++w) base += wave_sum[w];
  __syncthreads();
  if (t < kOrderBins) cnt[t] = base;  // first slot of the bin
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kOrderPer; ++k)
    if (bin[k] >= 0) p.seq_order[atomicAdd(&cnt[bin[k]], 1)] = t + k * kOrderThreads;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  // per-logit options (several-queries kernels only): the instantiations that hold them
  const bool opt = p.softcap > 0.0f || p.alibi_slopes != nullptr;
  if (p.seq_order)
    hipLaunchKernelGGL(pa_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, p);
  const size_t units = (size_t)p.num_seqs * p.num_kv_heads * p.num_parts;
  // several queries: units padded to a multiple of 8, times the groups of tiles
  const size_t items = p.multi_query
                           ? (units + 7) / 8 * 8 * (size_t)((p.num_q_tiles + p.tiles_per_item - 1) / p.tiles_per_item)
                           : units;
  if (p.token_rows)
    hipLaunchKernelGGL((pa_decode_kernel<kPagesPerStage, kRingDepth, false, false, PA_LOAD_AUX, true>),
                       dim3((unsigned)(items / p.kv_group)), dim3(64 * p.kv_group),
                       (unsigned)(p.kv_group * 2 * kVtBytes<kPagesPerStage>), stream, p);
  // V through LDS in every several-queries and per-slot kernel, measured
  // faster on MI355X (40/8 ctx 4096 x 256): two query tiles per item (4
  // queries: 372.9 -> 369.4 us), per-slot scales (339.8 -> 335.6 us), one
  // tile (3 queries 327.3 -> 321.9 us, ALiBi 333.0 -> 327.5, sinks 346.4 ->
  // 341.5, window 1024 94.0 -> 90.6; 64 x 1024, 2 queries 38.4 -> 36.1)
  else if (p.multi_query && opt && p.tiles_per_item == 3)
    hipLaunchKernelGGL((pa_decode_kernel<kThreeTilePagesPerStage, kRingDepth, false, true, PA_LOAD_AUX, false, 3, 1, true>),
                       dim3((unsigned)items), dim3(64), kThreeTilePagesPerStage * kPageBytes, stream, p);
  else if (p.multi_query && opt && p.tiles_per_item == 2)
    hipLaunchKernelGGL((pa_decode_kernel<kTwoTilePagesPerStage, kRingDepth, false, true, PA_LOAD_AUX, false, 2, 1, true>),
                       dim3((unsigned)items), dim3(64), kTwoTilePagesPerStage * kPageBytes, stream, p);
  else if (p.multi_query && opt)
    hipLaunchKernelGGL((pa_decode_kernel<kPagesPerStage, kRingDepth, false, true, PA_LOAD_AUX, false, 1, 1, true>),
                       dim3((unsigned)items), dim3(64), kPagesPerStage * kPageBytes, stream, p);
  else if (p.multi_query && p.tiles_per_item == 3)
    hipLaunchKernelGGL((pa_decode_kernel<kThreeTilePagesPerStage, kRingDepth, false, true, PA_LOAD_AUX, false, 3>),
                       dim3((unsigned)items), dim3(64), kThreeTilePagesPerStage * kPageBytes, stream, p);
  else if (p.multi_query && p.tiles_per_item == 2 && p.num_q_tiles > 2)
    hipLaunchKernelGGL((pa_decode_kernel<kTwoTilePagesPerStage, kRingDepth, false, true, 0, false, 2>),
                       dim3((unsigned)items), dim3(64), kTwoTilePagesPerStage * kPageBytes, stream, p);
  else if (p.multi_query && p.tiles_per_item == 2)
    hipLaunchKernelGGL((pa_decode_kernel<kTwoTilePagesPerStage, kRingDepth, false, true, PA_LOAD_AUX, false, 2>),
                       dim3((unsigned)items), dim3(64), kTwoTilePagesPerStage * kPageBytes, stream, p);
  else if (p.multi_query)
    hipLaunchKernelGGL((pa_decode_kernel<kPagesPerStage, kRingDepth, false, true, PA_LOAD_AUX, false, 1>),
                       dim3((unsigned)items), dim3(64), kPagesPerStage * kPageBytes, stream, p);
  else if (p.k_slot_scales)
    hipLaunchKernelGGL((pa_decode_kernel<kSlotScalePagesPerStage, kRingDepth, true, false, PA_LOAD_AUX, false, 1>),
                       dim3((unsigned)items), dim3(64), kSlotScalePagesPerStage * kPageBytes, stream, p);
  else if (p.waves_per_item == 2 && p.cached_loads)
    hipLaunchKernelGGL((pa_decode_kernel<kTwoWavePagesPerStage, kTwoWaveRingDepth, false, false, 0, false, 1, 2>),
                       dim3((unsigned)items), dim3(128), 2 * kTwoWavePagesPerStage * kPageBytes, stream, p);
  else if (p.waves_per_item == 2)
    hipLaunchKernelGGL((pa_decode_kernel<kTwoWavePagesPerStage, kTwoWaveRingDepth, false, false, PA_LOAD_AUX, false, 1, 2>),
                       dim3((unsigned)items), dim3(128), 2 * kTwoWavePagesPerStage * kPageBytes, stream, p);
  else if (p.cached_loads)
    hipLaunchKernelGGL((pa_decode_kernel<kPagesPerStage, kRingDepth, false, false, 0, false, 1>), dim3((unsigned)items),
                       dim3(64), kPagesPerStage * kPageBytes, stream, p);
  else  // V through LDS (two 16-byte loads a page instead of eight dword loads), with
        // either cache policy: a wave alone on its SIMD streams a page faster, which is
        // what the long items of a ragged batch are (measured on MI355X, working
        // sets in the Infinity Cache, graph replay: ragged 1..4000 x 256 at 8/1
        // 38.8 -> 28.8 us, 40/8 x 32 37.9 -> 27.6 us, 256 x {4000, 100, 100, 100}
        // 39.0 -> 28.4 us; uniform batches from 7% faster to 6% slower, e.g. 40/8
        // ctx 1024 x 16 12.0 -> 11.2 us, x 64 24.6 -> 26.2 us; on the streamed
        // sets: 40/8 ctx 4096 x 256 327.6 -> 326.9 us, ragged 216.7 -> 202.5 us)
    hipLaunchKernelGGL((pa_decode_kernel<kPagesPerStage, kRingDepth, false, false, PA_LOAD_AUX, false, 1>),
                       dim3((unsigned)items), dim3(64), kPagesPerStage * kPageBytes, stream, p);
  const size_t rows = p.multi_query ? (size_t)p.num_q_rows : (size_t)p.num_seqs;
  if (p.num_parts > 1 && rows > 0 && !p.fused_merge)
    hipLaunchKernelGGL(pa_merge_kernel, dim3((unsigned)(rows * p.num_heads)), dim3(kMergeThreads), 0, stream,
                       p);
  return hipGetLastError();
}

}  // namespace pa
