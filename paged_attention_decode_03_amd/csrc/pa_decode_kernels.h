// Internal interface between the C-ABI layer (pa_api.hip) and the gfx950
// kernels (pa_decode_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kHeadDim = 128;
constexpr int kBlockTokens = 16;
constexpr int kPageBytes = kHeadDim * kBlockTokens;  // one (block, kv head) page of fp8
constexpr int kMaxGroup = 16;                         // query heads per kv head (MFMA N)
constexpr int kMaxPagesPerPart = 256;                 // blocks per work item (LDS id buffer)

struct DecodeParams {
  const uint16_t* q;         // bf16 rows of [Hq][128], q_row_stride elements apart
  const uint8_t* k_cache;    // fp8 pages [8][16][16] (or token rows, below)
  const uint8_t* v_cache;    // fp8 pages [128][16]
  const int32_t* block_tables;  // [S] rows of W entries, bt_row_stride elements apart
  const int32_t* seq_lens;      // [S]
  int64_t q_row_stride;      // elements between consecutive q rows (>= Hq * 128)
  int64_t bt_row_stride;     // elements between consecutive block-table rows (>= W)
  const float* k_scale;      // [1] (per-tensor scales)
  const float* v_scale;      // [1]
  const float* k_slot_scales;  // [NB][Hkv][16] per-slot scales, or null for per-tensor
  const float* v_slot_scales;
  uint16_t* out;             // bf16 [rows][Hq][128], dense
  float* part_acc;           // [S][Hq][P][128] unnormalised partial outputs (P > 1 only)
  float* part_ml;            // [S][Hq][P][2]   (running max in log2 units, sum of weights)
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;             // num_heads / num_kv_heads, 1..16
  int32_t max_blocks;        // W, block-table row length
  uint32_t num_blocks_u32;   // physical blocks in the caches (capped at 2^31 - 1)
  int32_t num_parts;         // P, partitions per sequence
  int32_t pages_per_part;    // blocks per partition
  float scale_log2e;         // softmax scale * log2(e)
  int32_t cached_loads;      // plain decode: K/V loads with the default cache policy (else nt)
  // the several-queries kernel (its options included); cu_seqlens_q null: one
  // query per sequence
  int32_t multi_query;
  const int32_t* cu_seqlens_q;  // [S + 1] query row offsets
  int32_t num_q_rows;        // cu_seqlens_q[S]: rows of q and out
  int32_t q_tile;            // query tokens per work item (columns = q_tile * group <= 16)
  int32_t num_q_tiles;       // query tiles per sequence (from the host's max_seqlen_q)
  int32_t tiles_per_item;    // query tiles one work item holds (1 to 3)
  // options of the several-queries form (0 / null: off)
  int32_t window;            // a query at position p sees tokens p - window + 1 .. p
  float softcap;             // logit z -> softcap * tanh(z / softcap)
  float scale;               // softmax scale (natural units, for the softcap)
  const float* alibi_slopes;  // [Hq]: logit + slope * (t - p)
  const float* sinks;         // [Hq]: extra softmax term exp(sink) with no value
  // cache addressing, bytes from k_cache / v_cache: the page of kv head k in
  // block p at p * block_stride + k * head_stride (page layout); with token
  // rows (token_rows != 0), token j's 128 dims at p * block_stride +
  // j * token_stride + k * head_stride
  int32_t token_rows;
  int32_t kv_group;          // token rows: kv heads per workgroup (divides num_kv_heads, <= 8)
  int64_t block_stride;
  int64_t token_stride;
  int64_t head_stride;
  // longest-first dispatch: work items take sequence seq_order[i] for the i-th
  // sequence slot (written by the order kernel before the decode); null: in order
  int32_t* seq_order;
  // longest-first computed by each work item itself (one-wave workgroups,
  // num_seqs <= 512); excludes seq_order
  int32_t order_in_kernel;
  // longest-first with one query per sequence: sequence slots per round of
  // work items (one item per CU a round); every other round takes its slots in
  // reverse order.  0: slots in plain longest-first order
  int32_t lpt_round_slots;
  // waves per work item: 1, or 2 (the page-layout decode with one query per
  // sequence and per-tensor scales only)
  int32_t waves_per_item;
  // split contexts with few partitions (one query per sequence): the last
  // item of each (sequence, kv head) to finish merges the partitions itself
  // (no merge kernel).  unit_count: one arrival counter per (sequence, kv
  // head), zero before and after every call
  int32_t fused_merge;
  int32_t* unit_count;
};
// partitions a fused merge folds: measured on MI355X, 32/8 heads x 24
// sequences (4 partitions): ctx 1024 15.2 -> 14.7 us, ctx 4096 34.7 -> 34.0 us;
// at 8 partitions (40/8 x 16 sequences) the last item's loads made it slower
// than the merge kernel (ctx 1024 12.9 -> 13.9 us)
constexpr int kFusedMergeMaxParts = 4;
constexpr int kFusedMergeMaxLoads = 40;   // group size x partitions

// Enqueue the decode (and, when num_parts > 1, the merge) on `stream`.
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

}  // namespace pa
