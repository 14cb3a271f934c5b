// C ABI of libpagedattn.so (declared in include/paged_attention.h): argument
// validation, the shape-only split-KV planner, the per-device split-KV
// scratch, and the launch.
//
// Every check runs on the host before any HIP call, so a rejected call touches
// no device and needs no GPU.  Nothing here reads device memory or
// synchronises on the call path (vLLM pull request lishuoshuo-amd/vllm #3,
// Validation: no host synchronisation under torch's sync check; Details > Cut
// and precision: the kernel choice is made on the host from shapes so one
// captured graph uses one kernel).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "paged_attention.h"
#include "pa_cache_write.h"
#include "pa_decode_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

// Planner constants.
#ifndef PA_ITEMS_PER_CU
#define PA_ITEMS_PER_CU 2
#endif
#ifndef PA_SPLIT_ITEMS_PER_CU
#define PA_SPLIT_ITEMS_PER_CU 4
#endif
#ifndef PA_CACHED_LOAD_MAX_MIB
#define PA_CACHED_LOAD_MAX_MIB 320
#endif
#ifndef PA_TR_MAX_KV_GROUP
#define PA_TR_MAX_KV_GROUP 8
#endif
constexpr int kTokenRowMaxKvGroup = PA_TR_MAX_KV_GROUP;  // kv heads walking a sequence together
constexpr int kItemsPerCU = PA_ITEMS_PER_CU;  // from this many items per CU, no split
constexpr int kSplitItemsPerCU = PA_SPLIT_ITEMS_PER_CU;  // what a split aims for, per CU
// Token-row caches have no two-waves-per-item kernel, and a wave of theirs
// streams less than a page-layout wave: they split into at least the
// partitions the rule below gives, and further up to eight items per CU, with
// at most kTokenRowMaxParts partitions.  Measured on MI355X (NHD layout, graph
// replay, against the page layout's plan): 40/8 ctx 4096 x 64 sequences
// 169 -> 89 us (four partitions), x 128 178 -> 169 us (two), 32/8 ctx 4096 x
// 24 55.9 -> 45.8 us (eight), ctx 1024 x 24 19.1 -> 17.1 us (eight), 40/8 ctx
// 32768 x 4 52.0 -> 48.8 us (64); the packed layout, 64 sequences 168.5 ->
// 87.6 us.  256 partitions of one sequence lost (1 x 32768: 20.3 -> 21.5 us
// against 128), hence the cap.
constexpr int kTokenRowItemsPerCU = 8;
constexpr int kThreeTileUnitsPerCU = 8;  // (sequence, kv head) units for three query tiles an item
constexpr int kTokenRowMaxParts = 64;
// K/V working sets up to this size (about the 256 MB Infinity Cache and a
// little more) are read with the default cache policy, which lets repeated
// calls find the pages in that cache; larger ones stream past it (nt).
constexpr size_t kCachedLoadMaxBytes = (size_t)PA_CACHED_LOAD_MAX_MIB << 20;
constexpr int kDefaultCUs = 256;      // MI355X
constexpr int kMinPagesPerPart = 8;   // shorter partitions cost more in start-up and merge than they gain
constexpr int kMinPagesPerPartFewItems = 4;  // ... unless the items are at most one per CU
constexpr int kStagePages = 4;        // partitions are whole stages of every decode kernel (2 or 4 blocks)

struct Plan {
  int32_t num_parts;
  int32_t pages_per_part;
  bool longest_first;   // dispatch sequences longest first (order computed on the device)
  size_t order_offset;  // bytes into the scratch where that order lives
  size_t workspace_bytes;
};

// The front of the split-KV scratch holds the fused merge's arrival counters
// (one int per (sequence, kv head), up to kCounterSlots of them): zeroed when
// the scratch is allocated and left at zero by every call; partials and the
// longest-first order follow it, so no call writes over the counters.
constexpr size_t kCounterRegion = 4096;
constexpr int64_t kCounterSlots = kCounterRegion / sizeof(int32_t);

// Longest-first dispatch (an option): with ragged contexts, work items run
// about as long as their sequences, and items dispatched last set the end of
// the call.  A small kernel orders the sequences by length on the device (no
// host read) and the decode kernel takes its items in that order.  Measured on
// MI355X, 256 sequences of 1..4000 tokens at 40/8 heads: 202 -> 185 us with
// the order computed inside the work items (the order kernel instead: 188 us,
// its extra launch costing about 4.6 us); a loss of about 3 us when the
// contexts are all alike.
constexpr int kLongestFirstMaxSeqs = 8192;  // what the one-workgroup order kernel holds
constexpr int kInKernelOrderMaxSeqs = 512;  // what a work item orders by itself (8 per lane)
// Longest-first launches of up to this many items per CU run two waves per
// item (one per SIMD), so only two items a CU are resident and the rest start
// as those finish, longest first: greedy longest-first scheduling.  Measured
// on MI355X (graph replay, ragged 1..4000 x 256 sequences): 32/4 heads (4
// items per CU) 110.5 -> 96.1 us and 106.8 -> 89.9 us (seeds 0, 1); at 8
// items per CU (32/8, 40/8) within +-3%, so the rule stops at 4.  On uniform
// contexts it costs 1-8% more than longest-first alone.
constexpr int kLptTwoWaveItemsPerCU = 4;
// Longest-first without being asked, computed in the work items (no
// scratch): batches of at most kAutoLptMaxSeqs sequences with tables of at
// least kAutoLptMinBlocks blocks and at least eight (sequence, kv head) units
// per CU (where the plan is the same either way).  The items read their plain
// sequence's data while the order is made and keep it where every length
// falls in one bin, so a batch of equal lengths pays little.  Measured on
// MI355X (graph replay, plain -> this): ragged 1..4000 x 256 at 40/8 202.9 ->
// 184.5 us, 32/8 198.7 -> 181.1 us, the mixed batch 257.9 -> 233.2 us, at
// most 8 queries 230.9 -> 213.7 us; uniform 40/8 ctx 4096 x 256 329.8 ->
// 330.8 us, 32/8 324.7 -> 325.4 us, 3 queries 334.9 -> 336.3 us.  Outside
// these bounds the order cost more (ctx 1024 x 256 85.2 -> 87.0 us without
// the shortcut).  Results are bit-identical either way from 8 units per CU;
// at 4 (up to kLptTwoWaveItemsPerCU) the items run as two waves, whose sums
// agree with the plain order to rounding: ragged 1..4000 x 256 at 32/4 103.0
// -> 94.8, 99.3 -> 86.7, 102.8 -> 93.3 us (seeds 0-2), but equal lengths
// 1.7-3% slower (32/4 x 256 x 4096 168.2 -> 173.2 us, 40/8 x 128 x 4096
// 169.1 -> 172.0 us, 20/4 x 256 x 4096 169.6 -> 174.2 us); serving batches
// are ragged.
constexpr int kAutoLptUnitsPerCU = 4;
constexpr int kAutoLptMaxSeqs = 256;
constexpr int kAutoLptMinBlocks = 192;
#ifndef PA_LPT_IN_KERNEL
#define PA_LPT_IN_KERNEL 1
#endif

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape-only plan (no device data: it must not depend on seq_lens).  One
// partition per (sequence, kv head) when that already gives every CU two work
// items: every extra partition costs a start-up and a merge.  Fewer units:
// split each sequence's blocks into the largest power of two of partitions
// that keeps the items within four per CU.  Measured on MI355X (graph replay,
// 16..64 sequences at ctx 1024..4096 and 1..4 at 4096..32768): a CU streams
// at most ~25 GB/s, so every CU needs work, and items that divide evenly over
// the CUs with even partitions beat the same bytes in uneven pieces by 10-25%.
// Partitions hold at least kMinPagesPerPart blocks (kMinPagesPerPartFewItems
// where that leaves at most one item per CU), whole pipeline stages, and never
// more than pa::kMaxPagesPerPart blocks.
int make_plan(int32_t S, int32_t Hq, int32_t Hkv, int32_t W, int32_t num_cus, int32_t ppp_req,
              Plan* plan, int32_t q_tiles = 1, int64_t q_rows = -1, bool longest_first = false,
              bool token_rows = false, bool lpt_requested = false) {
  if (S < 0 || Hq <= 0 || Hkv <= 0 || W < 0 || ppp_req < 0)
    return fail(PA_ERR_SHAPE, "plan: negative or zero size (S=%d Hq=%d Hkv=%d W=%d ppp=%d)", S, Hq,
                Hkv, W, ppp_req);
  const int64_t Wc = W > 0 ? W : 1;
  int64_t ppp;
  if (ppp_req > 0) {
    ppp = ppp_req < Wc ? ppp_req : Wc;
  } else {
    const int64_t items = (int64_t)(S > 0 ? S : 1) * Hkv * (q_tiles > 0 ? q_tiles : 1);
    const int64_t cus = num_cus > 0 ? num_cus : kDefaultCUs;
    // a power of two of partitions, so that (table widths being powers of
    // two in practice) partitions are even and items divide over the CUs
    int64_t parts = 1;
    // exactly kItemsPerCU items per CU split in two as well (measured on
    // MI355X, 512 items, graph replay, two partitions merged in the decode
    // against two waves per item: 40/8 ctx 4096 x 64 sequences 91.0 -> 84.3
    // us, 32/8 x 64 92.5 -> 86.1 us, 20/4 x 128 93.8 -> 86.6 us, 32/4 x 128
    // 90.6 -> 84.8 us; ctx 1024 and 2048 within 1%; per-slot scales, which
    // have no two-waves form, 142.3 -> 91.0 us); longest-first dispatch keeps
    // them whole for its two waves per item
    if (items < cus * kItemsPerCU || (items == cus * kItemsPerCU && !lpt_requested))
      while (parts * 2 * items <= cus * kSplitItemsPerCU) parts *= 2;
    if (token_rows) {
      int64_t tr_parts = 1;
      while (tr_parts * 2 * items <= cus * kTokenRowItemsPerCU && tr_parts * 2 <= kTokenRowMaxParts)
        tr_parts *= 2;
      if (tr_parts > parts) parts = tr_parts;
    }
    if (parts > Wc) parts = Wc;
    ppp = ceil_div(Wc, parts < 1 ? 1 : parts);
    if (ppp < Wc) {
      if (ppp < kMinPagesPerPart) {
        ppp = kMinPagesPerPart;
        // where partitions of the minimum leave at most one item per CU,
        // halving them pays (two items per CU): measured on MI355X, one
        // sequence x 4096 at 40/8 heads 9.1 -> 8.4 us, 8/1 x 16 sequences x
        // 2048 9.1 -> 8.4 us; with more items it measured slower (4 sequences
        // x 4096: 11.7 -> 13.3 us)
        if (items * ceil_div(Wc, ppp) <= cus) ppp = kMinPagesPerPartFewItems;
      }
      ppp = ceil_div(ppp, kStagePages) * kStagePages;
      if (ppp > Wc) ppp = Wc;
    }
  }
  if (ppp > pa::kMaxPagesPerPart) ppp = pa::kMaxPagesPerPart;
  const int64_t parts = ceil_div(Wc, ppp);
  plan->num_parts = (int32_t)parts;
  plan->pages_per_part = (int32_t)ppp;
  const int64_t rows = q_rows >= 0 ? q_rows : S;
  const size_t partial_bytes =
      parts > 1 ? (size_t)rows * Hq * parts * (pa::kHeadDim + 2) * sizeof(float) : 0;
  plan->longest_first = longest_first && S >= 2 && S <= kLongestFirstMaxSeqs;
  plan->order_offset = kCounterRegion + ((partial_bytes + 255) & ~size_t(255));
  plan->workspace_bytes = plan->longest_first ? plan->order_offset + (size_t)S * sizeof(int32_t)
                          : partial_bytes     ? kCounterRegion + partial_bytes
                                              : 0;
  return PA_OK;
}

// Split-KV scratch: one buffer per (device, stream), so calls on different
// streams never share partials or arrival counters, while calls on one stream
// run in order.  A buffer that is outgrown is never freed: graphs captured
// earlier hold its address and keep using it on replay, so it stays allocated
// (and its counters at zero) until the process ends.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;
std::vector<void*> g_retired;  // outgrown buffers, still referenced by captured graphs
std::vector<int> g_cus;

int device_cus(int dev) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if ((int)g_cus.size() <= dev) g_cus.resize(dev + 1, 0);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = kDefaultCUs;
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

// The scratch of (dev, stream), grown to at least `bytes` (outside capture
// only: a capturing stream whose scratch is too small gets PA_ERR_WORKSPACE).
int ensure_workspace(int dev, hipStream_t stream, size_t bytes, void** out) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& ws = g_ws[std::make_pair(dev, (uintptr_t)stream)];
  if (ws.bytes >= bytes) {
    *out = ws.ptr;
    return PA_OK;
  }
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (stream != nullptr && hipStreamIsCapturing(stream, &st) != hipSuccess)
    return fail(PA_ERR_HIP, "hipStreamIsCapturing failed");
  if (st != hipStreamCaptureStatusNone)
    return fail(PA_ERR_WORKSPACE,
                "split-KV scratch of this stream needs %zu bytes but %zu are reserved and the stream "
                "is capturing; call pa_workspace_reserve for this stream before capture",
                bytes, ws.bytes);
  const size_t grow = (bytes + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);
  void* p = nullptr;
  if (hipMalloc(&p, grow) != hipSuccess) return fail(PA_ERR_HIP, "hipMalloc(%zu) for scratch failed", grow);
  // the arrival counters start at zero: cleared and waited for here, before
  // any call can use the buffer (never while `stream` captures)
  if (hipMemsetAsync(p, 0, kCounterRegion, stream) != hipSuccess || hipStreamSynchronize(stream) != hipSuccess) {
    (void)hipFree(p);
    return fail(PA_ERR_HIP, "clearing the scratch's counters failed");
  }
  if (ws.ptr) g_retired.push_back(ws.ptr);
  ws.ptr = p;
  ws.bytes = grow;
  *out = p;
  return PA_OK;
}

}  // namespace

// Split-KV scratch of the allocation-free entry point: a fixed array in the
// library's device memory (each GPU holds its own copy until the process
// ends).  In host code `scratch` only stands for the symbol: its device
// address on each GPU comes from hipGetSymbolAddress, kept per device below.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

std::vector<void*> g_fixed_scratch;  // per device: the address of `scratch` there

__global__ void clear_words_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// The device address of `scratch` on `dev` (the current device), looked up
// once per device.  That first time, the arrival counters at its front are
// cleared by a small kernel enqueued on `stream` (stream-ordered before the
// caller's decode; under capture it becomes part of the graph, where
// clearing counters that every call leaves at zero anyway is harmless).
int fixed_scratch(int dev, hipStream_t stream, void** out) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if ((int)g_fixed_scratch.size() <= dev) g_fixed_scratch.resize(dev + 1, nullptr);
  if (!g_fixed_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, "hipGetSymbolAddress of the fixed scratch failed: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, stream, (uint32_t*)p,
                       (int)(kCounterRegion / sizeof(uint32_t)));
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess) return fail(PA_ERR_HIP, "clearing the fixed scratch failed: %s", hipGetErrorString(le));
    g_fixed_scratch[dev] = p;
  }
  *out = g_fixed_scratch[dev];
  return PA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

// What a call reads beyond the plain decode's arguments.
struct Variant {
  bool slot_scales = false;                // k_scale / v_scale are [NB][Hkv][16] tables
  const int32_t* cu_seqlens_q = nullptr;   // several queries per sequence
  int32_t num_q_rows = 0;
  int32_t max_seqlen_q = 1;
  bool token_rows = false;                 // token-row cache layout with byte strides
  // cache addressing in bytes; page layout: 0 = dense (Hkv * 2048 per block, 2048 per kv head)
  int64_t block_stride = 0, token_stride = 0, head_stride = 0;
  // elements between rows of q and of the block table (0 = dense)
  int64_t q_row_stride = 0, bt_row_stride = 0;
  pa_attention_options options = {0, 0.0f, nullptr, nullptr, 0};
};

// The launch a call makes, from shapes alone.
struct CallPlan {
  Plan plan;
  int32_t q_tile;          // query tokens per tile (columns = q_tile * group <= 16)
  int32_t q_tiles;         // query tiles per sequence
  int32_t tiles_per_item;  // tiles one work item holds (1 to 3)
  int32_t q_items;         // work items per (sequence, kv head, partition)
  bool lpt_in_kernel;      // longest-first order computed inside the work items
};

int plan_call(int32_t S, int32_t Hq, int32_t Hkv, int32_t W, int32_t cus, int32_t ppp_req, bool mq,
              int32_t num_q_rows, int32_t max_seqlen_q, bool longest_first, bool token_rows,
              bool no_default_order, CallPlan* cp) {
  const int32_t G = Hq / Hkv;
  // query tokens per work item: as many as the 16 MFMA columns hold with the group
  cp->q_tile = mq ? (pa::kMaxGroup / G > 0 ? pa::kMaxGroup / G : 1) : 1;
  cp->q_tiles = mq ? (max_seqlen_q + cp->q_tile - 1) / cp->q_tile : 1;
  // query tiles per work item: up to three (one wave holds their accumulators
  // against the same K/V).  Three, at one page a stage, only where they make
  // one item of a sequence's three tiles and the (sequence, kv head) units
  // alone keep two waves per SIMD; otherwise items of two tiles, which for a
  // three-tile sequence means two items reading its pages.  Measured on
  // MI355X (graph replay, 40/8 heads, two -> three tiles an item; ragged
  // contexts 1..4000): 256 sequences with 8 queries in 40% of them (the rest
  // one) 323 -> 258 us, in 10% 315 -> 250 us, in all 334 -> 271 us, 256 x
  // 4096 all 8 505 -> 384 us, 64/4 heads x 512 sequences (3 queries in 40%)
  // 327 -> 271 us; but 128 ragged sequences (8 queries in 40%) 177 -> 194 us
  // and 64 x 4096 all 8 139 -> 186 us.  Six tiles (16 queries at G = 5): two
  // tiles an item win (256 ragged sequences, 16 queries in 40%: 325 us against
  // 432 us at three; 256 x 4096 all 16: 692 against 742 us); five likewise
  // (14 queries: 415 against 493 us).
  const int64_t ncus = cus > 0 ? cus : kDefaultCUs;
  const bool three = cp->q_tiles == 3 && (int64_t)(S > 0 ? S : 1) * Hkv >= kThreeTileUnitsPerCU * ncus;
  cp->tiles_per_item = cp->q_tiles <= 2 ? cp->q_tiles : (three ? 3 : 2);
  cp->q_items = (cp->q_tiles + cp->tiles_per_item - 1) / cp->tiles_per_item;
  // longest-first: computed by each work item where its workgroup is one wave
  // and the sequences few enough, else by the order kernel; by default on
  // large batches of long tables (kAutoLptUnitsPerCU), unless the caller
  // asks for the plain order or a sliding window bounds every item's pages
  // (the order ranks whole lengths; 40/8 x 256 x 4096, window 1024: 84.7 ->
  // 86.1 us with it)
  const bool auto_lpt = PA_LPT_IN_KERNEL && !token_rows && !no_default_order && S >= 2 && S <= kAutoLptMaxSeqs &&
                        W >= kAutoLptMinBlocks && (int64_t)S * Hkv >= kAutoLptUnitsPerCU * ncus;
  cp->lpt_in_kernel = PA_LPT_IN_KERNEL && (longest_first || auto_lpt) && !token_rows && S >= 2 &&
                      S <= kInKernelOrderMaxSeqs;
  return make_plan(S, Hq, Hkv, W, cus, ppp_req, &cp->plan, cp->q_items, mq ? num_q_rows : S,
                   longest_first && !cp->lpt_in_kernel, token_rows && !mq, longest_first);
}

int decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
           const int32_t* seq_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t head_size,
           int32_t block_size, int32_t W, int64_t NB, float scale, const float* k_scale,
           const float* v_scale, void* out, void* stream_ptr, int32_t ppp_req,
           const Variant& var = Variant(), bool use_fixed_scratch = false) {
  const bool slot_scales = var.slot_scales;
  const int32_t* cu_seqlens_q = var.cu_seqlens_q;
  const int32_t num_q_rows = var.num_q_rows;
  const int32_t max_seqlen_q = var.max_seqlen_q;
  g_last_error[0] = '\0';
  if (head_size != pa::kHeadDim)
    return fail(PA_ERR_UNSUPPORTED, "head_size %d unsupported (only %d)", head_size, pa::kHeadDim);
  if (block_size != pa::kBlockTokens)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d unsupported (only %d)", block_size,
                pa::kBlockTokens);
  if (S < 0 || Hq <= 0 || Hkv <= 0 || W < 0 || NB < 0 || ppp_req < 0)
    return fail(PA_ERR_SHAPE,
                "negative or zero size: num_seqs=%d num_heads=%d num_kv_heads=%d "
                "max_blocks_per_seq=%d num_blocks=%lld pages_per_partition=%d",
                S, Hq, Hkv, W, (long long)NB, ppp_req);
  if (Hq % Hkv != 0)
    return fail(PA_ERR_SHAPE, "num_heads %d is not a multiple of num_kv_heads %d", Hq, Hkv);
  const int32_t G = Hq / Hkv;
  if (G > pa::kMaxGroup)
    return fail(PA_ERR_UNSUPPORTED, "group size %d exceeds %d query heads per kv head", G,
                pa::kMaxGroup);
  if (!isfinite(scale)) return fail(PA_ERR_SHAPE, "scale is not finite");
  const pa_attention_options& opt = var.options;
  // the several-queries kernel serves several queries and every logit option
  const bool any_option = opt.sliding_window != 0 || opt.logits_soft_cap != 0.0f ||
                          opt.alibi_slopes != nullptr || opt.sinks != nullptr;
  const bool mq = cu_seqlens_q != nullptr || any_option;
  if (mq && (num_q_rows < 0 || max_seqlen_q < 0))
    return fail(PA_ERR_SHAPE, "negative num_q_tokens or max_seqlen_q");
  if (S == 0 || (mq && num_q_rows == 0)) return PA_OK;
  if (mq && max_seqlen_q == 0)
    return fail(PA_ERR_SHAPE, "max_seqlen_q must be positive when there are query tokens");
  if (opt.sliding_window < 0)
    return fail(PA_ERR_SHAPE, "sliding_window %d is negative", opt.sliding_window);
  if (!(opt.logits_soft_cap >= 0.0f) || !isfinite(opt.logits_soft_cap))
    return fail(PA_ERR_SHAPE, "logits_soft_cap must be finite and >= 0");
  if (((uintptr_t)opt.alibi_slopes & 3) || ((uintptr_t)opt.sinks & 3))
    return fail(PA_ERR_SHAPE, "misaligned alibi_slopes / sinks (4 B)");
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !k_scale || !v_scale || !out)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  if (W == 0 || NB == 0)
    return fail(PA_ERR_SHAPE, "max_blocks_per_seq and num_blocks must be positive when num_seqs > 0");

  const int64_t rows = mq ? num_q_rows : S;
  const int64_t row_elems = (int64_t)Hq * pa::kHeadDim;
  const int64_t qrs = var.q_row_stride ? var.q_row_stride : row_elems;
  const int64_t btrs = var.bt_row_stride ? var.bt_row_stride : W;
  if (qrs < row_elems || (qrs & 7))
    return fail(PA_ERR_LAYOUT, "q row stride %lld must be a multiple of 8 elements and at least %lld",
                (long long)qrs, (long long)row_elems);
  if (btrs < W)
    return fail(PA_ERR_LAYOUT, "block-table row stride %lld is below max_blocks_per_seq %d",
                (long long)btrs, W);
  const size_t out_bytes = (size_t)rows * row_elems * 2;
  const size_t q_bytes = ((size_t)(rows - 1) * qrs + row_elems) * 2;
  int64_t bstride = var.block_stride, hstride = var.head_stride;
  size_t cache_bytes;
  if (var.token_rows) {
    const int64_t bs = var.block_stride, ts = var.token_stride, hs = var.head_stride;
    if (bs <= 0 || ts <= 0 || hs <= 0 || (bs | ts | hs) & 15)
      return fail(PA_ERR_SHAPE, "token-row strides must be positive multiples of 16 bytes "
                                "(block %lld, token %lld, head %lld)",
                  (long long)bs, (long long)ts, (long long)hs);
    if (ts > (int64_t(1) << 26))
      return fail(PA_ERR_UNSUPPORTED, "token stride %lld exceeds 2^26 bytes", (long long)ts);
    // bytes from the cache base to the end of the last block's last row
    cache_bytes = (size_t)((NB - 1) * bs + (pa::kBlockTokens - 1) * ts + (Hkv - 1) * hs + pa::kHeadDim);
  } else {
    if (bstride == 0 && hstride == 0) {
      bstride = (int64_t)Hkv * pa::kPageBytes;
      hstride = pa::kPageBytes;
    }
    if (bstride <= 0 || hstride <= 0 || (bstride | hstride) & 15)
      return fail(PA_ERR_LAYOUT, "cache block / kv-head strides must be positive multiples of 16 bytes "
                                 "(block %lld, head %lld)", (long long)bstride, (long long)hstride);
    if (slot_scales && (bstride != (int64_t)Hkv * pa::kPageBytes || hstride != pa::kPageBytes))
      return fail(PA_ERR_LAYOUT, "per-slot scales need dense caches");
    cache_bytes = (size_t)((NB - 1) * bstride + (Hkv - 1) * hstride + pa::kPageBytes);
  }
  if (overlaps(out, out_bytes, q, q_bytes) || overlaps(out, out_bytes, k_cache, cache_bytes) ||
      overlaps(out, out_bytes, v_cache, cache_bytes) ||
      overlaps(out, out_bytes, block_tables, ((size_t)(S - 1) * btrs + W) * 4) ||
      overlaps(out, out_bytes, seq_lens, (size_t)S * 4) || overlaps(out, out_bytes, k_scale, 4) ||
      (mq && overlaps(out, out_bytes, cu_seqlens_q, (size_t)(S + 1) * 4)) ||
      overlaps(out, out_bytes, opt.alibi_slopes, opt.alibi_slopes ? (size_t)Hq * 4 : 0) ||
      overlaps(out, out_bytes, opt.sinks, opt.sinks ? (size_t)Hq * 4 : 0) ||
      overlaps(out, out_bytes, v_scale, 4))
    return fail(PA_ERR_ALIAS, "out overlaps an input");
  if (slot_scales && (overlaps(out, out_bytes, k_scale, (size_t)NB * Hkv * 64) ||
                      overlaps(out, out_bytes, v_scale, (size_t)NB * Hkv * 64)))
    return fail(PA_ERR_ALIAS, "out overlaps a scale table");
  if (var.token_rows && ((uintptr_t)v_cache & 15))
    return fail(PA_ERR_SHAPE, "misaligned v_cache (token rows: 16 B)");
  if (((uintptr_t)q & 15) || ((uintptr_t)k_cache & 15) || ((uintptr_t)v_cache & 3) ||
      ((uintptr_t)out & 7) || ((uintptr_t)block_tables & 3) || ((uintptr_t)seq_lens & 3))
    return fail(PA_ERR_SHAPE, "misaligned pointer (q, k_cache: 16 B; out: 8 B; others: 4 B)");
  if (slot_scales && (((uintptr_t)k_scale & 15) || ((uintptr_t)v_scale & 15)))
    return fail(PA_ERR_SHAPE, "scale tables must be 16-byte aligned");

  // --- past this point HIP is called
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  CallPlan cp;
  int rc = plan_call(S, Hq, Hkv, W, device_cus(dev), ppp_req, mq, num_q_rows, max_seqlen_q,
                     opt.longest_first > 0, var.token_rows, opt.sliding_window > 0 || opt.longest_first < 0,
                     &cp);
  if (rc) return rc;
  const Plan& plan = cp.plan;
  // one 64-lane block per work item, 256 lanes per merged row: keep both grids
  // within 2^32 lanes
  const int64_t units = (int64_t)S * Hkv * plan.num_parts;
  const int64_t items = mq ? (units + 7) / 8 * 8 * cp.q_items : units;
  const int64_t merge_rows = rows * Hq;
  if (items > (int64_t(1) << 26) || merge_rows > (int64_t(1) << 24))
    return fail(PA_ERR_UNSUPPORTED, "launch too large: %lld work items, %lld merged rows",
                (long long)items, (long long)merge_rows);
  hipStream_t stream = (hipStream_t)stream_ptr;

  pa::DecodeParams p;
  p.q = (const uint16_t*)q;
  p.k_cache = (const uint8_t*)k_cache;
  p.v_cache = (const uint8_t*)v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.q_row_stride = qrs;
  p.bt_row_stride = btrs;
  p.k_scale = slot_scales ? nullptr : k_scale;
  p.v_scale = slot_scales ? nullptr : v_scale;
  p.k_slot_scales = slot_scales ? k_scale : nullptr;
  p.v_slot_scales = slot_scales ? v_scale : nullptr;
  p.out = (uint16_t*)out;
  p.part_acc = nullptr;
  p.part_ml = nullptr;
  p.num_seqs = S;
  p.num_heads = Hq;
  p.num_kv_heads = Hkv;
  p.group = G;
  p.max_blocks = W;
  p.num_blocks_u32 = (uint32_t)(NB < INT32_MAX ? NB : INT32_MAX);
  p.num_parts = plan.num_parts;
  p.pages_per_part = plan.pages_per_part;
  p.scale_log2e = (float)((double)scale * 1.4426950408889634);
  // the plain decode reads a working set that fits the Infinity Cache with the
  // default policy (K and V of every table entry: an upper bound)
  p.cached_loads = (!mq && !slot_scales && !var.token_rows &&
                    (size_t)S * W * Hkv * 2 * pa::kPageBytes <= kCachedLoadMaxBytes)
                       ? 1 : 0;
  p.multi_query = mq ? 1 : 0;
  p.cu_seqlens_q = cu_seqlens_q;
  p.num_q_rows = (int32_t)rows;
  p.q_tile = cp.q_tile;
  p.num_q_tiles = cp.q_tiles;
  // more than one tile of queries: two tiles per item share the page reads
  p.tiles_per_item = cp.tiles_per_item;
  p.window = opt.sliding_window;
  p.softcap = opt.logits_soft_cap;
  p.scale = scale;
  p.alibi_slopes = opt.alibi_slopes;
  p.sinks = opt.sinks;
  p.token_rows = var.token_rows ? 1 : 0;
  // token rows: where the kv heads' rows interleave within a token's row
  // (head stride below token stride, as in [blocks, 16, kv_heads, 128]), the
  // largest divisor of Hkv up to 8 kv heads share a workgroup and read each
  // block together, as long as the launch keeps a workgroup per CU (measured on
  // MI355X, 40/8 NHD ctx 4096 x 16 sequences, 8 partitions: 8 kv heads a
  // workgroup 40.3 us, 4 30.0 us); a layout that keeps a (block, kv head)
  // together gains nothing from it
  p.kv_group = 1;
  if (var.token_rows && var.head_stride < var.token_stride) {
    const int64_t tr_items = (int64_t)S * Hkv * plan.num_parts;
    for (int g = kTokenRowMaxKvGroup; g >= 1; --g)
      if (Hkv % g == 0 && (g == 1 || tr_items / g >= device_cus(dev))) {
        p.kv_group = g;
        break;
      }
  }
  p.block_stride = bstride;
  p.token_stride = var.token_stride;
  p.head_stride = hstride;
  p.seq_order = nullptr;
  p.order_in_kernel = cp.lpt_in_kernel ? 1 : 0;
  // longest-first, one query per sequence, one wave per workgroup: slots in
  // snake order over rounds of one work item per CU (measured on MI355X,
  // ragged 1..4000 batches of 256 sequences: 40/8 181 -> 176 us, 32/8
  // 186 -> 180 us, 32/4 111 -> 105 us; 8/1 and uniform contexts unchanged)
  const int64_t items_per_slot = (int64_t)Hkv * plan.num_parts;
  p.lpt_round_slots = (!mq && !var.token_rows && (cp.lpt_in_kernel || plan.longest_first))
                          ? (int32_t)std::max<int64_t>(1, device_cus(dev) / items_per_slot)
                          : 0;
  // the last item of a split (sequence, kv head) merges its partitions where
  // they are few (one query per sequence): no merge kernel and no kernel
  // boundary before it
  p.fused_merge = (!mq && plan.num_parts > 1 && plan.num_parts <= pa::kFusedMergeMaxParts &&
                   (int64_t)G * plan.num_parts <= pa::kFusedMergeMaxLoads && (int64_t)S * Hkv <= kCounterSlots)
                      ? 1 : 0;
  p.unit_count = nullptr;
  // two waves per work item where one partition leaves more than one and at
  // most kLptTwoWaveItemsPerCU items per CU under longest-first dispatch
  // (without it such launches split into two partitions instead: see the
  // plan).  Measured on MI355X, 512 items, against one wave per item: 40/8
  // ctx 4096 x 64 sequences 95.7 -> 88.3 us, 20/4 ctx 4096 x 128 96.0 -> 87.8
  // us (two partitions: 84.3 and 86.6 us); with split contexts two waves
  // measured 3-10% slower
  const int64_t cus = device_cus(dev);
  const bool lpt_on = cp.lpt_in_kernel || plan.longest_first;
  p.waves_per_item = (!mq && !slot_scales && !var.token_rows && plan.num_parts == 1 && units > cus &&
                      units <= (lpt_on ? kLptTwoWaveItemsPerCU : 2) * cus)
                         ? 2 : 1;
  if (plan.workspace_bytes) {
    void* ws = nullptr;
    if (use_fixed_scratch) {
      // the fixed array of the allocation-free entry point: never grown
      if (plan.workspace_bytes > (size_t)PA_NOALLOC_SCRATCH_BYTES)
        return fail(PA_ERR_WORKSPACE,
                    "this plan needs %zu bytes of split-KV scratch; the fixed array holds %zu",
                    plan.workspace_bytes, (size_t)PA_NOALLOC_SCRATCH_BYTES);
      rc = fixed_scratch(dev, stream, &ws);
      if (rc) return rc;
    } else {
      rc = ensure_workspace(dev, stream, plan.workspace_bytes, &ws);
      if (rc) return rc;
    }
    p.unit_count = (int32_t*)ws;
    if (plan.num_parts > 1) {
      p.part_acc = (float*)((char*)ws + kCounterRegion);
      p.part_ml = p.part_acc + (size_t)p.num_q_rows * Hq * plan.num_parts * pa::kHeadDim;
    }
    if (plan.longest_first) p.seq_order = (int32_t*)((char*)ws + plan.order_offset);
  }
  const hipError_t err = pa::launch_decode(p, stream);
  if (err != hipSuccess) return fail(PA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return PA_OK;
}

// --- tensor descriptors (paged_decode_attention_desc)

bool fp8_bytes(int32_t dt) { return dt == PA_DTYPE_FP8_E4M3FN || dt == PA_DTYPE_UINT8; }

// Stride of dim i, or `want` when the dim has one element (its stride is then
// never used, and frameworks leave it arbitrary).
int64_t stride_or(const pa_tensor* t, int i, int64_t want) {
  return t->sizes[i] == 1 ? want : t->strides[i];
}

bool valid_desc(const pa_tensor* t) {
  if (t->ndim < 0 || t->ndim > PA_MAX_DIMS) return false;
  for (int i = 0; i < t->ndim; ++i)
    if (t->sizes[i] < 0 || t->strides[i] < 0) return false;
  return true;
}

int64_t numel(const pa_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->sizes[i];
  return n;
}

}  // namespace

extern "C" {

int paged_decode_attention_desc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                                const pa_tensor* block_tables, const pa_tensor* seq_lens, float scale,
                                const pa_tensor* k_scale, const pa_tensor* v_scale, const pa_tensor* out,
                                void* stream) {
  g_last_error[0] = '\0';
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !k_scale || !v_scale || !out)
    return fail(PA_ERR_NULL, "a tensor descriptor is NULL");
  for (const pa_tensor* t : {q, k_cache, v_cache, block_tables, seq_lens, k_scale, v_scale, out})
    if (!valid_desc(t))
      return fail(PA_ERR_SHAPE, "a descriptor has ndim outside 0..%d or a negative size or stride",
                  PA_MAX_DIMS);
  // dtypes
  if (q->dtype != PA_DTYPE_BF16 || out->dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "q and out must be bf16 (dtypes %d, %d)", q->dtype, out->dtype);
  if (!fp8_bytes(k_cache->dtype) || !fp8_bytes(v_cache->dtype))
    return fail(PA_ERR_DTYPE, "k_cache and v_cache must be fp8 e4m3fn (or its uint8 bytes)");
  if (block_tables->dtype != PA_DTYPE_INT32 || seq_lens->dtype != PA_DTYPE_INT32)
    return fail(PA_ERR_DTYPE, "block_tables and seq_lens must be int32");
  if (k_scale->dtype != PA_DTYPE_FP32 || v_scale->dtype != PA_DTYPE_FP32)
    return fail(PA_ERR_DTYPE, "k_scale and v_scale must be fp32");
  // ranks and sizes
  if (q->ndim != 3 || out->ndim != 3)
    return fail(PA_ERR_SHAPE, "q and out must be [num_seqs, num_heads, head_size]");
  const int64_t S = q->sizes[0], Hq = q->sizes[1], D = q->sizes[2];
  for (int i = 0; i < 3; ++i)
    if (out->sizes[i] != q->sizes[i]) return fail(PA_ERR_SHAPE, "out must have q's sizes");
  if (D != pa::kHeadDim) return fail(PA_ERR_UNSUPPORTED, "head_size %lld unsupported (only %d)", (long long)D, pa::kHeadDim);
  if (k_cache->ndim != 5)
    return fail(PA_ERR_SHAPE, "k_cache must be [num_blocks, num_kv_heads, head_size/16, block_size, 16]");
  const int64_t NB = k_cache->sizes[0], Hkv = k_cache->sizes[1], BS = k_cache->sizes[3];
  if (BS != pa::kBlockTokens)
    return fail(PA_ERR_UNSUPPORTED, "block_size %lld unsupported (only %d)", (long long)BS, pa::kBlockTokens);
  if (k_cache->sizes[2] * 16 != D || k_cache->sizes[4] != 16)
    return fail(PA_ERR_SHAPE, "k_cache's inner sizes must be [head_size/16, 16, 16]");
  const bool v5 = v_cache->ndim == 5;
  if (!(v_cache->ndim == 4 || (v5 && v_cache->sizes[2] == 1)))
    return fail(PA_ERR_SHAPE, "v_cache must be [num_blocks, num_kv_heads, head_size, block_size] "
                              "or [num_blocks, num_kv_heads, 1, head_size, block_size]");
  const int vd = v5 ? 3 : 2;  // v_cache's head_size dim
  if (v_cache->sizes[0] != NB || v_cache->sizes[1] != Hkv || v_cache->sizes[vd] != D ||
      v_cache->sizes[vd + 1] != BS)
    return fail(PA_ERR_SHAPE, "v_cache's sizes disagree with k_cache");
  if (block_tables->ndim != 2 || block_tables->sizes[0] != S)
    return fail(PA_ERR_SHAPE, "block_tables must be [num_seqs, max_blocks_per_seq]");
  const int64_t W = block_tables->sizes[1];
  if (seq_lens->ndim != 1 || seq_lens->sizes[0] != S) return fail(PA_ERR_SHAPE, "seq_lens must be [num_seqs]");
  if (numel(k_scale) != 1 || numel(v_scale) != 1)
    return fail(PA_ERR_SHAPE, "k_scale and v_scale must hold one element");
  if (S > INT32_MAX || Hq > INT32_MAX || Hkv > INT32_MAX || W > INT32_MAX || Hkv == 0)
    return fail(PA_ERR_SHAPE, "sizes out of range");
  // layouts (strides in elements)
  if (stride_or(q, 2, 1) != 1 || stride_or(q, 1, D) != D)
    return fail(PA_ERR_LAYOUT, "q's rows [num_heads, head_size] must be dense");
  if (stride_or(out, 2, 1) != 1 || stride_or(out, 1, D) != D || stride_or(out, 0, Hq * D) != Hq * D)
    return fail(PA_ERR_LAYOUT, "out must be dense");
  if (stride_or(k_cache, 4, 1) != 1 || stride_or(k_cache, 3, 16) != 16 || stride_or(k_cache, 2, 256) != 256)
    return fail(PA_ERR_LAYOUT, "k_cache's pages [head_size/16, 16, 16] must be dense");
  if (stride_or(v_cache, vd + 1, 1) != 1 || stride_or(v_cache, vd, BS) != BS)
    return fail(PA_ERR_LAYOUT, "v_cache's pages [head_size, block_size] must be dense");
  const int64_t page = D * BS;
  const int64_t kb = stride_or(k_cache, 0, Hkv * page), kh = stride_or(k_cache, 1, page);
  const int64_t vb = stride_or(v_cache, 0, Hkv * page), vh = stride_or(v_cache, 1, page);
  if (kb != vb || kh != vh)
    return fail(PA_ERR_LAYOUT, "k_cache and v_cache must have the same block and kv-head strides");
  if (stride_or(block_tables, 1, 1) != 1)
    return fail(PA_ERR_LAYOUT, "block_tables' rows must be dense");
  if (stride_or(seq_lens, 0, 1) != 1) return fail(PA_ERR_LAYOUT, "seq_lens must be dense");
  Variant var;
  var.block_stride = kb;
  var.head_stride = kh;
  var.q_row_stride = stride_or(q, 0, Hq * D);
  var.bt_row_stride = stride_or(block_tables, 0, W);
  return decode(q->data, k_cache->data, v_cache->data, (const int32_t*)block_tables->data,
                (const int32_t*)seq_lens->data, (int32_t)S, (int32_t)Hq, (int32_t)Hkv, (int32_t)D,
                (int32_t)BS, (int32_t)W, NB, scale, (const float*)k_scale->data,
                (const float*)v_scale->data, out->data, stream, 0, var);
}

int paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                           int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                           float scale, const float* k_scale, const float* v_scale, void* out,
                           void* stream) {
  return decode(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                head_size, block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, out,
                stream, 0);
}

int paged_decode_attention_split(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                                 int64_t num_blocks, float scale, const float* k_scale,
                                 const float* v_scale, void* out, void* stream,
                                 int32_t pages_per_partition) {
  return decode(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                head_size, block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, out,
                stream, pages_per_partition);
}

int paged_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                                   int64_t num_blocks, float scale, const float* k_scale,
                                   const float* v_scale, void* out, void* stream,
                                   int32_t pages_per_partition) {
  return decode(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                head_size, block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, out,
                stream, pages_per_partition, Variant(), true);
}

int paged_multi_query_attention(const void* q, const int32_t* cu_seqlens_q, int32_t num_q_tokens,
                                int32_t max_seqlen_q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                                int64_t num_blocks, float scale, const float* k_scale,
                                const float* v_scale, void* out, void* stream) {
  if (!cu_seqlens_q && num_seqs > 0) return fail(PA_ERR_NULL, "cu_seqlens_q is NULL");
  if (num_seqs > 0 && num_q_tokens > 0 && ((uintptr_t)cu_seqlens_q & 3))
    return fail(PA_ERR_SHAPE, "misaligned cu_seqlens_q (4 B)");
  Variant mq;
  mq.cu_seqlens_q = cu_seqlens_q;
  mq.num_q_rows = num_q_tokens;
  mq.max_seqlen_q = max_seqlen_q;
  return decode(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                head_size, block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, out,
                stream, 0, mq);
}

int paged_attention_unified(const void* q, const int32_t* cu_seqlens_q, int32_t num_q_tokens,
                            int32_t max_seqlen_q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                            float scale, const float* k_scale, const float* v_scale,
                            const pa_attention_options* options, void* out, void* stream) {
  g_last_error[0] = '\0';
  Variant mq;
  if (options) mq.options = *options;
  if (cu_seqlens_q) {
    if (num_seqs > 0 && num_q_tokens > 0 && ((uintptr_t)cu_seqlens_q & 3))
      return fail(PA_ERR_SHAPE, "misaligned cu_seqlens_q (4 B)");
    mq.cu_seqlens_q = cu_seqlens_q;
    mq.num_q_rows = num_q_tokens;
    mq.max_seqlen_q = max_seqlen_q;
  } else {
    // one query per sequence
    if (num_q_tokens != num_seqs)
      return fail(PA_ERR_SHAPE, "without cu_seqlens_q, num_q_tokens (%d) must equal num_seqs (%d)",
                  num_q_tokens, num_seqs);
    mq.num_q_rows = num_seqs;
  }
  return decode(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                head_size, block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, out,
                stream, 0, mq);
}

int paged_decode_attention_slot_scales(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_size, int32_t block_size,
                                       int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                       const float* k_slot_scales, const float* v_slot_scales,
                                       void* out, void* stream) {
  Variant ss;
  ss.slot_scales = true;
  return decode(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                head_size, block_size, max_blocks_per_seq, num_blocks, scale, k_slot_scales,
                v_slot_scales, out, stream, 0, ss);
}

int paged_decode_attention_nhd(const void* q, const void* k_cache, const void* v_cache,
                               int64_t block_stride, int64_t token_stride, int64_t head_stride,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, float scale, const float* k_scale,
                               const float* v_scale, void* out, void* stream) {
  Variant tr;
  tr.token_rows = true;
  tr.block_stride = block_stride;
  tr.token_stride = token_stride;
  tr.head_stride = head_stride;
  return decode(q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_heads, num_kv_heads,
                head_size, block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, out,
                stream, 0, tr);
}

int pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                   int32_t max_blocks_per_seq, int32_t num_compute_units,
                   int32_t pages_per_partition, int32_t* num_partitions, int32_t* pages_per_part,
                   size_t* workspace_bytes) {
  g_last_error[0] = '\0';
  Plan plan;
  const int rc = make_plan(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, num_compute_units,
                           pages_per_partition, &plan);
  if (rc) return rc;
  if (num_partitions) *num_partitions = plan.num_parts;
  if (pages_per_part) *pages_per_part = plan.pages_per_part;
  if (workspace_bytes) *workspace_bytes = plan.workspace_bytes;
  return PA_OK;
}

int pa_workspace_bytes(int32_t num_seqs, int32_t num_q_tokens, int32_t max_seqlen_q,
                       int32_t num_heads, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                       int32_t longest_first, int32_t token_rows, int device, size_t* bytes) {
  g_last_error[0] = '\0';
  if (!bytes) return fail(PA_ERR_NULL, "bytes is NULL");
  *bytes = 0;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0 ||
      num_q_tokens < 0 || max_seqlen_q < 0 || num_heads % num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "bad sizes (num_seqs=%d num_q_tokens=%d max_seqlen_q=%d num_heads=%d "
                              "num_kv_heads=%d max_blocks_per_seq=%d)",
                num_seqs, num_q_tokens, max_seqlen_q, num_heads, num_kv_heads, max_blocks_per_seq);
  if (num_heads / num_kv_heads > pa::kMaxGroup)
    return fail(PA_ERR_UNSUPPORTED, "group size %d exceeds %d", num_heads / num_kv_heads, pa::kMaxGroup);
  const bool mq = num_q_tokens > 0;
  if (num_seqs == 0 || (mq && max_seqlen_q == 0)) return PA_OK;
  int cus = kDefaultCUs;
  if (device >= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0)
      return fail(PA_ERR_HIP, "cannot read the compute-unit count of device %d", device);
    cus = n;
  }
  CallPlan cp;
  const int rc = plan_call(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, cus, 0, mq,
                           mq ? num_q_tokens : num_seqs, mq ? max_seqlen_q : 1, longest_first > 0,
                           token_rows != 0, false, &cp);
  if (rc) return rc;
  *bytes = cp.plan.workspace_bytes;
  return PA_OK;
}

int pa_workspace_reserve(int device, void* stream, size_t bytes) {
  g_last_error[0] = '\0';
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  if (device != cur && hipSetDevice(device) != hipSuccess)
    return fail(PA_ERR_HIP, "hipSetDevice(%d) failed", device);
  void* p = nullptr;
  const int rc = bytes ? ensure_workspace(device, (hipStream_t)stream, bytes, &p) : PA_OK;
  if (device != cur && hipSetDevice(cur) != hipSuccess && rc == PA_OK)
    return fail(PA_ERR_HIP, "hipSetDevice(%d) failed", cur);
  return rc;
}

int paged_kv_cache_write(const void* key, const void* value, int64_t key_token_stride,
                         int64_t value_token_stride, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size, int64_t num_blocks,
                         const float* k_scale, const float* v_scale, void* stream) {
  g_last_error[0] = '\0';
  if (head_size != pa::kHeadDim)
    return fail(PA_ERR_UNSUPPORTED, "head_size %d unsupported (only %d)", head_size, pa::kHeadDim);
  if (block_size != pa::kBlockTokens)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d unsupported (only %d)", block_size,
                pa::kBlockTokens);
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0)
    return fail(PA_ERR_SHAPE, "negative or zero size: num_tokens=%d num_kv_heads=%d num_blocks=%lld",
                num_tokens, num_kv_heads, (long long)num_blocks);
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping || !k_scale || !v_scale)
    return fail(PA_ERR_NULL, "a required pointer is NULL");
  const int64_t row = (int64_t)num_kv_heads * pa::kHeadDim;
  if (key_token_stride < row || value_token_stride < row || (key_token_stride & 1) ||
      (value_token_stride & 1))
    return fail(PA_ERR_SHAPE,
                "token strides (%lld, %lld) must be even and at least num_kv_heads * 128 = %lld",
                (long long)key_token_stride, (long long)value_token_stride, (long long)row);
  if (num_blocks == 0) return fail(PA_ERR_SHAPE, "num_blocks must be positive");
  // one 64-lane workgroup per (16 tokens, kv head): keep the grid within 2^32 lanes
  const int64_t cw_items = ((int64_t)num_tokens + pa::kBlockTokens - 1) / pa::kBlockTokens * num_kv_heads;
  if (cw_items > (int64_t(1) << 26))
    return fail(PA_ERR_UNSUPPORTED, "launch too large: %lld work items (16 tokens x kv head; at most 2^26)",
                (long long)cw_items);
  if (((uintptr_t)key & 3) || ((uintptr_t)value & 3) || ((uintptr_t)k_cache & 1) ||
      ((uintptr_t)slot_mapping & 7))
    return fail(PA_ERR_SHAPE, "misaligned pointer (key, value: 4 B; k_cache: 2 B; slot_mapping: 8 B)");
  const size_t cache_bytes = (size_t)num_blocks * num_kv_heads * pa::kPageBytes;
  const size_t key_bytes = ((size_t)(num_tokens - 1) * key_token_stride + row) * 2;
  const size_t value_bytes = ((size_t)(num_tokens - 1) * value_token_stride + row) * 2;
  if (overlaps(k_cache, cache_bytes, v_cache, cache_bytes))
    return fail(PA_ERR_ALIAS, "k_cache and v_cache overlap");
  for (const void* c : {(const void*)k_cache, (const void*)v_cache})
    if (overlaps(c, cache_bytes, key, key_bytes) || overlaps(c, cache_bytes, value, value_bytes) ||
        overlaps(c, cache_bytes, slot_mapping, (size_t)num_tokens * 8) ||
        overlaps(c, cache_bytes, k_scale, 4) || overlaps(c, cache_bytes, v_scale, 4))
      return fail(PA_ERR_ALIAS, "a cache overlaps an input");

  pa::CacheWriteParams p;
  p.key = (const uint16_t*)key;
  p.value = (const uint16_t*)value;
  p.key_stride = key_token_stride;
  p.value_stride = value_token_stride;
  p.k_cache = (uint8_t*)k_cache;
  p.v_cache = (uint8_t*)v_cache;
  p.slot_mapping = slot_mapping;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.num_tokens = num_tokens;
  p.num_kv_heads = num_kv_heads;
  p.num_blocks = num_blocks;
  p.vec16 = !((uintptr_t)key & 15) && !((uintptr_t)value & 15) && !(key_token_stride & 7) &&
            !(value_token_stride & 7) && !((uintptr_t)k_cache & 15) && !((uintptr_t)v_cache & 15);
  const hipError_t err = pa::launch_cache_write(p, (hipStream_t)stream);
  if (err != hipSuccess) return fail(PA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return PA_OK;
}

const char* pa_last_error(void) { return g_last_error; }

}  // extern "C"
