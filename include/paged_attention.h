/*
 * paged_attention.h -- C ABI of libpagedattn.so: single-token (decode) attention
 * over a paged fp8-e4m3fn KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The operation (vLLM pull request lishuoshuo-amd/vllm #3, Overview and
 * Details > Layout; API page vllm.v1.attention.backends.rocm_aiter_unified_attn,
 * RocmAiterUnifiedAttentionImpl.forward):
 *
 *   for every sequence s and query head h, with G = num_heads / num_kv_heads,
 *   kv head k = h / G and n = seq_lens[s]:
 *     token t (0 <= t < n) sits in physical block block_tables[s][t / 16], slot t % 16
 *     K_t = fp8(k_cache[block][k][:, slot, :]) * k_scale     (128 values)
 *     V_t = fp8(v_cache[block][k][:, slot])    * v_scale     (128 values)
 *     out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t) * V_t
 *
 * fp8 is the OCP e4m3fn format (largest finite 448, NaN = 0x7F / 0xFF).
 * Accumulation is fp32; out is rounded to bf16 (nearest even).  A sequence with
 * seq_lens[s] == 0 gets an all-zero output row.
 *
 * Memory: every pointer is device memory of the current HIP device, owned by
 * the caller and not retained after the call returns.  Calls are asynchronous:
 * they validate their arguments on the host, enqueue work on `stream` and
 * return; they never read device memory on the host and never synchronise, so
 * they may be captured into a HIP graph (the pull request's Validation ran
 * its decode under torch's host-sync check, and Details > Cut and precision
 * makes the kernel choice from shapes so that one captured graph keeps one
 * kernel).
 *
 * Split-KV scratch: calls whose plan splits contexts (pa_workspace_bytes > 0)
 * keep partial results and arrival counters in a scratch buffer the library
 * owns, one per (device, stream).  Calls on different streams therefore never
 * share it and may run concurrently; calls on one stream run in order.  The
 * buffer grows with hipMalloc when a call needs more, outside graph capture
 * only (that call also waits for `stream` once while it clears the new
 * buffer's counters); a capturing stream whose scratch is too small gets
 * PA_ERR_WORKSPACE, so reserve it first (pa_workspace_reserve, or one eager
 * call of the same shapes on that stream).  A graph uses the scratch of the
 * stream it was captured on: replaying it concurrently with other work that
 * uses that scratch (eager calls on that stream, other graphs captured there)
 * races.  An outgrown buffer is never freed (graphs captured before the
 * growth still use it); every buffer lives until the process ends.
 *
 * Errors: every check runs before any launch.  A failing call returns a
 * negative pa_status, launches nothing, and leaves a message for
 * pa_last_error() (thread-local).  No exception crosses the ABI; nothing aborts.
 * Conditions that only device memory could reveal are not reported: seq_lens
 * above 16 * max_blocks_per_seq are clamped to that, and a used block id
 * outside [0, num_blocks) reads as an all-zero page (zero K, V and slot
 * scales) without touching memory, so the result is defined but meaningless.
 */
#ifndef PAGED_ATTENTION_H_
#define PAGED_ATTENTION_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                            */
  PA_ERR_SHAPE = -2,       /* a size is negative or sizes disagree                  */
  PA_ERR_UNSUPPORTED = -3, /* head_size != 128, block_size != 16 or group > 16      */
  PA_ERR_ALIAS = -4,       /* out overlaps an input                                 */
  PA_ERR_WORKSPACE = -5,   /* split-KV scratch too small while `stream` captures    */
  PA_ERR_HIP = -6,         /* a HIP runtime call or a kernel launch failed          */
  PA_ERR_DTYPE = -7,       /* a tensor descriptor has the wrong element type        */
  PA_ERR_LAYOUT = -8       /* a stride the kernels need dense (or aligned) is not   */
} pa_status;

/*
 * Tensor descriptors (paged_decode_attention_desc).  Element types: */
typedef enum pa_dtype {
  PA_DTYPE_BF16 = 1,
  PA_DTYPE_FP8_E4M3FN = 2, /* OCP e4m3fn bytes                                       */
  PA_DTYPE_UINT8 = 3,      /* the same bytes seen as uint8 (accepted for the caches) */
  PA_DTYPE_INT32 = 4,
  PA_DTYPE_FP32 = 5
} pa_dtype;

#define PA_MAX_DIMS 5
/* data: device address of element [0, .., 0]; sizes and strides in elements
 * (strides >= 0); a dim of size 1 may have any stride. */
typedef struct pa_tensor {
  void* data;
  int32_t dtype; /* pa_dtype */
  int32_t ndim;  /* 0 .. PA_MAX_DIMS */
  int64_t sizes[PA_MAX_DIMS];
  int64_t strides[PA_MAX_DIMS];
} pa_tensor;

/* Bytes of the fixed split-KV array of paged_decode_attention_noalloc (per GPU). */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * Paged decode attention (see the top of this file for the operation).
 *
 *   q             bf16  [num_seqs][num_heads][head_size], dense
 *   k_cache       fp8   [num_blocks][num_kv_heads][head_size/16][16][16], dense:
 *                       per (block, kv head) one 2048-byte page holding, for each
 *                       16-dim chunk, the 16 slots' 16 dims
 *   v_cache       fp8   [num_blocks][num_kv_heads][head_size][16], dense: per
 *                       (block, kv head) one 2048-byte page holding, for each dim,
 *                       the 16 slots (the 5-D view [.., 1, head_size, 16] has the
 *                       same bytes)
 *   block_tables  int32 [num_seqs][max_blocks_per_seq], dense; logical block j of
 *                       sequence s is physical block block_tables[s][j]; entries at
 *                       or past ceil(seq_lens[s] / 16) may be read but are never
 *                       used, so they may hold anything
 *   seq_lens      int32 [num_seqs], tokens cached per sequence (current one included)
 *   num_heads     query heads; a positive multiple of num_kv_heads, group <= 16
 *   head_size     must be 128;  block_size must be 16
 *   num_blocks    physical blocks in each cache (sizes the caches for the alias check)
 *   scale         softmax scale applied to q.K (e.g. 1/sqrt(128)), host value
 *   k_scale       fp32 [1], device: dequantisation scale of the K cache
 *   v_scale       fp32 [1], device: dequantisation scale of the V cache
 *   out           bf16  [num_seqs][num_heads][head_size], dense, written in full;
 *                       must not overlap any input
 *   stream        hipStream_t to enqueue on (NULL: the default stream)
 *
 * num_seqs == 0 is a no-op returning PA_OK.
 */
int paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_size, int32_t block_size,
                           int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                           const float* k_scale, const float* v_scale, void* out,
                           void* stream);

/*
 * paged_decode_attention on tensor descriptors: the same operation, with the
 * element types and layouts checked at this boundary and the strides the
 * kernels can follow left free (the arguments of the API page's
 * RocmAiterUnifiedAttentionImpl.forward: query, key_cache / value_cache,
 * block_table, seqused_k, softmax_scale, k_descale / v_descale, output).
 *
 *   q             BF16  [num_seqs, num_heads, 128]: rows [num_heads, 128] dense,
 *                       the sequence stride free (a multiple of 8, >= num_heads * 128)
 *   k_cache       FP8_E4M3FN or UINT8 [num_blocks, num_kv_heads, 8, 16, 16]: each
 *                       (block, kv head) page dense, block and kv-head strides free
 *                       (multiples of 16)
 *   v_cache       FP8_E4M3FN or UINT8 [num_blocks, num_kv_heads, 128, 16] or
 *                       [num_blocks, num_kv_heads, 1, 128, 16]: pages dense, with
 *                       k_cache's block and kv-head strides
 *   block_tables  INT32 [num_seqs, max_blocks_per_seq]: rows dense, row stride free
 *   seq_lens      INT32 [num_seqs], dense
 *   k_scale, v_scale  FP32, one element each (device)
 *   out           BF16  q's sizes, dense, must not overlap any input
 *   scale, stream as for paged_decode_attention
 * Errors: PA_ERR_NULL (a NULL descriptor), PA_ERR_DTYPE (an element type),
 * PA_ERR_SHAPE (ranks and sizes), PA_ERR_UNSUPPORTED (head_size, block_size,
 * group), PA_ERR_LAYOUT (a stride that must be dense or aligned is not, or K
 * and V strides differ), then everything paged_decode_attention reports.
 */
int paged_decode_attention_desc(const pa_tensor* q, const pa_tensor* k_cache,
                                const pa_tensor* v_cache, const pa_tensor* block_tables,
                                const pa_tensor* seq_lens, float scale, const pa_tensor* k_scale,
                                const pa_tensor* v_scale, const pa_tensor* out, void* stream);

/*
 * The same operation with an explicit split-KV partition size: each sequence's
 * blocks are cut into partitions of `pages_per_partition` 16-token blocks,
 * computed independently and merged by a log-sum-exp reduction.  0 lets the
 * library choose (what paged_decode_attention does).  Results of different
 * partition sizes agree to rounding, not bit for bit; one size always gives
 * the same bits for the same inputs.
 */
int paged_decode_attention_split(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_size, int32_t block_size,
                                 int32_t max_blocks_per_seq, int64_t num_blocks,
                                 float scale, const float* k_scale, const float* v_scale,
                                 void* out, void* stream, int32_t pages_per_partition);

/*
 * paged_decode_attention_split that allocates nothing: for callers that
 * cannot call hipMalloc (code under HIP graph capture that must not grow a
 * scratch, tight serving loops, harnesses that forbid allocation).  The
 * split-KV partials and arrival counters live in a fixed array of
 * PA_NOALLOC_SCRATCH_BYTES (16 MiB) in the library's device memory, one copy
 * per GPU, held until the process ends; the caller passes inputs and out.
 *   pages_per_partition  as for paged_decode_attention_split; 0 = the
 *                        library's plan, which needs at most 8.5 MiB on a
 *                        256-CU MI355X
 * A call whose plan needs more than the array returns PA_ERR_WORKSPACE and
 * launches nothing.  All calls on one GPU share its array and find it as the
 * last call left it (the arrival counters back at zero): calls that overlap
 * on one GPU (two streams, concurrent graph replays) race and must not be
 * made.  The first call on a GPU that needs the array also enqueues, on
 * `stream`, one small kernel that clears its counters.  Otherwise (arguments,
 * result, errors) as paged_decode_attention_split.
 */
int paged_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                                   int64_t num_blocks, float scale, const float* k_scale,
                                   const float* v_scale, void* out, void* stream,
                                   int32_t pages_per_partition);

/*
 * Attention of several new query tokens per sequence over the paged cache,
 * causal (the multi-token form of the operation: API page
 * vllm.v1.attention.backends.rocm_aiter_unified_attn,
 * RocmAiterUnifiedAttentionImpl.forward with cu_seqlens_q / query_start_loc,
 * max_seqlen_q, seqused_k and causal=True; the new tokens' K/V are already in
 * the cache, e.g. written by paged_kv_cache_write).
 *
 * Sequence s owns query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1: its q_len
 * newest tokens.  Query i of a sequence with n = seq_lens[s] tokens sits at
 * position n - q_len + i and attends to cache tokens 0 .. n - q_len + i.
 *
 *   q, out          bf16 [num_q_tokens][num_heads][head_size], dense
 *   cu_seqlens_q    int32 [num_seqs + 1], device: cu[0] = 0, cu[num_seqs] = num_q_tokens,
 *                   non-decreasing
 *   max_seqlen_q    host bound on every q_len (the plan is sized from it; queries past it
 *                   are not computed); 0 < q_len <= seq_lens[s] is the caller's contract
 *                   (a query that would see no token gets zeros)
 * Each work item holds floor(16 / group) query tokens of one sequence (all the
 * group's heads for each), so the kernel is at its best for short q_len
 * (speculative or mixed decode); K/V are read once per query tile.  Other
 * arguments, scales, plan, scratch and errors as for paged_decode_attention.
 */
int paged_multi_query_attention(const void* q, const int32_t* cu_seqlens_q, int32_t num_q_tokens,
                                int32_t max_seqlen_q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                                int64_t num_blocks, float scale, const float* k_scale,
                                const float* v_scale, void* out, void* stream);

/*
 * Options of the unified attention call (API page
 * vllm.v1.attention.backends.rocm_aiter_unified_attn:
 * RocmAiterUnifiedAttentionImpl.__init__ takes sliding_window, logits_soft_cap,
 * alibi_slopes and sinks, and forward passes them as window_size, softcap,
 * alibi_slopes and sinks).  For the query at position p of head h:
 *   sliding_window   0: off; w > 0: it sees tokens max(0, p - w + 1) .. p
 *   logits_soft_cap  0: off; c > 0: the logit z = scale * q.K becomes c * tanh(z / c)
 *   alibi_slopes     NULL: off; else device fp32 [num_heads]: the logit gains
 *                    slopes[h] * (t - p), after the softcap
 *   sinks            NULL: off; else device fp32 [num_heads]: one more softmax
 *                    term exp(sinks[h]) that carries no value
 * and, for any call:
 *   longest_first    1: work items are dispatched longest sequence first;
 *                    0: the default order (longest first on the shapes given
 *                    below, else plain); -1: the plain order always.
 *                    Up to 512 sequences (block-table caches) each work item
 *                    finds its own sequence by a counting sort of the lengths;
 *                    otherwise, up to 8192 sequences, a small kernel orders them
 *                    first (about 4.6 us more); above that the order stays plain.
 *                    Where one partition per sequence gives 2 to 4 work items
 *                    per CU, each item then runs as two waves, so that few
 *                    items a CU are resident and the rest start longest first
 *                    as those finish.  Results equal the plain order's bit for
 *                    bit, except in that case, where the two waves' summation
 *                    order makes them agree to rounding (one shape still always
 *                    gives the same bits).  Pays off for ragged contexts (256
 *                    sequences of 1..4000 tokens on MI355X: 40/8 heads 202 ->
 *                    185 us, 32/4 heads 111 -> 96 us); when contexts are alike
 *                    it costs 0.2-0.6% with one wave per item and 1-8% with
 *                    two.  Every call of the
 *                    block layout (paged_decode_attention included) with no
 *                    sliding window and longest_first 0 orders longest first
 *                    by itself (paged_attention_unified with longest_first -1
 *                    and no row offsets is the decode in plain order) where
 *                    num_seqs <= 256, max_blocks_per_seq >= 192 and
 *                    num_seqs * num_kv_heads >= 4 per compute unit: bit for
 *                    bit the plain order's results from 8 units per CU, and
 *                    at 4 (two waves per item, as above) the same to
 *                    rounding; a batch whose lengths all fall in one bin
 *                    keeps the plain order.
 *                    The order kernel's scratch (4 bytes per sequence, after the
 *                    split-KV scratch rounded up to 256 bytes) is not in
 *                    pa_decode_plan's figure.
 */
typedef struct pa_attention_options {
  int32_t sliding_window;
  float logits_soft_cap;
  const float* alibi_slopes;
  const float* sinks;
  int32_t longest_first;
} pa_attention_options;

/*
 * paged_multi_query_attention with the options above (NULL options: none).
 * cu_seqlens_q may be NULL: one query per sequence (the decode; num_q_tokens
 * must equal num_seqs, max_seqlen_q is ignored), computed by the decode kernel
 * when no logit option is set.
 * Errors: PA_ERR_SHAPE for a negative window, a negative or non-finite cap,
 * misaligned option arrays, num_q_tokens != num_seqs without cu_seqlens_q;
 * otherwise as paged_multi_query_attention.  With a window, pages wholly
 * before every query's window are not read.
 */
int paged_attention_unified(const void* q, const int32_t* cu_seqlens_q, int32_t num_q_tokens,
                            int32_t max_seqlen_q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                            int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                            float scale, const float* k_scale, const float* v_scale,
                            const pa_attention_options* options, void* out, void* stream);

/*
 * paged_decode_attention over a token-row cache layout: each token's 128 fp8
 * dims are contiguous, and blocks, tokens and kv heads are reached by byte
 * strides (the flash-style caches of the API page
 * vllm.v1.attention.backends.rocm_aiter_unified_attn: the forward docstring's
 * [num_blocks, 2, block_size, num_kv_heads, head_size], and the
 * [blocks, tokens, kv_heads, head_size] views _split_kv_cache takes of the
 * packed and shuffled caches).  Token j of kv head k in physical block p:
 *   K bytes at k_cache + p * block_stride + j * token_stride + k * head_stride,
 *   V bytes at v_cache + the same offset.
 *   k_cache, v_cache   device, 16-byte aligned (K and V may share one allocation)
 *   block_stride, token_stride, head_stride
 *                      bytes, positive multiples of 16, token_stride <= 2^26
 * Same result as paged_decode_attention on the same bytes in the page layout
 * (bit for bit: the same arithmetic in the same order).  Other arguments, plan,
 * scratch and errors as for paged_decode_attention.
 */
int paged_decode_attention_nhd(const void* q, const void* k_cache, const void* v_cache,
                               int64_t block_stride, int64_t token_stride, int64_t head_stride,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                               int64_t num_blocks, float scale, const float* k_scale,
                               const float* v_scale, void* out, void* stream);

/*
 * paged_decode_attention with per-slot dequantisation scales: one fp32 K scale
 * and one V scale per (block, kv head, slot) instead of one per tensor (the
 * tables the asm decode of the vLLM pull request lishuoshuo-amd/vllm #3 reads,
 * Details > Scale tables):
 *   K_t = fp8(k_cache[...]) * k_slot_scales[block][kv head][slot], V likewise.
 *   k_slot_scales, v_slot_scales  fp32 [num_blocks][num_kv_heads][16], device,
 *                                 16-byte aligned; entries of slots outside every
 *                                 context are never used (they may hold NaN)
 * Other arguments, plan, scratch and errors as for paged_decode_attention.
 */
int paged_decode_attention_slot_scales(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_size, int32_t block_size,
                                       int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                                       const float* k_slot_scales, const float* v_slot_scales,
                                       void* out, void* stream);

/*
 * Launch plan of the one-query decode on block-layout caches
 * (paged_decode_attention, paged_decode_attention_split, _desc, _slot_scales)
 * for the given shapes: host arithmetic only, no device access.
 * num_compute_units: the device's CU count (256 on MI355X).
 * pages_per_partition: as in paged_decode_attention_split (0 = library's choice).
 * Outputs (any may be NULL): number of partitions per sequence, blocks per
 * partition, and the split-KV scratch bytes that plan needs (0 when it has one
 * partition).  Token-row caches (paged_decode_attention_nhd, which splits
 * more where one partition leaves one to eight work items per CU), several
 * queries per sequence and longest-first dispatch change the plan:
 * pa_workspace_bytes covers them.  Returns PA_OK or PA_ERR_SHAPE.
 */
int pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                   int32_t max_blocks_per_seq, int32_t num_compute_units,
                   int32_t pages_per_partition, int32_t* num_partitions,
                   int32_t* pages_per_part, size_t* workspace_bytes);

/*
 * Split-KV scratch bytes a call needs (0: none), for every entry point that
 * plans by itself (all but paged_decode_attention_split):
 *   num_q_tokens, max_seqlen_q  as for paged_multi_query_attention /
 *                               paged_attention_unified; 0, 0 for one query
 *                               per sequence
 *   longest_first               as in pa_attention_options
 *   token_rows                  nonzero for paged_decode_attention_nhd
 *   device                      the HIP device whose compute units the plan
 *                               uses, or -1 for MI355X's 256 (no device access)
 * *bytes receives the size.  Returns PA_OK, PA_ERR_NULL, PA_ERR_SHAPE,
 * PA_ERR_UNSUPPORTED or PA_ERR_HIP (no such device).
 */
int pa_workspace_bytes(int32_t num_seqs, int32_t num_q_tokens, int32_t max_seqlen_q,
                       int32_t num_heads, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                       int32_t longest_first, int32_t token_rows, int device, size_t* bytes);

/*
 * Make the split-KV scratch that calls on (device, stream) use at least
 * `bytes` large: hipMalloc, plus one wait for `stream` while the new buffer's
 * counters are cleared, so call it outside graph capture, before capturing
 * calls on that stream (pa_workspace_bytes gives the size).  An outgrown
 * buffer stays allocated (see the top of this file).  Returns PA_OK,
 * PA_ERR_WORKSPACE (the stream is capturing) or PA_ERR_HIP.
 */
int pa_workspace_reserve(int device, void* stream, size_t bytes);

/*
 * Fill the paged fp8 cache with new tokens (the cache update that precedes the
 * decode: API page vllm.v1.attention.backends.rocm_aiter_unified_attn,
 * do_kv_cache_update, which hands key, value, both caches, slot_mapping and the
 * per-tensor k/v scales to the cache writer; page layout as in the vLLM pull
 * request lishuoshuo-amd/vllm #3, Details > Layout).  For every token t with
 * slot = slot_mapping[t] >= 0, block = slot / 16, s = slot % 16, kv head k, dim d:
 *   k_cache[block][k][d/16][s][d%16] = fp8(key[t][k][d]   / k_scale)
 *   v_cache[block][k][d][s]          = fp8(value[t][k][d] / v_scale)
 * with the division in fp32 and fp8() = OCP e4m3fn, round to nearest even,
 * saturating to +-448 (infinities too); NaN stays NaN with its sign.
 *
 *   key, value        bf16, token t / kv head k / dim d at [t * stride + k * 128 + d];
 *                     4-byte aligned
 *   key_token_stride, value_token_stride
 *                     elements between consecutive tokens (even, >= num_kv_heads * 128:
 *                     key and value may be slices of a fused projection output)
 *   k_cache, v_cache  as for paged_decode_attention; only the addressed slots change
 *   slot_mapping      int64 [num_tokens]; negative = token not cached; a slot at or past
 *                     num_blocks * 16 cannot be reported without a device read and is
 *                     skipped
 *   num_tokens        0 is a no-op
 *   k_scale, v_scale  fp32 [1], device
 * Two tokens with the same slot race (one of them wins).  Asynchronous like
 * paged_decode_attention; errors as there, and PA_ERR_UNSUPPORTED when
 * ceil(num_tokens / 16) * num_kv_heads exceeds 2^26 (one 64-lane workgroup
 * each, within a 2^32-lane grid).
 */
int paged_kv_cache_write(const void* key, const void* value, int64_t key_token_stride,
                         int64_t value_token_stride, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size, int64_t num_blocks,
                         const float* k_scale, const float* v_scale, void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_H_ */
