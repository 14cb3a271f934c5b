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
 * they may be captured into a HIP graph.  Split-KV scratch is owned by the
 * library (one buffer per device, grown with hipMalloc outside capture only;
 * see pa_decode_reserve_workspace); the call that grows it also waits for
 * `stream` once (the new buffer's counters are cleared before any use).  Two calls that run concurrently on one
 * device (different streams or threads) must not both need the split-KV
 * scratch: they would share it, including the arrival counters at its front
 * (one per (sequence, kv head), zeroed when the scratch is allocated and left
 * at zero by every call), which overlapping calls could leave counting wrong
 * for the calls that follow.
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
  PA_ERR_HIP = -6          /* a HIP runtime call or a kernel launch failed          */
} pa_status;

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
 *   longest_first    0: off; 1: work items are dispatched longest sequence first.
 *                    Up to 512 sequences (block-table caches) each work item
 *                    finds its own sequence by a counting sort of the lengths;
 *                    otherwise, up to 8192 sequences, a small kernel orders them
 *                    first (about 4.6 us more); above that the order stays plain.
 *                    Same results, bit for bit; pays off for ragged contexts
 *                    (256 sequences of 1..4000 tokens at 40/8 heads on MI355X:
 *                    202 -> 185 us) and costs about 3 us when contexts are alike.
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
 * Launch plan for the given shapes (host arithmetic only; no device access).
 * num_compute_units: the device's CU count (256 on MI355X).
 * pages_per_partition: as in paged_decode_attention_split (0 = library's choice).
 * Outputs (any may be NULL): number of partitions per sequence, blocks per
 * partition, and the split-KV scratch bytes that plan needs (0 when it has one
 * partition).  Returns PA_OK or PA_ERR_SHAPE.
 */
int pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                   int32_t max_blocks_per_seq, int32_t num_compute_units,
                   int32_t pages_per_partition, int32_t* num_partitions,
                   int32_t* pages_per_part, size_t* workspace_bytes);

/*
 * Make the current device's split-KV scratch at least `bytes` large.
 * Growing it frees the old buffer (hipFree, which waits for the device) and
 * allocates a new one (hipMalloc), so do it outside graph capture: call it
 * before capturing a graph whose calls need scratch (pa_decode_plan gives the
 * size).  Returns PA_OK or PA_ERR_HIP (allocation failed).
 */
int pa_decode_reserve_workspace(size_t bytes);

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
 * ceil(num_tokens / 16) * num_kv_heads exceeds 2^31 - 1 (one workgroup each).
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
