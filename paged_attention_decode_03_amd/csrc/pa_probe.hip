// Bandwidth probes for the benchmark (libpa_probe.so, not part of the
// attention library): what MI355X's HBM delivers to plain reads, as the
// practical ceiling the decode kernel is measured against.
//
//   pa_probe_read_stream  one pass over a large buffer, each workgroup reading
//                         a contiguous chunk with 16-byte loads
//   pa_probe_page_gather  the decode's own access pattern without its
//                         arithmetic: one wave per (sequence, kv head) walks
//                         the block table and reads each 2 KiB K page and
//                         2 KiB V page (two 16-byte loads a lane per page),
//                         with a chosen stage size and ring depth
//
// Both fold what they read into one word per workgroup (so no load is dead)
// and write it to `sink`.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource: no format conversion, no swizzle
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;        // 16-byte loads in flight per thread

template <int AUX>
__global__ __launch_bounds__(kStreamThreads) void read_stream_kernel(const uint8_t* buf, uint64_t chunk,
                                                                     uint32_t* sink) {
  const uint8_t* base = buf + (uint64_t)blockIdx.x * chunk;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)chunk, kRsrcWord3);
  constexpr uint32_t kStep = kStreamThreads * 16 * kStreamUnroll;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint32_t off = threadIdx.x * 16; off < chunk; off += kStep) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + u * kStreamThreads * 16, 0, AUX));
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t part[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// One wave per (sequence, kv head) unit; pages of the unit's table row up to
// ceil(seq_len / 16), dense page layout (K and V pages of 2048 bytes at
// (block * Hkv + kv head) * 2048).  PPS pages a stage, a ring of NB stages
// (NB - 1 in flight while one is folded).
template <int PPS, int NB>
__global__ __launch_bounds__(64) void page_gather_kernel(const uint8_t* k_cache, const uint8_t* v_cache,
                                                         const int32_t* block_tables, const int32_t* seq_lens,
                                                         int num_kv_heads, int max_blocks, uint32_t* sink) {
  const int lane = threadIdx.x;
  const int unit = blockIdx.x;
  const int s = unit / num_kv_heads, kvh = unit % num_kv_heads;
  const int len = seq_lens[s];
  const int npages = min((len + 15) / 16, max_blocks);
  const int32_t* bt = block_tables + (size_t)s * max_blocks;
  const size_t page_stride = (size_t)num_kv_heads * 2048;
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 ring[NB][PPS][4];
  auto load = [&](u32x4 (&st)[PPS][4], int stage) {
#pragma unroll
    for (int pp = 0; pp < PPS; ++pp) {
      const int i = stage * PPS + pp;
      const int pid = __builtin_amdgcn_readfirstlane(i < npages ? bt[i] : 0);
      const int bytes = i < npages ? 2048 : 0;
      const size_t off = (size_t)pid * page_stride + (size_t)kvh * 2048;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k_cache + off), (short)0, bytes, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v_cache + off), (short)0, bytes, kRsrcWord3);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        st[pp][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, lane * 16 + 1024 * h, 0, 2));
        st[pp][2 + h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane * 16 + 1024 * h, 0, 2));
      }
    }
  };
  const int nsteps = (npages + PPS - 1) / PPS;
#pragma unroll
  for (int k = 0; k < NB - 1; ++k) load(ring[k], k);
  for (int st = 0; st < nsteps; st += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (st + k >= nsteps) break;
      // loads past the last page: zero-byte descriptors, no memory touched
      load(ring[(k + NB - 1) % NB], st + k + NB - 1);
#pragma unroll
      for (int pp = 0; pp < PPS; ++pp)
#pragma unroll
        for (int h = 0; h < 4; ++h) acc ^= ring[k][pp][h];
    }
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0) sink[unit] = x;
}

}  // namespace

extern "C" {

// Read bytes [0, blocks * chunk) of buf once: `blocks` workgroups of 256
// threads, workgroup b reading bytes [b * chunk, (b + 1) * chunk).  chunk must
// be a positive multiple of 16 below 2^31; sink holds `blocks` words.
// nontemporal: 1 = loads with the streaming hint, 0 = default policy.
// Returns 0, -2 (bad sizes) or -6 (launch failed).
int pa_probe_read_stream(const void* buf, uint64_t chunk, int32_t blocks, int32_t nontemporal,
                         uint32_t* sink, void* stream) {
  if (!buf || !sink || blocks <= 0 || chunk == 0 || (chunk & 15) || chunk >= (uint64_t(1) << 31)) return -2;
  if (nontemporal)
    hipLaunchKernelGGL(read_stream_kernel<2>, dim3(blocks), dim3(kStreamThreads), 0, (hipStream_t)stream,
                       (const uint8_t*)buf, chunk, sink);
  else
    hipLaunchKernelGGL(read_stream_kernel<0>, dim3(blocks), dim3(kStreamThreads), 0, (hipStream_t)stream,
                       (const uint8_t*)buf, chunk, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// The decode's page reads alone, over the same caches, table and lengths
// (dense page layout; every used block id must lie in the caches, seq_lens
// at most 16 * max_blocks).  sink holds num_seqs * num_kv_heads words.
// pages_per_stage: 1, 2 or 4; ring_depth: 2, 3 or 4 stages (depth - 1 in
// flight while one is folded); the decode itself reads 2 pages a stage in a
// ring of 2.
int pa_probe_page_gather(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                         int32_t max_blocks, int32_t pages_per_stage, int32_t ring_depth, uint32_t* sink,
                         void* stream) {
  if (!k_cache || !v_cache || !block_tables || !seq_lens || !sink || num_seqs <= 0 || num_kv_heads <= 0 ||
      max_blocks <= 0 || (int64_t)num_seqs * num_kv_heads > INT32_MAX)
    return -2;
  const dim3 grid(num_seqs * num_kv_heads), block(64);
  hipStream_t st = (hipStream_t)stream;
  const auto* kc = (const uint8_t*)k_cache;
  const auto* vc = (const uint8_t*)v_cache;
#define PA_PROBE_GATHER(P, D)                                                                         \
  if (pages_per_stage == P && ring_depth == D) {                                                      \
    hipLaunchKernelGGL((page_gather_kernel<P, D>), grid, block, 0, st, kc, vc, block_tables, seq_lens, \
                       num_kv_heads, max_blocks, sink);                                               \
    return hipGetLastError() == hipSuccess ? 0 : -6;                                                  \
  }
  PA_PROBE_GATHER(1, 2) PA_PROBE_GATHER(1, 3) PA_PROBE_GATHER(1, 4)
  PA_PROBE_GATHER(2, 2) PA_PROBE_GATHER(2, 3) PA_PROBE_GATHER(2, 4)
  PA_PROBE_GATHER(4, 2) PA_PROBE_GATHER(4, 3) PA_PROBE_GATHER(4, 4)
#undef PA_PROBE_GATHER
  return -2;
}

}  // extern "C"
