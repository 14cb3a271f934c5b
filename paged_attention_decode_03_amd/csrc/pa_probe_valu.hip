// A decode kernel whose dot products run on the vector ALUs instead of the
// matrix cores (libpa_probe.so, not part of the attention library): the
// benchmark times it beside the MFMA decode on the same inputs, so the choice
// of MFMA for qKᵀ and PV rests on a measurement.
//
// It computes what the library's one-query decode computes (vLLM pull request
// lishuoshuo-amd/vllm #3, Details: softmax(qKᵀ·scale)·V over a sequence's
// fp8-e4m3fn pages reached through its block table, per-tensor k/v scales):
// one wave per (sequence, kv head), the whole context in one pass (no split),
// dense page layout (K [blocks][kv heads][8][16][16], V [blocks][kv heads][128][16]).
//
// Per page of 16 tokens:
//   scores  lane (t = lane & 15, c = lane >> 4) dots dims 32c .. 32c + 31 of
//           token t with every head of the group (bf16 pairs, v_dot2 into
//           fp32; fp8 -> bf16 is exact), then the four partial sums are added
//           across the rows (permlane swaps), so every row holds the page's
//           16 scores of each head;
//   softmax online, in fp32: the page max over the 16 tokens (DPP row
//           rotations), the running max, 2^(z - m); each lane keeps its
//           token's share of the denominator, summed over the tokens once
//           at the end;
//   PV      lane l owns dims 2l and 2l + 1: its 32 V bytes (two dims x 16
//           tokens, contiguous in the page) are converted to fp32 and
//           multiplied with the page's weights of each head, which row 0
//           writes to LDS and every lane reads back (broadcast reads).
// Loads: two 16-byte K loads and two 16-byte V loads a lane per page, through
// buffer descriptors (zero bytes for pages past the context or block ids
// outside the caches), with the streaming hint, in a ring of three pages
// (two in flight while one is computed).  q stays in registers (16 a head), so
// groups of up to 6 heads run two waves per SIMD; 7 and 8 heads run one (the
// registers past 256 held in AGPRs).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource: no format conversion, no swizzle
constexpr int kAuxStream = 2;           // loads with the streaming (nontemporal) hint
constexpr int kMaxTable = 1024;         // table entries a sequence may use (block ids staged in LDS)

// Sum of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows); the
// same additions in the same order in every row, so all rows get equal bits.
__device__ __forceinline__ float sum_rows(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// x of the lane R places further along its 16-lane row (DPP row rotation)
template <int R>
__device__ __forceinline__ float row_rotate(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + R, 0xF, 0xF, false));
}

__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, row_rotate<8>(x));
  x = fmaxf(x, row_rotate<4>(x));
  x = fmaxf(x, row_rotate<2>(x));
  return fmaxf(x, row_rotate<1>(x));
}

__device__ __forceinline__ float row_sum(float x) {
  x += row_rotate<8>(x);
  x += row_rotate<4>(x);
  x += row_rotate<2>(x);
  return x + row_rotate<1>(x);
}

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct PageRegs {
  u32x4 k[2];  // token t, dims 32c .. 32c + 15 and 32c + 16 .. 32c + 31
  u32x4 v[2];  // dim 2l, tokens 0..15; dim 2l + 1, tokens 0..15
};

template <int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(G <= 6 ? 2 : 1))) void valu_decode_kernel(
    const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* block_tables,
    const int32_t* seq_lens, int num_kv_heads, int max_blocks, uint32_t num_blocks, float scale_log2e,
    const float* k_scale, const float* v_scale, uint16_t* out) {
  const int lane = threadIdx.x;
  const int unit = blockIdx.x;
  const int s = unit / num_kv_heads, kvh = unit % num_kv_heads;
  const int t = lane & 15, c = lane >> 4;
  const int L = min(max(seq_lens[s], 0), max_blocks * 16);
  const int npages = (L + 15) / 16;
  const size_t orow = ((size_t)s * num_kv_heads * G + (size_t)kvh * G) * 128;  // first head of the group
  if (L == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) *(uint32_t*)(out + orow + h * 128 + 2 * lane) = 0u;
    return;
  }

  __shared__ int32_t ids[kMaxTable];
  __shared__ __attribute__((aligned(16))) float wts[G][16];
  const int32_t* bt = block_tables + (size_t)s * max_blocks;
  for (int i = lane; i < npages; i += 64) ids[i] = bt[i];
  __syncthreads();

  // q, dims 32c .. 32c + 31 of each head, as bf16 pairs
  uint32_t qv[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4* src = (const u32x4*)(q + orow + h * 128 + 32 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u32x4 x = src[w];
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[h][4 * w + e] = x[e];
    }
  }
  const float c_log2 = scale_log2e * k_scale[0];
  const float vsc = v_scale[0];

  float m_run[G], l_lane[G], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.0f;
    acc[h][0] = acc[h][1] = 0.0f;
  }

  auto load = [&](PageRegs& pr, int i) {
    const bool in = i < npages;
    const int32_t pid = __builtin_amdgcn_readfirstlane(in ? ids[in ? i : 0] : 0);
    const bool used = in && (uint32_t)pid < num_blocks;
    const size_t off = ((size_t)(uint32_t)pid * num_kv_heads + kvh) * 2048;
    const int bytes = used ? 2048 : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(k_cache + (used ? off : 0)), (short)0, bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(v_cache + (used ? off : 0)), (short)0, bytes, kRsrcWord3);
    pr.k[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (2 * c) * 256 + t * 16, 0, kAuxStream));
    pr.k[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (2 * c + 1) * 256 + t * 16, 0, kAuxStream));
    pr.v[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane * 32, 0, kAuxStream));
    pr.v[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, lane * 32 + 16, 0, kAuxStream));
    __builtin_amdgcn_sched_barrier(0);
  };

  auto compute = [&](const PageRegs& pr, int i) {
    const bool last = i == npages - 1;
    // K, dims 32c + 2j and 32c + 2j + 1 in pair j (fp8 -> bf16 is exact)
    bf16x2 kb[16];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        kb[8 * hh + 2 * w] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pr.k[hh][w], 1.0f, false);
        kb[8 * hh + 2 * w + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pr.k[hh][w], 1.0f, true);
      }
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) d = __builtin_amdgcn_fdot2_f32_bf16(kb[j], __builtin_bit_cast(bf16x2, qv[h][j]), d, false);
      float z = sum_rows(d) * c_log2;  // log2 units
      if (last && i * 16 + t >= L) z = -INFINITY;
      // the page's first token is in the context, so the page max is finite
      const float m_new = fmaxf(m_run[h], row_max(z));
      alpha[h] = __builtin_amdgcn_exp2f(m_run[h] - m_new);  // 0 while m_run = -inf
      const float w = __builtin_amdgcn_exp2f(z - m_new);
      l_lane[h] = l_lane[h] * alpha[h] + w;
      m_run[h] = m_new;
      if (c == 0) wts[h][t] = w;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    // V of dims 2l, 2l + 1; bytes of tokens past the context (any value, even NaN) zeroed
    uint32_t vw[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vw[e] = pr.v[0][e];
      vw[4 + e] = pr.v[1][e];
    }
    if (last) {
      const int nv = L - i * 16;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int k = nv - 4 * w;
        const uint32_t mask = k >= 4 ? 0xFFFFFFFFu : (k <= 0 ? 0u : ((1u << (8 * k)) - 1u));
        vw[w] &= mask;
        vw[4 + w] &= mask;
      }
    }
    float vf[2][16];
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vw[4 * d + w], 1.0f, false);
        const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vw[4 * d + w], 1.0f, true);
        vf[d][4 * w] = a[0];
        vf[d][4 * w + 1] = a[1];
        vf[d][4 * w + 2] = b[0];
        vf[d][4 * w + 3] = b[1];
      }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float pw[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4v x = *(const f32x4v*)&wts[h][4 * k];
        pw[4 * k] = x[0];
        pw[4 * k + 1] = x[1];
        pw[4 * k + 2] = x[2];
        pw[4 * k + 3] = x[3];
      }
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        float a = acc[h][d] * alpha[h];
#pragma unroll
        for (int k = 0; k < 16; ++k) a = fmaf(pw[k], vf[d][k], a);
        acc[h][d] = a;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  };

  // pages a wave holds: two in flight while one is computed
  constexpr int kRing = 3;
  PageRegs ring[kRing];
#pragma unroll
  for (int k = 0; k < kRing - 1; ++k) load(ring[k], k);
  for (int i0 = 0; i0 < npages; i0 += kRing) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      const int i = i0 + k;
      if (i >= npages) break;
      load(ring[(k + kRing - 1) % kRing], i + kRing - 1);
      compute(ring[k], i);
    }
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float l = row_sum(l_lane[h]);
    const float inv = l > 0.0f ? vsc / l : 0.0f;
    *(uint32_t*)(out + orow + h * 128 + 2 * lane) = bf16_bits(acc[h][0] * inv) | (bf16_bits(acc[h][1] * inv) << 16);
  }
}

}  // namespace

extern "C" {

// The decode with its dot products on the vector ALUs: q bf16 [num_seqs,
// num_heads, 128] (dense), caches in the dense page layout above (fp8 e4m3fn
// bytes), block_tables int32 [num_seqs, max_blocks], seq_lens int32
// [num_seqs] (clamped to 16 * max_blocks), k_scale / v_scale one fp32 each on
// the device, out bf16 [num_seqs, num_heads, 128].  num_heads / num_kv_heads
// must be 1..8 and max_blocks at most 1024.  A block id outside
// [0, num_blocks) reads as a zero page.  Returns 0, -2 (bad arguments) or -6
// (launch failed).
int pa_probe_decode_valu(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                         int32_t max_blocks, int64_t num_blocks, float scale, const float* k_scale,
                         const float* v_scale, void* out, void* stream) {
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !k_scale || !v_scale || !out)
    return -2;
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_heads <= 0 || num_heads % num_kv_heads != 0 || max_blocks <= 0 ||
      max_blocks > kMaxTable || num_blocks <= 0 || (int64_t)num_seqs * num_kv_heads > INT32_MAX)
    return -2;
  const int G = num_heads / num_kv_heads;
  const uint32_t nb = (uint32_t)(num_blocks < (int64_t)UINT32_MAX ? num_blocks : (int64_t)UINT32_MAX);
  const float sl2e = (float)((double)scale * 1.4426950408889634);
  const dim3 grid(num_seqs * num_kv_heads), block(64);
  hipStream_t st = (hipStream_t)stream;
  const auto* qq = (const uint16_t*)q;
  const auto* kc = (const uint8_t*)k_cache;
  const auto* vc = (const uint8_t*)v_cache;
  auto* o = (uint16_t*)out;
#define PA_PROBE_VALU(GG)                                                                                       \
  case GG:                                                                                                      \
    hipLaunchKernelGGL(valu_decode_kernel<GG>, grid, block, 0, st, qq, kc, vc, block_tables, seq_lens,          \
                       num_kv_heads, max_blocks, nb, sl2e, k_scale, v_scale, o);                                \
    break;
  switch (G) {
    PA_PROBE_VALU(1) PA_PROBE_VALU(2) PA_PROBE_VALU(3) PA_PROBE_VALU(4)
    PA_PROBE_VALU(5) PA_PROBE_VALU(6) PA_PROBE_VALU(7) PA_PROBE_VALU(8)
    default:
      return -2;
  }
#undef PA_PROBE_VALU
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
