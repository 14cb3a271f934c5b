// gfx950 kernel that fills the paged fp8 KV cache: new tokens' bf16 keys and
// values are divided by the per-tensor scale, rounded to fp8 e4m3fn and
// scattered by slot into the page layout the decode kernel reads.
//
// The step is the cache update of the API page
// vllm.v1.attention.backends.rocm_aiter_unified_attn (do_kv_cache_update:
// key, value, the two caches, slot_mapping and the per-tensor k/v scales go
// to the cache writer); the page layout is that of the vLLM pull request
// lishuoshuo-amd/vllm #3 (Details > Layout): K [head_size/16][16 slots][16],
// V [head_size][16 slots] per (block, kv head).
//
// One wavefront per (group of 16 consecutive tokens, kv head).  When the group
// fills one block in order (the usual prefill pattern) the wave writes the two
// 2 KiB pages whole: each lane converts 2 tokens x 16 dims of K and 16 tokens x
// 2 dims of V and stores 32 contiguous bytes of each page.  Otherwise it walks
// the group token by token, two dims per lane: K as 2-byte stores into 16-byte
// slot rows, V as single bytes (a V page keeps a dim's 16 slots together, so
// one token touches a byte of every dim row).
// A negative slot is a token that is not cached; a slot past the caches is
// skipped too (the host cannot see device data to reject it).
#include <math.h>

#include "pa_cache_write.h"

namespace pa {
namespace {

template <typename T>
__device__ __forceinline__ T scalar_load(const T* ptr) {
  return *(const __attribute__((address_space(4))) T*)(ptr);
}

// Two fp32 values -> two fp8 e4m3fn codes (low byte = a): round to nearest
// even, saturate to +-448, NaN stays NaN with its sign (S.1111.111; the clamp
// turns a NaN into some number, whose code is then replaced).
__device__ __forceinline__ uint32_t fp8x2_saturate(float a, float b) {
  const float ca = fminf(fmaxf(a, -448.0f), 448.0f);
  const float cb = fminf(fmaxf(b, -448.0f), 448.0f);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
  if (a != a) r = (r & 0xFF00u) | (signbit(a) ? 0xFFu : 0x7Fu);
  if (b != b) r = (r & 0x00FFu) | ((signbit(b) ? 0xFFu : 0x7Fu) << 8);
  return r;
}

// The fp32 quotient x / s, correctly rounded.  FAST: Markstein's correction
// of the product with the rounded reciprocal r = RN(1 / s): q0 = RN(x r),
// e = x - q0 s (exact, one FMA), q = RN(q0 + e r) is the correctly rounded
// quotient whenever no step under- or overflows (the kernel checks the scale
// once; other scales take the division).  Where e is 0 (exact quotients, zeros, whose
// sign q0 keeps) or |q0| is far beyond fp8's range (saturated either way,
// infinities included) or q0 is NaN, q0 itself is that quotient's fp8 code.
template <bool FAST>
__device__ __forceinline__ float quot(float x, float s, float r) {
  if constexpr (FAST) {
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, s, x);
    const float q = __builtin_fmaf(e, r, q0);
    return (e != 0.0f && __builtin_fabsf(q0) <= 1.0e4f) ? q : q0;
  } else {
    return x / s;
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Four fp32 -> four fp8 codes in byte order a, b, c, d.
__device__ __forceinline__ uint32_t fp8x4_saturate(float a, float b, float c, float d) {
  return fp8x2_saturate(a, b) | (fp8x2_saturate(c, d) << 16);
}

constexpr int kWavesPerBlock = 4;
constexpr int kGroup = kBlockTokens;  // tokens per wave

// One token, two dims per lane (any slot pattern); kw / vw hold the lane's two
// bf16 key and value dims of the token; kr / vr the scales' reciprocals.
template <bool FAST>
__device__ __forceinline__ void write_token(const CacheWriteParams& p, int kvh, int64_t slot, int lane,
                                            uint32_t kw, uint32_t vw, float ks, float vs, float kr, float vr) {
  if (slot < 0 || slot >= p.num_blocks * kBlockTokens) return;
  const int64_t block = slot / kBlockTokens;
  const int j = (int)(slot % kBlockTokens);
  const int d = 2 * lane;
  const uint32_t kc = fp8x2_saturate(quot<FAST>(bf16_lo(kw), ks, kr), quot<FAST>(bf16_hi(kw), ks, kr));
  const uint32_t vc = fp8x2_saturate(quot<FAST>(bf16_lo(vw), vs, vr), quot<FAST>(bf16_hi(vw), vs, vr));
  const size_t page = ((size_t)block * p.num_kv_heads + kvh) * kPageBytes;
  *(uint16_t*)(p.k_cache + page + (d / 16) * 256 + j * 16 + (d % 16)) = (uint16_t)kc;
  uint8_t* vp = p.v_cache + page + (size_t)d * kBlockTokens + j;
  vp[0] = (uint8_t)(vc & 0xFFu);
  vp[kBlockTokens] = (uint8_t)(vc >> 8);
}

// Sixteen tokens that fill block `block` in slot order: whole-page writes.
template <bool FAST>
__device__ __forceinline__ void write_block(const CacheWriteParams& p, int t0, int kvh, int64_t block,
                                            int lane, float ks, float vs, float kr, float vr) {
  const size_t page = ((size_t)block * p.num_kv_heads + kvh) * kPageBytes;
  // K page bytes [32 l, 32 l + 32): chunk c = l / 8 (dims 16c..16c+15), slots 2(l%8), 2(l%8)+1
  {
    const int c = lane >> 3;
    const int j0 = 2 * (lane & 7);
    uint4 outw[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint16_t* src = p.key + (size_t)(t0 + j0 + u) * p.key_stride + kvh * kHeadDim + 16 * c;
      const uint4 lo = *(const uint4*)src;        // dims +0..7
      const uint4 hi = *(const uint4*)(src + 8);  // dims +8..15
      uint32_t w[4];
      const uint32_t in[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = fp8x4_saturate(quot<FAST>(bf16_lo(in[2 * q]), ks, kr), quot<FAST>(bf16_hi(in[2 * q]), ks, kr),
                              quot<FAST>(bf16_lo(in[2 * q + 1]), ks, kr), quot<FAST>(bf16_hi(in[2 * q + 1]), ks, kr));
      outw[u] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    uint4* dst = (uint4*)(p.k_cache + page + c * 256 + j0 * 16);
    dst[0] = outw[0];
    dst[1] = outw[1];
  }
  // V page bytes [32 l, 32 l + 32): dims 2l and 2l+1, all 16 slots of each
  {
    const int d = 2 * lane;
    float lo[kGroup], hi[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const uint32_t vw = *(const uint32_t*)(p.value + (size_t)(t0 + j) * p.value_stride + kvh * kHeadDim + d);
      lo[j] = quot<FAST>(bf16_lo(vw), vs, vr);
      hi[j] = quot<FAST>(bf16_hi(vw), vs, vr);
    }
    uint32_t a[4], b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = fp8x4_saturate(lo[4 * q], lo[4 * q + 1], lo[4 * q + 2], lo[4 * q + 3]);
      b[q] = fp8x4_saturate(hi[4 * q], hi[4 * q + 1], hi[4 * q + 2], hi[4 * q + 3]);
    }
    uint4* dst = (uint4*)(p.v_cache + page + (size_t)d * kBlockTokens);
    dst[0] = make_uint4(a[0], a[1], a[2], a[3]);
    dst[1] = make_uint4(b[0], b[1], b[2], b[3]);
  }
}

template <bool FAST>
__device__ __forceinline__ void cache_write_group(const CacheWriteParams& p, float ks, float vs, float kr, float vr) {
  const int lane = threadIdx.x & 63;
  // (the wave index read as wave-uniform: the token and head of the item, and
  // every address derived from them, stay scalar)
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t groups = ((int64_t)p.num_tokens + kGroup - 1) / kGroup;
  if (item >= groups * p.num_kv_heads) return;
  const int t0 = (int)(item / p.num_kv_heads) * kGroup;
  const int kvh = (int)(item % p.num_kv_heads);
  const int n = min(kGroup, p.num_tokens - t0);

  // slot of token t0 + lane (lanes past the group: -1)
  const int64_t my_slot = (lane < n) ? p.slot_mapping[t0 + lane] : -1;
  const int64_t s0 = (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(my_slot & 0xFFFFFFFF)) |
                     ((int64_t)__builtin_amdgcn_readfirstlane((int)(my_slot >> 32)) << 32);
  const bool in_order = (lane >= kGroup) || (my_slot == s0 + lane);
  const bool whole = p.vec16 && n == kGroup && s0 >= 0 && (s0 % kBlockTokens) == 0 &&
                     s0 < p.num_blocks * kBlockTokens && __builtin_amdgcn_ballot_w64(!in_order) == 0;
  if (whole) {
    write_block<FAST>(p, t0, kvh, s0 / kBlockTokens, lane, ks, vs, kr, vr);
    return;
  }
  // Any slot pattern: read every token's two dims first (the cache stores may
  // alias the inputs as far as the compiler knows, so loads interleaved with
  // them would wait for each store), then convert and store token by token.
  uint32_t kw[kGroup], vw[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const int t = t0 + min(i, n - 1);
    kw[i] = *(const uint32_t*)(p.key + t * p.key_stride + kvh * kHeadDim + 2 * lane);
    vw[i] = *(const uint32_t*)(p.value + t * p.value_stride + kvh * kHeadDim + 2 * lane);
  }
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    if (i >= n) break;
    const int64_t slot = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)(my_slot & 0xFFFFFFFF), i) |
                         ((int64_t)__builtin_amdgcn_readlane((int)(my_slot >> 32), i) << 32);
    write_token<FAST>(p, kvh, slot, lane, kw[i], vw[i], ks, vs, kr, vr);
  }
}

// Scales whose magnitude lies in [2^-60, 2^60]: then r is normal too, and for
// every quotient fp8 can tell from zero (|x / s| >= 2^-10) the remainder e is
// a normal number, so the FMA computes it exactly.  False for 0, subnormals,
// infinities and NaN.
__device__ __forceinline__ bool quotient_scale(float x) {
  const float a = __builtin_fabsf(x);
  return a >= 0x1p-60f && a <= 0x1p60f;
}

__global__ __launch_bounds__(64 * kWavesPerBlock) void pa_cache_write_kernel(const CacheWriteParams p) {
  const float ks = scalar_load(p.k_scale);
  const float vs = scalar_load(p.v_scale);
  const float kr = 1.0f / ks;
  const float vr = 1.0f / vs;
  // usable scales: the short quotient; anything else takes the division
  if (quotient_scale(ks) && quotient_scale(vs))
    cache_write_group<true>(p, ks, vs, kr, vr);
  else
    cache_write_group<false>(p, ks, vs, kr, vr);
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream) {
  const int64_t items = ((int64_t)p.num_tokens + kGroup - 1) / kGroup * p.num_kv_heads;
  const int64_t blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(pa_cache_write_kernel, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
