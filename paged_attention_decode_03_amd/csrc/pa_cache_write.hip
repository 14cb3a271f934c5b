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
// One wavefront per (group of 16 consecutive tokens, kv head).  Each lane
// converts one token's 32 dims of K and 2 dims of all 16 tokens' V.  K goes
// out as whole 16-byte rows (chunk, slot) of the K pages, whatever the slots;
// V rows keep a dim's 16 slots together, so the group is cut into runs of
// tokens whose slots follow each other in one block (one run filling a block
// in a prefill that starts on a block; two pieces of blocks where it starts
// inside one or where a sequence ends), and each run's bytes of a dim row go
// out in the widest aligned stores that cover them.  Rows of the key/value
// inputs without 16-byte alignment take a token-by-token walk instead (K as
// 2-byte stores, V as single bytes).
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

// One per-tensor scale s with what the short quotient needs: r = RN(1 / s)
// and the dividend bound lim = 512 s.
struct Scale {
  float s, r, lim;
};

// The fp32 quotient x / s, correctly rounded.  FAST: Markstein's correction
// of the product with the rounded reciprocal: q0 = RN(x r), e = q0 s - x
// (exact, one FMA), q = RN(q0 - e r) is the correctly rounded quotient when
// no step under- or overflows.  The kernel takes this path for scales in
// [2^-60, 2^60] only: then r is normal, and for every quotient fp8 can tell
// from zero (|x / s| >= 2^-10) e is a normal number, so the FMA is exact.
// Dividends beyond 512 s (quotients past 512, saturated to 448 either way,
// infinities included) are clamped to +-512 s first, so nothing overflows;
// the correction's signs keep the sign of a zero quotient.  NaN dividends
// are told apart by the caller.  Checked on the CPU against fp32 division
// for all 65536 bf16 dividends at 4000 scales: the same fp8 code every time.
template <bool FAST>
__device__ __forceinline__ float quot(float x, const Scale& sc) {
  if constexpr (FAST) {
    const float xc = __builtin_amdgcn_fmed3f(x, -sc.lim, sc.lim);  // (a NaN x: any value)
    const float q0 = xc * sc.r;
    const float e = __builtin_fmaf(q0, sc.s, -xc);
    return __builtin_fmaf(-e, sc.r, q0);
  } else {
    return x / sc.s;
  }
}

// Two quotients -> two fp8 e4m3fn codes (low byte = a): round to nearest
// even, saturate to +-448.  WITH_NAN: where na / nb is a NaN, the code is
// NaN with its sign (S.1111.111), whatever the clamp made of the quotient;
// without it the caller has made sure there is no NaN.
template <bool WITH_NAN>
__device__ __forceinline__ uint32_t fp8x2_code(float a, float b, float na, float nb) {
  // (the median of three is the clamp; a NaN gives some value, replaced below)
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
  if constexpr (WITH_NAN) {
    if (na != na) r = (r & 0xFF00u) | (signbit(na) ? 0xFFu : 0x7Fu);
    if (nb != nb) r = (r & 0x00FFu) | ((signbit(nb) ? 0xFFu : 0x7Fu) << 8);
  }
  return r;
}

// Two dividends -> their quotients' fp8 codes.  A NaN quotient comes from a
// NaN dividend on the short path (with the dividend's sign, as the division
// would give) and is taken from the quotient itself on the division path.
template <bool FAST, bool WITH_NAN>
__device__ __forceinline__ uint32_t code2(float x0, float x1, const Scale& sc) {
  const float q0 = quot<FAST>(x0, sc);
  const float q1 = quot<FAST>(x1, sc);
  return fp8x2_code<WITH_NAN>(q0, q1, FAST ? x0 : q0, FAST ? x1 : q1);
}

template <bool FAST, bool WITH_NAN>
__device__ __forceinline__ uint32_t code4(float a, float b, float c, float d, const Scale& sc) {
  return code2<FAST, WITH_NAN>(a, b, sc) | (code2<FAST, WITH_NAN>(c, d, sc) << 16);
}

// Lanes of the wave holding a NaN among a, b, c, d (one compare per value; the
// masks are wave-wide, so or-ing them costs scalar instructions only).
__device__ __forceinline__ uint64_t nan_lanes(float a, float b, float c, float d) {
  return __builtin_amdgcn_ballot_w64(a != a) | __builtin_amdgcn_ballot_w64(b != b) |
         __builtin_amdgcn_ballot_w64(c != c) | __builtin_amdgcn_ballot_w64(d != d);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One wave per workgroup: the waves of a launch spread over every CU (measured
// on MI355X, graph replay: 256 tokens x 8 kv heads at random slots 7.1 ->
// 6.6 us, 32768 tokens x 8 kv heads in whole blocks 38.3 -> 35.0 us, against
// four waves per workgroup; two: 7.4 / 35.5 us).
constexpr int kWavesPerBlock = 1;
constexpr int kGroup = kBlockTokens;  // tokens per wave
// Groups of more runs than this write V token by token (measured on MI355X,
// kernel trace: a decode step of 256 tokens x 8 kv heads at random slots 9.6
// us in a loop over each group's 16 runs of one token, 6.2 us token by token)
constexpr int kMaxRunsStored = 4;

// One token, two dims per lane (any slot pattern); kw / vw hold the lane's two
// bf16 key and value dims of the token.
template <bool FAST>
__device__ __forceinline__ void write_token(const CacheWriteParams& p, int kvh, int64_t slot, int lane,
                                            uint32_t kw, uint32_t vw, const Scale& ks, const Scale& vs) {
  if (slot < 0 || slot >= p.num_blocks * kBlockTokens) return;
  const int64_t block = slot / kBlockTokens;
  const int j = (int)(slot % kBlockTokens);
  const int d = 2 * lane;
  const uint32_t kc = code2<FAST, true>(bf16_lo(kw), bf16_hi(kw), ks);
  const uint32_t vc = code2<FAST, true>(bf16_lo(vw), bf16_hi(vw), vs);
  const size_t page = ((size_t)block * p.num_kv_heads + kvh) * kPageBytes;
  *(uint16_t*)(p.k_cache + page + (d / 16) * 256 + j * 16 + (d % 16)) = (uint16_t)kc;
  uint8_t* vp = p.v_cache + page + (size_t)d * kBlockTokens + j;
  vp[0] = (uint8_t)(vc & 0xFFu);
  vp[kBlockTokens] = (uint8_t)(vc >> 8);
}

// The lane's codes: kout[u] the 16 fp8 codes of kin[u] (16 dims of one
// token), vout[0] / vout[1] the codes of dims 2l / 2l + 1 of the group's 16
// tokens (byte t = token t).  The codes are made without NaN handling unless a
// NaN is in the wave's inputs (or the division path, where the scale may be one).
template <bool FAST, bool WITH_NAN>
__device__ __forceinline__ void block_codes(const uint32_t (&kin)[2][8], const uint32_t (&vin)[kGroup],
                                            const Scale& ks, const Scale& vs, uint4 (&kout)[2], uint4 (&vout)[2]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = code4<FAST, WITH_NAN>(bf16_lo(kin[u][2 * q]), bf16_hi(kin[u][2 * q]), bf16_lo(kin[u][2 * q + 1]),
                              bf16_hi(kin[u][2 * q + 1]), ks);
    kout[u] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  uint32_t a[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    a[q] = code4<FAST, WITH_NAN>(bf16_lo(vin[4 * q]), bf16_lo(vin[4 * q + 1]), bf16_lo(vin[4 * q + 2]),
                            bf16_lo(vin[4 * q + 3]), vs);
    b[q] = code4<FAST, WITH_NAN>(bf16_hi(vin[4 * q]), bf16_hi(vin[4 * q + 1]), bf16_hi(vin[4 * q + 2]),
                            bf16_hi(vin[4 * q + 3]), vs);
  }
  vout[0] = make_uint4(a[0], a[1], a[2], a[3]);
  vout[1] = make_uint4(b[0], b[1], b[2], b[3]);
}

// Bytes [x, x + 8) of a 16-byte row held as two 64-bit halves (x wave-uniform,
// 0 <= x <= 15; bytes past the row read as 0).
__device__ __forceinline__ uint64_t row_bytes(uint64_t lo, uint64_t hi, int x) {
  if (x >= 8) return hi >> (8 * (x - 8));
  if (x == 0) return lo;
  return (lo >> (8 * x)) | (hi << (64 - 8 * x));
}

// Slots [a, a + len) of two V page rows (dims d and d + 1: `row` and row + 16,
// 16-byte aligned) from the codes of tokens [o, o + len) of the group, held in
// token order (byte t = token t) as (la, ha) and (lb, hb).  The widest aligned
// stores that cover the range; a, len and o are wave-uniform, a + len <= 16.
__device__ __forceinline__ void store_rows(uint8_t* row, uint64_t la, uint64_t ha, uint64_t lb, uint64_t hb,
                                           int a, int len, int o) {
  if (a == 0 && len == kBlockTokens) {  // (then o = 0) the whole rows
    *(uint4*)row = make_uint4((uint32_t)la, (uint32_t)(la >> 32), (uint32_t)ha, (uint32_t)(ha >> 32));
    *(uint4*)(row + kBlockTokens) =
        make_uint4((uint32_t)lb, (uint32_t)(lb >> 32), (uint32_t)hb, (uint32_t)(hb >> 32));
    return;
  }
  const int end = a + len;
  for (int pos = a; pos < end;) {
    const uint64_t va = row_bytes(la, ha, pos - a + o);
    const uint64_t vb = row_bytes(lb, hb, pos - a + o);
    if ((pos & 7) == 0 && pos + 8 <= end) {
      *(uint64_t*)(row + pos) = va;
      *(uint64_t*)(row + kBlockTokens + pos) = vb;
      pos += 8;
    } else if ((pos & 3) == 0 && pos + 4 <= end) {
      *(uint32_t*)(row + pos) = (uint32_t)va;
      *(uint32_t*)(row + kBlockTokens + pos) = (uint32_t)vb;
      pos += 4;
    } else if ((pos & 1) == 0 && pos + 2 <= end) {
      *(uint16_t*)(row + pos) = (uint16_t)va;
      *(uint16_t*)(row + kBlockTokens + pos) = (uint16_t)vb;
      pos += 2;
    } else {
      row[pos] = (uint8_t)va;
      row[kBlockTokens + pos] = (uint8_t)vb;
      pos += 1;
    }
  }
}

// Any slot pattern, rows that allow 16-byte loads.  K: lane l converts token
// l & 15's dims of chunks l >> 4 and 4 + (l >> 4) and stores each as the
// whole 16-byte row (chunk, slot) of its page.  V: lane l converts dims 2l and
// 2l + 1 of all 16 tokens, and the group is cut into runs (tokens whose slots
// follow each other in one block: a whole block in a prefill that starts on a
// block, two pieces of blocks where it does not); each run's slots of the two
// dim rows are written with the widest aligned stores.  Runs of one block may
// come from two groups (a run that crosses a group boundary): each writes
// only its own tokens' bytes.
template <bool FAST>
__device__ __forceinline__ void write_runs(const CacheWriteParams& p, int t0, int n, int kvh, int lane,
                                           const Scale& ks, const Scale& vs) {
  const int jt = lane & 15;  // K: the lane's token; the lane of token jt in each row of 16
  const int c0 = lane >> 4;  // K: chunks c0 and c0 + 4
  const int d = 2 * lane;    // V: dims d and d + 1
  uint32_t kin[2][8], vin[kGroup];
  const int tk = t0 + min(jt, n - 1);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint16_t* src = p.key + (size_t)tk * p.key_stride + kvh * kHeadDim + 16 * (c0 + 4 * u);
    const uint4 lo = *(const uint4*)src;        // dims +0..7
    const uint4 hi = *(const uint4*)(src + 8);  // dims +8..15
    kin[u][0] = lo.x, kin[u][1] = lo.y, kin[u][2] = lo.z, kin[u][3] = lo.w;
    kin[u][4] = hi.x, kin[u][5] = hi.y, kin[u][6] = hi.z, kin[u][7] = hi.w;
  }
#pragma unroll
  for (int j = 0; j < kGroup; ++j)
    vin[j] = *(const uint32_t*)(p.value + (size_t)(t0 + min(j, n - 1)) * p.value_stride + kvh * kHeadDim + d);
  // The slot of token t0 + jt (tokens past the group: -1), read after the
  // inputs: read first, the wave waited for it before issuing them (measured
  // on MI355X, back to back, 32768 tokens x 8 kv heads in whole blocks 39.2
  // -> 35.4 us, 8 sequences of 3000-5000 44.5 -> 41.6 us, chunks starting
  // inside blocks 48.8 -> 46.3 us; with the unaligned-row walk in a kernel of
  // its own)
  const int64_t my_slot = (jt < n) ? p.slot_mapping[t0 + jt] : -1;
  bool nan = true;
  if constexpr (FAST) {
    uint64_t m = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < 8; q += 2)
        m |= nan_lanes(bf16_lo(kin[u][q]), bf16_hi(kin[u][q]), bf16_lo(kin[u][q + 1]), bf16_hi(kin[u][q + 1]));
#pragma unroll
    for (int j = 0; j < kGroup; j += 2)
      m |= nan_lanes(bf16_lo(vin[j]), bf16_hi(vin[j]), bf16_lo(vin[j + 1]), bf16_hi(vin[j + 1]));
    nan = m != 0;
  }
  uint4 kout[2], vout[2];
  if (nan)
    block_codes<FAST, true>(kin, vin, ks, vs, kout, vout);
  else
    block_codes<FAST, false>(kin, vin, ks, vs, kout, vout);

  const int64_t cap = p.num_blocks * kBlockTokens;
  const bool valid = jt < n && my_slot >= 0 && my_slot < cap;
  if (valid) {
    uint8_t* kp = p.k_cache + ((size_t)(my_slot / kBlockTokens) * p.num_kv_heads + kvh) * kPageBytes +
                  (my_slot % kBlockTokens) * 16;
    *(uint4*)(kp + c0 * 256) = kout[0];
    *(uint4*)(kp + (c0 + 4) * 256) = kout[1];
  }
  // the previous token's slot (lane jt - 1 of the row of 16; none for token 0)
  const uint32_t prev_lo = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)my_slot, 0x111, 0xF, 0xF, false);
  const uint32_t prev_hi = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)(my_slot >> 32), 0x111, 0xF, 0xF, false);
  const int64_t prev = (int64_t)(((uint64_t)prev_hi << 32) | prev_lo);
  // token jt continues the run of token jt - 1: the next slot of the same block
  const bool cont = valid && jt > 0 && prev >= 0 && my_slot == prev + 1 && (my_slot % kBlockTokens) != 0;
  uint64_t starts = __builtin_amdgcn_ballot_w64(lane < kGroup && valid && !cont);
  const uint64_t conts = __builtin_amdgcn_ballot_w64(lane < kGroup && cont);
  const uint64_t la = (uint64_t)vout[0].x | ((uint64_t)vout[0].y << 32);
  const uint64_t ha = (uint64_t)vout[0].z | ((uint64_t)vout[0].w << 32);
  const uint64_t lb = (uint64_t)vout[1].x | ((uint64_t)vout[1].y << 32);
  const uint64_t hb = (uint64_t)vout[1].z | ((uint64_t)vout[1].w << 32);
  if (__builtin_popcountll(starts) > kMaxRunsStored) {
    // many short runs (a decode step's scattered slots): token by token, the
    // two dim rows' bytes of each (no loop over runs)
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      if (i >= n) break;
      const int64_t s = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)(my_slot & 0xFFFFFFFF), i) |
                        ((int64_t)__builtin_amdgcn_readlane((int)(my_slot >> 32), i) << 32);
      if (s < 0 || s >= cap) continue;
      uint8_t* vp = p.v_cache + ((size_t)(s / kBlockTokens) * p.num_kv_heads + kvh) * kPageBytes +
                    (size_t)d * kBlockTokens + (s % kBlockTokens);
      vp[0] = (uint8_t)((i < 8 ? la : ha) >> (8 * (i & 7)));
      vp[kBlockTokens] = (uint8_t)((i < 8 ? lb : hb) >> (8 * (i & 7)));
    }
    return;
  }
  while (starts) {
    const int o = __builtin_ctzll(starts);
    starts &= starts - 1;
    const int len = 1 + __builtin_ctzll(~(conts >> (o + 1)));
    const int64_t s = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)(my_slot & 0xFFFFFFFF), o) |
                      ((int64_t)__builtin_amdgcn_readlane((int)(my_slot >> 32), o) << 32);
    uint8_t* row = p.v_cache + ((size_t)(s / kBlockTokens) * p.num_kv_heads + kvh) * kPageBytes +
                   (size_t)d * kBlockTokens;
    store_rows(row, la, ha, lb, hb, (int)(s % kBlockTokens), len, o);
  }
}

template <bool FAST, bool VEC16>
__device__ __forceinline__ void cache_write_group(const CacheWriteParams& p, const Scale& ks, const Scale& vs) {
  const int lane = threadIdx.x & 63;
  // (the wave index read as wave-uniform: the token and head of the item, and
  // every address derived from them, stay scalar)
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t groups = ((int64_t)p.num_tokens + kGroup - 1) / kGroup;
  if (item >= groups * p.num_kv_heads) return;
  const int t0 = (int)(item / p.num_kv_heads) * kGroup;
  const int kvh = (int)(item % p.num_kv_heads);
  const int n = min(kGroup, p.num_tokens - t0);

  if constexpr (VEC16) {
    write_runs<FAST>(p, t0, n, kvh, lane, ks, vs);
    return;
  }
  // Rows without 16-byte alignment: read every token's two dims first (the cache stores may
  // alias the inputs as far as the compiler knows, so loads interleaved with
  // them would wait for each store), then convert and store token by token.
  uint32_t kw[kGroup], vw[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const int t = t0 + min(i, n - 1);
    kw[i] = *(const uint32_t*)(p.key + t * p.key_stride + kvh * kHeadDim + 2 * lane);
    vw[i] = *(const uint32_t*)(p.value + t * p.value_stride + kvh * kHeadDim + 2 * lane);
  }
  // slot of token t0 + lane (lanes past the group: -1), after the inputs
  const int64_t my_slot = (lane < n) ? p.slot_mapping[t0 + lane] : -1;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    if (i >= n) break;
    const int64_t slot = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)(my_slot & 0xFFFFFFFF), i) |
                         ((int64_t)__builtin_amdgcn_readlane((int)(my_slot >> 32), i) << 32);
    write_token<FAST>(p, kvh, slot, lane, kw[i], vw[i], ks, vs);
  }
}

// Scales in [2^-60, 2^60] (positive): the short quotient's range.  False for
// negative scales, 0, subnormals, infinities and NaN.
__device__ __forceinline__ bool quotient_scale(float x) { return x >= 0x1p-60f && x <= 0x1p60f; }

// VEC16: rows that allow 16-byte loads (p.vec16), else the token walk.
// Registers for three waves per SIMD (168 VGPRs, no spills; four would spill):
// measured on MI355X against two, back to back, 32768 tokens x 8 kv heads in
// whole blocks 35.7 -> 32.5 us, 8 sequences of 3000-5000 41.0 -> 36.5 us, 64
// of 200-800 42.5 -> 38.3 us, chunks starting inside blocks 46.2 -> 44.0 us.
template <bool VEC16>
__global__ __launch_bounds__(64 * kWavesPerBlock) __attribute__((amdgpu_waves_per_eu(3))) void pa_cache_write_kernel(
    const CacheWriteParams p) {
  const float ks = scalar_load(p.k_scale);
  const float vs = scalar_load(p.v_scale);
  const Scale kq = {ks, 1.0f / ks, 512.0f * ks};
  const Scale vq = {vs, 1.0f / vs, 512.0f * vs};
  // usable scales: the short quotient; anything else takes the division
  if (quotient_scale(ks) && quotient_scale(vs))
    cache_write_group<true, VEC16>(p, kq, vq);
  else
    cache_write_group<false, VEC16>(p, kq, vq);
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream) {
  const int64_t items = ((int64_t)p.num_tokens + kGroup - 1) / kGroup * p.num_kv_heads;
  const int64_t blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  if (p.vec16)
    hipLaunchKernelGGL(pa_cache_write_kernel<true>, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0, stream, p);
  else
    hipLaunchKernelGGL(pa_cache_write_kernel<false>, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
