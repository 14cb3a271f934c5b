// Internal interface of the fp8 KV-cache write kernel (pa_cache_write.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_decode_kernels.h"

namespace pa {

struct CacheWriteParams {
  const uint16_t* key;       // bf16, token t / kv head k / dim d at [t * key_stride + k * 128 + d]
  const uint16_t* value;     // bf16, same with value_stride
  int64_t key_stride;        // elements between tokens
  int64_t value_stride;
  uint8_t* k_cache;          // fp8 [NB][Hkv][8][16][16]
  uint8_t* v_cache;          // fp8 [NB][Hkv][128][16]
  const int64_t* slot_mapping;  // [T]: block * 16 + slot, negative = not cached
  const float* k_scale;      // [1]
  const float* v_scale;      // [1]
  int32_t num_tokens;
  int32_t num_kv_heads;
  int64_t num_blocks;
  int32_t vec16;             // key/value rows allow 16-byte loads (whole-block path)
};

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream);

}  // namespace pa
