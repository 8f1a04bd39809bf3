// pa_write.h -- parameters of the KV-append kernel (pa_write.hip) and its launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct WriteParams {
  const void* k_new;        // [T][Hkv][D], source dtype
  const void* v_new;
  const int64_t* slot_ids;  // [T]: block * 16 + slot; < 0 skips the token
  void* k_pool;             // [num_blocks][16][Hkv][D], cache dtype
  void* v_pool;
  float* k_scale;           // int8 caches: [num_blocks][Hkv][16], or [Hkv] with head_scales
  float* v_scale;
  int32_t T, Hkv, num_blocks;
  int32_t write_v;          // 0 when the V pool is the K pool (written once)
  int32_t head_scales;      // int8: 1 -> k_scale / v_scale are given per head [Hkv], read only
};

// start / stop: NULL, or events stamped from the kernel's own dispatch.
hipError_t launch_cache_write(const WriteParams& p, int src_dtype, int kv_dtype, int D, hipStream_t st,
                              hipEvent_t start, hipEvent_t stop, bool* supported);

}  // namespace pa
