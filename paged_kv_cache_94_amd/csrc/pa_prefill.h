// pa_prefill.h -- parameters of the paged prefill kernel (pa_prefill.hip) and its launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct PrefillParams {
  void* out;                // [total][Hq][D] bf16
  const void* q;            // [total][Hq][D] bf16, sequence b's queries at rows q_start[b] ..
  const int32_t* q_start;   // [B+1]
  const void* k_pool;       // [num_blocks][16][Hkv][D], bf16 or int8
  const void* v_pool;
  const float* k_scale;     // int8: [num_blocks][Hkv][16], or [Hkv] with head_scales
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;  // cached tokens, this chunk included
  int32_t B, Hq, Hkv, G, maxb, window;
  int32_t ring;             // > 0: table rows are rings of this many entries
  int32_t head_scales;
  float scale_log2;         // caller's scale times log2(e)
  int32_t qt;               // query tokens per tile
  int32_t ntiles;           // tiles per (sequence, KV head) in the grid
};

// Rows (query token x head pairs) one workgroup takes at head_dim D.
constexpr int prefill_rows(int D) { return D >= 256 ? 64 : 128; }

hipError_t launch_prefill(const PrefillParams& p, int kv_dtype, int D, int64_t grid, hipStream_t st,
                          hipEvent_t start, hipEvent_t stop, bool* supported);

}  // namespace pa
