// pa_probe.hip -- a load-only kernel that measures how fast this part
// delivers a workload's cache tiles, for the roofline figures of the
// benchmark (libpa_probe.so; not part of the attention library's ABI).
//
// It reads exactly the (block, KV head) tiles one attention step reads, in
// the order and with the loads the matrix-core decode kernel uses -- each
// cached row front to back in 16-byte non-temporal pieces, LPR lanes per row,
// DEPTH tiles in flight per wavefront -- and does nothing with them but fold
// them into one word per wavefront (so the loads cannot be dropped). The
// pool layout is [num_blocks][16][Hkv][row_bytes] (tiniestgpt notes,
// "PagedAttention"); a tile id is phys * Hkv + g. Workgroup w streams tiles
// [w * per, (w + 1) * per) of the list, its wavefronts taking them in turn.
#include <hip/hip_ext.h>

#include "pa_device.h"
#include "pa_probe.h"

namespace pa {

template <int ROW_BYTES, bool TWO, int DEPTH>
__global__ void __launch_bounds__(512) pa_probe_kernel(const char* pool_k, const char* pool_v, const int32_t* tiles,
                                                        int32_t ntiles, int32_t Hkv, int32_t per, uint32_t* sink) {
  constexpr int LPR = ROW_BYTES / 16;
  constexpr int RPI = 64 / LPR;
  constexpr int NLOAD = kBlock / RPI;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int32_t tok_stride = token_stride_bytes(Hkv, ROW_BYTES);
  const int32_t tile_bytes = (kBlock - 1) * tok_stride + ROW_BYTES;
  const int32_t lane_off = (lane / LPR) * tok_stride + 16 * (lane % LPR);
  const int32_t t0 = (int32_t)min((int64_t)blockIdx.x * per, (int64_t)ntiles);
  const int32_t t1 = (int32_t)min((int64_t)t0 + per, (int64_t)ntiles);
  const int32_t mine = t1 > t0 + wave ? (t1 - t0 - wave + nw - 1) / nw : 0;
  uint4 buf[DEPTH][TWO ? 2 : 1][NLOAD];
  uint32_t acc = 0;
  auto fetch = [&](int32_t k, uint4 (&f)[TWO ? 2 : 1][NLOAD]) __attribute__((always_inline)) {
    const bool valid = k < mine;
    const int32_t id = valid ? tiles[t0 + wave + nw * k] : 0;
    const size_t off = tile_offset_bytes(id / Hkv, id % Hkv, Hkv, ROW_BYTES);
    const auto kd = buffer_rsrc(pool_k + off, valid ? tile_bytes : 0);
#pragma unroll
    for (int u = 0; u < NLOAD; ++u) f[0][u] = buffer_load16(kd, lane_off, u * RPI * tok_stride);
    if constexpr (TWO) {
      const auto vd = buffer_rsrc(pool_v + off, valid ? tile_bytes : 0);
#pragma unroll
      for (int u = 0; u < NLOAD; ++u) f[1][u] = buffer_load16(vd, lane_off, u * RPI * tok_stride);
    }
  };
  auto fold = [&](const uint4 (&f)[TWO ? 2 : 1][NLOAD]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < (TWO ? 2 : 1); ++t)
#pragma unroll
      for (int u = 0; u < NLOAD; ++u) acc ^= f[t][u].x ^ f[t][u].y ^ f[t][u].z ^ f[t][u].w;
  };
#pragma unroll
  for (int d = 0; d + 1 < DEPTH; ++d) fetch(d, buf[d]);
  for (int32_t k = 0; k < mine; k += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      fetch(k + d + DEPTH - 1, buf[(d + DEPTH - 1) % DEPTH]);
      fold(buf[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fold(buf[d]);
  sink[(size_t)blockIdx.x * nw * 64 + threadIdx.x] = acc;
}

template <int ROW_BYTES, bool TWO>
hipError_t probe_depth(int depth, dim3 grid, dim3 block, hipStream_t st, hipEvent_t e0, hipEvent_t e1,
                       const char* k, const char* v, const int32_t* tiles, int32_t n, int32_t Hkv, int32_t per,
                       uint32_t* sink) {
  switch (depth) {
    case 1: hipExtLaunchKernelGGL((pa_probe_kernel<ROW_BYTES, TWO, 1>), grid, block, 0, st, e0, e1, 0, k, v, tiles,
                                  n, Hkv, per, sink); break;
    case 2: hipExtLaunchKernelGGL((pa_probe_kernel<ROW_BYTES, TWO, 2>), grid, block, 0, st, e0, e1, 0, k, v, tiles,
                                  n, Hkv, per, sink); break;
    case 3: hipExtLaunchKernelGGL((pa_probe_kernel<ROW_BYTES, TWO, 3>), grid, block, 0, st, e0, e1, 0, k, v, tiles,
                                  n, Hkv, per, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa

extern "C" int pa_probe_read(const void* k_pool, const void* v_pool, const int32_t* tiles, int32_t ntiles,
                             int32_t row_bytes, int32_t num_kv_heads, int32_t workgroups, int32_t waves,
                             int32_t depth, uint32_t* sink, void* timing_start, void* timing_stop, void* stream) {
  if (!k_pool || !tiles || !sink || ntiles < 0 || num_kv_heads < 1 || workgroups < 1 || waves < 1 || waves > 8)
    return 1;
  if (depth < 1 || depth > 3) return 1;
  const int32_t per = (int32_t)(((int64_t)ntiles + workgroups - 1) / workgroups);
  const dim3 grid((unsigned)workgroups), block((unsigned)(64 * waves));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t e0 = reinterpret_cast<hipEvent_t>(timing_start), e1 = reinterpret_cast<hipEvent_t>(timing_stop);
  const char* k = reinterpret_cast<const char*>(k_pool);
  const char* v = reinterpret_cast<const char*>(v_pool);
  const bool two = v_pool && v_pool != k_pool;
  hipError_t e = hipErrorInvalidValue;
  switch (row_bytes) {
    case 128: e = two ? pa::probe_depth<128, true>(depth, grid, block, st, e0, e1, k, v, tiles, ntiles, num_kv_heads, per, sink)
                      : pa::probe_depth<128, false>(depth, grid, block, st, e0, e1, k, v, tiles, ntiles, num_kv_heads, per, sink);
              break;
    case 256: e = two ? pa::probe_depth<256, true>(depth, grid, block, st, e0, e1, k, v, tiles, ntiles, num_kv_heads, per, sink)
                      : pa::probe_depth<256, false>(depth, grid, block, st, e0, e1, k, v, tiles, ntiles, num_kv_heads, per, sink);
              break;
    case 512: e = two ? pa::probe_depth<512, true>(depth, grid, block, st, e0, e1, k, v, tiles, ntiles, num_kv_heads, per, sink)
                      : pa::probe_depth<512, false>(depth, grid, block, st, e0, e1, k, v, tiles, ntiles, num_kv_heads, per, sink);
              break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}
