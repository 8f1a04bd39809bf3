// pa_aux.hip -- the split-combine kernel and the debug gather kernel.
//
// Combine: when a sequence's key range is cut into S splits, split s leaves
// (m_s, l_s, o_s) -- its max score in base-2 units, its softmax sum and its
// unnormalised output. The merge is the online-softmax rule of the Lab 5
// handout ("Flash Attention") applied across splits:
//   M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One wavefront per output row; lanes cover the head dimension.
#include "pa_common.h"

namespace pa {

template <typename OutT, int D>
__global__ void __launch_bounds__(256) pa_combine_kernel(const Params p) {
  constexpr int PER = D / 64;   // dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = (int64_t)p.B * p.Hkv * p.rows;
  if (wid >= total) return;
  const int r = (int)(wid % p.rows);
  const int32_t unit = (int32_t)(wid / p.rows);
  const int32_t b = unit / p.Hkv;
  const int32_t g = unit % p.Hkv;
  const int32_t L = p.seq_lens[b];
  if (!len_ok(L, p)) return;
  const KeyRange kr = key_range(L, p.q_len, p.window);
  const int32_t ns = min(live_splits(kr, p.bps), p.splits);

  const size_t base = (size_t)unit * p.splits * p.rows + r;   // slot of split 0
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, p.ws_ml[(base + (size_t)s * p.rows) * 2]);
  const float Ms = M == -INFINITY ? 0.f : M;
  float num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  float den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t slot = base + (size_t)s * p.rows;
    const float w = fast_exp2(p.ws_ml[slot * 2] - Ms);
    den += w * p.ws_ml[slot * 2 + 1];
    const float* src = p.ws_acc + slot * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] += w * src[e];
  }
  const float inv = 1.f / den;
  const int t = r / p.G;
  const int h = g * p.G + r % p.G;
  OutT* out = reinterpret_cast<OutT*>(p.out) + (((size_t)b * p.q_len + t) * p.Hq + h) * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if constexpr (sizeof(OutT) == 4) {
      out[e] = num[e] * inv;
    } else {
      out[e] = (__bf16)(num[e] * inv);
    }
  }
}

// Debug gather: copy the cache rows the attention kernels would load, in
// logical key order, through the same key_range / row_offset_bytes helpers.
// grid.x covers tokens (one wavefront per token, 4 per workgroup), grid.y = sequence.
__global__ void __launch_bounds__(256) pa_gather_kernel(const Params p, const char* pool, int32_t row_bytes,
                                                          char* dst, int64_t dst_tokens) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int32_t b = blockIdx.y;
  const int32_t L = p.seq_lens[b];
  if (!len_ok(L, p)) return;
  const KeyRange kr = key_range(L, p.q_len, p.window);
  const int64_t n_keys = (int64_t)L - kr.lo0;
  if (w >= n_keys || w >= dst_tokens) return;
  const int32_t j = kr.lo0 + (int32_t)w;
  const int32_t phys = p.block_table[(size_t)b * p.maxb + j / kBlock];
  const int32_t words = row_bytes / 4;
  for (int32_t g = 0; g < p.Hkv; ++g) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(pool + row_offset_bytes(phys, j % kBlock, g, p.Hkv, row_bytes));
    uint32_t* out = reinterpret_cast<uint32_t*>(dst + (((size_t)b * dst_tokens + w) * p.Hkv + g) * (size_t)row_bytes);
    for (int32_t k = lane; k < words; k += 64) out[k] = src[k];
  }
}

hipError_t launch_combine(const Params& p, int q_dtype, int D, hipStream_t st) {
  const int64_t waves = (int64_t)p.B * p.Hkv * p.rows;
  const int grid = (int)((waves + 3) / 4);
  if (grid == 0) return hipSuccess;
  const bool bf16 = q_dtype == 1;
  switch (D) {
    case 64:
      if (bf16) hipLaunchKernelGGL((pa_combine_kernel<__bf16, 64>), dim3(grid), dim3(256), 0, st, p);
      else hipLaunchKernelGGL((pa_combine_kernel<float, 64>), dim3(grid), dim3(256), 0, st, p);
      break;
    case 128:
      if (bf16) hipLaunchKernelGGL((pa_combine_kernel<__bf16, 128>), dim3(grid), dim3(256), 0, st, p);
      else hipLaunchKernelGGL((pa_combine_kernel<float, 128>), dim3(grid), dim3(256), 0, st, p);
      break;
    case 256:
      if (bf16) hipLaunchKernelGGL((pa_combine_kernel<__bf16, 256>), dim3(grid), dim3(256), 0, st, p);
      else hipLaunchKernelGGL((pa_combine_kernel<float, 256>), dim3(grid), dim3(256), 0, st, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gather(const Params& p, int kv_dtype, int D, int which, void* dst, int64_t dst_tokens,
                         hipStream_t st) {
  const int32_t eb = kv_dtype == 0 ? 4 : (kv_dtype == 1 ? 2 : 1);
  const char* pool = reinterpret_cast<const char*>(which == 0 ? p.k_pool : p.v_pool);
  const int64_t gx = (dst_tokens + 3) / 4;
  if (gx == 0 || p.B == 0) return hipSuccess;
  hipLaunchKernelGGL(pa_gather_kernel, dim3((unsigned)gx, (unsigned)p.B), dim3(256), 0, st, p, pool, D * eb,
                     reinterpret_cast<char*>(dst), dst_tokens);
  return hipGetLastError();
}

}  // namespace pa
