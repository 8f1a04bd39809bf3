// pa_aux.hip -- the split-combine kernel and the debug gather kernel.
//
// Combine: when a sequence's key range is cut into S splits, split s leaves
// (m_s, l_s, o_s) -- its max score in base-2 units, its softmax sum and its
// unnormalised output. The merge is the online-softmax rule of the Lab 5
// handout ("Flash Attention") applied across splits:
//   M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One workgroup per output row; one thread per dim of the head.
#include "pa_common.h"

namespace pa {

template <typename OutT, int D>
__global__ void __launch_bounds__(D) pa_combine_kernel(const Params p) {
  // One workgroup per output row (unit, r); thread d owns dim d. The split's
  // (m, l) pair is the same for the whole workgroup (a uniform load).
  const int32_t row_id = blockIdx.x;
  const int r = row_id % p.rows;
  const int32_t unit = row_id / p.rows;
  const int32_t b = unit / p.Hkv;
  const int32_t g = unit % p.Hkv;
  const int32_t L = p.seq_lens[b];
  if (!len_ok(L, p)) return;
  // Slots holding this unit's partials: contiguous in both partitions.
  int64_t slot_first;
  int32_t ns;
  if (p.balanced) {
    // Workgroups w0..w1 each left a partial in slot w + unit; a unit inside a
    // single workgroup's slice was written out directly.
    const int32_t* pre = p.ws_prefix;
    const int32_t nb = pre[b + 1] - pre[b];
    if (nb == 0) return;
    const Balanced bal = balanced_split(pre, p.B, p.Hkv, p.nwg);
    const int64_t off = (int64_t)p.Hkv * pre[b] + (int64_t)g * nb;
    const int64_t w0 = off / bal.per, w1 = (off + nb - 1) / bal.per;
    if (w0 == w1) return;
    slot_first = w0 + unit;
    ns = (int32_t)(w1 - w0 + 1);
  } else {
    const KeyRange kr = key_range(L, p.q_len, p.window);
    slot_first = (int64_t)unit * p.splits;
    ns = min(live_splits(kr, p.bps), p.splits);
  }

  const size_t slot0 = (size_t)slot_first * p.rows + r;
  const size_t step = (size_t)p.rows;
  const float* ml = p.ws_ml + slot0 * 2;
  const float* acc = p.ws_acc + slot0 * D + threadIdx.x;
  const int lane = threadIdx.x & 63;

  // Split s's (m, l) sits in lane s % 64: the max and the weights come from
  // wave reductions, and every split's accumulator load below is independent.
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) M = fmaxf(M, ml[s * step * 2]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
  const float Ms = M == -INFINITY ? 0.f : M;
  float num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < ns; c0 += 64) {
    const int s = c0 + lane;
    float w = 0.f;
    if (s < ns) {
      w = fast_exp2(ml[s * step * 2] - Ms);
      den += w * ml[s * step * 2 + 1];
    }
    const int cnt = min(64, ns - c0);
#pragma unroll 8
    for (int j = 0; j < cnt; ++j) {
      const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
      num += wj * acc[(size_t)(c0 + j) * step * D];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += shfl_xor(den, off);
  const int t = r / p.G;
  const int h = g * p.G + r % p.G;
  OutT* out = reinterpret_cast<OutT*>(p.out) + (((size_t)b * p.q_len + t) * p.Hq + h) * D + threadIdx.x;
  if constexpr (sizeof(OutT) == 4) {
    *out = num / den;
  } else {
    *out = (__bf16)(num / den);
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
  const int64_t rows = (int64_t)p.B * p.Hkv * p.rows;
  if (rows == 0) return hipSuccess;
  if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)rows);
  const bool bf16 = q_dtype == 1;
  switch (D) {
    case 64:
      if (bf16) hipLaunchKernelGGL((pa_combine_kernel<__bf16, 64>), grid, dim3(64), 0, st, p);
      else hipLaunchKernelGGL((pa_combine_kernel<float, 64>), grid, dim3(64), 0, st, p);
      break;
    case 128:
      if (bf16) hipLaunchKernelGGL((pa_combine_kernel<__bf16, 128>), grid, dim3(128), 0, st, p);
      else hipLaunchKernelGGL((pa_combine_kernel<float, 128>), grid, dim3(128), 0, st, p);
      break;
    case 256:
      if (bf16) hipLaunchKernelGGL((pa_combine_kernel<__bf16, 256>), grid, dim3(256), 0, st, p);
      else hipLaunchKernelGGL((pa_combine_kernel<float, 256>), grid, dim3(256), 0, st, p);
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
