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

// Number of combine workgroups per output row: one per unit for aligned
// splits and the piece partition, one per workgroup boundary for the
// flattened-list partition (only units cut by a boundary have partials).
__host__ __device__ inline int64_t combine_groups(const Params& p) {
  return p.balanced == 1 ? (int64_t)(p.nwg > 1 ? p.nwg - 1 : 0) : (int64_t)p.B * p.Hkv;
}

constexpr int kCombineChunk = 64;   // partials whose loads are in flight together

template <typename OutT, int D>
__global__ void __launch_bounds__(D) pa_combine_kernel(const Params p) {
  // Workgroup (group, r): output row r of one unit; thread d owns dim d.
  const int r = blockIdx.x % p.rows;
  const int32_t grp = blockIdx.x / p.rows;
  const int lane = threadIdx.x & 63;
  int32_t b, g;
  int64_t slot_first;
  int32_t ns;
  if (p.balanced == 1) {
    // Boundary grp lies between workgroups grp and grp+1, at item x of the
    // flattened list. The unit holding x is merged here if it starts inside
    // workgroup grp (it is then cut by this boundary first); workgroups
    // w0..w1 left its partials in slots w + unit. The block prefix sums are
    // staged in LDS so the search below costs no memory round trips.
    __shared__ int32_t pre[kMaxBalancedSeqs + 1];
    for (int32_t i = threadIdx.x; i <= p.B; i += D) pre[i] = p.ws_prefix[i];
    __syncthreads();
    const Balanced bal = balanced_split(pre, p.B, p.Hkv, p.nwg);
    const int64_t x = (int64_t)(grp + 1) * bal.per;
    if (x >= bal.total) return;
    b = balanced_seq(pre, p.B, p.Hkv, x);
    const int32_t nb = pre[b + 1] - pre[b];
    const int64_t base = (int64_t)p.Hkv * pre[b];
    g = (int32_t)((x - base) / nb);
    const int64_t off = base + (int64_t)g * nb;
    if (off >= x || off < (int64_t)grp * bal.per) return;
    const int64_t w1 = (off + nb - 1) / bal.per;
    slot_first = grp + (int64_t)b * p.Hkv + g;
    ns = (int32_t)(w1 - grp + 1);
  } else {
    b = grp / p.Hkv;
    g = grp % p.Hkv;
    const int32_t L = p.seq_lens[b];
    if (!len_ok(L, p)) return;
    if (p.balanced == 2) {
      // Piece partition: unit (b, g) was cut into k pieces, owned by
      // workgroups kp[b] + g*k .. + k-1, each of which left its partial in
      // the slot of its own index; a unit of one piece was written out directly.
      const int32_t k = (p.ws_prefix[b + 1] - p.ws_prefix[b]) / p.Hkv;
      if (k <= 1) return;
      slot_first = p.ws_prefix[b] + (int64_t)g * k;
      ns = k;
    } else {
      const KeyRange kr = key_range(L, p.q_len, p.window);
      slot_first = (int64_t)grp * p.splits;
      ns = min(live_splits(kr, p.bps), p.splits);
    }
  }

  const size_t slot0 = (size_t)slot_first * p.rows + r;
  const size_t step = (size_t)p.rows;
  const float* ml = p.ws_ml + slot0 * 2;
  const float* acc = p.ws_acc + slot0 * D + threadIdx.x;

  // Chunks of up to 64 partials: every load of a chunk is issued before any
  // is used. Partial s's (m, l) sits in lane s % 64; the chunk max and the
  // weights come from wave reductions and v_readlane. Chunks after the first
  // rescale the running sums (online-softmax rule).
  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int32_t c0 = 0; c0 < ns; c0 += kCombineChunk) {
    const int32_t cnt = min(kCombineChunk, ns - c0);
    float a[kCombineChunk];
#pragma unroll
    for (int j = 0; j < kCombineChunk; ++j) a[j] = j < cnt ? acc[(size_t)(c0 + j) * step * D] : 0.f;
    const float ms = lane < cnt ? ml[(size_t)(c0 + lane) * step * 2] : -INFINITY;
    const float ls = lane < cnt ? ml[(size_t)(c0 + lane) * step * 2 + 1] : 0.f;
    float cm = ms;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cm = fmaxf(cm, shfl_xor(cm, off));
    const float Mn = fmaxf(M, cm);
    const float Ms = Mn == -INFINITY ? 0.f : Mn;
    const float resc = fast_exp2(M - Ms);   // 0 on the first chunk (M = -inf)
    num *= resc;
    den *= resc;
    M = Mn;
    const float w = lane < cnt ? fast_exp2(ms - Ms) : 0.f;
    float dl = w * ls;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dl += shfl_xor(dl, off);
    den += dl;
#pragma unroll
    for (int j = 0; j < kCombineChunk; ++j)
      num += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j)) * a[j];
  }
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
  const int64_t rows = combine_groups(p) * p.rows;
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
