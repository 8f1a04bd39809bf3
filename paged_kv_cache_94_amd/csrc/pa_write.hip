// pa_write.hip -- KV append: this step's new key and value rows go into the
// paged pools (tiniestgpt notes, "PagedAttention": pool[block][slot][head][dim],
// the step's tokens addressed by slot ids = block * 16 + slot).
//
// Each (token, KV head) row is carried by the 8 to 64 lanes that hold its
// bytes 16 at a time. A float cache takes the row as it is. An int8 cache
// takes the row quantized per token and head (tiniestgpt notes,
// "Quantization", KV cache quantization): the row's lanes find its largest
// magnitude with a lane reduction, scale = max / 127 (1 for an
// all-zero row), codes rint(x / scale) clamped to [-127, 127]. The divisions
// are IEEE binary32 (hipcc's default correctly rounded division) and rint
// rounds half to even, so the codes are those of any binary32 evaluation of
// the same formula. Scales are stored [block][head][slot].
#include <hip/hip_ext.h>

#include "pa_device.h"
#include "pa_write.h"

namespace pa {

namespace {

// Largest |x| over an aligned group of N lanes (N a power of two, <= 64); every lane gets it.
template <int N>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int off = N / 2; off >= 1; off >>= 1) x = fmaxf(x, shfl_xor(x, off));
  return x;
}

// Widen the 16 source bytes a lane holds to EPL floats (8 bf16 or 4 fp32).
template <bool SRC_BF16>
__device__ __forceinline__ void widen(const uint4& w, float* x) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  if constexpr (SRC_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, u[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __builtin_bit_cast(float, u[i]);
  }
}

// Quantize one lane's EPL values of a row whose LPR lanes hold it together;
// returns the packed codes (EPL bytes) and the row's scale. `given_mode`
// (uniform over the launch): quantize with `given`, the head's fixed scale,
// instead of the row's own max / 127.
template <bool SRC_BF16, int LPR>
__device__ __forceinline__ float quantize_lane(const uint4& w, uint32_t* packed, bool given_mode, float given) {
  constexpr int EPL = SRC_BF16 ? 8 : 4;
  float x[EPL];
  widen<SRC_BF16>(w, x);
  float scale = given;
  if (!given_mode) {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = group_max<LPR>(amax);
    scale = amax > 0.f ? amax / 127.0f : 1.0f;
  }
#pragma unroll
  for (int i = 0; i < EPL / 4; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float c = __builtin_rintf(x[4 * i + e] / scale);
      c = fminf(fmaxf(c, -127.0f), 127.0f);
      word |= (uint32_t)(uint8_t)(int8_t)(int32_t)c << (8 * e);
    }
    packed[i] = word;
  }
  return scale;
}

}  // namespace

// Each lane carries 16 source bytes of a row, so a row spans LPR = D * e_src / 16
// lanes (8 to 64) and a wavefront carries 64 / LPR rows; rows are (token, head)
// pairs in token-major order, so a wavefront's loads are one contiguous run.
template <bool SRC_BF16, int KV, int D>
__global__ void __launch_bounds__(256) pa_cache_write_kernel(const WriteParams p) {
  constexpr int ESRC = SRC_BF16 ? 2 : 4;
  constexpr int LPR = D * ESRC / 16;
  constexpr int RPW = 64 / LPR;
  constexpr int EPL = 16 / ESRC;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPR;
  const int64_t rows = (int64_t)p.T * p.Hkv;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const bool live_row = row < rows;
  const int64_t t = live_row ? row / p.Hkv : 0;
  const int32_t g = live_row ? (int32_t)(row % p.Hkv) : 0;
  const int64_t s = live_row ? p.slot_ids[t] : -1;
  // Skipped token, id outside the pool, or a lane past the last row: nothing is stored,
  // but the lane still takes part in the row maximum's shuffles.
  const bool store = s >= 0 && s < (int64_t)p.num_blocks * kBlock;
  const int32_t blk = store ? (int32_t)(s / kBlock) : 0;
  const int32_t slot = store ? (int32_t)(s % kBlock) : 0;
  const size_t in = ((size_t)t * p.Hkv + g) * D + (size_t)sub * EPL;                    // source element
  constexpr int ECACHE = KV == 2 ? 1 : ESRC;                                           // bytes per cache element
  const size_t at = row_offset_bytes(blk, slot, g, p.Hkv, D * ECACHE) + (size_t)sub * EPL * ECACHE;  // pool byte
  const uint4 zero = {0u, 0u, 0u, 0u};
  const uint4 wk = store ? *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.k_new) + in * ESRC) : zero;
  const uint4 wv = store && p.write_v
                       ? *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.v_new) + in * ESRC)
                       : zero;
  if constexpr (KV == 2) {
    const size_t sat = scale_tile_index(blk, g, p.Hkv) + slot;
    const bool hs = p.head_scales != 0;
    const float gk = hs && live_row ? p.k_scale[g] : 1.0f;
    const float gv = hs && live_row ? p.v_scale[g] : 1.0f;
    uint32_t ck[EPL / 4], cv[EPL / 4];
    const float sk = quantize_lane<SRC_BF16, LPR>(wk, ck, hs, gk);
    const float sv = quantize_lane<SRC_BF16, LPR>(wv, cv, hs, gv);
    if (store) {
      int8_t* dk = reinterpret_cast<int8_t*>(p.k_pool) + at;
      int8_t* dv = reinterpret_cast<int8_t*>(p.v_pool) + at;
      if constexpr (EPL == 8) {
        *reinterpret_cast<uint2*>(dk) = make_uint2(ck[0], ck[1]);
        if (p.write_v) *reinterpret_cast<uint2*>(dv) = make_uint2(cv[0], cv[1]);
      } else {
        *reinterpret_cast<uint32_t*>(dk) = ck[0];
        if (p.write_v) *reinterpret_cast<uint32_t*>(dv) = cv[0];
      }
      if (sub == 0 && !hs) {
        p.k_scale[sat] = sk;
        if (p.write_v) p.v_scale[sat] = sv;
      }
    }
  } else {
    static_assert(KV == (SRC_BF16 ? 1 : 0), "a float cache takes rows of its own type");
    if (store) {
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(p.k_pool) + at) = wk;
      if (p.write_v) *reinterpret_cast<uint4*>(reinterpret_cast<char*>(p.v_pool) + at) = wv;
    }
  }
}

namespace {
template <bool SRC_BF16, int KV>
hipError_t by_dim(const WriteParams& p, int D, hipStream_t st, hipEvent_t t0, hipEvent_t t1, bool* ok) {
  const int64_t rows = (int64_t)p.T * p.Hkv;
  // Rows per 256-thread workgroup: four wavefronts of 64 / LPR rows each.
  const int64_t per_wg = 4 * (64 / (D * (SRC_BF16 ? 2 : 4) / 16));
  const dim3 grid((unsigned)((rows + per_wg - 1) / per_wg)), block(256);
  *ok = true;
  switch (D) {
    case 64: hipExtLaunchKernelGGL((pa_cache_write_kernel<SRC_BF16, KV, 64>), grid, block, 0, st, t0, t1, 0, p); break;
    case 128: hipExtLaunchKernelGGL((pa_cache_write_kernel<SRC_BF16, KV, 128>), grid, block, 0, st, t0, t1, 0, p); break;
    case 256: hipExtLaunchKernelGGL((pa_cache_write_kernel<SRC_BF16, KV, 256>), grid, block, 0, st, t0, t1, 0, p); break;
    default: *ok = false; return hipSuccess;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_cache_write(const WriteParams& p, int src_dtype, int kv_dtype, int D, hipStream_t st,
                              hipEvent_t start, hipEvent_t stop, bool* supported) {
  *supported = false;
  if (p.T == 0) {
    *supported = true;
    return hipSuccess;
  }
  const bool bf16 = src_dtype == 1;
  if (kv_dtype == 2)
    return bf16 ? by_dim<true, 2>(p, D, st, start, stop, supported) : by_dim<false, 2>(p, D, st, start, stop, supported);
  if (kv_dtype == 1 && bf16) return by_dim<true, 1>(p, D, st, start, stop, supported);
  if (kv_dtype == 0 && !bf16) return by_dim<false, 0>(p, D, st, start, stop, supported);
  return hipSuccess;
}

}  // namespace pa
