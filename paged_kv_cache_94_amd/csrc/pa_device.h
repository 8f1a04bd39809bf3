// pa_device.h -- device helpers shared by every kernel of the library:
// the per-sequence key range (which logical blocks a step loads), the pool
// address of a cache row, wavefront reductions and bf16 packing.
//
// Everything here is gfx950 (CDNA4) code: 64-lane wavefronts, DPP lane
// permutations inside a 16-lane row, ds_bpermute across rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;   // tokens per cache block
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Parameters of one launch, passed by value to every kernel.
struct Params {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* ws_acc;        // [units][splits][rows][D] unnormalised partial outputs
  float* ws_ml;         // [units][splits][rows][2] running max (log2 units) and sum
  int32_t* visits;      // optional [B][Hkv][maxb] load counters
  int32_t B, q_len, Hq, Hkv, G, rows, maxb;
  int32_t window;
  float scale_log2;     // caller's scale times log2(e): scores live in base-2 exponent units
  int32_t splits, bps;  // splits per sequence and logical blocks per split
};

// Keys a step touches for one sequence (Lab 5 handout, "Sliding Window
// Attention": skip whole out-of-window blocks). Query t sits at p0 + t.
// With a window W every query sees p - W < j <= p; the union over the step's
// queries is [lo0, L-1], lo0 being query 0's first visible key.
struct KeyRange {
  int32_t p0;      // position of query 0
  int32_t lo0;     // first key any query sees
  int32_t blk_lo;  // first logical block loaded
  int32_t blk_hi;  // last logical block loaded
};

__device__ __forceinline__ KeyRange key_range(int32_t L, int32_t q_len, int32_t window) {
  KeyRange r;
  r.p0 = L - q_len;
  int32_t lo = 0;
  if (window > 0) {
    lo = r.p0 - window + 1;
    lo = lo < 0 ? 0 : lo;
  }
  r.lo0 = lo;
  r.blk_lo = lo / kBlock;
  r.blk_hi = (L - 1) / kBlock;
  return r;
}

// A sequence length the block table can map and that holds the step's queries.
template <typename P>
__device__ __forceinline__ bool len_ok(int32_t L, const P& p) {
  return L >= p.q_len && (int64_t)L <= (int64_t)p.maxb * kBlock;
}

// First key visible to query t (window rule) -- keys below it are masked.
__device__ __forceinline__ int32_t first_key(int32_t p0, int32_t t, int32_t window) {
  if (window <= 0) return 0;
  int32_t lo = p0 + t - window + 1;
  return lo < 0 ? 0 : lo;
}

// Number of context splits that hold work for a sequence.
__device__ __forceinline__ int32_t live_splits(const KeyRange& r, int32_t bps) {
  return (r.blk_hi - r.blk_lo + bps) / bps;
}

// Byte offset of (physical block, slot, kv head) row inside a pool laid out
// [num_blocks][16][Hkv][D] (tiniestgpt notes, "PagedAttention").
__device__ __forceinline__ size_t row_offset_bytes(int32_t phys, int32_t slot, int32_t g, int32_t Hkv,
                                                   int32_t row_bytes) {
  return ((size_t)((int64_t)phys * kBlock + slot) * Hkv + g) * (size_t)row_bytes;
}

// ---- lane permutations -------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppRor8 = 0x128;       // lane i <-> i^8 inside each 16-lane row

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

// Sum over the 8 lanes of an aligned lane octet; every lane gets the total.
__device__ __forceinline__ float octet_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

// Max / sum over the 8 octets of the wavefront (lanes that agree in bits 0..2).
__device__ __forceinline__ float octets_max(float x) {
  x = fmaxf(x, dpp<kDppRor8>(x));
  x = fmaxf(x, shfl_xor(x, 16));
  x = fmaxf(x, shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float octets_sum(float x) {
  x += dpp<kDppRor8>(x);
  x += shfl_xor(x, 16);
  x += shfl_xor(x, 32);
  return x;
}

// Max / sum over the 4 lanes that agree in bits 0..3 (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float quads16_max(float x) {
  x = fmaxf(x, shfl_xor(x, 16));
  x = fmaxf(x, shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float quads16_sum(float x) {
  x += shfl_xor(x, 16);
  x += shfl_xor(x, 32);
  return x;
}

// ---- bf16 <-> f32 ------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Round two floats to bf16 (nearest even) and pack them, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace pa
