// pa_aux.hip -- the split-combine kernel and the debug gather kernel.
//
// Combine: when a sequence's key range is cut into S splits, split s leaves
// (m_s, l_s, o_s) -- its max score in base-2 units, its softmax sum and its
// unnormalised output. The merge is the online-softmax rule of the Lab 5
// handout ("Flash Attention") applied across splits:
//   M = max_s m_s,  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One workgroup per unit to merge (or per workgroup boundary of the
// flattened-list partition), all query rows of it.
#include "pa_common.h"

namespace pa {

// Flattened-list partition: one combine workgroup per unit when there are
// fewer units than workgroup boundaries (few long contexts), else one per
// boundary. Either way only the units that a boundary cuts have partials.
__host__ __device__ inline bool combine_by_unit(const Params& p) {
  return (int64_t)p.B * p.Hkv < (int64_t)p.nwg - 1;
}

// Number of combine workgroups per output row: one per unit for aligned
// splits and the piece partition; for the flattened list, one per unit or
// one per workgroup boundary, whichever is fewer.
__host__ __device__ inline int64_t combine_groups(const Params& p) {
  if (p.balanced != 1) return (int64_t)p.B * p.Hkv;
  return combine_by_unit(p) ? (int64_t)p.B * p.Hkv : (int64_t)(p.nwg > 1 ? p.nwg - 1 : 0);
}

constexpr int kCombineWaves = 4;

// Workgroups per merged unit: one per group of kCombineWaves query rows, so
// that every wavefront merges one row (rows merged one after another by a
// wavefront chain their memory round trips), unless that would launch
// thousands of workgroups (2048 units x 5 row groups measured 3 us slower
// than one workgroup per unit).
// Few units cut into many slices (the flattened list merged per unit): one
// workgroup per (unit, row), whose wavefronts each merge a quarter of the
// row's splits and fold their results through LDS, so up to 64 splits cost
// one memory round trip.
__host__ __device__ inline bool combine_wide(const Params& p) {
  return p.balanced == 1 && combine_by_unit(p);
}

__host__ __device__ inline int combine_row_groups(const Params& p) {
  if (combine_wide(p)) return p.rows;
  return combine_groups(p) >= 1024 ? 1 : (p.rows + kCombineWaves - 1) / kCombineWaves;
}

// Workgroup (grp, rg) merges one unit's partials for query rows rg*4 + w,
// rg*4 + w + 4*RG, ... (w = its wavefront, RG workgroups per unit). For a
// row, lane s holds split s's (m, l) (64 splits at a time); the row max, the
// weights 2^(m_s - M) and the weighted sum of l come from wave reductions,
// and the D dims of the row are spread over the lanes (D/64 consecutive
// floats each), so every partial row is read with one coalesced load per
// lane. The first partial rows of a chunk are requested together with its
// (m, l), so a row costs one memory round trip once its unit's bounds are
// known.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Two consecutive floats through a buffer descriptor (zeros past its end).
// The words are copied out of the vector before the bit casts: a bit cast
// of a vector element read element 0 whatever the index with this compiler.
__device__ __forceinline__ float2 buffer_load_f32x2(__amdgpu_buffer_rsrc_t r, int32_t off) {
  const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  const uint32_t a = t[0], c = t[1];
  return make_float2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, c));
}

// Merge the rows r0, r0 + step, ... of one unit when a wavefront has several
// of them (many units, few workgroups per unit). A partial row is D floats,
// D/4 lanes x 16 bytes, so one load instruction of the wavefront fetches the
// rows of SPI = 256/D splits at once, and a batch of KF splits takes
// KF/SPI instructions. The next row's (m, l) pairs and first batch are
// requested before the current row is merged, so the rows' memory round
// trips overlap. Loads go through buffer descriptors that end after the
// chunk's last split: past it they return zeros without touching memory, so
// every path issues the same loads and the compiler waits for the current
// row's alone. Splits past the first batch (units of more than KF pieces)
// are loaded as the merge reaches them. Those no-op loads still take the
// address units' time, so a unit of few pieces gets a batch just large
// enough for them (combine_rows_sized).
constexpr int kCombineMaxRowsPerWave = 8;   // rows a wavefront of the pipelined merge can take

template <typename OutT, int D, int KF>
__device__ __forceinline__ void combine_rows_pipelined(const Params& p, int32_t b, int32_t g, int64_t slot_first,
                                                       int32_t ns, int r0, int step) {
  constexpr int LPS = D / 4;      // lanes per partial row
  constexpr int SPI = 64 / LPS;   // splits per load instruction
  constexpr int NI = KF / SPI;    // load instructions per batch
  static_assert(KF % SPI == 0 && KF >= SPI, "a batch is whole load instructions");
  const int lane = __lane_id();
  const int sl = lane / LPS;                  // this lane's split within an instruction
  const int32_t loff = (lane % LPS) * 16;     // this lane's 16 bytes of a partial row
  const int32_t S = p.rows * D * 4;           // bytes from one split's partial row to the next split's
  struct Batch {
    float m, l;          // lane s: split c0 + s of the chunk
    float v[NI][4];      // instruction i: split j0 + i*SPI + sl, dims loff/4 .. +3
  };
  auto load_ml = [&](int32_t r, int32_t c0, int32_t cnt, Batch& x) __attribute__((always_inline)) {
    const auto rm = buffer_rsrc(p.ws_ml + ((size_t)(slot_first + c0) * p.rows + r) * 2, cnt * p.rows * 8);
    const float2 ml = buffer_load_f32x2(rm, lane * p.rows * 8);
    x.m = lane < cnt ? ml.x : -INFINITY;
    x.l = lane < cnt ? ml.y : 0.f;
  };
  auto load_rows = [&](int32_t r, int32_t c0, int32_t j0, int32_t cnt, Batch& x) __attribute__((always_inline)) {
    const auto rs = buffer_rsrc(p.ws_acc + ((size_t)(slot_first + c0) * p.rows + r) * D, cnt * S);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint4 t = buffer_load16<0>(rs, (j0 + i * SPI + sl) * S + loff);
      x.v[i][0] = __builtin_bit_cast(float, t.x);
      x.v[i][1] = __builtin_bit_cast(float, t.y);
      x.v[i][2] = __builtin_bit_cast(float, t.z);
      x.v[i][3] = __builtin_bit_cast(float, t.w);
    }
  };
  // Fold a chunk's (m, l) into the running max M and denominator den,
  // rescaling o; returns this lane's weight 2^(m_s - M) (0 past the chunk).
  auto fold = [&](const Batch& x, int32_t cnt, float& M, float& den, float (&o)[4]) __attribute__((always_inline)) {
    float cm = x.m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cm = fmaxf(cm, shfl_xor(cm, off));
    const float Mn = fmaxf(M, cm);
    const float Ms = Mn == -INFINITY ? 0.f : Mn;
    const float resc = fast_exp2(M - Ms);   // 0 on the first chunk (M = -inf)
    den *= resc;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] *= resc;
    M = Mn;
    const float w = lane < cnt ? fast_exp2(x.m - Ms) : 0.f;
    float dl = w * x.l;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dl += shfl_xor(dl, off);
    den += dl;
    return w;
  };
  // o += weight(split j0 + i*SPI + sl) * its partial row, over the batch.
  auto accumulate = [&](const Batch& x, float w, int32_t j0, float (&o)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float ws;
      if constexpr (SPI == 1) {
        ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j0 + i));
      } else {
        ws = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((j0 + i * SPI + sl) << 2, __builtin_bit_cast(int, w)));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += ws * x.v[i][e];
    }
  };
  auto prefetch = [&](int32_t r, Batch& x) __attribute__((always_inline)) {
    const bool live = r < p.rows;   // a row past the unit's last loads nothing
    const int32_t cnt = live ? min(64, ns) : 0;
    const int32_t rr = live ? r : 0;
    load_ml(rr, 0, cnt, x);
    load_rows(rr, 0, 0, cnt, x);
  };
  auto merge = [&](int32_t r, Batch& x) __attribute__((always_inline)) {
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    float M = -INFINITY, den = 0.f;
    const int32_t cnt0 = min(64, ns);
    const float w0 = fold(x, cnt0, M, den, o);
    accumulate(x, w0, 0, o);
    if (ns > KF) {
      for (int32_t j0 = KF; j0 < cnt0; j0 += KF) {
        load_rows(r, 0, j0, cnt0, x);
        accumulate(x, w0, j0, o);
      }
      for (int32_t c0 = 64; c0 < ns; c0 += 64) {
        const int32_t cnt = min(64, ns - c0);
        load_ml(r, c0, cnt, x);
        load_rows(r, c0, 0, cnt, x);
        const float w = fold(x, cnt, M, den, o);
        accumulate(x, w, 0, o);
        for (int32_t j0 = KF; j0 < cnt; j0 += KF) {
          load_rows(r, c0, j0, cnt, x);
          accumulate(x, w, j0, o);
        }
      }
    }
    // Sum the SPI lane groups (each holds other splits' share of the same dims).
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (SPI == 4) o[e] += shfl_xor(o[e], 16);
      if constexpr (SPI >= 2) o[e] += shfl_xor(o[e], 32);
    }
    if (sl == 0) {
      const float inv = 1.f / den;
      const int t = r / p.G;
      const int h = g * p.G + r % p.G;
      OutT* out = reinterpret_cast<OutT*>(p.out) + (((size_t)b * p.q_len + t) * p.Hq + h) * D + loff / 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(OutT) == 4) {
          out[e] = o[e] * inv;
        } else {
          out[e] = (__bf16)(o[e] * inv);
        }
      }
    }
  };
  // Fully unrolled, so the two batches stay in fixed registers (a copy from
  // one to the other would wait for its loads).
  // The scheduling barriers keep the requests in row order (the compiler
  // otherwise issues the second row's first, and the first merge then waits
  // for both).
  Batch bt[2];
  prefetch(r0, bt[0]);
  __builtin_amdgcn_sched_barrier(0);
  prefetch(r0 + step, bt[1]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kCombineMaxRowsPerWave; ++i) {
    const int r = r0 + i * step;
    if (r >= p.rows) break;
    merge(r, bt[i & 1]);
    __builtin_amdgcn_sched_barrier(0);
    prefetch(r + 2 * step, bt[i & 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Batches of one or two load instructions for units of up to 256/D or
// 512/D pieces, else of 8 splits (C5's combine: 8 splits per batch measured
// 11.9 us, 4 measured 13.2 us and 16 measured 15.7 us for every unit alike).
template <typename OutT, int D>
__device__ __forceinline__ void combine_rows_sized(const Params& p, int32_t b, int32_t g, int64_t slot_first,
                                                   int32_t ns, int r0, int step) {
  constexpr int SPI = 256 / D;
  constexpr int KF2 = 2 * SPI < 8 ? 2 * SPI : 8;
  if (ns <= SPI) combine_rows_pipelined<OutT, D, SPI>(p, b, g, slot_first, ns, r0, step);
  else if (ns <= KF2) combine_rows_pipelined<OutT, D, KF2>(p, b, g, slot_first, ns, r0, step);
  else combine_rows_pipelined<OutT, D, 8>(p, b, g, slot_first, ns, r0, step);
}

template <typename OutT, int D, bool PIPE>
__global__ void __launch_bounds__(64 * kCombineWaves) pa_combine_kernel(const Params p) {
  constexpr int PER = D / 64;   // dims per lane
  const int rgs = combine_row_groups(p);
  const int32_t grp = blockIdx.x / rgs;
  const int rg = blockIdx.x % rgs;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int32_t b, g;
  int64_t slot_first;
  int32_t ns;
  if (p.balanced == 1) {
    // Flattened list: a unit is its p.seg_items leading items, then its
    // blocks. The item prefix sums are staged in LDS so the search below
    // costs no memory round trips.
    __shared__ int32_t pre[kMaxBalancedSeqs + 1];
    for (int32_t i = threadIdx.x; i <= p.B; i += 64 * kCombineWaves) pre[i] = p.ws_prefix[i];
    __syncthreads();
    const Balanced bal = balanced_split(pre, p.B, p.Hkv, p.nwg);
    if (combine_by_unit(p)) {
      // Unit grp: its blocks are items [blk0, blk0 + nb) (after its
      // p.seg_items leading items); workgroups w0..w1 hold them and left
      // their partials in slots w + unit, unless one workgroup held them all
      // and wrote the output itself.
      b = grp / p.Hkv;
      g = grp % p.Hkv;
      const int32_t items = pre[b + 1] - pre[b];
      if (items <= p.seg_items) return;   // no blocks
      const int64_t blk0 = (int64_t)p.Hkv * pre[b] + (int64_t)g * items + p.seg_items;
      const int64_t w0 = blk0 / bal.per;
      const int64_t w1 = (blk0 + (items - p.seg_items) - 1) / bal.per;
      if (w1 == w0) return;
      slot_first = w0 + grp;
      ns = (int32_t)(w1 - w0 + 1);
    } else {
      // Boundary grp lies between workgroups grp and grp+1, at item x. The
      // unit holding x is merged here if x cuts its blocks and they start
      // inside workgroup grp (this boundary then cuts them first); workgroups
      // grp..w1 left its partials in slots w + unit.
      const int64_t x = (int64_t)(grp + 1) * bal.per;
      if (x >= bal.total) return;
      b = balanced_seq(pre, p.B, p.Hkv, x);
      const int32_t items = pre[b + 1] - pre[b];
      const int64_t base = (int64_t)p.Hkv * pre[b];
      g = (int32_t)((x - base) / items);
      const int64_t blk0 = base + (int64_t)g * items + p.seg_items;   // the unit's first block item
      if (blk0 >= x || blk0 < (int64_t)grp * bal.per) return;
      const int64_t w1 = (blk0 + (items - p.seg_items) - 1) / bal.per;   // the last workgroup with its blocks
      slot_first = grp + (int64_t)b * p.Hkv + g;
      ns = (int32_t)(w1 - grp + 1);
    }
  } else {
    b = grp / p.Hkv;
    g = grp % p.Hkv;
    const int32_t L = p.seq_lens[b];
    if (p.balanced == 2) {
      // Piece partition: unit (b, g) was cut into k pieces, numbered
      // first + g*k .. + k-1 (sequence b's first piece number and its Hkv*k
      // pieces are in the workspace table), each of which left its partial
      // in the slot of its own number; a unit of one piece was written out
      // directly. The table entries are requested with the length (both are
      // in bounds whatever the length holds).
      const int32_t kp0 = p.ws_prefix[b];
      const int32_t cnt = p.ws_prefix[p.B + b];
      if (!len_ok(L, p)) return;
      const int32_t k = cnt / p.Hkv;
      if (k <= 1) return;
      slot_first = kp0 + (int64_t)g * k;
      ns = k;
    } else {
      if (!len_ok(L, p)) return;
      const KeyRange kr = key_range(L, p.q_len, p.window);
      slot_first = (int64_t)grp * p.splits;
      ns = min(live_splits(kr, p.bps), p.splits);
    }
  }

  if constexpr (PIPE) {
    // Wave-uniform values in scalar registers (the buffer descriptors need them there).
    const int64_t sf = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(slot_first >> 32)) << 32) |
                                 (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)slot_first));
    combine_rows_sized<OutT, D>(p, b, g, sf, __builtin_amdgcn_readfirstlane(ns),
                                    __builtin_amdgcn_readfirstlane(rg * kCombineWaves + wave), rgs * kCombineWaves);
    return;
  }
  // Merge partials s0 .. s0+nsw-1 of row r into (M, den, o).
  auto merge_row = [&](int r, int32_t s0, int32_t nsw, float& M, float& den, float (&o)[PER])
      __attribute__((always_inline)) {
    const size_t slot0 = ((size_t)slot_first + s0) * p.rows + r;   // partial s0+s of this row: slot0 + s*rows
    const float* ml = p.ws_ml + slot0 * 2;
    const float* acc = p.ws_acc + slot0 * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    M = -INFINITY;
    den = 0.f;
    // Partial rows j0 .. j0+NB-1 of the chunk starting at c0 (cnt of them), NB loads in flight.
    constexpr int NB = 16;
    float v[NB][PER];
    auto load_rows = [&](int32_t c0, int32_t j0, int32_t cnt) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const bool ok = j0 + j < cnt;
        const float* src = acc + (size_t)(c0 + j0 + j) * p.rows * D;
        if constexpr (PER == 4) {
          const float4 t = ok ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
          v[j][0] = t.x; v[j][1] = t.y; v[j][2] = t.z; v[j][3] = t.w;
        } else if constexpr (PER == 2) {
          const float2 t = ok ? *reinterpret_cast<const float2*>(src) : make_float2(0.f, 0.f);
          v[j][0] = t.x; v[j][1] = t.y;
        } else {
          v[j][0] = ok ? src[0] : 0.f;
        }
      }
    };
    for (int32_t c0 = 0; c0 < nsw; c0 += 64) {
      const int32_t cnt = min(64, nsw - c0);
      const float ms = lane < cnt ? ml[(size_t)(c0 + lane) * p.rows * 2] : -INFINITY;
      const float ls = lane < cnt ? ml[(size_t)(c0 + lane) * p.rows * 2 + 1] : 0.f;
      load_rows(c0, 0, cnt);
      float cm = ms;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) cm = fmaxf(cm, shfl_xor(cm, off));
      const float Mn = fmaxf(M, cm);
      const float Ms = Mn == -INFINITY ? 0.f : Mn;
      const float resc = fast_exp2(M - Ms);   // 0 on the first chunk (M = -inf)
      den *= resc;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] *= resc;
      M = Mn;
      const float w = lane < cnt ? fast_exp2(ms - Ms) : 0.f;
      float dl = w * ls;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dl += shfl_xor(dl, off);
      den += dl;
      // Accumulate the chunk's partial rows (the first NB are already requested).
      for (int32_t j0 = 0; j0 < cnt; j0 += NB) {
        if (j0 > 0) load_rows(c0, j0, cnt);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int jj = min(j0 + j, 63);
          const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), jj));
#pragma unroll
          for (int e = 0; e < PER; ++e) o[e] += wj * v[j][e];
        }
      }
    }
  };
  auto store_row = [&](int r, const float (&o)[PER], float den) __attribute__((always_inline)) {
    const float inv = 1.f / den;
    const int t = r / p.G;
    const int h = g * p.G + r % p.G;
    OutT* out = reinterpret_cast<OutT*>(p.out) + (((size_t)b * p.q_len + t) * p.Hq + h) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if constexpr (sizeof(OutT) == 4) {
        out[e] = o[e] * inv;
      } else {
        out[e] = (__bf16)(o[e] * inv);
      }
    }
  };
  if (combine_wide(p)) {
    // Row rg; wavefront w merges the w-th quarter of the splits, then
    // wavefront 0 folds the four (max, sum, row) results with the same rule.
    __shared__ float wide_o[kCombineWaves][64 * PER];
    __shared__ float wide_md[kCombineWaves][2];
    const int32_t q = (ns + kCombineWaves - 1) / kCombineWaves;
    const int32_t s0 = min(ns, wave * q);
    float o[PER], M, den;
    merge_row(rg, s0, min(ns - s0, q), M, den, o);
#pragma unroll
    for (int e = 0; e < PER; ++e) wide_o[wave][lane * PER + e] = o[e];
    if (lane == 0) {
      wide_md[wave][0] = M;
      wide_md[wave][1] = den;
    }
    __syncthreads();
    if (wave != 0) return;
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kCombineWaves; ++w) Mx = fmaxf(Mx, wide_md[w][0]);
    const float Ms = Mx == -INFINITY ? 0.f : Mx;
    float dsum = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kCombineWaves; ++w) {
      const float a = fast_exp2(wide_md[w][0] - Ms);   // 0 for a quarter with no splits
      dsum += a * wide_md[w][1];
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] += a * wide_o[w][lane * PER + e];
    }
    store_row(rg, o, dsum);
    return;
  }
  for (int r = rg * kCombineWaves + wave; r < p.rows; r += rgs * kCombineWaves) {
    float o[PER], M, den;
    merge_row(r, 0, ns, M, den, o);
    store_row(r, o, den);
  }
}

// Debug gather: copy the cache rows the attention kernels would load, in
// logical key order, through the same key_range / table_entry helpers and the
// same pool-addressing functions (tile_offset_bytes, token_stride_bytes) as the
// attention kernels and the append.
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
  const int32_t phys = p.block_table[(size_t)b * p.maxb + table_entry(p, j / kBlock)];
  const int32_t words = row_bytes / 4;
  for (int32_t g = 0; g < p.Hkv; ++g) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(pool + tile_offset_bytes(phys, g, p.Hkv, row_bytes) +
                                                               (size_t)(j % kBlock) * token_stride_bytes(p.Hkv, row_bytes));
    uint32_t* out = reinterpret_cast<uint32_t*>(dst + (((size_t)b * dst_tokens + w) * p.Hkv + g) * (size_t)row_bytes);
    for (int32_t k = lane; k < words; k += 64) out[k] = src[k];
  }
}

template <typename OutT, int D>
void launch_combine_as(const Params& p, dim3 grid, dim3 block, hipStream_t st) {
  // The pipelined instance when a wavefront merges more than one row (and
  // at most kCombineMaxRowsPerWave of them: 32 query rows at most).
  const int step = combine_row_groups(p) * kCombineWaves;
  if (p.rows > step && p.rows <= kCombineMaxRowsPerWave * step)
    hipLaunchKernelGGL((pa_combine_kernel<OutT, D, true>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((pa_combine_kernel<OutT, D, false>), grid, block, 0, st, p);
}

hipError_t launch_combine(const Params& p, int q_dtype, int D, hipStream_t st) {
  const int64_t groups = combine_groups(p) * combine_row_groups(p);
  if (groups == 0) return hipSuccess;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)groups), block(64 * kCombineWaves);
  const bool bf16 = q_dtype == 1;
  switch (D) {
    case 64:
      if (bf16) launch_combine_as<__bf16, 64>(p, grid, block, st);
      else launch_combine_as<float, 64>(p, grid, block, st);
      break;
    case 128:
      if (bf16) launch_combine_as<__bf16, 128>(p, grid, block, st);
      else launch_combine_as<float, 128>(p, grid, block, st);
      break;
    case 256:
      if (bf16) launch_combine_as<__bf16, 256>(p, grid, block, st);
      else launch_combine_as<float, 256>(p, grid, block, st);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__device__ __forceinline__ int32_t scale_bits(float ks, float vs) {
  int32_t bits = 0;
  if (!__builtin_isfinite(ks) || !__builtin_isfinite(vs)) bits |= 8;
  if (__builtin_fabsf(vs) >= 255.f) bits |= 16;
  return bits;
}

// Precondition check: one workgroup per sequence. Lengths: q_len <= L <=
// max_seq_len (and, linear tables, L <= maxb * 16). Table: every entry the
// step reads (logical blocks [blk_lo, blk_hi] through table_entry) lies in
// [0, num_blocks). Int8 scales (when check_scales): the K and V scales of
// every key some query sees (positions lo0 .. L-1, in a valid block) are
// finite, and the V scales are below 255 in magnitude. Bits as in pa.h: 1
// short, 2 long, 4 bad block, 8 non-finite scale, 16 value scale >= 255.
// queue_header (non-null when the call would use the piece queue): its
// "next" and "done" counters must all be zero; bit 32 in status[0] if not.
__global__ void __launch_bounds__(256) pa_validate_kernel(const Params p, int32_t num_blocks, int32_t max_seq_len,
                                                          int32_t check_scales, const int32_t* queue_header,
                                                          int32_t* status) {
  __shared__ int32_t bits;
  const int32_t b = blockIdx.x;
  if (threadIdx.x == 0) bits = 0;
  __syncthreads();
  const int32_t L = p.seq_lens[b];
  int32_t mine = 0;
  if (threadIdx.x == 0) {
    if (L < p.q_len) mine |= 1;
    if (L > max_seq_len || (p.ring == 0 && (int64_t)L > (int64_t)p.maxb * kBlock)) mine |= 2;
  }
  if (L >= 1) {
    const KeyRange kr = key_range(L, min(p.q_len, L), p.window);
    // Entries read for blocks blk_lo .. blk_hi; a length the table cannot hold is clamped to the row.
    const int32_t hi = p.ring > 0 ? kr.blk_hi : min(kr.blk_hi, p.maxb - 1);
    for (int32_t i = kr.blk_lo + (int32_t)threadIdx.x; i <= hi; i += blockDim.x) {
      const int32_t e = p.block_table[(size_t)b * p.maxb + table_entry(p, i)];
      if (e < 0 || e >= num_blocks) mine |= 4;
    }
    if (check_scales) {
      const int32_t key_end = p.ring > 0 ? L : min(L, p.maxb * kBlock);   // keys [lo0, key_end)
      const int32_t nkeys = key_end - kr.lo0;
      const int32_t H = p.Hkv;
      if (p.head_scales) {
        for (int32_t h = threadIdx.x; h < (nkeys > 0 ? H : 0); h += blockDim.x)
          mine |= scale_bits(p.k_scale[h], p.v_scale[h]);
      } else {
        for (int64_t f = threadIdx.x; f < (int64_t)max(nkeys, 0) * H; f += blockDim.x) {
          const int32_t j = kr.lo0 + (int32_t)(f / H), h = (int32_t)(f % H);
          const int32_t e = p.block_table[(size_t)b * p.maxb + table_entry(p, j / kBlock)];
          if (e < 0 || e >= num_blocks) continue;                        // already flagged as a bad block
          const size_t at = scale_tile_index(e, h, H) + j % kBlock;
          mine |= scale_bits(p.k_scale[at], p.v_scale[at]);
        }
      }
    }
  }
  if (mine) atomicOr(&bits, mine);
  if (queue_header && b == 0 && threadIdx.x < 2 * kQueueShards && queue_header[threadIdx.x * kQueueStride] != 0)
    atomicOr(status, 32);
  __syncthreads();
  if (threadIdx.x == 0) {
    status[1 + b] = bits;
    if (bits) atomicOr(status, bits);
  }
}

hipError_t launch_validate(const Params& p, int32_t num_blocks, int32_t max_seq_len, int check_scales,
                           const int32_t* queue_header, int32_t* status, hipStream_t st) {
  if (p.B == 0) return hipSuccess;
  hipLaunchKernelGGL(pa_validate_kernel, dim3((unsigned)p.B), dim3(256), 0, st, p, num_blocks, max_seq_len,
                     (int32_t)check_scales, queue_header, status);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) pa_zero_words_kernel(int32_t* p, int32_t n) {
  for (int32_t i = threadIdx.x; i < n; i += 256) p[i] = 0;
}

hipError_t launch_zero_words(int32_t* p, int32_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(pa_zero_words_kernel, dim3(1), dim3(256), 0, st, p, n);
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
