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
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
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
  int32_t splits, bps;  // aligned mode: splits per sequence and logical blocks per split
  int32_t balanced;     // 0: aligned splits; 1: flattened-list partition; 2: piece partition
  int32_t nwg;          // modes 1 and 2: workgroups of the launch
  int32_t seg_items;    // mode 1: items each non-empty unit counts beyond its blocks
  int32_t* ws_prefix;   // mode 1: [B+1] block prefix sums; mode 2: [B] first piece numbers, [B] piece counts (workgroup 0 writes)
  int32_t pieces;       // mode 2: pieces the partition aims for (nwg, or more when they are handed out)
  int32_t* ws_queue;    // mode 2, non-null: hand pieces out through this [2] counter pair (zero between calls)
  int32_t ring;         // > 0: each table row is a ring of this many entries (logical block i -> i mod ring)
  int32_t head_scales;  // int8: 1 -> k_scale / v_scale hold one scale per KV head
  uint64_t* stamps;     // builds with PA_STAMPS only: [grid][kStampSlots] phase timestamps, or null
};

// ---- phase stamps (a diagnostic build compiled with -DPA_STAMPS) ------------
//
// Thread 0 of a workgroup records the constant-rate real-time counter
// (s_memrealtime) at the phases of its work: slot 0 entry, 1 partition
// known, 2 exit, 3 the number of segments, then five per segment s (from
// slot 4 + 5s): segment start, first block consumed, block loop done,
// output or partial written, and the segment's block count (a count, not a
// time). The release build compiles all of it away.
constexpr int kStampSlots = 64;
constexpr int kStampPerSeg = 5;
constexpr int kStampSegments = (kStampSlots - 4) / kStampPerSeg;
enum { kStampEntry = 0, kStampPartition = 1, kStampExit = 2, kStampCount = 3, kStampSeg0 = 4 };

template <typename P>
__device__ __forceinline__ void stamp(const P& p, int slot) {
#ifdef PA_STAMPS
  if (p.stamps && threadIdx.x == 0 && slot < kStampSlots)
    p.stamps[(size_t)blockIdx.x * kStampSlots + slot] = __builtin_amdgcn_s_memrealtime();
#else
  (void)p;
  (void)slot;
#endif
}

template <typename P>
__device__ __forceinline__ void stamp_value(const P& p, int slot, uint64_t v) {
#ifdef PA_STAMPS
  if (p.stamps && threadIdx.x == 0 && slot < kStampSlots) p.stamps[(size_t)blockIdx.x * kStampSlots + slot] = v;
#else
  (void)p;
  (void)slot;
  (void)v;
#endif
}

// Table entry that holds logical block i (Lab 5 handout, "Ring KV Cache": in
// a ring of R blocks position t lives in slot t mod 16R, i.e. block i mod R).
template <typename P>
__device__ __forceinline__ int32_t table_entry(const P& p, int32_t i) {
  return p.ring > 0 ? i % p.ring : i;
}

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
  return L >= p.q_len && (p.ring > 0 || (int64_t)L <= (int64_t)p.maxb * kBlock);
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

// Logical blocks a step loads for one sequence (0 for a length the table cannot map).
template <typename P>
__device__ __forceinline__ int32_t seq_blocks(int32_t L, const P& p) {
  if (!len_ok(L, p)) return 0;
  const KeyRange r = key_range(L, p.q_len, p.window);
  return r.blk_hi - r.blk_lo + 1;
}

// Work-balanced partition. The work list is every (unit, block) pair, units
// u = b*Hkv + g in order, unit u's blocks contiguous: unit (b, g) starts at
// item Hkv*pre[b] + g*n_b where pre[b] = n_0 + ... + n_{b-1}. Workgroup w of
// nwg takes items [w*per, min(T, (w+1)*per)), per = ceil(T / nwg), so every
// workgroup streams the same number of blocks whatever the lengths are.
struct Balanced {
  int64_t total;  // T
  int64_t per;    // items per workgroup
};

__device__ __forceinline__ Balanced balanced_split(const int32_t* pre, int32_t B, int32_t Hkv, int32_t nwg) {
  Balanced s;
  s.total = (int64_t)Hkv * pre[B];
  s.per = (s.total + nwg - 1) / nwg;
  if (s.per < 1) s.per = 1;
  return s;
}

// The sequence whose units hold item x (0 <= x < T): the largest b with Hkv*pre[b] <= x.
__device__ __forceinline__ int32_t balanced_seq(const int32_t* pre, int32_t B, int32_t Hkv, int64_t x) {
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if ((int64_t)Hkv * pre[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP: shifts by
// 1, 2, 4 and 8 lanes inside each 16-lane row, then the last lane of a row
// is broadcast into the rows after it (row_bcast:15 into rows 1 and 3,
// row_bcast:31 into rows 2 and 3). A lane whose source falls outside its
// row, or whose row is masked off, adds 0. Every step is a VALU operation;
// nothing goes through LDS.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int32_t dpp_i32(int32_t x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ int32_t wave_scan_incl(int32_t x) {
  x += dpp_i32<0x111>(x);          // row_shr:1
  x += dpp_i32<0x112>(x);          // row_shr:2
  x += dpp_i32<0x114>(x);          // row_shr:4
  x += dpp_i32<0x118>(x);          // row_shr:8
  x += dpp_i32<0x142, 0xA>(x);     // row_bcast:15
  x += dpp_i32<0x143, 0xC>(x);     // row_bcast:31
  return x;
}
// Sum over the wavefront, the same value in every lane.
__device__ __forceinline__ int32_t wave_sum(int32_t x) {
  return __builtin_amdgcn_readlane(wave_scan_incl(x), 63);
}
// 64-bit sum of per-lane 32-bit values: the low and high 16-bit halves are
// summed separately (each total stays below 2^22 for 64 lanes).
__device__ __forceinline__ int64_t wave_sum_wide(int32_t x) {
  const uint32_t u = (uint32_t)x;
  const int64_t lo = wave_sum((int32_t)(u & 0xFFFFu));
  const int64_t hi = wave_sum((int32_t)(u >> 16));
  return lo + (hi << 16);
}

// Maximum over the wavefront of non-negative values (the same DPP steps as
// the scan; a lane whose source falls outside its row takes 0).
__device__ __forceinline__ int32_t wave_max_nonneg(int32_t x) {
  x = max(x, dpp_i32<0x111>(x));
  x = max(x, dpp_i32<0x112>(x));
  x = max(x, dpp_i32<0x114>(x));
  x = max(x, dpp_i32<0x118>(x));
  x = max(x, dpp_i32<0x142, 0xA>(x));
  x = max(x, dpp_i32<0x143, 0xC>(x));
  return __builtin_amdgcn_readlane(x, 63);
}

// Inclusive scans (wave_scans) or sums (wave_sums, the same value in every
// lane) of N values at once: each DPP step is applied to all N before the
// next, so no step waits on the result of the one before it.
template <int N>
__device__ __forceinline__ void wave_scans(int32_t (&x)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_i32<0x111>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_i32<0x112>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_i32<0x114>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_i32<0x118>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_i32<0x142, 0xA>(x[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] += dpp_i32<0x143, 0xC>(x[j]);
}
template <int N>
__device__ __forceinline__ void wave_sums(int32_t (&x)[N]) {
  wave_scans(x);
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] = __builtin_amdgcn_readlane(x[j], 63);
}

// 1/d to within a few ulps: the hardware estimate and two Newton steps.
// (The IEEE division sequence reads and writes VCC, which serializes
// neighbouring divisions; these chains overlap.)
__device__ __forceinline__ double recip(double d) {
  double r = __builtin_amdgcn_rcp(d);
  r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
  return __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
}

// ceil(n / d) for 0 <= n < 2^31 and 1 <= d < 2^31 by one double fma: the
// quotient (n + d - 1/2) / d lies at least 1/(2d) from every integer, and
// the error of the fma with an inverse good to a few ulps stays below
// (n/d + 1) * 2^-48, far smaller, so truncating it gives
// floor((n + d - 1) / d) exactly. The divisor's two constants are computed
// once for many numerators.
struct CeilDiv {
  double inv, bias;
};
__device__ __forceinline__ CeilDiv ceil_div_by(int32_t d) {
  const double inv = recip((double)d);
  return {inv, ((double)d - 0.5) * inv};
}
__device__ __forceinline__ int32_t ceil_div(double n, const CeilDiv& c) {
  return (int32_t)__builtin_fma(n, c.inv, c.bias);
}

// pre[0..B] = prefix sums of the list items per unit over the batch, and
// blo[0..B) = the first logical block each sequence loads, computed by wave 0
// of the workgroup (64 sequences per step, DPP scan); the caller synchronises
// the workgroup before reading them. A unit of sequence b counts its n_b
// blocks plus p.seg_items items ahead of them (none for a unit without
// blocks): the cost of one more segment in a workgroup's share.
template <typename P>
__device__ __forceinline__ void block_prefix(const P& p, int32_t* pre, int32_t* blo) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  if (lane == 0) pre[0] = 0;
  int32_t carry = 0;
  for (int32_t base = 0; base < p.B; base += 64) {
    const int32_t b = base + lane;
    const int32_t L = b < p.B ? p.seq_lens[b] : 0;
    const int32_t nb = b < p.B ? seq_blocks(L, p) : 0;
    const int32_t v = wave_scan_incl(nb > 0 ? nb + p.seg_items : 0);
    if (b < p.B) {
      pre[b + 1] = carry + v;
      blo[b] = key_range(L, p.q_len, p.window).blk_lo;
    }
    carry += __builtin_amdgcn_readlane(v, 63);
  }
}

// Piece partition. Unit (b, g) with n_b blocks is cut into
// k_b = ceil(n_b / per) pieces of ceil(n_b / k_b) blocks; `per` is the
// smallest count for which all pieces number at most p.pieces. With
// p.pieces == nwg each workgroup owns the piece of its own index (asked for
// through the launch-plan tuning); with more, workgroups take pieces from a
// queue until none are left, which evens out the time workgroups take for the
// same number of blocks.
//
// With by_size, pieces are numbered largest first, so that the last ones a
// queue hands out are the shortest and workgroups run out of work at nearly
// the same time. Sequences fall into kPieceClasses classes by the size c_b of
// their pieces, class floor(kPieceClasses * (per - c_b) / per) (class 0 the
// largest); the order is by class, then by b, then by (g, piece), so a unit's
// pieces stay consecutive. Without it (one piece per workgroup, where the
// order changes nothing) the order is by (b, g, piece). A sequence with no
// blocks has no pieces: its rank r has kp[r] == kp[r + 1] wherever it falls.
//
// Wave 0 fills nbs[b] = n_b, blo[b] = the first logical block sequence b
// loads, ord[r] = the sequence at rank r, and kp[0..B] = Hkv * (k_ord[0] + ...
// + k_ord[r-1]), the number of the first piece of rank r; the caller
// synchronises the workgroup before reading them. `per` is at least min_per
// (enough blocks for every wavefront of the workgroup). Needs p.pieces >=
// B * Hkv (checked on the host), which bounds the search below.
constexpr int kMaxPieceSeqs = 512;   // batch limit of the piece partition (its per-sequence tables live in LDS)
constexpr int kPieceClasses = 8;

template <typename P>
__device__ __forceinline__ void piece_prefix(const P& p, int32_t* nbs, int32_t* blo, int32_t* ord, int32_t* kp,
                                             int32_t min_per, bool by_size) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  // Lane l holds sequences l, l + 64, ... in registers: chunk i is b = 64 i + l.
  // Every length is requested at once (one memory round trip); lanes past the
  // batch count no blocks.
  constexpr int kChunks = kMaxPieceSeqs / 64;
  const int32_t nch = (p.B + 63) >> 6;
  int32_t L[kChunks], nb[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int32_t b = i * 64 + lane;
    L[i] = i < nch && b < p.B ? p.seq_lens[b] : 0;
  }
  int32_t lane_blocks = 0;
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    nb[i] = 0;
    if (i >= nch) continue;
    const int32_t b = i * 64 + lane;
    if (b < p.B) {
      nb[i] = seq_blocks(L[i], p);
      nbs[b] = nb[i];
      blo[b] = key_range(L[i], p.q_len, p.window).blk_lo;
    }
    lane_blocks += nb[i];   // at most 8 sequences of < 2^27 blocks
  }
  const int64_t total = wave_sum_wide(lane_blocks) * p.Hkv;
  double nbd[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) nbd[i] = (double)nb[i];
  // Bounds of the smallest fitting count: it is at least total / target, and
  // ceil(total / (target - units)) fits (pieces(per) <= total / per + units),
  // as does the longest unit (one piece each). The quotients are taken in
  // double (relative error far below 2^-40 for quotients below 2^31):
  // truncated, the first is at most its ceiling; the second is widened by
  // two, which keeps both bounds valid.
  const int64_t target = p.pieces;
  const int64_t units = (int64_t)p.B * p.Hkv;
  const int64_t spare = target - units;
  const double totd = (double)total;
  int32_t lo = (int32_t)fmin(totd * recip((double)target), 1073741824.0);
  int32_t hi;
  if (spare > 0) {
    hi = (int32_t)fmin(totd * recip((double)spare) + 2.0, 1073741824.0);
  } else {
    int32_t m = 0;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) m = nb[i] > m ? nb[i] : m;
    hi = wave_max_nonneg(m);
  }
  if (lo < min_per) lo = min_per;
  if (hi < lo) hi = lo;   // pieces() only falls as per grows
  // Search for the smallest fitting count in [lo, hi]. Each pass counts the
  // pieces (sum over units of ceil(n / x)) for kCand candidates x at once,
  // their divisions and wavefront sums side by side. pieces() only falls as
  // x grows, so each candidate moves lo or hi. The first pass tries the
  // counts around the one that fits if every unit's last piece is half full
  // (total / (target - units / 2)), which usually holds the answer; later
  // ones spread the candidates evenly over [lo, hi). B <= kMaxPieceSeqs
  // keeps every count far below 2^31.
  constexpr int kCand = 8;
  const int32_t guess = (int32_t)fmin(totd * recip((double)(target - units / 2)) + 1.0, 1073741824.0);
  for (bool first = true; lo < hi; first = false) {
    int32_t xs[kCand], cnt[kCand];
    CeilDiv dv[kCand];
#pragma unroll
    for (int c = 0; c < kCand; ++c) {
      const int32_t x = first ? guess - kCand / 2 + c : lo + (int32_t)((int64_t)(hi - lo) * (c + 1) / (kCand + 1));
      xs[c] = x < lo ? lo : (x > hi - 1 ? hi - 1 : x);
      dv[c] = ceil_div_by(xs[c]);
      cnt[c] = 0;
    }
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      if (i < nch) {
#pragma unroll
        for (int c = 0; c < kCand; ++c) cnt[c] += ceil_div(nbd[i], dv[c]);
      }
    wave_sums(cnt);
#pragma unroll
    for (int c = 0; c < kCand; ++c) {
      if ((int64_t)cnt[c] * p.Hkv <= target) hi = xs[c] < hi ? xs[c] : hi;
      else lo = xs[c] + 1 > lo ? xs[c] + 1 : lo;
    }
  }
  const int32_t per = lo;
  const CeilDiv by_per = ceil_div_by(per);
  if (!by_size) {
    if (lane == 0) kp[0] = 0;
    int32_t carry = 0;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      if (i >= nch) break;
      const int32_t b = i * 64 + lane;
      const int32_t v = wave_scan_incl(ceil_div(nbd[i], by_per) * p.Hkv);
      if (b < p.B) {
        ord[b] = b;
        kp[b + 1] = carry + v;
      }
      carry += __builtin_amdgcn_readlane(v, 63);
    }
    return;
  }
  // Class of each sequence (per and c_b are below 2^27, so 8 * per fits):
  // class >= j exactly when 8c <= (8 - j) per. Its rank inside its class is
  // the sequences of that class in earlier chunks plus those on lower lanes
  // of its own chunk, counted in 8-bit fields (at most 64 per chunk), four
  // classes to a word; the scans of all chunks run side by side.
  static_assert(kPieceClasses == 8, "classes are counted in 8-bit fields of two words");
  int32_t cls[kChunks], kk[kChunks], in[2 * kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    cls[i] = kk[i] = in[2 * i] = in[2 * i + 1] = 0;
    if (i >= nch) continue;
    const int32_t k = ceil_div(nbd[i], by_per);
    const int32_t c = k > 0 ? (nb[i] + k - 1) / k : 0;
    int32_t q = 0;
#pragma unroll
    for (int j = 1; j < kPieceClasses; ++j) q += 8 * c <= (8 - j) * per ? 1 : 0;
    const uint32_t one = i * 64 + lane < p.B ? 1u << (8 * (q & 3)) : 0u;
    cls[i] = q;
    kk[i] = k * p.Hkv;
    in[2 * i] = (int32_t)(q < 4 ? one : 0u);
    in[2 * i + 1] = (int32_t)(q < 4 ? 0u : one);
  }
  wave_scans(in);
  // Class starts (sequences per class: the fields of every chunk's last lane).
  int32_t off[kPieceClasses] = {};
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    if (i >= nch) break;
    const uint32_t ch_lo = (uint32_t)__builtin_amdgcn_readlane(in[2 * i], 63);
    const uint32_t ch_hi = (uint32_t)__builtin_amdgcn_readlane(in[2 * i + 1], 63);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      off[j + 1] += (ch_lo >> (8 * j)) & 0xFF;
      if (j < 3) off[j + 5] += (ch_hi >> (8 * j)) & 0xFF;
    }
  }
#pragma unroll
  for (int j = 1; j < kPieceClasses; ++j) off[j] += off[j - 1];
  // Each sequence to its rank, its piece count beside it (summed in place
  // below); off[] advances past each chunk's members of every class.
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    if (i >= nch) break;
    const int32_t b = i * 64 + lane;
    const int32_t q = cls[i];
    int32_t start = off[0];
#pragma unroll
    for (int j = 1; j < kPieceClasses; ++j) start = q == j ? off[j] : start;
    const uint32_t w = (uint32_t)(q < 4 ? in[2 * i] : in[2 * i + 1]);
    const int32_t r = start + (int32_t)((w >> (8 * (q & 3))) & 0xFF) - 1;
    if (b < p.B) {
      ord[r] = b;
      kp[r + 1] = kk[i];
    }
    const uint32_t ch_lo = (uint32_t)__builtin_amdgcn_readlane(in[2 * i], 63);
    const uint32_t ch_hi = (uint32_t)__builtin_amdgcn_readlane(in[2 * i + 1], 63);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      off[j] += (ch_lo >> (8 * j)) & 0xFF;
      off[4 + j] += (ch_hi >> (8 * j)) & 0xFF;
    }
  }
  // The counts were written by other lanes of this wavefront.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int32_t v[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) v[i] = i < nch && i * 64 + lane < p.B ? kp[i * 64 + lane + 1] : 0;
  wave_scans(v);
  int32_t carry = 0;
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    if (i >= nch) break;
    const int32_t r = i * 64 + lane;
    if (r < p.B) kp[r + 1] = carry + v[i];   // each lane rewrites only what it read
    carry += __builtin_amdgcn_readlane(v[i], 63);
  }
  if (lane == 0) kp[0] = 0;
}

// The piece of work a workgroup owns in the piece partition.
struct Piece {
  int32_t b, g;
  int32_t k;       // pieces of this unit (1: the workgroup writes the output itself)
  int32_t first;   // offset of its first block inside the unit's key range
  int32_t count;   // blocks it streams (>= 1)
};

// Piece w (< kp[B]) of the list: the sequence of the largest rank r with
// kp[r] <= w owns it (ranks without pieces have kp[r] == kp[r + 1] and are
// passed over).
__device__ __forceinline__ Piece piece_of(const int32_t* nbs, const int32_t* ord, const int32_t* kp, int32_t B,
                                          int32_t Hkv, int32_t w) {
  int32_t lo = 0, hi = B - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (kp[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  Piece pc;
  pc.b = ord[lo];
  pc.k = (kp[lo + 1] - kp[lo]) / Hkv;
  const int32_t r = w - kp[lo];
  pc.g = r / pc.k;
  const int32_t i = r % pc.k;
  const int32_t nb = nbs[pc.b];
  const int32_t len = (nb + pc.k - 1) / pc.k;   // (k-1)*len < nb: every piece is non-empty
  pc.first = i * len;
  pc.count = min(nb, pc.first + len) - pc.first;
  return pc;
}

// ---- pool addressing (tiniestgpt notes, "PagedAttention": the pool is
// [num_blocks][16][Hkv][D], a block-table entry names its first dimension) --
//
// Every kernel that reads or writes the cache, and the debug gather, forms
// its addresses from these three functions and nothing else, so the gather's
// bit-exact comparison with the oracle checks the attention kernels'
// addressing too.

// Bytes from one cached row (token) of a (block, KV head) tile to the next.
__device__ __forceinline__ int32_t token_stride_bytes(int32_t Hkv, int32_t row_bytes) { return Hkv * row_bytes; }

// Byte offset of the (physical block, KV head) tile: its slot-0 row. Rows of
// the tile follow at token_stride_bytes apart.
__device__ __forceinline__ size_t tile_offset_bytes(int32_t phys, int32_t g, int32_t Hkv, int32_t row_bytes) {
  return ((size_t)phys * kBlock * (size_t)Hkv + (size_t)g) * (size_t)row_bytes;
}

// Byte offset of the (physical block, slot, KV head) row.
__device__ __forceinline__ size_t row_offset_bytes(int32_t phys, int32_t slot, int32_t g, int32_t Hkv,
                                                   int32_t row_bytes) {
  return tile_offset_bytes(phys, g, Hkv, row_bytes) + (size_t)slot * (size_t)token_stride_bytes(Hkv, row_bytes);
}

// Index of the first of a (physical block, KV head) tile's 16 per-token int8
// scales in a [num_blocks][Hkv][16] scale array (one 64-byte run per tile).
__device__ __forceinline__ size_t scale_tile_index(int32_t phys, int32_t g, int32_t Hkv) {
  return ((size_t)phys * (size_t)Hkv + (size_t)g) * kBlock;
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

constexpr int kDppRowMirror = 0x140;  // lane i <-> 15-i inside each 16-lane row

// Sum over an aligned group of N (8 or 16) lanes; every lane of the group gets the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "lane groups of 8 or 16");
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  if constexpr (N == 16) x += dpp<kDppRowMirror>(x);
  return x;
}

// Max / sum across the 64/N groups of N lanes (lanes that agree in the low log2(N) bits).
template <int N>
__device__ __forceinline__ float across_groups_max(float x) {
  if constexpr (N == 8) x = fmaxf(x, dpp<kDppRor8>(x));
  x = fmaxf(x, shfl_xor(x, 16));
  x = fmaxf(x, shfl_xor(x, 32));
  return x;
}
template <int N>
__device__ __forceinline__ float across_groups_sum(float x) {
  if constexpr (N == 8) x += dpp<kDppRor8>(x);
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

// Online softmax with a lazily moved reference max: a row's reference moves
// only when a new score exceeds it by more than this many log2 units, so the
// accumulator is rescaled rarely; exp2 of (score - reference) stays below
// 2^kRescaleSlack.
constexpr float kRescaleSlack = 8.f;

// Copy a freshly loaded value into a register written by a VALU move (a DPP
// identity permutation). The wait for the load happens once, here; later
// reads of the copy inside a software-pipelined loop then never make the
// compiler wait on vector-memory loads issued after it (which it otherwise
// does conservatively across the loop's back edge).
__device__ __forceinline__ int32_t settle(int32_t v) {
  return __builtin_amdgcn_mov_dpp(v, 0xE4, 0xF, 0xF, true);   // quad_perm [0,1,2,3]
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over `bytes` bytes at `base` (gfx9 family: stride 0,
// descriptor word 3 = 0x00020000). A load at an offset past `bytes` returns 0
// and touches no memory, so a descriptor of zero bytes turns a load into a
// no-op that still counts as an issued load: a software pipeline can then
// issue the same loads on every path, which keeps the compiler's wait counts
// exact (a load issued on only some paths makes it wait for everything).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
constexpr int kCacheNonTemporal = 2;   // buffer cache policy: NT (data read once)

// voff: per-lane byte offset; soff: wave-uniform byte offset (a scalar register).
template <int CPOL = kCacheNonTemporal>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int32_t voff, int32_t soff = 0) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CPOL);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, int32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Mark a loaded value as used. A pipeline's last prefetch is dead once the
// loop exits; without a use on the exit path the compiler moves those loads
// behind the exit branch, which makes them conditional again (and its wait
// counts conservative).
__device__ __forceinline__ void keep_loaded(const uint4& v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  asm volatile("" ::"v"(x));
}
__device__ __forceinline__ void keep_loaded(float v) { asm volatile("" ::"v"(v)); }

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// ---- matrix-core operand helpers ---------------------------------------------

__device__ __forceinline__ uint32_t i8pair_to_bf16(uint32_t w, int byte0) {
  const float a = (float)(int32_t)(int8_t)(w >> (8 * byte0));
  const float b = (float)(int32_t)(int8_t)(w >> (8 * byte0 + 8));
  return pack_bf16(a, b);
}

// 16 int8 codes widened to 16 bf16 values (exact for |code| <= 127), in order.
__device__ __forceinline__ void i8x16_to_bf16(const uint4& w, uint4& lo, uint4& hi) {
  lo = make_uint4(i8pair_to_bf16(w.x, 0), i8pair_to_bf16(w.x, 2), i8pair_to_bf16(w.y, 0), i8pair_to_bf16(w.y, 2));
  hi = make_uint4(i8pair_to_bf16(w.z, 0), i8pair_to_bf16(w.z, 2), i8pair_to_bf16(w.w, 0), i8pair_to_bf16(w.w, 2));
}

// 16 int8 codes as 16 f16 values, exactly: with the sign bit flipped a code
// c reads as the unsigned byte c + 128; placed under the high byte 0x64 (the
// f16 pattern of 1024, whose spacing is 1) it reads as 1024 + c + 128, and a
// packed f16 subtraction of 1152 leaves c (every value is an integer below
// 2048, so nothing rounds). Five instructions per four codes.
typedef _Float16 f16x2h __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t i8pair_to_f16(uint32_t flipped, uint32_t sel) {
  const uint32_t bits = __builtin_amdgcn_perm(flipped, 0x64646464u, sel);
  const f16x2h v = __builtin_bit_cast(f16x2h, bits) - f16x2h{(_Float16)1152.f, (_Float16)1152.f};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void i8x16_to_f16_exact(const uint4& w, uint4& lo, uint4& hi) {
  // v_perm_b32 selectors: bytes 4..7 are the codes, bytes 0..3 the constant 0x64.
  constexpr uint32_t kLow = 0x00050004u, kHigh = 0x00070006u;
  const uint32_t x0 = w.x ^ 0x80808080u, x1 = w.y ^ 0x80808080u, x2 = w.z ^ 0x80808080u, x3 = w.w ^ 0x80808080u;
  lo = make_uint4(i8pair_to_f16(x0, kLow), i8pair_to_f16(x0, kHigh), i8pair_to_f16(x1, kLow), i8pair_to_f16(x1, kHigh));
  hi = make_uint4(i8pair_to_f16(x2, kLow), i8pair_to_f16(x2, kHigh), i8pair_to_f16(x3, kLow), i8pair_to_f16(x3, kHigh));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// ds_read_b64_tr_b16 at LDS address p: in each 16-lane group, lanes 4k..4k+3
// address row k (16 consecutive bf16) and lane i receives element i of the
// four rows -- a 4 x 16 bf16 tile read transposed.
__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<lds_char*>((const lds_char*)p)));
  return __builtin_bit_cast(uint2, v);
}

// 16-byte load with the non-temporal hint: cache rows are read exactly once
// per step, so they should not displace anything in L2 / the Infinity Cache.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace pa
