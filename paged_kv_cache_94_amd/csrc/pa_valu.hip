// pa_valu.hip -- vector-ALU paged decode attention for small query groups
// (rows = (Hq/Hkv) * q_len <= 512 / D) over fp32 or bf16 caches.
//
// One workgroup owns one (sequence, KV head, context split); its NW
// wavefronts take the split's logical blocks round-robin. Per block a
// wavefront reads the 16 cached rows of its KV head straight from HBM into
// registers: a group of LPT lanes (16 for rows of 256 bytes or more, else 8)
// covers LPT*16 bytes of one row with 16-byte loads, so every load
// instruction moves whole 128-byte lines of 64/LPT rows. The K rows are used
// for every query row of the group from registers (grouped-query attention,
// Lab 5 handout: heads share K/V without repeating them). Loads of the next
// block are issued before the current one is consumed (two register
// buffers per wavefront).
//
// Scores: each lane dots its slice of the row with the matching slice of
// every query row (bf16 pairs through v_dot2, fp32 through FMA), then a DPP
// sum over the lane group (quad_perm x2, half-row and row mirrors) gives
// every lane of the group the full score. The online softmax (Lab 5
// handout, "Flash Attention": running max m, running sum l, unnormalised
// output o, O = o/l; base-2 exponents, fp32 state) rescales o only when a
// row's max grows. A key no query may see is removed by select, never by
// multiplying with 0, so garbage in unused slots cannot leak in.
#include "pa_common.h"

namespace pa {

template <bool BF16, int D, int ROWS, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
pa_valu_kernel(const Params p) {
  constexpr int EB = BF16 ? 2 : 4;          // bytes per cache element
  constexpr int ROW_BYTES = D * EB;
  constexpr int LPT = ROW_BYTES >= 256 ? 16 : 8;   // lanes sharing one row: 16 B each, whole lines
  constexpr int TPI = 64 / LPT;             // rows per load instruction
  constexpr int TPL = kBlock / TPI;         // rows per lane per block
  constexpr int COLS = ROW_BYTES / (LPT * 16);
  constexpr int EPC = 16 / EB;              // elements per 16-byte chunk
  static_assert(COLS >= 1 && ROW_BYTES % (LPT * 16) == 0, "row must be whole 128-byte lines");
  // Two register buffers for K/V tiles when they fit next to q and the accumulators.
  constexpr int TILE_WORDS = TPL * COLS * 4;
  constexpr bool PIPE = 4 * TILE_WORDS + ROWS * COLS * (4 + EPC) <= 180;

  __shared__ float lds_acc[NW * ROWS * D];
  __shared__ float lds_ml[NW * ROWS * 2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: block indices and table reads stay scalar
  const int tsub = lane / LPT;
  const int part = lane % LPT;

  const int32_t g = blockIdx.x % p.Hkv;
  const int32_t bsplit = blockIdx.x / p.Hkv;
  const int32_t b = bsplit % p.B;
  const int32_t split = bsplit / p.B;

  const int32_t L = p.seq_lens[b];
  if (!len_ok(L, p)) return;   // broken precondition: touch nothing outside the arrays
  const KeyRange kr = key_range(L, p.q_len, p.window);
  const int32_t first = kr.blk_lo + split * p.bps;
  if (first > kr.blk_hi) return;
  const int32_t last = min(kr.blk_hi, first + p.bps - 1);

  // Query slices: row r = t * G + gi is query token t of head g*G + gi.
  uint32_t qw[ROWS][COLS][4];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    if (r < p.rows) {
      const int t = r / p.G;
      const int h = g * p.G + r % p.G;
      const char* qrow = reinterpret_cast<const char*>(p.q) + (((size_t)b * p.q_len + t) * p.Hq + h) * ROW_BYTES;
#pragma unroll
      for (int c = 0; c < COLS; ++c) {
        const uint4 v = load16(qrow + c * LPT * 16 + part * 16);
        qw[r][c][0] = v.x; qw[r][c][1] = v.y; qw[r][c][2] = v.z; qw[r][c][3] = v.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < COLS; ++c) qw[r][c][0] = qw[r][c][1] = qw[r][c][2] = qw[r][c][3] = 0u;
    }
  }

  float m[ROWS], l[ROWS], acc[ROWS][COLS][EPC];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int c = 0; c < COLS; ++c)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[r][c][e] = 0.f;
  }

  // Per-row visibility bounds: row r sees keys [lo_r, p0 + t_r].
  int32_t row_lo[ROWS], row_hi[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int t = r / p.G;
    row_lo[r] = first_key(kr.p0, t, p.window);
    row_hi[r] = r < p.rows ? kr.p0 + t : -1;
  }

  // A (block, KV head) tile: 16 rows of ROW_BYTES, tok_stride apart. Lane
  // (tsub, part) reads 16 bytes at column part*16 (+ c*LPT*16) of rows tsub + TPI*u.
  const int32_t tok_stride = token_stride_bytes(p.Hkv, ROW_BYTES);
  const int32_t tile_bytes = (kBlock - 1) * tok_stride + ROW_BYTES;
  const int32_t lane_off = tsub * tok_stride + part * 16;
  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(p.v_pool);
  const int32_t* table = p.block_table + (size_t)b * p.maxb;
  int32_t* visits = p.visits ? p.visits + ((size_t)b * p.Hkv + g) * p.maxb : nullptr;

  // One 16-token block: this lane's 16-byte slices of the K and V rows.
  using Tile = uint4[TPL][COLS];
  // The k-th block of this wavefront is first + wave + NW*k; lane k holds its
  // physical id (one coalesced read up front, then v_readlane per block, so no
  // block waits on a table read behind the K/V loads already in flight).
  int32_t cfirst = first;   // first block of the current chunk (at most 64 blocks per wavefront)
  int32_t nmine = 0;
  int32_t tbl = 0;

  // Block k of this wavefront (k >= nmine: a no-op load of zero bytes, so
  // every path through the pipeline issues the same loads).
  auto fetch = [&](int32_t k, Tile& kr_, Tile& vr_) __attribute__((always_inline)) {
    const bool valid = k < nmine;
    const int32_t phys = __builtin_amdgcn_readlane(tbl, valid ? k : 0);
    const size_t tile = tile_offset_bytes(phys, g, p.Hkv, ROW_BYTES);
    const auto kd = buffer_rsrc(kpool + tile, valid ? tile_bytes : 0);
    const auto vd = buffer_rsrc(vpool + tile, valid ? tile_bytes : 0);
#pragma unroll
    for (int u = 0; u < TPL; ++u)
#pragma unroll
      for (int c = 0; c < COLS; ++c) kr_[u][c] = buffer_load16(kd, lane_off + c * LPT * 16, TPI * u * tok_stride);
#pragma unroll
    for (int u = 0; u < TPL; ++u)
#pragma unroll
      for (int c = 0; c < COLS; ++c) vr_[u][c] = buffer_load16(vd, lane_off + c * LPT * 16, TPI * u * tok_stride);
  };
  auto keep = [&](const Tile& kr_, const Tile& vr_) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < TPL; ++u)
#pragma unroll
      for (int c = 0; c < COLS; ++c) {
        keep_loaded(kr_[u][c]);
        keep_loaded(vr_[u][c]);
      }
  };

  auto consume = [&](int32_t k, const Tile& kr_, const Tile& vr_) __attribute__((always_inline)) {
    const int32_t i = cfirst + wave + NW * k;   // logical block

    // q . k for every (row slot u, query row r), summed over the lanes sharing the row.
    float s[TPL][ROWS];
#pragma unroll
    for (int u = 0; u < TPL; ++u)
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float acc_s = 0.f;
#pragma unroll
        for (int c = 0; c < COLS; ++c) {
          const uint32_t kw[4] = {kr_[u][c].x, kr_[u][c].y, kr_[u][c].z, kr_[u][c].w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (BF16) {
              acc_s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[r][c][w]),
                                                      __builtin_bit_cast(bf16x2, kw[w]), acc_s, false);
            } else {
              acc_s = fmaf(__builtin_bit_cast(float, qw[r][c][w]), __builtin_bit_cast(float, kw[w]), acc_s);
            }
          }
        }
        s[u][r] = group_sum<LPT>(acc_s);
      }

    // Mask by select, scale to base-2 exponent units, per-row block max.
    bool tok_ok[TPL];
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
      const int32_t j = i * kBlock + tsub + TPI * u;
      tok_ok[u] = j < L && j >= kr.lo0;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const bool ok = j <= row_hi[r] && j >= row_lo[r];
        s[u][r] = ok ? s[u][r] * p.scale_log2 : -INFINITY;
      }
    }

    float pr[TPL][ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float mb = s[0][r];
#pragma unroll
      for (int u = 1; u < TPL; ++u) mb = fmaxf(mb, s[u][r]);
      mb = across_groups_max<LPT>(mb);
      const float mn = fmaxf(m[r], mb);
      if (__builtin_amdgcn_readfirstlane((int)(mn > m[r]))) {
        const float a = fast_exp2(m[r] - mn);   // 0 when m was -inf
        l[r] *= a;
#pragma unroll
        for (int c = 0; c < COLS; ++c)
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[r][c][e] *= a;
        m[r] = mn;
      }
      const float msafe = m[r] == -INFINITY ? 0.f : m[r];
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        pr[u][r] = fast_exp2(s[u][r] - msafe);
        l[r] += pr[u][r];
      }
    }

    // o += p * v; rows no query may see are zeroed first (they may hold anything).
#pragma unroll
    for (int u = 0; u < TPL; ++u)
#pragma unroll
      for (int c = 0; c < COLS; ++c) {
        const uint32_t vw[4] = {tok_ok[u] ? vr_[u][c].x : 0u, tok_ok[u] ? vr_[u][c].y : 0u,
                                tok_ok[u] ? vr_[u][c].z : 0u, tok_ok[u] ? vr_[u][c].w : 0u};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (BF16) {
            const float lo = bf16_lo(vw[w]);
            const float hi = bf16_hi(vw[w]);
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
              acc[r][c][2 * w] = fmaf(pr[u][r], lo, acc[r][c][2 * w]);
              acc[r][c][2 * w + 1] = fmaf(pr[u][r], hi, acc[r][c][2 * w + 1]);
            }
          } else {
            const float v = __builtin_bit_cast(float, vw[w]);
#pragma unroll
            for (int r = 0; r < ROWS; ++r) acc[r][c][w] = fmaf(pr[u][r], v, acc[r][c][w]);
          }
        }
      }
  };

  // Two-deep software pipeline: block k+1 is in flight while block k is consumed.
  for (; cfirst <= last; cfirst += 64 * NW) {
    const int32_t clast = min(last, cfirst + 64 * NW - 1);
    nmine = clast >= cfirst + wave ? (clast - cfirst - wave) / NW + 1 : 0;
    tbl = settle(lane < nmine ? table[table_entry(p, cfirst + wave + NW * lane)] : 0);
    // Debug load counts, kept out of the pipelined loop below.
    if (visits && lane < nmine) atomicAdd(visits + table_entry(p, cfirst + wave + NW * lane), 1);
    if constexpr (PIPE) {
      // Block k+1 is in flight while block k is consumed. The fetches are
      // unconditional (past the end they load zero bytes), so every path into
      // the loop head has the same loads outstanding and the compiler waits
      // only for the block it consumes.
      Tile ka, va, kb, vb;
      fetch(0, ka, va);
      for (int32_t k = 0; k < nmine; k += 2) {
        fetch(k + 1, kb, vb);
        consume(k, ka, va);
        if (k + 1 >= nmine) break;
        __builtin_amdgcn_sched_barrier(0);   // refill a buffer only once it is consumed
        fetch(k + 2, ka, va);
        consume(k + 1, kb, vb);
        __builtin_amdgcn_sched_barrier(0);
      }
      keep(ka, va);
      keep(kb, vb);
    } else {
      Tile ka, va;
      for (int32_t k = 0; k < nmine; ++k) {
        fetch(k, ka, va);
        consume(k, ka, va);
      }
    }
  }

  // Sum the lane groups (different rows, same slices), then hand off to LDS.
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    l[r] = across_groups_sum<LPT>(l[r]);
#pragma unroll
    for (int c = 0; c < COLS; ++c)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[r][c][e] = across_groups_sum<LPT>(acc[r][c][e]);
  }
  if (tsub == 0) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
      for (int c = 0; c < COLS; ++c)
#pragma unroll
        for (int e = 0; e < EPC; ++e) lds_acc[(wave * ROWS + r) * D + c * LPT * EPC + part * EPC + e] = acc[r][c][e];
    if (part == 0) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        lds_ml[(wave * ROWS + r) * 2] = m[r];
        lds_ml[(wave * ROWS + r) * 2 + 1] = l[r];
      }
    }
  }
  if constexpr (BF16) {
    merge_and_store<__bf16, D, ROWS, NW>(p, lds_acc, lds_ml, b, g, p.splits > 1 ? split : -1);
  } else {
    merge_and_store<float, D, ROWS, NW>(p, lds_acc, lds_ml, b, g, p.splits > 1 ? split : -1);
  }
}

namespace {
template <bool BF16, int D, int ROWS>
hipError_t launch_one(const Params& p, int nw, int grid, hipStream_t st, const Timing& tm, bool* ok) {
  *ok = true;
  switch (nw) {
    case 4: return launch_timed(pa_valu_kernel<BF16, D, ROWS, 4>, grid, 4 * 64, st, tm, p);
    case 8: return launch_timed(pa_valu_kernel<BF16, D, ROWS, 8>, grid, 8 * 64, st, tm, p);
  }
  *ok = false;
  return hipSuccess;
}

template <bool BF16, int D>
hipError_t by_rows(const Params& p, int rows_t, int nw, int grid, hipStream_t st, const Timing& tm, bool* ok) {
  // Query rows live in registers next to a row slice of D/8 elements: keep rows * D / 8 <= 64.
  switch (rows_t) {
    case 1: return launch_one<BF16, D, 1>(p, nw, grid, st, tm, ok);
    case 2: return launch_one<BF16, D, 2>(p, nw, grid, st, tm, ok);
    case 4: if constexpr (D <= 128) return launch_one<BF16, D, 4>(p, nw, grid, st, tm, ok); break;
    case 8: if constexpr (D <= 64) return launch_one<BF16, D, 8>(p, nw, grid, st, tm, ok); break;
  }
  *ok = false;
  return hipSuccess;
}
}  // namespace

hipError_t launch_valu(const Params& p, int q_dtype, int kv_dtype, int D, int rows_t, int nw, int grid,
                       hipStream_t st, const Timing& tm, bool* supported) {
  *supported = false;
  const bool bf16 = kv_dtype == 1;
  if (q_dtype != kv_dtype || kv_dtype > 1) return hipSuccess;
  switch (D) {
    case 64: return bf16 ? by_rows<true, 64>(p, rows_t, nw, grid, st, tm, supported)
                         : by_rows<false, 64>(p, rows_t, nw, grid, st, tm, supported);
    case 128: return bf16 ? by_rows<true, 128>(p, rows_t, nw, grid, st, tm, supported)
                          : by_rows<false, 128>(p, rows_t, nw, grid, st, tm, supported);
    case 256: return bf16 ? by_rows<true, 256>(p, rows_t, nw, grid, st, tm, supported)
                          : by_rows<false, 256>(p, rows_t, nw, grid, st, tm, supported);
  }
  return hipSuccess;
}

}  // namespace pa
