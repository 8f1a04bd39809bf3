// pa_prefill.hip -- paged prefill attention on the matrix cores: a chunk of
// query tokens per sequence, causal among themselves, over the sequence's
// history already in the paged cache (Lab 5 handout, "Flash Attention": a
// query block walks only the key blocks the causal rule lets it see, and a
// window layer also skips the blocks before its window, instead of scoring
// everything and masking; GQA without repeating K/V heads; an incomplete last
// tile masked). The softmax is the online form with fp32 state m, l and the
// accumulator, and O = o / l at the end (same section).
//
// Work: one workgroup of four wavefronts per (query tile, sequence, KV head).
// Its rows are (query token, query head) pairs of that KV head's group --
// 128 rows (64 at head_dim 256), each wavefront 16 or 32 of them -- so one
// K/V tile staged in LDS serves every row. Tiles of late query tokens, which
// see the most keys, are dispatched first.
//
// Per step of 32 keys (two cache blocks): every thread loads 16-byte pieces
// of the K and V rows along the cached rows and writes them to LDS as bf16
// (int8 codes widen exactly); the next step's loads are in flight while the
// current step is computed from the other LDS buffer. S^T = K Q^T uses the
// decode kernel's operand layout with v_mfma_f32_16x16x32_bf16 (Q^T in
// registers), the softmax is lane-local per row with a 4-lane max, and
// O^T += V^T P^T takes all 32 keys of a step in one instruction per output
// tile: V^T read transposed by ds_read_b64_tr_b16 from both 16-key halves,
// against one bf16 weight per key (rounded to nearest: each weight within a
// relative 2^-9, so O within 2^-9 max|V| of its exact value; the row sum l
// adds the same rounded weights, so O stays a convex combination of V rows).
// Keys outside the tile's range are staged as zeros and every score outside
// a row's [first visible key, own position] is removed by select; steps
// whose keys every row of the tile sees skip the masks.
//
// int8 caches: K codes widen to bf16 (the query's type, so S^T keeps the bf16
// MFMA) and V codes to f16, both exactly (|code| <= 127). The key scale, times
// the softmax's scale*log2(e), multiplies each score; the value scale
// multiplies each weight (dequantize after the gather, tiniestgpt notes, KV
// cache quantization). The weights then go to the matrix cores as one f16
// value each (11 significant bits, rounded to nearest), against the f16 V^T
// of both 16-key halves in one v_mfma_f32_16x16x32_f16 per output tile. A
// weight times its value scale must stay within f16 range: value scales
// below 255, i.e. dequantized values below ~32500 in magnitude.
//
// The running max is moved lazily: a row's reference max only changes when
// its block max exceeds it by more than kRescaleSlack (log2 units), so the
// accumulator is rescaled a handful of times per row instead of at nearly
// every step. The softmax is unchanged -- any reference value gives the same
// o / l -- and the weights stay below 2^kRescaleSlack, far from overflow.
#include <hip/hip_ext.h>

#include "pa_device.h"
#include "pa_prefill.h"

namespace pa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 f16x2 __attribute__((ext_vector_type(2)));

template <bool INT8, int D>
struct PrefillShape {
  static constexpr int NW = 4;
  static constexpr int MT = prefill_rows(D) / (NW * 16);   // 16-row tiles per wavefront
  static constexpr int C = D / 32;                         // contraction chunks of S^T
  static constexpr int TJ = D / 16;                        // 16-dim output tiles
  static constexpr int KB = 32;                            // keys per step
  static constexpr int EB = INT8 ? 1 : 2;
  static constexpr int ROW_BYTES = D * EB;
  static constexpr int LPR = ROW_BYTES / 16;               // 16-byte pieces per cached row
  static constexpr int NP = 2 * KB * LPR / (NW * 64);      // K and V pieces per thread per step
  // bf16 caches load straight into LDS (no staging registers), rows 2D bytes
  // apart with 16-byte chunks XOR-swizzled by row; int8 caches are staged
  // through registers (widened to bf16), rows padded to 2D + 32 bytes.
  static constexpr bool DIRECT = !INT8;
  static constexpr int RS = DIRECT ? D * 2 : D * 2 + 32;  // LDS row stride
  static constexpr int TILE = KB * RS;
  static constexpr int STAGE = 2 * TILE + (INT8 ? 2 * KB * 4 : 0);   // K tile, V tile, int8 scales
  static constexpr int NSTAGE = DIRECT && 3 * STAGE <= 72 * 1024 ? 3 : 2;
  static constexpr int BYTES = NSTAGE * STAGE;
  // Direct loads: one load instruction fills 1 KiB of LDS (64 lanes x 16 bytes),
  // RPI rows of CPR 16-byte chunks; IPW instructions per wavefront per tile.
  static constexpr int RPI = 1024 / (D * 2);
  static constexpr int CPR = D * 2 / 16;
  static constexpr int IPW = KB / RPI / NW;
  static_assert(NP >= 1 && (2 * KB * LPR) % (NW * 64) == 0, "piece split");
  static_assert(!DIRECT || (IPW >= 1 && IPW * RPI == 8 && NW == 4), "direct-load split: 8 rows per wavefront");
};

// Swizzle of the 16-byte chunks of LDS row `row` (direct-load layout): chunk c
// of the cached row is stored at chunk c ^ swz(row). Sixteen consecutive rows
// get distinct swizzles within one 256-byte bank sweep, so the K-operand reads
// (16 rows, one chunk) and the transposed V reads hit distinct banks.
template <int D>
__device__ __forceinline__ int lds_swz(int row) {
  return D >= 128 ? (row & 15) : ((row >> 1) & 7);
}

// s_waitcnt immediate waiting until at most n vector-memory operations are outstanding.
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) & 3) << 14 | (7 << 4) | (15 << 8);
}

// 16 bytes per lane from buffer `rsrc` at byte `voff` straight into LDS:
// lane i's bytes land at LDS address lds_base + 16 * i. Issued as assembly so
// that the compiler does not wait for these loads before every LDS access
// (it cannot tell which of them an LDS read depends on); the kernel waits for
// them itself (vmcnt, then a barrier) before reading the buffer they fill.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, int32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds_base)
               : "m0");
}

template <bool INT8, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
pa_prefill_kernel(const PrefillParams p) {
  using S = PrefillShape<INT8, D>;
  constexpr int MT = S::MT, C = S::C, TJ = S::TJ, KB = S::KB, LPR = S::LPR, NP = S::NP, RS = S::RS;
  constexpr int ROW_BYTES = S::ROW_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[S::BYTES];

  // The workgroup's tile: late query tiles first.
  const int32_t units = p.B * p.Hkv;
  const int32_t tile = p.ntiles - 1 - (int32_t)(blockIdx.x / units);
  const int32_t u = (int32_t)(blockIdx.x % units);
  const int32_t b = u / p.Hkv;
  const int32_t g = u - b * p.Hkv;
  const int32_t qs = p.q_start[b];
  const int32_t qn = p.q_start[b + 1] - qs;
  const int32_t t0 = tile * p.qt;
  if (t0 >= qn) return;
  const int32_t L = p.seq_lens[b];
  if (L < qn || (p.ring == 0 && (int64_t)L > (int64_t)p.maxb * kBlock)) return;   // broken precondition
  const int32_t tcount = min(p.qt, qn - t0);
  const int32_t pos_first = L - qn + t0;                    // position of the tile's first query
  const int32_t khi = pos_first + tcount - 1;               // last key any row sees (its own position)
  const int32_t klo = p.window > 0 ? max(0, pos_first - p.window + 1) : 0;
  const int32_t blk_lo = klo / kBlock;
  const int32_t nsteps = (khi / kBlock - blk_lo) / 2 + 1;
  // Keys every row of a full tile sees: [lo_all, pos_first] (the last row's
  // window start to the first row's position).
  const bool full_tile = tcount == p.qt && p.qt * p.G == S::NW * MT * 16;
  const int32_t lo_all = p.window > 0 ? max(0, khi - p.window + 1) : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int q4 = lane >> 4;

  // Rows of this lane: tile mt holds rows (wave*MT + mt)*16 + n; row r is
  // query token r / G of the tile and head g*G + r % G.
  bf16x8 qt[MT][C];
  int32_t row_lo[MT], row_hi[MT], row_tok[MT], row_head[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = (wave * MT + mt) * 16 + n;
    const int32_t tt = r / p.G;
    const bool live = tt < tcount;
    const int32_t pos = pos_first + tt;
    row_tok[mt] = live ? tt : -1;
    row_head[mt] = g * p.G + (r - tt * p.G);
    row_lo[mt] = p.window > 0 ? max(0, pos - p.window + 1) : 0;
    row_hi[mt] = live ? pos : -1;
    const char* qrow = reinterpret_cast<const char*>(p.q) +
                       ((size_t)(qs + t0 + (live ? tt : 0)) * p.Hq + row_head[mt]) * (size_t)D * 2;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (live) v = load16(qrow + (32 * c + 8 * q4) * 2);
      qt[mt][c] = __builtin_bit_cast(bf16x8, v);
    }
  }
  float ksh = 1.f, vsh = 1.f;   // per-head int8 scales (the key scale times scale*log2(e))
  if constexpr (INT8) {
    if (p.head_scales) {
      ksh = p.k_scale[g] * p.scale_log2;
      vsh = p.v_scale[g];
    }
  }

  f32x4 o[MT][TJ];
  float m[MT], l[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    m[mt] = -INFINITY;
    l[mt] = 0.f;
#pragma unroll
    for (int j = 0; j < TJ; ++j) o[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // This thread's pieces of a step: piece pi = tid + 256*k is K (pi < 32*LPR)
  // or V, cached row (pi % (32*LPR)) / LPR of the step, 16-byte chunk pi % LPR.
  // A wavefront's 64 pieces of one k lie in one half (one cache block) of one
  // of K and V, so its buffer descriptor is wave-uniform.
  const int32_t tok_stride = token_stride_bytes(p.Hkv, ROW_BYTES);
  const int32_t tile_bytes = (kBlock - 1) * tok_stride + ROW_BYTES;
  const int32_t* table = p.block_table + (size_t)b * p.maxb;
  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(p.v_pool);
  const bool token_scales = INT8 && !p.head_scales;
  const bool alias = p.v_pool == p.k_pool;   // V is K: its tile is loaded once and read as both

  // ---- direct-load path (bf16 caches) ----------------------------------------------------------
  // Step s's loads: the block pair blk_lo + 2s, +1 (a block past the range, or
  // a step past the last, loads through a zero-byte descriptor, so every step
  // issues the same number of loads and the waits below can count them).
  constexpr int NL = S::IPW * 2;   // load instructions per wavefront per step (K and V)
  // Block ids come 64 at a time, one per lane (logical blocks tbl_base ..
  // tbl_base + 63), and are picked per step with readlane: the only wait for
  // a table read happens when a new group of 64 is needed (every 32 steps).
  const int32_t blk_last = khi / kBlock;
  int32_t tbl_base = blk_lo;
  int32_t tbl = settle(table[table_entry(p, min(blk_lo + lane, blk_last))]);
  auto issue_direct = [&](int32_t s, char* buf) __attribute__((always_inline)) {
    const bool live = s < nsteps;
    const int32_t i0 = min(blk_lo + 2 * s, blk_last);
    const bool has1 = live && (i0 + 1) * kBlock <= khi;
    if (i0 + 1 >= tbl_base + 64) {           // wave-uniform: next group of block ids
      tbl_base = i0;
      tbl = settle(table[table_entry(p, min(tbl_base + lane, blk_last))]);   // the wait stays in this branch
    }
    // Wavefront w fills rows 8w .. 8w+7 of each tile (segments w*IPW ..), all
    // in cache block w / 2 of the step: one descriptor per tile per step.
    const bool mine1 = wave >= 2;
    const int32_t ph = __builtin_amdgcn_readlane(tbl, (mine1 && has1 ? i0 + 1 : i0) - tbl_base);
    const bool ok = mine1 ? has1 : live;
    const size_t tb = tile_offset_bytes(ph, g, p.Hkv, ROW_BYTES);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(buf) + wave * S::IPW * 1024;
#pragma unroll
    for (int t = 0; t < 2; ++t) {            // K tile, then V tile
      const char* pool = t == 0 || alias ? kpool : vpool;
      const bool skip = t == 1 && alias;     // V shares K's tile
      const auto d = buffer_rsrc(pool + tb, ok && !skip ? tile_bytes : 0);
#pragma unroll
      for (int k = 0; k < S::IPW; ++k) {
        const int row = (wave * S::IPW + k) * S::RPI + lane / S::CPR;   // row of the step's 32
        const int chunk = (lane % S::CPR) ^ lds_swz<D>(row);
        const int voff = (row % kBlock) * tok_stride + 16 * chunk;
        load_lds16(d, voff, lds0 + t * S::TILE + k * 1024);
      }
    }
  };
  // Zero the rows of step s's tiles whose keys lie outside [klo, khi] (edge steps only).
  auto zero_edges = [&](int32_t s, char* buf) __attribute__((always_inline)) {
    const int32_t key0 = (blk_lo + 2 * s) * kBlock;
    for (int pi = tid; pi < 2 * KB * S::CPR; pi += S::NW * 64) {
      const int t = pi / (KB * S::CPR);
      const int row = (pi / S::CPR) % KB;
      const int32_t key = key0 + row;
      if (key < klo || key > khi)
        *reinterpret_cast<uint4*>(buf + t * S::TILE + row * RS + 16 * (pi % S::CPR)) = make_uint4(0, 0, 0, 0);
    }
  };

  uint4 ld[NP];
  float lsc = 0.f;
  // Issue the loads of step s (the block pair blk_lo + 2s, +1; a block past
  // the range loads zero bytes).
  auto issue = [&](int32_t s) __attribute__((always_inline)) {
    const int32_t i0 = blk_lo + 2 * s;
    const bool has1 = (i0 + 1) * kBlock <= khi;
    const int32_t ph0 = table[table_entry(p, i0)];
    const int32_t ph1 = has1 ? table[table_entry(p, i0 + 1)] : 0;
    const size_t t0b = tile_offset_bytes(ph0, g, p.Hkv, ROW_BYTES);
    const size_t t1b = tile_offset_bytes(ph1, g, p.Hkv, ROW_BYTES);
    const auto k0 = buffer_rsrc(kpool + t0b, tile_bytes);
    const auto k1 = buffer_rsrc(kpool + t1b, has1 ? tile_bytes : 0);
    const auto v0 = buffer_rsrc(vpool + t0b, tile_bytes);
    const auto v1 = buffer_rsrc(vpool + t1b, has1 ? tile_bytes : 0);
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int base = 64 * wave + 256 * k;                 // wave-uniform
      const bool isv = base >= KB * LPR;
      const bool hi_half = (base % (KB * LPR)) / LPR >= kBlock;
      const int rem = (base % (KB * LPR)) + lane;
      const int voff = ((rem / LPR) % kBlock) * tok_stride + 16 * (rem % LPR);
      const auto d = isv ? (hi_half ? v1 : v0) : (hi_half ? k1 : k0);
      ld[k] = buffer_load16<0>(d, voff);
    }
    // Scales: lanes 0..31 of wavefront 0 (K) and 1 (V), one key each. A key of
    // a missing second block reads block 0's scale, which the masks ignore.
    if (token_scales && wave < 2 && lane < KB) {
      const float* sc = wave == 0 ? p.k_scale : p.v_scale;
      const int32_t ph = lane < kBlock ? ph0 : ph1;
      lsc = sc[scale_tile_index(ph, g, p.Hkv) + (lane % kBlock)];
    }
  };
  // Write step s's loaded pieces into LDS buffer `buf` as bf16; keys outside
  // [klo, khi] are written as zeros.
  auto stage = [&](int32_t s, char* buf) __attribute__((always_inline)) {
    const int32_t key0 = (blk_lo + 2 * s) * kBlock;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int pi = tid + 256 * k;
      const bool isv = pi >= KB * LPR;
      const int rem = pi % (KB * LPR);
      const int row = rem / LPR;
      const int chunk = rem % LPR;
      const int32_t key = key0 + row;
      const bool ok = key >= klo && key <= khi;
      uint4 w = ld[k];
      w.x = ok ? w.x : 0u;
      w.y = ok ? w.y : 0u;
      w.z = ok ? w.z : 0u;
      w.w = ok ? w.w : 0u;
      char* dst = buf + (isv ? S::TILE : 0) + row * RS;
      if constexpr (INT8) {
        uint4 lo, hi;
        if (isv) i8x16_to_f16_exact(w, lo, hi);
        else i8x16_to_bf16(w, lo, hi);
        // The two 16-byte halves go in swapped order in 32-byte chunks with
        // bit 2 set, so a store instruction covers every 16-byte slot of a
        // 128-byte span; the readers flip their half for those chunks.
        const int sw = ((chunk >> 2) & 1) * 16;
        *reinterpret_cast<uint4*>(dst + 32 * chunk + sw) = lo;
        *reinterpret_cast<uint4*>(dst + 32 * chunk + (16 - sw)) = hi;
      } else {
        *reinterpret_cast<uint4*>(dst + 16 * chunk) = w;
      }
    }
    // Key scales carry the softmax's scale*log2(e); a value scale of a key
    // outside [klo, khi] is stored as 0, so its weight (0) times it stays 0
    // whatever the unread scale slot holds.
    if (token_scales && wave < 2 && lane < KB) {
      const int32_t key = key0 + lane;
      const bool ok = key >= klo && key <= khi;
      reinterpret_cast<float*>(buf + 2 * S::TILE)[wave * KB + lane] =
          wave == 0 ? lsc * p.scale_log2 : (ok ? lsc : 0.f);
    }
  };

  // Step s from LDS buffer `buf`.
  auto compute = [&](int32_t s, const char* buf) __attribute__((always_inline)) {
    const int32_t key0 = (blk_lo + 2 * s) * kBlock;
    const bool interior = full_tile && key0 >= lo_all && key0 + KB - 1 <= pos_first;   // wave-uniform
    const char* kst = buf;
    const char* vst = S::DIRECT && alias ? buf : buf + S::TILE;
    const float* sst = reinterpret_cast<const float*>(buf + 2 * S::TILE);
    // S^T for both 16-key halves: lane l gets query row n, keys 16*half + 4*q4 .. +3.
    f32x4 sacc[MT][2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int krow = 16 * half + n;
      bf16x8 kop[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        // dims 32c + 8*q4 .. +7: 16-byte chunk 4c + q4 of the row (int8: its
        // halves swapped in 32-byte chunks 2c.. with bit 2 set, i.e. when c & 2)
        const int chunk = S::DIRECT ? ((4 * c + q4) ^ lds_swz<D>(krow)) : (4 * c + q4) ^ ((c >> 1) & 1);
        kop[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kst + krow * RS + 16 * chunk));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[c], qt[mt][c], acc, 0, 0, 0);
        sacc[mt][half] = acc;
      }
    }
    float ksc[8], vsc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ksc[e] = ksh;
      vsc[e] = vsh;
    }
    if (token_scales) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float4 a = *reinterpret_cast<const float4*>(sst + 16 * half + 4 * q4);
        const float4 v = *reinterpret_cast<const float4*>(sst + KB + 16 * half + 4 * q4);
        ksc[4 * half + 0] = a.x; ksc[4 * half + 1] = a.y; ksc[4 * half + 2] = a.z; ksc[4 * half + 3] = a.w;
        vsc[4 * half + 0] = v.x; vsc[4 * half + 1] = v.y; vsc[4 * half + 2] = v.z; vsc[4 * half + 3] = v.w;
      }
    }
    // Online softmax per row over the step's 32 keys; P leaves as hi/lo bf16
    // parts (bf16 caches) or as one f16 value per key times its value scale
    // (int8 caches; weight e of the lane is key 16*(e/4) + 4*q4 + e%4).
    bf16x8 pbv[MT];
    f16x8 pbh[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float sc[8];
      bool ok[8];
      float mb = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int32_t j = key0 + 16 * (e >> 2) + 4 * q4 + (e & 3);
        ok[e] = interior || (j >= row_lo[mt] && j <= row_hi[mt]);
        const float x = sacc[mt][e >> 2][e & 3] * (INT8 ? ksc[e] : p.scale_log2);
        sc[e] = ok[e] ? x : -INFINITY;
        mb = fmaxf(mb, sc[e]);
      }
      mb = quads16_max(mb);
      const bool grow = mb > m[mt] + kRescaleSlack;   // true for the first visible keys (m = -inf)
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? mb : m[mt];
        const float a = grow ? fast_exp2(m[mt] - mn) : 1.f;
        l[mt] *= a;
#pragma unroll
        for (int j = 0; j < TJ; ++j) o[mt][j] *= a;
        m[mt] = mn;
      }
      const float msafe = m[mt] == -INFINITY ? 0.f : m[mt];
      float pe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(sc[e] - msafe);
      if constexpr (INT8) {
        // A masked key's weight is exactly 0 (2^-inf), and its value scale is
        // finite (0 outside [klo, khi]).
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          l[mt] += pe[e];
          pbh[mt][e] = (_Float16)(pe[e] * vsc[e]);
        }
        continue;
      }
      // One bf16 weight per key; the row sum takes the same rounded weights,
      // so O stays a convex combination of the V rows.
      const uint4 pw = make_uint4(pack_bf16(pe[0], pe[1]), pack_bf16(pe[2], pe[3]), pack_bf16(pe[4], pe[5]),
                                  pack_bf16(pe[6], pe[7]));
      const uint32_t pwv[4] = {pw.x, pw.y, pw.z, pw.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        l[mt] += __builtin_bit_cast(float, pwv[i] << 16) + __builtin_bit_cast(float, pwv[i] & 0xFFFF0000u);
      pbv[mt] = __builtin_bit_cast(bf16x8, pw);
    }
    if constexpr (INT8) {
      // O^T += V^T P^T over all 32 keys: A holds the transposed f16 V reads of
      // both halves (lane: keys 4*q4 .. +3, then 16 + 4*q4 .. +3, one dim),
      // the order of the lane's weights in pbh.
      const int vrow0 = 4 * q4 + (n >> 2);
      const char* vread0 = vst + vrow0 * RS + 8 * (n & 1);
      const char* vread1 = vread0 + 16 * RS;
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int chunk = (2 * j + ((n & 3) >> 1)) ^ ((j >> 2) & 1);   // halves swapped when j & 4
        const uint2 a0 = lds_read_tr16(vread0 + 16 * chunk);
        const uint2 a1 = lds_read_tr16(vread1 + 16 * chunk);
        const f16x8 av = __builtin_bit_cast(f16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          o[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pbh[mt], o[mt][j], 0, 0, 0);
      }
      return;
    }
    // O^T += V^T P^T over all 32 keys: A holds the transposed V reads of both
    // halves (lane: keys 4*q4 .. +3, then 16 + 4*q4 .. +3, one dim), the order
    // of the lane's weights in pbv.
    const int vrow0 = 4 * q4 + (n >> 2);
    const char* vread0 = vst + vrow0 * RS + 8 * (n & 1);
    const char* vread1 = vread0 + 16 * RS;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      // dims 16j + 4*(n&3) .. +3: 16-byte chunk 2j + ((n&3) >> 1), half (n & 1); rows vrow0 and
      // vrow0 + 16 share a swizzle
      const int chunk = 2 * j + ((n & 3) >> 1);
      const int sw = S::DIRECT ? (chunk ^ lds_swz<D>(vrow0)) : chunk;
      const uint2 a0 = lds_read_tr16(vread0 + 16 * sw);
      const uint2 a1 = lds_read_tr16(vread1 + 16 * sw);
      const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(a0.x, a0.y, a1.x, a1.y));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        o[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pbv[mt], o[mt][j], 0, 0, 0);
    }
  };

  // Double-buffered key loop: step s+1's loads are in flight while step s is
  // computed; one barrier per step (buffer s&1 is rewritten two steps later,
  // after every wavefront has passed the barrier that follows its last read).
  if constexpr (S::DIRECT) {
    // NSTAGE LDS buffers; loads run NSTAGE - 1 steps ahead. At step s the
    // wavefront waits for its own loads of step s, the barrier makes every
    // wavefront's loads visible, and only then is buffer (s + NSTAGE - 1)
    // refilled: its last reader, step s - 1, is behind the barrier.
    constexpr int NS = S::NSTAGE;
#pragma unroll
    for (int k = 0; k + 1 < NS; ++k) issue_direct(k, smem + k * S::STAGE);
    for (int32_t s = 0; s < nsteps; ++s) {
      char* buf = smem + (s % NS) * S::STAGE;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * NL));
      __syncthreads();
      const int32_t key0 = (blk_lo + 2 * s) * kBlock;
      if (key0 < klo || key0 + KB - 1 > khi) {   // edge step: clear rows of keys no row may see
        zero_edges(s, buf);
        __syncthreads();
      }
      issue_direct(s + NS - 1, smem + ((s + NS - 1) % NS) * S::STAGE);
      compute(s, buf);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // loads past the last step (zero bytes) drain
  } else {
    issue(0);
    for (int32_t s = 0; s < nsteps; ++s) {
      char* buf = smem + (s & 1) * S::STAGE;
      stage(s, buf);
      if (s + 1 < nsteps) issue(s + 1);
      __syncthreads();
      compute(s, buf);
    }
  }

  // Row sums (the four lanes of a row each hold a quarter of the keys), then O / l.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) l[mt] = quads16_sum(l[mt]);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (row_tok[mt] < 0) continue;
    const float inv = 1.f / l[mt];
    __bf16* out = reinterpret_cast<__bf16*>(p.out) + ((size_t)(qs + t0 + row_tok[mt]) * p.Hq + row_head[mt]) * D + 4 * q4;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const f32x4 v = o[mt][j];
      *reinterpret_cast<uint2*>(out + 16 * j) =
          make_uint2(pack_bf16(v[0] * inv, v[1] * inv), pack_bf16(v[2] * inv, v[3] * inv));
    }
  }
}

namespace {
template <bool INT8>
hipError_t by_dim(const PrefillParams& p, int D, int64_t grid, hipStream_t st, hipEvent_t t0, hipEvent_t t1,
                  bool* ok) {
  *ok = true;
  const dim3 g((unsigned)grid), blk(256);
  switch (D) {
    case 64: hipExtLaunchKernelGGL((pa_prefill_kernel<INT8, 64>), g, blk, 0, st, t0, t1, 0, p); break;
    case 128: hipExtLaunchKernelGGL((pa_prefill_kernel<INT8, 128>), g, blk, 0, st, t0, t1, 0, p); break;
    case 256: hipExtLaunchKernelGGL((pa_prefill_kernel<INT8, 256>), g, blk, 0, st, t0, t1, 0, p); break;
    default: *ok = false; return hipSuccess;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int kv_dtype, int D, int64_t grid, hipStream_t st,
                          hipEvent_t start, hipEvent_t stop, bool* supported) {
  *supported = false;
  if (kv_dtype == 2) return by_dim<true>(p, D, grid, st, start, stop, supported);
  if (kv_dtype == 1) return by_dim<false>(p, D, grid, st, start, stop, supported);
  return hipSuccess;
}

}  // namespace pa
