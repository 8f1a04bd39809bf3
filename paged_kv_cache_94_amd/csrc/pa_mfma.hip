// pa_mfma.hip -- matrix-core paged decode attention for query groups of
// 8..32 rows per KV head (rows = (Hq/Hkv) * q_len): the Gemma4 global layer
// (16 query heads on one KV head), 8-head GQA over an int8 cache, and
// multi-token verify steps. Per 16-token block the two contractions are
// real small dense products -- S = Q K^T (rows x 16, depth D) and
// O += P V (rows x D, depth 16) -- so they run on MFMA; the softmax stays on
// the vector ALU in fp32.
//
// Layouts (lane l of the 64-lane wavefront; n = l & 15, q4 = l >> 4):
//  * Loads run along the cached rows: each group of D*e/16 lanes reads one
//    row of the (block, KV head) tile front to back in 16-byte pieces, so
//    every quad of lanes touches one cache line. (Reading the tile directly
//    in MFMA operand order -- 16 rows per instruction, 64 bytes each -- was
//    measured 15-40% slower on the same addresses.) Each wavefront writes
//    the block into its own LDS staging area as bf16 [16 tokens][D], rows
//    2D+32 bytes apart, and reads the operands back from there.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16 over D/32 chunks. The A operand is read from
//    the staged K tile (lane l: token n, dims 32c + 8*q4 .. +7, one 16-byte
//    LDS read per chunk); the B operand is Q^T, held in registers for the
//    whole segment. The result gives lane l query row n and tokens
//    4*q4 .. 4*q4+3 -- the B-operand layout P^T needs for the PV product,
//    and the row is lane-local, so the softmax needs lane exchanges only for
//    the max over the four lanes sharing a row.
//  * V is read with tokens along the contraction depth by ds_read_b64_tr_b16:
//    in each 16-lane group, lanes 4k..4k+3 address row k (token 4*q4+k, 16
//    consecutive dims) and lane i receives element i of the four rows -- the
//    A operand of O^T = V^T P^T for 16 dims.
//  * P is split into bf16 hi and lo parts; O^T += V^T [P_hi; P_lo] is one
//    v_mfma_f32_16x16x32_bf16 whose 32-deep contraction holds both parts
//    against the V^T slice read twice, so the weights keep ~16 bits while V
//    stays in its stored type.
//  * O^T accumulates in fp32: lane l ends with query row n and, per 16-dim
//    tile j, dims 16j + 4*q4 .. +3.
//  * int8 caches (tiniestgpt notes, KV cache quantization): codes are
//    gathered first and widened while staging, exactly (|code| <= 127): K
//    codes to bf16, and V codes to f16 when K and V have pools of their own
//    (a shared pool stages one bf16 tile for both). The key scale multiplies
//    the score of its token and the value scale is folded into P, which then
//    goes to the matrix cores as one f16 weight per key against the f16 V.
//    Each block's 16 key and 16 value scales come in with one load each and
//    pass through the staging area. A lane's 16 codes widen to 32 bytes,
//    stored as two 16-byte halves in an order that alternates between
//    128-byte spans, so the stores meet every LDS bank once.
//  * When v_pool == k_pool (Gemma4 global layer, shared W_K / W_V) the tile
//    is read from HBM once and staged once; it serves as both K and V.
#include "pa_common.h"

namespace pa {

template <int D, int MT, int NW, bool ALIAS>
struct MfmaLds {
  static constexpr int ROWS = 16 * MT;
  static constexpr int TJ = D / 16;                          // 16-dim output tiles per row tile
  // Staging, per wavefront: the block's K tile and (unless V aliases K) its
  // V tile as bf16 [16 tokens][D], rows RSTRIDE bytes apart (a 32-byte skew
  // keeps both the row-wise K reads and the transposed V reads free of bank
  // conflicts), then 32 floats for the int8 scales of the block.
  static constexpr int RSTRIDE = D * 2 + 32;
  static constexpr int TILE = 16 * RSTRIDE;
  static constexpr int WAVE_STAGE = TILE * (ALIAS ? 1 : 2) + 128;
  // Merge: output tile j belongs to wave j % NW. Once its block loop is
  // done, a wave parks in its own slot the NTO tiles it does not own,
  // [MT][NTO][64 lanes] float4 in increasing j (1 KiB per tile, lane-ordered,
  // so writes and reads are conflict-free), then its (m, l) per lane,
  // [MT][64] float2.
  static constexpr int NTO = TJ - TJ / NW;
  static constexpr int ML_OFF = MT * NTO * 1024;
  static constexpr int PARK = ML_OFF + MT * 64 * 8;
  // One slot per wave holds its staging area and later its parked tiles, so
  // a wave parks without waiting for the others to finish with their blocks.
  static constexpr int SLOT = WAVE_STAGE > PARK ? WAVE_STAGE : PARK;
  static constexpr int BYTES = NW * SLOT;
  // Position of tile j among the tiles wave w parks.
  static constexpr int park_index(int j, int w) {
    int c = 0;
    for (int x = 0; x < j; ++x) c += x % NW != w;
    return c;
  }
};

template <int V>
struct IntC {
  static constexpr int value = V;
};

// f(IntC<w>{}) for the wave-uniform w == wave: one code path per wave, so a
// wave's own tile indices are compile-time constants in f.
template <int W, int N, typename F>
__device__ __forceinline__ void for_this_wave(int wave, F& f) {
  if constexpr (W < N) {
    if (wave == W) f(IntC<W>{});
    else for_this_wave<W + 1, N>(wave, f);
  }
}

// Blocks a wavefront keeps in flight: as many as fit a register budget for
// the fetch buffers (FETCH_WORDS 32-bit registers per block), at most 4.
#ifndef PA_FETCH_BUDGET
#define PA_FETCH_BUDGET 64
#endif
constexpr int mfma_depth(int fetch_words) {
  const int d = PA_FETCH_BUDGET / fetch_words;
  return d < 1 ? 1 : (d > 4 ? 4 : d);
}

// Physical ids of the first chunk of a wavefront's blocks in a segment:
// lane j gets table[b][first + wave + NW*j]; lanes past the segment re-read
// its last entry, so only table entries of loaded blocks are ever read.
template <int NW>
__device__ __forceinline__ int32_t chunk_table(const Params& p, int32_t b, int32_t cfirst, int32_t last) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int32_t idx = min(cfirst + wave + NW * lane, last);
  return p.block_table[(size_t)b * p.maxb + table_entry(p, idx)];
}

// Barrier that orders LDS only. The merge exchanges data through LDS alone;
// a full __syncthreads() would also wait for every load in flight, among them
// the next segment's touch loads below.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int kTouch = 2;   // touch loads per lane for the next segment's first block

// What a segment's caller finds out about the segment after it: its first
// table chunk (a load in flight), thread 0's queue claim (an atomic in
// flight) and its KV head (-1: no next segment).
struct NextSeg {
  int32_t tbl = 0, claim = 0, g = -1;
};

// Attention of query rows (b, g) over logical blocks [first, last] of sequence
// b. slot < 0: write the normalised output; else write (m, l, o) to
// workspace slot `slot`. tbl0 = chunk_table(b, first, last), which the caller
// may have loaded ahead. next_fn() finds the segment after this one (a search
// in LDS, a table load and a queue claim); it runs once this segment's first
// loads are issued, so its latency hides under theirs, and its loads come back
// in pf and pf_claim: they are waited for right after this segment's block
// loop, when nothing else is in flight, so they reach the caller as settled
// values.
// pf_claim is thread 0's claim on the piece queue; it is handed to every
// wavefront through *claim_lds (read after this call returns). When pf holds
// the next segment's table entries (next_fn's g >= 0, its KV head), the wavefront
// ends by touching that segment's first block, one dword per 128-byte line,
// so it is on its way to L2 while the next segment starts and is found there
// when that segment loads it; the touch loads land in `touch`,
// which the next call consumes after its first barrier (which waits for every
// load anyway). Called uniformly by every wavefront of the workgroup.
template <bool INT8, bool ALIAS, int D, int MT, int NW, typename NextFn>
__device__ __forceinline__ void mfma_segment(const Params& p, char* smem, int32_t b, int32_t g, int32_t first,
                                             int32_t last, int64_t slot, int32_t tbl0, int32_t& pf,
                                             int32_t& pf_claim, int32_t* claim_lds, int32_t& seg,
                                             uint32_t (&touch)[kTouch], NextFn&& next_fn) {
  const int stamp_base = kStampSeg0 + kStampPerSeg * (seg < kStampSegments ? seg : kStampSegments);
  stamp(p, stamp_base);
  stamp_value(p, stamp_base + 4, (uint64_t)(last - first + 1));
  using Lds = MfmaLds<D, MT, NW, ALIAS>;
  constexpr int ROWS = Lds::ROWS;
  constexpr int C = D / 32;                           // contraction chunks of 32 dims
  constexpr int TJ = D / 16;                          // 16-dim output tiles
  constexpr int EB = INT8 ? 1 : 2;
  constexpr int ROW_BYTES = D * EB;
  // Tile loads run along the rows: LPR lanes cover one cached row with
  // 16-byte pieces, RPI rows per load instruction, NLOAD instructions per tile.
  constexpr int LPR = ROW_BYTES / 16;
  constexpr int RPI = 64 / LPR;
  constexpr int NLOAD = kBlock / RPI;
  // int8 caches with separate K and V stage the values as f16 and weigh them
  // with one f16 weight per key (a shared K/V tile serves as bf16 K, so it
  // keeps the bf16 weights of the other caches).
  constexpr bool F16V = INT8 && !ALIAS;
  // Cache rows are read once per step: the non-temporal hint keeps them from
  // displacing anything in L2 (measured 5% faster on 128-byte int8 rows too).
  constexpr int CPOL = kCacheNonTemporal;
  constexpr int RS = Lds::RSTRIDE;
  static_assert(D % 64 == 0 && LPR >= 4 && LPR <= 64, "head_dim must be 64, 128 or 256");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: block indices stay scalar
  const int n = lane & 15;
  const int q4 = lane >> 4;
  // Wait for the first chunk's table entries before issuing this segment's
  // query loads: a prefetched chunk then waits on nothing newer than itself.
  const int32_t tbl_first = settle(tbl0);
  // The sequence's length comes in with the queries and the first blocks;
  // only the masks need it.
  const int32_t L = p.seq_lens[b];
  KeyRange kr;                        // set once L has arrived (after the first loads are issued)
  int32_t row_lo[MT], row_hi[MT];     // per-row visible keys: [row_lo, row_hi]
  int32_t all_lo = 0, all_hi = -1;    // keys every live row sees: [all_lo, all_hi]

  // Q^T as the B operand: lane l holds query row n (+16 per tile), 8 dims per chunk.
  bf16x8 qt[MT][C];
#pragma unroll
  for (int tile = 0; tile < MT; ++tile) {
    const int r = n + 16 * tile;
    const bool live = r < p.rows;
    const int t = live ? r / p.G : 0;
    const int h = g * p.G + r % p.G;
    const char* qrow = reinterpret_cast<const char*>(p.q) + (((size_t)b * p.q_len + t) * p.Hq + h) * (size_t)D * 2;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (live) v = load16(qrow + (32 * c + 8 * q4) * 2);
      qt[tile][c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[MT][TJ];
  float m[MT], l[MT];
#pragma unroll
  for (int tile = 0; tile < MT; ++tile) {
    m[tile] = -INFINITY;
    l[tile] = 0.f;
#pragma unroll
    for (int j = 0; j < TJ; ++j) o[tile][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // A (block, KV head) tile: 16 rows of ROW_BYTES, tok_stride apart. Load
  // instruction u gives lane l row u*RPI + l/LPR, bytes 16*(l%LPR) .. +15:
  // every group of LPR lanes reads one row front to back.
  const int32_t tok_stride = token_stride_bytes(p.Hkv, ROW_BYTES);
  const int32_t tile_bytes = (kBlock - 1) * tok_stride + ROW_BYTES;
  const int ld_row = lane / LPR;                      // + u*RPI
  const int ld_chunk = lane % LPR;                    // 16-byte piece of the row
  const int32_t lane_off = ld_row * tok_stride + 16 * ld_chunk;
  const char* kpool = reinterpret_cast<const char*>(p.k_pool);
  const char* vpool = reinterpret_cast<const char*>(p.v_pool);
  const int32_t* table = p.block_table + (size_t)b * p.maxb;
  int32_t* visits = p.visits ? p.visits + ((size_t)b * p.Hkv + g) * p.maxb : nullptr;

  // This wavefront's staging area (bf16 K tile, V tile unless aliased, scales).
  // MFMA operands are read back from it: K as the A operand of S^T = K Q^T
  // (lane l: token n, dims 32c + 8*q4 .. +7, one 16-byte read), V transposed
  // with ds_read_b64_tr_b16 (lane l: row 4*q4 + (n>>2), dims 16j + 4*(n&3)).
  char* kst = smem + wave * Lds::SLOT;
  char* vst = ALIAS ? kst : kst + Lds::TILE;
  float* sst = reinterpret_cast<float*>(kst + Lds::TILE * (ALIAS ? 1 : 2));
  const char* kread = kst + n * RS + 16 * q4;
  const char* vread = vst + (4 * q4 + (n >> 2)) * RS + 8 * (n & 3);
  // int8 tiles: a lane widens 16 codes to 32 bytes and stores them as two
  // 16-byte halves. Lanes whose 32-byte chunk has bit 2 set (chunks 4-7,
  // 12-15) store the halves in swapped order, so each store instruction
  // covers every 16-byte slot of a 128-byte span instead of every other one.
  // Readers of those chunks flip bit 4 of the address (kread_x, vread_x).
  constexpr bool SWZ = INT8;
  const char* kread_x = SWZ ? kst + n * RS + ((16 * q4) ^ 16) : kread;
  const char* vread_x = SWZ ? vst + (4 * q4 + (n >> 2)) * RS + ((8 * (n & 3)) ^ 16) : vread;

  // One 16-token block as loaded: NLOAD 16-byte pieces of K (and V) rows, and
  // for int8 caches the scale of token l & 15 (K and V).
  struct Fetched {
    uint4 k[NLOAD];
    uint4 v[ALIAS ? 1 : NLOAD];
    float ks, vs;
  };
  // The k-th block of this wavefront is first + wave + NW*k; lane k holds its
  // physical id (one coalesced read up front, then v_readlane per block, so no
  // block waits on a table read behind the K/V loads already in flight).
  int32_t cfirst = first;   // first block of the current chunk (at most 64 blocks per wavefront)
  int32_t nmine = 0;
  int32_t tbl = 0;

  // Block k of this wavefront (k >= nmine: a no-op load of zero bytes, so
  // every path through the pipeline issues the same loads).
  auto keep = [&](const Fetched& f) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NLOAD; ++u) keep_loaded(f.k[u]);
    if constexpr (!ALIAS) {
#pragma unroll
      for (int u = 0; u < NLOAD; ++u) keep_loaded(f.v[u]);
    }
    if constexpr (INT8) {
      keep_loaded(f.ks);
      keep_loaded(f.vs);
    }
  };

  auto fetch = [&](int32_t k, Fetched& f) __attribute__((always_inline)) {
    const bool valid = k < nmine;
    const int32_t phys = __builtin_amdgcn_readlane(tbl, valid ? k : 0);
    const size_t tile = tile_offset_bytes(phys, g, p.Hkv, ROW_BYTES);
    const auto kd = buffer_rsrc(kpool + tile, valid ? tile_bytes : 0);
#pragma unroll
    for (int u = 0; u < NLOAD; ++u) f.k[u] = buffer_load16<CPOL>(kd, lane_off, u * RPI * tok_stride);
    if constexpr (!ALIAS) {
      const auto vd = buffer_rsrc(vpool + tile, valid ? tile_bytes : 0);
#pragma unroll
      for (int u = 0; u < NLOAD; ++u) f.v[u] = buffer_load16<CPOL>(vd, lane_off, u * RPI * tok_stride);
    }
    if constexpr (INT8) {
      // The block's 16 scales of this KV head: one 64-byte run ([block][head][slot]);
      // with per-head scales every lane reads the head's one scale.
      const size_t s0 = p.head_scales ? (size_t)g : scale_tile_index(phys, g, p.Hkv);
      const int32_t sbytes = valid ? (p.head_scales ? 4 : kBlock * 4) : 0;
      const int32_t soff = p.head_scales ? 0 : (lane & 15) * 4;
      f.ks = buffer_load_f32(buffer_rsrc(p.k_scale + s0, sbytes), soff);
      f.vs = buffer_load_f32(buffer_rsrc(p.v_scale + s0, sbytes), soff);
    }
  };

  // Write one loaded piece (row r, 16 bytes at byte 16*ld_chunk of the cached
  // row) into a staging tile as bf16; int8 codes widen to 32 bytes, as f16
  // for a V tile of the f16-value path.
  auto stage = [&](char* dst_tile, int r, const uint4& w, bool as_f16) __attribute__((always_inline)) {
    if constexpr (INT8) {
      uint4 lo, hi;
      if (F16V && as_f16) i8x16_to_f16_exact(w, lo, hi);
      else i8x16_to_bf16(w, lo, hi);
      char* dst = dst_tile + r * RS + 32 * ld_chunk;
      const int sw = ((ld_chunk >> 2) & 1) * 16;   // halves swapped in chunks with bit 2 set
      *reinterpret_cast<uint4*>(dst + sw) = lo;
      *reinterpret_cast<uint4*>(dst + (16 - sw)) = hi;
    } else {
      *reinterpret_cast<uint4*>(dst_tile + r * RS + 16 * ld_chunk) = w;
    }
  };

  // Stage block k of this wavefront in LDS as bf16 (waits for its loads). A
  // V row nobody may see can hold anything and is written as zeros (only
  // edge blocks have such rows); a K row's score is masked by select, so its
  // contents do not matter. The registers that held the block are free
  // afterwards.
  auto stage_block = [&](int32_t k, const Fetched& f) __attribute__((always_inline)) {
    const int32_t i = cfirst + wave + NW * k;   // logical block
    const bool edge = i * kBlock < kr.lo0 || i * kBlock + kBlock > L;
    __builtin_amdgcn_wave_barrier();   // the previous block's reads stay before these writes
#pragma unroll
    for (int u = 0; u < NLOAD; ++u) {
      const int r = ld_row + u * RPI;
      const int32_t jv = i * kBlock + r;
      const bool v_ok = !edge || (jv < L && jv >= kr.lo0);
      uint4 w = ALIAS ? f.k[u] : f.v[ALIAS ? 0 : u];
      if (edge) {
        w.x = v_ok ? w.x : 0u;
        w.y = v_ok ? w.y : 0u;
        w.z = v_ok ? w.z : 0u;
        w.w = v_ok ? w.w : 0u;
      }
      stage(vst, r, w, true);
      if constexpr (!ALIAS) stage(kst, r, f.k[u], false);
    }
    if constexpr (INT8) {
      if (lane < 32) sst[lane] = lane < 16 ? f.ks : f.vs;
    }
    __builtin_amdgcn_wave_barrier();   // these writes stay before this block's reads
  };

  // Attention over staged block k: scores, online softmax, P.V.
  auto compute = [&](int32_t k) __attribute__((always_inline)) {
    const int32_t i = cfirst + wave + NW * k;   // logical block
    // Every live row sees every key of an interior block (and those keys lie
    // in [lo0, L), so their scales are read): no masks. Padding rows (zero
    // queries) then score the block too; they are never merged into a live
    // row or written. Only the int8 path, whose vector work is on its critical
    // path, branches on it: on the bf16 paths the branches cost more than the
    // masks (global layer 27.8 against 26.9 us).
    const bool interior = INT8 && i * kBlock >= all_lo && i * kBlock + kBlock - 1 <= all_hi;

    // K operand chunks: token n, dims 32c + 8*q4 .. +7.
    bf16x8 kop[C];
#pragma unroll
    for (int c = 0; c < C; ++c)   // bytes 64c.. lie in 32-byte chunks 2c, 2c+1: swapped when c & 2
      kop[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>((SWZ && (c & 2) ? kread_x : kread) + 64 * c));
    float ksc[4], vsc[4];
    if constexpr (INT8) {
      const float4 a = *reinterpret_cast<const float4*>(sst + 4 * q4);
      const float4 v = *reinterpret_cast<const float4*>(sst + 16 + 4 * q4);
      ksc[0] = a.x; ksc[1] = a.y; ksc[2] = a.z; ksc[3] = a.w;
      vsc[0] = v.x; vsc[1] = v.y; vsc[2] = v.z; vsc[3] = v.w;
    }

    // Scores and softmax for every row tile; P leaves as hi/lo bf16 parts, or
    // (f16 values) as one f16 weight per key times its value scale, rounded
    // to nearest: 11 significant bits, so O moves by at most 2^-12 of the
    // weighted |V| sum; a weight stays below 2^kRescaleSlack, so with value
    // scales below 255 it stays in f16 range.
    bf16x8 pbv[MT];
    f16x4 pbh[MT];
#pragma unroll
    for (int tile = 0; tile < MT; ++tile) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[c], qt[tile][c], s, 0, 0, 0);

      // s[e] = score of query row n (+16*tile) against token 4*q4+e of block i.
      float sc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[e] = s[e] * p.scale_log2;
        if constexpr (INT8) sc[e] *= ksc[e];
      }
      if (!interior) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int32_t j = i * kBlock + 4 * q4 + e;
          sc[e] = j <= row_hi[tile] && j >= row_lo[tile] ? sc[e] : -INFINITY;
        }
      }
      float mb = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) mb = fmaxf(mb, sc[e]);
      mb = quads16_max(mb);
      // Lazy rescale: the row's reference max moves only when the block max
      // passes it by more than kRescaleSlack (log2 units); weights stay below
      // 2^kRescaleSlack and o / l is unchanged by the choice of reference.
      const bool grow = mb > m[tile] + kRescaleSlack;   // true for the first visible keys (m = -inf)
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? mb : m[tile];
        const float a = grow ? fast_exp2(m[tile] - mn) : 1.f;
        l[tile] *= a;
#pragma unroll
        for (int j = 0; j < TJ; ++j) o[tile][j] *= a;
        m[tile] = mn;
      }
      const float msafe = m[tile] == -INFINITY ? 0.f : m[tile];
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = fast_exp2(sc[e] - msafe);
        l[tile] += pe[e];
      }
      if constexpr (INT8) {
        if (interior) {
#pragma unroll
          for (int e = 0; e < 4; ++e) pe[e] *= vsc[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int32_t j = i * kBlock + 4 * q4 + e;
            pe[e] *= j < L && j >= kr.lo0 ? vsc[e] : 0.f;
          }
        }
      }
      if constexpr (F16V) {
        pbh[tile] = f16x4{(_Float16)pe[0], (_Float16)pe[1], (_Float16)pe[2], (_Float16)pe[3]};
        continue;
      }
      // P as hi + lo bf16 parts for the 32-deep PV contraction.
      float lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        lo[e] = pe[e] - __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)pe[e]) << 16);
      pbv[tile] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16(pe[0], pe[1]), pack_bf16(pe[2], pe[3]),
                                                        pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3])));
    }

    // O^T += V^T [P_hi; P_lo], one 16-dim tile at a time, V^T read transposed from LDS.
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const uint2 a = lds_read_tr16((SWZ && (j & 4) ? vread_x : vread) + 32 * j);   // chunk j
      if constexpr (F16V) {
        // One 16-deep product: lane l holds V^T for dim n, keys 4*q4 .. +3,
        // against its own four weights.
        const f16x4 av = __builtin_bit_cast(f16x4, a);
#pragma unroll
        for (int tile = 0; tile < MT; ++tile)
          o[tile][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pbh[tile], o[tile][j], 0, 0, 0);
      } else {
        const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, a.x, a.y));
#pragma unroll
        for (int tile = 0; tile < MT; ++tile)
          o[tile][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pbv[tile], o[tile][j], 0, 0, 0);
      }
    }
  };

  // Software pipeline: DEPTH blocks in flight per wavefront; block k+DEPTH-1
  // is requested before block k is staged and computed. The fetches are
  // unconditional (past the end they load zero bytes), so every path into
  // the loop head has the same loads outstanding and the compiler waits only
  // for the block it consumes. (Staging block k first and refilling its
  // buffer with block k+DEPTH before the computation measured slower on the
  // global layer and no faster elsewhere.)
  constexpr int FETCH_WORDS = NLOAD * 4 * (ALIAS ? 1 : 2) + (INT8 ? 2 : 0);
  constexpr int DEPTH = mfma_depth(FETCH_WORDS);
  // Blocks come in chunks of at most 64 per wavefront (one table entry per
  // lane); the next chunk's entries are loaded while this one streams. The
  // first chunk's loads are issued before the barrier that waits for the
  // previous segment's merge to release the staging area, so they overlap it.
  Fetched f[DEPTH];
  auto chunk_size = [&]() __attribute__((always_inline)) {
    const int32_t clast = min(last, cfirst + 64 * NW - 1);
    return clast >= cfirst + wave ? (clast - cfirst - wave) / NW + 1 : 0;
  };
  nmine = chunk_size();
  tbl = tbl_first;
#pragma unroll
  for (int d = 0; d + 1 < DEPTH; ++d) fetch(d, f[d]);
  const NextSeg next = next_fn();
  pf = next.tbl;
  pf_claim = next.claim;
  const int32_t next_g = next.g;
  __syncthreads();
  // The previous segment's touch loads have landed (the barrier waited for
  // every load); their values are dead from here on.
#pragma unroll
  for (int t = 0; t < kTouch; ++t) keep_loaded(__builtin_bit_cast(float, touch[t]));
  // Per-row visibility: row r (query t) sees keys [first_key(t), p0 + t].
  kr = key_range(L, p.q_len, p.window);
#pragma unroll
  for (int tile = 0; tile < MT; ++tile) {
    const int r = n + 16 * tile;
    const bool live = r < p.rows;
    const int t = live ? r / p.G : 0;
    row_lo[tile] = first_key(kr.p0, t, p.window);
    row_hi[tile] = live ? kr.p0 + t : -1;
  }
  all_lo = first_key(kr.p0, p.q_len - 1, p.window);   // the last query's window starts latest
  all_hi = kr.p0;                                      // the first query sees the fewest keys
  while (true) {
    const int32_t tbl_next = chunk_table<NW>(p, b, cfirst + 64 * NW, last);
    // Debug load counts, kept out of the pipelined loop below.
    if (visits && lane < nmine) atomicAdd(visits + table_entry(p, cfirst + wave + NW * lane), 1);
    if (nmine > 0) {
      for (int32_t k = 0;; k += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          fetch(k + d + DEPTH - 1, f[(d + DEPTH - 1) % DEPTH]);
          stage_block(k + d, f[d]);
          compute(k + d);
#ifdef PA_STAMPS
          if (k + d == 0 && cfirst == first) stamp(p, stamp_base + 1);
#endif
          if (k + d + 1 >= nmine) goto drained;
          __builtin_amdgcn_sched_barrier(0);   // refill a buffer only once it is consumed
        }
      }
    }
  drained:
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) keep(f[d]);
    cfirst += 64 * NW;
    if (cfirst > last) break;
    nmine = chunk_size();
    tbl = settle(tbl_next);
#pragma unroll
    for (int d = 0; d + 1 < DEPTH; ++d) fetch(d, f[d]);
  }
  stamp(p, stamp_base + 2);
  pf = settle(pf);
  pf_claim = settle(pf_claim);
  if (claim_lds && threadIdx.x == 0) *claim_lds = pf_claim;   // read by all after the merge's barrier

  // Row sums: the four lanes of a row each hold a quarter of the tokens.
#pragma unroll
  for (int tile = 0; tile < MT; ++tile) l[tile] = quads16_sum(l[tile]);

  // Merge the wavefronts through LDS. Output tile j (dims 16j..16j+15)
  // belongs to wave j % NW. A wave parks the tiles it does not own and its
  // (m, l) in its own slot as soon as its block loop is done (the slot held
  // only its own staging area), so parking overlaps the waves still
  // streaming. After one barrier every wave folds the other waves' copies of
  // its own tiles into its registers with the online-softmax rule and writes
  // them, so the fold and the stores are spread over all wavefronts. Lane l
  // holds the same (row, dims) in every wave: the fold is per lane. Each wave
  // runs its own copy of this code, in which its tiles are compile-time
  // constants: the others die once parked, which leaves the registers to
  // request all the parked copies a fold needs before the first is used.
  auto merge_as = [&](auto wc) __attribute__((always_inline)) {
    constexpr int W = decltype(wc)::value;
    constexpr int OWN = (TJ + NW - 1) / NW;   // at most this many tiles per wave
    char* mine = smem + W * Lds::SLOT;
#pragma unroll
    for (int tile = 0; tile < MT; ++tile) {
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if (j % NW == W) continue;
        const f32x4 v = o[tile][j];
        *reinterpret_cast<float4*>(mine + (tile * Lds::NTO + Lds::park_index(j, W)) * 1024 + 16 * lane) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
      *reinterpret_cast<float2*>(mine + Lds::ML_OFF + (tile * 64 + lane) * 8) = make_float2(m[tile], l[tile]);
    }
    lds_barrier();
#pragma unroll
    for (int tile = 0; tile < MT; ++tile) {
      float2 ml[NW];
      float4 x[OWN][NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (w == W) {
          ml[w] = make_float2(m[tile], l[tile]);
          continue;
        }
        const char* theirs = smem + w * Lds::SLOT;
        ml[w] = *reinterpret_cast<const float2*>(theirs + Lds::ML_OFF + (tile * 64 + lane) * 8);
#pragma unroll
        for (int j = W; j < TJ; j += NW)
          x[j / NW][w] =
              *reinterpret_cast<const float4*>(theirs + (tile * Lds::NTO + Lds::park_index(j, w)) * 1024 + 16 * lane);
      }
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, ml[w].x);
      const float Ms = M == -INFINITY ? 0.f : M;
      float a[NW];
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        a[w] = fast_exp2(ml[w].x - Ms);   // 0 for a wave that saw no key of this row
        L += a[w] * ml[w].y;
      }
#pragma unroll
      for (int j = W; j < TJ; j += NW) {
        f32x4 acc = o[tile][j] * a[W];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          if (w == W) continue;
          const float4 v = x[j / NW][w];
          acc += a[w] * f32x4{v.x, v.y, v.z, v.w};
        }
        o[tile][j] = acc;
      }
      m[tile] = M;
      l[tile] = L;
    }

#pragma unroll
    for (int tile = 0; tile < MT; ++tile) {
      const int r = n + 16 * tile;
      if (r >= p.rows) continue;
      const int t = r / p.G;
      const int h = g * p.G + r % p.G;
      if (slot >= 0) {
        const size_t row_slot = (size_t)slot * p.rows + r;
#pragma unroll
        for (int j = W; j < TJ; j += NW) {
          const f32x4 v = o[tile][j];
          *reinterpret_cast<float4*>(p.ws_acc + row_slot * D + 16 * j + 4 * q4) = make_float4(v[0], v[1], v[2], v[3]);
        }
        if (W == 0 && q4 == 0) {
          p.ws_ml[row_slot * 2] = m[tile];
          p.ws_ml[row_slot * 2 + 1] = l[tile];
        }
      } else {
        const float inv = 1.f / l[tile];
        __bf16* out = reinterpret_cast<__bf16*>(p.out) + (((size_t)b * p.q_len + t) * p.Hq + h) * D + 4 * q4;
#pragma unroll
        for (int j = W; j < TJ; j += NW) {
          const f32x4 v = o[tile][j];
          *reinterpret_cast<uint2*>(out + 16 * j) =
              make_uint2(pack_bf16(v[0] * inv, v[1] * inv), pack_bf16(v[2] * inv, v[3] * inv));
        }
      }
    }
  };
  for_this_wave<0, NW>(wave, merge_as);
  if (next_g >= 0) {
    constexpr int LR = (ROW_BYTES + 127) / 128;         // 128-byte lines per cached row
    constexpr int LB = kBlock * LR * (ALIAS ? 1 : 2);   // lines per block (K, and V unless aliased)
    constexpr int TL = (LB + 63) / 64;                  // touch loads per lane (the first block only)
    static_assert(TL <= kTouch, "touch loads");
    const int32_t phys = __builtin_amdgcn_readfirstlane(pf);   // lane 0: the next segment's first block
    const size_t tile = tile_offset_bytes(phys, next_g, p.Hkv, ROW_BYTES);
#pragma unroll
    for (int t = 0; t < TL; ++t) {
      // The lane's line is the same for every segment; pinned here (an empty
      // asm), so the compiler does not hoist what derives from it out of the
      // segment loop and keep it live through the block loops.
      int w = min(lane + 64 * t, LB - 1);
      asm volatile("" : "+v"(w));
      const char* base = ((w >= kBlock * LR) ? vpool : kpool) + tile + ((w / LR) % kBlock) * tok_stride +
                         128 * (w % LR);
      touch[t] = *reinterpret_cast<const uint32_t*>(base);
    }
  }
  stamp(p, stamp_base + 3);
  ++seg;
}


// MODE is the partition (Params::balanced): 0 aligned splits, 1 flattened
// list, 2 pieces. Each partition is its own kernel, which keeps the scalar
// registers of the other two out of its allocation.
template <bool INT8, bool ALIAS, int D, int MT, int NW, int MODE>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
pa_mfma_kernel(const Params p) {
  __shared__ __attribute__((aligned(16))) char smem[MfmaLds<D, MT, NW, ALIAS>::BYTES];
  int32_t seg = 0;   // segments this workgroup has run (phase stamps only)
  uint32_t touch[kTouch] = {};   // the next segment's touch loads (consumed by the call after)
  stamp(p, kStampEntry);
  auto done = [&]() __attribute__((always_inline)) {
    stamp_value(p, kStampCount, (uint64_t)seg);
    stamp(p, kStampExit);
  };
  if constexpr (MODE == 0) {
    // Aligned splits: workgroup (split, b, g) takes blocks [blk_lo + split*bps, ...] of sequence b.
    const int32_t g = blockIdx.x % p.Hkv;
    const int32_t bsplit = blockIdx.x / p.Hkv;
    const int32_t b = bsplit % p.B;
    const int32_t split = bsplit / p.B;
    const int32_t L = p.seq_lens[b];
    if (!len_ok(L, p)) return done();   // broken precondition: touch nothing outside the arrays
    const KeyRange kr = key_range(L, p.q_len, p.window);
    const int32_t first = kr.blk_lo + split * p.bps;
    if (first > kr.blk_hi) return done();
    const int32_t last = min(kr.blk_hi, first + p.bps - 1);
    const int64_t slot = p.splits > 1 ? (int64_t)(b * p.Hkv + g) * p.splits + split : -1;
    stamp(p, kStampPartition);
    int32_t none = 0, none_c = 0;
    mfma_segment<INT8, ALIAS, D, MT, NW>(p, smem, b, g, first, last, slot, chunk_table<NW>(p, b, first, last), none,
                                         none_c, nullptr, seg, touch, [] { return NextSeg{}; });
    return done();
  }
  __shared__ int32_t pre[balanced_seq_limit(NW) + 1];
  if constexpr (MODE == 2) {
    // Piece partition: each piece is one run of one unit; the slot of a
    // partial is the piece's own index.
    __shared__ int32_t nbs[kMaxPieceSeqs];
    __shared__ int32_t blo[kMaxPieceSeqs];
    __shared__ int32_t ord[kMaxPieceSeqs];
    __shared__ int32_t claims[2];
    // Queue shard of this workgroup: shard s hands out pieces s, s + kQueueShards, ...
    // (one counter per shard: claims on a single counter serialize at ~11 ns each).
    const int32_t shard = blockIdx.x % kQueueShards;
    int32_t* const qnext = p.ws_queue ? p.ws_queue + shard * kQueueStride : nullptr;
    int32_t* const qdone = qnext ? qnext + kQueueShards * kQueueStride : nullptr;
    // This workgroup's first two claims, from the second wavefront while the
    // first one searches the partition.
    static_assert(NW >= 2, "claims and partition search run on different wavefronts");
    if (qnext && threadIdx.x == 64) {
      claims[0] = atomicAdd(qnext, 1);
      claims[1] = atomicAdd(qnext, 1);
    }
    piece_prefix(p, nbs, blo, ord, pre, 2 * NW, qnext != nullptr);
    __syncthreads();
    stamp(p, kStampPartition);
    // For the combine: the number of sequence b's first piece, and its piece count.
    if (blockIdx.x == 0 && p.ws_prefix)
      for (int32_t r = threadIdx.x; r < p.B; r += NW * 64) {
        const int32_t b = ord[r];
        p.ws_prefix[b] = pre[r];
        p.ws_prefix[p.B + b] = pre[r + 1] - pre[r];
      }
    const int32_t npieces = pre[p.B];
    struct Run {
      int32_t b, g, first, last;
      int64_t slot;
    };
    auto run_of = [&](int32_t w) __attribute__((always_inline)) {
      const Piece pc = piece_of(nbs, ord, pre, p.B, p.Hkv, w);
      Run r;
      r.b = pc.b;
      r.g = pc.g;
      r.first = blo[pc.b] + pc.first;
      r.last = r.first + pc.count - 1;
      r.slot = pc.k > 1 ? (int64_t)w : -1;
      return r;
    };
    if (!p.ws_queue) {
      // Static: workgroup w owns piece w.
      const int32_t w = blockIdx.x;
      if (w >= npieces) return done();
      const Run r = run_of(w);
      int32_t none = 0, none_c = 0;
      mfma_segment<INT8, ALIAS, D, MT, NW>(p, smem, r.b, r.g, r.first, r.last, r.slot,
                                           chunk_table<NW>(p, r.b, r.first, r.last), none, none_c, nullptr, seg,
                                           touch, [] { return NextSeg{}; });
      return done();
    }
    // Queue: claims only grow, so a workgroup's pieces come in increasing
    // order. While piece w streams, the next piece's table entries load and
    // thread 0 claims the one after it.
    auto piece_of_claim = [&](int32_t c) __attribute__((always_inline)) {
      return c < 0 ? -1 : shard + kQueueShards * c;
    };
    int32_t w = piece_of_claim(claims[0]);
    int32_t w1 = piece_of_claim(claims[1]);
    int32_t tbl0 = 0;
    // A negative claim can only come from a header that was not zero-filled;
    // it ends the workgroup rather than naming a piece.
    Run r{};
    if (w >= 0 && w < npieces) {
      r = run_of(w);
      tbl0 = settle(chunk_table<NW>(p, r.b, r.first, r.last));
    }
    while (w >= 0 && w < npieces) {
      // The next piece's run is found once, inside the segment (under its
      // first loads), and carried into the next iteration (the search is
      // eight dependent LDS reads and three divisions).
      Run rn{};
      int32_t tbln = 0, claim = 0;
      auto next = [&]() __attribute__((always_inline)) {
        NextSeg nx;
        if (w1 >= 0 && w1 < npieces) {
          rn = run_of(w1);
          nx.tbl = chunk_table<NW>(p, rn.b, rn.first, rn.last);
          nx.g = rn.g;
        }
        if (threadIdx.x == 0) nx.claim = atomicAdd(qnext, 1);
        return nx;
      };
      mfma_segment<INT8, ALIAS, D, MT, NW>(p, smem, r.b, r.g, r.first, r.last, r.slot, tbl0, tbln, claim,
                                           &claims[0], seg, touch, next);
      w = w1;
      w1 = piece_of_claim(claims[0]);
      tbl0 = tbln;
      r = rn;
    }
    // The last workgroup of a shard out returns its counters to zero for the
    // next call (every claim on that shard has completed by then).
    const int32_t members = ((int32_t)gridDim.x - shard + kQueueShards - 1) / kQueueShards;
    if (threadIdx.x == 0 && atomicAdd(qdone, 1) == members - 1) {
      atomicExch(qnext, 0);
      atomicExch(qdone, 0);
    }
    return done();
  }
  if constexpr (MODE == 1) {
    // Flattened-list partition: this workgroup's slice of the flattened
    // (unit, item) list, cut at unit boundaries into segments. A unit's items
    // are p.seg_items leading ones, which stand for the cost of a segment
    // start and merge and load nothing, then its blocks; equal slices then
    // balance blocks plus segments. A slice's part of a unit that holds none
    // of its blocks is no segment. A segment holding all of a unit's blocks
    // writes the output directly; the others leave a partial in slot
    // (workgroup + unit), which is unique because both indices only grow
    // along the list. Each sequence's first loaded block sits in LDS next to
    // the prefix sums, so the next segment's table entries are loaded while a
    // segment streams, and a segment starts with one memory round trip (its
    // first blocks, queries and length together) instead of three.
    __shared__ int32_t blo[balanced_seq_limit(NW)];
    block_prefix(p, pre, blo);
    __syncthreads();
    stamp(p, kStampPartition);
    if (blockIdx.x == 0 && p.ws_prefix)
      for (int32_t b = threadIdx.x; b <= p.B; b += NW * 64) p.ws_prefix[b] = pre[b];
    const Balanced bal = balanced_split(pre, p.B, p.Hkv, p.nwg);
    const int64_t x0 = (int64_t)blockIdx.x * bal.per;
    const int64_t hi = min(bal.total, x0 + bal.per);
    if (x0 >= hi) return done();
    // The slice's part of the unit holding item x (from x on): unit (b, g),
    // the logical blocks [first, last] it covers (last < first: none), the
    // item after it, and whether it holds all of the unit's blocks.
    struct Seg {
      int32_t b, g, first, last;
      int64_t end;
      bool whole;
    };
    auto segment_at = [&](int64_t x) __attribute__((always_inline)) {
      Seg sg;
      sg.b = balanced_seq(pre, p.B, p.Hkv, x);
      const int32_t items = pre[sg.b + 1] - pre[sg.b];   // >= 1: x lies in this sequence's units
      const int64_t base = (int64_t)p.Hkv * pre[sg.b];
      sg.g = (int32_t)((x - base) / items);
      const int64_t off = base + (int64_t)sg.g * items;
      sg.end = min(hi, off + items);
      const int32_t b0 = max((int32_t)(x - off) - p.seg_items, 0);
      const int32_t b1 = (int32_t)(sg.end - off) - p.seg_items;   // past the last block (<= b0: none)
      sg.first = blo[sg.b] + b0;
      sg.last = blo[sg.b] + b1 - 1;
      sg.whole = b0 == 0 && b1 == items - p.seg_items;
      return sg;
    };
    // Only a slice that lies within a unit's leading items can begin without
    // blocks, and then it holds none at all.
    Seg cur = segment_at(x0);
    if (cur.last < cur.first) return done();
    int32_t tbl0 = settle(chunk_table<NW>(p, cur.b, cur.first, cur.last));
    while (true) {
      // The next segment's first table chunk loads while this one streams.
      // Only the slice's last part of a unit can hold no blocks.
      const bool more = cur.end < hi;
      Seg nxs{};
      int32_t tbln = 0;
      auto next = [&]() __attribute__((always_inline)) {
        NextSeg nx;
        if (more) {
          nxs = segment_at(cur.end);
          if (nxs.last >= nxs.first) {
            nx.tbl = chunk_table<NW>(p, nxs.b, nxs.first, nxs.last);
            nx.g = nxs.g;
          }
        }
        return nx;
      };
      const int64_t slot = cur.whole ? -1 : (int64_t)blockIdx.x + (int64_t)cur.b * p.Hkv + cur.g;
      int32_t none_c = 0;
      mfma_segment<INT8, ALIAS, D, MT, NW>(p, smem, cur.b, cur.g, cur.first, cur.last, slot, tbl0, tbln, none_c,
                                           nullptr, seg, touch, next);
      if (!more || nxs.last < nxs.first) break;
      cur = nxs;
      tbl0 = tbln;
    }
    return done();
  }
}

namespace {
template <bool INT8, bool ALIAS, int D, int MT, int NW>
hipError_t launch_mode(const Params& p, int grid, hipStream_t st, const Timing& tm, bool* ok) {
  *ok = true;
  switch (p.balanced) {
    case 0: return launch_timed(pa_mfma_kernel<INT8, ALIAS, D, MT, NW, 0>, grid, NW * 64, st, tm, p);
    case 1: return launch_timed(pa_mfma_kernel<INT8, ALIAS, D, MT, NW, 1>, grid, NW * 64, st, tm, p);
    case 2:
      if constexpr (NW >= 4) return launch_timed(pa_mfma_kernel<INT8, ALIAS, D, MT, NW, 2>, grid, NW * 64, st, tm, p);
      break;
  }
  *ok = false;
  return hipSuccess;
}

template <bool INT8, bool ALIAS, int D, int MT>
hipError_t launch_one(const Params& p, int nw, int grid, hipStream_t st, const Timing& tm, bool* ok) {
  *ok = false;
  switch (nw) {
    case 2: return launch_mode<INT8, ALIAS, D, MT, 2>(p, grid, st, tm, ok);
    case 4: return launch_mode<INT8, ALIAS, D, MT, 4>(p, grid, st, tm, ok);
    case 8: return launch_mode<INT8, ALIAS, D, MT, 8>(p, grid, st, tm, ok);
  }
  return hipSuccess;
}

template <bool INT8, bool ALIAS>
hipError_t by_shape(const Params& p, int D, int mt, int nw, int grid, hipStream_t st, const Timing& tm, bool* ok) {
  *ok = false;
  if (mt == 1) {
    if (D == 64) return launch_one<INT8, ALIAS, 64, 1>(p, nw, grid, st, tm, ok);
    if (D == 128) return launch_one<INT8, ALIAS, 128, 1>(p, nw, grid, st, tm, ok);
    if (D == 256) return launch_one<INT8, ALIAS, 256, 1>(p, nw, grid, st, tm, ok);
  } else if (mt == 2) {
    if (D == 64) return launch_one<INT8, ALIAS, 64, 2>(p, nw, grid, st, tm, ok);
    if (D == 128) return launch_one<INT8, ALIAS, 128, 2>(p, nw, grid, st, tm, ok);
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_mfma(const Params& p, int kv_dtype, int D, int row_tiles, int nw, int grid,
                       hipStream_t st, const Timing& tm, bool* supported) {
  *supported = false;
  const bool alias = p.v_pool == p.k_pool;
  if (kv_dtype == 2) {
    return alias ? by_shape<true, true>(p, D, row_tiles, nw, grid, st, tm, supported)
                 : by_shape<true, false>(p, D, row_tiles, nw, grid, st, tm, supported);
  }
  if (kv_dtype == 1) {
    return alias ? by_shape<false, true>(p, D, row_tiles, nw, grid, st, tm, supported)
                 : by_shape<false, false>(p, D, row_tiles, nw, grid, st, tm, supported);
  }
  return hipSuccess;
}

}  // namespace pa
