// pa_mfma.hip -- matrix-core paged decode attention for query groups of
// 8..32 rows per KV head (rows = (Hq/Hkv) * q_len): the Gemma4 global layer
// (16 query heads on one KV head), 8-head GQA over an int8 cache, and
// multi-token verify steps. Per 16-token block the two contractions are
// real small dense products -- S = Q K^T (rows x 16, depth D) and
// O += P V (rows x D, depth 16) -- so they run on MFMA; the softmax stays on
// the vector ALU in fp32.
//
// Layouts (lane l of the 64-lane wavefront; n = l & 15, q4 = l >> 4):
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16 over D/32 chunks. The A operand is the K tile
//    as loaded: lane l holds token n, 8 consecutive dims of chunk c. The B
//    operand is Q^T held in registers for the whole kernel. The result gives
//    lane l query row n and tokens 4*q4 .. 4*q4+3 -- exactly the B-operand
//    layout P^T needs for the PV product, and the row is lane-local, so the
//    running max / sum and the accumulator rescale need no lane exchange
//    except the max over the four lanes sharing a row.
//  * V has to be read with tokens along the contraction depth. The V tile is
//    loaded like K (token per lane) and transposed on the matrix core itself:
//    multiplying a 16x16 slice by the identity with v_mfma_f32_16x16x16_bf16
//    returns it with lane l holding one dim and four tokens, the A layout of
//    O^T = V^T P^T. The product is exact (bf16 values times 1.0).
//  * O^T accumulates in fp32; lane l ends with query row n and, per chunk,
//    8 consecutive dims.
//  * int8 caches (tiniestgpt notes, KV cache quantization): codes are
//    gathered first, widened to bf16 (exact for |code| <= 127), the key scale
//    multiplies the score of its token and the value scale is folded into P.
//  * When v_pool == k_pool (Gemma4 global layer, shared W_K / W_V) the tile
//    is read from HBM once and used as both K and V.
#include "pa_common.h"

namespace pa {

namespace {

// dim held by lane-group q4, element e (0..7) of 32-wide contraction chunk c.
template <bool INT8>
__device__ __forceinline__ int chunk_dim(int c, int q4, int e) {
  if constexpr (INT8) {
    return 64 * (c >> 1) + 16 * q4 + 8 * (c & 1) + e;   // 16-byte loads carry 16 dims
  } else {
    return 32 * c + 8 * q4 + e;                         // 16-byte loads carry 8 dims
  }
}

__device__ __forceinline__ uint32_t i8pair_to_bf16(uint32_t w, int byte0) {
  const float a = (float)(int32_t)(int8_t)(w >> (8 * byte0));
  const float b = (float)(int32_t)(int8_t)(w >> (8 * byte0 + 8));
  return pack_bf16(a, b);
}

}  // namespace

template <bool INT8, bool ALIAS, int D, int MT, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
pa_mfma_kernel(const Params p) {
  constexpr int ROWS = 16 * MT;
  constexpr int C = D / 32;                           // contraction chunks of 32 dims
  constexpr int EB = INT8 ? 1 : 2;
  constexpr int ROW_BYTES = D * EB;
  constexpr int NLOAD = ROW_BYTES / 64;               // 16-byte loads per lane per tile
  static_assert(D % 64 == 0, "head_dim must be a multiple of 64");

  __shared__ float lds_acc[(NW > 1 ? NW - 1 : 1) * ROWS * D];
  __shared__ float lds_ml[NW * ROWS * 2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int q4 = lane >> 4;

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

  // Q^T as the B operand: lane l holds query row n (+16 per tile), 8 dims per chunk.
  bf16x8 qt[MT][C];
  int32_t row_lo[MT], row_hi[MT];
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
      if (live) v = load16(qrow + chunk_dim<INT8>(c, q4, 0) * 2);
      qt[tile][c] = __builtin_bit_cast(bf16x8, v);
    }
    row_lo[tile] = first_key(kr.p0, t, p.window);
    row_hi[tile] = live ? kr.p0 + t : -1;
  }

  // Identity B operand for the transposing product: lane l holds column n,
  // contraction rows 4*q4 .. 4*q4+3.
  i16x4 ident;
#pragma unroll
  for (int e = 0; e < 4; ++e) ident[e] = (4 * q4 + e == n) ? (short)0x3F80 : (short)0;

  f32x4 o[MT][C][2];
  float m[MT], l[MT];
#pragma unroll
  for (int tile = 0; tile < MT; ++tile) {
    m[tile] = -INFINITY;
    l[tile] = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) o[tile][c][0] = o[tile][c][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t tok_stride = (size_t)p.Hkv * ROW_BYTES;
  const char* kbase = reinterpret_cast<const char*>(p.k_pool) + (size_t)g * ROW_BYTES + n * tok_stride;
  const char* vbase = reinterpret_cast<const char*>(p.v_pool) + (size_t)g * ROW_BYTES + n * tok_stride;
  const int32_t* table = p.block_table + (size_t)b * p.maxb;
  int32_t* visits = p.visits ? p.visits + ((size_t)b * p.Hkv + g) * p.maxb : nullptr;

  for (int32_t i = first + wave; i <= last; i += NW) {
    const int32_t phys = table[i];
    const size_t blk_off = (size_t)phys * kBlock * tok_stride;
    uint4 kraw[NLOAD], vraw[NLOAD];
#pragma unroll
    for (int u = 0; u < NLOAD; ++u) kraw[u] = load16(kbase + blk_off + (INT8 ? 16 * q4 + 64 * u : 16 * q4 + 64 * u));
    if constexpr (!ALIAS) {
#pragma unroll
      for (int u = 0; u < NLOAD; ++u) vraw[u] = load16(vbase + blk_off + 16 * q4 + 64 * u);
    }
    float ksc[4], vsc[4];
    if constexpr (INT8) {
      const float* ks = p.k_scale + ((size_t)phys * kBlock + 4 * q4) * p.Hkv + g;
      const float* vs = p.v_scale + ((size_t)phys * kBlock + 4 * q4) * p.Hkv + g;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ksc[e] = ks[(size_t)e * p.Hkv];
        vsc[e] = vs[(size_t)e * p.Hkv];
      }
    }
    if (visits && lane == 0) atomicAdd(visits + i, 1);
    if constexpr (ALIAS) {
#pragma unroll
      for (int u = 0; u < NLOAD; ++u) vraw[u] = kraw[u];
    }

    // Rows nobody may see can hold anything: zero this lane's V row (lane = token n).
    {
      const int32_t j = i * kBlock + n;
      const bool ok = j < L && j >= kr.lo0;
#pragma unroll
      for (int u = 0; u < NLOAD; ++u) {
        vraw[u].x = ok ? vraw[u].x : 0u;
        vraw[u].y = ok ? vraw[u].y : 0u;
        vraw[u].z = ok ? vraw[u].z : 0u;
        vraw[u].w = ok ? vraw[u].w : 0u;
      }
    }

    // Operands of chunk c as bf16x8 (int8 caches are widened here).
    bf16x8 ka[C], va[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if constexpr (INT8) {
        const uint4 kw = kraw[c >> 1];
        const uint4 vw = vraw[c >> 1];
        const uint32_t k0 = (c & 1) ? kw.z : kw.x, k1 = (c & 1) ? kw.w : kw.y;
        const uint32_t v0 = (c & 1) ? vw.z : vw.x, v1 = (c & 1) ? vw.w : vw.y;
        uint4 kb = make_uint4(i8pair_to_bf16(k0, 0), i8pair_to_bf16(k0, 2), i8pair_to_bf16(k1, 0), i8pair_to_bf16(k1, 2));
        uint4 vb = make_uint4(i8pair_to_bf16(v0, 0), i8pair_to_bf16(v0, 2), i8pair_to_bf16(v1, 0), i8pair_to_bf16(v1, 2));
        ka[c] = __builtin_bit_cast(bf16x8, kb);
        va[c] = __builtin_bit_cast(bf16x8, vb);
      } else {
        ka[c] = __builtin_bit_cast(bf16x8, kraw[c]);
        va[c] = __builtin_bit_cast(bf16x8, vraw[c]);
      }
    }

    // Transpose the V tile on the matrix core: vt[c][hh] holds dim slot n, tokens 4*q4..4*q4+3.
    uint32_t vt[C][2][2];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint4 w = __builtin_bit_cast(uint4, va[c]);
        i16x4 a;
        const uint32_t w0 = hh ? w.z : w.x, w1 = hh ? w.w : w.y;
        a[0] = (short)(w0 & 0xFFFF); a[1] = (short)(w0 >> 16);
        a[2] = (short)(w1 & 0xFFFF); a[3] = (short)(w1 >> 16);
        const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ident, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        vt[c][hh][0] = pack_bf16(t[0], t[1]);
        vt[c][hh][1] = pack_bf16(t[2], t[3]);
      }

#pragma unroll
    for (int tile = 0; tile < MT; ++tile) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qt[tile][c], s, 0, 0, 0);

      // s[e] = score of query row n (+16*tile) against token 4*q4+e of block i.
      float sc[4];
      float mb = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int32_t j = i * kBlock + 4 * q4 + e;
        const bool ok = j <= row_hi[tile] && j >= row_lo[tile];
        float x = s[e] * p.scale_log2;
        if constexpr (INT8) x *= ksc[e];
        sc[e] = ok ? x : -INFINITY;
        mb = fmaxf(mb, sc[e]);
      }
      mb = quads16_max(mb);
      const float mn = fmaxf(m[tile], mb);
      const bool grow = mn > m[tile];
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float a = grow ? fast_exp2(m[tile] - mn) : 1.f;
        l[tile] *= a;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) o[tile][c][hh] *= a;
        m[tile] = mn;
      }
      const float msafe = m[tile] == -INFINITY ? 0.f : m[tile];
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = fast_exp2(sc[e] - msafe);
        l[tile] += pe[e];
        if constexpr (INT8) {
          const int32_t j = i * kBlock + 4 * q4 + e;
          const bool vis = j < L && j >= kr.lo0;
          pe[e] *= vis ? vsc[e] : 0.f;
        }
      }
      i16x4 pb;
      {
        const uint32_t p01 = pack_bf16(pe[0], pe[1]);
        const uint32_t p23 = pack_bf16(pe[2], pe[3]);
        pb[0] = (short)(p01 & 0xFFFF); pb[1] = (short)(p01 >> 16);
        pb[2] = (short)(p23 & 0xFFFF); pb[3] = (short)(p23 >> 16);
      }
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          i16x4 a;
          a[0] = (short)(vt[c][hh][0] & 0xFFFF); a[1] = (short)(vt[c][hh][0] >> 16);
          a[2] = (short)(vt[c][hh][1] & 0xFFFF); a[3] = (short)(vt[c][hh][1] >> 16);
          o[tile][c][hh] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[tile][c][hh], 0, 0, 0);
        }
    }
  }

  // Row sums: the four lanes of a row each hold a quarter of the tokens.
#pragma unroll
  for (int tile = 0; tile < MT; ++tile) l[tile] = quads16_sum(l[tile]);

  // Merge the wavefronts: waves 1..NW-1 park their state in LDS, wave 0 folds it in.
  if (wave > 0) {
#pragma unroll
    for (int tile = 0; tile < MT; ++tile) {
      const int r = n + 16 * tile;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            lds_acc[((wave - 1) * ROWS + r) * D + chunk_dim<INT8>(c, q4, 4 * hh + e)] = o[tile][c][hh][e];
      if (q4 == 0) {
        lds_ml[(wave * ROWS + r) * 2] = m[tile];
        lds_ml[(wave * ROWS + r) * 2 + 1] = l[tile];
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;

  const int32_t unit = b * p.Hkv + g;
#pragma unroll
  for (int tile = 0; tile < MT; ++tile) {
    const int r = n + 16 * tile;
    float M = m[tile];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, lds_ml[(w * ROWS + r) * 2]);
    const float Ms = M == -INFINITY ? 0.f : M;
    float wsc[NW];
    float den = 0.f;
    wsc[0] = fast_exp2(m[tile] - Ms);
    den = wsc[0] * l[tile];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      wsc[w] = fast_exp2(lds_ml[(w * ROWS + r) * 2] - Ms);
      den += wsc[w] * lds_ml[(w * ROWS + r) * 2 + 1];
    }
    if (r >= p.rows) continue;
    const int t = r / p.G;
    const int h = g * p.G + r % p.G;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float v[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = wsc[0] * o[tile][c][hh][e];
#pragma unroll
          for (int w = 1; w < NW; ++w)
            x += wsc[w] * lds_acc[((w - 1) * ROWS + r) * D + chunk_dim<INT8>(c, q4, 4 * hh + e)];
          v[4 * hh + e] = x;
        }
      const int d0 = chunk_dim<INT8>(c, q4, 0);
      if (p.splits > 1) {
        const size_t slot = ((size_t)unit * p.splits + split) * p.rows + r;
        float4* dst = reinterpret_cast<float4*>(p.ws_acc + slot * D + d0);
        dst[0] = make_float4(v[0], v[1], v[2], v[3]);
        dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        if (c == 0 && q4 == 0) {
          p.ws_ml[slot * 2] = M;
          p.ws_ml[slot * 2 + 1] = den;
        }
      } else {
        const float inv = 1.f / den;
        uint4 pk = make_uint4(pack_bf16(v[0] * inv, v[1] * inv), pack_bf16(v[2] * inv, v[3] * inv),
                              pack_bf16(v[4] * inv, v[5] * inv), pack_bf16(v[6] * inv, v[7] * inv));
        __bf16* out = reinterpret_cast<__bf16*>(p.out) + (((size_t)b * p.q_len + t) * p.Hq + h) * D + d0;
        *reinterpret_cast<uint4*>(out) = pk;
      }
    }
  }
}

namespace {
template <bool INT8, bool ALIAS, int D, int MT>
hipError_t launch_one(const Params& p, int nw, int grid, hipStream_t st, bool* ok) {
  *ok = true;
  switch (nw) {
    case 4: hipLaunchKernelGGL((pa_mfma_kernel<INT8, ALIAS, D, MT, 4>), dim3(grid), dim3(256), 0, st, p); break;
    default: *ok = false; return hipSuccess;
  }
  return hipGetLastError();
}

template <bool INT8, bool ALIAS>
hipError_t by_shape(const Params& p, int D, int mt, int nw, int grid, hipStream_t st, bool* ok) {
  *ok = false;
  if (mt == 1) {
    if (D == 64) return launch_one<INT8, ALIAS, 64, 1>(p, nw, grid, st, ok);
    if (D == 128) return launch_one<INT8, ALIAS, 128, 1>(p, nw, grid, st, ok);
    if (D == 256) return launch_one<INT8, ALIAS, 256, 1>(p, nw, grid, st, ok);
  } else if (mt == 2) {
    if (D == 64) return launch_one<INT8, ALIAS, 64, 2>(p, nw, grid, st, ok);
    if (D == 128) return launch_one<INT8, ALIAS, 128, 2>(p, nw, grid, st, ok);
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_mfma(const Params& p, int kv_dtype, int D, int row_tiles, int nw, int grid,
                       hipStream_t st, bool* supported) {
  *supported = false;
  const bool alias = p.v_pool == p.k_pool;
  if (kv_dtype == 2) {
    return alias ? by_shape<true, true>(p, D, row_tiles, nw, grid, st, supported)
                 : by_shape<true, false>(p, D, row_tiles, nw, grid, st, supported);
  }
  if (kv_dtype == 1) {
    return alias ? by_shape<false, true>(p, D, row_tiles, nw, grid, st, supported)
                 : by_shape<false, false>(p, D, row_tiles, nw, grid, st, supported);
  }
  return hipSuccess;
}

}  // namespace pa
