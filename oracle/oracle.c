/*
 * oracle.c -- fp64 CPU oracle for one paged decode-attention step.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the HIP kernels, and it never sees their
 * results. It is deliberately plain and slow: every output row is computed
 * on its own, straight from the definition, in double precision.
 *
 * What it computes, and where each piece is defined:
 *
 *  - Attention for a new query over the cache (CS336 lecture 10 study guide,
 *    the decode-attention equation): the query is compared with every cached
 *    key it may see, the new token's own key included; the scores are scaled
 *    (by 1/sqrt(d_h) there; here by the caller's `scale`), passed through a
 *    softmax, and the output is the softmax-weighted sum of the values.
 *  - Paged storage (tiniestgpt notes, "PagedAttention: why it is needed"):
 *    the cache is a pool k_cache[block][slot][head][dim]; block_table[seq][i]
 *    names the physical block that holds logical block i of a sequence.
 *  - Sliding window (Lab 5 Gemma4 handout, "Sliding Window Attention" and
 *    "Ring KV Cache"): a local layer lets a position see only the most recent
 *    W tokens. Reading used here: W keys including the query's own position,
 *    i.e. key j is visible from position p iff p - W < j <= p; a ring of W
 *    slots holds exactly these. window <= 0 means a global (causal) layer.
 *  - Grouped-query attention (Lab 5, "Grouped Query Attention"): query heads
 *    share KV heads in contiguous groups, head h reads KV head h / (Hq/Hkv),
 *    the mapping obtained by repeating each KV head Hq/Hkv times.
 *  - Causal multi-token step (tiniestgpt notes, "Speculative decoding"): a
 *    verify step feeds q_len tokens; query t sits at position L - q_len + t,
 *    where L (seq_lens[b]) already counts all q_len new tokens.
 *  - Prefill over a paged cache (Lab 5, "Flash Attention": causal
 *    attention for q_len > 1 with history already in the cache): with
 *    q_start set, sequence b brings q_start[b+1] - q_start[b] query tokens
 *    of its own, packed one sequence after another, and query t of b sits at
 *    L - (q_start[b+1] - q_start[b]) + t.
 *  - int8 cache (tiniestgpt notes, "Quantization" / KV cache quantization):
 *    codes are gathered first and then dequantized, value = code * scale,
 *    with one scale per token per KV head (per-token granularity) or one
 *    per KV head for the whole cache (per-head granularity).
 *  - Ring cache for window layers (Lab 5, "Ring KV Cache"): a sequence owns
 *    a fixed ring of ring_blocks blocks and position t lives in ring slot
 *    t mod (ring_blocks * block_size), so logical block i sits in table
 *    entry i mod ring_blocks; newer tokens overwrite ones that have left
 *    the window. The ring must hold window + q_len - 1 tokens so that a
 *    step's own writes spare every key its queries see.
 *
 * The softmax is taken in the textbook two-pass form: the largest score is
 * subtracted before exponentiating, then the weights are normalised by their
 * sum. Both steps are exact rewrites of softmax; no blocking, no running
 * rescale, no split of the key range.
 */
#include <math.h>
#include <stdint.h>
/* ORC_MUTANT selects one planted mistake for the tests that prove the pins
 * catch it; the library the tests, the smoke check and the benchmark use is
 * always built with ORC_MUTANT == 0. */
#ifndef ORC_MUTANT
#define ORC_MUTANT 0
#endif
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_I8 = 2 };

enum {
  ORC_OK = 0,
  ORC_ERR_ARG = 1,       /* bad shape / null pointer */
  ORC_ERR_DATA = 2,      /* seq_len or block id out of range */
  ORC_ERR_NOMEM = 3
};

typedef struct {
  const void* q;            /* [B][q_len][Hq][D], q_dtype */
  const void* k_pool;       /* [num_blocks][block_size][Hkv][D], kv_dtype */
  const void* v_pool;       /* same shape and dtype */
  const float* k_scale;     /* [num_blocks][Hkv][block_size], int8 only */
  const float* v_scale;     /* same */
  const int32_t* block_table; /* [B][max_blocks] */
  const int32_t* seq_lens;  /* [B] */
  int32_t q_dtype, kv_dtype;
  int32_t B, q_len, Hq, Hkv, D, block_size, num_blocks, max_blocks;
  int32_t window;
  double scale;
  int32_t ring_blocks;      /* 0: block_table row is linear; > 0: a ring of this many entries */
  int32_t head_scales;      /* int8 only: 0 scales per token [num_blocks][Hkv][block_size]; 1 per head [Hkv] */
  const int32_t* q_start;   /* NULL: every sequence has q_len queries, q is [B][q_len][Hq][D]. Else [B+1]
                               offsets: q (and out) are [q_start[B]][Hq][D], q_len is unused */
} orc_problem;

/* Query tokens of sequence b. */
static int32_t seq_queries(const orc_problem* P, int b) {
  return P->q_start ? P->q_start[b + 1] - P->q_start[b] : P->q_len;
}

/* Largest query count of any sequence (the ring must hold window + that - 1). */
static int32_t max_queries(const orc_problem* P) {
  int32_t m = P->q_start ? 0 : P->q_len;
  if (P->q_start)
    for (int b = 0; b < P->B; ++b)
      if (seq_queries(P, b) > m) m = seq_queries(P, b);
  return m;
}

/* One stored element, widened to double. bf16 is the upper half of a binary32. */
static double elem(const void* base, int dtype, size_t i) {
  if (dtype == ORC_F32) return (double)((const float*)base)[i];
  if (dtype == ORC_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const int8_t*)base)[i];
}

static int check_problem(const orc_problem* P) {
  if (!P || !P->q || !P->k_pool || !P->v_pool || !P->block_table || !P->seq_lens) return ORC_ERR_ARG;
  if (P->B < 0 || P->Hq < 1 || P->Hkv < 1 || P->D < 1) return ORC_ERR_ARG;
  if (!P->q_start && P->q_len < 1) return ORC_ERR_ARG;
  if (P->q_start) {
    if (P->q_start[0] != 0) return ORC_ERR_ARG;
    for (int b = 0; b < P->B; ++b)
      if (seq_queries(P, b) < 0) return ORC_ERR_ARG;
  }
  if (P->block_size < 1 || P->num_blocks < 1 || P->max_blocks < 1) return ORC_ERR_ARG;
  if (P->Hq % P->Hkv != 0) return ORC_ERR_ARG;
  if (P->q_dtype != ORC_F32 && P->q_dtype != ORC_BF16) return ORC_ERR_ARG;
  if (P->kv_dtype != ORC_F32 && P->kv_dtype != ORC_BF16 && P->kv_dtype != ORC_I8) return ORC_ERR_ARG;
  if (P->kv_dtype == ORC_I8 && (!P->k_scale || !P->v_scale)) return ORC_ERR_ARG;
  if (P->head_scales != 0 && P->head_scales != 1) return ORC_ERR_ARG;
  if (P->ring_blocks < 0) return ORC_ERR_ARG;
  if (P->ring_blocks > 0) {
    if (P->window <= 0 || P->ring_blocks > P->max_blocks) return ORC_ERR_ARG;
    if ((int64_t)P->ring_blocks * P->block_size < (int64_t)P->window + max_queries(P) - 1) return ORC_ERR_ARG;
  }
  for (int b = 0; b < P->B; ++b) {
    int32_t L = P->seq_lens[b];
    if (L < seq_queries(P, b) || L < 1) return ORC_ERR_DATA;
    if (P->ring_blocks == 0 && (int64_t)L > (int64_t)P->max_blocks * P->block_size) return ORC_ERR_DATA;
    int32_t used = (L + P->block_size - 1) / P->block_size;
    if (P->ring_blocks > 0 && used > P->ring_blocks) used = P->ring_blocks;
    for (int i = 0; i < used; ++i) {
      int32_t blk = P->block_table[(size_t)b * P->max_blocks + i];
      if (blk < 0 || blk >= P->num_blocks) return ORC_ERR_DATA;
    }
  }
  return ORC_OK;
}

/* Position of query token t of sequence b, and the first key it may see. */
static void query_span(const orc_problem* P, int b, int t, int32_t* first, int32_t* last) {
  int32_t L = P->seq_lens[b];
#if ORC_MUTANT == 3
  int32_t p = L - 1; (void)t;
#else
  int32_t p = L - seq_queries(P, b) + t;
#endif
  int32_t lo = 0;
  if (P->window > 0) {
#if ORC_MUTANT == 2
    lo = p - P->window;
#else
    lo = p - P->window + 1;
#endif
    if (lo < 0) lo = 0;
  }
  *first = lo;
  *last = p;
}

/* Table entry that holds key j: logical block j / block_size, or in a ring the
 * block of ring slot j mod (ring_blocks * block_size). */
static int32_t table_entry(const orc_problem* P, int32_t j) {
  if (P->ring_blocks == 0) return j / P->block_size;
#if ORC_MUTANT == 12
  return (j % P->window) / P->block_size;
#else
  return (j % (P->ring_blocks * P->block_size)) / P->block_size;
#endif
}

/* Element index of (key j, kv head g, dim 0) of sequence b, through the block table. */
static size_t key_row(const orc_problem* P, int b, int32_t j, int g) {
  int32_t blk = P->block_table[(size_t)b * P->max_blocks + table_entry(P, j)];
  int32_t slot = j % P->block_size;
#if ORC_MUTANT == 4
  return (((size_t)blk * P->Hkv + g) * P->block_size + slot) * (size_t)P->D;
#else
  return (((size_t)blk * P->block_size + slot) * P->Hkv + g) * (size_t)P->D;
#endif
}

/* Scale of key j, kv head g of sequence b: one float per (token, head), stored
 * [block][head][slot] so that a block's scales for one head are contiguous;
 * or, per-head granularity, one float per head. */
static double key_scale(const float* s, const orc_problem* P, int b, int32_t j, int g) {
  if (P->kv_dtype != ORC_I8) return 1.0;
#if ORC_MUTANT == 13
  if (P->head_scales) return (double)s[0];
#else
  if (P->head_scales) return (double)s[g];
#endif
  int32_t blk = P->block_table[(size_t)b * P->max_blocks + table_entry(P, j)];
  int32_t slot = j % P->block_size;
  return (double)s[((size_t)blk * P->Hkv + g) * P->block_size + slot];
}

/* One output row: (sequence b, query token t, query head h) -> out[0..D). */
static int attend_row(const orc_problem* P, int b, int t, int h, double* out, double* scores) {
  const int D = P->D;
#if ORC_MUTANT == 1
  const int g = h % P->Hkv;
#else
  const int g = h / (P->Hq / P->Hkv);
#endif
  int32_t lo, p;
  query_span(P, b, t, &lo, &p);
  const size_t qtok = P->q_start ? (size_t)P->q_start[b] + t : (size_t)b * P->q_len + t;
  const size_t qrow = (qtok * P->Hq + h) * (size_t)D;
  const int32_t n = p - lo + 1;

  for (int32_t j = lo; j <= p; ++j) {
    size_t kr = key_row(P, b, j, g);
    double ks = key_scale(P->k_scale, P, b, j, g);
    double dot = 0.0;
#if ORC_MUTANT == 8
    for (int d = 1; d < D; ++d) dot += elem(P->q, P->q_dtype, qrow + d) * (elem(P->k_pool, P->kv_dtype, kr + d) * ks);
#else
    for (int d = 0; d < D; ++d) dot += elem(P->q, P->q_dtype, qrow + d) * (elem(P->k_pool, P->kv_dtype, kr + d) * ks);
#endif
#if ORC_MUTANT == 5
    scores[j - lo] = dot;
#else
    scores[j - lo] = P->scale * dot;
#endif
  }
  double m = -INFINITY;
  for (int32_t i = 0; i < n; ++i)
    if (scores[i] > m) m = scores[i];
  double z = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    scores[i] = exp(scores[i] - m);
    z += scores[i];
  }
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int32_t j = lo; j <= p; ++j) {
    size_t vr = key_row(P, b, j, g);
#if ORC_MUTANT == 7
    double vs = key_scale(P->k_scale, P, b, j, g);
#else
    double vs = key_scale(P->v_scale, P, b, j, g);
#endif
    double w = scores[j - lo];
    for (int d = 0; d < D; ++d) out[d] += w * (elem(P->v_pool, P->kv_dtype, vr + d) * vs);
  }
#if ORC_MUTANT != 6
  for (int d = 0; d < D; ++d) out[d] /= z;
#else
  (void)z;
#endif
  return ORC_OK;
}

/*
 * Attention output in fp64.
 *   rows == NULL: every row, out is [B][q_len][Hq][D] ([q_start[B]][Hq][D] with q_start).
 *   rows != NULL: only the listed rows, row index r = (b*q_len + t)*Hq + h
 *                 ((q_start[b] + t)*Hq + h with q_start), out is [n_rows][D].
 * nthreads <= 0 uses the OpenMP default. Returns an ORC_* code.
 */
int oracle_attention(const orc_problem* P, const int64_t* rows, int64_t n_rows, double* out, int nthreads) {
  int rc = check_problem(P);
  if (rc != ORC_OK) return rc;
  if (!out) return ORC_ERR_ARG;
  const int64_t tokens = P->q_start ? (int64_t)P->q_start[P->B] : (int64_t)P->B * P->q_len;
  const int64_t total = tokens * P->Hq;
  const int64_t n = rows ? n_rows : total;
  if (rows) {
    for (int64_t i = 0; i < n_rows; ++i)
      if (rows[i] < 0 || rows[i] >= total) return ORC_ERR_ARG;
  }
  int32_t max_len = 1;
  for (int b = 0; b < P->B; ++b)
    if (P->seq_lens[b] > max_len) max_len = P->seq_lens[b];
  int err = ORC_OK;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)max_len);
    if (!scores) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      err = ORC_ERR_NOMEM;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
      for (int64_t i = 0; i < n; ++i) {
        int64_t r = rows ? rows[i] : i;
        int h = (int)(r % P->Hq);
        int64_t bt = r / P->Hq;
        int b, t;
        if (P->q_start) {   /* the sequence whose query range holds token bt */
          b = 0;
          while (P->q_start[b + 1] <= bt) ++b;
          t = (int)(bt - P->q_start[b]);
        } else {
          t = (int)(bt % P->q_len);
          b = (int)(bt / P->q_len);
        }
        attend_row(P, b, t, h, out + (size_t)i * P->D, scores);
      }
      free(scores);
    }
  }
  return err;
}

/* Number of threads oracle_attention would use for nthreads <= 0. */
int oracle_default_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Logical blocks that hold at least one key visible to at least one query
 * row of the sequence, counted per table entry: vis[b][e] = the number of
 * such logical blocks whose keys table entry e holds (vis is
 * [B][max_blocks]). A linear table gives 0 or 1; in a ring, the entry that
 * holds both the oldest and the newest keys of the window counts 2. Found by
 * listing every visible key.
 */
int oracle_visited_blocks(const orc_problem* P, int32_t* vis) {
  int rc = check_problem(P);
  if (rc != ORC_OK) return rc;
  if (!vis) return ORC_ERR_ARG;
  memset(vis, 0, sizeof(int32_t) * (size_t)P->B * P->max_blocks);
  for (int b = 0; b < P->B; ++b) {
    const int32_t L = P->seq_lens[b];
    const int32_t nlog = (L + P->block_size - 1) / P->block_size;
    uint8_t* seen = (uint8_t*)calloc((size_t)nlog, 1);
    if (!seen) return ORC_ERR_NOMEM;
    for (int t = 0; t < seq_queries(P, b); ++t) {
      int32_t lo, p;
      query_span(P, b, t, &lo, &p);
      for (int32_t j = lo; j <= p; ++j) seen[j / P->block_size] = 1;
    }
    for (int32_t i = 0; i < nlog; ++i)
      if (seen[i]) vis[(size_t)b * P->max_blocks + table_entry(P, i * P->block_size)] += 1;
    free(seen);
  }
  return ORC_OK;
}

/*
 * Raw bytes of the keys (which == 0) or values (which == 1) that some query
 * row of each sequence can see, in increasing key order, all KV heads:
 * dst is [B][dst_tokens][Hkv][D] elements of the cache type; for sequence b,
 * entry w holds key first(b) + w where first(b) is the first key visible to
 * query token 0. Entries past the visible range are left untouched.
 */
int oracle_gather(const orc_problem* P, int which, void* dst, int64_t dst_tokens) {
  int rc = check_problem(P);
  if (rc != ORC_OK) return rc;
  if (!dst || (which != 0 && which != 1) || dst_tokens < 0) return ORC_ERR_ARG;
  const void* pool = which == 0 ? P->k_pool : P->v_pool;
  const size_t esz = P->kv_dtype == ORC_F32 ? 4 : (P->kv_dtype == ORC_BF16 ? 2 : 1);
  const size_t row_bytes = esz * (size_t)P->D;
  for (int b = 0; b < P->B; ++b) {
    int32_t lo0, p0, lo_last, p_last;
    if (seq_queries(P, b) < 1) continue;
    query_span(P, b, 0, &lo0, &p0);
    query_span(P, b, seq_queries(P, b) - 1, &lo_last, &p_last);
    if ((int64_t)(p_last - lo0 + 1) > dst_tokens) return ORC_ERR_ARG;
    for (int32_t j = lo0; j <= p_last; ++j)
      for (int g = 0; g < P->Hkv; ++g) {
        size_t src = key_row(P, b, j, g) * esz;
        size_t off = ((((size_t)b * dst_tokens) + (size_t)(j - lo0)) * P->Hkv + g) * row_bytes;
        memcpy((char*)dst + off, (const char*)pool + src, row_bytes);
      }
  }
  return ORC_OK;
}

/*
 * KV append: the rows of this step's new tokens go into the paged pools
 * (tiniestgpt notes, "PagedAttention": pool[block][slot][head][dim], the
 * step's tokens addressed by their slot ids; "Quantization", KV cache
 * quantization: one scale per token per KV head).
 *   slot_ids[t] = physical_block * block_size + slot; t is skipped if < 0.
 *   Float caches take the rows unchanged (src dtype == cache dtype).
 *   An int8 cache takes, per (token, KV head), scale = max_d |x_d| / 127
 *   (1 for an all-zero row) and codes rint(x_d / scale) clamped to
 *   [-127, 127], in binary32 with round-half-even -- the quantizer of the
 *   input recipe, in the precision its integer codes are decided in.
 *   Scales are stored [num_blocks][Hkv][block_size].
 *   Per-head granularity (tiniestgpt notes: per_head, a smaller scale
 *   table): the scale of head g is given, s[g]; the codes are
 *   rint(x_d / s[g]) clamped to [-127, 127] and no scale is written.
 */
typedef struct {
  const void* k_new;        /* [T][Hkv][D], src dtype */
  const void* v_new;        /* same */
  const int64_t* slot_ids;  /* [T] */
  void* k_pool;             /* [num_blocks][block_size][Hkv][D], kv dtype */
  void* v_pool;             /* same */
  float* k_scale;           /* [num_blocks][Hkv][block_size], int8 only */
  float* v_scale;           /* same */
  int32_t src_dtype, kv_dtype;
  int32_t T, Hkv, D, block_size, num_blocks;
  int32_t head_scales;      /* int8 only: 1 -> k_scale / v_scale are [Hkv], given, read only */
} orc_write;

/* One element of a float source row as binary32 (bf16 widens exactly). */
static float src_elem(const void* base, int dtype, size_t i) {
  if (dtype == ORC_F32) return ((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

static void write_row(const orc_write* W, const void* src, void* pool, float* scales, int64_t t, int g,
                      int32_t blk, int32_t slot) {
  const int D = W->D;
  const size_t in = ((size_t)t * W->Hkv + g) * (size_t)D;
  const size_t at = (((size_t)blk * W->block_size + slot) * W->Hkv + g) * (size_t)D;
  if (W->kv_dtype != ORC_I8) {
    const size_t esz = W->kv_dtype == ORC_F32 ? 4 : 2;
    memcpy((char*)pool + at * esz, (const char*)src + in * esz, esz * (size_t)D);
    return;
  }
  float scale;
  if (W->head_scales) {
#if ORC_MUTANT == 14
    scale = scales[0];
#else
    scale = scales[g];
#endif
  } else {
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
      float a = fabsf(src_elem(src, W->src_dtype, in + d));
      if (a > amax) amax = a;
    }
#if ORC_MUTANT == 9
    scale = amax > 0.0f ? amax / 128.0f : 1.0f;
#else
    scale = amax > 0.0f ? amax / 127.0f : 1.0f;
#endif
  }
  int8_t* codes = (int8_t*)pool + at;
  for (int d = 0; d < D; ++d) {
#if ORC_MUTANT == 10
    float c = truncf(src_elem(src, W->src_dtype, in + d) / scale);
#else
    float c = rintf(src_elem(src, W->src_dtype, in + d) / scale);   /* default rounding: to nearest, ties even */
#endif
    if (c > 127.0f) c = 127.0f;
    if (c < -127.0f) c = -127.0f;
    codes[d] = (int8_t)c;
  }
  if (W->head_scales) return;
#if ORC_MUTANT == 11
  scales[((size_t)blk * W->block_size + slot) * W->Hkv + g] = scale;
#else
  scales[((size_t)blk * W->Hkv + g) * W->block_size + slot] = scale;
#endif
}

int oracle_cache_write(const orc_write* W) {
  if (!W || !W->k_new || !W->v_new || !W->slot_ids || !W->k_pool || !W->v_pool) return ORC_ERR_ARG;
  if (W->T < 0 || W->Hkv < 1 || W->D < 1 || W->block_size < 1 || W->num_blocks < 1) return ORC_ERR_ARG;
  if (W->src_dtype != ORC_F32 && W->src_dtype != ORC_BF16) return ORC_ERR_ARG;
  if (W->head_scales != 0 && (W->head_scales != 1 || W->kv_dtype != ORC_I8)) return ORC_ERR_ARG;
  if (W->kv_dtype == ORC_I8) {
    if (!W->k_scale || !W->v_scale) return ORC_ERR_ARG;
  } else if (W->kv_dtype != W->src_dtype) {
    return ORC_ERR_ARG;
  }
  const int64_t slots = (int64_t)W->num_blocks * W->block_size;
  for (int64_t t = 0; t < W->T; ++t)
    if (W->slot_ids[t] >= slots) return ORC_ERR_DATA;
  for (int64_t t = 0; t < W->T; ++t) {
    const int64_t s = W->slot_ids[t];
    if (s < 0) continue;
    const int32_t blk = (int32_t)(s / W->block_size), slot = (int32_t)(s % W->block_size);
    for (int g = 0; g < W->Hkv; ++g) {
      write_row(W, W->k_new, W->k_pool, W->k_scale, t, g, blk, slot);
      write_row(W, W->v_new, W->v_pool, W->v_scale, t, g, blk, slot);
    }
  }
  return ORC_OK;
}

