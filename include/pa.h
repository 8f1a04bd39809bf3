/*
 * pa.h -- paged decode attention on AMD Instinct MI355X (gfx950).
 *
 * One attention step of a decoder over a paged KV cache: every query token
 * gathers its sequence's keys and values through a block table, takes the
 * softmax of its scaled dot products with the keys it may see, and returns
 * the weighted sum of the matching values.
 *
 *   - Cache layout (tiniestgpt inference notes, "PagedAttention: why it is
 *     needed"): a physical pool k_cache[block][slot][head][dim] and a table
 *     block_table[seq][i] naming the physical block of logical block i.
 *   - The operation (CS336 lecture 10 study guide, decode-attention
 *     equation): a = softmax(q [K_1..K_n]^T * scale), y = a [V_1..V_n]; the
 *     step's own key and value are already in the cache.
 *   - Grouped-query attention (Lab 5 Gemma4 handout, "Grouped Query
 *     Attention"): query head h reads KV head h / (Hq / Hkv); KV heads are
 *     never copied per query head.
 *   - Sliding window (Lab 5, "Sliding Window Attention" and "Ring KV Cache"):
 *     with window W > 0 a query at position p sees keys p-W < j <= p, the W
 *     most recent tokens including itself. Blocks holding no such key are
 *     never loaded (the handout's "skip out-of-window blocks rather than
 *     compute then mask").
 *   - int8 cache (tiniestgpt notes, "Quantization", KV cache quantization):
 *     the same interface; codes are gathered first and dequantized after
 *     the gather, value = code * scale, one fp32 scale per token per KV head.
 *   - Verify step (tiniestgpt notes, "Speculative decoding"): q_len tokens
 *     of one sequence at once, causal among themselves.
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or keeps them. Arrays are dense and
 *     row-major in the shapes given below.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *     stream). A return of PA_OK means the work was enqueued; device-side
 *     data errors are not detected (see the preconditions).
 *   - The library keeps no state between calls except a per-device cache of
 *     the compute-unit count, and reads no environment variable: the launch
 *     plan depends only on the arguments (pa_args.tuning overrides it
 *     explicitly). It is safe to call from several host threads.
 *   - On failure the entry point returns a PA_ERR_* code, enqueues nothing,
 *     and pa_last_error() returns a message for the calling thread.
 *
 * Preconditions on device data (not checked by the kernels):
 *   q_len <= seq_lens[b] <= max_seq_len <= max_blocks_per_seq * block_size,
 *   and block_table[b][i] in [0, num_blocks) for every logical block i that
 *   holds a key visible to some query of sequence b. Other table entries
 *   and cache slots past seq_lens[b] are never read.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* pa_stream_t; /* a hipStream_t */
typedef struct ihipEvent_t* pa_event_t;   /* a hipEvent_t */

/* Element types. q and out share one type; the cache may be int8. */
enum { PA_F32 = 0, PA_BF16 = 1, PA_INT8 = 2 };

/* Return codes. */
enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, bad shape, Hq % Hkv != 0, q_len rule broken, non-finite scale */
  PA_ERR_UNSUPPORTED = 2, /* head_dim / block_size / dtype / group combination not built */
  PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than pa_workspace_size() */
  PA_ERR_HIP = 4,         /* the HIP runtime reported an error while enqueuing */
  PA_ERR_NO_BLOCKS = 5    /* block allocator (pa_alloc.h): too few free blocks; nothing changed */
};

/*
 * Explicit overrides of the launch plan, for tests and tuning experiments
 * (pa_args.tuning). A zero field keeps the library's own choice; every
 * partition computes the same attention up to floating-point rounding order.
 * A request the chosen kernel cannot honour returns PA_ERR_UNSUPPORTED.
 */
enum {
  PA_PART_AUTO = 0,      /* the library's choice */
  PA_PART_ALIGNED = 1,   /* each workgroup owns one aligned split of one (sequence, KV head) */
  PA_PART_LIST = 2,      /* matrix-core kernel: equal shares of the flattened (sequence, KV head, block) list,
                            each unit charged tuning.segment_blocks blocks beyond its own */
  PA_PART_PIECES = 3,    /* matrix-core kernel: units cut into near-equal pieces, one per workgroup */
  PA_PART_QUEUE = 4      /* matrix-core kernel: pieces handed out through the workspace queue, largest
                            first */
};

typedef struct {
  int32_t waves;              /* wavefronts per workgroup: 4 or 8 (also 2 for the matrix-core kernel); 0 auto */
  int32_t blocks_per_wave;    /* aligned splits without num_splits: blocks per wavefront per split; 0 auto */
  int32_t partition;          /* PA_PART_* */
  int32_t pieces_per_wg;      /* PA_PART_QUEUE: pieces per workgroup the queue aims for, 1..64; 0 auto
                                 (the plan then keeps at least two pieces per unit; an explicit count
                                 at least one) */
  int32_t oversub;            /* list / piece partitions: workgroups per resident slot, 1..64; 0 auto */
  int32_t segment_blocks;     /* list partition: what one more segment (a unit a workgroup's share
                                 starts in or crosses into) costs, in blocks of streaming: each
                                 unit counts as its blocks plus this many; 1..4096, -1 none (equal
                                 blocks per workgroup), 0 auto */
} pa_tuning;

typedef struct {
  void* out;                  /* [B][q_len][Hq][D], q_dtype */
  const void* q;              /* [B][q_len][Hq][D], q_dtype */
  const void* k_pool;         /* [num_blocks][block_size][Hkv][D], kv_dtype */
  const void* v_pool;         /* same shape; may equal k_pool (keys and values shared, read once) */
  const float* k_scale;       /* int8 cache only: [num_blocks][Hkv][block_size], one fp32 per (token,
                                 KV head), a block's 16 scales of one head contiguous; or [Hkv],
                                 one per KV head, when scale_per_head is 1; else NULL */
  const float* v_scale;       /* int8 cache only: same shape; else NULL. When v_pool == k_pool the
                                 values are the keys, so v_scale must equal k_scale. With separate
                                 pools every V scale a step reads must be below 255 in magnitude:
                                 each weight (at most 2^8) times its value scale reaches the matrix
                                 cores as one f16 value (pa_validate flags larger ones) */
  const int32_t* block_table; /* [B][max_blocks_per_seq] physical block ids; with ring_blocks > 0 each
                                 row's first ring_blocks entries form the sequence's ring */
  const int32_t* seq_lens;    /* [B] cached tokens per sequence, this step's q_len tokens included */
  int32_t num_seqs;           /* B >= 0 (B == 0 enqueues nothing) */
  int32_t q_len;              /* query tokens per sequence; query t sits at position seq_len - q_len + t */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv, divides Hq */
  int32_t head_dim;           /* D: 64, 128 or 256 */
  int32_t block_size;         /* tokens per cache block: 16 */
  int32_t num_blocks;         /* blocks in each pool */
  int32_t max_blocks_per_seq; /* row length of block_table */
  int32_t max_seq_len;        /* host-side upper bound on seq_lens[]; sizes the launch, no device sync
                                 (at most max_blocks_per_seq * block_size unless ring_blocks > 0) */
  int32_t window;             /* <= 0: every earlier key; > 0: the W most recent keys */
  float scale;                /* multiplies q.k before the softmax (1/sqrt(D) for standard attention) */
  int32_t q_dtype;            /* PA_F32 or PA_BF16 (also the output type) */
  int32_t kv_dtype;           /* PA_F32, PA_BF16 or PA_INT8 */
  int32_t num_splits;         /* 0: the library picks the context split; > 0: split each sequence's
                                 key range into this many parts (more if a part would exceed
                                 64 blocks per wavefront of the chosen kernel) */
  void* workspace;            /* device scratch for split partials and the piece queue,
                                 caller-owned, 16-byte aligned; may be NULL when
                                 pa_workspace_size() returns 0. Its first 4096 bytes must be
                                 zero before the first call that uses it; every call leaves
                                 them zero again, so one zero-fill at allocation is enough.
                                 Calls that share a workspace must not run concurrently. */
  size_t workspace_bytes;     /* size of workspace */
  int32_t* debug_visits;      /* NULL, or [B][Hkv][max_blocks_per_seq] zeroed by the caller: the
                                 kernels add 1 for every (sequence, KV head, logical block) they load */
  pa_event_t timing_start;    /* NULL, or a timing-enabled event: stamped when the attention kernel starts */
  pa_event_t timing_stop;     /* NULL, or a timing-enabled event: stamped when it completes (before any combine
                                 kernel). Both come from the kernel's own dispatch (hipExtLaunchKernel), so
                                 their interval is the kernel's execution time with no marker overhead. */
  int32_t ring_blocks;        /* 0: logical block i of a sequence is table entry i. > 0: ring cache for a
                                 window layer (Lab 5, "Ring KV Cache"): position t lives in ring slot
                                 t mod (ring_blocks * block_size), so logical block i is entry
                                 i mod ring_blocks. Needs window > 0, ring_blocks <= max_blocks_per_seq and
                                 ring_blocks * block_size >= window + q_len - 1 (a step's own keys must
                                 not overwrite keys its queries see). debug_visits then counts per
                                 table entry. */
  int32_t scale_per_head;     /* int8 caches: 0 scales per token (k_scale layout above); 1 one scale
                                 per KV head for the whole cache, k_scale / v_scale [Hkv] (tiniestgpt
                                 notes, "Quantization": per_head granularity, a smaller scale table) */
  const pa_tuning* tuning;    /* NULL: the library's launch plan; else explicit overrides (host memory,
                                 read during the call only) */
  void* debug_stamps;         /* NULL, or (a library built with -DPA_STAMPS, libpa_stamps.so) a device
                                 buffer of grid x 64 uint64 that the matrix-core kernel fills with the
                                 real-time counter at each workgroup's phases (slot 0 entry, 1 partition
                                 known, 2 exit, 3 segment count, then per segment s at 4 + 4s: start,
                                 first block consumed, block loop done, result written). The release
                                 library never writes it. */
} pa_args;

/* Plan the library would use for these arguments (informational). */
typedef struct {
  int32_t kernel;             /* 0: vector-ALU kernel, 1: matrix-core (MFMA) kernel */
  int32_t rows;               /* query rows per KV head = (Hq/Hkv) * q_len */
  int32_t waves_per_group;    /* wavefronts cooperating on one (sequence, KV head, split) */
  int32_t splits;             /* aligned partition: context splits per sequence (1: no combine kernel) */
  int32_t blocks_per_split;   /* aligned partition: logical blocks per split */
  int32_t grid;               /* workgroups of the attention kernel */
  int32_t balanced;           /* 0: each workgroup owns one split of one (sequence, KV head);
                                 1: every workgroup takes an equal share of the flattened
                                 (sequence, KV head, block) list, cut where a unit ends,
                                 each unit counted segment_blocks blocks longer;
                                 2: units are cut into near-equal pieces, one per workgroup
                                 or (queue != 0) handed out largest first to the workgroups
                                 in turn */
  int32_t pieces;             /* partition 2: most pieces the partition can produce */
  int32_t queue;              /* partition 2: 1 if pieces go out through the workspace queue */
  int32_t segment_blocks;     /* partition 1: blocks each unit is charged beyond its own (0: none) */
  size_t workspace_bytes;     /* == pa_workspace_size() */
} pa_plan_info;

/*
 * Bytes of workspace the call needs for these arguments (0 when the key
 * range is not split). Depends on the shapes, max_seq_len, window,
 * num_splits, tuning and the device's compute-unit count; never on device
 * data. Returns (size_t)-1 if the arguments are invalid.
 */
size_t pa_workspace_size(const pa_args* args);

/* Fill *info with the plan for args. Returns a PA_* code. */
int pa_plan(const pa_args* args, pa_plan_info* info);

/*
 * Single-token decode step (q_len must be 1) over an fp32 or bf16 cache;
 * kv_dtype must equal q_dtype. Defined by the decode-attention equation of
 * the CS336 lecture 10 study guide with the paging, GQA and window rules
 * above.
 */
int pa_decode(const pa_args* args, pa_stream_t stream);

/*
 * Single-token decode step (q_len must be 1) over an int8 cache with
 * per-token, per-KV-head fp32 scales (tiniestgpt notes, KV cache
 * quantization: gather the int8 codes, then dequantize). q_dtype must be
 * PA_BF16, kv_dtype PA_INT8, and k_scale / v_scale non-NULL; with separate
 * K and V pools the value scales must stay below 255 (see v_scale).
 */
int pa_decode_int8(const pa_args* args, pa_stream_t stream);

/*
 * Multi-token verify step, q_len >= 1 (tiniestgpt notes, "Speculative
 * decoding": the target model scores the last known token plus the drafts
 * in one pass). Query t of sequence b sits at position seq_lens[b]-q_len+t
 * and sees keys up to and including its own position (and, with a window,
 * only the W most recent of them). Any supported cache type.
 */
int pa_verify(const pa_args* args, pa_stream_t stream);

/*
 * pa_verify without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc. Same arguments, kernels and results as pa_verify,
 * except that args->workspace must be NULL and workspace_bytes 0: the split
 * partials, prefix sums and piece queue go to a static device array of the
 * library, 64 MiB per GPU, held from the first use on a GPU until the
 * process ends. A call whose plan needs more (pa_workspace_size() >
 * 67108864) returns PA_ERR_WORKSPACE and enqueues nothing. Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other host
 * threads, other streams) race and must be ordered by the caller. The queue
 * counters are cleared by a small kernel on `stream` before a call that
 * uses them. The call itself allocates nothing; its first call on a device
 * looks up the array's address there (hipGetSymbolAddress).
 */
int pa_verify_noalloc(const pa_args* args, pa_stream_t stream);

/*
 * Debug: copy the raw cache rows that the attention kernels would load
 * (which = 0: keys, 1: values) into dst, [B][dst_tokens][Hkv][D] elements of
 * kv_dtype. Entry w of sequence b holds key first(b)+w, first(b) being the
 * first key visible to query token 0; entries past seq_lens[b]-1 are left
 * untouched. It computes the key range, the table entry of a logical
 * block and a row's pool address with the device functions the attention,
 * prefill and append kernels use for theirs (the tile of a (block, KV head)
 * and the stride from one token's row to the next), so a bit-exact
 * comparison checks that shared addressing; the order in which a kernel's
 * lanes read the rows of a tile is checked by the poisoned parity tests.
 * dst_tokens must be >= window + q_len - 1 (window > 0) or >= max_seq_len.
 */
int pa_debug_gather(const pa_args* args, int32_t which, void* dst, int64_t dst_tokens,
                    pa_stream_t stream);

/* Status bits written by pa_validate. */
enum {
  PA_BAD_LEN_SHORT = 1, /* seq_len < q_len */
  PA_BAD_LEN_LONG = 2,  /* seq_len > max_seq_len, or (linear table) > max_blocks_per_seq * block_size */
  PA_BAD_BLOCK = 4,     /* a table entry the step would read is outside [0, num_blocks) */
  PA_BAD_SCALE = 8,     /* int8: a K or V scale of a key the step sees is NaN or infinite */
  PA_BIG_V_SCALE = 16,  /* int8: a V scale of a key the step sees is 255 or more in magnitude; only
                           decode over a shared K/V pool takes it (see pa_args.v_scale and
                           pa_prefill's v_scale) */
  PA_BAD_WORKSPACE = 32 /* (entry 0 only) the call would hand pieces out through the workspace queue
                           and the queue's counters in the workspace header are not zero */
};

/*
 * Check on the device the preconditions the attention kernels trust (the
 * sequence lengths and the block-table entries a step reads; tiniestgpt
 * notes, "PagedAttention": block_table[seq][i] names a block of the pool).
 * d_status: device int32 [num_seqs + 1]. Entry 1 + b receives the PA_BAD_*
 * bits of sequence b (0 when it is fine); entry 0 receives the OR of all
 * of them and must be zero before the call. Only table entries inside each
 * row are read, whatever the lengths say. For an int8 cache with both scale
 * arrays given, the scales of the keys some query of the step sees
 * (positions max(0, L - q_len - window + 1) .. L - 1 with a window, else
 * 0 .. L - 1; only those in valid blocks) are checked as well; scales of
 * other slots are never used and may hold anything. Without a window this
 * covers every key of a pa_prefill chunk that ends at L. When the plan for
 * these arguments hands pieces out through the workspace queue and a
 * workspace is given, its header's queue counters are checked too
 * (PA_BAD_WORKSPACE in entry 0). Same argument rules as pa_verify (q and
 * out must be non-NULL but are not read). Asynchronous on stream.
 */
int pa_validate(const pa_args* args, int32_t* d_status, pa_stream_t stream);

/*
 * KV append: write this step's new key and value rows into the paged pools
 * (tiniestgpt notes, "PagedAttention": the pool is [block][slot][head][dim]
 * and a step's tokens are addressed by slot ids; "Quantization", KV cache
 * quantization, per-token granularity: one scale per token per KV head).
 */
typedef struct {
  const void* k_new;          /* [num_tokens][Hkv][D], src_dtype */
  const void* v_new;          /* same shape and dtype; must equal k_new when v_pool == k_pool */
  const int64_t* slot_ids;    /* [num_tokens]: physical_block * block_size + slot. A negative id skips
                                 the token; an id >= num_blocks * block_size is a precondition
                                 violation and is never written (the token is skipped) */
  void* k_pool;               /* [num_blocks][block_size][Hkv][D], kv_dtype */
  void* v_pool;               /* same; may equal k_pool (then the rows are written once) */
  float* k_scale;             /* int8 cache only: [num_blocks][Hkv][block_size]; else NULL */
  float* v_scale;             /* int8 cache only: same; else NULL. Must equal k_scale when v_pool == k_pool */
  int32_t num_tokens;         /* T >= 0 (0 enqueues nothing) */
  int32_t num_kv_heads;       /* Hkv */
  int32_t head_dim;           /* D: 64, 128 or 256 */
  int32_t block_size;         /* 16 */
  int32_t num_blocks;         /* blocks in each pool */
  int32_t src_dtype;          /* PA_F32 or PA_BF16 */
  int32_t kv_dtype;           /* PA_INT8, or the same float type as src_dtype */
  pa_event_t timing_start;    /* NULL, or a timing-enabled event stamped when the append kernel starts */
  pa_event_t timing_stop;     /* NULL, or one stamped when it completes (the kernel's own dispatch) */
  int32_t scale_per_head;     /* int8 cache: 0 per-token scales, computed and written as above; 1 the
                                 given per-head scales k_scale / v_scale [Hkv] (read only): codes are
                                 rint(x / s[head]) clamped to [-127, 127]. Scales must be finite, > 0. */
} pa_write_args;

/*
 * Write the rows. A float cache receives them unchanged. An int8 cache
 * receives, per (token, KV head), scale = max_d |x_d| / 127 (1 for an
 * all-zero row) and codes rint(x_d / scale) clamped to [-127, 127], in IEEE
 * binary32 with round-half-even, and the scale at k_scale[block][head][slot].
 * Tokens whose slots repeat within one call race (one of them wins). All
 * pointers are device pointers owned by the caller; rows and pools 16-byte
 * aligned, slot ids and scales 8-byte aligned; asynchronous on stream.
 * Returns PA_OK, PA_ERR_INVALID_ARG (null pointer with num_tokens > 0,
 * misaligned pointer, dtype mismatch, aliased pools with different rows),
 * PA_ERR_UNSUPPORTED
 * (head_dim / block_size / dtype not built) or PA_ERR_HIP.
 */
int pa_cache_write(const pa_write_args* args, pa_stream_t stream);

/*
 * Paged prefill: a chunk of query tokens per sequence, causal among
 * themselves, over the sequence's history already in the cache (Lab 5,
 * "Flash Attention": q_len > 1 with cached history, global and window
 * layers, GQA without repeating K/V, key blocks outside a query tile's
 * causal and window range never loaded). The chunk's own keys and values
 * must be in the cache first (pa_cache_write). Sequence b brings
 * q_start[b+1] - q_start[b] >= 0 query tokens, packed one sequence after
 * another; its query t sits at position seq_lens[b] - (q_start[b+1] -
 * q_start[b]) + t and sees keys j with j <= position (and position - j <
 * window when window > 0).
 */
typedef struct {
  void* out;                  /* [total_q][Hq][D] bf16 */
  const void* q;              /* [total_q][Hq][D] bf16 */
  const int32_t* q_start;     /* [num_seqs + 1] device int32, q_start[0] = 0, non-decreasing,
                                 q_start[num_seqs] = total_q */
  const void* k_pool;         /* [num_blocks][block_size][Hkv][D], bf16 or int8 */
  const void* v_pool;         /* same; may equal k_pool */
  const float* k_scale;       /* int8 only: as in pa_args (per token, or per head with scale_per_head) */
  const float* v_scale;       /* int8 only (equal to k_scale when v_pool == k_pool): every value
                                 scale the chunk's keys use must be below 255
                                 (dequantized values below ~32500 in magnitude): the kernel hands
                                 each softmax weight (<= 256) times its value scale to the matrix
                                 cores as one f16 value; larger scales overflow it */
  const int32_t* block_table; /* [B][max_blocks_per_seq]; ring rows with ring_blocks > 0 */
  const int32_t* seq_lens;    /* [B] cached tokens, this chunk's included; >= the chunk's length */
  int32_t num_seqs;           /* B >= 0 */
  int32_t total_q;            /* q_start[B] (host copy; sizes nothing on the device) */
  int32_t max_q_len;          /* host upper bound on any sequence's query count; sizes the grid */
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* Hkv; Hq / Hkv <= 128 (64 at head_dim 256) */
  int32_t head_dim;           /* 64, 128 or 256 */
  int32_t block_size;         /* 16 */
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_seq_len;        /* host upper bound on seq_lens[] */
  int32_t window;             /* <= 0: every earlier key; > 0: the W most recent keys */
  float scale;                /* multiplies q.k */
  int32_t q_dtype;            /* PA_BF16 */
  int32_t kv_dtype;           /* PA_BF16 or PA_INT8 */
  int32_t ring_blocks;        /* as in pa_args; the ring must hold window + max_q_len - 1 keys */
  int32_t scale_per_head;     /* as in pa_args */
  pa_event_t timing_start;    /* NULL, or an event stamped when the prefill kernel starts */
  pa_event_t timing_stop;     /* NULL, or one stamped when it completes */
} pa_prefill_args;

/* Enqueue the prefill attention on stream. Returns PA_OK, PA_ERR_INVALID_ARG
 * (NULL pointer, bad sizes, a ring too small for the chunk, misaligned
 * pointers: q, out and the pools must be 16-byte aligned), PA_ERR_UNSUPPORTED
 * (fp32, head_dim, block_size, or a query group too large) or PA_ERR_HIP.
 * Sequences whose q_start range is empty write nothing. */
int pa_prefill(const pa_prefill_args* args, pa_stream_t stream);

/* Static description of a return code. */
const char* pa_strerror(int code);

/* Message describing the calling thread's most recent failure ("" if none). */
const char* pa_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int pa_version(void);

/* Identifier of the sources this library was built from: 16 hex digits of
 * a SHA-256 over the C/HIP sources and headers, computed by the build. A
 * binding that has the sources can compare it with their current hash and
 * refuse a library built from other sources. */
const char* pa_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
