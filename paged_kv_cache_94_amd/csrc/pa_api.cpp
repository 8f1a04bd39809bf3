// pa_api.cpp -- the C entry points declared in include/pa.h: argument
// checks, the launch plan (kernel family, context splits, workspace) and
// the launches. Host code only; the kernels live in the .hip files.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "pa.h"
#include "pa_common.h"
#include "pa_error.h"
#include "pa_prefill.h"
#include "pa_write.h"

namespace {

using pa::fail;

// Compute units per device, looked up once per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

using pa::kWsHeader;

struct Plan {
  int kernel = 0;       // 0 valu, 1 mfma
  int rows = 0;         // G * q_len
  int rows_t = 0;       // compiled rows (valu) or 16 * row tiles (mfma)
  int row_tiles = 0;
  int nw = 4;
  int splits = 1;
  int bps = 1;
  int n_blk_max = 0;
  int balanced = 0;     // 1: flattened-list partition, 2: piece partition (both over nwg workgroups)
  int nwg = 0;
  int64_t pieces = 0;   // piece partition: pieces aimed for
  bool queue = false;   // piece partition: pieces handed out through the workspace queue
  int seg_blocks = 0;   // list partition: blocks each unit is charged beyond its own
  int64_t slots = 0;    // workspace partial slots
  int64_t grid = 0;
  size_t ws_bytes = 0;
};


enum Entry { kDecode, kDecodeInt8, kVerify, kAny, kGather };

int validate(const pa_args* a, Entry entry) {
  if (!a) return fail(PA_ERR_INVALID_ARG, "args is NULL");
  if (a->num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs < 0");
  if (a->q_len < 1) return fail(PA_ERR_INVALID_ARG, "q_len must be >= 1 (got %d)", a->q_len);
  if ((entry == kDecode || entry == kDecodeInt8) && a->q_len != 1)
    return fail(PA_ERR_INVALID_ARG, "single-token decode needs q_len == 1 (got %d); use pa_verify", a->q_len);
  if (a->num_q_heads < 1 || a->num_kv_heads < 1 || a->num_q_heads % a->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                a->num_q_heads, a->num_kv_heads);
  if (a->block_size != pa::kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size must be 16 (got %d)", a->block_size);
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256 (got %d)", a->head_dim);
  if (a->q_dtype != PA_F32 && a->q_dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "q_dtype must be PA_F32 or PA_BF16");
  if (a->kv_dtype != PA_F32 && a->kv_dtype != PA_BF16 && a->kv_dtype != PA_INT8)
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype must be PA_F32, PA_BF16 or PA_INT8");
  if (entry == kDecode && a->kv_dtype == PA_INT8)
    return fail(PA_ERR_INVALID_ARG, "int8 caches go through pa_decode_int8");
  if (entry == kDecodeInt8 && (a->kv_dtype != PA_INT8 || a->q_dtype != PA_BF16))
    return fail(PA_ERR_INVALID_ARG, "pa_decode_int8 needs q_dtype PA_BF16 and kv_dtype PA_INT8");
  if (entry != kGather && a->kv_dtype == PA_INT8 && (!a->k_scale || !a->v_scale))
    return fail(PA_ERR_INVALID_ARG, "int8 cache needs k_scale and v_scale");
  if (a->kv_dtype == PA_INT8 && a->v_pool == a->k_pool && a->v_scale != a->k_scale)
    return fail(PA_ERR_INVALID_ARG, "values that alias the keys (v_pool == k_pool) need v_scale == k_scale");
  if (a->kv_dtype != PA_INT8 && a->kv_dtype != a->q_dtype)
    return fail(PA_ERR_UNSUPPORTED, "a floating-point cache must have the query's dtype");
  if (a->kv_dtype == PA_INT8 && a->q_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "an int8 cache needs bf16 queries");
  if (!std::isfinite(a->scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
  if (a->num_blocks < 1 || a->max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARG, "num_blocks and max_blocks_per_seq must be >= 1");
  if (a->max_seq_len < a->q_len)
    return fail(PA_ERR_INVALID_ARG, "max_seq_len (%d) must be >= q_len (%d)", a->max_seq_len, a->q_len);
  if (a->ring_blocks < 0) return fail(PA_ERR_INVALID_ARG, "ring_blocks must be >= 0");
  if (a->ring_blocks > 0) {
    if (a->window <= 0) return fail(PA_ERR_INVALID_ARG, "a ring cache needs a window");
    if (a->ring_blocks > a->max_blocks_per_seq)
      return fail(PA_ERR_INVALID_ARG, "ring_blocks (%d) exceeds max_blocks_per_seq (%d)", a->ring_blocks,
                  a->max_blocks_per_seq);
    if ((int64_t)a->ring_blocks * a->block_size < (int64_t)a->window + a->q_len - 1)
      return fail(PA_ERR_INVALID_ARG, "a ring of %d blocks cannot hold window + q_len - 1 = %lld keys",
                  a->ring_blocks, (long long)a->window + a->q_len - 1);
  } else if ((int64_t)a->max_seq_len > (int64_t)a->max_blocks_per_seq * a->block_size) {
    return fail(PA_ERR_INVALID_ARG, "max_seq_len (%d) exceeds max_blocks_per_seq * block_size", a->max_seq_len);
  }
  if (a->scale_per_head != 0 && (a->scale_per_head != 1 || a->kv_dtype != PA_INT8))
    return fail(PA_ERR_INVALID_ARG, "scale_per_head is 0, or 1 for an int8 cache");
  if (a->num_splits < 0) return fail(PA_ERR_INVALID_ARG, "num_splits must be >= 0");
  if (a->num_seqs > 0 && (!a->out || !a->q || !a->k_pool || !a->v_pool || !a->block_table || !a->seq_lens))
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  return PA_OK;
}

int make_plan(const pa_args* a, Plan* pl) {
  const int G = a->num_q_heads / a->num_kv_heads;
  const int D = a->head_dim;
  static const pa_tuning kNoTuning = {0, 0, PA_PART_AUTO, 0, 0, 0};
  const pa_tuning& tu = a->tuning ? *a->tuning : kNoTuning;
  Plan P;
  P.rows = G * a->q_len;
  const int valu_max_rows = 512 / D;   // query rows the vector kernel keeps in registers
  if (a->kv_dtype == PA_INT8 || (a->q_dtype == PA_BF16 && P.rows > valu_max_rows)) {
    P.kernel = 1;
    P.row_tiles = (P.rows + 15) / 16;
    P.rows_t = 16 * P.row_tiles;
    if (P.row_tiles > 2 || (P.row_tiles == 2 && D > 128))
      return fail(PA_ERR_UNSUPPORTED, "matrix-core kernel supports up to 32 query rows per KV head (D <= 128) "
                  "or 16 (D = 256); got %d rows, D = %d", P.rows, D);
  } else {
    if (P.rows > valu_max_rows)
      return fail(PA_ERR_UNSUPPORTED, "fp32 path supports at most %d query rows per KV head at D = %d (got %d)",
                  valu_max_rows, D, P.rows);
    P.kernel = 0;
    P.rows_t = 1;
    while (P.rows_t < P.rows) P.rows_t *= 2;
  }
  P.nw = P.kernel == 1 ? 4 : 8;   // matrix-core: two 4-wave workgroups per CU measured faster than one of 8

  // Explicit overrides (pa_tuning): checked against what the chosen kernel supports.
  if (tu.waves != 0 && tu.waves != 4 && tu.waves != 8 && !(P.kernel == 1 && tu.waves == 2))
    return fail(PA_ERR_UNSUPPORTED, "tuning.waves = %d: the %s kernel takes 4 or 8%s", tu.waves,
                P.kernel ? "matrix-core" : "vector", P.kernel ? " (or 2)" : "");
  if (tu.blocks_per_wave < 0 || tu.blocks_per_wave > 64)
    return fail(PA_ERR_INVALID_ARG, "tuning.blocks_per_wave must be 0..64 (got %d)", tu.blocks_per_wave);
  if (tu.partition < PA_PART_AUTO || tu.partition > PA_PART_QUEUE)
    return fail(PA_ERR_INVALID_ARG, "tuning.partition must be a PA_PART_* value (got %d)", tu.partition);
  if (P.kernel == 0 && tu.partition > PA_PART_ALIGNED)
    return fail(PA_ERR_UNSUPPORTED, "the vector kernel only takes aligned splits");
  if (a->num_splits > 0 && tu.partition > PA_PART_ALIGNED)
    return fail(PA_ERR_INVALID_ARG, "num_splits asks for aligned splits; tuning.partition asks otherwise");
  if (tu.pieces_per_wg < 0 || tu.pieces_per_wg > 64 || tu.oversub < 0 || tu.oversub > 64)
    return fail(PA_ERR_INVALID_ARG, "tuning.pieces_per_wg and tuning.oversub must be 0..64");
  if (tu.segment_blocks < -1 || tu.segment_blocks > 4096)
    return fail(PA_ERR_INVALID_ARG, "tuning.segment_blocks must be -1..4096 (got %d)", tu.segment_blocks);
  const bool nw_forced = tu.waves != 0;
  if (nw_forced) P.nw = tu.waves;

  const int bs = a->block_size;
  int n_blk_max = (a->max_seq_len + bs - 1) / bs;
  if (a->window > 0) {
    const int64_t span = (int64_t)a->window + a->q_len - 1;   // keys the step can see
    const int64_t blocks = (span + bs - 2) / bs + 1;         // worst alignment
    if (blocks < n_blk_max) n_blk_max = (int)blocks;
  }
  if (n_blk_max < 1) n_blk_max = 1;
  P.n_blk_max = n_blk_max;

  const int64_t units = (int64_t)a->num_seqs * a->num_kv_heads;
  int S;
  if (a->num_splits > 0) {
    S = a->num_splits < n_blk_max ? a->num_splits : n_blk_max;
  } else {
    // Each wavefront should stream 4..16 blocks (enough to keep its two-deep
    // pipeline busy, few enough that long sequences are cut into workgroups
    // the dispatcher can balance). Work is estimated from max_seq_len alone
    // (no device read): every sequence spans the window when there is one,
    // otherwise half the longest context on average.
    const int64_t slots = (int64_t)cu_count() * 8;           // resident wavefronts at 2 per SIMD
    const int64_t per_unit = a->window > 0 ? n_blk_max : (n_blk_max + 1) / 2;
    int64_t bpw = (units * per_unit + slots - 1) / (slots > 0 ? slots : 1);
    bpw = bpw < 4 ? 4 : (bpw > 16 ? 16 : bpw);
    if (tu.blocks_per_wave > 0) bpw = tu.blocks_per_wave;
    const int64_t bps = bpw * P.nw;
    S = (int)((n_blk_max + bps - 1) / bps);
    if (S < 1) S = 1;
  }
  P.bps = (n_blk_max + S - 1) / S;
  P.splits = (n_blk_max + P.bps - 1) / P.bps;
  P.grid = units * P.splits;
  P.slots = P.splits > 1 ? units * P.splits : 0;

  // The matrix-core kernel defaults to a work-balanced partition over as
  // many workgroups as are resident at once (two per compute unit at 4
  // waves, one at 8). With many units (sequence, KV head), units are cut on
  // the device into near-equal pieces handed out to the workgroups through a
  // sharded queue in the workspace. Otherwise, and for batches beyond the
  // piece partition's LDS tables, each workgroup takes an equal share of the
  // flattened (unit, block) list, each unit charged a segment's cost. One
  // piece per workgroup is available on request. Forced splits and the
  // vector kernel keep the aligned splits.
  const int part = tu.partition;
  const bool balanced = P.kernel == 1 && a->num_splits == 0 && part != PA_PART_ALIGNED;
  if (balanced && a->num_seqs > pa::balanced_seq_limit(P.nw)) {
    if (part != PA_PART_AUTO)
      return fail(PA_ERR_UNSUPPORTED, "the balanced partitions take at most %d sequences at %d waves",
                  pa::balanced_seq_limit(P.nw), P.nw);
  } else if (balanced) {
    // Few units (at most one per two CUs): one 8-wave workgroup per CU
    // streams them as fast as two of 4 waves and leaves half the partials to
    // merge (16 sequences of 4K-32K tokens on one KV head: kernel 29.4 vs
    // 29.2 us, step 34.9 vs 37.0 us).
    if (!nw_forced && 2 * units <= (int64_t)cu_count()) P.nw = 8;
    P.nwg = cu_count() * (8 / P.nw);   // as many workgroups as are resident at once (2 wavefronts per SIMD)
    if (tu.oversub > 0) P.nwg *= tu.oversub;
    // Measured on MI355X: the flattened list with segment charges for few
    // units (16 long contexts on one KV head: kernel 27.3 vs 28.2 us for one
    // piece per workgroup, step 33.3 vs 34.2 us; equal items per workgroup
    // where pieces of different units differ in size) and for about as many
    // units as workgroups (512 units of 1-4K tokens: 81 us vs 89-98 us
    // through the queue), the queue for many (2048 units of lognormal
    // length: 306 us vs 310 us for the flattened list).
    const bool few = 2 * units <= P.nwg;
    const bool many = units >= 2 * (int64_t)P.nwg;
    const bool pieces_ok = a->num_seqs <= pa::kMaxPieceSeqs && P.nw >= 4;
    const bool queue_ok = P.nwg >= pa::kQueueShards;
    bool pieces, queue;
    switch (part) {
      case PA_PART_LIST:
        pieces = queue = false;
        break;
      case PA_PART_PIECES:
        if (!pieces_ok || !few)
          return fail(PA_ERR_UNSUPPORTED, "one piece per workgroup needs at most %d sequences, 4+ waves and "
                      "2 x units <= workgroups (%lld units, %d workgroups)", pa::kMaxPieceSeqs,
                      (long long)units, P.nwg);
        pieces = true;
        queue = false;
        break;
      case PA_PART_QUEUE:
        if (!pieces_ok || !queue_ok)
          return fail(PA_ERR_UNSUPPORTED, "queued pieces need at most %d sequences, 4+ waves and %d+ workgroups",
                      pa::kMaxPieceSeqs, pa::kQueueShards);
        pieces = queue = true;
        break;
      default:
        pieces = pieces_ok && many && queue_ok;
        queue = pieces;
        break;
    }
    P.balanced = pieces ? 2 : 1;
    P.grid = P.nwg;
    if (pieces) {
      P.queue = queue;
      const int64_t per_wg = tu.pieces_per_wg > 0 ? tu.pieces_per_wg : 4;
      P.pieces = queue ? per_wg * P.nwg : P.nwg;
      // The device's search for the piece size needs at least one piece per
      // unit; the plan's own choice keeps twice that, an explicit request
      // (tuning.pieces_per_wg) only the minimum.
      if (P.pieces < 2 * units) P.pieces = tu.pieces_per_wg > 0 ? std::max<int64_t>(P.pieces, units) : 2 * units;
      P.slots = P.pieces;
    } else {
      P.queue = false;
      P.pieces = 0;
      P.slots = P.nwg + units;
      // Equal blocks per workgroup leave the workgroups whose share crosses
      // more unit boundaries behind: each segment costs a start and a merge,
      // measured at ~3.5 + 1.2 us on MI355X (int8 GQA layer, 512 workgroups).
      // Each unit is therefore charged, besides its blocks, the blocks a
      // workgroup streams in that time at its share of ~6 TB/s.
      if (tu.segment_blocks > 0) {
        P.seg_blocks = tu.segment_blocks;
      } else if (tu.segment_blocks == 0) {
        const bool int8 = a->kv_dtype == PA_INT8;
        const double row_bytes = (double)D * (int8 ? 1 : a->kv_dtype == PA_BF16 ? 2 : 4);
        const double block_bytes = pa::kBlock * row_bytes * (a->v_pool == a->k_pool ? 1 : 2) +
                                   (int8 ? 2.0 * pa::kBlock * sizeof(float) : 0.0);
        const long c = std::lround(4.7e-6 * 6.0e12 / P.nwg / block_bytes);
        P.seg_blocks = (int)std::min<long>(std::max<long>(c, 1), 4096);
      }
    }
  }
  if (P.grid > 0x7FFFFFFF || P.pieces > 0x7FFFFFFF) return fail(PA_ERR_UNSUPPORTED, "launch too large");
  // Workspace: a 4 KiB header holding the piece-queue counters (zero between
  // calls; no other partition writes the header), then the partials and the
  // prefix sums.
  if (P.slots > 0) {
    P.ws_bytes = kWsHeader + (size_t)P.slots * P.rows * (size_t)(D + 2) * sizeof(float);
    if (P.balanced) P.ws_bytes += (size_t)(2 * a->num_seqs + 1) * sizeof(int32_t);
  } else {
    P.ws_bytes = 0;
  }
  *pl = P;
  return PA_OK;
}

pa::Params make_params(const pa_args* a, const Plan& P) {
  pa::Params p{};
  p.out = a->out;
  p.q = a->q;
  p.k_pool = a->k_pool;
  p.v_pool = a->v_pool;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  // Workspace: the header (queue words), acc [slots][rows][D] f32, then
  // (m, l) [slots][rows][2] f32, then (balanced modes) a sequence table of
  // 2B+1 int32: block prefix sums [B+1] (list partition), or first piece
  // numbers [B] and piece counts [B] (piece partition).
  const size_t acc_bytes = (size_t)P.slots * P.rows * a->head_dim * sizeof(float);
  const size_t ml_bytes = (size_t)P.slots * P.rows * 2 * sizeof(float);
  char* ws = reinterpret_cast<char*>(a->workspace);
  char* body = ws + kWsHeader;
  p.ws_acc = P.ws_bytes ? reinterpret_cast<float*>(body) : nullptr;
  p.ws_ml = P.ws_bytes ? reinterpret_cast<float*>(body + acc_bytes) : nullptr;
  p.ws_prefix = (P.ws_bytes && P.balanced) ? reinterpret_cast<int32_t*>(body + acc_bytes + ml_bytes) : nullptr;
  p.ws_queue = (P.ws_bytes && P.queue) ? reinterpret_cast<int32_t*>(ws) : nullptr;
  p.pieces = (int32_t)P.pieces;
  p.balanced = P.balanced;
  p.nwg = P.nwg;
  p.seg_items = P.balanced == 1 ? P.seg_blocks : 0;
  p.visits = a->debug_visits;
  p.stamps = reinterpret_cast<uint64_t*>(a->debug_stamps);
  p.B = a->num_seqs;
  p.q_len = a->q_len;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.G = a->num_q_heads / a->num_kv_heads;
  p.rows = P.rows;
  p.maxb = a->max_blocks_per_seq;
  p.window = a->window;
  p.scale_log2 = a->scale * pa::kLog2e;
  p.splits = P.splits;
  p.bps = P.bps;
  p.ring = a->ring_blocks;
  p.head_scales = a->scale_per_head;
  return p;
}

// Enqueue the attention kernel (and the combine kernel when the plan splits)
// for arguments already validated and planned; the workspace is checked.
int launch_plan(const pa_args* a, const Plan& P, pa_stream_t stream) {
  if (P.ws_bytes) {
    if (!a->workspace || a->workspace_bytes < P.ws_bytes)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", P.ws_bytes,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(a->workspace) % 16)
      return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  const pa::Params p = make_params(a, P);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  pa::Timing tm;
  tm.start = reinterpret_cast<hipEvent_t>(a->timing_start);
  tm.stop = reinterpret_cast<hipEvent_t>(a->timing_stop);
  hipError_t e;
  bool supported = false;
  if (P.kernel == 0)
    e = pa::launch_valu(p, a->q_dtype, a->kv_dtype, a->head_dim, P.rows_t, P.nw, (int)P.grid, st, tm, &supported);
  else
    e = pa::launch_mfma(p, a->kv_dtype, a->head_dim, P.row_tiles, P.nw, (int)P.grid, st, tm, &supported);
  if (!supported)
    return fail(PA_ERR_UNSUPPORTED, "no kernel built for D=%d rows=%d q_dtype=%d kv_dtype=%d", a->head_dim, P.rows,
                a->q_dtype, a->kv_dtype);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "attention kernel launch: %s", hipGetErrorString(e));
  if (P.slots > 0) {
    e = pa::launch_combine(p, a->q_dtype, a->head_dim, st);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

int run(const pa_args* a, pa_stream_t stream, Entry entry) {
  pa::clear_error();
  int rc = validate(a, entry);
  if (rc) return rc;
  Plan P;
  rc = make_plan(a, &P);
  if (rc) return rc;
  if (a->num_seqs == 0) return PA_OK;
  return launch_plan(a, P, stream);
}

}  // namespace

// ---- pa_verify_noalloc: the workspace in a static device array ----------------
//
// For callers that cannot allocate device memory (HIP graph capture, serving
// loops that forbid it). The split partials, prefix sums and piece queue live
// in `scratch`, one copy per GPU, zero when the library's code object is
// loaded and kept until the process ends. On the host this name only stands
// for the symbol: host code never hands it to a kernel or a copy, and uses
// instead the device address hipGetSymbolAddress returns for the current
// device (looked up once per device, then cached).
namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::atomic<void*> g_scratch[kMaxDevices];

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d is past the library's table", dev);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PA_OK;
}
}  // namespace

extern "C" {

size_t pa_workspace_size(const pa_args* a) {
  pa::clear_error();
  if (validate(a, kAny)) return (size_t)-1;
  Plan P;
  if (make_plan(a, &P)) return (size_t)-1;
  return P.ws_bytes;
}

int pa_plan(const pa_args* a, pa_plan_info* info) {
  pa::clear_error();
  if (!info) return fail(PA_ERR_INVALID_ARG, "info is NULL");
  int rc = validate(a, kAny);
  if (rc) return rc;
  Plan P;
  rc = make_plan(a, &P);
  if (rc) return rc;
  info->kernel = P.kernel;
  info->rows = P.rows;
  info->waves_per_group = P.nw;
  info->splits = P.splits;
  info->blocks_per_split = P.bps;
  info->grid = (int32_t)P.grid;
  info->balanced = P.balanced;
  info->pieces = (int32_t)P.pieces;
  info->queue = P.queue ? 1 : 0;
  info->segment_blocks = P.balanced == 1 ? P.seg_blocks : 0;
  info->workspace_bytes = P.ws_bytes;
  return PA_OK;
}

int pa_decode(const pa_args* a, pa_stream_t stream) { return run(a, stream, kDecode); }
int pa_decode_int8(const pa_args* a, pa_stream_t stream) { return run(a, stream, kDecodeInt8); }
int pa_verify(const pa_args* a, pa_stream_t stream) { return run(a, stream, kVerify); }

int pa_verify_noalloc(const pa_args* a, pa_stream_t stream) {
  pa::clear_error();
  int rc = validate(a, kVerify);
  if (rc) return rc;
  if (a->workspace || a->workspace_bytes)
    return fail(PA_ERR_INVALID_ARG, "pa_verify_noalloc uses the library's scratch array: pass no workspace");
  Plan P;
  rc = make_plan(a, &P);
  if (rc) return rc;
  if (a->num_seqs == 0) return PA_OK;
  if (P.ws_bytes > kScratchBytes)
    return fail(PA_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the library's array holds %zu "
                "(use pa_verify with a workspace)", P.ws_bytes, kScratchBytes);
  pa_args b = *a;
  if (P.ws_bytes) {
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    b.workspace = ws;
    b.workspace_bytes = kScratchBytes;
    if (P.queue) {
      // The piece queue's counters must start at zero; a previous call on
      // this GPU leaves them so, but they are cleared here by a small kernel
      // on the call's own stream (no memset node if the call is captured).
      const hipError_t e = pa::launch_zero_words(reinterpret_cast<int32_t*>(ws), (int32_t)(kWsHeader / 4),
                                                 reinterpret_cast<hipStream_t>(stream));
      if (e != hipSuccess) return fail(PA_ERR_HIP, "scratch clear launch: %s", hipGetErrorString(e));
    }
  }
  return launch_plan(&b, P, stream);
}

int pa_debug_gather(const pa_args* a, int32_t which, void* dst, int64_t dst_tokens, pa_stream_t stream) {
  pa::clear_error();
  int rc = validate(a, kGather);
  if (rc) return rc;
  if (which != 0 && which != 1) return fail(PA_ERR_INVALID_ARG, "which must be 0 (keys) or 1 (values)");
  if (a->num_seqs > 0 && !dst) return fail(PA_ERR_INVALID_ARG, "dst is NULL");
  // The widest visible key range a sequence can have; dst must hold it.
  int64_t need = a->max_seq_len;
  if (a->window > 0 && (int64_t)a->window + a->q_len - 1 < need) need = (int64_t)a->window + a->q_len - 1;
  if (dst_tokens < need)
    return fail(PA_ERR_INVALID_ARG, "dst_tokens (%lld) must be >= %lld", (long long)dst_tokens, (long long)need);
  if (a->num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "debug gather handles at most 65535 sequences");
  if (a->num_seqs == 0) return PA_OK;
  Plan P;
  rc = make_plan(a, &P);
  if (rc) return rc;
  const pa::Params p = make_params(a, P);
  hipError_t e = pa::launch_gather(p, a->kv_dtype, a->head_dim, which, dst, dst_tokens,
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "gather kernel launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_validate(const pa_args* a, int32_t* d_status, pa_stream_t stream) {
  pa::clear_error();
  int rc = validate(a, kGather);   // the attention pointers are not used here
  if (rc) return rc;
  if (!d_status) return fail(PA_ERR_INVALID_ARG, "d_status is NULL");
  if (a->num_seqs > 0x7FFFFFFF - 1) return fail(PA_ERR_UNSUPPORTED, "too many sequences");
  if (a->num_seqs == 0) return PA_OK;
  Plan P;
  rc = make_plan(a, &P);
  if (rc) return rc;
  const pa::Params p = make_params(a, P);
  const int check_scales = a->kv_dtype == PA_INT8 && a->k_scale && a->v_scale;
  // The piece queue's counters must be zero when a call starts (each call
  // leaves them so): check them when the call would use the queue.
  const int32_t* header = (P.queue && a->workspace && a->workspace_bytes >= P.ws_bytes)
                              ? reinterpret_cast<const int32_t*>(a->workspace)
                              : nullptr;
  const hipError_t e = pa::launch_validate(p, a->num_blocks, a->max_seq_len, check_scales, header, d_status,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "validate kernel launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_cache_write(const pa_write_args* a, pa_stream_t stream) {
  pa::clear_error();
  if (!a) return fail(PA_ERR_INVALID_ARG, "args is NULL");
  if (a->num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
  if (a->num_kv_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (a->num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (a->block_size != pa::kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size must be 16 (got %d)", a->block_size);
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256 (got %d)", a->head_dim);
  if (a->src_dtype != PA_F32 && a->src_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "src_dtype must be PA_F32 or PA_BF16");
  if (a->scale_per_head != 0 && (a->scale_per_head != 1 || a->kv_dtype != PA_INT8))
    return fail(PA_ERR_INVALID_ARG, "scale_per_head is 0, or 1 for an int8 cache");
  if (a->kv_dtype == PA_INT8) {
    if (a->num_tokens > 0 && (!a->k_scale || !a->v_scale))
      return fail(PA_ERR_INVALID_ARG, "an int8 cache needs k_scale and v_scale");
  } else if (a->kv_dtype != a->src_dtype) {
    return fail(PA_ERR_INVALID_ARG, "a floating-point cache must have the rows' dtype");
  }
  if (a->num_tokens == 0) return PA_OK;
  if (!a->k_new || !a->v_new || !a->slot_ids || !a->k_pool || !a->v_pool)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  for (const void* ptr : {a->k_new, a->v_new, (const void*)a->k_pool, (const void*)a->v_pool})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
      return fail(PA_ERR_INVALID_ARG, "rows and pools must be 16-byte aligned");
  for (const void* ptr : {(const void*)a->slot_ids, (const void*)a->k_scale, (const void*)a->v_scale})
    if (reinterpret_cast<uintptr_t>(ptr) % 8 != 0)
      return fail(PA_ERR_INVALID_ARG, "slot ids and scales must be 8-byte aligned");
  const bool alias = a->v_pool == a->k_pool;
  if (alias && a->v_new != a->k_new)
    return fail(PA_ERR_INVALID_ARG, "v_pool is k_pool but v_new is not k_new");
  if (alias && a->kv_dtype == PA_INT8 && a->v_scale != a->k_scale)
    return fail(PA_ERR_INVALID_ARG, "v_pool is k_pool but v_scale is not k_scale");
  if ((int64_t)a->num_tokens * a->num_kv_heads > (int64_t)0x7FFFFFFF * 4)
    return fail(PA_ERR_UNSUPPORTED, "launch too large");
  pa::WriteParams p{};
  p.k_new = a->k_new;
  p.v_new = a->v_new;
  p.slot_ids = a->slot_ids;
  p.k_pool = a->k_pool;
  p.v_pool = a->v_pool;
  p.k_scale = a->k_scale;
  p.v_scale = alias ? a->k_scale : a->v_scale;
  p.T = a->num_tokens;
  p.Hkv = a->num_kv_heads;
  p.num_blocks = a->num_blocks;
  p.write_v = alias ? 0 : 1;
  p.head_scales = a->scale_per_head;
  bool supported = false;
  const hipError_t e = pa::launch_cache_write(p, a->src_dtype, a->kv_dtype, a->head_dim,
                                              reinterpret_cast<hipStream_t>(stream),
                                              reinterpret_cast<hipEvent_t>(a->timing_start),
                                              reinterpret_cast<hipEvent_t>(a->timing_stop), &supported);
  if (!supported) return fail(PA_ERR_UNSUPPORTED, "no append kernel for these dtypes / head_dim");
  if (e != hipSuccess) return fail(PA_ERR_HIP, "append kernel launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_prefill(const pa_prefill_args* a, pa_stream_t stream) {
  pa::clear_error();
  if (!a) return fail(PA_ERR_INVALID_ARG, "args is NULL");
  if (a->num_seqs < 0 || a->total_q < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs and total_q must be >= 0");
  if (a->num_q_heads < 1 || a->num_kv_heads < 1 || a->num_q_heads % a->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                a->num_q_heads, a->num_kv_heads);
  if (a->block_size != pa::kBlock) return fail(PA_ERR_UNSUPPORTED, "block_size must be 16 (got %d)", a->block_size);
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256 (got %d)", a->head_dim);
  if (a->q_dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "prefill takes bf16 queries");
  if (a->kv_dtype != PA_BF16 && a->kv_dtype != PA_INT8)
    return fail(PA_ERR_UNSUPPORTED, "prefill takes a bf16 or int8 cache");
  const int G = a->num_q_heads / a->num_kv_heads;
  const int rows = pa::prefill_rows(a->head_dim);
  if (G > rows) return fail(PA_ERR_UNSUPPORTED, "query group of %d heads exceeds %d rows", G, rows);
  if (!std::isfinite(a->scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
  if (a->num_blocks < 1 || a->max_blocks_per_seq < 1)
    return fail(PA_ERR_INVALID_ARG, "num_blocks and max_blocks_per_seq must be >= 1");
  if (a->scale_per_head != 0 && (a->scale_per_head != 1 || a->kv_dtype != PA_INT8))
    return fail(PA_ERR_INVALID_ARG, "scale_per_head is 0, or 1 for an int8 cache");
  if (a->kv_dtype == PA_INT8 && (!a->k_scale || !a->v_scale))
    return fail(PA_ERR_INVALID_ARG, "an int8 cache needs k_scale and v_scale");
  if (a->kv_dtype == PA_INT8 && a->v_pool == a->k_pool && a->v_scale != a->k_scale)
    return fail(PA_ERR_INVALID_ARG, "values that alias the keys (v_pool == k_pool) need v_scale == k_scale");
  if (a->num_seqs == 0 || a->total_q == 0) return PA_OK;
  if (a->max_q_len < 1) return fail(PA_ERR_INVALID_ARG, "max_q_len must be >= 1");
  if (a->max_seq_len < a->max_q_len)
    return fail(PA_ERR_INVALID_ARG, "max_seq_len (%d) must be >= max_q_len (%d)", a->max_seq_len, a->max_q_len);
  if (a->ring_blocks < 0) return fail(PA_ERR_INVALID_ARG, "ring_blocks must be >= 0");
  if (a->ring_blocks > 0) {
    if (a->window <= 0) return fail(PA_ERR_INVALID_ARG, "a ring cache needs a window");
    if (a->ring_blocks > a->max_blocks_per_seq)
      return fail(PA_ERR_INVALID_ARG, "ring_blocks exceeds max_blocks_per_seq");
    if ((int64_t)a->ring_blocks * a->block_size < (int64_t)a->window + a->max_q_len - 1)
      return fail(PA_ERR_INVALID_ARG, "a ring of %d blocks cannot hold window + max_q_len - 1 keys", a->ring_blocks);
  } else if ((int64_t)a->max_seq_len > (int64_t)a->max_blocks_per_seq * a->block_size) {
    return fail(PA_ERR_INVALID_ARG, "max_seq_len (%d) exceeds max_blocks_per_seq * block_size", a->max_seq_len);
  }
  if (!a->out || !a->q || !a->q_start || !a->k_pool || !a->v_pool || !a->block_table || !a->seq_lens)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  for (const void* ptr : {(const void*)a->out, a->q, a->k_pool, a->v_pool})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
      return fail(PA_ERR_INVALID_ARG, "q, out and the pools must be 16-byte aligned");
  pa::PrefillParams p{};
  p.out = a->out;
  p.q = a->q;
  p.q_start = a->q_start;
  p.k_pool = a->k_pool;
  p.v_pool = a->v_pool;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.block_table = a->block_table;
  p.seq_lens = a->seq_lens;
  p.B = a->num_seqs;
  p.Hq = a->num_q_heads;
  p.Hkv = a->num_kv_heads;
  p.G = G;
  p.maxb = a->max_blocks_per_seq;
  p.window = a->window;
  p.ring = a->ring_blocks;
  p.head_scales = a->scale_per_head;
  p.scale_log2 = a->scale * pa::kLog2e;
  p.qt = rows / G;
  p.ntiles = (a->max_q_len + p.qt - 1) / p.qt;
  const int64_t grid = (int64_t)p.ntiles * a->num_seqs * a->num_kv_heads;
  if (grid > 0x7FFFFFFF) return fail(PA_ERR_UNSUPPORTED, "launch too large");
  bool supported = false;
  const hipError_t e = pa::launch_prefill(p, a->kv_dtype, a->head_dim, grid, reinterpret_cast<hipStream_t>(stream),
                                          reinterpret_cast<hipEvent_t>(a->timing_start),
                                          reinterpret_cast<hipEvent_t>(a->timing_stop), &supported);
  if (!supported) return fail(PA_ERR_UNSUPPORTED, "no prefill kernel for this head_dim / dtype");
  if (e != hipSuccess) return fail(PA_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_version(void) { return 10100; }

#ifndef PA_BUILD_ID
#define PA_BUILD_ID "unknown"
#endif
const char* pa_build_id(void) { return PA_BUILD_ID; }

}  // extern "C"
