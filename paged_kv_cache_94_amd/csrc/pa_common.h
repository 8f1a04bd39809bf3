// pa_common.h -- the part of every attention kernel that follows the block
// loop: merging the wavefronts of a workgroup and writing either the final
// output or the split partials, plus the list of kernel entry points the
// host dispatcher instantiates.
#pragma once

#include <hip/hip_ext.h>

#include "pa_device.h"

namespace pa {

// Merge NW wavefront states through LDS and write the result.
//
// Each wavefront contributes, per query row r < ROWS, its running max m[r]
// (log2 units), its running sum l[r] and its unnormalised accumulator
// acc[r][0..D); merging uses the online-softmax rule (Lab 5 handout, "Flash
// Attention": rescale by 2^(m_w - M) before adding, O = o / l at the end).
//
// lds_acc: [NW][ROWS][D] floats, lds_ml: [NW][ROWS][2] floats. The caller
// has already stored its share and the merge starts with a barrier.
// split == -1 writes out = o / l in OutT; otherwise (m, l, o) go to the
// workspace slot of this split.
template <typename OutT, int D, int ROWS, int NW>
__device__ __forceinline__ void merge_and_store(const Params& p, const float* lds_acc, const float* lds_ml,
                                                int32_t b, int32_t g, int32_t split) {
  __syncthreads();
  const int tid = threadIdx.x;
  const int rows = p.rows;
  const int32_t unit = b * p.Hkv + g;
  for (int idx = tid; idx < ROWS * D; idx += NW * 64) {
    const int r = idx / D;
    const int d = idx % D;
    if (r >= rows) break;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, lds_ml[(w * ROWS + r) * 2]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = lds_ml[(w * ROWS + r) * 2];
        const float s = fast_exp2(mw - M);
        num += s * lds_acc[(w * ROWS + r) * D + d];
        den += s * lds_ml[(w * ROWS + r) * 2 + 1];
      }
    }
    if (split < 0) {
      const int t = r / p.G;
      const int h = g * p.G + r % p.G;
      OutT* out = reinterpret_cast<OutT*>(p.out) + (((size_t)b * p.q_len + t) * p.Hq + h) * D;
      const float v = num / den;
      if constexpr (sizeof(OutT) == 4) {
        out[d] = v;
      } else {
        out[d] = (__bf16)v;
      }
    } else {
      const size_t slot = ((size_t)unit * p.splits + split) * rows + r;
      p.ws_acc[slot * D + d] = num;
      if (d == 0) {
        p.ws_ml[slot * 2] = M;
        p.ws_ml[slot * 2 + 1] = den;
      }
    }
  }
}

}  // namespace pa

// Host-side launchers, one per kernel family (defined in the .hip files).
namespace pa {
// Batch limits of the balanced partitions (their per-sequence tables live in LDS).
constexpr int kMaxBalancedSeqs = 2048;   // flattened-list partition: block prefix sums and first blocks
// Workgroups of one or two wavefronts run four to eight to a compute unit, so
// their LDS share is smaller: their prefix table holds fewer sequences.
constexpr int balanced_seq_limit(int nw) { return nw >= 4 ? kMaxBalancedSeqs : 1024; }
// Piece queue in the workspace header: kQueueShards "next" counters, then as
// many "done" counters, each on its own 64-byte line (int32 index stride 16).
constexpr int kQueueShards = 8;
constexpr int kQueueStride = 16;
constexpr size_t kWsHeader = 4096;      // workspace bytes before the partials

struct LaunchShape {
  int kernel;   // 0 valu, 1 mfma
  int rows_t;   // compiled row count (>= rows)
  int nw;       // waves per workgroup
  int grid;     // workgroups
};
// Optional timing of the attention kernel. The kernel goes through
// hipExtLaunchKernel, which stamps the two events from the kernel's own
// dispatch (its start and its completion) rather than from separate marker
// commands queued around it, so the interval is the kernel's execution time.
struct Timing {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename K>
inline hipError_t launch_timed(K kernel, int grid, int threads, hipStream_t st, const Timing& tm, const Params& p) {
  hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, st, tm.start, tm.stop, 0, p);
  return hipGetLastError();
}

hipError_t launch_valu(const Params& p, int q_dtype, int kv_dtype, int D, int rows_t, int nw, int grid,
                       hipStream_t st, const Timing& tm, bool* supported);
hipError_t launch_mfma(const Params& p, int kv_dtype, int D, int row_tiles, int nw, int grid,
                       hipStream_t st, const Timing& tm, bool* supported);
hipError_t launch_combine(const Params& p, int q_dtype, int D, hipStream_t st);
hipError_t launch_validate(const Params& p, int32_t num_blocks, int32_t max_seq_len, int check_scales,
                           const int32_t* queue_header, int32_t* status, hipStream_t st);
hipError_t launch_gather(const Params& p, int kv_dtype, int D, int which, void* dst, int64_t dst_tokens,
                         hipStream_t st);
// Zero n int32 words at p with a small kernel (one workgroup; vector stores).
hipError_t launch_zero_words(int32_t* p, int32_t n, hipStream_t st);
}  // namespace pa
