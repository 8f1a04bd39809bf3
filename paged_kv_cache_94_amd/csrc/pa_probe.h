// pa_probe.h -- the read-ceiling probe of libpa_probe.so (a measurement
// kernel for the benchmark, outside the attention library's ABI).
#pragma once

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

// Stream the cache tiles tiles[0..ntiles) (id = phys * num_kv_heads + g) of a
// pool laid out [num_blocks][16][num_kv_heads][row_bytes] (v_pool NULL or
// equal to k_pool: keys only), workgroup w taking tiles [w * per, (w + 1) *
// per), per = ceil(ntiles / workgroups), its `waves` wavefronts in turn, with
// `depth` tiles in flight per wavefront. sink: device uint32
// [workgroups * waves * 64]. timing_start / timing_stop: NULL or HIP events
// stamped by the kernel's own dispatch. Returns 0, 1 (bad argument) or 2
// (launch error). Device pointers; asynchronous on stream.
int pa_probe_read(const void* k_pool, const void* v_pool, const int32_t* tiles, int32_t ntiles, int32_t row_bytes,
                  int32_t num_kv_heads, int32_t workgroups, int32_t waves, int32_t depth, uint32_t* sink,
                  void* timing_start, void* timing_stop, void* stream);

#ifdef __cplusplus
}
#endif
