/* A decode step driven from plain C through the library's C ABI (include/pa.h),
 * with device memory from the HIP runtime's C API and no Python or torch, checked
 * against the fp64 oracle (oracle/oracle.c, compiled into this test program).
 *
 * Workload: the tiny fp32 decode (2 sequences of 37 and 70 cached tokens, 4 query
 * heads on 2 KV heads, head_dim 64, 16-token blocks) with its blocks scattered
 * over a 16-block pool. Inputs come from a fixed linear congruential generator.
 * Exit status 0 when max |err| <= 1e-5 and the two error paths report what they
 * should; 1 otherwise. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "pa.h"

#include "../../oracle/oracle.c"

enum { B = 2, HQ = 4, HKV = 2, D = 64, BS = 16, NB = 16, MAXB = 5 };

static uint32_t lcg_state = 12345u;
static float uniform_pm1(void) {   /* test data in [-1, 1) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)((lcg_state >> 8) * (1.0 / 16777216.0)) * 2.0f - 1.0f;
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));            \
      return 1;                                                                \
    }                                                                          \
  } while (0)

int main(void) {
  static float q[B * HQ * D], kp[NB * BS * HKV * D], vp[NB * BS * HKV * D], out[B * HQ * D];
  static double ref[B * HQ * D];
  const int32_t lens[B] = {37, 70};
  /* Physical blocks, handed to the sequences from a fixed permutation of the pool. */
  const int32_t perm[NB] = {11, 3, 14, 0, 7, 9, 2, 13, 5, 1, 15, 8, 4, 12, 6, 10};
  int32_t table[B * MAXB];
  int used = 0;
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < MAXB; ++i) table[b * MAXB + i] = i * BS < lens[b] ? perm[used++] : 0;
  for (size_t i = 0; i < sizeof q / sizeof q[0]; ++i) q[i] = uniform_pm1();
  for (size_t i = 0; i < sizeof kp / sizeof kp[0]; ++i) kp[i] = uniform_pm1();
  for (size_t i = 0; i < sizeof vp / sizeof vp[0]; ++i) vp[i] = uniform_pm1();

  void *dq, *dk, *dv, *dout, *dtable, *dlens;
  HIP_OK(hipMalloc(&dq, sizeof q));
  HIP_OK(hipMalloc(&dk, sizeof kp));
  HIP_OK(hipMalloc(&dv, sizeof vp));
  HIP_OK(hipMalloc(&dout, sizeof out));
  HIP_OK(hipMalloc(&dtable, sizeof table));
  HIP_OK(hipMalloc(&dlens, sizeof lens));
  HIP_OK(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, kp, sizeof kp, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, vp, sizeof vp, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dtable, table, sizeof table, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dlens, lens, sizeof lens, hipMemcpyHostToDevice));

  pa_args a = {0};
  a.out = dout;
  a.q = dq;
  a.k_pool = dk;
  a.v_pool = dv;
  a.block_table = (const int32_t*)dtable;
  a.seq_lens = (const int32_t*)dlens;
  a.num_seqs = B;
  a.q_len = 1;
  a.num_q_heads = HQ;
  a.num_kv_heads = HKV;
  a.head_dim = D;
  a.block_size = BS;
  a.num_blocks = NB;
  a.max_blocks_per_seq = MAXB;
  a.max_seq_len = 70;
  a.window = 0;
  a.scale = 0.125f;
  a.q_dtype = PA_F32;
  a.kv_dtype = PA_F32;

  const size_t ws = pa_workspace_size(&a);
  void* dws = NULL;
  if (ws > 0) {
    HIP_OK(hipMalloc(&dws, ws));
    HIP_OK(hipMemset(dws, 0, ws));
    a.workspace = dws;
    a.workspace_bytes = ws;
  }
  int rc = pa_decode(&a, NULL);
  if (rc != PA_OK) {
    fprintf(stderr, "pa_decode: %s (%s)\n", pa_strerror(rc), pa_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));

  orc_problem P;
  memset(&P, 0, sizeof P);
  P.q = q;
  P.k_pool = kp;
  P.v_pool = vp;
  P.block_table = table;
  P.seq_lens = lens;
  P.q_dtype = ORC_F32;
  P.kv_dtype = ORC_F32;
  P.B = B;
  P.q_len = 1;
  P.Hq = HQ;
  P.Hkv = HKV;
  P.D = D;
  P.block_size = BS;
  P.num_blocks = NB;
  P.max_blocks = MAXB;
  P.window = 0;
  P.scale = 0.125;
  if (oracle_attention(&P, NULL, 0, ref, 1) != ORC_OK) {
    fprintf(stderr, "oracle failed\n");
    return 1;
  }
  double err = 0.0;
  for (int i = 0; i < B * HQ * D; ++i) err = fmax(err, fabs((double)out[i] - ref[i]));
  printf("decode from C: max|err| vs fp64 oracle = %.3e\n", err);

  /* Error paths: a NULL query pointer, and a head count the KV heads do not divide. */
  pa_args bad = a;
  bad.q = NULL;
  const int rc_null = pa_decode(&bad, NULL);
  bad = a;
  bad.num_q_heads = 3;
  const int rc_heads = pa_decode(&bad, NULL);
  printf("NULL q -> %s; Hq = 3 over Hkv = 2 -> %s\n", pa_strerror(rc_null), pa_strerror(rc_heads));

  hipFree(dq);
  hipFree(dk);
  hipFree(dv);
  hipFree(dout);
  hipFree(dtable);
  hipFree(dlens);
  if (dws) hipFree(dws);
  return err <= 1e-5 && rc_null == PA_ERR_INVALID_ARG && rc_heads == PA_ERR_INVALID_ARG ? 0 : 1;
}
