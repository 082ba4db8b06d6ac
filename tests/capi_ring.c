/* Plain C client of include/ra.h that runs one device's ring forward on the
 * GPU with nothing but the HIP runtime's C API and libra_amd.so (no Python,
 * no torch). Built by the package build into _lib/ra_capi_ring; run by
 * tests/test_gpu_capi.py, which writes the inputs and checks the output.
 *
 *   ra_capi_ring <in> <out> <n_ring> <rank> <len> <hq> <hkv> <d> <layout> <causal>
 *
 * <in>:  q [len, hq, d] then k, v [n_ring, len, hkv, d], bf16 (raw 16-bit
 *        words, batch 1, blocks in the layout's token order)
 * <out>: out [len, hq, d] then lse [len, hq], float32
 * Exit status 0 on success; on failure a message on stderr and status 1. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ra.h"

static int fail(const char* what, const char* detail) {
  fprintf(stderr, "ra_capi_ring: %s: %s\n", what, detail);
  return 1;
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_));   \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 11) return fail("usage", "in out n_ring rank len hq hkv d layout causal");
  ra_problem p;
  memset(&p, 0, sizeof p);
  p.dtype = RA_BF16;
  p.batch = 1;
  p.n_ring = atoi(argv[3]);
  p.rank = atoi(argv[4]);
  p.q_len = p.kv_len = atoll(argv[5]);
  p.hq = atoi(argv[6]);
  p.hkv = atoi(argv[7]);
  p.head_dim = atoi(argv[8]);
  p.layout = atoi(argv[9]);
  p.causal = atoi(argv[10]);
  p.scale = 0.0f;
  if (p.n_ring < 1 || p.q_len < 1 || p.hq < 1 || p.hkv < 1 || p.head_dim < 1) return fail("arguments", "out of range");

  const size_t nq = (size_t)p.q_len * p.hq * p.head_dim;
  const size_t nkv = (size_t)p.n_ring * p.kv_len * p.hkv * p.head_dim;
  const size_t nrow = (size_t)p.q_len * p.hq;
  uint16_t* h_in = (uint16_t*)malloc((nq + 2 * nkv) * sizeof(uint16_t));
  float* h_out = (float*)malloc((nq + nrow) * sizeof(float));
  if (!h_in || !h_out) return fail("malloc", "host buffers");
  FILE* f = fopen(argv[1], "rb");
  if (!f) return fail("open", argv[1]);
  const size_t got = fread(h_in, sizeof(uint16_t), nq + 2 * nkv, f);
  fclose(f);
  if (got != nq + 2 * nkv) return fail("read", "input file shorter than the shapes");

  const size_t ws_bytes = ra_ring_workspace_bytes(&p);
  if (ws_bytes == 0) return fail("ra_ring_workspace_bytes", ra_last_error());
  void *d_q, *d_k, *d_v, *d_ws;
  float *d_out, *d_lse;
  HIP_OK(hipMalloc(&d_q, nq * 2));
  HIP_OK(hipMalloc(&d_k, nkv * 2));
  HIP_OK(hipMalloc(&d_v, nkv * 2));
  HIP_OK(hipMalloc((void**)&d_out, nq * 4));
  HIP_OK(hipMalloc((void**)&d_lse, nrow * 4));
  HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMemcpy(d_q, h_in, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_k, h_in + nq, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_v, h_in + nq + nkv, nkv * 2, hipMemcpyHostToDevice));

  hipStream_t compute, copy;
  HIP_OK(hipStreamCreate(&compute));
  HIP_OK(hipStreamCreate(&copy));
  const ra_status st = ra_ring_fwd(&p, d_q, d_k, d_v, d_out, d_lse, d_ws, ws_bytes, (void*)compute, (void*)copy);
  if (st != RA_OK) return fail("ra_ring_fwd", ra_last_error());
  HIP_OK(hipStreamSynchronize(compute));
  HIP_OK(hipMemcpy(h_out, d_out, nq * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_out + nq, d_lse, nrow * 4, hipMemcpyDeviceToHost));

  f = fopen(argv[2], "wb");
  if (!f) return fail("open", argv[2]);
  const size_t put = fwrite(h_out, sizeof(float), nq + nrow, f);
  fclose(f);
  if (put != nq + nrow) return fail("write", argv[2]);

  HIP_OK(hipStreamDestroy(copy));
  HIP_OK(hipStreamDestroy(compute));
  HIP_OK(hipFree(d_ws));
  HIP_OK(hipFree(d_lse));
  HIP_OK(hipFree(d_out));
  HIP_OK(hipFree(d_v));
  HIP_OK(hipFree(d_k));
  HIP_OK(hipFree(d_q));
  free(h_out);
  free(h_in);
  return 0;
}
