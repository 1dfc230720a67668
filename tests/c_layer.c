/* A plain C caller of bsga_layer on one GPU, with no Python in the process:
 * reads Q, K, V (bf16 bits, [H][N][64] each, one after the other) from a
 * file, allocates device memory and the workspace with the HIP runtime, runs
 * one layer on the null stream and writes, in this order, probs [H][B][B]
 * float32, row_ptr [H*B+1] int32, col_idx [nnz] int32, O [H][N][64] bf16
 * bits and LSE [H][N] float32 to the output file.
 * usage: c_layer IN OUT frames patches_per_frame special_per_frame heads
 *        block rho tau                                                   */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "bsga.h"

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}
#define HIP(x) \
  if (!hip_ok((x), #x)) return 1
#define BSGA(x)                                                        \
  do {                                                                 \
    const int st_ = (x);                                               \
    if (st_ != BSGA_OK) {                                              \
      fprintf(stderr, "%s: %s\n", #x, bsga_status_string(st_));        \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static int write_all(FILE* f, const void* p, size_t bytes) {
  return fwrite(p, 1, bytes, f) == bytes;
}

int main(int argc, char** argv) {
  bsga_shape s;
  double rho, tau;
  int32_t B = 0;
  int64_t cap = 0, nnz;
  size_t ws_bytes = 0, n, nel;
  uint16_t *h_qkv, *h_o;
  float *h_probs, *h_lse;
  int32_t *h_rp, *h_ci;
  void *q, *k, *v, *o, *lse, *probs, *rp, *ci, *ws = NULL;
  FILE* f;
  if (argc != 10) {
    fprintf(stderr, "usage: c_layer IN OUT frames P S heads block rho tau\n");
    return 2;
  }
  s.frames = atoi(argv[3]);
  s.patches_per_frame = atoi(argv[4]);
  s.special_per_frame = atoi(argv[5]);
  s.heads = atoi(argv[6]);
  s.head_dim = 64;
  s.block = atoi(argv[7]);
  rho = atof(argv[8]);
  tau = atof(argv[9]);
  BSGA(bsga_num_blocks(&s, &B));
  BSGA(bsga_csr_capacity(&s, &cap));
  BSGA(bsga_workspace_bytes(&s, BSGA_OP_LAYER, &ws_bytes));
  n = (size_t)s.frames * (size_t)(s.patches_per_frame + s.special_per_frame);
  nel = (size_t)s.heads * n * 64;

  h_qkv = (uint16_t*)malloc(3 * nel * sizeof(uint16_t));
  f = fopen(argv[1], "rb");
  if (!h_qkv || !f || fread(h_qkv, sizeof(uint16_t), 3 * nel, f) != 3 * nel) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  fclose(f);

  HIP(hipMalloc(&q, nel * 2));
  HIP(hipMalloc(&k, nel * 2));
  HIP(hipMalloc(&v, nel * 2));
  HIP(hipMalloc(&o, nel * 2));
  HIP(hipMalloc(&lse, (size_t)s.heads * n * 4));
  HIP(hipMalloc(&probs, (size_t)s.heads * B * B * 4));
  HIP(hipMalloc(&rp, ((size_t)s.heads * B + 1) * 4));
  HIP(hipMalloc(&ci, (size_t)cap * 4));
  if (ws_bytes) HIP(hipMalloc(&ws, ws_bytes));
  HIP(hipMemcpy(q, h_qkv, nel * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(k, h_qkv + nel, nel * 2, hipMemcpyHostToDevice));
  HIP(hipMemcpy(v, h_qkv + 2 * nel, nel * 2, hipMemcpyHostToDevice));

  BSGA(bsga_layer(&s, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, NULL, rho, tau,
                  (float*)probs, (int32_t*)rp, (int32_t*)ci, cap, (uint16_t*)o, (float*)lse, ws,
                  ws_bytes, NULL));
  HIP(hipDeviceSynchronize());

  h_probs = (float*)malloc((size_t)s.heads * B * B * 4);
  h_rp = (int32_t*)malloc(((size_t)s.heads * B + 1) * 4);
  h_o = (uint16_t*)malloc(nel * 2);
  h_lse = (float*)malloc((size_t)s.heads * n * 4);
  if (!h_probs || !h_rp || !h_o || !h_lse) return 1;
  HIP(hipMemcpy(h_probs, probs, (size_t)s.heads * B * B * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(h_rp, rp, ((size_t)s.heads * B + 1) * 4, hipMemcpyDeviceToHost));
  nnz = h_rp[(size_t)s.heads * B];
  h_ci = (int32_t*)malloc((size_t)(nnz > 0 ? nnz : 1) * 4);
  if (!h_ci) return 1;
  if (nnz > 0) HIP(hipMemcpy(h_ci, ci, (size_t)nnz * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(h_o, o, nel * 2, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(h_lse, lse, (size_t)s.heads * n * 4, hipMemcpyDeviceToHost));

  f = fopen(argv[2], "wb");
  if (!f || !write_all(f, h_probs, (size_t)s.heads * B * B * 4) ||
      !write_all(f, h_rp, ((size_t)s.heads * B + 1) * 4) || !write_all(f, h_ci, (size_t)nnz * 4) ||
      !write_all(f, h_o, nel * 2) || !write_all(f, h_lse, (size_t)s.heads * n * 4)) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(f);
  HIP(hipFree(q));
  HIP(hipFree(k));
  HIP(hipFree(v));
  HIP(hipFree(o));
  HIP(hipFree(lse));
  HIP(hipFree(probs));
  HIP(hipFree(rp));
  HIP(hipFree(ci));
  if (ws) HIP(hipFree(ws));
  free(h_qkv);
  free(h_probs);
  free(h_rp);
  free(h_ci);
  free(h_o);
  free(h_lse);
  printf("ok nnz %lld\n", (long long)nnz);
  return 0;
}
