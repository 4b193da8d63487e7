/*
 * The path through the C ABI alone (no Python, no PyTorch): block masses,
 * selection and sparse attention on one layer read from a file.
 *
 * usage: losa_path INPUT OUTPUT
 * INPUT  (little endian): int32 batch, heads, tokens, tokens_alloc, head_dim,
 *        q_block, k_block; float64 p; then Q, K, V as bf16 bit patterns
 *        [batch, heads, tokens_alloc, head_dim]; then fp32 masses
 *        [batch, heads, n_q, n_k] to select from.
 * OUTPUT: fp32 M from losa_block_mass; int32 row_ptr [rows + 1], col_idx
 *        [row_ptr[rows]] and order [rows] from losa_select on the given
 *        masses; fp32 O from losa_sparse_attn on those lists.
 * Exit status: 0 on success, 2 on a HIP error, 3 on a library error, 1 on
 * bad input.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "losa.h"

#define HIP_OK(x)                                                                          \
  do {                                                                                     \
    hipError_t e_ = (x);                                                                   \
    if (e_ != hipSuccess) {                                                                \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                      \
      return 2;                                                                            \
    }                                                                                      \
  } while (0)
#define LOSA_OK_(x)                                                                        \
  do {                                                                                     \
    losa_status s_ = (x);                                                                  \
    if (s_ != LOSA_OK) {                                                                   \
      fprintf(stderr, "%s failed: %s\n", #x, losa_status_string(s_));                     \
      return 3;                                                                            \
    }                                                                                      \
  } while (0)

static void* read_all(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s INPUT OUTPUT\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 1;
  int32_t hdr[7];
  double p;
  if (fread(hdr, sizeof hdr, 1, in) != 1 || fread(&p, sizeof p, 1, in) != 1) return 1;
  losa_shape s;
  memset(&s, 0, sizeof s);
  s.batch = hdr[0];
  s.heads = hdr[1];
  s.tokens = hdr[2];
  s.tokens_alloc = hdr[3];
  s.head_dim = hdr[4];
  s.q_block = hdr[5];
  s.k_block = hdr[6];
  s.dtype = LOSA_BF16;
  s.softmax_scale = 0.0f;
  const int64_t d = s.head_dim, Na = s.tokens_alloc;
  const int64_t strides[3] = {s.heads * Na * d, Na * d, d};
  memcpy(s.q_stride, strides, sizeof strides);
  memcpy(s.k_stride, strides, sizeof strides);
  memcpy(s.v_stride, strides, sizeof strides);
  memcpy(s.o_stride, strides, sizeof strides);
  const int64_t nq = (s.tokens + s.q_block - 1) / s.q_block, nk = (s.tokens + s.k_block - 1) / s.k_block;
  const int64_t rows = (int64_t)s.batch * s.heads * nq;
  const size_t elems = (size_t)s.batch * s.heads * Na * d;
  uint16_t* hq = read_all(in, elems * 2);
  uint16_t* hk = read_all(in, elems * 2);
  uint16_t* hv = read_all(in, elems * 2);
  float* hm = read_all(in, (size_t)rows * nk * 4);
  fclose(in);
  if (!hq || !hk || !hv || !hm) return 1;

  void *q, *k, *v, *o, *ws_m, *ws_s, *ws_a;
  float *m_gpu, *m_in;
  int32_t *rp, *ci, *ord;
  size_t b_m, b_s, b_a;
  LOSA_OK_(losa_block_mass_workspace(&s, &b_m));
  LOSA_OK_(losa_select_workspace(&s, &b_s));
  LOSA_OK_(losa_sparse_attn_workspace(&s, &b_a));
  HIP_OK(hipMalloc(&q, elems * 2));
  HIP_OK(hipMalloc(&k, elems * 2));
  HIP_OK(hipMalloc(&v, elems * 2));
  HIP_OK(hipMalloc(&o, elems * 4));
  HIP_OK(hipMalloc((void**)&m_gpu, rows * nk * 4));
  HIP_OK(hipMalloc((void**)&m_in, rows * nk * 4));
  HIP_OK(hipMalloc((void**)&rp, (rows + 1) * 4));
  HIP_OK(hipMalloc((void**)&ci, rows * nk * 4));
  HIP_OK(hipMalloc((void**)&ord, rows * 4));
  HIP_OK(hipMalloc(&ws_m, b_m ? b_m : 1));
  HIP_OK(hipMalloc(&ws_s, b_s ? b_s : 1));
  HIP_OK(hipMalloc(&ws_a, b_a ? b_a : 1));
  HIP_OK(hipMemcpy(q, hq, elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, elems * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(m_in, hm, rows * nk * 4, hipMemcpyHostToDevice));

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  LOSA_OK_(losa_block_mass(&s, q, k, m_gpu, ws_m, b_m, st));
  LOSA_OK_(losa_select(&s, m_in, &p, 1, rp, ci, rows * nk, ord, ws_s, b_s, st));
  LOSA_OK_(losa_sparse_attn(&s, q, k, v, rp, ci, ord, o, LOSA_F32, ws_a, b_a, st));
  HIP_OK(hipStreamSynchronize(st));

  float* out_m = malloc(rows * nk * 4);
  int32_t* out_rp = malloc((rows + 1) * 4);
  float* out_o = malloc(elems * 4);
  int32_t* out_ord = malloc(rows * 4);
  if (!out_m || !out_rp || !out_o || !out_ord) return 1;
  HIP_OK(hipMemcpy(out_m, m_gpu, rows * nk * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out_rp, rp, (rows + 1) * 4, hipMemcpyDeviceToHost));
  const int64_t nnz = out_rp[rows];
  int32_t* out_ci = malloc((nnz ? nnz : 1) * 4);
  if (!out_ci) return 1;
  HIP_OK(hipMemcpy(out_ci, ci, nnz * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out_ord, ord, rows * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out_o, o, elems * 4, hipMemcpyDeviceToHost));

  FILE* out = fopen(argv[2], "wb");
  if (!out) return 1;
  fwrite(out_m, 4, rows * nk, out);
  fwrite(out_rp, 4, rows + 1, out);
  fwrite(out_ci, 4, nnz, out);
  fwrite(out_ord, 4, rows, out);
  fwrite(out_o, 4, elems, out);
  fclose(out);
  printf("losa_path: abi %d, %lld rows, %lld kept blocks\n", losa_abi_version(), (long long)rows, (long long)nnz);
  HIP_OK(hipStreamDestroy(st));
  return 0;
}
