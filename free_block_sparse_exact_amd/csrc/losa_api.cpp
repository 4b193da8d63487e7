// C ABI of the library: argument validation (before any HIP call),
// workspace sizing and kernel dispatch.  See include/losa.h for the contract.
#include "losa.h"

#include <math.h>
#include <string.h>

#include "losa_internal.hpp"

namespace {

using losa::Geom;

bool is_block(int x) { return x == 32 || x == 64 || x == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool strides_ok(const int64_t s[3], int head_dim, int elem_multiple) {
  for (int t = 0; t < 3; ++t)
    if (s[t] <= 0 || s[t] % elem_multiple != 0) return false;
  return s[2] >= head_dim;
}

// Shape checks shared by every call.  Fills g on success.
losa_status make_geom(const losa_shape* s, Geom* g) {
  if (!s) return LOSA_ERR_NULL;
  if (s->reserved != 0) return LOSA_ERR_INVALID_ARG;
  if (s->batch < 1 || s->heads < 1 || s->tokens < 1) return LOSA_ERR_INVALID_ARG;
  if (s->dtype != LOSA_F32 && s->dtype != LOSA_BF16) return LOSA_ERR_INVALID_ARG;
  if (!(s->softmax_scale == s->softmax_scale) || isinf(s->softmax_scale)) return LOSA_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128) return LOSA_ERR_UNSUPPORTED;
  if (!is_block(s->q_block) || !is_block(s->k_block)) return LOSA_ERR_UNSUPPORTED;
  const int64_t nq = ((int64_t)s->tokens + s->q_block - 1) / s->q_block;
  const int64_t nk = ((int64_t)s->tokens + s->k_block - 1) / s->k_block;
  if (nk > LOSA_MAX_KEY_BLOCKS) return LOSA_ERR_UNSUPPORTED;
  const int64_t need = nq * s->q_block > nk * s->k_block ? nq * s->q_block : nk * s->k_block;
  if (s->tokens_alloc < need) return LOSA_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)s->batch * s->heads * nq;
  if (rows * nk >= ((int64_t)1 << 31)) return LOSA_ERR_UNSUPPORTED;   // int32 CSR offsets
  if ((int64_t)s->batch * s->heads > 65535) return LOSA_ERR_UNSUPPORTED;     // grid z of the V transpose
  g->B = s->batch;
  g->H = s->heads;
  g->N = s->tokens;
  g->Na = s->tokens_alloc;
  g->D = s->head_dim;
  g->R = s->q_block;
  g->C = s->k_block;
  g->nq = (int)nq;
  g->nk = (int)nk;
  g->bf16 = s->dtype == LOSA_BF16;
  g->scale = s->softmax_scale > 0.f ? s->softmax_scale : 1.0f / sqrtf((float)s->head_dim);
  g->scale_log2 = g->scale * 1.4426950408889634f;
  memcpy(g->qs, s->q_stride, sizeof g->qs);
  memcpy(g->ks, s->k_stride, sizeof g->ks);
  memcpy(g->vs, s->v_stride, sizeof g->vs);
  memcpy(g->os, s->o_stride, sizeof g->os);
  return LOSA_OK;
}

losa_status check_input(const Geom& g, const void* p, const int64_t st[3]) {
  if (!p) return LOSA_ERR_NULL;
  if (!aligned16(p) || !strides_ok(st, g.D, g.bf16 ? 8 : 4)) return LOSA_ERR_INVALID_ARG;
  return LOSA_OK;
}

losa_status hip_status(hipError_t e) { return e == hipSuccess ? LOSA_OK : LOSA_ERR_HIP; }

size_t mass_ws(const Geom& g) { return losa::mass_ws_bytes(g); }

}  // namespace

extern "C" {

int32_t losa_abi_version(void) { return LOSA_ABI_VERSION; }

const char* losa_status_string(losa_status status) {
  switch (status) {
    case LOSA_OK: return "ok";
    case LOSA_ERR_NULL: return "a required pointer is NULL";
    case LOSA_ERR_INVALID_ARG: return "invalid argument (size, stride, alignment or parameter)";
    case LOSA_ERR_UNSUPPORTED: return "unsupported shape (head_dim, block size or problem size)";
    case LOSA_ERR_WORKSPACE: return "workspace too small or misaligned";
    case LOSA_ERR_CAPACITY: return "col_idx capacity below batch*heads*n_q*n_k";
    case LOSA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

losa_status losa_block_mass_workspace(const losa_shape* shape, size_t* bytes) {
  Geom g;
  if (!bytes) return LOSA_ERR_NULL;
  const losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  *bytes = mass_ws(g);
  return LOSA_OK;
}

losa_status losa_block_mass(const losa_shape* shape, const void* Q, const void* K, float* M, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if ((st = check_input(g, Q, g.qs)) != LOSA_OK) return st;
  if ((st = check_input(g, K, g.ks)) != LOSA_OK) return st;
  if (!M || !ws) return LOSA_ERR_NULL;
  if (!aligned16(M)) return LOSA_ERR_INVALID_ARG;
  if (ws_bytes < mass_ws(g) || !aligned16(ws)) return LOSA_ERR_WORKSPACE;
  return hip_status(losa::launch_block_mass(g, Q, K, M, ws, stream));
}

losa_status losa_select_workspace(const losa_shape* shape, size_t* bytes) {
  Geom g;
  if (!bytes) return LOSA_ERR_NULL;
  const losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  *bytes = losa::select_ws_bytes(g, nullptr, nullptr);
  return LOSA_OK;
}

}  // extern "C"

namespace {

// Checks shared by losa_select and losa_select_noalloc (everything but the
// workspace); fills g and pt.
losa_status select_args(const losa_shape* shape, const float* M, const double* p, int32_t n_p,
                        const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity, Geom* g,
                        losa::PTable* pt) {
  losa_status st = make_geom(shape, g);
  if (st != LOSA_OK) return st;
  if (!M || !p || !row_ptr || !col_idx) return LOSA_ERR_NULL;
  if (n_p != 1 && n_p != g->H) return LOSA_ERR_INVALID_ARG;
  if (n_p > 1 && n_p > LOSA_MAX_HEADS_P) return LOSA_ERR_UNSUPPORTED;
  memset(pt, 0, sizeof *pt);
  pt->per_head = n_p > 1;
  for (int t = 0; t < n_p; ++t) {
    if (!(p[t] > 0.0 && p[t] <= 1.0)) return LOSA_ERR_INVALID_ARG;
    pt->P[t] = (uint64_t)floor(p[t] * 4294967296.0 + 0.5);
  }
  if (col_capacity < (int64_t)g->rows() * g->nk) return LOSA_ERR_CAPACITY;
  return LOSA_OK;
}

}  // namespace

extern "C" {

losa_status losa_select(const losa_shape* shape, const float* M, const double* p, int32_t n_p, int32_t* row_ptr,
                        int32_t* col_idx, int64_t col_capacity, int32_t* order, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  Geom g;
  losa::PTable pt;
  const losa_status st = select_args(shape, M, p, n_p, row_ptr, col_idx, col_capacity, &g, &pt);
  if (st != LOSA_OK) return st;
  if (!ws) return LOSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return LOSA_ERR_WORKSPACE;
  losa::SelectWs layout;
  if (ws_bytes < losa::select_ws_bytes(g, &layout, reinterpret_cast<char*>(ws))) return LOSA_ERR_WORKSPACE;
  return hip_status(losa::launch_select(g, M, pt, row_ptr, col_idx, order, layout, stream));
}

losa_status losa_select_noalloc(const losa_shape* shape, const float* M, const double* p, int32_t n_p,
                                int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* order,
                                hipStream_t stream) {
  Geom g;
  losa::PTable pt;
  const losa_status st = select_args(shape, M, p, n_p, row_ptr, col_idx, col_capacity, &g, &pt);
  if (st != LOSA_OK) return st;
  if (losa::select_ws_bytes(g, nullptr, nullptr) > LOSA_SELECT_SCRATCH_BYTES) return LOSA_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (losa::select_scratch(&scratch) != hipSuccess) return LOSA_ERR_HIP;
  losa::SelectWs layout;
  losa::select_ws_bytes(g, &layout, reinterpret_cast<char*>(scratch));
  return hip_status(losa::launch_select(g, M, pt, row_ptr, col_idx, order, layout, stream));
}

losa_status losa_sparse_attn_workspace(const losa_shape* shape, size_t* bytes) {
  Geom g;
  if (!bytes) return LOSA_ERR_NULL;
  const losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  *bytes = losa::attn_ws_bytes(g);
  return LOSA_OK;
}

losa_status losa_sparse_attn(const losa_shape* shape, const void* Q, const void* K, const void* V,
                             const int32_t* row_ptr, const int32_t* col_idx, const int32_t* order, void* O,
                             losa_dtype o_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if ((st = check_input(g, Q, g.qs)) != LOSA_OK) return st;
  if ((st = check_input(g, K, g.ks)) != LOSA_OK) return st;
  if ((st = check_input(g, V, g.vs)) != LOSA_OK) return st;
  if (!row_ptr || !col_idx || !O) return LOSA_ERR_NULL;
  if (o_dtype != LOSA_F32 && o_dtype != LOSA_BF16) return LOSA_ERR_INVALID_ARG;
  if (!aligned16(O) || !strides_ok(g.os, g.D, o_dtype == LOSA_BF16 ? 8 : 4)) return LOSA_ERR_INVALID_ARG;
  const size_t need = losa::attn_ws_bytes(g);
  if (need > 0) {
    if (!ws) return LOSA_ERR_NULL;
    if (ws_bytes < need || !aligned16(ws)) return LOSA_ERR_WORKSPACE;
  }
  return hip_status(losa::launch_sparse_attn(g, Q, K, V, row_ptr, col_idx, order, O, o_dtype == LOSA_BF16, ws,
                                             stream));
}

losa_status losa_sparse_attn_threshold_workspace(const losa_shape* shape, size_t* bytes) {
  Geom g;
  if (!bytes) return LOSA_ERR_NULL;
  const losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if (!losa::mfma_path(g)) return LOSA_ERR_UNSUPPORTED;
  *bytes = losa::attn_threshold_ws_bytes(g);
  return LOSA_OK;
}

losa_status losa_sparse_attn_threshold(const losa_shape* shape, const void* Q, const void* K, const void* V,
                                       const double* theta, int32_t n_theta, void* O, losa_dtype o_dtype,
                                       int32_t* kept_count, uint32_t* kept_mask, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if (!losa::mfma_path(g)) return LOSA_ERR_UNSUPPORTED;
  if ((st = check_input(g, Q, g.qs)) != LOSA_OK) return st;
  if ((st = check_input(g, K, g.ks)) != LOSA_OK) return st;
  if ((st = check_input(g, V, g.vs)) != LOSA_OK) return st;
  if (!theta || !O || !ws) return LOSA_ERR_NULL;
  if (n_theta != 1 && n_theta != g.H) return LOSA_ERR_INVALID_ARG;
  if (n_theta > 1 && n_theta > LOSA_MAX_HEADS_P) return LOSA_ERR_UNSUPPORTED;
  if (o_dtype != LOSA_F32 && o_dtype != LOSA_BF16) return LOSA_ERR_INVALID_ARG;
  if (!aligned16(O) || !strides_ok(g.os, g.D, o_dtype == LOSA_BF16 ? 8 : 4)) return LOSA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(kept_count) & 3u) != 0 || (reinterpret_cast<uintptr_t>(kept_mask) & 3u) != 0)
    return LOSA_ERR_INVALID_ARG;
  losa::InPass ip;
  memset(&ip, 0, sizeof ip);
  ip.per_head = n_theta > 1;
  for (int t = 0; t < n_theta; ++t) {
    if (!(theta[t] > 0.0 && theta[t] <= 1.0)) return LOSA_ERR_INVALID_ARG;
    ip.ln_theta[t] = log(theta[t]);
  }
  ip.ln_c = log((double)g.C);
  ip.ln_last = log((double)(g.N - (g.nk - 1) * g.C));
  if (ws_bytes < losa::attn_threshold_ws_bytes(g) || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return LOSA_ERR_WORKSPACE;
  return hip_status(losa::launch_sparse_attn_threshold(g, Q, K, V, ip, O, o_dtype == LOSA_BF16, kept_count,
                                                       kept_mask, ws, stream));
}

losa_status losa_dense_attn_mass_workspace(const losa_shape* shape, size_t* bytes) {
  Geom g;
  if (!bytes) return LOSA_ERR_NULL;
  const losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  *bytes = losa::dense_ws_bytes(g);
  return LOSA_OK;
}

losa_status losa_dense_attn_mass(const losa_shape* shape, const void* Q, const void* K, const void* V, float* M,
                                 void* O, losa_dtype o_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if ((st = check_input(g, Q, g.qs)) != LOSA_OK) return st;
  if ((st = check_input(g, K, g.ks)) != LOSA_OK) return st;
  if ((st = check_input(g, V, g.vs)) != LOSA_OK) return st;
  if (!M || !O || !ws) return LOSA_ERR_NULL;
  if (o_dtype != LOSA_F32 && o_dtype != LOSA_BF16) return LOSA_ERR_INVALID_ARG;
  if (!aligned16(M)) return LOSA_ERR_INVALID_ARG;
  if (!aligned16(O) || !strides_ok(g.os, g.D, o_dtype == LOSA_BF16 ? 8 : 4)) return LOSA_ERR_INVALID_ARG;
  if (ws_bytes < losa::dense_ws_bytes(g) || !aligned16(ws)) return LOSA_ERR_WORKSPACE;
  return hip_status(losa::launch_dense_attn_mass(g, Q, K, V, M, O, o_dtype == LOSA_BF16, ws, stream));
}

losa_status losa_sparse_attn_mass_workspace(const losa_shape* shape, size_t* bytes) {
  Geom g;
  if (!bytes) return LOSA_ERR_NULL;
  const losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if (!losa::mfma_path(g)) return LOSA_ERR_UNSUPPORTED;
  *bytes = losa::sparse_mass_ws_bytes(g);
  return LOSA_OK;
}

losa_status losa_sparse_attn_mass(const losa_shape* shape, const void* Q, const void* K, const void* V,
                                  const int32_t* row_ptr, const int32_t* col_idx, const int32_t* order,
                                  float* M, void* O, losa_dtype o_dtype, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if (!losa::mfma_path(g)) return LOSA_ERR_UNSUPPORTED;
  if ((st = check_input(g, Q, g.qs)) != LOSA_OK) return st;
  if ((st = check_input(g, K, g.ks)) != LOSA_OK) return st;
  if ((st = check_input(g, V, g.vs)) != LOSA_OK) return st;
  if (!row_ptr || !col_idx || !M || !O || !ws) return LOSA_ERR_NULL;
  if (o_dtype != LOSA_F32 && o_dtype != LOSA_BF16) return LOSA_ERR_INVALID_ARG;
  if (!aligned16(M)) return LOSA_ERR_INVALID_ARG;
  if (!aligned16(O) || !strides_ok(g.os, g.D, o_dtype == LOSA_BF16 ? 8 : 4)) return LOSA_ERR_INVALID_ARG;
  if (ws_bytes < losa::sparse_mass_ws_bytes(g) || !aligned16(ws)) return LOSA_ERR_WORKSPACE;
  return hip_status(losa::launch_sparse_attn_mass(g, Q, K, V, row_ptr, col_idx, order, M, O,
                                                  o_dtype == LOSA_BF16, ws, stream));
}

losa_status losa_pooled_mass_workspace(const losa_shape* shape, size_t* bytes) {
  Geom g;
  if (!bytes) return LOSA_ERR_NULL;
  const losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  *bytes = losa::pooled_ws_bytes(g);
  return LOSA_OK;
}

losa_status losa_pooled_mass(const losa_shape* shape, const void* Q, const void* K, float* P, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if ((st = check_input(g, Q, g.qs)) != LOSA_OK) return st;
  if ((st = check_input(g, K, g.ks)) != LOSA_OK) return st;
  if (!P || !ws) return LOSA_ERR_NULL;
  if (!aligned16(P)) return LOSA_ERR_INVALID_ARG;
  if (ws_bytes < losa::pooled_ws_bytes(g) || !aligned16(ws)) return LOSA_ERR_WORKSPACE;
  return hip_status(losa::launch_pooled_mass(g, Q, K, P, ws, stream));
}

losa_status losa_retained_mass(const losa_shape* shape, const float* M, const int32_t* row_ptr,
                               const int32_t* col_idx, float* kept, hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if (!M || !row_ptr || !col_idx || !kept) return LOSA_ERR_NULL;
  return hip_status(losa::launch_retained_mass(g, M, row_ptr, col_idx, kept, stream));
}

losa_status losa_select_threshold_workspace(const losa_shape* shape, size_t* bytes) {
  return losa_select_workspace(shape, bytes);
}

losa_status losa_select_threshold(const losa_shape* shape, const float* M, const double* theta, int32_t n_theta,
                                  int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* order, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if (!M || !theta || !row_ptr || !col_idx || !ws) return LOSA_ERR_NULL;
  if (n_theta != 1 && n_theta != g.H) return LOSA_ERR_INVALID_ARG;
  if (n_theta > 1 && n_theta > LOSA_MAX_HEADS_P) return LOSA_ERR_UNSUPPORTED;
  losa::ThetaTable tt;
  memset(&tt, 0, sizeof tt);
  tt.per_head = n_theta > 1;
  for (int t = 0; t < n_theta; ++t) {
    if (!(theta[t] > 0.0 && theta[t] <= 1.0)) return LOSA_ERR_INVALID_ARG;
    tt.t[t] = theta[t];
  }
  if (col_capacity < (int64_t)g.rows() * g.nk) return LOSA_ERR_CAPACITY;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return LOSA_ERR_WORKSPACE;
  losa::SelectWs layout;
  if (ws_bytes < losa::select_ws_bytes(g, &layout, reinterpret_cast<char*>(ws))) return LOSA_ERR_WORKSPACE;
  return hip_status(losa::launch_select_threshold(g, M, tt, row_ptr, col_idx, order, layout, stream));
}

losa_status losa_qk_drift_workspace(const losa_shape* shape, size_t* bytes) {
  Geom g;
  if (!bytes) return LOSA_ERR_NULL;
  const losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  *bytes = losa::drift_ws_bytes(g);
  return LOSA_OK;
}

losa_status losa_qk_drift(const losa_shape* shape, const void* Q, const void* K, const void* Q_ref,
                          const void* K_ref, double tau, double* drift, int32_t* refresh, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if ((st = check_input(g, Q, g.qs)) != LOSA_OK) return st;
  if ((st = check_input(g, K, g.ks)) != LOSA_OK) return st;
  if ((st = check_input(g, Q_ref, g.qs)) != LOSA_OK) return st;
  if ((st = check_input(g, K_ref, g.ks)) != LOSA_OK) return st;
  if (!drift || !ws) return LOSA_ERR_NULL;
  if (!(tau == tau)) return LOSA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(drift) & 7u) != 0 || (reinterpret_cast<uintptr_t>(refresh) & 3u) != 0)
    return LOSA_ERR_INVALID_ARG;
  if (ws_bytes < losa::drift_ws_bytes(g) || !aligned16(ws)) return LOSA_ERR_WORKSPACE;
  return hip_status(losa::launch_qk_drift(g, Q, K, Q_ref, K_ref, tau, drift, refresh, ws, stream));
}

losa_status losa_merge_lists_workspace(const losa_shape* shape, size_t* bytes) {
  return losa_select_workspace(shape, bytes);
}

losa_status losa_merge_lists(const losa_shape* shape, const int32_t* take_b, const int32_t* row_ptr_a,
                             const int32_t* col_idx_a, const int32_t* row_ptr_b, const int32_t* col_idx_b,
                             int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity, int32_t* order, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  Geom g;
  losa_status st = make_geom(shape, &g);
  if (st != LOSA_OK) return st;
  if (!take_b || !row_ptr_a || !col_idx_a || !row_ptr_b || !col_idx_b || !row_ptr || !col_idx || !ws)
    return LOSA_ERR_NULL;
  if (col_capacity < (int64_t)g.rows() * g.nk) return LOSA_ERR_CAPACITY;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return LOSA_ERR_WORKSPACE;
  losa::SelectWs layout;
  if (ws_bytes < losa::select_ws_bytes(g, &layout, reinterpret_cast<char*>(ws))) return LOSA_ERR_WORKSPACE;
  return hip_status(losa::launch_merge_lists(g, take_b, row_ptr_a, col_idx_a, row_ptr_b, col_idx_b, row_ptr,
                                             col_idx, order, layout, stream));
}

}  // extern "C"
