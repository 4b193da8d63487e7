// Internal interface between the C ABI (losa_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace losa {

// Validated geometry of one call, derived from losa_shape on the host.
struct Geom {
  int B, H, N, Na, D, R, C, nq, nk;
  int bf16;          // 1: Q/K/V are bf16, 0: f32
  float scale;       // softmax scale (1/sqrt(d) by default)
  float scale_log2;  // scale * log2(e): scores in log2 units
  int64_t qs[3], ks[3], vs[3], os[3];
  __host__ __device__ int rows() const { return B * H * nq; }
};

// Per-head fixed-point selection thresholds P = floor(p * 2^32 + 1/2),
// passed by value as a kernel argument.
constexpr int kMaxHeadsP = 128;
struct PTable {
  uint64_t P[kMaxHeadsP];
  int per_head;  // 0: P[0] for every head
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// True when the bf16 matrix-core kernels cover this geometry.
inline bool mfma_path(const Geom& g) {
  return g.bf16 && (g.D == 64 || g.D == 128) && (g.R == 64 || g.R == 128);
}

// Block masses.  Workspace: on the matrix-core path the per-(query row, key
// block) partial sums and a packed copy of K; otherwise the row log-sum-exp.
size_t mass_ws_bytes(const Geom& g);
hipError_t launch_block_mass(const Geom& g, const void* Q, const void* K, float* M, void* ws,
                             hipStream_t stream);

// Selection.
struct SelectWs {
  int32_t* counts;      // [rows] kept blocks per row
  uint32_t* keep;       // [rows][keep_words] the kept blocks as bits (bit j%32 of word j/32)
  int keep_words;       // ceil(nk / 32)
  int32_t* local_off;   // [rows] kept blocks of the head's earlier rows
  int32_t* head_total;  // [B*H] kept blocks per head
  int32_t* head_base;   // [B*H] first col_idx slot of each head
  int32_t* done;        // [1] finished workgroups of the order kernel (cleared by the count kernel before it)
  int32_t* ranked;      // [rows] row of rank r in head h at h * nq + r
  int32_t* gkey;        // [B*H*ngh] count of each work group's first row
  int32_t* bucket_start;  // [B*H][nk + 2] first rank in the head of count nk - b (b = nk + 1: n_q)
  int ngh;              // work groups per head: ceil(nq / kGroupRows)
};
constexpr int kGroupRows = 32;    // rows per work group of the budget order (one XCD's CUs)
size_t select_ws_bytes(const Geom& g, SelectWs* layout, char* base);
hipError_t launch_select(const Geom& g, const float* M, const PTable& pt, int32_t* row_ptr,
                         int32_t* col_idx, int32_t* order, const SelectWs& ws, hipStream_t stream);
// Device address of the selector's file-scope scratch array on the current
// device (looked up once per device).
hipError_t select_scratch(void** ptr);
// Online block thresholding: per-head theta (or one for all) by value.
struct ThetaTable {
  double t[kMaxHeadsP];
  int per_head;  // 0: t[0] for every head
};
hipError_t launch_select_threshold(const Geom& g, const float* M, const ThetaTable& tt, int32_t* row_ptr,
                                   int32_t* col_idx, int32_t* order, const SelectWs& ws, hipStream_t stream);
// Row offsets of each head and (want_order) the work order's ranks and
// group slots from the kept counts in ws.counts, one launch; the writing
// kernel after it stores row_ptr and order (shared by the selector, online
// thresholding and the list merge).
void launch_order(const Geom& g, const SelectWs& ws, int32_t* row_ptr, bool want_order, hipStream_t stream);
// Per-head choice between two list sets (selector workspace).
hipError_t launch_merge_lists(const Geom& g, const int32_t* take_b, const int32_t* rpa, const int32_t* cia,
                              const int32_t* rpb, const int32_t* cib, int32_t* row_ptr, int32_t* col_idx,
                              int32_t* order, const SelectWs& ws, hipStream_t stream);

// Query-key drift per head since a reference step.
size_t drift_ws_bytes(const Geom& g);
hipError_t launch_qk_drift(const Geom& g, const void* Q, const void* K, const void* Qr, const void* Kr, double tau,
                           double* drift, int32_t* refresh, void* ws, hipStream_t stream);

hipError_t launch_retained_mass(const Geom& g, const float* M, const int32_t* row_ptr,
                                const int32_t* col_idx, float* kept, hipStream_t stream);

// Sparse attention.  Workspace: packed K and V on the matrix-core path, none
// otherwise.  Null row_ptr/col_idx (SIMT path only) means every key block.
size_t attn_ws_bytes(const Geom& g);
hipError_t launch_sparse_attn(const Geom& g, const void* Q, const void* K, const void* V,
                              const int32_t* row_ptr, const int32_t* col_idx, const int32_t* order,
                              void* O, int o_bf16, void* ws, hipStream_t stream);

// Dense attention with exact block masses in one pass (construction step).
size_t dense_ws_bytes(const Geom& g);
// The same kernel over a row's listed blocks only (matrix-core shapes only):
// sparse attention plus the masses within the lists.
size_t sparse_mass_ws_bytes(const Geom& g);
hipError_t launch_sparse_attn_mass(const Geom& g, const void* Q, const void* K, const void* V,
                                   const int32_t* row_ptr, const int32_t* col_idx, const int32_t* order,
                                   float* M, void* O, int o_bf16, void* ws, hipStream_t stream);
hipError_t launch_dense_attn_mass(const Geom& g, const void* Q, const void* K, const void* V, float* M, void* O,
                                  int o_bf16, void* ws, hipStream_t stream);

// Sparse attention with on-the-fly block thresholding against the pooled
// proxy: ln(theta) per head (or one for all) and the log of the valid keys of
// a full and of the last key block, all computed on the host.
struct InPass {
  double ln_theta[kMaxHeadsP];
  int per_head;
  double ln_c, ln_last;
};
size_t attn_threshold_ws_bytes(const Geom& g);
hipError_t launch_sparse_attn_threshold(const Geom& g, const void* Q, const void* K, const void* V, const InPass& ip,
                                        void* O, int o_bf16, int32_t* kept_count, uint32_t* kept_mask, void* ws,
                                        hipStream_t stream);
// Block means of bf16 Q (query blocks) and K (key blocks) in fp64:
// qbar [B*H*nq][D], kbar [B*H*nk][D].
void launch_block_means64(const Geom& g, const void* Q, const void* K, double* qbar, double* kbar, hipStream_t st);

// Pooled proxy masses (block-mean Q and K, block-weighted softmax).
size_t pooled_ws_bytes(const Geom& g);
hipError_t launch_pooled_mass(const Geom& g, const void* Q, const void* K, float* P, void* ws, hipStream_t stream);

}  // namespace losa
