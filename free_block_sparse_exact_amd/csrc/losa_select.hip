// Retained-mass (top-p) key-block selection to CSR (LoSA page, Methodology
// Summary, one-time pattern construction: per head and query block, sort
// the key blocks by decreasing mass and keep the shortest prefix whose
// cumulative mass reaches p times the block's total).
//
// Kernels, in launch order:
//   fill        zero the count histogram (a kernel, not a memset, so the
//               sequence can sit inside a captured graph);
//   cut         one workgroup per row: sort keys (mass desc, index asc) in
//               LDS with a bitonic network, integer prefix sums, find the
//               kept count s and the sort key kappa of the last kept block;
//               bump the histogram of counts for the work order;
//   scan        one workgroup: exclusive scan of counts -> row_ptr, and of
//               the count histogram -> per-(count, row chunk) offsets;
//   compact     one workgroup per row: block j is kept iff its sort key is
//               <= kappa; write kept indices ascending at row_ptr[row];
//   place       one workgroup per chunk of rows: stable placement of rows
//               by count, descending -> order.
//
// Sort key of block j with (sanitised) mass bits u: ((2^32-1-u) << 32) | j.
// For non-negative floats the bit pattern orders like the value, so an
// ascending sort of keys is (mass descending, index ascending), and "kept"
// is exactly "key <= key of the s-th block".
//
// Exact cumulative sums: e = binary exponent of the row maximum (max = f*2^e,
// 1/2 <= f < 1), q_j = ceil(m_j * 2^(51-e)) as uint64 (<= 2^51 each, so a row
// of up to 4096 blocks sums below 2^63), T = ceil(P * sum q / 2^32) with a
// 128-bit product, s = least prefix length with sum >= T; P = 2^32 keeps all.
#include "losa_device.hpp"
#include "losa_internal.hpp"

namespace losa {
namespace {

constexpr int kSelThreads = 256;

__device__ __forceinline__ uint32_t sanitized_bits(float m) {
  // NaN, +-inf, negatives and -0 count as mass 0.
  return (m > 0.f && m < __builtin_huge_valf()) ? __float_as_uint(m) : 0u;
}

__device__ __forceinline__ uint64_t sort_key(uint32_t u, int j) {
  return ((uint64_t)(0xFFFFFFFFu - u) << 32) | (uint32_t)j;
}

// frexp exponent of the float with bits u > 0.
__device__ __forceinline__ int frexp_exp(uint32_t u) {
  const uint32_t ef = u >> 23;
  if (ef != 0) return (int)ef - 126;
  const uint32_t frac = u & 0x7FFFFFu;
  return (31 - __clz(frac)) + 1 - 149;
}

// q = ceil(m * 2^(51 - e)) for the float with bits u (u = 0 -> 0).
__device__ __forceinline__ uint64_t fixed_units(uint32_t u, int e) {
  if (u == 0) return 0;
  const uint32_t ef = u >> 23, frac = u & 0x7FFFFFu;
  const uint64_t mant = ef ? (uint64_t)(frac | 0x800000u) : (uint64_t)frac;
  const int e2 = ef ? (int)ef - 150 : -149;  // m = mant * 2^e2
  const int sh = e2 + 51 - e;
  if (sh >= 0) return mant << sh;
  const int rs = -sh;
  if (rs >= 63) return 1;  // 0 < m*2^(51-e) < 1
  return (mant + ((uint64_t)1 << rs) - 1) >> rs;
}

// ceil(P * total / 2^32), P <= 2^32, total < 2^64 (product < 2^96).
__device__ __forceinline__ uint64_t threshold(uint64_t P, uint64_t total) {
  const uint64_t lo = P * total;
  const uint64_t hi = __umul64hi(P, total);
  return ((hi << 32) | (lo >> 32)) + ((lo & 0xFFFFFFFFull) != 0 ? 1 : 0);
}

// Inclusive scan of a uint64 over the workgroup (blockDim = kSelThreads).
__device__ __forceinline__ uint64_t block_inclusive_scan_u64(uint64_t v, uint64_t* wsum, uint64_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int ww = 0; ww < kSelThreads / 64; ++ww) {
    const uint64_t s = wsum[ww];
    if (ww < w) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

__device__ __forceinline__ int block_sum_i32(int v, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  if (lane == 0) wsum[w] = v;
  __syncthreads();
  int all = 0;
#pragma unroll
  for (int ww = 0; ww < kSelThreads / 64; ++ww) all += wsum[ww];
  __syncthreads();
  return all;
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x)
    p[t] = v;
}

// One workgroup per row.  Dynamic LDS: npad uint64 keys.
__global__ __launch_bounds__(kSelThreads) void cut_kernel(const Geom g, const float* __restrict__ M,
                                                          const PTable pt, int npad,
                                                          int32_t* __restrict__ counts,
                                                          uint64_t* __restrict__ kappa,
                                                          int32_t* __restrict__ chunk_hist, int nchunk) {
  extern __shared__ uint64_t keys[];
  __shared__ uint64_t wsum64[kSelThreads / 64];
  __shared__ int wsum32[kSelThreads / 64];
  __shared__ uint32_t wmax[kSelThreads / 64];
  const int row = blockIdx.x;
  const int h = (row / g.nq) % g.H;
  const uint64_t P = pt.P[pt.per_head ? h : 0];
  const int nk = g.nk;
  const float* Mrow = M + (int64_t)row * nk;

  uint32_t umax = 0;
  for (int j = threadIdx.x; j < npad; j += kSelThreads) {
    uint64_t key = ~0ull;
    if (j < nk) {
      const uint32_t u = sanitized_bits(Mrow[j]);
      umax = umax > u ? umax : u;
      key = sort_key(u, j);
    }
    keys[j] = key;
  }
  umax = wave_max_u32(umax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = umax;
  __syncthreads();
#pragma unroll
  for (int ww = 0; ww < kSelThreads / 64; ++ww) umax = umax > wmax[ww] ? umax : wmax[ww];

  // Bitonic sort, ascending.
  for (int k = 2; k <= npad; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int t = threadIdx.x; t < (npad >> 1); t += kSelThreads) {
        const int a = ((t & ~(jj - 1)) << 1) | (t & (jj - 1));
        const int bb = a + jj;
        const uint64_t ka = keys[a], kb = keys[bb];
        const bool up = (a & k) == 0;
        if ((ka > kb) == up) { keys[a] = kb; keys[bb] = ka; }
      }
      __syncthreads();
    }
  }

  int s;
  if (P == (1ull << 32)) {
    s = nk;
  } else {
    const int e = umax ? frexp_exp(umax) : 0;
    // Each thread owns a contiguous run of sorted positions.
    const int per = (npad + kSelThreads - 1) / kSelThreads;
    const int p0 = threadIdx.x * per;
    uint64_t run = 0;
    for (int t = 0; t < per; ++t) {
      const int pos = p0 + t;
      if (pos < nk) run += fixed_units(0xFFFFFFFFu - (uint32_t)(keys[pos] >> 32), e);
    }
    uint64_t total;
    const uint64_t incl = block_inclusive_scan_u64(run, wsum64, &total);
    const uint64_t T = threshold(P, total);
    uint64_t pre = incl - run;
    int below = 0;
    for (int t = 0; t < per; ++t) {
      const int pos = p0 + t;
      if (pos < nk) {
        pre += fixed_units(0xFFFFFFFFu - (uint32_t)(keys[pos] >> 32), e);
        below += pre < T ? 1 : 0;
      }
    }
    below = block_sum_i32(below, wsum32);
    s = below + 1;
    if (s > nk) s = nk;
  }
  if (threadIdx.x == 0) {
    counts[row] = s;
    kappa[row] = keys[s - 1];
    if (chunk_hist) atomicAdd(&chunk_hist[(int64_t)(nk - s) * nchunk + row / kOrderChunk], 1);
  }
}

// Single workgroup of 1024 threads: exclusive scans.
__device__ void block_exclusive_scan_i32(int32_t* data, int n, int32_t* out, int32_t* out_total,
                                         int* wsum) {
  const int nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int p0 = threadIdx.x * per;
  int run = 0;
  for (int t = 0; t < per; ++t) {
    const int pos = p0 + t;
    if (pos < n) run += data[pos];
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = nt >> 6;
  int v = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int before = 0, all = 0;
  for (int ww = 0; ww < nw; ++ww) {
    const int s = wsum[ww];
    if (ww < w) before += s;
    all += s;
  }
  __syncthreads();
  int pre = before + v - run;
  for (int t = 0; t < per; ++t) {
    const int pos = p0 + t;
    if (pos < n) {
      const int x = data[pos];
      out[pos] = pre;
      pre += x;
    }
  }
  if (threadIdx.x == 0 && out_total) *out_total = all;
  __syncthreads();
}

__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts, int rows,
                                                    int32_t* __restrict__ row_ptr, int32_t* chunk_hist,
                                                    int hist_len) {
  __shared__ int wsum[16];
  block_exclusive_scan_i32(const_cast<int32_t*>(counts), rows, row_ptr, row_ptr + rows, wsum);
  if (chunk_hist) block_exclusive_scan_i32(chunk_hist, hist_len, chunk_hist, nullptr, wsum);
}

// One workgroup per row: ascending compaction of {j : key_j <= kappa}.
__global__ __launch_bounds__(kSelThreads) void compact_kernel(const Geom g, const float* __restrict__ M,
                                                              const uint64_t* __restrict__ kappa,
                                                              const int32_t* __restrict__ row_ptr,
                                                              int32_t* __restrict__ col_idx) {
  __shared__ int wsum[kSelThreads / 64];
  const int row = blockIdx.x;
  const int nk = g.nk;
  const float* Mrow = M + (int64_t)row * nk;
  const uint64_t kap = kappa[row];
  const int per = (nk + kSelThreads - 1) / kSelThreads;
  const int j0 = threadIdx.x * per;
  unsigned flags = 0;  // per <= 16 since nk <= 4096
  int cnt = 0;
  for (int t = 0; t < per; ++t) {
    const int j = j0 + t;
    if (j < nk && sort_key(sanitized_bits(Mrow[j]), j) <= kap) {
      flags |= 1u << t;
      ++cnt;
    }
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int v = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int ww = 0; ww < kSelThreads / 64; ++ww)
    if (ww < w) before += wsum[ww];
  int pos = row_ptr[row] + before + v - cnt;
  for (int t = 0; t < per; ++t)
    if (flags & (1u << t)) col_idx[pos++] = j0 + t;
}

// One workgroup (kOrderChunk threads) per chunk of rows: stable placement by
// count descending.  chunk_hist holds, after the scan, the first output slot
// of each (nk - count, chunk) pair; waves take turns so that rows keep their
// index order within a count.
__global__ __launch_bounds__(kOrderChunk) void place_kernel(const int32_t* __restrict__ counts, int rows,
                                                            int nk, const int32_t* __restrict__ chunk_hist,
                                                            int nchunk, int32_t* __restrict__ order) {
  extern __shared__ int run[];  // [nk + 1] slots already used by earlier waves of this chunk
  const int chunk = blockIdx.x;
  for (int v = threadIdx.x; v <= nk; v += blockDim.x) run[v] = 0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = chunk * kOrderChunk + threadIdx.x;
  const int bucket = row < rows ? nk - counts[row] : 0;
  for (int turn = 0; turn < kOrderChunk / 64; ++turn) {
    __syncthreads();
    if (w == turn) {
      bool todo = row < rows;
      while (true) {
        const uint64_t am = __ballot(todo);
        if (am == 0) break;
        const int leader = __ffsll((unsigned long long)am) - 1;
        const int b0 = __shfl(bucket, leader, kWave);
        const bool match = todo && bucket == b0;
        const uint64_t mm = __ballot(match);
        const int base = chunk_hist[(int64_t)b0 * nchunk + chunk] + run[b0];
        if (match) {
          const int rank = __popcll(mm & ((1ull << lane) - 1));
          order[base + rank] = row;
          todo = false;
        }
        __builtin_amdgcn_wave_barrier();
        if (lane == leader) run[b0] += __popcll(mm);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
}

__global__ __launch_bounds__(64) void retained_kernel(const Geom g, const float* __restrict__ M,
                                                      const int32_t* __restrict__ row_ptr,
                                                      const int32_t* __restrict__ col_idx,
                                                      float* __restrict__ kept) {
  const int row = blockIdx.x;
  const float* Mrow = M + (int64_t)row * g.nk;
  float k = 0.f, a = 0.f;
  for (int p = row_ptr[row] + threadIdx.x; p < row_ptr[row + 1]; p += 64) k += Mrow[col_idx[p]];
  for (int j = threadIdx.x; j < g.nk; j += 64) a += Mrow[j];
  k = wave_sum(k);
  a = wave_sum(a);
  if (threadIdx.x == 0) { kept[2 * row] = k; kept[2 * row + 1] = a; }
}

int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace

size_t select_ws_bytes(const Geom& g, SelectWs* layout, char* base) {
  const int rows = g.rows();
  const int nchunk = (rows + kOrderChunk - 1) / kOrderChunk;
  size_t off = 0;
  const size_t counts_off = off;
  off = align_up(off + (size_t)rows * sizeof(int32_t), 256);
  const size_t kappa_off = off;
  off = align_up(off + (size_t)rows * sizeof(uint64_t), 256);
  const size_t hist_off = off;
  off = align_up(off + (size_t)(g.nk + 1) * nchunk * sizeof(int32_t), 256);
  if (layout) {
    layout->counts = reinterpret_cast<int32_t*>(base + counts_off);
    layout->kappa = reinterpret_cast<uint64_t*>(base + kappa_off);
    layout->chunk_hist = reinterpret_cast<int32_t*>(base + hist_off);
    layout->nchunk = nchunk;
  }
  return off;
}

hipError_t launch_select(const Geom& g, const float* M, const PTable& pt, int32_t* row_ptr, int32_t* col_idx,
                         int32_t* order, const SelectWs& ws, hipStream_t st) {
  const int rows = g.rows();
  const int npad = next_pow2(g.nk < 2 ? 2 : g.nk);
  const int hist_len = (g.nk + 1) * ws.nchunk;
  int32_t* hist = order ? ws.chunk_hist : nullptr;
  if (hist) {
    const int blocks = (hist_len + 255) / 256 < 1024 ? (hist_len + 255) / 256 : 1024;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(blocks), dim3(256), 0, st, hist, (int64_t)hist_len, 0);
  }
  hipLaunchKernelGGL(cut_kernel, dim3(rows), dim3(kSelThreads), (size_t)npad * sizeof(uint64_t), st, g, M, pt,
                     npad, ws.counts, ws.kappa, hist, ws.nchunk);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, (const int32_t*)ws.counts, rows, row_ptr, hist,
                     hist_len);
  hipLaunchKernelGGL(compact_kernel, dim3(rows), dim3(kSelThreads), 0, st, g, M, (const uint64_t*)ws.kappa,
                     (const int32_t*)row_ptr, col_idx);
  if (order)
    hipLaunchKernelGGL(place_kernel, dim3(ws.nchunk), dim3(kOrderChunk), (size_t)(g.nk + 1) * sizeof(int), st,
                       (const int32_t*)ws.counts, rows, g.nk, (const int32_t*)hist, ws.nchunk, order);
  return hipGetLastError();
}

hipError_t launch_retained_mass(const Geom& g, const float* M, const int32_t* row_ptr, const int32_t* col_idx,
                                float* kept, hipStream_t st) {
  hipLaunchKernelGGL(retained_kernel, dim3(g.rows()), dim3(64), 0, st, g, M, row_ptr, col_idx, kept);
  return hipGetLastError();
}

}  // namespace losa
