// Retained-mass (top-p) key-block selection to CSR (LoSA page, Methodology
// Summary, one-time pattern construction: per head and query block, sort
// the key blocks by decreasing mass and keep the shortest prefix whose
// cumulative mass reaches p times the block's total).
//
// Kernels, in launch order:
//   cut         the cut in (mass desc, index asc) order over exact integer
//               units, without sorting -> the kept count s and the sort key
//               kappa of the last kept block, and the row's kept blocks
//               (sort key <= kappa) as bits: one wave per row (n_k <= 2048)
//               by a radix select over the range of the row's keys, or one
//               workgroup per row by radix select;
//   chunk       one workgroup per chunk of up to 256 rows of one head:
//               histogram of counts and kept total of the chunk (LDS, then
//               plain stores: no global atomics, nothing to clear
//               beforehand, so the sequence can sit inside a captured graph);
//   offsets     one thread per count: exclusive scan, head by head, over
//               the head's row chunks of that count's histogram column
//               (-> the head's rows of that count); the last workgroup to
//               finish scans the per-chunk kept totals (-> first CSR slot
//               per chunk, and row_ptr[rows]);
//   place       one workgroup per chunk: row_ptr of its rows (chunk base +
//               scan of counts), and each row's stable rank by count,
//               descending, inside its head (-> ranked rows, group keys);
//   group_order one workgroup: the work groups (32 ranks of one head) by
//               their first count, descending, stable -> each group's slot;
//   scatter     one thread per rank: the row into its group's slots -> order;
//   compact     one wave per row: from the kept bits, the kept indices
//               ascending at row_ptr[row] (the masses are read once, by the
//               cut).
//
// The same chunk / offsets / place kernels also serve two other list
// builders here: online block thresholding (threshold kernel: counts, then
// the kept indices) and the per-head merge of two list sets (pick_counts,
// then copy_lists).
//
// Work order: each (batch, head)'s n_q rows ranked by kept count,
// descending, ties by row index; the ranks cut into groups of 32 (what one
// XCD's CUs run side by side); groups longest first by their first row's
// count, ties by head and group; ranks in order inside a group.
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
#include "losa.h"
#include "losa_device.hpp"
#include "losa_internal.hpp"

#include <mutex>

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

// Orders this wave's LDS accesses across its lanes (the waves of a
// workgroup work on different rows and do not meet).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The active lanes of this wave whose key equals this lane's (0 <= key <
// 2^nbits): one ballot per key bit, so a wave of many distinct keys costs
// no more than a wave of one.
__device__ __forceinline__ uint64_t match_lanes(int key, bool active, int nbits) {
  uint64_t eq = __ballot(active);
  for (int i = 0; i < nbits; ++i) {
    const bool bit = (key >> i) & 1;
    const uint64_t bm = __ballot(bit);
    eq &= bit ? bm : ~bm;
  }
  return eq;
}

// Chunk c covers rows h * nq + k * kOrderChunk + [0, kOrderChunk) of head
// h = c / cph, k = c % cph (cph chunks per head), cut at the head's end.
struct ChunkRows {
  int row, valid, head;
  __device__ ChunkRows(int chunk, int nq, int cph) {
    head = chunk / cph;
    const int local = (chunk - head * cph) * kOrderChunk + (int)threadIdx.x;
    valid = local < nq;
    row = head * nq + local;
  }
};

// One workgroup per chunk: the chunk's histogram of nk - count (built in
// LDS, stored whole, zeros included) and its kept total.  Workgroup 0 also
// clears the offsets kernel's done counter.  Plain stores only, so nothing
// needs clearing beforehand.
__global__ __launch_bounds__(kOrderChunk) void chunk_kernel(const int32_t* __restrict__ counts, int nq, int cph,
                                                            int nk, int32_t* __restrict__ hist,
                                                            int32_t* __restrict__ chunk_sum, int32_t* done) {
  extern __shared__ int hl[];  // [nk + 1]
  __shared__ int wsum[kOrderChunk / 64];
  const int chunk = blockIdx.x;
  for (int x = threadIdx.x; x <= nk; x += blockDim.x) hl[x] = 0;
  __syncthreads();
  const ChunkRows cr(chunk, nq, cph);
  const int cnt = cr.valid ? counts[cr.row] : 0;
  if (cr.valid) atomicAdd(&hl[nk - cnt], 1);
  int v = cnt;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
  __syncthreads();
  int32_t* hrow = hist + (int64_t)chunk * (nk + 1);
  for (int x = threadIdx.x; x <= nk; x += blockDim.x) hrow[x] = hl[x];
  if (threadIdx.x == 0) {
    int t = 0;
#pragma unroll
    for (int ww = 0; ww < kOrderChunk / 64; ++ww) t += wsum[ww];
    chunk_sum[chunk] = t;
    if (chunk == 0) *done = 0;
  }
}

// Most key blocks one thread of the cut kernel owns.
constexpr int kMaxPer = LOSA_MAX_KEY_BLOCKS / kSelThreads;
static_assert(kMaxPer == 16, "the workgroup cut kernel serves rows of 2049 to 4096 blocks");

// ORs the run of bits (bit t for block j0 + t, at most 32 of them) into an
// LDS bit array of the row (bit j%32 of word j/32); the run may straddle two
// words.
__device__ __forceinline__ void or_bit_run(uint32_t* words, int j0, uint32_t bits) {
  if (bits == 0) return;
  const int w = j0 >> 5, sh = j0 & 31;
  atomicOr(&words[w], bits << sh);
  if (sh != 0 && (bits >> (32 - sh)) != 0) atomicOr(&words[w + 1], bits >> (32 - sh));
}

// One workgroup per row.  Finds the kept count s and the sort key kappa of
// the s-th block in (mass desc, index asc) order without sorting: a radix
// select, most significant digit first, over the inverted mass bits
// ku = 2^32-1-u (ascending ku = descending mass), four passes of 8 bits.
// Each pass sums the fixed-point units q of the remaining candidates per
// digit and keeps the first non-empty digit at which the running sum
// (everything before it included) reaches T; after the last pass the
// candidates share one mass, and the cut within them falls by index.
// Thread t owns the contiguous blocks [t*per, t*per + per), so thread order
// is index order; kPer >= per bounds the per-thread register arrays.  The
// row's kept count goes to counts, its kept blocks as bits to keep (the
// blocks whose sort key is at most kappa's, kappa being the s-th block's).
template <int kPer>
__global__ __launch_bounds__(kSelThreads) void cut_kernel(const Geom g, const float* __restrict__ M,
                                                          const PTable pt, int32_t* __restrict__ counts,
                                                          uint32_t* __restrict__ keep) {
  __shared__ uint64_t hsum[256];
  __shared__ uint32_t hnz[256];
  __shared__ uint64_t wsum64[kSelThreads / 64];
  __shared__ int wsum32[kSelThreads / 64];
  __shared__ uint32_t wred[kSelThreads / 64];
  __shared__ uint64_t s_below;
  __shared__ int s_jcut;
  __shared__ uint32_t s_keep[LOSA_MAX_KEY_BLOCKS / 32];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = (row / g.nq) % g.H;
  const uint64_t P = pt.P[pt.per_head ? h : 0];
  const int nk = g.nk;
  const float* Mrow = M + (int64_t)row * nk;
  const int per = (nk + kSelThreads - 1) / kSelThreads;
  const int j0 = tid * per;
  const int mine = max(0, min(per, nk - j0));  // valid blocks of this thread
  if (tid == 0) s_jcut = 0;

  uint32_t ku[kPer];
  uint32_t umax = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const uint32_t u = t < mine ? sanitized_bits(Mrow[j0 + t]) : 0u;
    ku[t] = 0xFFFFFFFFu - u;
    umax = umax > u ? umax : u;
  }
  umax = wave_max_u32(umax);
  if (lane == 0) wred[w] = umax;
  __syncthreads();
#pragma unroll
  for (int ww = 0; ww < kSelThreads / 64; ++ww) umax = umax > wred[ww] ? umax : wred[ww];
  __syncthreads();

  int s;
  uint64_t kap;
  if (P == (1ull << 32)) {  // keep everything
    s = nk;
    kap = ~0ull;
  } else {
    const int e = umax ? frexp_exp(umax) : 0;
    uint64_t q[kPer];
    uint64_t run = 0;
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      q[t] = t < mine ? fixed_units(0xFFFFFFFFu - ku[t], e) : 0;
      run += q[t];
    }
    uint64_t total;
    block_inclusive_scan_u64(run, wsum64, &total);
    const uint64_t T = threshold(P, total);

    uint32_t prefix = 0;  // digits fixed so far
    uint64_t below = 0;   // units of all blocks ordered before the candidates
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hsum[tid] = 0;
      hnz[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int t = 0; t < kPer; ++t) {
        if (t < mine && ((uint64_t)ku[t] >> (shift + 8)) == prefix) {
          const int d = (ku[t] >> shift) & 255;
          atomicAdd(reinterpret_cast<unsigned long long*>(&hsum[d]), (unsigned long long)q[t]);
          hnz[d] = 1;
        }
      }
      __syncthreads();
      const uint64_t hs = hsum[tid];
      uint64_t all;
      const uint64_t cum = block_inclusive_scan_u64(hs, wsum64, &all);  // bins in ascending digit order
      const bool hit = hnz[tid] != 0 && below + cum >= T;
      const uint64_t bal = __ballot(hit);
      if (lane == 0) wred[w] = bal ? (uint32_t)(w * 64 + __builtin_ctzll(bal)) : 0xFFFFFFFFu;
      __syncthreads();
      uint32_t bin = wred[0];
#pragma unroll
      for (int ww = 1; ww < kSelThreads / 64; ++ww) bin = bin < wred[ww] ? bin : wred[ww];
      bin = bin < 255u ? bin : 255u;  // a hit always exists: the candidates' units reach T
      if ((uint32_t)tid == bin) s_below = below + cum - hs;
      __syncthreads();
      below = s_below;
      prefix = (prefix << 8) | bin;
    }
    // The cut lies among the blocks whose inverted bits equal prefix (all
    // with units qu): the need-th of them in index order.
    const uint64_t qu = fixed_units(0xFFFFFFFFu - prefix, e);
    uint64_t need = 1;
    if (below < T && qu > 0) need = (T - below + qu - 1) / qu;
    int nbelow = 0, nties = 0;
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      if (t < mine) {
        nbelow += ku[t] < prefix ? 1 : 0;
        nties += ku[t] == prefix ? 1 : 0;
      }
    }
    nbelow = block_sum_i32(nbelow, wsum32);
    uint64_t tie_all;
    const uint64_t tie_incl = block_inclusive_scan_u64((uint64_t)nties, wsum64, &tie_all);
    uint64_t rank = tie_incl - (uint64_t)nties;  // ties owned by earlier threads
    if (need > rank && need <= tie_incl) {
#pragma unroll
      for (int t = 0; t < kPer; ++t) {
        if (t < mine && ku[t] == prefix) {
          ++rank;
          if (rank == need) s_jcut = j0 + t;
        }
      }
    }
    __syncthreads();
    s = nbelow + (int)need;
    kap = sort_key(0xFFFFFFFFu - prefix, s_jcut);
  }
  const int nw = (nk + 31) / 32;
  if (tid < nw) s_keep[tid] = 0;
  __syncthreads();
  uint32_t bits = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t)
    if (t < mine && sort_key(0xFFFFFFFFu - ku[t], j0 + t) <= kap) bits |= 1u << t;
  or_bit_run(s_keep, j0, bits);
  __syncthreads();
  for (int x = tid; x < nw; x += kSelThreads) keep[(int64_t)row * nw + x] = s_keep[x];
  if (tid == 0) counts[row] = s;
}

// Wave reductions with a wave-uniform result: DPP within each 16-lane row
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror 4, row_ror 8 leave
// every lane with its row's total), then the four row totals read from
// lanes 0, 16, 32, 48.  All 64 lanes must be active.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;

__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)v, l); }

template <int kCtrl>
__device__ __forceinline__ uint64_t add_dpp_u64(uint64_t x) {
  return x + (((uint64_t)dpp_u32<kCtrl>((uint32_t)(x >> 32)) << 32) | dpp_u32<kCtrl>((uint32_t)x));
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  v = add_dpp_u64<kDppXor1>(v);
  v = add_dpp_u64<kDppXor2>(v);
  v = add_dpp_u64<kDppRor4>(v);
  v = add_dpp_u64<kDppRor8>(v);
  uint64_t t = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) t += ((uint64_t)lane_u32((uint32_t)(v >> 32), 16 * r) << 32) | lane_u32((uint32_t)v, 16 * r);
  return t;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  v += (int)dpp_u32<kDppXor1>((uint32_t)v);
  v += (int)dpp_u32<kDppXor2>((uint32_t)v);
  v += (int)dpp_u32<kDppRor4>((uint32_t)v);
  v += (int)dpp_u32<kDppRor8>((uint32_t)v);
  return (int)(lane_u32(v, 0) + lane_u32(v, 16) + lane_u32(v, 32) + lane_u32(v, 48));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u32<kDppXor1>(v));
  v = min(v, dpp_u32<kDppXor2>(v));
  v = min(v, dpp_u32<kDppRor4>(v));
  v = min(v, dpp_u32<kDppRor8>(v));
  return min(min(lane_u32(v, 0), lane_u32(v, 16)), min(lane_u32(v, 32), lane_u32(v, 48)));
}

__device__ __forceinline__ uint32_t wave_max_u32_uniform(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppRor4>(v));
  v = max(v, dpp_u32<kDppRor8>(v));
  return max(max(lane_u32(v, 0), lane_u32(v, 16)), max(lane_u32(v, 32), lane_u32(v, 48)));
}

// One wave per row (four rows per workgroup), no workgroup barriers.  The
// cut is the least inverted-bits value v with F(v) = sum of the units q of
// the blocks with ku <= v reaching T, found over the range of the blocks'
// ku (F only steps at those values, so v is one of them, and F(v - 1) < T)
// by a radix select.  Among the blocks with ku = v (equal masses, equal units)
// the cut falls on the need-th in index order.  Lane l owns the contiguous
// blocks [l*per, l*per + per), per <= kPer, so lane order is index order.
// The row's kept count goes to counts, its kept blocks as bits to keep.
template <int kPer>
__global__ __launch_bounds__(256) void cut_wave_kernel(const Geom g, const float* __restrict__ M, const PTable pt,
                                                       int32_t* __restrict__ counts,
                                                       uint32_t* __restrict__ keep) {
  __shared__ uint64_t cut_hist[4][256];  // per wave: units per digit of the radix select, then the kept bits
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= g.rows()) return;  // whole waves only
  const int h = (row / g.nq) % g.H;
  const uint64_t P = pt.P[pt.per_head ? h : 0];
  const int nk = g.nk;
  const float* Mrow = M + (int64_t)row * nk;
  const int per = (nk + kWave - 1) / kWave;
  const int j0 = lane * per;
  const int mine = max(0, min(per, nk - j0));

  uint32_t ku[kPer];
  uint32_t umax = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const uint32_t u = t < mine ? sanitized_bits(Mrow[j0 + t]) : 0u;
    ku[t] = 0xFFFFFFFFu - u;
    umax = umax > u ? umax : u;
  }
  umax = wave_max_u32_uniform(umax);

  int s;
  uint64_t kap;
  if (P == (1ull << 32)) {  // keep everything
    s = nk;
    kap = ~0ull;
  } else {
    const int e = umax ? frexp_exp(umax) : 0;
    uint64_t q[kPer];
    uint64_t run = 0;
    uint32_t lo = 0xFFFFFFFFu, hi = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      q[t] = t < mine ? fixed_units(0xFFFFFFFFu - ku[t], e) : 0;
      run += q[t];
      if (t < mine) kmin = kmin < ku[t] ? kmin : ku[t];
      if (q[t] > 0) {
        lo = lo < ku[t] ? lo : ku[t];
        hi = hi > ku[t] ? hi : ku[t];
      }
    }
    const uint64_t T = threshold(P, wave_sum_u64(run));
    uint32_t v;
    if (T == 0) {
      v = wave_min_u32(kmin);  // the first block in sorted order
    } else {  // T > 0: some block has units, and F(max ku of those) = total >= T
      // F steps only at keys of blocks with units, all in [lo, hi]: a radix
      // select over rel = ku - lo, most significant 8-bit digit of the
      // range first.  Each pass sums the units of the blocks still in the
      // prefix's range per digit (this wave's histogram in LDS, exact u64
      // sums) and keeps the least digit at which acc + the running sum
      // reaches T.  At most four passes, against up to 32 bisection steps
      // that each re-sum the whole row.
      lo = wave_min_u32(lo);
      hi = wave_max_u32_uniform(hi);
      const uint32_t width = hi - lo;
      uint64_t* hist = cut_hist[threadIdx.x >> 6];
      uint32_t rel[kPer];
#pragma unroll
      for (int t = 0; t < kPer; ++t) rel[t] = ku[t] - lo;
      uint32_t pre = 0;  // digits found so far
      uint64_t acc = 0;  // units of the blocks below the prefix's range
      for (int top = width ? 32 - __builtin_clz(width) : 0; top > 0;) {
        const int shift = top > 8 ? top - 8 : 0;
        const uint32_t dmask = (1u << (top - shift)) - 1u;
        const uint32_t above = top >= 32 ? 0u : (0xFFFFFFFFu << top);
        hist[4 * lane] = 0;
        hist[4 * lane + 1] = 0;
        hist[4 * lane + 2] = 0;
        hist[4 * lane + 3] = 0;
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < kPer; ++t)
          if (q[t] > 0 && ((rel[t] ^ pre) & above) == 0)
            atomicAdd(reinterpret_cast<unsigned long long*>(hist + ((rel[t] >> shift) & dmask)),
                      (unsigned long long)q[t]);
        wave_lds_sync();
        uint64_t c[4];  // inclusive sums of this lane's digits 4 lane .. 4 lane + 3
        c[0] = hist[4 * lane];
#pragma unroll
        for (int k = 1; k < 4; ++k) c[k] = c[k - 1] + hist[4 * lane + k];
        uint64_t inc = c[3];  // inclusive scan over lanes
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const uint32_t xl = __shfl_up((uint32_t)inc, o, kWave), xh = __shfl_up((uint32_t)(inc >> 32), o, kWave);
          if (lane >= o) inc += ((uint64_t)xh << 32) | xl;
        }
        const uint64_t base = acc + (inc - c[3]);
        // this lane's least digit reaching T (4: none), and the units below it
        int k = 4;
        uint64_t bel = 0;
#pragma unroll
        for (int kk = 3; kk >= 0; --kk)
          if (base + c[kk] >= T) {
            k = kk;
            bel = kk ? c[kk - 1] : 0;
          }
        // some lane hits: acc plus all units in the prefix's range is F(end of the range) >= T
        const uint64_t hit = __ballot(k < 4);
        const int lf = __builtin_ctzll(hit);
        const uint32_t digit = 4u * lf + (uint32_t)__builtin_amdgcn_readlane(k, lf);
        const uint64_t add = (inc - c[3]) + bel;
        acc += ((uint64_t)lane_u32((uint32_t)(add >> 32), lf) << 32) | lane_u32((uint32_t)add, lf);
        pre |= digit << shift;
        top = shift;
        wave_lds_sync();  // every lane has read the histogram before the next pass clears it
      }
      v = lo + pre;
    }
    uint64_t below = 0;
    int nbelow = 0, nties = 0;
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      if (t < mine) {
        below += ku[t] < v ? q[t] : 0;
        nbelow += ku[t] < v ? 1 : 0;
        nties += ku[t] == v ? 1 : 0;
      }
    }
    below = wave_sum_u64(below);
    const uint64_t qu = fixed_units(0xFFFFFFFFu - v, e);
    uint64_t need = 1;
    if (below < T && qu > 0) need = (T - below + qu - 1) / qu;
    int incl = nties;  // ties owned by lanes <= this one
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int x = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += x;
    }
    int jcut = -1;
    int rank = incl - nties;
    if ((int64_t)need > rank && (int64_t)need <= incl) {
#pragma unroll
      for (int t = 0; t < kPer; ++t) {
        if (t < mine && ku[t] == v) {
          ++rank;
          if (rank == (int)need) jcut = j0 + t;
        }
      }
    }
    const uint64_t owner = __ballot(jcut >= 0);
    jcut = __builtin_amdgcn_readlane(jcut, owner ? __builtin_ctzll(owner) : 0);
    s = wave_sum_i32(nbelow) + (int)need;
    kap = sort_key(0xFFFFFFFFu - v, jcut < 0 ? 0 : jcut);
  }
  // The kept blocks (sort key <= kappa) as bits, assembled in this wave's LDS
  // (at most 64 words: n_k <= 2048 here), then stored coalesced.
  uint32_t* words = reinterpret_cast<uint32_t*>(cut_hist[threadIdx.x >> 6]);
  const int nw = (nk + 31) / 32;
  wave_lds_sync();  // the histogram's last reads are done
  words[lane] = 0;
  wave_lds_sync();
  uint32_t bits = 0;
#pragma unroll
  for (int t = 0; t < kPer; ++t)
    if (t < mine && sort_key(0xFFFFFFFFu - ku[t], j0 + t) <= kap) bits |= 1u << t;
  or_bit_run(words, j0, bits);
  wave_lds_sync();
  if (lane < nw) keep[(int64_t)row * nw + lane] = words[lane];
  if (lane == 0) counts[row] = s;
}

// Exclusive scan of data[0, n) into out by one workgroup (a multiple of 64
// threads, wsum holding one int per wave); in place is allowed.
__device__ void block_exclusive_scan_i32(const int32_t* data, int n, int32_t* out, int32_t* out_total,
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

// One thread per count bucket b = nk - count: within each head, the column
// hist[.][b] over the head's cph chunks becomes its exclusive scan, and
// bucket[head][b] the head's total.  The last workgroup to finish (counted
// in *done) turns chunk_sum into the first CSR slot of each chunk and writes
// row_ptr[rows].
__global__ __launch_bounds__(256) void offsets_kernel(int nk, int nchunk, int cph, int rows,
                                                      int32_t* __restrict__ hist, int32_t* chunk_sum,
                                                      int32_t* __restrict__ bucket, int32_t* done,
                                                      int32_t* __restrict__ row_ptr) {
  __shared__ int wsum[256 / 64];
  __shared__ int last;
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b <= nk) {
    int run = 0, k = 0, h = 0;  // running total, chunk within the head, head
    auto step = [&](int c, int v) {
      if (k == 0) run = 0;
      hist[(int64_t)c * (nk + 1) + b] = run;
      run += v;
      if (++k == cph) {
        bucket[(int64_t)h * (nk + 1) + b] = run;
        k = 0;
        ++h;
      }
    };
    int c = 0;
    for (; c + 8 <= nchunk; c += 8) {  // eight loads in flight per thread
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hist[(int64_t)(c + u) * (nk + 1) + b];
#pragma unroll
      for (int u = 0; u < 8; ++u) step(c + u, v[u]);
    }
    for (; c < nchunk; ++c) step(c, hist[(int64_t)c * (nk + 1) + b]);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(done, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();
  block_exclusive_scan_i32(chunk_sum, nchunk, chunk_sum, row_ptr + rows, wsum);
}

// One wave per row (four rows per workgroup): the row's kept bits (from the
// cut, 4 bytes per 32 blocks instead of the masses again) are loaded once,
// one word per lane; for each 64 blocks lane l writes block 64 s + l, if
// kept, at row_ptr[row] plus the number kept before it.
__global__ __launch_bounds__(256) void compact_kernel(const Geom g, const uint32_t* __restrict__ keep,
                                                      const int32_t* __restrict__ row_ptr,
                                                      int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= g.rows()) return;  // whole waves only
  const int nk = g.nk, nw = (nk + 31) / 32;  // nw <= 128
  const uint32_t* kr = keep + (int64_t)row * nw;
  const uint32_t w0 = lane < nw ? kr[lane] : 0u, w1 = 64 + lane < nw ? kr[64 + lane] : 0u;
  const uint64_t lt = (1ull << lane) - 1ull;
  int pos = row_ptr[row];
  for (int s = 0; 64 * s < nk; ++s) {  // blocks [64 s, 64 s + 64): words 2s, 2s + 1
    const int a = 2 * s, b = 2 * s + 1;
    const uint32_t lo = __builtin_amdgcn_readlane(a < 64 ? w0 : w1, a & 63);
    const uint32_t hi = __builtin_amdgcn_readlane(b < 64 ? w0 : w1, b & 63);
    const uint64_t m = ((uint64_t)hi << 32) | lo;
    if ((m >> lane) & 1ull) col_idx[pos + __popcll(m & lt)] = 64 * s + lane;
    pos += __popcll(m);
  }
}

// One workgroup (kOrderChunk threads) per chunk of rows.  row_ptr of the
// chunk's rows: the chunk's first CSR slot plus the scan of their counts.
// Then (if the work order is wanted) each row's rank r in its head by count
// descending, stable: h * nq + r is h * nq + (rows of the head with a larger
// count: the exclusive scan of bucket[h]) + hist[chunk][nk - c] (rows of
// count c in earlier chunks of the head) plus the rows of that count already
// placed by earlier waves of this chunk; waves take turns so that rows keep
// their index order within a count.  ranked[h * nq + r] = row, and the rows
// of rank r = 0 mod kGroupRows record their count as their group's key.
__global__ __launch_bounds__(kOrderChunk) void place_kernel(const int32_t* __restrict__ counts, int nq, int cph,
                                                            int nk, const int32_t* __restrict__ hist,
                                                            const int32_t* __restrict__ bucket,
                                                            const int32_t* __restrict__ chunk_base,
                                                            int32_t* __restrict__ row_ptr,
                                                            int32_t* __restrict__ ranked, int ngh,
                                                            int32_t* __restrict__ gkey) {
  extern __shared__ int run[];  // [nk + 1] next free slot of each count, relative to the head's first
  __shared__ int wsum[kOrderChunk / 64];
  __shared__ int wscan[kOrderChunk / 64];
  const int chunk = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const ChunkRows cr(chunk, nq, cph);
  const int row = cr.row;
  const int cnt = cr.valid ? counts[row] : 0;
  int v = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int before = chunk_base[chunk];
#pragma unroll
  for (int ww = 0; ww < kOrderChunk / 64; ++ww)
    if (ww < w) before += wsum[ww];
  if (cr.valid) row_ptr[row] = before + v - cnt;
  if (!ranked) return;
  block_exclusive_scan_i32(bucket + (int64_t)cr.head * (nk + 1), nk + 1, run, nullptr, wscan);
  const int32_t* hrow = hist + (int64_t)chunk * (nk + 1);
  const int head0 = cr.head * nq;
  const int bkt = nk - cnt;
  const int nbits = 32 - __builtin_clz(nk);  // bkt <= nk
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int turn = 0; turn < kOrderChunk / 64; ++turn) {  // waves in row order: the ranks are stable
    __syncthreads();
    if (w == turn) {
      const uint64_t eq = match_lanes(bkt, cr.valid, nbits);
      if (cr.valid) {
        const int r = hrow[bkt] + run[bkt] + __popcll(eq & lt);  // rank within the head
        ranked[head0 + r] = row;
        if (r % kGroupRows == 0) gkey[cr.head * ngh + r / kGroupRows] = cnt;  // the group's first count
      }
      wave_lds_sync();  // every lane has read run[] before the first lane of each key moves it on
      if (cr.valid && (eq & lt) == 0) run[bkt] += __popcll(eq);
    }
  }
}

// The work order's groups: group (h, k) holds ranks [k * kGroupRows,
// (k + 1) * kGroupRows) of head h (the last group of a head holds
// nq - (ngh - 1) * kGroupRows rows when nq is not a multiple of kGroupRows);
// groups run by key descending, ties by group index (head, then k).  One
// workgroup: a counting sort over the keys in LDS (all groups, and the short
// head-last groups) and a stable placement in group-index order.  A group's
// first slot is kGroupRows * R - (kGroupRows - last) * S, with R the groups
// and S the short groups placed before it.
__global__ __launch_bounds__(256) void group_order_kernel(int ngroups, int ngh, int last, int nk,
                                                          const int32_t* __restrict__ gkey,
                                                          int32_t* __restrict__ gstart) {
  extern __shared__ int gl[];  // [2][nk + 1]: groups, then short groups, per key bucket nk - key
  __shared__ int wsum[256 / 64];
  int* all = gl;
  int* shrt = gl + nk + 1;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int x = threadIdx.x; x < 2 * (nk + 1); x += 256) gl[x] = 0;
  __syncthreads();
  const bool has_short = last < kGroupRows;
  const int nbits = 32 - __builtin_clz(nk);  // nk - key <= nk
  for (int gi = threadIdx.x; gi < ngroups; gi += 256) {
    const int b = nk - gkey[gi];
    atomicAdd(&all[b], 1);
    if (has_short && gi % ngh == ngh - 1) atomicAdd(&shrt[b], 1);
  }
  __syncthreads();
  block_exclusive_scan_i32(all, nk + 1, all, nullptr, wsum);  // now the next slot per bucket
  block_exclusive_scan_i32(shrt, nk + 1, shrt, nullptr, wsum);
  for (int t0 = 0; t0 < ngroups; t0 += 256) {
    const int gi = t0 + (int)threadIdx.x;
    const bool valid = gi < ngroups;
    const int b = valid ? nk - gkey[gi] : 0;
    const bool is_short = valid && has_short && gi % ngh == ngh - 1;
    for (int turn = 0; turn < 4; ++turn) {  // waves in group order: the slots are stable
      __syncthreads();
      if (w == turn) {
        const uint64_t eq = match_lanes(b, valid, nbits);
        const uint64_t es = eq & __ballot(is_short);
        const uint64_t lt = (1ull << lane) - 1ull;
        if (valid) {
          const int R = all[b] + __popcll(eq & lt), S = shrt[b] + __popcll(es & lt);
          gstart[gi] = kGroupRows * R - (kGroupRows - last) * S;
        }
        wave_lds_sync();  // every lane has read the slots before the first lane of each key moves them on
        if (valid && (eq & lt) == 0) {
          all[b] += __popcll(eq);
          shrt[b] += __popcll(es);
        }
      }
    }
  }
}

// order[first slot of the row's group + rank within the group] = row.
__global__ __launch_bounds__(256) void scatter_order_kernel(int rows, int nq, int ngh,
                                                            const int32_t* __restrict__ ranked,
                                                            const int32_t* __restrict__ gstart,
                                                            int32_t* __restrict__ order) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= rows) return;
  const int h = p / nq, r = p - h * nq;
  order[gstart[h * ngh + r / kGroupRows] + r % kGroupRows] = ranked[p];
}

// Online block thresholding (the Sol-Attn page's block thresholding during
// the online-softmax pass): visiting the row's key blocks in index order,
// block j is kept when m_j >= theta * max(m_0 .. m_j), on the sanitised fp32
// masses, compared in fp64.  One wave per row, 64 blocks per step: coalesced
// loads, an inclusive max scan across the wave, and the running maximum
// carried from the previous step.  kWrite = false: the kept count into
// counts[row]; true: the kept indices, ascending, from row_ptr[row].
template <bool kWrite>
__global__ __launch_bounds__(256) void threshold_kernel(const Geom g, const float* __restrict__ M, const ThetaTable tt,
                                                        int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= g.rows()) return;  // the whole wave
  const int nk = g.nk;
  const double theta = tt.t[tt.per_head ? (row / g.nq) % g.H : 0];
  const float* Mrow = M + (int64_t)row * nk;
  int32_t* dst = kWrite ? col_idx + row_ptr[row] : nullptr;
  float carry = 0.f;  // largest mass before this step's blocks
  int kept = 0;
  for (int j0 = 0; j0 < nk; j0 += kWave) {
    const int j = j0 + lane;
    const float x = j < nk ? __uint_as_float(sanitized_bits(Mrow[j])) : 0.f;
    float run = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const float y = __shfl_up(run, o, kWave);
      if (lane >= o) run = fmaxf(run, y);
    }
    run = fmaxf(run, carry);
    const bool keep = j < nk && (double)x >= theta * (double)run;
    const uint64_t bal = __ballot(keep);
    if (kWrite && keep) dst[kept + __popcll(bal & ((1ull << lane) - 1))] = j;
    kept += __popcll(bal);
    carry = __shfl(run, kWave - 1, kWave);
  }
  if (!kWrite && lane == 0) counts[row] = kept;
}

// List merge: row r takes its count from set b when its head is flagged,
// from set a otherwise (clamped to [0, nk], so a malformed count cannot
// place a row outside the output).
__global__ __launch_bounds__(256) void pick_counts_kernel(int rows, int nq, int nk, const int32_t* __restrict__ take_b,
                                                          const int32_t* __restrict__ rpa,
                                                          const int32_t* __restrict__ rpb,
                                                          int32_t* __restrict__ counts) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int32_t* rp = take_b[r / nq] ? rpb : rpa;
  counts[r] = min(max(rp[r + 1] - rp[r], 0), nk);
}

// One wave per row: copy the chosen set's indices to row_ptr[r].
__global__ __launch_bounds__(256) void copy_lists_kernel(int rows, int nq, const int32_t* __restrict__ take_b,
                                                         const int32_t* __restrict__ rpa,
                                                         const int32_t* __restrict__ cia,
                                                         const int32_t* __restrict__ rpb,
                                                         const int32_t* __restrict__ cib,
                                                         const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ row_ptr,
                                                         int32_t* __restrict__ col_idx) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const bool b = take_b[r / nq] != 0;
  const int32_t* src = (b ? cib : cia) + (b ? rpb : rpa)[r];
  int32_t* dst = col_idx + row_ptr[r];
  const int n = counts[r];
  for (int t = threadIdx.x & 63; t < n; t += 64) dst[t] = src[t];
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

}  // namespace

size_t select_ws_bytes(const Geom& g, SelectWs* layout, char* base) {
  const int rows = g.rows();
  const int heads = g.B * g.H;
  const int cph = (g.nq + kOrderChunk - 1) / kOrderChunk;
  const int nchunk = heads * cph;
  size_t off = 0;
  const size_t counts_off = off;
  off = align_up(off + (size_t)rows * sizeof(int32_t), 256);
  const int keep_words = (g.nk + 31) / 32;
  const size_t keep_off = off;
  off = align_up(off + (size_t)rows * keep_words * sizeof(uint32_t), 256);
  const size_t hist_off = off;  // then chunk_sum and done
  off = align_up(off + ((size_t)(g.nk + 1) * nchunk + nchunk + 1) * sizeof(int32_t), 256);
  const size_t bucket_off = off;
  off = align_up(off + (size_t)heads * (g.nk + 1) * sizeof(int32_t), 256);
  const int ngh = (g.nq + kGroupRows - 1) / kGroupRows;
  const size_t ranked_off = off;
  off = align_up(off + (size_t)rows * sizeof(int32_t), 256);
  const size_t gkey_off = off;  // then gstart
  off = align_up(off + (size_t)2 * heads * ngh * sizeof(int32_t), 256);
  if (layout) {
    layout->counts = reinterpret_cast<int32_t*>(base + counts_off);
    layout->keep = reinterpret_cast<uint32_t*>(base + keep_off);
    layout->keep_words = keep_words;
    layout->chunk_hist = reinterpret_cast<int32_t*>(base + hist_off);
    layout->chunk_sum = layout->chunk_hist + (size_t)(g.nk + 1) * nchunk;
    layout->done = layout->chunk_sum + nchunk;
    layout->bucket = reinterpret_cast<int32_t*>(base + bucket_off);
    layout->nchunk = nchunk;
    layout->cph = cph;
    layout->ranked = reinterpret_cast<int32_t*>(base + ranked_off);
    layout->gkey = reinterpret_cast<int32_t*>(base + gkey_off);
    layout->gstart = layout->gkey + (size_t)heads * ngh;
    layout->ngh = ngh;
  }
  return off;
}

hipError_t launch_select(const Geom& g, const float* M, const PTable& pt, int32_t* row_ptr, int32_t* col_idx,
                         int32_t* order, const SelectWs& ws, hipStream_t st) {
  const int rows = g.rows();
  // Up to 2048 key blocks a wave per row; beyond, a workgroup
  // per row (radix select), which spreads a long row over 256 threads.  The
  // per-thread arrays are unrolled, so the instance fits the row closely.
  const int per = (g.nk + kWave - 1) / kWave;
  if (per <= 32) {
    auto cut = per <= 2 ? cut_wave_kernel<2> : per <= 4 ? cut_wave_kernel<4> : per <= 8 ? cut_wave_kernel<8>
             : per <= 12 ? cut_wave_kernel<12> : per <= 16 ? cut_wave_kernel<16> : per <= 20 ? cut_wave_kernel<20>
             : per <= 24 ? cut_wave_kernel<24> : cut_wave_kernel<32>;
    hipLaunchKernelGGL(cut, dim3((rows + 3) / 4), dim3(256), 0, st, g, M, pt, ws.counts, ws.keep);
  } else {
    const int per_t = (g.nk + kSelThreads - 1) / kSelThreads;
    auto cut = per_t <= 12 ? cut_kernel<12> : cut_kernel<kMaxPer>;
    hipLaunchKernelGGL(cut, dim3(rows), dim3(kSelThreads), 0, st, g, M, pt, ws.counts, ws.keep);
  }
  launch_offsets_and_order(g, ws, row_ptr, order, st);
  hipLaunchKernelGGL(compact_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, g, (const uint32_t*)ws.keep,
                     (const int32_t*)row_ptr, col_idx);
  return hipGetLastError();
}

hipError_t launch_select_threshold(const Geom& g, const float* M, const ThetaTable& tt, int32_t* row_ptr,
                                   int32_t* col_idx, int32_t* order, const SelectWs& ws, hipStream_t st) {
  const int rows = g.rows();
  const dim3 grid((rows + 3) / 4);
  hipLaunchKernelGGL(threshold_kernel<false>, grid, dim3(256), 0, st, g, M, tt, ws.counts, (const int32_t*)nullptr,
                     (int32_t*)nullptr);
  launch_offsets_and_order(g, ws, row_ptr, order, st);
  hipLaunchKernelGGL(threshold_kernel<true>, grid, dim3(256), 0, st, g, M, tt, (int32_t*)nullptr,
                     (const int32_t*)row_ptr, col_idx);
  return hipGetLastError();
}

hipError_t launch_merge_lists(const Geom& g, const int32_t* take_b, const int32_t* rpa, const int32_t* cia,
                              const int32_t* rpb, const int32_t* cib, int32_t* row_ptr, int32_t* col_idx,
                              int32_t* order, const SelectWs& ws, hipStream_t st) {
  const int rows = g.rows();
  hipLaunchKernelGGL(pick_counts_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, rows, g.nq, g.nk, take_b, rpa,
                     rpb, ws.counts);
  launch_offsets_and_order(g, ws, row_ptr, order, st);
  hipLaunchKernelGGL(copy_lists_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, rows, g.nq, take_b, rpa, cia, rpb,
                     cib, (const int32_t*)ws.counts, (const int32_t*)row_ptr, col_idx);
  return hipGetLastError();
}

// From the kept counts in ws.counts: row_ptr, and (order != NULL) the work order.
void launch_offsets_and_order(const Geom& g, const SelectWs& ws, int32_t* row_ptr, int32_t* order, hipStream_t st) {
  const int rows = g.rows();
  const size_t hist_lds = (size_t)(g.nk + 1) * sizeof(int);
  hipLaunchKernelGGL(chunk_kernel, dim3(ws.nchunk), dim3(kOrderChunk), hist_lds, st, (const int32_t*)ws.counts,
                     g.nq, ws.cph, g.nk, ws.chunk_hist, ws.chunk_sum, ws.done);
  hipLaunchKernelGGL(offsets_kernel, dim3((g.nk + 1 + 255) / 256), dim3(256), 0, st, g.nk, ws.nchunk, ws.cph,
                     rows, ws.chunk_hist, ws.chunk_sum, ws.bucket, ws.done, row_ptr);
  hipLaunchKernelGGL(place_kernel, dim3(ws.nchunk), dim3(kOrderChunk), hist_lds, st, (const int32_t*)ws.counts,
                     g.nq, ws.cph, g.nk, (const int32_t*)ws.chunk_hist, (const int32_t*)ws.bucket,
                     (const int32_t*)ws.chunk_sum, row_ptr, order ? ws.ranked : nullptr, ws.ngh, ws.gkey);
  if (!order) return;
  const int ngroups = g.B * g.H * ws.ngh;
  const int last = g.nq - (ws.ngh - 1) * kGroupRows;
  hipLaunchKernelGGL(group_order_kernel, dim3(1), dim3(256), 2 * hist_lds, st, ngroups, ws.ngh, last, g.nk,
                     (const int32_t*)ws.gkey, ws.gstart);
  hipLaunchKernelGGL(scatter_order_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, rows, g.nq, ws.ngh,
                     (const int32_t*)ws.ranked, (const int32_t*)ws.gstart, order);
}

// Scratch of the allocation-free selector: one array per device, placed by
// the code object loader.  In host code `scratch` names a host-side stand-in,
// not device memory; the device address comes from hipGetSymbolAddress and is
// what the kernels are given.
static __device__ __align__(256) unsigned char scratch[LOSA_SELECT_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t select_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_retained_mass(const Geom& g, const float* M, const int32_t* row_ptr, const int32_t* col_idx,
                                float* kept, hipStream_t st) {
  hipLaunchKernelGGL(retained_kernel, dim3(g.rows()), dim3(64), 0, st, g, M, row_ptr, col_idx, kept);
  return hipGetLastError();
}

}  // namespace losa
