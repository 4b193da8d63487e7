// Retained-mass (top-p) key-block selection to CSR (LoSA page, Methodology
// Summary, one-time pattern construction: per head and query block, sort
// the key blocks by decreasing mass and keep the shortest prefix whose
// cumulative mass reaches p times the block's total).
//
// Kernels, in launch order:
//   cut         the cut in (mass desc, index asc) order over exact integer
//               units, without sorting -> the kept count s and the row's
//               kept blocks as bits: one wave per row (n_k <= 64 * 31) or
//               one workgroup per row (up to 4096); the row arrives through
//               LDS from coalesced buffer loads, one radix pass over the
//               range of its masses finds the band of masses that holds the
//               cut, and the cut is taken among the (usually few) blocks of
//               that band, with further radix passes when the band is wide;
//   order       one workgroup per (batch, head): the exclusive scan of the
//               head's counts (its rows' offsets inside the head) and, when
//               the work order is wanted, the head's rows ranked by count (a
//               bitonic sort of unique keys in LDS) with, for every count,
//               the first rank in the head that holds it (binary searches
//               over the sorted keys); the last workgroup to finish scans
//               the heads' totals (-> each head's first CSR slot,
//               row_ptr[rows]);
//   compact     one wave per row: row_ptr[row]; the first order slot of the
//               row's work group, counted from every head's count bucket
//               starts (the groups that come before it in the order); and
//               from the kept bits the kept indices ascending from
//               row_ptr[row] (the masses are read once, by the cut).
//
// The same order kernel also serves two other list builders here: online
// block thresholding (threshold kernel: counts, then the kept indices) and
// the per-head merge of two list sets (pick_counts, then copy_lists).
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

// Orders this wave's LDS accesses across its lanes (the waves of a
// workgroup work on different rows and do not meet).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ORs the run of bits (bit t for block j0 + t, at most 32 of them) into an
// LDS bit array of the row (bit j%32 of word j/32); the run may straddle two
// words.
__device__ __forceinline__ void or_bit_run(uint32_t* words, int j0, uint32_t bits) {
  if (bits == 0) return;
  const int w = j0 >> 5, sh = j0 & 31;
  atomicOr(&words[w], bits << sh);
  if (sh != 0 && (bits >> (32 - sh)) != 0) atomicOr(&words[w + 1], bits >> (32 - sh));
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

// Inclusive scans over the wave by DPP moves (no LDS): within each 16-lane
// row by shifts of 1, 2, 4 and 8 (lanes shifted in from outside the row add
// 0), then lane 15 of rows 0 and 2 into rows 1 and 3, and lane 31 into rows
// 2 and 3.  All 64 lanes must be active.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp0_u32(uint32_t v) {  // lanes without a source get 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp0_u32<0x111>(v);
  v += dpp0_u32<0x112>(v);
  v += dpp0_u32<0x114>(v);
  v += dpp0_u32<0x118>(v);
  v += dpp0_u32<0x142, 0xA>(v);
  v += dpp0_u32<0x143, 0xC>(v);
  return v;
}
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint64_t dpp0_add_u64(uint64_t v) {
  return v + (((uint64_t)dpp0_u32<kCtrl, kRowMask>((uint32_t)(v >> 32)) << 32) |
              dpp0_u32<kCtrl, kRowMask>((uint32_t)v));
}
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  v = dpp0_add_u64<0x111>(v);
  v = dpp0_add_u64<0x112>(v);
  v = dpp0_add_u64<0x114>(v);
  v = dpp0_add_u64<0x118>(v);
  v = dpp0_add_u64<0x142, 0xA>(v);
  v = dpp0_add_u64<0x143, 0xC>(v);
  return v;
}

// The units of block mass bits u with the row's frexp exponent e:
// ceil(m * 2^(51 - e)), exact.
__device__ __forceinline__ uint64_t row_units(uint32_t u, int e) {
  const int ef = (int)(u >> 23);
  if (ef >= 99 + e && ef > 0) return (uint64_t)((u & 0x7FFFFFu) | 0x800000u) << (ef - 99 - e);
  return fixed_units(u, e);
}

// One wave per row (four rows per workgroup), no workgroup barriers.  The
// cut is the least inverted-bits value v with F(v) = sum of the units q of
// the blocks with ku <= v reaching T (F only steps at the blocks' keys, so v
// is one of them, and F(v - 1) < T); in mass bits u = 2^32 - 1 - ku that is
// the largest uv with the units of the blocks of u >= uv reaching T.  Among
// the blocks with u = uv (equal masses, equal units) the cut falls on the
// need-th in index order.  Lane l owns the contiguous blocks [l kPer,
// l kPer + kPer) (kPer odd, 64 kPer >= nk; blocks past nk read as 0), so lane
// order is index order.
//
// The search runs over rel = umax - u in [0, umax - umin] (umin: the least
// positive mass).  A radix pass over the top 8 bits of the range (units
// summed per digit in an LDS histogram) finds the digit whose band of masses
// holds the cut; when at most 64 blocks fall in that band (the usual case)
// they are listed in index order and each listed block's cumulative units are
// counted directly against the others; otherwise further radix passes of 8
// bits narrow the band.  Units are mant << (exponent shift) for masses within
// 2^27 of the row maximum (exact, no rounding) and the general ceil rule for
// smaller or denormal ones.  The row's kept count goes to counts, its kept
// blocks as bits to keep.
template <int kPer>
__global__ __launch_bounds__(256) void cut_wave_kernel(const Geom g, const float* __restrict__ M, const PTable pt,
                                                       int32_t* __restrict__ counts,
                                                       uint32_t* __restrict__ keep, int32_t* __restrict__ done) {
  static_assert(kPer % 2 == 1 && kPer <= 31, "odd runs: lanes reading runs of kPer words hit distinct banks");
  // per wave: the staged row (kept for the listing); the radix histogram, then the listed blocks, then the
  // kept bits
  __shared__ uint32_t stage_all[4][64 * kPer];
  __shared__ uint64_t hist_all[4][256];
  __shared__ uint32_t eq_all[4][64];  // per wave: each lane's tie bits, from the listed band
  // wave-uniform values live in scalar registers (the buffer descriptor too)
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * 4 + wv;
  if (row == 0 && lane == 0) *done = 0;  // the order kernel's counter
  if (row >= g.rows()) return;           // whole waves only
  const int h = (row / g.nq) % g.H;
  const uint64_t P = pt.P[pt.per_head ? h : 0];
  const int nk = g.nk;
  const int j0 = lane * kPer;
  uint32_t* stage = stage_all[wv];
  uint64_t* hist = hist_all[wv];

  // The row through LDS: coalesced loads of block 64 c + lane (buffer loads:
  // blocks past the row's end read as 0 without a memory access), then each
  // lane reads back its own run.
  {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(M + (int64_t)row * nk), (short)0, nk * 4, 0x00020000);
    uint32_t x[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) x[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, (64 * c + lane) * 4, 0, 0);
#pragma unroll
    for (int c = 0; c < kPer; ++c) stage[64 * c + lane] = sanitized_bits(__uint_as_float(x[c]));
  }
  wave_lds_sync();
  uint32_t u[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) u[t] = stage[j0 + t];
  uint32_t umax = 0, umin = 0xFFFFFFFFu;  // largest mass; least positive mass
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    umax = max(umax, u[t]);
    umin = min(umin, u[t] ? u[t] : 0xFFFFFFFFu);
  }
  umax = wave_max_u32_uniform(umax);

  int s;
  uint32_t gt = 0, eq = 0;  // this lane's blocks with u > uv, and with u == uv (bit t: block j0 + t)
  int jcut = nk;            // kept: u > uv, or u == uv and index <= jcut
  if (P == (1ull << 32)) {  // keep everything
    s = nk;
#pragma unroll
    for (int t = 0; t < kPer; ++t) gt |= (j0 + t < nk ? 1u : 0u) << t;
  } else {
    const int e = umax ? frexp_exp(umax) : 0;
    const int c = 99 + e;
    const uint32_t fast_lo = (uint32_t)max(c, 1) << 23;  // masses with bits >= this take the shift rule
    uint64_t q[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const uint32_t mant = u[t] ? ((u[t] & 0x7FFFFFu) | 0x800000u) : 0u;
      q[t] = (uint64_t)mant << (((int)(u[t] >> 23) - c) & 63);
    }
    if (__ballot(umin < fast_lo)) {  // masses below 2^-27 of the row maximum, or denormal: the rounded rule
#pragma unroll
      for (int t = 0; t < kPer; ++t)
        if (u[t] != 0 && u[t] < fast_lo) q[t] = fixed_units(u[t], e);
    }
    uint64_t run = 0;
#pragma unroll
    for (int t = 0; t < kPer; ++t) run += q[t];
    const uint64_t T = threshold(P, wave_sum_u64(run));
    uint64_t below = 0;   // units of the blocks with u > uv
    uint32_t uv = umax;   // T == 0, or one positive mass value: the cut is at the largest mass
    bool listed = false;  // the cut found among the listed blocks of a band (their ties in eq)
    if (T != 0) {
      umin = wave_min_u32(umin);
      const uint32_t width = umax - umin;
      // rel = umax - u: in [0, width] for masses, umax > width for zeros (which
      // add no units to any bin and lie outside every band cut at width)
      uint32_t rel[kPer];
#pragma unroll
      for (int t = 0; t < kPer; ++t) rel[t] = umax - u[t];
      uint32_t pre = 0;  // digits found so far
      uint64_t acc = 0;  // units of the blocks below the prefix's range
      int top = width ? 32 - __builtin_clz(width) : 0;
      for (int pass = 0; top > 0 && !listed; ++pass) {
        const int shift = top > 8 ? top - 8 : 0;
        const uint32_t dmask = (1u << (top - shift)) - 1u;
        const uint32_t above = top >= 32 ? 0u : (0xFFFFFFFFu << top);
        hist[4 * lane] = 0;
        hist[4 * lane + 1] = 0;
        hist[4 * lane + 2] = 0;
        hist[4 * lane + 3] = 0;
        wave_lds_sync();
        if (pass == 0) {  // every block: zeros add 0 to some bin
#pragma unroll
          for (int t = 0; t < kPer; ++t)
            atomicAdd(reinterpret_cast<unsigned long long*>(hist + ((rel[t] >> shift) & dmask)),
                      (unsigned long long)q[t]);
        } else {  // the blocks in the prefix's range (a zero, if there, adds 0)
#pragma unroll
          for (int t = 0; t < kPer; ++t)
            if (((rel[t] ^ pre) & above) == 0)
              atomicAdd(reinterpret_cast<unsigned long long*>(hist + ((rel[t] >> shift) & dmask)),
                        (unsigned long long)q[t]);
        }
        wave_lds_sync();
        uint64_t cs[4];  // inclusive sums of this lane's digits 4 lane .. 4 lane + 3
        cs[0] = hist[4 * lane];
#pragma unroll
        for (int k = 1; k < 4; ++k) cs[k] = cs[k - 1] + hist[4 * lane + k];
        const uint64_t inc = wave_incl_scan_u64(cs[3]);  // inclusive scan over lanes
        const uint64_t base = acc + (inc - cs[3]);
        // this lane's least digit reaching T (4: none), and the units below it
        int k = 4;
        uint64_t bel = 0;
#pragma unroll
        for (int kk = 3; kk >= 0; --kk)
          if (base + cs[kk] >= T) {
            k = kk;
            bel = kk ? cs[kk - 1] : 0;
          }
        // some lane hits: acc plus all units in the prefix's range is F(end of the range) >= T
        const uint64_t hit = __ballot(k < 4);
        const int lf = __builtin_ctzll(hit);
        const uint32_t digit = 4u * lf + (uint32_t)__builtin_amdgcn_readlane(k, lf);
        const uint64_t add = (inc - cs[3]) + bel;
        acc += ((uint64_t)lane_u32((uint32_t)(add >> 32), lf) << 32) | lane_u32((uint32_t)add, lf);
        pre |= digit << shift;
        top = shift;
        wave_lds_sync();  // every lane has read the histogram before it is cleared or reused
        if (top == 0) break;
        // the blocks of the chosen digit: rel in [pre, pre + 2^top); listed when at most 64
        const uint32_t span = min((1u << top) - 1u, width - pre);  // the band ends at width: zeros stay out
        uint32_t smask = 0;
#pragma unroll
        for (int t = 0; t < kPer; ++t) smask |= (rel[t] - pre <= span ? 1u : 0u) << t;
        const int cnt = __popc(smask);
        const int incl = (int)wave_incl_scan_u32((uint32_t)cnt);  // listed blocks of lanes <= this one
        const int nlist = __builtin_amdgcn_readlane(incl, 63);
        if (nlist > 64) continue;
        // (mass bits, index) and units of each listed block, in index order
        int at = incl - cnt;
        while (smask) {
          const int t = __builtin_ctz(smask);
          smask &= smask - 1u;
          const uint32_t uj = stage[j0 + t];
          hist[2 * at] = (uint64_t)uj | ((uint64_t)(j0 + t) << 32);
          hist[2 * at + 1] = row_units(uj, e);
          ++at;
        }
        wave_lds_sync();
        const uint32_t ui = lane < nlist ? (uint32_t)hist[2 * lane] : 0u;
        uint64_t fle = acc, flt = acc;  // units of the blocks with u >= ui, and with u > ui
        for (int x = 0; x < nlist; ++x) {
          const uint32_t ux = (uint32_t)hist[2 * x];
          const uint64_t qx = hist[2 * x + 1];
          fle += ux >= ui ? qx : 0;
          flt += ux > ui ? qx : 0;
        }
        // the cut: the largest listed mass whose cumulative units reach T
        uv = wave_max_u32_uniform(lane < nlist && fle >= T ? ui : 0u);
        const bool tie = lane < nlist && ui == uv;
        const uint64_t at_v = __ballot(tie);
        const int lv = __builtin_ctzll(at_v);
        below = ((uint64_t)lane_u32((uint32_t)(flt >> 32), lv) << 32) | lane_u32((uint32_t)flt, lv);
        // every block of mass uv lies in the band, so the listed ties are all of
        // them: their bits go to the owning lanes' tie words
        uint32_t* eqw = eq_all[wv];
        eqw[lane] = 0;
        wave_lds_sync();
        if (tie) {
          const int j = (int)(hist[2 * lane] >> 32);
          atomicOr(&eqw[j / kPer], 1u << (j % kPer));
        }
        wave_lds_sync();
        eq = eqw[lane];
        listed = true;
        wave_lds_sync();  // the list is read before its space is reused
      }
      if (!listed) {
        uv = umax - pre;
        below = acc;
      }
    }
    const uint64_t qu = row_units(uv, e);
    uint64_t need = 1;  // one tie is enough unless T lies beyond the first
    if (below < T && qu > 0 && T - below > qu) need = (T - below + qu - 1) / qu;
#pragma unroll
    for (int t = 0; t < kPer; ++t) gt |= (u[t] > uv ? 1u : 0u) << t;
    if (!listed) {
#pragma unroll
      for (int t = 0; t < kPer; ++t) eq |= (u[t] == uv ? 1u : 0u) << t;
      if (uv == 0) {  // an all-zero row: blocks past nk (read as 0) are no ties
        const int nv = min(max(nk - j0, 0), kPer);
        eq &= nv >= 32 ? 0xFFFFFFFFu : (1u << nv) - 1u;
      }
    }
    const int nties = __popc(eq);
    const int incl = (int)wave_incl_scan_u32((uint32_t)nties);  // ties owned by lanes <= this one
    // the need-th tie in index order: in the lane whose ties cover it
    const int before = incl - nties;
    int jc = -1;
    if ((int64_t)need > before && (int64_t)need <= incl) {
      uint32_t w = eq;
      for (int r = before + 1; r < (int)need; ++r) w &= w - 1u;
      jc = j0 + __builtin_ctz(w);
    }
    const uint64_t owner = __ballot(jc >= 0);
    jcut = __builtin_amdgcn_readlane(jc, owner ? __builtin_ctzll(owner) : 0);
    s = wave_sum_i32(__popc(gt)) + (int)need;
  }
  // The kept blocks (u > uv, or u == uv up to jcut) as bits, assembled in this
  // wave's LDS (at most 64 words: n_k <= 2048 here), then stored coalesced.
  const int upto = jcut - j0 + 1;  // ties at t < upto are kept
  const uint32_t tmask = upto >= 32 ? 0xFFFFFFFFu : (upto <= 0 ? 0u : (1u << upto) - 1u);
  const uint32_t bits = gt | (eq & tmask);
  uint32_t* words = reinterpret_cast<uint32_t*>(hist);
  const int nw = (nk + 31) / 32;
  words[lane] = 0;
  wave_lds_sync();
  or_bit_run(words, j0, bits);
  wave_lds_sync();
  if (lane < nw) keep[(int64_t)row * nw + lane] = words[lane];
  if (lane == 0) counts[row] = s;
}

// One workgroup (four waves) per row, for rows of more than 64 * 31 blocks:
// the wave kernel's search with block-wide reductions.  Thread t owns the
// contiguous blocks [t kPer, t kPer + kPer) (kPer odd, 256 kPer >= nk;
// blocks past nk read as 0), so thread order is index order.
template <int kPer>
__global__ __launch_bounds__(kSelThreads) void cut_group_kernel(const Geom g, const float* __restrict__ M,
                                                                const PTable pt, int32_t* __restrict__ counts,
                                                                uint32_t* __restrict__ keep,
                                                                int32_t* __restrict__ done) {
  static_assert(kPer % 2 == 1 && kPer <= 31, "odd runs: threads reading runs of kPer words hit distinct banks");
  __shared__ uint32_t stage[kSelThreads * kPer];  // the staged row
  __shared__ uint64_t hist[256];                  // the radix histogram, then the listed blocks
  __shared__ uint32_t words[kSelThreads];         // each thread's tie bits, then the row's kept bits
  __shared__ uint64_t r64[4];
  __shared__ uint32_t r32[4];
  __shared__ uint64_t s_u64[2];
  __shared__ int s_i32[2];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (row == 0 && tid == 0) *done = 0;  // the order kernel's counter
  const int h = (row / g.nq) % g.H;
  const uint64_t P = pt.P[pt.per_head ? h : 0];
  const int nk = g.nk;
  const int j0 = tid * kPer;

  // block-wide reductions: each wave's value (uniform), then the four in LDS
  auto block_max_u32 = [&](uint32_t v) {
    v = wave_max_u32_uniform(v);
    if (lane == 0) r32[w] = v;
    __syncthreads();
    const uint32_t r = max(max(r32[0], r32[1]), max(r32[2], r32[3]));
    __syncthreads();
    return r;
  };
  auto block_min_u32 = [&](uint32_t v) {
    v = wave_min_u32(v);
    if (lane == 0) r32[w] = v;
    __syncthreads();
    const uint32_t r = min(min(r32[0], r32[1]), min(r32[2], r32[3]));
    __syncthreads();
    return r;
  };
  auto block_sum_u64 = [&](uint64_t v) {
    v = wave_sum_u64(v);
    if (lane == 0) r64[w] = v;
    __syncthreads();
    const uint64_t r = (r64[0] + r64[1]) + (r64[2] + r64[3]);
    __syncthreads();
    return r;
  };
  // inclusive scan over the block's threads (thread order)
  auto block_incl_scan_u32 = [&](uint32_t v) {
    v = wave_incl_scan_u32(v);
    if (lane == 63) r32[w] = v;
    __syncthreads();
    uint32_t before = 0;
    for (int ww = 0; ww < w; ++ww) before += r32[ww];
    __syncthreads();
    return v + before;
  };

  {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(M + (int64_t)row * nk), (short)0, nk * 4, 0x00020000);
    uint32_t x[kPer];
#pragma unroll
    for (int c = 0; c < kPer; ++c) x[c] = __builtin_amdgcn_raw_buffer_load_b32(rs, (kSelThreads * c + tid) * 4, 0, 0);
#pragma unroll
    for (int c = 0; c < kPer; ++c) stage[kSelThreads * c + tid] = sanitized_bits(__uint_as_float(x[c]));
  }
  __syncthreads();
  uint32_t u[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) u[t] = stage[j0 + t];
  uint32_t umax = 0, umin = 0xFFFFFFFFu;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    umax = max(umax, u[t]);
    umin = min(umin, u[t] ? u[t] : 0xFFFFFFFFu);
  }
  umax = block_max_u32(umax);

  int s;
  uint32_t gt = 0, eq = 0;
  int jcut = nk;
  if (P == (1ull << 32)) {
    s = nk;
#pragma unroll
    for (int t = 0; t < kPer; ++t) gt |= (j0 + t < nk ? 1u : 0u) << t;
  } else {
    const int e = umax ? frexp_exp(umax) : 0;
    const int c = 99 + e;
    const uint32_t fast_lo = (uint32_t)max(c, 1) << 23;
    uint64_t q[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const uint32_t mant = u[t] ? ((u[t] & 0x7FFFFFu) | 0x800000u) : 0u;
      q[t] = (uint64_t)mant << (((int)(u[t] >> 23) - c) & 63);
    }
    if (__ballot(umin < fast_lo)) {
#pragma unroll
      for (int t = 0; t < kPer; ++t)
        if (u[t] != 0 && u[t] < fast_lo) q[t] = fixed_units(u[t], e);
    }
    uint64_t run = 0;
#pragma unroll
    for (int t = 0; t < kPer; ++t) run += q[t];
    const uint64_t T = threshold(P, block_sum_u64(run));
    uint64_t below = 0;
    uint32_t uv = umax;
    bool listed = false;
    if (T != 0) {
      umin = block_min_u32(umin);
      const uint32_t width = umax - umin;
      uint32_t rel[kPer];
#pragma unroll
      for (int t = 0; t < kPer; ++t) rel[t] = umax - u[t];
      uint32_t pre = 0;
      uint64_t acc = 0;
      int top = width ? 32 - __builtin_clz(width) : 0;
      for (int pass = 0; top > 0 && !listed; ++pass) {
        const int shift = top > 8 ? top - 8 : 0;
        const uint32_t dmask = (1u << (top - shift)) - 1u;
        const uint32_t above = top >= 32 ? 0u : (0xFFFFFFFFu << top);
        hist[tid] = 0;
        __syncthreads();
        if (pass == 0) {
#pragma unroll
          for (int t = 0; t < kPer; ++t)
            atomicAdd(reinterpret_cast<unsigned long long*>(hist + ((rel[t] >> shift) & dmask)),
                      (unsigned long long)q[t]);
        } else {
#pragma unroll
          for (int t = 0; t < kPer; ++t)
            if (((rel[t] ^ pre) & above) == 0)
              atomicAdd(reinterpret_cast<unsigned long long*>(hist + ((rel[t] >> shift) & dmask)),
                        (unsigned long long)q[t]);
        }
        __syncthreads();
        // thread t holds digit t: inclusive scan of the units over the digits
        const uint64_t hv = hist[tid];
        uint64_t inc = wave_incl_scan_u64(hv);
        if (lane == 63) r64[w] = inc;
        __syncthreads();
        for (int ww = 0; ww < w; ++ww) inc += r64[ww];
        const uint64_t hitm = __ballot(acc + inc >= T);  // the least digit reaching T, by wave
        if (lane == 0) r32[w] = hitm ? (uint32_t)(64 * w + __builtin_ctzll(hitm)) : 0xFFFFFFFFu;
        __syncthreads();
        const uint32_t digit = min(min(r32[0], r32[1]), min(r32[2], r32[3]));  // exists: acc + all >= T
        if ((uint32_t)tid == digit) s_u64[0] = acc + inc - hv;
        __syncthreads();
        acc = s_u64[0];
        pre |= digit << shift;
        top = shift;
        if (top == 0) break;
        const uint32_t span = min((1u << top) - 1u, width - pre);
        uint32_t smask = 0;
#pragma unroll
        for (int t = 0; t < kPer; ++t) smask |= (rel[t] - pre <= span ? 1u : 0u) << t;
        const int cnt = __popc(smask);
        const int incl = (int)block_incl_scan_u32((uint32_t)cnt);
        if (tid == kSelThreads - 1) s_i32[0] = incl;
        __syncthreads();
        const int nlist = s_i32[0];
        if (nlist > 64) continue;
        int at = incl - cnt;
        while (smask) {
          const int t = __builtin_ctz(smask);
          smask &= smask - 1u;
          const uint32_t uj = stage[j0 + t];
          hist[2 * at] = (uint64_t)uj | ((uint64_t)(j0 + t) << 32);
          hist[2 * at + 1] = row_units(uj, e);
          ++at;
        }
        __syncthreads();
        // wave 0 resolves the cut among the listed blocks
        if (w == 0) {
          const uint32_t ui = lane < nlist ? (uint32_t)hist[2 * lane] : 0u;
          uint64_t fle = acc, flt = acc;
          for (int x = 0; x < nlist; ++x) {
            const uint32_t ux = (uint32_t)hist[2 * x];
            const uint64_t qx = hist[2 * x + 1];
            fle += ux >= ui ? qx : 0;
            flt += ux > ui ? qx : 0;
          }
          const uint32_t cut = wave_max_u32_uniform(lane < nlist && fle >= T ? ui : 0u);
          const uint64_t at_v = __ballot(lane < nlist && ui == cut);
          const int lv = __builtin_ctzll(at_v);
          if (lane == 0) {
            s_u64[1] = ((uint64_t)lane_u32((uint32_t)(flt >> 32), lv) << 32) | lane_u32((uint32_t)flt, lv);
            s_i32[1] = (int)cut;
          }
        }
        words[tid] = 0;
        __syncthreads();
        uv = (uint32_t)s_i32[1];
        below = s_u64[1];
        // the ties: every block of mass uv lies in the band and is listed
        if (tid < nlist && (uint32_t)hist[2 * tid] == uv) {
          const int j = (int)(hist[2 * tid] >> 32);
          atomicOr(&words[j / kPer], 1u << (j % kPer));
        }
        __syncthreads();
        eq = words[tid];
        listed = true;
        __syncthreads();
      }
      if (!listed) {
        uv = umax - pre;
        below = acc;
      }
    }
    const uint64_t qu = row_units(uv, e);
    uint64_t need = 1;
    if (below < T && qu > 0 && T - below > qu) need = (T - below + qu - 1) / qu;
#pragma unroll
    for (int t = 0; t < kPer; ++t) gt |= (u[t] > uv ? 1u : 0u) << t;
    if (!listed) {
#pragma unroll
      for (int t = 0; t < kPer; ++t) eq |= (u[t] == uv ? 1u : 0u) << t;
      if (uv == 0) {
        const int nv = min(max(nk - j0, 0), kPer);
        eq &= nv >= 32 ? 0xFFFFFFFFu : (1u << nv) - 1u;
      }
    }
    const int nties = __popc(eq);
    const int incl = (int)block_incl_scan_u32((uint32_t)nties);
    const int before = incl - nties;
    if ((int64_t)need > before && (int64_t)need <= incl) {
      uint32_t wd = eq;
      for (int r = before + 1; r < (int)need; ++r) wd &= wd - 1u;
      s_i32[0] = j0 + __builtin_ctz(wd);  // one thread owns the need-th tie
    }
    const int nbelow = (int)block_incl_scan_u32((uint32_t)__popc(gt));  // thread 255: all
    if (tid == kSelThreads - 1) s_i32[1] = nbelow;
    __syncthreads();
    jcut = s_i32[0];
    s = s_i32[1] + (int)need;
  }
  const int upto = jcut - j0 + 1;
  const uint32_t tmask = upto >= 32 ? 0xFFFFFFFFu : (upto <= 0 ? 0u : (1u << upto) - 1u);
  const uint32_t bits = gt | (eq & tmask);
  const int nw = (nk + 31) / 32;
  words[tid] = 0;
  __syncthreads();
  or_bit_run(words, j0, bits);
  __syncthreads();
  for (int x = tid; x < nw; x += kSelThreads) keep[(int64_t)row * nw + x] = words[x];
  if (tid == 0) counts[row] = s;
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

// The first col_idx slot of row's list: its head's first slot plus the kept
// blocks of the head's earlier rows (both written by order_kernel); lane 0 of
// the row's wave stores it as row_ptr[row].  With a work order, the wave also
// fills one order slot, reading its row index as a rank position p (rank r
// of head h): the work group (h, r / 32) has the key x = gkey (its first
// count); the groups before it are k = r / 32 of its own head, and of every
// other head h' those with a key > x, or >= x when h' < h (ties by head):
// ceil(rows of h' with count > x (or >= x) / 32), from h''s bucket starts;
// among them the short ones (each head's last group, nq - 32 (ngh - 1) rows)
// come from the heads' last keys the same way.  order[32 R - (32 - last) S +
// r mod 32] = ranked[p] (a slot outside [0, rows) cannot arise and is not
// written).
__device__ __forceinline__ int finish_row(const Geom& g, const SelectWs& ws, int row, int lane, int32_t* row_ptr,
                                          int32_t* order) {
  const int nq = g.nq, nk = g.nk, h = row / nq;
  const int start = ws.head_base[h] + ws.local_off[row];
  if (lane == 0) row_ptr[row] = start;
  if (order) {
    const int heads = g.B * g.H, ngh = ws.ngh, r = row - h * nq, k = r / kGroupRows;
    const int lastn = nq - (ngh - 1) * kGroupRows;
    const int x = ws.gkey[h * ngh + k], b = nk - x;
    int R = k, S = 0;
    for (int h0 = 0; h0 < heads; h0 += kWave) {  // the other heads, 64 at a time
      const int hh = h0 + lane;
      int t = 0, sh = 0;
      if (hh < heads && hh != h) {
        const int32_t* bs = ws.bucket_start + (int64_t)hh * (nk + 2);
        t = ((hh < h ? bs[b + 1] : bs[b]) + kGroupRows - 1) / kGroupRows;
        if (lastn < kGroupRows) {
          const int y = ws.gkey[hh * ngh + ngh - 1];
          sh = (hh < h ? y >= x : y > x) ? 1 : 0;
        }
      }
      R += wave_sum_i32(t);
      S += wave_sum_i32(sh);
    }
    const int slot = kGroupRows * R - (kGroupRows - lastn) * S + r % kGroupRows;
    if (lane == 0 && (unsigned)slot < (unsigned)g.rows()) order[slot] = ws.ranked[row];
  }
  return start;
}

// One wave per row (four rows per workgroup): the row's kept bits (from the
// cut, 4 bytes per 32 blocks instead of the masses again) are loaded once,
// one word per lane; for each 64 blocks (a wave-uniform 64-bit mask m) lane
// l writes block 64 s + l, if kept, at the row's first slot plus the kept
// blocks before it (all 64 when m is full: the common case, one coalesced
// store of consecutive indices).
__global__ __launch_bounds__(256) void compact_kernel(const Geom g, const uint32_t* __restrict__ keep,
                                                      const SelectWs ws, int32_t* __restrict__ row_ptr,
                                                      int32_t* __restrict__ order, int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= g.rows()) return;  // whole waves only
  const int nk = g.nk, nw = (nk + 31) / 32;  // nw <= 128
  const uint32_t* kr = keep + (int64_t)row * nw;
  const uint32_t w0 = lane < nw ? kr[lane] : 0u, w1 = 64 + lane < nw ? kr[64 + lane] : 0u;
  int pos = finish_row(g, ws, row, lane, row_ptr, order);
  // the row's slots lie inside the capacity checked on the host (rows * nk <
  // 2^31) unless the offsets are not the order kernel's; then nothing is written
  if (pos < 0 || (int64_t)pos + ws.counts[row] > (int64_t)g.rows() * nk) return;
  int32_t* dst = col_idx + pos;
  for (int s = 0; 64 * s < nk; ++s) {  // blocks [64 s, 64 s + 64): words 2s, 2s + 1
    const int a = 2 * s, b = 2 * s + 1;
    const uint32_t lo = __builtin_amdgcn_readlane(a < 64 ? w0 : w1, a & 63);
    const uint32_t hi = __builtin_amdgcn_readlane(b < 64 ? w0 : w1, b & 63);
    if ((lo & hi) == 0xFFFFFFFFu) {  // all 64 kept
      dst[lane] = 64 * s + lane;
      dst += 64;
    } else {
      const uint64_t m = ((uint64_t)hi << 32) | lo;
      if ((m >> lane) & 1ull) dst[__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u))] = 64 * s + lane;
      dst += __popcll(m);
    }
  }
}

constexpr int kOrderThreads = 1024;

// x from lane (lane ^ J), by DPP moves and gfx950 lane swaps (no LDS); every
// lane must be active.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
  if constexpr (J == 1) {
    return dpp_u32<0xB1>(x);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (J == 2) {
    return dpp_u32<0x4E>(x);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (J == 4) {
    return dpp_u32<0x141>(dpp_u32<0x1B>(x));  // quad_perm [3, 2, 1, 0] (xor 3), then row_half_mirror (xor 7)
  } else if constexpr (J == 8) {
    return dpp_u32<0x128>(x);  // row_ror 8 (xor 8 within a 16-lane row)
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);  // rows (0,0,2,2), (1,1,3,3)
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane distances 1 .. 32");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);  // halves (lo,lo), (hi,hi)
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

// One in-wave compare-exchange of a bitonic stage: element i keeps the
// smaller key when it is the lower of its pair in an ascending block (or the
// upper in a descending one), else the larger.
template <int J>
__device__ __forceinline__ uint32_t bitonic_cx(uint32_t x, int i, int k) {
  const uint32_t y = xor_lane<J>(x);
  return (((i & J) == 0) == ((i & k) == 0)) ? min(x, y) : max(x, y);
}

// In-wave stages of a block of size k, distances min(k/2, 32) down to 1.
__device__ __forceinline__ uint32_t bitonic_wave(uint32_t x, int i, int k) {
  if (k >= 64) x = bitonic_cx<32>(x, i, k);
  if (k >= 32) x = bitonic_cx<16>(x, i, k);
  if (k >= 16) x = bitonic_cx<8>(x, i, k);
  if (k >= 8) x = bitonic_cx<4>(x, i, k);
  if (k >= 4) x = bitonic_cx<2>(x, i, k);
  return bitonic_cx<1>(x, i, k);
}

// Ascending bitonic sort of the n keys in s[] (LDS, n a power of two, at
// least 64) by the whole workgroup (a multiple of 64 threads).  Compare-
// exchange distances of 64 or more go through LDS with a barrier each;
// shorter ones stay inside a wave (key i on lane i mod 64, partners by lane
// exchange), with all stages of block sizes 2 to 64 in one register pass.
__device__ void bitonic_sort_lds(uint32_t* s, int n) {
  const int nt = blockDim.x;
  for (int i = threadIdx.x; i < n; i += nt) {  // whole waves: n and nt are multiples of 64
    uint32_t x = s[i];
    for (int k = 2; k <= 64; k <<= 1) x = bitonic_wave(x, i, k);
    s[i] = x;
  }
  __syncthreads();
  for (int k = 128; k <= n; k <<= 1) {
    for (int j = k >> 1; j >= 64; j >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += nt) {
        const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1)), b = a + j;  // the i-th pair of this stage
        const uint32_t x = s[a], y = s[b];
        if ((x > y) == ((a & k) == 0)) {
          s[a] = y;
          s[b] = x;
        }
      }
      __syncthreads();
    }
    for (int i = threadIdx.x; i < n; i += nt) s[i] = bitonic_wave(s[i], i, k);
    __syncthreads();
  }
}

__host__ __device__ inline int pow2_at_least(int n) {
  int p = 64;  // the sort's least size
  while (p < n) p <<= 1;
  return p;
}

// Exclusive scan of the per-thread values v over the workgroup (wsum: one
// int per wave); the total goes to *total when given.
__device__ __forceinline__ int block_exclusive_scan_reg(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int ww = 0; ww < nw; ++ww) {
    const int s = wsum[ww];
    if (ww < w) before += s;
    all += s;
  }
  __syncthreads();
  if (total) *total = all;
  return before + inc - v;
}

// Row offsets and the work order's ranks from the kept counts, one
// workgroup per (batch, head), then a hand-off to the last workgroup to
// finish (*done must be 0 on entry: the count kernel before clears it).
//   per head h: local_off[row] = the kept blocks of the head's earlier rows,
//     head_total[h]; when the order is wanted, the head's rows ranked by
//     count descending, ties by row: a sort of the unique keys
//     (nk - count) << 14 | local row (nq <= 16384) -> ranked[h nq + r] = row
//     of rank r, gkey[h ngh + k] = the count of rank 32 k (the first, largest,
//     of work group k), and bucket_start[h][b] = the first rank of bucket
//     b = nk - count (b = nk + 1: nq);
//   last workgroup: head_base = exclusive scan of head_total, row_ptr[rows].
// The work groups' order slots follow per row from these (finish_row).
// The counts are read once, each thread a contiguous run of at most 16.
__global__ __launch_bounds__(kOrderThreads) void order_kernel(const Geom g, const int32_t* __restrict__ counts,
                                                              const SelectWs ws, int32_t* __restrict__ row_ptr,
                                                              int want_order) {
  extern __shared__ uint32_t ol[];  // sort keys
  __shared__ int wsum[kOrderThreads / 64];
  __shared__ int last;
  const int h = blockIdx.x, nq = g.nq, nk = g.nk, tid = threadIdx.x;
  {
    const int32_t* hc = counts + (int64_t)h * nq;
    const int per = (nq + (int)blockDim.x - 1) / (int)blockDim.x, i0 = tid * per;  // per <= 16
    int cnt[16];
    int run = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      cnt[k] = (k < per && i0 + k < nq) ? hc[i0 + k] : 0;
      run += cnt[k];
    }
    int off = block_exclusive_scan_reg(run, wsum, ws.head_total + h);
    int32_t* lo = ws.local_off + (int64_t)h * nq;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < per && i0 + k < nq) {
        lo[i0 + k] = off;
        off += cnt[k];
      }
    if (want_order) {
      const int n = pow2_at_least(nq);
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (k < per && i0 + k < n) {
          const int i = i0 + k;
          ol[i] = i < nq ? ((uint32_t)(nk - min(max(cnt[k], 0), nk)) << 14) | (uint32_t)i : 0xFFFFFFFFu;
        }
      for (int i = per * (int)blockDim.x + tid; i < n; i += blockDim.x) ol[i] = 0xFFFFFFFFu;  // beyond the runs
      __syncthreads();
      bitonic_sort_lds(ol, n);
      int32_t* ranked = ws.ranked + (int64_t)h * nq;
      int32_t* gkey = ws.gkey + (int64_t)h * ws.ngh;
      int32_t* bst = ws.bucket_start + (int64_t)h * (nk + 2);
      for (int r = tid; r < nq; r += blockDim.x) {
        const uint32_t k = ol[r];
        ranked[r] = h * nq + (int)(k & 0x3FFFu);
        if (r % kGroupRows == 0) gkey[r / kGroupRows] = nk - (int)(k >> 14);
      }
      // bucket b starts at the first rank whose key is at least b << 14: a
      // binary search over the sorted keys (padding keys are all ones)
      const int lg = 31 - __builtin_clz(n);
      for (int b = tid; b <= nk + 1; b += blockDim.x) {
        const uint32_t kb = (uint32_t)b << 14;
        int lo = 0;  // keys before lo are < kb
        for (int step = n >> 1, it = 0; it <= lg; ++it, step >>= 1)
          if (step > 0 && ol[lo + step - 1] < kb) lo += step;
        if (lo < n && ol[lo] < kb) ++lo;
        bst[b] = min(lo, nq);
      }
    }
  }
  __syncthreads();  // the workgroup's stores are done (to L2) ...
  if (tid == 0) {
    __threadfence();  // ... and made visible to every XCD before the count moves
    last = atomicAdd(ws.done, 1) == (int)gridDim.x - 1;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  block_exclusive_scan_i32(ws.head_total, gridDim.x, ws.head_base, row_ptr + (int64_t)gridDim.x * nq, wsum);
}

// Online block thresholding (the Sol-Attn page's block thresholding during
// the online-softmax pass): visiting the row's key blocks in index order,
// block j is kept when m_j >= theta * max(m_0 .. m_j), on the sanitised fp32
// masses, compared in fp64.  One wave per row, 64 blocks per step: coalesced
// loads, an inclusive max scan across the wave, and the running maximum
// carried from the previous step.  kWrite = false: the kept count into
// ws.counts[row] (and the order kernel's done counter cleared); true: the
// kept indices, ascending, from the row's first slot, with row_ptr and the
// work order stored.
template <bool kWrite>
__global__ __launch_bounds__(256) void threshold_kernel(const Geom g, const float* __restrict__ M, const ThetaTable tt,
                                                        const SelectWs ws, int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ order, int32_t* __restrict__ col_idx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (!kWrite && blockIdx.x == 0 && threadIdx.x == 0) *ws.done = 0;
  if (row >= g.rows()) return;  // the whole wave
  const int nk = g.nk;
  const double theta = tt.t[tt.per_head ? (row / g.nq) % g.H : 0];
  const float* Mrow = M + (int64_t)row * nk;
  int32_t* dst = kWrite ? col_idx + finish_row(g, ws, row, lane, row_ptr, order) : nullptr;
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
  if (!kWrite && lane == 0) ws.counts[row] = kept;
}

// List merge: row r takes its count from set b when its head is flagged,
// from set a otherwise (clamped to [0, nk], so a malformed count cannot
// place a row outside the output).  Also clears the order kernel's done
// counter.
__global__ __launch_bounds__(256) void pick_counts_kernel(int rows, int nq, int nk, const int32_t* __restrict__ take_b,
                                                          const int32_t* __restrict__ rpa,
                                                          const int32_t* __restrict__ rpb, const SelectWs ws) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r == 0) *ws.done = 0;
  if (r >= rows) return;
  const int32_t* rp = take_b[r / nq] ? rpb : rpa;
  ws.counts[r] = min(max(rp[r + 1] - rp[r], 0), nk);
}

// One wave per row: copy the chosen set's indices to the row's first slot
// (row_ptr and the work order stored on the way).
__global__ __launch_bounds__(256) void copy_lists_kernel(const Geom g, const int32_t* __restrict__ take_b,
                                                         const int32_t* __restrict__ rpa,
                                                         const int32_t* __restrict__ cia,
                                                         const int32_t* __restrict__ rpb,
                                                         const int32_t* __restrict__ cib, const SelectWs ws,
                                                         int32_t* __restrict__ row_ptr, int32_t* __restrict__ order,
                                                         int32_t* __restrict__ col_idx) {
  const int r = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), rows = g.rows(), nq = g.nq;
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const bool b = take_b[r / nq] != 0;
  const int32_t* src = (b ? cib : cia) + (b ? rpb : rpa)[r];
  int32_t* dst = col_idx + finish_row(g, ws, r, lane, row_ptr, order);
  const int n = ws.counts[r];
  for (int t = lane; t < n; t += 64) dst[t] = src[t];
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
  const size_t rows = (size_t)g.rows();
  const size_t heads = (size_t)g.B * g.H;
  const int keep_words = (g.nk + 31) / 32;
  const int ngh = (g.nq + kGroupRows - 1) / kGroupRows;
  size_t off = 0;
  auto take = [&](size_t ints) {
    const size_t at = off;
    off = align_up(off + ints * sizeof(int32_t), 256);
    return reinterpret_cast<int32_t*>(base + at);
  };
  int32_t* counts = take(rows);
  int32_t* keep = take(rows * keep_words);
  int32_t* local_off = take(rows);
  int32_t* head_total = take(2 * heads + 1);  // then head_base and done
  int32_t* ranked = take(rows);
  int32_t* gkey = take(heads * (size_t)ngh);
  int32_t* bucket_start = take(heads * (size_t)(g.nk + 2));
  if (layout) {
    layout->counts = counts;
    layout->keep = reinterpret_cast<uint32_t*>(keep);
    layout->keep_words = keep_words;
    layout->local_off = local_off;
    layout->head_total = head_total;
    layout->head_base = head_total + heads;
    layout->done = head_total + 2 * heads;
    layout->ranked = ranked;
    layout->gkey = gkey;
    layout->bucket_start = bucket_start;
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
  const int per = ((g.nk + kWave - 1) / kWave) | 1;  // odd runs per lane
  if (per <= 31) {
    using CutFn = void (*)(const Geom, const float*, const PTable, int32_t*, uint32_t*, int32_t*);
    static const CutFn cuts[16] = {cut_wave_kernel<1>,  cut_wave_kernel<3>,  cut_wave_kernel<5>,  cut_wave_kernel<7>,
                                   cut_wave_kernel<9>,  cut_wave_kernel<11>, cut_wave_kernel<13>, cut_wave_kernel<15>,
                                   cut_wave_kernel<17>, cut_wave_kernel<19>, cut_wave_kernel<21>, cut_wave_kernel<23>,
                                   cut_wave_kernel<25>, cut_wave_kernel<27>, cut_wave_kernel<29>, cut_wave_kernel<31>};
    hipLaunchKernelGGL(cuts[per / 2], dim3((rows + 3) / 4), dim3(256), 0, st, g, M, pt, ws.counts, ws.keep, ws.done);
  } else {  // 1985 .. 4096 blocks: a workgroup per row, odd runs of 9 .. 17 per thread
    using CutFn = void (*)(const Geom, const float*, const PTable, int32_t*, uint32_t*, int32_t*);
    static const CutFn cuts[5] = {cut_group_kernel<9>, cut_group_kernel<11>, cut_group_kernel<13>,
                                  cut_group_kernel<15>, cut_group_kernel<17>};
    const int per_t = ((g.nk + kSelThreads - 1) / kSelThreads) | 1;
    hipLaunchKernelGGL(cuts[(per_t - 9) / 2], dim3(rows), dim3(kSelThreads), 0, st, g, M, pt, ws.counts, ws.keep,
                       ws.done);
  }
  launch_order(g, ws, row_ptr, order != nullptr, st);
  hipLaunchKernelGGL(compact_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, g, (const uint32_t*)ws.keep, ws,
                     row_ptr, order, col_idx);
  return hipGetLastError();
}

hipError_t launch_select_threshold(const Geom& g, const float* M, const ThetaTable& tt, int32_t* row_ptr,
                                   int32_t* col_idx, int32_t* order, const SelectWs& ws, hipStream_t st) {
  const int rows = g.rows();
  const dim3 grid((rows + 3) / 4);
  hipLaunchKernelGGL(threshold_kernel<false>, grid, dim3(256), 0, st, g, M, tt, ws, (int32_t*)nullptr,
                     (int32_t*)nullptr, (int32_t*)nullptr);
  launch_order(g, ws, row_ptr, order != nullptr, st);
  hipLaunchKernelGGL(threshold_kernel<true>, grid, dim3(256), 0, st, g, M, tt, ws, row_ptr, order, col_idx);
  return hipGetLastError();
}

hipError_t launch_merge_lists(const Geom& g, const int32_t* take_b, const int32_t* rpa, const int32_t* cia,
                              const int32_t* rpb, const int32_t* cib, int32_t* row_ptr, int32_t* col_idx,
                              int32_t* order, const SelectWs& ws, hipStream_t st) {
  const int rows = g.rows();
  hipLaunchKernelGGL(pick_counts_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, rows, g.nq, g.nk, take_b, rpa,
                     rpb, ws);
  launch_order(g, ws, row_ptr, order != nullptr, st);
  hipLaunchKernelGGL(copy_lists_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, g, take_b, rpa, cia, rpb, cib, ws,
                     row_ptr, order, col_idx);
  return hipGetLastError();
}

void launch_order(const Geom& g, const SelectWs& ws, int32_t* row_ptr, bool want_order, hipStream_t st) {
  const size_t lds = want_order ? (size_t)pow2_at_least(g.nq) * sizeof(uint32_t) : 0;
  hipLaunchKernelGGL(order_kernel, dim3(g.B * g.H), dim3(kOrderThreads), lds, st, g, (const int32_t*)ws.counts, ws,
                     row_ptr, want_order ? 1 : 0);
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
