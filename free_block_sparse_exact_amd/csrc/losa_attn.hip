// Frozen-pattern block-sparse attention (LoSA page, Methodology Summary:
// sparse attention with a frozen pattern -- each query attends to the valid
// tokens of its row's kept key blocks, softmax normalised over those keys
// only; discarded keys leave the denominator).
//
// bf16 matrix-core path (d in {64, 128}, R in {64, 128}):
//   * a pre-pass packs K and V into lane-major operand copies per 32-token
//     chunk (the exact register images of the MFMA A operands), so every
//     operand load is 64 lanes x 16 contiguous bytes -- with K and V read in
//     their natural layouts each 1 KB load split into ~48 cache accesses and
//     the texture data path, not the matrix cores, set the pace;
//   * one workgroup (four waves, one per SIMD) per 64-query tile of a row
//     (two per row when R = 128), dispatched in the caller's budget order
//     with an XCD-aware mapping.  The waves split the row's 32-key chunks
//     (wave kw takes chunks kw, kw+4, ...), each keeping its own online-
//     softmax state for all 64 queries; the four key groups are merged
//     through LDS at the end.  Each wave holds its Q tile as MFMA B operands
//     in AGPRs (only matrix instructions read it);
//   * S^T = K Q^T and O^T += V^T P^T on 16x16x32 bf16 MFMA.  K rows are fed
//     in the permuted order kappa(kt, rho) = 8*(rho>>2) + 4*kt + (rho&3), so
//     lane l ends up holding the eight consecutive keys 8*(l>>4)+[0,8) of
//     query (l & 15): exactly the k-layout of the P^T operand, so P goes from
//     the S accumulators to the next MFMA without any exchange;
//   * no per-score maximum and no rescaling of O inside the loop (see the
//     main loop); row sums use the bf16-rounded probabilities, matching the
//     numerator, and come from the matrix cores: one more MFMA per query
//     tile and chunk multiplies P^T by a block of ones, whose every row is
//     then the column sums of P^T (replacing sixteen dot products and the
//     adds per chunk: config 1 5.79 -> 5.49 ms, config 3 152.3 -> 150.4 ms
//     on one box);
//   * a two-stage software pipeline (scores of chunk t+1 beside the softmax
//     and P.V of chunk t), chunk keys read from registers, and the MFMA form
//     with vector-register results (built with -amdgpu-mfma-vgpr-form).
#include "losa_device.hpp"
#include "losa_internal.hpp"
#include "losa_pack.hpp"

namespace losa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// A row sum against the wave's reference above this bound (or not finite)
// sends the wave to the exact two-pass path once its chunks are done: with
// every probability, and so the row sum, at most 2^100, neither P nor P.V
// can have overflowed.
constexpr float kLBound = 1.2676506e30f;  // 2^100

// On-the-fly block thresholding (Sol-Attn page: blocks are chosen while the
// online softmax runs, by comparing each block's proxy score with a
// threshold, without materialising a proxy map).  The proxy of key block j
// for this query block is a_j = scale * qbar . kbar_j + ln|B_j| (pooled
// score, weighted by the block's valid keys; fp64 throughout, the fp32 softmax
// scale widened exactly); in index order, the order of the online pass, block
// j is kept when a_j >= ln(theta) + max(a_0 .. a_j).  The kept blocks go to
// list[] in ascending order, in LDS; the return value is their number.  The
// whole workgroup (256 threads) takes part.  scratch: D + nk doubles and nk
// bytes of LDS, free for the call.  mask_row (or null): the kept blocks as
// bits, 32 per word.
template <int D>
__device__ int inpass_list(const Geom& g, const double* __restrict__ qbar_row, const double* __restrict__ kbar_bh,
                           double ln_t, double ln_c, double ln_last, double* scratch, int32_t* list,
                           uint32_t* __restrict__ mask_row) {
  __shared__ double s_wmax[4];
  __shared__ int s_wcnt[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nk = g.nk;
  double* qv = scratch;       // [D]
  double* av = scratch + D;   // [nk]
  uint8_t* kf = reinterpret_cast<uint8_t*>(av + nk);  // [nk] keep flags
  if (tid < D) qv[tid] = qbar_row[tid];
  __syncthreads();
  // Pooled scores, four blocks per wave and step: lane l takes block
  // jb + l/16 and its D/16 dimensions from (l%16)*D/16 (contiguous 16-byte
  // loads), then the 16 lanes of a block add their partial sums.  Eight steps
  // are loaded before any is used, so their loads overlap.
  {
    constexpr int E = D / 16;  // doubles per lane
    constexpr int kSteps = 8;
    const int part = lane & 15, sub4 = lane >> 4;
    double qr[E];
#pragma unroll
    for (int e = 0; e < E; ++e) qr[e] = qv[part * E + e];
    const double sc = (double)g.scale;
    for (int jb0 = 4 * w; jb0 < nk; jb0 += 16 * kSteps) {
      double2 kk[kSteps][E / 2];
#pragma unroll
      for (int t = 0; t < kSteps; ++t) {
        const int j = jb0 + 16 * t + sub4;
        const double2* kj = reinterpret_cast<const double2*>(kbar_bh + (int64_t)min(j, nk - 1) * D + part * E);
#pragma unroll
        for (int e = 0; e < E / 2; ++e) kk[t][e] = kj[e];
      }
#pragma unroll
      for (int t = 0; t < kSteps; ++t) {
        const int j = jb0 + 16 * t + sub4;
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < E / 2; ++e) {
          s = __builtin_fma(qr[2 * e], kk[t][e].x, s);
          s = __builtin_fma(qr[2 * e + 1], kk[t][e].y, s);
        }
        s += __shfl_xor(s, 8, 16);
        s += __shfl_xor(s, 4, 16);
        s += __shfl_xor(s, 2, 16);
        s += __shfl_xor(s, 1, 16);
        if (part == 0 && j < nk) av[j] = s * sc + (j == nk - 1 ? ln_last : ln_c);
      }
    }
  }
  __syncthreads();
  // Running maximum in index order: thread t owns blocks [t*per, t*per + per).
  const int per = (nk + 255) / 256, j0 = tid * per, j1 = min(nk, j0 + per);
  double m = -__builtin_huge_val();
  for (int j = j0; j < j1; ++j) m = __builtin_fmax(m, av[j]);
  double incl = m;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o, 64);
    if (lane >= o) incl = __builtin_fmax(incl, y);
  }
  double run = __shfl_up(incl, 1, 64);
  if (lane == 0) run = -__builtin_huge_val();
  if (lane == 63) s_wmax[w] = incl;
  __syncthreads();
  for (int ww = 0; ww < w; ++ww) run = __builtin_fmax(run, s_wmax[ww]);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) {
    run = __builtin_fmax(run, av[j]);
    const bool keep = av[j] >= ln_t + run;
    kf[j] = keep ? 1 : 0;
    cnt += keep ? 1 : 0;
  }
  // Exclusive scan of the counts in thread order: the list stays ascending.
  int ci = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(ci, o, 64);
    if (lane >= o) ci += y;
  }
  if (lane == 63) s_wcnt[w] = ci;
  __syncthreads();
  int off = ci - cnt, total = 0;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    const int c = s_wcnt[ww];
    if (ww < w) off += c;
    total += c;
  }
  for (int j = j0; j < j1; ++j)
    if (kf[j]) list[off++] = j;
  if (mask_row) {
    for (int x = tid; x < (nk + 31) / 32; x += 256) {
      uint32_t word = 0;
      for (int b = 0; b < 32 && 32 * x + b < nk; ++b) word |= (uint32_t)kf[32 * x + b] << b;
      mask_row[x] = word;
    }
  }
  __syncthreads();  // the list is complete, and the scratch free again
  return total;
}

// Workgroup: 4 waves (one per SIMD), one per key group.  Wave kw keeps the
// running state of all 64 queries of the tile (4 query tiles of 16: every
// K and V operand feeds four MFMAs) over the chunks kw, kw+4, kw+8, ... of
// the row; the four key groups are merged through LDS at the end.  (With 32
// queries per wave two waves fit a SIMD, but each K/V chunk is then read by
// two waves and the texture path saturates: measured slower.)
//
// kInPass: the row's blocks are not given but chosen inside this kernel by
// on-the-fly thresholding (inpass_list) into an LDS list; rows run in index
// order (their budgets are not known beforehand).
template <int D, bool kInPass>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(
    const Geom g, const __bf16* __restrict__ Q, const __bf16* __restrict__ Kp, const __bf16* __restrict__ Vp,
    int nch, const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const int32_t* __restrict__ order, void* O, int o_bf16, const double* __restrict__ qbar,
    const double* __restrict__ kbar, const InPass ip, int32_t* __restrict__ kept_count,
    uint32_t* __restrict__ kept_mask, int32_t* __restrict__ list_ws) {
  constexpr int DC = D / 32, DT = D / 16, kQT = 4;
  constexpr int LD = D + 4;   // merge slot row stride (floats)
  extern __shared__ float lds[];  // merge slots [4][64][LD] f32, maxima [4][64], row sums [4][64]; in-pass list [nk]
  const int qhalves = g.R / 64;
  const int tix = xcd_block_task(blockIdx.x, gridDim.x);
  const int ridx = tix / qhalves, qsub = tix - ridx * qhalves;
  const int row = (!kInPass && order) ? order[ridx] : ridx;
  const int bh = row / g.nq, i = row - bh * g.nq;
  const int b = bh / g.H, h = bh - b * g.H;
  const int lane = threadIdx.x & 63, kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const __bf16* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const __bf16* Kbh = Kp + (int64_t)bh * nch * (32 * D);
  const __bf16* Vbh = Vp + (int64_t)bh * nch * (32 * D);
  const int row0 = i * g.R + qsub * 64;

  // Q as the B operand of S^T = K Q^T, held in registers for the whole row
  // (padding rows -> 0).
  bf16x8 qop[kQT][DC];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qrow = row0 + qt * 16 + lr;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      bf16x8 v = load_bf16x8(Qbh + (int64_t)qrow * g.qs[2] + dc * 32 + lg * 8);
      if (qrow >= g.N) v = bf16x8{};
      asm("" : "+a"(v));  // only matrix instructions read Q: keep it in AGPRs (waits once, per row)
      qop[qt][dc] = v;
    }
  }

  f32x4 o[DT][kQT];
  float m[kQT], l[kQT];
  f32x4 lsum[kQT];  // row sums from the matrix cores (see pv)
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    m[qt] = kNegInf;
    l[qt] = 0.f;
    lsum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const float c = g.scale_log2;
  int beg, end;
  int32_t* list = reinterpret_cast<int32_t*>(lds + 4 * 64 * LD + 512);  // in-pass kept blocks
  const int32_t* lst;  // the row's list: block lst[p] at position p in [0, end - beg)
  if constexpr (kInPass) {
    const double ln_t = ip.ln_theta[ip.per_head ? h : 0];
    uint32_t* mask_row = (kept_mask && qsub == 0) ? kept_mask + (int64_t)row * ((g.nk + 31) / 32) : nullptr;
    const int n = inpass_list<D>(g, qbar + (int64_t)row * D, kbar + (int64_t)bh * g.nk * D, ln_t, ip.ln_c,
                                 ip.ln_last, reinterpret_cast<double*>(lds), list, mask_row);
    if (kept_count && qsub == 0 && threadIdx.x == 0) kept_count[row] = n;
    // The loop reads the list from this task's slot in global memory, as it
    // reads a CSR row: read from LDS, the compiler scheduled the loop's
    // operand loads so that every trip waited for all of them (the in-pass
    // call took 15-23% longer than the sparse attention on the same blocks;
    // 3-14% of it is recovered this way).
    int32_t* gl = list_ws + (int64_t)tix * g.nk;
    for (int x = threadIdx.x; x < n; x += 256) gl[x] = list[x];
    __syncthreads();  // the whole list is written before any wave reads it
    beg = 0;
    end = n;
    lst = gl;
  } else {
    beg = row_ptr[row];
    end = row_ptr[row + 1];
    lst = col_idx + beg;
  }
  // Block at position p of the row's list.
  auto list_at = [&](int p) -> int { return lst[p]; };
  const int sub = g.C / 32;
  const int nchunk = (end - beg) * sub;

  auto chunk_key = [&](int u) -> int {
    const int p = u / sub;
    return list_at(p) * g.C + (u - p * sub) * 32;
  };
  // Operand loads from the packed copies: 64 lanes x 16 contiguous bytes each.
  auto load_k = [&](int kb, bf16x8 (&kop)[2][DC]) {
    const __bf16* kc = Kbh + (int64_t)(kb >> 5) * (32 * D) + lane * 8;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) kop[kt][dc] = load_bf16x8(kc + (kt * DC + dc) * 512);
  };
  auto load_v = [&](int kb, bf16x8 (&vop)[DT]) {
    const __bf16* vc = Vbh + (int64_t)(kb >> 5) * (32 * D) + lane * 8;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vop[dt] = load_bf16x8(vc + dt * 512);
  };
  // S^T for one chunk: acc[kt][qt][r] = score of key kb + 8*lg + 4*kt + r for
  // query qt*16 + lr.
  auto scores = [&](const bf16x8 (&kop)[2][DC], f32x4 (&acc)[2][kQT]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) acc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)  // each K operand's four uses back to back
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) acc[kt][qt] = mfma_bf16(kop[kt][dc], qop[qt][dc], acc[kt][qt]);
    }
  };
  // Padding keys of the last block's tail leave the softmax.
  auto mask_tail = [&](int kb, f32x4 (&acc)[2][kQT]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool dead = kb + lg * 8 + kt * 4 + r >= g.N;
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt)
          if (dead) acc[kt][qt][r] = kNegInf;
      }
  };
  // Probabilities p = 2^(s*c - m) against the wave's fixed reference m, packed
  // to bf16 (the row sums are taken from these packed values by pv).
  auto probs = [&](const f32x4 (&acc)[2][kQT], bf16x8 (&pop)[kQT]) {
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      const float nm = -m[qt];
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(acc[e >> 2][qt][e & 3], c, nm));
      pop[qt] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
    }
  };
  auto chunk_max = [&](const f32x4 (&acc)[2][kQT], float (&mx)[kQT]) {
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      float t = mx[qt];
#pragma unroll
      for (int e = 0; e < 8; ++e) t = fmaxf(t, acc[e >> 2][qt][e & 3]);
      mx[qt] = t;
    }
  };
  auto lanes_max = [&](float (&mx)[kQT]) {
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      mx[qt] = rows_max(mx[qt]);
    }
  };
  // O^T += V^T P^T, and the row sums: a block of ones as the A operand makes
  // every row of lsum[qt] the column sums of P^T, so each lane holds the full
  // sum of its query over the wave's chunks (element 0 is used).
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  auto pv = [&](const bf16x8 (&vop)[DT], const bf16x8 (&pop)[kQT]) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) o[dt][qt] = mfma_bf16(vop[dt], pop[qt], o[dt][qt]);
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) lsum[qt] = mfma_bf16(ones, pop[qt], lsum[qt]);
  };

  auto scores_qt = [&](const bf16x8 (&kop)[2][DC], int qt, f32x4 (&acc)[2][kQT]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      acc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) acc[kt][qt] = mfma_bf16(kop[kt][dc], qop[qt][dc], acc[kt][qt]);
    }
  };
  auto probs_qt = [&](const f32x4 (&acc)[2][kQT], int qt, bf16x8& pq) {
    const float nm = -m[qt];
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(acc[e >> 2][qt][e & 3], c, nm));
    pq = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
  };
  auto pv_qt = [&](const bf16x8 (&vop)[DT], int qt, const bf16x8& pq) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][qt] = mfma_bf16(vop[dt], pq, o[dt][qt]);
    lsum[qt] = mfma_bf16(ones, pq, lsum[qt]);
  };

  // No maximum is tracked per score and O is never rescaled inside the loop:
  // the reference m is fixed at the wave's first chunk's maximum plus
  // kHeadroom (log2 units).  Later chunks may exceed the first chunk's
  // maximum by up to kHeadroom + 100 - log2(their count) before the row sum
  // passes kLBound; terms more than ~60 below the maximum are negligible
  // either way.  If the row sum passes kLBound or is not finite (an
  // overflow, a reference that is not finite, or a NaN input) the wave, once
  // through its chunks, drops its partial sums and recomputes them in two
  // passes (exact maximum first), so all probabilities are <= 1.  The loop
  // has a single exit: an early exit makes the register allocator shuffle the
  // O accumulators on every trip.
  //
  // Software pipeline: iteration t takes the query tiles in turn -- the
  // softmax of chunk t, the score MFMAs of chunk t+1 into the same
  // accumulators, P.V of chunk t -- in the compiler's own interleaving
  // (asking it to alternate one MFMA with one or two vector instructions
  // measured 3.5% and 6% slower on the HunyuanVideo 720p layer, and no
  // faster elsewhere; all scores of chunk t+1 into a second buffer, copied
  // back each trip, 0.8% slower there).  K of chunk t+2 and V of chunk t+1
  // are requested once the iteration's MFMAs have read K and V.
  //
  // Padding keys of the last block score exactly 0 against the zero rows of
  // the packed K, which can lie far above every real score of a row, so they
  // must leave the softmax; the loop itself does no masking.  With C <= 128 a
  // wave owns at most one 32-key chunk of the last block: a partly padded one
  // is moved to the front of the wave's sequence (the first chunk is masked
  // explicitly), a wholly padded one is dropped.  Indices within a row are
  // distinct, so the last block occurs at most once.
  constexpr float kHeadroom = 64.0f;
  int nmine = nchunk > kw ? (nchunk - kw + 3) / 4 : 0;
  int swap_a = 0, swap_b = 0;  // positions exchanged in the wave's chunk sequence
  if (g.N != g.nk * g.C && nmine > 0) {
    const int n = end - beg;
    int pos = -1;  // position of the last block in the row's list
    for (int base = 0; base < n; base += 4 * kWave) {
      uint64_t hit[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int x = base + j * kWave + lane;
        hit[j] = __ballot(x < n && list_at(x) == g.nk - 1);
      }
#pragma unroll
      for (int j = 3; j >= 0; --j)
        if (hit[j]) pos = base + j * kWave + __builtin_ctzll(hit[j]);
      if (pos >= 0) break;
    }
    if (pos >= 0) {
      for (int s = 0; s < sub; ++s) {
        const int u = pos * sub + s;
        if ((u & 3) != kw) continue;
        const int key0 = (g.nk - 1) * g.C + 32 * s, t = u >> 2;
        if (key0 >= g.N) {             // wholly padding: move it last and drop it
          swap_a = t;
          swap_b = nmine - 1;
          --nmine;
        } else if (key0 + 32 > g.N) {  // partly padding: move it first
          swap_b = t;
        }
      }
    }
  }
  auto key_of = [&](int t) {
    t = t < nmine ? t : nmine - 1;
    t = t == swap_a ? swap_b : (t == swap_b ? swap_a : t);
    return chunk_key(kw + 4 * t);
  };
  // The loop reads its chunk keys from registers: lane j of a window holds
  // key_of(base + j), so a key costs one lane read instead of a dependent
  // scalar load of col_idx.  Two windows cover 128 chunks; the next one is
  // loaded 64 iterations before it is needed.
  const int sub_shift = __builtin_ctz(sub);
  auto key_window = [&](int base) -> int {
    int t = base + lane;
    t = t < nmine ? t : nmine - 1;
    t = t == swap_a ? swap_b : (t == swap_b ? swap_a : t);
    const int u = kw + 4 * t, p = u >> sub_shift;
    return list_at(p) * g.C + (u - (p << sub_shift)) * 32;
  };
  bool fallback = false;
  bf16x8 kop[2][DC], vop[DT];
  if (nmine > 0) {
    int kb = key_of(0);
    load_k(kb, kop);
    load_v(kb, vop);
    f32x4 acc[2][kQT];
    scores(kop, acc);
    load_k(key_of(1), kop);
    if (kb + 32 > g.N) mask_tail(kb, acc);
    {
      float mx[kQT];
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) mx[qt] = kNegInf;
      chunk_max(acc, mx);
      lanes_max(mx);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) m[qt] = mx[qt] * c + kHeadroom;  // -inf: forces the fallback
    }
    bool over_any = false;
    int win_base = 0;
    int win0 = key_window(0), win1 = key_window(64);
    for (int t = 0; t < nmine; ++t) {
      if (t == win_base + 64) {  // keys t+1, t+2 now lie in [win_base + 64, win_base + 128)
        win_base += 64;
        win0 = win1;
        win1 = key_window(win_base + 64);
      }
      auto key_at = [&](int i) {  // both lanes read, then a select: no branch inside the body
        const int r = i - win_base;
        const int k0 = __builtin_amdgcn_readlane(win0, r & 63), k1 = __builtin_amdgcn_readlane(win1, r & 63);
        return r < 64 ? k0 : k1;
      };
      // per query tile: the softmax of chunk t, the scores of chunk t+1 into
      // the registers just read (the last iteration recomputes the last
      // chunk), P.V of chunk t -- no second score buffer and no copies
      bf16x8 pop[kQT];
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) {
        probs_qt(acc, qt, pop[qt]);
        scores_qt(kop, qt, acc);
        pv_qt(vop, qt, pop[qt]);
      }
      load_k(key_at(t + 2), kop);
      load_v(key_at(t + 1), vop);
    }
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) over_any |= !(lsum[qt][0] <= kLBound);
    fallback = __any(over_any);
  }
  if (fallback) {
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      lsum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[qt] = kNegInf;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int t = 0; t < nmine; ++t) {
      const int kb2 = key_of(t);
      load_k(kb2, kop);
      f32x4 acc[2][kQT];
      scores(kop, acc);
      if (kb2 + 32 > g.N) mask_tail(kb2, acc);
      chunk_max(acc, m);
    }
    lanes_max(m);
    bool any_key = false;
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      any_key |= m[qt] != kNegInf;
      m[qt] *= c;
    }
    if (__any(any_key)) {  // a key row is common to all queries, so the maxima are all finite
      for (int t = 0; t < nmine; ++t) {
        const int kb2 = key_of(t);
        load_k(kb2, kop);
        load_v(kb2, vop);
        f32x4 acc[2][kQT];
        scores(kop, acc);
        if (kb2 + 32 > g.N) mask_tail(kb2, acc);
        bf16x8 pop[kQT];
        probs(acc, pop);
        pv(vop, pop);
      }
    }
  }

  // Row sums: every lane already holds its query's sum over the wave's chunks.
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) l[qt] = lsum[qt][0];

  // Merge the four key groups in one step: every wave parks its partial O,
  // maxima and row sums in its own LDS slot, then wave kw combines dims
  // [kw*D/4, (kw+1)*D/4) of all 64 queries from the four slots and stores
  // them (a chain of three pairwise merges through one slot took ~5 us per
  // workgroup, measured with one-block lists).
  constexpr int DTW = DT / 4;  // dim tiles merged and stored per wave
  float* slot = lds + kw * (64 * LD);
  float* sm = lds + 4 * 64 * LD;  // [4][64] maxima
  float* sl = sm + 4 * 64;        // [4][64] row sums
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qi = qt * 16 + lr;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(slot + qi * LD + dt * 16 + lg * 4) = o[dt][qt];
    if (lg == 0) {
      sm[kw * 64 + qi] = m[qt];
      sl[kw * 64 + qi] = l[qt];
    }
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qi = qt * 16 + lr;
    float mw[4], a[4], mm = kNegInf, lt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = sm[w * 64 + qi];
      mm = fmaxf(mm, mw[w]);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      a[w] = mw[w] == kNegInf ? 0.f : fast_exp2(mw[w] - mm);
      lt += a[w] * sl[w * 64 + qi];
    }
    const int qrow = row0 + qi;
    const float inv = (qrow < g.N && lt > 0.f) ? 1.0f / lt : 0.f;
    const int64_t obase = b * g.os[0] + h * g.os[1] + (int64_t)qrow * g.os[2];
#pragma unroll
    for (int dd = 0; dd < DTW; ++dd) {
      const int dt = kw * DTW + dd;
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w)
        v += *reinterpret_cast<const f32x4*>(lds + w * (64 * LD) + qi * LD + dt * 16 + lg * 4) * a[w];
      v *= inv;
      const int d0 = dt * 16 + lg * 4;
      if (o_bf16) {
        u32x2 pk;
        pk[0] = pack_bf16x2(v[0], v[1]);
        pk[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(O) + obase + d0) = pk;
      } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(O) + obase + d0) = v;
      }
    }
  }
}

// ------------------------------------------------------------------ SIMT path
// One thread per query row (R threads per workgroup), K and V tiles of 32
// keys staged through LDS, fp32 arithmetic.
template <typename T, int D>
__global__ __launch_bounds__(128) void attn_simt_kernel(const Geom g, const T* __restrict__ Q,
                                                        const T* __restrict__ K, const T* __restrict__ V,
                                                        const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ col_idx,
                                                        const int32_t* __restrict__ order, void* O,
                                                        int o_bf16) {
  const int ridx = blockIdx.x;
  const int row = order ? order[ridx] : ridx;
  const int bh = row / g.nq, i = row - bh * g.nq;
  const int b = bh / g.H, h = bh - b * g.H;
  const int qrow = i * g.R + threadIdx.x;
  const bool valid = qrow < g.N;
  const T* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const T* Kbh = K + b * g.ks[0] + h * g.ks[1];
  const T* Vbh = V + b * g.vs[0] + h * g.vs[1];
  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? (float)Qbh[(int64_t)qrow * g.qs[2] + d] : 0.f;
    o[d] = 0.f;
  }
  __shared__ float ks[32][D], vs[32][D];
  float m = kNegInf, l = 0.f;
  const float c = g.scale_log2;
  // no lists: every key block (dense attention)
  const int beg = row_ptr ? row_ptr[row] : 0, end = row_ptr ? row_ptr[row + 1] : g.nk;
  for (int p = beg; p < end; ++p) {
    const int j = col_idx ? col_idx[p] : p;
    const int kend = min((j + 1) * g.C, g.N);
    for (int kb = j * g.C; kb < kend; kb += 32) {
      for (int idx = threadIdx.x; idx < 32 * D; idx += blockDim.x) {
        const int kk = idx / D, d = idx - kk * D;
        const bool in = kb + kk < kend;
        ks[kk][d] = in ? (float)Kbh[(int64_t)(kb + kk) * g.ks[2] + d] : 0.f;
        vs[kk][d] = in ? (float)Vbh[(int64_t)(kb + kk) * g.vs[2] + d] : 0.f;
      }
      __syncthreads();
      const int nkk = min(32, kend - kb);
      for (int kk = 0; kk < nkk; ++kk) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(q[d], ks[kk][d], dot);
        const float x = dot * c;
        const float mn = fmaxf(m, x);
        const float a = fast_exp2(m - mn);
        const float pe = fast_exp2(x - mn);
        l = l * a + pe;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], a, pe * vs[kk][d]);
        m = mn;
      }
      __syncthreads();
    }
  }
  const float inv = (valid && l > 0.f) ? 1.0f / l : 0.f;
  const int64_t obase = b * g.os[0] + h * g.os[1] + (int64_t)qrow * g.os[2];
  if (o_bf16) {
    __bf16* Ob = reinterpret_cast<__bf16*>(O) + obase;
#pragma unroll
    for (int d = 0; d < D; ++d) Ob[d] = (__bf16)(o[d] * inv);
  } else {
    float* Of = reinterpret_cast<float*>(O) + obase;
#pragma unroll
    for (int d = 0; d < D; ++d) Of[d] = o[d] * inv;
  }
}

int vt_chunks(const Geom& g) { return packed_chunks(g); }

template <int D>
hipError_t launch_mfma(const Geom& g, const void* Q, const void* K, const void* V, const int32_t* row_ptr,
                       const int32_t* col_idx, const int32_t* order, void* O, int o_bf16, void* ws,
                       hipStream_t st) {
  const int nch = vt_chunks(g);
  __bf16* Kp = reinterpret_cast<__bf16*>(ws);
  __bf16* Vp = Kp + (size_t)g.B * g.H * nch * 32 * D;
  hipLaunchKernelGGL((pack_kv_kernel<D, true>), dim3((unsigned)(nch / 2), g.B * g.H), dim3(256), 0, st, g,
                     (const __bf16*)K, (const __bf16*)V, Kp, Vp, nch);
  const size_t lds = (size_t)(4 * 64 * (D + 4) + 512) * sizeof(float);  // 137 KB at d = 128
  InPass none;
  none.per_head = 0;
  hipLaunchKernelGGL((attn_bf16_kernel<D, false>), dim3(g.rows() * (g.R / 64)), dim3(256), lds, st,
                     g, (const __bf16*)Q, (const __bf16*)Kp, (const __bf16*)Vp, nch, row_ptr, col_idx, order, O,
                     o_bf16, (const double*)nullptr, (const double*)nullptr, none, (int32_t*)nullptr,
                     (uint32_t*)nullptr, (int32_t*)nullptr);
  return hipGetLastError();
}

// Bytes of the fp64 block means of Q [B*H*nq][D] and of K [B*H*nk][D].
size_t means_bytes(const Geom& g) {
  return align_up((size_t)g.B * g.H * g.nq * g.D * sizeof(double), 256) +
         align_up((size_t)g.B * g.H * g.nk * g.D * sizeof(double), 256);
}

template <int D>
hipError_t launch_inpass(const Geom& g, const void* Q, const void* K, const void* V, const InPass& ip, void* O,
                         int o_bf16, int32_t* kept_count, uint32_t* kept_mask, void* ws, hipStream_t st) {
  char* base = reinterpret_cast<char*>(ws);
  double* qbar = reinterpret_cast<double*>(base);
  double* kbar = reinterpret_cast<double*>(base + align_up((size_t)g.B * g.H * g.nq * g.D * sizeof(double), 256));
  launch_block_means64(g, Q, K, qbar, kbar, st);
  int32_t* list_ws = reinterpret_cast<int32_t*>(base + means_bytes(g) + attn_ws_bytes(g));
  const int nch = vt_chunks(g);
  __bf16* Kp = reinterpret_cast<__bf16*>(base + means_bytes(g));
  __bf16* Vp = Kp + (size_t)g.B * g.H * nch * 32 * D;
  hipLaunchKernelGGL((pack_kv_kernel<D, true>), dim3((unsigned)(nch / 2), g.B * g.H), dim3(256), 0, st, g,
                     (const __bf16*)K, (const __bf16*)V, Kp, Vp, nch);
  // merge slots, maxima and row sums, then the kept-block list (153 KB at d = 128, n_k = 4096)
  const size_t lds = (size_t)(4 * 64 * (D + 4) + 512) * sizeof(float) + (size_t)g.nk * sizeof(int32_t);
  hipLaunchKernelGGL((attn_bf16_kernel<D, true>), dim3(g.rows() * (g.R / 64)), dim3(256), lds, st, g,
                     (const __bf16*)Q, (const __bf16*)Kp, (const __bf16*)Vp, nch, (const int32_t*)nullptr,
                     (const int32_t*)nullptr, (const int32_t*)nullptr, O, o_bf16, (const double*)qbar,
                     (const double*)kbar, ip, kept_count, kept_mask, list_ws);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_simt(const Geom& g, const void* Q, const void* K, const void* V, const int32_t* row_ptr,
                       const int32_t* col_idx, const int32_t* order, void* O, int o_bf16, hipStream_t st) {
  hipLaunchKernelGGL((attn_simt_kernel<T, D>), dim3(g.rows()), dim3(g.R), 0, st, g, (const T*)Q, (const T*)K,
                     (const T*)V, row_ptr, col_idx, order, O, o_bf16);
  return hipGetLastError();
}

}  // namespace

size_t attn_ws_bytes(const Geom& g) {
  if (!mfma_path(g)) return 0;
  return 2 * (size_t)g.B * g.H * g.D * (size_t)vt_chunks(g) * 32 * sizeof(uint16_t);  // packed K and V
}

// In-pass thresholding workspace: the block means, the packed K and V, then
// one list slot of n_k int32 per task (workgroup).
size_t attn_threshold_ws_bytes(const Geom& g) {
  return means_bytes(g) + attn_ws_bytes(g) + (size_t)g.rows() * (g.R / 64) * g.nk * sizeof(int32_t);
}

hipError_t launch_sparse_attn_threshold(const Geom& g, const void* Q, const void* K, const void* V, const InPass& ip,
                                        void* O, int o_bf16, int32_t* kept_count, uint32_t* kept_mask, void* ws,
                                        hipStream_t stream) {
  return g.D == 128 ? launch_inpass<128>(g, Q, K, V, ip, O, o_bf16, kept_count, kept_mask, ws, stream)
                    : launch_inpass<64>(g, Q, K, V, ip, O, o_bf16, kept_count, kept_mask, ws, stream);
}

hipError_t launch_sparse_attn(const Geom& g, const void* Q, const void* K, const void* V,
                              const int32_t* row_ptr, const int32_t* col_idx, const int32_t* order,
                              void* O, int o_bf16, void* ws, hipStream_t stream) {
  if (mfma_path(g))
    return g.D == 128 ? launch_mfma<128>(g, Q, K, V, row_ptr, col_idx, order, O, o_bf16, ws, stream)
                      : launch_mfma<64>(g, Q, K, V, row_ptr, col_idx, order, O, o_bf16, ws, stream);
  if (g.bf16)
    return g.D == 128 ? launch_simt<__bf16, 128>(g, Q, K, V, row_ptr, col_idx, order, O, o_bf16, stream)
                      : launch_simt<__bf16, 64>(g, Q, K, V, row_ptr, col_idx, order, O, o_bf16, stream);
  return g.D == 128 ? launch_simt<float, 128>(g, Q, K, V, row_ptr, col_idx, order, O, o_bf16, stream)
                    : launch_simt<float, 64>(g, Q, K, V, row_ptr, col_idx, order, O, o_bf16, stream);
}

}  // namespace losa
