// Exact block attention masses (LoSA page, Motivation Summary: block
// attention mass; Methodology Summary: masses at the construction step are
// exact, not estimated).
//
//   M[b,h,i,j] = (1/valid rows of block i) * sum over rows q of block i and
//                valid keys k of block j of exp(s_qk - lse_q),
// with s = q.k * scale and lse_q the log-sum-exp of row q over all valid keys.
//
// bf16 matrix-core path (d in {64, 128}, R in {64, 128}): ONE pass over K.
// A workgroup holds two query groups of 64 rows (the halves of one 128-row
// block, or two neighbouring 64-row blocks of one head), two waves each; the
// two waves of a group split the KEY BLOCKS (wave w takes blocks j = w,
// w+2, ...).  For every query the group fixes one reference m, the largest
// score of its waves' first chunks (log2 units; scores are pre-multiplied by
// scale*log2(e)); each wave sums 2^(s*c - m) per key block, writes that
// per-(query, block) sum to a workspace S and keeps the row total.  Once
// the two waves' totals are added, the group reads S back:
//   M[i,j] = (1/rows) * sum_q S[q,j] / total_q
// (for a 128-row block, the two halves' sums over their rows added first).
// The scores and exponentials are computed once (a two-pass form computes
// both twice); S costs 4 bytes per (query row, key block) of HBM traffic each
// way.  S^T = K Q^T is formed with 16x16x32 bf16 MFMA: lane l owns query
// (l & 15) of each 16-query tile and 4 keys per 16-key tile.
//
// fp32 inputs (and bf16 shapes outside the matrix-core path) take a SIMT
// two-pass path: row maximum and sum first, then the block sums.
#include "losa_blocksum.hpp"
#include "losa_device.hpp"
#include "losa_internal.hpp"
#include "losa_pack.hpp"

namespace losa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// ------------------------------------------------------------------ bf16 MFMA

template <int D>
struct QTile {
  static constexpr int DC = D / 32;
  bf16x8 op[4][DC];  // B operand: 4 query tiles of 16 rows x D

  // Rows at or beyond n_valid are padding and may hold anything: they are
  // replaced by zeros so that no non-finite value reaches a reduction.
  __device__ __forceinline__ void load(const __bf16* Qbh, int64_t ts, int row0, int n_valid, int lr, int lg) {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const int row = row0 + qt * 16 + lr;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        bf16x8 v = load_bf16x8(Qbh + (int64_t)row * ts + dc * 32 + lg * 8);
        if (row >= n_valid) v = bf16x8{};
        op[qt][dc] = v;
      }
    }
  }
};

// K operand of one 32-key chunk from the packed copy (64 lanes x 16
// contiguous bytes per load).  acc[kt][qt][r] then holds the score of key
// kb + 8*lg + 4*kt + r (the packed row order) for query qt*16 + lr.
template <int D>
__device__ __forceinline__ void load_kchunk(const __bf16* Kpbh, int kb, int lane, bf16x8 (&kop)[2][D / 32]) {
  constexpr int DC = D / 32;
  const __bf16* kc = Kpbh + (int64_t)(kb >> 5) * (32 * D) + lane * 8;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kop[kt][dc] = load_bf16x8(kc + (kt * DC + dc) * 512);
}

template <int D>
__device__ __forceinline__ void chunk_scores(const QTile<D>& q, const bf16x8 (&kop)[2][D / 32], f32x4 (&acc)[2][4]) {
  constexpr int DC = D / 32;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) a = mfma_bf16(kop[kt][dc], q.op[qt][dc], a);
      acc[kt][qt] = a;
    }
}

__device__ __forceinline__ void mask_tail(int kb, int n_valid, int lg, f32x4 (&acc)[2][4]) {
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool dead = kb + lg * 8 + kt * 4 + r >= n_valid;
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
        if (dead) acc[kt][qt][r] = kNegInf;
    }
}

// Grid: workgroups of 256 threads (four waves), three per CU (151
// registers: three waves per SIMD).  A workgroup holds two query groups of
// 64 rows, two waves each; the two waves of a group split the key blocks
// (wave kw takes blocks kw, kw + 2, ...), so both groups read every K chunk
// side by side on one CU.  R = 128: the groups are the halves of one query
// block (B*H*nq workgroups) and their partial masses are added in LDS.
// R = 64 (kPair): the groups are two neighbouring query blocks of one head
// (B*H*ceil(nq/2) workgroups), each writing its own row of M.  (Eight waves
// for R = 128, four per group, leave room for one workgroup per CU: two
// waves per SIMD; one workgroup per group streams every K chunk to two CUs,
// twice the traffic beyond L2.)
//
// Reference.  The two waves of a query group share one reference per query:
// the largest score of their first chunks, exchanged through LDS before the
// sweep (no headroom).  It is an actual score of the row, so it is at most
// the row's log-sum-exp: every term 2^(s*c - m) is at least the probability
// it stands for.  A key whose probability is a normal fp32 number (>= 2^-126)
// therefore never lands in the range the exponential flushes to zero, and the
// masses keep fp32's relative precision down to that range; only keys of
// probability below 2^-126 may be lost, at most C * 2^-126 per mass.  With
// one reference per query the row total is a plain sum over the waves and the
// per-query factor is 1 / total: no exponential of a reference difference,
// which could itself flush when the waves' first chunks differ widely.
//
// A term can only exceed 1 when a later score exceeds the first chunks'
// maximum; if a block sum or a row total leaves [0, 2^100] (a score ~83 above
// it; or a non-finite input), the whole workgroup recomputes against the
// exact maximum of the row (every term <= 1), overwriting its S entries.
template <int D, bool kPair>
__global__ __launch_bounds__(256, 2) void mass_bf16_kernel(const Geom g, const __bf16* __restrict__ Q,
                                                           const __bf16* __restrict__ Kp, int nch,
                                                           float* __restrict__ S, float* __restrict__ M) {
  constexpr int QG = 2, WPG = 2;              // query groups, waves per group
  constexpr float kSumBound = 1.2676506e30f;  // 2^100
  __shared__ float s_ref[QG][WPG][64], s_tot[QG][WPG][64], s_f[QG][WPG][64];
  __shared__ int s_over;
  extern __shared__ float part[];  // [QG][nk] the halves' partial masses (R = 128)
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = w / WPG, kw = w - grp * WPG;
  const int lr = lane & 15, lg = lane >> 4;
  // row: the query block whose row of M (and, with kPair, S) this group
  // serves; i: its index in the head; valid: false for the missing second
  // block of a head with odd n_q (its waves do no work).
  int row, bh, i;
  bool valid = true;
  if constexpr (kPair) {
    const int nq2 = (g.nq + 1) >> 1;
    const int task = xcd_task(blockIdx.x, g.B * g.H * nq2);
    bh = task / nq2;
    i = 2 * (task - bh * nq2) + grp;
    valid = i < g.nq;
    row = bh * g.nq + i;
  } else {
    row = xcd_task(blockIdx.x, g.B * g.H * g.nq);
    bh = row / g.nq;
    i = row - bh * g.nq;
  }
  const int b = bh / g.H, h = bh - b * g.H;
  const __bf16* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const __bf16* Kpbh = Kp + (int64_t)bh * nch * (32 * D);
  const int row0 = kPair ? i * g.R : i * g.R + grp * 64;
  // [nk][64] of this query group
  float* Sg = S + (kPair ? (int64_t)row : (int64_t)row * QG + grp) * g.nk * 64;

  QTile<D> q;
  // A missing block reads rows 0..63 (allocated for every head) as padding:
  // all of them zero, no access beyond n_q * R.
  q.load(Qbh, g.qs[2], valid ? row0 : 0, valid ? g.N : 0, lr, lg);

  const float c = g.scale_log2;
  const int sub = g.C / 32, sub_shift = __builtin_ctz(sub);
  const int nb = valid && g.nk > kw ? (g.nk - kw + WPG - 1) / WPG : 0;  // my key blocks kw, kw+WPG, ...
  const int nu = nb * sub;                                      // their 32-key chunks
  auto chunk_kb = [&](int u) { return (kw + WPG * (u >> sub_shift)) * g.C + 32 * (u & (sub - 1)); };

  // Block sums: lane (lg, lr) holds partial sums over its keys for queries
  // qt*16 + lr, qt = 0..3; the totals over the four lane groups are formed so
  // that lane (lg, lr) ends with the one for query lg*16 + lr (the one it
  // stores): two values swapped with the lane 32 away, then one with the lane
  // 16 away.
  auto reduce_mine = [&](const float (&v)[4]) -> float { return rows_sum_own(v); };
  // The query group's common reference for the queries of this lane's four
  // tiles, from its waves' entries in s_ref (scaled, log2 units).
  float m[4];
  auto common_ref = [&]() {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      float mm = s_ref[grp][0][qt * 16 + lr];
#pragma unroll
      for (int ww = 1; ww < WPG; ++ww) mm = fmaxf(mm, s_ref[grp][ww][qt * 16 + lr]);
      m[qt] = mm;
    }
  };
  auto publish_ref = [&](const float (&mx)[4]) {  // lane (lg, lr) holds query lg*16 + lr's entry
    s_ref[grp][kw][lane] = (lg == 0 ? mx[0] : lg == 1 ? mx[1] : lg == 2 ? mx[2] : mx[3]) * c;
  };

  // One sweep over my chunks against m (acc0: the scores of chunk 0 when
  // have0).  tot = this lane's query's total.  Returns whether some sum left
  // [0, 2^100].
  float tot;
  bool over;
  float blk[4];
  auto consume = [&](const f32x4 (&acc)[2][4], int u) {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const float nm = -m[qt];
      // Seeded with the first term rather than 0 (0 + x is not folded, since
      // it would differ for x = -0): four fewer additions per chunk, the same
      // sums (no term is -0).
      float sum = fast_exp2(__builtin_fmaf(acc[0][qt][0], c, nm));
#pragma unroll
      for (int e = 1; e < 8; ++e) sum += fast_exp2(__builtin_fmaf(acc[e >> 2][qt][e & 3], c, nm));
      blk[qt] += sum;
    }
    if ((u & (sub - 1)) == sub - 1) {  // block complete: store this lane's query's sum, add it to the total
      const int j = kw + WPG * (u >> sub_shift);
      const float v = reduce_mine(blk);
      tot += v;
      over |= !(v <= kSumBound);
      Sg[(int64_t)j * 64 + lane] = v;  // lane = query lg*16 + lr
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) blk[qt] = 0.f;
    }
  };
  auto sweep = [&](const f32x4 (&acc0)[2][4], bool have0) -> bool {
    over = false;
    tot = 0.f;
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) blk[qt] = 0.f;
    if (have0) consume(acc0, 0);
    const int u0 = have0 ? 1 : 0;
    bf16x8 kop[2][D / 32];
    if (u0 < nu) load_kchunk<D>(Kpbh, chunk_kb(u0), lane, kop);
    for (int u = u0; u < nu; ++u) {
      const int kb = chunk_kb(u);
      f32x4 acc[2][4];
      chunk_scores<D>(q, kop, acc);
      if (u + 1 < nu) load_kchunk<D>(Kpbh, chunk_kb(u + 1), lane, kop);
      if (__builtin_expect(kb + 32 > g.N, 0)) mask_tail(kb, g.N, lg, acc);
      consume(acc, u);
    }
    over |= !(tot <= kSumBound);
    return __any(over);
  };

  // Chunk 0's scores and their maximum per query (-inf for a wave without key
  // blocks), shared through LDS: the common reference.
  f32x4 acc0[2][4];
  {
    float mx[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) mx[qt] = kNegInf;
    if (nu > 0) {
      bf16x8 kop[2][D / 32];
      load_kchunk<D>(Kpbh, chunk_kb(0), lane, kop);
      chunk_scores<D>(q, kop, acc0);
      if (chunk_kb(0) + 32 > g.N) mask_tail(chunk_kb(0), g.N, lg, acc0);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        float t = acc0[0][qt][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) t = fmaxf(t, acc0[e >> 2][qt][e & 3]);
        mx[qt] = rows_max(t);  // finite: a key block's first chunk holds a valid key
      }
    }
    publish_ref(mx);
    if (threadIdx.x == 0) s_over = 0;
  }
  __syncthreads();
  common_ref();
  tot = 0.f;
  if (nu > 0 && sweep(acc0, true) && lane == 0) s_over = 1;
  __syncthreads();
  if (s_over) {
    // Exact maximum of the row (over every wave's keys), then the sums again
    // against it: all terms <= 1.
    float mx[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) mx[qt] = kNegInf;
    bf16x8 kop[2][D / 32];
    for (int u = 0; u < nu; ++u) {
      const int kb = chunk_kb(u);
      load_kchunk<D>(Kpbh, kb, lane, kop);
      f32x4 acc[2][4];
      chunk_scores<D>(q, kop, acc);
      if (kb + 32 > g.N) mask_tail(kb, g.N, lg, acc);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx[qt] = fmaxf(mx[qt], acc[e >> 2][qt][e & 3]);
    }
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) mx[qt] = rows_max(mx[qt]);
    publish_ref(mx);  // every wave read the first references before the barrier above
    __syncthreads();
    common_ref();
    tot = 0.f;
    if (nu > 0) sweep(acc0, false);
  }

  // Row totals: the four key groups' totals against the common reference add
  // up directly; the factor for the query this lane stored is 1 / total (0
  // for padding rows).
  s_tot[grp][kw][lane] = tot;
  __syncthreads();
  float f = 0.f;
  {
    const float l = s_tot[grp][0][lane] + s_tot[grp][1][lane];
    if (row0 + lane < g.N) f = 1.0f / l;
  }
  s_f[grp][kw][lane] = f;
  __syncthreads();  // every lane reads all 64 factors of its wave
  const float inv_rows = valid ? 1.0f / (float)min(g.R, g.N - i * g.R) : 0.f;
  float* Mrow = M + (int64_t)row * g.nk;
  auto block_of = [kw](int bb) { return kw + WPG * bb; };
  if constexpr (kPair) {
    blocks_from_sums(Sg, s_f[grp][kw], nb, inv_rows, Mrow, lane, block_of);  // nothing when !valid (nb = 0)
  } else {
    blocks_from_sums(Sg, s_f[grp][kw], nb, 1.0f, part + grp * g.nk, lane, block_of);
    __syncthreads();
    for (int j = threadIdx.x; j < g.nk; j += blockDim.x) {
      float v = part[j];
#pragma unroll
      for (int gg = 1; gg < QG; ++gg) v += part[gg * g.nk + j];
      Mrow[j] = v * inv_rows;
    }
  }
}

// ------------------------------------------------------------------ SIMT path
// fp32 (or bf16 with shapes the matrix-core kernels do not cover).  One
// thread per query row, K staged through LDS in 32-key tiles.

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

template <typename T, int D>
__global__ __launch_bounds__(64) void lse_simt_kernel(const Geom g, const T* __restrict__ Q,
                                                      const T* __restrict__ K, float2* __restrict__ ml) {
  const int tiles = (g.N + 63) / 64;
  const int task = blockIdx.x;
  const int bh = task / tiles, t = task - bh * tiles;
  const int b = bh / g.H, h = bh - b * g.H;
  const int row = t * 64 + threadIdx.x;
  const bool valid = row < g.N;
  const T* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const T* Kbh = K + b * g.ks[0] + h * g.ks[1];
  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = valid ? to_f32(Qbh[(int64_t)row * g.qs[2] + d]) : 0.f;
  __shared__ float ks[32][D];
  float m = kNegInf, s = 0.f;
  const float c = g.scale_log2;
  for (int kb = 0; kb < g.N; kb += 32) {
    for (int idx = threadIdx.x; idx < 32 * D; idx += 64) {
      const int kk = idx / D, d = idx - kk * D;
      ks[kk][d] = kb + kk < g.N ? to_f32(Kbh[(int64_t)(kb + kk) * g.ks[2] + d]) : 0.f;
    }
    __syncthreads();
    const int nkk = min(32, g.N - kb);
    for (int kk = 0; kk < nkk; ++kk) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(q[d], ks[kk][d], dot);
      const float x = dot * c;
      const float mn = fmaxf(m, x);
      s = s * fast_exp2(m - mn) + fast_exp2(x - mn);
      m = mn;
    }
    __syncthreads();
  }
  // the row maximum and the sum against it (log2 units); the block sums are
  // taken against the maximum, so every key of probability >= 2^-126 yields a
  // normal term, and divided by the sum afterwards
  if (row < g.Na) ml[(int64_t)bh * g.Na + row] = float2{m, s};
}

template <typename T, int D>
__global__ __launch_bounds__(128) void block_simt_kernel(const Geom g, const T* __restrict__ Q,
                                                         const T* __restrict__ K,
                                                         const float2* __restrict__ ml,
                                                         float* __restrict__ M) {
  const int task = blockIdx.x;
  const int bh = task / g.nq, i = task - bh * g.nq;
  const int b = bh / g.H, h = bh - b * g.H;
  const int row = i * g.R + threadIdx.x;
  const bool valid = row < g.N;
  const T* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const T* Kbh = K + b * g.ks[0] + h * g.ks[1];
  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = valid ? to_f32(Qbh[(int64_t)row * g.qs[2] + d]) : 0.f;
  const float2 rm = valid ? ml[(int64_t)bh * g.Na + row] : float2{0.f, 0.f};
  const float mref = rm.x, inv_l = valid ? 1.0f / rm.y : 0.f;
  __shared__ float ks[32][D];
  __shared__ float red[128];
  const float c = g.scale_log2;
  const float inv_rows = 1.0f / (float)min(g.R, g.N - i * g.R);
  for (int j = 0; j < g.nk; ++j) {
    float tot = 0.f;
    const int kend = min((j + 1) * g.C, g.N);
    for (int kb = j * g.C; kb < kend; kb += 32) {
      for (int idx = threadIdx.x; idx < 32 * D; idx += blockDim.x) {
        const int kk = idx / D, d = idx - kk * D;
        ks[kk][d] = kb + kk < kend ? to_f32(Kbh[(int64_t)(kb + kk) * g.ks[2] + d]) : 0.f;
      }
      __syncthreads();
      const int nkk = min(32, kend - kb);
      for (int kk = 0; kk < nkk; ++kk) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(q[d], ks[kk][d], dot);
        tot += fast_exp2(dot * c - mref);
      }
      __syncthreads();
    }
    red[threadIdx.x] = tot * inv_l;
    __syncthreads();
    if (threadIdx.x == 0) {
      float v = 0.f;
      for (int tt = 0; tt < (int)blockDim.x; ++tt) v += red[tt];
      M[(int64_t)task * g.nk + j] = v * inv_rows;
    }
    __syncthreads();
  }
}

template <typename T, int D>
hipError_t launch_simt(const Geom& g, const void* Q, const void* K, float* M, float2* ml, hipStream_t st) {
  const int tiles = (g.N + 63) / 64;
  hipLaunchKernelGGL((lse_simt_kernel<T, D>), dim3(g.B * g.H * tiles), dim3(64), 0, st, g,
                     (const T*)Q, (const T*)K, ml);
  hipLaunchKernelGGL((block_simt_kernel<T, D>), dim3(g.rows()), dim3(g.R), 0, st, g, (const T*)Q,
                     (const T*)K, (const float2*)ml, M);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const Geom& g, const void* Q, const void* K, float* M, float* S, __bf16* Kp,
                       hipStream_t st) {
  const int nch = packed_chunks(g);
  hipLaunchKernelGGL((pack_kv_kernel<D, false>), dim3((unsigned)(nch / 2), g.B * g.H), dim3(256), 0, st, g,
                     (const __bf16*)K, (const __bf16*)nullptr, Kp, (__bf16*)nullptr, nch);
  if (g.R == 64)
    hipLaunchKernelGGL((mass_bf16_kernel<D, true>), dim3(g.B * g.H * ((g.nq + 1) / 2)), dim3(256), 0, st, g,
                       (const __bf16*)Q, (const __bf16*)Kp, nch, S, M);
  else
    hipLaunchKernelGGL((mass_bf16_kernel<D, false>), dim3(g.rows()), dim3(256), (size_t)2 * g.nk * sizeof(float),
                       st, g, (const __bf16*)Q, (const __bf16*)Kp, nch, S, M);
  return hipGetLastError();
}

}  // namespace

// Workspace.  Matrix-core path: per-(query row, key block) sums S, fp32
// [B*H*nq][R/64][nk][64], then the packed K.  SIMT path: per row the maximum
// score (log2 units) and the sum of 2^(s - max), fp32 pairs [B*H][N_alloc].
static size_t mass_s_bytes(const Geom& g) {
  return align_up((size_t)g.B * g.H * g.nq * (g.R / 64) * g.nk * 64 * sizeof(float), 256);
}

size_t mass_ws_bytes(const Geom& g) {
  if (mfma_path(g)) return mass_s_bytes(g) + (size_t)g.B * g.H * packed_chunks(g) * 32 * g.D * sizeof(uint16_t);
  return (size_t)g.B * g.H * g.Na * sizeof(float2);
}

hipError_t launch_block_mass(const Geom& g, const void* Q, const void* K, float* M, void* ws,
                             hipStream_t stream) {
  if (mfma_path(g)) {
    float* S = reinterpret_cast<float*>(ws);
    __bf16* Kp = reinterpret_cast<__bf16*>(reinterpret_cast<char*>(ws) + mass_s_bytes(g));
    return g.D == 128 ? launch_mfma<128>(g, Q, K, M, S, Kp, stream) : launch_mfma<64>(g, Q, K, M, S, Kp, stream);
  }
  float2* ml = reinterpret_cast<float2*>(ws);
  if (g.bf16)
    return g.D == 128 ? launch_simt<__bf16, 128>(g, Q, K, M, ml, stream)
                      : launch_simt<__bf16, 64>(g, Q, K, M, ml, stream);
  return g.D == 128 ? launch_simt<float, 128>(g, Q, K, M, ml, stream)
                    : launch_simt<float, 64>(g, Q, K, M, ml, stream);
}

}  // namespace losa
