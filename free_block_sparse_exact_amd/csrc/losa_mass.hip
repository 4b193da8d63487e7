// Exact block attention masses (LoSA page, Motivation Summary: block
// attention mass; Methodology Summary: masses at the construction step are
// exact, not estimated).
//
//   M[b,h,i,j] = (1/valid rows of block i) * sum over rows q of block i and
//                valid keys k of block j of exp(s_qk - lse_q),
// with s = q.k * scale and lse_q the log-sum-exp of row q over all valid keys.
//
// bf16 matrix-core path (d in {64, 128}, R in {64, 128}): ONE pass over K.
// A workgroup owns one query block (R/64 groups of 64 rows, four waves per
// group); the waves of a group split the KEY BLOCKS (wave w takes blocks
// j = w, w+4, ...).  For every query a wave fixes a reference m at its first
// chunk's maximum plus kHeadroom (log2 units; scores are pre-multiplied by
// scale*log2(e)), sums 2^(s*c - m) per key block, writes that per-(query,
// block) sum to a workspace S and keeps the row total.  Once the four waves
// are merged, lse_q is known, and the workgroup reads S back:
//   M[i,j] = (1/rows) * sum_q S[q,j] * 2^(m_q,w(j) - lse_q).
// The scores and exponentials are computed once (a two-pass form computes
// both twice); S costs 4 bytes per (query row, key block) of HBM traffic each
// way.  S^T = K Q^T is formed with 16x16x32 bf16 MFMA: lane l owns query
// (l & 15) of each 16-query tile and 4 keys per 16-key tile.
//
// fp32 inputs (and bf16 shapes outside the matrix-core path) take a SIMT
// two-pass path: row log-sum-exp first, then the block sums.
#include "losa_blocksum.hpp"
#include "losa_device.hpp"
#include "losa_internal.hpp"
#include "losa_pack.hpp"

namespace losa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

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

// Grid: B*H*nq workgroups of 256*QG threads (QG = R/64 query groups), two
// waves per SIMD.  A term 2^(s*c - m) can only overflow if a score exceeds the
// wave's first-chunk maximum by more than ~190 (log2 units); terms more than
// ~60 below the row maximum flush to 0, negligible against it.  If a block sum
// or the row total leaves [0, 2^100] (or m is not finite), the wave recomputes
// its blocks against its exact maximum instead, overwriting its S entries.
template <int D, int QG>
__global__ __launch_bounds__(256 * QG, 2 / QG) void mass_bf16_kernel(const Geom g, const __bf16* __restrict__ Q,
                                                                     const __bf16* __restrict__ Kp, int nch,
                                                                     float* __restrict__ S, float* __restrict__ M) {
  constexpr float kHeadroom = 64.0f;
  constexpr float kSumBound = 1.2676506e30f;  // 2^100
  __shared__ float s_ref[QG][4][64], s_tot[QG][4][64], s_f[QG][4][64];
  extern __shared__ float part[];  // [QG][nk] per-group partial masses (QG > 1)
  const int rows = g.B * g.H * g.nq;
  const int task = xcd_task(blockIdx.x, rows);
  const int bh = task / g.nq, i = task - bh * g.nq;
  const int b = bh / g.H, h = bh - b * g.H;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = w >> 2, kw = w & 3;
  const int lr = lane & 15, lg = lane >> 4;
  const __bf16* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const __bf16* Kpbh = Kp + (int64_t)bh * nch * (32 * D);
  const int row0 = i * g.R + grp * 64;
  float* Sg = S + ((int64_t)task * QG + grp) * g.nk * 64;  // [nk][64] of this query group

  QTile<D> q;
  q.load(Qbh, g.qs[2], row0, g.N, lr, lg);

  const float c = g.scale_log2;
  const int sub = g.C / 32, sub_shift = __builtin_ctz(sub);
  const int nb = g.nk > kw ? (g.nk - kw + 3) / 4 : 0;  // my key blocks kw, kw+4, ...
  const int nu = nb * sub;                              // their 32-key chunks
  auto chunk_kb = [&](int u) { return (kw + 4 * (u >> sub_shift)) * g.C + 32 * (u & (sub - 1)); };

  // Block sums: lane (lg, lr) holds partial sums over its keys for queries
  // qt*16 + lr, qt = 0..3; the totals over the four lane groups are formed so
  // that lane (lg, lr) ends with the one for query lg*16 + lr (the one it
  // stores): two values swapped with the lane 32 away, then one with the lane
  // 16 away.
  auto reduce_mine = [&](const float (&v)[4]) -> float { return rows_sum_own(v); };

  // One sweep over my chunks against the reference m (fixed_from_first: m is
  // set from the first chunk).  tot = this lane's query's total.  Returns
  // whether a sum left [0, 2^100].
  float m[4], tot;
  auto sweep = [&](bool fixed_from_first) -> bool {
    bool over = false;
    float blk[4];
    tot = 0.f;
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) blk[qt] = 0.f;
    bf16x8 kop[2][D / 32];
    load_kchunk<D>(Kpbh, chunk_kb(0), lane, kop);
    for (int u = 0; u < nu; ++u) {
      const int kb = chunk_kb(u);
      f32x4 acc[2][4];
      chunk_scores<D>(q, kop, acc);
      if (u + 1 < nu) load_kchunk<D>(Kpbh, chunk_kb(u + 1), lane, kop);
      if (__builtin_expect(kb + 32 > g.N, 0)) mask_tail(kb, g.N, lg, acc);
      if (fixed_from_first && u == 0) {
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          float mx = acc[0][qt][0];
#pragma unroll
          for (int e = 1; e < 8; ++e) mx = fmaxf(mx, acc[e >> 2][qt][e & 3]);
          mx = rows_max(mx);
          m[qt] = mx * c + kHeadroom;  // finite: the first chunk holds a valid key
        }
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const float nm = -m[qt];
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += fast_exp2(__builtin_fmaf(acc[e >> 2][qt][e & 3], c, nm));
        blk[qt] += sum;
      }
      if ((u & (sub - 1)) == sub - 1) {  // block complete: store this lane's query's sum, add it to the total
        const int j = kw + 4 * (u >> sub_shift);
        const float v = reduce_mine(blk);
        tot += v;
        over |= !(v <= kSumBound);
        Sg[(int64_t)j * 64 + lane] = v;  // lane = query lg*16 + lr
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) blk[qt] = 0.f;
      }
    }
    over |= !(tot <= kSumBound);
    return __any(over);
  };

#pragma unroll
  for (int qt = 0; qt < 4; ++qt) m[qt] = kNegInf;
  tot = 0.f;
  if (nu > 0 && sweep(true)) {
    // Exact maximum over my keys, then the sums again against it (all terms <= 1).
    bf16x8 kop[2][D / 32];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) m[qt] = kNegInf;
    for (int u = 0; u < nu; ++u) {
      const int kb = chunk_kb(u);
      load_kchunk<D>(Kpbh, kb, lane, kop);
      f32x4 acc[2][4];
      chunk_scores<D>(q, kop, acc);
      if (kb + 32 > g.N) mask_tail(kb, g.N, lg, acc);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int e = 0; e < 8; ++e) m[qt] = fmaxf(m[qt], acc[e >> 2][qt][e & 3]);
    }
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      m[qt] = rows_max(m[qt]);
      m[qt] *= c;
    }
    sweep(false);
  }

  // Merge the four key groups of each query: lse_q, then this wave's factor
  // 2^(m - lse) for the query its lane stored (padding rows get 0).
  s_ref[grp][kw][lane] = lg == 0 ? m[0] : lg == 1 ? m[1] : lg == 2 ? m[2] : m[3];  // lane = query lg*16 + lr
  s_tot[grp][kw][lane] = tot;
  __syncthreads();
  float f = 0.f;
  {
    float mm = kNegInf;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) mm = fmaxf(mm, s_ref[grp][ww][lane]);
    float l = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
      if (s_ref[grp][ww][lane] != kNegInf) l += s_tot[grp][ww][lane] * fast_exp2(s_ref[grp][ww][lane] - mm);
    const float mine = s_ref[grp][kw][lane];
    if (row0 + lane < g.N && mine != kNegInf) f = fast_exp2(mine - mm) / l;
  }
  s_f[grp][kw][lane] = f;
  __syncthreads();  // every lane reads all 64 factors of its wave
  const float inv_rows = 1.0f / (float)min(g.R, g.N - i * g.R);
  float* Mrow = M + (int64_t)task * g.nk;
  if (QG == 1) blocks_from_sums(Sg, s_f[grp][kw], kw, nb, inv_rows, Mrow, lane);
  else blocks_from_sums(Sg, s_f[grp][kw], kw, nb, 1.0f, part + grp * g.nk, lane);
  if (QG > 1) {
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
                                                      const T* __restrict__ K, float* __restrict__ lse2) {
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
  if (row < g.Na) lse2[(int64_t)bh * g.Na + row] = m + __log2f(s);
}

template <typename T, int D>
__global__ __launch_bounds__(128) void block_simt_kernel(const Geom g, const T* __restrict__ Q,
                                                         const T* __restrict__ K,
                                                         const float* __restrict__ lse2,
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
  const float l2 = valid ? lse2[(int64_t)bh * g.Na + row] : kPosInf;
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
        tot += fast_exp2(dot * c - l2);
      }
      __syncthreads();
    }
    red[threadIdx.x] = tot;
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
hipError_t launch_simt(const Geom& g, const void* Q, const void* K, float* M, float* lse2, hipStream_t st) {
  const int tiles = (g.N + 63) / 64;
  hipLaunchKernelGGL((lse_simt_kernel<T, D>), dim3(g.B * g.H * tiles), dim3(64), 0, st, g,
                     (const T*)Q, (const T*)K, lse2);
  hipLaunchKernelGGL((block_simt_kernel<T, D>), dim3(g.rows()), dim3(g.R), 0, st, g, (const T*)Q,
                     (const T*)K, (const float*)lse2, M);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const Geom& g, const void* Q, const void* K, float* M, float* S, __bf16* Kp,
                       hipStream_t st) {
  const int nch = packed_chunks(g);
  hipLaunchKernelGGL((pack_kv_kernel<D, false>), dim3((unsigned)(nch / 2), g.B * g.H), dim3(256), 0, st, g,
                     (const __bf16*)K, (const __bf16*)nullptr, Kp, (__bf16*)nullptr, nch);
  if (g.R == 64)
    hipLaunchKernelGGL((mass_bf16_kernel<D, 1>), dim3(g.rows()), dim3(256), 0, st, g, (const __bf16*)Q,
                       (const __bf16*)Kp, nch, S, M);
  else
    hipLaunchKernelGGL((mass_bf16_kernel<D, 2>), dim3(g.rows()), dim3(512), (size_t)2 * g.nk * sizeof(float), st,
                       g, (const __bf16*)Q, (const __bf16*)Kp, nch, S, M);
  return hipGetLastError();
}

}  // namespace

// Workspace.  Matrix-core path: per-(query row, key block) sums S, fp32
// [B*H*nq][R/64][nk][64], then the packed K.  SIMT path: the row log-sum-exp
// in log2 units, fp32 [B*H][N_alloc].
static size_t mass_s_bytes(const Geom& g) {
  return align_up((size_t)g.B * g.H * g.nq * (g.R / 64) * g.nk * 64 * sizeof(float), 256);
}

size_t mass_ws_bytes(const Geom& g) {
  if (mfma_path(g)) return mass_s_bytes(g) + (size_t)g.B * g.H * packed_chunks(g) * 32 * g.D * sizeof(uint16_t);
  return (size_t)g.B * g.H * g.Na * sizeof(float);
}

hipError_t launch_block_mass(const Geom& g, const void* Q, const void* K, float* M, void* ws,
                             hipStream_t stream) {
  if (mfma_path(g)) {
    float* S = reinterpret_cast<float*>(ws);
    __bf16* Kp = reinterpret_cast<__bf16*>(reinterpret_cast<char*>(ws) + mass_s_bytes(g));
    return g.D == 128 ? launch_mfma<128>(g, Q, K, M, S, Kp, stream) : launch_mfma<64>(g, Q, K, M, S, Kp, stream);
  }
  float* lse2 = reinterpret_cast<float*>(ws);
  if (g.bf16)
    return g.D == 128 ? launch_simt<__bf16, 128>(g, Q, K, M, lse2, stream)
                      : launch_simt<__bf16, 64>(g, Q, K, M, lse2, stream);
  return g.D == 128 ? launch_simt<float, 128>(g, Q, K, M, lse2, stream)
                    : launch_simt<float, 64>(g, Q, K, M, lse2, stream);
}

}  // namespace losa
