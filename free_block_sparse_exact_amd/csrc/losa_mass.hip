// Exact block attention masses (LoSA page, Motivation Summary: block
// attention mass; Methodology Summary: masses at the construction step are
// exact, not estimated).
//
// Two passes over K per query tile:
//   pass 1  row log-sum-exp: a flash-style sweep over all valid keys keeping
//           a running maximum and sum (log2 units: scores are pre-multiplied
//           by scale*log2(e));
//   pass 2  M[b,h,i,j] = (1/valid rows of block i) * sum over rows q of block
//           i and valid keys k of block j of exp2(s_qk - lse2_q).
// Both passes compute the same scores with the same instruction sequence, so
// pass 2 sees exactly the scores pass 1 normalised.
//
// bf16 matrix-core path (d in {64, 128}, R in {64, 128}): a workgroup of four
// waves owns a 64-row query tile; the waves split the KEYS (wave w takes
// 32-key chunks w, w+4, ...), each holding the whole tile's Q as the B
// operand, so K is read straight from global memory into registers with no
// LDS staging and no wave reads another's keys.  S^T = K Q^T is formed with
// 16x16x32 bf16 MFMA: lane l then owns query (l & 15) of each 16-query tile
// and 4 keys per 16-key tile, so the per-query statistics live in lanes.
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

// Pass 1.  Grid: B*H*ceil(N/64) workgroups of 256 threads (two per CU).
// Each lane keeps, per query, a sum of 2^(s*c - m) over its own keys against
// a reference m fixed at its first chunk's maximum plus kHeadroom (log2
// units): no per-score maximum.  A term can only overflow if a later score
// exceeds that maximum by more than ~190; terms more than ~85 below it flush
// to 0, negligible against the maximum term.  If a lane's sum ever leaves
// (0, 2^100] the wave recomputes its chunks in two passes (exact per-lane
// maximum first).  Lanes, then waves, are merged at the end.
template <int D>
__global__ __launch_bounds__(256, 2) void lse_bf16_kernel(const Geom g, const __bf16* __restrict__ Q,
                                                          const __bf16* __restrict__ Kp, int nch,
                                                          float* __restrict__ lse2) {
  constexpr float kHeadroom = 64.0f;
  constexpr float kSumBound = 1.2676506e30f;  // 2^100
  const int tiles = (g.N + 63) / 64;
  const int task = xcd_task(blockIdx.x, g.B * g.H * tiles);
  const int bh = task / tiles, t = task - bh * tiles;
  const int b = bh / g.H, h = bh - b * g.H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const __bf16* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const __bf16* Kpbh = Kp + (int64_t)bh * nch * (32 * D);

  QTile<D> q;
  q.load(Qbh, g.qs[2], t * 64, g.N, lr, lg);
  float m[4], s[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) { m[qt] = kNegInf; s[qt] = 0.f; }

  const float c = g.scale_log2;
  const int nchunks = (g.N + 31) / 32;
  const int nmine = nchunks > w ? (nchunks - w + 3) / 4 : 0;
  bool fallback = false;
  if (nmine > 0) {
    bf16x8 kop[2][D / 32];
    load_kchunk<D>(Kpbh, w * 32, lane, kop);
    for (int it = 0; it < nmine; ++it) {
      const int kb = (w + 4 * it) * 32;
      f32x4 acc[2][4];
      chunk_scores<D>(q, kop, acc);
      if (it + 1 < nmine) load_kchunk<D>(Kpbh, kb + 128, lane, kop);
      if (__builtin_expect(kb + 32 > g.N, 0)) mask_tail(kb, g.N, lg, acc);
      if (it == 0) {
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          float mx = acc[0][qt][0];
#pragma unroll
          for (int e = 1; e < 8; ++e) mx = fmaxf(mx, acc[e >> 2][qt][e & 3]);
          m[qt] = mx * c + kHeadroom;  // -inf (all masked) forces the fallback
        }
      }
      bool over = false;
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const float nm = -m[qt];
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += fast_exp2(__builtin_fmaf(acc[e >> 2][qt][e & 3], c, nm));
        s[qt] += sum;
        over |= !(s[qt] <= kSumBound);
      }
      if (__builtin_expect(__any(over), 0)) { fallback = true; break; }
    }
  }
  if (fallback) {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) { m[qt] = kNegInf; s[qt] = 0.f; }
    bf16x8 kop[2][D / 32];
    for (int it = 0; it < nmine; ++it) {
      const int kb = (w + 4 * it) * 32;
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
    for (int qt = 0; qt < 4; ++qt) m[qt] *= c;
    for (int it = 0; it < nmine; ++it) {
      const int kb = (w + 4 * it) * 32;
      load_kchunk<D>(Kpbh, kb, lane, kop);
      f32x4 acc[2][4];
      chunk_scores<D>(q, kop, acc);
      if (kb + 32 > g.N) mask_tail(kb, g.N, lg, acc);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const float nm = m[qt] == kNegInf ? 0.f : -m[qt];
#pragma unroll
        for (int e = 0; e < 8; ++e) s[qt] += fast_exp2(__builtin_fmaf(acc[e >> 2][qt][e & 3], c, nm));
      }
    }
  }

  // Merge the four lanes that share each query, then the four waves.
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float mo = __shfl_xor(m[qt], o, kWave);
      const float so = __shfl_xor(s[qt], o, kWave);
      const float mn = fmaxf(m[qt], mo);
      float acc = 0.f;
      if (m[qt] != kNegInf) acc += s[qt] * fast_exp2(m[qt] - mn);
      if (mo != kNegInf) acc += so * fast_exp2(mo - mn);
      m[qt] = mn;
      s[qt] = acc;
    }
  }
  __shared__ float sm[4][64], ss[4][64];
  if (lg == 0) {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) { sm[w][qt * 16 + lr] = m[qt]; ss[w][qt * 16 + lr] = s[qt]; }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int qi = threadIdx.x;
    float mm = kNegInf;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) mm = fmaxf(mm, sm[ww][qi]);
    float tot = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
      if (sm[ww][qi] != kNegInf) tot += ss[ww][qi] * fast_exp2(sm[ww][qi] - mm);
    const int row = t * 64 + qi;
    lse2[(int64_t)bh * g.Na + row] = mm + __log2f(tot);
  }
}

// Pass 2.  Grid: B*H*nq workgroups of 256*QG threads (QG = R/64 query groups),
// two waves per SIMD.  Key block j goes to key group j % 4; its 32-key chunks
// are summed as exp2(s*c - lse2_q) and reduced over the wave.
template <int D, int QG>
__global__ __launch_bounds__(256 * QG, 2 / QG) void block_bf16_kernel(const Geom g, const __bf16* __restrict__ Q,
                                                                      const __bf16* __restrict__ Kp, int nch,
                                                                      const float* __restrict__ lse2,
                                                                      float* __restrict__ M) {
  extern __shared__ float part[];  // [QG][nk]
  const int rows = g.B * g.H * g.nq;
  const int task = xcd_task(blockIdx.x, rows);
  const int bh = task / g.nq, i = task - bh * g.nq;
  const int b = bh / g.H, h = bh - b * g.H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int grp = w >> 2, kw = w & 3;
  const int lr = lane & 15, lg = lane >> 4;
  const __bf16* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const __bf16* Kpbh = Kp + (int64_t)bh * nch * (32 * D);
  const int row0 = i * g.R + grp * 64;

  QTile<D> q;
  q.load(Qbh, g.qs[2], row0, g.N, lr, lg);
  float l2[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int row = row0 + qt * 16 + lr;
    l2[qt] = row < g.N ? lse2[(int64_t)bh * g.Na + row] : kPosInf;  // padding rows add 0
  }

  const float c = g.scale_log2;
  const int sub = g.C / 32;
  for (int j = kw; j < g.nk; j += 4) {
    float tot = 0.f;
    for (int sc = 0; sc < sub; ++sc) {
      const int kb = j * g.C + sc * 32;
      if (kb >= g.N) break;
      bf16x8 kop[2][D / 32];
      load_kchunk<D>(Kpbh, kb, lane, kop);
      f32x4 acc[2][4];
      chunk_scores<D>(q, kop, acc);
      if (__builtin_expect(kb + 32 > g.N, 0)) mask_tail(kb, g.N, lg, acc);
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const float nl = -l2[qt];
#pragma unroll
        for (int e = 0; e < 8; ++e) tot += fast_exp2(__builtin_fmaf(acc[e >> 2][qt][e & 3], c, nl));
      }
    }
    tot = wave_sum(tot);
    if (lane == 0) part[grp * g.nk + j] = tot;
  }
  __syncthreads();
  const float inv_rows = 1.0f / (float)min(g.R, g.N - i * g.R);
  float* Mrow = M + (int64_t)task * g.nk;
  for (int j = threadIdx.x; j < g.nk; j += blockDim.x) {
    float v = part[j];
#pragma unroll
    for (int gg = 1; gg < QG; ++gg) v += part[gg * g.nk + j];
    Mrow[j] = v * inv_rows;
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
hipError_t launch_mfma(const Geom& g, const void* Q, const void* K, float* M, float* lse2, __bf16* Kp,
                       hipStream_t st) {
  const int nch = packed_chunks(g);
  hipLaunchKernelGGL((pack_kv_kernel<D, false>), dim3((unsigned)(nch / 2), g.B * g.H), dim3(256), 0, st, g,
                     (const __bf16*)K, (const __bf16*)nullptr, Kp, (__bf16*)nullptr, nch);
  const int tiles = (g.N + 63) / 64;
  hipLaunchKernelGGL((lse_bf16_kernel<D>), dim3(g.B * g.H * tiles), dim3(256), 0, st, g, (const __bf16*)Q,
                     (const __bf16*)Kp, nch, lse2);
  const size_t lds = (size_t)(g.R / 64) * g.nk * sizeof(float);
  if (g.R == 64)
    hipLaunchKernelGGL((block_bf16_kernel<D, 1>), dim3(g.rows()), dim3(256), lds, st, g, (const __bf16*)Q,
                       (const __bf16*)Kp, nch, (const float*)lse2, M);
  else
    hipLaunchKernelGGL((block_bf16_kernel<D, 2>), dim3(g.rows()), dim3(512), lds, st, g, (const __bf16*)Q,
                       (const __bf16*)Kp, nch, (const float*)lse2, M);
  return hipGetLastError();
}

}  // namespace

size_t mass_ws_bytes(const Geom& g) {
  size_t n = align_up((size_t)g.B * g.H * g.Na * sizeof(float), 256);  // row log-sum-exp (log2 units)
  if (mfma_path(g)) n += (size_t)g.B * g.H * packed_chunks(g) * 32 * g.D * sizeof(uint16_t);  // packed K
  return n;
}

hipError_t launch_block_mass(const Geom& g, const void* Q, const void* K, float* M, void* ws,
                             hipStream_t stream) {
  float* lse2 = reinterpret_cast<float*>(ws);
  __bf16* Kp = reinterpret_cast<__bf16*>(reinterpret_cast<char*>(ws) +
                                         align_up((size_t)g.B * g.H * g.Na * sizeof(float), 256));
  if (mfma_path(g)) return g.D == 128 ? launch_mfma<128>(g, Q, K, M, lse2, Kp, stream)
                                      : launch_mfma<64>(g, Q, K, M, lse2, Kp, stream);
  if (g.bf16)
    return g.D == 128 ? launch_simt<__bf16, 128>(g, Q, K, M, lse2, stream)
                      : launch_simt<__bf16, 64>(g, Q, K, M, lse2, stream);
  return g.D == 128 ? launch_simt<float, 128>(g, Q, K, M, lse2, stream)
                    : launch_simt<float, 64>(g, Q, K, M, lse2, stream);
}

}  // namespace losa
