// Query-key drift per (batch, head) since a reference step, for the
// drift-triggered refresh of frozen lists (HASTE page, temporal mask reuse:
// mask prediction is skipped while queries and keys have drifted little
// since it was last made).  For head g = b * H + h, over its valid tokens:
//   drift[2g]     = ||Q_g - Qref_g||_F / ||Qref_g||_F
//   drift[2g + 1] = ||K_g - Kref_g||_F / ||Kref_g||_F
// (0 when both norms are 0, +inf when only the reference's is), and
// refresh[g] = 1 when either drift exceeds tau.
//
// HBM-bound: each element of Q, K, Q_ref and K_ref is read once, in
// 16-byte loads, all of a thread's loads in flight together.  Differences,
// squares and sums are fp64 (a difference of two bf16 or fp32 values is
// exact there), added in a fixed order -- per-workgroup partials, then one
// wave per head -- so the result is deterministic and needs no atomics and
// no cleared memory.
#include "losa.h"
#include "losa_device.hpp"
#include "losa_internal.hpp"

namespace losa {
namespace {

constexpr int kDriftThreads = 256;
constexpr int kDriftElems = 8192;  // elements of one tensor per workgroup: 64 tokens at d = 128

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum of squared differences and of squared reference values over 16 bytes.
template <bool kBf16>
__device__ __forceinline__ void accumulate16(const uint4& a, const uint4& r, double& dd, double& rr) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w};
  const uint32_t rv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if constexpr (kBf16) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t sh = half ? 0u : 16u;  // low half first: its bits move to the top
        const double x = (double)__uint_as_float((av[w] << sh) & 0xffff0000u);
        const double y = (double)__uint_as_float((rv[w] << sh) & 0xffff0000u);
        const double d = x - y;
        dd = __builtin_fma(d, d, dd);
        rr = __builtin_fma(y, y, rr);
      }
    } else {
      const double x = (double)__uint_as_float(av[w]);
      const double y = (double)__uint_as_float(rv[w]);
      const double d = x - y;
      dd = __builtin_fma(d, d, dd);
      rr = __builtin_fma(y, y, rr);
    }
  }
}

// Grid (chunk, head g, tensor t): tokens [chunk * tok, min(N, +tok)) of
// tensor t (0 = Q, 1 = K) of head g.  kPer = 16-byte vectors per thread.
template <bool kBf16, int kPer>
__global__ __launch_bounds__(kDriftThreads) void drift_partial_kernel(const Geom g, const char* __restrict__ Q,
                                                                      const char* __restrict__ K,
                                                                      const char* __restrict__ Qr,
                                                                      const char* __restrict__ Kr, int tok,
                                                                      int nchunk, double2* __restrict__ part) {
  __shared__ double red[2][kDriftThreads / 64];
  const int chunk = blockIdx.x, gh = blockIdx.y, t = blockIdx.z;
  const int b = gh / g.H, h = gh - b * g.H;
  const int64_t* st = t ? g.ks : g.qs;
  const char* cur = t ? K : Q;
  const char* ref = t ? Kr : Qr;
  constexpr int esz = kBf16 ? 2 : 4;
  const int vpr = g.D * esz / 16;  // 16-byte vectors per token
  const int n0 = chunk * tok;
  const int nv = (min(g.N, n0 + tok) - n0) * vpr;
  const int64_t base = ((int64_t)b * st[0] + (int64_t)h * st[1] + (int64_t)n0 * st[2]) * esz;
  uint4 a[kPer], r[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int v = threadIdx.x + u * kDriftThreads;
    if (v < nv) {
      const int n = v / vpr, c = v - n * vpr;
      const int64_t off = base + (int64_t)n * st[2] * esz + c * 16;
      a[u] = *reinterpret_cast<const uint4*>(cur + off);
      r[u] = *reinterpret_cast<const uint4*>(ref + off);
    }
  }
  double dd = 0.0, rr = 0.0;
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if ((int)threadIdx.x + u * kDriftThreads < nv) accumulate16<kBf16>(a[u], r[u], dd, rr);
  dd = wave_sum_f64(dd);
  rr = wave_sum_f64(rr);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = dd;
    red[1][w] = rr;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sd = 0.0, sr = 0.0;
#pragma unroll
    for (int ww = 0; ww < kDriftThreads / 64; ++ww) {
      sd += red[0][ww];
      sr += red[1][ww];
    }
    part[((int64_t)gh * 2 + t) * nchunk + chunk] = make_double2(sd, sr);
  }
}

// ||diff|| / ||ref|| from the two sums of squares; 0/0 = 0, x/0 = inf, NaN
// (a NaN among the valid tokens) stays NaN.
__device__ __forceinline__ double rel_norm(double dd, double rr) {
  if (rr > 0.0) return sqrt(dd) / sqrt(rr);
  if (rr == 0.0) return dd > 0.0 ? __builtin_inf() : dd;
  return rr;
}

// One wave per head: lane l adds the partials l, l + 64, ... of Q and of K,
// then the wave adds the lanes' sums.
__global__ __launch_bounds__(64) void drift_final_kernel(int nchunk, const double2* __restrict__ part, double tau,
                                                         double* __restrict__ drift, int32_t* __restrict__ refresh) {
  const int gh = blockIdx.x;
  double out[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const double2* p = part + ((int64_t)gh * 2 + t) * nchunk;
    double dd = 0.0, rr = 0.0;
    for (int c = threadIdx.x; c < nchunk; c += 64) {
      const double2 x = p[c];
      dd += x.x;
      rr += x.y;
    }
    out[t] = rel_norm(wave_sum_f64(dd), wave_sum_f64(rr));
  }
  if (threadIdx.x == 0) {
    drift[2 * gh] = out[0];
    drift[2 * gh + 1] = out[1];
    if (refresh) refresh[gh] = (out[0] > tau || out[1] > tau) ? 1 : 0;
  }
}

int drift_tokens(const Geom& g) { return kDriftElems / g.D; }
int drift_chunks(const Geom& g) { return (g.N + drift_tokens(g) - 1) / drift_tokens(g); }

}  // namespace

size_t drift_ws_bytes(const Geom& g) {
  return align_up((size_t)g.B * g.H * 2 * drift_chunks(g) * sizeof(double2), 256);
}

hipError_t launch_qk_drift(const Geom& g, const void* Q, const void* K, const void* Qr, const void* Kr, double tau,
                           double* drift, int32_t* refresh, void* ws, hipStream_t st) {
  const int tok = drift_tokens(g), nchunk = drift_chunks(g);
  double2* part = reinterpret_cast<double2*>(ws);
  const dim3 grid(nchunk, g.B * g.H, 2);
  auto cq = reinterpret_cast<const char*>(Q);
  auto ck = reinterpret_cast<const char*>(K);
  auto cqr = reinterpret_cast<const char*>(Qr);
  auto ckr = reinterpret_cast<const char*>(Kr);
  // tok * D = kDriftElems elements per workgroup: kDriftElems * esz / 16 vectors over kDriftThreads threads
  if (g.bf16)
    hipLaunchKernelGGL((drift_partial_kernel<true, kDriftElems * 2 / 16 / kDriftThreads>), grid, dim3(kDriftThreads),
                       0, st, g, cq, ck, cqr, ckr, tok, nchunk, part);
  else
    hipLaunchKernelGGL((drift_partial_kernel<false, kDriftElems * 4 / 16 / kDriftThreads>), grid,
                       dim3(kDriftThreads), 0, st, g, cq, ck, cqr, ckr, tok, nchunk, part);
  hipLaunchKernelGGL(drift_final_kernel, dim3(g.B * g.H), dim3(64), 0, st, nchunk, (const double2*)part, tau, drift,
                     refresh);
  return hipGetLastError();
}

}  // namespace losa
