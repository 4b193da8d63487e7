// Pooled proxy masses: the coarse block-mass estimate that per-step top-p
// methods rely on and that the LoSA page contrasts with exact masses
// (Motivation Summary: the estimates SVG2 and SpargeAttn use lose accuracy
// just where 99% recall is wanted).  The pages give no formula; this
// library takes the plainest block-pooled reading:
//
//   P[b,h,i,j] = |B_j| exp(qbar_i . kbar_j * scale) / sum_j' |B_j'| exp(qbar_i . kbar_j' * scale),
//
// with qbar_i, kbar_j the means over the valid tokens of query block i and
// key block j, and |B_j| the number of valid keys of block j (each pooled key
// stands for its block's keys).  Rows sum to 1 like the exact masses, so the
// same selector turns P into lists; P equals M whenever the scores are
// constant on every (query block, key block) pair.
//
// Two kernels, both bound by memory, not arithmetic: block means of Q and K
// (every valid token read once, fp32 sums), then one workgroup per query
// block for the n_k pooled scores and the block-weighted softmax.
#include "losa_device.hpp"
#include "losa_internal.hpp"

namespace losa {
namespace {

// Mean over the valid tokens of block x (size blk) of X[b, h, :, :] -> out[bh][x][D],
// accumulated and stored in Acc (fp32 for the pooled proxy masses; fp64 for the
// on-the-fly thresholding inside the attention pass, whose block sums of bf16
// inputs are then exact and whose means are correctly rounded).
// Grid (n_blocks, B*H), 256 threads: thread = (token group, dimension).
template <typename T, int D, typename Acc>
__global__ __launch_bounds__(256) void pool_kernel(const Geom g, const T* __restrict__ X, int64_t s0, int64_t s1,
                                                   int64_t s2, int blk, int nblk, Acc* __restrict__ out) {
  constexpr int G = 256 / D;  // token groups
  __shared__ Acc part[G][D];
  const int x = blockIdx.x, bh = blockIdx.y;
  const int b = bh / g.H, h = bh - b * g.H;
  const int d = threadIdx.x % D, grp = threadIdx.x / D;
  const int t0 = x * blk, t1 = min(t0 + blk, g.N);
  const T* Xbh = X + b * s0 + h * s1;
  Acc acc = 0;
  for (int t = t0 + grp; t < t1; t += G) acc += (Acc)(float)Xbh[(int64_t)t * s2 + d];
  part[grp][d] = acc;
  __syncthreads();
  if (grp == 0) {
    Acc s = 0;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) s += part[gg][d];
    out[((int64_t)bh * nblk + x) * D + d] = s / (Acc)(t1 - t0);
  }
}

// One workgroup per query block row r = (b*H + h)*nq + i: scores of qbar_i
// against the n_k pooled keys (log2 units), then the block-weighted softmax.
template <int D>
__global__ __launch_bounds__(256) void proxy_kernel(const Geom g, const float* __restrict__ qbar,
                                                    const float* __restrict__ kbar, float* __restrict__ P) {
  extern __shared__ float sc[];  // [nk] scores
  __shared__ __attribute__((aligned(16))) float qv[D];
  __shared__ float red[256 / kWave];
  const int r = blockIdx.x;
  const int bh = r / g.nq;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  if (tid < D) qv[tid] = qbar[(int64_t)r * D + tid];
  __syncthreads();
  const float* kb = kbar + (int64_t)bh * g.nk * D;
  float mx = -__builtin_huge_valf();
  for (int j = tid; j < g.nk; j += 256) {
    const f32x4* kj = reinterpret_cast<const f32x4*>(kb + (int64_t)j * D);  // 16-byte loads of the row
    float s = 0.f;
#pragma unroll 8
    for (int e = 0; e < D / 4; ++e) {
      const f32x4 k4 = kj[e], q4 = *reinterpret_cast<const f32x4*>(qv + 4 * e);
      s = __builtin_fmaf(q4[0], k4[0], s);
      s = __builtin_fmaf(q4[1], k4[1], s);
      s = __builtin_fmaf(q4[2], k4[2], s);
      s = __builtin_fmaf(q4[3], k4[3], s);
    }
    s *= g.scale_log2;
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int ww = 1; ww < 256 / kWave; ++ww) mx = fmaxf(mx, red[ww]);
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j < g.nk; j += 256) {
    const float wj = (float)min(g.C, g.N - j * g.C) * fast_exp2(sc[j] - mx);
    sc[j] = wj;
    sum += wj;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  sum = 0.f;
#pragma unroll
  for (int ww = 0; ww < 256 / kWave; ++ww) sum += red[ww];
  const float inv = 1.0f / sum;
  float* Prow = P + (int64_t)r * g.nk;
  for (int j = tid; j < g.nk; j += 256) Prow[j] = sc[j] * inv;
}

template <typename T, int D>
hipError_t launch(const Geom& g, const void* Q, const void* K, float* P, float* qbar, float* kbar, hipStream_t st) {
  hipLaunchKernelGGL((pool_kernel<T, D, float>), dim3(g.nq, g.B * g.H), dim3(256), 0, st, g, (const T*)Q, g.qs[0],
                     g.qs[1], g.qs[2], g.R, g.nq, qbar);
  hipLaunchKernelGGL((pool_kernel<T, D, float>), dim3(g.nk, g.B * g.H), dim3(256), 0, st, g, (const T*)K, g.ks[0],
                     g.ks[1], g.ks[2], g.C, g.nk, kbar);
  hipLaunchKernelGGL((proxy_kernel<D>), dim3(g.rows()), dim3(256), (size_t)g.nk * sizeof(float), st, g,
                     (const float*)qbar, (const float*)kbar, P);
  return hipGetLastError();
}

template <int D>
void launch_means64(const Geom& g, const __bf16* Q, const __bf16* K, double* qbar, double* kbar, hipStream_t st) {
  hipLaunchKernelGGL((pool_kernel<__bf16, D, double>), dim3(g.nq, g.B * g.H), dim3(256), 0, st, g, Q, g.qs[0],
                     g.qs[1], g.qs[2], g.R, g.nq, qbar);
  hipLaunchKernelGGL((pool_kernel<__bf16, D, double>), dim3(g.nk, g.B * g.H), dim3(256), 0, st, g, K, g.ks[0],
                     g.ks[1], g.ks[2], g.C, g.nk, kbar);
}

}  // namespace

void launch_block_means64(const Geom& g, const void* Q, const void* K, double* qbar, double* kbar, hipStream_t st) {
  if (g.D == 128)
    launch_means64<128>(g, (const __bf16*)Q, (const __bf16*)K, qbar, kbar, st);
  else
    launch_means64<64>(g, (const __bf16*)Q, (const __bf16*)K, qbar, kbar, st);
}

// Workspace: qbar fp32 [B*H*nq][D], then kbar fp32 [B*H*nk][D].
size_t pooled_ws_bytes(const Geom& g) {
  return align_up((size_t)g.B * g.H * g.nq * g.D * sizeof(float), 256) +
         align_up((size_t)g.B * g.H * g.nk * g.D * sizeof(float), 256);
}

hipError_t launch_pooled_mass(const Geom& g, const void* Q, const void* K, float* P, void* ws, hipStream_t stream) {
  char* base = reinterpret_cast<char*>(ws);
  float* qbar = reinterpret_cast<float*>(base);
  float* kbar = reinterpret_cast<float*>(base + align_up((size_t)g.B * g.H * g.nq * g.D * sizeof(float), 256));
  if (g.bf16)
    return g.D == 128 ? launch<__bf16, 128>(g, Q, K, P, qbar, kbar, stream)
                      : launch<__bf16, 64>(g, Q, K, P, qbar, kbar, stream);
  return g.D == 128 ? launch<float, 128>(g, Q, K, P, qbar, kbar, stream)
                    : launch<float, 64>(g, Q, K, P, qbar, kbar, stream);
}

}  // namespace losa
