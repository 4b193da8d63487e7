// Frozen-pattern block-sparse attention (LoSA page, Methodology Summary:
// sparse attention with a frozen pattern -- each query attends to the valid
// tokens of its row's kept key blocks, softmax normalised over those keys
// only; discarded keys leave the denominator).
//
// bf16 matrix-core path (d in {64, 128}, R in {64, 128}):
//   * one workgroup (4 waves) per 64-query tile of a row (two per row when
//     R = 128); tiles are dispatched in the caller's budget order;
//   * the row's kept blocks are cut into 32-key chunks and the waves split
//     the chunks (wave w takes chunks w, w+4, ...).  Each wave keeps the
//     whole tile's Q as a B operand and its own online-softmax state
//     (running max m, sum l, O^T accumulators) for all 64 queries, and reads
//     its K chunk and V chunk straight from global memory into registers --
//     no LDS in the main loop;
//   * S^T = K Q^T and O^T += V^T P^T on 16x16x32 bf16 MFMA.  K rows are fed
//     in the permuted order kappa(kt, rho) = 8*(rho>>2) + 4*kt + (rho&3) so
//     that lane l ends up holding the eight consecutive keys 8*(l>>4)+[0,8)
//     of every query (l & 15): exactly the k-layout of the P^T operand, so P
//     goes from the S accumulators to the next MFMA without any exchange;
//   * V is consumed as V^T (keys contiguous per lane): a transpose kernel
//     writes a head_dim-major copy of V into the workspace first;
//   * the max is raised lazily: O and l are rescaled only when a new score
//     exceeds the running max by more than 8 (log2 units), so probabilities
//     stay below 2^8 and the rescale is rare after the first chunk;
//   * the four waves' partial states are merged through LDS at the end.
#include "losa_device.hpp"
#include "losa_internal.hpp"

namespace losa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazyMax = 8.0f;

// V [B,H,Na,D] (strided) -> Vt [B*H][D][Lt] bf16, zero for tokens >= N.
// 64x64 tiles through LDS.  Grid: (Lt/64, D/64, B*H), 256 threads.
__global__ __launch_bounds__(256) void transpose_v_kernel(const Geom g, const __bf16* __restrict__ V,
                                                          __bf16* __restrict__ Vt, int64_t Lt) {
  __shared__ uint16_t tile[64][66];
  const int t0 = blockIdx.x * 64, d0 = blockIdx.y * 64, bh = blockIdx.z;
  const int b = bh / g.H, h = bh - b * g.H;
  const __bf16* Vbh = V + b * g.vs[0] + h * g.vs[1];
  const uint16_t* Vu = reinterpret_cast<const uint16_t*>(Vbh);
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    const int tt = idx >> 6, dd = idx & 63;
    const int tok = t0 + tt;
    tile[tt][dd] = tok < g.N ? Vu[(int64_t)tok * g.vs[2] + d0 + dd] : (uint16_t)0;
  }
  __syncthreads();
  uint16_t* out = reinterpret_cast<uint16_t*>(Vt) + ((int64_t)bh * g.D + d0) * Lt;
  for (int idx = threadIdx.x; idx < 64 * 64; idx += 256) {
    const int dd = idx >> 6, tt = idx & 63;
    out[(int64_t)dd * Lt + t0 + tt] = tile[tt][dd];
  }
}

template <int D>
struct AttnState {
  static constexpr int DT = D / 16;
  f32x4 o[DT][4];  // O^T: lane holds query (l & 15) of tile qt, dims dt*16 + 4*(l>>4) + r
  float m[4], l[4];
};

template <int D>
__global__ __launch_bounds__(256) void attn_bf16_kernel(const Geom g, const __bf16* __restrict__ Q,
                                                        const __bf16* __restrict__ K,
                                                        const __bf16* __restrict__ Vt, int64_t Lt,
                                                        const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ col_idx,
                                                        const int32_t* __restrict__ order, void* O,
                                                        int o_bf16) {
  constexpr int DC = D / 32, DT = D / 16;
  extern __shared__ float lds[];  // merge slot: [64][D + 4] floats + m[64] + l[64]
  const int qhalves = g.R / 64;
  const int tix = blockIdx.x;
  const int ridx = tix / qhalves, qh = tix - ridx * qhalves;
  const int row = order ? order[ridx] : ridx;
  const int bh = row / g.nq, i = row - bh * g.nq;
  const int b = bh / g.H, h = bh - b * g.H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const __bf16* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const __bf16* Kbh = K + b * g.ks[0] + h * g.ks[1];
  const __bf16* Vbh = Vt + (int64_t)bh * D * Lt;
  const int row0 = i * g.R + qh * 64;

  // Q as the B operand of S^T = K Q^T (padding rows -> 0).
  bf16x8 qop[4][DC];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int qrow = row0 + qt * 16 + lr;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      bf16x8 v = load_bf16x8(Qbh + (int64_t)qrow * g.qs[2] + dc * 32 + lg * 8);
      if (qrow >= g.N) v = bf16x8{};
      qop[qt][dc] = v;
    }
  }

  AttnState<D> st;
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    st.m[qt] = kNegInf;
    st.l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const float c = g.scale_log2;
  const int beg = row_ptr[row], end = row_ptr[row + 1];
  const int sub = g.C / 32;
  const int nchunk = (end - beg) * sub;
  // K row fed to A-operand row rho of key tile kt.
  const int krow0 = ((lr >> 2) << 3) + (lr & 3);

  for (int u = w; u < nchunk; u += 4) {
    const int p = u / sub, sc = u - p * sub;
    const int j = col_idx[beg + p];
    const int kb = j * g.C + sc * 32;
    if (kb >= g.N) continue;  // chunk lies wholly in the padding of the last block

    bf16x8 kop[2][DC];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        kop[kt][dc] = load_bf16x8(Kbh + (int64_t)(kb + krow0 + kt * 4) * g.ks[2] + dc * 32 + lg * 8);
    bf16x8 vop[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vop[dt] = load_bf16x8(Vbh + (int64_t)(dt * 16 + lr) * Lt + kb + lg * 8);

    f32x4 acc[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) a = mfma_bf16(kop[kt][dc], qop[qt][dc], a);
        acc[kt][qt] = a;
      }

    // acc[kt][qt][r] is the score of key kb + 8*lg + 4*kt + r.
    const bool partial = kb + 32 > g.N;
    float x[4][8];
    float mx[4];
    bool need = false;
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = acc[kt][qt][r] * c;
          if (partial && kb + lg * 8 + kt * 4 + r >= g.N) v = kNegInf;
          x[qt][kt * 4 + r] = v;
        }
      float t = fmaxf(fmaxf(fmaxf(x[qt][0], x[qt][1]), fmaxf(x[qt][2], x[qt][3])),
                      fmaxf(fmaxf(x[qt][4], x[qt][5]), fmaxf(x[qt][6], x[qt][7])));
      t = fmaxf(t, __shfl_xor(t, 16, kWave));
      t = fmaxf(t, __shfl_xor(t, 32, kWave));
      mx[qt] = t;
      need |= t > st.m[qt] + kLazyMax;
    }
    if (__any(need)) {
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        if (mx[qt] > st.m[qt] + kLazyMax) {
          const float alpha = fast_exp2(st.m[qt] - mx[qt]);  // 0 on the first chunk
          st.l[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) st.o[dt][qt] *= alpha;
          st.m[qt] = mx[qt];
        }
      }
    }
    bf16x8 pop[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      float pe[8];
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pe[e] = fast_exp2(x[qt][e] - st.m[qt]);
        rs += pe[e];
      }
      st.l[qt] += rs;
      u32x4 pk;
      pk[0] = pack_bf16x2(pe[0], pe[1]);
      pk[1] = pack_bf16x2(pe[2], pe[3]);
      pk[2] = pack_bf16x2(pe[4], pe[5]);
      pk[3] = pack_bf16x2(pe[6], pe[7]);
      pop[qt] = __builtin_bit_cast(bf16x8, pk);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) st.o[dt][qt] = mfma_bf16(vop[dt], pop[qt], st.o[dt][qt]);
  }

  // Row sums: combine the four lane groups that share each query.
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    st.l[qt] += __shfl_xor(st.l[qt], 16, kWave);
    st.l[qt] += __shfl_xor(st.l[qt], 32, kWave);
  }

  // Merge the waves' partial states: 3 -> 2 -> 1 -> 0 through one LDS slot.
  constexpr int LD = D + 4;
  float* so = lds;
  float* sm = lds + 64 * LD;
  float* sl = sm + 64;
  for (int src = 3; src >= 1; --src) {
    __syncthreads();
    if (w == src) {
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int qi = qt * 16 + lr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<f32x4*>(so + qi * LD + dt * 16 + lg * 4) = st.o[dt][qt];
        if (lg == 0) { sm[qi] = st.m[qt]; sl[qi] = st.l[qt]; }
      }
    }
    __syncthreads();
    if (w == src - 1) {
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int qi = qt * 16 + lr;
        const float mo = sm[qi], lo = sl[qi];
        const float mn = fmaxf(st.m[qt], mo);
        const float a = st.m[qt] == kNegInf ? 0.f : fast_exp2(st.m[qt] - mn);
        const float ao = mo == kNegInf ? 0.f : fast_exp2(mo - mn);
        st.m[qt] = mn;
        st.l[qt] = st.l[qt] * a + lo * ao;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f32x4 oo = *reinterpret_cast<const f32x4*>(so + qi * LD + dt * 16 + lg * 4);
          st.o[dt][qt] = st.o[dt][qt] * a + oo * ao;
        }
      }
    }
  }

  if (w == 0) {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const int qrow = row0 + qt * 16 + lr;
      const float inv = (qrow < g.N && st.l[qt] > 0.f) ? 1.0f / st.l[qt] : 0.f;
      const int64_t obase = b * g.os[0] + h * g.os[1] + (int64_t)qrow * g.os[2];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 v = st.o[dt][qt] * inv;
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
  const int beg = row_ptr[row], end = row_ptr[row + 1];
  for (int p = beg; p < end; ++p) {
    const int j = col_idx[p];
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

int64_t vt_len(const Geom& g) { return (int64_t)align_up((size_t)g.nk * g.C, 64); }

template <int D>
hipError_t launch_mfma(const Geom& g, const void* Q, const void* K, const void* V, const int32_t* row_ptr,
                       const int32_t* col_idx, const int32_t* order, void* O, int o_bf16, void* ws,
                       hipStream_t st) {
  const int64_t Lt = vt_len(g);
  __bf16* Vt = reinterpret_cast<__bf16*>(ws);
  hipLaunchKernelGGL(transpose_v_kernel, dim3((unsigned)(Lt / 64), D / 64, g.B * g.H), dim3(256), 0, st, g,
                     (const __bf16*)V, Vt, Lt);
  const size_t lds = (size_t)(64 * (D + 4) + 128) * sizeof(float);
  hipLaunchKernelGGL((attn_bf16_kernel<D>), dim3(g.rows() * (g.R / 64)), dim3(256), lds, st, g,
                     (const __bf16*)Q, (const __bf16*)K, (const __bf16*)Vt, Lt, row_ptr, col_idx, order, O,
                     o_bf16);
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
  return (size_t)g.B * g.H * g.D * (size_t)vt_len(g) * sizeof(uint16_t);
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
