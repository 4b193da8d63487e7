// Packing of K (and V) into lane-major MFMA operand images, shared by the
// block-mass and sparse-attention kernels.
#pragma once

#include "losa_device.hpp"
#include "losa_internal.hpp"

namespace losa {

// 32-token chunks in the packed copies (even, so 64-token pack tiles cover them).
inline int packed_chunks(const Geom& g) { return (int)(align_up((size_t)g.nk * g.C, 64) / 32); }

// K and V -> lane-major operand copies, one 32-token chunk at a time, so that
// every operand load in the attention kernel is 64 lanes x 16 contiguous
// bytes (lane order), the pattern the vector memory path coalesces fully.
//   Kp[bh][c][kt][dc][lane][8]: row 32c + 8*((lane&15)>>2) + 4*kt + (lane&3)
//       of K, elements dc*32 + (lane>>4)*8 + [0,8) (the A operand of S^T = K Q^T
//       for key tile kt and k-step dc);
//   Vp[bh][c][dt][lane][8]: V[32c + (lane>>4)*8 + e][dt*16 + (lane&15)]
//       for e in [0,8) (the A operand of O^T += V^T P^T for dim tile dt).
// Tokens >= N are written as zeros.  Grid: (nch / 2, B*H) with nch even;
// each workgroup packs 64 tokens (two chunks), V through an LDS tile (rows
// read and staged 16 bytes at a time, then gathered column-wise).
// kWithV = false packs K only (Vp unused).
template <int D, bool kWithV>
__global__ __launch_bounds__(256) void pack_kv_kernel(const Geom g, const __bf16* __restrict__ K,
                                                      const __bf16* __restrict__ V, __bf16* __restrict__ Kp,
                                                      __bf16* __restrict__ Vp, int nch) {
  constexpr int DC = D / 32, DT = D / 16;
  constexpr int VP = D + 8;  // LDS row pitch (elements): rows stay 16-byte aligned
  __shared__ __attribute__((aligned(16))) uint16_t vt[64][VP];
  const int t0 = blockIdx.x * 64, bh = blockIdx.y;
  const int b = bh / g.H, h = bh - b * g.H;
  const __bf16* Kbh = K + b * g.ks[0] + h * g.ks[1];
  const __bf16* Vbh = kWithV ? V + b * g.vs[0] + h * g.vs[1] : nullptr;
  if (kWithV) {
    for (int idx = threadIdx.x; idx < 64 * D / 8; idx += 256) {
      const int tt = idx / (D / 8), d8 = idx - tt * (D / 8);
      const int tok = t0 + tt;
      bf16x8 v = bf16x8{};
      if (tok < g.N) v = load_bf16x8(Vbh + (int64_t)tok * g.vs[2] + d8 * 8);
      *reinterpret_cast<bf16x8*>(&vt[tt][d8 * 8]) = v;
    }
  }
  const int64_t cbase = (int64_t)bh * nch + (t0 >> 5);
  // K: 2 chunks x 2 key tiles x DC k-steps x 64 lanes pieces of 16 bytes.
  for (int idx = threadIdx.x; idx < 2 * 2 * DC * 64; idx += 256) {
    const int lane = idx & 63, rest = idx >> 6;
    const int dc = rest % DC, kt = (rest / DC) & 1, cc = rest / (2 * DC);
    const int lr = lane & 15;
    const int tok = t0 + cc * 32 + ((lr >> 2) << 3) + kt * 4 + (lr & 3);
    bf16x8 v = bf16x8{};
    if (tok < g.N) v = load_bf16x8(Kbh + (int64_t)tok * g.ks[2] + dc * 32 + (lane >> 4) * 8);
    *reinterpret_cast<bf16x8*>(Kp + ((cbase + cc) * 2 * DC * 64 + idx - cc * 2 * DC * 64) * 8) = v;
  }
  if (!kWithV) return;
  __syncthreads();
  // V: 2 chunks x DT dim tiles x 64 lanes pieces of 16 bytes.
  for (int idx = threadIdx.x; idx < 2 * DT * 64; idx += 256) {
    const int lane = idx & 63, dt = (idx >> 6) % DT, cc = idx / (DT * 64);
    const int dv = dt * 16 + (lane & 15), k0 = cc * 32 + (lane >> 4) * 8;
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = vt[k0 + j][dv];
    u32x4 pk;
    pk[0] = e[0] | ((uint32_t)e[1] << 16);
    pk[1] = e[2] | ((uint32_t)e[3] << 16);
    pk[2] = e[4] | ((uint32_t)e[5] << 16);
    pk[3] = e[6] | ((uint32_t)e[7] << 16);
    *reinterpret_cast<u32x4*>(Vp + ((cbase + cc) * DT * 64 + idx - cc * DT * 64) * 8) = pk;
  }
}

}  // namespace losa
