// Final step of the one-pass block masses (shared by the mass and the
// construction kernels): a wave has written, for each of its key blocks j,
// the per-query sums S[j][q] (q = 0..63, relative to the wave's references)
// and knows each query's factor f[q] = 2^(m_q - lse_q) (0 for padding rows).
// The block's mass over these 64 queries is sum_q S[j][q] * f[q].
#pragma once

#include "losa_device.hpp"

namespace losa {

// Lane l takes the wave's block number b0 + l (block j = block_of(b0 + l)):
// its 64 sums are 256 contiguous bytes, read as 16 independent 16-byte loads,
// against f from LDS (the same address in every lane, so the reads
// broadcast).  One memory round trip per 64 blocks and no cross-lane
// reduction.  dst[j] = scale * mass of block j.
template <typename BlockOf>
__device__ __forceinline__ void blocks_from_sums(const float* __restrict__ Sg, const float* f, int nb, float scale,
                                                 float* dst, int lane, BlockOf block_of) {
  for (int b0 = 0; b0 < nb; b0 += kWave) {
    const int bb = b0 + lane;
    if (bb < nb) {
      const int j = block_of(bb);
      const f32x4* src = reinterpret_cast<const f32x4*>(Sg + (int64_t)j * 64);
      f32x4 s4[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) s4[c] = src[c];
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const f32x4 f4 = *reinterpret_cast<const f32x4*>(f + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(s4[c][e], f4[e], acc);
      }
      dst[j] = acc * scale;
    }
  }
}

// The wave's blocks are kw, kw+4, ... (every key block in turn).
__device__ __forceinline__ void blocks_from_sums(const float* __restrict__ Sg, const float* f, int kw, int nb,
                                                 float scale, float* dst, int lane) {
  blocks_from_sums(Sg, f, nb, scale, dst, lane, [kw](int bb) { return kw + 4 * bb; });
}

}  // namespace losa
