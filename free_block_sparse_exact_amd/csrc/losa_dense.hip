// Dense self-attention that also accumulates the exact block masses, in one
// pass over K and V: the construction step of the LoSA page (Methodology
// Summary: the pattern is built at one dense step from exact block masses;
// Experiments Summary: the construction step's kernel is a full attention
// pass that also sums the exact block masses).
//
//   O(q)    = softmax over all valid keys of s = q.k * scale, times V;
//   M[i,j]  = (1/valid rows of block i) * sum over rows q of block i and
//             valid keys k of block j of exp(s_qk - lse_q)
// (M is exactly what losa_block_mass computes).
//
// bf16 matrix-core path (d in {64, 128}, R in {64, 128}): the sparse
// attention kernel's structure over the full key range.  One workgroup (four
// waves, one per SIMD) per 64-query tile; wave kw takes the key BLOCKS
// j = kw, kw+4, ... (all their 32-key chunks).  The four waves share one
// fixed reference m per query: the largest score of their first chunks
// (log2 units), exchanged through LDS before the main loop, with no
// headroom.  Being an actual score of the row, m is at most its log-sum-exp,
// so each term p = 2^(s*c - m) is at least the probability it stands for: a
// key of probability >= 2^-126 is never flushed by the exponential, and the
// block sums keep fp32's relative precision down to there (at most C * 2^-126
// is lost per mass, from keys of smaller probability).  p rounded to bf16
// feeds the P.V product and its normaliser (the row sums, taken on the
// matrix cores by one more MFMA per query tile against a block of ones), p
// in fp32 feeds the block sums.  At the end of a block the wave stores the
// block sum of each query to the workspace S (as the mass kernel does); with
// one reference the partial O, row sums and row totals of the four waves
// simply add, and M follows from S divided by the row total.  If a wave's
// row sum ends above 2^100 or not finite (a score ~100 above the first
// chunks' maximum, or a non-finite input) or O is not finite, the whole
// workgroup recomputes against the exact maximum of the row.
//
// Padding keys of the last block score exactly 0 against the zero rows of
// the packed K and must leave the softmax: the wave that owns the last block
// processes it first, its partly padded chunk at the very front (the first
// chunk is masked explicitly), so the pipelined loop does no masking.
//
// With CSR lists (kLists) the same kernel runs over each row's listed blocks
// only: O is then the frozen-pattern sparse attention, and M the masses
// within the lists -- the softmax of that attention summed per listed block
// (0 outside the list), the exact weights a reduced search (GSRS card: a
// top-p search that, after the first, looks only among blocks an earlier
// search kept, its weights taken from the attention pass) selects from.
#include "losa_blocksum.hpp"
#include "losa_device.hpp"
#include "losa_internal.hpp"
#include "losa_pack.hpp"

namespace losa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
// A row sum above this bound (or not finite) after the wave's chunks sends the
// workgroup to the exact path: with every probability at most 2^100, neither
// P, nor P.V, nor a block sum can have overflowed.
constexpr float kLBound = 1.2676506e30f;  // 2^100

template <int D, bool kLists>
__global__ __launch_bounds__(256, 1) void dense_bf16_kernel(const Geom g, const __bf16* __restrict__ Q,
                                                            const __bf16* __restrict__ Kp,
                                                            const __bf16* __restrict__ Vp, int nch,
                                                            const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ col_idx,
                                                            const int32_t* __restrict__ order,
                                                            float* __restrict__ S, float* __restrict__ Mout,
                                                            void* O, int o_bf16) {
  constexpr int DC = D / 32, DT = D / 16, kQT = 4;
  constexpr int LD = D + 4;       // merge slot row stride (floats)
  extern __shared__ float lds[];  // merge slots [4][64][LD] f32, maxima [4][64], row sums [4][64]
  __shared__ float s_ref[4][64], s_tot[4][64], s_f[4][64];
  __shared__ int s_over;
  const int qhalves = g.R / 64;
  const int rows = g.rows();
  // Lists come in the caller's work order (rows by budget), dealt to the XCDs
  // in blocks of 32 tasks like the sparse attention; dense rows are spread
  // in contiguous ranges per XCD.
  const int tix = kLists ? xcd_block_task(blockIdx.x, gridDim.x) : xcd_task(blockIdx.x, rows * qhalves);
  const int ridx = tix / qhalves, qsub = tix - ridx * qhalves;
  const int row = (kLists && order) ? order[ridx] : ridx;
  const int bh = row / g.nq, i = row - bh * g.nq;
  const int b = bh / g.H, h = bh - b * g.H;
  const int lane = threadIdx.x & 63, kw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const __bf16* Qbh = Q + b * g.qs[0] + h * g.qs[1];
  const __bf16* Kbh = Kp + (int64_t)bh * nch * (32 * D);
  const __bf16* Vbh = Vp + (int64_t)bh * nch * (32 * D);
  const int row0 = i * g.R + qsub * 64;
  float* Sg = S + (int64_t)tix * g.nk * 64;  // [nk][64] of this query tile

  // Q as the B operand of S^T = K Q^T (padding rows -> 0), kept in AGPRs.
  bf16x8 qop[kQT][DC];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qrow = row0 + qt * 16 + lr;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      bf16x8 v = load_bf16x8(Qbh + (int64_t)qrow * g.qs[2] + dc * 32 + lg * 8);
      if (qrow >= g.N) v = bf16x8{};
      asm("" : "+a"(v));
      qop[qt][dc] = v;
    }
  }

  f32x4 o[DT][kQT];
  float m[kQT], l[kQT], blk[kQT], tot = 0.f;
  f32x4 lsum[kQT];  // row sums of the bf16 P from the matrix cores (see pv)
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    m[qt] = kNegInf;
    l[qt] = 0.f;
    lsum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    blk[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c = g.scale_log2;

  // The row's blocks: every block (dense), or the listed ones.  Wave kw owns
  // list positions kw, kw+4, ... with all their valid chunks.  The last key
  // block (nk - 1) is partly padding unless N = nk*C: the wave that owns it
  // takes it first, its final (partly padded) chunk at the very front, and
  // drops its wholly padded chunks, so only the first chunk needs masking.
  const int beg = kLists ? row_ptr[row] : 0;
  const int n = kLists ? row_ptr[row + 1] - beg : g.nk;
  auto block_at = [&](int pos) -> int { return kLists ? col_idx[beg + pos] : pos; };
  const int sub = g.C / 32, sub_shift = __builtin_ctz(sub), c_shift = __builtin_ctz(g.C);
  const int nb = n > kw ? (n - kw + 3) / 4 : 0;
  const int last = g.nk - 1;
  const int sub_last = (g.N - last * g.C + 31) / 32;  // valid chunks of the last block
  int lp = -1;                                        // position of the last block in the row
  if (g.N != g.nk * g.C) {
    if (!kLists) {
      lp = last;
    } else {
      for (int base = 0; base < n; base += 4 * kWave) {
        uint64_t hit[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int x = base + jj * kWave + lane;
          hit[jj] = __ballot(x < n && col_idx[beg + x] == last);
        }
#pragma unroll
        for (int jj = 3; jj >= 0; --jj)
          if (hit[jj]) lp = base + jj * kWave + __builtin_ctzll(hit[jj]);
        if (lp >= 0) break;
      }
    }
  }
  const bool own_last = lp >= 0 && (lp & 3) == kw;
  const int o_last = lp >> 2;  // ordinal of the last block among this wave's blocks (when own_last)
  const int nmine = own_last ? (nb - 1) * sub + sub_last : nb * sub;
  // Chunk t of the wave -> its first key, with bit 0 set if it closes its block.
  auto seq_key = [&](int t) -> int {
    t = t < nmine ? t : nmine - 1;
    int j, sc;
    bool ends;
    if (own_last && t < sub_last) {
      j = last;
      sc = t == 0 ? sub_last - 1 : t - 1;
      ends = t == sub_last - 1;
    } else {
      const int tt = own_last ? t - sub_last : t;
      int ord = tt >> sub_shift;
      ord += (own_last && ord >= o_last) ? 1 : 0;
      j = block_at(kw + 4 * ord);
      sc = tt & (sub - 1);
      ends = sc == sub - 1;
    }
    return (j * g.C + 32 * sc) | (ends ? 1 : 0);
  };
  // The loop reads chunk keys from registers: lane x of a window holds
  // seq_key(base + x), so a key costs one lane read (two windows cover 128
  // chunks; the next is loaded 64 iterations before it is needed).
  auto key_window = [&](int base) -> int { return seq_key(base + lane); };

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
  // acc[kt][qt][r] = score of key kb + 8*lg + 4*kt + r for query qt*16 + lr.
  auto scores = [&](const bf16x8 (&kop)[2][DC], f32x4 (&acc)[2][kQT]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) acc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) acc[kt][qt] = mfma_bf16(kop[kt][dc], qop[qt][dc], acc[kt][qt]);
    }
  };
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
  // p = 2^(s*c - m): fp32 into the block sums, bf16 into P (and, by pv, into
  // the row sums).
  auto probs = [&](const f32x4 (&acc)[2][kQT], bf16x8 (&pop)[kQT]) {
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      const float nm = -m[qt];
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(__builtin_fmaf(acc[e >> 2][qt][e & 3], c, nm));
      blk[qt] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
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
  // every row of lsum[qt] the column sums of P^T (each lane ends with its
  // query's full sum over the wave's chunks).
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
  // Block end: lane (lg, lr) stores the block sum of query lg*16 + lr (sums
  // over the four lane groups formed by a transpose-reduce: two values swapped
  // with the lane 32 away, then one with the lane 16 away).
  auto block_end = [&](int j) {
    const float v = rows_sum_own(blk);
    tot += v;
    Sg[(int64_t)j * 64 + lane] = v;
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) blk[qt] = 0.f;
  };

  // The query's common reference from the four waves' entries in s_ref.
  auto common_ref = [&]() {
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      float mm = s_ref[0][qt * 16 + lr];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) mm = fmaxf(mm, s_ref[ww][qt * 16 + lr]);
      m[qt] = mm;
    }
  };
  auto publish_ref = [&](const float (&mx)[kQT]) {  // lane (lg, lr) writes query lg*16 + lr's entry
    s_ref[kw][lane] = (lg == 0 ? mx[0] : lg == 1 ? mx[1] : lg == 2 ? mx[2] : mx[3]) * c;
  };
  bf16x8 kop[2][DC], vop[DT];
  f32x4 acc[2][kQT];
  {
    float mx[kQT];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) mx[qt] = kNegInf;
    if (nmine > 0) {
      const int kb = seq_key(0) & ~1;
      load_k(kb, kop);
      load_v(kb, vop);
      scores(kop, acc);
      load_k(seq_key(1) & ~1, kop);
      if (kb + 32 > g.N) mask_tail(kb, acc);
      chunk_max(acc, mx);
      lanes_max(mx);  // finite: the chunk holds a valid key
    }
    publish_ref(mx);
    if (threadIdx.x == 0) s_over = 0;
  }
  __syncthreads();
  common_ref();
  if (nmine > 0) {
    bool over_any = false;
    int win_base = 0;
    int win0 = key_window(0), win1 = key_window(64);
    for (int t = 0; t < nmine; ++t) {
      if (t == win_base + 64) {  // keys t..t+2 now lie in [win_base + 64, win_base + 128)
        win_base += 64;
        win0 = win1;
        win1 = key_window(win_base + 64);
      }
      auto key_at = [&](int x) {  // both windows read, then a select: no branch inside the body
        const int r = x - win_base;
        const int k0 = __builtin_amdgcn_readlane(win0, r & 63), k1 = __builtin_amdgcn_readlane(win1, r & 63);
        return r < 64 ? k0 : k1;
      };
      f32x4 accn[2][kQT];
      scores(kop, accn);  // chunk t+1 (the last iteration recomputes the last chunk)
      load_k(key_at(t + 2) & ~1, kop);
      bf16x8 pop[kQT];
      probs(acc, pop);  // chunk t
      pv(vop, pop);
      load_v(key_at(t + 1) & ~1, vop);
      // Three vector instructions per MFMA: the block sums add 32 to the
      // sparse attention loop's ~110 per 64 MFMAs, and with two per MFMA the
      // rest bunched up in one stretch (config 3: 179 against 170 ms).
#pragma unroll
      for (int s = 0; s < 64 + kQT; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // then three vector ALU ops
      }
      const int kt_cur = key_at(t);
      if (kt_cur & 1) block_end(kt_cur >> c_shift);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) acc[kt][qt] = accn[kt][qt];
    }
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) over_any |= !(lsum[qt][0] <= kLBound);
    // O itself must be finite (its probabilities may reach 2^100)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
        for (int e = 0; e < 4; ++e) over_any |= !(__builtin_fabsf(o[dt][qt][e]) <= 3.0e38f);
    if (__any(over_any) && lane == 0) s_over = 1;
  }
  __syncthreads();
  if (s_over) {
    // Exact maximum of the row over every wave's keys, then O, the row sums
    // and the block sums again against it (all probabilities <= 1).
    tot = 0.f;
    float mx[kQT];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      lsum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      mx[qt] = kNegInf;
      blk[qt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int t = 0; t < nmine; ++t) {
      const int kb2 = seq_key(t) & ~1;
      load_k(kb2, kop);
      f32x4 acc2[2][kQT];
      scores(kop, acc2);
      if (kb2 + 32 > g.N) mask_tail(kb2, acc2);
      chunk_max(acc2, mx);
    }
    lanes_max(mx);
    publish_ref(mx);  // every wave read the first references before the barrier above
    __syncthreads();
    common_ref();
    for (int t = 0; t < nmine; ++t) {
      const int key = seq_key(t);
      const int kb2 = key & ~1, jt = key >> c_shift;
      const bool ends = (key & 1) != 0;
      load_k(kb2, kop);
      load_v(kb2, vop);
      f32x4 acc2[2][kQT];
      scores(kop, acc2);
      if (kb2 + 32 > g.N) mask_tail(kb2, acc2);
      bf16x8 pop[kQT];
      probs(acc2, pop);
      pv(vop, pop);
      if (ends) block_end(jt);
    }
  }

  // Row sums of P: every lane already holds its query's sum over the wave's chunks.
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) l[qt] = lsum[qt][0];
  // Block-sum total of the query this lane stored (lg*16 + lr).
  s_tot[kw][lane] = tot;

  // Merge the four key groups for O in one step: every wave parks its partial
  // O and row sums in its own LDS slot, then wave kw adds up dims
  // [kw*D/4, (kw+1)*D/4) of all 64 queries from the four slots and stores
  // them (one reference for all four: plain sums).
  {
    constexpr int DTW = DT / 4;
    float* slot = lds + kw * (64 * LD);
    float* sl = lds + 4 * 64 * LD + 4 * 64;  // [4][64] row sums
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      const int qi = qt * 16 + lr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(slot + qi * LD + dt * 16 + lg * 4) = o[dt][qt];
      if (lg == 0) sl[kw * 64 + qi] = l[qt];
    }
    __syncthreads();
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      const int qi = qt * 16 + lr;
      const float lt = (sl[qi] + sl[64 + qi]) + (sl[128 + qi] + sl[192 + qi]);
      const int qrow = row0 + qi;
      const float inv = (qrow < g.N && lt > 0.f) ? 1.0f / lt : 0.f;
      const int64_t obase = b * g.os[0] + h * g.os[1] + (int64_t)qrow * g.os[2];
#pragma unroll
      for (int dd = 0; dd < DTW; ++dd) {
        const int dt = kw * DTW + dd;
        const float* src = lds + qi * LD + dt * 16 + lg * 4;
        f32x4 v = (*reinterpret_cast<const f32x4*>(src) + *reinterpret_cast<const f32x4*>(src + 64 * LD)) +
                  (*reinterpret_cast<const f32x4*>(src + 2 * 64 * LD) +
                   *reinterpret_cast<const f32x4*>(src + 3 * 64 * LD));
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

  // Masses: the stored query's factor 1 / (its row total against the common
  // reference; 0 for padding rows), then M from S (s_tot was written before
  // the merge's barrier).
  {
    const float lt = (s_tot[0][lane] + s_tot[1][lane]) + (s_tot[2][lane] + s_tot[3][lane]);
    s_f[kw][lane] = (row0 + lane < g.N && lt > 0.f) ? 1.0f / lt : 0.f;
    __syncthreads();  // every lane reads all 64 factors of its wave
    const float inv_rows = 1.0f / (float)min(g.R, g.N - i * g.R);
    float* Mrow = Mout + ((int64_t)qsub * rows + row) * g.nk;
    if (kLists) {  // blocks outside the list get 0, then the listed ones their mass
      for (int x = threadIdx.x; x < g.nk; x += blockDim.x) Mrow[x] = 0.f;
      __syncthreads();
      blocks_from_sums(Sg, s_f[kw], nb, inv_rows, Mrow, lane, [&](int bb) { return block_at(kw + 4 * bb); });
    } else {
      blocks_from_sums(Sg, s_f[kw], kw, nb, inv_rows, Mrow, lane);
    }
  }
}

// M = Mh[0] + Mh[1]: the two 64-query halves of 128-row query blocks (two
// addends, so the order of addition cannot change the result).
__global__ __launch_bounds__(256) void add_halves_kernel(const float* __restrict__ Mh, float* __restrict__ M,
                                                         int64_t n) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < n) M[k] = Mh[k] + Mh[n + k];
}

struct DenseWs {
  __bf16* Kp;
  __bf16* Vp;
  float* S;
  float* Mh;  // R = 128 only
};

size_t dense_layout(const Geom& g, char* base, DenseWs* w) {
  const size_t packed = (size_t)g.B * g.H * packed_chunks(g) * 32 * g.D * sizeof(uint16_t);
  const size_t s = align_up((size_t)g.B * g.H * g.nq * g.R * g.nk * sizeof(float), 256);
  const size_t mh = g.R == 64 ? 0 : align_up((size_t)2 * g.rows() * g.nk * sizeof(float), 256);
  if (w) {
    w->Kp = reinterpret_cast<__bf16*>(base);
    w->Vp = reinterpret_cast<__bf16*>(base + align_up(packed, 256));
    w->S = reinterpret_cast<float*>(base + 2 * align_up(packed, 256));
    w->Mh = reinterpret_cast<float*>(base + 2 * align_up(packed, 256) + s);
  }
  return 2 * align_up(packed, 256) + s + mh;
}

template <int D>
hipError_t launch_mfma(const Geom& g, const void* Q, const void* K, const void* V, const int32_t* row_ptr,
                       const int32_t* col_idx, const int32_t* order, float* M, void* O, int o_bf16, void* ws,
                       hipStream_t st) {
  DenseWs w;
  dense_layout(g, reinterpret_cast<char*>(ws), &w);
  const int nch = packed_chunks(g);
  hipLaunchKernelGGL((pack_kv_kernel<D, true>), dim3((unsigned)(nch / 2), g.B * g.H), dim3(256), 0, st, g,
                     (const __bf16*)K, (const __bf16*)V, w.Kp, w.Vp, nch);
  const int tiles = g.rows() * (g.R / 64);
  const size_t lds = (size_t)(4 * 64 * (D + 4) + 512) * sizeof(float);  // 137 KB at d = 128
  float* Mout = g.R == 64 ? M : w.Mh;
  if (row_ptr)
    hipLaunchKernelGGL((dense_bf16_kernel<D, true>), dim3(tiles), dim3(256), lds, st, g, (const __bf16*)Q,
                       (const __bf16*)w.Kp, (const __bf16*)w.Vp, nch, row_ptr, col_idx, order, w.S, Mout, O,
                       o_bf16);
  else
    hipLaunchKernelGGL((dense_bf16_kernel<D, false>), dim3(tiles), dim3(256), lds, st, g, (const __bf16*)Q,
                       (const __bf16*)w.Kp, (const __bf16*)w.Vp, nch, nullptr, nullptr, nullptr, w.S, Mout, O,
                       o_bf16);
  if (g.R != 64) {
    const int64_t n = (int64_t)g.rows() * g.nk;
    hipLaunchKernelGGL(add_halves_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const float*)w.Mh, M, n);
  }
  return hipGetLastError();
}

}  // namespace

size_t dense_ws_bytes(const Geom& g) {
  if (mfma_path(g)) return dense_layout(g, nullptr, nullptr);
  return mass_ws_bytes(g);  // the separate mass and attention kernels
}

hipError_t launch_dense_attn_mass(const Geom& g, const void* Q, const void* K, const void* V, float* M, void* O,
                                  int o_bf16, void* ws, hipStream_t stream) {
  if (mfma_path(g))
    return g.D == 128 ? launch_mfma<128>(g, Q, K, V, nullptr, nullptr, nullptr, M, O, o_bf16, ws, stream)
                      : launch_mfma<64>(g, Q, K, V, nullptr, nullptr, nullptr, M, O, o_bf16, ws, stream);
  // Other shapes: the SIMT mass kernels, then the SIMT attention kernel over
  // every key block (no lists).
  hipError_t e = launch_block_mass(g, Q, K, M, ws, stream);
  if (e != hipSuccess) return e;
  return launch_sparse_attn(g, Q, K, V, nullptr, nullptr, nullptr, O, o_bf16, nullptr, stream);
}

size_t sparse_mass_ws_bytes(const Geom& g) { return mfma_path(g) ? dense_layout(g, nullptr, nullptr) : 0; }

hipError_t launch_sparse_attn_mass(const Geom& g, const void* Q, const void* K, const void* V,
                                   const int32_t* row_ptr, const int32_t* col_idx, const int32_t* order,
                                   float* M, void* O, int o_bf16, void* ws, hipStream_t stream) {
  return g.D == 128 ? launch_mfma<128>(g, Q, K, V, row_ptr, col_idx, order, M, O, o_bf16, ws, stream)
                    : launch_mfma<64>(g, Q, K, V, row_ptr, col_idx, order, M, O, o_bf16, ws, stream);
}

}  // namespace losa
