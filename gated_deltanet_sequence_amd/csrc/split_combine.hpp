// Middle step of the sequence-split forward pass: the start states of the
// segments of each sequence.  Segment g maps a state S entering it to
// S M_g + tilde_g (M_g: its transition, tilde_g: its state from a zero
// start; both computed by the pipelined kernel in MAP_SPLIT_A mode), so
//   start_0 = S_0,   start_{g+1} = start_g M_g + tilde_g.
// [P1] §2.3 (composition of affine maps) and §3.3 (splitting a long
// sequence into parts evaluated in parallel, then joined).
//
// Each row of a state evolves alone (the transition multiplies from the
// right), so a workgroup owns ROWS rows of one sequence and walks all its
// segments without synchronising with other workgroups.  fp32 throughout.
//
// The walk is a chain of G-1 dependent steps, so the time of one step is
// what counts.  A step is a small dense product, [ROWS x D] = [ROWS x D]
// [D x D] + [ROWS x D], done with the fp32 MFMA v_mfma_f32_16x16x4f32: one
// wave per 16-column tile of the result, D / 4 MFMAs per step.  M_g is
// staged in LDS with coalesced 16-byte loads (16-column blocks swizzled so
// that the four k rows a B fragment spans fall in different banks), and the
// next segments' M and tilde are loaded into registers several steps ahead.
// The rows' current state stays in LDS transposed (prevT[k][i]), so that the
// A fragment of every MFMA is one contiguous 256-byte read.  Both LDS
// buffers are doubled, which leaves one barrier per step and lets the next
// M go to LDS while the MFMAs run.
#pragma once

#include "gdn_common.hpp"

namespace gdn {
namespace split {

constexpr int ROWS = 16;  // rows of a state per workgroup: one MFMA tile

// Threads of a workgroup: one wave per 16-column tile.
template <int D>
constexpr int threads_for() {
  return 64 * (D / 16);
}

// Loads into registers the transition of segment `seg` (all of it, as 16-byte
// vectors in a coalesced order) and this thread's four entries of its
// zero-start state (rows r0 + ib .. r0 + ib + 3, column jj).
template <int D>
__device__ __forceinline__ void fetch_step(f32x4 (&mr)[D * D / 4 / threads_for<D>()], f32x4& tr,
                                           const float* trans, const float* tilde, int64_t seg, int r0, int t,
                                           int ib, int jj) {
  constexpr int64_t DD = (int64_t)D * D;
  constexpr int NT = threads_for<D>();
  const f32x4* M = reinterpret_cast<const f32x4*>(trans + seg * DD);
#pragma unroll
  for (int v = 0; v < D * D / 4 / NT; ++v) mr[v] = M[t + NT * v];
  const float* Tl = tilde + seg * DD + (int64_t)(r0 + ib) * D + jj;
  tr = f32x4{Tl[0], Tl[D], Tl[2 * D], Tl[3 * D]};
}

// Where M_g[k][n] sits in an LDS buffer of M: row-major, its 16-column
// blocks XOR-swizzled by k & 3, so that the four k rows one B fragment spans
// fall in different banks.
template <int D>
__device__ __forceinline__ int m_at(int k, int n) {
  return k * D + (n ^ (16 * (k & 3)));
}

// One step of the walk: start_{g+1} = start_g M_g + tilde_g for this
// workgroup's rows.  M_g is in LDS buffer Mc and start_g in Pc; the step
// writes start_{g+1} to Pn and, while it runs its MFMAs, M_{g+1} (from the
// registers mr) to Mn.  Every buffer it reads was written before the last
// barrier and every buffer it writes was last read before it, so one
// barrier per step suffices.  The registers (mr, tr) are then refilled with
// segment `next`; the refill is unconditional (past the last segment the
// caller passes the last one again): a conditional one leaves the compiler
// merging register sets, which makes it wait for every load in flight.
template <int D>
__device__ __forceinline__ void combine_step(f32x4 (&mr)[D * D / 4 / threads_for<D>()], f32x4& tr,
                                             const f32x4 (&mn)[D * D / 4 / threads_for<D>()],
                                             const float* Mc, float* Mn, const float* Pc, float* Pn, float* out,
                                             const float* trans, const float* tilde, int64_t next, bool store_next,
                                             int r0, int t, int ib, int jj) {
  constexpr int NT = threads_for<D>();
  constexpr int NV = D * D / 4 / NT;
  const int lane = t % 64, ct = t / 64;
  f32x4 acc = tr;
  // A[i][kk] = start_g[i][4 kb + kk] (i = lane % 16, kk = lane / 16),
  // B[kk][j] = M_g[4 kb + kk][16 ct + j] (j = lane % 16)
  const float* pa = Pc + lane;
  const int kk = lane / 16, n = 16 * ct + lane % 16;
#pragma unroll
  for (int kb = 0; kb < D / 4; ++kb)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[64 * kb], Mc[m_at<D>(4 * kb + kk, n)], acc, 0, 0, 0);
  if (store_next) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e = 4 * (t + NT * v);
      *reinterpret_cast<f32x4*>(&Mn[m_at<D>(e / D, e % D)]) = mn[v];
    }
  }
  // refill once mr and tr are dead, so that the loads land in place
  fetch_step<D>(mr, tr, trans, tilde, next, r0, t, ib, jj);
  // acc[r] = start_{g+1}[ib + r][jj]
  *reinterpret_cast<f32x4*>(&Pn[jj * 16 + ib]) = acc;
#pragma unroll
  for (int r = 0; r < 4; ++r) out[(ib + r) * D + jj] = acc[r];
  __syncthreads();
}

// ws layout (floats, D x D per state): tilde[nseq * (G-1)], trans[nseq * (G-1)],
// start[nseq * G] (start[seq * G + g]); index seq * (G-1) + g for the first two.
// Grid: nseq * (D / ROWS) workgroups of threads_for<D>() threads.  DEPTH
// register sets keep the loads of the next DEPTH segments in flight.
template <int D>
__global__ __launch_bounds__(threads_for<D>()) void split_combine_kernel(const float* __restrict__ s0,
                                                                        float* __restrict__ ws, int nseq, int G) {
  static_assert(D == 64 || D == 128, "state width");
  constexpr int NT = threads_for<D>();
  constexpr int NV = D * D / 4 / NT;  // 16-byte vectors of M per thread: 4 (D = 64) or 8 (D = 128)
  constexpr int DEPTH = D == 128 ? 3 : 4;
  constexpr int64_t DD = (int64_t)D * D;
  __shared__ __attribute__((aligned(16))) float Ms[2][D * D];
  __shared__ __attribute__((aligned(16))) float prevT[2][D * ROWS];

  constexpr int blocks_per_seq = D / ROWS;
  const int seq = blockIdx.x / blocks_per_seq;
  const int r0 = (blockIdx.x % blocks_per_seq) * ROWS;
  if (seq >= nseq) return;
  const int t = threadIdx.x;
  if constexpr (POISON_LDS) {
    lds_poison(Ms, t, NT);
    lds_poison(prevT, t, NT);
    __syncthreads();
  }
  const int lane = t % 64;
  const int ib = 4 * (lane / 16), jj = 16 * (t / 64) + lane % 16;
  const int64_t per = (int64_t)nseq * (G - 1);
  const float* tilde = ws;
  const float* trans = ws + per * DD;
  float* start = ws + 2 * per * DD;
  const int64_t seg0 = (int64_t)seq * (G - 1);

  // register set s holds the M and tilde of the steps g = s (mod DEPTH); the
  // M of a step goes to LDS during the step before it
  f32x4 mr[DEPTH][NV];
  f32x4 tr[DEPTH];
#pragma unroll
  for (int s = 0; s < DEPTH; ++s)
    if (G > 1) fetch_step<D>(mr[s], tr[s], trans, tilde, seg0 + (s + 1 < G ? s : G - 2), r0, t, ib, jj);

  {
    float* out = start + ((int64_t)seq * G) * DD + (int64_t)r0 * D;
    const float* in = s0 ? s0 + (int64_t)seq * DD + (int64_t)r0 * D : nullptr;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (in) x = f32x4{in[ib * D + jj], in[(ib + 1) * D + jj], in[(ib + 2) * D + jj], in[(ib + 3) * D + jj]};
    *reinterpret_cast<f32x4*>(&prevT[0][jj * 16 + ib]) = x;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(ib + r) * D + jj] = x[r];
    if (G > 1) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int e = 4 * (t + NT * v);
        *reinterpret_cast<f32x4*>(&Ms[0][m_at<D>(e / D, e % D)]) = mr[0][v];
      }
    }
  }
  __syncthreads();
  // Step g reads Ms[g & 1] and prevT[g & 1] and writes Ms[(g+1) & 1] (from
  // register set (g+1) % DEPTH) and prevT[(g+1) & 1].  The walk runs whole
  // groups of 2 DEPTH steps with no branch between them, so that every
  // register set and buffer index is known at compile time (a branch would
  // also make the compiler wait for loads of later steps), then the rest.
  int g0 = 0;
  for (; g0 + 2 * DEPTH < G; g0 += 2 * DEPTH) {
#pragma unroll
    for (int u = 0; u < 2 * DEPTH; ++u) {
      const int g = g0 + u, s = u % DEPTH, s1 = (u + 1) % DEPTH, b = u & 1;
      float* out = start + ((int64_t)seq * G + g + 1) * DD + (int64_t)r0 * D;
      const int64_t next = seg0 + (g + DEPTH + 1 < G ? g + DEPTH : G - 2);
      combine_step<D>(mr[s], tr[s], mr[s1], Ms[b], Ms[b ^ 1], prevT[b], prevT[b ^ 1], out, trans, tilde,
                      next, true, r0, t, ib, jj);
    }
  }
#pragma unroll
  for (int u = 0; u + 1 < 2 * DEPTH; ++u) {
    const int g = g0 + u, s = u % DEPTH, s1 = (u + 1) % DEPTH, b = u & 1;
    if (g + 1 < G) {
      float* out = start + ((int64_t)seq * G + g + 1) * DD + (int64_t)r0 * D;
      const int64_t next = seg0 + (g + DEPTH + 1 < G ? g + DEPTH : G - 2);
      combine_step<D>(mr[s], tr[s], mr[s1], Ms[b], Ms[b ^ 1], prevT[b], prevT[b ^ 1], out, trans, tilde,
                      next, g + 2 < G, r0, t, ib, jj);
    }
  }
}

}  // namespace split
}  // namespace gdn
