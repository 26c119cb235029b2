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
#pragma once

#include "gdn_common.hpp"

namespace gdn {
namespace split {

constexpr int ROWS = 8;
constexpr int THREADS = 256;

// ws layout (floats, d x d per state): tilde[nseq * (G-1)], trans[nseq * (G-1)],
// start[nseq * G] (start[seq * G + g]); index seq * (G-1) + g for the first two.
__global__ __launch_bounds__(THREADS) void split_combine_kernel(const float* __restrict__ s0,
                                                               float* __restrict__ ws, int nseq,
                                                               int G, int d) {
  __shared__ float prev[ROWS][128];
  const int blocks_per_seq = d / ROWS;
  const int seq = blockIdx.x / blocks_per_seq;
  const int r0 = (blockIdx.x % blocks_per_seq) * ROWS;
  if (seq >= nseq) return;
  const int64_t dd = (int64_t)d * d, per = (int64_t)nseq * (G - 1);
  const float* tilde = ws;
  const float* trans = ws + per * dd;
  float* start = ws + 2 * per * dd;
  const int nout = ROWS * d / THREADS;  // outputs per thread: 4 (d = 128) or 2 (d = 64)

  // start_0 = S_0 (a copy, so that the caller's final state may alias S_0)
  for (int e = threadIdx.x; e < ROWS * d; e += THREADS) {
    const int i = e / d, j = e % d;
    const float x = s0 ? s0[(int64_t)seq * dd + (int64_t)(r0 + i) * d + j] : 0.f;
    prev[i][j] = x;
    start[((int64_t)seq * G) * dd + (int64_t)(r0 + i) * d + j] = x;
  }
  __syncthreads();
  for (int g = 0; g + 1 < G; ++g) {
    const int64_t idx = (int64_t)seq * (G - 1) + g;
    const float* M = trans + idx * dd;
    const float* Tl = tilde + idx * dd;
    float* out = start + ((int64_t)seq * G + g + 1) * dd;
    float acc[4];
    for (int u = 0; u < nout; ++u) {
      const int e = threadIdx.x + THREADS * u, i = e / d, j = e % d;
      float a = Tl[(int64_t)(r0 + i) * d + j];
      for (int kk = 0; kk < d; ++kk) a = fmaf(prev[i][kk], M[(int64_t)kk * d + j], a);
      acc[u] = a;
    }
    __syncthreads();
    for (int u = 0; u < nout; ++u) {
      const int e = threadIdx.x + THREADS * u, i = e / d, j = e % d;
      prev[i][j] = acc[u];
      out[(int64_t)(r0 + i) * d + j] = acc[u];
    }
    __syncthreads();
  }
}

}  // namespace split
}  // namespace gdn
