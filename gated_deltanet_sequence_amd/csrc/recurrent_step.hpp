// Single-token decode step of the gated delta rule on gfx950.
//
// Sources (web pages, by title and section):
//   [P1] "Gated DeltaNet GPU并行实现：拆解线性注意力循环的两种高效方案"
//        §1.2 each token's state depends on the previous one; §2.1 delta rule
//        with its erase term.
//   [P3] "线性注意力机制与Gated DeltaNet的优化实践"
//        §3.1 a one-step gated state update applied in place to a global fp32
//        state (that kernel has no erase term and no output; this one has
//        both and touches the state once).
//
// Per (n,h) and value row i of the fp32 state S (dv x dk):
//     rk_i = S_i . k,  rq_i = S_i . q                (row dots, pre-decay state)
//     u_i  = beta (v_i - alpha rk_i)
//     o_i  = alpha rq_i + (k . q) u_i
//     S_i <- alpha S_i + u_i k^T                     (written in place)
// Every row is independent, so the state is read once and written once.
// Two more token updates share the kernel (template argument GATE):
//   - a per-dimension gate alpha in R^dk ([P1] §2.2 vector gate), which decays
//     the key columns: S <- S Diag(alpha) (I - beta k k^T) + beta v k^T.  The
//     decay moves onto the vectors of the row dots, rk_i = S_i . (alpha o k)
//     and rq_i = S_i . (alpha o q); then u_i = beta (v_i - rk_i),
//     o_i = rq_i + (k . q) u_i and S_i <- alpha o S_i + u_i k^T;
//   - gated linear attention without the erase term ([P3] §2.3):
//     u_i = beta v_i, o_i = alpha rq_i + (k . q) u_i, S_i <- alpha S_i + u_i k^T
//     (no rk).
//
// Layout of one workgroup (NT threads) = one head: LPR = dk/4 consecutive
// lanes hold one row as float4s (a 16-byte coalesced load per lane), and
// NT/LPR row groups stride over the dv rows.  NT = 512 for d = 128 keeps a
// lane's share of the state at 8 rows (about 70 VGPRs, 7 waves per SIMD), so
// enough heads are resident per CU for their loads and stores to overlap;
// with 256 threads (16 rows per lane) only 4 waves fit and the step runs
// measurably slower than an in-place read-modify-write of the same bytes.
// The per-row dot products are reduced across the LPR lanes with a halving
// exchange: each step sends half of the still-partial rows to the partner
// lane, so every step halves the values a lane carries instead of reducing
// every row separately.
#pragma once

#include "gdn_common.hpp"

namespace gdn {

// Sum over the LPR lanes of one row group for R rows at once.  On return,
// lane x (x = lane % LPR) holds the full sum of row rowsel(x) in v[0].
template <int LPR, int R>
__device__ __forceinline__ void halving_row_reduce(float (&v)[R], int x) {
  int n = R;
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) {
    if (n > 1) {
      const bool hi = (x & off) != 0;
      const int h = n / 2;
#pragma unroll
      for (int m = 0; m < R / 2; ++m) {
        if (m < h) {
          const float send = hi ? v[m] : v[m + h];
          const float keep = hi ? v[m + h] : v[m];
          v[m] = keep + __shfl_xor(send, off, 64);
        }
      }
      n = h;
    } else {
      v[0] += __shfl_xor(v[0], off, 64);
    }
  }
}

// Which of a lane's R rows it holds after halving_row_reduce.
template <int LPR, int R>
__device__ __forceinline__ int halving_row_index(int x) {
  int idx = 0, n = R;
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) {
    if (n > 1) {
      n /= 2;
      if (x & off) idx += n;
    }
  }
  return idx;
}

enum StepGate : int { STEP_SCALAR = 0, STEP_VEC = 1, STEP_GLA = 2 };

template <class T, int DK, int DV, int NT, int GATE = STEP_SCALAR>
__global__ __launch_bounds__(NT) void recurrent_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    float* __restrict__ state, T* __restrict__ o, int64_t nheads) {
  constexpr int LPR = DK / 4;        // lanes per row
  constexpr int RG = NT / LPR;       // row groups
  constexpr int R = DV / RG;         // rows per lane
  static_assert(LPR <= 64 && (LPR & (LPR - 1)) == 0, "row must fit a wave");
  static_assert(R >= 1 && (R & (R - 1)) == 0 && R <= LPR, "rows per lane");

  const int64_t head = blockIdx.x;
  if (head >= nheads) return;
  const int tid = threadIdx.x;
  const int x = tid % LPR;          // float4 column index within the row
  const int grp = tid / LPR;        // row group: rows grp + RG*m

  float* S = state + head * (int64_t)DV * DK;
  const T* kh = k + head * DK;
  const T* qh = q + head * DK;
  // scalar gate a, or this lane's four key columns of a per-dimension gate
  float av[4];
  if constexpr (GATE == STEP_VEC) {
    const float4 a4 = *reinterpret_cast<const float4*>(alpha + head * DK + 4 * x);
    av[0] = a4.x, av[1] = a4.y, av[2] = a4.z, av[3] = a4.w;
  } else {
    const float a = alpha[head];
    av[0] = av[1] = av[2] = av[3] = a;
  }
  const float b = beta[head];

  float kk[4], qq[4], ka[4], qa[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kk[e] = Elem<T>::to_f32(kh[4 * x + e]);
    qq[e] = Elem<T>::to_f32(qh[4 * x + e]);
    // vectors of the row dots: the per-dimension decay folded into them
    ka[e] = GATE == STEP_VEC ? av[e] * kk[e] : kk[e];
    qa[e] = GATE == STEP_VEC ? av[e] * qq[e] : qq[e];
  }

  float4 s[R];
#pragma unroll
  for (int m = 0; m < R; ++m)
    s[m] = *reinterpret_cast<const float4*>(S + (int64_t)(grp + RG * m) * DK + 4 * x);

  float rk[R], rq[R];
#pragma unroll
  for (int m = 0; m < R; ++m) {
    rk[m] = GATE == STEP_GLA ? 0.f : s[m].x * ka[0] + s[m].y * ka[1] + s[m].z * ka[2] + s[m].w * ka[3];
    rq[m] = s[m].x * qa[0] + s[m].y * qa[1] + s[m].z * qa[2] + s[m].w * qa[3];
  }
  float kq[1] = {kk[0] * qq[0] + kk[1] * qq[1] + kk[2] * qq[2] + kk[3] * qq[3]};
  if constexpr (GATE != STEP_GLA) halving_row_reduce<LPR, R>(rk, x);
  halving_row_reduce<LPR, R>(rq, x);
  halving_row_reduce<LPR, 1>(kq, x);

  // This lane now owns row grp + RG*mi of the head.
  const int mi = halving_row_index<LPR, R>(x);
  const int row = grp + RG * mi;
  const float vr = Elem<T>::to_f32(v[head * DV + row]);
  float u, out;
  if constexpr (GATE == STEP_SCALAR) {
    u = b * (vr - av[0] * rk[0]);
    out = av[0] * rq[0] + kq[0] * u;
  } else if constexpr (GATE == STEP_VEC) {
    u = b * (vr - rk[0]);
    out = rq[0] + kq[0] * u;
  } else {
    u = b * vr;
    out = av[0] * rq[0] + kq[0] * u;
  }
  // Rows are held by LPR/R lanes each; the lowest of them writes o.
  constexpr int DUP = LPR / R;
  if ((x & (DUP - 1)) == 0) o[head * DV + row] = Elem<T>::from_f32(out);

  // Gather u for every row this lane updates: row grp + RG*m is held by the
  // lanes whose halving index is m.
#pragma unroll
  for (int m = 0; m < R; ++m) {
    // lane offset within the row group whose halving index equals m
    int src = 0, n = R, mm = m;
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) {
      if (n > 1) {
        n /= 2;
        if (mm >= n) { src |= off; mm -= n; }
      }
    }
    const int base = tid - x;  // first lane of this row group
    const float um = __shfl(u, (base + src) & 63, 64);
    float4 w = s[m];
    w.x = av[0] * w.x + um * kk[0];
    w.y = av[1] * w.y + um * kk[1];
    w.z = av[2] * w.z + um * kk[2];
    w.w = av[3] * w.w + um * kk[3];
    *reinterpret_cast<float4*>(S + (int64_t)(grp + RG * m) * DK + 4 * x) = w;
  }
}

}  // namespace gdn
