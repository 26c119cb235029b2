// Chunked forward pass of the gated delta rule on gfx950.
//
// Sources (web pages, by title and section):
//   [P1] "Gated DeltaNet GPU并行实现：拆解线性注意力循环的两种高效方案"
//        §2.1-2.3 the per-token update is an affine map of the state and maps
//        compose; §3.2 chunked evaluation: inside a chunk the work is dense
//        matmuls, across chunks the state is carried serially (T/C rounds);
//        §3.3 chunk-wise mode: one workgroup carries every chunk of its
//        sequence so the serial carry never leaves the workgroup; §4.1 layout
//        change done once per tile, not per op; §4.4 fp32 state, bf16 matmul
//        inputs with fp32 accumulation; §5.2 (third pitfall) gates are used as
//        given, never renormalised.
//
// The chunk algebra (derived from the per-token loop; checked in fp64 by the
// oracle tests).  For one chunk of C tokens with start state S (dv x dk), gate
// log-prefix g_r = sum_{s<=r} log alpha_s, D_rs = exp(g_r - g_s) for s <= r:
//     L    = strictly-lower( diag(beta) (D o K K^T) )
//     Tinv = (I + L)^-1
//     U    = Tinv ( diag(beta) V - diag(beta e^g) K S^T )
//     O    = diag(e^g) Q S^T + (D o Q K^T)_{s<=r} U
//     S'   = e^{g_C} S + U^T diag(e^{g_C - g}) K
// U is formed from S directly (K S^T first, one Tinv product after), which
// needs no separate W = Tinv diag(beta e^g) K factor.
//
// Work split.  Rows of S (value dims) evolve independently, so one workgroup
// owns a DVS-row slice of one (b,h) state and walks all chunks of that
// sequence; the S-independent chunk products (K K^T, K Q^T, the inverse) are
// recomputed by each slice's workgroup.  The fp32 state slice lives in MFMA
// accumulators for the whole sequence; a bf16 copy in LDS feeds the products.
//
// The library uses this kernel for fp32 inputs (d = 64); bf16 inputs take the
// pipelined kernel of chunk_fwd_pipe.hpp.
//
// All tensors are dense row-major; pointers are 16-byte aligned (checked on
// the host).
#pragma once

#include "gdn_common.hpp"

namespace gdn {

template <class T, int DK, int DVS, int C>
struct ChunkSmem {
  static constexpr int PAD = 16 / (int)sizeof(T);  // 16-byte row padding
  static constexpr int LDK = DK + PAD;              // stride of dk-long rows
  static constexpr int LDC = C + PAD;               // stride of C-long rows
  T K[C * LDK];       // keys of the chunk, [token][dk]
  T Q[C * LDK];       // queries, [token][dk]
  T Kt[DK * LDC];     // keys transposed, [dk][token]
  T V[C * DVS];       // value slice, [token][dvs]
  T S[DVS * LDK];     // operand copy of the state slice, [dv][dk]
  T Yt[DVS * LDC];    // right-hand side of the triangular system, [dv][token]
  T Ut[DVS * LDC];    // U^T, [dv][token]
  T Uh[DVS * LDC];    // U^T scaled by exp(g_C - g_r), [dv][token]
  T Ti[C * LDC];      // (I + L)^-1, [token][token]
  T Tt[C * LDC];      // its transpose while it is being built
  T Lb[C * LDC];      // L, operand copy
  T P[C * LDC];       // D o Q K^T (lower incl. diagonal), [r][s]
  T Mt[32 * LDC];     // partial products of the blocked inverse (transposed)
  float Ld[4][16][17];  // fp32 diagonal 16x16 blocks of L
  float g[C];         // log2-prefix of alpha
  float beta[C];
  float eg[C];        // 2^g
  float beg[C];       // beta * 2^g
  float el[C];        // 2^(g_C - g)
};

// Pairs (s-block, r-block) with s-block <= r-block of a 4x4 block grid.
__device__ __forceinline__ void lower_pair(int p, int& sb, int& rb) {
  // p: 0..9 -> (0,0),(0,1),(1,1),(0,2),(1,2),(2,2),(0,3),(1,3),(2,3),(3,3)
  rb = (p >= 1) + (p >= 3) + (p >= 6);
  sb = p - rb * (rb + 1) / 2;
}

template <class T, int DK, int DVS, int C, int NW>
__global__ __launch_bounds__(NW * 64) void chunk_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* initial_state, T* __restrict__ o, float* final_state,
    int nchain, int64_t Tlen, int DV, int xcd_map) {
  static_assert(C == 64, "one gate lane per token: C equals the wave width");
  static_assert(DK % 16 == 0 && DVS % 16 == 0, "16x16 tiles");
  using Sm = ChunkSmem<T, DK, DVS, C>;
  constexpr int LDK = Sm::LDK;
  constexpr int LDC = Sm::LDC;
  constexpr int NT = NW * 64;
  constexpr int VEC = 16 / (int)sizeof(T);             // elements per 16-byte vector
  constexpr int NQK = (C * DK / VEC + NT - 1) / NT;    // vectors per thread, Q or K
  constexpr int NVV = (C * DVS / VEC + NT - 1) / NT;   // vectors per thread, V
  constexpr int IB = DVS / 16;                         // value-row tiles
  constexpr int JB = DK / 16;                          // key-column tiles
  constexpr int RB = C / 16;                           // token tiles
  constexpr int NST = (JB * IB + NW - 1) / NW;         // state tiles per wave
  constexpr int NOT = (IB * RB + NW - 1) / NW;         // output tiles per wave

  __shared__ Sm sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;  // tile column owned by this lane
  const int lg = lane >> 4;  // tile row group (rows 4*lg .. 4*lg+3)

  // Workgroup -> (sequence, value slice).  Consecutive workgroups go to
  // different XCDs round-robin; with xcd_map the slices of one sequence share
  // an XCD (and its L2) so their identical Q/K tile reads hit the same cache.
  const int NS = DV / DVS;
  int chain, slice;
  {
    const int w = blockIdx.x;
    if (xcd_map) {
      const int x = w & 7, r = w >> 3;
      slice = r % NS;
      chain = (r / NS) * 8 + x;
    } else {
      chain = w / NS;
      slice = w % NS;
    }
  }
  if (chain >= nchain) return;

  const T* qc = q + (int64_t)chain * Tlen * DK;
  const T* kc = k + (int64_t)chain * Tlen * DK;
  const T* vc = v + (int64_t)chain * Tlen * DV + slice * DVS;
  const float* ac = alpha + (int64_t)chain * Tlen;
  const float* bc = beta + (int64_t)chain * Tlen;
  T* oc = o + (int64_t)chain * Tlen * DV + slice * DVS;
  const int64_t st_off = ((int64_t)chain * DV + (int64_t)slice * DVS) * DK;

  // Zero the triangular buffers once: their upper blocks are never written
  // and must read as zero.
  for (int e = tid; e < C * LDC; e += NT) {
    sm.Ti[e] = Elem<T>::from_f32(0.f);
    sm.Tt[e] = Elem<T>::from_f32(0.f);
    sm.P[e] = Elem<T>::from_f32(0.f);
    sm.Lb[e] = Elem<T>::from_f32(0.f);
  }

  // State slice: S^T tiles [j-block][i-block] in MFMA accumulators.
  f32x4 Sacc[NST];
#pragma unroll
  for (int m = 0; m < NST; ++m) {
    const int t = wave + NW * m;
    Sacc[m] = zero4();
    if (t < JB * IB) {
      const int jb = t / IB, ib = t % IB;
      const int i = ib * 16 + lr, j = jb * 16 + 4 * lg;
      if (initial_state) {
        const float4 s4 = *reinterpret_cast<const float4*>(initial_state + st_off + (int64_t)i * DK + j);
        Sacc[m] = f32x4{s4.x, s4.y, s4.z, s4.w};
      }
      store4<T>(&sm.S[i * LDK + j], Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
    }
  }

  const int64_t nchunks = (Tlen + C - 1) / C;

  // Register staging of the next chunk's tiles (prefetch).
  uint4 rq[NQK], rk[NQK], rv[NVV];
  auto load_chunk = [&](int64_t ch) {
    const int64_t t0 = ch * C;
#pragma unroll
    for (int it = 0; it < NQK; ++it) {
      const int vi = tid + NT * it;
      const int r = vi / (DK / VEC), cg = vi % (DK / VEC);
      const bool ok = vi < C * DK / VEC && t0 + r < Tlen;
      const int64_t off = (t0 + r) * DK + cg * VEC;
      rq[it] = ok ? *reinterpret_cast<const uint4*>(qc + off) : make_uint4(0, 0, 0, 0);
      rk[it] = ok ? *reinterpret_cast<const uint4*>(kc + off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int it = 0; it < NVV; ++it) {
      const int vi = tid + NT * it;
      const int r = vi / (DVS / VEC), cg = vi % (DVS / VEC);
      const bool ok = vi < C * DVS / VEC && t0 + r < Tlen;
      rv[it] = ok ? *reinterpret_cast<const uint4*>(vc + (t0 + r) * DV + cg * VEC)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage_chunk = [&]() {
#pragma unroll
    for (int it = 0; it < NQK; ++it) {
      const int vi = tid + NT * it;
      if (vi < C * DK / VEC) {
        const int r = vi / (DK / VEC), cg = vi % (DK / VEC);
        *reinterpret_cast<uint4*>(&sm.Q[r * LDK + cg * VEC]) = rq[it];
        *reinterpret_cast<uint4*>(&sm.K[r * LDK + cg * VEC]) = rk[it];
        const T* ke = reinterpret_cast<const T*>(&rk[it]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) sm.Kt[(cg * VEC + e) * LDC + r] = ke[e];
      }
    }
#pragma unroll
    for (int it = 0; it < NVV; ++it) {
      const int vi = tid + NT * it;
      if (vi < C * DVS / VEC) {
        const int r = vi / (DVS / VEC), cg = vi % (DVS / VEC);
        *reinterpret_cast<uint4*>(&sm.V[r * DVS + cg * VEC]) = rv[it];
      }
    }
  };

  if (nchunks > 0) load_chunk(0);

  for (int64_t ch = 0; ch < nchunks; ++ch) {
    __syncthreads();  // previous chunk finished reading every tile buffer
    stage_chunk();
    if (wave == 0) {
      // a2: gate log-prefix (base 2) over the chunk, one lane per token.
      // Tokens past the end act as identity maps: alpha = 1, beta = 0.
      const int64_t t = ch * C + lane;
      const bool ok = t < Tlen;
      const float a = ok ? ac[t] : 1.f;
      const float b = ok ? bc[t] : 0.f;
      float gs = fmaxf(fast_log2(a), LOG2_ALPHA_MIN);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(gs, off, 64);
        if (lane >= off) gs += y;
      }
      const float glast = __shfl(gs, 63, 64);
      const float e = fast_exp2(gs);
      sm.g[lane] = gs;
      sm.beta[lane] = b;
      sm.eg[lane] = e;
      sm.beg[lane] = b * e;
      sm.el[lane] = fast_exp2(glast - gs);
    }
    if (ch + 1 < nchunks) load_chunk(ch + 1);
    __syncthreads();

    // a3: Gram products on the lower block triangle, in [s][r] orientation so
    // each lane writes four consecutive s of row r.
    //   L[r][s] = beta_r D_rs (k_r . k_s), s < r      P[r][s] = D_rs (q_r . k_s), s <= r
    for (int u = wave; u < 20; u += NW) {
      const int kind = u / 10;  // 0: L, 1: P
      int sb, rb;
      lower_pair(u % 10, sb, rb);
      f32x4 acc = Mma<T>::template run<DK>(zero4(), &sm.K[sb * 16 * LDK], LDK,
                                            &(kind == 0 ? sm.K : sm.Q)[rb * 16 * LDK], LDK, lane);
      const int r = rb * 16 + lr;
      const int s0 = sb * 16 + 4 * lg;
      const float gr = sm.g[r];
      float val[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = s0 + e;
        const bool in = kind == 0 ? (s < r) : (s <= r);
        const float d = in ? fast_exp2(gr - sm.g[s]) : 0.f;
        val[e] = (kind == 0 ? sm.beta[r] : 1.f) * d * acc[e];
      }
      T* dst = kind == 0 ? sm.Lb : sm.P;
      store4<T>(&dst[r * LDC + s0], val[0], val[1], val[2], val[3]);
      if (kind == 0 && sb == rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Ld[sb][r - rb * 16][s0 - sb * 16 + e] = val[e];
      }
    }
    __syncthreads();

    // a4: Tinv = (I + L)^-1, blocked.  Level 0: the four unit-lower 16x16
    // diagonal blocks by forward substitution in fp32 (lane = block, column).
    if (wave == 0) {
      const int b = lane >> 4, c = lane & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < r; ++s) acc -= sm.Ld[b][r][s] * x[s];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sm.Ti[(16 * b + r) * LDC + 16 * b + c] = Elem<T>::from_f32(x[r]);
        sm.Tt[(16 * b + c) * LDC + 16 * b + r] = Elem<T>::from_f32(x[r]);
      }
    }
    __syncthreads();
    // Level 1: Ti[a][b] = -Ti[a][a] L[a][b] Ti[b][b] for (a,b) = (1,0), (3,2).
    if (wave < 2) {
      const int p = wave, a = 2 * p + 1, b = 2 * p;
      f32x4 acc = Mma<T>::template run<16>(zero4(), &sm.Lb[16 * a * LDC + 16 * b], LDC,
                                            &sm.Tt[16 * b * LDC + 16 * b], LDC, lane);
      store4<T>(&sm.Mt[(16 * p + lr) * LDC + 4 * lg], acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();
    if (wave < 2) {
      const int p = wave, a = 2 * p + 1, b = 2 * p;
      f32x4 acc = Mma<T>::template run<16>(zero4(), &sm.Ti[16 * a * LDC + 16 * a], LDC,
                                            &sm.Mt[16 * p * LDC], LDC, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sm.Ti[(16 * a + 4 * lg + e) * LDC + 16 * b + lr] = Elem<T>::from_f32(-acc[e]);
      store4<T>(&sm.Tt[(16 * b + lr) * LDC + 16 * a + 4 * lg], -acc[0], -acc[1], -acc[2], -acc[3]);
    }
    __syncthreads();
    // Level 2: Ti[hi][lo] = -Ti[hi][hi] L[hi][lo] Ti[lo][lo] on 32x32 halves.
    for (int u = wave; u < 4; u += NW) {
      const int rb2 = u >> 1, cb2 = u & 1;
      f32x4 acc = Mma<T>::template run<32>(zero4(), &sm.Lb[(32 + 16 * rb2) * LDC], LDC,
                                            &sm.Tt[16 * cb2 * LDC], LDC, lane);
      store4<T>(&sm.Mt[(16 * cb2 + lr) * LDC + 16 * rb2 + 4 * lg], acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();
    for (int u = wave; u < 4; u += NW) {
      const int rb2 = u >> 1, cb2 = u & 1;
      f32x4 acc = Mma<T>::template run<32>(zero4(), &sm.Ti[(32 + 16 * rb2) * LDC + 32], LDC,
                                            &sm.Mt[16 * cb2 * LDC], LDC, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sm.Ti[(32 + 16 * rb2 + 4 * lg + e) * LDC + 16 * cb2 + lr] = Elem<T>::from_f32(-acc[e]);
    }
    __syncthreads();

    // a5 (1): Y = diag(beta) V - diag(beta e^g) K S^T  (tiles [r][i]), and the
    // inter-chunk part of the output, e^g (S Q^T) (tiles [i][r], kept live).
    for (int t = wave; t < RB * IB; t += NW) {
      const int rb = t / IB, ib = t % IB;
      f32x4 acc = Mma<T>::template run<DK>(zero4(), &sm.K[rb * 16 * LDK], LDK,
                                            &sm.S[ib * 16 * LDK], LDK, lane);
      const int i = ib * 16 + lr;
      const int r0 = rb * 16 + 4 * lg;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + e;
        y[e] = sm.beta[r] * Elem<T>::to_f32(sm.V[r * DVS + i]) - sm.beg[r] * acc[e];
      }
      store4<T>(&sm.Yt[i * LDC + r0], y[0], y[1], y[2], y[3]);
    }
    f32x4 Oacc[NOT];
#pragma unroll
    for (int m = 0; m < NOT; ++m) {
      const int t = wave + NW * m;
      Oacc[m] = zero4();
      if (t < IB * RB) {
        const int ib = t / RB, rb = t % RB;
        Oacc[m] = Mma<T>::template run<DK>(zero4(), &sm.S[ib * 16 * LDK], LDK,
                                           &sm.Q[rb * 16 * LDK], LDK, lane);
        const float sc = sm.eg[rb * 16 + lr];
        Oacc[m] *= sc;
      }
    }
    __syncthreads();

    // a5 (2): U = Tinv Y (tiles [r][i]); store U^T and U^T scaled by e^{g_C - g}.
    for (int t = wave; t < RB * IB; t += NW) {
      const int rb = t / IB, ib = t % IB;
      f32x4 acc = Mma<T>::template run<C>(zero4(), &sm.Ti[rb * 16 * LDC], LDC,
                                           &sm.Yt[ib * 16 * LDC], LDC, lane);
      const int i = ib * 16 + lr;
      const int r0 = rb * 16 + 4 * lg;
      store4<T>(&sm.Ut[i * LDC + r0], acc[0], acc[1], acc[2], acc[3]);
      store4<T>(&sm.Uh[i * LDC + r0], acc[0] * sm.el[r0], acc[1] * sm.el[r0 + 1],
                acc[2] * sm.el[r0 + 2], acc[3] * sm.el[r0 + 3]);
    }
    __syncthreads();

    // a5 (3) + a6: O^T += U^T P^T and store; S^T <- e^{g_C} S^T + K^T Uh^T.
#pragma unroll
    for (int m = 0; m < NOT; ++m) {
      const int t = wave + NW * m;
      if (t < IB * RB) {
        const int ib = t / RB, rb = t % RB;
        Oacc[m] = Mma<T>::template run<C>(Oacc[m], &sm.Ut[ib * 16 * LDC], LDC,
                                          &sm.P[rb * 16 * LDC], LDC, lane);
        const int64_t tok = ch * C + rb * 16 + lr;
        if (tok < Tlen)
          store4<T>(oc + tok * DV + ib * 16 + 4 * lg, Oacc[m][0], Oacc[m][1], Oacc[m][2], Oacc[m][3]);
      }
    }
    const float decay = sm.eg[C - 1];
#pragma unroll
    for (int m = 0; m < NST; ++m) {
      const int t = wave + NW * m;
      if (t < JB * IB) {
        const int jb = t / IB, ib = t % IB;
        Sacc[m] *= decay;
        Sacc[m] = Mma<T>::template run<C>(Sacc[m], &sm.Kt[jb * 16 * LDC], LDC,
                                          &sm.Uh[ib * 16 * LDC], LDC, lane);
        const int i = ib * 16 + lr, j = jb * 16 + 4 * lg;
        store4<T>(&sm.S[i * LDK + j], Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
      }
    }
  }

  // a6: final state slice (fp32).
  if (final_state) {
#pragma unroll
    for (int m = 0; m < NST; ++m) {
      const int t = wave + NW * m;
      if (t < JB * IB) {
        const int jb = t / IB, ib = t % IB;
        const int i = ib * 16 + lr, j = jb * 16 + 4 * lg;
        *reinterpret_cast<float4*>(final_state + st_off + (int64_t)i * DK + j) =
            make_float4(Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
      }
    }
  }
}

}  // namespace gdn
