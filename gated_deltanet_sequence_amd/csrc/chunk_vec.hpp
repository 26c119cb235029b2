// Chunked forward pass of the gated delta rule with a per-dimension gate (or
// a scalar gate, as the special case of equal columns), bf16 or fp32 inputs,
// d_k = d_v = 64 or 128, on gfx950.
//
// Sources (web pages, by title and section):
//   [P1] "Gated DeltaNet GPU并行实现：拆解线性注意力循环的两种高效方案"
//        §2.2 the forgetting gate may be a scalar or a vector (one factor per
//        dimension); §3.2 chunked evaluation (dense products inside a chunk,
//        serial state carry between chunks); §4.4 fp32 state, bf16 matmul
//        inputs with fp32 accumulation (fp32 inputs: fp32 products
//        throughout).
//
// The recurrence.  alpha_t in [0,1]^{d_k} decays the key columns of the state:
//     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//     o_t = S_t q_t.
//
// Chunk algebra (derived from the token loop as for the scalar gate).  For a
// chunk with start state S, let G_r[j] = sum_{s <= r} log2 alpha_s[j] (the
// decay of key column j from the chunk start through token r) and write
// x~ = 2^G o x for a token row x.  Then per token pair s <= r the decay
// between them is 2^(G_r - G_s) per column, so
//     A_qk[r][s] = q~_r . (2^-G_s o k_s),   A_kk[r][s] = k~_r . (2^-G_s o k_s)
//     L = strictly-lower(diag(beta) A_kk),  Ti = (I + L)^-1,  P = lower(A_qk)
//     U = Ti diag(beta) (V - K~ S^T)
//     O = Q~ S^T + P U
//     S' = S Diag(2^(G_C)) + U^T Kbar,   Kbar_s = 2^(G_C - G_s) o k_s.
// The per-column decay of the scalar-gate masks moves into the operands: the
// products stay plain matrix products (MFMA), the masks only zero the upper
// triangle.  All factors are at most 1 except 2^-G_s, which is at most
// 2^100 while the chunk decays by no more than 2^-100 in every column
// (SAFE_MIN); then every factor and product lies in the normal fp32/bf16
// range.  A chunk that decays more in some column (strong gates, a gate of
// 0) forms A_qk and A_kk element by element from 2^(G_r - G_s) <= 1 instead
// (slow, exact; such chunks carry almost nothing across anyway).
//
// Work split: rows of S (value dimensions) evolve independently, so one
// workgroup owns a 16-row value slice of one sequence and walks all its
// chunks; the S-independent chunk products are recomputed by each slice's
// workgroup.  The fp32 state slice lives in MFMA accumulators, a copy in the
// input type in LDS feeds the products; four waves in seven barrier-separated
// steps per chunk.  The chunk is 32 tokens: the fp32 table of G (32 x d_k)
// and the four operand copies of q and k it needs per chunk then fit in LDS
// next to the chunk matrices (bf16: 48.8 KB at d_k = 64, 80.8 KB at 128;
// fp32: 137 KB at d_k = 128).  Under 80 KB, two workgroups share a CU (the
// bf16 instances ask the compiler for two waves per SIMD).
//
// With a scalar gate (VG = false: alpha is [.., T] and every key column
// decays alike) the same algebra holds with G_r[j] = g_r for all j; that
// instance is the library's path for fp32 inputs and for 32-token chunks (a
// 64-token chunk's fp32 buffers would exceed the LDS at d_k = 128).  The GLA
// instance evaluates gated linear attention without the delta rule (L = 0,
// U = diag(beta) V), and the PREP instance is the first pass of the two-pass
// route (the chunk records, no state).  The second pass of that route walks
// the records: vec_state_kernel (four waves per slice, three barriers per
// chunk; fp32 records) and vec_state_pipe_kernel (one wave per slice and a
// loader wave, one barrier per chunk; bf16 records).
#pragma once

#include "gdn_common.hpp"
#include "chunk_fwd_pipe.hpp"  // ChainMap: the chain -> (sequence, token range) map of the sequence split

namespace gdn {
namespace vec {

constexpr int C = 32;      // tokens per chunk
constexpr int DVS = 16;    // value rows per workgroup
constexpr int NW = 4;      // waves
constexpr int NT = NW * 64;
constexpr float SAFE_MIN = -100.f;  // log2 of the least chunk decay the factored products take
constexpr int LDR = 20;    // row stride (floats) of the fp32 diagonal blocks of L

// Order this wave's earlier LDS accesses before its later ones (one wave
// hands data to other lanes of itself through LDS): the LDS unit runs one
// wave's instructions in order, so draining the counter suffices; the
// empty asm keeps the compiler from moving memory accesses across.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

template <class T, int DK>
struct __attribute__((aligned(16))) Smem {
  static constexpr int PAD = 16 / (int)sizeof(T);  // 16-byte row padding
  static constexpr int LDK = DK + PAD;  // rows of d_k
  static constexpr int LDC = C + PAD;   // rows of C
  static constexpr int VEC16 = 16 / (int)sizeof(T);
  T Qs[C * LDK];    // 2^G o q, [token][dk]
  T Kr[C * LDK];    // 2^G o k
  T Kh[C * LDK];    // 2^-G o k (Gram columns); raw k in chunks on the exact path
  T Qr[C * LDK];    // raw q (exact path)
  T Kbt[DK * LDC];  // (2^(G_C - G) o k)^T, [dk][token]
  T V[C * DVS];     // value slice, [token][dvs]
  T S[DVS * LDK];   // operand copy of the state slice, [dv][dk]
  union {
    T Yt[DVS * LDC];  // right-hand side of the triangular system, [dv][token]
    float tot[NT / DK][DK];  // gate scan: log2 sums of each token group per column
                             // (dead by the time Yt is written, and Yt by the next scan)
  };
  T Ut[DVS * LDC];  // U^T
  T Ti[C * LDC];    // (I + L)^-1, [token][token]
  T Lb[C * LDC];    // L, operand copy
  T P[C * LDC];     // lower(A_qk), [r][s]
  T Mt[sizeof(T) == 2 ? VEC16 : 16 * LDC];  // partial product of the blocked inverse (fp32;
                                            // bf16 keeps it in registers)
  float Ld[2][16][LDR];  // fp32 diagonal 16x16 blocks of L (rows 16-byte aligned)
  float G[C * (DK + 4)]; // log2-prefix of alpha per key column, [token][dk], rows padded by 16 bytes
  float beta[C];
  float Ec[DK];          // 2^(G_C) per key column
  int exactw[NW];        // per wave: a column of this chunk decays below 2^SAFE_MIN
};

// Eight or four values -> one 16-byte vector of T.
__device__ __forceinline__ void store_vec(bf16_t* p, const float (&x)[8]) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                            pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}
__device__ __forceinline__ void store_vec(float* p, const float (&x)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// Two-pass evaluation (gdn_chunk_fwd_vecgate_2pass).  The S-independent part
// of a chunk (gate scan, scaled operands, L, (I+L)^-1, P) does not depend on
// the value slice, yet the single-pass kernel repeats it in every slice's
// workgroup.  The first pass (the PREP instance of chunk_vec_kernel) computes
// it once per chunk and writes the buffers the
// state products need, verbatim in their LDS layout, to a record in the
// caller's workspace; the second pass (vec_state_kernel) walks the chunks of
// every value slice from those records.
constexpr int MAP_PREP = 3;  // ChainMap mode of the PREP instance (cm.L: first
                             // token of the tile, cm.G: chunks per sequence in
                             // the tile, cm.ws: the records; the grid holds
                             // cm.nseq * ng workgroups, each taking one of ng
                             // groups of consecutive chunks of a sequence, so
                             // that the next chunk's inputs load while one is
                             // computed)
template <class T, int DK>
struct VecRec {
  using Sm = Smem<T, DK>;
  static constexpr int QS = 0;                                             // 2^G o q     [C][LDK]
  static constexpr int KR = QS + C * Sm::LDK * (int)sizeof(T);             // 2^G o k     [C][LDK]
  static constexpr int KBT = KR + C * Sm::LDK * (int)sizeof(T);            // Kbar^T      [DK][LDC]
  static constexpr int TI = KBT + DK * Sm::LDC * (int)sizeof(T);           // (I + L)^-1  [C][LDC]
  static constexpr int PM = TI + C * Sm::LDC * (int)sizeof(T);             // P           [C][LDC]
  static constexpr int EC = PM + C * Sm::LDC * (int)sizeof(T);             // 2^(G_C)     [DK] fp32
  static constexpr int BETA = EC + DK * 4;                                 // beta        [C] fp32
  static constexpr int BYTES = (BETA + C * 4 + 1023) / 1024 * 1024;        // whole KiB
};

// VG: alpha is [.., T, DK] (per-dimension gate); otherwise [.., T] (scalar).
// cm maps workgroups to (sequence, token range) chains as for the pipelined
// kernel (gdn::pipe::ChainMap): whole sequences (MAP_SEQ), or the first and
// the last launch of the sequence split (MAP_SPLIT_A: segment states from a
// zero start and segment transitions from the identity with V read as zero,
// no output; MAP_SPLIT_C: every segment from its start state in cm.ws).  The
// per-token maps stay affine with a per-dimension gate, so the split and its
// combine step are the same.
// PREP: the first pass of the two-pass evaluation (cm.mode == MAP_PREP): a
// workgroup walks one group of consecutive chunks of a sequence in the tile,
// with no state and no output, and writes each chunk's record to cm.ws.
// GLA: gated linear attention without the delta rule ([P3] §2.3; scalar gate,
// MAP_SEQ only): L = 0, so Ti = I and U = Y = diag(beta) V, with no K S^T
// term; the gate scan, P, the output and the state update are unchanged.
template <class T, int DK, bool VG, bool PREP = false, bool GLA = false>
__global__ __launch_bounds__(NT, sizeof(T) == 2 ? 2 : 1) void chunk_vec_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* initial_state, T* __restrict__ o, float* final_state,
    gdn::pipe::ChainMap cm, int DV, int xcd_map) {
  using Sm = Smem<T, DK>;
  constexpr int LDK = Sm::LDK;
  constexpr int LDC = Sm::LDC;
  constexpr int LDG = DK + 4;                    // row stride of the gate table
  constexpr int VEC = 16 / (int)sizeof(T);      // elements per 16-byte vector
  constexpr int NQK = C * DK / VEC / NT;         // vectors per thread, q or k
  constexpr int NVV = C * DVS / VEC;             // vectors of V (threads 0 .. NVV-1)
  constexpr int IB = DVS / 16;
  constexpr int JB = DK / 16;
  constexpr int RB = C / 16;
  constexpr int NST = (JB * IB + NW - 1) / NW;   // state tiles per wave
  static_assert(NQK * NT * VEC == C * DK, "q/k vectors spread evenly");
  static_assert(NVV <= NT && DK <= NT && C <= 64, "one thread per V vector, key column, token");
  static_assert(RB == 2, "the blocked inverse below is for two 16-token blocks");
  static_assert(IB * RB == 2 && NW == 4, "wave roles below: one Y wave, two output waves");
  static_assert(!(GLA && (PREP || VG)), "gated linear attention: scalar gate, single pass");
  constexpr int NG = NT / DK;                    // token groups of the gate scan
  constexpr int TPG = C / NG;                    // tokens per group

  __shared__ Sm sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int lg = lane >> 4;

  const int NS = DV / DVS;
  int chain, slice;
  if constexpr (PREP) {
    chain = blockIdx.x;
    slice = 0;
  } else {
    const int w = blockIdx.x;
    if (xcd_map) {
      // the slices of one sequence land on one XCD and share its L2
      const int x = w & 7, r = w >> 3;
      slice = r % NS;
      chain = (r / NS) * 8 + x;
    } else {
      chain = w / NS;
      slice = w % NS;
    }
  }
  if (chain >= gdn::pipe::map_chains(cm)) return;

  // this chain's sequence, token range, start and end state, and whether it
  // reads V and writes output
  const int64_t dd = (int64_t)DK * DV;  // floats per state
  int seq = chain;
  int64_t t0 = 0, Tlen = cm.T;
  bool v_on = true, o_on = true, s0_ident = false;
  const float* s0 = initial_state ? initial_state + (int64_t)chain * dd : nullptr;
  float* sT = final_state ? final_state + (int64_t)chain * dd : nullptr;
  int prep_first = 0;  // PREP: the first chunk of this workgroup within the tile
  if constexpr (PREP) {
    // chain = (sequence, group of consecutive chunks of the tile)
    const int ng = (int)gridDim.x / cm.nseq;
    const int gsz = (cm.G + ng - 1) / ng;
    seq = chain / ng;
    prep_first = (chain % ng) * gsz;
    const int nc = max(0, min(gsz, cm.G - prep_first));
    t0 = cm.L + (int64_t)prep_first * C;
    Tlen = max((int64_t)0, min((int64_t)nc * C, cm.T - t0));
    v_on = false;
    s0 = nullptr;
    sT = nullptr;
  } else if (cm.mode == gdn::pipe::MAP_SPLIT_A) {
    const int per = cm.nseq * (cm.G - 1);
    const int kind = chain / per, r = chain % per;
    seq = r / (cm.G - 1);
    t0 = (int64_t)(r % (cm.G - 1)) * cm.L;
    Tlen = cm.L;
    o_on = false;
    v_on = kind == 0;
    s0_ident = kind == 1;
    s0 = nullptr;
    sT = cm.ws + ((int64_t)kind * per + r) * dd;
  } else if (cm.mode == gdn::pipe::MAP_SPLIT_C) {
    seq = chain / cm.G;
    const int g = chain % cm.G;
    t0 = (int64_t)g * cm.L;
    Tlen = g == cm.G - 1 ? cm.T - t0 : cm.L;
    s0 = cm.ws + (2 * (int64_t)cm.nseq * (cm.G - 1) + (int64_t)seq * cm.G + g) * dd;
    sT = g == cm.G - 1 && final_state ? final_state + (int64_t)seq * dd : nullptr;
  }
  const int64_t tok0 = (int64_t)seq * cm.T + t0;  // first token in memory
  const T* qc = q + tok0 * DK;
  const T* kc = k + tok0 * DK;
  const T* vc = v + tok0 * DV + slice * DVS;
  const float* ac = alpha + tok0 * (VG ? DK : 1);
  const float* bc = beta + tok0;
  T* oc = o + tok0 * DV + slice * DVS;
  const int64_t st_off = (int64_t)slice * DVS * DK;  // this slice's rows within s0 / sT

  if constexpr (POISON_LDS) {
    lds_poison(sm, tid, NT);
    __syncthreads();
  }
  // The upper blocks of the triangular buffers are never written and must
  // read as zero.
  for (int e = tid; e < C * LDC; e += NT) {
    sm.Ti[e] = Elem<T>::from_f32(0.f);
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
      if (s0_ident) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[m][e] = slice * DVS + i == j + e ? 1.f : 0.f;
      } else if (s0) {
        const float4 s4 = *reinterpret_cast<const float4*>(s0 + st_off + (int64_t)i * DK + j);
        Sacc[m] = f32x4{s4.x, s4.y, s4.z, s4.w};
      }
      store4<T>(&sm.S[i * LDK + j], Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
    }
  }

  const int64_t nchunks = (Tlen + C - 1) / C;

  // Register staging of the next chunk (prefetch): q, k vectors, a V vector,
  // the gates of one key column over one group of TPG tokens and beta of one
  // token.  Every load is unconditional, so that it stays in flight until its
  // use in the next chunk: tokens past the end reread the last token, and the
  // uses below mask them (zero q, k, v, alpha = 1, beta = 0: identity maps).
  const int gj = tid % DK, gg = tid / DK;  // gate column and token group of this thread
  uint4 rq[NQK], rk[NQK], rv;
  float ra[TPG], rbt;
  auto load_chunk = [&](int64_t ch) {
    // chunk base pointers (uniform) and 32-bit offsets; rows past the end
    // are clamped to the chunk's last valid row
    const int64_t t0 = ch * C;
    const int rmax = (int)(Tlen - 1 - t0 < C - 1 ? Tlen - 1 - t0 : C - 1);
    const T* qb = qc + t0 * DK;
    const T* kb = kc + t0 * DK;
    const T* vb = vc + t0 * DV;
    const float* ab = ac + t0 * (VG ? DK : 1);
    const float* bb = bc + t0;
#pragma unroll
    for (int it = 0; it < NQK; ++it) {
      const int vi = tid + NT * it;
      const int r = vi % C, cg = vi / C;  // token fastest (see the operands below)
      const int off = min(r, rmax) * DK + cg * VEC;
      rq[it] = *reinterpret_cast<const uint4*>(qb + off);
      rk[it] = *reinterpret_cast<const uint4*>(kb + off);
    }
    {
      const int vi = tid % NVV;
      const int r = vi / (DVS / VEC), cg = vi % (DVS / VEC);
      rv = *reinterpret_cast<const uint4*>(vb + min(r, rmax) * DV + cg * VEC);
    }
#pragma unroll
    for (int i = 0; i < TPG; ++i) {
      const int rr = min(gg * TPG + i, rmax);
      ra[i] = ab[VG ? rr * DK + gj : rr];
    }
    rbt = bb[min(tid % C, rmax)];
  };

  if (nchunks > 0) load_chunk(0);

  for (int64_t ch = 0; ch < nchunks; ++ch) {
    __syncthreads();  // the previous chunk has finished with every buffer

    // Gate table, as a scan over the chunk's tokens per key column: thread
    // (group gg, column gj) sums log2 alpha over its TPG tokens; the sums of
    // the earlier groups are added once every group's total is in LDS.
    float gl[TPG];
    {
      float g = 0.f;
#pragma unroll
      for (int i = 0; i < TPG; ++i) {
        g += fmaxf(fast_log2(ch * C + gg * TPG + i < Tlen ? ra[i] : 1.f), LOG2_ALPHA_MIN);
        gl[i] = g;
      }
      sm.tot[gg][gj] = g;
    }
    if (tid < C) sm.beta[tid] = ch * C + tid < Tlen ? rbt : 0.f;
    if (tid < NVV) {
      const int r = tid / (DVS / VEC), cg = tid % (DVS / VEC);
      *reinterpret_cast<uint4*>(&sm.V[r * DVS + cg * VEC]) = v_on && ch * C + r < Tlen ? rv : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    {
      float off = 0.f;
#pragma unroll
      for (int h = 0; h < NG - 1; ++h) off += h < gg ? sm.tot[h][gj] : 0.f;
#pragma unroll
      for (int i = 0; i < TPG; ++i) sm.G[(gg * TPG + i) * LDG + gj] = gl[i] + off;
      bool low = false;
      if (gg == NG - 1) {
        const float gC = gl[TPG - 1] + off;
        sm.Ec[gj] = fast_exp2(gC);
        low = gC < SAFE_MIN;
      }
      const bool any = __builtin_amdgcn_ballot_w64(low) != 0;
      if (lane == 0) sm.exactw[wave] = any ? 1 : 0;
    }
    __syncthreads();
    bool exact = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) exact = exact || sm.exactw[w] != 0;

    // Operands: 2^G o q, 2^G o k, 2^-G o k (raw q, k on the exact path), and
    // (2^(G_C - G) o k)^T (as 2^-G 2^(G_C) when the factors are in range).
    // A thread holds VEC keys of one token, with the token fastest over the
    // lanes: the transposed writes of K^T are then consecutive elements
    // (conflict-free), and the padded rows of G and of the operand copies
    // keep the row-wise accesses conflict-free too.
#pragma unroll
    for (int it = 0; it < NQK; ++it) {
      const int vi = tid + NT * it;
      const int r = vi % C, cg = vi / C;
      const int j0 = cg * VEC;
      float g[VEC], gc[VEC];
#pragma unroll
      for (int h = 0; h < VEC / 4; ++h) {
        const float4 g4 = *reinterpret_cast<const float4*>(&sm.G[r * LDG + j0 + 4 * h]);
        const float4 c4 = exact ? *reinterpret_cast<const float4*>(&sm.G[(C - 1) * LDG + j0 + 4 * h])
                                : *reinterpret_cast<const float4*>(&sm.Ec[j0 + 4 * h]);
        g[4 * h] = g4.x; g[4 * h + 1] = g4.y; g[4 * h + 2] = g4.z; g[4 * h + 3] = g4.w;
        gc[4 * h] = c4.x; gc[4 * h + 1] = c4.y; gc[4 * h + 2] = c4.z; gc[4 * h + 3] = c4.w;
      }
      const bool live = ch * C + r < Tlen;
      const uint4 zq = live ? rq[it] : make_uint4(0, 0, 0, 0);
      const uint4 zk = live ? rk[it] : make_uint4(0, 0, 0, 0);
      const T* qe = reinterpret_cast<const T*>(&zq);
      const T* ke = reinterpret_cast<const T*>(&zk);
      float qs[VEC], kr[VEC], kh[VEC];
      if (!exact) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float qv = Elem<T>::to_f32(qe[e]), kv = Elem<T>::to_f32(ke[e]);
          const float eg = fast_exp2(g[e]), ei = fast_exp2(-g[e]);
          qs[e] = qv * eg;
          kr[e] = kv * eg;
          kh[e] = kv * ei;
          sm.Kbt[(j0 + e) * LDC + r] = Elem<T>::from_f32(kh[e] * gc[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float qv = Elem<T>::to_f32(qe[e]), kv = Elem<T>::to_f32(ke[e]);
          const float eg = fast_exp2(g[e]);
          qs[e] = qv * eg;
          kr[e] = kv * eg;
          kh[e] = kv;
          sm.Kbt[(j0 + e) * LDC + r] = Elem<T>::from_f32(kv * fast_exp2(gc[e] - g[e]));
        }
        *reinterpret_cast<uint4*>(&sm.Qr[r * LDK + j0]) = zq;
      }
      if (o_on) store_vec(&sm.Qs[r * LDK + j0], qs);
      if constexpr (!GLA) store_vec(&sm.Kr[r * LDK + j0], kr);
      store_vec(&sm.Kh[r * LDK + j0], kh);
    }
    if (ch + 1 < nchunks) load_chunk(ch + 1);
    __syncthreads();

    // Gram products on the lower block triangle in [s][r] orientation (each
    // lane holds four consecutive s of one row r):
    //   L[r][s] = beta_r A_kk[r][s] (s < r),  P[r][s] = A_qk[r][s] (s <= r).
    // Tiles u = 0..5: kind u / 3 (0: L, 1: P), block pair (sb, rb) =
    // (0,0), (0,1), (1,1).
    // The three L tiles run here, on waves 0..2; the three P tiles (needed
    // only by the output) run in the next step on the waves that are not
    // building the inverse, and not at all without output.
    auto gram_tile = [&](int u) {
      const int kind = u / 3, pr = u % 3;
      const int rb = pr >= 1 ? 1 : 0, sb = pr == 1 ? 0 : rb;
      const int r = rb * 16 + lr;
      const int s0 = sb * 16 + 4 * lg;
      const float rowf = kind == 0 ? sm.beta[r] : 1.f;  // read before the products, unconditionally
      float val[4];
      if (!exact) {
        const f32x4 acc = Mma<T>::template run<DK>(zero4(), &sm.Kh[sb * 16 * LDK], LDK,
                                                   &(kind == 0 ? sm.Kr : sm.Qs)[rb * 16 * LDK], LDK, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = acc[e];
      } else {
        // A[r][s] = sum_j x_r[j] k_s[j] 2^(G_r[j] - G_s[j]), every factor <= 1
        const T* xr = &(kind == 0 ? sm.Kh : sm.Qr)[r * LDK];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = s0 + e;
          const T* ks = &sm.Kh[s * LDK];
          float acc = 0.f;
          if (s <= r) {
            for (int j = 0; j < DK; ++j)
              acc += Elem<T>::to_f32(xr[j]) * Elem<T>::to_f32(ks[j]) * fast_exp2(sm.G[r * LDG + j] - sm.G[s * LDG + j]);
          }
          val[e] = acc;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = s0 + e;
        const bool in = s < r + kind;  // L: s < r, P: s <= r
        val[e] = in ? rowf * val[e] : 0.f;
      }
      T* dst = kind == 0 ? sm.Lb : sm.P;
      store4<T>(&dst[r * LDC + s0], val[0], val[1], val[2], val[3]);
      if (kind == 0 && sb == rb)
        *reinterpret_cast<float4*>(&sm.Ld[sb][r - rb * 16][s0 - sb * 16]) = make_float4(val[0], val[1], val[2], val[3]);
    };
    // (Without the delta rule there is no L: the P tiles run here instead.)
    if (wave < 3 && (!GLA || o_on)) gram_tile(GLA ? 3 + wave : wave);
    __syncthreads();

    f32x4 Oacc = zero4();
    if (wave == 0) {
      if constexpr (!GLA) {
      // Ti = (I + L)^-1, blocked, on this wave alone: the two unit-lower 16x16
      // diagonal blocks by forward substitution in fp32 (lane = block,
      // column; each band of four L columns read as float4 rows one band
      // ahead) ...
      if (lane < 32) {
        const int b = lane >> 4, c = lane & 15;
        const float* Lr = &sm.Ld[b][0][0];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
        float4 lq[2][16];
        auto band_read = [&](int Q, float4 (&dst)[16]) {
#pragma unroll
          for (int r = 4 * Q + 1; r < 16; ++r) dst[r] = *reinterpret_cast<const float4*>(Lr + r * LDR + 4 * Q);
        };
        auto band = [&](int Q, const float4 (&l)[16]) {
#pragma unroll
          for (int s = 4 * Q; s < 4 * Q + 4; ++s) {
#pragma unroll
            for (int r = s + 1; r < 16; ++r) {
              const float4 l4 = l[r];
              const float lrs = (s & 3) == 0 ? l4.x : (s & 3) == 1 ? l4.y : (s & 3) == 2 ? l4.z : l4.w;
              x[r] = fmaf(-lrs, x[s], x[r]);
            }
          }
        };
        band_read(0, lq[0]);
        band_read(1, lq[1]);
        band(0, lq[0]);
        band_read(2, lq[0]);
        band(1, lq[1]);
        band_read(3, lq[1]);
        band(2, lq[0]);
        band(3, lq[1]);
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Ti[(16 * b + r) * LDC + 16 * b + c] = Elem<T>::from_f32(x[r]);
        // column c of Ti[0][0] is row c of its transpose: 16 consecutive
        // elements, written over the diagonal block L[0][0] of the operand
        // copy of L, which only the forward substitution (from the fp32
        // copy) needed
        if (b == 0) {
#pragma unroll
          for (int h = 0; h < 16 / VEC; ++h) {
            float xv[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) xv[e] = x[VEC * h + e];
            store_vec(&sm.Lb[c * LDC + VEC * h], xv);
          }
        }
      }
      wave_lds_sync();
      // ... then the off-diagonal block Ti[1][0] = -Ti[1][1] L[1][0] Ti[0][0].
      const f32x4 m = Mma<T>::template run<16>(zero4(), &sm.Lb[16 * LDC], LDC, &sm.Lb[0], LDC, lane);
      f32x4 acc;
      if constexpr (sizeof(T) == 2) {
        // M = L[1][0] Ti[0][0] is in the accumulator layout, which is the B
        // operand layout of the 16-deep product: no round trip through LDS
        const i16x4_t av = __builtin_bit_cast(i16x4_t, *reinterpret_cast<const uint2*>(&sm.Ti[(16 + lr) * LDC + 16 + 4 * lg]));
        const i16x4_t bv = __builtin_bit_cast(i16x4_t, make_uint2(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3])));
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, zero4(), 0, 0, 0);
      } else {
        store4<T>(&sm.Mt[lr * LDC + 4 * lg], m[0], m[1], m[2], m[3]);
        wave_lds_sync();
        acc = Mma<T>::template run<16>(zero4(), &sm.Ti[16 * LDC + 16], LDC, &sm.Mt[0], LDC, lane);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.Ti[(16 + 4 * lg + e) * LDC + lr] = Elem<T>::from_f32(-acc[e]);
      }
    } else if (PREP && wave == 1) {
      gram_tile(5);
    } else if (wave == 1) {
      // Y = diag(beta) (V - K~ S^T), tiles [r][i], meanwhile.  Without the
      // delta rule Y = diag(beta) V is U already and goes to U^T.
#pragma unroll
      for (int t = 0; t < RB * IB; ++t) {
        const int rb = t / IB, ib = t % IB;
        f32x4 acc = zero4();
        if constexpr (!GLA)
          acc = Mma<T>::template run<DK>(zero4(), &sm.Kr[rb * 16 * LDK], LDK, &sm.S[ib * 16 * LDK], LDK, lane);
        const int i = ib * 16 + lr;
        const int r0 = rb * 16 + 4 * lg;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = r0 + e;
          y[e] = sm.beta[r] * (Elem<T>::to_f32(sm.V[r * DVS + i]) - acc[e]);
        }
        store4<T>(&(GLA ? sm.Ut : sm.Yt)[i * LDC + r0], y[0], y[1], y[2], y[3]);
      }
      if (o_on && !GLA) gram_tile(5);
    } else if (o_on) {
      // the inter-chunk part of the output, S Q~^T (tile [i][r] of this
      // output wave, kept live until the output is finished)
      const int t = wave - 2;
      const int ib = t / RB, rb = t % RB;
      if constexpr (!PREP)
        Oacc = Mma<T>::template run<DK>(zero4(), &sm.S[ib * 16 * LDK], LDK, &sm.Qs[rb * 16 * LDK], LDK, lane);
      if constexpr (!GLA) gram_tile(3 + t);
    }
    __syncthreads();

    if constexpr (PREP) {
      // the chunk's record: the buffers the state products read, verbatim
      using R = VecRec<T, DK>;
      char* rec = reinterpret_cast<char*>(cm.ws) + ((int64_t)seq * cm.G + prep_first + ch) * R::BYTES;
      auto put = [&](int off, const void* src, int bytes) {
        const uint4* s16 = reinterpret_cast<const uint4*>(src);
        uint4* d16 = reinterpret_cast<uint4*>(rec + off);
        for (int e = tid; e < bytes / 16; e += NT) d16[e] = s16[e];
      };
      put(R::QS, sm.Qs, (int)sizeof(sm.Qs));
      put(R::KR, sm.Kr, (int)sizeof(sm.Kr));
      put(R::KBT, sm.Kbt, (int)sizeof(sm.Kbt));
      put(R::TI, sm.Ti, (int)sizeof(sm.Ti));
      put(R::PM, sm.P, (int)sizeof(sm.P));
      put(R::EC, sm.Ec, (int)sizeof(sm.Ec));
      put(R::BETA, sm.beta, (int)sizeof(sm.beta));
      continue;
    }

    // U = Ti Y (tiles [r][i]), stored as U^T.
    if (!GLA && wave < RB * IB) {
      const int t = wave;
      const int rb = t / IB, ib = t % IB;
      const f32x4 acc = Mma<T>::template run<C>(zero4(), &sm.Ti[rb * 16 * LDC], LDC, &sm.Yt[ib * 16 * LDC], LDC, lane);
      const int i = ib * 16 + lr;
      const int r0 = rb * 16 + 4 * lg;
      store4<T>(&sm.Ut[i * LDC + r0], acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();

    // O^T += U^T P^T and store (output waves); S^T <- Diag(2^(G_C)) S^T +
    // Kbar^T U (every wave, its state tiles).
    if (wave >= 2 && o_on) {
      const int t = wave - 2;
      const int ib = t / RB, rb = t % RB;
      Oacc = Mma<T>::template run<C>(Oacc, &sm.Ut[ib * 16 * LDC], LDC, &sm.P[rb * 16 * LDC], LDC, lane);
      const int64_t tk = ch * C + rb * 16 + lr;
      if (tk < Tlen) store4<T>(oc + tk * DV + ib * 16 + 4 * lg, Oacc[0], Oacc[1], Oacc[2], Oacc[3]);
    }
#pragma unroll
    for (int m = 0; m < NST; ++m) {
      const int t = wave + NW * m;
      if (t < JB * IB) {
        const int jb = t / IB, ib = t % IB;
        const int i = ib * 16 + lr, j = jb * 16 + 4 * lg;
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[m][e] *= sm.Ec[j + e];
        Sacc[m] = Mma<T>::template run<C>(Sacc[m], &sm.Kbt[jb * 16 * LDC], LDC, &sm.Ut[ib * 16 * LDC], LDC, lane);
        store4<T>(&sm.S[i * LDK + j], Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
      }
    }
  }

  // final state slice (fp32)
  if (sT) {
#pragma unroll
    for (int m = 0; m < NST; ++m) {
      const int t = wave + NW * m;
      if (t < JB * IB) {
        const int jb = t / IB, ib = t % IB;
        const int i = ib * 16 + lr, j = jb * 16 + 4 * lg;
        *reinterpret_cast<float4*>(sT + st_off + (int64_t)i * DK + j) =
            make_float4(Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
      }
    }
  }
}

// Register staging of the second pass: a record as NR 16-byte vectors per
// thread of NTH (N16 in all), and one V vector.  (Native vectors: an array of
// the uint4 structs under a guard was kept in scratch memory.)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <int NR, int N16, int NTH>
__device__ __forceinline__ void rec_load(u32x4 (&rr)[NR], const char* src, int tid) {
  const u32x4* s16 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int e = tid + NTH * n;
    if (N16 % NTH == 0 || e < N16) rr[n] = s16[e];
  }
}
template <int NR, int N16, int NTH>
__device__ __forceinline__ void rec_stage(const u32x4 (&rr)[NR], char* dst, int tid) {
  u32x4* d16 = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int e = tid + NTH * n;
    if (N16 % NTH == 0 || e < N16) d16[e] = rr[n];
  }
}
template <class T>
__device__ __forceinline__ u32x4 v_load(const T* vc, int c, int r, int col, int64_t Tlen, int DV, bool has_v) {
  const int64_t tk = (int64_t)c * C + r;
  return has_v && tk < Tlen ? *reinterpret_cast<const u32x4*>(vc + tk * DV + col) : u32x4{0u, 0u, 0u, 0u};
}

// Second pass of the two-pass evaluation: one workgroup per (chain, SL
// consecutive 16-row value slices), a chain being a sequence's chunks
// [c0, c0 + nct) of the tile or, in a sequence split (cm), one segment of
// them, walks its chunks from their records (rec: [sequence][chunk of the
// tile] records of VecRec<T, DK>::BYTES; in a split the segment states from
// a zero start and the segment transitions from the identity with V read as
// zero, then every segment from its start state, with cm.ws laid out as for
// the single-pass split), each slice's state in the MFMA accumulators of its
// own four waves; the slices of a workgroup share the records in LDS.  Per
// chunk, three barrier-separated steps: Y = diag(beta) (V - K~ S^T) (waves
// 0, 1 of a slice) beside the inter-chunk output S Q~^T (waves 2, 3); U = Ti Y
// (waves 0, 1); the output O = S Q~^T + P U (waves 2, 3) and the state update
// (every wave).  The next chunk's record and V are loaded into registers
// while a chunk is computed and written to the other of two LDS record
// buffers in its last step.  s0 (NULL: zero) is read before sT (NULL: not
// stored) is written, by the same workgroup, so they may alias.
template <class T, int DK, int SL>
__global__ __launch_bounds__(NT * SL, SL == 1 && sizeof(T) == 2 ? 2 : 1) void vec_state_kernel(
    const T* __restrict__ v, const char* __restrict__ rec, const float* s0, T* __restrict__ o,
    float* sT, int nseq, int64_t Tseq, int64_t c0, int nct, int DV, int xcd_map, gdn::pipe::ChainMap cm) {
  using Sm = Smem<T, DK>;
  using R = VecRec<T, DK>;
  constexpr int NTH = NT * SL;
  constexpr int LDK = Sm::LDK;
  constexpr int LDC = Sm::LDC;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int NVV = C * DVS / VEC;             // 16-byte vectors of one slice's V
  constexpr int N16 = R::BYTES / 16;             // 16-byte vectors of a record
  constexpr int NR = (N16 + NTH - 1) / NTH;      // per thread
  constexpr int JB = DK / 16;
  constexpr int IB = DVS / 16;
  constexpr int RB = C / 16;
  constexpr int NST = (JB * IB + NW - 1) / NW;
  static_assert(IB == 1 && RB == 2 && NW == 4, "wave roles below: two Y waves, two output waves");
  static_assert(NVV <= NT, "one thread of the slice's waves per V vector");

  __shared__ __attribute__((aligned(16))) char recb[2][R::BYTES];
  __shared__ __attribute__((aligned(16))) T Vb[2][SL][C * DVS];
  __shared__ __attribute__((aligned(16))) T Ssh[SL][DVS * LDK];  // operand copy of each state slice
  __shared__ __attribute__((aligned(16))) T Yt[SL][DVS * LDC];
  __shared__ __attribute__((aligned(16))) T Ut[SL][DVS * LDC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = wave_all / NW;    // slice of this wave within the workgroup
  const int wave = wave_all % NW; // role within the slice
  const int ts = tid % NT;        // thread within the slice's waves
  const int lr = lane & 15;
  const int lg = lane >> 4;

  const int NSG = DV / (DVS * SL);  // slice groups per sequence
  int chain, sg;
  {
    const int w = blockIdx.x;
    if (xcd_map) {
      const int x = w & 7, r = w >> 3;
      sg = r % NSG;
      chain = (r / NSG) * 8 + x;
    } else {
      chain = w / NSG;
      sg = w % NSG;
    }
  }
  if (chain >= gdn::pipe::map_chains(cm)) return;
  const int slice = sg * SL + h;
  const int64_t dd = (int64_t)DK * DV;
  if constexpr (POISON_LDS) {
    lds_poison(recb, tid, NT * SL);
    lds_poison(Vb, tid, NT * SL);
    lds_poison(Ssh, tid, NT * SL);
    lds_poison(Yt, tid, NT * SL);
    lds_poison(Ut, tid, NT * SL);
    __syncthreads();
  }

  // this chain's sequence, chunks of the tile, start and end state, and
  // whether it reads V and writes output (cm.mode as for chunk_vec_kernel:
  // whole sequences, or the first and last launch of a sequence split, whose
  // segments are cm.L tokens; the tile then holds the whole sequence)
  int seq = chain, cf = 0, ncc = nct;
  bool v_on = true, o_on = true, ident = false;
  const float* s0c = s0 ? s0 + (int64_t)chain * dd : nullptr;
  float* sTc = sT ? sT + (int64_t)chain * dd : nullptr;
  if (cm.mode == gdn::pipe::MAP_SPLIT_A) {
    const int per = nseq * (cm.G - 1);
    const int kind = chain / per, r = chain % per;
    seq = r / (cm.G - 1);
    ncc = (int)(cm.L / C);
    cf = (r % (cm.G - 1)) * ncc;
    o_on = false;
    v_on = kind == 0;
    ident = kind == 1;
    s0c = nullptr;
    sTc = cm.ws + ((int64_t)kind * per + r) * dd;
  } else if (cm.mode == gdn::pipe::MAP_SPLIT_C) {
    seq = chain / cm.G;
    const int g = chain % cm.G;
    cf = g * (int)(cm.L / C);
    ncc = g == cm.G - 1 ? nct - cf : (int)(cm.L / C);
    s0c = cm.ws + (2 * (int64_t)nseq * (cm.G - 1) + (int64_t)seq * cm.G + g) * dd;
    sTc = g == cm.G - 1 && sT ? sT + (int64_t)seq * dd : nullptr;
  }
  const int64_t st_off = (int64_t)slice * DVS * DK;          // this slice's rows within a state
  const int64_t tok0 = (int64_t)seq * Tseq + (c0 + cf) * C;  // first token of the chain in memory
  const int64_t Tlen = Tseq - (c0 + cf) * C;                 // tokens of the sequence from there
  const T* vc = v + tok0 * DV + slice * DVS;
  T* oc = o + tok0 * DV + slice * DVS;
  const char* rc = rec + ((int64_t)seq * nct + cf) * R::BYTES;
  T* Sh = Ssh[h];
  T* Yh = Yt[h];
  T* Uh = Ut[h];

  f32x4 Sacc[NST];
#pragma unroll
  for (int m = 0; m < NST; ++m) {
    const int t = wave + NW * m;
    Sacc[m] = zero4();
    if (t < JB * IB) {
      const int j = t * 16 + 4 * lg;
      if (ident) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[m][e] = slice * DVS + lr == j + e ? 1.f : 0.f;
      } else if (s0c) {
        const float4 s4 = *reinterpret_cast<const float4*>(s0c + st_off + (int64_t)lr * DK + j);
        Sacc[m] = f32x4{s4.x, s4.y, s4.z, s4.w};
      }
      store4<T>(&Sh[lr * LDK + j], Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
    }
  }

  // register staging of the records (all threads) and of each slice's V (V
  // rows past the end of the sequence are written as zero), two chunks ahead:
  // while chunk c is computed, the records of chunks c+1 (set A) and c+2 (set
  // B) are in flight; at its end, c+1 goes to LDS and c+3 is requested into
  // the set that held it.  The loop is unrolled by two so that the two
  // register sets stay static.
  u32x4 rA[NR], rB[NR], vA = u32x4{0u, 0u, 0u, 0u}, vB = u32x4{0u, 0u, 0u, 0u};
  const bool has_v = ts < NVV;       // this thread stages a V vector
  const bool read_v = has_v && v_on;  // ... read from v (else zero)
  const int vr = ts / (DVS / VEC), vcg = ts % (DVS / VEC);  // token, 16-byte column group of this V vector
  if (ncc > 0) {
    rec_load<NR, N16, NTH>(rA, rc, tid);
    vA = v_load<T>(vc, 0, vr, vcg * VEC, Tlen, DV, read_v);
    rec_stage<NR, N16, NTH>(rA, recb[0], tid);
    if (has_v) reinterpret_cast<u32x4*>(Vb[0][h])[ts] = vA;
  }
  if (ncc > 1) {
    rec_load<NR, N16, NTH>(rA, rc + R::BYTES, tid);
    vA = v_load<T>(vc, 1, vr, vcg * VEC, Tlen, DV, read_v);
  }
  if (ncc > 2) {
    rec_load<NR, N16, NTH>(rB, rc + 2 * R::BYTES, tid);
    vB = v_load<T>(vc, 2, vr, vcg * VEC, Tlen, DV, read_v);
  }

  // one chunk: its products, then the next record from set `nx` to LDS and
  // the record three chunks ahead into `nx`
  auto chunk = [&](int c, u32x4 (&nx)[NR], u32x4& nv) {
    const int b = c & 1;
    const T* Qs = reinterpret_cast<const T*>(recb[b] + R::QS);
    const T* Kr = reinterpret_cast<const T*>(recb[b] + R::KR);
    const T* Kbt = reinterpret_cast<const T*>(recb[b] + R::KBT);
    const T* Ti = reinterpret_cast<const T*>(recb[b] + R::TI);
    const T* Pm = reinterpret_cast<const T*>(recb[b] + R::PM);
    const float* Ec = reinterpret_cast<const float*>(recb[b] + R::EC);
    const float* be = reinterpret_cast<const float*>(recb[b] + R::BETA);
    const T* Vh = Vb[b][h];
    __syncthreads();  // this chunk's record, V and the state copies are in LDS

    f32x4 Oacc = zero4();
    if (wave < 2) {
      // Y = diag(beta) (V - K~ S^T), tile [r][i] with rb = wave
      const int rb = wave;
      const f32x4 acc = Mma<T>::template run<DK>(zero4(), &Kr[rb * 16 * LDK], LDK, Sh, LDK, lane);
      const int r0 = rb * 16 + 4 * lg;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = be[r0 + e] * (Elem<T>::to_f32(Vh[(r0 + e) * DVS + lr]) - acc[e]);
      store4<T>(&Yh[lr * LDC + r0], y[0], y[1], y[2], y[3]);
    } else {
      // S Q~^T, tile [i][r] with rb = wave - 2, kept live until the output is finished
      Oacc = Mma<T>::template run<DK>(zero4(), Sh, LDK, &Qs[(wave - 2) * 16 * LDK], LDK, lane);
    }
    __syncthreads();

    // U = Ti Y (tile [r][i] with rb = wave), stored as U^T
    if (wave < 2) {
      const int rb = wave;
      const f32x4 acc = Mma<T>::template run<C>(zero4(), &Ti[rb * 16 * LDC], LDC, Yh, LDC, lane);
      store4<T>(&Uh[lr * LDC + rb * 16 + 4 * lg], acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();

    // the output (waves 2, 3) and the state update (every wave); the next
    // chunk's record goes to the other buffer
    if (wave >= 2) {
      const int rb = wave - 2;
      Oacc = Mma<T>::template run<C>(Oacc, Uh, LDC, &Pm[rb * 16 * LDC], LDC, lane);
      const int64_t tk = (int64_t)c * C + rb * 16 + lr;
      if (o_on && tk < Tlen) store4<T>(oc + tk * DV + 4 * lg, Oacc[0], Oacc[1], Oacc[2], Oacc[3]);
    }
#pragma unroll
    for (int m = 0; m < NST; ++m) {
      const int t = wave + NW * m;
      if (t < JB * IB) {
        const int j = t * 16 + 4 * lg;
#pragma unroll
        for (int e = 0; e < 4; ++e) Sacc[m][e] *= Ec[j + e];
        Sacc[m] = Mma<T>::template run<C>(Sacc[m], &Kbt[t * 16 * LDC], LDC, Uh, LDC, lane);
        store4<T>(&Sh[lr * LDK + j], Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
      }
    }
    if (c + 1 < ncc) {
      rec_stage<NR, N16, NTH>(nx, recb[b ^ 1], tid);
      if (has_v) reinterpret_cast<u32x4*>(Vb[b ^ 1][h])[ts] = nv;
      if (c + 3 < ncc) {
        rec_load<NR, N16, NTH>(nx, rc + (int64_t)(c + 3) * R::BYTES, tid);
        nv = v_load<T>(vc, c + 3, vr, vcg * VEC, Tlen, DV, read_v);
      }
    }
  };
  for (int c = 0; c < ncc; c += 2) {
    chunk(c, rA, vA);
    if (c + 1 < ncc) chunk(c + 1, rB, vB);
  }

  if (sTc) {
#pragma unroll
    for (int m = 0; m < NST; ++m) {
      const int t = wave + NW * m;
      if (t < JB * IB) {
        const int j = t * 16 + 4 * lg;
        *reinterpret_cast<float4*>(sTc + st_off + (int64_t)lr * DK + j) =
            make_float4(Sacc[m][0], Sacc[m][1], Sacc[m][2], Sacc[m][3]);
      }
    }
  }
}


// Second pass for bf16 records, pipelined: one state wave per 16-row value
// slice (SL slices per workgroup) and one loader wave.  The loader moves each
// chunk's record and value slices into LDS with LDS-DMA loads, two chunks
// ahead into three buffers, and waits only for the next chunk, so a period
// has a single barrier.  A state wave keeps its slice of S^T ([dk][dv], 16
// columns) in MFMA accumulators and evaluates the chunk in registers, every
// product a 16x16x32 bf16 MFMA whose 32-deep reduction index runs in the
// order of two stacked accumulator tiles (row 4g + e of the first tile, then
// of the second, for lane group g = lane / 16): an accumulator pair is then
// an operand as it stands, and the LDS operand of the other side is read as
// two 8-byte halves per lane in the same order.  Per chunk (tokens r, s;
// slice columns i; key columns j):
//   Z = K~ S^T            [r][i]   (the state before the chunk)
//   O^T = S Q~^T          [i][r]
//   Y = diag(beta) (V - Z)
//   U = Ti Y              [r][i]
//   O^T += U^T P^T        [i][r]   -> o, 8 bytes per lane and token
//   S^T = diag(Ec) S^T + Kbar^T U
// The operands are rounded to bf16 where the 32-token kernel rounds them (S,
// Y, U), with fp32 accumulation; only the order of the sums differs.  Chains
// and the sequence-split modes are those of vec_state_kernel, whose
// arguments this kernel takes.
template <int DK, int SL>
__global__ __launch_bounds__(64 * (SL + 1), 1) void vec_state_pipe_kernel(
    const bf16_t* __restrict__ v, const char* __restrict__ rec, const float* s0, bf16_t* __restrict__ o,
    float* sT, int nseq, int64_t Tseq, int64_t c0, int nct, int DV, int xcd_map, gdn::pipe::ChainMap cm) {
  using namespace gdn::pipe;
  using R = VecRec<bf16_t, DK>;
  using Sm = Smem<bf16_t, DK>;
  constexpr int LDK = Sm::LDK;
  constexpr int LDC = Sm::LDC;
  constexpr int KB = DK / 32;        // 32-deep key blocks
  constexpr int JB = DK / 16;        // 16-row key tiles of S^T
  constexpr int NREC = R::BYTES / 1024;  // 1 KiB LDS-DMA loads per record
  constexpr int NLD = NREC + SL;         // loads per chunk (record, value slices)
  static_assert(R::BYTES % 1024 == 0 && NLD < 64, "record loads and their wait count");
  // s_waitcnt vmcnt(NLD), other counters not waited for (vmcnt bits [3:0], [15:14])
  constexpr int WAIT_NEXT = 0x0f70 | (NLD & 15) | ((NLD >> 4) << 14);
  static_assert(C == 32 && DVS == 16, "two 16-token blocks, 16-column slices");

  __shared__ __attribute__((aligned(1024))) char recb[3][R::BYTES];
  __shared__ __attribute__((aligned(16))) bf16_t Vb[3][SL][C * DVS];  // [token][column] per slice

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // < SL: state wave of slice `wave`; else loader
  const int lr = lane & 15;
  const int lg = lane >> 4;

  const int NSG = DV / (DVS * SL);
  int chain, sg;
  {
    const int w = blockIdx.x;
    if (xcd_map) {
      const int x = w & 7, r = w >> 3;
      sg = r % NSG;
      chain = (r / NSG) * 8 + x;
    } else {
      chain = w / NSG;
      sg = w % NSG;
    }
  }
  if (chain >= map_chains(cm)) return;
  const int64_t dd = (int64_t)DK * DV;
  if constexpr (POISON_LDS) {
    lds_poison(recb, tid, 64 * (SL + 1));
    lds_poison(Vb, tid, 64 * (SL + 1));
    __syncthreads();
  }

  // the chain: as for vec_state_kernel
  int seq = chain, cf = 0, ncc = nct;
  bool v_on = true, o_on = true, ident = false;
  const float* s0c = s0 ? s0 + (int64_t)chain * dd : nullptr;
  float* sTc = sT ? sT + (int64_t)chain * dd : nullptr;
  if (cm.mode == MAP_SPLIT_A) {
    const int per = nseq * (cm.G - 1);
    const int kind = chain / per, r = chain % per;
    seq = r / (cm.G - 1);
    ncc = (int)(cm.L / C);
    cf = (r % (cm.G - 1)) * ncc;
    o_on = false;
    v_on = kind == 0;
    ident = kind == 1;
    s0c = nullptr;
    sTc = cm.ws + ((int64_t)kind * per + r) * dd;
  } else if (cm.mode == MAP_SPLIT_C) {
    seq = chain / cm.G;
    const int g = chain % cm.G;
    cf = g * (int)(cm.L / C);
    ncc = g == cm.G - 1 ? nct - cf : (int)(cm.L / C);
    s0c = cm.ws + (2 * (int64_t)nseq * (cm.G - 1) + (int64_t)seq * cm.G + g) * dd;
    sTc = g == cm.G - 1 && sT ? sT + (int64_t)seq * dd : nullptr;
  }
  const int64_t tok0 = (int64_t)seq * Tseq + (c0 + cf) * C;  // first token of the chain in memory
  const int64_t Tlen = Tseq - (c0 + cf) * C;                 // tokens of the sequence from there
  const char* rc = rec + ((int64_t)seq * nct + cf) * R::BYTES;

  // this workgroup's value columns; tokens past the sequence fall outside the
  // buffer range and read as zeros, as does everything with v_on off
  const bf16_t* vg = v + tok0 * DV + sg * SL * DVS;
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vg, v_on && Tlen > 0 ? (uint32_t)(Tlen * DV * 2) : 0u);
  if (wave == SL) {
    // ---------------------------------------------------------------- loader
    // value slice s of chunk c: lane i fetches half i % 2 of token i / 2 (a
    // token's 16 columns are 32 bytes)
    const uint32_t voff = (uint32_t)((lane >> 1) * DV * 2 + (lane & 1) * 16);
    auto issue = [&](int c) {
      const int b = c % 3;
      const __amdgpu_buffer_rsrc_t rr = make_rsrc(rc + (int64_t)c * R::BYTES, (uint32_t)R::BYTES);
#pragma unroll
      for (int n = 0; n < NREC; ++n)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void*)&recb[b][n * 1024], 16, (uint32_t)(16 * lane),
                                                 n * 1024, 0, 0);
      const uint32_t v0 = (uint32_t)(c * C * DV * 2);
#pragma unroll
      for (int s = 0; s < SL; ++s)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)&Vb[b][s][0], 16, voff, (int)(v0 + s * DVS * 2), 0,
                                                 0);
    };
    if (ncc > 0) issue(0);
    if (ncc > 1) {
      issue(1);
      __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
    } else {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    }
    lds_barrier_keep_dma();
    for (int c = 0; c < ncc; ++c) {
      // buffer (c + 2) % 3 held chunk c - 1, read before the last barrier
      if (c + 2 < ncc) {
        issue(c + 2);
        __builtin_amdgcn_s_waitcnt(WAIT_NEXT);  // chunk c + 1 has landed
      } else {
        __builtin_amdgcn_s_waitcnt(0x0f70);
      }
      lds_barrier_keep_dma();
    }
    return;
  }

  // ------------------------------------------------------------ state wave
  const int slice = sg * SL + wave;
  const int64_t st_off = (int64_t)slice * DVS * DK;  // this slice's rows within a state
  bf16_t* oc = o + tok0 * DV + slice * DVS;
  // Sacc[jb]: S^T tile [j = 16 jb + 4 lg + e][i = lr]
  f32x4 Sacc[JB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    const int j = jb * 16 + 4 * lg;
    Sacc[jb] = zero4();
    if (ident) {
#pragma unroll
      for (int e = 0; e < 4; ++e) Sacc[jb][e] = slice * DVS + lr == j + e ? 1.f : 0.f;
    } else if (s0c) {
      const float4 s4 = *reinterpret_cast<const float4*>(s0c + st_off + (int64_t)lr * DK + j);
      Sacc[jb] = f32x4{s4.x, s4.y, s4.z, s4.w};
    }
  }
  lds_barrier_keep_dma();

  // per-lane byte offsets of the two 8-byte halves of a fragment row
  const int koff = 8 * lg;  // + 32 for the second half
  for (int c = 0; c < ncc; ++c) {
    const char* rb_ = recb[c % 3];
    const lptr Qb = lane_base(rb_ + R::QS, lr * LDK * 2 + koff);
    const lptr Kb = lane_base(rb_ + R::KR, lr * LDK * 2 + koff);
    const lptr Bt = lane_base(rb_ + R::KBT, lr * LDC * 2 + koff);
    const lptr Tb = lane_base(rb_ + R::TI, lr * LDC * 2 + koff);
    const lptr Pb = lane_base(rb_ + R::PM, lr * LDC * 2 + koff);
    const char* Ec = rb_ + R::EC;
    const char* be = rb_ + R::BETA;
    const bf16_t* Vh = Vb[c % 3][wave];

    // Four phases separated by scheduling fences, so that each phase's LDS
    // reads are in flight while the previous phase's products run (left to
    // itself the compiler issues every read just before its use, and the
    // period then waits for dozens of LDS round trips in a row).
    // 1: the operands of Z and the decay; S as an operand
    uint2 kr[2][KB][2];
    float4 ec[JB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int pp = 0; pp < KB; ++pp) {
        const int off = rb * 16 * LDK * 2 + pp * 64;
        kr[rb][pp][0] = ld3<uint2>(Kb, off);
        kr[rb][pp][1] = ld3<uint2>(Kb, off + 32);
      }
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) ec[jb] = lds_at<float4>(Ec, (jb * 16 + 4 * lg) * 4);
    bf16x8_t Sop[KB];
#pragma unroll
    for (int pp = 0; pp < KB; ++pp) Sop[pp] = pack_op(Sacc[2 * pp], Sacc[2 * pp + 1]);
    __builtin_amdgcn_sched_barrier(0);

    // 2: Z = K~ S^T; the decay diag(Ec) S^T; reads for the output and Y
    uint2 qs[2][KB][2];
    float4 b4[2];
    float vv[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int pp = 0; pp < KB; ++pp) {
        const int off = rb * 16 * LDK * 2 + pp * 64;
        qs[rb][pp][0] = ld3<uint2>(Qb, off);
        qs[rb][pp][1] = ld3<uint2>(Qb, off + 32);
      }
      const int r0 = rb * 16 + 4 * lg;
      b4[rb] = lds_at<float4>(be, r0 * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[rb][e] = bf16_to_f32(Vh[(r0 + e) * DVS + lr]);
    }
    f32x4 Z[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      Z[rb] = zero4();
#pragma unroll
      for (int pp = 0; pp < KB; ++pp) Z[rb] = mfma(as_op(kr[rb][pp][0], kr[rb][pp][1]), Sop[pp], Z[rb]);
    }
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      Sacc[jb][0] *= ec[jb].x;
      Sacc[jb][1] *= ec[jb].y;
      Sacc[jb][2] *= ec[jb].z;
      Sacc[jb][3] *= ec[jb].w;
    }
    __builtin_amdgcn_sched_barrier(0);

    // 3: O^T = S Q~^T; Y = diag(beta) (V - Z), rows r = 16 rb + 4 lg + e;
    // reads for U, the output and the state update
    uint2 ti[2][2], pm[2][2], kt[JB][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int off = rb * 16 * LDC * 2;
      ti[rb][0] = ld3<uint2>(Tb, off);
      ti[rb][1] = ld3<uint2>(Tb, off + 32);
      pm[rb][0] = ld3<uint2>(Pb, off);
      pm[rb][1] = ld3<uint2>(Pb, off + 32);
    }
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int off = jb * 16 * LDC * 2;
      kt[jb][0] = ld3<uint2>(Bt, off);
      kt[jb][1] = ld3<uint2>(Bt, off + 32);
    }
    f32x4 O[2], Y[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      O[rb] = zero4();
#pragma unroll
      for (int pp = 0; pp < KB; ++pp) O[rb] = mfma(Sop[pp], as_op(qs[rb][pp][0], qs[rb][pp][1]), O[rb]);
      const float bb[4] = {b4[rb].x, b4[rb].y, b4[rb].z, b4[rb].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) Y[rb][e] = bb[e] * (vv[rb][e] - Z[rb][e]);
    }
    const bf16x8_t Yop = pack_op(Y[0], Y[1]);
    __builtin_amdgcn_sched_barrier(0);

    // 4: U = Ti Y; O^T += U^T P^T and o (token 16 rb + lr, columns 4 lg ..
    // 4 lg + 3); S^T += Kbar^T U
    f32x4 U[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) U[rb] = mfma(as_op(ti[rb][0], ti[rb][1]), Yop, zero4());
    const bf16x8_t Uop = pack_op(U[0], U[1]);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) O[rb] = mfma(Uop, as_op(pm[rb][0], pm[rb][1]), O[rb]);
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) Sacc[jb] = mfma(as_op(kt[jb][0], kt[jb][1]), Uop, Sacc[jb]);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int64_t tk = (int64_t)c * C + rb * 16 + lr;
      if (o_on && tk < Tlen) store4<bf16_t>(oc + tk * DV + 4 * lg, O[rb][0], O[rb][1], O[rb][2], O[rb][3]);
    }
    lds_barrier_keep_dma();
  }

  if (sTc) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int j = jb * 16 + 4 * lg;
      *reinterpret_cast<float4*>(sTc + st_off + (int64_t)lr * DK + j) =
          make_float4(Sacc[jb][0], Sacc[jb][1], Sacc[jb][2], Sacc[jb][3]);
    }
  }
}

}  // namespace vec
}  // namespace gdn
