// Parallel-scan route of the gated delta rule on gfx950 (the pages' other
// route besides the chunked one, kept for the route comparison).
//
// Sources (web pages, by title and section):
//   [P1] "Gated DeltaNet GPU并行实现：拆解线性注意力循环的两种高效方案"
//        §2.3 each token is an affine map of the state and maps compose
//        associatively; §3.1 evaluate the recurrence as a parallel scan over
//        those maps; §3.4 / §5.1 the scan and chunked routes compared.
//
// The token map is S -> S A_t + B_t with A_t = alpha_t (I - beta_t k_t k_t^T)
// and B_t = beta_t v_t k_t^T.  The scan is blocked: every block of L tokens
// of a sequence is reduced to its map (A_blk, B_blk), the blocks' start
// states follow from the exclusive scan over those maps
// (start_{g+1} = start_g A_g + B_g, split_combine_kernel), and every block
// then replays its tokens from its start state to write the outputs.
//   AGG: blocks 0 .. G-2, kind 0: B_blk (zero start, with V), kind 1: A_blk
//        (identity start, V read as zero); written to ws slots tilde, trans.
//   OUT: blocks 0 .. G-1 from ws slot start, output o; the last block's
//        state is the final state.  With G = 1 the start slots are laid out
//        as an initial state [nseq, D, D]: the token-by-token forward pass
//        passes the initial state itself as ws, or NULL for a zero start.
// Reducing a block to its map is the token loop itself on the stacked state
// [B; A] (a rank-1 update per token, O(d^2) instead of a d^3 product).
//
// VEC: a per-dimension gate alpha_t in (0,1]^{d_k} ([P1] §2.2 allows a vector
// gate) that decays the key columns of the state, A_t = Diag(alpha_t)(I -
// beta_t k_t k_t^T); alpha is then [B,H,T,d_k].  The maps stay affine, so the
// same blocked scan applies.
//
// Layout: a workgroup owns 16 rows of one state; 16 consecutive lanes hold a
// row (D / 16 columns each), and row dot products are summed across those
// lanes with DPP rotations.  Tokens are staged 32 at a time in LDS.
#pragma once

#include "gdn_common.hpp"

namespace gdn {
namespace scan {

enum { SCAN_AGG = 0, SCAN_OUT = 1 };
constexpr int TPR = 16;              // threads per state row
constexpr int THREADS = 256;
constexpr int RPW = THREADS / TPR;   // rows per workgroup
constexpr int TILE = 32;             // tokens per LDS tile (the scan route)
constexpr int SHORT_TILE = 8;        // tokens per tile for short sequences


// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
// Each step reads lanes inside the row only, so bound_ctrl (and the old
// value 0) never applies; with them the compiler fuses the DPP move into the
// add (v_add_f32_dpp), one instruction per step instead of two.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, true));  // row_ror:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, true));  // row_ror:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, true));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, true));   // quad [1,0,3,2]
  return v;
}

// Workgroups per launch.
__host__ __device__ inline int64_t scan_blocks(int mode, int nseq, int G, int D) {
  const int64_t per = mode == SCAN_AGG ? 2 * (int64_t)(G - 1) : (int64_t)G;
  return (int64_t)nseq * per * (D / RPW);
}

// A tile's inputs are loaded in words of EPW elements: bf16 pairs as 32-bit
// words (the compiler would otherwise pack two 16-bit loads into a register
// as soon as they land, waiting for them), fp32 one element per word.
template <class E> struct TileWord {
  typedef float type;
  static constexpr int EPW = 1;
  static __device__ __forceinline__ float elem(float w, int) { return w; }
};
template <> struct TileWord<bf16_t> {
  typedef uint32_t type;
  static constexpr int EPW = 2;
  static __device__ __forceinline__ float elem(uint32_t w, int h) {
    return Elem<bf16_t>::to_f32((bf16_t)(w >> (16 * h)));
  }
};

// Words of one tile's value rows (TL x RPW elements) per thread, at least
// one: with short tiles the threads past the rows reread the tile's last
// word and do not stage it.
template <class E, int TL> struct VWords {
  static constexpr int value = (TL * RPW / TileWord<E>::EPW + THREADS - 1) / THREADS;
};

// Loads one tile's inputs into registers (the tile goes to LDS after the
// current one has been computed): keys and queries (TL x D, word
// p = tid + THREADS i holds elements EPW p ..), per-dimension gates (element
// tid + THREADS i), this workgroup's value rows (TL x RPW, in words like
// the keys), scalar gates (threads below TL).  Every load is
// unconditional: past the n tokens of a ragged tile it reads the last token
// again, and the tile is masked when it goes to LDS.  (A conditional load
// ends in a register copy that waits for it, which would serialize the
// loads.)
template <class E, int D, bool VEC, int TL>
__device__ __forceinline__ void fetch_tile(typename TileWord<E>::type (&kreg)[TL * D / THREADS / TileWord<E>::EPW],
                                           typename TileWord<E>::type (&qreg)[TL * D / THREADS / TileWord<E>::EPW],
                                           typename TileWord<E>::type (&vreg)[(VWords<E, TL>::value)],
                                           float (&avreg)[VEC ? TL * D / THREADS : 1], float& areg, float& breg,
                                           const E* q, const E* k, const E* v, const float* alpha, const float* beta,
                                           int64_t base, int64_t tt, int n, int rg, int tid) {
  typedef typename TileWord<E>::type W;
  constexpr int EPW = TileWord<E>::EPW;
#pragma unroll
  for (int i = 0; i < TL * D / THREADS / EPW; ++i) {
    const int e = EPW * (tid + THREADS * i), c = e % D;
    const int t = e / D < n ? e / D : n - 1;
    kreg[i] = *reinterpret_cast<const W*>(k + (base + tt + t) * D + c);
    qreg[i] = *reinterpret_cast<const W*>(q + (base + tt + t) * D + c);
  }
  if constexpr (VEC) {
#pragma unroll
    for (int i = 0; i < TL * D / THREADS; ++i) {
      const int e = tid + THREADS * i, c = e % D;
      const int t = e / D < n ? e / D : n - 1;
      avreg[i] = alpha[(base + tt + t) * D + c];
    }
  }
#pragma unroll
  for (int i = 0; i < VWords<E, TL>::value; ++i) {
    int e = EPW * (tid + THREADS * i);
    e = e < TL * RPW ? e : TL * RPW - EPW;
    const int r = e % RPW;
    const int t = e / RPW < n ? e / RPW : n - 1;
    vreg[i] = *reinterpret_cast<const W*>(v + (base + tt + t) * D + rg * RPW + r);
  }
  if (tid < TL) {
    const int t = tid < n ? tid : n - 1;
    if constexpr (!VEC) areg = alpha[base + tt + t];
    breg = beta[base + tt + t];
  }
}

// TL: tokens per LDS tile (TILE for the scan route, SHORT_TILE for short
// sequences: a smaller LDS footprint, so more workgroups share a CU).
template <class E, int D, bool VEC = false, int TL = TILE>
__global__ __launch_bounds__(THREADS) void scan_tokens_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, E* __restrict__ o,
    float* final_state, int mode, int nseq, int G, int64_t T, int64_t L,
    float* ws) {  // ws and final_state may be one array (G = 1: the start state is the initial state)
  constexpr int CPT = D / TPR;  // columns per thread
  static_assert(TL * D % (THREADS * TileWord<E>::EPW) == 0 && TL <= THREADS, "tile words spread evenly");
  __shared__ float ks[TL][D], qs[TL][D];
  __shared__ float vs[TL][RPW], os[TL][RPW];
  __shared__ float as_[TL], bs_[TL];
  __shared__ float av[VEC ? TL : 1][VEC ? D : 1];  // per-dimension gates

  int64_t b = blockIdx.x;
  const int rg = (int)(b % (D / RPW));
  b /= D / RPW;
  int seq, g, kind;
  if (mode == SCAN_AGG) {
    kind = (int)(b % 2);
    b /= 2;
    g = (int)(b % (G - 1));
    seq = (int)(b / (G - 1));
  } else {
    kind = 2;
    g = (int)(b % G);
    seq = (int)(b / G);
  }
  if (seq >= nseq) return;
  const int tid = threadIdx.x, rl = tid / TPR, x = tid % TPR;
  if constexpr (POISON_LDS) {
    lds_poison(ks, tid, THREADS);
    lds_poison(qs, tid, THREADS);
    lds_poison(vs, tid, THREADS);
    lds_poison(os, tid, THREADS);
    lds_poison(as_, tid, THREADS);
    lds_poison(bs_, tid, THREADS);
    lds_poison(av, tid, THREADS);
    __syncthreads();
  }
  const int row = rg * RPW + rl;
  const int c0 = x * CPT;
  const int64_t t0 = (int64_t)g * L;
  const int64_t len = (mode == SCAN_OUT && g == G - 1) ? T - t0 : L;
  const int64_t dd = (int64_t)D * D, per = (int64_t)nseq * (G - 1);
  const int64_t base = (int64_t)seq * T + t0;  // first token in memory

  float s[CPT];
  if (kind == 0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) s[j] = 0.f;
  } else if (kind == 1) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) s[j] = row == c0 + j ? 1.f : 0.f;
  } else if (!ws) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) s[j] = 0.f;
  } else {
    const float* st = ws + (2 * per + (int64_t)seq * G + g) * dd + (int64_t)row * D + c0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) s[j] = st[j];
  }
  // The start state is in registers before the tiles are: left pending, its
  // loads would make the compiler wait for every load in flight (the next
  // tile's too) at the first token of each tile.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  // Tiles are software-pipelined: the next tile's inputs are loaded into
  // registers while the current one is computed, and go to LDS after it.
  typedef typename TileWord<E>::type W;
  constexpr int EPW = TileWord<E>::EPW;
  constexpr int NKQ = TL * D / THREADS / EPW, NV = VWords<E, TL>::value;
  W kreg[NKQ], qreg[NKQ], vreg[NV];
  float avreg[VEC ? TL * D / THREADS : 1];
  float areg = 1.f, breg = 0.f;
  if (len > 0)
    fetch_tile<E, D, VEC, TL>(kreg, qreg, vreg, avreg, areg, breg, q, k, v, alpha, beta, base, 0,
                              (int)(len < TL ? len : TL), rg, tid);
  for (int64_t tt = 0; tt < len; tt += TL) {
    const int n = (int)(len - tt < TL ? len - tt : TL);
    // stage the tile: keys, queries, this workgroup's value rows, gates
#pragma unroll
    for (int i = 0; i < NKQ; ++i) {
      const int e = EPW * (tid + THREADS * i), t = e / D, c = e % D;
      const bool in = t < n;
#pragma unroll
      for (int h = 0; h < EPW; ++h) {
        ks[t][c + h] = in ? TileWord<E>::elem(kreg[i], h) : 0.f;
        qs[t][c + h] = in ? TileWord<E>::elem(qreg[i], h) : 0.f;
      }
    }
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < TL * D / THREADS; ++i) {
        const int e = tid + THREADS * i, t = e / D, c = e % D;
        av[t][c] = t < n ? avreg[i] : 1.f;
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = EPW * (tid + THREADS * i), t = e / RPW, r = e % RPW;
      if (e < TL * RPW) {
#pragma unroll
        for (int h = 0; h < EPW; ++h) vs[t][r + h] = (t < n && kind != 1) ? TileWord<E>::elem(vreg[i], h) : 0.f;
      }
    }
    if (tid < TL) {
      as_[tid] = (!VEC && tid < n) ? areg : 1.f;
      bs_[tid] = tid < n ? breg : 0.f;
    }
    __syncthreads();
    if (tt + TL < len) {
      const int64_t nt = tt + TL;
      fetch_tile<E, D, VEC, TL>(kreg, qreg, vreg, avreg, areg, breg, q, k, v, alpha, beta, base, nt,
                                (int)(len - nt < TL ? len - nt : TL), rg, tid);
    }
    for (int t = 0; t < n; ++t) {
      const float a = as_[t], bt = bs_[t];
      float kr[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) kr[j] = ks[t][c0 + j];
      // S <- alpha S;  r = S k;  u = beta (v - r);  S <- S + u k^T
      float r = 0.f;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        s[j] *= VEC ? av[t][c0 + j] : a;
        r = fmaf(s[j], kr[j], r);
      }
      r = row16_sum(r);
      const float u = bt * (vs[t][rl] - r);
#pragma unroll
      for (int j = 0; j < CPT; ++j) s[j] = fmaf(u, kr[j], s[j]);
      if (mode == SCAN_OUT) {
        float oq = 0.f;
#pragma unroll
        for (int j = 0; j < CPT; ++j) oq = fmaf(s[j], qs[t][c0 + j], oq);
        oq = row16_sum(oq);
        if (x == 0) os[t][rl] = oq;
      }
    }
    __syncthreads();
    if (mode == SCAN_OUT) {
      for (int e = tid; e < n * RPW; e += THREADS) {
        const int t = e / RPW, r = e % RPW;
        o[(base + tt + t) * D + rg * RPW + r] = Elem<E>::from_f32(os[t][r]);
      }
    }
  }

  float* dst = nullptr;
  if (mode == SCAN_AGG) dst = ws + ((int64_t)kind * per + (int64_t)seq * (G - 1) + g) * dd;
  else if (g == G - 1 && final_state) dst = final_state + (int64_t)seq * dd;
  if (dst) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) dst[(int64_t)row * D + c0 + j] = s[j];
  }
}

}  // namespace scan
}  // namespace gdn
