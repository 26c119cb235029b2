// Pipelined chunked forward pass of the gated delta rule for bf16 inputs,
// d_k = d_v = 128, 64-token chunks, on gfx950.
//
// Sources (web pages, by title and section):
//   [P1] "Gated DeltaNet GPU并行实现：拆解线性注意力循环的两种高效方案"
//        §3.2 chunked evaluation (dense products inside a chunk, serial state
//        carry between chunks); §3.3 chunk-wise mode (one workgroup walks all
//        chunks of its sequence); §4.3 give the heavy matmuls to most of the
//        waves and the serial state recurrence to few, with double-buffered
//        tiles so they overlap; §4.4 fp32 state, bf16 matmul operands with
//        fp32 accumulation.
//
// Chunk algebra (as in chunk_fwd.hpp): for a chunk with start state S,
//   g = log2-prefix of alpha, D_rs = 2^(g_r - g_s) (s <= r)
//   L = strictly-lower(diag(beta) (D o K K^T)),   Ti = (I + L)^-1
//   P = (D o Q K^T) on s <= r
//   U = Ti (diag(beta) V - diag(beta 2^g) K S^T)
//   O = diag(2^g) Q S^T + P U
//   S' = 2^(g_C) S + U^T diag(2^(g_C - g)) K
//
// Workgroup = 4 waves (one per SIMD), one (sequence, 32-row value slice) per
// workgroup, one barrier per period.  In period p:
//   wave 0 (state)   runs the S-dependent part of chunk p.  The fp32 state
//                    slice stays in MFMA accumulators for the whole sequence,
//                    and so do Z = K S^T, Y, U and O: an accumulator tile holds
//                    4 consecutive rows per lane, so two vertically adjacent
//                    tiles are a valid 32-deep MFMA operand once the k index is
//                    permuted as kappa(g, e) = e < 4 ? 4g + e : 16 + 4g + e - 4.
//                    The LDS operands it meets (Q, K, P, Ti) are stored with
//                    their columns in that same kappa order.
//   wave 1 (stage+P) writes chunk p+1 (K, Q, V^T, gate tables) into LDS from
//                    registers loaded one period earlier, issues the loads of
//                    chunk p+2, and builds P for chunk p+1.
//   wave 2 (inverse) builds Ti = (I + L)^-1 of chunk p+1 from L.
//   wave 3 (L)       builds L of chunk p+2 from keys it loaded one period
//                    earlier, then issues the loads of chunk p+3.
// Every buffer a wave writes in period p is read by another wave only after
// the barrier that ends period p, and no buffer is rewritten while another wave
// still reads it (double buffering by chunk parity).
//
// Cost model this code is written for (gfx950, measured): a wave64 VALU op
// occupies its SIMD for 4 cycles and a 16x16x32 bf16 MFMA for 16, so every
// role keeps its per-chunk VALU count small: LDS addresses are per-lane bases
// fixed before the chunk loop plus compile-time offsets, and global traffic
// goes through buffer instructions whose descriptors hold the sequence base in
// scalar registers.  Reads past the end of a sequence return zero and stores
// past it are dropped by the buffer range check, so the ragged last chunk
// needs no per-element predicates.
//
// LDS layout.  K and Q tiles are 64 rows x 128 columns (bf16) with the
// columns of each 32-column block in kappa order; the sixteen 16-byte octets
// of a row are XOR-swizzled by f(row) = ((row & 3) << 2) | ((row >> 2) & 3),
// which keeps both the 16-lane b128 fragment reads (16 consecutive rows, one
// octet) and the transposed 8-byte reads (4 consecutive rows x 4 chunks) free
// of bank conflicts.  P and Ti are 64 x 64 with kappa-ordered columns and
// octets swizzled by (row >> 1) & 7.
#pragma once

#include "gdn_common.hpp"

namespace gdn {
namespace pipe {

constexpr int C = 64;
constexpr int DK = 128;
constexpr int DVS = 32;
constexpr int LDT = 72;  // padded stride (elements) of 64-wide scratch rows
constexpr int LDD = 20;  // stride (floats) of the fp32 diagonal blocks of L

enum { G_BETA = 0, G_BEG = 1, G_EG = 2, G_EL = 3, G_LOG = 4, G_N = 5 };

struct __attribute__((aligned(16))) Smem {
  bf16_t K[2][C * DK];      // kappa-ordered, swizzled
  bf16_t Q[2][C * DK];
  bf16_t P[2][C * C];       // kappa-ordered columns, swizzled
  bf16_t Ti[2][C * C];
  bf16_t Vt[2][DVS * LDT];  // value slice transposed: [value col][token]
  float gate[2][G_N][C];
  float egl[2][4];          // 2^(g_C)
  bf16_t Lb[2][C * LDT];    // L row-major (operands of the blocked inverse)
  float Ld[2][4][16][LDD];  // fp32 diagonal 16x16 blocks of L
  bf16_t Trm[C * LDT];      // inverse being built, row-major
  bf16_t Tt[C * LDT];       // its transpose
  bf16_t Mt[32 * LDT];      // partial products of the blocked inverse
  float lg3[2][C];          // L wave: log2-prefix and beta of its chunk
};

__device__ __forceinline__ int swz_kq(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int swz_pt(int row) { return (row >> 1) & 7; }

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0), word 3 = 0x00020000 (gfx9 family untyped access)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float buf_ldf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void buf_st8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t lo, uint32_t hi) {
  const u32x2_t v = {lo, hi};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}

template <class T>
__device__ __forceinline__ T lds_at(const char* base, int off) {
  return *reinterpret_cast<const T*>(base + off);
}
template <class T>
__device__ __forceinline__ void lds_put(char* base, int off, T v) {
  *reinterpret_cast<T*>(base + off) = v;
}
__device__ __forceinline__ bf16x8_t as_op(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
// Two vertically adjacent accumulator tiles -> one kappa-ordered operand.
__device__ __forceinline__ bf16x8_t pack_op(const f32x4& lo, const f32x4& hi) {
  return as_op(make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]),
                          pack2(hi[2], hi[3])));
}
__device__ __forceinline__ f32x4 mfma(bf16x8_t a, bf16x8_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Order this wave's LDS writes before its later LDS reads (single-wave
// producer/consumer through LDS).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float wave_prefix_sum(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Byte offset of the b128 MFMA fragment (rows 0..15, 32-column block blk) of
// lane (lr, lg) in a kappa-ordered swizzled tile with `noct` octets per row;
// row block rb adds rb * 16 * noct * 16 bytes.
__device__ __forceinline__ int frag_base(int lr, int lg, int blk, int noct, int swz) {
  return lr * noct * 16 + (((4 * blk + lg) ^ swz) << 4);
}

// Per-sequence buffer descriptors.
struct Seq {
  __amdgpu_buffer_rsrc_t q, k, v, a, b, o;
  int64_t T;
};

// ============================================================ wave 0: state
struct StateAddr {
  int kq[4];   // fragment base per 32-column block
  int pt[2];   // P / Ti fragment base per 32-token block
  int tr[4];   // transposed-read supplier base per pair of key blocks
  int vt;      // V^T read base
  uint32_t o;  // lane part of the output byte offset
};

__device__ __forceinline__ StateAddr state_addr(int lane, int DV) {
  const int lr = lane & 15, lg = lane >> 4;
  StateAddr A;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) A.kq[pp] = frag_base(lr, lg, pp, 16, swz_kq(lr));
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) A.pt[pp] = frag_base(lr, lg, pp, 8, swz_pt(lr));
  const int sr = lr >> 2, sq = lane & 3;  // supplier token row / 4-column chunk
  const int t = 4 * lg + sr;              // supplier token of the first read
  const int sw = (sr << 2) | lg;          // = swz_kq(t + 16 m) for every m
#pragma unroll
  for (int h = 0; h < 4; ++h) A.tr[h] = t * 256 + (((4 * h + sq) ^ sw) << 4);
  A.vt = lr * (LDT * 2) + lg * 8;
  A.o = (uint32_t)((lr * DV + 4 * lg) * 2);
  return A;
}

__device__ __forceinline__ void state_chunk(Smem& sm, const Seq& sq, const StateAddr& A,
                                            f32x4 (&Sacc)[2][8], int64_t p, int DV, int lane) {
  const int buf = (int)(p & 1);
  const char* Kb = reinterpret_cast<const char*>(sm.K[buf]);
  const char* Qb = reinterpret_cast<const char*>(sm.Q[buf]);
  const char* Tb = reinterpret_cast<const char*>(sm.Ti[buf]);
  const char* Pb = reinterpret_cast<const char*>(sm.P[buf]);
  const char* Vb = reinterpret_cast<const char*>(sm.Vt[buf]);
  const float* gt = &sm.gate[buf][0][0];
  const int lr = lane & 15, lg = lane >> 4;

  // Operands of S for contractions over the key index.
  bf16x8_t Sop[2][4];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) Sop[ib][pp] = pack_op(Sacc[ib][2 * pp], Sacc[ib][2 * pp + 1]);
  // The decay of the carried state does not depend on this chunk's products.
  const float decay = sm.egl[buf][0];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) Sacc[ib][jb] *= decay;

  // O1 = S Q^T (tiles [ib][rb]) and Z = K S^T (tiles [rb][ib]).
  f32x4 Oacc[2][4], Z[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    bf16x8_t qf[4], kf[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      qf[pp] = as_op(lds_at<uint4>(Qb, A.kq[pp] + rb * 4096));
      kf[pp] = as_op(lds_at<uint4>(Kb, A.kq[pp] + rb * 4096));
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      f32x4 ao = zero4(), az = zero4();
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        ao = mfma(Sop[ib][pp], qf[pp], ao);
        az = mfma(kf[pp], Sop[ib][pp], az);
      }
      Oacc[ib][rb] = ao;
      Z[rb][ib] = az;
    }
  }
  // Y = beta V - beta 2^g Z, packed as kappa operands [ib][32-token block].
  bf16x8_t Yop[2][2];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib) {
    f32x4 y[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const float4 b4 = *reinterpret_cast<const float4*>(gt + G_BETA * C + 16 * rb + 4 * lg);
      const float4 g4 = *reinterpret_cast<const float4*>(gt + G_BEG * C + 16 * rb + 4 * lg);
      const uint2 vv = lds_at<uint2>(Vb, A.vt + ib * 16 * LDT * 2 + rb * 32);
      y[rb][0] = b4.x * __uint_as_float(vv.x << 16) - g4.x * Z[rb][ib][0];
      y[rb][1] = b4.y * __uint_as_float(vv.x & 0xffff0000u) - g4.y * Z[rb][ib][1];
      y[rb][2] = b4.z * __uint_as_float(vv.y << 16) - g4.z * Z[rb][ib][2];
      y[rb][3] = b4.w * __uint_as_float(vv.y & 0xffff0000u) - g4.w * Z[rb][ib][3];
    }
    Yop[ib][0] = pack_op(y[0], y[1]);
    Yop[ib][1] = pack_op(y[2], y[3]);
  }
  // O1 carries the factor 2^g of its token column.
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const float eg = gt[G_EG * C + 16 * rb + lr];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) Oacc[ib][rb] *= eg;
  }
  // U = Ti Y (tiles [rb][ib]); Ti is lower triangular, so row block rb only
  // needs the 32-token blocks pp <= rb/2 (the upper blocks inside them are zero).
  f32x4 U[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    bf16x8_t tf[2];
#pragma unroll
    for (int pp = 0; pp <= rb / 2; ++pp) tf[pp] = as_op(lds_at<uint4>(Tb, A.pt[pp] + rb * 2048));
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      f32x4 acc = zero4();
#pragma unroll
      for (int pp = 0; pp <= rb / 2; ++pp) acc = mfma(tf[pp], Yop[ib][pp], acc);
      U[rb][ib] = acc;
    }
  }
  // Operands of U: plain (for O) and scaled by 2^(g_C - g_s) (for S).
  bf16x8_t Uop[2][2], Uh[2][2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const float4 e0 = *reinterpret_cast<const float4*>(gt + G_EL * C + 32 * pp + 4 * lg);
    const float4 e1 = *reinterpret_cast<const float4*>(gt + G_EL * C + 32 * pp + 16 + 4 * lg);
    const f32x4 s0 = {e0.x, e0.y, e0.z, e0.w}, s1 = {e1.x, e1.y, e1.z, e1.w};
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      Uop[ib][pp] = pack_op(U[2 * pp][ib], U[2 * pp + 1][ib]);
      Uh[ib][pp] = pack_op(U[2 * pp][ib] * s0, U[2 * pp + 1][ib] * s1);
    }
  }
  // O^T += U^T P^T, then store this chunk's outputs (the range check of the
  // output descriptor drops rows past the end of the sequence).
  const uint32_t obase = (uint32_t)(p * C * DV * 2) + A.o;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    bf16x8_t pf[2];
#pragma unroll
    for (int pp = 0; pp <= rb / 2; ++pp) pf[pp] = as_op(lds_at<uint4>(Pb, A.pt[pp] + rb * 2048));
    const uint32_t orow = obase + (uint32_t)(rb * 16 * DV * 2);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      f32x4 acc = Oacc[ib][rb];
#pragma unroll
      for (int pp = 0; pp <= rb / 2; ++pp) acc = mfma(Uop[ib][pp], pf[pp], acc);
      buf_st8(sq.o, orow + ib * 32, pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
    }
  }
  // S^T += K^T Uh, with K^T fragments from transposed LDS reads: within each
  // 16-lane group, lane (4*r + q) supplies the address of 4 columns (chunk q)
  // of token row r, and lane m receives column m of the four rows, i.e. 4
  // consecutive tokens of one key column.
  typedef __attribute__((address_space(3))) i16x4_t lds_v4;
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) {
    bf16x8_t kt[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int off = A.tr[jb >> 1] + (jb & 1) * 8 + pp * 32 * 256;
      const i16x4_t a4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(Kb + off));
      const i16x4_t b4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(Kb + off + 16 * 256));
      const uint2 ua = __builtin_bit_cast(uint2, a4), ub = __builtin_bit_cast(uint2, b4);
      kt[pp] = as_op(make_uint4(ua.x, ua.y, ub.x, ub.y));
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      f32x4 acc = Sacc[ib][jb];
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) acc = mfma(kt[pp], Uh[ib][pp], acc);
      Sacc[ib][jb] = acc;
    }
  }
}

// ============================================================ wave 1: stage + P
// Register image of one chunk: k/q[it] = 8 columns (8*(lane%16) ..) of token
// 4*it + lane/16; v[it] = 8 slice columns (8*(lane%4) ..) of token 16*it + lane/4.
struct ChunkRegs {
  uint4 k[16];
  uint4 q[16];
  uint4 v[4];
  float a, b;  // alpha, beta of token `lane`
};

struct StageAddr {
  uint32_t gkq;   // global byte offset (lane part) of k/q[0]
  uint32_t gv;    // global byte offset (lane part) of v[0]
  int wkq[4][2];  // LDS write offsets of the two 4-column halves, per (it & 3)
  int wvt;        // V^T write base
  int kq[4];      // fragment bases (as the state wave)
  int pw[2];      // P write base per 32-token block of s
};

__device__ __forceinline__ StageAddr stage_addr(int lane, int DV) {
  const int lr = lane & 15, lg = lane >> 4;
  StageAddr A;
  A.gkq = (uint32_t)(lg * DK * 2 + lr * 16);
  A.gv = (uint32_t)((lane >> 2) * DV * 2 + (lane & 3) * 16);
  // columns 8*lr .. +7 of a row: 32-column block lr/4, 4-column groups
  // 2*(lr&1) and 2*(lr&1)+1, in the upper kappa half when (lr>>1)&1
  const int blk = lr >> 2, q0 = 2 * (lr & 1), half = (lr >> 1) & 1;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int sw = (lg << 2) | m;  // swz_kq(4*it + lg) when it & 3 == m
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      A.wkq[m][hh] = lg * 256 + (((4 * blk + q0 + hh) ^ sw) << 4) + half * 8;
  }
  A.wvt = (lane & 3) * 8 * (LDT * 2) + (lane >> 2) * 2;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) A.kq[pp] = frag_base(lr, lg, pp, 16, swz_kq(lr));
#pragma unroll
  for (int h = 0; h < 2; ++h) A.pw[h] = lr * 128 + (((4 * h + lg) ^ swz_pt(lr)) << 4);
  return A;
}

__device__ __forceinline__ void load_chunk(ChunkRegs& R, const Seq& sq, const StageAddr& A,
                                           int64_t c, int DV, int lane) {
  const uint32_t kq0 = (uint32_t)(c * C * DK * 2) + A.gkq;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    R.k[it] = buf_ld16(sq.k, kq0 + it * 4 * DK * 2);
    R.q[it] = buf_ld16(sq.q, kq0 + it * 4 * DK * 2);
  }
  const uint32_t v0 = (uint32_t)(c * C * DV * 2) + A.gv;
#pragma unroll
  for (int it = 0; it < 4; ++it) R.v[it] = buf_ld16(sq.v, v0 + it * 16 * DV * 2);
  const int64_t t = c * C + lane;
  const float a = buf_ldf(sq.a, (uint32_t)(t * 4));
  const float b = buf_ldf(sq.b, (uint32_t)(t * 4));
  R.a = t < sq.T ? a : 1.f;  // tokens past the end: identity maps
  R.b = t < sq.T ? b : 0.f;
}

__device__ __forceinline__ void stage_chunk(Smem& sm, const ChunkRegs& R, const StageAddr& A,
                                            int64_t c, int lane) {
  const int buf = (int)(c & 1);
  char* Kb = reinterpret_cast<char*>(sm.K[buf]);
  char* Qb = reinterpret_cast<char*>(sm.Q[buf]);
  char* Vb = reinterpret_cast<char*>(sm.Vt[buf]);
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int o0 = A.wkq[it & 3][0] + it * 4 * 256;
    const int o1 = A.wkq[it & 3][1] + it * 4 * 256;
    lds_put<uint2>(Kb, o0, make_uint2(R.k[it].x, R.k[it].y));
    lds_put<uint2>(Kb, o1, make_uint2(R.k[it].z, R.k[it].w));
    lds_put<uint2>(Qb, o0, make_uint2(R.q[it].x, R.q[it].y));
    lds_put<uint2>(Qb, o1, make_uint2(R.q[it].z, R.q[it].w));
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const uint32_t w[4] = {R.v[it].x, R.v[it].y, R.v[it].z, R.v[it].w};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      lds_put<bf16_t>(Vb, A.wvt + (2 * x) * LDT * 2 + it * 32, (bf16_t)(w[x] & 0xffffu));
      lds_put<bf16_t>(Vb, A.wvt + (2 * x + 1) * LDT * 2 + it * 32, (bf16_t)(w[x] >> 16));
    }
  }
  // gate tables, one lane per token
  const float gs = wave_prefix_sum(fast_log2(R.a), lane);
  const float glast = __shfl(gs, 63, 64);
  const float eg = fast_exp2(gs);
  float* gt = &sm.gate[buf][0][0];
  gt[G_BETA * C + lane] = R.b;
  gt[G_BEG * C + lane] = R.b * eg;
  gt[G_EG * C + lane] = eg;
  gt[G_EL * C + lane] = fast_exp2(glast - gs);
  gt[G_LOG * C + lane] = gs;
  if (lane == 0) sm.egl[buf][0] = fast_exp2(glast);
}

// P of chunk c from the staged buffers c & 1 (after a wave fence).
__device__ __forceinline__ void build_p(Smem& sm, const StageAddr& A, int64_t c, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int buf = (int)(c & 1);
  const char* Kb = reinterpret_cast<const char*>(sm.K[buf]);
  const char* Qb = reinterpret_cast<const char*>(sm.Q[buf]);
  const float* gt = &sm.gate[buf][0][0];
  char* Pb = reinterpret_cast<char*>(sm.P[buf]);
  bf16x8_t kf[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) kf[b][pp] = as_op(lds_at<uint4>(Kb, A.kq[pp] + b * 4096));
  // tiles [s-block sb][r-block rb], sb <= rb: element (s, r) = k_s . q_r
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    bf16x8_t qf[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) qf[pp] = as_op(lds_at<uint4>(Qb, A.kq[pp] + rb * 4096));
    const float gr = gt[G_LOG * C + 16 * rb + lr];
#pragma unroll
    for (int sb = 0; sb <= rb; ++sb) {
      f32x4 acc = zero4();
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) acc = mfma(kf[sb][pp], qf[pp], acc);
      const float4 g4 = *reinterpret_cast<const float4*>(gt + G_LOG * C + 16 * sb + 4 * lg);
      float val[4] = {fast_exp2(gr - g4.x) * acc[0], fast_exp2(gr - g4.y) * acc[1],
                      fast_exp2(gr - g4.z) * acc[2], fast_exp2(gr - g4.w) * acc[3]};
      if (sb == rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (4 * lg + e <= lr) ? val[e] : 0.f;
      }
      lds_put<uint2>(Pb, A.pw[sb >> 1] + (sb & 1) * 8 + rb * 2048,
                     make_uint2(pack2(val[0], val[1]), pack2(val[2], val[3])));
    }
  }
}

// ============================================================ wave 2: inverse
// Ti = (I + L)^-1 of chunk c from L buffers c & 1 into Ti buffer c & 1.
__device__ __forceinline__ void build_inverse(Smem& sm, int64_t c, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int lb = (int)(c & 1);
  // level 0: unit-lower 16x16 diagonal blocks by forward substitution, fp32,
  // lane = (block lg, column lr); column-oriented so the row updates of one
  // step are independent.
  {
    const float* Lblk = &sm.Ld[lb][lg][0][0];
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == lr) ? 1.f : 0.f;
#pragma unroll
    for (int s = 0; s < 15; ++s) {
#pragma unroll
      for (int r = s + 1; r < 16; ++r) x[r] -= Lblk[r * LDD + s] * x[s];
    }
    bf16_t* trm = &sm.Trm[(16 * lg) * LDT + 16 * lg + lr];
#pragma unroll
    for (int r = 0; r < 16; ++r) trm[r * LDT] = f32_to_bf16(x[r]);
    uint4* tt = reinterpret_cast<uint4*>(&sm.Tt[(16 * lg + lr) * LDT + 16 * lg]);
    tt[0] = make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7]));
    tt[1] = make_uint4(pack2(x[8], x[9]), pack2(x[10], x[11]), pack2(x[12], x[13]), pack2(x[14], x[15]));
  }
  wave_lds_fence();
  // level 1: T[a][b] = -T[a][a] L[a][b] T[b][b], (a,b) = (1,0), (3,2)
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const int a = 2 * pr + 1, b = 2 * pr;
    f32x4 acc = Mma<bf16_t>::template run<16>(zero4(), &sm.Lb[lb][16 * a * LDT + 16 * b], LDT,
                                              &sm.Tt[16 * b * LDT + 16 * b], LDT, lane);
    store4<bf16_t>(&sm.Mt[(16 * pr + lr) * LDT + 4 * lg], acc[0], acc[1], acc[2], acc[3]);
  }
  wave_lds_fence();
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const int a = 2 * pr + 1, b = 2 * pr;
    f32x4 acc = Mma<bf16_t>::template run<16>(zero4(), &sm.Trm[16 * a * LDT + 16 * a], LDT,
                                              &sm.Mt[16 * pr * LDT], LDT, lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.Trm[(16 * a + 4 * lg + e) * LDT + 16 * b + lr] = f32_to_bf16(-acc[e]);
    store4<bf16_t>(&sm.Tt[(16 * b + lr) * LDT + 16 * a + 4 * lg], -acc[0], -acc[1], -acc[2], -acc[3]);
  }
  wave_lds_fence();
  // level 2: T[hi][lo] = -T[hi][hi] L[hi][lo] T[lo][lo] on 32x32 halves
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int rb2 = u >> 1, cb2 = u & 1;
    f32x4 acc = Mma<bf16_t>::template run<32>(zero4(), &sm.Lb[lb][(32 + 16 * rb2) * LDT], LDT,
                                              &sm.Tt[16 * cb2 * LDT], LDT, lane);
    store4<bf16_t>(&sm.Mt[(16 * cb2 + lr) * LDT + 16 * rb2 + 4 * lg], acc[0], acc[1], acc[2], acc[3]);
  }
  wave_lds_fence();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int rb2 = u >> 1, cb2 = u & 1;
    f32x4 acc = Mma<bf16_t>::template run<32>(zero4(), &sm.Trm[(32 + 16 * rb2) * LDT + 32], LDT,
                                              &sm.Mt[16 * cb2 * LDT], LDT, lane);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sm.Trm[(32 + 16 * rb2 + 4 * lg + e) * LDT + 16 * cb2 + lr] = f32_to_bf16(-acc[e]);
  }
  wave_lds_fence();
  // copy the ten lower 16x16 blocks into the kappa-ordered, swizzled Ti buffer
  char* Tb = reinterpret_cast<char*>(sm.Ti[lb]);
  const char* Rb = reinterpret_cast<const char*>(sm.Trm);
  const int rd = lr * LDT * 2 + lg * 8;
  int wr[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) wr[h] = lr * 128 + (((4 * h + lg) ^ swz_pt(lr)) << 4);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b <= a; ++b) {
      const uint2 val = lds_at<uint2>(Rb, rd + a * 16 * LDT * 2 + b * 32);
      lds_put<uint2>(Tb, wr[b >> 1] + (b & 1) * 8 + a * 2048, val);
    }
}

// ============================================================ wave 3: L
// Keys of one chunk in MFMA fragment layout: kf[rb][pp] = columns
// 32pp + 8*(lane/16) .. +7 of token 16rb + lane%16.
struct FragRegs {
  uint4 kf[4][4];
  float a, b;  // alpha, beta of token `lane`
};

__device__ __forceinline__ void load_frags(FragRegs& R, const Seq& sq, int64_t c, int lane) {
  const uint32_t base =
      (uint32_t)(c * C * DK * 2) + (uint32_t)((lane & 15) * DK * 2 + (lane >> 4) * 16);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) R.kf[rb][pp] = buf_ld16(sq.k, base + rb * 16 * DK * 2 + pp * 64);
  const int64_t t = c * C + lane;
  const float a = buf_ldf(sq.a, (uint32_t)(t * 4));
  const float b = buf_ldf(sq.b, (uint32_t)(t * 4));
  R.a = t < sq.T ? a : 1.f;
  R.b = t < sq.T ? b : 0.f;
}

__device__ __forceinline__ void build_l(Smem& sm, const FragRegs& R, int64_t c, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int lb = (int)(c & 1);
  const float gs = wave_prefix_sum(fast_log2(R.a), lane);
  sm.lg3[0][lane] = gs;
  sm.lg3[1][lane] = R.b;
  wave_lds_fence();
  // tiles [s-block sb][r-block rb], sb <= rb: element (s, r) = k_s . k_r
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int r = 16 * rb + lr;
    const float gr = sm.lg3[0][r];
    const float br = sm.lg3[1][r];
#pragma unroll
    for (int sb = 0; sb <= rb; ++sb) {
      f32x4 acc = zero4();
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) acc = mfma(as_op(R.kf[sb][pp]), as_op(R.kf[rb][pp]), acc);
      const float4 g4 = *reinterpret_cast<const float4*>(&sm.lg3[0][16 * sb + 4 * lg]);
      float val[4] = {br * fast_exp2(gr - g4.x) * acc[0], br * fast_exp2(gr - g4.y) * acc[1],
                      br * fast_exp2(gr - g4.z) * acc[2], br * fast_exp2(gr - g4.w) * acc[3]};
      if (sb == rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (4 * lg + e < lr) ? val[e] : 0.f;
        *reinterpret_cast<float4*>(&sm.Ld[lb][rb][lr][4 * lg]) = make_float4(val[0], val[1], val[2], val[3]);
      }
      store4<bf16_t>(&sm.Lb[lb][r * LDT + 16 * sb + 4 * lg], val[0], val[1], val[2], val[3]);
    }
  }
}

// ============================================================ kernel
__global__ __launch_bounds__(256) void chunk_fwd_pipe_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* initial_state, bf16_t* __restrict__ o, float* final_state, int nchain,
    int64_t Tlen, int DV, int xcd_map) {
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int lg = lane >> 4;

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

  Seq sq;
  sq.T = Tlen;
  {
    const uint32_t kq_bytes = (uint32_t)(Tlen * DK * 2);
    sq.q = make_rsrc(q + (int64_t)chain * Tlen * DK, kq_bytes);
    sq.k = make_rsrc(k + (int64_t)chain * Tlen * DK, kq_bytes);
    // value / output slice: the descriptor range ends with the sequence
    const int64_t vs = (int64_t)chain * Tlen * DV + slice * DVS;
    const uint32_t v_bytes = (uint32_t)((Tlen * DV - slice * DVS) * 2);
    sq.v = make_rsrc(v + vs, v_bytes);
    sq.o = make_rsrc(o + vs, v_bytes);
    sq.a = make_rsrc(alpha + (int64_t)chain * Tlen, (uint32_t)(Tlen * 4));
    sq.b = make_rsrc(beta + (int64_t)chain * Tlen, (uint32_t)(Tlen * 4));
  }
  const int64_t nch = (Tlen + C - 1) / C;
  const int64_t st_off = ((int64_t)chain * DV + (int64_t)slice * DVS) * DK;

  // Zero the triangular buffers: their strictly-upper blocks are never
  // written but are read as zero by 32-deep products.
  {
    uint32_t* z = reinterpret_cast<uint32_t*>(&sm.P[0][0]);
    for (int e = tid; e < 2 * 2 * C * C / 2; e += 256) z[e] = 0u;  // P and Ti
    uint32_t* z2 = reinterpret_cast<uint32_t*>(&sm.Trm[0]);
    for (int e = tid; e < 2 * C * LDT / 2; e += 256) z2[e] = 0u;  // Trm and Tt
  }

  // Each role runs its own loop over periods p = -2 .. nch-1 with exactly one
  // workgroup barrier per period, so all four waves meet at every barrier.
  if (wave == 0) {
    const StateAddr A = state_addr(lane, DV);
    f32x4 Sacc[2][8];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        Sacc[ib][jb] = zero4();
        if (initial_state) {
          const int i = 16 * ib + lr, j = 16 * jb + 4 * lg;
          const float4 s4 = *reinterpret_cast<const float4*>(initial_state + st_off + (int64_t)i * DK + j);
          Sacc[ib][jb] = f32x4{s4.x, s4.y, s4.z, s4.w};
        }
      }
    __syncthreads();
    for (int64_t p = -2; p < nch; ++p) {
      if (p >= 0) state_chunk(sm, sq, A, Sacc, p, DV, lane);
      __syncthreads();
    }
    if (final_state) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
          const int i = 16 * ib + lr, j = 16 * jb + 4 * lg;
          *reinterpret_cast<float4*>(final_state + st_off + (int64_t)i * DK + j) =
              make_float4(Sacc[ib][jb][0], Sacc[ib][jb][1], Sacc[ib][jb][2], Sacc[ib][jb][3]);
        }
    }
  } else if (wave == 1) {
    const StageAddr A = stage_addr(lane, DV);
    ChunkRegs R;
    __syncthreads();
    for (int64_t p = -2; p < nch; ++p) {
      const int64_t c1 = p + 1, c2 = p + 2;
      const bool have1 = c1 >= 0 && c1 < nch;
      if (have1) stage_chunk(sm, R, A, c1, lane);
      if (c2 < nch) load_chunk(R, sq, A, c2, DV, lane);
      if (have1) {
        wave_lds_fence();
        build_p(sm, A, c1, lane);
      }
      __syncthreads();
    }
  } else if (wave == 2) {
    __syncthreads();
    for (int64_t p = -2; p < nch; ++p) {
      const int64_t c1 = p + 1;
      if (c1 >= 0 && c1 < nch) build_inverse(sm, c1, lane);
      __syncthreads();
    }
  } else {
    FragRegs R;
    if (nch > 0) load_frags(R, sq, 0, lane);
    __syncthreads();
    for (int64_t p = -2; p < nch; ++p) {
      const int64_t c2 = p + 2, c3 = p + 3;
      if (c2 < nch) build_l(sm, R, c2, lane);
      if (c3 < nch) load_frags(R, sq, c3, lane);
      __syncthreads();
    }
  }
}

}  // namespace pipe
}  // namespace gdn
