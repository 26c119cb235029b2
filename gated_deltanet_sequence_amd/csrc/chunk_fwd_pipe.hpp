// Pipelined chunked forward pass of the gated delta rule for bf16 inputs,
// d_k = d_v = 128 or 64, 64-token chunks, on gfx950.  The LDS layout always
// holds 128 keys; with d = 64 the keys 64..127 are zero in LDS (their loads
// read past the buffer range, which returns zero) and in the state, and the
// instance with KB = 2 key blocks skips the products over them.
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
// Chunk algebra (derived by unrolling the per-token update inside a chunk;
// [P1] §2.1-2.3): for a chunk with start state S,
//   g = log2-prefix of alpha, D_rs = 2^(g_r - g_s) (s <= r)
//   L = strictly-lower(diag(beta) (D o K K^T)),   Ti = (I + L)^-1
//   P = (D o Q K^T) on s <= r
//   U = Ti (diag(beta) V - diag(beta 2^g) K S^T)
//   O = diag(2^g) Q S^T + P U
//   S' = 2^(g_C) S + U^T diag(2^(g_C - g)) K
//
// Workgroup = 8 wave slots (7 working waves), one (sequence, 32-row value
// slice) per workgroup, one workgroup barrier per period.  Waves 0..3 run on
// four different SIMDs and wave w + 4 shares the SIMD of wave w: the state
// waves share their SIMDs only with the prefetch wave and the empty slot, the
// P wave shares with the loader, and the L wave with the inverse.  In period p:
//   waves 0, 1 (state)  each own 16 rows of the value slice.  They finish the
//                       output of chunk p-1 (O += P U) and run the S-dependent
//                       part of chunk p.  The fp32 state stays in MFMA
//                       accumulators for the whole sequence.
//   wave 2 (P)          builds P of chunk p.
//   wave 3 (L)          builds L of chunk p+2 from its keys in LDS; it issues
//                       no global loads.  (Without the delta rule it moves Q
//                       instead, see the kernel.)
//   wave 4 (prefetch)   touches the cache lines of chunk p+3 (the key lines
//                       of chunk p+5) so that later loads hit L2, and never
//                       waits for those loads.
//   wave 6 (loader)     moves V and Q of chunk p+1 and K of chunk p+3 into
//                       LDS with LDS-DMA loads, builds the gate tables of
//                       chunk p+3 from gates it loaded one period earlier and
//                       loads the gates of chunk p+4.
//   wave 7 (inverse)    builds Ti = (I + L)^-1 of chunk p+1.
// Every buffer written in period p is read by another wave only after the
// barrier that ends period p, and none is rewritten while another wave still
// reads it (double buffering by chunk parity).
//
// Operand layouts.  An MFMA accumulator tile gives each lane 4 consecutive
// rows of one column; two vertically adjacent tiles form one 32-deep operand
// whose k index runs kappa(g, e) = e < 4 ? 4g + e : 16 + 4g + e - 4 over the
// lane's eight values.  The key index of the state is relabelled so that this
// kappa order is the natural column order of q and k: internal key
// 32b + 16h + 4a + e is global key 32b + 8a + 4h + e.  Hence K and Q sit in
// LDS in their global layout (rows of 256 bytes, 16-byte octets XOR-swizzled
// per row) and the relabelling only touches the addresses of the initial and
// final state.  Token-indexed operands (P, Ti) keep kappa order where an
// accumulator meets them.  Transposed operands (K^T, V^T, Ti) come from the
// gfx950 transposed LDS read.
#pragma once

#include "gdn_common.hpp"
#include <type_traits>

namespace gdn {
namespace pipe {

constexpr int C = 64;
constexpr int DK = 128;
constexpr int DVS = 32;   // value columns per workgroup
// Wave slots and roles.  Waves 0..3 run on four different SIMDs and wave
// w + 4 shares the SIMD of wave w; slot 5 is left empty (that wave exits at
// once), so the second state wave has a SIMD of its own.
constexpr int NWAVES = 8;
constexpr int W_P = 2, W_L = 3, W_PREFETCH = 4, W_IDLE = 5, W_LOADER = 6, W_INV = 7;
// Without the delta rule the P wave builds the first PSPLIT tiles of P and
// the idle inverse slot (SIMD 3) the rest (2.4 % faster than all ten on the
// P wave, which shares SIMD 2 with the loader).
constexpr int PSPLIT = 5;
constexpr int TTS = 72;   // row stride (elements) of Ti^T
constexpr int LDR = 20;   // row stride (floats) of the fp32 diagonal blocks of L

enum { G_BETA = 0, G_ER = 1, G_EG = 2, G_EL = 3, G_LOG = 4, G_N = 5 };

// How far ahead K and Q are fetched without the delta rule (GLA): the period
// is then short enough that the loader's DMA round trip becomes the critical
// path, so K, Q are loaded two chunks ahead and each load has two periods to
// land (measured 9 % faster than one chunk ahead).  The otherwise idle L wave
// moves Q there, so that the loader's own loads per period shrink (one wave
// moves only so many bytes per clock; 2.4 % faster).  With the delta
// rule, Q is loaded one chunk ahead and K three (see k_buf below).
template <bool GLA> constexpr int KQ_AHEAD = GLA ? 2 : 1;

// The prefetch wave touches every 128-byte line of chunk
// p + PREFETCH_AHEAD + KQ_AHEAD - 1 in period p, so that the loads of the
// later periods find their lines in L2.  Two periods before the loader's DMA
// of that chunk is the measured optimum: at four or more periods, lines are
// evicted before use and HBM traffic rises above the algorithmic bytes
// (1.34x at five); at one the lines arrive too late for the DMA and the
// kernel is 40 % slower; three is as fast as two.  With the delta rule the
// key lines of chunk p+5 are touched instead, two periods before their DMA.
constexpr int PREFETCH_AHEAD = 3;

// Targets of LDS-DMA loads are arrays of their own: the compiler then sees
// that the LDS reads which follow such a load in the same wave touch other
// objects, and does not wait for the load before them.
// GLA: K and Q of chunk c in lds_K[c % 3], lds_Q[c % 3] (two chunks ahead).
// Delta rule: K of chunk c in lds_K4[c % 4], loaded three chunks ahead, so
// that the L wave reads its keys of chunk c from LDS two periods before the
// chunk instead of loading them from global memory (loads of one wave that
// miss L2 hold up the later loads of the whole CU: the L wave's own key loads
// cost about 5 % of the period); Q of chunk c in lds_Q2[c % 2], one chunk
// ahead.  V of chunk c in lds_V[c % 2], one chunk ahead.  Rows [token][key]
// with octets swizzled by swz_kq(token).
__shared__ __attribute__((aligned(16))) bf16_t lds_K[3][C * DK];
__shared__ __attribute__((aligned(16))) bf16_t lds_Q[3][C * DK];
__shared__ __attribute__((aligned(16))) bf16_t lds_K4[4][C * DK];
__shared__ __attribute__((aligned(16))) bf16_t lds_Q2[2][C * DK];
template <bool GLA>
__device__ __forceinline__ bf16_t* k_buf(int64_t c) {
  if constexpr (GLA) return lds_K[c % 3];
  else return lds_K4[c & 3];
}
template <bool GLA>
__device__ __forceinline__ bf16_t* q_buf(int64_t c) {
  if constexpr (GLA) return lds_Q[c % 3];
  else return lds_Q2[c & 1];
}
__shared__ __attribute__((aligned(16))) bf16_t lds_V[2][C * DVS];  // [token][slice column]
__shared__ __attribute__((aligned(16))) uint32_t lds_touch[64];    // landing area of the L2 prefetch (never read)
__shared__ __attribute__((aligned(16))) float lds_gst[2][C];        // alpha, beta of the next chunk, landed by LDS-DMA

struct __attribute__((aligned(16))) Smem {
  bf16_t P[2][C * C];       // [r][s], s kappa-ordered, octets swizzled by swz_p(r)
  bf16_t Tt[2][C * TTS];    // Ti^T: [s][t]
  float gate[4][G_N][C];    // written three periods before the last use: four buffers
  float egl[4][4];          // 2^(g_C), and 1 where the decay factors of P and L may be split
  float Ld[2][4][16 * LDR + 4];  // strictly-lower diagonal 16x16 blocks of L, fp32
                                // (blocks padded by 16 bytes: the inverse reads
                                // the four blocks at once without bank conflicts)
  bf16_t Lo[2][6][64 * 4];  // off-diagonal 16x16 blocks of L, MFMA A-operand order
};

// The decay 2^(g_r - g_s) of P and L is split into 2^(g_r - g_C) 2^(g_C - g_s)
// when g_C >= SPLIT_MIN; whether it is, is uniform over the wave.
constexpr float SPLIT_MIN = -120.f;
__device__ __forceinline__ bool split_decay(const Smem& sm, int64_t c) {
  return __builtin_amdgcn_readfirstlane(__float_as_int(sm.egl[c & 3][1])) != 0;
}

// XOR applied to the 16-byte octet index of K/Q row `row`.  LDS bank rules on
// gfx950 (64 banks of 4 bytes): a 16-byte read serves 16 lanes per cycle,
// taken from one half-wave by the bit parity of (lane / 4) mod 8; an 8-byte
// or transposed read serves a half-wave per cycle.  With this XOR the
// fragment reads (16 consecutive rows, one octet) are conflict-free and the
// transposed reads of the state update (4 rows x 4 octets per 16 lanes, one
// 8-byte half) reach the 2-way minimum that a fixed half allows.
__device__ __forceinline__ int swz_kq(int row) { return ((row & 3) << 2) | (3 * ((row >> 3) & 1)); }
__device__ __forceinline__ int swz_p(int row) { return (row >> 1) & 7; }

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0), word 3 = 0x00020000 (gfx9 family untyped access)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// voff: per-lane byte offset; soff: wave-uniform byte offset (scalar register)
__device__ __forceinline__ uint4 buf_ld16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
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
// gfx950 transposed read: within each 16-lane group, lane m receives element
// m % 4 of the 8-byte rows whose addresses lanes m/4, m/4 + 4, m/4 + 8 and
// m/4 + 12 supply.
__device__ __forceinline__ uint2 lds_tr(const char* base, int off) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
  return __builtin_bit_cast(uint2, v);
}
// LDS pointer of one lane: buffer start plus a per-lane offset, computed once
// per period.  The empty asm hides the sum from the optimiser, which would
// otherwise fold the per-read constants into per-read address registers;
// this way every read adds its constant in the instruction's offset field.
typedef const __attribute__((address_space(3))) char* lptr;
__device__ __forceinline__ lptr lane_base(const void* buf, int lane_off) {
  uint32_t a = (uint32_t)(uintptr_t)(lptr)buf + (uint32_t)lane_off;
  asm volatile("" : "+v"(a));
  return (lptr)(uintptr_t)a;
}
template <class T> struct Ld3;
template <> struct Ld3<uint4> {
  static __device__ __forceinline__ uint4 get(lptr p) {
    const u32x4_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
};
template <> struct Ld3<uint2> {
  static __device__ __forceinline__ uint2 get(lptr p) {
    const u32x2_t v = *reinterpret_cast<const __attribute__((address_space(3))) u32x2_t*>(p);
    return make_uint2(v.x, v.y);
  }
};
template <class T>
__device__ __forceinline__ T ld3(lptr base, int off) { return Ld3<T>::get(base + off); }
__device__ __forceinline__ uint2 tr3(lptr base, int off) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
  return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ bf16x8_t as_op(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_op(uint2 lo, uint2 hi) {
  return as_op(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
__device__ __forceinline__ i16x4_t as_op4(uint2 u) { return __builtin_bit_cast(i16x4_t, u); }

__device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
// One accumulator tile -> 16-deep operand (4 values per lane).
__device__ __forceinline__ uint2 pack_tile(const f32x4& t) {
  return make_uint2(pack2(t[0], t[1]), pack2(t[2], t[3]));
}
// Two vertically adjacent accumulator tiles -> one kappa-ordered operand.
__device__ __forceinline__ bf16x8_t pack_op(const f32x4& lo, const f32x4& hi) {
  return as_op(pack_tile(lo), pack_tile(hi));
}
__device__ __forceinline__ f32x4 mfma(bf16x8_t a, bf16x8_t b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_op4(a), as_op4(b), c, 0, 0, 0);
}
__device__ __forceinline__ float4 as_f4(f32x4 v) { return make_float4(v[0], v[1], v[2], v[3]); }
// Order this wave's LDS writes before its later LDS reads (single-wave
// producer/consumer through LDS).  The LDS unit executes the instructions of
// one wave in issue order, and the compiler keeps a read after a write to the
// same array, so draining the LDS counter is enough.  (A memory-model fence
// here would also wait for the wave's outstanding LDS-DMA loads.)
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier that orders LDS only.  A full __syncthreads() also waits
// for every outstanding global load and store of the wave (vmcnt(0)), which
// would drain the loads that are meant to stay in flight across periods.
// Data that crosses a barrier here lives in LDS; LDS-DMA loads are waited for
// explicitly by the wave that issues them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier for the wave that keeps LDS-DMA prefetch loads in flight across
// periods: an LDS-scope release fence would wait for those loads too (they
// write LDS), so this drains only the LDS counter (the wave's own LDS writes
// are complete) and stops the compiler from moving memory operations across.
__device__ __forceinline__ void lds_barrier_keep_dma() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round trips):
// row_shr 1, 2, 4, 8 scan each row of 16 lanes; row_bcast15 and row_bcast31
// then add the totals of the preceding rows.  Lanes without a source take 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_src(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x += dpp_src<0x111, 0xf>(x);  // row_shr:1
  x += dpp_src<0x112, 0xf>(x);  // row_shr:2
  x += dpp_src<0x114, 0xf>(x);  // row_shr:4
  x += dpp_src<0x118, 0xf>(x);  // row_shr:8
  x += dpp_src<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_src<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ float lane63(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Per-sequence buffer descriptors.
struct Seq {
  __amdgpu_buffer_rsrc_t q, k, v, a, b, o;
  int64_t T;
  int dk;  // key width of q, k and the state in global memory: 128, or 64
           // (then keys 64..127 are zero in LDS and in the state)
};

// Global key column of the first of the 4 state values a lane holds in
// accumulator tile jb (the relabelling described at the top of the file).
__device__ __forceinline__ int state_col(int jb, int lg) {
  return 32 * (jb >> 1) + 8 * lg + 4 * (jb & 1);
}

// ============================================================ waves 0, 1: state
struct StateAddr {
  int frag[4];  // K/Q fragment (token row lr, octet 4pp + lg) per key block pp
  int ktr[4];   // K^T supplier address per key block
  int vtr;      // V^T supplier address
  int ttr;      // Ti supplier address (rows of Ti^T)
  int pfr[2];   // P fragment per 32-token block
  uint32_t o;   // lane part of the output byte offset
};

__device__ __forceinline__ StateAddr state_addr(int lane, int X, int DV) {
  const int lr = lane & 15, lg = lane >> 4;
  const int a = lr & 3, r = lr >> 2;  // as a supplier of transposed reads
  StateAddr A;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    A.frag[pp] = lr * 256 + (((4 * pp + lg) ^ swz_kq(lr)) << 4);
    // token 4 lg + r (+ 32-token and 16-token offsets added per read), whose
    // swizzle is swz_kq(4 lg + r); key octet 4 pp + a
    A.ktr[pp] = (4 * lg + r) * 256 + (((4 * pp + a) ^ swz_kq(4 * lg + r)) << 4);
  }
  // value rows of 64 bytes; the 16-byte slot index is XORed with 2 on rows
  // with bit 2 set, which makes these transposed reads conflict-free
  A.vtr = (4 * lg + r) * (DVS * 2) + (((2 * X + (a >> 1)) ^ (2 * (lg & 1))) << 4) + 8 * (a & 1);
  A.ttr = (4 * lg + r) * (TTS * 2) + 8 * a;
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) A.pfr[pp] = lr * 128 + (((4 * pp + lg) ^ swz_p(lr)) << 4);
  A.o = (uint32_t)((lr * DV + 16 * X + 4 * lg) * 2);
  return A;
}

struct StateRegs {
  f32x4 S[8];        // state tiles: value row lr, internal keys 16 jb + 4 lg + e
  f32x4 Oprev[4];    // Q S^T part of the previous chunk's output (per 16-token block)
  bf16x8_t Uprev[2]; // U of the previous chunk as kappa operands
  bf16x8_t Kpre[3][4];  // key fragments of the next chunk's first three 16-token
                        // blocks, read at the end of a period (delta rule)
};

// One period of a state wave: with FINISH, the output of chunk c - 1
// (Oprev + Uprev P^T) is completed and stored; with CHAIN, the S-dependent
// part of chunk c runs.  Both sit in one basic block, and the LDS reads are
// software-pipelined: every operand is read one step before the products
// that use it (scheduling barriers keep the order), while the register
// footprint stays within what two waves per SIMD can hold.
__device__ __forceinline__ void finish_output(const Seq& sq, const StateAddr& A, const StateRegs& R,
                                              const bf16x8_t (&pf)[4][2], int64_t c, int DV) {
  const uint32_t obase = (uint32_t)(c * C * DV * 2) + A.o;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    f32x4 acc = R.Oprev[rb];
#pragma unroll
    for (int pp = 0; pp <= rb / 2; ++pp) acc = mfma(R.Uprev[pp], pf[rb][pp], acc);
    buf_st8(sq.o, obase + (uint32_t)(rb * 16 * DV * 2), pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
  }
}
__device__ __forceinline__ void read_p(const Smem& sm, const StateAddr& A, int64_t c, bf16x8_t (&pf)[4][2]) {
  const lptr pb[2] = {lane_base(sm.P[c & 1], A.pfr[0]), lane_base(sm.P[c & 1], A.pfr[1])};
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int pp = 0; pp <= rb / 2; ++pp) pf[rb][pp] = as_op(ld3<uint4>(pb[pp], rb * 2048));
}

// PRE: the key fragments of blocks 0, 1 and 2 of chunk c are in R.Kpre (read
// at the end of the previous period, so that their LDS latency falls in the
// barrier wait instead of delaying the first products of this period: at the
// start of a period every wave issues its LDS reads at once, and the state
// waves' reads queue behind the others').
// OUT = false: no output (the first launch of the sequence split, which
// needs only the state): no Q S^T, no P U, no stores.
template <bool FINISH_, bool CHAIN, bool GLA, bool PRE = false, bool OUT = true, int KB = 4>
__device__ __forceinline__ void state_period(const Smem& sm, const Seq& sq, const StateAddr& A,
                                             StateRegs& R, int64_t c, int DV, int lane) {
  constexpr int JB = 2 * KB;  // state tiles of 16 keys that can be nonzero
  constexpr bool FINISH = FINISH_ && OUT;
  const int lr = lane & 15, lg = lane >> 4;
  bf16x8_t pf[4][2];
  if constexpr (!CHAIN) {
    read_p(sm, A, c - 1, pf);
    finish_output(sq, A, R, pf, c - 1, DV);
    return;
  }
  const int buf = (int)(c & 1);
  lptr kf_b[4], qf_b[4], kt_b[4];
#pragma unroll
  for (int pp = 0; pp < KB; ++pp) {
    kf_b[pp] = lane_base(k_buf<GLA>(c), A.frag[pp]);
    qf_b[pp] = lane_base(q_buf<GLA>(c), A.frag[pp]);
    kt_b[pp] = lane_base(k_buf<GLA>(c), A.ktr[pp]);
  }
  const lptr v_b = lane_base(lds_V[buf], A.vtr);
  const lptr t_b = lane_base(sm.Tt[buf], A.ttr);
  const int gb = (int)(c & 3);
  const float* gt = &sm.gate[gb][0][0];
  const float decay = sm.egl[gb][0];

  // The chain of this chunk is ordered so that VALU work runs beside
  // independent MFMAs: Z = K S^T first, then O1 = S Q^T while Y is formed
  // from Z, U = Ti Y while O1 is scaled, the previous chunk's O2 while the
  // operands of U are packed, and finally the state update.
  bf16x8_t Sop[4];
#pragma unroll
  for (int pp = 0; pp < KB; ++pp) Sop[pp] = pack_op(R.S[2 * pp], R.S[2 * pp + 1]);

  // ---- Z = K S^T (tile per 16-token block, rows = token).  The fragments
  // of the 16-token blocks K0..K3, Q0..Q3 pass through a ring of three
  // register slots (block n in slot n % 3), read two blocks ahead of their
  // products; the decay of the carried state fills the gaps.
  f32x4 Z[4];
  bf16x8_t fr[3][4];
  auto read_block = [&](int n) {
    if (GLA && n < 4) return;  // without the delta rule K S^T is not needed
    if (!OUT && n >= 4) return;  // no output: Q is not needed
#pragma unroll
    for (int pp = 0; pp < KB; ++pp)
      fr[n % 3][pp] = PRE && n < 3 ? R.Kpre[n][pp]
                                   : as_op(n < 4 ? ld3<uint4>(kf_b[pp], n * 4096) : ld3<uint4>(qf_b[pp], (n - 4) * 4096));
  };
  // V and the gates of Y, read during the products of blocks 1..3
  uint2 vv[4];
  float4 b4[4], g4[4];
  read_block(0);
  read_block(1);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    read_block(rb + 2);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (rb == 1) vv[h] = tr3(v_b, h * 16 * DVS * 2);
      if (rb == 2) b4[h] = *reinterpret_cast<const float4*>(gt + G_BETA * C + 16 * h + 4 * lg);
      if (!GLA && rb == 3) g4[h] = *reinterpret_cast<const float4*>(gt + G_EG * C + 16 * h + 4 * lg);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 az = zero4();
    if constexpr (!GLA) {
#pragma unroll
      for (int pp = 0; pp < KB; ++pp) az = mfma(fr[rb % 3][pp], Sop[pp], az);
    }
    if (2 * rb < JB) {
      R.S[2 * rb] *= decay;
      R.S[2 * rb + 1] *= decay;
    }
    Z[rb] = az;
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- O1 = S Q^T (rows = value, columns = token) while Y = beta (V -
  // 2^g Z) is formed; Ti, the output gates and P are read meanwhile.
  f32x4 O1[4], y[4];
  bf16x8_t tf[4][2];
  f32x4 el[4];
  float eg[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (rb < 2) read_block(rb + 6);  // Q block rb sits in slot (4 + rb) % 3
    if (!GLA && rb == 2) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int pp = 0; pp <= tb / 2; ++pp) {
          const int off = pp * 32 * TTS * 2 + tb * 32;
          tf[tb][pp] = as_op(tr3(t_b, off), tr3(t_b, off + 16 * TTS * 2));
        }
    }
    if (rb == 3) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float4 e = *reinterpret_cast<const float4*>(gt + G_EL * C + 16 * h + 4 * lg);
        el[h] = f32x4{e.x, e.y, e.z, e.w};
        eg[h] = gt[G_EG * C + 16 * h + lr];
      }
      if constexpr (FINISH) read_p(sm, A, c - 1, pf);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (OUT) {
      f32x4 ao = zero4();
#pragma unroll
      for (int pp = 0; pp < KB; ++pp) ao = mfma(Sop[pp], fr[(4 + rb) % 3][pp], ao);
      O1[rb] = ao;
    }
    if constexpr (GLA) {
      y[rb][0] = b4[rb].x * __uint_as_float(vv[rb].x << 16);
      y[rb][1] = b4[rb].y * __uint_as_float(vv[rb].x & 0xffff0000u);
      y[rb][2] = b4[rb].z * __uint_as_float(vv[rb].y << 16);
      y[rb][3] = b4[rb].w * __uint_as_float(vv[rb].y & 0xffff0000u);
    } else {
      y[rb][0] = b4[rb].x * fmaf(-g4[rb].x, Z[rb][0], __uint_as_float(vv[rb].x << 16));
      y[rb][1] = b4[rb].y * fmaf(-g4[rb].y, Z[rb][1], __uint_as_float(vv[rb].x & 0xffff0000u));
      y[rb][2] = b4[rb].z * fmaf(-g4[rb].z, Z[rb][2], __uint_as_float(vv[rb].y << 16));
      y[rb][3] = b4[rb].w * fmaf(-g4[rb].w, Z[rb][3], __uint_as_float(vv[rb].y & 0xffff0000u));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const bf16x8_t Yop[2] = {pack_op(y[0], y[1]), pack_op(y[2], y[3])};
  // the first K^T operands of the state update (ring of four slots, tile jb
  // in slot jb % 4, read three tiles ahead of its products)
  bf16x8_t kt[4][2];
  auto read_kt = [&](int jb, bf16x8_t (&dst)[2]) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int off = (jb & 1) * 8 + pp * 32 * 256;
      dst[pp] = as_op(tr3(kt_b[jb >> 1], off), tr3(kt_b[jb >> 1], off + 16 * 256));
    }
  };
  read_kt(0, kt[0]);
  read_kt(1, kt[1]);
  read_kt(2, kt[2]);
  static_assert(JB >= 4, "the K^T ring and the key pre-reads below assume at least four state tiles");
  __builtin_amdgcn_sched_barrier(0);
  // ---- U = Ti Y (Ti lower triangular: row block rb needs the 32-token blocks
  // pp <= rb/2, the upper 16x16 blocks inside them are zero) while O1 takes
  // the factor 2^g of its token column.
  f32x4 U[4], Onew[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if constexpr (GLA) {
      U[rb] = y[rb];  // Ti = I
    } else {
      f32x4 acc = zero4();
#pragma unroll
      for (int pp = 0; pp <= rb / 2; ++pp) acc = mfma(tf[rb][pp], Yop[pp], acc);
      U[rb] = acc;
    }
    if constexpr (OUT) Onew[rb] = O1[rb] * eg[rb];
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- output of the previous chunk while the operands of U are packed:
  // plain (for O) and scaled by 2^(g_C - g_s) (for S).
  f32x4 Ofin[4];
  if constexpr (FINISH) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 acc = R.Oprev[rb];
#pragma unroll
      for (int pp = 0; pp <= rb / 2; ++pp) acc = mfma(R.Uprev[pp], pf[rb][pp], acc);
      Ofin[rb] = acc;
    }
  }
  if constexpr (OUT) {
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) R.Oprev[rb] = Onew[rb];
  }
  bf16x8_t Uh[2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    if constexpr (OUT) R.Uprev[pp] = pack_op(U[2 * pp], U[2 * pp + 1]);
    Uh[pp] = pack_op(U[2 * pp] * el[2 * pp], U[2 * pp + 1] * el[2 * pp + 1]);
  }
  if constexpr (FINISH) {
    const uint32_t obase = (uint32_t)((c - 1) * C * DV * 2) + A.o;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      buf_st8(sq.o, obase + (uint32_t)(rb * 16 * DV * 2), pack2(Ofin[rb][0], Ofin[rb][1]),
              pack2(Ofin[rb][2], Ofin[rb][3]));
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- S^T += K^T Uh with K^T from transposed reads: supplier lane (a, r) of
  // a 16-lane group addresses 4 key columns of token 4 lg + r.  The operands
  // of tile jb + 3 are read while the products of tile jb run; in the last
  // tiles (delta rule) the key fragments of the next chunk's blocks 0, 1 and
  // 2 are read instead.  The next chunk's keys are in LDS already (loaded three
  // chunks ahead); after the last chunk the reads fetch unused values.
  lptr kn_b[4];
  if constexpr (!GLA) {
#pragma unroll
    for (int pp = 0; pp < KB; ++pp) kn_b[pp] = lane_base(k_buf<GLA>(c + 1), A.frag[pp]);
  }
  // (the key pre-reads run in the last three tiles but one: JB - 4 .. JB - 2)
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    if (jb < JB - 3) read_kt(jb + 3, kt[(jb + 3) % 4]);
    if (!GLA && jb >= JB - 4 && jb <= JB - 2) {
#pragma unroll
      for (int pp = 0; pp < KB; ++pp)
        R.Kpre[jb - (JB - 4)][pp] = as_op(ld3<uint4>(kn_b[pp], (jb - (JB - 4)) * 4096));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = R.S[jb];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) acc = mfma(kt[jb % 4][pp], Uh[pp], acc);
    R.S[jb] = acc;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ============================================================ K, Q, V into LDS
// LDS-DMA loads of chunk c.  Lane i of a 16-byte LDS-DMA
// load writes bytes 16 i .. 16 i + 15 after the uniform LDS base, so each lane
// fetches the global octet that the swizzled layout puts there: for K and Q,
// instruction it covers tokens 4 it .. 4 it + 3 and lane (lr, lg) fills
// physical octet lr of token 4 it + lg, i.e. key octet lr ^ swz_kq(4 it + lg)
// (swz_kq of token 4 it + lg depends on it only through it & 3).
struct DmaAddr {
  uint32_t kq[4];  // per it & 3
  uint32_t v;
};
// With dk = 64 a lane whose key octet is 8 or more reads past the end of the
// buffer range, which returns zero, so those LDS octets are written as zero.
constexpr uint32_t OOB_OFFSET = 0x80000000u;
__device__ __forceinline__ DmaAddr dma_addr(int lane, int DV, int dk) {
  const int lr = lane & 15, lg = lane >> 4;
  DmaAddr A;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int ko = lr ^ swz_kq(4 * m + lg);
    A.kq[m] = 8 * ko < dk ? (uint32_t)(lg * dk * 2 + (ko << 4)) : OOB_OFFSET;
  }
  // lane -> token 16 it + lane / 4, physical slot lane % 4 (see vtr)
  A.v = (uint32_t)((lane >> 2) * DV * 2 + (((lane & 3) ^ (2 * ((lane >> 4) & 1))) << 4));
  return A;
}
// K (or Q) of chunk c into dst: 16 LDS-DMA loads.
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t src, bf16_t* dst, const Seq& sq, const DmaAddr& A,
                                         int64_t c) {
  const uint32_t row = (uint32_t)(sq.dk * 2), kq0 = (uint32_t)(c * C) * row;
#pragma unroll
  for (int it = 0; it < 16; ++it)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)&dst[it * 512], 16, A.kq[it & 3],
                                             (int)(kq0 + it * 4 * row), 0, 0);
}
// V of chunk c (4 loads) into buffer c % 2.
__device__ __forceinline__ void dma_v(const Seq& sq, const DmaAddr& A, int64_t c, int DV) {
  const int buf = (int)(c & 1);
  const uint32_t v0 = (uint32_t)(c * C * DV * 2);
#pragma unroll
  for (int it = 0; it < 4; ++it)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.v, (lds_void*)&lds_V[buf][it * 512], 16, A.v,
                                             (int)(v0 + it * 16 * DV * 2), 0, 0);
}

// ============================================================ prefetch wave
// L2 prefetch of chunk c: one 4-byte load per 128-byte line, landing in a
// scratch word of LDS (an LDS-DMA load has a side effect, so it is kept, and
// no register waits for it).  The four slice workgroups of a sequence split
// the key and query lines; each touches its own value lines.  All 64 lanes
// take part in every load (lanes 32..63 repeat the lines of lanes 0..31), so
// the descriptors stay uniform.
__device__ __forceinline__ void prefetch_keys(const Seq& sq, int64_t c, int slice, int lane) {
  const uint32_t kq = (uint32_t)(c * C * sq.dk * 2) + (uint32_t)((32 * slice + (lane & 31)) * 128);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.k, (lds_void*)&lds_touch[0], 4, kq, 0, 0, 0);
}
__device__ __forceinline__ void prefetch_rest(const Seq& sq, int64_t c, int slice, int DV, int lane, bool q_on = true) {
  lds_void* land = (lds_void*)&lds_touch[0];
  const uint32_t kq = (uint32_t)(c * C * sq.dk * 2) + (uint32_t)((32 * slice + (lane & 31)) * 128);
  if (q_on) __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.q, land, 4, kq, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.v, land, 4, (uint32_t)((c * C + lane) * DV * 2), 0, 0, 0);
  const uint32_t g = (uint32_t)(c * C * 4 + (lane & 1) * 128);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.a, land, 4, g, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.b, land, 4, g, 0, 0, 0);
}

// ============================================================ P wave
// The 10 lower 16x16 tiles of a 64x64 chunk matrix, in the order the P and
// L waves build them: (row block rb, column block sb), sb <= rb.
constexpr int TILE_RB[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
constexpr int TILE_SB[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

// Tiles TB .. TE-1 of P of chunk c.  Tiles are software-pipelined: the
// products of tile t + 1 are issued before the decay, mask and store of tile t.
template <bool GLA, int TB = 0, int TE = 10, int KB = 4>
__device__ __forceinline__ void build_p(Smem& sm, const StateAddr& A, int64_t c, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int buf = (int)(c & 1);
  lptr kf_b[4], qf_b[4];
#pragma unroll
  for (int pp = 0; pp < KB; ++pp) {
    kf_b[pp] = lane_base(k_buf<GLA>(c), A.frag[pp]);
    qf_b[pp] = lane_base(q_buf<GLA>(c), A.frag[pp]);
  }
  const float* gt = &sm.gate[c & 3][0][0];
  char* Pb = reinterpret_cast<char*>(sm.P[buf]);
  int pw[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) pw[h] = lr * 128 + (((4 * h + lg) ^ swz_p(lr)) << 4);
  bf16x8_t kf[4][4], qf[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int pp = 0; pp < KB; ++pp) kf[b][pp] = as_op(ld3<uint4>(kf_b[pp], b * 4096));
#pragma unroll
  for (int b = 0; b < (TB == 0 ? 2 : 4); ++b)
#pragma unroll
    for (int pp = 0; pp < KB; ++pp) qf[b][pp] = as_op(ld3<uint4>(qf_b[pp], b * 4096));
  // decay of element (s, r): 2^(g_r - g_C) 2^(g_C - g_s) when split, else
  // 2^(g_r - g_s) from the log table
  const bool split = split_decay(sm, c);
  float gr[4];
  float4 gs4[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    gr[b] = gt[(split ? G_ER : G_LOG) * C + 16 * b + lr];
    gs4[b] = *reinterpret_cast<const float4*>(gt + (split ? G_EL : G_LOG) * C + 16 * b + 4 * lg);
  }
  // element (s, r) = k_s . q_r of tile t
  auto tile = [&](int t) {
    f32x4 acc = zero4();
#pragma unroll
    for (int pp = 0; pp < KB; ++pp) acc = mfma(kf[TILE_SB[t]][pp], qf[TILE_RB[t]][pp], acc);
    return acc;
  };
  auto run = [&](auto SPLIT) {
    f32x4 acc[2];
    acc[TB & 1] = tile(TB);
#pragma unroll
    for (int t = TB; t < TE; ++t) {
      const int rb = TILE_RB[t], sb = TILE_SB[t];
      if (TB == 0 && sb == 0 && rb >= 1 && rb < 3) {
#pragma unroll
        for (int pp = 0; pp < KB; ++pp) qf[rb + 1][pp] = as_op(ld3<uint4>(qf_b[pp], (rb + 1) * 4096));
      }
      if (t + 1 < TE) acc[(t + 1) & 1] = tile(t + 1);
      __builtin_amdgcn_sched_barrier(0);
      const f32x4 a = acc[t & 1];
      const float g[4] = {gs4[sb].x, gs4[sb].y, gs4[sb].z, gs4[sb].w};
      float val[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        val[e] = decltype(SPLIT)::value ? a[e] * g[e] * gr[rb] : fast_exp2(gr[rb] - g[e]) * a[e];
      if (sb == rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (4 * lg + e <= lr) ? val[e] : 0.f;
      }
      lds_put<uint2>(Pb, pw[sb >> 1] + (sb & 1) * 8 + rb * 2048,
                     make_uint2(pack2(val[0], val[1]), pack2(val[2], val[3])));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (split)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// ============================================================ L wave
// Keys of one chunk in MFMA fragment layout: kf[rb][pp] = key octet 4 pp + lg
// of token 16 rb + lr, read from K in LDS with the fragment addresses of the
// state waves.
struct FragRegs {
  uint4 kf[4][4];
};

template <bool GLA, int KB = 4>
__device__ __forceinline__ void read_frags(FragRegs& R, const StateAddr& A, int64_t c) {
#pragma unroll
  for (int pp = 0; pp < KB; ++pp) {
    const lptr b = lane_base(k_buf<GLA>(c), A.frag[pp]);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) R.kf[rb][pp] = ld3<uint4>(b, rb * 4096);
  }
}

// Gate tables of chunk c (alpha, beta of token `lane` as loaded, 0 past the
// end): beta, 2^(g - g_C), 2^g, 2^(g_C - g), g and 2^(g_C), with g the
// log2-prefix of alpha.  The decay 2^(g_r - g_s) of P and L is the product
// 2^(g_r - g_C) 2^(g_C - g_s) of two table entries when g_C >= SPLIT_MIN (both
// factors then lie in the normal fp32 range); otherwise P and L take one exp2
// per element.
__device__ __forceinline__ void build_gates(Smem& sm, float ra, float rb, int64_t c, int64_t T, int lane) {
  float* gt = &sm.gate[c & 3][0][0];
  // tokens past the end are identity maps (alpha 1, beta 0)
  const bool live = c * C + lane < T;
  const float a = live ? ra : 1.f, b = live ? rb : 0.f;
  const float gs = wave_prefix_sum(fmaxf(fast_log2(a), LOG2_ALPHA_MIN));
  const float glast = lane63(gs);
  gt[G_BETA * C + lane] = b;
  gt[G_ER * C + lane] = fast_exp2(gs - glast);
  gt[G_EG * C + lane] = fast_exp2(gs);
  gt[G_EL * C + lane] = fast_exp2(glast - gs);
  gt[G_LOG * C + lane] = gs;
  if (lane == 0) {
    sm.egl[c & 3][0] = fast_exp2(glast);
    sm.egl[c & 3][1] = glast >= SPLIT_MIN ? 1.f : 0.f;
  }
}
// L of chunk c: diagonal blocks as fp32 rows, off-diagonal blocks as bf16 in
// the order in which the inverse consumes them as MFMA A operands.  The row
// factor beta_r multiplies the decay (split as in build_p), and the tiles are
// software-pipelined as in build_p.
template <int KB = 4>
__device__ __forceinline__ void build_l(Smem& sm, const FragRegs& R, int64_t c, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int lb = (int)(c & 1);
  const float* gt = &sm.gate[c & 3][0][0];
  const bool split = split_decay(sm, c);
  float grb[4], br[4];
  float4 gs4[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    grb[b] = gt[(split ? G_ER : G_LOG) * C + 16 * b + lr];
    br[b] = gt[G_BETA * C + 16 * b + lr];
    gs4[b] = *reinterpret_cast<const float4*>(gt + (split ? G_EL : G_LOG) * C + 16 * b + 4 * lg);
  }
  // tile t: lane holds k_r . k_s for r = 16rb + lr, s = 16sb + 4lg + e
  auto tile = [&](int t) {
    f32x4 acc = zero4();
#pragma unroll
    for (int pp = 0; pp < KB; ++pp) acc = mfma(as_op(R.kf[TILE_SB[t]][pp]), as_op(R.kf[TILE_RB[t]][pp]), acc);
    return acc;
  };
  auto run = [&](auto SPLIT) {
    float rf[4];  // row factor: beta_r 2^(g_r - g_C) when split, else g_r
#pragma unroll
    for (int b = 0; b < 4; ++b) rf[b] = decltype(SPLIT)::value ? br[b] * grb[b] : grb[b];
    f32x4 acc[2];
    acc[0] = tile(0);
#pragma unroll
    for (int t = 0; t < 10; ++t) {
      const int rb = TILE_RB[t], sb = TILE_SB[t];
      if (t + 1 < 10) acc[(t + 1) & 1] = tile(t + 1);
      __builtin_amdgcn_sched_barrier(0);
      const f32x4 a = acc[t & 1];
      const float g[4] = {gs4[sb].x, gs4[sb].y, gs4[sb].z, gs4[sb].w};
      float val[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        val[e] = decltype(SPLIT)::value ? a[e] * g[e] * rf[rb] : fast_exp2(rf[rb] - g[e]) * (a[e] * br[rb]);
      if (sb == rb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (4 * lg + e < lr) ? val[e] : 0.f;
        *reinterpret_cast<float4*>(&sm.Ld[lb][rb][lr * LDR + 4 * lg]) = make_float4(val[0], val[1], val[2], val[3]);
      } else {
        const int tix = rb * (rb - 1) / 2 + sb;
        *reinterpret_cast<uint2*>(&sm.Lo[lb][tix][lane * 4]) =
            make_uint2(pack2(val[0], val[1]), pack2(val[2], val[3]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (split)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// ============================================================ loader wave
// In period p the loader builds the gate tables of chunk p+3 (gates loaded one
// period earlier) and loads the gates of chunk p+4, V and Q of chunk p+1 and
// K of chunk p+3 (GLA: V of p+1, K and Q of p+2), and ends the period once
// they are in LDS (the prefetch wave has pulled their lines into L2 two
// periods earlier).
// Before the first period: the gate tables of chunk 0, and the gates of
// chunk 1 (in registers for the delta rule, landed in lds_gst by LDS-DMA for
// GLA); for the delta rule also K of chunk 0.
template <bool GLA>
__device__ __forceinline__ void loader_prologue(Smem& sm, const Seq& sq, const DmaAddr& D, int64_t nch, float& ga,
                                                float& gb, int lane) {
  ga = gb = 0.f;
  if (nch > 0) {
    if constexpr (!GLA) dma_rows(sq.k, k_buf<GLA>(0), sq, D, 0);
    build_gates(sm, buf_ldf(sq.a, (uint32_t)(lane * 4)), buf_ldf(sq.b, (uint32_t)(lane * 4)), 0, sq.T, lane);
    if constexpr (GLA) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.a, (lds_void*)&lds_gst[0][0], 4, lane * 4, C * 4, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.b, (lds_void*)&lds_gst[1][0], 4, lane * 4, C * 4, 0, 0);
    } else {
      ga = buf_ldf(sq.a, (uint32_t)((C + lane) * 4));
      gb = buf_ldf(sq.b, (uint32_t)((C + lane) * 4));
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no load is pending when the loop starts
}

// One period of the loader.  Every global load of the period is issued first,
// and the gate tables of chunk p+3 are built while they fly, from the gates
// loaded one period earlier.
//   delta rule: the gates go to registers and the wait is vmcnt(0).
//   GLA: K is two chunks ahead (Q too, moved by the L wave) and the wait
//   leaves this period's 16 K loads in flight (vmcnt(16)).  The gates then
//   go through LDS (lds_gst) by LDS-DMA: in registers, the compiler would
//   wait for every load before their use, since its count ignores LDS-DMA
//   loads.
template <bool GLA, bool OUT = true>
__device__ __forceinline__ void loader_period(Smem& sm, const Seq& sq, const DmaAddr& D, int64_t p, int64_t nch,
                                              int DV, float& ga, float& gb, int lane) {
  constexpr int KA = KQ_AHEAD<GLA>;
  if constexpr (!GLA) {
    float na = 0.f, nb = 0.f;
    if (p + 3 < nch) {
      const uint32_t t4 = (uint32_t)(((p + 4) * C + lane) * 4);
      na = buf_ldf(sq.a, t4);
      nb = buf_ldf(sq.b, t4);
    }
    if (p + 1 >= 0 && p + 1 < nch) {
      dma_v(sq, D, p + 1, DV);
      if (OUT) dma_rows(sq.q, q_buf<GLA>(p + 1), sq, D, p + 1);
    }
    if (p + 3 >= 0 && p + 3 < nch) dma_rows(sq.k, k_buf<GLA>(p + 3), sq, D, p + 3);
    if (p + 3 < nch) build_gates(sm, ga, gb, p + 3, sq.T, lane);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    ga = na;
    gb = nb;
  } else {
    if (p + 3 < nch) {
      // The gates that landed one period earlier are complete: that period
      // ended with a wait for every load but its last 16 (the K loads).  The read is
      // asm because the compiler's own wait before a read of an LDS-DMA
      // target would be vmcnt(0), i.e. also for the K loads in flight.  It
      // completes (lgkmcnt(0)) before the DMA below rewrites the gates.
      const uint32_t ga_addr = (uint32_t)(uintptr_t)(lds_void*)&lds_gst[0][lane];
      asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(ga), "=&v"(gb)
                   : "v"(ga_addr), "i"(C * 4)
                   : "memory");
      const uint32_t t4 = (uint32_t)(((p + 4) * C) * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.a, (lds_void*)&lds_gst[0][0], 4, lane * 4, (int)t4, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sq.b, (lds_void*)&lds_gst[1][0], 4, lane * 4, (int)t4, 0, 0);
    }
    if (p + 1 >= 0 && p + 1 < nch) dma_v(sq, D, p + 1, DV);
    const bool kq_next = p + KA >= 0 && p + KA < nch;
    if (kq_next) dma_rows(sq.k, k_buf<GLA>(p + KA), sq, D, p + KA);  // Q: the L wave
    if (p + 3 < nch) build_gates(sm, ga, gb, p + 3, sq.T, lane);
    static_assert(KA == 2, "the wait below leaves this period's 16 K loads in flight");
    if (kq_next)
      __builtin_amdgcn_s_waitcnt(0x4f70);  // vmcnt(16): vmcnt bits [15:14] = 1, [3:0] = 0
    else
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  }
}

// ============================================================ inverse wave
// Forward substitution over key columns 4Q .. 4Q+3 of one unit-lower 16x16
// block: x[r] -= L[r][s] x[s] for s in the band and r > s.  The band's rows of
// L (float4, read by all 16 lanes of a group at once) are read one band ahead.
template <int Q>
__device__ __forceinline__ void subst_read(float4 (&lq)[16], const float* Lr) {
#pragma unroll
  for (int r = 4 * Q + 1; r < 16; ++r) lq[r] = *reinterpret_cast<const float4*>(Lr + r * LDR + 4 * Q);
}
template <int Q>
__device__ __forceinline__ void subst_band(float (&x)[16], const float4 (&lq)[16]) {
#pragma unroll
  for (int s = 4 * Q; s < 4 * Q + 4; ++s) {
#pragma unroll
    for (int r = s + 1; r < 16; ++r) {
      const float4 l4 = lq[r];
      const float lrs = (s & 3) == 0 ? l4.x : (s & 3) == 1 ? l4.y : (s & 3) == 2 ? l4.z : l4.w;
      x[r] = fmaf(-lrs, x[s], x[r]);
    }
  }
}

__device__ __forceinline__ void build_inverse(Smem& sm, int64_t c, const float (&xinit)[16], int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int lb = (int)(c & 1);
  char* Tb = reinterpret_cast<char*>(sm.Tt[lb]);
  // off-diagonal blocks of L, needed only after the diagonal blocks are done
  uint2 Lop[6];
#pragma unroll
  for (int t = 0; t < 6; ++t) Lop[t] = *reinterpret_cast<const uint2*>(&sm.Lo[lb][t][lane * 4]);
  {
    const float* Lr = &sm.Ld[lb][lg][0];
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = xinit[r];
    float4 la[16], lbb[16];
    subst_read<0>(la, Lr);
    subst_read<1>(lbb, Lr);
    __builtin_amdgcn_sched_barrier(0);
    subst_band<0>(x, la);
    subst_read<2>(la, Lr);
    __builtin_amdgcn_sched_barrier(0);
    subst_band<1>(x, lbb);
    subst_read<3>(lbb, Lr);
    __builtin_amdgcn_sched_barrier(0);
    subst_band<2>(x, la);
    subst_band<3>(x, lbb);
    // column lr of block lg = row (16 lg + lr) of Ti^T, columns 16 lg .. +15
    char* dst = Tb + (16 * lg + lr) * (TTS * 2) + 32 * lg;
    lds_put<uint4>(dst, 0, make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])));
    lds_put<uint4>(dst, 16, make_uint4(pack2(x[8], x[9]), pack2(x[10], x[11]), pack2(x[12], x[13]), pack2(x[14], x[15])));
  }
  wave_lds_fence();
  // B operand of T_cc: lane holds T_cc[4lg + e][lr] = Ti^T[16c + lr][16c + 4lg + e]
  uint2 Bd[3];
#pragma unroll
  for (int cc = 0; cc < 3; ++cc) Bd[cc] = lds_at<uint2>(Tb, (16 * cc + lr) * (TTS * 2) + (16 * cc + 4 * lg) * 2);
  // A operand of T_aa: lane holds T_aa[lr][4lg + e], from transposed reads of Ti^T
  uint2 Ad[4];
  {
    const int a = lr & 3, r = lr >> 2;
#pragma unroll
    for (int aa = 1; aa < 4; ++aa)
      Ad[aa] = lds_tr(Tb, (16 * aa + 4 * lg + r) * (TTS * 2) + (16 * aa + 4 * a) * 2);
  }
  // T blocks below the diagonal as B operands: Tb_[a][b]
  uint2 Tbo[4][3];
#pragma unroll
  for (int a = 1; a < 4; ++a) {
#pragma unroll
    for (int b = a - 1; b >= 0; --b) {
      f32x4 m = zero4();
#pragma unroll
      for (int cc = b; cc < a; ++cc) m = mfma16(Lop[a * (a - 1) / 2 + cc], cc == b ? Bd[b] : Tbo[cc][b], m);
      const f32x4 t = mfma16(Ad[a], pack_tile(-m), zero4());
      Tbo[a][b] = pack_tile(t);
      // lane holds T_ab[4lg + e][lr] -> Ti^T[16b + lr][16a + 4lg + e]
      lds_put<uint2>(Tb, (16 * b + lr) * (TTS * 2) + (16 * a + 4 * lg) * 2, Tbo[a][b]);
    }
  }
}

// ============================================================ kernel
// How the workgroups of one launch map onto (sequence, token range) pairs.
//   SEQ:     chain i is sequence i, all T tokens; state from initial_state[i]
//            (zero if NULL) to final_state[i] (skipped if NULL).
//   SPLIT_A: the first G-1 segments of L tokens of every sequence, twice:
//            kind 0 from a zero state with V (chain state -> ws slot
//            "tilde"), kind 1 from the identity with V read as zero (-> slot
//            "trans"); no output.  Kind 1 gives the segment's transition M:
//            a state S entering the segment leaves it as S M + tilde.
//   SPLIT_C: all G segments of every sequence, segment g starting from ws
//            slot "start", with output; the last segment's state goes to
//            final_state.
// ws holds tilde and trans, nseq * (G-1) states of d x d floats each
// (index seq * (G-1) + g), then start, nseq * G states (index seq * G + g;
// start of segment 0 is a copy of initial_state).
enum { MAP_SEQ = 0, MAP_SPLIT_A = 1, MAP_SPLIT_C = 2 };
struct ChainMap {
  int mode, nseq, G;
  int64_t T, L;  // tokens per sequence, tokens per segment (a multiple of C)
  float* ws;
};
__host__ __device__ inline int map_chains(const ChainMap& m) {
  return m.mode == MAP_SEQ ? m.nseq : m.mode == MAP_SPLIT_A ? 2 * m.nseq * (m.G - 1) : m.nseq * m.G;
}

// GLA: gated linear attention without the delta rule ([P3] §2.3),
// S_t = alpha_t S_{t-1} + beta_t v_t k_t^T.  Its chunk form is the one above
// with L = 0 (so Ti = I) and U = Y = diag(beta) V: the L and inverse waves
// stay idle, and the state waves compute neither K S^T nor the product by Ti.
// The state chain is then only the decayed accumulation of U^T K.
// OUT = false (delta rule only): the first launch of the sequence split,
// which needs the segment states and no output; the P wave, the loads of Q
// and the output products are left out.
// KB: 32-key blocks that can be nonzero, dk / 32.  With dk = 64 (KB = 2) the
// keys 64..127 are zero in LDS and in the state, so the products over them
// and the state tiles of those keys are skipped.
template <bool GLA, bool OUT = true, int KB = 4>
__global__ __launch_bounds__(64 * NWAVES) void chunk_fwd_pipe_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta,
    const float* initial_state, bf16_t* __restrict__ o, float* final_state, ChainMap cm,
    int DV, int dk, int xcd_map) {
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15;
  const int lg = lane >> 4;

  const int NS = DV / DVS;
  const int nchain = map_chains(cm);
  int chain, slice;
  {
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
  if (chain >= nchain) return;

  // this chain's sequence, token range, start and end state, and whether it
  // reads V and writes output
  const int64_t dd = (int64_t)dk * DV;  // floats per state
  int seq = chain;
  int64_t t0 = 0, Tlen = cm.T;
  bool v_on = true, o_on = true, s0_ident = false;
  const float* s0 = initial_state ? initial_state + (int64_t)chain * dd : nullptr;
  float* sT = final_state ? final_state + (int64_t)chain * dd : nullptr;
  if (cm.mode == MAP_SPLIT_A) {
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
  } else if (cm.mode == MAP_SPLIT_C) {
    seq = chain / cm.G;
    const int g = chain % cm.G;
    t0 = (int64_t)g * cm.L;
    Tlen = g == cm.G - 1 ? cm.T - t0 : cm.L;
    s0 = cm.ws + (2 * (int64_t)cm.nseq * (cm.G - 1) + (int64_t)seq * cm.G + g) * dd;
    sT = g == cm.G - 1 && final_state ? final_state + (int64_t)seq * dd : nullptr;
  }

  Seq sq;
  sq.T = Tlen;
  {
    sq.dk = dk;
    const int64_t tok = (int64_t)seq * cm.T + t0;  // first token in memory
    const uint32_t kq_bytes = (uint32_t)(Tlen * dk * 2);
    sq.q = make_rsrc(q + tok * dk, kq_bytes);
    sq.k = make_rsrc(k + tok * dk, kq_bytes);
    // value / output slice: the descriptor range ends with the token range;
    // an empty range reads zeros and drops stores
    const int64_t vs = tok * DV + slice * DVS;
    const uint32_t v_bytes = (uint32_t)((Tlen * DV - slice * DVS) * 2);
    sq.v = make_rsrc(v + vs, v_on ? v_bytes : 0u);
    sq.o = make_rsrc(o + vs, o_on ? v_bytes : 0u);
    sq.a = make_rsrc(alpha + tok, (uint32_t)(Tlen * 4));
    sq.b = make_rsrc(beta + tok, (uint32_t)(Tlen * 4));
  }
  const int64_t nch = (Tlen + C - 1) / C;

  if constexpr (POISON_LDS) {
    lds_poison(sm, tid, 64 * NWAVES);
    if constexpr (GLA) {
      lds_poison(lds_K, tid, 64 * NWAVES);
      lds_poison(lds_Q, tid, 64 * NWAVES);
      lds_poison(lds_gst, tid, 64 * NWAVES);
    } else {
      lds_poison(lds_K4, tid, 64 * NWAVES);
      lds_poison(lds_Q2, tid, 64 * NWAVES);
    }
    lds_poison(lds_V, tid, 64 * NWAVES);
    __syncthreads();
  }

  // Zero P and Ti^T: their blocks above the diagonal are never written but
  // are read as zero by 32-deep products.
  {
    uint32_t* z = reinterpret_cast<uint32_t*>(&sm.P[0][0]);
    for (int e = tid; e < 2 * C * C / 2; e += 64 * NWAVES) z[e] = 0u;
    uint32_t* z2 = reinterpret_cast<uint32_t*>(&sm.Tt[0][0]);
    for (int e = tid; e < 2 * C * TTS / 2; e += 64 * NWAVES) z2[e] = 0u;
  }

  // The empty slot only helps to zero P and Ti^T.  Its stores are complete
  // before it ends, and a barrier waits only for waves that have not ended.
  if (wave == W_IDLE) {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    return;
  }

  // Each role runs its own loop over periods p = -2 .. nch with exactly one
  // workgroup barrier per period, so all waves meet at every barrier.
  if (wave < 2) {
    const int X = wave;
    const StateAddr A = state_addr(lane, X, DV);
    const int st_row = slice * DVS + 16 * X + lr;  // value row of the state
    StateRegs R;
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      R.S[jb] = zero4();
      if (s0_ident) {
#pragma unroll
        for (int e = 0; e < 4; ++e) R.S[jb][e] = st_row == state_col(jb, lg) + e ? 1.f : 0.f;
      } else if (s0 && state_col(jb, lg) < dk) {
        const float4 s4 = *reinterpret_cast<const float4*>(s0 + (int64_t)st_row * dk + state_col(jb, lg));
        R.S[jb] = f32x4{s4.x, s4.y, s4.z, s4.w};
      }
    }
    // the set-up barrier, periods -2 and -1 (nothing to do yet), chunk 0, the
    // steady state (output of chunk p-1 and chain of chunk p), the last output
    lds_barrier();
    lds_barrier();
    lds_barrier();
    if (nch > 0) {
      state_period<false, true, GLA, false, OUT, KB>(sm, sq, A, R, 0, DV, lane);
      lds_barrier();
      for (int64_t p = 1; p < nch; ++p) {
        state_period<true, true, GLA, !GLA, OUT, KB>(sm, sq, A, R, p, DV, lane);
        lds_barrier();
      }
      if (OUT) state_period<true, false, GLA, false, true, KB>(sm, sq, A, R, nch, DV, lane);
    }
    lds_barrier();
    if (sT) {
#pragma unroll
      for (int jb = 0; jb < 8; ++jb)
        if (state_col(jb, lg) < dk)
          *reinterpret_cast<float4*>(sT + (int64_t)st_row * dk + state_col(jb, lg)) = as_f4(R.S[jb]);
    }
  } else if (wave == W_P) {
    const StateAddr A = state_addr(lane, 0, DV);
    lds_barrier();
    for (int64_t p = -2; p <= nch; ++p) {
      // With the delta rule the P wave has slack: it starts its LDS reads
      // about 500 cycles into the period, behind those of the state waves,
      // whose chain is longer (without it, P is as long as the state waves).
      if constexpr (!GLA) __builtin_amdgcn_s_sleep(8);
      if (OUT && p >= 0 && p < nch) build_p<GLA, 0, GLA ? PSPLIT : 10, KB>(sm, A, p, lane);
      lds_barrier();
    }
  } else if (GLA && wave == W_L) {
    // without the delta rule the L wave moves Q, two chunks ahead, and keeps
    // each period's 16 loads in flight across the barrier
    const DmaAddr D = dma_addr(lane, DV, dk);
    lds_barrier();
    for (int64_t p = -2; p <= nch; ++p) {
      const bool q_next = p + 2 >= 0 && p + 2 < nch;
      if (q_next) {
        dma_rows(sq.q, q_buf<GLA>(p + 2), sq, D, p + 2);
        __builtin_amdgcn_s_waitcnt(0x4f70);  // vmcnt(16)
      } else {
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      }
      lds_barrier_keep_dma();
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);
  } else if (wave == W_L) {
    const StateAddr A = state_addr(lane, 0, DV);
    FragRegs R;
    lds_barrier();
    for (int64_t p = -2; p <= nch; ++p) {
      if (!GLA && p + 2 < nch) {
        read_frags<GLA, KB>(R, A, p + 2);
        build_l<KB>(sm, R, p + 2, lane);
      }
      lds_barrier();
    }
  } else if (wave == W_LOADER) {
    const DmaAddr D = dma_addr(lane, DV, dk);
    float ga, gb;
    loader_prologue<GLA>(sm, sq, D, nch, ga, gb, lane);
    lds_barrier();
    for (int64_t p = -2; p <= nch; ++p) {
      loader_period<GLA, OUT>(sm, sq, D, p, nch, DV, ga, gb, lane);
      if constexpr (GLA)
        lds_barrier_keep_dma();  // this period's K loads stay in flight
      else
        lds_barrier();
    }
  } else if (GLA && wave == W_INV) {
    // without the delta rule this slot builds the last tiles of P
    const StateAddr A = state_addr(lane, 0, DV);
    lds_barrier();
    for (int64_t p = -2; p <= nch; ++p) {
      if (p >= 0 && p < nch) build_p<GLA, PSPLIT, 10, KB>(sm, A, p, lane);
      lds_barrier();
    }
  } else if (wave == W_INV) {
    // The inverse is the longest role of a period and shares its SIMD with the
    // L wave, which has slack: it takes the higher issue priority (about 1 %
    // faster, alternating on one GPU).
    __builtin_amdgcn_s_setprio(3);
    // column lr of the identity: the start of the forward substitution
    float xinit[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) xinit[r] = (r == lr) ? 1.f : 0.f;
    lds_barrier();
    for (int64_t p = -2; p <= nch; ++p) {
      if (!GLA && p + 1 >= 0 && p + 1 < nch) build_inverse(sm, p + 1, xinit, lane);
      lds_barrier();
    }
  } else if (wave == W_PREFETCH) {
    // the L2 prefetch, issued by a wave that never waits for it
    lds_barrier();
    for (int64_t p = -2; p <= nch; ++p) {
      if constexpr (GLA) {
        constexpr int PA = PREFETCH_AHEAD + KQ_AHEAD<GLA> - 1;
        if (p + PA < nch) {
          prefetch_keys(sq, p + PA, slice, lane);
          prefetch_rest(sq, p + PA, slice, DV, lane);
        }
      } else {
        if (p + 5 < nch) prefetch_keys(sq, p + 5, slice, lane);
        if (p + 3 < nch) prefetch_rest(sq, p + 3, slice, DV, lane, OUT);
      }
      lds_barrier_keep_dma();
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no LDS-DMA write outlives the workgroup
  }
}

}  // namespace pipe
}  // namespace gdn
