// Host side of libgdn.so: argument validation, dispatch over the compiled
// instantiations and launch on the caller's stream.  The C ABI is declared in
// include/gdn.h.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "gdn.h"
#include "chunk_fwd_pipe.hpp"
#include "chunk_vec.hpp"
#include "recurrent_step.hpp"
#include "split_combine.hpp"
#include "scan_route.hpp"

namespace {

using gdn::bf16_t;

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

struct Range {
  const void* p;
  int64_t bytes;
};

// Size limits shared by every entry point: at most 2^31 - 1 sequences and
// tokens, and 2^48 token-sequences, so that byte counts (times d * 4 <= 2^9)
// stay far inside int64.
constexpr int64_t MAX_SEQS = 0x7fffffff, MAX_TOKENS = 0x7fffffff, MAX_SEQ_TOKENS = int64_t(1) << 48;
bool too_large(int64_t B, int64_t H, int64_t T) {
  if (B > MAX_SEQS || H > MAX_SEQS || T > MAX_TOKENS) return true;
  const int64_t n = B * H;  // < 2^62
  return n > MAX_SEQS || (T > 0 && n > MAX_SEQ_TOKENS / T);
}

// The pipelined bf16 kernel addresses one sequence's q, k, v and o through
// 32-bit buffer offsets: T * d * 2 bytes must stay under 2^31.
bool pipe_len_ok(int64_t T, int64_t dk, int64_t dv) {
  return T * dk * 2 <= 0x7fffffff && T * dv * 2 <= 0x7fffffff;
}

bool overlaps(Range a, Range b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

template <bool GLA = false>
int launch_chunk_pipe(const void* q, const void* k, const void* v, const float* alpha,
                      const float* beta, const float* s0, void* o, float* sT,
                      const gdn::pipe::ChainMap& cm, int64_t dk, int64_t dv, hipStream_t stream) {
  const int64_t nchain = gdn::pipe::map_chains(cm);
  const int64_t nblocks = nchain * (dv / gdn::pipe::DVS);
  if (nblocks > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  // one sequence's q, k or v must fit a 32-bit buffer range
  if (cm.T * dk * 2 > 0x7fffffff || cm.T * dv * 2 > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  const int xcd_map = (nchain % 8) == 0;
  // the first launch of the sequence split needs no output; with dk = 64
  // the products over the zero keys 64..127 are skipped (two key blocks)
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)nblocks), dim3(64 * gdn::pipe::NWAVES), 0, stream,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                       alpha, beta, s0, static_cast<bf16_t*>(o), sT, cm, (int)dv, (int)dk, xcd_map);
  };
  const bool no_out = !GLA && cm.mode == gdn::pipe::MAP_SPLIT_A;
  if (dk == 64) {
    if (no_out) launch(gdn::pipe::chunk_fwd_pipe_kernel<false, false, 2>);
    else launch(gdn::pipe::chunk_fwd_pipe_kernel<GLA, true, 2>);
  } else {
    if (no_out) launch(gdn::pipe::chunk_fwd_pipe_kernel<false, false, 4>);
    else launch(gdn::pipe::chunk_fwd_pipe_kernel<GLA, true, 4>);
  }
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn::pipe::ChainMap seq_map(int64_t nchain, int64_t T) {
  gdn::pipe::ChainMap cm{};
  cm.mode = gdn::pipe::MAP_SEQ;
  cm.nseq = (int)nchain;
  cm.G = 1;
  cm.T = T;
  cm.L = T;
  cm.ws = nullptr;
  return cm;
}

// Segments for the sequence-split pass: G segments of L tokens (a multiple of
// the chunk size; the last one shorter), chosen so that its first launch
// (2 (G-1) chains per sequence) still fits the device's CUs in one wave of
// workgroups and every segment has at least MIN_SEG tokens.  G = 1 means no
// split.  So does a plan of two segments: its first and last launches then
// run T/2 tokens each, one after the other, which is the plain pass's T
// tokens plus the extra launches.  Three segments take 2T/3.
constexpr int64_t MIN_SEG = 512;
void split_plan(int64_t nseq, int64_t T, int64_t dv, int& G, int64_t& L) {
  G = 1;
  L = T;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) {
    (void)hipGetLastError();
    return;
  }
  const int64_t ns = dv / gdn::pipe::DVS;
  int64_t g = 1 + ncu / (2 * nseq * ns);
  g = g < T / MIN_SEG ? g : T / MIN_SEG;
  if (g < 3) return;
  const int64_t C = gdn::pipe::C;
  L = ((T + g - 1) / g + C - 1) / C * C;
  G = (int)((T + L - 1) / L);
  if (G < 3) {
    G = 1;
    L = T;
  }
}

// Blocks of the scan route: L tokens (a multiple of the staging tile), about
// sqrt(32 T), which balances the per-block token loops (length L) against
// the sequential chain of block maps (length T / L).
void scan_plan(int64_t T, int& G, int64_t& L) {
  const int64_t tile = gdn::scan::TILE;
  int64_t l = 1;
  while (l * l < 32 * T) l *= 2;
  L = (l + tile - 1) / tile * tile;
  G = T > 0 ? (int)((T + L - 1) / L) : 1;
}
size_t scan_ws_bytes(int64_t nseq, int G, int64_t d) {
  return (size_t)(2 * nseq * (G - 1) + nseq * G) * (size_t)(d * d) * sizeof(float);
}

template <class E, int D, bool VEC>
int launch_scan(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                const float* s0, void* o, float* sT, int64_t nseq, int64_t T, float* ws, hipStream_t stream) {
  int G;
  int64_t L;
  scan_plan(T, G, L);
  using namespace gdn::scan;
  const E* qq = static_cast<const E*>(q);
  const E* kk = static_cast<const E*>(k);
  const E* vv = static_cast<const E*>(v);
  E* oo = static_cast<E*>(o);
  if (G > 1) {
    const int64_t nb = scan_blocks(SCAN_AGG, (int)nseq, G, D);
    if (nb > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((scan_tokens_kernel<E, D, VEC>), dim3((unsigned)nb), dim3(THREADS), 0, stream, qq, kk,
                       vv, alpha, beta, oo, sT, (int)SCAN_AGG, (int)nseq, G, T, L, ws);
    if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;
  }
  hipLaunchKernelGGL(gdn::split::split_combine_kernel<D>, dim3((unsigned)(nseq * (D / gdn::split::ROWS))),
                     dim3(gdn::split::threads_for<D>()), 0, stream, s0, ws, (int)nseq, G);
  if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;
  const int64_t nb = scan_blocks(SCAN_OUT, (int)nseq, G, D);
  if (nb > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((scan_tokens_kernel<E, D, VEC>), dim3((unsigned)nb), dim3(THREADS), 0, stream, qq, kk, vv,
                     alpha, beta, oo, sT, (int)SCAN_OUT, (int)nseq, G, T, L, ws);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t split_ws_bytes(int64_t nseq, int G, int64_t d) {
  return G < 2 ? 0 : (size_t)(2 * nseq * (G - 1) + nseq * G) * (size_t)(d * d) * sizeof(float);
}

template <class E, int DK, int DV, int GATE>
int launch_step(const void* q, const void* k, const void* v, const float* alpha,
                const float* beta, float* state, void* o, int64_t nheads, hipStream_t stream) {
  if (nheads > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  constexpr int NT = DK == 128 ? 512 : 256;
  hipLaunchKernelGGL((gdn::recurrent_step_kernel<E, DK, DV, NT, GATE>), dim3((unsigned)nheads), dim3(NT), 0,
                     stream, static_cast<const E*>(q), static_cast<const E*>(k),
                     static_cast<const E*>(v), alpha, beta, state, static_cast<E*>(o), nheads);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace

extern "C" {

const char* gdn_strerror(int code) {
  switch (code) {
    case GDN_OK: return "success";
    case GDN_ERR_INVALID_ARG: return "invalid argument (NULL pointer, negative size, bad dtype or overlapping output)";
    case GDN_ERR_UNSUPPORTED: return "unsupported shape or chunk size (dk == dv in {64,128}; chunk_size 64, or 32 where documented)";
    case GDN_ERR_ALIGNMENT: return "tensor pointer not 16-byte aligned";
    case GDN_ERR_HIP: return "HIP runtime error while launching";
    default: return "unknown gdn error code";
  }
}

const char* gdn_version(void) { return "0.1.0"; }

}  // extern "C"

namespace {
// Argument checks shared by the forward entry points: GDN_OK, or the error.
int check_fwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
              const float* initial_state, void* o, float* final_state, int64_t B, int64_t H,
              int64_t T, int64_t dk, int64_t dv, int64_t chunk_size, gdn_dtype dtype,
              bool alpha_per_dim = false) {
  if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0 || chunk_size <= 0) return GDN_ERR_INVALID_ARG;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (too_large(B, H, T)) return GDN_ERR_UNSUPPORTED;
  const int64_t nchain = B * H;
  const bool has_tokens = nchain > 0 && T > 0;
  if (has_tokens && (!q || !k || !v || !alpha || !beta || !o)) return GDN_ERR_INVALID_ARG;
  if (dk != dv || (dk != 64 && dk != 128) || chunk_size != 64) return GDN_ERR_UNSUPPORTED;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(alpha) || misaligned(beta) ||
      misaligned(initial_state) || misaligned(o) || misaligned(final_state))
    return GDN_ERR_ALIGNMENT;
  const int64_t esz = dtype == GDN_BF16 ? 2 : 4;
  if (has_tokens) {
    const Range ro{o, nchain * T * dv * esz};
    const Range ins[] = {{q, nchain * T * dk * esz}, {k, nchain * T * dk * esz},
                         {v, nchain * T * dv * esz}, {alpha, nchain * T * (alpha_per_dim ? dk : 1) * 4},
                         {beta, nchain * T * 4},     {initial_state, nchain * dv * dk * 4},
                         {final_state, nchain * dv * dk * 4}};
    for (const Range& r : ins)
      if (overlaps(ro, r)) return GDN_ERR_INVALID_ARG;
  }
  if (nchain > 0 && final_state) {
    // The final state is written while other workgroups still read the
    // inputs: it must be disjoint from them, and from the initial state
    // unless it is that very state (each workgroup reads its part first).
    const Range rs{final_state, nchain * dv * dk * 4};
    const Range ins[] = {{q, nchain * T * dk * esz},
                         {k, nchain * T * dk * esz},
                         {v, nchain * T * dv * esz},
                         {alpha, nchain * T * (alpha_per_dim ? dk : 1) * 4},
                         {beta, nchain * T * 4}};
    for (const Range& r : ins)
      if (overlaps(rs, r)) return GDN_ERR_INVALID_ARG;
    if (initial_state != final_state && overlaps(rs, Range{initial_state, nchain * dv * dk * 4}))
      return GDN_ERR_INVALID_ARG;
  }
  return GDN_OK;
}
}  // namespace

namespace {
// The three launches of the sequence-split pass on workspace ws (G >= 2).
int split_launches(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                   const float* initial_state, void* o, float* final_state, int64_t nchain, int64_t T,
                   int64_t dk, int64_t dv, int G, int64_t L, float* ws, hipStream_t stream) {
  gdn::pipe::ChainMap cm{};
  cm.nseq = (int)nchain;
  cm.G = G;
  cm.T = T;
  cm.L = L;
  cm.ws = ws;
  // 1: per segment, the state from zero and the transition (first G-1 segments)
  cm.mode = gdn::pipe::MAP_SPLIT_A;
  int r = launch_chunk_pipe(q, k, v, alpha, beta, nullptr, o, nullptr, cm, dk, dv, stream);
  if (r != GDN_OK) return r;
  // 2: the start state of every segment
  if (dk == 128)
    hipLaunchKernelGGL(gdn::split::split_combine_kernel<128>, dim3((unsigned)(nchain * (128 / gdn::split::ROWS))),
                       dim3(gdn::split::threads_for<128>()), 0, stream, initial_state, cm.ws, (int)nchain, G);
  else
    hipLaunchKernelGGL(gdn::split::split_combine_kernel<64>, dim3((unsigned)(nchain * (64 / gdn::split::ROWS))),
                       dim3(gdn::split::threads_for<64>()), 0, stream, initial_state, cm.ws, (int)nchain, G);
  if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;
  // 3: every segment from its start state, with output
  cm.mode = gdn::pipe::MAP_SPLIT_C;
  return launch_chunk_pipe(q, k, v, alpha, beta, nullptr, o, final_state, cm, dk, dv, stream);
}

// Scratch of gdn_chunk_fwd_split_noalloc: one copy in the memory of every
// device the library runs on, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host it is only a stand-in for
// the symbol): the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress and kept in noalloc_ptr.
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[NOALLOC_MAX_DEVICES] = {};
}  // namespace

static __device__ __align__(256) unsigned char scratch[GDN_SPLIT_NOALLOC_SCRATCH_BYTES];

namespace {
// Device address of the current device's scratch (looked up on the first call
// on that device, with that device current).
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return GDN_ERR_HIP;
  }
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return GDN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (!noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return GDN_ERR_HIP;
    }
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return GDN_OK;
}
}  // namespace

namespace {
// The 32-token chunk kernel of chunk_vec.hpp: the per-dimension gate (VG),
// and the scalar gate for fp32 inputs and for a requested chunk size of 32.
// vec_dispatch calls f(T{}, DK) with the element type and key width of the
// instantiation that serves dtype, dk.
template <bool VG, class F>
int vec_dispatch(gdn_dtype dtype, int64_t dk, F&& f) {
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (dtype == GDN_F32) return dk == 128 ? f(float{}, D128{}) : f(float{}, D64{});
  return dk == 128 ? f(bf16_t{}, D128{}) : f(bf16_t{}, D64{});
}

template <bool VG, class T, int DK, bool GLA = false>
int launch_vec_t(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                 const float* initial_state, void* o, float* final_state, const gdn::pipe::ChainMap& cm,
                 int64_t dv, hipStream_t stream) {
  const int64_t nchain = gdn::pipe::map_chains(cm);
  const int64_t nblocks = nchain * (dv / gdn::vec::DVS);
  if (nblocks > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  const int xcd_map = (nchain % 8) == 0;
  hipLaunchKernelGGL((gdn::vec::chunk_vec_kernel<T, DK, VG, false, GLA>), dim3((unsigned)nblocks), dim3(gdn::vec::NT), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), alpha,
                     beta, initial_state, static_cast<T*>(o), final_state, cm, (int)dv, xcd_map);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}
template <bool VG, bool GLA = false>
int launch_vec(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
               const float* initial_state, void* o, float* final_state, const gdn::pipe::ChainMap& cm,
               int64_t dk, int64_t dv, gdn_dtype dtype, hipStream_t stream) {
  return vec_dispatch<VG>(dtype, dk, [&](auto t, auto dkc) {
    return launch_vec_t<VG, decltype(t), decltype(dkc)::value, GLA>(q, k, v, alpha, beta, initial_state, o,
                                                                    final_state, cm, dv, stream);
  });
}

// Segments of the vector-gate split: as split_plan, but the first launch
// may hold as many workgroups as the kernel's occupancy puts on the device
// at once (two per CU at d = 64 in bf16, one otherwise), and segments are
// multiples of the 32-token chunk.
template <bool VG>
void vec_split_plan(int64_t nseq, int64_t T, int64_t dk, int64_t dv, gdn_dtype dtype, int& G, int64_t& L) {
  G = 1;
  L = T;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) {
    (void)hipGetLastError();
    return;
  }
  const int per_cu = vec_dispatch<VG>(dtype, dk, [&](auto t, auto dkc) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(&gdn::vec::chunk_vec_kernel<decltype(t), decltype(dkc)::value, VG>),
            gdn::vec::NT, 0) != hipSuccess) {
      (void)hipGetLastError();
      n = 1;
    }
    return n > 0 ? n : 1;
  });
  const int64_t ns = dv / gdn::vec::DVS;
  int64_t g = 1 + (int64_t)ncu * per_cu / (2 * nseq * ns);
  g = g < T / MIN_SEG ? g : T / MIN_SEG;
  if (g < 3) return;
  const int64_t C = gdn::vec::C;
  L = ((T + g - 1) / g + C - 1) / C * C;
  G = (int)((T + L - 1) / L);
  if (G < 3) {
    G = 1;
    L = T;
  }
}

// The combine step of a sequence split: the start state of every segment.
int launch_combine(int64_t dk, const float* initial_state, float* ws, int64_t nchain, int G, hipStream_t stream) {
  if (dk == 128)
    hipLaunchKernelGGL(gdn::split::split_combine_kernel<128>, dim3((unsigned)(nchain * (128 / gdn::split::ROWS))),
                       dim3(gdn::split::threads_for<128>()), 0, stream, initial_state, ws, (int)nchain, G);
  else
    hipLaunchKernelGGL(gdn::split::split_combine_kernel<64>, dim3((unsigned)(nchain * (64 / gdn::split::ROWS))),
                       dim3(gdn::split::threads_for<64>()), 0, stream, initial_state, ws, (int)nchain, G);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// The three launches of the vector-gate split on workspace ws (G >= 2).
int vec_split_launches(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                       const float* initial_state, void* o, float* final_state, int64_t nchain, int64_t T,
                       int64_t dk, int64_t dv, gdn_dtype dtype, int G, int64_t L, float* ws,
                       hipStream_t stream) {
  gdn::pipe::ChainMap cm{};
  cm.nseq = (int)nchain;
  cm.G = G;
  cm.T = T;
  cm.L = L;
  cm.ws = ws;
  cm.mode = gdn::pipe::MAP_SPLIT_A;
  int r = launch_vec<true>(q, k, v, alpha, beta, nullptr, o, nullptr, cm, dk, dv, dtype, stream);
  if (r != GDN_OK) return r;
  r = launch_combine(dk, initial_state, ws, nchain, G, stream);
  if (r != GDN_OK) return r;
  cm.mode = gdn::pipe::MAP_SPLIT_C;
  return launch_vec<true>(q, k, v, alpha, beta, nullptr, o, final_state, cm, dk, dv, dtype, stream);
}

// Two-pass per-dimension gate.  The workspace holds the state carried from
// one tile of chunks to the next (B*H*dk*dv floats), then the records of one
// tile (B*H*tile records).  A tile is at most VEC2P_TILE chunks per sequence
// (8192 tokens; the main workload's shape in one tile, 553 MB of records).
// Measured at that shape: tiles of 64, 128, 256 chunks took 0.542, 0.524 and
// 0.511 ms, longer tiles the same; at B=1, H=8, T=16384, d=64: 0.456, 0.411,
// 0.384 ms, and 0.373 ms for 512.
constexpr int64_t VEC2P_TILE = 256;

int64_t vec2p_rec_bytes(int64_t dk, gdn_dtype dtype) {
  return vec_dispatch<true>(dtype, dk, [](auto t, auto dkc) {
    return (int)gdn::vec::VecRec<decltype(t), decltype(dkc)::value>::BYTES;
  });
}

int device_cus() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return ncu;
}

// The first pass over chunks [c0, c0 + n) of every sequence: groups of
// consecutive chunks per sequence, about as many workgroups as the device
// holds at once (two per CU), each walking its chunks.
template <class T, int DK>
int vec2p_prep(const void* q, const void* k, const void* v, const float* alpha, const float* beta, void* o,
               int64_t nseq, int64_t Tseq, int64_t dv, char* rec, int64_t c0, int64_t n, int ncu,
               hipStream_t stream) {
  gdn::pipe::ChainMap cm{};
  cm.mode = gdn::vec::MAP_PREP;
  cm.nseq = (int)nseq;
  cm.G = (int)n;
  cm.T = Tseq;
  cm.L = c0 * gdn::vec::C;
  cm.ws = reinterpret_cast<float*>(rec);
  int64_t ng = ncu > 0 ? 2 * (int64_t)ncu / nseq : n;
  ng = ng < 1 ? 1 : ng > n ? n : ng;
  if (nseq * ng > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gdn::vec::chunk_vec_kernel<T, DK, true, true>), dim3((unsigned)(nseq * ng)),
                     dim3(gdn::vec::NT), 0, stream, static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), alpha, beta, nullptr, static_cast<T*>(o), nullptr, cm, (int)dv, 0);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// Resident workgroups per CU of a kernel at `threads` threads (0 when the
// runtime cannot tell).
int occupancy(const void* kern, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, threads, 0) != hipSuccess) {
    (void)hipGetLastError();
    n = 0;
  }
  return n;
}
// The pipelined second pass for bf16 records with SL value slices per
// workgroup (SL state waves and a loader wave).
template <int DK, int SL>
const void* vec_pipe_kernel() {
  return reinterpret_cast<const void*>(&gdn::vec::vec_state_pipe_kernel<DK, SL>);
}
template <int DK, int SL>
int vec_pipe_occupancy() {
  static const int n = occupancy(vec_pipe_kernel<DK, SL>(), 64 * (SL + 1));
  return n;
}
// Value slices per workgroup of the pipelined second pass over nchain chains
// of ns slices: the fewest (1, 2 or 4) with which every workgroup is resident
// at once; else 4, which shares each record among the most slices.
template <int DK>
int vec_pipe_slices(int64_t nchain, int64_t ns) {
  const int ncu = device_cus();
  if (ncu > 0) {
    if (nchain * ns <= (int64_t)vec_pipe_occupancy<DK, 1>() * ncu) return 1;
    if (ns % 2 == 0 && nchain * (ns / 2) <= (int64_t)vec_pipe_occupancy<DK, 2>() * ncu) return 2;
  }
  return ns % 4 == 0 ? 4 : ns % 2 == 0 ? 2 : 1;
}

// The second pass over the chains of cm (cm.nseq = the sequences): bf16
// records go to the pipelined kernel (its slices per workgroup chosen here),
// fp32 records to vec_state_kernel with sl value slices per workgroup.
template <class T, int DK>
int vec2p_state(int sl, const void* v, const char* rec, const float* in, void* o, float* out, int64_t nseq,
                int64_t Tseq, int64_t c0, int64_t n, int64_t dv, const gdn::pipe::ChainMap& cm,
                hipStream_t stream) {
  const int64_t nchain = gdn::pipe::map_chains(cm);
  const int xcd_map = (nchain % 8) == 0;
  if constexpr (std::is_same<T, bf16_t>::value) {
    const int64_t ns = dv / gdn::vec::DVS;
    const int spw = vec_pipe_slices<DK>(nchain, ns);
    const int64_t nblocks = nchain * (ns / spw);
    if (nblocks > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
    auto launch = [&](auto slc) {
      constexpr int S = decltype(slc)::value;
      hipLaunchKernelGGL((gdn::vec::vec_state_pipe_kernel<DK, S>), dim3((unsigned)nblocks), dim3(64 * (S + 1)), 0,
                         stream, static_cast<const bf16_t*>(v), rec, in, static_cast<bf16_t*>(o), out, (int)nseq,
                         Tseq, c0, (int)n, (int)dv, xcd_map, cm);
    };
    if (spw == 4)
      launch(std::integral_constant<int, 4>{});
    else if (spw == 2)
      launch(std::integral_constant<int, 2>{});
    else
      launch(std::integral_constant<int, 1>{});
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  }
  const int64_t nblocks = nchain * (dv / (gdn::vec::DVS * sl));
  if (nblocks > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  if (sl == 2)
    hipLaunchKernelGGL((gdn::vec::vec_state_kernel<T, DK, 2>), dim3((unsigned)nblocks), dim3(gdn::vec::NT * 2), 0,
                       stream, static_cast<const T*>(v), rec, in, static_cast<T*>(o), out, (int)nseq, Tseq, c0,
                       (int)n, (int)dv, xcd_map, cm);
  else
    hipLaunchKernelGGL((gdn::vec::vec_state_kernel<T, DK, 1>), dim3((unsigned)nblocks), dim3(gdn::vec::NT), 0,
                       stream, static_cast<const T*>(v), rec, in, static_cast<T*>(o), out, (int)nseq, Tseq, c0,
                       (int)n, (int)dv, xcd_map, cm);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// Sequence split of the two-pass route (few sequences: the second pass is a
// chain of T/32 chunks per workgroup): as for the single-pass split, the
// first G-1 segments from a zero start and from the identity (V read as
// zero), the combine step, then every segment from its start state.  The
// records of the whole sequences are written once by the first pass.  G is
// the largest value whose first launch fits the device at the second pass's
// occupancy, with segments of at least VEC2P_MIN_SEG tokens; below 3, no split.
constexpr int64_t VEC2P_MIN_SEG = 256;
void vec2p_split_plan(int64_t nseq, int64_t T, int64_t dk, int64_t dv, gdn_dtype dtype, int& G, int64_t& L) {
  G = 1;
  L = T;
  const int ncu = device_cus();
  if (ncu <= 0) return;
  const int per_cu = vec_dispatch<true>(dtype, dk, [&](auto t, auto dkc) {
    constexpr int DK = decltype(dkc)::value;
    // bf16: chains x slices resident at four slices per workgroup (the
    // second pass's slice count adapts to its launch)
    if constexpr (std::is_same<decltype(t), bf16_t>::value) return 4 * vec_pipe_occupancy<DK, 4>();
    return occupancy(reinterpret_cast<const void*>(&gdn::vec::vec_state_kernel<decltype(t), DK, 1>), gdn::vec::NT);
  });
  if (per_cu <= 0) return;
  const int64_t ns = dv / gdn::vec::DVS;
  int64_t g = 1 + (int64_t)per_cu * ncu / (2 * nseq * ns);
  g = g < T / VEC2P_MIN_SEG ? g : T / VEC2P_MIN_SEG;
  if (g < 3) return;
  const int64_t C = gdn::vec::C;
  L = ((T + g - 1) / g + C - 1) / C * C;
  G = (int)((T + L - 1) / L);
  if (G < 3) {
    G = 1;
    L = T;
  }
}

template <class T, int DK>
int vec2p_launches_t(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                     const float* initial_state, void* o, float* final_state, int64_t nseq, int64_t Tseq,
                     int64_t dv, char* ws, int64_t tile, int G, int64_t L, hipStream_t stream) {
  const int64_t nch = (Tseq + gdn::vec::C - 1) / gdn::vec::C;
  const int ncu = device_cus();
  if (G >= 3) {
    // split: ws = the split's states, then the records of every chunk
    float* sws = reinterpret_cast<float*>(ws);
    char* rec = ws + split_ws_bytes(nseq, G, DK);
    int r = vec2p_prep<T, DK>(q, k, v, alpha, beta, o, nseq, Tseq, dv, rec, 0, nch, ncu, stream);
    if (r != GDN_OK) return r;
    gdn::pipe::ChainMap cm{};
    cm.nseq = (int)nseq;
    cm.G = G;
    cm.T = Tseq;
    cm.L = L;
    cm.ws = sws;
    cm.mode = gdn::pipe::MAP_SPLIT_A;
    r = vec2p_state<T, DK>(1, v, rec, nullptr, o, nullptr, nseq, Tseq, 0, nch, dv, cm, stream);
    if (r != GDN_OK) return r;
    r = launch_combine(DK, initial_state, sws, nseq, G, stream);
    if (r != GDN_OK) return r;
    cm.mode = gdn::pipe::MAP_SPLIT_C;
    return vec2p_state<T, DK>(1, v, rec, nullptr, o, final_state, nseq, Tseq, 0, nch, dv, cm, stream);
  }
  // tiles: ws = the carried state, then the records of one tile.  Two value
  // slices per workgroup of the second pass (sharing the records in LDS) when
  // that still fills the device: at the main workload's shape 0.63 -> 0.55
  // ms; with fewer sequences one slice per workgroup is faster (B=1, H=8,
  // T=16384, d=64: 0.45 vs 0.55 ms).
  float* carry = reinterpret_cast<float*>(ws);
  char* rec = ws + nseq * DK * dv * 4;
  const int sl = ncu > 0 && nseq * (dv / gdn::vec::DVS) >= 2 * (int64_t)ncu ? 2 : 1;
  gdn::pipe::ChainMap cm{};
  cm.mode = gdn::pipe::MAP_SEQ;
  cm.nseq = (int)nseq;
  int64_t c0 = 0;
  do {
    const int64_t n = tile < nch - c0 ? tile : nch - c0;  // 0 when there are no chunks
    if (n > 0) {
      const int r = vec2p_prep<T, DK>(q, k, v, alpha, beta, o, nseq, Tseq, dv, rec, c0, n, ncu, stream);
      if (r != GDN_OK) return r;
    }
    const float* in = c0 == 0 ? initial_state : carry;
    float* out = c0 + n >= nch ? final_state : carry;
    const int r = vec2p_state<T, DK>(sl, v, rec, in, o, out, nseq, Tseq, c0, n, dv, cm, stream);
    if (r != GDN_OK) return r;
    c0 += n;
  } while (c0 < nch);
  return GDN_OK;
}

// Workspace of the two-pass route: with a split, the split's states and the
// records of whole sequences; else the carried state and one tile's records.
int64_t vec2p_split_bytes(int64_t nseq, int64_t T, int G, int64_t dk, gdn_dtype dtype) {
  const int64_t nch = (T + gdn::vec::C - 1) / gdn::vec::C;
  return (int64_t)split_ws_bytes(nseq, G, dk) + nseq * nch * vec2p_rec_bytes(dk, dtype);
}
}  // namespace

extern "C" {

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                  const float* beta, const float* initial_state, void* o, float* final_state,
                  int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk_size,
                  gdn_dtype dtype, void* hip_stream) {
  // chunk sizes: 64, and 32 (the 32-token kernel)
  const bool c32 = chunk_size == gdn::vec::C;
  const int rc = check_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                           c32 ? 64 : chunk_size, dtype);
  if (rc != GDN_OK) return rc;
  if (dtype == GDN_BF16 && !c32 && !pipe_len_ok(T, dk, dv)) return GDN_ERR_UNSUPPORTED;
  const int64_t nchain = B * H;
  if (nchain == 0) return GDN_OK;
  if (T == 0 && !final_state) return GDN_OK;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (dtype == GDN_BF16 && !c32)
    return launch_chunk_pipe(q, k, v, alpha, beta, initial_state, o, final_state, seq_map(nchain, T),
                             dk, dv, stream);
  // fp32 (at either chunk size: 64-token fp32 buffers exceed the LDS at
  // d = 128, and the result does not depend on the chunk size beyond
  // rounding) and chunk size 32: chunks of 32 tokens
  return launch_vec<false>(q, k, v, alpha, beta, initial_state, o, final_state, seq_map(nchain, T), dk, dv,
                           dtype, stream);
}

int gla_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                  const float* beta, const float* initial_state, void* o, float* final_state,
                  int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk_size,
                  gdn_dtype dtype, void* hip_stream) {
  // chunk sizes and dtypes as gdn_chunk_fwd: bf16 64-token chunks on the
  // pipelined kernel, fp32 and 32-token chunks on the 32-token kernel
  const bool c32 = chunk_size == gdn::vec::C;
  const int rc = check_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                           c32 ? 64 : chunk_size, dtype);
  if (rc != GDN_OK) return rc;
  if (dtype == GDN_BF16 && !c32 && !pipe_len_ok(T, dk, dv)) return GDN_ERR_UNSUPPORTED;
  const int64_t nchain = B * H;
  if (nchain == 0) return GDN_OK;
  if (T == 0 && !final_state) return GDN_OK;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (dtype == GDN_BF16 && !c32)
    return launch_chunk_pipe<true>(q, k, v, alpha, beta, initial_state, o, final_state, seq_map(nchain, T),
                                   dk, dv, stream);
  return launch_vec<false, true>(q, k, v, alpha, beta, initial_state, o, final_state, seq_map(nchain, T), dk,
                                 dv, dtype, stream);
}

size_t gdn_scan_fwd_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                              gdn_dtype dtype) {
  if (B <= 0 || H <= 0 || T < 0 || dk != dv || (dk != 64 && dk != 128) ||
      (dtype != GDN_F32 && dtype != GDN_BF16) || too_large(B, H, T))
    return 0;
  int G;
  int64_t L;
  scan_plan(T, G, L);
  return scan_ws_bytes(B * H, G, dk);
}

}  // extern "C"

namespace {
// The token-by-token forward pass: the scan route's replay kernel with one
// block per sequence (G = 1), starting from the initial state itself (or a
// zero state) and writing the final state; no workspace and no other launch.
constexpr int64_t SHORT_T = 64;  // up to this length, tiles of SHORT_TILE tokens
template <class E, int D, bool VEC>
int launch_recurrent(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                     const float* s0, void* o, float* sT, int64_t nseq, int64_t T, hipStream_t stream) {
  using namespace gdn::scan;
  const int64_t nb = scan_blocks(SCAN_OUT, (int)nseq, 1, D);
  if (nb > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  if (T <= SHORT_T)
    hipLaunchKernelGGL((scan_tokens_kernel<E, D, VEC, SHORT_TILE>), dim3((unsigned)nb), dim3(THREADS), 0, stream,
                       static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v), alpha, beta,
                       static_cast<E*>(o), sT, (int)SCAN_OUT, (int)nseq, 1, T, T, const_cast<float*>(s0));
  else
    hipLaunchKernelGGL((scan_tokens_kernel<E, D, VEC>), dim3((unsigned)nb), dim3(THREADS), 0, stream,
                       static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v), alpha, beta,
                       static_cast<E*>(o), sT, (int)SCAN_OUT, (int)nseq, 1, T, T, const_cast<float*>(s0));
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

template <bool VEC>
int recurrent_fwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                  const float* initial_state, void* o, float* final_state, int64_t B, int64_t H, int64_t T,
                  int64_t dk, int64_t dv, gdn_dtype dtype, void* hip_stream) {
  const int rc = check_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                           64, dtype, VEC);
  if (rc != GDN_OK) return rc;
  const int64_t nseq = B * H;
  if (nseq == 0 || (T == 0 && !final_state)) return GDN_OK;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (dtype == GDN_BF16)
    return dk == 128 ? launch_recurrent<bf16_t, 128, VEC>(q, k, v, alpha, beta, initial_state, o, final_state, nseq, T, stream)
                     : launch_recurrent<bf16_t, 64, VEC>(q, k, v, alpha, beta, initial_state, o, final_state, nseq, T, stream);
  return dk == 128 ? launch_recurrent<float, 128, VEC>(q, k, v, alpha, beta, initial_state, o, final_state, nseq, T, stream)
                   : launch_recurrent<float, 64, VEC>(q, k, v, alpha, beta, initial_state, o, final_state, nseq, T, stream);
}

template <bool VEC>
int scan_fwd(const void* q, const void* k, const void* v, const float* alpha, const float* beta,
             const float* initial_state, void* o, float* final_state, int64_t B, int64_t H, int64_t T,
             int64_t dk, int64_t dv, gdn_dtype dtype, void* workspace, size_t workspace_bytes,
             void* hip_stream) {
  const int rc = check_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                           64, dtype, VEC);
  if (rc != GDN_OK) return rc;
  const int64_t nseq = B * H;
  if (nseq == 0) return GDN_OK;
  if (T == 0 && !final_state) return GDN_OK;
  int G;
  int64_t L;
  scan_plan(T, G, L);
  const size_t need = scan_ws_bytes(nseq, G, dk);
  if (!workspace || workspace_bytes < need) return GDN_ERR_INVALID_ARG;
  if (misaligned(workspace)) return GDN_ERR_ALIGNMENT;
  {
    const int64_t esz = dtype == GDN_BF16 ? 2 : 4;
    const Range rw{workspace, (int64_t)need};
    const Range others[] = {{q, nseq * T * dk * esz}, {k, nseq * T * dk * esz},
                            {v, nseq * T * dv * esz}, {o, nseq * T * dv * esz},
                            {alpha, nseq * T * (VEC ? dk : 1) * 4}, {beta, nseq * T * 4},
                            {initial_state, nseq * dv * dk * 4}, {final_state, nseq * dv * dk * 4}};
    for (const Range& r : others)
      if (overlaps(rw, r)) return GDN_ERR_INVALID_ARG;
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  float* ws = static_cast<float*>(workspace);
  if (dtype == GDN_BF16)
    return dk == 128 ? launch_scan<bf16_t, 128, VEC>(q, k, v, alpha, beta, initial_state, o, final_state, nseq, T, ws, stream)
                     : launch_scan<bf16_t, 64, VEC>(q, k, v, alpha, beta, initial_state, o, final_state, nseq, T, ws, stream);
  return dk == 128 ? launch_scan<float, 128, VEC>(q, k, v, alpha, beta, initial_state, o, final_state, nseq, T, ws, stream)
                   : launch_scan<float, 64, VEC>(q, k, v, alpha, beta, initial_state, o, final_state, nseq, T, ws, stream);
}
}  // namespace

extern "C" {

int gdn_recurrent_fwd(const void* q, const void* k, const void* v, const float* alpha,
                      const float* beta, const float* initial_state, void* o, float* final_state,
                      int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, gdn_dtype dtype,
                      void* hip_stream) {
  return recurrent_fwd<false>(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv, dtype,
                              hip_stream);
}

int gdn_recurrent_fwd_vecgate(const void* q, const void* k, const void* v, const float* alpha,
                              const float* beta, const float* initial_state, void* o, float* final_state,
                              int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, gdn_dtype dtype,
                              void* hip_stream) {
  return recurrent_fwd<true>(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv, dtype,
                             hip_stream);
}

int gdn_scan_fwd(const void* q, const void* k, const void* v, const float* alpha,
                 const float* beta, const float* initial_state, void* o, float* final_state,
                 int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, gdn_dtype dtype,
                 void* workspace, size_t workspace_bytes, void* hip_stream) {
  return scan_fwd<false>(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv, dtype,
                         workspace, workspace_bytes, hip_stream);
}

int gdn_scan_fwd_vecgate(const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const float* initial_state, void* o, float* final_state,
                         int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, gdn_dtype dtype,
                         void* workspace, size_t workspace_bytes, void* hip_stream) {
  return scan_fwd<true>(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv, dtype,
                        workspace, workspace_bytes, hip_stream);
}

int gdn_chunk_fwd_vecgate(const void* q, const void* k, const void* v, const float* alpha,
                          const float* beta, const float* initial_state, void* o, float* final_state,
                          int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk_size,
                          gdn_dtype dtype, void* hip_stream) {
  // the shared checks with the scalar path's chunk size; this route's own below
  const int rc = check_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                           chunk_size > 0 ? 64 : chunk_size, dtype, true);
  if (rc != GDN_OK) return rc;
  if (chunk_size != gdn::vec::C) return GDN_ERR_UNSUPPORTED;
  const int64_t nchain = B * H;
  if (nchain == 0 || (T == 0 && !final_state)) return GDN_OK;
  return launch_vec<true>(q, k, v, alpha, beta, initial_state, o, final_state, seq_map(nchain, T), dk, dv, dtype,
                          static_cast<hipStream_t>(hip_stream));
}

size_t gdn_chunk_fwd_vecgate_2pass_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                             int64_t chunk_size, gdn_dtype dtype) {
  if (B <= 0 || H <= 0 || T < 0 || dk != dv || (dk != 64 && dk != 128) || chunk_size != gdn::vec::C ||
      (dtype != GDN_BF16 && dtype != GDN_F32) || too_large(B, H, T))
    return 0;
  const int64_t nch = (T + gdn::vec::C - 1) / gdn::vec::C;
  const int64_t tile = nch < VEC2P_TILE ? (nch > 0 ? nch : 1) : VEC2P_TILE;
  int64_t need = B * H * (dk * dv * 4 + tile * vec2p_rec_bytes(dk, dtype));
  int G = 1;
  int64_t L = T;
  if (T > 0) vec2p_split_plan(B * H, T, dk, dv, dtype, G, L);
  if (G >= 3) {
    const int64_t split = vec2p_split_bytes(B * H, T, G, dk, dtype);
    need = split > need ? split : need;
  }
  return (size_t)need;
}

int gdn_chunk_fwd_vecgate_2pass(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* initial_state, void* o, float* final_state,
                                int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk_size,
                                gdn_dtype dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  const int rc = check_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                           chunk_size > 0 ? 64 : chunk_size, dtype, true);
  if (rc != GDN_OK) return rc;
  if (chunk_size != gdn::vec::C) return GDN_ERR_UNSUPPORTED;
  const int64_t nseq = B * H;
  if (nseq == 0 || (T == 0 && !final_state)) return GDN_OK;
  const int64_t rec = vec2p_rec_bytes(dk, dtype);
  const int64_t carry = nseq * dk * dv * 4;
  const int64_t nch = (T + gdn::vec::C - 1) / gdn::vec::C;
  if (!workspace || (int64_t)workspace_bytes < carry + nseq * rec) return GDN_ERR_INVALID_ARG;
  if (misaligned(workspace)) return GDN_ERR_ALIGNMENT;
  // a split when planned and the workspace holds it, else tiles
  int G = 1;
  int64_t L = T;
  if (T > 0) vec2p_split_plan(nseq, T, dk, dv, dtype, G, L);
  int64_t used = 0, tile = 0;
  if (G >= 3 && vec2p_split_bytes(nseq, T, G, dk, dtype) <= (int64_t)workspace_bytes) {
    used = vec2p_split_bytes(nseq, T, G, dk, dtype);
  } else {
    G = 1;
    tile = ((int64_t)workspace_bytes - carry) / (nseq * rec);
    if (tile > VEC2P_TILE) tile = VEC2P_TILE;
    if (tile > nch) tile = nch;
    used = carry + (tile > 0 ? tile : 1) * nseq * rec;
  }
  {
    const Range rw{workspace, used};
    const int64_t esz = dtype == GDN_BF16 ? 2 : 4;
    const Range others[] = {{q, nseq * T * dk * esz}, {k, nseq * T * dk * esz},
                            {v, nseq * T * dv * esz}, {o, nseq * T * dv * esz},
                            {alpha, nseq * T * dk * 4}, {beta, nseq * T * 4},
                            {initial_state, nseq * dv * dk * 4}, {final_state, nseq * dv * dk * 4}};
    for (const Range& r : others)
      if (overlaps(rw, r)) return GDN_ERR_INVALID_ARG;
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  return vec_dispatch<true>(dtype, dk, [&](auto t, auto dkc) {
    return vec2p_launches_t<decltype(t), decltype(dkc)::value>(q, k, v, alpha, beta, initial_state, o, final_state,
                                                              nseq, T, dv, ws, tile, G, L, stream);
  });
}

size_t gdn_chunk_fwd_vecgate_split_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                             int64_t chunk_size, gdn_dtype dtype) {
  if (B <= 0 || H <= 0 || T <= 0 || dk != dv || (dk != 64 && dk != 128) || chunk_size != gdn::vec::C ||
      (dtype != GDN_BF16 && dtype != GDN_F32) || too_large(B, H, T))
    return 0;
  int G;
  int64_t L;
  vec_split_plan<true>(B * H, T, dk, dv, dtype, G, L);
  return split_ws_bytes(B * H, G, dk);
}

int gdn_chunk_fwd_vecgate_split(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* initial_state, void* o, float* final_state,
                                int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk_size,
                                gdn_dtype dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  const int rc = check_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                           chunk_size > 0 ? 64 : chunk_size, dtype, true);
  if (rc != GDN_OK) return rc;
  if (chunk_size != gdn::vec::C) return GDN_ERR_UNSUPPORTED;
  const int64_t nchain = B * H;
  int G = 1;
  int64_t L = T;
  if (nchain > 0 && T > 0) vec_split_plan<true>(nchain, T, dk, dv, dtype, G, L);
  if (G < 2)
    return gdn_chunk_fwd_vecgate(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv, chunk_size,
                                 dtype, hip_stream);
  const size_t need = split_ws_bytes(nchain, G, dk);
  if (!workspace || workspace_bytes < need) return GDN_ERR_INVALID_ARG;
  if (misaligned(workspace)) return GDN_ERR_ALIGNMENT;
  {
    const Range rw{workspace, (int64_t)need};
    const int64_t esz = dtype == GDN_BF16 ? 2 : 4;
    const Range others[] = {{q, nchain * T * dk * esz}, {k, nchain * T * dk * esz},
                            {v, nchain * T * dv * esz}, {o, nchain * T * dv * esz},
                            {alpha, nchain * T * dk * 4}, {beta, nchain * T * 4},
                            {initial_state, nchain * dv * dk * 4}, {final_state, nchain * dv * dk * 4}};
    for (const Range& r : others)
      if (overlaps(rw, r)) return GDN_ERR_INVALID_ARG;
  }
  return vec_split_launches(q, k, v, alpha, beta, initial_state, o, final_state, nchain, T, dk, dv, dtype, G, L,
                            static_cast<float*>(workspace), static_cast<hipStream_t>(hip_stream));
}

size_t gdn_chunk_fwd_split_workspace(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                                     int64_t chunk_size, gdn_dtype dtype) {
  if (B <= 0 || H <= 0 || T <= 0 || dk != dv || (dk != 64 && dk != 128) || chunk_size != 64 ||
      dtype != GDN_BF16 || too_large(B, H, T) || !pipe_len_ok(T, dk, dv))
    return 0;
  int G;
  int64_t L;
  split_plan(B * H, T, dv, G, L);
  return split_ws_bytes(B * H, G, dk);
}

int gdn_chunk_fwd_split(const void* q, const void* k, const void* v, const float* alpha,
                        const float* beta, const float* initial_state, void* o, float* final_state,
                        int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk_size,
                        gdn_dtype dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  const int rc = check_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                           chunk_size, dtype);
  if (rc != GDN_OK) return rc;
  if (dtype == GDN_BF16 && !pipe_len_ok(T, dk, dv)) return GDN_ERR_UNSUPPORTED;
  const int64_t nchain = B * H;
  int G = 1;
  int64_t L = T;
  if (dtype == GDN_BF16 && nchain > 0 && T > 0) split_plan(nchain, T, dv, G, L);
  if (G < 2)
    return gdn_chunk_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                         chunk_size, dtype, hip_stream);
  const size_t need = split_ws_bytes(nchain, G, dk);
  if (!workspace || workspace_bytes < need) return GDN_ERR_INVALID_ARG;
  if (misaligned(workspace)) return GDN_ERR_ALIGNMENT;
  {
    const Range rw{workspace, (int64_t)need};
    const int64_t esz = 2;
    const Range others[] = {{q, nchain * T * dk * esz}, {k, nchain * T * dk * esz},
                            {v, nchain * T * dv * esz}, {o, nchain * T * dv * esz},
                            {alpha, nchain * T * 4},    {beta, nchain * T * 4},
                            {initial_state, nchain * dv * dk * 4}, {final_state, nchain * dv * dk * 4}};
    for (const Range& r : others)
      if (overlaps(rw, r)) return GDN_ERR_INVALID_ARG;
  }
  return split_launches(q, k, v, alpha, beta, initial_state, o, final_state, nchain, T, dk, dv, G, L,
                        static_cast<float*>(workspace), static_cast<hipStream_t>(hip_stream));
}

int gdn_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* initial_state, void* o, float* final_state,
                                int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk_size,
                                gdn_dtype dtype, void* hip_stream) {
  const int rc = check_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                           chunk_size, dtype);
  if (rc != GDN_OK) return rc;
  if (dtype == GDN_BF16 && !pipe_len_ok(T, dk, dv)) return GDN_ERR_UNSUPPORTED;
  const int64_t nchain = B * H;
  int G = 1;
  int64_t L = T;
  if (dtype == GDN_BF16 && nchain > 0 && T > 0) split_plan(nchain, T, dv, G, L);
  if (G < 2)
    return gdn_chunk_fwd(q, k, v, alpha, beta, initial_state, o, final_state, B, H, T, dk, dv,
                         chunk_size, dtype, hip_stream);
  if (split_ws_bytes(nchain, G, dk) > GDN_SPLIT_NOALLOC_SCRATCH_BYTES) return GDN_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const int r = noalloc_scratch(&ws);
  if (r != GDN_OK) return r;
  return split_launches(q, k, v, alpha, beta, initial_state, o, final_state, nchain, T, dk, dv, G, L,
                        static_cast<float*>(ws), static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"

namespace {

// The decode steps share validation and dispatch; a per-dimension gate has
// dk entries per head, a scalar gate one.
template <int GATE>
int step_entry(const void* q, const void* k, const void* v, const float* alpha,
               const float* beta, float* state, void* o, int64_t N, int64_t H,
               int64_t dk, int64_t dv, gdn_dtype dtype, void* hip_stream) {
  if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_INVALID_ARG;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (too_large(N, H, 0)) return GDN_ERR_UNSUPPORTED;
  const int64_t nheads = N * H;
  if (nheads > 0 && (!q || !k || !v || !alpha || !beta || !state || !o)) return GDN_ERR_INVALID_ARG;
  if (dk != dv || (dk != 64 && dk != 128)) return GDN_ERR_UNSUPPORTED;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(alpha) || misaligned(beta) ||
      misaligned(state) || misaligned(o))
    return GDN_ERR_ALIGNMENT;
  const int64_t esz = dtype == GDN_BF16 ? 2 : 4;
  const int64_t gate_entries = GATE == gdn::STEP_VEC ? dk : 1;
  if (nheads > 0) {
    const Range ro{o, nheads * dv * esz};
    const Range ins[] = {{q, nheads * dk * esz},        {k, nheads * dk * esz}, {v, nheads * dv * esz},
                         {alpha, nheads * gate_entries * 4}, {beta, nheads * 4},
                         {state, nheads * dv * dk * 4}};
    for (const Range& r : ins)
      if (overlaps(ro, r)) return GDN_ERR_INVALID_ARG;
    // the state is rewritten in place while other heads read the token inputs
    const Range rs{state, nheads * dv * dk * 4};
    for (int i = 0; i < 5; ++i)
      if (overlaps(rs, ins[i])) return GDN_ERR_INVALID_ARG;
  }
  if (nheads == 0) return GDN_OK;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (dtype == GDN_BF16) {
    if (dk == 128) return launch_step<bf16_t, 128, 128, GATE>(q, k, v, alpha, beta, state, o, nheads, stream);
    return launch_step<bf16_t, 64, 64, GATE>(q, k, v, alpha, beta, state, o, nheads, stream);
  }
  if (dk == 128) return launch_step<float, 128, 128, GATE>(q, k, v, alpha, beta, state, o, nheads, stream);
  return launch_step<float, 64, 64, GATE>(q, k, v, alpha, beta, state, o, nheads, stream);
}

}  // namespace

extern "C" {

int gdn_recurrent_step(const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, float* state, void* o, int64_t N, int64_t H,
                       int64_t dk, int64_t dv, gdn_dtype dtype, void* hip_stream) {
  return step_entry<gdn::STEP_SCALAR>(q, k, v, alpha, beta, state, o, N, H, dk, dv, dtype, hip_stream);
}

int gdn_recurrent_step_vecgate(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, float* state, void* o, int64_t N, int64_t H,
                               int64_t dk, int64_t dv, gdn_dtype dtype, void* hip_stream) {
  return step_entry<gdn::STEP_VEC>(q, k, v, alpha, beta, state, o, N, H, dk, dv, dtype, hip_stream);
}

int gla_recurrent_step(const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, float* state, void* o, int64_t N, int64_t H,
                       int64_t dk, int64_t dv, gdn_dtype dtype, void* hip_stream) {
  return step_entry<gdn::STEP_GLA>(q, k, v, alpha, beta, state, o, N, H, dk, dv, dtype, hip_stream);
}

}  // extern "C"
