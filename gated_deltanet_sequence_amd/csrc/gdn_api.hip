// Host side of libgdn.so: argument validation, dispatch over the compiled
// instantiations and launch on the caller's stream.  The C ABI is declared in
// include/gdn.h.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "chunk_fwd.hpp"
#include "chunk_fwd_pipe.hpp"
#include "recurrent_step.hpp"

namespace {

using gdn::bf16_t;

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

struct Range {
  const void* p;
  int64_t bytes;
};

bool overlaps(Range a, Range b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

template <class E, int DK, int DVS, int C, int NW>
int launch_chunk(const void* q, const void* k, const void* v, const float* alpha,
                 const float* beta, const float* s0, void* o, float* sT, int64_t nchain,
                 int64_t T, int64_t dv, hipStream_t stream) {
  const int ns = (int)(dv / DVS);
  const int64_t nblocks = nchain * ns;
  if (nblocks > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  const int xcd_map = (nchain % 8) == 0;
  hipLaunchKernelGGL((gdn::chunk_fwd_kernel<E, DK, DVS, C, NW>), dim3((unsigned)nblocks),
                     dim3(NW * 64), 0, stream, static_cast<const E*>(q), static_cast<const E*>(k),
                     static_cast<const E*>(v), alpha, beta, s0, static_cast<E*>(o), sT,
                     (int)nchain, T, (int)dv, xcd_map);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int launch_chunk_pipe(const void* q, const void* k, const void* v, const float* alpha,
                      const float* beta, const float* s0, void* o, float* sT, int64_t nchain,
                      int64_t T, int64_t dk, int64_t dv, hipStream_t stream) {
  const int64_t nblocks = nchain * (dv / gdn::pipe::DVS);
  if (nblocks > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  // one sequence's q, k or v must fit a 32-bit buffer range
  if (T * dk * 2 > 0x7fffffff || T * dv * 2 > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  const int xcd_map = (nchain % 8) == 0;
  hipLaunchKernelGGL(gdn::pipe::chunk_fwd_pipe_kernel, dim3((unsigned)nblocks), dim3(64 * gdn::pipe::NWAVES), 0,
                     stream, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), alpha, beta, s0, static_cast<bf16_t*>(o), sT,
                     (int)nchain, T, (int)dv, (int)dk, xcd_map);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

template <class E, int DK, int DV>
int launch_step(const void* q, const void* k, const void* v, const float* alpha,
                const float* beta, float* state, void* o, int64_t nheads, hipStream_t stream) {
  if (nheads > 0x7fffffff) return GDN_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gdn::recurrent_step_kernel<E, DK, DV>), dim3((unsigned)nheads), dim3(256), 0,
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
    case GDN_ERR_UNSUPPORTED: return "unsupported shape or chunk size (dk == dv in {64,128}, chunk_size 64; fp32 needs dk == 64)";
    case GDN_ERR_ALIGNMENT: return "tensor pointer not 16-byte aligned";
    case GDN_ERR_HIP: return "HIP runtime error while launching";
    default: return "unknown gdn error code";
  }
}

const char* gdn_version(void) { return "0.1.0"; }

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                  const float* beta, const float* initial_state, void* o, float* final_state,
                  int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, int64_t chunk_size,
                  gdn_dtype dtype, void* hip_stream) {
  if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0 || chunk_size <= 0) return GDN_ERR_INVALID_ARG;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  const int64_t nchain = B * H;
  const bool has_tokens = nchain > 0 && T > 0;
  if (has_tokens && (!q || !k || !v || !alpha || !beta || !o)) return GDN_ERR_INVALID_ARG;
  if (dk != dv || (dk != 64 && dk != 128) || chunk_size != 64) return GDN_ERR_UNSUPPORTED;
  if (dtype == GDN_F32 && dk != 64) return GDN_ERR_UNSUPPORTED;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(alpha) || misaligned(beta) ||
      misaligned(initial_state) || misaligned(o) || misaligned(final_state))
    return GDN_ERR_ALIGNMENT;
  const int64_t esz = dtype == GDN_BF16 ? 2 : 4;
  if (has_tokens) {
    const Range ro{o, nchain * T * dv * esz};
    const Range ins[] = {{q, nchain * T * dk * esz}, {k, nchain * T * dk * esz},
                         {v, nchain * T * dv * esz}, {alpha, nchain * T * 4},
                         {beta, nchain * T * 4},     {initial_state, nchain * dv * dk * 4},
                         {final_state, nchain * dv * dk * 4}};
    for (const Range& r : ins)
      if (overlaps(ro, r)) return GDN_ERR_INVALID_ARG;
  }
  if (nchain == 0) return GDN_OK;
  if (T == 0 && !final_state) return GDN_OK;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (dtype == GDN_BF16)
    return launch_chunk_pipe(q, k, v, alpha, beta, initial_state, o, final_state, nchain, T, dk, dv,
                             stream);
  return launch_chunk<float, 64, 16, 64, 4>(q, k, v, alpha, beta, initial_state, o, final_state,
                                            nchain, T, dv, stream);
}

int gdn_recurrent_step(const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, float* state, void* o, int64_t N, int64_t H,
                       int64_t dk, int64_t dv, gdn_dtype dtype, void* hip_stream) {
  if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_INVALID_ARG;
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  const int64_t nheads = N * H;
  if (nheads > 0 && (!q || !k || !v || !alpha || !beta || !state || !o)) return GDN_ERR_INVALID_ARG;
  if (dk != dv || (dk != 64 && dk != 128)) return GDN_ERR_UNSUPPORTED;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(alpha) || misaligned(beta) ||
      misaligned(state) || misaligned(o))
    return GDN_ERR_ALIGNMENT;
  const int64_t esz = dtype == GDN_BF16 ? 2 : 4;
  if (nheads > 0) {
    const Range ro{o, nheads * dv * esz};
    const Range ins[] = {{q, nheads * dk * esz}, {k, nheads * dk * esz}, {v, nheads * dv * esz},
                         {alpha, nheads * 4},    {beta, nheads * 4},     {state, nheads * dv * dk * 4}};
    for (const Range& r : ins)
      if (overlaps(ro, r)) return GDN_ERR_INVALID_ARG;
  }
  if (nheads == 0) return GDN_OK;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (dtype == GDN_BF16) {
    if (dk == 128) return launch_step<bf16_t, 128, 128>(q, k, v, alpha, beta, state, o, nheads, stream);
    return launch_step<bf16_t, 64, 64>(q, k, v, alpha, beta, state, o, nheads, stream);
  }
  if (dk == 128) return launch_step<float, 128, 128>(q, k, v, alpha, beta, state, o, nheads, stream);
  return launch_step<float, 64, 64>(q, k, v, alpha, beta, state, o, nheads, stream);
}

}  // extern "C"
