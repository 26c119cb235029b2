// Device helpers shared by the gated-delta-rule kernels (gfx950 / CDNA4).
//
// bf16 is kept as raw uint16_t storage; MFMA operands are reinterpreted as
// the compiler's __bf16 vectors.  Matrix products use the gfx950 MFMA
// instructions on 16x16 output tiles:
//   bf16: v_mfma_f32_16x16x32_bf16 (8 k-values per lane), or the 16x16x16
//         variant (4 k-values per lane) when a product's depth is 16;
//   fp32: v_mfma_f32_16x16x4_f32 (1 k-value per lane).
// Lane l (of 64) supplies row (l % 16) of A and column (l % 16) of B at the
// k-slice chosen by l / 16, and receives rows 4*(l/16) .. 4*(l/16)+3 of
// column (l % 16) of the 16x16 fp32 result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Lower bound applied to log2(alpha): a gate of 0 then gives decay factors
// that are 0 in fp32 without turning differences of prefix sums into NaN.
constexpr float LOG2_ALPHA_MIN = -200.f;

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 values -> packed bf16 pair (low half = a), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
// Native base-2 exponential / logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Debug build (GDN_POISON_LDS=1, libgdn_debug.so): every kernel first fills
// its LDS with a NaN pattern (0x7fc0 as bf16, 0x7fc07fc0 as fp32), before
// its own initialisation, so that a read of LDS that nothing wrote shows up
// as NaN in the results.  The release build compiles the fills away.
#ifndef GDN_POISON_LDS
#define GDN_POISON_LDS 0
#endif
constexpr bool POISON_LDS = GDN_POISON_LDS != 0;
template <class T>
__device__ __forceinline__ void lds_poison(T& obj, int tid, int nthreads) {
  if constexpr (POISON_LDS) {
    static_assert(sizeof(T) % 4 == 0, "LDS objects are whole words");
    uint32_t* w = reinterpret_cast<uint32_t*>(&obj);
    for (int i = tid; i < (int)(sizeof(T) / 4); i += nthreads) w[i] = 0x7fc07fc0u;
  }
}

template <class T> struct Elem;
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ bf16_t from_f32(float f) { return f32_to_bf16(f); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f32(float x) { return x; }
  static __device__ __forceinline__ float from_f32(float f) { return f; }
};

// Four consecutive elements packed for one store (8 B for bf16, 16 B for fp32).
template <class T> struct Pack4;
template <> struct Pack4<bf16_t> {
  typedef uint2 type;
  static __device__ __forceinline__ uint2 make(float a, float b, float c, float d) {
    return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
  }
};
template <> struct Pack4<float> {
  typedef float4 type;
  static __device__ __forceinline__ float4 make(float a, float b, float c, float d) {
    return make_float4(a, b, c, d);
  }
};

template <class T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
  *reinterpret_cast<typename Pack4<T>::type*>(p) = Pack4<T>::make(a, b, c, d);
}

// acc (16x16 tile) += A(16 x K) * B(K x 16).
//   a: first row of A; row stride lda elements; k contiguous within a row.
//   b: first column of B stored as a row (i.e. B^T row-major); stride ldb.
template <class T> struct Mma;

template <> struct Mma<bf16_t> {
  template <int K>
  static __device__ __forceinline__ f32x4 run(f32x4 acc, const bf16_t* a, int lda,
                                              const bf16_t* b, int ldb, int lane) {
    const int r = lane & 15, g = lane >> 4;
    if constexpr (K % 32 == 0) {
      const bf16_t* pa = a + r * lda + g * 8;
      const bf16_t* pb = b + r * ldb + g * 8;
#pragma unroll
      for (int k0 = 0; k0 < K; k0 += 32) {
        bf16x8_t av = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(pa + k0));
        bf16x8_t bv = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(pb + k0));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
      }
    } else {
      static_assert(K % 16 == 0, "bf16 product depth must be a multiple of 16");
      const bf16_t* pa = a + r * lda + g * 4;
      const bf16_t* pb = b + r * ldb + g * 4;
#pragma unroll
      for (int k0 = 0; k0 < K; k0 += 16) {
        i16x4_t av = __builtin_bit_cast(i16x4_t, *reinterpret_cast<const uint2*>(pa + k0));
        i16x4_t bv = __builtin_bit_cast(i16x4_t, *reinterpret_cast<const uint2*>(pb + k0));
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, acc, 0, 0, 0);
      }
    }
    return acc;
  }
};

template <> struct Mma<float> {
  template <int K>
  static __device__ __forceinline__ f32x4 run(f32x4 acc, const float* a, int lda,
                                              const float* b, int ldb, int lane) {
    static_assert(K % 4 == 0, "fp32 product depth must be a multiple of 4");
    const int r = lane & 15, g = lane >> 4;
    const float* pa = a + r * lda + g;
    const float* pb = b + r * ldb + g;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k0], pb[k0], acc, 0, 0, 0);
    return acc;
  }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace gdn
