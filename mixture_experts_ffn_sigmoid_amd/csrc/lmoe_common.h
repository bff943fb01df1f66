// Shared device helpers of the gfx950 Stable LatentMoE kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

typedef uint16_t bf16_t;  // bf16 bit pattern in memory
typedef _Float16 f16_t;   // IEEE binary16
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int V>
struct IntC {
  static constexpr int value = V;
};

// Compile-time loop: f(IntC<0>{}), ..., f(IntC<N-1>{}).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    sfor<N, I + 1>(f);
  }
}

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16, round to nearest even, NaN kept NaN: one v_cvt_pk_bf16_f32.
// (Checked on the device against the bitwise rounding rule, add 0x7FFF plus
// the kept lsb and truncate, over every non-NaN fp32 pattern: no difference.
// The bitwise form with its NaN test compiles to a divergent branch per value.)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kSize = 4;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <>
struct Elem<f16_t> {
  static constexpr int kSize = 2;
  __device__ __forceinline__ static float load(const f16_t* p) { return (float)*p; }
  __device__ __forceinline__ static void store(f16_t* p, float v) { *p = (f16_t)v; }
};
template <>
struct Elem<bf16_t> {
  static constexpr int kSize = 2;
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
};

// 8 bf16 (16 bytes) -> 8 fp16.  Exact for |w| in [2^-14, 65504]; smaller
// magnitudes keep fp16's subnormal absolute precision (2^-24).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 in) {
  u32x4 out;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float lo = __uint_as_float(in[w] << 16);
    const float hi = __uint_as_float(in[w] & 0xFFFF0000u);
    out[w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return out;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }

// 1/x from the hardware reciprocal v_rcp_f32 (about 1 ulp; 1/inf = 0).  A
// correctly rounded reciprocal compiles to a ten-instruction division sequence.
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh from one hardware exp and one reciprocal: tanh|x| = (1 - e) / (1 + e),
// e = exp(-2|x|) in (0, 1], so nothing overflows; absolute error ~1e-7.
__device__ __forceinline__ float tanh_fast(float x) {
  const float e = __expf(-2.0f * fabsf(x));
  return copysignf((1.0f - e) * rcp_fast(1.0f + e), x);
}

// SiTU-GLU hidden: beta1*tanh(g/beta1)*sigmoid(g) * beta2*tanh(u/beta2), fp32.
// inv_b1 = 1/beta1, inv_b2 = 1/beta2.
__device__ __forceinline__ float situ_hidden(float g, float u, float beta1, float beta2,
                                             float inv_b1, float inv_b2) {
  const float sig = rcp_fast(1.0f + __expf(-g));  // exp(-g) = inf gives 0
  const float gate = beta1 * tanh_fast(g * inv_b1) * sig;
  const float up = beta2 * tanh_fast(u * inv_b2);
  return gate * up;
}

// Hardware dispatches workgroup w to XCD (w mod 8).  Renumber so that each
// XCD works on one contiguous range of logical tile ids: neighbouring tiles
// (which share operand panels) then share that XCD's L2.
__device__ __forceinline__ int xcd_contiguous_id(int w, int total) {
  constexpr int kXcd = 8;
  int q = total / kXcd, r = total % kXcd;
  int x = w % kXcd, i = w / kXcd;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace lmoe
