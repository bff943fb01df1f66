// Sum of the p-weighted routed slots of each token (the deterministic form of
// the scatter-add) fused with the latent RMSNorm that feeds W_up.
#pragma once

#include "lmoe_common.h"

namespace lmoe {
// Internal linkage: every translation unit that launches these kernels
// carries its own copy.
namespace {

constexpr int kMaxLatent = 8192;  // 8 float4 per thread of a 256-thread workgroup

// Four consecutive elements (8- or 16-byte aligned) widened to fp32.
template <typename TS>
__device__ __forceinline__ f32x4 load4(const TS* p) {
  f32x4 r;
  if constexpr (sizeof(TS) == 4) {
    r = *(const f32x4*)p;
  } else {
    TS tmp[4];
    *(u32x2*)tmp = *(const u32x2*)p;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = Elem<TS>::load(tmp + q);
  }
  return r;
}

// One workgroup per token n (slots of type TS, summed in fp32):
//   u[c] = sum_{j < k} slots[(n k + j) l + c]      (slot order)
//   u_out[n, c] = u[c]                               (if u_out)
//   dst[n, c]   = T(w[c] u[c] / sqrt(mean(u^2) + eps)) (if dst; w = 1 when rms_w is NULL)
// With fp16 dst, *range_flag = 1 when a stored value is not finite in fp16.
template <typename TS, typename T>
__global__ __launch_bounds__(256) void combine_rmsnorm_kernel(const TS* __restrict__ slots, int k,
                                                              int ell, float* __restrict__ u_out,
                                                              const float* __restrict__ rms_w,
                                                              float eps, T* __restrict__ dst,
                                                              int64_t ld_dst, int32_t* __restrict__ range_flag) {
  constexpr int kVec = kMaxLatent / 1024;
  __shared__ float red[4];
  const int64_t n = blockIdx.x;
  const int t = threadIdx.x;
  f32x4 u[kVec];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const int c = 4 * t + 1024 * i;
    u[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c < ell) {
      const TS* src = slots + (n * k * ell + c);
      int j = 0;
      for (; j + 4 <= k; j += 4) {  // four slots' loads in flight, summed in slot order
        const f32x4 a = load4(src + (int64_t)j * ell), b = load4(src + (int64_t)(j + 1) * ell);
        const f32x4 cc = load4(src + (int64_t)(j + 2) * ell), d = load4(src + (int64_t)(j + 3) * ell);
#pragma unroll
        for (int q = 0; q < 4; ++q) u[i][q] = (((u[i][q] + a[q]) + b[q]) + cc[q]) + d[q];
      }
      for (; j < k; ++j) {
        const f32x4 a = load4(src + (int64_t)j * ell);
#pragma unroll
        for (int q = 0; q < 4; ++q) u[i][q] += a[q];
      }
      ss += u[i][0] * u[i][0] + u[i][1] * u[i][1] + u[i][2] * u[i][2] + u[i][3] * u[i][3];
      if (u_out) *(f32x4*)(u_out + n * ell + c) = u[i];
    }
  }
  if (!dst) return;  // uniform
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  const float total = (red[0] + red[1]) + (red[2] + red[3]);
  const float r = 1.0f / sqrtf(total / (float)ell + eps);
  bool out_of_range = false;
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const int c = 4 * t + 1024 * i;
    if (c < ell) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float w = rms_w ? rms_w[c + q] : 1.f;
        const float v = u[i][q] * r * w;
        if constexpr (__is_same(T, f16_t)) out_of_range |= !(fabsf(v) < 65520.0f);
        Elem<T>::store(dst + n * ld_dst + c + q, v);
      }
    }
  }
  if (out_of_range && range_flag) *range_flag = 1;
}

}  // namespace
}  // namespace lmoe
