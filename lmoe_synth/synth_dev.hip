/* Device side of the seeded input generator (same definition as the host
 * side, see synth_core.h).  Used to materialise the large weight sets
 * (tens of GB) directly in HBM.  Plain C ABI; returns hipError_t as int. */
#include <hip/hip_runtime.h>
#include "synth_core.h"

namespace {

__global__ void fill_normal_f32(float* dst, int64_t start, int64_t count, uint64_t key,
                                double scale, int64_t row_len, int64_t rows_mult, double row_mult) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += stride)
    dst[j] = (float)lmoe_synth_normal_value(key, (uint64_t)(start + j), scale, row_len, rows_mult,
                                            row_mult);
}

__global__ void fill_normal_bf16(uint16_t* dst, int64_t start, int64_t count, uint64_t key,
                                 double scale, int64_t row_len, int64_t rows_mult, double row_mult) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += stride) {
    float f = (float)lmoe_synth_normal_value(key, (uint64_t)(start + j), scale, row_len, rows_mult,
                                             row_mult);
    dst[j] = lmoe_synth_f32_to_bf16(f);
  }
}

__global__ void fill_uniform_f32(float* dst, int64_t start, int64_t count, uint64_t key, double lo,
                                 double hi) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += stride)
    dst[j] = (float)lmoe_synth_uniform(key, (uint64_t)(start + j), lo, hi);
}

unsigned grid_for(int64_t count) {
  int64_t g = (count + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

extern "C" {

int lmoe_synth_dev_fill_normal_f32(float* dst, int64_t start, int64_t count, uint64_t seed,
                                   uint32_t tensor_id, double scale, int64_t row_len,
                                   int64_t rows_mult, double row_mult, void* stream) {
  if (count <= 0) return 0;
  fill_normal_f32<<<grid_for(count), 256, 0, (hipStream_t)stream>>>(
      dst, start, count, lmoe_synth_key(seed, tensor_id), scale, row_len, rows_mult, row_mult);
  return (int)hipGetLastError();
}

int lmoe_synth_dev_fill_normal_bf16(uint16_t* dst, int64_t start, int64_t count, uint64_t seed,
                                    uint32_t tensor_id, double scale, int64_t row_len,
                                    int64_t rows_mult, double row_mult, void* stream) {
  if (count <= 0) return 0;
  fill_normal_bf16<<<grid_for(count), 256, 0, (hipStream_t)stream>>>(
      dst, start, count, lmoe_synth_key(seed, tensor_id), scale, row_len, rows_mult, row_mult);
  return (int)hipGetLastError();
}

int lmoe_synth_dev_fill_uniform_f32(float* dst, int64_t start, int64_t count, uint64_t seed,
                                    uint32_t tensor_id, double lo, double hi, void* stream) {
  if (count <= 0) return 0;
  fill_uniform_f32<<<grid_for(count), 256, 0, (hipStream_t)stream>>>(
      dst, start, count, lmoe_synth_key(seed, tensor_id), lo, hi);
  return (int)hipGetLastError();
}

}  // extern "C"
