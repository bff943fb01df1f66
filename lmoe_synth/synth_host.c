/* Host (CPU, OpenMP) side of the seeded input generator.  See synth_core.h
 * for the definition.  `start` is the element index of dst[0] inside the
 * tensor, so any slice (one expert, a few rows) can be regenerated alone. */
#include "synth_core.h"

void lmoe_synth_fill_normal_f32(float* dst, int64_t start, int64_t count, uint64_t seed,
                                uint32_t tensor_id, double scale, int64_t row_len,
                                int64_t rows_mult, double row_mult) {
  const uint64_t key = lmoe_synth_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) {
    dst[j] = (float)lmoe_synth_normal_value(key, (uint64_t)(start + j), scale, row_len, rows_mult,
                                            row_mult);
  }
}

void lmoe_synth_fill_normal_bf16(uint16_t* dst, int64_t start, int64_t count, uint64_t seed,
                                 uint32_t tensor_id, double scale, int64_t row_len,
                                 int64_t rows_mult, double row_mult) {
  const uint64_t key = lmoe_synth_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) {
    float f = (float)lmoe_synth_normal_value(key, (uint64_t)(start + j), scale, row_len, rows_mult,
                                             row_mult);
    dst[j] = lmoe_synth_f32_to_bf16(f);
  }
}

void lmoe_synth_fill_uniform_f32(float* dst, int64_t start, int64_t count, uint64_t seed,
                                 uint32_t tensor_id, double lo, double hi) {
  const uint64_t key = lmoe_synth_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) {
    dst[j] = (float)lmoe_synth_uniform(key, (uint64_t)(start + j), lo, hi);
  }
}
