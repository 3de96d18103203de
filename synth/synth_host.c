/* Host filler of the seeded generator (plain C, built with gcc, OpenMP).
 * Used by the oracle side of the tests and by the CPU baseline. */
#include <stddef.h>
#include <stdint.h>
#include "synth_core.h"

/* out[i] for global element indices start .. start+n-1 of tensor (seed, tid).
 * row_len > 0 and row_mult != NULL: element g = start+i belongs to row g/row_len
 * and is multiplied by row_mult[g/row_len - row0] (row0 = start/row_len) after
 * the scale multiply. */
void synth_fill_f32(float *out, size_t n, uint64_t seed, uint64_t tid, uint64_t start,
                    float scale, const float *row_mult, uint64_t row_len) {
  const uint64_t key = synth_key(seed, tid);
  const uint64_t row0 = row_len ? start / row_len : 0;
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) {
    uint64_t g = start + (uint64_t)i;
    float v = (float)synth_centred(key, g) * scale;
    if (row_mult && row_len) v = v * row_mult[g / row_len - row0];
    out[i] = v;
  }
}

void synth_fill_bf16(uint16_t *out, size_t n, uint64_t seed, uint64_t tid, uint64_t start,
                     float scale, const float *row_mult, uint64_t row_len) {
  const uint64_t key = synth_key(seed, tid);
  const uint64_t row0 = row_len ? start / row_len : 0;
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) {
    uint64_t g = start + (uint64_t)i;
    float v = (float)synth_centred(key, g) * scale;
    if (row_mult && row_len) v = v * row_mult[g / row_len - row0];
    out[i] = synth_f32_to_bf16(v);
  }
}

uint64_t synth_splitmix_output(uint64_t state, uint64_t j) { return synth_draw(state, j); }
