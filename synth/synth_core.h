/* Seeded synthetic-input generator shared by the host and device fillers.
 *
 * This file holds no arithmetic of the layer; it only turns (seed, tensor id,
 * element index) into a reproducible, approximately normal number, so that the
 * CPU oracle and the GPU path can be fed bit-identical inputs without copying
 * multi-GB weight banks between them.
 *
 * Definition (counter based, random access):
 *   mix64      the SplitMix64 output function (Steele, Lea & Flood, "Fast
 *              splittable pseudorandom number generators", OOPSLA 2014; the
 *              64-bit finaliser constants of Vigna's reference code).
 *   key        = mix64(mix64(seed + G) + tensor_id), G = 0x9E3779B97F4A7C15.
 *   draw(j)    = mix64(key + (j + 1) * G)   -- the (j+1)-th SplitMix64 output of
 *              a generator whose state starts at `key`.
 *   element i  uses draws 3i, 3i+1, 3i+2: their twelve 16-bit fields u_0..u_11
 *              are summed (Irwin-Hall with 12 terms: mean 6*65535, standard
 *              deviation sqrt(65536^2-1) ~= 65536), centred as
 *              c_i = sum - 393210 (an integer, |c_i| <= 393210, exact in fp32),
 *              and scaled:  v_i = fp32(c_i) * scale  (one IEEE fp32 multiply,
 *              round to nearest even), where scale = fp32(std / 65536).
 *              An optional per-row multiplier is applied as a second fp32
 *              multiply; rows with multiplier 1 are unchanged.
 *   bf16 output rounds v_i to nearest even.
 * Every step is integer or a single correctly rounded fp32 operation, so the
 * host and device fillers produce identical bits.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H
#include <stdint.h>

#ifndef SYNTH_FN
#define SYNTH_FN static inline
#endif

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t tensor_id) {
  return synth_mix64(synth_mix64(seed + SYNTH_GOLDEN) + tensor_id);
}

SYNTH_FN uint64_t synth_draw(uint64_t key, uint64_t j) {
  return synth_mix64(key + (j + 1) * SYNTH_GOLDEN);
}

SYNTH_FN int32_t synth_centred(uint64_t key, uint64_t i) {
  uint64_t s = 0;
  for (int d = 0; d < 3; ++d) {
    uint64_t r = synth_draw(key, 3 * i + (uint64_t)d);
    s += (r & 0xFFFFu) + ((r >> 16) & 0xFFFFu) + ((r >> 32) & 0xFFFFu) + (r >> 48);
  }
  return (int32_t)((int64_t)s - 393210);
}

/* fp32 -> bf16 bits, round to nearest even; NaN kept quiet. */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  if ((v.u & 0x7F800000u) == 0x7F800000u && (v.u & 0x007FFFFFu)) return (uint16_t)((v.u >> 16) | 0x40u);
  uint32_t lsb = (v.u >> 16) & 1u;
  v.u += 0x7FFFu + lsb;
  return (uint16_t)(v.u >> 16);
}

#endif
