// Device filler of the seeded generator: the same definition as the host
// filler, evaluated one element per thread, so multi-GB synthetic weight banks
// are produced in place in HBM.
#include <hip/hip_runtime.h>
#define SYNTH_FN __host__ __device__ static inline
#include "synth_core.h"

template <bool BF16>
__global__ void synth_fill_kernel(void *out, uint64_t n, uint64_t key, uint64_t start, float scale,
                                  const float *row_mult, uint64_t row_len, uint64_t row0) {
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    uint64_t g = start + i;
    float v = __fmul_rn((float)synth_centred(key, g), scale);
    if (row_mult) v = __fmul_rn(v, row_mult[g / row_len - row0]);
    if (BF16) ((uint16_t *)out)[i] = synth_f32_to_bf16(v);
    else ((float *)out)[i] = v;
  }
}

extern "C" int synth_fill_device(void *out, uint64_t n, int bf16, uint64_t seed, uint64_t tid,
                                 uint64_t start, float scale, const float *row_mult_dev,
                                 uint64_t row_len, void *stream) {
  if (n == 0) return 0;
  if (!out || (row_mult_dev && row_len == 0)) return -1;
  const uint64_t key = synth_key(seed, tid);
  const uint64_t row0 = row_len ? start / row_len : 0;
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = (hipStream_t)stream;
  if (bf16)
    synth_fill_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(out, n, key, start, scale, row_mult_dev, row_len, row0);
  else
    synth_fill_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(out, n, key, start, scale, row_mult_dev, row_len, row0);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
