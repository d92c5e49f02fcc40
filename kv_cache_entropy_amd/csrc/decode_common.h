// rANS decoding pieces shared by the HIP kernels that read containers.
//
// Container format (written by dq_encode): bytes 0..3 hold the final encoder
// state x (little endian, 2^23 <= x < 2^31); the following bytes are the
// renormalisation bytes in reading order; the rest is zero.  Decoding symbol
// i: slot = x mod 4096 selects the symbol s (cum_s <= slot < cum_{s+1}),
// x <- f_s * (x >> 12) + slot - cum_s, then one byte is shifted in if
// x < 2^23 (every f >= 16, so one byte always restores the interval).
#pragma once

#include <hip/hip_runtime.h>

#include "dq_internal.h"

namespace dq {

// LUT entry for slot u (8 bytes):
//   .x = f_s | s << 24        (mad24 reads only the low 24 bits: f_s)
//   .y = (u - cum_s) | r_s << 16   (r_s = fp16 reconstruction level)
__device__ __forceinline__ void build_lut(uint2 *lut, const Tables &t, int tid, int nthreads) {
  for (int u = tid; u < (int)kM; u += nthreads) {
    int s = 0;
    while (s + 1 < t.levels && (int)t.cum[s + 1] <= u) ++s;
    lut[u] = make_uint2((uint32_t)t.freq[s] | ((uint32_t)s << 24),
                        (uint32_t)(u - (int)t.cum[s]) | ((uint32_t)t.recon[s] << 16));
  }
}

// One decode step; returns the LUT entry so callers can take the symbol
// (e.x >> 24) or the fp16 level (e.y >> 16).
__device__ __forceinline__ uint2 rans_step(uint32_t &x, const uint2 *lut) {
  const uint2 e = lut[x & (kM - 1)];
  x = __umul24(e.x, x >> kMBits) + (e.y & 0xFFFFu);
  return e;
}

__device__ __forceinline__ uint64_t dev_splitmix64(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace dq
