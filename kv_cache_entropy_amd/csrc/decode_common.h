// rANS decoding pieces shared by the HIP kernels that read containers.
//
// Container format (written by dq_encode): bytes 0..3 hold the final encoder
// state x (little endian, 2^23 <= x < 2^31); the following bytes are the
// renormalisation bytes in reading order; the rest is zero.  Decoding symbol
// i: slot = x mod 4096 selects the symbol s (cum_s <= slot < cum_{s+1}),
// x <- f_s * (x >> 12) + slot - cum_s, then one byte is shifted in if
// x < 2^23 (every f >= 16, so one byte always restores the interval).
//
// Decode tables in LDS, per codec (4352 bytes):
//   sym8[4096]   slot -> 8 * symbol (one byte, so the slot itself is the LDS
//                address and the byte is already the symbol-table offset)
//   symtab[16]   symbol -> {f, cum | fp16 level << 16}
// The byte table is read at a random slot per lane; the symbol table has at
// most 16 distinct entries, so its reads are mostly broadcasts.
#pragma once

#include <hip/hip_runtime.h>

#include "dq_internal.h"

namespace dq {

constexpr int kSymTabBytes = kMaxLevels * 8;
constexpr int kDecodeTableBytes = (int)kM + kSymTabBytes;

__device__ __forceinline__ void build_tables(uint8_t *sym8, uint2 *symtab, const Tables &t, int tid,
                                             int nthreads) {
  // the symbol of slot u is the number of k >= 1 with cum[k] <= u (cum
  // rises strictly): a count over uniform indices, so each cum[k] is a
  // scalar read.  A search with a per-lane index into the argument block
  // would be a chain of dependent memory loads per slot, 12 us per launch.
  for (int u = tid; u < (int)kM; u += nthreads) {
    uint32_t s = 0;
#pragma unroll
    for (int k = 1; k < kMaxLevels; ++k) s += (k < t.levels && (int)t.cum[k] <= u) ? 1u : 0u;
    sym8[u] = (uint8_t)(8 * s);
  }
  if (tid < kMaxLevels)
    symtab[tid] = tid < t.levels ? make_uint2(t.freq[tid], (uint32_t)t.cum[tid] | ((uint32_t)t.recon[tid] << 16))
                                 : make_uint2(0u, 0u);
}

// Per-slot tables: slot u -> the entry of its symbol, {f, cum | fp16 level
// << 16}.  The 16 entries go to `symtab` first; after a barrier each slot
// copies its symbol's (the symbol counted as in build_tables).
__device__ __forceinline__ void build_slot_tables(uint2 *ent, uint2 *symtab, const Tables &t, int tid,
                                                  int nthreads) {
  if (tid < kMaxLevels)
    symtab[tid] = tid < t.levels ? make_uint2(t.freq[tid], (uint32_t)t.cum[tid] | ((uint32_t)t.recon[tid] << 16))
                                 : make_uint2(0u, 0u);
  __syncthreads();
  for (int u = tid; u < (int)kM; u += nthreads) {
    uint32_t s = 0;
#pragma unroll
    for (int k = 1; k < kMaxLevels; ++k) s += (k < t.levels && (int)t.cum[k] <= u) ? 1u : 0u;
    ent[u] = symtab[s];
  }
}

// The state update of a decode step, given the symbol-table entry e of the
// symbol that x's slot selects.
__device__ __forceinline__ uint32_t rans_advance(uint32_t x, uint2 e) {
  return __umul24(e.x, x >> kMBits) + ((x & (kM - 1)) - (e.y & 0xFFFFu));
}

// The same update with the slot (x mod 4096) already at hand.
__device__ __forceinline__ uint32_t rans_advance_slot(uint32_t x, uint32_t slot, uint2 e) {
  return __umul24(e.x, x >> kMBits) + (slot - (e.y & 0xFFFFu));
}

// One decode step without the renormalisation; returns the symbol-table
// entry (.y >> 16 = fp16 level) and the symbol.
__device__ __forceinline__ uint2 rans_step(uint32_t &x, const uint8_t *sym8, const uint2 *symtab, uint32_t &s) {
  const uint32_t s8 = sym8[x & (kM - 1)];
  s = s8 >> 3;
  const uint2 e = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint8_t *>(symtab) + s8);
  x = rans_advance(x, e);
  return e;
}

__device__ __forceinline__ uint64_t dev_splitmix64(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace dq
