// Internal definitions shared by the library's host code and HIP kernels.
// (Not shared with anything outside kv_cache_entropy_amd/csrc.)
#pragma once

#include <stdint.h>

#include "../../include/dq.h"

namespace dq {

constexpr int kD = 128;                 // head dimension
constexpr int kMBits = 12;              // rANS table precision
constexpr uint32_t kM = 1u << kMBits;   // 4096
constexpr uint32_t kLow = 1u << 23;     // rANS state lower bound
constexpr uint32_t kFMin = 16;          // smallest frequency: one renorm byte per step
constexpr int kMaxLevels = 16;
constexpr int kMaxHalf = kMaxLevels / 2;
constexpr int kMaxC = DQ_MAX_CONTAINER;

// Everything a kernel needs to know about one codec; passed by value as a
// kernel argument, so hot calls touch no device-side tables.
struct Tables {
  int32_t levels;   // L
  int32_t half;     // L / 2
  int32_t C;        // container bytes
  int32_t step64;   // cell width * 64
  int32_t hkv;      // kv heads
  int32_t pad0;
  uint64_t seed;    // rotation seed
  uint16_t freq[kMaxLevels];
  uint16_t cum[kMaxLevels + 1];
  uint16_t recon[kMaxLevels];          // fp16 bits of the reconstruction level
  uint16_t pad1;
  // encoder: exact floor(x / f) = mulhi(x, magic) >> shift for x < 2^31
  // (Granlund & Montgomery, PLDI 1994, with N = 31, l = ceil(log2 f))
  uint32_t magic[kMaxLevels];
  uint8_t shift[kMaxLevels];
  float cost[kMaxLevels];              // log2(4096 / f), drift estimate only
  float saving[kMaxHalf];              // log2(f_{m-1} / f_m) for magnitude m >= 1
};

}  // namespace dq

struct dq_codec {
  dq_codec_desc desc;  // resolved
  dq::Tables t;
};

namespace dq {
// host helpers implemented in codec.cpp
uint64_t host_splitmix64(uint64_t seed, uint64_t n);
}  // namespace dq
