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

// Length band of the encoder's drift.  Encoding one symbol from a state
// x >= f * 2^11 (always true after renormalisation) changes log2(x) by
// log2(4096 / f) + d with |d| < log2(1 + 2^-11); emitting a byte from
// x >= 2^23 takes 8 + e bits with 0 <= e < log2(1 + 255 * 2^-23), at most
// once per symbol.  Starting from 2^23 and ending in [2^23, 2^31), a stream
// of B renorm bytes has 8 B <= I + eps < 8 B + 8, with I the sum of
// log2(4096 / f) over its symbols and -0.095760 < eps < 0.090147 over 128
// symbols, so it fits C bytes iff I + eps < 8 (C - 3).  In fixed point
// (kCostFrac fraction bits, each cost rounded: at most 64 units of total
// rounding) the two bounds below are widened by 64 + 16 units.  The band
// they leave, 0.186 bits, is narrower than the smallest saving of one
// move, which the codec check keeps at or above log2(1.15) = 0.2016 bits.
constexpr int kCostFrac = 20;
constexpr uint32_t kEpsHiFx = 94526u + 80u;   // ceil(0.0901465 * 2^20) + margin
constexpr uint32_t kEpsLoFx = 100412u + 80u;  // ceil(0.0957599 * 2^20) + margin

// Everything a kernel needs to know about one codec; passed by value as a
// kernel argument, so hot calls touch no device-side tables.
struct Tables {
  int32_t levels;   // L
  int32_t half;     // L / 2
  int32_t C;        // container bytes
  int32_t step64;   // cell width * 64
  int32_t hkv;      // kv heads
  int32_t order;    // drift order: 0 magnitude, 1 rate-distortion
  uint64_t seed;    // rotation seed
  uint16_t freq[kMaxLevels];
  uint16_t cum[kMaxLevels + 1];
  uint16_t recon[kMaxLevels];          // fp16 bits of the reconstruction level
  uint16_t pad1;
  // encoder: exact floor(x / f) = mulhi(x, magic) >> shift for x < 2^31
  // (Granlund & Montgomery, PLDI 1994, with N = 31, l = ceil(log2 f))
  uint32_t magic[kMaxLevels];
  uint8_t shift[kMaxLevels];
  uint32_t cost_fx[kMaxLevels];        // log2(4096 / f) * 2^20, rounded
  uint32_t saving_fx[kMaxHalf];        // cost_fx[h + m] - cost_fx[h + m - 1], magnitude m >= 1
  float rd_w[kMaxHalf];                // rate-distortion weight of a move from magnitude m
};

}  // namespace dq

struct dq_codec {
  dq_codec_desc desc;  // resolved
  dq::Tables t;
};

namespace dq {
// host helpers implemented in codec.cpp
uint64_t host_splitmix64(uint64_t seed, uint64_t n);
int64_t knob(int k);  // value set by dq_set_knob, -1 when not forced
}  // namespace dq
