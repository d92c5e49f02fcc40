// One-wave-per-vector encode: the core shared by dq_encode's small-batch
// kernels and the append inside decode attention.
//
// Steps per vector ("D-Quant: Entropy Coding Meets KV Cache at 2.26 Bits",
// Why Fixed Width Is a Ceiling and Drift: Bending Variable Back to Fixed):
// rotate (randomized Walsh-Hadamard), fp16 norm, quantise on the analytic
// N(0,1) cells, rANS into the container, and drift the first candidates of
// the fixed order one level inward until the stream fits.  Lane l holds
// coordinates l and l + 64; the drift search is one parallel pass: a
// bitonic sort of the wave's 128 (key, index) pairs gives every candidate
// its rank in the drift order, and lane l runs the rANS pass with the first
// k0 + l candidates moved, so the lowest
// lane whose stream fits is the answer (the length never increases along
// the order).
//
// Arithmetic that decides a symbol is fp32 in a fixed order (butterfly
// widths 1..64, halving-tree sum of squares); the build uses
// -ffp-contract=off and keeps denormals, so the result is reproducible bit
// for bit.
#pragma once

#include <hip/hip_runtime.h>

#include "decode_common.h"

namespace dq {

constexpr int kWaveScr = 128;  // renorm bytes a candidate stream can emit: one per symbol at most

__device__ __forceinline__ float half_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp16 nearest to sqrt(S) (ties to even), exactly: a candidate from the
// hardware square root and conversion, then corrected against the squared
// midpoints to its neighbours.  Midpoints of adjacent fp16 values have at
// most 12 significant bits, so mid * mid is exact in fp32 and the compares
// decide the rounding of the exact square root.
__device__ __forceinline__ uint32_t norm_half(float S) {
  if (S != S) return 0x7E00u;
  if (S == __builtin_inff()) return 0x7C00u;
  uint32_t hb = __builtin_bit_cast(uint16_t, (_Float16)__builtin_sqrtf(S));
  if (hb < 0x7C00u) {
    const float hv = half_to_float(hb);
    const float up = hb == 0x7BFFu ? 65536.0f : half_to_float(hb + 1);
    const float mid = (hv + up) * 0.5f;
    const float m2 = mid * mid;
    if (S > m2 || (S == m2 && (hb & 1u))) ++hb;
  }
  if (hb > 0u) {
    const float hv = hb == 0x7C00u ? 65536.0f : half_to_float(hb);
    const float lo = half_to_float(hb - 1);
    const float mid = (lo + hv) * 0.5f;
    const float m2 = mid * mid;
    if (S < m2 || (S == m2 && (hb & 1u))) --hb;
  }
  return hb;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Coder constants per symbol (etab) and the rate-distortion key terms per
// magnitude (rdtab), built once per block by the first threads.
//   etab[s] = {f << 19 (emit bound), magic, cum, (M - f) | shift << 16}
//   rdtab[m] = {l_m + l_{m-1}, w_m}
__device__ __forceinline__ void wave_encode_tables(const Tables &t, uint4 *etab, float2 *rdtab, int tid) {
  if (tid < t.levels) {
    const uint32_t f = t.freq[tid];
    etab[tid] = make_uint4(f << 19, t.magic[tid], t.cum[tid], (kM - f) | ((uint32_t)t.shift[tid] << 16));
  }
  if (tid >= 1 && tid < t.half)
    rdtab[tid] = make_float2(half_to_float(t.recon[t.half + tid]) + half_to_float(t.recon[t.half + tid - 1]),
                             t.rd_w[tid]);
}

// Per-wave LDS scratch.  rows >= C - 3: a stream longer than C - 4 bytes
// does not fit anyway, so only its length, not its bytes, must be right.
struct WaveEncodeScratch {
  uint32_t *ent;  // [128] s0 | sd << 8 | rank << 16
  uint8_t *mag;   // [128] magnitude cell (4-byte aligned: read as words)
  uint8_t *scr;   // [rows][64] renorm bytes, lane-minor
  int rows;
};

struct WaveEncodeResult {
  uint32_t nh;   // fp16 norm bits
  uint32_t okx;  // final encoder state of the fitting stream
  int win;       // lane that found it (-1: none)
  int okB;       // its renorm bytes
  int moves;     // symbols moved inward
  int passes;    // full passes that moved every candidate
  bool bad, zero;
  uint32_t sym[2];  // final symbols of coordinates lane and lane + 64
};

// Encodes the vector at xp (bf16 [128]) of kv head g.  CLAMP keeps the
// scratch writes inside rows < kWaveScr (unneeded when rows == kWaveScr).
template <bool RD, bool CLAMP>
__device__ __forceinline__ void wave_encode_vector(const uint16_t *xp, int g, const Tables &t, const uint4 *etab,
                                                   const float2 *rdtab, const WaveEncodeScratch &L, int lane,
                                                   WaveEncodeResult &r) {
  const int h = t.half, C = t.C;
  const float x0 = __uint_as_float((uint32_t)xp[lane] << 16);
  const float x1 = __uint_as_float((uint32_t)xp[lane + 64] << 16);

  // ||x||^2: level 64 in-lane, then levels 32 .. 1 across lanes
  float sq = x0 * x0 + x1 * x1;
#pragma unroll
  for (int wd = 32; wd >= 1; wd >>= 1) {
    const float o = __shfl_down(sq, wd);
    if (lane < wd) sq = sq + o;
  }
  const float S = __shfl(sq, 0);

  // y = H * D * x
  const uint64_t s0w = dev_splitmix64(t.seed, 2ull * (uint64_t)g);
  const uint64_t s1w = dev_splitmix64(t.seed, 2ull * (uint64_t)g + 1ull);
  float u0 = ((s0w >> lane) & 1ull) ? -x0 : x0;
  float u1 = ((s1w >> lane) & 1ull) ? -x1 : x1;
#pragma unroll
  for (int wd = 1; wd < 64; wd <<= 1) {
    const float p0 = __shfl_xor(u0, wd), p1 = __shfl_xor(u1, wd);
    const bool hi = lane & wd;
    u0 = hi ? p0 - u0 : u0 + p0;
    u1 = hi ? p1 - u1 : u1 + p1;
  }
  {
    const float p = u0, q = u1;
    u0 = p + q;
    u1 = p - q;
  }

  const uint32_t nh = norm_half(S);
  const float nf = half_to_float(nh);
  const bool zero = nh == 0u;
  const bool bad = (nh & 0x7C00u) == 0x7C00u;
  const bool degenerate = zero || bad;
  float thr[kMaxHalf];
#pragma unroll
  for (int k = 1; k < kMaxHalf; ++k)
    thr[k] = (k < h && !degenerate) ? (float)(k * t.step64) * nf * 0.015625f : __builtin_inff();
  uint32_t sA[2], mA[2];
  float yA[2];
  const float ys[2] = {u0, u1};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float ay = degenerate ? 0.0f : __builtin_fabsf(ys[e]);
    uint32_t m = 0;
#pragma unroll
    for (int k = 1; k < kMaxHalf; ++k) m += ay >= thr[k] ? 1u : 0u;
    sA[e] = (degenerate || ys[e] >= 0.0f) ? (uint32_t)h + m : (uint32_t)(h - 1) - m;
    mA[e] = m;
    yA[e] = ay;
  }
  uint32_t *E = L.ent;
  uint8_t *Mg = L.mag;
  uint8_t *scol = L.scr;
  const int rows = L.rows;

  int moves = 0, passes = 0, okB = 0;
  uint32_t okx = 0, kwin = 0;
  int win = -1;
  for (int outer = 0; outer < 2 * kD && win < 0; ++outer) {
    // ranks of the candidates (magnitude >= 1) in drift order.  Magnitude
    // order compares (m desc, |y| asc); rate-distortion order compares its
    // key (2|y| - n (l_m + l_{m-1})) * w_m ascending, n (l_m + l_{m-1})
    // being exact in fp32.  Both then break ties by index.
    float kA[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float key = yA[e];
      if (RD && mA[e] >= 1u) {
        const float2 rr = rdtab[mA[e]];
        const float tt = nf * rr.x;
        key = (2.0f * yA[e] - tt) * rr.y;
      }
      kA[e] = key;
    }
    // Ranks by a bitonic sort of the wave's 128 (key, index) pairs, position
    // lane + 64 e holding element e of the lane.  The 64-bit key orders
    // non-candidates last, then (magnitude order) m descending, then the
    // drift-order key ascending as sortable bits (-0 folded into +0, so that
    // keys equal as floats tie), then the index: distinct keys, so a
    // candidate's place is the number of candidates before it.
    uint64_t v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t kb = __float_as_uint(kA[e] + 0.0f);
      const uint32_t lo = (kb & 0x80000000u) ? ~kb : (kb | 0x80000000u);
      const uint32_t cls = mA[e] >= 1u ? (RD ? 0u : 15u - mA[e]) : 16u;
      v[e] = ((uint64_t)cls << 40) | ((uint64_t)lo << 8) | (uint64_t)(lane + 64 * e);
    }
#pragma unroll
    for (int k = 2; k <= kD; k <<= 1) {
#pragma unroll
      for (int j = k >> 1; j >= 1; j >>= 1) {
        if (j == 64) {  // partners in the same lane (k = 128: ascending)
          const uint64_t a0 = v[0], a1 = v[1];
          v[0] = a0 < a1 ? a0 : a1;
          v[1] = a0 < a1 ? a1 : a0;
        } else {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int p = lane + 64 * e;
            const uint32_t whi = (uint32_t)__shfl_xor((int)(uint32_t)(v[e] >> 32), j);
            const uint32_t wlo = (uint32_t)__shfl_xor((int)(uint32_t)v[e], j);
            const uint64_t w = ((uint64_t)whi << 32) | wlo;
            const bool take_min = ((p & k) == 0) == ((p & j) == 0);
            const bool less = v[e] < w;
            v[e] = take_min == less ? v[e] : w;
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) Mg[(int)(v[e] & 0x7Fu)] = (uint8_t)(lane + 64 * e);
    wave_sync_lds();
    int rank[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) rank[e] = Mg[lane + 64 * e];
    int total = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) total += __popcll(__ballot(mA[e] >= 1u));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t sd = mA[e] >= 1u ? (sA[e] >= (uint32_t)h ? sA[e] - 1u : sA[e] + 1u) : sA[e];
      const uint32_t rk = mA[e] >= 1u ? (uint32_t)rank[e] : 255u;
      E[lane + 64 * e] = sA[e] | (sd << 8) | (rk << 16);
    }
    wave_sync_lds();
    for (int k0 = 0; k0 <= total && win < 0; k0 += 64) {
      const uint32_t k = (uint32_t)(k0 + lane);
      uint32_t x = kLow;
      int pos = rows - 1;
      // the symbol and coder-constant reads of a step do not depend on the
      // state: unrolled, they run ahead of the state chain
#pragma unroll 8
      for (int i = kD - 1; i >= 0; --i) {
        const uint32_t en = E[i];
        const uint32_t s = ((en >> 16) & 0xFFu) < k ? ((en >> 8) & 0xFFu) : (en & 0xFFu);
        const uint4 c = etab[s];
        scol[(CLAMP ? max(pos, 0) : pos) * 64 + lane] = (uint8_t)x;
        const bool emit = x >= c.x;
        x = emit ? x >> 8 : x;
        pos -= emit ? 1 : 0;
        const uint32_t q = __umulhi(x, c.y) >> (c.w >> 16);
        x = x + c.z + __umul24(q, c.w & 0xFFFFu);
      }
      const int B = rows - 1 - pos;
      const bool fits = 4 + B <= C && (int)k <= total;
      const uint64_t vote = __ballot(fits);
      if (vote) {
        win = __ffsll((unsigned long long)vote) - 1;
        okB = __shfl(B, win);
        okx = (uint32_t)__shfl((int)x, win);
        kwin = (uint32_t)(k0 + win);
        moves += k0 + win;
      }
    }
    if (win < 0) {
      // every candidate moved and the stream still does not fit: keep the
      // moves and rank again on the new symbols
      moves += total;
      ++passes;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (mA[e] >= 1u) {
          sA[e] = sA[e] >= (uint32_t)h ? sA[e] - 1u : sA[e] + 1u;
          mA[e] -= 1u;
        }
      }
    }
  }
  wave_sync_lds();
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t en = E[lane + 64 * e];
    r.sym[e] = win < 0 ? sA[e] : (((en >> 16) & 0xFFu) < kwin ? ((en >> 8) & 0xFFu) : (en & 0xFFu));
  }
  r.nh = nh;
  r.okx = okx;
  r.win = win;
  r.okB = okB;
  r.moves = moves;
  r.passes = passes;
  r.bad = bad;
  r.zero = zero;
}

// Writes the container [final state LE][renorm bytes in decode order][zero
// pad] and the fp16 norm of an encoded vector.
__device__ __forceinline__ void wave_store_container(const WaveEncodeResult &r, const WaveEncodeScratch &L, int C,
                                                     uint8_t *dst, uint16_t *norm_dst, int lane) {
  for (int j = lane; j < C; j += 64) {
    uint8_t b;
    if (j < 4) b = (uint8_t)(r.okx >> (8 * j));
    else b = (j - 4 < r.okB) ? L.scr[(L.rows - r.okB + (j - 4)) * 64 + r.win] : (uint8_t)0;
    dst[j] = b;
  }
  if (lane == 0) *norm_dst = (uint16_t)r.nh;
}

}  // namespace dq
