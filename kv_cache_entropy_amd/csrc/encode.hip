// dq_encode: bf16 K or V vectors -> fixed-size rANS containers.
//
// Pipeline per vector ("D-Quant: Entropy Coding Meets KV Cache at 2.26
// Bits", Why Fixed Width Is a Ceiling and Drift: Bending Variable Back to
// Fixed; "D-Quant: Driftable Entropy Coding for KV Cache Quantization",
// abstract):
//   rotate (randomized Walsh-Hadamard) -> normalise (fp16 norm) -> quantise
//   (uniform cells on the analytic N(0,1) model) -> rANS into the container
//   -> if the stream does not fit, drift the first candidates of a fixed
//   order one level inward until it does.
//
// MI355X mapping: one lane owns one vector end to end.  The rotation runs on
// the 128 coordinates in VGPRs (fully unrolled butterflies); the symbols stay
// in VGPRs as 4-bit fields, so a rANS pass is a straight unrolled chain whose
// only memory access is the per-symbol coder constants in LDS.  Renorm bytes
// go to a double-buffered LDS scratch, lane-minor, so the last fitting
// stream survives a later trial pass.  The drift search moves one candidate
// at a time around an estimate of the number of moves, so a drifted vector
// usually costs three passes.  Lanes of a wave take consecutive tokens of one
// kv head, so their containers are adjacent in the pool.
//
// Arithmetic that decides a symbol is fp32 in a fixed order (butterfly
// widths 1..64, halving-tree sum of squares); the build uses
// -ffp-contract=off and keeps denormals, so the result is reproducible
// bit for bit.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "dq_internal.h"

namespace dq {
namespace {

constexpr int kThreads = 128;
constexpr int kScr = 128;  // renorm bytes per lane and buffer: at most one per symbol

struct EncodeArgs {
  const uint16_t *x;
  int64_t T, stride_t, stride_h;
  const int64_t *slots;
  int64_t num_slots;
  uint8_t *cont;
  uint16_t *norm;
  dq_stats *stats;
};

__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t n) {
  uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

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

__device__ __forceinline__ uint32_t nib(const uint32_t (&w)[16], int i) {
  return (w[i >> 3] >> (4 * (i & 7))) & 15u;
}
__device__ __forceinline__ uint32_t bit(const uint32_t (&w)[4], int i) {
  return (w[i >> 5] >> (i & 31)) & 1u;
}
__device__ __forceinline__ uint32_t magnitude(uint32_t s, int h) {
  return s >= (uint32_t)h ? s - (uint32_t)h : (uint32_t)(h - 1) - s;
}

// One lane's vector during the drift search: the quantised symbols before
// the current drift pass (4 bits each), the drift flags, and |y_i| (the
// order key inside a magnitude group).  The current symbols (with the
// flagged coordinates one level inward) live in the lane's LDS column.
struct Vec {
  float ay[kD];
  uint32_t sym0[16];
  uint32_t fl[4];
};

// Among the members of group mask gm: the unflagged one with the smallest
// (|y|, index) -- the next candidate in drift order -- or, with flagged, the
// flagged one with the largest (|y|, index) -- the last candidate taken;
// -1 if there is none.
__device__ __forceinline__ int extreme_in_group(const Vec &v, const uint32_t (&gm)[4], bool flagged) {
  float best = 0.0f;
  int bi = -1;
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    const bool member = bit(gm, i) && ((bit(v.fl, i) != 0u) == flagged);
    const bool better = flagged ? (v.ay[i] >= best) : (v.ay[i] < best);
    const bool take = member && (bi < 0 || better);
    best = take ? v.ay[i] : best;
    bi = take ? i : bi;
  }
  return bi;
}

__device__ __forceinline__ void group_mask(const Vec &v, int h, int g, uint32_t (&gm)[4]) {
  gm[0] = gm[1] = gm[2] = gm[3] = 0u;
#pragma unroll
  for (int i = 0; i < kD; ++i) gm[i >> 5] |= (magnitude(nib(v.sym0, i), h) == (uint32_t)g ? 1u : 0u) << (i & 31);
}

// Moves coordinate i (dynamic) one level inward, or back out (undo), in the
// LDS symbol column, and toggles its flag.  A moved symbol stays on its side
// of zero, so the current value alone tells the direction.
__device__ __forceinline__ void toggle(Vec &v, uint8_t *symL, int i, int h, bool undo, int lane) {
  uint8_t *p = symL + i * kThreads + lane;
  const uint32_t s = *p;
  const bool pos = s >= (uint32_t)h;
  *p = (uint8_t)((pos != undo) ? s - 1u : s + 1u);
#pragma unroll
  for (int j = 0; j < 4; ++j) v.fl[j] ^= ((i >> 5) == j) ? (1u << (i & 31)) : 0u;
}

template <int MAXH>
__device__ __forceinline__ int cnt_at(const int (&cnt)[MAXH], int m) {
  int r = 0;
#pragma unroll
  for (int q = 1; q < MAXH; ++q) r = (q == m) ? cnt[q] : r;
  return r;
}

// One rANS pass over the lane's LDS symbol column (pushed 127 -> 0).
// Renorm bytes go to the lane's scratch column from the end backwards (rows
// kScr - B .. kScr - 1 are then in the decoder's reading order); the byte
// store is unconditional and simply overwritten when no byte is emitted.
__device__ __forceinline__ int rans_pass(const uint8_t *symL, const uint4 *etab, uint8_t *buf, int lane,
                                         uint32_t *xfinal) {
  uint32_t x = kLow;
  int pos = kScr - 1;
#pragma unroll 4
  for (int i = kD - 1; i >= 0; --i) {
    const uint4 e = etab[symL[i * kThreads + lane]];  // {f << 19, magic, cum, (4096 - f) | shift << 16}
    buf[pos * kThreads + lane] = (uint8_t)x;
    const bool emit = x >= e.x;
    x = emit ? x >> 8 : x;
    pos -= emit ? 1 : 0;
    const uint32_t q = __umulhi(x, e.y) >> (e.w >> 16);
    x = x + e.z + __umul24(q, e.w & 0xFFFFu);
  }
  *xfinal = x;
  return kScr - 1 - pos;
}

enum : int { kPhInit, kPhFirst, kPhDown, kPhUp, kPhDone };
enum : int { kActNone, kActPrefix, kActAdd, kActRemove, kActCommit };

template <int MAXH>
__global__ void __launch_bounds__(kThreads) encode_kernel(EncodeArgs a, Tables t) {
  __shared__ uint4 etab[kMaxLevels];
  __shared__ uint8_t scr[2][kScr * kThreads];  // double-buffered renorm bytes
  __shared__ uint8_t symcol[kD * kThreads];     // current symbols, lane-minor
  __shared__ uint32_t bstat[6 + kMaxC + 1];

  const int lane = threadIdx.x;
  if (lane < t.levels) {
    const uint32_t f = t.freq[lane];
    etab[lane] = make_uint4(f << 19, t.magic[lane], t.cum[lane], (kM - f) | ((uint32_t)t.shift[lane] << 16));
  }
  for (int k = lane; k < 6 + kMaxC + 1; k += kThreads) bstat[k] = 0u;
  __syncthreads();

  const int h = t.half;
  const int C = t.C;
  const int64_t nvec = a.T * (int64_t)t.hkv;
  const int64_t vid = (int64_t)blockIdx.x * kThreads + lane;
  if (vid < nvec) {
    const int g = (int)(vid / a.T);
    const int64_t tok = vid - (int64_t)g * a.T;
    const int64_t slot = a.slots[tok];
    const bool in_pool = slot >= 0 && slot < a.num_slots;  // out-of-range slots write nothing
    const uint4 *src = reinterpret_cast<const uint4 *>(a.x + tok * a.stride_t + (int64_t)g * a.stride_h);
    uint32_t xw[64];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 w = src[j];
      xw[4 * j + 0] = w.x;
      xw[4 * j + 1] = w.y;
      xw[4 * j + 2] = w.z;
      xw[4 * j + 3] = w.w;
    }
    // bf16 element i as fp32 bits
#define DQ_ELEM(i) ((xw[(i) >> 1] << (16 * (1 - ((i) & 1)))) & 0xFFFF0000u)
    // ||x||^2 by the halving tree: i + 64, then i + 32, ..., i + 1
    float sq[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float a0 = __uint_as_float(DQ_ELEM(i));
      const float a1 = __uint_as_float(DQ_ELEM(i + 64));
      sq[i] = a0 * a0 + a1 * a1;
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) sq[i] = sq[i] + sq[i + w];
    const float S = sq[0];

    // y = H * D * x: signs from SplitMix64 words 2g, 2g + 1, then fp32
    // butterflies of width 1, 2, ..., 64
    const uint64_t s0 = splitmix64(t.seed, 2ull * (uint64_t)g);
    const uint64_t s1 = splitmix64(t.seed, 2ull * (uint64_t)g + 1ull);
    float y[kD];
#pragma unroll
    for (int i = 0; i < kD; ++i) {
      const uint64_t sw = i < 64 ? s0 : s1;
      const uint32_t flip = (uint32_t)((sw >> (i & 63)) & 1ull) << 31;
      y[i] = __uint_as_float(DQ_ELEM(i) ^ flip);
    }
#undef DQ_ELEM
#pragma unroll
    for (int w = 1; w < kD; w <<= 1)
#pragma unroll
      for (int i = 0; i < kD; ++i)
        if ((i & w) == 0) {
          const float p = y[i], q = y[i + w];
          y[i] = p + q;
          y[i + w] = p - q;
        }

    const uint32_t nh = norm_half(S);
    const float nf = half_to_float(nh);
    const bool zero = nh == 0u;
    const bool bad = (nh & 0x7C00u) == 0x7C00u;
    const bool degenerate = zero || bad;

    // quantise: m_i = #{k in 1..h-1 : |y_i| >= k * step * n_h}; each
    // threshold is an integer times an fp16 value times 2^-6, exact in fp32
    Vec v;
    float thr[MAXH];
#pragma unroll
    for (int k = 1; k < MAXH; ++k)
      thr[k] = (k < h && !degenerate) ? (float)(k * t.step64) * nf * 0.015625f : __builtin_inff();
    int ge[MAXH];
#pragma unroll
    for (int k = 0; k < MAXH; ++k) ge[k] = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) v.sym0[j] = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) v.fl[j] = 0u;
#pragma unroll
    for (int i = 0; i < kD; ++i) {
      const float ay = degenerate ? 0.0f : __builtin_fabsf(y[i]);
      v.ay[i] = ay;
      uint32_t m = 0;
#pragma unroll
      for (int k = 1; k < MAXH; ++k) {
        const uint32_t c = ay >= thr[k] ? 1u : 0u;
        m += c;
        ge[k] += (int)c;
      }
      const uint32_t sy = (degenerate || y[i] >= 0.0f) ? (uint32_t)h + m : (uint32_t)(h - 1) - m;
      v.sym0[i >> 3] |= sy << (4 * (i & 7));
    }
    // current symbols into the lane's LDS column
    uint8_t *symL = symcol;
#pragma unroll
    for (int i = 0; i < kD; ++i) symL[i * kThreads + lane] = (uint8_t)nib(v.sym0, i);

    // ---- drift search: a per-lane state machine around one rANS pass.
    // Passes alternate between the two scratch buffers, so the last fitting
    // stream is still there after a trial pass that does not fit.
    int buf = 1, okbuf = -1, okB = 0;
    uint32_t okx = 0;
    int moves = 0, passes = 0, k = 0, total = 0, gb = 0, taken = 0;
    int cnt[MAXH];
#pragma unroll
    for (int m = 0; m < MAXH; ++m) cnt[m] = 0;
    uint32_t gm[4] = {0u, 0u, 0u, 0u};
    bool first_round = true;
    int phase = kPhInit;
    for (int guard = 0; phase != kPhDone && guard < 4 * kD; ++guard) {
      uint32_t xf;
      buf ^= 1;
      const int B = rans_pass(symL, etab, scr[buf], lane, &xf);
      const bool fits = 4 + B <= C;
      if (fits) {
        okbuf = buf;
        okB = B;
        okx = xf;
      }
      int act = kActNone;
      if (phase == kPhInit) {
        if (fits) {
          phase = kPhDone;
        } else {
          // group sizes and the estimated number of moves: shed the excess
          // bits greedily in drift order at each group's per-move saving
          float sigma_c = 0.0f;
          total = 0;
          if (first_round) {
#pragma unroll
            for (int m = 0; m < MAXH; ++m) {
              const int above = (m + 1 < MAXH) ? ge[m + 1] : 0;
              const int c = (m == 0 ? kD : ge[m]) - above;
              if (m >= 1) cnt[m] = c;
              if (m < h) sigma_c += (float)c * t.cost[h + m];
            }
          } else {
#pragma unroll
            for (int m = 1; m < MAXH; ++m) cnt[m] = 0;
#pragma unroll
            for (int i = 0; i < kD; ++i) {
              const uint32_t mg = magnitude(nib(v.sym0, i), h);
#pragma unroll
              for (int m = 1; m < MAXH; ++m) cnt[m] += mg == (uint32_t)m ? 1 : 0;
            }
            int c0 = kD;
#pragma unroll
            for (int m = 1; m < MAXH; ++m) {
              c0 -= cnt[m];
              if (m < h) sigma_c += (float)cnt[m] * t.cost[h + m];
            }
            sigma_c += (float)c0 * t.cost[h];
          }
#pragma unroll
          for (int m = 1; m < MAXH; ++m) total += cnt[m];
          float need = sigma_c - 8.0f * (float)(C - 4) - 4.0f;
          int khat = 0;
#pragma unroll
          for (int m = MAXH - 1; m >= 1; --m) {
            if (m < h && need > 0.0f) {
              const float sv = t.saving[m];
              int take = (int)ceilf(need / sv);
              take = take < cnt[m] ? take : cnt[m];
              khat += take;
              need -= (float)take * sv;
            }
          }
          khat = khat < 1 ? 1 : (khat > total ? total : khat);
          k = khat > 1 ? khat - 1 : 1;
          act = kActPrefix;
          phase = kPhFirst;
        }
      } else if (phase == kPhFirst || phase == kPhDown) {
        if (fits) {
          if (k == 1) {
            phase = kPhDone;
          } else {
            act = kActRemove;  // try one candidate fewer
            phase = kPhDown;
          }
        } else if (phase == kPhDown) {
          ++k;  // prefix k - 1 failed: the previous pass (prefix k) is the answer
          phase = kPhDone;
        } else {
          act = kActAdd;
          phase = kPhUp;
        }
      } else {  // kPhUp
        if (fits) phase = kPhDone;
        else act = kActAdd;
      }
      if (act == kActAdd && k >= total) act = kActCommit;

      if (act == kActPrefix) {
        // first k candidates: whole groups above the boundary, then the
        // smallest members of the boundary group
        int kk = k, rest = 0;
        bool full = false;
        gb = h - 1;
#pragma unroll
        for (int m = MAXH - 1; m >= 1; --m) {
          if (m < h && kk > 0) {
            gb = m;
            if (kk >= cnt[m]) {
              kk -= cnt[m];
              full = true;
              rest = cnt[m];
            } else {
              full = false;
              rest = kk;
              kk = 0;
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) v.fl[j] = 0u;
#pragma unroll
        for (int i = 0; i < kD; ++i) {
          const uint32_t s0 = nib(v.sym0, i);
          const uint32_t mg = magnitude(s0, h);
          const bool f = mg > (uint32_t)gb || (full && mg == (uint32_t)gb);
          v.fl[i >> 5] |= (f ? 1u : 0u) << (i & 31);
          symL[i * kThreads + lane] = (uint8_t)(f ? (s0 >= (uint32_t)h ? s0 - 1u : s0 + 1u) : s0);
        }
        group_mask(v, h, gb, gm);
        taken = rest;
        if (!full)
          for (int j = 0; j < rest; ++j) toggle(v, symL, extreme_in_group(v, gm, false), h, false, lane);
      } else if (act == kActAdd || act == kActRemove) {
        const bool add = act == kActAdd;
        // move the boundary when the current boundary group has nothing left
        if (add ? (taken == cnt_at<MAXH>(cnt, gb)) : (taken == 0)) {
          int m = add ? gb - 1 : gb + 1;
          while (add ? (m > 1 && cnt_at<MAXH>(cnt, m) == 0) : (m < h - 1 && cnt_at<MAXH>(cnt, m) == 0))
            m += add ? -1 : 1;
          gb = m;
          taken = add ? 0 : cnt_at<MAXH>(cnt, gb);
          group_mask(v, h, gb, gm);
        }
        toggle(v, symL, extreme_in_group(v, gm, !add), h, !add, lane);
        taken += add ? 1 : -1;
        k += add ? 1 : -1;
      } else if (act == kActCommit) {
        // every candidate moved and the stream still does not fit: keep the
        // moves and search again on the new symbols (the all-innermost
        // vector always fits)
        moves += total;
        ++passes;
#pragma unroll
        for (int i = 0; i < kD; ++i) {
          const uint32_t s0 = nib(v.sym0, i);
          const uint32_t sn = bit(v.fl, i) ? (s0 >= (uint32_t)h ? s0 - 1u : s0 + 1u) : s0;
          v.sym0[i >> 3] = (v.sym0[i >> 3] & ~(15u << (4 * (i & 7)))) | (sn << (4 * (i & 7)));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) v.fl[j] = 0u;
        k = 0;
        first_round = false;
        phase = kPhInit;
      }
    }
    if (phase == kPhDone) moves += k;

    // container: [final state, little endian][renorm bytes][zero pad]
    if (in_pool && okbuf >= 0) {
      uint8_t *dst = a.cont + ((int64_t)g * a.num_slots + slot) * C;
      dst[0] = (uint8_t)okx;
      dst[1] = (uint8_t)(okx >> 8);
      dst[2] = (uint8_t)(okx >> 16);
      dst[3] = (uint8_t)(okx >> 24);
      const uint8_t *sb = scr[okbuf];
      for (int j = 0; j < C - 4; ++j) dst[4 + j] = j < okB ? sb[(kScr - okB + j) * kThreads + lane] : (uint8_t)0;
      a.norm[(int64_t)g * a.num_slots + slot] = (uint16_t)nh;
    }

    if (a.stats) {
      atomicAdd(&bstat[0], 1u);
      if (moves) {
        atomicAdd(&bstat[1], 1u);
        atomicAdd(&bstat[2], (uint32_t)moves);
      }
      if (passes) atomicAdd(&bstat[3], (uint32_t)passes);
      if (bad) atomicAdd(&bstat[4], 1u);
      if (zero) atomicAdd(&bstat[5], 1u);
      atomicAdd(&bstat[6 + 4 + okB], 1u);
    }
  }
  if (a.stats) {
    __syncthreads();
    unsigned long long *gs = reinterpret_cast<unsigned long long *>(a.stats);
    for (int q = lane; q < 6 + kMaxC + 1; q += kThreads)
      if (bstat[q]) atomicAdd(gs + q, (unsigned long long)bstat[q]);
  }
}

// ---------------------------------------------------------------------------
// Small batches (a decode step appends one token per sequence): one wave per
// vector, so the latency is a single rANS pass instead of a serial search.
//  - rotation and norm cooperatively: lane l holds coordinates l and l + 64;
//    the butterflies of width 1..32 pair lanes l and l ^ w, width 64 pairs
//    the two values in a lane (the same fp32 operations in the same order as
//    the per-lane path); the sum of squares follows the same halving tree;
//  - every drift candidate gets its rank in the drift order (magnitude
//    descending, |y| ascending, index ascending) by a broadcast scan;
//  - lane l runs the rANS pass with the first k0 + l candidates moved one
//    level inward; the lowest lane whose stream fits is the answer (the
//    length never increases along the order, so every lower lane failed).
constexpr int kWaveVecs = 4;  // vectors (waves) per block

__global__ void __launch_bounds__(64 * kWaveVecs) encode_wave_kernel(EncodeArgs a, Tables t) {
  __shared__ uint4 etab[kMaxLevels];
  __shared__ uint32_t ent[kWaveVecs][kD];          // s0 | sd << 8 | rank << 16
  __shared__ float yabs[kWaveVecs][kD];
  __shared__ uint8_t mag[kWaveVecs][kD];
  __shared__ uint8_t scr[kWaveVecs][kScr * 64];   // renorm bytes, lane-minor
  const int tid = threadIdx.x;
  if (tid < t.levels) {
    const uint32_t f = t.freq[tid];
    etab[tid] = make_uint4(f << 19, t.magic[tid], t.cum[tid], (kM - f) | ((uint32_t)t.shift[tid] << 16));
  }
  __syncthreads();
  const int w = tid >> 6, lane = tid & 63;
  const int64_t nvec = a.T * (int64_t)t.hkv;
  const int64_t vid = (int64_t)blockIdx.x * kWaveVecs + w;
  if (vid >= nvec) return;  // whole wave exits together
  const int h = t.half, C = t.C;
  const int g = (int)(vid / a.T);
  const int64_t tok = vid - (int64_t)g * a.T;
  const int64_t slot = a.slots[tok];
  const uint16_t *xp = a.x + tok * a.stride_t + (int64_t)g * a.stride_h;
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
  const uint64_t s0w = splitmix64(t.seed, 2ull * (uint64_t)g);
  const uint64_t s1w = splitmix64(t.seed, 2ull * (uint64_t)g + 1ull);
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
  uint32_t *E = ent[w];
  float *Y = yabs[w];
  uint8_t *Mg = mag[w];
  uint8_t *scol = scr[w];

  int moves = 0, passes = 0, okB = 0;
  uint32_t okx = 0;
  int win = -1;
  for (int outer = 0; outer < 2 * kD && win < 0; ++outer) {
    // ranks of the candidates (magnitude >= 1) in drift order
    Mg[lane] = (uint8_t)mA[0];
    Mg[lane + 64] = (uint8_t)mA[1];
    Y[lane] = yA[0];
    Y[lane + 64] = yA[1];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int rank[2] = {0, 0};
    for (int j = 0; j < kD; ++j) {
      const uint32_t mj = Mg[j];
      const float yj = Y[j];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = lane + 64 * e;
        const bool before = mj >= 1u && (mj > mA[e] || (mj == mA[e] && (yj < yA[e] || (yj == yA[e] && j < i))));
        rank[e] += before ? 1 : 0;
      }
    }
    int total = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) total += __popcll(__ballot(mA[e] >= 1u));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t sd = mA[e] >= 1u ? (sA[e] >= (uint32_t)h ? sA[e] - 1u : sA[e] + 1u) : sA[e];
      const uint32_t rk = mA[e] >= 1u ? (uint32_t)rank[e] : 255u;
      E[lane + 64 * e] = sA[e] | (sd << 8) | (rk << 16);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int k0 = 0; k0 <= total && win < 0; k0 += 64) {
      const uint32_t k = (uint32_t)(k0 + lane);
      uint32_t x = kLow;
      int pos = kScr - 1;
      for (int i = kD - 1; i >= 0; --i) {
        const uint32_t en = E[i];
        const uint32_t s = ((en >> 16) & 0xFFu) < k ? ((en >> 8) & 0xFFu) : (en & 0xFFu);
        const uint4 c = etab[s];
        scol[pos * 64 + lane] = (uint8_t)x;
        const bool emit = x >= c.x;
        x = emit ? x >> 8 : x;
        pos -= emit ? 1 : 0;
        const uint32_t q = __umulhi(x, c.y) >> (c.w >> 16);
        x = x + c.z + __umul24(q, c.w & 0xFFFFu);
      }
      const int B = kScr - 1 - pos;
      const bool fits = 4 + B <= C && (int)k <= total;
      const uint64_t vote = __ballot(fits);
      if (vote) {
        win = __ffsll((unsigned long long)vote) - 1;
        okB = __shfl(B, win);
        okx = (uint32_t)__shfl((int)x, win);
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

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (win >= 0 && slot >= 0 && slot < a.num_slots) {
    uint8_t *dst = a.cont + ((int64_t)g * a.num_slots + slot) * C;
    for (int j = lane; j < C; j += 64) {
      uint8_t b;
      if (j < 4) b = (uint8_t)(okx >> (8 * j));
      else b = (j - 4 < okB) ? scol[(kScr - okB + (j - 4)) * 64 + win] : (uint8_t)0;
      dst[j] = b;
    }
    if (lane == 0) a.norm[(int64_t)g * a.num_slots + slot] = (uint16_t)nh;
  }
  if (a.stats && lane == 0) {
    unsigned long long *gs = reinterpret_cast<unsigned long long *>(a.stats);
    atomicAdd(gs + 0, 1ull);
    if (moves) {
      atomicAdd(gs + 1, 1ull);
      atomicAdd(gs + 2, (unsigned long long)moves);
    }
    if (passes) atomicAdd(gs + 3, (unsigned long long)passes);
    if (bad) atomicAdd(gs + 4, 1ull);
    if (zero) atomicAdd(gs + 5, 1ull);
    atomicAdd(gs + 6 + 4 + okB, 1ull);
  }
}

constexpr int64_t kWavePathMax = 16384;  // vectors: below this, latency wins

template <int MAXH>
hipError_t launch(const EncodeArgs &a, const Tables &t, hipStream_t s) {
  const int64_t nvec = a.T * (int64_t)t.hkv;
  const unsigned blocks = (unsigned)((nvec + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(encode_kernel<MAXH>, dim3(blocks), dim3(kThreads), 0, s, a, t);
  return hipGetLastError();
}

}  // namespace
}  // namespace dq

extern "C" int dq_encode(dq_codec_t codec, const void *x, int64_t T, int64_t stride_t,
                         int64_t stride_h, const int64_t *slots, int64_t num_slots,
                         uint8_t *cont, uint16_t *norm, dq_stats *stats,
                         dq_stream_t stream) {
  if (!codec || T < 0) return DQ_ERR_INVALID;
  if (T == 0) return DQ_OK;
  if (!x || !slots || !cont || !norm || num_slots < 1) return DQ_ERR_INVALID;
  const dq::Tables &t = codec->t;
  // 16-byte vector loads: the base and both strides must keep rows aligned
  if ((reinterpret_cast<uintptr_t>(x) & 15u) || (stride_t & 7) || (stride_h & 7) || stride_t < 0 ||
      stride_h < 0)
    return DQ_ERR_INVALID;
  if (T > ((int64_t)1 << 40) / t.hkv || num_slots > ((int64_t)1 << 40) / t.C) return DQ_ERR_INVALID;
  dq::EncodeArgs a{static_cast<const uint16_t *>(x), T, stride_t, stride_h, slots, num_slots,
                   cont, norm, stats};
  hipStream_t s = static_cast<hipStream_t>(stream);
  // DQ_ENCODE_WAVE_MAX overrides the batch size (vectors) up to which the
  // wave-per-vector kernel runs; both kernels write identical bytes
  int64_t wave_max = dq::kWavePathMax;
  if (const char *ev = getenv("DQ_ENCODE_WAVE_MAX")) wave_max = atoll(ev);
  hipError_t e;
  if (T * (int64_t)t.hkv <= wave_max && T * (int64_t)t.hkv <= ((int64_t)1 << 30)) {
    const int64_t nvec = T * (int64_t)t.hkv;
    hipLaunchKernelGGL(dq::encode_wave_kernel, dim3((unsigned)((nvec + dq::kWaveVecs - 1) / dq::kWaveVecs)),
                       dim3(64 * dq::kWaveVecs), 0, s, a, t);
    e = hipGetLastError();
  } else {
    e = t.half <= 4 ? dq::launch<4>(a, t, s) : dq::launch<8>(a, t, s);
  }
  return e == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}
