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
// the 128 coordinates in VGPRs (fully unrolled butterflies); the symbols and
// the renorm bytes then live in LDS, lane-minor ([i][lane]), so the serial
// rANS chain of every lane reads symbol i of all lanes from one contiguous
// 128-byte row.  Lanes of a wave take consecutive tokens of one kv head, so
// their containers are adjacent in the pool.  The drift search is a per-lane
// state machine around a single rANS pass, so lanes that need more passes
// simply stay active while the others idle.
//
// Arithmetic that decides a symbol is fp32 in a fixed order (butterfly
// widths 1..64, halving-tree sum of squares); the build uses
// -ffp-contract=off and keeps denormals, so the result is reproducible
// bit for bit.
#include <hip/hip_runtime.h>

#include "dq_internal.h"

namespace dq {
namespace {

constexpr int kThreads = 128;
constexpr int kScr = 128;  // renorm bytes per lane: at most one per symbol

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

// Per-lane view of one vector during the drift search.
struct Vec {
  float ay[kD];      // |y_i|: drift order within a magnitude group
  uint32_t mag[16];  // magnitude cell m_i, 4 bits each
  uint32_t neg[4];   // 1: y_i < 0
  uint32_t fl[4];    // 1: coordinate moved one level inward
};

// Writes the current symbols (base symbols with the drift flags applied) to
// the lane's LDS column.
__device__ __forceinline__ void materialize(const Vec &v, int h, uint8_t *sym, int lane) {
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    const uint32_t m = nib(v.mag, i) - bit(v.fl, i);
    const uint32_t s = bit(v.neg, i) ? (uint32_t)(h - 1) - m : (uint32_t)h + m;
    sym[i * kThreads + lane] = (uint8_t)s;
  }
}

// Flags the not-yet-flagged member of magnitude group g with the smallest
// (|y|, index) and updates its LDS symbol; false if the group has none left.
__device__ __forceinline__ bool add_smallest(Vec &v, uint32_t g, int h, uint8_t *sym, int lane) {
  float best = __builtin_inff();
  int bi = -1;
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    const bool take = nib(v.mag, i) == g && !bit(v.fl, i) && (bi < 0 || v.ay[i] < best);
    best = take ? v.ay[i] : best;
    bi = take ? i : bi;
  }
  if (bi < 0) return false;
#pragma unroll
  for (int j = 0; j < 4; ++j) v.fl[j] |= ((bi >> 5) == j) ? (1u << (bi & 31)) : 0u;
  // one level inward: toward the innermost pair (h - 1, h)
  const uint32_t s = sym[bi * kThreads + lane];
  sym[bi * kThreads + lane] = (uint8_t)(s >= (uint32_t)h ? s - 1u : s + 1u);
  (void)h;
  return true;
}

// Flags exactly the first k candidates of the drift order (magnitude
// descending, then |y| ascending, then index ascending) and materialises
// the symbols.  Returns the group holding the k-th candidate.
template <int MAXH>
__device__ __forceinline__ uint32_t set_prefix(Vec &v, const int (&cnt)[MAXH], int k, int h, uint8_t *sym, int lane) {
  v.fl[0] = v.fl[1] = v.fl[2] = v.fl[3] = 0u;
  uint32_t gb = (uint32_t)(h - 1);
  int rest = 0;
#pragma unroll
  for (int m = MAXH - 1; m >= 1; --m) {
    if (m < h && k > 0) {
      gb = (uint32_t)m;
      if (k >= cnt[m]) {
#pragma unroll
        for (int i = 0; i < kD; ++i) v.fl[i >> 5] |= (nib(v.mag, i) == (uint32_t)m ? 1u : 0u) << (i & 31);
        k -= cnt[m];
      } else {
        rest = k;
        k = 0;
      }
    }
  }
  materialize(v, h, sym, lane);
  for (int j = 0; j < rest; ++j) add_smallest(v, gb, h, sym, lane);
  return gb;
}

template <int MAXH>
__device__ __forceinline__ int count_at(const int (&cnt)[MAXH], int m) {
  int r = 0;
#pragma unroll
  for (int q = 1; q < MAXH; ++q) r = q == m ? cnt[q] : r;
  return r;
}

// One rANS pass over the lane's current symbols (pushed 127 -> 0).  Renorm
// bytes go to the lane's scratch column from the end backwards, so rows
// kScr - B .. kScr - 1 are already in the decoder's reading order.
__device__ __forceinline__ int rans_pass(const uint4 *etab, const uint8_t *sym, uint8_t *scr, int lane,
                                         uint32_t *xfinal) {
  uint32_t x = kLow;
  int pos = kScr - 1;
  for (int i = kD - 1; i >= 0; --i) {
    const uint32_t s = sym[i * kThreads + lane];
    const uint4 e = etab[s];  // {f << 19, magic, cum, (4096 - f) | shift << 16}
    if (x >= e.x) {
      scr[pos * kThreads + lane] = (uint8_t)x;
      --pos;
      x >>= 8;
    }
    const uint32_t q = __umulhi(x, e.y) >> (e.w >> 16);
    x = x + e.z + __umul24(q, e.w & 0xFFFFu);
  }
  *xfinal = x;
  return kScr - 1 - pos;
}

enum : int { kPhInit = 0, kPhFirst = 1, kPhDown = 2, kPhUp = 3, kPhFinal = 4, kPhDone = 5 };
enum : int { kActNone = 0, kActPrefix = 1, kActNext = 2, kActCommit = 3 };

template <int MAXH>
__global__ void __launch_bounds__(kThreads) encode_kernel(EncodeArgs a, Tables t) {
  __shared__ uint4 etab[kMaxLevels];
  __shared__ uint8_t sym[kD * kThreads];
  __shared__ uint8_t scr[kScr * kThreads];
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
    for (int j = 0; j < 16; ++j) v.mag[j] = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v.neg[j] = 0u;
      v.fl[j] = 0u;
    }
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
      v.mag[i >> 3] |= m << (4 * (i & 7));
      v.neg[i >> 5] |= ((degenerate || y[i] >= 0.0f) ? 0u : 1u) << (i & 31);
    }
    materialize(v, h, sym, lane);

    // drift search: a per-lane state machine around one rANS pass.  Each
    // iteration runs the pass on the current symbols, records the result if
    // it is the candidate answer, and picks one action for the symbols.
    int cnt[MAXH];
    cnt[0] = 0;
    int total = 0;
    int k = 0, moves = 0, passes = 0, B = 0;
    uint32_t gb = 0, xfin = 0;
    int phase = kPhInit;
    int guard = 0;  // bounded: every lane leaves the loop (search needs < 3 * 128 passes)
    while (phase != kPhDone && ++guard < 1024) {
      uint32_t xf;
      const int Bp = rans_pass(etab, sym, scr, lane, &xf);
      const bool fits = 4 + Bp <= C;
      int act = kActNone;
      if (phase == kPhInit) {
        if (fits) {
          B = Bp;
          xfin = xf;
          phase = kPhDone;
        } else {
          // group sizes and the estimated number of moves: shed the excess
          // bits greedily in drift order using the per-move savings
          float sigma_c = 0.0f;
          total = 0;
#pragma unroll
          for (int m = 0; m < MAXH; ++m) {
            const int above = (m + 1 < MAXH) ? ge[m + 1] : 0;
            const int c = (m == 0 ? kD : ge[m]) - above;
            if (m < h) sigma_c += (float)c * t.cost[h + m];
            if (m >= 1) {
              cnt[m] = c;
              total += c;
            }
          }
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
          // prefix k fits: try one shorter while possible
          B = Bp;
          xfin = xf;
          if (k == 1) {
            phase = kPhDone;
          } else {
            --k;
            act = kActPrefix;
            phase = kPhDown;
          }
        } else if (phase == kPhDown) {
          // prefix k + 1 was the shortest that fits: redo it (scratch)
          ++k;
          act = kActPrefix;
          phase = kPhFinal;
        } else {
          act = kActNext;
          phase = kPhUp;
        }
      } else if (phase == kPhFinal) {
        B = Bp;
        xfin = xf;
        phase = kPhDone;
      } else {  // kPhUp: prefix k did not fit before this pass added one
        if (fits) {
          B = Bp;
          xfin = xf;
          phase = kPhDone;
        } else {
          act = kActNext;
        }
      }
      if (act == kActNext && k >= total) act = kActCommit;
      if (act == kActPrefix) {
        gb = set_prefix<MAXH>(v, cnt, k, h, sym, lane);
      } else if (act == kActNext) {
        // next candidate: the boundary group's smallest unflagged member,
        // else the next non-empty group inward
        if (!add_smallest(v, gb, h, sym, lane)) {
          int m = (int)gb - 1;
          while (m > 1 && count_at<MAXH>(cnt, m) == 0) --m;
          gb = (uint32_t)m;
          add_smallest(v, gb, h, sym, lane);
        }
        ++k;
      } else if (act == kActCommit) {
        // every candidate moved and the stream still does not fit: commit
        // and search again on the new symbols (the all-innermost vector
        // always fits)
        moves += total;
        ++passes;
#pragma unroll
        for (int i = 0; i < kD; ++i) v.mag[i >> 3] -= bit(v.fl, i) << (4 * (i & 7));
#pragma unroll
        for (int q = 1; q < MAXH; ++q) ge[q] = 0;
#pragma unroll
        for (int i = 0; i < kD; ++i) {
          const uint32_t m = nib(v.mag, i);
#pragma unroll
          for (int q = 1; q < MAXH; ++q) ge[q] += m >= (uint32_t)q ? 1 : 0;
        }
        v.fl[0] = v.fl[1] = v.fl[2] = v.fl[3] = 0u;
        k = 0;
        materialize(v, h, sym, lane);
        phase = kPhInit;
      }
    }
    moves += k;

    // container: [final state, little endian][renorm bytes][zero pad]
    if (in_pool) {
    uint8_t *dst = a.cont + ((int64_t)g * a.num_slots + slot) * C;
    dst[0] = (uint8_t)xfin;
    dst[1] = (uint8_t)(xfin >> 8);
    dst[2] = (uint8_t)(xfin >> 16);
    dst[3] = (uint8_t)(xfin >> 24);
    for (int j = 0; j < C - 4; ++j) dst[4 + j] = j < B ? scr[(kScr - B + j) * kThreads + lane] : (uint8_t)0;
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
      atomicAdd(&bstat[6 + 4 + B], 1u);
    }
  }
  if (a.stats) {
    __syncthreads();
    unsigned long long *gs = reinterpret_cast<unsigned long long *>(a.stats);
    for (int q = lane; q < 6 + kMaxC + 1; q += kThreads)
      if (bstat[q]) atomicAdd(gs + q, (unsigned long long)bstat[q]);
  }
}

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
  hipError_t e = t.half <= 4 ? dq::launch<4>(a, t, s) : dq::launch<8>(a, t, s);
  return e == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}
