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
// Two kernels write the same bytes:
//  - encode_kernel (large batches, e.g. a prompt): one lane owns one vector
//    end to end.  The rotation runs on the 128 coordinates in VGPRs (fully
//    unrolled butterflies); the symbols are packed 4 bits each in
//    registers.  The drift is planned before any pass from the ideal code
//    length, which decides whether a prefix of moves fits except inside a
//    band narrower than one move's saving; then one rANS pass runs, or two
//    when the undecided prefix is tried first.  Renorm bytes go to the
//    lane's column of an LDS scratch.  Lanes of a wave take consecutive
//    tokens of one kv head, so their containers are adjacent in the pool.
//  - encode_wave_kernel (small batches, e.g. one appended token per
//    sequence): one wave owns one vector, so the batch fills the chip with
//    waves instead of lanes and the serial search becomes one parallel
//    pass: lane l tries the first k0 + l candidates.
//
// Arithmetic that decides a symbol is fp32 in a fixed order (butterfly
// widths 1..64, halving-tree sum of squares); the build uses
// -ffp-contract=off and keeps denormals, so the result is reproducible
// bit for bit.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "dq_internal.h"
#include "encode_wave.h"

namespace dq {
namespace {

constexpr int kThreads = 128;
constexpr int kScr = 128;  // renorm bytes per lane and buffer: at most one per symbol
// In-group selection keys: the offset of |y| bits above the group threshold
// is clamped to a span (at most kKeySpan, so keys fit 32 bits); a clamped
// key is (span + 1) * 128 + index, above every unclamped one.  Inner groups
// never clamp at the full span: their |y| spans at most a factor 2, 2^23
// bits of offset.  The outermost group's could reach 16 times its
// threshold only for a norm rounded far down in fp16's subnormal range.
constexpr uint32_t kKeySpan = (1u << 25) - 2u;

struct EncodeArgs {
  const uint16_t *x;
  int64_t T, stride_t, stride_h;
  const int64_t *slots;
  int64_t num_slots;
  uint8_t *cont;
  uint16_t *norm;
  dq_stats *stats;
  uint32_t key_span;  // in-group key span; smaller values only to test the float-scan fallback
};

__device__ __forceinline__ uint32_t nib(const uint32_t (&w)[16], int i) {
  return (w[i >> 3] >> (4 * (i & 7))) & 15u;
}
__device__ __forceinline__ uint32_t bit(const uint32_t (&w)[4], int i) {
  return (w[i >> 5] >> (i & 31)) & 1u;
}
__device__ __forceinline__ uint32_t magnitude(uint32_t s, int h) {
  return s >= (uint32_t)h ? s - (uint32_t)h : (uint32_t)(h - 1) - s;
}

// The smallest (|y|, index) among the members of gm not yet in fl, -1 if
// none: the next candidate of a magnitude group in drift order.  Every |y|
// is finite, so starting from +inf needs no "found yet" test, and the strict
// compare keeps the lowest index among equal values.  The two halves are
// scanned separately so every index is an inline constant (0..63); on a tie
// the lower half wins.
__device__ __forceinline__ int next_in_group(const float (&ay)[kD], const uint32_t (&gm)[4],
                                             const uint32_t (&fl)[4]) {
  uint32_t mw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) mw[q] = gm[q] & ~fl[q];
  float best[2];
  int bi[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    best[half] = __builtin_inff();
    bi[half] = -1;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const int i = 64 * half + j;
      const bool take = ((mw[i >> 5] >> (i & 31)) & 1u) && ay[i] < best[half];
      best[half] = take ? ay[i] : best[half];
      bi[half] = take ? j : bi[half];
    }
  }
  return best[1] < best[0] ? 64 + bi[1] : bi[0];
}

// The candidate not yet in fl with the smallest (key, index), for the
// rate-distortion order: rk holds each candidate's key as sortable bits
// (below 2^32 - 1) and ~0 for the other coordinates; a taken candidate's
// key is masked to ~0.  Halves as in next_in_group, so indices are inline
// constants and a tie goes to the lower index.
__device__ __forceinline__ int next_by_key(const uint32_t (&rk)[kD], const uint32_t (&fl)[4]) {
  uint32_t best[2];
  int bi[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    best[half] = ~0u;
    bi[half] = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const int i = 64 * half + j;
      const uint32_t v = rk[i] | (uint32_t)__builtin_amdgcn_sbfe((int)fl[i >> 5], i & 31, 1);
      const bool take = v < best[half];
      best[half] = take ? v : best[half];
      bi[half] = take ? j : bi[half];
    }
  }
  return best[1] < best[0] ? 64 + bi[1] : bi[0];
}

// One rANS pass over the packed symbols (pushed 127 -> 0).  Renorm bytes go
// to the lane's scratch column from the end backwards (rows kScr - B ..
// kScr - 1 are then in the decoder's reading order); the byte store is
// unconditional and simply overwritten when no byte is emitted.  The coder
// constants do not depend on the state, so their loads run ahead of it.
__device__ __forceinline__ int rans_pass(const uint32_t (&sym)[16], const uint4 *etab, uint8_t *buf, int lane,
                                         uint32_t *xfinal) {
  uint32_t x = kLow;
  int pos = kScr - 1;
#pragma unroll
  for (int i = kD - 1; i >= 0; --i) {
    const uint4 e = etab[nib(sym, i)];  // {f << 19, magic, cum, (4096 - f) | shift << 16}
    buf[pos * kThreads + lane] = (uint8_t)x;
    const bool emit = x >= e.x;
    x = emit ? x >> 8 : x;
    pos -= emit ? 1 : 0;
    const uint32_t q = __umulhi(x, e.y) >> (e.w >> 16);
    x = x + e.z + __umul24(q, e.w & 0xFFFFu);
    if ((i & 7) == 0) __builtin_amdgcn_sched_barrier(0);  // loads run at most 8 steps ahead
  }
  *xfinal = x;
  return kScr - 1 - pos;
}


// Makes the packed words opaque to the compiler, so nibbles extracted in one
// region are not kept alive for reuse in the next one.
template <int N>
__device__ __forceinline__ void opaque(uint32_t (&w)[N]) {
#pragma unroll
  for (int j = 0; j < N; ++j) asm volatile("" : "+v"(w[j]));
}

// y = H * D * x for one bf16 vector: signs from the SplitMix64 words (made
// opaque so the 128 sign masks are not hoisted out of a loop), then fp32
// butterflies of width 1, 2, ..., 64.  With S != nullptr also ||x||^2 by the
// halving tree (i + 64, then i + 32, ..., i + 1).
__device__ __forceinline__ void rotate(const uint4 *src, uint64_t s0, uint64_t s1, float (&y)[kD], float *S) {
  uint32_t xw[64];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint4 w = src[j];
    xw[4 * j + 0] = w.x;
    xw[4 * j + 1] = w.y;
    xw[4 * j + 2] = w.z;
    xw[4 * j + 3] = w.w;
  }
  opaque(xw);  // a second rotation of the same vector is recomputed, not reused
  // bf16 element i as fp32 bits
#define DQ_ELEM(i) ((xw[(i) >> 1] << (16 * (1 - ((i) & 1)))) & 0xFFFF0000u)
  if (S) {
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
    *S = sq[0];
  }
  uint32_t sgn[4] = {(uint32_t)s0, (uint32_t)(s0 >> 32), (uint32_t)s1, (uint32_t)(s1 >> 32)};
  opaque(sgn);
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    const uint32_t flip = ((sgn[i >> 5] >> (i & 31)) & 1u) << 31;
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
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ uint32_t inward(uint32_t s, int h) { return s >= (uint32_t)h ? s - 1u : s + 1u; }

// Moves packed symbol i (a per-lane index) one level inward: its word is
// picked out by selects, updated, and put back by selects.
__device__ __forceinline__ void move_inward(uint32_t (&sym)[16], int i, int h) {
  const int wi = i >> 3, sh = 4 * (i & 7);
  uint32_t w = sym[0];
#pragma unroll
  for (int j = 1; j < 16; ++j) w = wi == j ? sym[j] : w;
  const uint32_t sv = (w >> sh) & 15u;
  w = (w & ~(15u << sh)) | (inward(sv, h) << sh);
#pragma unroll
  for (int j = 0; j < 16; ++j) sym[j] = wi == j ? w : sym[j];
}

constexpr int kStatWords = 6 + kMaxC + 1;  // per-block stats, flushed once

// The block's coder tables (and rate-distortion terms when RD), stats zeroed.
template <bool RD>
__device__ __forceinline__ void block_setup(const Tables &t, uint4 *etab, float2 *rdtab, uint32_t *bstat,
                                            int lane) {
  if (lane < t.levels) {
    const uint32_t f = t.freq[lane];
    etab[lane] = make_uint4(f << 19, t.magic[lane], t.cum[lane], (kM - f) | ((uint32_t)t.shift[lane] << 16));
  }
  if (RD && lane < kMaxHalf)
    rdtab[lane] = (lane >= 1 && lane < t.half)
                      ? make_float2(half_to_float(t.recon[t.half + lane]) + half_to_float(t.recon[t.half + lane - 1]),
                                    t.rd_w[lane])
                      : make_float2(0.0f, 0.0f);
  for (int k = lane; k < kStatWords; k += kThreads) bstat[k] = 0u;
  __syncthreads();
}

__device__ __forceinline__ void flush_stats(const EncodeArgs &a, const uint32_t *bstat, int lane) {
  if (a.stats) {
    __syncthreads();
    unsigned long long *gs = reinterpret_cast<unsigned long long *>(a.stats);
    for (int q = lane; q < kStatWords; q += kThreads)
      if (bstat[q]) atomicAdd(gs + q, (unsigned long long)bstat[q]);
  }
}

// The serial encode of vector vid by one lane, drift search included; lane
// is also its column of the renorm scratch.  Stats go to the block's bstat.
template <int MAXH, bool RD>  // RD: rate-distortion drift order
__device__ __forceinline__ void encode_vector(const EncodeArgs &a, const Tables &t, int64_t vid,
                                              const uint4 *etab, const float2 *rdtab, uint8_t *scr,
                                              uint32_t *bstat, int lane) {
  const int h = t.half;
  const int C = t.C;
  {
    const int g = (int)(vid / a.T);
    const int64_t tok = vid - (int64_t)g * a.T;
    const int64_t slot = a.slots[tok];
    const bool in_pool = slot >= 0 && slot < a.num_slots;  // out-of-range slots write nothing
    const uint4 *src = reinterpret_cast<const uint4 *>(a.x + tok * a.stride_t + (int64_t)g * a.stride_h);
    const uint64_t s0 = dev_splitmix64(t.seed, 2ull * (uint64_t)g);
    const uint64_t s1 = dev_splitmix64(t.seed, 2ull * (uint64_t)g + 1ull);

    // ---- drift.  I(k), the ideal code length of the symbols after the
    // first k moves (sum of log2(4096 / f), fixed point), decides whether
    // prefix k fits except inside a band narrower than one move's saving
    // (kEpsHiFx, kEpsLoFx), so at most one k per round is undecided.  The
    // plan and the choice of the moved symbols come first; then one rANS
    // pass, or two when the undecided prefix is tried first.  A round in
    // which even every move is too long commits them and plans again (rare:
    // the rotated coordinates are recomputed then, so they are not kept
    // through the passes).
    const uint32_t lim = (uint32_t)(8 * (C - 3)) << kCostFrac;
    const uint32_t sure_lo = lim - kEpsHiFx;  // I(k) below: fits
    const uint32_t sure_hi = lim + kEpsLoFx;  // I(k) at or above: does not fit
    uint32_t sym0[16];                        // symbols at the start of the round, 4 bits each
    int cnt[MAXH];                            // candidates per magnitude in the round
    uint32_t I = 0u;
    uint32_t nh = 0u;
    bool zero = false, bad = false;
    int moves = 0, passes = 0, okB = -1;
    uint32_t okx = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) sym0[j] = 0u;
#pragma unroll
    for (int m = 0; m < MAXH; ++m) cnt[m] = 0;

    for (int round = 0; okB < 0 && round <= MAXH; ++round) {
      if (round == 0) {
        float y[kD], S;
        rotate(src, s0, s1, y, &S);
        nh = norm_half(S);
        zero = nh == 0u;
        bad = (nh & 0x7C00u) == 0x7C00u;
        const bool degenerate = zero || bad;
        // quantise: m_i = #{k in 1..h-1 : |y_i| >= k * step * n_h}; each
        // threshold is an integer times an fp16 value times 2^-6, exact in fp32
        const float nf = half_to_float(nh);
        float thr[MAXH];
#pragma unroll
        for (int k = 1; k < MAXH; ++k)
          thr[k] = (k < h && !degenerate) ? (float)(k * t.step64) * nf * 0.015625f : __builtin_inff();
        // magnitude histogram: 8-bit counters, m = 0..3 in hl, 4..7 in hh
        uint32_t hl = 0u, hh = 0u;
#pragma unroll
        for (int i = 0; i < kD; ++i) {
          const float ay = degenerate ? 0.0f : __builtin_fabsf(y[i]);
          uint32_t m = 0;
#pragma unroll
          for (int k = 1; k < MAXH; ++k) m += ay >= thr[k] ? 1u : 0u;
          const uint32_t inc = 1u << (8 * (m & 3u));
          hl += m < 4u ? inc : 0u;
          hh += m < 4u ? 0u : inc;
          const uint32_t sy = (degenerate || y[i] >= 0.0f) ? (uint32_t)h + m : (uint32_t)(h - 1) - m;
          sym0[i >> 3] |= sy << (4 * (i & 7));
          if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);  // one packed word at a time
        }
#pragma unroll
        for (int m = 0; m < MAXH; ++m) {
          const int c = (int)(((m < 4 ? hl : hh) >> (8 * (m & 3))) & 0xFFu);
          if (m >= 1) cnt[m] = c;
          if (m < h) I += (uint32_t)c * t.cost_fx[h + m];
        }
      }

      opaque(sym0);
      int ks = 0, total = 0;
      uint32_t Ik = I, Iprev = 0xFFFFFFFFu;  // I(ks), I(ks - 1)
      if constexpr (!RD) {
      // plan: the smallest k with I(k) < sure_lo takes whole magnitude
      // groups, outermost first, each move saving saving_fx[m]
#pragma unroll
      for (int m = MAXH - 1; m >= 1; --m) {
        if (m < h) {
          total += cnt[m];
          if (Ik >= sure_lo && cnt[m] > 0) {
            const uint32_t sv = t.saving_fx[m];
            const uint32_t need = (Ik - sure_lo) / sv + 1u;
            const uint32_t take = need < (uint32_t)cnt[m] ? need : (uint32_t)cnt[m];
            Iprev = Ik - (take - 1u) * sv;
            Ik -= take * sv;
            ks += (int)take;
          }
        }
      }
      const bool sure = Ik < sure_lo;
      const bool undecided = sure ? (ks >= 1 && Iprev < sure_hi) : (Ik < sure_hi);

      if (sure || undecided) {
        // the first k candidates: whole groups above the boundary group gb,
        // then its `rest` smallest members; `nxt` is candidate k + 1 when
        // the undecided prefix k is tried first
        const int k = undecided ? (sure ? ks - 1 : total) : ks;
        int kk = k, rest = 0, gb = h - 1;
        bool full = false;
#pragma unroll
        for (int m = MAXH - 1; m >= 1; --m) {
          if (m < h && kk > 0) {
            gb = m;
            full = kk >= cnt[m];
            rest = full ? cnt[m] : kk;
            kk -= rest;
          }
        }
        uint32_t fl[4] = {0u, 0u, 0u, 0u}, gm[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kD; ++i) {
          const uint32_t mg = magnitude(nib(sym0, i), h);
          fl[i >> 5] |= (mg > (uint32_t)gb || (full && mg == (uint32_t)gb) ? 1u : 0u) << (i & 31);
          gm[i >> 5] |= (mg == (uint32_t)gb ? 1u : 0u) << (i & 31);
        }
        int nxt = -1;
        const bool want_next = undecided && sure;
        // The order inside a group needs |y|: the rotation runs again rather
        // than keep 128 values alive since quantisation.  The boundary
        // group's members first become integer keys, (|y| bits above the
        // bits of the group's threshold) * 128 + 128 + index, 0 for the
        // other coordinates.  Keys order as (|y|, index) do, so an
        // extraction is one subtract and a minimum per coordinate.  The
        // float scans remain for what the keys cannot rank: a next candidate
        // from a lower group, and |y| far enough above the threshold that
        // its key saturates (possible only in the outermost group).
        bool scan = want_next && (full || rest == cnt[gb]);
        const int want = full ? 0 : rest + (want_next && !scan ? 1 : 0);
        int got = 0;
        if (want > 0) {
          opaque(sym0);
          float ay[kD];
          rotate(src, s0, s1, ay, nullptr);
          // the threshold of the members' magnitude before the rounds that
          // moved every candidate, computed as quantisation did
          const float nf = half_to_float(nh);
          const uint32_t blo = __float_as_uint((float)((gb + passes) * t.step64) * nf * 0.015625f);
          const uint32_t span = a.key_span, sat = (span << 7) + 128u;  // keys >= sat are clamped
          uint32_t key[kD];
#pragma unroll
          for (int i = 0; i < kD; ++i) {
            const uint32_t d = (__float_as_uint(ay[i]) & 0x7FFFFFFFu) - blo;  // members: |y| >= threshold
            const uint32_t kv = (min(d, span) << 7) + (128u + (uint32_t)i);
            const uint32_t mask = (uint32_t)__builtin_amdgcn_sbfe((int)gm[i >> 5], i & 31, 1);
            key[i] = kv & mask;
          }
          uint32_t p1 = 1u;  // every key taken so far is below p1
          for (int j = 0; j < want; ++j) {
            // min over (key - p1) mod 2^32: a member not yet taken gives key
            // - p1 < 2^32 - p1, the others give at least 2^32 - p1
            uint32_t best = ~0u;
#pragma unroll
            for (int i = 0; i < kD; i += 2) best = min(best, min(key[i] - p1, key[i + 1] - p1));
            const uint32_t kw = best + p1;
            if (kw == 0u || kw >= sat) {
              scan = true;
              break;
            }
            p1 = kw + 1u;
            const int i = (int)(kw & 127u);
            if (j < rest) {
#pragma unroll
              for (int q = 0; q < 4; ++q) fl[q] |= ((i >> 5) == q) ? (1u << (i & 31)) : 0u;
              ++got;
            } else {
              nxt = i;
            }
          }
        }
        if (scan) {
          opaque(sym0);
          opaque(fl);
          float ay[kD];
          rotate(src, s0, s1, ay, nullptr);
#pragma unroll
          for (int i = 0; i < kD; ++i) ay[i] = __builtin_fabsf(ay[i]);
          if (!full)
            for (int j = got; j < rest; ++j) {
              const int i = next_in_group(ay, gm, fl);
#pragma unroll
              for (int q = 0; q < 4; ++q) fl[q] |= ((i >> 5) == q) ? (1u << (i & 31)) : 0u;
            }
          if (want_next) {
            if (full || rest == cnt[gb]) {
              // the boundary group is used up: the next lower non-empty group
              int m = k == 0 ? h - 1 : gb - 1;
              while (m > 1 && cnt[m] == 0) --m;
#pragma unroll
              for (int i = 0; i < kD; ++i) {
                const uint32_t mg = magnitude(nib(sym0, i), h);
                gm[i >> 5] = (gm[i >> 5] & ~(1u << (i & 31))) | ((mg == (uint32_t)m ? 1u : 0u) << (i & 31));
              }
            }
            nxt = next_in_group(ay, gm, fl);
          }
        }
        opaque(sym0);
        opaque(fl);
        // symbols of prefix k
        uint32_t sym[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) sym[j] = 0u;
#pragma unroll
        for (int i = 0; i < kD; ++i) {
          const uint32_t s = nib(sym0, i);
          sym[i >> 3] |= (bit(fl, i) ? inward(s, h) : s) << (4 * (i & 7));
        }
        for (int attempt = 0; attempt < 2; ++attempt) {
          uint32_t xf;
          const int B = rans_pass(sym, etab, scr, lane, &xf);
          if (4 + B <= C) {
            okB = B;
            okx = xf;
            moves += k + attempt;
            break;
          }
          if (nxt < 0) break;
          // prefix k did not fit: prefix k + 1 does
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int sh = 4 * (nxt & 7);
            const uint32_t s = (sym[j] >> sh) & 15u;
            sym[j] = ((nxt >> 3) == j) ? ((sym[j] & ~(15u << sh)) | (inward(s, h) << sh)) : sym[j];
          }
          nxt = -1;
        }
      }
      } else {
        // Rate-distortion order: candidates (m >= 1) ascending in the key
        // (2|y| - n (l_m + l_{m-1})) * w_m, then in index, so the groups
        // interleave.  I(every move) decides first whether any prefix can
        // fit; otherwise candidates are taken in key order, each saving
        // saving_fx[m], until I(k) < sure_lo.
        uint32_t Iall = I;
#pragma unroll
        for (int m = 1; m < MAXH; ++m)
          if (m < h) {
            total += cnt[m];
            Iall -= (uint32_t)cnt[m] * t.saving_fx[m];
          }
        uint32_t fl[4] = {0u, 0u, 0u, 0u};
        int k = 0, nxt = -1;
        bool go = true;
        if (I < sure_lo) {
          // fits as it is
        } else if (Iall >= sure_hi) {
          go = false;  // not even every move fits
          Ik = Iall;
        } else if (Iall >= sure_lo) {
          // only the prefix of every move can fit
          k = total;
          Ik = Iall;
#pragma unroll
          for (int i = 0; i < kD; ++i) fl[i >> 5] |= (magnitude(nib(sym0, i), h) >= 1u ? 1u : 0u) << (i & 31);
        } else {
          opaque(sym0);
          float ay[kD];
          rotate(src, s0, s1, ay, nullptr);
          const float nf = half_to_float(nh);
          uint32_t rk[kD];
#pragma unroll
          for (int i = 0; i < kD; ++i) {
            const uint32_t mg = magnitude(nib(sym0, i), h);
            const float2 rr = rdtab[mg];
            const float tt = nf * rr.x;  // exact: 11 x 12 significant bits
            const float key = (2.0f * __builtin_fabsf(ay[i]) - tt) * rr.y;
            const uint32_t kb = __float_as_uint(key + 0.0f);  // -0 -> +0
            const uint32_t lo = (kb & 0x80000000u) ? ~kb : (kb | 0x80000000u);
            rk[i] = mg >= 1u ? lo : ~0u;
          }
          int last = 0;
          do {  // ends by the last candidate: I(every move) < sure_lo
            const int c = next_by_key(rk, fl);
            // c's magnitude: its packed word by selects (c varies by lane)
            uint32_t w = sym0[0];
#pragma unroll
            for (int j = 1; j < 16; ++j) w = (c >> 3) == j ? sym0[j] : w;
            const uint32_t mc = magnitude((w >> (4 * (c & 7))) & 15u, h);
            uint32_t sv = 0u;
#pragma unroll
            for (int m = 1; m < MAXH; ++m) sv = mc == (uint32_t)m ? t.saving_fx[m] : sv;
            Iprev = Ik;
            Ik -= sv;
#pragma unroll
            for (int q = 0; q < 4; ++q) fl[q] |= ((c >> 5) == q) ? (1u << (c & 31)) : 0u;
            ++k;
            last = c;
          } while (Ik >= sure_lo);
          if (Iprev < sure_hi) {
            // prefix k - 1 may fit too: it is tried first
#pragma unroll
            for (int q = 0; q < 4; ++q) fl[q] &= ((last >> 5) == q) ? ~(1u << (last & 31)) : ~0u;
            nxt = last;
            --k;
          }
        }
        if (go) {
          opaque(sym0);
          opaque(fl);
          uint32_t sym[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) sym[j] = 0u;
#pragma unroll
          for (int i = 0; i < kD; ++i) {
            const uint32_t s = nib(sym0, i);
            sym[i >> 3] |= (bit(fl, i) ? inward(s, h) : s) << (4 * (i & 7));
          }
          for (int attempt = 0; attempt < 2; ++attempt) {
            uint32_t xf;
            const int B = rans_pass(sym, etab, scr, lane, &xf);
            if (4 + B <= C) {
              okB = B;
              okx = xf;
              moves += k + attempt;
              break;
            }
            if (nxt < 0) break;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int sh = 4 * (nxt & 7);
              const uint32_t s = (sym[j] >> sh) & 15u;
              sym[j] = ((nxt >> 3) == j) ? ((sym[j] & ~(15u << sh)) | (inward(s, h) << sh)) : sym[j];
            }
            nxt = -1;
          }
        }
      }
      if (okB < 0) {
        // every candidate of the round moves one level inward; the plan is
        // made again on the new symbols (the all-innermost vector fits)
        moves += total;
        ++passes;
        opaque(sym0);
#pragma unroll
        for (int i = 0; i < kD; ++i) {
          const uint32_t s = nib(sym0, i);
          const uint32_t sn = magnitude(s, h) >= 1u ? inward(s, h) : s;
          sym0[i >> 3] = (sym0[i >> 3] & ~(15u << (4 * (i & 7)))) | (sn << (4 * (i & 7)));
        }
#pragma unroll
        for (int m = 1; m < MAXH; ++m) cnt[m] = (m + 1 < MAXH) ? cnt[m + 1] : 0;
        I = Ik;
      }
    }

    // container: [final state, little endian][renorm bytes][zero pad]
    if (in_pool && okB >= 0) {
      uint8_t *dst = a.cont + ((int64_t)g * a.num_slots + slot) * C;
      dst[0] = (uint8_t)okx;
      dst[1] = (uint8_t)(okx >> 8);
      dst[2] = (uint8_t)(okx >> 16);
      dst[3] = (uint8_t)(okx >> 24);
      for (int j = 0; j < C - 4; ++j) dst[4 + j] = j < okB ? scr[(kScr - okB + j) * kThreads + lane] : (uint8_t)0;
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
      atomicAdd(&bstat[6 + 4 + (okB < 0 ? 0 : okB)], 1u);
    }
  }
}

// Single pass: one lane per vector, the drift search inline.
template <int MAXH, bool RD>
__global__ void __launch_bounds__(kThreads, 2) encode_kernel(EncodeArgs a, Tables t) {
  __shared__ uint4 etab[kMaxLevels];
  __shared__ float2 rdtab[kMaxHalf];        // {l_m + l_{m-1}, w_m}; entry 0 unused
  __shared__ uint8_t scr[kScr * kThreads];  // renorm bytes, lane-minor
  __shared__ uint32_t bstat[kStatWords];
  const int lane = threadIdx.x;
  block_setup<RD>(t, etab, rdtab, bstat, lane);
  const int64_t nvec = a.T * (int64_t)t.hkv;
  const int64_t vid = (int64_t)blockIdx.x * kThreads + lane;
  if (vid < nvec) encode_vector<MAXH, RD>(a, t, vid, etab, rdtab, scr, bstat, lane);
  flush_stats(a, bstat, lane);
}

// Quantisation of the rotated coordinates against thresholds thr[1..NK]
// (the magnitude is the count of those |y| reaches), packed 4 bits per
// symbol, with the magnitude histogram as 8-bit counters (m = 0..3 in hl,
// 4..7 in hh).
template <int NK, int MAXH>
__device__ __forceinline__ void quantize(const float (&y)[kD], const float (&thr)[MAXH], int h, bool degenerate,
                                         uint32_t (&sym0)[16], uint32_t &hl, uint32_t &hh) {
#pragma unroll
  for (int j = 0; j < 16; ++j) sym0[j] = 0u;
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    const float ay = __builtin_fabsf(y[i]);
    uint32_t m = 0;
#pragma unroll
    for (int k = 1; k <= NK; ++k) m += ay >= thr[k] ? 1u : 0u;
    const uint32_t inc = 1u << (8 * (m & 3u));
    if (NK < 4) {
      hl += inc;
    } else {
      hl += m < 4u ? inc : 0u;
      hh += m < 4u ? 0u : inc;
    }
    const uint32_t sy = (degenerate || y[i] >= 0.0f) ? (uint32_t)h + m : (uint32_t)(h - 1) - m;
    sym0[i >> 3] |= sy << (4 * (i & 7));
    // finish each packed word and the counts here: otherwise the compiler
    // keeps all 128 magnitudes, and y for their signs
    if ((i & 7) == 7) asm volatile("" : "+v"(sym0[i >> 3]), "+v"(hl), "+v"(hh));
  }
}

// Two passes for large batches.  encode_vector keeps neither the rotated
// coordinates nor the plan across its rounds: its in-group order needs |y|
// again, so it rotates a second time, and a wave runs every path that one of
// its lanes takes.  Nearly every value vector and about half the keys drift
// at the default widths, so:
//  - encode_fast_kernel runs round 0 of the search with y kept in registers
//    from the first rotation: the plan, the in-group keys made from y, the
//    one or two rANS passes.  The cases it leaves are rare: a vector whose
//    round 0 cannot fit (more rounds), a key at the span's clamp.  Those
//    in-pool vectors get kPendingNorm in their norm slot;
//  - encode_rest_kernel gathers the pending vectors of 8192 consecutive
//    ones into a list and runs encode_vector on it.  Vectors outside the
//    pool write nothing either way; with stats, the second pass counts them.
// Round 0 makes the same choices in the same order as encode_vector, so
// bytes, norms and stats are those of encode_kernel.  (Slots of one call are
// distinct: with a slot given twice, which vector's container remains is
// unspecified, as in one pass, and the stats may count only that one.)
constexpr uint16_t kPendingNorm = 0xFFFFu;  // never a norm: norm_half gives NaN as 0x7E00
constexpr int kRestRange = 8192;            // vectors per encode_rest_kernel block

// NK: the thresholds quantisation tests (h - 1 when the launch knows h,
// as for 6 levels; MAXH - 1 covers every h up to MAXH)
template <int MAXH, bool RD, int NK = MAXH - 1>
__global__ void __launch_bounds__(kThreads, 2) encode_fast_kernel(EncodeArgs a, Tables t) {
  __shared__ uint4 etab[kMaxLevels];
  __shared__ float2 rdtab[kMaxHalf];
  __shared__ uint8_t scr[kScr * kThreads];
  __shared__ uint32_t bstat[kStatWords];
  const int lane = threadIdx.x;
  block_setup<RD>(t, etab, rdtab, bstat, lane);
  const int h = t.half;
  const int C = t.C;
  const int64_t nvec = a.T * (int64_t)t.hkv;
  const int64_t vid = (int64_t)blockIdx.x * kThreads + lane;
  if (vid < nvec) {
    const int g = (int)(vid / a.T);
    const int64_t tok = vid - (int64_t)g * a.T;
    const int64_t slot = a.slots[tok];
    if (slot >= 0 && slot < a.num_slots) {
      const uint4 *src = reinterpret_cast<const uint4 *>(a.x + tok * a.stride_t + (int64_t)g * a.stride_h);
      const uint64_t s0 = dev_splitmix64(t.seed, 2ull * (uint64_t)g);
      const uint64_t s1 = dev_splitmix64(t.seed, 2ull * (uint64_t)g + 1ull);
      float y[kD], S;
      rotate(src, s0, s1, y, &S);
      const uint32_t nh = norm_half(S);
      const bool zero = nh == 0u;
      const bool bad = (nh & 0x7C00u) == 0x7C00u;
      const bool degenerate = zero || bad;
      // quantisation and the magnitude histogram, as in encode_vector; a
      // degenerate vector's thresholds are NaN, so every |y| (inf too)
      // compares below them: all magnitudes 0, as encode_vector's |y| = 0
      const float nf = half_to_float(nh);
      float thr[MAXH];
#pragma unroll
      for (int k = 1; k < MAXH; ++k)
        thr[k] = degenerate ? __builtin_nanf("")
                            : (k < h ? (float)(k * t.step64) * nf * 0.015625f : __builtin_inff());
      uint32_t sym0[16];
      uint32_t hl = 0u, hh = 0u;
      quantize<NK>(y, thr, h, degenerate, sym0, hl, hh);
      int cnt[MAXH];
      uint32_t I = 0u;
#pragma unroll
      for (int m = 0; m < MAXH; ++m) {
        const int c = (int)(((m < 4 ? hl : hh) >> (8 * (m & 3))) & 0xFFu);
        cnt[m] = m >= 1 ? c : 0;
        if (m < h) I += (uint32_t)c * t.cost_fx[h + m];
      }
      const uint32_t lim = (uint32_t)(8 * (C - 3)) << kCostFrac;
      const uint32_t sure_lo = lim - kEpsHiFx;
      const uint32_t sure_hi = lim + kEpsLoFx;

      // round 0 of the search: the moved candidates fl, their count k, and
      // nxt, the one more tried second when prefix k is undecided
      bool pending = false;
      uint32_t sym[16];  // the symbols of prefix k
#pragma unroll
      for (int j = 0; j < 16; ++j) sym[j] = 0u;
      int k = 0, nxt = -1, total = 0;
      uint32_t Ik = I, Iprev = 0xFFFFFFFFu;
      if constexpr (!RD) {
        int ks = 0;
#pragma unroll
        for (int m = MAXH - 1; m >= 1; --m) {
          if (m < h) {
            total += cnt[m];
            if (Ik >= sure_lo && cnt[m] > 0) {
              const uint32_t sv = t.saving_fx[m];
              const uint32_t need = (Ik - sure_lo) / sv + 1u;
              const uint32_t take = need < (uint32_t)cnt[m] ? need : (uint32_t)cnt[m];
              Iprev = Ik - (take - 1u) * sv;
              Ik -= take * sv;
              ks += (int)take;
            }
          }
        }
        const bool sure = Ik < sure_lo;
        const bool undecided = sure ? (ks >= 1 && Iprev < sure_hi) : (Ik < sure_hi);
        pending = !(sure || undecided);  // every move of the round is too long
        k = undecided ? (sure ? ks - 1 : total) : ks;
        int kk = k, rest = 0, gb = h - 1;
        bool full = false;
#pragma unroll
        for (int m = MAXH - 1; m >= 1; --m) {
          if (m < h && kk > 0) {
            gb = m;
            full = kk >= cnt[m];
            rest = full ? cnt[m] : kk;
            kk -= rest;
          }
        }
        const bool want_next = undecided && sure;
        // When the undecided prefix uses up the boundary group, the next
        // candidate is the smallest |y| of the next lower non-empty group
        // (encode_vector's float scan): every member of the boundary group
        // moves, and the keys are made for that lower group (kg) instead,
        // so one extraction gives it.  No such group: the second kernel.
        const bool scan = want_next && (full || rest == cnt[gb]);
        int kg = gb;
        if (scan) {
          const int start = k == 0 ? h - 1 : gb - 1;
          bool found = false;
#pragma unroll
          for (int m = MAXH - 1; m >= 1; --m)
            if (!found && m <= start && cnt[m] > 0) {
              kg = m;
              found = true;
            }
          pending = pending || !found;
        }
        const bool whole = full || scan;  // the boundary group moves whole
        const int taken = scan ? 0 : rest;  // members taken in key order
        const int want = pending ? 0 : (scan ? 1 : (full ? 0 : rest + (want_next ? 1 : 0)));
        // one pass: the symbols with the whole-group moves applied, and the
        // key group's in-group keys made from y, as encode_vector makes them
        // from its second rotation (the same bits); 0 for the others
        const uint32_t blo = __float_as_uint((float)(kg * t.step64) * nf * 0.015625f);
        const uint32_t span = a.key_span, sat = (span << 7) + 128u;  // keys >= sat are clamped
        uint32_t key[kD];
        if constexpr (MAXH == 4) {
          // up to 8 levels, symbols below 8: eight nibbles of a packed word
          // at a time.  Per nibble, t = s + 8 - h has bit 3 iff s >= h, and
          // its low 3 bits give the magnitude (s - h, or h - 1 - s flipped
          // from them); a symbol moves iff its magnitude >= gb + (full ? 0
          // : 1), one level inward (s + 1 below h, s - 1 from h on).  No
          // nibble carries into the next: every sum stays below 16.
          const uint32_t hb = 0x11111111u * (uint32_t)(8 - h);
          const uint32_t tb = 0x11111111u * (uint32_t)(8 - (whole ? gb : gb + 1));
          const uint32_t gbb = 0x11111111u * (uint32_t)kg;
          // 2 (|y| bits - blo): the shift drops y's sign bit; exact for
          // members, whose |y| >= the threshold; keys as in the other loop
          const uint32_t nblo2 = 0u - (blo << 1), span2 = span << 1;
#pragma unroll
          for (int w = 0; w < 16; ++w) {
            const uint32_t x = sym0[w];
            const uint32_t tt = x + hb;
            const uint32_t gen = (tt >> 3) & 0x11111111u;  // 1 where s >= h
            const uint32_t ltn = gen ^ 0x11111111u;        // 1 where s < h
            const uint32_t mag = (tt ^ ((ltn << 3) - ltn)) & 0x77777777u;
            const uint32_t mv = ((mag + tb) >> 3) & 0x11111111u;
            sym[w] = x + (mv & ltn) - (mv & gen);
            // bit 3 of each nibble: magnitude == kg (z == 0)
            const uint32_t z = mag ^ gbb;
            const uint32_t eq = ~((z | 0x88888888u) - 0x11111111u) & 0x88888888u;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int i = 8 * w + j;
              const uint32_t dd = min((__float_as_uint(y[i]) << 1) + nblo2, span2);
              key[i] = ((dd << 6) + (128u + (uint32_t)i)) & (uint32_t)__builtin_amdgcn_sbfe((int)eq, 4 * j + 3, 1);
              asm volatile("" : "+v"(key[i]));  // made here, while eq is at hand
            }
            asm volatile("" : "+v"(sym[w]));
          }
        } else {
#pragma unroll
          for (int i = 0; i < kD; ++i) {
            const uint32_t sv = nib(sym0, i);
            const uint32_t mg = magnitude(sv, h);
            const bool move = mg > (uint32_t)gb || (whole && mg == (uint32_t)gb);
            sym[i >> 3] |= (move ? inward(sv, h) : sv) << (4 * (i & 7));
            const uint32_t d = (__float_as_uint(y[i]) & 0x7FFFFFFFu) - blo;  // members: |y| >= threshold
            key[i] = mg == (uint32_t)kg ? (min(d, span) << 7) + (128u + (uint32_t)i) : 0u;
            asm volatile("" : "+v"(key[i]));  // made here, while mg is at hand
            if ((i & 7) == 7) asm volatile("" : "+v"(sym[i >> 3]));
          }
        }
        uint32_t p1 = 1u;  // every key taken so far is below p1
        for (int j = 0; j < want; ++j) {
          // min over (key - p1) mod 2^32: a member not yet taken gives key
          // - p1 < 2^32 - p1, the others give at least 2^32 - p1
          uint32_t best = ~0u;
#pragma unroll
          for (int i = 0; i < kD; i += 2) best = min(best, min(key[i] - p1, key[i + 1] - p1));
          const uint32_t kw = best + p1;
          if (kw == 0u || kw >= sat) {
            pending = true;  // a clamped key: the float scan ranks it
            break;
          }
          p1 = kw + 1u;
          const int i = (int)(kw & 127u);
          if (j < taken) move_inward(sym, i, h);
          else nxt = i;
        }
      } else {
        uint32_t fl[4] = {0u, 0u, 0u, 0u};
        uint32_t Iall = I;
#pragma unroll
        for (int m = 1; m < MAXH; ++m)
          if (m < h) {
            total += cnt[m];
            Iall -= (uint32_t)cnt[m] * t.saving_fx[m];
          }
        if (I < sure_lo) {
          // fits as it is
        } else if (Iall >= sure_hi) {
          pending = true;  // not even every move fits: more rounds
        } else if (Iall >= sure_lo) {
          k = total;
#pragma unroll
          for (int i = 0; i < kD; ++i) fl[i >> 5] |= (magnitude(nib(sym0, i), h) >= 1u ? 1u : 0u) << (i & 31);
        } else {
          opaque(sym0);
          uint32_t rk[kD];
#pragma unroll
          for (int i = 0; i < kD; ++i) {
            const uint32_t mg = magnitude(nib(sym0, i), h);
            const float2 rr = rdtab[mg];
            const float tt = nf * rr.x;
            const float key = (2.0f * __builtin_fabsf(y[i]) - tt) * rr.y;
            const uint32_t kb = __float_as_uint(key + 0.0f);
            const uint32_t lo = (kb & 0x80000000u) ? ~kb : (kb | 0x80000000u);
            rk[i] = mg >= 1u ? lo : ~0u;
          }
          int last = 0;
          do {
            const int c = next_by_key(rk, fl);
            uint32_t w = sym0[0];
#pragma unroll
            for (int j = 1; j < 16; ++j) w = (c >> 3) == j ? sym0[j] : w;
            const uint32_t mc = magnitude((w >> (4 * (c & 7))) & 15u, h);
            uint32_t sv = 0u;
#pragma unroll
            for (int m = 1; m < MAXH; ++m) sv = mc == (uint32_t)m ? t.saving_fx[m] : sv;
            Iprev = Ik;
            Ik -= sv;
#pragma unroll
            for (int q = 0; q < 4; ++q) fl[q] |= ((c >> 5) == q) ? (1u << (c & 31)) : 0u;
            ++k;
            last = c;
          } while (Ik >= sure_lo);
          if (Iprev < sure_hi) {
#pragma unroll
            for (int q = 0; q < 4; ++q) fl[q] &= ((last >> 5) == q) ? ~(1u << (last & 31)) : ~0u;
            nxt = last;
            --k;
          }
        }
        opaque(sym0);
        opaque(fl);
#pragma unroll
        for (int i = 0; i < kD; ++i) {
          const uint32_t sv = nib(sym0, i);
          sym[i >> 3] |= (bit(fl, i) ? inward(sv, h) : sv) << (4 * (i & 7));
        }
      }

      int okB = -1, moves = 0;
      uint32_t okx = 0u;
      if (!pending) {
        for (int attempt = 0; attempt < 2; ++attempt) {
          uint32_t xf;
          const int B = rans_pass(sym, etab, scr, lane, &xf);
          if (4 + B <= C) {
            okB = B;
            okx = xf;
            moves = k + attempt;
            break;
          }
          if (nxt < 0) break;
          move_inward(sym, nxt, h);
          nxt = -1;
        }
      }
      const int64_t at = (int64_t)g * a.num_slots + slot;
      if (okB >= 0) {
        uint8_t *dst = a.cont + at * C;
        dst[0] = (uint8_t)okx;
        dst[1] = (uint8_t)(okx >> 8);
        dst[2] = (uint8_t)(okx >> 16);
        dst[3] = (uint8_t)(okx >> 24);
        for (int j = 0; j < C - 4; ++j) dst[4 + j] = j < okB ? scr[(kScr - okB + j) * kThreads + lane] : (uint8_t)0;
        a.norm[at] = (uint16_t)nh;
        if (a.stats) {
          atomicAdd(&bstat[0], 1u);
          if (moves) {
            atomicAdd(&bstat[1], 1u);
            atomicAdd(&bstat[2], (uint32_t)moves);
          }
          if (bad) atomicAdd(&bstat[4], 1u);
          if (zero) atomicAdd(&bstat[5], 1u);
          atomicAdd(&bstat[6 + 4 + okB], 1u);
        }
      } else {
        a.norm[at] = kPendingNorm;  // more rounds: the second pass
      }
    }
  }
  flush_stats(a, bstat, lane);
}

template <int MAXH, bool RD>
__global__ void __launch_bounds__(kThreads, 2) encode_rest_kernel(EncodeArgs a, Tables t) {
  __shared__ uint4 etab[kMaxLevels];
  __shared__ float2 rdtab[kMaxHalf];
  __shared__ uint8_t scr[kScr * kThreads];
  __shared__ uint32_t bstat[kStatWords];
  __shared__ uint16_t list[kRestRange];  // pending vectors, as offsets in the block's range
  __shared__ uint32_t nlist;
  const int lane = threadIdx.x;
  if (lane == 0) nlist = 0u;
  block_setup<RD>(t, etab, rdtab, bstat, lane);
  const int64_t nvec = a.T * (int64_t)t.hkv;
  const int64_t v0 = (int64_t)blockIdx.x * kRestRange;
  const int64_t v1 = min(v0 + (int64_t)kRestRange, nvec);
  // (head, token) of the range's first vector once; the others step from
  // it (no division per vector when a head holds at least a range), four
  // vectors per lane per round so that their loads overlap
  const int64_t g0 = v0 / a.T, r0 = v0 - g0 * a.T;
  constexpr int kU = 4;
  for (int64_t c = 0; c < v1 - v0; c += kU * kThreads) {
    int64_t slot[kU], head[kU];
    bool live[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t off = c + u * kThreads + lane;
      live[u] = off < v1 - v0;
      int64_t r = r0 + off, g = g0;
      if (a.T >= kRestRange) {
        if (r >= a.T) {  // the range spans at most two heads
          r -= a.T;
          ++g;
        }
      } else {
        g += r / a.T;
        r -= (r / a.T) * a.T;
      }
      head[u] = g;
      slot[u] = live[u] ? a.slots[r] : -1;
    }
    bool pend[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      pend[u] = live[u] && ((slot[u] >= 0 && slot[u] < a.num_slots)
                                ? a.norm[head[u] * a.num_slots + slot[u]] == kPendingNorm
                                : a.stats != nullptr);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // the wave's pending lanes take consecutive list entries
      const uint64_t m = __ballot(pend[u]);
      uint32_t base = 0u;
      if ((lane & 63) == 0 && m) base = atomicAdd(&nlist, (uint32_t)__popcll(m));
      base = (uint32_t)__shfl((int)base, 0);
      const uint32_t rank =
          __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (pend[u]) list[base + rank] = (uint16_t)(c + u * kThreads + lane);
    }
  }
  __syncthreads();
  const int n = (int)nlist;
  for (int j = 0; j < n; j += kThreads)
    if (j + lane < n) encode_vector<MAXH, RD>(a, t, v0 + list[j + lane], etab, rdtab, scr, bstat, lane);
  flush_stats(a, bstat, lane);
}

// ---------------------------------------------------------------------------
// Small batches (a decode step appends one token per sequence): one wave per
// vector, so the latency is a single rANS pass instead of a serial search.
//  - rotation and norm cooperatively: lane l holds coordinates l and l + 64;
//    the butterflies of width 1..32 pair lanes l and l ^ w, width 64 pairs
//    the two values in a lane (the same fp32 operations in the same order as
//    the per-lane path); the sum of squares follows the same halving tree;
//  - every drift candidate gets its rank in the drift order (magnitude
//    descending, |y| ascending, index ascending) from a bitonic sort of the
//    wave's 128 (key, index) pairs;
//  - lane l runs the rANS pass with the first k0 + l candidates moved one
//    level inward; the lowest lane whose stream fits is the answer (the
//    length never increases along the order, so every lower lane failed).
constexpr int kWaveVecs = 4;  // vectors (waves) per block

// One block's vectors (kWaveVecs of them) of a wave-per-vector encode; the
// block index is passed in so one launch can serve two streams (K and V).
template <bool RD>  // drift order: rate-distortion (true) or magnitude (false)
__device__ __forceinline__ void wave_encode_block(const EncodeArgs &a, const Tables &t, int64_t block) {
  __shared__ uint4 etab[kMaxLevels];
  __shared__ float2 rdtab[kMaxHalf];
  __shared__ uint32_t ent[kWaveVecs][kD];
  __shared__ __attribute__((aligned(16))) uint8_t mag[kWaveVecs][kD];  // read as words
  __shared__ uint8_t scr[kWaveVecs][kWaveScr * 64];
  __shared__ uint32_t bstat[6 + kMaxC + 1];  // per-block stats, flushed once
  const int tid = threadIdx.x;
  for (int k = tid; k < 6 + kMaxC + 1; k += 64 * kWaveVecs) bstat[k] = 0u;
  wave_encode_tables(t, etab, rdtab, tid);
  __syncthreads();
  const int w = tid >> 6, lane = tid & 63;
  const int64_t nvec = a.T * (int64_t)t.hkv;
  const int64_t vid = block * kWaveVecs + w;
  if (vid < nvec) {  // whole waves; every wave reaches the block barrier below
    const int g = (int)(vid / a.T);
    const int64_t tok = vid - (int64_t)g * a.T;
    const int64_t slot = a.slots[tok];
    const WaveEncodeScratch L{ent[w], mag[w], scr[w], kWaveScr};
    WaveEncodeResult r;
    wave_encode_vector<RD, false>(a.x + tok * a.stride_t + (int64_t)g * a.stride_h, g, t, etab, rdtab, L, lane, r);
    if (r.win >= 0 && slot >= 0 && slot < a.num_slots)
      wave_store_container(r, L, t.C, a.cont + ((int64_t)g * a.num_slots + slot) * t.C,
                           a.norm + (int64_t)g * a.num_slots + slot, lane);
    if (a.stats && lane == 0) {
      atomicAdd(&bstat[0], 1u);
      if (r.moves) {
        atomicAdd(&bstat[1], 1u);
        atomicAdd(&bstat[2], (uint32_t)r.moves);
      }
      if (r.passes) atomicAdd(&bstat[3], (uint32_t)r.passes);
      if (r.bad) atomicAdd(&bstat[4], 1u);
      if (r.zero) atomicAdd(&bstat[5], 1u);
      atomicAdd(&bstat[6 + 4 + r.okB], 1u);
    }
  }
  if (a.stats) {
    __syncthreads();
    unsigned long long *gs = reinterpret_cast<unsigned long long *>(a.stats);
    for (int q = tid; q < 6 + kMaxC + 1; q += 64 * kWaveVecs)
      if (bstat[q]) atomicAdd(gs + q, (unsigned long long)bstat[q]);
  }
}

template <bool RD>
__global__ void __launch_bounds__(64 * kWaveVecs) encode_wave_kernel(EncodeArgs a, Tables t) {
  wave_encode_block<RD>(a, t, blockIdx.x);
}

// K and V of the same tokens in one launch: blocks [0, nbk) take K, the
// rest V (a decode step's append is then one launch, not two).
template <bool RD>
__global__ void __launch_bounds__(64 * kWaveVecs) encode_wave_kv_kernel(EncodeArgs ak, Tables tk, EncodeArgs av,
                                                                        Tables tv, int64_t nbk) {
  if ((int64_t)blockIdx.x < nbk) wave_encode_block<RD>(ak, tk, blockIdx.x);
  else wave_encode_block<RD>(av, tv, blockIdx.x - nbk);
}

constexpr int64_t kWavePathMax = 16384;  // vectors: below this, latency wins

// One pass or two (DQ_KNOB_ENCODE_TWO_PASS: 0 one, 1 two; the library takes
// two); the bytes are the same.
template <int MAXH>
hipError_t launch(const EncodeArgs &a, const Tables &t, hipStream_t s) {
  const int64_t nvec = a.T * (int64_t)t.hkv;
  const unsigned blocks = (unsigned)((nvec + kThreads - 1) / kThreads);
  if (knob(DQ_KNOB_ENCODE_TWO_PASS) != 0) {
    const unsigned rest = (unsigned)((nvec + kRestRange - 1) / kRestRange);
    // 6 levels (h = 3) test two thresholds instead of MAXH - 1 = 3
    bool six = false;
    if constexpr (MAXH == 4) six = t.half == 3;
    if (t.order == 1) {
      if constexpr (MAXH == 4)
        if (six) hipLaunchKernelGGL((encode_fast_kernel<4, true, 2>), dim3(blocks), dim3(kThreads), 0, s, a, t);
      if (!six) hipLaunchKernelGGL((encode_fast_kernel<MAXH, true>), dim3(blocks), dim3(kThreads), 0, s, a, t);
      hipLaunchKernelGGL((encode_rest_kernel<MAXH, true>), dim3(rest), dim3(kThreads), 0, s, a, t);
    } else {
      if constexpr (MAXH == 4)
        if (six) hipLaunchKernelGGL((encode_fast_kernel<4, false, 2>), dim3(blocks), dim3(kThreads), 0, s, a, t);
      if (!six) hipLaunchKernelGGL((encode_fast_kernel<MAXH, false>), dim3(blocks), dim3(kThreads), 0, s, a, t);
      hipLaunchKernelGGL((encode_rest_kernel<MAXH, false>), dim3(rest), dim3(kThreads), 0, s, a, t);
    }
    return hipGetLastError();
  }
  if (t.order == 1) hipLaunchKernelGGL((encode_kernel<MAXH, true>), dim3(blocks), dim3(kThreads), 0, s, a, t);
  else hipLaunchKernelGGL((encode_kernel<MAXH, false>), dim3(blocks), dim3(kThreads), 0, s, a, t);
  return hipGetLastError();
}

}  // namespace
}  // namespace dq

// Validates a dq_encode call and fills its kernel arguments.
static int encode_args(dq_codec_t codec, const void *x, int64_t T, int64_t stride_t, int64_t stride_h,
                       const int64_t *slots, int64_t num_slots, uint8_t *cont, uint16_t *norm, dq_stats *stats,
                       dq::EncodeArgs *a) {
  if (!codec || T < 0) return DQ_ERR_INVALID;
  if (T == 0) return DQ_OK;
  if (!x || !slots || !cont || !norm || num_slots < 1) return DQ_ERR_INVALID;
  const dq::Tables &t = codec->t;
  // 16-byte vector loads: the base and both strides must keep rows aligned
  if ((reinterpret_cast<uintptr_t>(x) & 15u) || (stride_t & 7) || (stride_h & 7) || stride_t < 0 ||
      stride_h < 0)
    return DQ_ERR_INVALID;
  if (T > ((int64_t)1 << 40) / t.hkv || num_slots > ((int64_t)1 << 40) / t.C) return DQ_ERR_INVALID;
  // one lane per vector in blocks of kThreads: the grid bounds the batch
  if (T * (int64_t)t.hkv > ((int64_t)1 << 38)) return DQ_ERR_UNSUPPORTED;
  // DQ_KNOB_ENCODE_KEY_SPAN narrows the in-group keys' span so that the
  // float scans they fall back to run more often (same bytes either way)
  uint32_t span = dq::kKeySpan;
  const int64_t forced = dq::knob(DQ_KNOB_ENCODE_KEY_SPAN);
  if (forced >= 0) span = forced < (int64_t)dq::kKeySpan ? (uint32_t)forced : dq::kKeySpan;
  *a = dq::EncodeArgs{static_cast<const uint16_t *>(x), T, stride_t, stride_h, slots, num_slots, cont, norm, stats,
                      span};
  return DQ_OK;
}

// Does a batch of this codec take the wave-per-vector kernel?
// DQ_KNOB_ENCODE_WAVE_MAX overrides the batch size (vectors) up to which
// it does; both kernels write identical bytes.
static bool wave_path(const dq::Tables &t, int64_t T) {
  const int64_t forced = dq::knob(DQ_KNOB_ENCODE_WAVE_MAX);
  const int64_t wave_max = forced >= 0 ? forced : dq::kWavePathMax;
  const int64_t nvec = T * (int64_t)t.hkv;
  return nvec <= wave_max && nvec <= ((int64_t)1 << 30);
}

static hipError_t launch_encode(const dq::EncodeArgs &a, const dq::Tables &t, hipStream_t s) {
  if (wave_path(t, a.T)) {
    const int64_t nvec = a.T * (int64_t)t.hkv;
    const dim3 grid((unsigned)((nvec + dq::kWaveVecs - 1) / dq::kWaveVecs)), block(64 * dq::kWaveVecs);
    if (t.order == 1) hipLaunchKernelGGL(dq::encode_wave_kernel<true>, grid, block, 0, s, a, t);
    else hipLaunchKernelGGL(dq::encode_wave_kernel<false>, grid, block, 0, s, a, t);
    return hipGetLastError();
  }
  return t.half <= 4 ? dq::launch<4>(a, t, s) : dq::launch<8>(a, t, s);
}

extern "C" int dq_encode(dq_codec_t codec, const void *x, int64_t T, int64_t stride_t,
                         int64_t stride_h, const int64_t *slots, int64_t num_slots,
                         uint8_t *cont, uint16_t *norm, dq_stats *stats,
                         dq_stream_t stream) {
  dq::EncodeArgs a{};
  const int st = encode_args(codec, x, T, stride_t, stride_h, slots, num_slots, cont, norm, stats, &a);
  if (st || T == 0) return st;
  return launch_encode(a, codec->t, static_cast<hipStream_t>(stream)) == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

extern "C" int dq_encode_kv(dq_codec_t ck, dq_codec_t cv, const void *k, const void *v, int64_t T,
                            int64_t stride_t, int64_t stride_h, const int64_t *slots, int64_t num_slots,
                            uint8_t *k_cont, uint16_t *k_norm, uint8_t *v_cont, uint16_t *v_norm,
                            dq_stats *k_stats, dq_stats *v_stats, dq_stream_t stream) {
  if (!ck || !cv || ck->t.hkv != cv->t.hkv) return DQ_ERR_INVALID;
  dq::EncodeArgs ak{}, av{};
  int st = encode_args(ck, k, T, stride_t, stride_h, slots, num_slots, k_cont, k_norm, k_stats, &ak);
  if (st) return st;
  st = encode_args(cv, v, T, stride_t, stride_h, slots, num_slots, v_cont, v_norm, v_stats, &av);
  if (st || T == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dq::Tables &tk = ck->t, &tv = cv->t;
  if (wave_path(tk, T) && wave_path(tv, T) && tk.order == tv.order) {
    const int64_t nbk = (T * (int64_t)tk.hkv + dq::kWaveVecs - 1) / dq::kWaveVecs;
    const dim3 grid((unsigned)(2 * nbk)), block(64 * dq::kWaveVecs);
    if (tk.order == 1) hipLaunchKernelGGL(dq::encode_wave_kv_kernel<true>, grid, block, 0, s, ak, tk, av, tv, nbk);
    else hipLaunchKernelGGL(dq::encode_wave_kv_kernel<false>, grid, block, 0, s, ak, tk, av, tv, nbk);
    return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
  }
  if (launch_encode(ak, tk, s) != hipSuccess) return DQ_ERR_HIP;
  return launch_encode(av, tv, s) == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}
