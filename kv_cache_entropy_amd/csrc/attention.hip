// dq_attn_decode: GQA split-K decode attention over rANS containers.
//
// "D-Quant: Driftable Entropy Coding for KV Cache Quantization" (abstract):
// fixed-size per-token streams give attention regular, fixed-stride memory
// access and let it dequantise in parallel; "D-Quant: Entropy Coding Meets KV
// Cache at 2.26 Bits" (intro, So What): the entropy decoder runs inside the
// attention kernel.
//
// Two kernels on the caller's stream (three when a decode step's appended
// tokens are encoded by a launch of their own, append_encode_kernel):
//  1. attn_splitk: persistent waves; a work item is (sequence, kv head,
//     context chunk).  The item first rotates its own query, q~ = H * D_K *
//     q in fp32, kept as an fp16 hi/lo pair (hi + lo carries ~22 bits) in
//     the MFMA operand layout.  Because H * H = 128 I, q . khat = q~ . (n *
//     r(s)) / 128: scores are computed directly on the decoded levels, no
//     inverse rotation of K.  Per 64-token tile a wave copies the tile's K
//     and V containers (64 * C contiguous bytes each, fixed stride) into its
//     LDS slice with 16-byte loads; every lane then rANS-decodes one token's
//     container through an LDS table (slot -> f, slot - cum, fp16 level).
//     K: every 4 decoded symbols form the B operand of a 4x4x4 MFMA
//     (16 blocks = the wave's 64 tokens) against q~ (4 heads), so the decoded
//     keys never leave registers.  Online softmax in fp32 (exp2 domain).
//     V: decoded levels are written transposed into an LDS tile [dim][token]
//     and contracted with p * n_v (an fp16 hi/lo pair, so ~22 bits) by
//     4x4x4 MFMAs whose 16 blocks cover 64 dims.  Each item leaves
//     (m, l, acc[4][128]) in the workspace.
//  2. combine: log-sum-exp merge of an item's chunks, then the inverse
//     rotation D_V * H / 128 and the store.
// Chunked prefill (attn_prefill_shared_kernel, attn_prefill_kernel) reuses
// the decode pieces with many query rows per decoded tile.
#include "decode_common.h"
#include "encode_wave.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>
#include <utility>

namespace dq {
namespace {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
static_assert(kTile == DQ_PAGE_TOKENS, "a page is one attention tile");
constexpr int kVtStride = 66;    // halves per V-tile row: 33 dwords, spreads LDS banks
constexpr int kPass = 32;        // dims per V-tile pass (per-block prefill)
constexpr int kDPass = 16;       // dims per V-tile pass (decode attention)
constexpr int kPart = 132;       // floats per (item, head): acc[128], m, l, pad
constexpr int kLutBytes = 2 * kDecodeTableBytes;  // K and V decode tables
// K and V encoder constants of the append (etab, rdtab), static too
constexpr int kAppendLdsBytes = 2 * (kMaxLevels * 16 + kMaxHalf * 8);
constexpr int kStaticLds = kLutBytes + kAppendLdsBytes;
// Per-slot decode tables (slot -> {f, cum | fp16 level << 16}), 32 KB per
// codec: one LDS read per decode step instead of a byte read and a
// dependent entry read.
constexpr int kSlotTableBytes = (int)kM * 8;
constexpr int kSlotLds = 2 * kSlotTableBytes + 2 * kSymTabBytes + kAppendLdsBytes + 16;

struct AttnArgs {
  const uint16_t *q;
  int B, Hq, Hkv, group;
  const uint8_t *kc;
  const uint16_t *kn;
  const uint8_t *vc;
  const uint16_t *vn;
  int64_t S;
  const int64_t *seq_start;  // contiguous layout, or
  const int32_t *pages;      // [B][max_pages] 64-token page ids (paged layout)
  int max_pages;
  const int32_t *seq_len;
  float qk_scale;  // sm_scale * log2(e) / 128
  int chunk, nc;
  // decode split: chunk c covers tiles [c cq + min(c, cr), (c + 1) cq +
  // min(c + 1, cr)) of a sequence, so the nc chunks of a max_len sequence
  // differ by at most one tile
  int cq, cr;
  int64_t n_items;
  float *part;
  uint16_t *qrot;
  void *out;
  int out_bf16;
  int waves_per_block;
  int Tq, tb, nqb;  // prefill: query tokens, tokens per 16-row block, blocks per sequence
  // decode with append: the new token of sequence b (bf16 [128] at
  // k_new / v_new + b * new_stride_b + g * new_stride_h) sits at position
  // seq_len[b] - 1 and is encoded into the pools by the launch itself
  const uint16_t *k_new, *v_new;
  int64_t new_stride_b, new_stride_h;
  uint8_t *kc_w, *vc_w;  // the pools, writable
  uint16_t *kn_w, *vn_w;
  dq_stats *k_stats, *v_stats;
  float *part_new;  // [B][Hkv][4][kPart]: the new token's own partial
  int64_t n_enc;    // encode items run by the split-K launch (0: a launch of their own ran them)
  int skip_last;    // 1 with an append: the chunks cover the len - 1 older tokens
  // work queue: null, or a counter (zero at launch) from which each wave
  // takes its next item, for launches whose items take several rounds
  unsigned int *queue;
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- rotate q
// q~ = H * D_K * q for one query head, in fp32, by one wave: lane l ends with
// dims l (v0) and l + 64 (v1).  Width 64 pairs d with d + 64 inside the lane;
// widths 32..1 go across lanes.  w0, w1: the sign words of the kv group.
__device__ __forceinline__ void rotate_q_head(const uint16_t *qp, uint64_t w0, uint64_t w1, int lane, float &v0,
                                              float &v1) {
  v0 = __uint_as_float((uint32_t)qp[lane] << 16);
  v1 = __uint_as_float((uint32_t)qp[lane + 64] << 16);
  if ((w0 >> lane) & 1ull) v0 = -v0;
  if ((w1 >> lane) & 1ull) v1 = -v1;
  const float t0 = v0 + v1, t1 = v0 - v1;
  v0 = t0;
  v1 = t1;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const float p0 = __shfl_xor(v0, w), p1 = __shfl_xor(v1, w);
    const bool hi = lane & w;
    v0 = hi ? p0 - v0 : v0 + p0;
    v1 = hi ? p1 - v1 : v1 + p1;
  }
}

// The rotated query of kv group g of sequence b as the QK MFMAs read it: an
// fp16 hi + lo pair per value, staged through `tmp` (2 KB of the wave's LDS
// slice) as [dim group][head][hi x4, lo x4] and read back so that lane l
// holds dim groups l / 4 and 16 + l / 4 of head l mod 4.  Heads past the
// group size are zero.  Each split-K item rotates its own query (a few
// hundred instructions against the item's tiles), so no launch precedes
// the attention.
__device__ __forceinline__ void rotate_q_wave(const AttnArgs &a, uint64_t kseed, int b, int g, uint16_t *tmp,
                                              uint4 (&qreg)[2], int lane) {
  const uint64_t w0 = dev_splitmix64(kseed, 2ull * (uint64_t)g);
  const uint64_t w1 = dev_splitmix64(kseed, 2ull * (uint64_t)g + 1ull);
  const int d0 = lane, d1 = lane + 64;
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    uint16_t h0 = 0, l0 = 0, h1 = 0, l1 = 0;
    if (hh < a.group) {
      float v0, v1;
      rotate_q_head(a.q + ((int64_t)b * a.Hq + g * a.group + hh) * kD, w0, w1, lane, v0, v1);
      const _Float16 f0 = (_Float16)v0, f1 = (_Float16)v1;
      h0 = __builtin_bit_cast(uint16_t, f0);
      h1 = __builtin_bit_cast(uint16_t, f1);
      l0 = __builtin_bit_cast(uint16_t, (_Float16)(v0 - (float)f0));
      l1 = __builtin_bit_cast(uint16_t, (_Float16)(v1 - (float)f1));
    }
    const int i0 = ((d0 >> 2) * 4 + hh) * 8 + (d0 & 3), i1 = ((d1 >> 2) * 4 + hh) * 8 + (d1 & 3);
    tmp[i0] = h0;
    tmp[i0 + 4] = l0;
    tmp[i1] = h1;
    tmp[i1 + 4] = l1;
  }
  wave_sync();
  const uint4 *t4 = reinterpret_cast<const uint4 *>(tmp);
  qreg[0] = t4[lane];
  qreg[1] = t4[64 + lane];
}

// The rotated query of kv group g of sequence b in fp32 for the VALU QK
// variant: dst[4 d + h] = q~_h[d] (2 KB, heads past the group size zero),
// visible to the whole wave when this returns.
__device__ __forceinline__ void rotate_q_global(const AttnArgs &a, uint64_t kseed, int b, int g, float *dst,
                                                int lane) {
  const uint64_t w0 = dev_splitmix64(kseed, 2ull * (uint64_t)g);
  const uint64_t w1 = dev_splitmix64(kseed, 2ull * (uint64_t)g + 1ull);
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    float v0 = 0.0f, v1 = 0.0f;
    if (hh < a.group) rotate_q_head(a.q + ((int64_t)b * a.Hq + g * a.group + hh) * kD, w0, w1, lane, v0, v1);
    dst[4 * lane + hh] = v0;
    dst[4 * (lane + 64) + hh] = v1;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");  // stores done, stale L1 lines dropped
}

// Four floats at one address for the whole wave (a typed global load, so it
// waits on the vector-memory counter, not the LDS one).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) f32x4 global_f32x4;
__device__ __forceinline__ f32x4 load_global_f4(const float *p) { return *(global_f32x4 *)p; }

__device__ __forceinline__ uint32_t load_le32(const uint8_t *p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

// ---------------------------------------------------------------- split-K
// Per-wave LDS slice (byte offsets), identical on host and device.
struct WaveLayout {
  int kst, vst, pl, vt, bytes;
};
// full_v (latency mode): the V tile holds all 128 dims, not one 32-dim pass.
__host__ __device__ inline WaveLayout wave_layout(int Ck, int Cv, bool full_v = false) {
  WaveLayout w;
  w.kst = 0;
  w.vst = w.kst + ((kTile * Ck + 31) & ~15);
  w.pl = w.vst + ((kTile * Cv + 31) & ~15);
  w.vt = w.pl + 2 * 4 * kTile * 2;  // P: [head][token quad][hi x4, lo x4] fp16
  w.bytes = w.vt + (full_v ? kD : kDPass) * kVtStride * 2;
  w.bytes = (w.bytes + 15) & ~15;
  return w;
}

// Container bytes of one 64-token tile, fetched into registers one tile
// ahead (NQ 16-byte pieces per lane) and committed to LDS when needed.
template <int NQ>
struct TileRegs {
  uint4 q[NQ];
  int off;
};

// A 16-byte load from global memory, typed as such: a generic (flat) load
// would also count on the LDS counter, and while one is in flight every
// wait for an LDS result has to be a wait for all of them.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4 global_u32x4;
__device__ __forceinline__ uint4 load_global16(uintptr_t p) {
  const u32x4 v = *(global_u32x4 *)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int NQ>
__device__ __forceinline__ void fetch(TileRegs<NQ> &r, const uint8_t *src, int nbytes, const uint8_t *pool,
                                      const uint8_t *pool_end, int lane) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(src);
  const uintptr_t a0 = a & ~(uintptr_t)15;
  r.off = (int)(a - a0);
  const int n16 = (r.off + nbytes + 15) >> 4;
  const uintptr_t beg = reinterpret_cast<uintptr_t>(pool), end = reinterpret_cast<uintptr_t>(pool_end);
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int i = lane + 64 * k;
    const uintptr_t p = a0 + 16 * (uintptr_t)i;
    r.q[k] = (i < n16 && p >= beg && p + 16 <= end) ? load_global16(p) : make_uint4(0, 0, 0, 0);
  }
}

template <int NQ>
__device__ __forceinline__ void commit(const TileRegs<NQ> &r, uint8_t *dst, int nbytes, int lane) {
  const int n16 = (r.off + nbytes + 15) >> 4;
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int i = lane + 64 * k;
    if (i < n16) *reinterpret_cast<uint4 *>(dst + 16 * i) = r.q[k];
  }
}

// The token of a 64-token tile that lane l decodes: the even tokens in
// lanes 0..31, the odd ones in 32..63.  The LDS serves a wave 32 lanes at a
// time, and the streams of one half then start 2 C bytes apart (17 dwords
// for C = 34), so their byte reads spread over the banks.
__device__ __forceinline__ int lane_token(int lane) { return ((lane & 31) << 1) | (lane >> 5); }

struct DecTab {
  const uint8_t *sym8;
  const uint2 *symtab;
  const uint2 *ent;  // per-slot entries (null: sym8 and symtab)
};

// Byte renormalisation.  Stream positions are 32-bit LDS addresses.  The
// next byte is loaded unconditionally (the load is volatile so the compiler
// cannot sink it into a branch): the select then stays branch-free and the
// load overlaps the table lookups of the step.  The empty asm makes each new
// position an opaque value, so every step advances the pointer with one
// add-with-carry instead of re-deriving it from older positions.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef const __attribute__((address_space(3))) uint8_t lds_u8;
typedef const volatile __attribute__((address_space(3))) uint8_t lds_byte;
__device__ __forceinline__ lds_u8 *to_lds(const uint8_t *p) {
  return (lds_u8 *)p;  // p points into LDS (a container staged by this wave)
}
__device__ __forceinline__ uint32_t next_byte(lds_u8 *p) { return *(lds_byte *)p; }
__device__ __forceinline__ void renorm(uint32_t &x, lds_u8 *&p, uint32_t byte) {
  const bool need = x < kLow;
  x = need ? ((x << 8) | byte) : x;
  p += need ? 1 : 0;
  asm("" : "+v"(p));
}

// Renormalisation four steps at a time.  A step shifts in at most one byte,
// so the 4 stream bytes at p cover a group of 4 steps: they are read once
// (two aligned dwords, then a byte shift) and each step takes the next one
// of them.  sel is the v_perm selector of (x << 8) | window byte k: its low
// byte is k, the number of bytes the group has taken so far.
typedef const volatile __attribute__((address_space(3))) u32x2_a4 lds_u32x2_a4;
constexpr uint32_t kSel0 = 0x06050400u;
// (The two dwords are loaded first and shifted later, so the caller can
// issue other loads before waiting for them.)
__device__ __forceinline__ uint2 byte_window_load(lds_u8 *p) {
  const uint32_t a = (uint32_t)(uintptr_t)p;
  const u32x2_a4 d = *(lds_u32x2_a4 *)(uintptr_t)(a & ~3u);
  return make_uint2(d.x, d.y);
}
__device__ __forceinline__ uint32_t byte_window_shift(uint2 d, lds_u8 *p) {
  return __builtin_amdgcn_alignbyte(d.y, d.x, (uint32_t)(uintptr_t)p);  // bytes p .. p + 3
}
__device__ __forceinline__ void renorm_window(uint32_t &x, uint32_t w, uint32_t &sel) {
  const bool need = x < kLow;
  const uint32_t y = __builtin_amdgcn_perm(x, w, sel);
  x = need ? y : x;
  sel += need ? 1u : 0u;
  asm("" : "+v"(sel));  // one add-with-carry per step; the group's count is sel - kSel0
}

// The two table reads of a decode step (slot -> 8 * symbol, then the symbol
// entry), volatile so that their order across chains is kept.
typedef const volatile __attribute__((address_space(3))) u32x2 lds_u32x2;
__device__ __forceinline__ uint32_t lookup_sym8(const DecTab &t, uint32_t x) {
  return *(lds_byte *)to_lds(t.sym8 + (x & (kM - 1)));
}
__device__ __forceinline__ uint2 lookup_symtab(const DecTab &t, uint32_t s8) {
  const u32x2 e = *(lds_u32x2 *)to_lds(reinterpret_cast<const uint8_t *>(t.symtab) + s8);
  return make_uint2(e.x, e.y);
}
// The entry of a slot from the per-slot table: one read per step.
__device__ __forceinline__ uint2 lookup_slot(const DecTab &t, uint32_t slot) {
  const u32x2 e = *(lds_u32x2 *)to_lds(reinterpret_cast<const uint8_t *>(t.ent) + (slot << 3));
  return make_uint2(e.x, e.y);
}
// x's slot, as an opaque value: the table address (slot * 8) and the state
// update (slot - cum) then share one AND instead of the compiler's
// (x << 3) & 0x7FF8 beside x & 0xFFF.
__device__ __forceinline__ uint32_t slot_of(uint32_t x) {
  uint32_t s = x & (kM - 1);
  asm("" : "+v"(s));
  return s;
}

// f(std::integral_constant<int, i>()) for i = 0 .. N-1, so that i can feed
// the constant operands of a builtin (the MFMA broadcast block)
template <typename F, int... I>
__device__ __forceinline__ void unroll_impl(F &f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>()), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F &&f) {
  unroll_impl(f, std::make_integer_sequence<int, N>());
}


// P (hi, lo) x the 16 dims of a V-tile pass: 8 MFMAs whose blocks are (4
// dim quads) x (4 token quarters).  Token quad 4 q + c of P sits in block c
// of quarter q and is broadcast within the quarter (cbsz 2, abid c); vrow is
// this lane's row (dim lane mod 16) at its quarter's tokens (16 (lane / 16)
// onwards).  The hi and lo products accumulate into the same registers, hi
// first: the partial of each dim is summed over the quarters at the end.
template <int P>
__device__ __forceinline__ void pv_pass(const uint32_t *vrow, half4 Ph, half4 Pl, floatx4 (&acc)[8]) {
  // the pass's four operands are read first: one LDS round trip, not four
  half4 V[4];
  unroll<4>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    V[c] = __builtin_bit_cast(half4, make_uint2(vrow[2 * c], vrow[2 * c + 1]));
  });
  unroll<4>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    acc[P] = __builtin_amdgcn_mfma_f32_4x4x4f16(Ph, V[c], acc[P], 2, c, 0);
    acc[P] = __builtin_amdgcn_mfma_f32_4x4x4f16(Pl, V[c], acc[P], 2, c, 0);
  });
}

// This lane's P operand: 16 bytes (hi x4, lo x4) of token quad lane / 4 for
// head lane mod 4, read once per tile.
__device__ __forceinline__ void load_p(const uint16_t *pl, int lane, half4 &Ph, half4 &Pl) {
  const int th = lane >> 5, row = lane & 31;
  const uint4 pq = *reinterpret_cast<const uint4 *>(pl + ((lane & 3) * 16 + th * 8 + (row >> 2)) * 8);
  Ph = __builtin_bit_cast(half4, make_uint2(pq.x, pq.y));
  Pl = __builtin_bit_cast(half4, make_uint2(pq.z, pq.w));
}

// Decodes one K tile (scores into sc) and/or one V tile (PV into acc),
// interleaving the two independent rANS chains of each lane.
// K: after every 4 symbols (dim group G), sc += q~[4 heads][4 dims] x
//   levels[4 dims] on a 4x4x4 MFMA.  The query of group G sits in block
//   G mod 16 of register set G / 16 (lanes 4b .. 4b + 3 hold groups b and
//   16 + b, one head each, hi then lo) and is broadcast to every block
//   (cbsz 4, abid G mod 16).  The lane's own 4 levels are the B column, and
//   the lane ends with its token's scores for the 4 heads.
// V: levels go to the transposed LDS tile, 16 dims per pass; each pass is
//   contracted with P (hi, then lo) by pv_pass.  P is read from LDS once
//   per tile.
// SLOT: each step reads its entry from the per-slot table (one LDS round
// trip); otherwise the slot's symbol, then the symbol's entry.
//
// FULLV (latency mode): K and V of the same tile; the V levels of all 128
// dims stay in the V tile for pv_full after the tile's softmax, and no PV
// runs inside the pass.
//
// VQK (measurement variant): the K scores as fp32 fused multiply-adds on the
// vector ALU, sc[h] += level * q~_h[d] in dim order, with q~ read from
// global memory (qg, [dim][head]) one group of 4 dims ahead: qb holds the
// first group's values on entry and, on return, those the next pass starts
// with (loaded before the caller's next tile fetch, which they then need
// not wait for).
template <bool DK, bool DV, bool FULLV = false, bool SLOT = false, bool VQK = false>
__device__ __forceinline__ void tile_pass(const DecTab tk, const DecTab tv, const uint8_t *kb,
                                          const uint8_t *vb, const uint4 (&qreg)[2], const uint16_t *pl,
                                          uint16_t *vt, floatx4 &sc, floatx4 (&acc)[8], int lane,
                                          const float *qg = nullptr, f32x4 *qb = nullptr) {
  half4 Ph = {}, Pl = {};
  if (DV && !FULLV) load_p(pl, lane, Ph, Pl);
  const uint32_t *vrow = reinterpret_cast<const uint32_t *>(vt) + (lane & 15) * (kVtStride / 2) + (lane >> 4) * 8;
  uint32_t xk = 0, xv = 0;
  lds_u8 *pk = nullptr, *pv = nullptr;
  if (DK) {
    xk = load_le32(kb);
    pk = to_lds(kb + 4);
  }
  if (DV) {
    xv = load_le32(vb);
    pv = to_lds(vb + 4);
  }
  uint16_t *col = vt + lane;
  unroll<kD / kDPass>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    unroll<kDPass / 4>([&](auto gc) {
      constexpr int gq = decltype(gc)::value;
      constexpr int G = p * (kDPass / 4) + gq;
      uint32_t lv[4];
      uint32_t wk = 0, wv = 0, selk = kSel0, selv = kSel0;
      uint2 dwk = make_uint2(0, 0), dwv = make_uint2(0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // the two chains' loads are issued in this order (volatile), so
        // each LDS round trip of one chain overlaps the other's.  The
        // group's renormalisation bytes are read in its first step, after
        // the table read that step's renorm waits for anyway: in the order
        // results are used (LDS returns in order), never on their own.
        uint32_t ak = 0, av = 0;
        uint2 ek = make_uint2(0, 0), ev = make_uint2(0, 0);
        if (SLOT) {
          if (DK) ak = slot_of(xk);
          if (DV) av = slot_of(xv);
          if (DK) ek = lookup_slot(tk, ak);
          if (DK && j == 0) dwk = byte_window_load(pk);
          if (DV) ev = lookup_slot(tv, av);
          if (DV && j == 0) dwv = byte_window_load(pv);
        } else {
          uint32_t sk = 0, sv = 0;
          if (DK) sk = lookup_sym8(tk, xk);
          if (DV) sv = lookup_sym8(tv, xv);
          if (DK && j == 0) dwk = byte_window_load(pk);
          if (DV && j == 0) dwv = byte_window_load(pv);
          if (DK) ek = lookup_symtab(tk, sk);
          if (DV) ev = lookup_symtab(tv, sv);
        }
        if (j == 0) {
          // the windows' byte shifts (and so their waits) stay below the
          // step's loads
          __builtin_amdgcn_sched_barrier(0);
          if (DK) wk = byte_window_shift(dwk, pk);
          if (DV) wv = byte_window_shift(dwv, pv);
        }
        if (DK) {
          xk = SLOT ? rans_advance_slot(xk, ak, ek) : rans_advance(xk, ek);
          renorm_window(xk, wk, selk);
          lv[j] = ek.y;
        }
        if (DV) {
          xv = SLOT ? rans_advance_slot(xv, av, ev) : rans_advance(xv, ev);
          renorm_window(xv, wv, selv);
          col[((FULLV ? p * kDPass : 0) + gq * 4 + j) * kVtStride] = (uint16_t)(ev.y >> 16);
        }
      }
      if (DK) pk += selk - kSel0;
      if (DV) pv += selv - kSel0;
      if (DK && VQK) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float l = (float)__builtin_bit_cast(_Float16, (uint16_t)(lv[j] >> 16));
#pragma unroll
          for (int h = 0; h < 4; ++h) sc[h] = __builtin_fmaf(l, qb[j][h], sc[h]);
        }
        // the next group's q~ (after the last group: the next pass's first)
        constexpr int Gn = (G + 1) % (kD / 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) qb[j] = load_global_f4(qg + 4 * (4 * Gn + j));
      } else if (DK) {
        const uint32_t b01 = __builtin_amdgcn_perm(lv[1], lv[0], 0x07060302u);
        const uint32_t b23 = __builtin_amdgcn_perm(lv[3], lv[2], 0x07060302u);
        const half4 Bk = __builtin_bit_cast(half4, make_uint2(b01, b23));
        const uint4 &q = qreg[G >> 4];
        sc = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4, make_uint2(q.x, q.y)), Bk, sc, 4,
                                                G & 15, 0);
        sc = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4, make_uint2(q.z, q.w)), Bk, sc, 4,
                                                G & 15, 0);
      }
    });
    if (DV && !FULLV) {
      wave_sync();
      pv_pass<p>(vrow, Ph, Pl, acc);
      wave_sync();
    }
  });
}

// Latency mode: PV of a whole tile whose V levels (128 dims) are in vt and
// whose P is in pl.
__device__ __forceinline__ void pv_full(const uint16_t *pl, const uint16_t *vt, floatx4 (&acc)[8], int lane) {
  half4 Ph, Pl;
  load_p(pl, lane, Ph, Pl);
  const uint32_t *v32 = reinterpret_cast<const uint32_t *>(vt);
  unroll<kD / kDPass>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    pv_pass<p>(v32 + (p * kDPass + (lane & 15)) * (kVtStride / 2) + (lane >> 4) * 8, Ph, Pl, acc);
  });
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) v = fmaxf(v, __shfl_xor(v, w));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int w = 1; w < 64; w <<= 1) v += __shfl_xor(v, w);
  return v;
}

// Online softmax for one tile.  Lane t holds its token's scores for the 4
// heads (sc) and its own K and V norms; m_run is per head (same in every
// lane), l_lane is this lane's share of the per-head sum (reduced once per
// item).  Writes P = p * n_v (fp16) to LDS and rescales the V accumulators.
// The running max only has to bound the scores, not equal their maximum:
// while no score of the tile exceeds it (checked with one vote), the tile
// reuses it and skips the reductions and the rescale; p stays <= 1.
__device__ __forceinline__ void softmax_tile(const floatx4 &sc, uint32_t nk_bits, uint32_t nv_bits, bool valid,
                                             float qk_scale, float (&m_run)[4], float (&l_lane)[4],
                                             uint16_t *pl, floatx4 (&acc)[8], int lane) {
  const float nk = (float)__builtin_bit_cast(_Float16, (uint16_t)nk_bits);
  const float nv = (float)__builtin_bit_cast(_Float16, (uint16_t)nv_bits);
  float s[4];
  bool over = false;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    s[h] = valid ? sc[h] * nk * qk_scale : -__builtin_inff();
    over |= s[h] > m_run[h];  // also true while m_run is still -inf
  }
  if (__builtin_amdgcn_read_exec() & __ballot(over)) {
    float alpha[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float m_new = fmaxf(m_run[h], wave_max(s[h]));
      alpha[h] = exp2f(m_run[h] - m_new);
      l_lane[h] *= alpha[h];
      m_run[h] = m_new;
    }
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
      for (int h = 0; h < 4; ++h) acc[p][h] *= alpha[h];
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float p = valid ? exp2f(s[h] - m_run[h]) : 0.0f;
    l_lane[h] += p;
    // P = p * n_v as an fp16 pair (hi + lo carries ~22 bits): one fp16
    // rounding alone would cost up to 2^-11 of an output of norm size
    const float pv = valid ? p * nv : 0.0f;
    const _Float16 hi = (_Float16)pv;
    uint16_t *q8 = pl + (h * 16 + (lane >> 2)) * 8 + (lane & 3);
    q8[0] = __builtin_bit_cast(uint16_t, hi);
    q8[4] = __builtin_bit_cast(uint16_t, (_Float16)(pv - (float)hi));
  }
}

// An item's partial: the four token quarters of every dim are summed
// across lanes l, l ^ 16, l ^ 32, l ^ 48; lanes 0..15 hold dims 16p + l.
// Then m and the wave-summed l of each head.
__device__ __forceinline__ void write_partial(float *dst, const floatx4 (&acc)[8], const float (&m_run)[4],
                                              const float (&l_lane)[4], int lane) {
#pragma unroll
  for (int p = 0; p < kD / kDPass; ++p) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float v = acc[p][h];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) dst[h * kPart + p * kDPass + lane] = v;
    }
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float l = wave_sum(l_lane[h]);
    if (lane == h) {
      dst[h * kPart + 128] = m_run[h];
      dst[h * kPart + 129] = l;
    }
  }
}

// Append: one wave encodes the new token's K (isv false) or V vector of
// (b, g) into the pool and writes that token's own attention partial from
// the symbols it chose: the K wave the scores (m = s_h, l = 1), the V wave
// n_v * level (p = 1).  The chunk items then cover the older tokens only,
// and the combine merges this partial like any other, so no item waits for
// the encode.  scratch: the wave's LDS slice.
template <bool RD>
__device__ __forceinline__ void append_vector(const AttnArgs &a, const Tables &t, const uint4 *etab,
                                              const float2 *rdtab, uint8_t *scratch, bool isv, int b, int g,
                                              int lane) {
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int pos = a.seq_len[b] - 1;
  int64_t slot = -1;
  if (pos >= 0) {
    if (!a.pages) slot = a.seq_start[b] + pos;
    else if (pos / kTile < a.max_pages) slot = (int64_t)a.pages[(int64_t)b * a.max_pages + pos / kTile] * kTile + pos % kTile;
  }
  const uint16_t *xp = (isv ? a.v_new : a.k_new) + (int64_t)b * a.new_stride_b + (int64_t)g * a.new_stride_h;
  const WaveEncodeScratch L{reinterpret_cast<uint32_t *>(scratch), scratch + 4 * kD, scratch + 5 * kD,
                            min(kWaveScr, t.C - 3)};
  WaveEncodeResult r;
  wave_encode_vector<RD, true>(xp, g, t, etab, rdtab, L, lane, r);
  if (r.win >= 0 && slot >= 0 && slot < a.S) {
    const int64_t idx = (int64_t)g * a.S + slot;
    wave_store_container(r, L, t.C, (isv ? a.vc_w : a.kc_w) + idx * t.C, (isv ? a.vn_w : a.kn_w) + idx, lane);
  }
  dq_stats *st = isv ? a.v_stats : a.k_stats;
  if (st && lane == 0) {
    unsigned long long *gs = reinterpret_cast<unsigned long long *>(st);
    atomicAdd(gs + 0, 1ull);
    if (r.moves) {
      atomicAdd(gs + 1, 1ull);
      atomicAdd(gs + 2, (unsigned long long)r.moves);
    }
    if (r.passes) atomicAdd(gs + 3, (unsigned long long)r.passes);
    if (r.bad) atomicAdd(gs + 4, 1ull);
    if (r.zero) atomicAdd(gs + 5, 1ull);
    atomicAdd(gs + 6 + 4 + r.okB, 1ull);
  }
  if (pos < 0) return;
  float *P = a.part_new + bg * 4 * kPart;
  const float n = half_to_float(r.nh);
  const float lam0 = half_to_float(t.recon[r.sym[0]]), lam1 = half_to_float(t.recon[r.sym[1]]);
  if (!isv) {
    // s_h = q~_h . levels * n_k * scale, with q~ as the QK MFMAs see it (the
    // fp16 hi + lo pair of each rotated value); heads past the group: 0
    const uint64_t w0 = dev_splitmix64(t.seed, 2ull * (uint64_t)g);
    const uint64_t w1 = dev_splitmix64(t.seed, 2ull * (uint64_t)g + 1ull);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float q0 = 0.0f, q1 = 0.0f;
      if (h < a.group) {
        float v0, v1;
        rotate_q_head(a.q + ((int64_t)b * a.Hq + g * a.group + h) * kD, w0, w1, lane, v0, v1);
        const _Float16 f0 = (_Float16)v0, f1 = (_Float16)v1;
        q0 = (float)f0 + (float)(_Float16)(v0 - (float)f0);
        q1 = (float)f1 + (float)(_Float16)(v1 - (float)f1);
      }
      float dot = q0 * lam0 + q1 * lam1;
#pragma unroll
      for (int w = 1; w < 64; w <<= 1) dot += __shfl_xor(dot, w);
      if (lane == h) {
        P[h * kPart + 128] = dot * n * a.qk_scale;
        P[h * kPart + 129] = 1.0f;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      P[h * kPart + lane] = n * lam0;
      P[h * kPart + lane + 64] = n * lam1;
    }
  }
}

// LAT (latency mode, for batches that leave waves idle): each tile's K and
// V are decoded in one pass, then its softmax and PV; an item of n tiles
// takes n passes instead of n + 1 (a K-only first and a V-only last), at
// the price of a whole V tile in LDS and so fewer waves per CU.  The
// arithmetic and its order are those of the pipelined mode.
// SLOT: the per-slot decode tables (64 KB for K and V), so a decode step is
// one LDS round trip; otherwise the byte table and the symbol entries.
template <int NQ, bool APPEND, bool LAT = false, bool SLOT = false, bool VQK = false>
__global__ void __launch_bounds__(NQ == 3 ? 768 : 256) attn_splitk_kernel(AttnArgs a, Tables tk, Tables tv) {
  static_assert(!(LAT && SLOT), "latency mode keeps the byte tables: its whole V tiles leave no room");
  static_assert(!VQK || (SLOT && !APPEND), "the VALU QK variant is built for the plain per-slot-table kernel");
  // decode tables at fixed LDS addresses (static), per-wave slices after them
  __shared__ uint2 slot_ent[2][SLOT ? kM : 1];
  __shared__ uint8_t sym8[2][SLOT ? 1 : kM];
  __shared__ uint2 symtab[2][kMaxLevels];
  __shared__ uint4 etab[2][APPEND ? kMaxLevels : 1];
  __shared__ float2 rdtab[2][APPEND ? kMaxHalf : 1];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const DecTab dk{sym8[0], symtab[0], SLOT ? slot_ent[0] : nullptr};
  const DecTab dv{sym8[1], symtab[1], SLOT ? slot_ent[1] : nullptr};
  if (SLOT) {
    build_slot_tables(slot_ent[0], symtab[0], tk, threadIdx.x, blockDim.x);
    build_slot_tables(slot_ent[1], symtab[1], tv, threadIdx.x, blockDim.x);
  } else {
    build_tables(sym8[0], symtab[0], tk, threadIdx.x, blockDim.x);
    build_tables(sym8[1], symtab[1], tv, threadIdx.x, blockDim.x);
  }
  if (APPEND) {
    wave_encode_tables(tk, etab[0], rdtab[0], threadIdx.x);
    wave_encode_tables(tv, etab[1], rdtab[1], threadIdx.x);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // P and the V tile are indexed by lane: the token order inside a tile never shows
  const int tok = lane_token(lane);
  const int Ck = tk.C, Cv = tv.C;
  const WaveLayout L = wave_layout(Ck, Cv, LAT);
  uint8_t *base = smem + (size_t)wave * L.bytes;
  uint8_t *kst = base + L.kst;
  uint8_t *vst = base + L.vst;
  uint16_t *pl = reinterpret_cast<uint16_t *>(base + L.pl);
  uint16_t *vt = reinterpret_cast<uint16_t *>(base + L.vt);

  const uint8_t *kpool_end = a.kc + (size_t)a.Hkv * a.S * Ck;
  const uint8_t *vpool_end = a.vc + (size_t)a.Hkv * a.S * Cv;
  const int64_t W = (int64_t)gridDim.x * a.waves_per_block;

  // items [0, n_enc): the append's encodes (K of every (b, g), then V);
  // then the attention items, each one chunk of one (b, g)
  const int64_t n_enc = APPEND ? a.n_enc : 0;
  const int64_t n_half = (int64_t)a.B * a.Hkv;
  // items in turn: statically every W-th one, or from the work queue.  The
  // static deal suits one round of equal items; a ragged batch over several
  // rounds would leave one wave all the chunks of a long sequence (the
  // deal repeats with period W, a multiple of B * Hkv), so there each wave
  // takes the next item from the queue when it is done with one.
  auto grab = [&](int64_t cur) -> int64_t {
    if (!a.queue) return cur + W;
    unsigned int t = 0u;
    if (lane == 0) t = atomicAdd(a.queue, 1u);
    return (int64_t)(unsigned int)__shfl((int)t, 0);
  };
  int64_t it = a.queue ? grab(0) : (int64_t)blockIdx.x * a.waves_per_block + wave;
  for (; APPEND && it < n_enc; it = grab(it)) {
    const bool isv = it >= n_half;
    const int64_t e = isv ? it - n_half : it;
    const int b = (int)(e / a.Hkv), g = (int)(e - (int64_t)(e / a.Hkv) * a.Hkv);
    wave_sync();  // the slice is free
    // one call per kernel argument: a reference chosen at run time would put
    // both tables in scratch memory
    if (isv) {
      if (tv.order == 1) append_vector<true>(a, tv, etab[1], rdtab[1], base, true, b, g, lane);
      else append_vector<false>(a, tv, etab[1], rdtab[1], base, true, b, g, lane);
    } else {
      if (tk.order == 1) append_vector<true>(a, tk, etab[0], rdtab[0], base, false, b, g, lane);
      else append_vector<false>(a, tk, etab[0], rdtab[0], base, false, b, g, lane);
    }
  }
  // items are chunk-major: a wave's items in successive rounds are chunks
  // c, c + W / nbg, ..., which pairs the one-tile-longer first chunks with
  // the shorter last ones when the items fill whole rounds
  const int64_t nbg = (int64_t)a.B * a.Hkv;
  for (; it < n_enc + a.n_items; it = grab(it)) {
    const int64_t item = it - n_enc;
    const int c = (int)(item / nbg);
    const int64_t bg = item - (int64_t)c * nbg;
    const int b = (int)(bg / a.Hkv), g = (int)(bg - (int64_t)b * a.Hkv);
    const int64_t pidx = bg * a.nc + c;  // the partial's slot
    // a paged sequence never reads past its row of the page table; with an
    // append the newest token is not part of any chunk
    const int len0 = a.seq_len[b] - a.skip_last;
    const int len = a.pages ? min(len0, a.max_pages * kTile) : len0;
    const int t0 = (c * a.cq + min(c, a.cr)) * kTile;
    if (t0 >= len) continue;
    const int t1 = min(t0 + (a.cq + (c < a.cr ? 1 : 0)) * kTile, len);
    const int ntiles = (t1 - t0 + kTile - 1) / kTile;
    const int64_t plane0 = (int64_t)g * a.S;
    // pool index of the first token of tile `tile` of this item: a page is
    // one tile, so a tile's containers are contiguous in either layout
    // (the sequence's start is read once per item: a read per tile would
    // follow the tile prefetch, and waiting for it would wait for that too)
    const int64_t seq0 = a.pages ? 0 : a.seq_start[b];
    auto tile_base = [&](int tile) -> int64_t {
      const int t = t0 + tile * kTile;
      return a.pages ? plane0 + (int64_t)a.pages[(int64_t)b * a.max_pages + t / kTile] * kTile
                     : plane0 + seq0 + t;
    };

    wave_sync();  // the previous item's LDS reads are done
    // rotated query of this (sequence, kv head): lane l holds dim groups
    // l / 4 and 16 + l / 4 of head l mod 4 (8 VGPRs for the whole item)
    uint4 qreg[2] = {};
    const float *qg = nullptr;
    f32x4 qb[4];  // VQK: the q~ group a K pass starts with
    if (VQK) {
      // the item's partial slot holds q~ until the partial overwrites it
      float *qs = a.part + pidx * 4 * kPart;
      rotate_q_global(a, tk.seed, b, g, qs, lane);
      qg = qs;
#pragma unroll
      for (int j = 0; j < 4; ++j) qb[j] = load_global_f4(qg + 4 * j);
    } else {
      rotate_q_wave(a, tk.seed, b, g, vt, qreg, lane);
    }

    // this lane's token norms for a tile (0 outside the pool plane)
    auto norms = [&](int64_t tbase, uint32_t &nk, uint32_t &nv) {
      const int64_t idx = tbase + tok;
      const bool ok = idx >= (int64_t)g * a.S && idx < (int64_t)(g + 1) * a.S;
      nk = ok ? a.kn[idx] : 0u;
      nv = ok ? a.vn[idx] : 0u;
    };
    TileRegs<NQ> rk, rv;
    if (LAT) {
      uint32_t nkc, nvc, nkn = 0, nvn = 0;  // norms of the current and the next tile
      const int64_t base0 = tile_base(0);
      fetch<NQ>(rk, a.kc + base0 * Ck, kTile * Ck, a.kc, kpool_end, lane);
      fetch<NQ>(rv, a.vc + base0 * Cv, kTile * Cv, a.vc, vpool_end, lane);
      norms(base0, nkc, nvc);
      float m_run[4], l_lane[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        m_run[h] = -__builtin_inff();
        l_lane[h] = 0.0f;
      }
      floatx4 acc[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) acc[p] = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < ntiles; ++j) {
        wave_sync();  // every read of the staging buffers, P and the V tile is done
        commit<NQ>(rk, kst, kTile * Ck, lane);
        commit<NQ>(rv, vst, kTile * Cv, lane);
        const int koff = rk.off, voff = rv.off;
        wave_sync();
        if (j + 1 < ntiles) {
          const int64_t base1 = tile_base(j + 1);
          fetch<NQ>(rk, a.kc + base1 * Ck, kTile * Ck, a.kc, kpool_end, lane);
          fetch<NQ>(rv, a.vc + base1 * Cv, kTile * Cv, a.vc, vpool_end, lane);
          norms(base1, nkn, nvn);
        }
        floatx4 sc = {0.f, 0.f, 0.f, 0.f};
        tile_pass<true, true, true>(dk, dv, kst + koff + tok * Ck, vst + voff + tok * Cv, qreg, pl, vt, sc, acc,
                                    lane);
        softmax_tile(sc, nkc, nvc, j * kTile + tok < t1 - t0, a.qk_scale, m_run, l_lane, pl, acc, lane);
        wave_sync();  // P and the V tile are complete
        pv_full(pl, vt, acc, lane);
        nkc = nkn;
        nvc = nvn;
      }
      write_partial(a.part + pidx * 4 * kPart, acc, m_run, l_lane, lane);
      continue;
    }
    uint32_t nk0, nv0, nk1 = 0, nv1 = 0;
    // prologue: K of tile 0
    const int64_t base0 = tile_base(0);
    int64_t vbase = base0;  // V tile to fetch next
    fetch<NQ>(rk, a.kc + base0 * Ck, kTile * Ck, a.kc, kpool_end, lane);
    norms(base0, nk0, nv0);
    commit<NQ>(rk, kst, kTile * Ck, lane);
    const int koff0 = rk.off;
    wave_sync();
    fetch<NQ>(rv, a.vc + vbase * Cv, kTile * Cv, a.vc, vpool_end, lane);
    if (ntiles > 1) {
      const int64_t base1 = tile_base(1);
      fetch<NQ>(rk, a.kc + base1 * Ck, kTile * Ck, a.kc, kpool_end, lane);
      norms(base1, nk1, nv1);
      vbase = base1;
    }
    float m_run[4], l_lane[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      m_run[h] = -__builtin_inff();
      l_lane[h] = 0.0f;
    }
    floatx4 acc[8];  // [0..3]: P hi contributions, [4..7]: P lo
#pragma unroll
    for (int p = 0; p < 8; ++p) acc[p] = floatx4{0.f, 0.f, 0.f, 0.f};
    floatx4 sc = {0.f, 0.f, 0.f, 0.f};
    tile_pass<true, false, false, SLOT, VQK>(dk, dv, kst + koff0 + tok * Ck, nullptr, qreg, pl, vt, sc, acc, lane,
                                             qg, qb);
    softmax_tile(sc, nk0, nv0, tok < t1 - t0, a.qk_scale, m_run, l_lane, pl, acc, lane);

    for (int j = 0; j < ntiles; ++j) {
      const bool next = j + 1 < ntiles;
      wave_sync();  // every read of the staging buffers is done
      commit<NQ>(rv, vst, kTile * Cv, lane);
      const int voff = rv.off;
      int koff = 0;
      if (next) {
        commit<NQ>(rk, kst, kTile * Ck, lane);
        koff = rk.off;
      }
      wave_sync();
      // prefetch the next iteration's tiles into registers; the K tile's
      // base first (in a paged pool a page-table read, which would otherwise
      // wait for the V tile's loads issued before it)
      uint32_t nk2 = 0, nv2 = 0;
      const int64_t base2 = j + 2 < ntiles ? tile_base(j + 2) : 0;
      if (next) fetch<NQ>(rv, a.vc + vbase * Cv, kTile * Cv, a.vc, vpool_end, lane);
      if (j + 2 < ntiles) {
        fetch<NQ>(rk, a.kc + base2 * Ck, kTile * Ck, a.kc, kpool_end, lane);
        norms(base2, nk2, nv2);
        vbase = base2;
      }
      if (next) {
        sc = floatx4{0.f, 0.f, 0.f, 0.f};
        tile_pass<true, true, false, SLOT, VQK>(dk, dv, kst + koff + tok * Ck, vst + voff + tok * Cv, qreg, pl, vt,
                                                sc, acc, lane, qg, qb);
        softmax_tile(sc, nk1, nv1, (j + 1) * kTile + tok < t1 - t0, a.qk_scale, m_run, l_lane, pl, acc, lane);
      } else {
        tile_pass<false, true, false, SLOT, VQK>(dk, dv, nullptr, vst + voff + tok * Cv, qreg, pl, vt, sc, acc, lane,
                                                 qg, qb);
      }
      nk1 = nk2;
      nv1 = nv2;
    }

    write_partial(a.part + pidx * 4 * kPart, acc, m_run, l_lane, lane);
  }
}

// Zeroes the split-K work queue's counter (a kernel, not a memset, so the
// call stays capturable in a HIP graph).
__global__ void __launch_bounds__(64) queue_reset_kernel(unsigned int *counter) {
  if (threadIdx.x == 0) *counter = 0u;
}

// ---------------------------------------------------------------- combine
// The append's encodes as a launch of their own, for batches whose
// attention items already fill every round of resident waves: one wave per
// new vector (K of every (b, g), then V), each writing its container and
// its token's own partial exactly as inside the split-K launch.
constexpr int kAppendWaves = 4;  // waves per block
__host__ __device__ inline int append_scratch_bytes(int C) {
  const int rows = C - 3 < kWaveScr ? C - 3 : kWaveScr;
  return 5 * kD + rows * 64;  // ent [128] words, mag [128] bytes, renorm rows
}
__global__ void __launch_bounds__(64 * kAppendWaves) append_encode_kernel(AttnArgs a, Tables tk, Tables tv) {
  __shared__ uint4 etab[2][kMaxLevels];
  __shared__ float2 rdtab[2][kMaxHalf];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  wave_encode_tables(tk, etab[0], rdtab[0], threadIdx.x);
  wave_encode_tables(tv, etab[1], rdtab[1], threadIdx.x);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n_half = (int64_t)a.B * a.Hkv;
  const int64_t it = (int64_t)blockIdx.x * kAppendWaves + wave;
  if (it >= 2 * n_half) return;  // whole waves; no block barrier follows
  const bool isv = it >= n_half;
  const int64_t e = isv ? it - n_half : it;
  const int b = (int)(e / a.Hkv), g = (int)(e - (int64_t)(e / a.Hkv) * a.Hkv);
  const int C = tk.C > tv.C ? tk.C : tv.C;
  uint8_t *scratch = smem + (size_t)wave * ((append_scratch_bytes(C) + 15) & ~15);
  if (isv) {
    if (tv.order == 1) append_vector<true>(a, tv, etab[1], rdtab[1], scratch, true, b, g, lane);
    else append_vector<false>(a, tv, etab[1], rdtab[1], scratch, true, b, g, lane);
  } else {
    if (tk.order == 1) append_vector<true>(a, tk, etab[0], rdtab[0], scratch, false, b, g, lane);
    else append_vector<false>(a, tk, etab[0], rdtab[0], scratch, false, b, g, lane);
  }
}

// Log-sum-exp merge of a row's partials for the 128 threads of a block
// (thread d owns dim d): partial c sits at src + c * stride floats (acc
// [0, 128), m at 128, l at 129), plus an optional extra one (pe).  Returns
// sum_c w_c acc_c[d] / sum_c w_c l_c with w_c = 2^(m_c - M), M the largest
// m; a partial with m = -inf (no visible token) weighs nothing.  The maxima
// and weights are taken 128 partials at a time, one per thread, so the
// latency is that of a few loads, not of n dependent ones; each thread then
// sums its dim in partial order.
// The same merge for n <= kFewParts partials (a decode step over a few long
// chunks per sequence): every thread loads the few (m, l) pairs itself, so
// there is no exchange, no barrier and no loop over kD slots.  The weights
// are lse_merge's (below); acc and l are summed in partial order, the extra
// partial last.
constexpr int kFewParts = 4;
__device__ __forceinline__ float lse_merge_few(const float *src, int64_t stride, int n, const float *pe) {
  const int d = threadIdx.x;
  float av[kFewParts], mv[kFewParts], lv[kFewParts];
#pragma unroll
  for (int j = 0; j < kFewParts; ++j) {
    av[j] = 0.0f;
    mv[j] = -__builtin_inff();
    lv[j] = 0.0f;
    if (j < n) {  // n is the same for the whole block
      av[j] = src[(int64_t)j * stride + d];
      mv[j] = src[(int64_t)j * stride + 128];
      lv[j] = src[(int64_t)j * stride + 129];
    }
  }
  float ae = 0.0f, me = -__builtin_inff(), le = 0.0f;
  if (pe) {
    ae = pe[d];
    me = pe[128];
    le = pe[129];
  }
  float M = me;
#pragma unroll
  for (int j = 0; j < kFewParts; ++j) M = fmaxf(M, mv[j]);
  float o = 0.0f, L = 0.0f;
#pragma unroll
  for (int j = 0; j < kFewParts; ++j) {
    const float w = mv[j] != -__builtin_inff() ? exp2f(mv[j] - M) : 0.0f;
    if (w != 0.0f) {
      o += w * av[j];
      L += w * lv[j];
    }
  }
  if (pe) {
    const float w = exp2f(me - M);
    o += w * ae;
    L += w * le;
  }
  return L > 0.0f ? o / L : 0.0f;  // an empty row (a caller error) gives zeros
}

__device__ __forceinline__ float lse_merge(const float *src, int64_t stride, int n, const float *pe, float *red,
                                           float *wts) {
  const int d = threadIdx.x;
  // Every load that does not wait on the maximum is issued first: this
  // dim's values of the first kD partials, and the (m, l) of the partials
  // this thread weighs in the first two rounds.  A merge of up to kD
  // partials then costs one memory round trip instead of three.
  const int cnt0 = min(n, kD);
  float av[kD];
#pragma unroll
  for (int j = 0; j < kD; ++j) av[j] = j < cnt0 ? src[(int64_t)j * stride + d] : 0.0f;
  float mr[2] = {-__builtin_inff(), -__builtin_inff()}, lr[2] = {0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < 2; ++r)
    if (d + r * kD < n) {
      mr[r] = src[(int64_t)(d + r * kD) * stride + 128];
      lr[r] = src[(int64_t)(d + r * kD) * stride + 129];
    }
  float M = pe ? pe[128] : -__builtin_inff();
  M = fmaxf(M, fmaxf(mr[0], mr[1]));
  for (int c = d + 2 * kD; c < n; c += kD) M = fmaxf(M, src[(int64_t)c * stride + 128]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) M = fmaxf(M, __shfl_xor(M, w));
  if ((d & 63) == 0) red[d >> 6] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  float Lp = 0.0f, o = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kD) {
    const int cnt = min(kD, n - c0);
    float w = 0.0f;
    if (d < cnt) {
      const float *p = src + (int64_t)(c0 + d) * stride;
      const bool held = c0 < 2 * kD;
      const float m = held ? (c0 == 0 ? mr[0] : mr[1]) : p[128];
      if (m != -__builtin_inff()) {
        w = exp2f(m - M);
        Lp += w * (held ? (c0 == 0 ? lr[0] : lr[1]) : p[129]);
      }
    }
    __syncthreads();  // the previous round's weights are read
    wts[d] = w;
    __syncthreads();
    if (c0 == 0) {
#pragma unroll
      for (int j = 0; j < kD; ++j)
        if (j < cnt && wts[j] != 0.0f) o += wts[j] * av[j];
      continue;
    }
    const float *p = src + (int64_t)c0 * stride + d;
    int j = 0;
    for (; j + 4 <= cnt; j += 4) {
      const float a0 = p[(int64_t)j * stride], a1 = p[(int64_t)(j + 1) * stride];
      const float a2 = p[(int64_t)(j + 2) * stride], a3 = p[(int64_t)(j + 3) * stride];
      if (wts[j] != 0.0f) o += wts[j] * a0;
      if (wts[j + 1] != 0.0f) o += wts[j + 1] * a1;
      if (wts[j + 2] != 0.0f) o += wts[j + 2] * a2;
      if (wts[j + 3] != 0.0f) o += wts[j + 3] * a3;
    }
    for (; j < cnt; ++j)
      if (wts[j] != 0.0f) o += wts[j] * p[(int64_t)j * stride];
  }
  if (pe) {
    const float w = exp2f(pe[128] - M);
    if (d == 0) Lp += w * pe[129];
    o += w * pe[d];
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) Lp += __shfl_xor(Lp, w);
  __syncthreads();  // red[0..1] and wts are free again
  if ((d & 63) == 0) red[d >> 6] = Lp;
  __syncthreads();
  const float L = red[0] + red[1];
  return L > 0.0f ? o / L : 0.0f;  // an empty row (a caller error) gives zeros
}

__global__ void __launch_bounds__(128) combine_kernel(AttnArgs a, uint64_t vseed) {
  __shared__ float buf[kD];
  __shared__ float wts[kD];
  __shared__ float red[2];
  const int d = threadIdx.x;
  const int b = blockIdx.x / a.Hq, h = blockIdx.x - b * a.Hq;
  const int g = h / a.group, hh = h - g * a.group;
  const int len = a.seq_len[b];
  // with an append the chunks hold the len - 1 older tokens and the new
  // token's partial sits apart
  const bool extra = a.part_new != nullptr && len >= 1;
  const int lc = a.part_new != nullptr ? len - 1 : len;
  // chunks holding tokens: those starting below tile L = ceil(lc / 64)
  // (the first cr chunks have cq + 1 tiles, the others cq >= 1)
  const int L = max(0, (lc + kTile - 1) / kTile), big = a.cr * (a.cq + 1);
  const int n = min(a.nc, L <= big ? (L + a.cq) / (a.cq + 1) : a.cr + (L - big + a.cq - 1) / a.cq);
  const float *src = a.part + (((int64_t)b * a.Hkv + g) * a.nc) * 4 * kPart + hh * kPart;
  const float *pe = extra ? a.part_new + ((int64_t)b * a.Hkv + g) * 4 * kPart + hh * kPart : nullptr;
  // an empty sequence (a caller error) gives a zero row
  buf[d] = n <= kFewParts ? lse_merge_few(src, 4 * kPart, n, pe) : lse_merge(src, 4 * kPart, n, pe, red, wts);
  // inverse rotation: o = D_V * H * o' / 128 (H * H = 128 I)
#pragma unroll
  for (int w = 1; w < kD; w <<= 1) {
    __syncthreads();
    const float v = buf[d], pv = buf[d ^ w];
    __syncthreads();
    buf[d] = (d & w) ? pv - v : v + pv;
  }
  __syncthreads();
  const uint64_t sw = dev_splitmix64(vseed, 2ull * (uint64_t)g + (uint64_t)(d >> 6));
  float r = buf[d] * 0.0078125f;
  if ((sw >> (d & 63)) & 1ull) r = -r;
  const int64_t oi = ((int64_t)b * a.Hq + h) * kD + d;
  if (a.out_bf16) {
    const uint32_t u = __float_as_uint(r);
    const uint32_t rb = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
    reinterpret_cast<uint16_t *>(a.out)[oi] = (r != r) ? (uint16_t)0x7FC0u : (uint16_t)rb;
  } else {
    reinterpret_cast<float *>(a.out)[oi] = r;
  }
}

// ---------------------------------------------------------------- prefill
// Chunked prefill: the last Tq cached tokens of each sequence are queries;
// query j (position L - Tq + j) attends causally to tokens 0..its position.
// An item is (sequence, kv head, block of tb = 16 / group query tokens,
// context chunk): every decoded tile serves 16 query rows (row r = token
// r / group of the block, head r % group of the kv group).
//  - QK: as in decode, each lane decodes one token and its 4 levels per
//    step are the B column of 4x4x4 MFMAs; the four row groups' query
//    operands (fp16 hi/lo) sit in lanes 0..3 and are broadcast (cbsz 4).
//  - softmax per row with the causal mask; P (hi/lo) to LDS as
//    [row][token quad][hi x4, lo x4].
//  - PV: 16x16x16 MFMAs of P (16 rows x 16 tokens) with the transposed V
//    tile (16 tokens x 16 dims); lane l ends with rows 4 (l / 16) + i of
//    dim 16 db + l % 16.
constexpr int kRows = 16;
// rotated queries, halves per (b, g, block) in either layout:
//   per-block decode: [dim quad][lane][row group][hi4 lo4]
//   shared decode:    [32-dim block][lane][hi8 lo8], lane 16 j + r holding
//                     dims 8 j .. 8 j + 7 of the block for row r (the B
//                     operand of a 16x16x32 MFMA)
constexpr int kQrotPrefill = 32 * 4 * 4 * 8;

typedef float floatx4v __attribute__((ext_vector_type(4)));

template <bool SHARED>
__global__ void __launch_bounds__(64) rotate_qp_kernel(AttnArgs a, uint64_t kseed) {
  const int lane = threadIdx.x;
  // block = ((b * nqb + qb) * tb + tl) * Hq + h
  int64_t blk = blockIdx.x;
  const int h = (int)(blk % a.Hq);
  blk /= a.Hq;
  const int tl = (int)(blk % a.tb);
  blk /= a.tb;
  const int qb = (int)(blk % a.nqb);
  const int b = (int)(blk / a.nqb);
  const int g = h / a.group, hh = h - g * a.group;
  const int tq = qb * a.tb + tl;
  const int r = tl * a.group + hh, i = r & 3, rg = r >> 2;
  uint16_t *dst = a.qrot + (((int64_t)b * a.Hkv + g) * a.nqb + qb) * kQrotPrefill;
  const int d0 = lane, d1 = lane + 64;
  auto at = [&](int d) {
    return SHARED ? (((d >> 5) * 64 + ((d & 31) >> 3) * 16 + r) * 16) + (d & 7)
                  : ((((d >> 2) * 4 + i) * 4 + rg) * 8) + (d & 3);
  };
  const int lo = SHARED ? 8 : 4;  // offset of the lo half
  if (tq >= a.Tq) {
    dst[at(d0)] = 0; dst[at(d0) + lo] = 0; dst[at(d1)] = 0; dst[at(d1) + lo] = 0;
    return;
  }
  const uint16_t *qp = a.q + (((int64_t)b * a.Tq + tq) * a.Hq + h) * kD;
  const uint64_t w0 = dev_splitmix64(kseed, 2ull * (uint64_t)g);
  const uint64_t w1 = dev_splitmix64(kseed, 2ull * (uint64_t)g + 1ull);
  float v0 = __uint_as_float((uint32_t)qp[d0] << 16);
  float v1 = __uint_as_float((uint32_t)qp[d1] << 16);
  if ((w0 >> lane) & 1ull) v0 = -v0;
  if ((w1 >> lane) & 1ull) v1 = -v1;
  float t0 = v0 + v1, t1 = v0 - v1;
  v0 = t0;
  v1 = t1;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const float p0 = __shfl_xor(v0, w), p1 = __shfl_xor(v1, w);
    const bool hi = lane & w;
    v0 = hi ? p0 - v0 : v0 + p0;
    v1 = hi ? p1 - v1 : v1 + p1;
  }
  const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
  const _Float16 l0 = (_Float16)(v0 - (float)h0), l1 = (_Float16)(v1 - (float)h1);
  dst[at(d0)] = __builtin_bit_cast(uint16_t, h0);
  dst[at(d0) + lo] = __builtin_bit_cast(uint16_t, l0);
  dst[at(d1)] = __builtin_bit_cast(uint16_t, h1);
  dst[at(d1) + lo] = __builtin_bit_cast(uint16_t, l1);
}

__host__ __device__ inline WaveLayout prefill_layout(int Ck, int Cv) {
  WaveLayout w;
  w.kst = 0;
  w.vst = w.kst + ((kTile * Ck + 31) & ~15);
  w.pl = w.vst + ((kTile * Cv + 31) & ~15);
  w.vt = w.pl + kRows * kTile * 2 * 2;  // P: [16 rows][16 quads][hi4 lo4]
  w.bytes = w.vt + kPass * kVtStride * 2;
  w.bytes = (w.bytes + 15) & ~15;
  return w;
}

template <bool DK, bool DV>
__device__ __forceinline__ void prefill_tile_pass(const DecTab tk, const DecTab tv, const uint8_t *kb,
                                                  const uint8_t *vb, const uint4 *qg, const uint16_t *pl,
                                                  uint16_t *vt, floatx4 (&sc)[4], floatx4 (&acc)[8], int lane) {
  const bool qlane = lane < 4;
  uint4 qn[4] = {};
  if (DK && qlane) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) qn[rg] = qg[lane * 4 + rg];
  }
  uint32_t xk = 0, xv = 0;
  lds_u8 *pk = nullptr, *pv = nullptr;
  if (DK) {
    xk = load_le32(kb);
    pk = to_lds(kb + 4);
  }
  if (DV) {
    xv = load_le32(vb);
    pv = to_lds(vb + 4);
  }
  uint16_t *col = vt + lane;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    for (int gq = 0; gq < kPass / 4; ++gq) {
      const int gnext = p * (kPass / 4) + gq + 1;
      uint32_t lv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // the two chains' loads are issued in this order (volatile), so
        // each LDS round trip of one chain overlaps the other's
        uint32_t bk = 0, bv = 0, sk = 0, sv = 0;
        uint2 ek = make_uint2(0, 0), ev = make_uint2(0, 0);
        if (DK) bk = next_byte(pk);
        if (DV) bv = next_byte(pv);
        if (DK) sk = lookup_sym8(tk, xk);
        if (DV) sv = lookup_sym8(tv, xv);
        if (DK) ek = lookup_symtab(tk, sk);
        if (DV) ev = lookup_symtab(tv, sv);
        if (DK) {
          xk = rans_advance(xk, ek);
          renorm(xk, pk, bk);
          lv[j] = ek.y;
        }
        if (DV) {
          xv = rans_advance(xv, ev);
          renorm(xv, pv, bv);
          col[(gq * 4 + j) * kVtStride] = (uint16_t)(ev.y >> 16);
        }
      }
      if (DK) {
        const uint32_t b01 = __builtin_amdgcn_perm(lv[1], lv[0], 0x07060302u);
        const uint32_t b23 = __builtin_amdgcn_perm(lv[3], lv[2], 0x07060302u);
        const half4 Bk = __builtin_bit_cast(half4, make_uint2(b01, b23));
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          sc[rg] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4, make_uint2(qn[rg].x, qn[rg].y)), Bk,
                                                      sc[rg], 4, 0, 0);
          sc[rg] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4, make_uint2(qn[rg].z, qn[rg].w)), Bk,
                                                      sc[rg], 4, 0, 0);
        }
        // next dim group's query operands, in flight during its decode
        if (qlane && gnext < 32) {
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) qn[rg] = qg[(gnext * 4 + lane) * 4 + rg];
        }
      }
    }
    if (DV) {
      wave_sync();
      const int m = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        // P rows x tokens 16 kc .. 16 kc + 15: this lane's row m, tokens 4 kq .. 4 kq + 3
        const uint4 pp = *reinterpret_cast<const uint4 *>(pl + (m * 16 + kc * 4 + kq) * 8);
        const half4 Ph = __builtin_bit_cast(half4, make_uint2(pp.x, pp.y));
        const half4 Pl = __builtin_bit_cast(half4, make_uint2(pp.z, pp.w));
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          // V tokens 16 kc + 4 kq .. + 3 of dim 16 db + m (of this pass)
          const uint32_t *r = reinterpret_cast<const uint32_t *>(vt + (16 * db + m) * kVtStride + 16 * kc + 4 * kq);
          const half4 V = __builtin_bit_cast(half4, make_uint2(r[0], r[1]));
          acc[2 * p + db] = __builtin_amdgcn_mfma_f32_16x16x16f16(Ph, V, acc[2 * p + db], 0, 0, 0);
          acc[2 * p + db] = __builtin_amdgcn_mfma_f32_16x16x16f16(Pl, V, acc[2 * p + db], 0, 0, 0);
        }
      }
      wave_sync();
    }
  }
}

// Online softmax for one tile and 16 rows.  Lane = token (absolute position
// tpos); row r is valid for it when tpos <= pos0 + r / group (causal) and
// the token is inside the item's range.
__device__ __forceinline__ void prefill_softmax(const floatx4 (&sc)[4], uint32_t nk_bits, uint32_t nv_bits,
                                                bool in_range, int tpos, int pos0, int group, float qk_scale,
                                                float (&m_run)[kRows], float (&l_lane)[kRows], uint16_t *pl,
                                                floatx4 (&acc)[8], int lane) {
  const float nk = (float)__builtin_bit_cast(_Float16, (uint16_t)nk_bits);
  const float nv = (float)__builtin_bit_cast(_Float16, (uint16_t)nv_bits);
  float s[kRows];
  bool ok[kRows];
  bool over = false;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    ok[r] = in_range && tpos <= pos0 + r / group;
    s[r] = ok[r] ? sc[r >> 2][r & 3] * nk * qk_scale : -__builtin_inff();
    over |= s[r] > m_run[r];
  }
  if (__builtin_amdgcn_read_exec() & __ballot(over)) {
    float alpha[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const float m_new = fmaxf(m_run[r], wave_max(s[r]));
      alpha[r] = m_new == -__builtin_inff() ? 1.0f : exp2f(m_run[r] - m_new);
      l_lane[r] *= alpha[r];
      m_run[r] = m_new;
    }
    // acc[db][i] holds row 4 (lane / 16) + i
    const int q4 = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = q4 == 0 ? alpha[i] : q4 == 1 ? alpha[4 + i] : q4 == 2 ? alpha[8 + i] : alpha[12 + i];
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db][i] *= ai;
    }
  }
  uint16_t *q8 = pl + (lane >> 2) * 8 + (lane & 3);
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const float p = ok[r] ? exp2f(s[r] - m_run[r]) : 0.0f;
    l_lane[r] += p;
    const float pv = p * nv;
    const _Float16 hi = (_Float16)pv;
    q8[r * 16 * 8] = __builtin_bit_cast(uint16_t, hi);
    q8[r * 16 * 8 + 4] = __builtin_bit_cast(uint16_t, (_Float16)(pv - (float)hi));
  }
}

// Larger containers (NQ 5, 9) hold more tile bytes per lane: those variants
// run one wave per SIMD, with the whole register file, so nothing spills.
template <int NQ>
__global__ void __launch_bounds__(NQ == 3 ? 512 : 256) attn_prefill_kernel(AttnArgs a, Tables tk, Tables tv) {
  __shared__ uint8_t sym8[2][kM];
  __shared__ uint2 symtab[2][kMaxLevels];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const DecTab dk{sym8[0], symtab[0]};
  const DecTab dv{sym8[1], symtab[1]};
  build_tables(sym8[0], symtab[0], tk, threadIdx.x, blockDim.x);
  build_tables(sym8[1], symtab[1], tv, threadIdx.x, blockDim.x);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int tok = lane_token(lane);
  const int wave = threadIdx.x >> 6;
  const int Ck = tk.C, Cv = tv.C;
  const WaveLayout L = prefill_layout(Ck, Cv);
  uint8_t *base = smem + (size_t)wave * L.bytes;
  uint8_t *kst = base + L.kst;
  uint8_t *vst = base + L.vst;
  uint16_t *pl = reinterpret_cast<uint16_t *>(base + L.pl);
  uint16_t *vt = reinterpret_cast<uint16_t *>(base + L.vt);
  const uint8_t *kpool_end = a.kc + (size_t)a.Hkv * a.S * Ck;
  const uint8_t *vpool_end = a.vc + (size_t)a.Hkv * a.S * Cv;
  const int64_t W = (int64_t)gridDim.x * a.waves_per_block;

  for (int64_t item = (int64_t)blockIdx.x * a.waves_per_block + wave; item < a.n_items; item += W) {
    const int c = (int)(item % a.nc);
    int64_t rest = item / a.nc;
    const int qb = (int)(rest % a.nqb);
    const int64_t bg = rest / a.nqb;
    const int b = (int)(bg / a.Hkv), g = (int)(bg - (int64_t)b * a.Hkv);
    const int len = a.seq_len[b];
    const int pos0 = len - a.Tq + qb * a.tb;                  // position of the block's first query
    const int pmax = pos0 + min(a.tb, a.Tq - qb * a.tb) - 1;  // of its last
    const int t0 = c * a.chunk;
    if (t0 > pmax || pmax < 0) continue;
    const int t1 = min(t0 + a.chunk, pmax + 1);
    const int ntiles = (t1 - t0 + kTile - 1) / kTile;
    const int64_t plane0 = (int64_t)g * a.S;
    const int64_t seq0 = a.seq_start[b];  // read once per item, not after each tile prefetch
    auto tile_base = [&](int tile) -> int64_t { return plane0 + seq0 + t0 + tile * kTile; };

    wave_sync();
    const uint4 *qr = reinterpret_cast<const uint4 *>(a.qrot + ((bg * a.nqb) + qb) * kQrotPrefill);
    auto norms = [&](int64_t tbase, uint32_t &nk, uint32_t &nv) {
      const int64_t idx = tbase + tok;
      const bool ok = idx >= plane0 && idx < plane0 + a.S;
      nk = ok ? a.kn[idx] : 0u;
      nv = ok ? a.vn[idx] : 0u;
    };
    TileRegs<NQ> rk, rv;
    uint32_t nk0, nv0, nk1 = 0, nv1 = 0;
    const int64_t base0 = tile_base(0);
    int64_t vbase = base0;
    fetch<NQ>(rk, a.kc + base0 * Ck, kTile * Ck, a.kc, kpool_end, lane);
    norms(base0, nk0, nv0);
    commit<NQ>(rk, kst, kTile * Ck, lane);
    const int koff0 = rk.off;
    wave_sync();
    fetch<NQ>(rv, a.vc + vbase * Cv, kTile * Cv, a.vc, vpool_end, lane);
    if (ntiles > 1) {
      const int64_t base1 = tile_base(1);
      fetch<NQ>(rk, a.kc + base1 * Ck, kTile * Ck, a.kc, kpool_end, lane);
      norms(base1, nk1, nv1);
      vbase = base1;
    }
    float m_run[kRows], l_lane[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      m_run[r] = -__builtin_inff();
      l_lane[r] = 0.0f;
    }
    floatx4 acc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    floatx4 sc[4];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) sc[rg] = floatx4{0.f, 0.f, 0.f, 0.f};
    prefill_tile_pass<true, false>(dk, dv, kst + koff0 + tok * Ck, nullptr, qr, pl, vt, sc, acc, lane);
    prefill_softmax(sc, nk0, nv0, t0 + tok < t1, t0 + tok, pos0, a.group, a.qk_scale, m_run, l_lane, pl, acc,
                    lane);

    for (int j = 0; j < ntiles; ++j) {
      const bool next = j + 1 < ntiles;
      wave_sync();
      commit<NQ>(rv, vst, kTile * Cv, lane);
      const int voff = rv.off;
      int koff = 0;
      if (next) {
        commit<NQ>(rk, kst, kTile * Ck, lane);
        koff = rk.off;
      }
      wave_sync();
      uint32_t nk2 = 0, nv2 = 0;
      const int64_t base2 = j + 2 < ntiles ? tile_base(j + 2) : 0;
      if (next) fetch<NQ>(rv, a.vc + vbase * Cv, kTile * Cv, a.vc, vpool_end, lane);
      if (j + 2 < ntiles) {
        fetch<NQ>(rk, a.kc + base2 * Ck, kTile * Ck, a.kc, kpool_end, lane);
        norms(base2, nk2, nv2);
        vbase = base2;
      }
      if (next) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) sc[rg] = floatx4{0.f, 0.f, 0.f, 0.f};
        prefill_tile_pass<true, true>(dk, dv, kst + koff + tok * Ck, vst + voff + tok * Cv, qr, pl, vt, sc, acc,
                                      lane);
        const int tp = t0 + (j + 1) * kTile + tok;
        prefill_softmax(sc, nk1, nv1, tp < t1, tp, pos0, a.group, a.qk_scale, m_run, l_lane, pl, acc, lane);
      } else {
        prefill_tile_pass<false, true>(dk, dv, nullptr, vst + voff + tok * Cv, qr, pl, vt, sc, acc, lane);
      }
      nk1 = nk2;
      nv1 = nv2;
    }

    // partial: lane l holds rows 4 (l / 16) + i of dims 16 db + l % 16
    float *dst = a.part + item * kRows * kPart;
    const int q4 = lane >> 4, dn = lane & 15;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(4 * q4 + i) * kPart + 16 * db + dn] = acc[db][i];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const float l = wave_sum(l_lane[r]);
      if (lane == r) {
        dst[r * kPart + 128] = m_run[r];
        dst[r * kPart + 129] = l;
      }
    }
  }
}

// ---------------------------------------------------------------- prefill, shared decode
// For containers of up to 35 bytes (the LDS holds 8 staging slices of 64
// containers beside the level tiles).  A block of kSbWaves waves takes an
// item (sequence, kv head, kSbWaves consecutive query blocks of 16 rows,
// context chunk).  The chunk goes by in rounds of kRoundTiles tiles: waves
// 0..3 decode K of the round's tiles and waves 4..7 V, one container per
// lane, into fp16 level tiles in LDS; then every wave runs its own 16 rows
// over those tiles on 16x16x32 MFMAs.  A tile is decoded once for the
// item's 128 rows instead of once per 16.
//
// Scores are formed transposed, S^T = K q~^T (tokens x rows), so that each
// lane ends with 4 tokens of one row (lane l: row l mod 16, tokens 4 (l / 16)
// .. + 3 of each 16-token block).  After the softmax those values, two
// 16-token blocks at a time, are as they stand the B operand of
// O^T = V^T P^T, and the running max and sum are one value per lane.
constexpr int kSbWaves = 8;
constexpr int kRoundTiles = 4;
// Level tiles, fp16, rows padded by one dword pair (K) or one dword (V) so
// that the 16 rows x 2 chunks a half-wave reads for an MFMA operand spread
// over the banks (at most two-way), with every address a per-lane base plus
// an immediate:
//   K: [token][dims], 132 halves a row (8-byte operand reads stay aligned)
//   V: [dim][tokens],  66 halves a row (operands read as two dwords)
constexpr int kKlRow = kD + 4, kVlRow = kTile + 2;
constexpr int kLvHalves = kTile * kKlRow;  // = kD * kVlRow: one K or V level tile
static_assert(kTile * kKlRow == kD * kVlRow, "K and V level tiles share a size");
typedef _Float16 half4a __attribute__((ext_vector_type(4), aligned(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half8a __attribute__((ext_vector_type(8), aligned(8)));

__host__ __device__ inline size_t prefill_shared_lds(int Ck, int Cv) {
  const int cmax = Ck > Cv ? Ck : Cv;
  return (size_t)2 * kRoundTiles * kLvHalves * 2 + 2 * kRoundTiles * kTile * 4 +
         (size_t)kSbWaves * ((kTile * cmax + 31) & ~15);
}

// One container per lane, a single rANS chain: K levels go to the K tile
// four at a time, V levels one per step to the V tile.
template <bool V>
__device__ __forceinline__ void decode_levels(const DecTab t, const uint8_t *cb, uint16_t *dst, int tok) {
  uint32_t x = load_le32(cb);
  lds_u8 *p = to_lds(cb + 4);
#pragma unroll
  for (int G = 0; G < kD / 4; ++G) {
    uint32_t lv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t bt = next_byte(p);
      const uint32_t s8 = lookup_sym8(t, x);
      const uint2 e = lookup_symtab(t, s8);
      x = rans_advance(x, e);
      renorm(x, p, bt);
      lv[j] = e.y;
      if (V) dst[(4 * G + j) * kVlRow + tok] = (uint16_t)(e.y >> 16);
    }
    if (!V) {
      const uint32_t b01 = __builtin_amdgcn_perm(lv[1], lv[0], 0x07060302u);
      const uint32_t b23 = __builtin_amdgcn_perm(lv[3], lv[2], 0x07060302u);
      *reinterpret_cast<uint2 *>(dst + tok * kKlRow + 4 * G) = make_uint2(b01, b23);
    }
  }
}

// One decoded tile against this wave's 16 rows: S^T, the online softmax of
// each row (lane l: row l mod 16), and O^T += V^T P^T, on 16x16x32 MFMAs.
// A lane's 8-value k group is 8 consecutive dims for S^T; for O^T it is the
// 4 tokens 4 (l / 16) + i of each of two 16-token blocks, the tokens the
// lane holds scores for (the order inside a group is free, as long as both
// operands use the same one).  tpos0 is the position of the tile's first
// token; a token is visible to a row when it lies before t1 and at or
// before the row's query position qpos.
__device__ __forceinline__ void shared_tile(const uint16_t *kt, const uint16_t *vtl, const float *knl,
                                            const float *vnl, const half8 (&qh)[4], const half8 (&ql)[4],
                                            int tpos0, int t1, int qpos, float &m_run, float &l_run,
                                            floatx4 (&acc)[8], int lane) {
  const int m = lane & 15, kq = lane >> 4;
  floatx4 st[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) st[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < kD / 32; ++kb) {
    half8 A[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) A[tb] = *reinterpret_cast<const half8a *>(kt + (16 * tb + m) * kKlRow + 32 * kb + 8 * kq);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) st[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[tb], qh[kb], st[tb], 0, 0, 0);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) st[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[tb], ql[kb], st[tb], 0, 0, 0);
  }
  // token 16 tb + 4 kq + i of the tile is visible when 16 tb + i <= lim
  const int lim = min(t1 - 1, qpos) - tpos0 - 4 * kq;
  float mx = -__builtin_inff();
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const float4 nk = *reinterpret_cast<const float4 *>(knl + 16 * tb + 4 * kq);  // n_k * scale
    const float nkv[4] = {nk.x, nk.y, nk.z, nk.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st[tb][i] = 16 * tb + i <= lim ? st[tb][i] * nkv[i] : -__builtin_inff();
      mx = fmaxf(mx, st[tb][i]);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(m_run, mx);
  if (__builtin_amdgcn_read_exec() & __ballot(m_new > m_run)) {
    const float alpha = m_new > m_run ? exp2f(m_run - m_new) : 1.0f;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;
    m_run = m_new;
  }
  // a row with nothing visible yet keeps m = -inf; its scores are -inf too
  const float m_use = m_run == -__builtin_inff() ? 0.0f : m_run;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    half8 ph, pl;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tb = 2 * h + u;
      const float4 nv = *reinterpret_cast<const float4 *>(vnl + 16 * tb + 4 * kq);
      const float nvv[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(st[tb][i] - m_use);
        l_run += p;
        // P = p * n_v as an fp16 pair, as in decode attention
        const float pv = p * nvv[i];
        const _Float16 hi = (_Float16)pv;
        ph[4 * u + i] = hi;
        pl[4 * u + i] = (_Float16)(pv - (float)hi);
      }
    }
    half8 A[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t *row = vtl + (16 * db + m) * kVlRow + 32 * h + 4 * kq;
      const half4a v0 = *reinterpret_cast<const half4a *>(row);
      const half4a v1 = *reinterpret_cast<const half4a *>(row + 16);
      A[db] = half8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[db], ph, acc[db], 0, 0, 0);
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[db], pl, acc[db], 0, 0, 0);
  }
}

template <int NQ>
__global__ void __launch_bounds__(64 * kSbWaves) attn_prefill_shared_kernel(AttnArgs a, Tables tk, Tables tv) {
  __shared__ uint8_t sym8[2][kM];
  __shared__ uint2 symtab[2][kMaxLevels];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const DecTab dk{sym8[0], symtab[0]};
  const DecTab dv{sym8[1], symtab[1]};
  build_tables(sym8[0], symtab[0], tk, threadIdx.x, blockDim.x);
  build_tables(sym8[1], symtab[1], tv, threadIdx.x, blockDim.x);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok = lane_token(lane);
  // decode role: K (waves 0..3) or V (4..7) of the round's tile wave mod 4
  const bool isv = wave >= kRoundTiles;
  const int dtile = wave & (kRoundTiles - 1);
  const int C = isv ? tv.C : tk.C;
  const int cmax = tk.C > tv.C ? tk.C : tv.C;
  uint16_t *kl = reinterpret_cast<uint16_t *>(smem);
  uint16_t *vl = kl + kRoundTiles * kLvHalves;
  float *knl = reinterpret_cast<float *>(vl + kRoundTiles * kLvHalves);
  float *vnl = knl + kRoundTiles * kTile;
  uint8_t *stg = reinterpret_cast<uint8_t *>(vnl + kRoundTiles * kTile) + wave * ((kTile * cmax + 31) & ~15);
  const uint8_t *pool = isv ? a.vc : a.kc;
  const uint8_t *pool_end = pool + (size_t)a.Hkv * a.S * C;
  const uint16_t *norm = isv ? a.vn : a.kn;
  const int m = lane & 15, kq = lane >> 4;
  const int nsb = (a.nqb + kSbWaves - 1) / kSbWaves;

  for (int64_t item = blockIdx.x; item < a.n_items; item += gridDim.x) {
    const int c = (int)(item % a.nc);
    const int64_t rest = item / a.nc;
    const int sb = (int)(rest % nsb);
    const int64_t bg = rest / nsb;
    const int b = (int)(bg / a.Hkv), g = (int)(bg - (int64_t)b * a.Hkv);
    const int len = a.seq_len[b];
    const int qb = sb * kSbWaves + wave;  // this wave's query block
    const bool qvalid = qb < a.nqb;
    const int qb_last = min(sb * kSbWaves + kSbWaves, a.nqb) - 1;
    // position of the item's last query row, and of this wave's first and last
    const int pmax = len - a.Tq + min(qb_last * a.tb + a.tb, a.Tq) - 1;
    const int pos0 = len - a.Tq + qb * a.tb;
    const int pend = pos0 + a.tb - 1;
    const int t0 = c * a.chunk;
    if (t0 > pmax || pmax < 0) continue;  // the same for the whole block
    const int t1 = min(t0 + a.chunk, pmax + 1);
    const int ntiles = (t1 - t0 + kTile - 1) / kTile;
    const int64_t plane0 = (int64_t)g * a.S;
    const int64_t sbase = plane0 + a.seq_start[b] + t0;  // pool index of token t0
    const int qpos = pos0 + m / a.group;                   // query position of this lane's row

    half8 qh[4], ql[4];
    if (qvalid) {
      const uint4 *qg = reinterpret_cast<const uint4 *>(a.qrot + ((bg * a.nqb) + qb) * kQrotPrefill);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        qh[kb] = __builtin_bit_cast(half8, qg[(kb * 64 + lane) * 2]);
        ql[kb] = __builtin_bit_cast(half8, qg[(kb * 64 + lane) * 2 + 1]);
      }
    }
    float m_run = -__builtin_inff(), l_run = 0.0f;
    floatx4 acc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = floatx4{0.f, 0.f, 0.f, 0.f};

    TileRegs<NQ> rr;
    if (dtile < ntiles) fetch<NQ>(rr, pool + sbase * C + (int64_t)dtile * kTile * C, kTile * C, pool, pool_end, lane);
    for (int r0 = 0; r0 < ntiles; r0 += kRoundTiles) {
      const int tile = r0 + dtile;
      if (tile < ntiles) {  // the same for the whole wave
        commit<NQ>(rr, stg, kTile * C, lane);
        const int off = rr.off;
        wave_sync();
        const int64_t idx = sbase + (int64_t)tile * kTile + tok;
        const bool ok = idx >= plane0 && idx < plane0 + a.S;
        const float nrm = ok ? (float)__builtin_bit_cast(_Float16, norm[idx]) : 0.0f;
        if (tile + kRoundTiles < ntiles)
          fetch<NQ>(rr, pool + (sbase + (int64_t)(tile + kRoundTiles) * kTile) * C, kTile * C, pool, pool_end, lane);
        // one call per kernel argument (a table chosen at run time would go to scratch)
        if (isv) {
          decode_levels<true>(dv, stg + off + tok * C, vl + dtile * kLvHalves, tok);
          vnl[dtile * kTile + tok] = nrm;
        } else {
          decode_levels<false>(dk, stg + off + tok * C, kl + dtile * kLvHalves, tok);
          knl[dtile * kTile + tok] = nrm * a.qk_scale;
        }
      }
      __syncthreads();  // the round's level tiles and norms are complete
      if (qvalid) {
        for (int tt = 0; tt < kRoundTiles; ++tt) {
          const int tp0 = t0 + (r0 + tt) * kTile;
          if (r0 + tt >= ntiles || tp0 > pend) break;  // later tiles are masked for every row
          shared_tile(kl + tt * kLvHalves, vl + tt * kLvHalves, knl + tt * kTile, vnl + tt * kTile, qh, ql, tp0, t1,
                      qpos, m_run, l_run, acc, lane);
        }
      }
      __syncthreads();  // every read of the round's tiles is done
    }

    if (qvalid) {
      // partial of (b, g, qb, c): lane l holds dims 16 db + 4 (l / 16) + i of row l mod 16
      float *dst = a.part + ((((int64_t)b * a.Hkv + g) * a.nqb + qb) * a.nc + c) * kRows * kPart + m * kPart;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[16 * db + 4 * kq + i] = acc[db][i];
      float l = l_run + __shfl_xor(l_run, 16);
      l += __shfl_xor(l, 32);
      if (kq == 0) {
        dst[128] = m_run;
        dst[129] = l;
      }
    }
  }
}

__global__ void __launch_bounds__(128) prefill_combine_kernel(AttnArgs a, uint64_t vseed) {
  __shared__ float buf[kD];
  __shared__ float wts[kD];
  __shared__ float red[2];
  const int d = threadIdx.x;
  int64_t blk = blockIdx.x;  // (b * Tq + tq) * Hq + h
  const int h = (int)(blk % a.Hq);
  blk /= a.Hq;
  const int tq = (int)(blk % a.Tq);
  const int b = (int)(blk / a.Tq);
  const int g = h / a.group, hh = h - g * a.group;
  const int qb = tq / a.tb, r = (tq - qb * a.tb) * a.group + hh;
  const int pos = a.seq_len[b] - a.Tq + tq;
  const int n = pos < 0 ? 0 : min(pos / a.chunk + 1, a.nc);
  const float *src = a.part + ((((int64_t)b * a.Hkv + g) * a.nqb + qb) * a.nc) * kRows * kPart + r * kPart;
  // a chunk with no token visible to the row has m = -inf and weighs nothing
  buf[d] = lse_merge(src, kRows * kPart, n, nullptr, red, wts);
#pragma unroll
  for (int w = 1; w < kD; w <<= 1) {
    __syncthreads();
    const float v = buf[d], pv = buf[d ^ w];
    __syncthreads();
    buf[d] = (d & w) ? pv - v : v + pv;
  }
  __syncthreads();
  const uint64_t sw = dev_splitmix64(vseed, 2ull * (uint64_t)g + (uint64_t)(d >> 6));
  float rv = buf[d] * 0.0078125f;
  if ((sw >> (d & 63)) & 1ull) rv = -rv;
  const int64_t oi = (((int64_t)b * a.Tq + tq) * a.Hq + h) * kD + d;
  if (a.out_bf16) {
    const uint32_t u = __float_as_uint(rv);
    const uint32_t rb = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    reinterpret_cast<uint16_t *>(a.out)[oi] = (rv != rv) ? (uint16_t)0x7FC0u : (uint16_t)rb;
  } else {
    reinterpret_cast<float *>(a.out)[oi] = rv;
  }
}

// ---------------------------------------------------------------- planning
struct Plan {
  int chunk, nc, cq, cr, waves_per_block, blocks_cap, nq;
  bool lat;   // latency mode (whole V tiles in LDS, fewer waves per CU)
  bool slot;  // per-slot decode tables (one LDS round trip per decode step)
  int64_t n_items;
  size_t lds, qrot_bytes, part_bytes, part_new_bytes, queue_bytes, total;
};

// CU count of the current device, read once per process (thread-safe static
// initialisation; the library plans for the one device it runs on)
int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
  }();
  return cus;
}

// Context split.  A launch deals its items (units x nc, the nc chunks of a
// max_len sequence balanced to within one tile) round-robin to W resident
// waves, so it takes about ceil(units * nc / W) rounds of (longest chunk +
// c0) token-times, c0 being an item's fixed cost (a K-only and a V-only tile
// pass and the partial; about 32 tokens on MI355X).  The chunk count from a
// chunk length of 64 to 2048 tokens (only max_len is known here, and ragged
// batches need the finer items to balance) minimising that is chosen; W is a
// fixed function of the
// CU count, so the workspace size depends only on the call's shape.  Small
// batches get one-tile chunks: an item is then a K pass and a V pass, the
// shortest latency a wave can give a tile.
// DQ_KNOB_SPLIT_TOKENS forces a chunk (tests use it).
int64_t choose_chunk(int64_t units, int64_t max_len, int64_t W) {
  const int64_t c0 = 32;
  int64_t best = 1024, best_cost = INT64_MAX;
  for (int64_t chunk = kTile; chunk <= 4096; chunk += kTile) {
    const int64_t nc = (max_len + chunk - 1) / chunk;
    const int64_t tiles = (max_len + kTile - 1) / kTile;
    const int64_t span = ((tiles + nc - 1) / nc) * kTile;  // the longest of nc balanced chunks
    const int64_t rounds = (units * nc + W - 1) / W;
    // chunks past 2048 tokens only when the items then fill one round: a
    // wave takes a single item, and a ragged batch's longest items are no
    // longer than two of the finer split's would be together
    if (chunk > 2048 && rounds > 1) continue;
    const int64_t cost = rounds * (span + c0);
    if (cost < best_cost) {
      best_cost = cost;
      best = chunk;
    }
    if (nc == 1) break;  // larger chunks change nothing
  }
  const int64_t forced = knob(DQ_KNOB_SPLIT_TOKENS);
  if (forced >= kTile && forced % kTile == 0) best = forced;
  return best;
}

int make_plan(int B, int Hq, int Hkv, int64_t max_len, int Ck, int Cv, Plan *pl) {
  (void)Hq;
  const int cus = device_cus();
  if (cus <= 0) return DQ_ERR_HIP;
  const int cmax = Ck > Cv ? Ck : Cv;
  pl->nq = cmax <= 47 ? 3 : (cmax <= 79 ? 5 : 9);  // 16-byte pieces per lane per tile
  const int wb = wave_layout(Ck, Cv).bytes;
  const int lds_cap = 160 * 1024;
  int wpb = pl->nq == 3 ? 12 : 4;  // three waves per SIMD when the LDS allows (larger C: fewer)
  const int64_t forced_w = knob(DQ_KNOB_SPLITK_WAVES);
  if (forced_w >= 1 && forced_w < wpb) wpb = (int)forced_w;
  while (wpb > 1 && kStaticLds + wpb * wb > lds_cap) wpb -= wpb > 4 ? 4 : 1;
  if (kStaticLds + wpb * wb > lds_cap) return DQ_ERR_UNSUPPORTED;
  // chunk: aim for ~8 items per resident wave (8 waves per CU) if every
  // sequence were max_len; independent of C so the workspace size is too
  const int64_t chunk = choose_chunk((int64_t)B * Hkv, max_len, (int64_t)cus * 12);
  const int64_t nc = (max_len + chunk - 1) / chunk;
  const int64_t tiles = (max_len + kTile - 1) / kTile;  // >= nc
  pl->chunk = (int)chunk;
  pl->nc = (int)nc;
  pl->cq = nc > 0 ? (int)(tiles / nc) : 1;
  pl->cr = nc > 0 ? (int)(tiles % nc) : 0;
  pl->waves_per_block = wpb;
  pl->n_items = (int64_t)B * Hkv * nc;
  pl->lds = (size_t)wpb * wb;  // dynamic part; the decode tables are static
  // latency mode when its fewer resident waves still take every item in one
  // round (small batches); DQ_KNOB_LATENCY_MODE forces it on (1) or off (0)
  pl->lat = false;
  if (pl->nq == 3) {
    const int lwb = wave_layout(Ck, Cv, true).bytes;
    int lwpb = (lds_cap - kStaticLds) / lwb;
    lwpb = lwpb > 12 ? 12 : lwpb;
    bool lat = lwpb >= 1 && pl->n_items <= (int64_t)cus * lwpb;
    const int64_t forced = knob(DQ_KNOB_LATENCY_MODE);
    if (forced >= 0) lat = lwpb >= 1 && forced == 1;
    if (lat) {
      pl->lat = true;
      pl->waves_per_block = lwpb;
      pl->lds = (size_t)lwpb * lwb;
    }
  }
  // per-slot tables where their 64 KB fit beside the waves' slices
  // (containers up to 38 bytes at 12 waves); DQ_KNOB_SLOT_TABLE forces them
  // off (0) or on (1, where they fit)
  pl->slot = false;
  if (!pl->lat && pl->nq == 3) {
    bool slot = kSlotLds + pl->waves_per_block * wb <= lds_cap;
    const int64_t forced = knob(DQ_KNOB_SLOT_TABLE);
    if (forced == 0) slot = false;
    pl->slot = slot;
  }
  pl->blocks_cap = cus;  // one block per CU at most; fewer when the items are few
  pl->qrot_bytes = 0;  // each item rotates its own query
  pl->part_bytes = ((size_t)pl->n_items * 4 * kPart * sizeof(float) + 255) & ~(size_t)255;
  pl->part_new_bytes = (size_t)B * Hkv * 4 * kPart * sizeof(float);  // the append's own partials
  pl->queue_bytes = 256;  // the work queue's counter
  pl->total = pl->qrot_bytes + pl->part_bytes + pl->part_new_bytes + pl->queue_bytes;
  return DQ_OK;
}

template <int NQ, bool APPEND, bool LAT = false, bool SLOT = false, bool VQK = false>
hipError_t launch_splitk(const Plan &pl, const AttnArgs &a, const Tables &tk, const Tables &tv, hipStream_t s) {
  // dynamic LDS beyond the default limit, requested once (thread-safe static)
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void *>(attn_splitk_kernel<NQ, APPEND, LAT, SLOT, VQK>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - (SLOT ? kSlotLds : kStaticLds));
  if (attr != hipSuccess) return attr;
  // the append's encode items (if this launch runs them) come first, one per wave
  const int64_t n = a.n_items + (APPEND ? a.n_enc : 0);
  const int64_t want = (n + pl.waves_per_block - 1) / pl.waves_per_block;
  const int blocks = (int)(want < pl.blocks_cap ? want : pl.blocks_cap);
  hipLaunchKernelGGL((attn_splitk_kernel<NQ, APPEND, LAT, SLOT, VQK>), dim3((unsigned)blocks),
                     dim3(64 * pl.waves_per_block), pl.lds, s, a, tk, tv);
  return hipGetLastError();
}

struct PrefillPlan {
  int chunk, nc, waves_per_block, blocks, nq, tb, nqb;
  bool shared;  // shared-decode kernel (items of kSbWaves query blocks)
  int64_t n_items;
  size_t lds, qrot_bytes, part_bytes, total;
};

// Context split of the shared-decode kernel.  One block per CU takes items
// (units x nc) in turn; an item of span s tokens costs about
// ceil(s / 256) rounds of 4 tiles plus a fixed quarter round.  The chunk (a
// multiple of 64) minimising ceil(items / CUs) x that is chosen.
// DQ_KNOB_SPLIT_TOKENS forces a chunk, as for decode.
int64_t choose_prefill_chunk(int64_t units, int64_t max_len, int cus) {
  const int64_t rt = (int64_t)kRoundTiles * kTile;
  int64_t best = max_len, best_cost = INT64_MAX;
  for (int64_t chunk = rt;; chunk += rt) {
    const int64_t nc = (max_len + chunk - 1) / chunk;
    const int64_t span = nc == 1 ? max_len : chunk;
    const int64_t cost = ((units * nc + cus - 1) / cus) * (4 * ((span + rt - 1) / rt) + 1);
    if (cost < best_cost) {
      best_cost = cost;
      best = nc == 1 ? ((max_len + kTile - 1) / kTile) * kTile : chunk;
    }
    if (nc == 1) break;
  }
  const int64_t forced = knob(DQ_KNOB_SPLIT_TOKENS);
  if (forced >= kTile && forced % kTile == 0) best = forced;
  return best;
}

// Ck, Cv pick the kernel: the shared-decode one when its LDS fits (C up to
// 35), the per-block one otherwise.
int make_prefill_plan(int B, int Tq, int Hq, int Hkv, int64_t max_len, int Ck, int Cv, PrefillPlan *pl) {
  const int cus = device_cus();
  if (cus <= 0) return DQ_ERR_HIP;
  const int group = Hq / Hkv;
  pl->tb = kRows / group;
  pl->nqb = (Tq + pl->tb - 1) / pl->tb;
  const int cmax = Ck > Cv ? Ck : Cv;
  pl->nq = cmax <= 47 ? 3 : (cmax <= 79 ? 5 : 9);
  const int64_t qunits = (int64_t)B * Hkv * pl->nqb;  // (sequence, kv head, query block)
  pl->shared = pl->nq == 3 && kLutBytes + prefill_shared_lds(Ck, Cv) <= 160 * 1024;
  if (pl->shared) {
    const int64_t units = (int64_t)B * Hkv * ((pl->nqb + kSbWaves - 1) / kSbWaves);
    const int64_t chunk = choose_prefill_chunk(units, max_len, cus);
    pl->chunk = (int)chunk;
    pl->nc = (int)((max_len + chunk - 1) / chunk);
    pl->waves_per_block = kSbWaves;
    pl->n_items = units * pl->nc;
    pl->lds = prefill_shared_lds(Ck, Cv);
    pl->blocks = (int)(pl->n_items < cus ? pl->n_items : cus);
  } else {
    const int wb = prefill_layout(Ck, Cv).bytes;
    int wpb = pl->nq == 3 ? 8 : 4;  // the kernel's launch bounds
    while (wpb > 1 && kLutBytes + wpb * wb > 160 * 1024) wpb -= 1;
    if (kLutBytes + wpb * wb > 160 * 1024) return DQ_ERR_UNSUPPORTED;
    const int64_t chunk = choose_chunk(qunits, max_len, (int64_t)cus * 8);
    pl->chunk = (int)chunk;
    pl->nc = (int)((max_len + chunk - 1) / chunk);
    pl->waves_per_block = wpb;
    pl->n_items = qunits * pl->nc;
    pl->lds = (size_t)wpb * wb;
    const int64_t want_blocks = (pl->n_items + wpb - 1) / wpb;
    pl->blocks = (int)(want_blocks < cus ? want_blocks : cus);
  }
  pl->qrot_bytes = ((size_t)qunits * kQrotPrefill * 2 + 255) & ~(size_t)255;
  pl->part_bytes = (size_t)qunits * pl->nc * kRows * kPart * sizeof(float);
  pl->total = pl->qrot_bytes + pl->part_bytes;
  return DQ_OK;
}

template <int NQ>
hipError_t launch_prefill_shared(const PrefillPlan &pl, const AttnArgs &a, const Tables &tk, const Tables &tv,
                                 hipStream_t s) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void *>(attn_prefill_shared_kernel<NQ>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - kLutBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(attn_prefill_shared_kernel<NQ>, dim3((unsigned)pl.blocks), dim3(64 * kSbWaves), pl.lds, s, a,
                     tk, tv);
  return hipGetLastError();
}

template <int NQ>
hipError_t launch_prefill(const PrefillPlan &pl, const AttnArgs &a, const Tables &tk, const Tables &tv,
                          hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(attn_prefill_kernel<NQ>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     160 * 1024 - kLutBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(attn_prefill_kernel<NQ>, dim3((unsigned)pl.blocks), dim3(64 * pl.waves_per_block), pl.lds, s,
                     a, tk, tv);
  return hipGetLastError();
}

}  // namespace
}  // namespace dq

extern "C" int dq_attn_prefill_workspace(int32_t B, int32_t Tq, int32_t Hq, int32_t Hkv, int64_t max_len,
                                         size_t *bytes) {
  if (!bytes || B < 1 || Tq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || max_len < Tq) return DQ_ERR_INVALID;
  const int group = Hq / Hkv;
  if (group != 1 && group != 2 && group != 4) return DQ_ERR_UNSUPPORTED;
  // the kernel (and with it the split) depends on the container sizes, which
  // this call does not know: the larger need of the two kernels
  dq::PrefillPlan p1, p2;
  int st = dq::make_prefill_plan(B, Tq, Hq, Hkv, max_len, 34, 34, &p1);
  if (st) return st;
  st = dq::make_prefill_plan(B, Tq, Hq, Hkv, max_len, 64, 64, &p2);
  if (st) return st;
  *bytes = p1.total > p2.total ? p1.total : p2.total;
  return DQ_OK;
}

extern "C" int dq_attn_prefill(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B, int32_t Tq, int32_t Hq,
                               const uint8_t *k_cont, const uint16_t *k_norm, const uint8_t *v_cont,
                               const uint16_t *v_norm, int64_t num_slots, const int64_t *seq_start,
                               const int32_t *seq_len, int64_t max_len, float sm_scale, int32_t out_dtype,
                               void *out, void *workspace, size_t ws_bytes, dq_stream_t stream) {
  if (!ck || !cv || !q || !k_cont || !k_norm || !v_cont || !v_norm || !seq_start || !seq_len || !out ||
      !workspace)
    return DQ_ERR_INVALID;
  const int Hkv = ck->t.hkv;
  if (cv->t.hkv != Hkv || B < 1 || Tq < 1 || Hq < 1 || Hq % Hkv || num_slots < 1 || max_len < Tq)
    return DQ_ERR_INVALID;
  const int group = Hq / Hkv;
  if (group != 1 && group != 2 && group != 4) return DQ_ERR_UNSUPPORTED;
  if (out_dtype != 0 && out_dtype != 1) return DQ_ERR_INVALID;
  if (max_len > (int64_t)1 << 31) return DQ_ERR_INVALID;
  const uintptr_t kca = reinterpret_cast<uintptr_t>(k_cont), vca = reinterpret_cast<uintptr_t>(v_cont);
  if ((kca & 15u) || (vca & 15u) || ((num_slots * ck->t.C) & 15) || ((num_slots * cv->t.C) & 15))
    return DQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return DQ_ERR_INVALID;
  dq::PrefillPlan pl;
  int st = dq::make_prefill_plan(B, Tq, Hq, Hkv, max_len, ck->t.C, cv->t.C, &pl);
  if (st) return st;
  size_t need = 0;
  st = dq_attn_prefill_workspace(B, Tq, Hq, Hkv, max_len, &need);
  if (st) return st;
  if (ws_bytes < need || pl.total > need) return DQ_ERR_WORKSPACE;

  dq::AttnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = group;
  a.kc = k_cont;
  a.kn = k_norm;
  a.vc = v_cont;
  a.vn = v_norm;
  a.S = num_slots;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.qk_scale = sm_scale * 1.4426950408889634f / 128.0f;
  a.chunk = pl.chunk;
  a.nc = pl.nc;
  a.n_items = pl.n_items;
  a.qrot = static_cast<uint16_t *>(workspace);
  a.part = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pl.qrot_bytes);
  a.out = out;
  a.out_bf16 = out_dtype;
  a.waves_per_block = pl.waves_per_block;
  a.Tq = Tq;
  a.tb = pl.tb;
  a.nqb = pl.nqb;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rot_blocks = (int64_t)B * pl.nqb * pl.tb * Hq;
  hipError_t e;
  if (pl.shared) {
    hipLaunchKernelGGL(dq::rotate_qp_kernel<true>, dim3((unsigned)rot_blocks), dim3(64), 0, s, a, ck->t.seed);
    e = dq::launch_prefill_shared<3>(pl, a, ck->t, cv->t, s);
  } else {
    hipLaunchKernelGGL(dq::rotate_qp_kernel<false>, dim3((unsigned)rot_blocks), dim3(64), 0, s, a, ck->t.seed);
    e = pl.nq == 3   ? dq::launch_prefill<3>(pl, a, ck->t, cv->t, s)
        : pl.nq == 5 ? dq::launch_prefill<5>(pl, a, ck->t, cv->t, s)
                     : dq::launch_prefill<9>(pl, a, ck->t, cv->t, s);
  }
  if (e != hipSuccess) return DQ_ERR_HIP;
  hipLaunchKernelGGL(dq::prefill_combine_kernel, dim3((unsigned)((int64_t)B * Tq * Hq)), dim3(128), 0, s, a,
                     cv->t.seed);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

extern "C" int dq_attn_decode_workspace(int32_t B, int32_t Hq, int32_t Hkv, int64_t max_len, size_t *bytes) {
  if (!bytes || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || max_len < 1) return DQ_ERR_INVALID;
  // the plan depends on C only through the LDS split, not the workspace size
  dq::Plan pl;
  const int st = dq::make_plan(B, Hq, Hkv, max_len, 34, 34, &pl);
  if (st) return st;
  *bytes = pl.total;
  return DQ_OK;
}

// The new tokens of a decode step with append (null: no append).
struct AppendArgs {
  const void *k_new, *v_new;
  int64_t stride_b, stride_h;
  dq_stats *k_stats, *v_stats;
};

static int attn_decode(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B, int32_t Hq, const uint8_t *k_cont,
                       const uint16_t *k_norm, const uint8_t *v_cont, const uint16_t *v_norm, int64_t num_slots,
                       const int64_t *seq_start, const int32_t *pages, int32_t max_pages,
                       const int32_t *seq_len, int64_t max_len, float sm_scale, int32_t out_dtype, void *out,
                       void *workspace, size_t ws_bytes, dq_stream_t stream, hipEvent_t split_begin,
                       hipEvent_t split_end, const AppendArgs *app = nullptr) {
  if (!ck || !cv || !q || !k_cont || !k_norm || !v_cont || !v_norm || (!seq_start && !pages) || !seq_len ||
      !out || !workspace)
    return DQ_ERR_INVALID;
  if (app && (!app->k_new || !app->v_new || (reinterpret_cast<uintptr_t>(app->k_new) & 1u) ||
              (reinterpret_cast<uintptr_t>(app->v_new) & 1u)))
    return DQ_ERR_INVALID;
  if (pages && (max_pages < 1 || max_len > (int64_t)max_pages * dq::kTile)) return DQ_ERR_INVALID;
  const int Hkv = ck->t.hkv;
  if (cv->t.hkv != Hkv || B < 1 || Hq < 1 || Hq % Hkv || num_slots < 1 || max_len < 1) return DQ_ERR_INVALID;
  const int group = Hq / Hkv;
  if (group != 1 && group != 2 && group != 4) return DQ_ERR_UNSUPPORTED;
  if (out_dtype != 0 && out_dtype != 1) return DQ_ERR_INVALID;
  if (max_len > (int64_t)1 << 31) return DQ_ERR_INVALID;
  const uintptr_t kca = reinterpret_cast<uintptr_t>(k_cont), vca = reinterpret_cast<uintptr_t>(v_cont);
  if ((kca & 15u) || (vca & 15u) || ((num_slots * ck->t.C) & 15) || ((num_slots * cv->t.C) & 15))
    return DQ_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(q) & 15u) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return DQ_ERR_INVALID;
  dq::Plan pl;
  int st = dq::make_plan(B, Hq, Hkv, max_len, ck->t.C, cv->t.C, &pl);
  if (st) return st;
  size_t need = 0;
  st = dq_attn_decode_workspace(B, Hq, Hkv, max_len, &need);
  if (st) return st;
  if (ws_bytes < need || pl.total > need) return DQ_ERR_WORKSPACE;

  dq::AttnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = group;
  a.kc = k_cont;
  a.kn = k_norm;
  a.vc = v_cont;
  a.vn = v_norm;
  a.S = num_slots;
  a.seq_start = seq_start;
  a.pages = pages;
  a.max_pages = pages ? max_pages : 0;
  a.seq_len = seq_len;
  a.qk_scale = sm_scale * 1.4426950408889634f / 128.0f;
  a.chunk = pl.chunk;
  a.nc = pl.nc;
  a.cq = pl.cq;
  a.cr = pl.cr;
  a.n_items = pl.n_items;
  a.qrot = nullptr;  // the split-K items rotate their own queries
  a.part = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pl.qrot_bytes);
  a.out = out;
  a.out_bf16 = out_dtype;
  a.waves_per_block = pl.waves_per_block;
  if (app) {
    a.k_new = static_cast<const uint16_t *>(app->k_new);
    a.v_new = static_cast<const uint16_t *>(app->v_new);
    a.new_stride_b = app->stride_b;
    a.new_stride_h = app->stride_h;
    // the append entry points take the pools as writable
    a.kc_w = const_cast<uint8_t *>(k_cont);
    a.vc_w = const_cast<uint8_t *>(v_cont);
    a.kn_w = const_cast<uint16_t *>(k_norm);
    a.vn_w = const_cast<uint16_t *>(v_norm);
    a.k_stats = app->k_stats;
    a.v_stats = app->v_stats;
    a.part_new = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + pl.qrot_bytes + pl.part_bytes);
    // The encodes ride in the split-K launch when they fit in the slack of
    // its last round of resident waves (small batches: they are then free);
    // otherwise they would lengthen every wave that takes one, and a launch
    // of their own before the attention costs less.
    const int64_t W = (int64_t)pl.blocks_cap * pl.waves_per_block;
    const int64_t n_enc = 2 * (int64_t)B * Hkv;
    bool fuse = (pl.n_items + n_enc + W - 1) / W == (pl.n_items + W - 1) / W;
    const int64_t forced = dq::knob(DQ_KNOB_APPEND_FUSE);  // tests force either way
    if (forced >= 0) fuse = forced == 1;
    a.n_enc = fuse ? n_enc : 0;
    a.skip_last = 1;
  }
  // the work queue when the items take several rounds of resident waves
  {
    const int64_t W = (int64_t)pl.blocks_cap * pl.waves_per_block;
    bool queue = !pl.lat && pl.n_items + a.n_enc > W;
    const int64_t forced = dq::knob(DQ_KNOB_WORK_QUEUE);  // tests force either way
    if (forced >= 0) queue = forced == 1;
    if (queue)
      a.queue = reinterpret_cast<unsigned int *>(static_cast<uint8_t *>(workspace) + pl.qrot_bytes +
                                                 pl.part_bytes + pl.part_new_bytes);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.queue) hipLaunchKernelGGL(dq::queue_reset_kernel, dim3(1), dim3(64), 0, s, a.queue);
  if (app && a.n_enc == 0) {
    const int C = ck->t.C > cv->t.C ? ck->t.C : cv->t.C;
    const size_t lds = (size_t)dq::kAppendWaves * ((dq::append_scratch_bytes(C) + 15) & ~15);
    const int64_t blocks = (2 * (int64_t)B * Hkv + dq::kAppendWaves - 1) / dq::kAppendWaves;
    hipLaunchKernelGGL(dq::append_encode_kernel, dim3((unsigned)blocks), dim3(64 * dq::kAppendWaves), lds, s, a,
                       ck->t, cv->t);
  }
  if (split_begin && hipEventRecord(split_begin, s) != hipSuccess) return DQ_ERR_HIP;
  hipError_t e;
  if (pl.lat)  // latency mode (only for the 3-piece tile fetch)
    e = app && a.n_enc > 0 ? dq::launch_splitk<3, true, true>(pl, a, ck->t, cv->t, s)
                           : dq::launch_splitk<3, false, true>(pl, a, ck->t, cv->t, s);
  else if (pl.slot)  // three-piece tile fetch with the per-slot tables
    e = app && a.n_enc > 0            ? dq::launch_splitk<3, true, false, true>(pl, a, ck->t, cv->t, s)
        : dq::knob(DQ_KNOB_QK_VALU) == 1 ? dq::launch_splitk<3, false, false, true, true>(pl, a, ck->t, cv->t, s)
                                         : dq::launch_splitk<3, false, false, true>(pl, a, ck->t, cv->t, s);
  else if (app && a.n_enc > 0)  // the variant with the encode loop only when it has encodes to run
    e = pl.nq == 3   ? dq::launch_splitk<3, true>(pl, a, ck->t, cv->t, s)
        : pl.nq == 5 ? dq::launch_splitk<5, true>(pl, a, ck->t, cv->t, s)
                     : dq::launch_splitk<9, true>(pl, a, ck->t, cv->t, s);
  else
    e = pl.nq == 3   ? dq::launch_splitk<3, false>(pl, a, ck->t, cv->t, s)
        : pl.nq == 5 ? dq::launch_splitk<5, false>(pl, a, ck->t, cv->t, s)
                     : dq::launch_splitk<9, false>(pl, a, ck->t, cv->t, s);
  if (e != hipSuccess) return DQ_ERR_HIP;
  if (split_end && hipEventRecord(split_end, s) != hipSuccess) return DQ_ERR_HIP;
  hipLaunchKernelGGL(dq::combine_kernel, dim3((unsigned)(B * Hq)), dim3(128), 0, s, a, cv->t.seed);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}

extern "C" int dq_attn_decode(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B, int32_t Hq,
                              const uint8_t *k_cont, const uint16_t *k_norm, const uint8_t *v_cont,
                              const uint16_t *v_norm, int64_t num_slots, const int64_t *seq_start,
                              const int32_t *seq_len, int64_t max_len, float sm_scale, int32_t out_dtype,
                              void *out, void *workspace, size_t ws_bytes, dq_stream_t stream) {
  return attn_decode(ck, cv, q, B, Hq, k_cont, k_norm, v_cont, v_norm, num_slots, seq_start, nullptr, 0, seq_len,
                     max_len, sm_scale, out_dtype, out, workspace, ws_bytes, stream, nullptr, nullptr);
}

extern "C" int dq_attn_decode_paged(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B, int32_t Hq,
                                    const uint8_t *k_cont, const uint16_t *k_norm, const uint8_t *v_cont,
                                    const uint16_t *v_norm, int64_t num_slots, const int32_t *pages,
                                    int32_t max_pages, const int32_t *seq_len, int64_t max_len, float sm_scale,
                                    int32_t out_dtype, void *out, void *workspace, size_t ws_bytes,
                                    dq_stream_t stream) {
  if (!pages) return DQ_ERR_INVALID;
  return attn_decode(ck, cv, q, B, Hq, k_cont, k_norm, v_cont, v_norm, num_slots, nullptr, pages, max_pages,
                     seq_len, max_len, sm_scale, out_dtype, out, workspace, ws_bytes, stream, nullptr, nullptr);
}

extern "C" int dq_attn_decode_timed(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B, int32_t Hq,
                                    const uint8_t *k_cont, const uint16_t *k_norm, const uint8_t *v_cont,
                                    const uint16_t *v_norm, int64_t num_slots, const int64_t *seq_start,
                                    const int32_t *seq_len, int64_t max_len, float sm_scale, int32_t out_dtype,
                                    void *out, void *workspace, size_t ws_bytes, dq_stream_t stream,
                                    void *split_begin, void *split_end) {
  return attn_decode(ck, cv, q, B, Hq, k_cont, k_norm, v_cont, v_norm, num_slots, seq_start, nullptr, 0, seq_len,
                     max_len, sm_scale, out_dtype, out, workspace, ws_bytes, stream,
                     static_cast<hipEvent_t>(split_begin), static_cast<hipEvent_t>(split_end));
}

extern "C" int dq_attn_decode_append(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B, int32_t Hq,
                                     const void *k_new, const void *v_new, int64_t new_stride_b,
                                     int64_t new_stride_h, uint8_t *k_cont, uint16_t *k_norm, uint8_t *v_cont,
                                     uint16_t *v_norm, int64_t num_slots, const int64_t *seq_start,
                                     const int32_t *seq_len, int64_t max_len, float sm_scale, int32_t out_dtype,
                                     void *out, void *workspace, size_t ws_bytes, dq_stats *k_stats,
                                     dq_stats *v_stats, dq_stream_t stream) {
  const AppendArgs app{k_new, v_new, new_stride_b, new_stride_h, k_stats, v_stats};
  return attn_decode(ck, cv, q, B, Hq, k_cont, k_norm, v_cont, v_norm, num_slots, seq_start, nullptr, 0, seq_len,
                     max_len, sm_scale, out_dtype, out, workspace, ws_bytes, stream, nullptr, nullptr, &app);
}

extern "C" int dq_attn_decode_append_timed(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B, int32_t Hq,
                                           const void *k_new, const void *v_new, int64_t new_stride_b,
                                           int64_t new_stride_h, uint8_t *k_cont, uint16_t *k_norm,
                                           uint8_t *v_cont, uint16_t *v_norm, int64_t num_slots,
                                           const int64_t *seq_start, const int32_t *seq_len, int64_t max_len,
                                           float sm_scale, int32_t out_dtype, void *out, void *workspace,
                                           size_t ws_bytes, dq_stats *k_stats, dq_stats *v_stats,
                                           dq_stream_t stream, void *split_begin, void *split_end) {
  const AppendArgs app{k_new, v_new, new_stride_b, new_stride_h, k_stats, v_stats};
  return attn_decode(ck, cv, q, B, Hq, k_cont, k_norm, v_cont, v_norm, num_slots, seq_start, nullptr, 0, seq_len,
                     max_len, sm_scale, out_dtype, out, workspace, ws_bytes, stream,
                     static_cast<hipEvent_t>(split_begin), static_cast<hipEvent_t>(split_end), &app);
}

extern "C" int dq_attn_decode_paged_append(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B, int32_t Hq,
                                           const void *k_new, const void *v_new, int64_t new_stride_b,
                                           int64_t new_stride_h, uint8_t *k_cont, uint16_t *k_norm,
                                           uint8_t *v_cont, uint16_t *v_norm, int64_t num_slots,
                                           const int32_t *pages, int32_t max_pages, const int32_t *seq_len,
                                           int64_t max_len, float sm_scale, int32_t out_dtype, void *out,
                                           void *workspace, size_t ws_bytes, dq_stats *k_stats,
                                           dq_stats *v_stats, dq_stream_t stream) {
  if (!pages) return DQ_ERR_INVALID;
  const AppendArgs app{k_new, v_new, new_stride_b, new_stride_h, k_stats, v_stats};
  return attn_decode(ck, cv, q, B, Hq, k_cont, k_norm, v_cont, v_norm, num_slots, nullptr, pages, max_pages,
                     seq_len, max_len, sm_scale, out_dtype, out, workspace, ws_bytes, stream, nullptr, nullptr,
                     &app);
}

// ---------------------------------------------------------------- no-alloc decode
// dq_attn_decode_noalloc's workspace: a device array of fixed size, one copy
// per GPU, held until the process ends.  Host code never passes `scratch`
// itself (in host code the name is a stand-in, not a device address): the
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and only that address reaches the kernels.
static __device__ __align__(256) uint8_t scratch[DQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up on its first call).
int scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DQ_ERR_UNSUPPORTED;
  void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DQ_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DQ_OK;
}
}  // namespace

extern "C" int dq_attn_decode_noalloc(dq_codec_t ck, dq_codec_t cv, const void *q, int32_t B, int32_t Hq,
                                      const uint8_t *k_cont, const uint16_t *k_norm, const uint8_t *v_cont,
                                      const uint16_t *v_norm, int64_t num_slots, const int64_t *seq_start,
                                      const int32_t *seq_len, int64_t max_len, float sm_scale,
                                      int32_t out_dtype, void *out, dq_stream_t stream) {
  void *ws = nullptr;
  const int st = scratch_address(&ws);
  if (st) return st;
  // the same checks and kernels as dq_attn_decode; a call whose workspace
  // need exceeds the array returns DQ_ERR_WORKSPACE before any launch
  return attn_decode(ck, cv, q, B, Hq, k_cont, k_norm, v_cont, v_norm, num_slots, seq_start, nullptr, 0, seq_len,
                     max_len, sm_scale, out_dtype, out, ws, (size_t)DQ_NOALLOC_SCRATCH_BYTES, stream, nullptr,
                     nullptr);
}
