// dq_decode_symbols: containers -> the 128 symbols each (inspection and
// checking path; attention decodes inside its own kernel).  One lane per
// container; the decode table lives in LDS.  Bytes past the container read
// as zero and are never fetched, so arbitrary (even corrupted) containers
// decode without touching memory outside their C bytes.
#include "decode_common.h"

namespace dq {
namespace {

constexpr int kThreads = 256;

struct DecodeArgs {
  const uint8_t *cont;
  int64_t num_slots;
  int32_t head;
  const int64_t *slots;
  int64_t n;
  uint8_t *sym;
  uint32_t *final_state;
  int32_t *consumed;
};

__global__ void __launch_bounds__(kThreads) decode_symbols_kernel(DecodeArgs a, Tables t) {
  __shared__ uint8_t sym8[kM];
  __shared__ uint2 symtab[kMaxLevels];
  build_tables(sym8, symtab, t, threadIdx.x, kThreads);
  __syncthreads();
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= a.n) return;
  const int C = t.C;
  uint8_t *out = a.sym + j * kD;
  const int64_t slot = a.slots[j];
  if (slot < 0 || slot >= a.num_slots) {  // out of range: zeros, state 0
    for (int i = 0; i < kD; i += 4) *reinterpret_cast<uint32_t *>(out + i) = 0u;
    if (a.final_state) a.final_state[j] = 0u;
    if (a.consumed) a.consumed[j] = 0;
    return;
  }
  const uint8_t *c = a.cont + ((int64_t)a.head * a.num_slots + slot) * C;
  uint32_t x = (uint32_t)c[0] | ((uint32_t)c[1] << 8) | ((uint32_t)c[2] << 16) | ((uint32_t)c[3] << 24);
  int p = 4;
  for (int i = 0; i < kD; i += 4) {
    uint32_t packed = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t sy;
      rans_step(x, sym8, symtab, sy);
      packed |= sy << (8 * q);
      if (x < kLow) {
        const uint32_t b = p < C ? (uint32_t)c[p] : 0u;
        x = (x << 8) | b;
        ++p;
      }
    }
    *reinterpret_cast<uint32_t *>(out + i) = packed;
  }
  if (a.final_state) a.final_state[j] = x;
  if (a.consumed) a.consumed[j] = p;
}

}  // namespace
}  // namespace dq

extern "C" int dq_decode_symbols(dq_codec_t codec, const uint8_t *cont, int64_t num_slots,
                                 int32_t head, const int64_t *slots, int64_t n, uint8_t *sym_out,
                                 uint32_t *final_state, int32_t *consumed, dq_stream_t stream) {
  if (!codec || n < 0) return DQ_ERR_INVALID;
  if (n == 0) return DQ_OK;
  if (!cont || !slots || !sym_out || num_slots < 1) return DQ_ERR_INVALID;
  if (head < 0 || head >= codec->t.hkv) return DQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(sym_out) & 3u) return DQ_ERR_INVALID;
  dq::DecodeArgs a{cont, num_slots, head, slots, n, sym_out, final_state, consumed};
  const unsigned blocks = (unsigned)((n + dq::kThreads - 1) / dq::kThreads);
  hipLaunchKernelGGL(dq::decode_symbols_kernel, dim3(blocks), dim3(dq::kThreads), 0,
                     static_cast<hipStream_t>(stream), a, codec->t);
  return hipGetLastError() == hipSuccess ? DQ_OK : DQ_ERR_HIP;
}
