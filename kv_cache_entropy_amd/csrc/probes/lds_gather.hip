// Throughput of random LDS gathers shaped like a rANS decode step, as a
// function of the dependent chains in flight (chains per lane x waves per
// CU).  Each step of a chain reads the table entry at its state's slot
// (x mod 4096) and updates the state from it, so every read depends on the
// one before, as in the decode attention kernels.  One block per CU (a pad
// fills the rest of the LDS); every index is masked into its table.
//
// Tables:
//   slot8  4096 x 8 B per-slot entries {f, cum | level << 16} (32 KB)
//   slot4  4096 x 4 B per-slot entries {f, slot - cum} (16 KB)
//   byte   4096 x 1 B symbol table (4 KB), then the symbol's 8-byte entry
//          from a 16-entry table: two dependent reads per step
//
// Prints, per table and shape, chain-steps per CU-cycle at 2.4 GHz and a
// checksum of the final states.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef const volatile __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef const volatile __attribute__((address_space(3))) uint32_t lds_u32;
typedef const volatile __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kSteps = 2048;  // per chain
constexpr int kPadWords = 24 * 1024;

enum { kSlot8 = 0, kSlot4 = 1, kByte = 2 };

template <int TAB, int C, int T>
__global__ void __launch_bounds__(T) gather(uint32_t *out) {
  __shared__ uint2 e8[4096];
  __shared__ uint32_t e4[4096];
  __shared__ uint8_t s8[4096];
  __shared__ uint2 sym[16];
  __shared__ uint32_t pad[kPadWords];  // one block per CU
  for (int i = threadIdx.x; i < kPadWords; i += T) pad[i] = (uint32_t)i;
  for (int i = threadIdx.x; i < 4096; i += T) {
    const uint32_t s = ((uint32_t)i * 7u) >> 12;  // 7 symbols, contiguous slot ranges
    const uint32_t cum = (4096u * s + 6u) / 7u, nxt = (4096u * (s + 1u) + 6u) / 7u;
    e8[i] = make_uint2(nxt - cum, cum | ((0x3C00u + s) << 16));
    e4[i] = (nxt - cum) | (((uint32_t)i - cum) << 16);
    s8[i] = (uint8_t)(8u * s);
  }
  if (threadIdx.x < 16) {
    const uint32_t s = threadIdx.x < 7 ? threadIdx.x : 6u;
    const uint32_t cum = (4096u * s + 6u) / 7u, nxt = (4096u * (s + 1u) + 6u) / 7u;
    sym[threadIdx.x] = make_uint2(nxt - cum, cum | ((0x3C00u + s) << 16));
  }
  __syncthreads();
  uint32_t x[C];
#pragma unroll
  for (int c = 0; c < C; ++c) x[c] = ((0x12345u + 977u * c) * (threadIdx.x + 1u) + blockIdx.x * 31u) | (1u << 23);
  uint32_t acc = 0;
  for (int k = 0; k < kSteps / 8; ++k) {
#pragma unroll 4
    for (int j = 0; j < 8; ++j) {
      uint32_t f[C], d[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t u = x[c] & 4095u;
        if (TAB == kSlot8) {
          const u32x2 a = *(lds_u32x2 *)((const uint8_t *)e8 + (u << 3));
          f[c] = a.x;
          d[c] = u - (a.y & 0xFFFFu);
          acc += a.y >> 16;
        } else if (TAB == kSlot4) {
          const uint32_t a = *(lds_u32 *)((const uint8_t *)e4 + (u << 2));
          f[c] = a & 0xFFFFu;
          d[c] = a >> 16;
        } else {
          const uint32_t s = *(lds_u8 *)(s8 + u);
          const u32x2 a = *(lds_u32x2 *)((const uint8_t *)sym + s);
          f[c] = a.x;
          d[c] = u - (a.y & 0xFFFFu);
          acc += a.y >> 16;
        }
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t y = __umul24(f[c], x[c] >> 12) + d[c];
        x[c] = y < (1u << 23) ? (y << 8) | ((uint32_t)(k + j + c) & 255u) : y;
      }
    }
  }
  uint32_t r = acc ^ pad[(threadIdx.x * 7u) % kPadWords];
#pragma unroll
  for (int c = 0; c < C; ++c) r ^= x[c];
  out[blockIdx.x * 1024 + threadIdx.x] = r;
}

template <int TAB, int C, int T>
int run(const char *name, uint32_t *d, int blocks) {
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 1;
  for (int w = 0; w < 2; ++w) hipLaunchKernelGGL((gather<TAB, C, T>), dim3(blocks), dim3(T), 0, 0, d);
  if (hipEventRecord(a, 0) != hipSuccess) return 1;
  const int reps = 5;
  for (int r = 0; r < reps; ++r) hipLaunchKernelGGL((gather<TAB, C, T>), dim3(blocks), dim3(T), 0, 0, d);
  if (hipEventRecord(b, 0) != hipSuccess || hipEventSynchronize(b) != hipSuccess) return 1;
  float ms = 0.0f;
  if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return 1;
  uint32_t h[4];
  if (hipMemcpy(h, d, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return 1;
  const double steps = (double)blocks * T * C * kSteps;  // chain-steps per launch
  printf("| %s | %d | %2d | %.3f | %.2f | %08x |\n", name, C, T / 64, ms / reps,
         steps / (ms / reps * 1e-3) / blocks / 2.4e9, h[0] ^ h[1]);
  hipEventDestroy(a);
  hipEventDestroy(b);
  return 0;
}

}  // namespace

int main() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
    fprintf(stderr, "no GPU\n");
    return 1;
  }
  uint32_t *d = nullptr;
  if (hipMalloc(&d, (size_t)cus * 1024 * sizeof(uint32_t)) != hipSuccess) return 1;
  printf("%d CUs, one block per CU, %d dependent steps per chain\n\n", cus, kSteps);
  printf("| table | chains per lane | waves per CU | ms per launch | chain-steps per CU-cycle | checksum |\n");
  printf("|---|---:|---:|---:|---:|---|\n");
  int e = 0;
  e |= run<kSlot8, 1, 768>("slot8", d, cus);
  e |= run<kSlot8, 2, 256>("slot8", d, cus);
  e |= run<kSlot8, 2, 512>("slot8", d, cus);
  e |= run<kSlot8, 2, 768>("slot8", d, cus);
  e |= run<kSlot8, 2, 1024>("slot8", d, cus);
  e |= run<kSlot8, 4, 768>("slot8", d, cus);
  e |= run<kSlot8, 4, 1024>("slot8", d, cus);
  e |= run<kSlot8, 8, 768>("slot8", d, cus);
  e |= run<kSlot4, 2, 768>("slot4", d, cus);
  e |= run<kSlot4, 4, 1024>("slot4", d, cus);
  e |= run<kByte, 2, 768>("byte", d, cus);
  e |= run<kByte, 4, 1024>("byte", d, cus);
  hipFree(d);
  return e;
}
