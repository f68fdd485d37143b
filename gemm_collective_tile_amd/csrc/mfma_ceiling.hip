// The dense fp16 MFMA rate this chip sustains with no memory traffic. Every
// wave issues v_mfma_f32_32x32x16_f16 over eight independent accumulators
// (128 registers per lane), round robin, its operands in registers.
//
// With random operands, eight operand sets of random fp16 values (random
// signs and mantissas, magnitudes in [0.5, 2)) rotate from one instruction to
// the next, so the multipliers switch as they do on GEMM data; otherwise the
// operands are the same constants throughout. On a chip whose package power
// limit binds under MFMA load, the first rate is the ceiling a GEMM on random
// data can approach and the second the rate of the MFMA pipes when power does
// not bind; the two differ by the clock the chip holds.
#include "mfma_ceiling.hpp"

#include <vector>

namespace iris {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// random sign, exponent 14 or 15 (binary16 bias 15), random 10-bit mantissa
__device__ __forceinline__ _Float16 random_half(uint32_t x) {
  const uint32_t h = mix32(x);
  const uint16_t bits = (uint16_t)(((h & 1u) << 15) | ((14u + ((h >> 1) & 1u)) << 10) | ((h >> 2) & 0x3ffu));
  return __builtin_bit_cast(_Float16, bits);
}

template <bool RANDOM>
__global__ __launch_bounds__(256) void mfma_ceiling_kernel(float* out, int iters, unsigned long long* stamps) {
  const uint32_t l = threadIdx.x;
  h8 a[8], b[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[s][e] = RANDOM ? random_half(l * 131u + s * 17u + e) : (_Float16)(((l + e) & 7) * 0.001f);
      b[s][e] = RANDOM ? random_half(l * 977u + s * 29u + e + 7777u) : (_Float16)(((l * 3 + e) & 7) * 0.001f);
    }
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
    // operand sets named at compile time (a runtime index would put them in
    // scratch memory)
#pragma unroll
    for (int k = 0; k < 8; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[RANDOM ? k : 0], b[RANDOM ? (k + 3) & 7 : 0], acc[k], 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[k][r];
  if (l == 0) {
    stamps[blockIdx.x * 2] = __builtin_amdgcn_s_memtime() - t0;
    stamps[blockIdx.x * 2 + 1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  out[blockIdx.x * 256 + l] = sum;  // keeps the accumulation live
}

template <bool RANDOM>
hipError_t launch(int grid, int iters, hipStream_t s, float* out, unsigned long long* stamps) {
  hipLaunchKernelGGL((mfma_ceiling_kernel<RANDOM>), dim3(grid), dim3(256), 0, s, out, iters, stamps);
  return hipGetLastError();
}

}  // namespace

hipError_t mfma_ceiling_run(bool random_operands, int iters, int grid, hipStream_t s, float* ms, double* cycles,
                            double* ticks) {
  float* out = nullptr;
  unsigned long long* stamps = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipMalloc(&out, (size_t)grid * 256 * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&stamps, (size_t)grid * 2 * sizeof(unsigned long long));
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  auto run = [&](int n) { return random_operands ? launch<true>(grid, n, s, out, stamps) : launch<false>(grid, n, s, out, stamps); };
  if (e == hipSuccess) e = run(64);  // warm-up
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) e = run(iters);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
  std::vector<unsigned long long> st((size_t)grid * 2);
  if (e == hipSuccess) e = hipMemcpy(st.data(), stamps, st.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    *cycles = 0.0;
    *ticks = 0.0;
    for (int i = 0; i < grid; ++i) {
      *cycles += (double)st[(size_t)i * 2];
      *ticks += (double)st[(size_t)i * 2 + 1];
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (stamps) (void)hipFree(stamps);
  if (out) (void)hipFree(out);
  return e;
}

}  // namespace iris
