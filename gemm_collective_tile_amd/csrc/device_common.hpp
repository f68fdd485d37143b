// Device-side building blocks shared by the GEMM tile, the comm units and the
// scheduler: vector types, buffer-resource loads, fp16 packing, fast integer
// division and the agent-scope flag protocol.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iris {

typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxW = 16;
constexpr int kThreads = 256;  // every fused/comm workgroup is 4 wave64s

// ----------------------------------------------------------------- buffers
// gfx9 raw buffer resource: stride 0, num_records in bytes; a load whose
// offset is >= num_records returns 0 and a store there is dropped. That is
// how edge tiles are masked without branches.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOob = 0x80000000u;  // an offset past any num_records used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Agent-coherent 16-byte store (sc1 cache policy): the write goes through
// the XCD's L2, so once this wave's vmcnt reaches zero the data is visible
// to every XCD and no L2 write-back is needed before a flag that publishes
// it (agent-scope relaxed atomic stores use the same policy).
constexpr int kPolicySc1 = 16;
__device__ __forceinline__ void buf_store16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kPolicySc1);
}

// ----------------------------------------------------------- plain vectors
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }
// streaming forms for data touched once (non-temporal cache policy)
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4*)p); }

__device__ __forceinline__ f16x8 as_h8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ u32x4 as_u4(f16x8 v) { return __builtin_bit_cast(u32x4, v); }

// ------------------------------------------------------------ fast divide
// n / d for 32-bit unsigned n and a divisor fixed per unit of work
// (round-up multiply-high method: m = floor(2^32 (2^l - d) / d) + 1,
// l = ceil(log2 d); q = (hi(m n) + ((n - hi(m n)) >> 1)) >> (l - 1)).
struct FastDiv {
  uint32_t d, m, s;  // s = l - 1, or 0xffffffff for d == 1
  __host__ __device__ static FastDiv make(uint32_t d) {
    FastDiv f;
    f.d = d;
    if (d <= 1) {
      f.m = 0;
      f.s = 0xffffffffu;
      return f;
    }
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    f.m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
    f.s = l - 1;
    return f;
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    if (s == 0xffffffffu) return n;
    const uint32_t t = __umulhi(m, n);
    return (t + ((n - t) >> 1)) >> s;
  }
};

// ---------------------------------------------------- flags and counters
// Producer: all threads store data, the workgroup barriers, then one thread
// publishes with an agent-scope release. Consumer: one thread observes the
// flag, issues an agent-scope acquire fence, then the workgroup barriers
// before anyone reads the data.
__device__ __forceinline__ int ld_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ int fetch_add(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every vector memory operation this wave issued has completed
// (its stores have reached L2). A workgroup barrier alone does not do this on
// gfx9, so a producer drains its stores before the barrier that precedes the
// one-thread release of a flag.
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }

__device__ __forceinline__ uint64_t stamp_now() { return wall_clock64(); }

}  // namespace iris
