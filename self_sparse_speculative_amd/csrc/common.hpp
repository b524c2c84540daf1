// Shared device helpers for the S3R kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s3r {

constexpr int kWave = 64;
constexpr int kPage = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef uint16_t bf16_t;  // bfloat16 bit pattern

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Low and high bfloat16 of a packed 32-bit word.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float fmax_nan_free(float a, float b) { return a > b ? a : b; }

// Exponent base 2 that returns 0 for -inf inputs (v_exp_f32 already does).
__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes of one wave that hand data to each other through LDS (a transpose)
// need this between the writes and the reads: without it the compiler may,
// reasoning one lane at a time, reuse an earlier read of the same address in
// lanes that did not write in between. Wave-scope fences emit no wait of
// their own; LDS operations of one wave complete in order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Keeps the loads issued before it where they are in program order (no
// instruction of its own): software pipelining needs the next step's loads
// issued early, and the compiler otherwise sinks each load to its first use.
__device__ __forceinline__ void pin_issued_loads() { asm volatile("" ::: "memory"); }

// 16-byte global loads and stores carrying the nontemporal hint (the `nt`
// bit of the vector memory instructions): for streams a kernel touches once,
// so that they do not displace lines that are still to be reused from L2 and
// the Infinity Cache. They pay where every lane's 16 B chunk completes whole
// 128 B lines within one instruction (gathered 256 B rows, V rows read 8 rows
// x 128 B at a time, records written as runs); the verification's K
// fragments, whose lines are completed by two instructions, keep ordinary
// loads, which measured 9 % faster there.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t load_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ uint4 load_nt16_u4(const void* p) {
  const u32x4_t w = load_nt16(p);
  return make_uint4(w.x, w.y, w.z, w.w);
}

__device__ __forceinline__ void store_nt16(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// Ordered split of [0, n) into `parts` contiguous chunks of `chunk` elements.
__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace s3r
