// Building blocks of the LDS-pipelined MFMA kernels (gfx950): LDS-DMA loads,
// LDS fragment reads issued by inline asm (so the compiler does not wait for
// every outstanding DMA load before them), compile-time s_waitcnt counts, and
// compile-time loops for pinning an instruction order.
#pragma once

#include <type_traits>

#include "gemm_common.h"

namespace moe {
namespace gemm {

#define LDS3 __attribute__((address_space(3)))

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const LDS3 char*)p));
}

// s_waitcnt vmcnt(N) with a compile-time N (0..63).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  if constexpr (N == 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  else if constexpr (N == 5) asm volatile("s_waitcnt lgkmcnt(5)" ::: "memory");
  else if constexpr (N == 9) asm volatile("s_waitcnt lgkmcnt(9)" ::: "memory");
  else if constexpr (N == 10) asm volatile("s_waitcnt lgkmcnt(10)" ::: "memory");
  else if constexpr (N == 12) asm volatile("s_waitcnt lgkmcnt(12)" ::: "memory");
  else if constexpr (N == 13) asm volatile("s_waitcnt lgkmcnt(13)" ::: "memory");
  else static_assert(N == 0, "add the count");
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <typename T>
__device__ __forceinline__ void tie(T& v) {
  asm volatile("" : "+v"(v));
}

template <int IMM>
__device__ __forceinline__ bf16x8_t ds_read16(uint32_t addr) {
  bf16x8_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(IMM));
  return v;
}

template <int IMM>
__device__ __forceinline__ i16x4_t ds_read_tr(uint32_t addr) {
  i16x4_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(IMM));
  return v;
}

// 16 bytes per lane from the buffer into LDS at lds_base + 16 * lane (lds_base is
// a wave-uniform LDS byte address), with cache policy CPOL (0 or kCpolNT).
template <int CPOL = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS3 void*)(uintptr_t)lds_base, 16, voff, 0, 0, CPOL);
}

// c += a * b with c held in VGPRs
__device__ __forceinline__ void mfma_in_vgprs(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

__device__ __forceinline__ bf16x8_t join(i16x4_t lo, i16x4_t hi) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace gemm
}  // namespace moe
