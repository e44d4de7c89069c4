// Internal helpers and launcher declarations shared by the HIP sources.
// Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Wave-uniform value as an SGPR (the caller guarantees uniformity).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

// Raw buffer resource over `bytes` bytes at `base`: loads past the end return
// zero and stores past the end are dropped, with no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Cache-policy field of a load: non-temporal. The caches treat the bytes as
// streamed (read once) rather than keeping them for reuse.
constexpr int kCpolNT = 2;

// 16 bytes at voffset, with cache policy CPOL (0 or kCpolNT).
template <int CPOL = 0>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset) {
  const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, static_cast<int>(voffset), 0, CPOL);
  return make_uint4(static_cast<uint32_t>(v.x), static_cast<uint32_t>(v.y), static_cast<uint32_t>(v.z),
                    static_cast<uint32_t>(v.w));
}

__device__ __forceinline__ void buffer_store16(uint4 v, __amdgpu_buffer_rsrc_t rsrc, uint32_t voffset) {
  const i32x4_t d = {static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(d, rsrc, static_cast<int>(voffset), 0, 0);
}

// Launchers (host side). Each returns hipSuccess or the launch error.
hipError_t launch_route_topk(const float* logits, int32_t* idx, float* w, int64_t T, int E, int k,
                             hipStream_t stream);

size_t dispatch_workspace_bytes(int64_t T, int k, int E);
// byte offset of the debug error word in the dispatch workspace; SIZE_MAX in release builds
size_t dispatch_debug_word_offset();
// the allocation-free dispatch's per-GPU workspace: its size, and its device address on the current device
constexpr size_t kDispatchScratchBytes = MOE_DISPATCH_SCRATCH_BYTES;
hipError_t dispatch_scratch(void** ptr);
hipError_t launch_dispatch(const void* x, size_t row_bytes, const int32_t* idx, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* pair_pos, void* x_perm,
                           void* workspace, int64_t T, int k, int E, int e_begin, int e_end,
                           int64_t n_max, hipStream_t stream);

hipError_t launch_grouped_gemm_bf16(const void* x_perm, const int32_t* offsets, const void* w_gu,
                                    const void* w_dn, void* h, void* y, int d, int d_ff, int e_begin,
                                    int e_loc, int64_t n_max, int64_t T, int k, int E,
                                    hipStream_t stream);
// a = x_perm (perm == nullptr) or x, whose rows the gate/up loads gather through perm (or, with a_blk,
// a copy of them gathered into a_blk in 32-column blocks of n_max rows first; a_blk then has
// blocked_rows_workspace_bytes(n_max, d) bytes);
// gu != nullptr (with perm only): the gate/up pre-activations [G | U] are written there too
hipError_t launch_grouped_gemm_lds(const void* a, const int32_t* perm, int64_t T, int k, const int32_t* offsets,
                                   const void* w_gu, const void* w_dn, void* h, void* y, void* gu, int d, int d_ff,
                                   int e_begin, int e_loc, int64_t n_max, int grid_gate_up, int grid_down,
                                   void* a_blk, hipStream_t stream);
// Whether the gathered gate/up rows are copied in 32-column blocks first; the workspace then holds
// the copy (blocked_rows_bytes) and, after it, one tile count per XCD for the gate/up launch's pacing
bool grouped_gemm_blocked_rows(int64_t n_max, int e_loc, int d, int d_ff);
size_t blocked_rows_bytes(int64_t n_max, int d);
size_t blocked_rows_workspace_bytes(int64_t n_max, int d);
// Gate/up rows gathered from x through perm, no x_perm (bf16, d and d_ff multiples of 32);
// gu != nullptr: [G | U] of every local row is kept there as well; a_blk: see launch_grouped_gemm_lds.
hipError_t launch_grouped_gemm_gather(const void* x, const int32_t* perm, const int32_t* offsets,
                                      const void* w_gu, const void* w_dn, void* h, void* y, void* gu, int d,
                                      int d_ff, int e_begin, int e_loc, int64_t n_max, int64_t T, int k,
                                      void* a_blk, hipStream_t stream);
hipError_t launch_grouped_gemm_f32(const float* x_perm, const int32_t* offsets, const float* w_gu,
                                   const float* w_dn, float* h, float* y, int d, int d_ff,
                                   int e_begin, int e_loc, int64_t n_max, hipStream_t stream);

// w == nullptr: unit weights (the gradient of the row gather)
hipError_t launch_combine(const void* y, const int32_t* pair_pos, const float* w, void* out,
                          int64_t T, int k, int d, int64_t n_max, bool bf16, hipStream_t stream);

// x_perm rows [0, N_loc) = x[perm[offsets[e_begin] + r] / k]
hipError_t launch_gather_rows(const void* x, size_t row_bytes, const int32_t* perm, const int32_t* offsets,
                              void* x_perm, int k, int e_begin, int e_end, int64_t n_max, hipStream_t stream);

// C[rows, N] = A[rows, K] @ B_e[K, N] (N-contiguous weights, row stride ldb) per local expert
hipError_t launch_grouped_gemm_plain(const void* a, const void* b, void* c, const int32_t* offsets, int e_begin,
                                     int e_loc, int K, int N, int ldb, int64_t n_max, int grid, hipStream_t stream);
// C[rows, N] = A[rows, K] @ B_e[N, K]^T (K-contiguous weights), A in 32-column blocks of n_max rows. With
// swiglu_bwd, A = dY, B = W_dn and C receives [dG | dU], blocked the same way, from the [G | U] rows in gu (row
// stride ldc = 2 N); without, A is that [dG | dU] (K = 2 d_ff) and C is row-major (row stride ldc)
hipError_t launch_grouped_gemm_nt(const void* a, const void* b, void* c, const void* gu, const int32_t* offsets,
                                  int e_begin, int e_loc, int K, int N, int ldc, int64_t n_max, bool swiglu_bwd,
                                  int grid, hipStream_t stream);
// rows [0, N_loc) of the row-major [n_max][cols] src into dst in 32-column blocks of n_max rows
hipError_t launch_to_blocked(const void* src, void* dst, const int32_t* offsets, int e_begin, int e_end, int cols,
                             int64_t n_max, hipStream_t stream);
// dW_e[M, N] = A_e^T @ B_e over each local expert's rows (A [rows][M], B [rows][N];
// b_blocked: B in the 32-column blocked layout of the backward's [dG | dU], n_max rows)
hipError_t launch_grouped_gemm_tn(const void* src_a, const void* src_b, void* dw, const int32_t* offsets,
                                  int e_begin, int e_loc, int M, int N, int64_t n_max, bool b_blocked, int grid,
                                  hipStream_t stream);
// persistent-grid size for a row-tiled grouped GEMM with n_tiles column tiles
int grouped_gemm_grid(int64_t n_max, int e_loc, int n_tiles);
int device_cu_count();

hipError_t launch_combine_backward(const void* d_out, const void* y, const int32_t* pair_pos, const float* w,
                                   void* d_y, float* d_w, int64_t T, int k, int d, int64_t n_max, bool bf16,
                                   hipStream_t stream);
hipError_t launch_route_topk_backward(const int32_t* idx, const float* w, const float* d_w, float* d_logits,
                                      int64_t T, int E, int k, hipStream_t stream);

}  // namespace moe
