// Internal helpers shared by the grouped-GEMM kernels: the per-expert tile walk
// read from device offsets, buffer-resource access, and small math.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace gemm {

constexpr int kThreads = 256;  // 4 waves per workgroup

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Per-workgroup tile prefix over the local experts, derived from the device offsets.
struct TileMap {
  int mstart[kMaxExperts + 1];  // row-tile prefix per expert
  int rstart[kMaxExperts + 1];  // first row of each expert, relative to the local segment
};

// Rows are clamped to [0, n_max): with a caller-supplied topk_idx that repeats an
// id inside a token, local pairs could exceed n_max; those rows are dropped
// rather than written past the end of H and Y.
//
// Row tiles of an expert with R rows: BM-row tiles, and the remainder R % BM as
// one more, shorter tile -- unless MERGE_TAIL > 0, the remainder is at most
// MERGE_TAIL rows and there is a full tile to absorb it, in which case the
// last full tile grows to BM + remainder rows instead.
template <int BM, int MERGE_TAIL = 0>
__device__ __forceinline__ int row_tiles(int rows) {
  const int full = rows / BM, rem = rows % BM;
  if (MERGE_TAIL > 0 && full > 0 && rem <= MERGE_TAIL) return full;
  return full + (rem > 0);
}

template <int BM, int MERGE_TAIL = 0>
__device__ void build_tile_map(TileMap& tm, const int32_t* __restrict__ offsets, int e_begin,
                               int e_loc, int n_max) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int base = offsets[e_begin];
    int carry = 0;
    for (int e0 = 0; e0 < e_loc; e0 += kWave) {
      const int e = e0 + lane;
      int rows = 0, start = 0;
      if (e < e_loc) {
        start = min(offsets[e_begin + e] - base, n_max);
        rows = min(offsets[e_begin + e + 1] - base, n_max) - start;
      }
      const int mt = row_tiles<BM, MERGE_TAIL>(rows);
      int incl = mt;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (e < e_loc) {
        tm.mstart[e] = carry + incl - mt;
        tm.rstart[e] = start;
      }
      carry += __shfl(incl, kWave - 1);
    }
    if (lane == 0) {
      tm.mstart[e_loc] = carry;
      tm.rstart[e_loc] = min(offsets[e_begin + e_loc] - base, n_max);
    }
  }
  __syncthreads();
}

struct TileCoord {
  int e, mt, nt;
};

// Expert e with mstart[e]*n_tiles <= tile < mstart[e+1]*n_tiles (empty experts own no ids).
__device__ __forceinline__ TileCoord find_tile(const TileMap& tm, int tile, int n_tiles, int e_loc) {
  int lo = 0, hi = e_loc;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tm.mstart[mid] * n_tiles <= tile) lo = mid;
    else hi = mid;
  }
  // values read from LDS are not known to be wave-uniform: pin them to SGPRs
  lo = uniform(lo);
  const int ms = uniform(tm.mstart[lo]);
  const int mt_e = uniform(tm.mstart[lo + 1]) - ms;
  const int local = tile - ms * n_tiles;
  return {lo, local % mt_e, local / mt_e};
}

// Workgroup -> first tile id: each XCD (workgroups are dealt to the 8 XCDs
// round-robin) gets a contiguous range of ids.
__device__ __forceinline__ int xcd_remap(int b, int G) {
  return (G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b;
}


__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// SiLU for results that are rounded to bf16 next: hardware exp2 and reciprocal,
// a few ulp of fp32, far below bf16's half-ulp of 2^-9.
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Hides a value from loop-invariant code motion, so offsets derived from it are
// recomputed (one add each) instead of being hoisted into many live registers.
template <typename T>
__device__ __forceinline__ T opaque(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.

}  // namespace gemm
}  // namespace moe
