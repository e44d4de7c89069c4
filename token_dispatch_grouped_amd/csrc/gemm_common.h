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

// Tile map with the experts ordered by the height of their tiles, largest first:
// class 0 = more than 128 rows (tiles of 256 or 288 rows), then (64, 128],
// (32, 64], (0, 32], empty last; stable by expert id inside a class. Walked in
// snake order (see snake_tile), the costly tiles start in the first round and
// the second round's cheap tiles go to the workgroups whose first tiles were
// cheap. When every expert is in one class the order is the plain expert order.
struct SortedTileMap {
  int mstart[kMaxExperts + 1];  // row-tile prefix over positions
  int eid[kMaxExperts];         // local expert at each position
  int rstart[kMaxExperts + 1];  // first row of each expert (by expert id), relative to the local segment
  int classes;                  // height classes that hold at least one expert with rows
  int tall;                     // positions [0, tall) hold the class-0 experts
};

__device__ __forceinline__ int height_class(int rows) {
  return rows > 128 ? 0 : rows > 64 ? 1 : rows > 32 ? 2 : rows > 0 ? 3 : 4;
}

template <int BM, int MERGE_TAIL>
__device__ void build_sorted_tile_map(SortedTileMap& tm, const int32_t* __restrict__ offsets, int e_begin,
                                      int e_loc, int n_max) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int base = offsets[e_begin];
    auto rows_of = [&](int e) {
      const int start = min(offsets[e_begin + e] - base, n_max);
      return min(offsets[e_begin + e + 1] - base, n_max) - start;
    };
    // pass 1: experts per class, and the row starts
    int cnt[5] = {0, 0, 0, 0, 0};
    for (int e0 = 0; e0 < e_loc; e0 += kWave) {
      const int e = e0 + lane;
      const int c = e < e_loc ? height_class(rows_of(e)) : 5;
      if (e < e_loc) tm.rstart[e] = min(offsets[e_begin + e] - base, n_max);
#pragma unroll
      for (int q = 0; q < 5; ++q) cnt[q] += __popcll(__ballot(c == q));
    }
    if (lane == 0) {
      tm.rstart[e_loc] = min(offsets[e_begin + e_loc] - base, n_max);
      tm.classes = (cnt[0] > 0) + (cnt[1] > 0) + (cnt[2] > 0) + (cnt[3] > 0);
      tm.tall = cnt[0];
    }
    int cbase[5];
    cbase[0] = 0;
#pragma unroll
    for (int q = 1; q < 5; ++q) cbase[q] = cbase[q - 1] + cnt[q - 1];
    // pass 2: position = class base + rank inside the class; row tiles parked in mstart
    const uint64_t below = (uint64_t{1} << lane) - 1;
    for (int e0 = 0; e0 < e_loc; e0 += kWave) {
      const int e = e0 + lane;
      const int rows = e < e_loc ? rows_of(e) : 0;
      const int c = e < e_loc ? height_class(rows) : 5;
      int pos = 0;
#pragma unroll
      for (int q = 0; q < 5; ++q) {
        const uint64_t m = __ballot(c == q);
        if (c == q) pos = cbase[q] + __popcll(m & below);
        cbase[q] += __popcll(m);
      }
      if (e < e_loc) {
        tm.eid[pos] = e;
        tm.mstart[pos] = row_tiles<BM, MERGE_TAIL>(rows);
      }
    }
    // pass 3: exclusive prefix of the row tiles over positions (a position may
    // have been written by another lane: the fences keep the reads after the writes)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    int carry = 0;
    for (int p0 = 0; p0 < e_loc; p0 += kWave) {
      const int p = p0 + lane;
      const int mt = p < e_loc ? tm.mstart[p] : 0;
      int incl = mt;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (p < e_loc) tm.mstart[p] = carry + incl - mt;
      carry += __shfl(incl, kWave - 1);
    }
    if (lane == 0) tm.mstart[e_loc] = carry;
  }
  __syncthreads();
}

struct SortedTile {
  int e, mt, nt, mt_e;
};

// Row tiles of an expert are walked in groups of kRowGroup: inside a group the
// row tile is fastest, then the column block; the last group holds the rest.
constexpr int kRowGroup = 4;

// Position p with mstart[p]*n_tiles <= tile < mstart[p+1]*n_tiles; empty experts
// own no ids. Inside an expert, groups of kRowGroup row tiles, row tile fastest
// inside a group: 32 consecutive ids (a round of one XCD's workgroups) cover 4
// row tiles x 8 column blocks of a tall expert, so each weight panel crosses to
// that XCD's L2 once per 4 row tiles and each row tile's activations once per 8
// column blocks. An expert of at most kRowGroup row tiles is walked as by
// find_tile.
__device__ __forceinline__ SortedTile find_sorted_tile(const SortedTileMap& tm, int tile, int n_tiles, int e_loc) {
  int lo = 0, hi = e_loc;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tm.mstart[mid] * n_tiles <= tile) lo = mid;
    else hi = mid;
  }
  lo = uniform(lo);
  const int ms = uniform(tm.mstart[lo]);
  const int mt_e = uniform(tm.mstart[lo + 1]) - ms;
  const int local = tile - ms * n_tiles;
  const int full = mt_e / kRowGroup * kRowGroup;  // row tiles in whole groups
  int mt, nt;
  if (local < full * n_tiles) {
    const int g = local / (kRowGroup * n_tiles), off = local - g * kRowGroup * n_tiles;
    mt = g * kRowGroup + off % kRowGroup;
    nt = off / kRowGroup;
  } else {
    const int rest = mt_e - full, off = local - full * n_tiles;
    mt = full + off % rest;
    nt = off / rest;
  }
  return {uniform(tm.eid[lo]), uniform(mt), uniform(nt), mt_e};
}

// Tile of round i for a workgroup whose XCD-remapped index is r: rounds go
// forward and backward in turn over the tile ids.
__device__ __forceinline__ int snake_tile(int i, int r, int G) {
  return (i & 1) ? (i + 1) * G - 1 - r : i * G + r;
}


// Byte offset of element (row, col) of a [rows][cols] bf16 matrix stored in
// 32-column blocks of n_rows rows: block col / 32 holds [n_rows][32]. A K = 32
// stage of a tile's rows is then one contiguous run, where row-major rows give
// one 64-byte piece per row.
__device__ __forceinline__ uint32_t blk_off(int row, int col, int n_rows) {
  return static_cast<uint32_t>((col >> 5) * n_rows + row) * 64u + static_cast<uint32_t>(col & 31) * 2u;
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
