// Grouped expert FFN over one rank's local experts: gate/up GEMM with a fused
// SwiGLU epilogue, then the down GEMM.
//
// What is computed: experts_forward of "Paralelismo de especialistas"
// (transformers v5.23.0, pt), section "Adicionando uma implementação", on
// weights sharded along the expert dimension (GroupedGemmParallel), with the
// packed gate_up_proj [hidden, 2*expert_dim] of "Paralelismo de tensor para
// inferência", section "Estratégias empacotadas" (gate = first half of the
// columns, up = second half) and SwiGLU = silu(gate) * up. The down projection
// is [d_ff, d] per expert.
//
// Design (bf16, gfx950):
//   * v_mfma_f32_32x32x16_bf16, fp32 accumulation. A workgroup of 4 waves owns a
//     256 x 256 tile of the product (2 x 2 waves of 128 x 128 = 4 x 4 MFMA
//     blocks each) and walks K in steps of 64 through two LDS buffers
//     (2 x 64 KB), one barrier per step; global loads for step s+1 are in
//     flight while step s runs on the matrix cores.
//   * Both operands live in LDS K-contiguous, [row][64] bf16, with the 16-byte
//     chunk index XOR-swizzled by (r ^ r>>3) & 7 so the MFMA fragment reads
//     (16 rows x 16 bytes) hit distinct banks.
//   * The weights keep the pages' layout [K, N] (N contiguous). Each thread
//     loads an 8 x 8 block (8 rows of 16 bytes, coalesced along N), transposes
//     it in registers and stores 8 K-contiguous 16-byte rows, so no weight
//     repacking is needed.
//   * Gate/up: a tile takes 128 gate columns and the matching 128 up columns;
//     each wave holds gate and up accumulators for the same outputs, so SwiGLU
//     runs on registers and only H (bf16) is written.
//   * Tiles: per local expert, ceil(rows / 256) row tiles x column tiles. Every
//     workgroup derives the per-expert tile prefix from the device offsets
//     (no host sync), then walks tile ids persistently. Ids run row-tile
//     fastest, so neighbouring ids share one weight panel, and the workgroup ->
//     id map gives each XCD a contiguous id range, so a panel is fetched into
//     one XCD's L2 and reused there. Empty experts own no tiles: their weights
//     are never read.
//   * Operands are read with raw buffer loads (one SGPR resource per tile and a
//     single VGPR offset per operand): rows past the expert's end and K rows past
//     the end of an expert's weights read as zero, so the only predicate-free
//     hazard, a K tail that is not a multiple of 64, multiplies finite row
//     data by zero weight rows. Results leave through buffer stores whose
//     resource ends at the tile's last valid row.
//
// fp32 (small parity workload): a plain VALU tiled kernel with the same tile walk.

#include <atomic>

#include "gemm_common.h"

namespace moe {
namespace {

using namespace gemm;

constexpr int kBM = 256;       // rows per tile
constexpr int kBN = 256;       // weight columns per tile (128 gate + 128 up for SwiGLU)
constexpr int kBK = 64;        // K per pipeline step
constexpr int kTileElems = 256 * kBK;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// LDS element offset of the 16-byte chunk c (0..7) of row r of a [256][64] tile.
__device__ __forceinline__ int lds_off(int r, int c) { return r * kBK + ((c ^ swz(r)) << 3); }

template <bool SWIGLU>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A,        // [rows, K] local rows (x_perm or H)
    const uint16_t* __restrict__ B,        // [e_loc][K][ldb]
    uint16_t* __restrict__ C,              // [rows, N]
    const int32_t* __restrict__ offsets,   // [E+1] global
    int e_begin, int e_loc, int K, int N, int ldb, int n_max) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][kTileElems];  // [buf][A|B]
  __shared__ TileMap tm;
  build_tile_map<kBM>(tm, offsets, e_begin, e_loc, n_max);

  constexpr int kOutCols = SWIGLU ? kBN / 2 : kBN;  // output columns per tile
  const int n_tiles = (N + kOutCols - 1) / kOutCols;
  const int total = uniform(tm.mstart[e_loc]) * n_tiles;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t b_expert_bytes = static_cast<uint32_t>(K) * ldb * 2u;
  const int ksteps = (K + kBK - 1) / kBK;

  // A loads: 16-byte chunk a_c of rows a_r + 32*i; B loads: 8 columns b_cb*8.., 8 K-rows b_kb*8..
  const int a_c = tid & 7, a_r = tid >> 3;
  const int b_cb = tid & 31, b_kb = tid >> 5;
  const uint32_t a_row_bytes = static_cast<uint32_t>(K) * 2u;
  const uint32_t b_row_bytes = static_cast<uint32_t>(ldb) * 2u;

  // MFMA fragment LDS offsets (elements) for k-chunk 0; chunk ch adds (ch ^ swz) * 8
  auto bcol = [&](int ni) {
    return SWIGLU ? ((ni < 2) ? wn * 64 + ni * 32 : 128 + wn * 64 + (ni - 2) * 32) : wn * 128 + ni * 32;
  };

  for (int tile = xcd_remap(blockIdx.x, gridDim.x); tile < total; tile += gridDim.x) {
    const TileCoord tc = find_tile(tm, tile, n_tiles, e_loc);
    const int row0 = uniform(tm.rstart[tc.e]) + tc.mt * kBM;
    const int rows_valid = min(kBM, uniform(tm.rstart[tc.e + 1]) - row0);
    const int n0 = tc.nt * kOutCols;

    const __amdgpu_buffer_rsrc_t ra_src =
        make_rsrc(A + static_cast<int64_t>(row0) * K, static_cast<uint32_t>(rows_valid) * a_row_bytes);
    const __amdgpu_buffer_rsrc_t rb_src =
        make_rsrc(B + static_cast<int64_t>(tc.e) * K * ldb, b_expert_bytes);
    const uint32_t a_voff = static_cast<uint32_t>(a_r) * a_row_bytes + a_c * 16u;
    int b_col = b_cb * 8;
    if (SWIGLU) b_col = b_col < 128 ? n0 + b_col : N + n0 + (b_col - 128);
    else b_col += n0;
    const uint32_t b_voff = static_cast<uint32_t>(b_kb * 8) * b_row_bytes + static_cast<uint32_t>(b_col) * 2u;

    uint4 ra[8], rb[8];
    auto load_global = [&](int ks) {
      const uint32_t av = opaque(a_voff + ks * (kBK * 2u));
      const uint32_t bv = opaque(b_voff + ks * kBK * b_row_bytes);
#pragma unroll
      for (int i = 0; i < 8; ++i) ra[i] = buffer_load16(ra_src, av + i * 32u * a_row_bytes);
#pragma unroll
      for (int i = 0; i < 8; ++i) rb[i] = buffer_load16(rb_src, bv + i * b_row_bytes);
    };
    auto store_lds = [&](int buf) {
      uint16_t* sa = smem[buf][0];
      uint16_t* sb = smem[buf][1];
      // every row offset derives from one opaque base
      const int a_base = opaque(a_r * kBK);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = a_r + 32 * i;
        *reinterpret_cast<uint4*>(sa + a_base + 32 * i * kBK + ((a_c ^ swz(r)) << 3)) = ra[i];
      }
      // transpose the 8 (k) x 8 (n) block: column j gets k = 0..7 contiguous
      const uint32_t* v = reinterpret_cast<const uint32_t*>(rb);  // v[4*i + q]: row i, cols 2q, 2q+1
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = j >> 1;
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t lo = v[4 * (2 * m) + q], hi = v[4 * (2 * m + 1) + q];
          o[m] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        *reinterpret_cast<uint4*>(sb + lds_off(b_cb * 8 + j, b_kb)) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < ksteps) load_global(ks + 1);
      const uint16_t* sa = smem[cur][0];
      const uint16_t* sb = smem[cur][1];
      // fragment rows: row = base + (lane & 31) with base a multiple of 32, so
      // swz(row) = (l ^ (base/8 + l/8)) & 7 with l = lane & 31
      const int fl = opaque(lane & 31);
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int ch = 2 * kk + (lane >> 5);
        bf16x8_t fa[4], fb[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          fa[mi] = *reinterpret_cast<const bf16x8_t*>(sa + lds_off(wm * 128 + mi * 32 + fl, ch));
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          fb[ni] = *reinterpret_cast<const bf16x8_t*>(sb + lds_off(bcol(ni) + fl, ch));
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
      }
      if (ks + 1 < ksteps) store_lds(cur ^ 1);
      __syncthreads();
    }

    // Epilogue: lane holds column (lane & 31), rows 8*(r/4) + 4*(lane/32) + r%4 of each
    // 32 x 32 block. Buffer stores over this tile's valid rows drop rows past the
    // expert's end; a column past N gets an offset beyond the resource (the resource
    // is < 2^31 bytes and row offsets are < 2^31, so the sum cannot wrap).
    const __amdgpu_buffer_rsrc_t rc_src = make_rsrc(
        C + static_cast<int64_t>(row0) * N, static_cast<uint32_t>(rows_valid) * static_cast<uint32_t>(N) * 2u);
    constexpr int kStoreBlocks = SWIGLU ? 2 : 4;
    uint32_t col_off[kStoreBlocks];
#pragma unroll
    for (int ni = 0; ni < kStoreBlocks; ++ni) {
      const int col = n0 + (SWIGLU ? wn * 64 : wn * 128) + ni * 32 + (lane & 31);
      col_off[ni] = col < N ? static_cast<uint32_t>(col) * 2u : 0x80000000u;
    }
    const uint32_t c_row_bytes = static_cast<uint32_t>(N) * 2u;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const uint32_t row_off = static_cast<uint32_t>(row) * c_row_bytes;
#pragma unroll
        for (int ni = 0; ni < kStoreBlocks; ++ni) {
          const float v = SWIGLU ? silu_fast(acc[mi][ni][r]) * acc[mi][ni + 2][r] : acc[mi][ni][r];
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), rc_src,
                                                static_cast<int>(row_off + col_off[ni]), 0, 0);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 path

// K = 64 per stage, with every load of a stage issued before any is stored to
// LDS: the small fp32 products are latency-bound, one memory round trip per stage
// (T = 64 layer: GEMM 105 us with 16-wide stages loaded one element at a time,
// 49 us so; issuing the next stage's loads before computing this one: 57 us).
constexpr int kFBM = 64, kFBN = 64, kFBK = 64;

template <bool SWIGLU>
__global__ __launch_bounds__(kThreads) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C,
    const int32_t* __restrict__ offsets, int e_begin, int e_loc, int K, int N, int ldb, int n_max) {
  __shared__ float As[kFBK][kFBM + 1];
  __shared__ float Bg[kFBK][kFBN];
  __shared__ float Bu[kFBK][kFBN];
  __shared__ TileMap tm;
  build_tile_map<kFBM>(tm, offsets, e_begin, e_loc, n_max);
  const int n_tiles = (N + kFBN - 1) / kFBN;
  const int total = tm.mstart[e_loc] * n_tiles;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  const int64_t b_expert = static_cast<int64_t>(K) * ldb;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const TileCoord tc = find_tile(tm, tile, n_tiles, e_loc);
    const int row0 = tm.rstart[tc.e] + tc.mt * kFBM;
    const int row_end = tm.rstart[tc.e + 1];
    const int n0 = tc.nt * kFBN;
    const float* Bexp = B + static_cast<int64_t>(tc.e) * b_expert;
    float g[4][4] = {}, u[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kFBK) {
      constexpr int kLoads = kFBM * kFBK / kThreads;  // per thread and operand
      float av[kLoads], gv[kLoads], uv[kLoads];
#pragma unroll
      for (int q = 0; q < kLoads; ++q) {
        const int i = q * kThreads + tid;
        const int r = i / kFBK, kk = i % kFBK;
        const int gr = min(row0 + r, row_end - 1);
        av[q] = (k0 + kk < K) ? A[static_cast<int64_t>(gr) * K + k0 + kk] : 0.f;
        const int kb = i / kFBN, c = i % kFBN;
        const bool ok = (k0 + kb < K) && (n0 + c < N);
        const float* brow = Bexp + static_cast<int64_t>(k0 + kb) * ldb;
        gv[q] = ok ? brow[n0 + c] : 0.f;
        uv[q] = (SWIGLU && ok) ? brow[N + n0 + c] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < kLoads; ++q) {
        const int i = q * kThreads + tid;
        As[i % kFBK][i / kFBK] = av[q];
        Bg[i / kFBN][i % kFBN] = gv[q];
        if (SWIGLU) Bu[i / kFBN][i % kFBN] = uv[q];
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kFBK; ++kk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = As[kk][ty * 4 + i];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            g[i][j] = fmaf(a, Bg[kk][tx * 4 + j], g[i][j]);
            if (SWIGLU) u[i][j] = fmaf(a, Bu[kk][tx * 4 + j], u[i][j]);
          }
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + ty * 4 + i;
      if (row >= row_end) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (col < N) C[static_cast<int64_t>(row) * N + col] = SWIGLU ? silu(g[i][j]) * u[i][j] : g[i][j];
      }
    }
  }
}

// CU count of the current device, queried once per device. Atomic, so that
// callers launching from several host threads at once read and fill it safely.
int device_cus() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Persistent grid: enough workgroups to fill the chip, never more than the
// host-side upper bound on tiles (row tiles <= n_max/BM + e_loc per column tile).
int grid_for(int64_t n_max, int e_loc, int bm, int n_tiles, int per_cu) {
  const int64_t upper = (n_max / bm + e_loc) * static_cast<int64_t>(n_tiles);
  const int64_t fill = static_cast<int64_t>(device_cus()) * per_cu;
  int64_t g = upper < fill ? upper : fill;
  if (g > 8) g &= ~int64_t{7};  // a multiple of the 8 XCDs
  return static_cast<int>(g < 1 ? 1 : g);
}

}  // namespace

int grouped_gemm_grid(int64_t n_max, int e_loc, int n_tiles) { return grid_for(n_max, e_loc, kBM, n_tiles, 1); }

int device_cu_count() { return device_cus(); }

hipError_t launch_grouped_gemm_bf16(const void* x_perm, const int32_t* offsets, const void* w_gu,
                                    const void* w_dn, void* h, void* y, int d, int d_ff, int e_begin,
                                    int e_loc, int64_t n_max, int64_t T, int k, int E,
                                    hipStream_t stream) {
  (void)T;
  (void)k;
  (void)E;
  if (n_max == 0) return hipSuccess;
  const int g1 = grid_for(n_max, e_loc, kBM, (d_ff + 127) / 128, 1);
  const int g2 = grid_for(n_max, e_loc, kBM, (d + 255) / 256, 1);
  // The LDS-pipelined kernel needs K (d for gate/up, d_ff for down) in whole
  // 32-wide stages; other multiples of 8 take the register-staged kernel.
  if (d % 32 == 0 && d_ff % 32 == 0)
    return launch_grouped_gemm_lds(x_perm, nullptr, T, k, offsets, w_gu, w_dn, h, y, nullptr, d, d_ff, e_begin,
                                   e_loc, n_max, g1, g2, nullptr, stream);
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, dim3(g1), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(x_perm), static_cast<const uint16_t*>(w_gu),
                     static_cast<uint16_t*>(h), offsets, e_begin, e_loc, d, d_ff, 2 * d_ff,
                     static_cast<int>(n_max));
  hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, dim3(g2), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_dn),
                     static_cast<uint16_t*>(y), offsets, e_begin, e_loc, d_ff, d, d,
                     static_cast<int>(n_max));
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_gather(const void* x, const int32_t* perm, const int32_t* offsets,
                                      const void* w_gu, const void* w_dn, void* h, void* y, void* gu, int d,
                                      int d_ff, int e_begin, int e_loc, int64_t n_max, int64_t T, int k,
                                      void* a_blk, hipStream_t stream) {
  if (n_max == 0) return hipSuccess;
  const int g1 = grid_for(n_max, e_loc, kBM, (d_ff + 127) / 128, 1);
  const int g2 = grid_for(n_max, e_loc, kBM, (d + 255) / 256, 1);
  return launch_grouped_gemm_lds(x, perm, T, k, offsets, w_gu, w_dn, h, y, gu, d, d_ff, e_begin, e_loc, n_max, g1,
                                 g2, a_blk, stream);
}

hipError_t launch_grouped_gemm_f32(const float* x_perm, const int32_t* offsets, const float* w_gu,
                                   const float* w_dn, float* h, float* y, int d, int d_ff,
                                   int e_begin, int e_loc, int64_t n_max, hipStream_t stream) {
  if (n_max == 0) return hipSuccess;
  const int g1 = grid_for(n_max, e_loc, kFBM, (d_ff + kFBN - 1) / kFBN, 4);
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3(g1), dim3(kThreads), 0, stream, x_perm, w_gu, h,
                     offsets, e_begin, e_loc, d, d_ff, 2 * d_ff, static_cast<int>(n_max));
  const int g2 = grid_for(n_max, e_loc, kFBM, (d + kFBN - 1) / kFBN, 4);
  hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3(g2), dim3(kThreads), 0, stream, h, w_dn, y,
                     offsets, e_begin, e_loc, d_ff, d, d, static_cast<int>(n_max));
  return hipGetLastError();
}

}  // namespace moe
