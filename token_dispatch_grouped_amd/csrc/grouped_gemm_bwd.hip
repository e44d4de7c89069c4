// Backward of the grouped expert FFN: the four products of its gradient.
//
// What is computed is the chain rule through experts_forward of "Paralelismo de
// especialistas" (transformers v5.23.0, pt), section "Adicionando uma
// implementação", with the packed gate_up_proj of "Paralelismo de tensor para
// inferência", section "Estratégias empacotadas", and SwiGLU = silu(gate) * up.
// For each local expert e with rows R (its segment of the dispatched rows):
//     dH    = dY @ W_dn[e]^T, then dG = dH * U * silu'(G), dU = dH * silu(G)
//     dX    = [dG | dU] @ W_gu[e]^T
//     dW_dn = H^T @ dY
//     dW_gu = X^T @ [dG | dU]
// with fp32 accumulation and bf16 (RNE) results.
//
// Two tile kinds share the forward kernel's pipeline (LDS-DMA stages of K = 32,
// four stages, reads and loads issued one per MFMA slot):
//   * NT (dH, dX): row tiles of an expert's rows as in the forward; both operands
//     are K-contiguous rows (the activations, and the weights read along their
//     contiguous dimension, which is the product's K here), so both are staged
//     as [row][32] and read with ds_read_b128.
//   * TN (dW): a tile is 256 x 256 of one expert's weight gradient and K runs
//     over the expert's rows (any count, zero included); both operands are
//     row-major activations with M or N contiguous, so both are staged as
//     [k][256] and read back transposed with ds_read_b64_tr_b16.
// Waves: 2 x 2, each 128 x 128 (4 x 4 MFMA blocks of 32 x 32).
//
// The A operands of both NT products live in the workspace in 32-column blocks
// of all N_max rows (see blk_off): [dG | dU], which exists only between the
// launches, and a copy of dY made for the purpose. A K = 32 stage of an NT row
// tile is then one contiguous 16 KB run instead of 256 pieces of 64 bytes (on
// dense8, dX went from 1.70 to 1.50 ms and dH from 1.01 to 0.90 with their
// operands addressed as blocks); a TN stage over [dG | dU] (32 rows of a
// 256-column slice) is eight 2 KB runs.
#include "lds_pipe.h"

namespace moe {
namespace {

using namespace gemm;

constexpr int kBK = 32;
constexpr int kStages = 4;
constexpr int kOpStageBytes = 256 * kBK * 2;  // 16 KB: a 256-row (or 256-column) operand stage
constexpr int kNTAStageBytes = 288 * kBK * 2; // 18 KB: NT activation stage, room for a 288-row tile
constexpr int MI = 4, NI = 4;                 // 32 x 32 blocks per wave

enum Mode { kNT = 0, kTN = 1 };
enum Epi { kPlain = 0, kSwigluBwd = 1 };

template <int MODE>
struct Frags;
template <>
struct Frags<kNT> {
  bf16x8_t a[MI + 1], b[NI];  // a[MI]: the shared extra row block of a 288-row tile
};
template <>
struct Frags<kTN> {
  i16x4_t a[MI][2], b[NI][2];
};

// One operand of a tile as the DMA and the fragment reads see it.
struct Operand {
  const uint16_t* base;  // first element of the tile's rows (KROWS) or k-rows (KMAJOR) at stage 0
  uint32_t bytes;        // bytes from base that are valid (past them: zeros)
  uint32_t stage_step;   // bytes base advances per stage
  uint32_t voff[5];      // per-lane byte offsets of this wave's loads (4, or 5 for 288 rows)
  int slot[5];           // 1 KB LDS slot of each load inside the stage
  uint32_t voff_tail[4]; // KMAJOR over blocks: voff, or past the buffer for k-rows past the tile's
  int tail_stage;        // last rows, in stage tail_stage (-1: none)
};


// KROWS operand ([row][K], K contiguous) of ROWS rows (256 or 288): load j of a
// stage covers rows 16j..16j+15, lane L row 16j + L/4, 16-byte chunk
// (L & 3) ^ ((row >> 2) & 3). With 288 rows there are 18 loads for 4 waves: each
// wave issues 5, the two spare ones repeating a load (same bytes, same place).
template <int ROWS>
__device__ __forceinline__ Operand krows_operand(const uint16_t* rows, int valid_rows, int ld, int wave, int lane) {
  constexpr int kInstr = ROWS / 16, kPer = (kInstr + 3) / 4;
  Operand op;
  op.base = rows;
  op.bytes = static_cast<uint32_t>(valid_rows) * static_cast<uint32_t>(ld) * 2u;
  op.stage_step = kBK * 2;
#pragma unroll
  for (int jj = 0; jj < kPer; ++jj) {
    const int j = (wave * kPer + jj) % kInstr;
    op.slot[jj] = j;
    const int r = 16 * j + (lane >> 2);
    const int c = (lane & 3) ^ ((lane >> 4) & 3);
    op.voff[jj] = static_cast<uint32_t>(r) * static_cast<uint32_t>(ld) * 2u + static_cast<uint32_t>(c) * 16u;
  }
  return op;
}

// KMAJOR operand ([k][ld], the tile's 256 columns from col0): load j of a stage
// covers k-rows 2j, 2j+1, lane L k-row 2j + L/32, chunk (L & 31) ^ (4 * (k & 3)).
__device__ __forceinline__ Operand kmajor_operand(const uint16_t* krows, int valid_krows, int ld, int col0, int wave,
                                                  int lane) {
  Operand op;
  op.base = krows;
  op.bytes = static_cast<uint32_t>(valid_krows) * static_cast<uint32_t>(ld) * 2u;
  op.stage_step = static_cast<uint32_t>(kBK) * static_cast<uint32_t>(ld) * 2u;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int j = wave * 4 + jj;
    op.slot[jj] = j;
    const int kl = 2 * j + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (kl & 3));
    op.voff[jj] = (static_cast<uint32_t>(kl) * static_cast<uint32_t>(ld) + static_cast<uint32_t>(col0 + 8 * c)) * 2u;
  }
  op.tail_stage = -1;
  return op;
}

// KROWS operand over the blocked layout: rows row0.. of a [n_rows][K] matrix in
// 32-column blocks, so a stage is one contiguous run of its rows. Rows past the
// tile's valid rows read whatever lies there (or zeros past the buffer): an NT
// output row depends on its own A row only, and those output rows are not stored.
template <int ROWS>
__device__ __forceinline__ Operand kblk_rows_operand(const uint16_t* buf, int row0, int n_rows, int K, int wave,
                                                     int lane) {
  constexpr int kInstr = ROWS / 16, kPer = (kInstr + 3) / 4;
  Operand op;
  op.base = buf + static_cast<int64_t>(row0) * 32;
  op.bytes = static_cast<uint32_t>(K) * static_cast<uint32_t>(n_rows) * 2u - static_cast<uint32_t>(row0) * 64u;
  op.stage_step = static_cast<uint32_t>(n_rows) * 64u;
#pragma unroll
  for (int jj = 0; jj < kPer; ++jj) {
    const int j = (wave * kPer + jj) % kInstr;
    op.slot[jj] = j;
    const int r = 16 * j + (lane >> 2);
    const int c = (lane & 3) ^ ((lane >> 4) & 3);
    op.voff[jj] = static_cast<uint32_t>(r) * 64u + static_cast<uint32_t>(c) * 16u;
  }
  op.tail_stage = -1;
  return op;
}

// KMAJOR operand over the blocked layout: k-rows r0.. (valid_krows of them) of a
// [n_rows][ld] matrix in 32-column blocks, the tile's 256 columns from col0; the
// same LDS image as kmajor_operand. The extent of a buffer resource cannot stop
// at the tile's last k-row here (the next rows of each block follow it), so the
// loads of the last stage take voff_tail, which sends the lanes of k-rows past
// valid_krows past the buffer (zeros).
__device__ __forceinline__ Operand kblk_kmajor_operand(const uint16_t* buf, int r0, int valid_krows, int n_rows,
                                                       int ld, int col0, int wave, int lane) {
  Operand op;
  op.base = buf + static_cast<int64_t>(r0) * 32;
  op.bytes = static_cast<uint32_t>(ld) * static_cast<uint32_t>(n_rows) * 2u - static_cast<uint32_t>(r0) * 64u;
  op.stage_step = kBK * 64u;
  const int last = (valid_krows + kBK - 1) / kBK - 1;  // -1: no rows
  const int rem = valid_krows - last * kBK;             // k-rows of the last stage
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int j = wave * 4 + jj;
    op.slot[jj] = j;
    const int kl = 2 * j + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (kl & 3));
    op.voff[jj] = blk_off(kl, col0 + 8 * c, n_rows);
    op.voff_tail[jj] = kl < rem ? op.voff[jj] : 0x80000000u;
  }
  op.tail_stage = rem < kBK ? last : -1;
  return op;
}

// The bytes left are clamped at zero with a signed max (every size here is below
// 2^31): the unsigned form becomes a saturating subtract, which has only a vector
// instruction, and a resource held in vector registers makes the compiler wrap
// every load that uses it in a loop over the distinct values of the wave.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(const Operand& op, int s) {
  const int adv = s * static_cast<int>(op.stage_step);
  const int left = static_cast<int>(op.bytes) - adv;
  return make_rsrc(reinterpret_cast<const char*>(op.base) + adv, static_cast<uint32_t>(uniform(left > 0 ? left : 0)));
}

// Byte offset, inside a KROWS stage, of block-row base `rb` (a multiple of 32)
// for slice kk: lane reads row rb + l31, logical chunk 2 kk + lane / 32.
__device__ __forceinline__ uint32_t krows_read(int rb, int kk, int lane) {
  const int l31 = lane & 31;
  const int c = (2 * kk + (lane >> 5)) ^ ((l31 >> 2) & 3);
  return static_cast<uint32_t>((rb + l31) * kBK + c * 8) * 2u;
}

// Byte offset, inside a KMAJOR stage, of column block `cb`: two transposed reads
// (imm 0 and 2048, plus 8192 for slice 1) give lane l column cb + l % 32, k 8(l/32)..+7.
__device__ __forceinline__ uint32_t kmajor_read(int cb, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int kl = (g >> 1) * 8 + (i >> 2);
  const int n = cb + (g & 1) * 16 + 4 * (i & 3);
  return static_cast<uint32_t>(kl * 256 + (((n >> 3) ^ (4 * (kl & 3))) * 8) + (n & 4)) * 2u;
}

__device__ __forceinline__ float sigmoid_fast(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// mfma c += a * b with c held in VGPRs (the 256 accumulation registers are full)
__device__ __forceinline__ void mfma_vgpr(f32x16_t& c, const bf16x8_t& a, const bf16x8_t& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

// up_off (kSwigluBwd): columns between gate and up halves of C and gu (= N).
// XR (NT only): 1 for a 288-row tile, whose rows 256..287 every wave shares: each
// wave multiplies them by two of its four column blocks. The second wave row keeps
// its column blocks in swapped slots (block = slot ^ 2), so that both wave rows use
// slots 0 and 1 for the extra rows and together cover all four blocks.
// BBLK (TN): B is a blocked KMAJOR operand (kblk_kmajor_operand), whose last
// stage takes its tail offsets. CBLK (NT with kSwigluBwd): C is the blocked
// [dG | dU] of cblk_rows rows, C pointing at its start and (crow0, ccol0) the
// tile's origin in it; otherwise C points at the tile's origin, row stride ldc.
template <int MODE, int EPI, int XR, bool BBLK = false, bool CBLK = false>
__device__ __forceinline__ void bwd_tile(uint16_t* smem, const Operand& opa, const Operand& opb, int ksteps,
                                         uint16_t* __restrict__ C, int c_rows, int c_cols, int ldc,
                                         const uint16_t* __restrict__ gu, int up_off, int cblk_rows = 0,
                                         int crow0 = 0, int ccol0 = 0) {
  static_assert(XR == 0 || MODE == kNT, "extra rows only in NT tiles");
  constexpr int MX = XR ? 2 : 0;                                     // extra MFMA blocks per wave
  constexpr int NA = XR ? 5 : 4;                                     // activation loads per wave per stage
  constexpr int PER = NA + 4;                                        // DMA loads per wave per stage
  constexpr int kAStage = MODE == kNT ? kNTAStageBytes : kOpStageBytes;
  const int lane = lane_id();
  const int wave = uniform(static_cast<int>(threadIdx.x) / kWave);
  const int wm = wave / 2, wn = wave % 2;
  const int l31 = lane & 31;
  const uint32_t sA = uniform(static_cast<int>(lds_addr(smem)));
  const uint32_t sB = sA + kStages * kAStage;
  // column block of B slot ni
  auto blk = [&](int ni) { return XR && wm ? ni ^ 2 : ni; };

  // fragment read offsets
  uint32_t a_rd[2], a_rd_x[2], b_rd_lo[2], b_rd_hi[2], at_rd[MI], bt_rd[NI];
  if constexpr (MODE == kNT) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      a_rd[kk] = krows_read(wm * 128, kk, lane);
      a_rd_x[kk] = krows_read(256, kk, lane);
      b_rd_lo[kk] = krows_read(wn * 128 + blk(0) * 32, kk, lane);  // slots 0, 1
      b_rd_hi[kk] = krows_read(wn * 128 + blk(2) * 32, kk, lane);  // slots 2, 3
    }
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i) at_rd[i] = kmajor_read(wm * 128 + i * 32, lane);
#pragma unroll
    for (int i = 0; i < NI; ++i) bt_rd[i] = kmajor_read(wn * 128 + i * 32, lane);
  }
  // LDS reads of one 16-wide K slice: the A blocks (and the extra row block), then
  // the B blocks (KROWS: one ds_read_b128 each; KMAJOR: two transposed reads each)
  constexpr int R = MODE == kNT ? MI + XR + NI : 2 * (MI + NI);
  auto read_one = [&](Frags<MODE>& f, int buf, auto kk_c, auto r_c) {
    constexpr int kk = decltype(kk_c)::value, r = decltype(r_c)::value;
    if constexpr (MODE == kNT) {
      if constexpr (r < MI) {
        f.a[r] = ds_read16<r * 2048>(sA + buf * kAStage + a_rd[kk]);
      } else if constexpr (r < MI + XR) {
        f.a[MI] = ds_read16<0>(sA + buf * kAStage + a_rd_x[kk]);
      } else {
        constexpr int ni = r - MI - XR;
        f.b[ni] = ds_read16<(ni & 1) * 2048>(sB + buf * kOpStageBytes + (ni < 2 ? b_rd_lo[kk] : b_rd_hi[kk]));
      }
    } else {
      constexpr int blk_i = (r % (2 * MI)) / 2, h = r % 2;
      if constexpr (r < 2 * MI) f.a[blk_i][h] = ds_read_tr<kk * 8192 + h * 2048>(sA + buf * kAStage + at_rd[blk_i]);
      else f.b[blk_i][h] = ds_read_tr<kk * 8192 + h * 2048>(sB + buf * kOpStageBytes + bt_rd[blk_i]);
    }
  };
  auto tie_frags = [&](Frags<MODE>& f) {
    if constexpr (MODE == kNT) {
#pragma unroll
      for (int i = 0; i < MI + XR; ++i) tie(f.a[i]);
#pragma unroll
      for (int i = 0; i < NI; ++i) tie(f.b[i]);
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        tie(f.a[i][0]);
        tie(f.a[i][1]);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        tie(f.b[i][0]);
        tie(f.b[i][1]);
      }
    }
  };

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  f32x16_t acc_x[MX > 0 ? MX : 1];
#pragma unroll
  for (int x = 0; x < MX; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_x[x][r] = 0.f;

  // MFMA q of a slice: the extra row block first (its VGPR results are next read
  // NM - MX MFMAs later, also after the last slice), then row-major over mi, ni
  auto mfma_one = [&](const auto& f, auto q_c) {  // f: Frags<MODE> (a generic parameter, so
    constexpr int q = decltype(q_c)::value;       // that the unused branch is not instantiated)
    if constexpr (q < MX) {
      mfma_vgpr(acc_x[q], f.a[MI], f.b[q]);
    } else {
      constexpr int mi = (q - MX) / NI, ni = (q - MX) % NI;
      if constexpr (MODE == kNT)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
      else
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join(f.a[mi][0], f.a[mi][1]),
                                                              join(f.b[ni][0], f.b[ni][1]), acc[mi][ni], 0, 0, 0);
    }
  };

  // DMA of one stage: loads 0..NA-1 the A operand, then 4 of the B operand
  struct StageLoads {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t la, lb;
    bool tail_b;  // BBLK: B's loads take their tail offsets
  };
  auto stage_loads = [&](int s) {
    const int buf = s % kStages;
    return StageLoads{stage_rsrc(opa, s), stage_rsrc(opb, s), sA + buf * kAStage, sB + buf * kOpStageBytes,
                      BBLK && s == opb.tail_stage};
  };
  auto dma_one = [&](const StageLoads& st, auto j_c) {
    constexpr int j = decltype(j_c)::value;
    if constexpr (j < NA) {
      dma16(st.ra, opa.voff[j], st.la + opa.slot[j] * 1024);
    } else if constexpr (BBLK) {
      dma16(st.rb, st.tail_b ? opb.voff_tail[j - NA] : opb.voff[j - NA], st.lb + opb.slot[j - NA] * 1024);
    } else {
      dma16(st.rb, opb.voff[j - NA], st.lb + opb.slot[j - NA] * 1024);
    }
  };
  auto wait_stage = [&](int s) {
    const int after = min(kStages - 2, ksteps - 1 - s);
    static_for<0, kStages - 1>([&](auto a_c) {
      constexpr int a = decltype(a_c)::value;
      if (after == a) wait_vmcnt<a * PER>();
    });
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  constexpr int NM = MI * NI + MX;
  // reads per MFMA: all of a slice's reads go out in the first three quarters of
  // the slice, so the last has a quarter slice of MFMAs to land
  constexpr int RPM = (R + (NM * 3 / 4) - 1) / (NM * 3 / 4);

  // One stage, as in the forward kernel: slice 0 carries slice 1's reads; the
  // stage barrier; slice 1 carries the next stage's slice-0 reads and the DMA of
  // stage ks + kStages, one load per two MFMAs.
  Frags<MODE> f0, f1;
  auto stage = [&](int ks, auto dma_c, auto more_c) {
    constexpr bool DMA = decltype(dma_c)::value, MORE = decltype(more_c)::value;
    const int buf = ks % kStages;
    wait_lgkmcnt<0>();
    tie_frags(f0);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NM>([&](auto q_c) {
      constexpr int q = decltype(q_c)::value;
      mfma_one(f0, q_c);
      __builtin_amdgcn_sched_barrier(0);
      static_for<(q * RPM < R ? q * RPM : R), ((q + 1) * RPM < R ? (q + 1) * RPM : R)>(
          [&](auto r) { read_one(f1, buf, K1{}, r); });
      __builtin_amdgcn_sched_barrier(0);
    });
    wait_lgkmcnt<0>();
    tie_frags(f1);
    if constexpr (MORE) {
      wait_stage(ks + 1);
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_sched_barrier(0);
    StageLoads st;
    if constexpr (DMA) st = stage_loads(ks + kStages);
    const int nbuf = (ks + 1) % kStages;
    static_for<0, NM>([&](auto q_c) {
      constexpr int q = decltype(q_c)::value;
      mfma_one(f1, q_c);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MORE)
        static_for<(q * RPM < R ? q * RPM : R), ((q + 1) * RPM < R ? (q + 1) * RPM : R)>(
            [&](auto r) { read_one(f0, nbuf, K0{}, r); });
      if constexpr (DMA && q % 2 == 0 && q / 2 < PER) dma_one(st, std::integral_constant<int, q / 2>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (DMA) static_for<((NM + 1) / 2 < PER ? (NM + 1) / 2 : PER), PER>([&](auto j) { dma_one(st, j); });
    __builtin_amdgcn_sched_barrier(0);
  };

  if (ksteps > 0) {
    for (int s = 0; s < kStages - 1 && s < ksteps; ++s) {
      const StageLoads st = stage_loads(s);
      static_for<0, PER>([&](auto j) { dma_one(st, j); });
    }
    wait_stage(0);
    __builtin_amdgcn_s_barrier();
    if (kStages - 1 < ksteps) {
      const StageLoads st = stage_loads(kStages - 1);
      static_for<0, PER>([&](auto j) { dma_one(st, j); });
    }
    static_for<0, R>([&](auto r) { read_one(f0, 0, K0{}, r); });
    int ks = 0;
    for (; ks + kStages < ksteps; ++ks) stage(ks, std::true_type{}, std::true_type{});
    for (; ks + 1 < ksteps; ++ks) stage(ks, std::false_type{}, std::true_type{});
    stage(ks, std::false_type{}, std::false_type{});
  }

  // ---- epilogue: C is c_rows x c_cols (row stride ldc) at the tile origin --------
  const __amdgpu_buffer_rsrc_t rc =
      CBLK ? make_rsrc(C, static_cast<uint32_t>(cblk_rows) * static_cast<uint32_t>(ldc) * 2u)
           : make_rsrc(C, static_cast<uint32_t>(c_rows) * static_cast<uint32_t>(ldc) * 2u);
  // ---- epilogue: C goes out through LDS (the stage buffers are free after the K
  // loop), 64 rows at a time, as 16-byte vectors of 8 columns, so that a store
  // moves two whole rows of the tile instead of one element per lane (an eighth
  // of the store instructions, whose issue was a fifth of the TN kernel's time).
  // The passes take wave row p / 2's blocks mi = 2 (p % 2) and the next; a
  // 288-row NT tile's extra 32 rows, a part of which every wave holds, go in a
  // fifth pass. Row pitch 264 floats: the two half-waves of a staging write
  // (rows 4 apart) land in different bank halves.
  constexpr int kPitch = 256 + 8;
  float* stg = reinterpret_cast<float*>(smem);
  const int tid = static_cast<int>(threadIdx.x);
  // one 32 x 32 block into staged rows row_base.., lane column col
  auto stage_block = [&](const f32x16_t& a, int row_base, int col) {
#pragma unroll
    for (int r = 0; r < 16; ++r) stg[(row_base + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * kPitch + col] = a[r];
  };
  auto stage_pass = [&](int p) {
    if (wm == (p >> 1)) {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) stage_block(acc[2 * (p & 1) + m2][ni], m2 * 32, wn * 128 + blk(ni) * 32 + l31);
    }
  };
  auto stage_extra = [&] {
#pragma unroll
    for (int x = 0; x < MX; ++x) stage_block(acc_x[x], 0, wn * 128 + blk(x) * 32 + l31);
  };
  // 8-column chunk i of a pass: staged row rl, column col; byte offset of C row
  // row0 + rl at column col (c_cols is a multiple of 32, so a chunk is all in
  // range or all out; rows past c_rows fall outside the buffer and are dropped)
  auto chunk = [&](int i, int row0, int& rl, int& col, int cshift) {
    const int c = tid + i * kThreads;
    rl = c >> 5;
    col = (c & 31) * 8;
    return col < c_cols ? static_cast<uint32_t>(row0 + rl) * static_cast<uint32_t>(ldc) * 2u +
                              static_cast<uint32_t>(col + cshift) * 2u
                        : 0x80000000u;
  };
  // byte offset in C of tile row row0 + rl, tile column col + cshift (past the
  // buffer for rows past c_rows and columns past c_cols): the blocked [dG | dU]
  // with CBLK (ldc = its column count), else row-major from the tile's origin
  auto cstore = [&](int rl, int row0, int col, int cshift) -> uint32_t {
    if constexpr (CBLK) {
      return row0 + rl < c_rows && col < c_cols ? blk_off(crow0 + row0 + rl, ccol0 + col + cshift, cblk_rows)
                                                : 0x80000000u;
    } else {
      return col < c_cols ? static_cast<uint32_t>(row0 + rl) * static_cast<uint32_t>(ldc) * 2u +
                                static_cast<uint32_t>(col + cshift) * 2u
                          : 0x80000000u;
    }
  };
  auto staged8 = [&](int rl, int col, float* h) {
    const float4 h0 = *reinterpret_cast<const float4*>(stg + rl * kPitch + col);
    const float4 h1 = *reinterpret_cast<const float4*>(stg + rl * kPitch + col + 4);
    h[0] = h0.x, h[1] = h0.y, h[2] = h0.z, h[3] = h0.w, h[4] = h1.x, h[5] = h1.y, h[6] = h1.z, h[7] = h1.w;
  };
  if constexpr (EPI == kSwigluBwd && MODE == kNT) {
    // C = [dG | dU] from the staged dH and G, U of the same elements (gu has
    // C's layout); each pass's G and U loads go out before its rows are
    // staged, so their latency runs under the staging
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gu, static_cast<uint32_t>(c_rows) * static_cast<uint32_t>(ldc) * 2u);
    auto finish_rows = [&](int row0, auto nr_c, auto&& stage_fn) {
      constexpr int NR = decltype(nr_c)::value;
      constexpr int kChunks = NR * 256 / 8 / kThreads;  // 8-column chunks per thread
      uint4 gv[kChunks], uv[kChunks];
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        int rl, col;
        gv[i] = buffer_load16(rg, chunk(i, row0, rl, col, 0));
        uv[i] = buffer_load16(rg, chunk(i, row0, rl, col, up_off));
      }
      stage_fn();
      __syncthreads();  // the staged rows are in LDS
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        int rl, col;
        chunk(i, row0, rl, col, 0);
        float dh[8];
        staged8(rl, col, dh);
        const uint32_t gw[4] = {gv[i].x, gv[i].y, gv[i].z, gv[i].w}, uw[4] = {uv[i].x, uv[i].y, uv[i].z, uv[i].w};
        uint32_t dgw[4], duw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t dgp = 0, dup = 0;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const float g = bf16_to_f32(static_cast<uint16_t>(gw[q] >> (16 * hh)));
            const float u = bf16_to_f32(static_cast<uint16_t>(uw[q] >> (16 * hh)));
            const float s = sigmoid_fast(g);
            const float d = dh[2 * q + hh];
            dgp |= static_cast<uint32_t>(f32_to_bf16_rne(d * u * (s * (1.0f + g * (1.0f - s))))) << (16 * hh);
            dup |= static_cast<uint32_t>(f32_to_bf16_rne(d * g * s)) << (16 * hh);
          }
          dgw[q] = dgp;
          duw[q] = dup;
        }
        buffer_store16(make_uint4(dgw[0], dgw[1], dgw[2], dgw[3]), rc, cstore(rl, row0, col, 0));
        buffer_store16(make_uint4(duw[0], duw[1], duw[2], duw[3]), rc, cstore(rl, row0, col, up_off));
      }
      __syncthreads();  // the staged rows are read before the next ones are written
    };
    __syncthreads();  // every wave is done with the K loop's LDS stages
#pragma unroll
    for (int p = 0; p < 4; ++p) finish_rows(64 * p, std::integral_constant<int, 64>{}, [&] { stage_pass(p); });
    if constexpr (MX > 0) finish_rows(256, std::integral_constant<int, 32>{}, stage_extra);
  } else {
    // plain C, rounded to bf16
    auto write_rows = [&](int row0, auto nr_c) {
      constexpr int NR = decltype(nr_c)::value;
      __syncthreads();  // the staged rows are in LDS
#pragma unroll
      for (int i = 0; i < NR * 256 / 8 / kThreads; ++i) {
        int rl, col;
        const uint32_t off = chunk(i, row0, rl, col, 0);
        float h[8];
        staged8(rl, col, h);
        uint32_t w4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w4[q] = static_cast<uint32_t>(f32_to_bf16_rne(h[2 * q])) |
                  (static_cast<uint32_t>(f32_to_bf16_rne(h[2 * q + 1])) << 16);
        buffer_store16(make_uint4(w4[0], w4[1], w4[2], w4[3]), rc, off);
      }
      __syncthreads();  // the staged rows are read before the next ones are written
    };
    __syncthreads();  // every wave is done with the K loop's LDS stages
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      stage_pass(p);
      write_rows(64 * p, std::integral_constant<int, 64>{});
    }
    if constexpr (MX > 0) {
      stage_extra();
      write_rows(256, std::integral_constant<int, 32>{});
    }
  }
}

// NT: C[rows, N] = A[rows, K] @ B_e[N, K]^T over row tiles of each local expert,
// A in the blocked layout (blk_off, n_max rows, K columns).
// EPI = kSwigluBwd: A = dY, B = W_dn (N = d_ff, K = d), gu = [G | U] of the same
// rows (row stride ldc = 2 N), C = [dG | dU], blocked (n_max rows, ldc columns).
// EPI = kPlain: A = that [dG | dU] (K = 2 d_ff), B = W_gu, C = dX row-major (row
// stride ldc).
template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_nt_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    const uint16_t* __restrict__ gu, const int32_t* __restrict__ offsets, int e_begin, int e_loc, int K, int N,
    int ldc, int n_max) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kStages * (288 + 256) * kBK];
  __shared__ SortedTileMap tm;
  // a remainder of at most 32 rows rides on the expert's last full tile (288 rows)
  build_sorted_tile_map<256, 32>(tm, offsets, e_begin, e_loc, n_max);
  const int n_tiles = (N + 255) / 256;
  const int total = uniform(tm.mstart[e_loc]) * n_tiles;
  const int lane = lane_id();
  const int wave = uniform(static_cast<int>(threadIdx.x) / kWave);
  const int G = gridDim.x, r = xcd_remap(blockIdx.x, G);
  for (int i = 0;; ++i) {
    const int tile = snake_tile(i, r, G);
    if (tile >= total) break;  // later rounds hold only larger ids
    const SortedTile tc = find_sorted_tile(tm, tile, n_tiles, e_loc);
    const int row0 = uniform(tm.rstart[tc.e]) + tc.mt * 256;
    const int rows = tc.mt == tc.mt_e - 1 ? uniform(tm.rstart[tc.e + 1]) - row0 : 256;
    const int n0 = tc.nt * 256;
    const uint16_t* Bexp = B + static_cast<int64_t>(tc.e) * N * K;
    const Operand opb = krows_operand<256>(Bexp + static_cast<int64_t>(n0) * K, N - n0, K, wave, lane);
    if constexpr (EPI == kSwigluBwd) {
      const uint16_t* gut = gu + static_cast<int64_t>(row0) * ldc + n0;
      if (rows > 256) {
        const Operand opa = kblk_rows_operand<288>(A, row0, n_max, K, wave, lane);
        bwd_tile<kNT, EPI, 1, false, true>(smem, opa, opb, K / kBK, C, rows, N - n0, ldc, gut, N, n_max, row0, n0);
      } else {
        const Operand opa = kblk_rows_operand<256>(A, row0, n_max, K, wave, lane);
        bwd_tile<kNT, EPI, 0, false, true>(smem, opa, opb, K / kBK, C, rows, N - n0, ldc, gut, N, n_max, row0, n0);
      }
    } else {
      uint16_t* Ct = C + static_cast<int64_t>(row0) * ldc + n0;
      if (rows > 256) {
        const Operand opa = kblk_rows_operand<288>(A, row0, n_max, K, wave, lane);
        bwd_tile<kNT, EPI, 1>(smem, opa, opb, K / kBK, Ct, rows, N - n0, ldc, nullptr, 0);
      } else {
        const Operand opa = kblk_rows_operand<256>(A, row0, n_max, K, wave, lane);
        bwd_tile<kNT, EPI, 0>(smem, opa, opb, K / kBK, Ct, rows, N - n0, ldc, nullptr, 0);
      }
    }
    __builtin_amdgcn_s_barrier();
  }
}

// Tile `rem` of an expert's m_tiles x n_tiles output grid, walked in groups of
// kRowGroup m-tiles, the m-tile fastest inside a group (the last group holds the
// rest). 32 consecutive ids (one XCD's workgroups in a round) then cover 4
// m-tiles x 8 n-tiles: each k-slice of an A column block crosses to that XCD's
// L2 once per 8 tiles and each B column block once per 4 (with the n-tile
// fastest, every tile fetched its own B block).
__device__ __forceinline__ void grouped_mn(int rem, int m_tiles, int n_tiles, int& mt, int& nt) {
  const int full = m_tiles / kRowGroup * kRowGroup;
  if (rem < full * n_tiles) {
    const int g = rem / (kRowGroup * n_tiles), off = rem - g * kRowGroup * n_tiles;
    mt = g * kRowGroup + off % kRowGroup;
    nt = off / kRowGroup;
  } else {
    const int rest = m_tiles - full, off = rem - full * n_tiles;
    mt = full + off % rest;
    nt = off / rest;
  }
}

// TN: dW_e[M, N] = A_e^T @ B_e with A = src_a [rows][M], B = src_b [rows][N]
// over each local expert's rows (K = its row count; none gives zeros). BBLK: B is
// the blocked [dG | dU] (blk_off, n_max rows).
template <bool BBLK>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_tn_kernel(
    const uint16_t* __restrict__ src_a, const uint16_t* __restrict__ src_b, uint16_t* __restrict__ dW,
    const int32_t* __restrict__ offsets, int e_begin, int e_loc, int M, int N, int n_max) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kStages * 2 * 256 * kBK];
  const int m_tiles = (M + 255) / 256, n_tiles = (N + 255) / 256;
  const int per_e = m_tiles * n_tiles;
  const int total = e_loc * per_e;
  const int lane = lane_id();
  const int wave = uniform(static_cast<int>(threadIdx.x) / kWave);
  const int base = offsets[e_begin];
  for (int tile = xcd_remap(blockIdx.x, gridDim.x); tile < total; tile += gridDim.x) {
    const int e = tile / per_e;
    int mt, nt;
    grouped_mn(tile - e * per_e, m_tiles, n_tiles, mt, nt);
    mt = uniform(mt);
    nt = uniform(nt);
    const int r0 = uniform(min(offsets[e_begin + e] - base, n_max));
    const int rows = uniform(min(offsets[e_begin + e + 1] - base, n_max)) - r0;
    const int m0 = mt * 256, n0 = nt * 256;
    const Operand opa = kmajor_operand(src_a + static_cast<int64_t>(r0) * M, rows, M, m0, wave, lane);
    const Operand opb = BBLK ? kblk_kmajor_operand(src_b, r0, rows, n_max, N, n0, wave, lane)
                             : kmajor_operand(src_b + static_cast<int64_t>(r0) * N, rows, N, n0, wave, lane);
    bwd_tile<kTN, kPlain, 0, BBLK>(smem, opa, opb, (rows + kBK - 1) / kBK,
                          dW + static_cast<int64_t>(e) * M * N + static_cast<int64_t>(m0) * N + n0, M - m0, N - n0, N,
                          nullptr, 0);
    __builtin_amdgcn_s_barrier();
  }
}

// Rows [0, N_loc) of a row-major [N_max][cols] matrix into the blocked layout
// (blk_off, n_max rows): one 16-byte chunk of 8 columns per thread. Eight
// consecutive threads take rows 2m and 2m + 1 of one 32-column block (one
// 128-byte line of the destination), the next eight the next block: a wave reads
// two whole 512-byte row pieces and writes eight whole lines.
__global__ __launch_bounds__(kThreads) void to_blocked_kernel(const uint4* __restrict__ src, uint16_t* __restrict__ dst,
                                                             const int32_t* __restrict__ offsets, int e_begin,
                                                             int e_end, int cols, int n_max) {
  const int n_loc = min(offsets[e_end] - offsets[e_begin], n_max);
  const int nb = cols / 32;
  const int64_t items = static_cast<int64_t>((n_loc + 1) / 2) * nb * 8;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; it < items;
       it += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int sub = static_cast<int>(it & 3), rp = static_cast<int>((it >> 2) & 1);
    const int64_t rest = it >> 3;
    const int m = static_cast<int>(rest / nb), b = static_cast<int>(rest - static_cast<int64_t>(m) * nb);
    const int r = 2 * m + rp;
    if (r < n_loc)
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(dst) + blk_off(r, b * 32 + sub * 8, n_max)) =
          src[static_cast<int64_t>(r) * (cols / 8) + b * 4 + sub];
  }
}

}  // namespace

hipError_t launch_to_blocked(const void* src, void* dst, const int32_t* offsets, int e_begin, int e_end, int cols,
                             int64_t n_max, hipStream_t stream) {
  int64_t blocks = (n_max * (cols / 8) + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(to_blocked_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(src), static_cast<uint16_t*>(dst), offsets, e_begin, e_end, cols,
                     static_cast<int>(n_max));
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_nt(const void* a, const void* b, void* c, const void* gu, const int32_t* offsets,
                                  int e_begin, int e_loc, int K, int N, int ldc, int64_t n_max, bool swiglu_bwd,
                                  int grid, hipStream_t stream) {
  if (swiglu_bwd) {
    hipLaunchKernelGGL(grouped_gemm_nt_kernel<kSwigluBwd>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), static_cast<uint16_t*>(c),
                       static_cast<const uint16_t*>(gu), offsets, e_begin, e_loc, K, N, ldc, static_cast<int>(n_max));
  } else {
    hipLaunchKernelGGL(grouped_gemm_nt_kernel<kPlain>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), static_cast<uint16_t*>(c),
                       nullptr, offsets, e_begin, e_loc, K, N, ldc, static_cast<int>(n_max));
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_tn(const void* src_a, const void* src_b, void* dw, const int32_t* offsets,
                                  int e_begin, int e_loc, int M, int N, int64_t n_max, bool b_blocked, int grid,
                                  hipStream_t stream) {
  if (b_blocked)
    hipLaunchKernelGGL(grouped_gemm_tn_kernel<true>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(src_a), static_cast<const uint16_t*>(src_b),
                       static_cast<uint16_t*>(dw), offsets, e_begin, e_loc, M, N, static_cast<int>(n_max));
  else
    hipLaunchKernelGGL(grouped_gemm_tn_kernel<false>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(src_a), static_cast<const uint16_t*>(src_b),
                       static_cast<uint16_t*>(dw), offsets, e_begin, e_loc, M, N, static_cast<int>(n_max));
  return hipGetLastError();
}

}  // namespace moe
