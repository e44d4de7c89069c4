// Grouped expert GEMM, pipelined variant for K a multiple of 32 (every
// workload's d and d_ff): operands go from HBM straight into LDS and the
// N-contiguous weights are read back transposed by the LDS unit.
//
// What is computed is the same as the register-staged kernel in
// grouped_gemm.hip: experts_forward of "Paralelismo de especialistas"
// (transformers v5.23.0, pt), section "Adicionando uma implementação", on the
// packed gate_up_proj of "Paralelismo de tensor para inferência", section
// "Estratégias empacotadas", with SwiGLU = silu(gate) * up, then the down
// projection.
//
// Design (gfx950):
//   * Four LDS stages of K = 32 (18 KB of activations, room for 288 rows, + 16 KB
//     of weights each, 136 KB in all). Each stage is filled by buffer_load ... lds (16 bytes per
//     lane, written to LDS without passing through registers), issued three
//     stages ahead of its use, so about 3 x 1000 MFMA cycles of HBM/L2 latency
//     are covered without staging registers.
//   * Activations sit in LDS as [row][32] (64-byte rows) with the 16-byte chunk
//     index XOR-ed by (row >> 2) & 3; 16 consecutive fragment rows then hit 16
//     distinct bank groups. Weights sit as [k][256] in the pages' N-contiguous
//     order with the chunk index XOR-ed by 4 * (k & 3); ds_read_b64_tr_b16 turns
//     each 4 (k) x 16 (n) block into per-lane 4-k columns, two of which form a
//     v_mfma_f32_32x32x16_bf16 B operand. No weight repacking, no VALU transpose.
//   * LDS reads are issued by inline asm with explicit lgkmcnt waits, so the
//     compiler does not serialise them behind the outstanding LDS-DMA loads.
//     Fragments for the next 16-wide K slice are read while the current slice's
//     MFMAs run, one read after each MFMA, and the DMA loads go one after every
//     second MFMA: with one wave per SIMD, a burst of other instructions would
//     leave the matrix unit idle. sched_barriers keep that order in place.
//   * Row tiles are 256 rows. A remainder of at most 32 rows rides on the
//     expert's last full tile, which becomes 288 rows: every wave also takes
//     half of its weight blocks against the shared 32-row block (their two
//     accumulators live in VGPRs, the other 256 registers being full). A larger
//     remainder gets its own tile of the smallest of 32/64/128/256 rows that
//     covers it. Wave layouts: 2 x 2 waves of (H/2) x 128 for H >= 64, 1 x 4
//     waves of 32 x 64 for H = 32.
//   * Half-width tiles (128 weight columns, five stages in the same LDS) for
//     balance: the last round's tiles when they would fill at most half of the
//     workgroups, and a last column block that is at most half full.
//   * Tile walk: persistent workgroups, experts ordered by the height class of
//     their tiles, rounds walked in snake order, each XCD given a contiguous
//     range of tile ids (gemm_common.h). Epilogue: bf16 buffer stores bounded by
//     the tile's valid rows; SAVE also keeps the gate/up pre-activations.
//   * Activation rows come as x_perm / H rows (64 bytes of each row per stage),
//     gathered from x through perm in the loads, or, when each row is read by
//     enough column tiles to pay for a copy, from a copy of the gathered rows in
//     32-column blocks (gather_blocked_kernel), where a stage of a row tile is one
//     contiguous run.
#include <type_traits>

#include "lds_pipe.h"

namespace moe {
namespace {

using namespace gemm;

constexpr int kBK = 32;                       // K per stage
constexpr int kStages = 4;
constexpr int kPaceStride = 32;  // ints between the per-XCD tile counts (one 128-byte line each)
constexpr int kPacePolls = 64;
constexpr int kARows = 288;                   // rows an activation stage holds
constexpr int kAStageElems = kARows * kBK;    // 18 KB
constexpr int kBStageElems = 256 * kBK;       // 16 KB
constexpr uint32_t kAStageBytes = kAStageElems * 2;
constexpr uint32_t kBStageBytes = kBStageElems * 2;

struct Frags {
  bf16x8_t a[5];   // A blocks (32 rows each); a[MI] is the extra block of a 288-row tile
  i16x4_t b[4][2]; // B blocks (32 columns each), two 4-k halves
};

// H = rows of the tile: 32, 64, 128, 256 or 288. A 288-row tile is a 256-row
// tile plus one 32-row block (rows 256..287) that every wave shares: each wave
// computes it against half of its own weight blocks. BN = weight columns of the
// tile: 256, or 128 for a half-width tile (the two halves of a tile split for
// balance, or a last column block that is at most half full).
template <int H, int BN>
struct Layout {
  static constexpr int WM = H >= 64 ? 2 : 1;       // waves along M
  static constexpr int WN = 4 / WM;                // waves along N
  static constexpr int MI = H / WM / 32;           // 32-row MFMA blocks per wave (regular part)
  static constexpr int NI = BN / WN / 32;          // 32-column MFMA blocks per wave
  static constexpr int XR = (H - WM * MI * 32) / 32;  // shared extra row blocks (0 or 1)
  // extra MFMA blocks per wave: half of four blocks, or one of two (with SwiGLU the
  // two wave rows then hold the gate and the up half of one pair between them)
  static constexpr int MX = XR ? (NI == 4 ? 2 : 1) : 0;
  static constexpr int A_INSTR = H / 16;           // 1 KB DMA instructions per activation stage
  static constexpr int A_PER_WAVE = (A_INSTR + 3) / 4;
  static constexpr int B_PER_WAVE = BN / 64;       // 1 KB DMA instructions per weight stage, per wave
  static constexpr int PER = B_PER_WAVE + A_PER_WAVE;  // DMA instructions per stage per wave
  static constexpr int LDS_READS = MI + XR + 2 * NI;
  static constexpr int NMFMA = MI * NI + MX;       // MFMAs per 16-wide K slice
  static_assert(XR == 0 || (XR == 1 && WM == 2), "one shared extra row block, two waves along M");
  static_assert(BN == 256 || BN == 128, "full or half-width tiles");
};

// Where activation rows come from (AM): kAInOrder, rows of A in order (x_perm,
// H); kAGather, row r of the local segment is row perm_seg[r] / k of A (the
// token's hidden state in x, the row gather of the dispatch done by the loads);
// kABlocked, row r of A stored in 32-column blocks of n_rows rows (blk_off).
enum AMode { kAInOrder = 0, kAGather = 1, kABlocked = 2 };
struct ARows {
  const int32_t* perm_seg;  // perm + offsets[e_begin]
  int k;
  uint32_t a_bytes;         // bytes of A (T * K * 2)
  int n_rows;               // rows of a blocked A
};

// BSTREAM: the tile's weight panel is read by no other row tile (its expert has
// one), so its loads carry the non-temporal policy.
template <bool SWIGLU, int AM, bool SAVE, int H, int BN, bool BSTREAM>
__device__ __forceinline__ void gemm_tile(uint16_t* smem, const uint16_t* __restrict__ A,
                                          const uint16_t* __restrict__ Bexp, uint16_t* __restrict__ C,
                                          uint16_t* __restrict__ GU, int row0, int rows_valid, int n0, int K, int N,
                                          int ldb, const ARows& ar) {
  static_assert(!SAVE || SWIGLU, "pre-activations are kept only by the gate/up product");
  constexpr bool GATHER = AM == kAGather, BLK = AM == kABlocked;
  using L = Layout<H, BN>;
  constexpr int MI = L::MI, NI = L::NI, WM = L::WM, WN = L::WN, PER = L::PER;
  // A half-width tile does half the MFMA work per stage, so the same lookahead
  // in stages covers half the time: it runs five stages (four ahead) in the
  // room of the full-width tile's four.
  constexpr int NS = BN == 256 ? kStages : 5;
  constexpr uint32_t kBBytes = BN * kBK * 2;  // weight stage
  static_assert(NS * (kAStageBytes + kBBytes) <= kStages * (kAStageBytes + kBStageBytes), "stages fit");
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = uniform(tid / kWave);
  const int wm = wave / WN, wn = wave % WN;
  const int ksteps = K / kBK;

  const uint32_t sA_base = uniform(static_cast<int>(lds_addr(smem)));
  const uint32_t sB_base = sA_base + NS * kAStageBytes;

  // ---- DMA: per-lane byte offsets, constant over the tile ---------------------------
  // Activation instruction j covers rows 16j..16j+15: lane L brings row 16j + L/4,
  // logical chunk (L & 3) ^ ((row >> 2) & 3) into LDS slot L. Slots beyond the
  // A_INSTR instructions repeat an earlier instruction (identical bytes to the same
  // place), so every wave issues PER loads per stage.
  // blocked: stage s of the tile's rows starts s * n_rows * 64 bytes after row0's first block
  const uint16_t* a_tile = GATHER ? A : BLK ? A + static_cast<int64_t>(row0) * 32 : A + static_cast<int64_t>(row0) * K;
  const uint32_t a_bytes =
      GATHER ? ar.a_bytes
      : BLK  ? static_cast<uint32_t>(ar.n_rows) * static_cast<uint32_t>(K) * 2u - static_cast<uint32_t>(row0) * 64u
             : static_cast<uint32_t>(rows_valid) * static_cast<uint32_t>(K) * 2u;
  const uint32_t a_stage_bytes = BLK ? static_cast<uint32_t>(ar.n_rows) * 64u : kBK * 2u;
  const uint32_t b_bytes = static_cast<uint32_t>(K) * static_cast<uint32_t>(ldb) * 2u;
  uint32_t a_voff[L::A_PER_WAVE];
  int a_slot[L::A_PER_WAVE];
#pragma unroll
  for (int jj = 0; jj < L::A_PER_WAVE; ++jj) {
    const int j = (wave * L::A_PER_WAVE + jj) % L::A_INSTR;
    a_slot[jj] = j;
    const int r = 16 * j + (lane >> 2);
    const int c = (lane & 3) ^ ((lane >> 4) & 3);
    if (BLK) {
      // rows past the tile's valid rows point past the buffer (zeros)
      a_voff[jj] = r < rows_valid ? static_cast<uint32_t>(r) * 64u + static_cast<uint32_t>(c) * 16u : 0x80000000u;
    } else if (GATHER) {
      // the token's row; rows past the tile's valid rows point past the buffer (zeros)
      const uint32_t src = r < rows_valid ? static_cast<uint32_t>(ar.perm_seg[row0 + r] / ar.k) * static_cast<uint32_t>(K) * 2u
                                          : 0x80000000u;
      a_voff[jj] = src + static_cast<uint32_t>(c) * 16u;
    } else {
      a_voff[jj] = static_cast<uint32_t>(r) * static_cast<uint32_t>(K) * 2u + static_cast<uint32_t>(c) * 16u;
    }
  }
  // Weight instruction j covers RPI k-rows of the stage (2 at BN = 256, 4 at 128):
  // lane L brings k-row RPI j + L / CPR, logical chunk (L % CPR) ^ (4 * (k & 3))
  // (8 columns) into LDS slot L. With SwiGLU the first half of a row's chunks are
  // gate columns and the second half the matching up columns.
  constexpr int CPR = BN / 8, RPI = 64 / CPR;
  uint32_t b_voff[L::B_PER_WAVE];
#pragma unroll
  for (int jj = 0; jj < L::B_PER_WAVE; ++jj) {
    const int j = wave * L::B_PER_WAVE + jj;
    const int kl = RPI * j + lane / CPR;
    const int c = (lane % CPR) ^ (4 * (kl & 3));
    // 8 columns from n0 + 8 * (chunk within its half); past N they would be the
    // next row's (or the up half's) first columns, so they point past the buffer
    // and load zeros without a fetch (the last column block of N = 2880)
    const int cc = SWIGLU && c >= CPR / 2 ? c - CPR / 2 : c;
    const int col = (SWIGLU && c >= CPR / 2 ? N : 0) + n0 + 8 * cc;
    b_voff[jj] = n0 + 8 * cc < N
                     ? (static_cast<uint32_t>(kl) * static_cast<uint32_t>(ldb) + static_cast<uint32_t>(col)) * 2u
                     : 0x80000000u;
  }

  // ---- fragment reads ----------------------------------------------------------------
  const int l31 = lane & 31;
  uint32_t a_rd[2], a_rd_x[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int row = wm * (MI * 32) + l31;
    const int c = (2 * kk + (lane >> 5)) ^ ((l31 >> 2) & 3);
    a_rd[kk] = static_cast<uint32_t>(row * kBK + c * 8) * 2u;
    a_rd_x[kk] = static_cast<uint32_t>((WM * MI * 32 + l31) * kBK + c * 8) * 2u;  // extra row block
  }
  // B-tile column of register slot ni (SwiGLU: slots [0, NI/2) gate, the rest
  // the matching up columns; with one block per wave, waves 0 and 1 take gate
  // blocks and waves 2 and 3 the matching up blocks). In a 288-row tile the
  // second wave row holds its blocks in swapped slots, so that every wave's
  // share of the extra row block uses slot 0 (and X1 = (SwiGLU ? NI/2 : 1) when
  // it takes two): the gate/up pair or plain blocks that the other wave row does
  // not take. With two blocks per wave that share is one block, and under
  // SwiGLU the first wave row holds the gate half and the second the up half.
  constexpr int X1 = SWIGLU ? NI / 2 : 1;
  auto bcol = [&](int ni) {
    constexpr int half = NI / 2;
    if constexpr (SWIGLU && NI == 1) return wn < 2 ? wn * 32 : BN / 2 + (wn - 2) * 32;
    if (L::XR) ni = wm ? (SWIGLU || NI == 2 ? ni ^ 1 : ni ^ 2) : ni;
    if (SWIGLU) return ni < half ? wn * (BN / 2 / WN) + ni * 32 : BN / 2 + wn * (BN / 2 / WN) + (ni - half) * 32;
    return wn * (BN / WN) + ni * 32;
  };
  uint32_t b_rd[NI];
  {
    const int g = lane >> 4, i = lane & 15;
    const int kl = (g >> 1) * 8 + (i >> 2);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = bcol(ni) + (g & 1) * 16 + 4 * (i & 3);
      b_rd[ni] = static_cast<uint32_t>(kl * BN + (((n >> 3) ^ (4 * (kl & 3))) * 8) + (n & 4)) * 2u;
    }
  }
  const uint32_t sA_addr = sA_base, sB_addr = sB_base;
  constexpr int R = L::LDS_READS, NM = L::NMFMA;

  // LDS read number r of a 16-wide K slice kk: r < MI an activation block, then
  // the two 4-k halves of each weight block.
  auto read_one = [&](Frags& f, int buf, auto kk_c, auto r_c) {
    constexpr int kk = decltype(kk_c)::value, r = decltype(r_c)::value;
    if constexpr (r < MI) {
      f.a[r] = ds_read16<r * 2048>(sA_addr + buf * kAStageBytes + a_rd[kk]);
    } else if constexpr (r < MI + L::XR) {
      f.a[MI] = ds_read16<0>(sA_addr + buf * kAStageBytes + a_rd_x[kk]);
    } else {
      constexpr int ni = (r - MI - L::XR) / 2, h = (r - MI - L::XR) % 2;
      f.b[ni][h] = ds_read_tr<kk * 32 * BN + h * 8 * BN>(sB_addr + buf * kBBytes + b_rd[ni]);
    }
  };
  auto tie_frags = [&](Frags& f) {
#pragma unroll
    for (int mi = 0; mi < MI + L::XR; ++mi) tie(f.a[mi]);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      tie(f.b[ni][0]);
      tie(f.b[ni][1]);
    }
  };

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  f32x16_t acc_x[L::MX > 0 ? L::MX : 1];  // this wave's share of the extra row block
#pragma unroll
  for (int x = 0; x < L::MX; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_x[x][r] = 0.f;

  // MFMA number q of a slice: first this wave's share of the extra row block (so
  // that its results, written outside the compiler's view, are next read at least
  // NMFMA - MX MFMAs later, also in the last slice), then row-major over mi, ni.
  auto mfma_one = [&](const Frags& f, auto q_c) {
    constexpr int q = decltype(q_c)::value;
    if constexpr (q < L::MX) {
      // The accumulators are full; these two live in ordinary VGPRs, which the
      // compiler only allocates for an MFMA written out here.
      constexpr int ni = q == 0 ? 0 : X1;
      mfma_in_vgprs(acc_x[q], f.a[MI], join(f.b[ni][0], f.b[ni][1]));
    } else {
      constexpr int mi = (q - L::MX) / NI, ni = (q - L::MX) % NI;
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], join(f.b[ni][0], f.b[ni][1]), acc[mi][ni], 0,
                                                            0, 0);
    }
  };

  // ---- DMA, one instruction at a time -------------------------------------------------
  struct StageLoads {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t la, lb;  // LDS byte addresses of the stage's buffers
  };
  auto stage_loads = [&](int s) {
    const int buf = s % NS;
    const uint32_t a_adv = static_cast<uint32_t>(s) * a_stage_bytes;
    return StageLoads{make_rsrc(reinterpret_cast<const char*>(a_tile) + a_adv, a_bytes - a_adv),
                      make_rsrc(Bexp + static_cast<int64_t>(s) * kBK * ldb,
                                b_bytes - static_cast<uint32_t>(s) * kBK * ldb * 2u),
                      sA_base + buf * kAStageBytes, sB_base + buf * kBBytes};
  };
  // load j of a stage: j < A_PER_WAVE activations, then this wave's B_PER_WAVE weight loads
  auto dma_one = [&](const StageLoads& st, auto j_c) {
    constexpr int j = decltype(j_c)::value;
    if constexpr (j < L::A_PER_WAVE) dma16(st.ra, a_voff[j], st.la + a_slot[j] * 1024);
    else
      dma16<BSTREAM ? kCpolNT : 0>(st.rb, b_voff[j - L::A_PER_WAVE],
                                   st.lb + (wave * L::B_PER_WAVE + (j - L::A_PER_WAVE)) * 1024);
  };

  // ---- pipeline -------------------------------------------------------------------------
  // Stage s lands in buffer s % NS; it is issued NS - 1 stages ahead. When a
  // wave waits for stage s, min(NS - 2, ksteps - 1 - s) later stages of its own
  // loads may still be in flight.
  auto wait_stage = [&](int s) {
    const int after = min(NS - 2, ksteps - 1 - s);
    if constexpr (NS > 4) {
      if (after >= 3) {
        wait_vmcnt<3 * PER>();
        return;
      }
    }
    if (after >= 2) wait_vmcnt<2 * PER>();
    else if (after == 1) wait_vmcnt<PER>();
    else wait_vmcnt<0>();
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;

  // One stage. With a single wave per SIMD, the matrix unit idles whenever the
  // wave stops to issue a burst of other instructions, so every LDS read and
  // every DMA load is issued in the shadow of an MFMA: slice 0 (fragments f0)
  // carries slice 1's reads, one per MFMA; then the stage barrier; slice 1
  // carries the next stage's slice-0 reads, one per MFMA, and the DMA of stage
  // ks + NS, one per two MFMAs.
  Frags f0, f1;
  auto stage = [&](int ks, auto dma_c, auto more_c) {
    constexpr bool DMA = decltype(dma_c)::value, MORE = decltype(more_c)::value;
    const int buf = ks % NS;
    wait_lgkmcnt<0>();  // f0 (read during the previous stage) has landed
    tie_frags(f0);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NM>([&](auto q) {
      mfma_one(f0, q);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(q)::value < R) read_one(f1, buf, K1{}, q);
      __builtin_amdgcn_sched_barrier(0);
    });
    static_for<(NM < R ? NM : R), R>([&](auto r) { read_one(f1, buf, K1{}, r); });
    wait_lgkmcnt<0>();  // this wave's reads of stage ks are complete
    tie_frags(f1);
    if constexpr (MORE) {
      wait_stage(ks + 1);
      __builtin_amdgcn_s_barrier();  // stage ks+1 landed for every wave; nobody reads stage ks any more
    }
    __builtin_amdgcn_sched_barrier(0);
    StageLoads st;
    if constexpr (DMA) st = stage_loads(ks + NS);
    const int nbuf = (ks + 1) % NS;
    static_for<0, NM>([&](auto q_c) {
      constexpr int q = decltype(q_c)::value;
      mfma_one(f1, q_c);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MORE && q < R) read_one(f0, nbuf, K0{}, q_c);
      if constexpr (DMA && q % 2 == 0 && q / 2 < PER) dma_one(st, std::integral_constant<int, q / 2>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (MORE) static_for<(NM < R ? NM : R), R>([&](auto r) { read_one(f0, nbuf, K0{}, r); });
    if constexpr (DMA) static_for<((NM + 1) / 2 < PER ? (NM + 1) / 2 : PER), PER>([&](auto j) { dma_one(st, j); });
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: stages 0..NS-2 in flight, stage 0 landed, stage NS-1
  // issued, slice 0 of stage 0 requested
  for (int s = 0; s < NS - 1 && s < ksteps; ++s) {
    const StageLoads st = stage_loads(s);
    static_for<0, PER>([&](auto j) { dma_one(st, j); });
  }
  wait_stage(0);
  __builtin_amdgcn_s_barrier();
  if (NS - 1 < ksteps) {
    const StageLoads st = stage_loads(NS - 1);
    static_for<0, PER>([&](auto j) { dma_one(st, j); });
  }
  static_for<0, R>([&](auto r) { read_one(f0, 0, K0{}, r); });

  int ks = 0;
  for (; ks + NS < ksteps; ++ks) stage(ks, std::true_type{}, std::true_type{});
  for (; ks + 1 < ksteps; ++ks) stage(ks, std::false_type{}, std::true_type{});
  stage(ks, std::false_type{}, std::false_type{});

  // ---- epilogue: bf16 results through buffer stores over the tile's valid rows --------
  const __amdgpu_buffer_rsrc_t rc_src = make_rsrc(
      C + static_cast<int64_t>(row0) * N, static_cast<uint32_t>(rows_valid) * static_cast<uint32_t>(N) * 2u);
  const uint32_t c_row_bytes = static_cast<uint32_t>(N) * 2u;
  auto col_off = [&](int ni) -> uint32_t {  // output column of register slot ni (gate slot for SwiGLU)
    const int col = n0 + bcol(ni) + l31;
    return col < N ? static_cast<uint32_t>(col) * 2u : 0x80000000u;
  };
  auto store = [&](float v, int row, uint32_t coff) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), rc_src,
                                          static_cast<int>(static_cast<uint32_t>(row) * c_row_bytes + coff), 0, 0);
  };
  auto acc_row = [&](int r) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); };  // row of element r in a block

  // SAVE: the pre-activations go to GU [rows][2 N] (gate columns, then the up
  // columns) as they are read for H, at the output column of the pair: G at
  // column c and U at column N + c of the row.
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(
      SAVE ? GU + static_cast<int64_t>(row0) * 2 * N : GU,
      SAVE ? static_cast<uint32_t>(rows_valid) * static_cast<uint32_t>(N) * 4u : 0u);
  auto save = [&](float v, int row, uint32_t coff, bool up) {
    if constexpr (SAVE) {
      const uint32_t o = coff + (up ? c_row_bytes : 0u);  // an out-of-range coff stays out of range
      __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), rg,
                                            static_cast<int>(static_cast<uint32_t>(row) * 2u * c_row_bytes + o), 0,
                                            0);
    }
  };

  // Where a gate block and its up block sit in different waves (one block per
  // wave; or the shared extra row block of a half-width 288-row tile), the up
  // wave hands its 16 accumulators per lane over through LDS, in the activation
  // buffer the last stages left untouched (stage ksteps - NS's, free since its barrier).
  constexpr bool XCH_MAIN = SWIGLU && NI == 1;
  constexpr bool XCH_X = SWIGLU && L::MX == 1;
  float up_in[16];
  if constexpr (XCH_MAIN || XCH_X) {
    const uint32_t xbyte = (ksteps % NS) * kAStageBytes;
    float* xch = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + xbyte);
    const bool giver = XCH_MAIN ? wn >= 2 : wm == 1;
    const int slot = XCH_MAIN ? (wn & 1) : wn;
    float4* mine = reinterpret_cast<float4*>(xch) + slot * 256 + lane;
    if (giver) {
      const f32x16_t& v = XCH_MAIN ? acc[0][0] : acc_x[0];
#pragma unroll
      for (int j = 0; j < 4; ++j) mine[64 * j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    }
    __syncthreads();
    if (!giver) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 u = mine[64 * j];
        up_in[4 * j] = u.x;
        up_in[4 * j + 1] = u.y;
        up_in[4 * j + 2] = u.z;
        up_in[4 * j + 3] = u.w;
      }
    }
  }

  if constexpr (XCH_MAIN) {  // 32 rows: waves 0 and 1 write silu(gate) * up, waves 2 and 3 keep their up
    if (wn < 2) {
      const uint32_t coff = col_off(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float gv = acc[0][0][r];
        store(silu_fast(gv) * up_in[r], acc_row(r), coff);
        save(gv, acc_row(r), coff, false);
      }
    } else if constexpr (SAVE) {
      const int c = n0 + (wn - 2) * 32 + l31;  // the output column of this up block
      const uint32_t coff = c < N ? static_cast<uint32_t>(c) * 2u : 0x80000000u;
#pragma unroll
      for (int r = 0; r < 16; ++r) save(acc[0][0][r], acc_row(r), coff, true);
    }
  } else if constexpr (SWIGLU && NI == 2 && L::XR) {
    // half-width 288-row tile: the second wave row holds its up block in slot 0
    const int gs = wm;  // gate slot
    const uint32_t coff = col_off(gs);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float a0 = acc[mi][0][r], a1 = acc[mi][1][r];
        const float gv = gs ? a1 : a0, uv = gs ? a0 : a1;
        const int row = wm * (MI * 32) + mi * 32 + acc_row(r);
        store(silu_fast(gv) * uv, row, coff);
        save(gv, row, coff, false);
        save(uv, row, coff, true);
      }
  } else {
    constexpr int kStoreBlocks = SWIGLU ? NI / 2 : NI;
    uint32_t coff[kStoreBlocks];
#pragma unroll
    for (int ni = 0; ni < kStoreBlocks; ++ni) coff[ni] = col_off(ni);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * (MI * 32) + mi * 32 + acc_row(r);
#pragma unroll
        for (int ni = 0; ni < kStoreBlocks; ++ni) {
          if constexpr (SWIGLU) {
            const float gv = acc[mi][ni][r], uv = acc[mi][ni + NI / 2][r];
            store(silu_fast(gv) * uv, row, coff[ni]);
            save(gv, row, coff[ni], false);
            save(uv, row, coff[ni], true);
          } else {
            store(acc[mi][ni][r], row, coff[ni]);
          }
        }
      }
    }
  }
  if constexpr (L::MX > 0) {  // the extra row block (rows WM * MI * 32 ...)
    const int row0x = WM * MI * 32;
    if constexpr (XCH_X) {  // gate half here in the first wave row, up half handed over by the second
      const uint32_t coff = col_off(0);
      if (wm == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          store(silu_fast(acc_x[0][r]) * up_in[r], row0x + acc_row(r), coff);
          save(acc_x[0][r], row0x + acc_row(r), coff, false);
        }
      } else if constexpr (SAVE) {  // slot 0 of the second wave row is the up block of the same columns
        const uint32_t ucoff = col_off(1);
#pragma unroll
        for (int r = 0; r < 16; ++r) save(acc_x[0][r], row0x + acc_row(r), ucoff, true);
      }
    } else if constexpr (SWIGLU) {  // slot 0 with its up pair X1
      const uint32_t coff = col_off(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        store(silu_fast(acc_x[0][r]) * acc_x[1][r], row0x + acc_row(r), coff);
        save(acc_x[0][r], row0x + acc_row(r), coff, false);
        save(acc_x[1][r], row0x + acc_row(r), coff, true);
      }
    } else {  // slots 0 .. MX-1
#pragma unroll
      for (int x = 0; x < L::MX; ++x) {
        const uint32_t coff = col_off(x);
#pragma unroll
        for (int r = 0; r < 16; ++r) store(acc_x[x][r], row0x + acc_row(r), coff);
      }
    }
  }
}

// The tile height for rows_valid rows (a last row tile is the smallest that covers them).
template <bool SWIGLU, int AM, bool SAVE, int BN, bool BSTREAM>
__device__ __forceinline__ void run_tile(uint16_t* smem, const uint16_t* __restrict__ A,
                                         const uint16_t* __restrict__ Bexp, uint16_t* __restrict__ C,
                                         uint16_t* __restrict__ GU, int row0, int rows_valid, int n0, int K, int N,
                                         int ldb, const ARows& ar) {
  if (rows_valid > 256)
    gemm_tile<SWIGLU, AM, SAVE, 288, BN, BSTREAM>(smem, A, Bexp, C, GU, row0, rows_valid, n0, K, N, ldb, ar);
  else if (rows_valid > 128)
    gemm_tile<SWIGLU, AM, SAVE, 256, BN, BSTREAM>(smem, A, Bexp, C, GU, row0, rows_valid, n0, K, N, ldb, ar);
  else if (rows_valid > 64)
    gemm_tile<SWIGLU, AM, SAVE, 128, BN, BSTREAM>(smem, A, Bexp, C, GU, row0, rows_valid, n0, K, N, ldb, ar);
  else if (rows_valid > 32)
    gemm_tile<SWIGLU, AM, SAVE, 64, BN, BSTREAM>(smem, A, Bexp, C, GU, row0, rows_valid, n0, K, N, ldb, ar);
  else
    gemm_tile<SWIGLU, AM, SAVE, 32, BN, BSTREAM>(smem, A, Bexp, C, GU, row0, rows_valid, n0, K, N, ldb, ar);
}

// SAVE: the gate/up launch also writes its pre-activations [G | U] to GU.
template <bool SWIGLU, int AM, bool SAVE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_lds_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    uint16_t* __restrict__ GU, const int32_t* __restrict__ offsets, int e_begin, int e_loc, int K, int N, int ldb,
    int n_max, const int32_t* __restrict__ perm, int k, uint32_t a_bytes, int* __restrict__ xcd_done) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kStages * (kAStageElems + kBStageElems)];
  __shared__ SortedTileMap tm;
  // a remainder of at most 32 rows rides on the expert's last full tile (288 rows)
  build_sorted_tile_map<256, 32>(tm, offsets, e_begin, e_loc, n_max);

  constexpr int kOutCols = SWIGLU ? 128 : 256;
  const int n_tiles = (N + kOutCols - 1) / kOutCols;
  const int total = uniform(tm.mstart[e_loc]) * n_tiles;
  const int64_t b_expert = static_cast<int64_t>(K) * ldb;
  ARows ar{nullptr, k, a_bytes, n_max};
  if (AM == kAGather) ar.perm_seg = perm + offsets[e_begin];

  // Balance: when the last round would keep at most half of the workgroups busy
  // and every expert's tiles have the same height class (so that the rounds
  // before it end together), its tiles are split into half-width tiles, two per
  // tile, and that round takes a little over half as long. With several classes
  // the tiles come tallest class first, so every workgroup's earlier rounds were
  // full-height tiles; there only the last round's tiles of class-0 experts are
  // split, when their halves and the round's other (lighter) tiles still fit in
  // one round (skew256's gate/up: 16 full tiles past four rounds became 32 half
  // tiles beside the 144 light ones). A last column block with at most half of
  // its columns in range is computed as a half-width tile when it has more than
  // 32 rows (a 32-row tile streams weights, and measured no faster at half width).
  const int G = gridDim.x, r = xcd_remap(blockIdx.x, G);
  const int rounds = (total + G - 1) / G;
  const int last = total - (rounds - 1) * G;
  const int tall_last = min(max(uniform(tm.mstart[uniform(tm.tall)]) * n_tiles - (rounds - 1) * G, 0), last);
  const int n_split = uniform(tm.classes) == 1 ? last : tall_last;  // last-round tiles split in two
  const bool split = total > 0 && n_split > 0 && last + n_split <= G;
  const bool narrow_last = N - (n_tiles - 1) * kOutCols <= kOutCols / 2;
  // Pacing (blocked activation rows): the rows of a blocked copy
  // arrive fast enough that the workgroups of one XCD drift apart by more k-steps
  // than its L2 holds, and re-fetch their round's shared rows and weight panels.
  // A workgroup that runs a tile ahead of most of its XCD waits at the tile
  // boundary. xcd_done holds one count per XCD, zeroed by the copy kernel.
  const bool pace = AM == kABlocked && xcd_done != nullptr && (G & 7) == 0;
  const int per_xcd = G >> 3;
  for (int i = 0;; ++i) {
    int tile, part = 0;  // part: 0 the whole tile, 1 or 2 its first or second half
    if (split && i == rounds - 1) {
      const int h = (i & 1) ? G - 1 - r : r;  // items of the round in the snake's direction
      if (h < 2 * n_split) {
        tile = (rounds - 1) * G + (h >> 1);
        part = 1 + (h & 1);
      } else {
        tile = (rounds - 1) * G + n_split + (h - 2 * n_split);
        if (tile >= total) break;
      }
    } else {
      tile = snake_tile(i, r, G);
      if (tile >= total) break;  // later rounds hold only larger ids
    }
    if (pace && i > 0 && uniform(static_cast<int>(threadIdx.x)) < kWave) {
      // this workgroup has finished i tiles: count it, then wait (a bounded number
      // of polls) until all but a quarter of its XCD's workgroups have as well
      int* ctr = xcd_done + (blockIdx.x & 7) * kPaceStride;
      int seen = 0;
      if (lane_id() == 0) seen = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
      seen = __builtin_amdgcn_readfirstlane(seen);
      for (int poll = 0; poll < kPacePolls && seen < i * per_xcd - per_xcd / 4; ++poll) {
        __builtin_amdgcn_s_sleep(4);
        seen = __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
    }
    const SortedTile tc = find_sorted_tile(tm, tile, n_tiles, e_loc);
    const int row0 = uniform(tm.rstart[tc.e]) + tc.mt * 256;
    const int row_end = uniform(tm.rstart[tc.e + 1]);
    const int rows_valid = tc.mt == tc.mt_e - 1 ? row_end - row0 : 256;
    const int n0 = tc.nt * kOutCols + (part == 2 ? kOutCols / 2 : 0);
    if (n0 >= N) break;  // second half of a last column block that is at most half full
    const bool half = part != 0 || (narrow_last && tc.nt == n_tiles - 1 && rows_valid > 32);
    const uint16_t* Bexp = B + static_cast<int64_t>(tc.e) * b_expert;
    // An expert with one row tile reads each weight panel once: stream it past the
    // caches, which then keep the rows and panels that are read again. (Measured:
    // decode256's GEMM 6 % faster, ep8_share128's 1-2 %; on dense8, where four row
    // tiles share each panel, the same policy was 6 % slower.)
    const bool stream = tc.mt_e == 1;
    if (half) {
      if (stream) run_tile<SWIGLU, AM, SAVE, 128, true>(smem, A, Bexp, C, GU, row0, rows_valid, n0, K, N, ldb, ar);
      else run_tile<SWIGLU, AM, SAVE, 128, false>(smem, A, Bexp, C, GU, row0, rows_valid, n0, K, N, ldb, ar);
    } else {
      if (stream) run_tile<SWIGLU, AM, SAVE, 256, true>(smem, A, Bexp, C, GU, row0, rows_valid, n0, K, N, ldb, ar);
      else run_tile<SWIGLU, AM, SAVE, 256, false>(smem, A, Bexp, C, GU, row0, rows_valid, n0, K, N, ldb, ar);
    }
    // every wave has waited for its last LDS reads; the next tile's loads may land
    __builtin_amdgcn_s_barrier();
  }
  // done: no workgroup of this XCD waits for this one any more
  if (pace && threadIdx.x == 0)
    __hip_atomic_fetch_add(xcd_done + (blockIdx.x & 7) * kPaceStride, 1 << 24, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// The local rows of x (row r = x[perm[offsets[e_begin] + r] / k]) into a_blk in
// 32-column blocks of n_max rows (blk_off), for the gate/up launch to read as
// contiguous stages. One 16-byte chunk of 8 columns per thread; eight
// consecutive threads take rows 2m and 2m + 1 of one 32-column block (one
// 128-byte line of the copy), the next eight the next block, so a wave reads two
// whole 512-byte row pieces and writes eight whole lines.
__global__ __launch_bounds__(kThreads) void gather_blocked_kernel(const uint4* __restrict__ x,
                                                                  const int32_t* __restrict__ perm,
                                                                  const int32_t* __restrict__ offsets,
                                                                  uint16_t* __restrict__ a_blk, int e_begin, int e_end,
                                                                  int k, int d, int n_max, int* __restrict__ xcd_done) {
  if (blockIdx.x == 0 && threadIdx.x < 8) xcd_done[threadIdx.x * kPaceStride] = 0;  // for the gate/up launch
  const int seg0 = offsets[e_begin];
  const int n_loc = min(offsets[e_end] - seg0, n_max);
  const int nb = d / 32;
  const int64_t items = static_cast<int64_t>((n_loc + 1) / 2) * nb * 8;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; it < items;
       it += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int sub = static_cast<int>(it & 3), rp = static_cast<int>((it >> 2) & 1);
    const int64_t rest = it >> 3;
    const int m = static_cast<int>(rest / nb), b = static_cast<int>(rest - static_cast<int64_t>(m) * nb);
    const int r = 2 * m + rp;
    if (r < n_loc) {
      const int64_t tok = perm[seg0 + r] / k;
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(a_blk) + blk_off(r, b * 32 + sub * 8, n_max)) =
          x[tok * (d / 8) + b * 4 + sub];
    }
  }
}

}  // namespace

size_t blocked_rows_bytes(int64_t n_max, int d) { return static_cast<size_t>(n_max) * d * 2; }

size_t blocked_rows_workspace_bytes(int64_t n_max, int d) {
  return blocked_rows_bytes(n_max, d) + 8 * kPaceStride * sizeof(int);
}

bool grouped_gemm_blocked_rows(int64_t n_max, int e_loc, int d, int d_ff) {
  // Each gathered row is read by d_ff / 128 gate/up column tiles. Measured (one
  // box): the copy paid on dense8 (112 tiles: gate/up -80 us for a 25 us copy)
  // and ep8_share128 (23: -27 us for 12 us), not on skew256 (16: -67 us for 85
  // us); tiles of few rows (decode) gain nothing. So: at least 20 column tiles,
  // and at least 128 rows per local expert on average (by N_max), for d, d_ff
  // multiples of 32 and a copy addressable in 31 bits.
  return d % 32 == 0 && d_ff % 32 == 0 && d_ff / 128 >= 20 && e_loc > 0 && n_max / e_loc >= 128 &&
         n_max * d * 2 + 64 <= INT32_MAX;
}

hipError_t launch_grouped_gemm_lds(const void* a, const int32_t* perm, int64_t T, int k, const int32_t* offsets,
                                   const void* w_gu, const void* w_dn, void* h, void* y, void* gu, int d, int d_ff,
                                   int e_begin, int e_loc, int64_t n_max, int grid_gate_up, int grid_down,
                                   void* a_blk, hipStream_t stream) {
  const uint16_t* wgu = static_cast<const uint16_t*>(w_gu);
  uint16_t* hh = static_cast<uint16_t*>(h);
  uint16_t* g = static_cast<uint16_t*>(gu);
  const int nm = static_cast<int>(n_max);
  if (perm != nullptr && a_blk != nullptr) {  // rows gathered into a blocked copy first
    int64_t blocks = ((n_max + 1) / 2 * (d / 32) * 8 + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    // the per-XCD tile counts of the pacing follow the copy in the workspace
    int* xcd_done = reinterpret_cast<int*>(static_cast<char*>(a_blk) + blocked_rows_bytes(n_max, d));
    hipLaunchKernelGGL(gather_blocked_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(a), perm, offsets, static_cast<uint16_t*>(a_blk), e_begin,
                       e_begin + e_loc, k, d, nm, xcd_done);
    const uint16_t* ab = static_cast<const uint16_t*>(a_blk);
    if (gu != nullptr)
      hipLaunchKernelGGL((grouped_gemm_lds_kernel<true, kABlocked, true>), dim3(grid_gate_up), dim3(kThreads), 0,
                         stream, ab, wgu, hh, g, offsets, e_begin, e_loc, d, d_ff, 2 * d_ff, nm, nullptr, k, 0u,
                         xcd_done);
    else
      hipLaunchKernelGGL((grouped_gemm_lds_kernel<true, kABlocked, false>), dim3(grid_gate_up), dim3(kThreads), 0,
                         stream, ab, wgu, hh, nullptr, offsets, e_begin, e_loc, d, d_ff, 2 * d_ff, nm, nullptr, k, 0u,
                         xcd_done);
  } else if (perm != nullptr) {  // activation rows gathered from x by perm in the loads
    const uint32_t a_bytes = static_cast<uint32_t>(T * d * 2);
    const uint16_t* x = static_cast<const uint16_t*>(a);
    if (gu != nullptr)
      hipLaunchKernelGGL((grouped_gemm_lds_kernel<true, kAGather, true>), dim3(grid_gate_up), dim3(kThreads), 0,
                         stream, x, wgu, hh, g, offsets, e_begin, e_loc, d, d_ff, 2 * d_ff, nm, perm, k, a_bytes,
                         nullptr);
    else
      hipLaunchKernelGGL((grouped_gemm_lds_kernel<true, kAGather, false>), dim3(grid_gate_up), dim3(kThreads), 0,
                         stream, x, wgu, hh, nullptr, offsets, e_begin, e_loc, d, d_ff, 2 * d_ff, nm, perm, k,
                         a_bytes, nullptr);
  } else {
    hipLaunchKernelGGL((grouped_gemm_lds_kernel<true, kAInOrder, false>), dim3(grid_gate_up), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a), wgu, hh, nullptr, offsets, e_begin, e_loc, d, d_ff, 2 * d_ff,
                       nm, nullptr, k, 0u, nullptr);
  }
  hipLaunchKernelGGL((grouped_gemm_lds_kernel<false, kAInOrder, false>), dim3(grid_down), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_dn),
                     static_cast<uint16_t*>(y), nullptr, offsets, e_begin, e_loc, d_ff, d, d, nm, nullptr, k, 0u,
                     nullptr);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_plain(const void* a, const void* b, void* c, const int32_t* offsets, int e_begin,
                                     int e_loc, int K, int N, int ldb, int64_t n_max, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((grouped_gemm_lds_kernel<false, kAInOrder, false>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), static_cast<uint16_t*>(c),
                     nullptr, offsets, e_begin, e_loc, K, N, ldb, static_cast<int>(n_max), nullptr, 1, 0u, nullptr);
  return hipGetLastError();
}

}  // namespace moe
