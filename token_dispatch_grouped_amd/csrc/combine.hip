// Weighted combine of the expert outputs back to token order.
//
// What is computed follows "Paralelismo de especialistas" (transformers v5.23.0,
// pt), sections "Despacho de tokens" (results are combined with the routing
// weights) and "Adicionando uma implementação" (the weighted expert output of
// every token the rank holds): out[t] = sum_j w[t,j] * y[pair_pos[t*k+j]] over
// the token's local pairs, in slot order, in fp32; zero if it has none.
//
// Design: one wave per token (grid-stride), or per part of a token's row when
// the batch is short. The token's k row indices and
// weights come in with one vector load (a lane per slot); a ballot gives the
// local slots, visited in slot order through readlane two at a time (both rows'
// loads in flight together), and a token with none writes its zero row
// directly. Each lane owns kChunks 16-byte column chunks per pass; loads and
// stores go through buffer resources bounded by the row, so there is no branch
// between them. HBM-bound: N_loc*d*b read + T*d*b written.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <bool BF16>
struct Vec;

template <>
struct Vec<true> {  // 8 bf16 per 16 bytes
  static constexpr int kN = 8;
  __device__ static void load(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static uint4 store(const float* f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16_rne(f[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16_rne(f[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <>
struct Vec<false> {  // 4 fp32 per 16 bytes
  static constexpr int kN = 4;
  __device__ static void load(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static uint4 store(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

// kChunks: 16-byte chunks per lane per pass over a row (a pass covers kChunks KB).
// A wave takes one part of a token's row (vectors [cb, ce)): the whole row, or,
// for short batches, one of `split` parts of `span` vectors.
template <bool BF16, bool UNIT, int kChunks>
__global__ __launch_bounds__(kThreads) void combine_kernel(const uint4* __restrict__ y,
                                                           const int32_t* __restrict__ pair_pos,
                                                           const float* __restrict__ w,
                                                           uint4* __restrict__ out, int64_t T, int k,
                                                           int row_vec, int64_t n_max, int split, int span) {
  using V = Vec<BF16>;
  const int lane = lane_id();
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  const int64_t items = T * split;
  for (int64_t it = uniform(static_cast<int>(blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave)); it < items;
       it += nwaves) {
    const int64_t t = it / split;
    const int cb = static_cast<int>(it - t * split) * span;
    const int ce = min(row_vec, cb + span);
    // slots j0..j0+63 of this token, one per lane; local ones are visited in slot order
    const int64_t pbase = t * k;
    bool any = false;
    for (int j0 = 0; j0 < k; j0 += kWave) {
      const int j = j0 + lane;
      const int r = j < k ? pair_pos[pbase + j] : -1;
      any = any || __ballot(r >= 0 && r < n_max) != 0;
    }
    uint4* dst = out + t * row_vec;
    if (!any) {
      for (int c = cb + lane; c < ce; c += kWave) dst[c] = make_uint4(0, 0, 0, 0);
      continue;
    }
    for (int c0 = cb; c0 < ce; c0 += kChunks * kWave) {
      // buffers over this block of kChunks * kWave vectors of the part: lanes past
      // its end load zero and their stores are dropped, with no branch
      const uint32_t bytes = static_cast<uint32_t>(min(kChunks * kWave, ce - c0)) * 16u;
      float acc[kChunks][V::kN];
#pragma unroll
      for (int q = 0; q < kChunks; ++q)
#pragma unroll
        for (int i = 0; i < V::kN; ++i) acc[q][i] = 0.f;
      for (int j0 = 0; j0 < k; j0 += kWave) {
        const int j = j0 + lane;
        const int rl = j < k ? pair_pos[pbase + j] : -1;
        const float wl = UNIT ? 1.f : (j < k ? w[pbase + j] : 0.f);
        uint64_t mask = __ballot(rl >= 0 && rl < n_max);
        // local slots two at a time, both rows' loads in flight together, added in slot order
        while (mask) {
          const int s0 = __ffsll(static_cast<unsigned long long>(mask)) - 1;
          mask &= mask - 1;
          const int r0 = __builtin_amdgcn_readlane(rl, s0);
          const float w0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wl), s0));
          const bool two = mask != 0;
          int r1 = 0;
          float w1 = 0.f;
          if (two) {
            const int s1 = __ffsll(static_cast<unsigned long long>(mask)) - 1;
            mask &= mask - 1;
            r1 = __builtin_amdgcn_readlane(rl, s1);
            w1 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wl), s1));
          }
          const __amdgpu_buffer_rsrc_t b0 = make_rsrc(y + static_cast<int64_t>(r0) * row_vec + c0, bytes);
          const __amdgpu_buffer_rsrc_t b1 = make_rsrc(y + static_cast<int64_t>(r1) * row_vec + c0, two ? bytes : 0u);
          // each row of y is read once: streamed past the caches (measured, one box:
          // skew256 78 -> 74.5 us, decode256 7.9 -> 7.3 us, dense8 and ep8_share128 the same)
          uint4 v0[kChunks], v1[kChunks];
#pragma unroll
          for (int q = 0; q < kChunks; ++q)
            v0[q] = buffer_load16<kCpolNT>(b0, static_cast<uint32_t>(q * kWave + lane) * 16u);
#pragma unroll
          for (int q = 0; q < kChunks; ++q)
            v1[q] = buffer_load16<kCpolNT>(b1, static_cast<uint32_t>(q * kWave + lane) * 16u);
          __builtin_amdgcn_sched_barrier(0);  // both rows' loads in flight before the first use
#pragma unroll
          for (int q = 0; q < kChunks; ++q) {
            float f[V::kN];
            V::load(v0[q], f);
#pragma unroll
            for (int i = 0; i < V::kN; ++i) acc[q][i] = fmaf(w0, f[i], acc[q][i]);
          }
          // a select rather than a branch, so the second row's loads are not sunk
          // behind the first row's arithmetic
#pragma unroll
          for (int q = 0; q < kChunks; ++q) {
            float f[V::kN];
            V::load(v1[q], f);
#pragma unroll
            for (int i = 0; i < V::kN; ++i) {
              const float t = fmaf(w1, f[i], acc[q][i]);
              acc[q][i] = two ? t : acc[q][i];
            }
          }
        }
      }
      const __amdgpu_buffer_rsrc_t bd = make_rsrc(dst + c0, bytes);
#pragma unroll
      for (int q = 0; q < kChunks; ++q)
        buffer_store16(V::store(acc[q]), bd, static_cast<uint32_t>(q * kWave + lane) * 16u);
    }
  }
}

}  // namespace

hipError_t launch_combine(const void* y, const int32_t* pair_pos, const float* w, void* out,
                          int64_t T, int k, int d, int64_t n_max, bool bf16, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int row_vec = bf16 ? d / 8 : d / 4;
  // Chunks per lane and pass, by row length (measured, one box, timing each in the
  // layer): rows of more than 8 KB take 8 (skew256's 14 KB rows: 45 us, against
  // 49 with 4 and 56 with 2); 6-8 KB rows take 4 (dense8: 18.7 us against 20.2
  // with 8); shorter rows take 2 (ep8_share128's 5.6 KB: 15.7 us against 17.5):
  // fewer registers, so more of the token waves are resident at once.
  const int chunks = row_vec > 512 ? 8 : row_vec > 384 ? 4 : 2;
  // A short batch (decode) has too few token waves to keep the memory system
  // busy, so its rows are cut into one part per pass, a wave each (decode256:
  // 10.4 -> 7.3 us, decode32 10.2 -> 7.1; dense8's 4096 tokens measured 2 %
  // slower cut, ep8_share128's 8192 the same).
  const int passes = (row_vec + chunks * kWave - 1) / (chunks * kWave);
  const int split = T * passes <= 4096 ? passes : 1;
  const int span = split == 1 ? row_vec : chunks * kWave;
  int64_t blocks = (T * split + (kThreads / kWave) - 1) / (kThreads / kWave);
  if (blocks > 4096) blocks = 4096;
#define MOE_COMBINE_LAUNCH(B, U, C)                                                                          \
  hipLaunchKernelGGL((combine_kernel<B, U, C>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, \
                     static_cast<const uint4*>(y), pair_pos, w, static_cast<uint4*>(out), T, k, row_vec, n_max, split, span)
#define MOE_COMBINE_CHUNKS(B, U)            \
  if (chunks == 8) MOE_COMBINE_LAUNCH(B, U, 8); \
  else if (chunks == 4) MOE_COMBINE_LAUNCH(B, U, 4); \
  else MOE_COMBINE_LAUNCH(B, U, 2)
  // w == nullptr: every local pair has weight 1 (the gradient of the row gather)
  if (bf16) {
    if (w) MOE_COMBINE_CHUNKS(true, false);
    else MOE_COMBINE_CHUNKS(true, true);
  } else {
    if (w) MOE_COMBINE_CHUNKS(false, false);
    else MOE_COMBINE_CHUNKS(false, true);
  }
#undef MOE_COMBINE_CHUNKS
#undef MOE_COMBINE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
