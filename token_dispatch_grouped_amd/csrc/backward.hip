// Backward of the combine and of the router's softmax over the top-k.
//
// What is computed is the chain rule through two steps of "Paralelismo de
// especialistas" (transformers v5.23.0, pt): the combine of section "Despacho de
// tokens" (out[t] = sum_j w[t,j] * y[pair_pos[t*k+j]] over local pairs) and the
// routing weights of section "Adicionando uma implementação" (top_k_weights =
// softmax over the k selected logits):
//   d_y[r]     = w[t,j] * d_out[t]          for the local pair (t, j) at row r
//   d_w[t,j]   = <d_out[t], y[r]>           (0 for a pair that is not local)
//   d_logit[t, idx[t,j]] = w[t,j] * (d_w[t,j] - sum_i w[t,i] * d_w[t,i]), 0 elsewhere
// The selection itself is piecewise constant and passes no gradient.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// One wave per token. Per local slot, one pass over the row: d_y gets w * d_out
// (fp32 product, rounded once), and each lane's part of the dot product is
// summed in a fixed order, so d_w is deterministic. bf16 rows move as 16-byte
// vectors (8 elements per lane and load; d is a multiple of 8), two of them per
// lane in flight per operand.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_backward_kernel(
    const void* __restrict__ d_out, const void* __restrict__ y, const int32_t* __restrict__ pair_pos,
    const float* __restrict__ w, void* __restrict__ d_y, float* __restrict__ d_w, int64_t T, int k, int d,
    int64_t n_max) {
  const int lane = lane_id();
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  for (int64_t t = uniform(static_cast<int>(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave)); t < T;
       t += nwaves) {
    const int64_t pbase = t * k;
    for (int j0 = 0; j0 < k; j0 += kWave) {
      const int j = j0 + lane;
      const int rl = j < k ? pair_pos[pbase + j] : -1;
      const float wl = j < k ? w[pbase + j] : 0.f;
      const bool local = rl >= 0 && rl < n_max;
      if (j < k && !local) d_w[pbase + j] = 0.f;
      uint64_t mask = __ballot(local);
      while (mask) {
        const int src = __ffsll(static_cast<unsigned long long>(mask)) - 1;
        mask &= mask - 1;
        const int64_t r = __builtin_amdgcn_readlane(rl, src);
        const float wj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wl), src));
        float dot = 0.f;
        if (BF16) {
          // 16-byte vectors, kPer per lane per pass; buffers bounded by the row, so
          // lanes past its end load zeros (adding nothing) and their stores drop
          constexpr int kPer = 2;
          const int row_vec = d / 8;
          const uint4* go = static_cast<const uint4*>(d_out) + t * row_vec;
          const uint4* yr = static_cast<const uint4*>(y) + r * row_vec;
          uint4* dy = static_cast<uint4*>(d_y) + r * row_vec;
          for (int c0 = 0; c0 < row_vec; c0 += kPer * kWave) {
            const uint32_t bytes = static_cast<uint32_t>(min(kPer * kWave, row_vec - c0)) * 16u;
            const __amdgpu_buffer_rsrc_t bg = make_rsrc(go + c0, bytes);
            const __amdgpu_buffer_rsrc_t by = make_rsrc(yr + c0, bytes);
            const __amdgpu_buffer_rsrc_t bd = make_rsrc(dy + c0, bytes);
            uint4 gv[kPer], yv[kPer];
#pragma unroll
            for (int q = 0; q < kPer; ++q) gv[q] = buffer_load16(bg, static_cast<uint32_t>(q * kWave + lane) * 16u);
#pragma unroll
            for (int q = 0; q < kPer; ++q) yv[q] = buffer_load16(by, static_cast<uint32_t>(q * kWave + lane) * 16u);
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
              const uint32_t g4[4] = {gv[q].x, gv[q].y, gv[q].z, gv[q].w};
              const uint32_t y4[4] = {yv[q].x, yv[q].y, yv[q].z, yv[q].w};
              uint32_t o4[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float g0 = __uint_as_float(g4[i] << 16), g1 = __uint_as_float(g4[i] & 0xFFFF0000u);
                const float y0 = __uint_as_float(y4[i] << 16), y1 = __uint_as_float(y4[i] & 0xFFFF0000u);
                dot = fmaf(g0, y0, dot);
                dot = fmaf(g1, y1, dot);
                o4[i] = static_cast<uint32_t>(f32_to_bf16_rne(wj * g0)) |
                        (static_cast<uint32_t>(f32_to_bf16_rne(wj * g1)) << 16);
              }
              buffer_store16(make_uint4(o4[0], o4[1], o4[2], o4[3]), bd, static_cast<uint32_t>(q * kWave + lane) * 16u);
            }
          }
        } else {
          const float* go = static_cast<const float*>(d_out) + t * d;
          const float* yr = static_cast<const float*>(y) + r * d;
          float* dy = static_cast<float*>(d_y) + r * d;
          for (int c = lane; c < d; c += kWave) {
            const float g = go[c];
            dot = fmaf(g, yr[c], dot);
            dy[c] = wj * g;
          }
        }
        dot = wave_sum(dot);
        if (lane == src) d_w[pbase + j0 + src] = dot;
      }
    }
  }
}

// One wave per token, the token's gradient row assembled in LDS: zeros, then the
// k selected entries (ids of a token are distinct), then one coalesced copy out.
// Every wave of a block runs the same number of iterations, so the block
// barriers are uniform.
__global__ __launch_bounds__(kThreads) void route_topk_backward_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ w, const float* __restrict__ d_w,
    float* __restrict__ d_logits, int64_t T, int E, int k) {
  __shared__ float rows[kWavesPerBlock][kMaxExperts];
  const int lane = lane_id();
  const int wv = static_cast<int>(threadIdx.x) / kWave;
  float* row = rows[wv];
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock; t0 < T;
       t0 += static_cast<int64_t>(gridDim.x) * kWavesPerBlock) {
    const int64_t t = t0 + wv;
    const bool active = t < T;
    for (int e = lane; e < E; e += kWave) row[e] = 0.f;
    float s = 0.f;
    if (active)
      for (int j = lane; j < k; j += kWave) s = fmaf(w[t * k + j], d_w[t * k + j], s);
    s = wave_sum(s);
    __syncthreads();
    if (active)
      for (int j = lane; j < k; j += kWave) {
        const int e = idx[t * k + j];
        const float wj = w[t * k + j];
        if (e >= 0 && e < E) row[e] = wj * (d_w[t * k + j] - s);
      }
    __syncthreads();
    if (active)
      for (int e = lane; e < E; e += kWave) d_logits[t * E + e] = row[e];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_combine_backward(const void* d_out, const void* y, const int32_t* pair_pos, const float* w,
                                   void* d_y, float* d_w, int64_t T, int k, int d, int64_t n_max, bool bf16,
                                   hipStream_t stream) {
  if (T == 0) return hipSuccess;
  int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 4096) blocks = 4096;
  if (bf16)
    hipLaunchKernelGGL(combine_backward_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                       d_out, y, pair_pos, w, d_y, d_w, T, k, d, n_max);
  else
    hipLaunchKernelGGL(combine_backward_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       stream, d_out, y, pair_pos, w, d_y, d_w, T, k, d, n_max);
  return hipGetLastError();
}

hipError_t launch_route_topk_backward(const int32_t* idx, const float* w, const float* d_w, float* d_logits,
                                      int64_t T, int E, int k, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  int64_t blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(route_topk_backward_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, idx,
                     w, d_w, d_logits, T, E, k);
  return hipGetLastError();
}

}  // namespace moe
