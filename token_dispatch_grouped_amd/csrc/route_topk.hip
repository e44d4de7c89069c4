// Router top-k with softmax over the selected logits, one token per lane group.
//
// What is computed follows "Paralelismo de especialistas" (transformers v5.23.0,
// pt), section "Adicionando uma implementação" (top_k_index / top_k_weights):
// the k largest logits of each token in descending order, equal logits to the
// lower expert id (signed zeros equal), and weights = softmax of those k logits.
//
// Design: G lanes (a power of two, G <= 32) share one token and each lane keeps
// VPL logits in registers, expert e = g + v*G, so a group's loads are contiguous.
// A logit and its id form one 64-bit key (order-preserving float bits << 32 |
// ~id), so "larger value, then lower id" is a plain unsigned max and every key
// is unique. Each lane sorts its keys once (a bitonic network in registers);
// each of the k rounds is then a group maximum of the lanes' largest keys (DPP
// moves inside each 16-lane row, readlane across rows), and the owning lane
// drops its largest key. HBM-bound: T*E*4 bytes read.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t orderable(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_orderable(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// 64-bit DPP move within a row of 16 lanes (every lane reads a lane of its own row).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xF, 0xF,
                                             false);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Maximum over each aligned group of G lanes, returned to every lane of the
// group: DPP steps inside a row of 16, then the row maxima by readlane.
template <int G>
__device__ __forceinline__ uint64_t group_max(uint64_t v) {
  if constexpr (G >= 2) v = umax64(v, dpp_u64<kQuadSwap1>(v));
  if constexpr (G >= 4) v = umax64(v, dpp_u64<kQuadSwap2>(v));
  if constexpr (G >= 8) v = umax64(v, dpp_u64<kRowHalfMirror>(v));
  if constexpr (G >= 16) v = umax64(v, dpp_u64<kRowMirror>(v));
  if constexpr (G >= 32) {
    const uint64_t r01 = umax64(readlane_u64(v, 0), readlane_u64(v, 16));
    const uint64_t r23 = umax64(readlane_u64(v, 32), readlane_u64(v, 48));
    if constexpr (G == 32) v = lane_id() < 32 ? r01 : r23;
    else v = umax64(r01, r23);
  }
  return v;
}

// Hides a key from the optimiser, so that "c ? a[i] : a[j]" on two entries of
// a register array stays a two-way select instead of being rewritten as a
// variable-index extract (a select chain over the whole array).
__device__ __forceinline__ uint64_t opaque64(uint64_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Keys a[0..N) into descending order: a bitonic network with compile-time
// indices, so every key stays in a register.
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&a)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t x = opaque64(a[i]), y = opaque64(a[j]);
          const bool gt = x > y;
          const uint64_t hi = gt ? x : y, lo = gt ? y : x;
          if ((i & size) == 0) {  // descending pair (the final pass, size = N, is descending throughout)
            a[i] = hi;
            a[j] = lo;
          } else {
            a[i] = lo;
            a[j] = hi;
          }
        }
      }
}

// KW: keys a lane keeps after sorting: a lane gives up at most min(k, VPL) keys,
// so with k <= KW or KW = VPL its head after any round < k is among its KW
// largest. KMAX: the largest k the instantiation takes (it sizes the result slots).
template <int G, int VPL, int KW, int KMAX>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ w, int64_t T, int E,
                                                         int k) {
  constexpr int kTokensPerWave = kWave / G;
  constexpr int NS = (KMAX + G - 1) / G;  // result slots per lane: round r goes to lane r % G, slot r / G
  const int lane = lane_id();
  const int g = lane % G;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int64_t t = wave * kTokensPerWave + lane / G;
  const bool active = t < T;

  // All VPL loads are issued before any is used: a lane with nothing to load
  // reads element 0 (T >= 1) and its key is set to zero afterwards, so no load
  // sits behind a branch that would wait for it.
  // When the group's lanes hold exactly a token's row (E = G * VPL, VPL a
  // multiple of 4), lane g takes experts [g * VPL, (g + 1) * VPL) with 16-byte
  // loads (4 % faster on E = 128 and 256 than VPL strided 4-byte loads); which
  // lane holds which expert does not change the result.
  float x[VPL];
  const bool contig = VPL % 4 == 0 && E == G * VPL;
  if (contig) {
#pragma unroll
    for (int q = 0; q < VPL / 4; ++q) {
      const float4 v4 = *reinterpret_cast<const float4*>(logits + (active ? t * E + g * VPL + 4 * q : 0));
      x[4 * q] = v4.x;
      x[4 * q + 1] = v4.y;
      x[4 * q + 2] = v4.z;
      x[4 * q + 3] = v4.w;
    }
  } else {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = g + v * G;
      x[v] = logits[active && e < E ? t * E + e : 0];
    }
  }
  uint64_t key[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = contig ? g * VPL + v : g + v * G;
    const uint64_t kv = (static_cast<uint64_t>(orderable(x[v])) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
    key[v] = active && e < E ? kv : 0;
  }
  sort_desc(key);

  float sel_val[NS];
  int sel_id[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    sel_val[s] = 0.f;
    sel_id[s] = 0;
  }
  float top = 0.f, sum = 0.f;
  for (int r = 0; r < k; ++r) {
    // the group's largest remaining key is the largest of the lanes' heads; its
    // owner (keys are unique) drops its head
    const uint64_t best = group_max<G>(key[0]);
    const bool own = key[0] == best;
#pragma unroll
    for (int i = 0; i + 1 < KW; ++i) key[i] = own ? opaque64(key[i + 1]) : opaque64(key[i]);
    key[KW - 1] = own ? 0 : key[KW - 1];
    const float val = from_orderable(static_cast<uint32_t>(best >> 32));
    const int id = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
    if (r == 0) top = val;
    sum += expf(val - top);
    if (r % G == g) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (s == r / G) {
          sel_val[s] = val;
          sel_id[s] = id;
        }
    }
  }
  if (!active) return;
  const float inv = 1.0f / sum;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int r = s * G + g;
    if (r < k) {
      idx[t * k + r] = sel_id[s];
      w[t * k + r] = expf(sel_val[s] - top) * inv;
    }
  }
}

template <int G, int VPL, int KW, int KMAX>
hipError_t launch_gk(const float* logits, int32_t* idx, float* w, int64_t T, int E, int k, hipStream_t stream) {
  constexpr int kThreads = 256;
  constexpr int64_t kTokensPerBlock = (kThreads / kWave) * (kWave / G);
  const int64_t blocks = (T + kTokensPerBlock - 1) / kTokensPerBlock;
  hipLaunchKernelGGL((route_topk_kernel<G, VPL, KW, KMAX>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, logits, idx, w, T, E, k);
  return hipGetLastError();
}

// k <= 8 (every workload) keeps at most 8 keys per lane after the sort
template <int G, int VPL>
hipError_t launch_g(const float* logits, int32_t* idx, float* w, int64_t T, int E, int k, hipStream_t stream) {
  constexpr int KW8 = VPL < 8 ? VPL : 8;
  if (k <= KW8) return launch_gk<G, VPL, KW8, KW8>(logits, idx, w, T, E, k, stream);
  return launch_gk<G, VPL, VPL, G * VPL>(logits, idx, w, T, E, k, stream);
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int32_t* idx, float* w, int64_t T, int E, int k,
                             hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // G lanes per token, VPL logits per lane (G * VPL >= E). Per token, a round costs
  // about G * (c1 * VPL + c2 * log2 G) lane-slots: the per-lane scan grows with VPL,
  // the group maximum with G log G, so small experts counts take one lane per
  // expert and larger ones 8-32 lanes with more logits each.
  if (E <= 1) return launch_g<1, 1>(logits, idx, w, T, E, k, stream);
  if (E <= 2) return launch_g<2, 1>(logits, idx, w, T, E, k, stream);
  if (E <= 4) return launch_g<4, 1>(logits, idx, w, T, E, k, stream);
  if (E <= 8) return launch_g<8, 1>(logits, idx, w, T, E, k, stream);
  if (E <= 16) return launch_g<8, 2>(logits, idx, w, T, E, k, stream);
  if (E <= 32) return launch_g<8, 4>(logits, idx, w, T, E, k, stream);
  if (E <= 64) return launch_g<8, 8>(logits, idx, w, T, E, k, stream);
  if (E <= 128) return launch_g<16, 8>(logits, idx, w, T, E, k, stream);
  if (E <= 256) return launch_g<16, 16>(logits, idx, w, T, E, k, stream);
  if (E <= 512) return launch_g<16, 32>(logits, idx, w, T, E, k, stream);
  return launch_g<32, 32>(logits, idx, w, T, E, k, stream);
}

}  // namespace moe
