// Token dispatch on one rank: per-expert histogram, prefix-sum offsets, stable
// permutation of (token, expert) pairs, and the gather of local rows.
//
// What is computed follows "Paralelismo de especialistas" (transformers v5.23.0,
// pt): section "Despacho de tokens" (each (token, expert) pair goes to the rank
// owning the expert, which computes only its own experts) and section "Como os
// tamanhos se combinam" (a rank owns one contiguous block of experts, so its
// pairs are one contiguous segment of the expert-sorted pair list).
//
// Design (four small launches, all bounded by the pair count or HBM):
//   1. count   : one workgroup per chunk of kDispatchChunk flat pairs builds an
//                LDS histogram and stores it expert-major: ws[e * n_chunks + c].
//   2. scan    : one workgroup scans ws in place (exclusive, expert-major). Entry
//                (e, c) becomes the first sorted slot of chunk c's pairs of
//                expert e; counts and offsets fall out of the same scan.
//   3. scatter : each chunk walks its pairs in order, 256 at a time. A wave
//                finds the lanes holding the same expert with a ballot loop;
//                the rank among them is a popcount, and per-wave counts in LDS
//                order the waves. Slot = chunk base + running count + rank, so
//                the order inside an expert is the flat-pair order (stable).
//   4. gather  : one wave per local row copies x[token] into x_perm with 16-byte
//                loads and stores; the row count is read on the device.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                                  int32_t* __restrict__ ws,
                                                                  int64_t P, int E, int n_chunks) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kDispatchChunk;
  for (int i = threadIdx.x; i < kDispatchChunk; i += kThreads) {
    const int64_t p = base + i;
    if (p < P) {
      const int e = idx[p];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads)
    ws[static_cast<int64_t>(e) * n_chunks + blockIdx.x] = hist[e];
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void dispatch_scan_kernel(int32_t* __restrict__ ws,
                                                                     int32_t* __restrict__ counts,
                                                                     int32_t* __restrict__ offsets,
                                                                     int E, int n_chunks) {
  __shared__ int part[kScanThreads];
  __shared__ int off_s[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int64_t L = static_cast<int64_t>(E) * n_chunks;
  const int64_t per = (L + kScanThreads - 1) / kScanThreads;
  const int64_t b = tid * per;
  const int64_t end = b + per < L ? b + per : L;
  int s = 0;
  for (int64_t i = b; i < end; ++i) s += ws[i];
  part[tid] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;  // exclusive prefix of this thread's range
  for (int64_t i = b; i < end; ++i) {
    const int v = ws[i];
    if (i % n_chunks == 0) off_s[i / n_chunks] = run;
    ws[i] = run;
    run += v;
  }
  if (tid == kScanThreads - 1) off_s[E] = part[kScanThreads - 1];
  if (n_chunks == 0)
    for (int e = tid; e <= E; e += kScanThreads) off_s[e] = 0;
  __syncthreads();
  for (int e = tid; e < E; e += kScanThreads) {
    offsets[e] = off_s[e];
    counts[e] = off_s[e + 1] - off_s[e];
  }
  if (tid == 0) offsets[E] = off_s[E];
}

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ ws,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ pair_pos, int64_t P, int E, int n_chunks, int e_begin, int e_end) {
  constexpr int kWaves = kThreads / kWave;
  __shared__ int run[kMaxExperts];            // pairs of each expert placed so far by this chunk
  __shared__ int wcnt[kWaves][kMaxExperts];   // per-wave counts of the current pass
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const int chunk = blockIdx.x;
  const int seg0 = offsets[e_begin];
  const uint64_t lt_mask = (uint64_t{1} << lane) - 1;
  for (int e = tid; e < E; e += kThreads) run[e] = 0;

  for (int pass = 0; pass < kDispatchChunk / kThreads; ++pass) {
    for (int i = tid; i < kWaves * E; i += kThreads) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int64_t p = static_cast<int64_t>(chunk) * kDispatchChunk + pass * kThreads + tid;
    int e = -1;
    bool valid = false;
    if (p < P) {
      e = idx[p];
      valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
      if (!valid) pair_pos[p] = -1;
    }
    // lanes of this wave holding the same expert (ballot loop over distinct ids)
    uint64_t remaining = __ballot(valid);
    uint64_t peers = 0;
    while (remaining) {
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int le = __shfl(e, leader);
      const uint64_t m = __ballot(valid && e == le);
      if (valid && e == le) peers = m;
      remaining &= ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wv][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = ws[static_cast<int64_t>(e) * n_chunks + chunk] + run[e] + rank;
      for (int w2 = 0; w2 < wv; ++w2) pos += wcnt[w2][e];
      perm[pos] = static_cast<int32_t>(p);
      pair_pos[p] = (e >= e_begin && e < e_end) ? pos - seg0 : -1;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kThreads) {
      int add = 0;
      for (int w2 = 0; w2 < kWaves; ++w2) add += wcnt[w2][x];
      run[x] += add;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void dispatch_gather_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, uint4* __restrict__ x_perm, int e_begin, int e_end, int k,
    int row_vec, int n_max) {
  const int seg0 = offsets[e_begin];
  // rows past n_max (only reachable when topk_idx repeats an id in a token) are dropped
  const int n_loc = min(offsets[e_end] - seg0, n_max);
  const int lane = lane_id();
  const int nwaves = gridDim.x * (kThreads / kWave);
  for (int r = uniform(blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave); r < n_loc; r += nwaves) {
    const int tok = uniform(perm[seg0 + r] / k);
    const uint4* src = x + static_cast<int64_t>(tok) * row_vec;
    uint4* dst = x_perm + static_cast<int64_t>(r) * row_vec;
    int c = lane;
    for (; c + 3 * kWave < row_vec; c += 4 * kWave) {
      const uint4 a0 = src[c], a1 = src[c + kWave], a2 = src[c + 2 * kWave], a3 = src[c + 3 * kWave];
      dst[c] = a0;
      dst[c + kWave] = a1;
      dst[c + 2 * kWave] = a2;
      dst[c + 3 * kWave] = a3;
    }
    for (; c < row_vec; c += kWave) dst[c] = src[c];
  }
}

}  // namespace

size_t dispatch_workspace_bytes(int64_t T, int k, int E) {
  const int64_t P = T * k;
  const int64_t n_chunks = (P + kDispatchChunk - 1) / kDispatchChunk;
  return static_cast<size_t>(n_chunks * E) * sizeof(int32_t);
}

hipError_t launch_dispatch(const void* x, size_t row_bytes, const int32_t* idx, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* pair_pos, void* x_perm,
                           void* workspace, int64_t T, int k, int E, int e_begin, int e_end,
                           int64_t n_max, hipStream_t stream) {
  const int64_t P = T * k;
  const int n_chunks = static_cast<int>((P + kDispatchChunk - 1) / kDispatchChunk);
  int32_t* ws = static_cast<int32_t*>(workspace);
  if (n_chunks > 0) {
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(n_chunks), dim3(kThreads), 0, stream, idx, ws, P,
                       E, n_chunks);
  }
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, ws, counts,
                     offsets, E, n_chunks);
  if (n_chunks == 0) return hipGetLastError();
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(n_chunks), dim3(kThreads), 0, stream, idx, ws,
                     offsets, perm, pair_pos, P, E, n_chunks, e_begin, e_end);
  const int row_vec = static_cast<int>(row_bytes / 16);
  const int64_t waves_needed = n_max;  // one wave per row at most
  int64_t blocks = (waves_needed + (kThreads / kWave) - 1) / (kThreads / kWave);
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(dispatch_gather_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, static_cast<const uint4*>(x), perm, offsets, static_cast<uint4*>(x_perm),
                     e_begin, e_end, k, row_vec, static_cast<int>(n_max));
  return hipGetLastError();
}

}  // namespace moe
