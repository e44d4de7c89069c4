// Token dispatch on one rank: per-expert histogram, prefix-sum offsets, stable
// permutation of (token, expert) pairs, and the gather of local rows.
//
// What is computed follows "Paralelismo de especialistas" (transformers v5.23.0,
// pt): section "Despacho de tokens" (each (token, expert) pair goes to the rank
// owning the expert, which computes only its own experts) and section "Como os
// tamanhos se combinam" (a rank owns one contiguous block of experts, so its
// pairs are one contiguous segment of the expert-sorted pair list).
//
// Design, by the number of flat pairs P = T*k (every path gives the same
// stable permutation; the row gather of moe_dispatch follows as one more launch):
//   P <= 2048  : one workgroup does everything (dispatch_small_kernel);
//   P <= 65536 : one launch, a workgroup per 1024 pairs that counts every pair
//                itself (dispatch_onepass_kernel);
//   P <= 131072: two launches (E < 512), per-chunk histograms of 2048 pairs,
//                then a workgroup per 512 pairs that scans the whole table and
//                places its pairs (dispatch_scan_scatter_kernel);
//   larger     : four launches over per-chunk histograms in the workspace:
//   1. count   : one workgroup per chunk of 256 (or 1024) flat pairs builds an
//                LDS histogram and stores it expert-major: ws[e * n_chunks + c].
//   2. scan    : two launches with one wave per expert: per-expert totals,
//                then counts, offsets and the first sorted slot of chunk c's
//                pairs of expert e, stored chunk-major.
//   3. scatter : each chunk stages its E first slots in LDS and walks its
//                pairs in order, 256 at a time. A wave
//                finds the lanes holding the same expert with a ballot loop;
//                the rank among them is a popcount, and per-wave counts in LDS
//                order the waves. Slot = chunk base + running count + rank, so
//                the order inside an expert is the flat-pair order (stable).
//   4. gather  : one wave per part of a local row copies x[token] into x_perm with 16-byte
//                loads and stores; the row count is read on the device.
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Debug builds (MOE_DEBUG defined) also count the ids outside [0, E): an extra
// histogram row E (bucket E) whose total is the error word at the start of the
// workspace. Release builds drop such ids without counting them.
#ifdef MOE_DEBUG
constexpr int kDebugRows = 1;
#else
constexpr int kDebugRows = 0;
#endif
// ints before the histogram tables: the debug error word, padded to 256 bytes
constexpr int kWsHead = kDebugRows * 64;

// CMAJOR: the table is stored chunk-major, ws[chunk * rows + e], for the
// two-launch path, whose scan reads one expert's counts per thread.
template <int CHUNK, bool CMAJOR = false>
__global__ __launch_bounds__(kThreads) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                                  int32_t* __restrict__ ws,
                                                                  int64_t P, int E, int n_chunks) {
  __shared__ int hist[kMaxExperts + kDebugRows];
  const int rows = E + kDebugRows;
  for (int e = threadIdx.x; e < rows; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * CHUNK;
  for (int i = threadIdx.x; i < CHUNK; i += kThreads) {
    const int64_t p = base + i;
    if (p < P) {
      const int e = idx[p];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&hist[e], 1);
      else if (kDebugRows) atomicAdd(&hist[E], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < rows; e += kThreads)
    ws[CMAJOR ? static_cast<int64_t>(blockIdx.x) * rows + e : static_cast<int64_t>(e) * n_chunks + blockIdx.x] =
        hist[e];
}

constexpr int kScanWavesPerBlock = kThreads / kWave;

// Scan of the (expert, chunk) histogram, in two launches with one wave per
// expert so that every expert's row is read with many loads in flight:
//   totals: tot[e] = sum over chunks of the histogram row of expert e;
//   bases : every workgroup scans the <= 1024 totals in LDS (offsets), then each
//           wave prefix-sums its expert's row and stores the first sorted slot
//           of every (chunk, expert) pair chunk-major, base[c * E + e], so that
//           a scatter workgroup reads its E bases as one contiguous row.
//           Workgroup 0 also writes counts and offsets.
__global__ __launch_bounds__(kThreads) void dispatch_zero_counts_kernel(int32_t* __restrict__ counts,
                                                                        int32_t* __restrict__ offsets,
                                                                        int32_t* __restrict__ err_word, int E) {
  for (int e = threadIdx.x; e <= E; e += kThreads) {
    if (e < E) counts[e] = 0;
    offsets[e] = 0;
  }
  if (kDebugRows && threadIdx.x == 0) err_word[0] = 0;
}

// `rows` is E, or E + 1 in debug builds (the last total is the count of ids
// outside [0, E), and also goes to the error word).
__global__ __launch_bounds__(kThreads) void dispatch_totals_kernel(const int32_t* __restrict__ ws,
                                                                   int32_t* __restrict__ tot,
                                                                   int32_t* __restrict__ err_word, int E,
                                                                   int n_chunks) {
  const int lane = lane_id();
  const int e = blockIdx.x * kScanWavesPerBlock + threadIdx.x / kWave;
  if (e >= E + kDebugRows) return;
  const int32_t* row = ws + static_cast<int64_t>(e) * n_chunks;
  int s = 0;
  for (int c = lane; c < n_chunks; c += kWave) s += row[c];
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) {
    tot[e] = s;
    if (kDebugRows && e == E) err_word[0] = s;
  }
}

__global__ __launch_bounds__(kThreads) void dispatch_bases_kernel(const int32_t* __restrict__ ws,
                                                                  const int32_t* __restrict__ tot,
                                                                  int32_t* __restrict__ base,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets, int E,
                                                                  int n_chunks) {
  __shared__ int off_s[kMaxExperts + 1];
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  if (wv == 0) {
    // the <= 1024 totals: lane L scans the run of kTotRun experts from L * kTotRun
    constexpr int kTotRun = (kMaxExperts + kWave - 1) / kWave;
    const int e0 = lane * kTotRun;
    int v[kTotRun];
#pragma unroll
    for (int i = 0; i < kTotRun; ++i) v[i] = e0 + i < E ? tot[e0 + i] : 0;
    int run = 0;
#pragma unroll
    for (int i = 0; i < kTotRun; ++i) run += v[i];
    int incl = run;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int off_e = incl - run;
#pragma unroll
    for (int i = 0; i < kTotRun; ++i) {
      if (e0 + i < E) {
        off_s[e0 + i] = off_e;
        if (blockIdx.x == 0) {
          offsets[e0 + i] = off_e;
          counts[e0 + i] = v[i];
        }
      }
      off_e += v[i];
    }
    const int all = __shfl(incl, kWave - 1);
    if (lane == 0) {
      off_s[E] = all;
      if (blockIdx.x == 0) offsets[E] = all;
    }
  }
  __syncthreads();
  const int e = blockIdx.x * kScanWavesPerBlock + wv;
  if (e >= E) return;
  const int32_t* row = ws + static_cast<int64_t>(e) * n_chunks;
  int carry = off_s[e];
  // Batches of 64 * kRun chunks: lane L takes the run of kRun consecutive chunks
  // from L * kRun, loads them all before adding, sums its run, and one wave scan
  // of the run sums places every run. A batch costs one load latency and one
  // scan, where a chunk per lane and pass cost one of each per 64 chunks.
  constexpr int kRun = 8;
  for (int b0 = 0; b0 < n_chunks; b0 += kWave * kRun) {
    const int c0 = b0 + lane * kRun;
    int v[kRun];
#pragma unroll
    for (int i = 0; i < kRun; ++i) v[i] = c0 + i < n_chunks ? row[c0 + i] : 0;
    int run = 0;
#pragma unroll
    for (int i = 0; i < kRun; ++i) run += v[i];
    int incl = run;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    int slot = carry + incl - run;  // first sorted slot of chunk c0 for expert e
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      if (c0 + i < n_chunks) base[static_cast<int64_t>(c0 + i) * E + e] = slot;
      slot += v[i];
    }
    carry += __shfl(incl, kWave - 1);
  }
}

template <int CHUNK>
__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ pair_pos, int64_t P, int E, int e_begin, int e_end) {
  constexpr int kWaves = kThreads / kWave;
  constexpr int kPasses = CHUNK / kThreads;
  __shared__ int run[kMaxExperts];            // next sorted slot of each expert for this chunk
  __shared__ int wcnt[kWaves][kMaxExperts];   // per-wave counts of the current pass
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const int chunk = blockIdx.x;
  const int seg0 = offsets[e_begin];
  const uint64_t lt_mask = (uint64_t{1} << lane) - 1;
  // every pass's expert id is loaded up front so the loads overlap
  int ids[kPasses];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int64_t p = static_cast<int64_t>(chunk) * CHUNK + pass * kThreads + tid;
    ids[pass] = p < P ? idx[p] : -1;
  }
  const int32_t* brow = base + static_cast<int64_t>(chunk) * E;
  for (int e = tid; e < E; e += kThreads) run[e] = brow[e];

#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    for (int i = tid; i < kWaves * E; i += kThreads) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int64_t p = static_cast<int64_t>(chunk) * CHUNK + pass * kThreads + tid;
    const int e = ids[pass];
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    if (p < P && !valid) pair_pos[p] = -1;
    // lanes of this wave holding the same expert (ballot loop over distinct ids)
    uint64_t remaining = __ballot(valid);
    uint64_t peers = 0;
    while (remaining) {
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int le = __builtin_amdgcn_readlane(e, leader);  // leader is wave-uniform
      const uint64_t m = __ballot(valid && e == le);
      if (valid && e == le) peers = m;
      remaining &= ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wv][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = run[e] + rank;
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
    __syncthreads();  // wcnt is read above before the next pass clears it
  }
}

// Up to kSmallPairs pairs: the whole dispatch in one workgroup of 1024 threads
// (histogram, scan and the same stable scatter, one pass per 1024 pairs), so a
// decode-sized batch pays one launch instead of four.
constexpr int kSmallThreads = 1024;
constexpr int kSmallPairs = 2048;

__global__ __launch_bounds__(kSmallThreads) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ pair_pos, int32_t* __restrict__ err_word, int P, int E,
    int e_begin, int e_end) {
  constexpr int kWaves = kSmallThreads / kWave;
  constexpr int kPasses = kSmallPairs / kSmallThreads;
  __shared__ int run[kMaxExperts + 1];        // histogram, then the next sorted slot of each expert
  __shared__ int wcnt[kWaves][kMaxExperts];   // per-wave counts of the current pass
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const uint64_t lt_mask = (uint64_t{1} << lane) - 1;
  int ids[kPasses];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int p = pass * kSmallThreads + tid;
    ids[pass] = p < P ? idx[p] : -1;
  }
  __shared__ int bad;  // ids outside [0, E) (debug builds)
  for (int e = tid; e < E; e += kSmallThreads) run[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    if (static_cast<unsigned>(ids[pass]) < static_cast<unsigned>(E)) atomicAdd(&run[ids[pass]], 1);
    else if (kDebugRows && pass * kSmallThreads + tid < P) atomicAdd(&bad, 1);
  }
  __syncthreads();
  if (kDebugRows && tid == 0) err_word[0] = bad;
  if (wv == 0) {  // exclusive scan: counts, offsets, and each expert's first slot
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int v = e < E ? run[e] : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      if (e < E) {
        counts[e] = v;
        offsets[e] = carry + incl - v;
        run[e] = carry + incl - v;
      }
      carry += __shfl(incl, kWave - 1);
    }
    if (lane == 0) {
      offsets[E] = carry;
      run[E] = carry;
    }
  }
  __syncthreads();
  const int seg0 = run[e_begin];  // the first local slot (read before any pass moves run)
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    if (pass * kSmallThreads >= P) break;  // uniform
    for (int i = tid; i < kWaves * E; i += kSmallThreads) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int p = pass * kSmallThreads + tid;
    const int e = ids[pass];
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    if (p < P && !valid) pair_pos[p] = -1;
    uint64_t remaining = __ballot(valid);
    uint64_t peers = 0;
    while (remaining) {
      const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
      const int le = __builtin_amdgcn_readlane(e, leader);
      const uint64_t m = __ballot(valid && e == le);
      if (valid && e == le) peers = m;
      remaining &= ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wv][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = run[e] + rank;
      for (int w2 = 0; w2 < wv; ++w2) pos += wcnt[w2][e];
      perm[pos] = p;
      pair_pos[p] = (e >= e_begin && e < e_end) ? pos - seg0 : -1;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kSmallThreads) {
      int add = 0;
      for (int w2 = 0; w2 < kWaves; ++w2) add += wcnt[w2][x];
      run[x] += add;
    }
    __syncthreads();
  }
}

// Up to kOnePassPairs pairs (more than one workgroup takes): one launch, one
// workgroup of 1024 threads per chunk of 1024 pairs. Every workgroup counts all
// the pairs itself, those before its chunk apart from the rest, so no table of
// chunk counts has to pass between launches; it scans the counts into offsets
// and its chunk's first slots, then places its chunk's pairs with the same
// stable ballot ranking as the other paths (workgroup 0 writes counts and
// offsets). Each workgroup reads all T*k ids from L2, n_chunks * T*k * 4 bytes in
// all; past kOnePassPairs the four-launch path reads less.
constexpr int kOnePassPairs = 65536;

__global__ __launch_bounds__(kSmallThreads) void dispatch_onepass_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ pair_pos, int32_t* __restrict__ err_word, int P, int E,
    int e_begin, int e_end) {
  constexpr int kWaves = kSmallThreads / kWave;
  constexpr int kUnroll = 8;                  // ids per thread in flight while counting
  __shared__ int run[kMaxExperts];            // counts before the chunk, then the chunk's next slot per expert
  __shared__ int rest[kMaxExperts + 1];       // counts from the chunk on, then the offsets
  __shared__ int wcnt[kWaves][kMaxExperts];   // per-wave counts of the chunk's pass
  __shared__ int bad;                         // ids outside [0, E) (debug builds)
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const uint64_t lt_mask = (uint64_t{1} << lane) - 1;
  const int c0 = blockIdx.x * kSmallThreads;  // the chunk's first pair
  const int p = c0 + tid;
  const int e = p < P ? idx[p] : -1;
  for (int x = tid; x < E; x += kSmallThreads) {
    run[x] = 0;
    rest[x] = 0;
  }
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int b = 0; b < P; b += kSmallThreads * kUnroll) {
    int ids[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = b + u * kSmallThreads + tid;
      ids[u] = q < P ? idx[q] : -1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = b + u * kSmallThreads + tid;
      if (static_cast<unsigned>(ids[u]) < static_cast<unsigned>(E)) atomicAdd(q < c0 ? &run[ids[u]] : &rest[ids[u]], 1);
      else if (kDebugRows && q < P) atomicAdd(&bad, 1);
    }
  }
  __syncthreads();
  if (kDebugRows && blockIdx.x == 0 && tid == 0) err_word[0] = bad;
  if (wv == 0) {  // counts and their exclusive scan; run[x] becomes the chunk's first slot of expert x
    int carry = 0;
    for (int x0 = 0; x0 < E; x0 += kWave) {
      const int x = x0 + lane;
      const int before = x < E ? run[x] : 0;
      const int v = x < E ? before + rest[x] : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const int first = carry + incl - v;
      if (x < E) {
        if (blockIdx.x == 0) {
          counts[x] = v;
          offsets[x] = first;
        }
        rest[x] = first;
        run[x] = first + before;
      }
      carry += __shfl(incl, kWave - 1);
    }
    if (lane == 0) {
      rest[E] = carry;
      if (blockIdx.x == 0) offsets[E] = carry;
    }
  }
  for (int i = tid; i < kWaves * E; i += kSmallThreads) wcnt[i / E][i % E] = 0;
  __syncthreads();
  const int seg0 = rest[e_begin];
  const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
  if (p < P && !valid) pair_pos[p] = -1;
  uint64_t remaining = __ballot(valid);
  uint64_t peers = 0;
  while (remaining) {
    const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
    const int le = __builtin_amdgcn_readlane(e, leader);
    const uint64_t m = __ballot(valid && e == le);
    if (valid && e == le) peers = m;
    remaining &= ~m;
  }
  const int rank = __popcll(peers & lt_mask);
  if (valid && rank == 0) wcnt[wv][e] = __popcll(peers);
  __syncthreads();
  if (valid) {
    int pos = run[e] + rank;
    for (int w2 = 0; w2 < wv; ++w2) pos += wcnt[w2][e];
    perm[pos] = p;
    pair_pos[p] = (e >= e_begin && e < e_end) ? pos - seg0 : -1;
  }
}

// Past kOnePassPairs, up to kFusedPairs pairs and kFusedThreads table rows (E,
// plus the debug row): two launches. The count launch
// stores a histogram per chunk of kFusedChunk pairs (at most kWave chunks),
// chunk-major. Then one workgroup per kFusedSub pairs (a quarter of a chunk, so
// that every CU ranks pairs) reads the whole table from L2 (rows x n_chunks x 4
// bytes, 64 KB at E = 256): a thread per expert loads that expert's count in
// every chunk at once and adds them, the total and the part before its chunk.
// It counts the pairs of its chunk before its quarter itself (at most 1536 ids,
// in LDS), scans the totals into offsets (workgroup 0 writes counts and
// offsets) and places its pairs by the same stable ballot ranking as the other
// paths. This folds the totals and bases launches of the larger path into the
// scatter.
constexpr int kFusedChunk = 2048;
constexpr int kFusedSub = 512;
constexpr int kFusedThreads = 512;
constexpr int64_t kFusedPairs = static_cast<int64_t>(kFusedChunk) * kWave;

__global__ __launch_bounds__(kFusedThreads) void dispatch_scan_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ ws, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ pair_pos,
    int32_t* __restrict__ err_word, int P, int E, int n_chunks, int e_begin, int e_end) {
  constexpr int kWaves = kFusedThreads / kWave;
  constexpr int kSubs = kFusedChunk / kFusedSub;     // quarters per chunk
  constexpr int kBefore = kFusedSub * (kSubs - 1) / kFusedThreads;  // ids before the quarter, per thread
  __shared__ int run[kMaxExperts];          // pairs before this quarter, then its next slot per expert
  __shared__ int tot[kMaxExperts + 1];      // the offsets
  __shared__ int wsum[kWaves];              // per-wave sums of the totals
  __shared__ int wcnt[kWaves][kMaxExperts]; // per-wave counts
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const int sub = blockIdx.x;
  const int chunk = sub / kSubs;
  const int c0 = chunk * kFusedChunk;        // the chunk's first pair
  const int q0 = sub * kFusedSub;            // the quarter's first pair
  const uint64_t lt_mask = (uint64_t{1} << lane) - 1;
  const int p = q0 + tid;
  const int e = p < P ? idx[p] : -1;
  int prev[kBefore];                         // ids of the chunk before the quarter
#pragma unroll
  for (int u = 0; u < kBefore; ++u) {
    const int q = c0 + u * kFusedThreads + tid;
    prev[u] = q < q0 ? idx[q] : -1;
  }
  // thread x holds expert x's count in every chunk (rows <= kFusedThreads), loaded
  // with the ids, before the first barrier
  const int rows = E + kDebugRows;
  const int x = tid;
  int v[kWave];
#pragma unroll
  for (int c = 0; c < kWave; ++c) v[c] = x < rows && c < n_chunks ? ws[static_cast<int64_t>(c) * rows + x] : 0;
  if (x < E) run[x] = 0;
  for (int i = tid; i < kWaves * E; i += kFusedThreads) wcnt[i / E][i % E] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kBefore; ++u)
    if (static_cast<unsigned>(prev[u]) < static_cast<unsigned>(E)) atomicAdd(&run[prev[u]], 1);
  int all = 0, before = 0;
#pragma unroll
  for (int c = 0; c < kWave; ++c) {
    all += v[c];
    before += c < chunk ? v[c] : 0;
  }
  if (kDebugRows && x == E && sub == 0) err_word[0] = all;  // ids outside [0, E)
  // exclusive scan of the totals over the workgroup: a scan inside each wave,
  // then the sums of the waves before
  const int cnt = x < E ? all : 0;
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wsum[wv] = incl;
  __syncthreads();
  int first = incl - cnt, grand = 0;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) {
    first += w2 < wv ? wsum[w2] : 0;
    grand += wsum[w2];
  }
  if (x < E) {
    if (sub == 0) {
      counts[x] = cnt;
      offsets[x] = first;
    }
    tot[x] = first;
    run[x] += first + before;  // the quarter's first slot of expert x
  }
  if (x == 0) {
    tot[E] = grand;
    if (sub == 0) offsets[E] = grand;
  }
  __syncthreads();
  const int seg0 = tot[e_begin];
  const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
  if (p < P && !valid) pair_pos[p] = -1;
  uint64_t remaining = __ballot(valid);
  uint64_t peers = 0;
  while (remaining) {
    const int leader = __ffsll(static_cast<unsigned long long>(remaining)) - 1;
    const int le = __builtin_amdgcn_readlane(e, leader);
    const uint64_t m = __ballot(valid && e == le);
    if (valid && e == le) peers = m;
    remaining &= ~m;
  }
  const int rank = __popcll(peers & lt_mask);
  if (valid && rank == 0) wcnt[wv][e] = __popcll(peers);
  __syncthreads();
  if (valid) {
    int pos = run[e] + rank;
    for (int w2 = 0; w2 < wv; ++w2) pos += wcnt[w2][e];
    perm[pos] = p;
    pair_pos[p] = (e >= e_begin && e < e_end) ? pos - seg0 : -1;
  }
}

// Rows are copied in parts of kGatherVec 16-byte vectors (2 per lane), one part
// per wave at a time, so that a few long rows still spread over many waves. Two
// per lane, with more parts and waves, measured faster than 4 or 8 on every
// workload (dense8 21.0 us against 21.5 with 8, skew256 15.0 against 16.7,
// ep8_share128 10.0 against 11.2).
constexpr int kGatherPerLane = 2;
constexpr int kGatherVec = kWave * kGatherPerLane;

__global__ __launch_bounds__(kThreads) void dispatch_gather_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, uint4* __restrict__ x_perm, int e_begin, int e_end, int k,
    int row_vec, int parts, int n_max) {
  const int seg0 = offsets[e_begin];
  // rows past n_max (only reachable when topk_idx repeats an id in a token) are dropped
  const int n_loc = min(offsets[e_end] - seg0, n_max);
  const int lane = lane_id();
  const int nwaves = gridDim.x * (kThreads / kWave);
  const int64_t items = static_cast<int64_t>(n_loc) * parts;
  for (int64_t it = uniform(blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave); it < items; it += nwaves) {
    const int r = static_cast<int>(it / parts);
    const int c0 = static_cast<int>(it - static_cast<int64_t>(r) * parts) * kGatherVec;
    const int tok = uniform(perm[seg0 + r] / k);
    // buffers over the part's vectors of this row: lanes past the row end load zero
    // and their stores are dropped, with no branch between the loads
    const uint32_t bytes = static_cast<uint32_t>(min(kGatherVec, row_vec - c0)) * 16u;
    const __amdgpu_buffer_rsrc_t src = make_rsrc(x + static_cast<int64_t>(tok) * row_vec + c0, bytes);
    const __amdgpu_buffer_rsrc_t dst = make_rsrc(x_perm + static_cast<int64_t>(r) * row_vec + c0, bytes);
    uint4 v[kGatherPerLane];
#pragma unroll
    for (int i = 0; i < kGatherPerLane; ++i) v[i] = buffer_load16(src, static_cast<uint32_t>(i * kWave + lane) * 16u);
#pragma unroll
    for (int i = 0; i < kGatherPerLane; ++i) buffer_store16(v[i], dst, static_cast<uint32_t>(i * kWave + lane) * 16u);
  }
}

}  // namespace

// Pairs per chunk: 256 (one pass of a workgroup, and four times the workgroups of
// 1024-pair chunks), unless the (expert, chunk) tables would pass 4M entries.
int dispatch_chunk(int64_t P, int E) {
  const int64_t n256 = (P + 255) / 256;
  return n256 * E <= (int64_t{1} << 22) ? 256 : 1024;
}

size_t dispatch_workspace_bytes(int64_t T, int k, int E) {
  const int64_t P = T * k;
  const int chunk = dispatch_chunk(P, E);
  const int64_t n_chunks = (P + chunk - 1) / chunk;
  const int64_t rows = E + kDebugRows;
  if (n_chunks == 0) return kWsHead * sizeof(int32_t);
  // (debug: the error word), per-(expert, chunk) counts, per-(chunk, expert) first slots, per-expert totals
  return (kWsHead + static_cast<size_t>(n_chunks * rows) + static_cast<size_t>(n_chunks * E) + rows) *
         sizeof(int32_t);
}

size_t dispatch_debug_word_offset() { return kDebugRows ? 0 : SIZE_MAX; }

// Workspace of the allocation-free dispatch: one array in each GPU's copy of
// the code object, held until the process ends. Every call on a GPU shares it.
static __device__ __align__(256) int32_t scratch[kDispatchScratchBytes / sizeof(int32_t)];

hipError_t dispatch_scratch(void** ptr) {
  // The array's device address on each GPU, looked up once per device with that
  // device current (the host-side name is not a device address).
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_dispatch(const void* x, size_t row_bytes, const int32_t* idx, int32_t* counts,
                           int32_t* offsets, int32_t* perm, int32_t* pair_pos, void* x_perm,
                           void* workspace, int64_t T, int k, int E, int e_begin, int e_end,
                           int64_t n_max, hipStream_t stream) {
  const int64_t P = T * k;
  int32_t* err_word = static_cast<int32_t*>(workspace);  // read by the kernels in debug builds only
  if (P > 0 && P <= kSmallPairs) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kSmallThreads), 0, stream, idx, counts, offsets, perm,
                       pair_pos, err_word, static_cast<int>(P), E, e_begin, e_end);
    if (x_perm == nullptr) return hipGetLastError();
    return launch_gather_rows(x, row_bytes, perm, offsets, x_perm, k, e_begin, e_end, n_max, stream);
  }
  if (P > kSmallPairs && P <= kOnePassPairs) {
    const int blocks = static_cast<int>((P + kSmallThreads - 1) / kSmallThreads);
    hipLaunchKernelGGL(dispatch_onepass_kernel, dim3(blocks), dim3(kSmallThreads), 0, stream, idx, counts, offsets,
                       perm, pair_pos, err_word, static_cast<int>(P), E, e_begin, e_end);
    if (x_perm == nullptr) return hipGetLastError();
    return launch_gather_rows(x, row_bytes, perm, offsets, x_perm, k, e_begin, e_end, n_max, stream);
  }
  int32_t* ws = static_cast<int32_t*>(workspace) + kWsHead;
  if (P > kOnePassPairs && P <= kFusedPairs && E + kDebugRows <= kFusedThreads) {
    const int n_fused = static_cast<int>((P + kFusedChunk - 1) / kFusedChunk);
    hipLaunchKernelGGL((dispatch_count_kernel<kFusedChunk, true>), dim3(n_fused), dim3(kThreads), 0, stream, idx, ws,
                       P, E, n_fused);
    const int n_subs = static_cast<int>((P + kFusedSub - 1) / kFusedSub);
    hipLaunchKernelGGL(dispatch_scan_scatter_kernel, dim3(n_subs), dim3(kFusedThreads), 0, stream, idx, ws, counts,
                       offsets, perm, pair_pos, err_word, static_cast<int>(P), E, n_fused, e_begin, e_end);
    if (x_perm == nullptr) return hipGetLastError();
    return launch_gather_rows(x, row_bytes, perm, offsets, x_perm, k, e_begin, e_end, n_max, stream);
  }
  const int chunk = dispatch_chunk(P, E);
  const int n_chunks = static_cast<int>((P + chunk - 1) / chunk);
  const int rows = E + kDebugRows;
  if (n_chunks > 0) {
    if (chunk == 256)
      hipLaunchKernelGGL(dispatch_count_kernel<256>, dim3(n_chunks), dim3(kThreads), 0, stream, idx, ws, P, E,
                         n_chunks);
    else
      hipLaunchKernelGGL(dispatch_count_kernel<1024>, dim3(n_chunks), dim3(kThreads), 0, stream, idx, ws, P, E,
                         n_chunks);
  }
  int32_t* bases = ws + static_cast<int64_t>(n_chunks) * rows;
  int32_t* tot = bases + static_cast<int64_t>(n_chunks) * E;
  const int scan_blocks = (E + kScanWavesPerBlock - 1) / kScanWavesPerBlock;
  if (n_chunks == 0) {
    // no pairs: counts and offsets are all zero (tot is the E zeros the totals pass would give)
    hipLaunchKernelGGL(dispatch_zero_counts_kernel, dim3(1), dim3(kThreads), 0, stream, counts, offsets, err_word,
                       E);
    return hipGetLastError();
  }
  const int total_blocks = (rows + kScanWavesPerBlock - 1) / kScanWavesPerBlock;
  hipLaunchKernelGGL(dispatch_totals_kernel, dim3(total_blocks), dim3(kThreads), 0, stream, ws, tot, err_word, E,
                     n_chunks);
  hipLaunchKernelGGL(dispatch_bases_kernel, dim3(scan_blocks), dim3(kThreads), 0, stream, ws, tot, bases, counts,
                     offsets, E, n_chunks);
  if (chunk == 256)
    hipLaunchKernelGGL(dispatch_scatter_kernel<256>, dim3(n_chunks), dim3(kThreads), 0, stream, idx, bases, offsets,
                       perm, pair_pos, P, E, e_begin, e_end);
  else
    hipLaunchKernelGGL(dispatch_scatter_kernel<1024>, dim3(n_chunks), dim3(kThreads), 0, stream, idx, bases, offsets,
                       perm, pair_pos, P, E, e_begin, e_end);
  if (x_perm == nullptr) return hipGetLastError();  // indices only: the rows are gathered by the GEMM
  return launch_gather_rows(x, row_bytes, perm, offsets, x_perm, k, e_begin, e_end, n_max, stream);
}

hipError_t launch_gather_rows(const void* x, size_t row_bytes, const int32_t* perm, const int32_t* offsets,
                              void* x_perm, int k, int e_begin, int e_end, int64_t n_max, hipStream_t stream) {
  const int row_vec = static_cast<int>(row_bytes / 16);
  const int parts = (row_vec + kGatherVec - 1) / kGatherVec;
  const int64_t waves_needed = n_max * parts;  // one wave per row part at most
  int64_t blocks = (waves_needed + (kThreads / kWave) - 1) / (kThreads / kWave);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(dispatch_gather_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, static_cast<const uint4*>(x), perm, offsets, static_cast<uint4*>(x_perm),
                     e_begin, e_end, k, row_vec, parts, static_cast<int>(n_max));
  return hipGetLastError();
}

}  // namespace moe
