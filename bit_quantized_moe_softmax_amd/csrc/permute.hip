// Permute: stable counting sort of the (token, slot) pairs by expert.
//
// Gives each expert a contiguous run of rows, the expert-major order in which the
// Flash-MoE runtime streams only the routed experts ("Hy4-preview Flash-MoE STQ1_0",
// expert-major sidecar).  Pairs go in chunks of 1024; within a chunk each pair's rank among
// equal experts comes from wave ballots (same-expert lanes found bit by bit) plus per-wave
// counts in LDS -- the output order is fixed by the pair index, never by atomics.
// Up to 8191 pairs one workgroup of 16 waves does everything (LDS histogram, block scan,
// then the chunks in turn).  From 8192 pairs the chunks run in parallel, in four launches
// that use the outputs as scratch (chunks x E <= P is required, so E <= 1024 fits): (1) one
// workgroup per chunk counts its pairs per expert into sorted_pair; (2) one workgroup sums
// the counts into the expert offsets and each chunk's first position per expert, written
// into pair_pos; (3) one workgroup per chunk places its pairs into sorted_pair; (4) pair_pos
// from sorted_pair, -1 for unrouted pairs and past the routed positions.
// A pair whose expert id lies outside [0, E) (an expert with no slot, or a corrupted id) is
// not routed: it gets pair_pos -1, takes no sorted position (offsets[E] counts only the
// routed pairs), and sorted_pair is -1 from offsets[E] on.  No id is used as an index
// before that check.
#include "moe_device.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxE = 1024;

__global__ __launch_bounds__(kThreads) void permute_kernel(const int32_t* __restrict__ ids,
                                                           int P, int E, int nbits,
                                                           int32_t* __restrict__ sorted_pair,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ pair_pos) {
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_base[kMaxE];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_routed;
  __shared__ uint8_t s_wc[kWaves][kMaxE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;

  for (int e = tid; e < E; e += kThreads) s_cnt[e] = 0;
  __syncthreads();
  for (int f = tid; f < P; f += kThreads) {
    const int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();

  // exclusive scan of s_cnt[0..E) (E <= 1024: one value per thread)
  {
    const int c = tid < E ? s_cnt[tid] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wsum[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int w2 = 0; w2 < wv; ++w2) before += s_wsum[w2];
    const int excl = before + incl - c;
    if (tid < E) {
      s_base[tid] = excl;
      offsets[tid] = excl;
    }
    if (tid == E - 1) {
      offsets[E] = excl + c;
      s_routed = excl + c;
    }
  }
  __syncthreads();
  for (int pos = s_routed + tid; pos < P; pos += kThreads) sorted_pair[pos] = -1;

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < P; c0 += kThreads) {
    // clear the per-wave counts of this chunk
    for (int i = tid; i < kWaves * E; i += kThreads) s_wc[i / E][i % E] = 0;
    __syncthreads();
    const int f = c0 + tid;
    const int ef = f < P ? ids[f] : -1;
    const bool valid = ef >= 0 && ef < E;
    const int e = valid ? ef : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      peers &= bit ? ones : ~ones;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) s_wc[wv][e] = (uint8_t)__popcll(peers);
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w2 = 0; w2 < wv; ++w2) pre += s_wc[w2][e];
      const int pos = s_base[e] + pre + rank;
      sorted_pair[pos] = f;
      pair_pos[f] = pos;
    } else if (f < P) {
      pair_pos[f] = -1;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += kThreads) {
      int s = 0;
      for (int w2 = 0; w2 < kWaves; ++w2) s += s_wc[w2][e2];
      s_base[e2] += s;
    }
    __syncthreads();
  }
}

// ---- the parallel path (P >= kParMin, chunks x E <= P)
constexpr int kParMin = 8192;

// (1) counts of chunk c per expert -> cnt[c E + e]
__global__ __launch_bounds__(kThreads) void permute_count_kernel(const int32_t* __restrict__ ids, int P,
                                                                 int E, int32_t* __restrict__ cnt) {
  __shared__ int s_cnt[kMaxE];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < E; e += kThreads) s_cnt[e] = 0;
  __syncthreads();
  const int f = c * kThreads + tid;
  if (f < P) {
    const int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) cnt[(size_t)c * E + e] = s_cnt[e];
}

// (2) one workgroup, thread e: offsets[e] (exclusive scan of the experts' totals) and
// base[c E + e] = offsets[e] + the pairs of expert e in chunks before c
__global__ __launch_bounds__(kThreads) void permute_scan_kernel(const int32_t* __restrict__ cnt, int nch,
                                                                int E, int32_t* __restrict__ base,
                                                                int32_t* __restrict__ offsets) {
  __shared__ int s_wsum[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // the counts of 8 chunks are loaded together: one memory round trip per 8 chunks
  constexpr int kB = 8;
  auto batch = [&](int c0, int* v) {
#pragma unroll
    for (int j = 0; j < kB; ++j) v[j] = c0 + j < nch ? cnt[(size_t)(c0 + j) * E + tid] : 0;
  };
  int c_tot = 0;
  if (tid < E)
    for (int c0 = 0; c0 < nch; c0 += kB) {
      int v[kB];
      batch(c0, v);
#pragma unroll
      for (int j = 0; j < kB; ++j) c_tot += v[j];
    }
  int incl = c_tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_wsum[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w2 = 0; w2 < wv; ++w2) before += s_wsum[w2];
  const int excl = before + incl - c_tot;
  if (tid < E) {
    offsets[tid] = excl;
    int run = excl;
    for (int c0 = 0; c0 < nch; c0 += kB) {
      int v[kB];
      batch(c0, v);
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        if (c0 + j < nch) base[(size_t)(c0 + j) * E + tid] = run;
        run += v[j];
      }
    }
  }
  if (tid == E - 1) offsets[E] = excl + c_tot;
}

// (3) chunk c: each routed pair's sorted position = its chunk's base for the expert + the
// pairs of the same expert before it in the chunk
__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(const int32_t* __restrict__ ids, int P,
                                                                   int E, int nbits,
                                                                   const int32_t* __restrict__ base,
                                                                   int32_t* __restrict__ sorted_pair) {
  __shared__ int s_base[kMaxE];
  __shared__ uint8_t s_wc[kWaves][kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, c = blockIdx.x;
  for (int e = tid; e < E; e += kThreads) s_base[e] = base[(size_t)c * E + e];
  for (int i = tid; i < kWaves * E; i += kThreads) s_wc[i / E][i % E] = 0;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int f = c * kThreads + tid;
  const int ef = f < P ? ids[f] : -1;
  const bool valid = ef >= 0 && ef < E;
  const int e = valid ? ef : 0;
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t ones = __ballot(valid && bit);
    peers &= bit ? ones : ~ones;
  }
  const int rank = __popcll(peers & lt_mask);
  if (valid && rank == 0) s_wc[wv][e] = (uint8_t)__popcll(peers);
  __syncthreads();
  if (valid) {
    int pre = 0;
    for (int w2 = 0; w2 < wv; ++w2) pre += s_wc[w2][e];
    sorted_pair[s_base[e] + pre + rank] = f;
  }
}

// (4) pair_pos from sorted_pair; -1 for unrouted pairs and for sorted positions past the
// routed ones (each entry of either output is written once)
__global__ __launch_bounds__(256) void permute_finish_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                             const int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_pair,
                                                             int32_t* __restrict__ pair_pos) {
  const int routed = offsets[E];
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < P; i += gridDim.x * blockDim.x) {
    if (i < routed) pair_pos[sorted_pair[i]] = i;
    else sorted_pair[i] = -1;
    const int e = ids[i];
    if (e < 0 || e >= E) pair_pos[i] = -1;
  }
}

}  // namespace

hipError_t moe_launch_permute(const int32_t* ids, int P, int E, int32_t* sorted_pair,
                              int32_t* offsets, int32_t* pair_pos, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const long nch = ((long)P + kThreads - 1) / kThreads;
  if (P < kParMin || nch * E > P) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kThreads), 0, s, ids, P, E, nbits,
                       sorted_pair, offsets, pair_pos);
    return hipGetLastError();
  }
  int32_t* cnt = sorted_pair;   // (1) -> (2), consumed before (3) writes sorted_pair
  int32_t* base = pair_pos;     // (2) -> (3), consumed before (4) writes pair_pos
  hipLaunchKernelGGL(permute_count_kernel, dim3((unsigned)nch), dim3(kThreads), 0, s, ids, P, E, cnt);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kThreads), 0, s, cnt, (int)nch, E, base, offsets);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)nch), dim3(kThreads), 0, s, ids, P, E, nbits,
                     base, sorted_pair);
  const long nb = ((long)P + 255) / 256;
  hipLaunchKernelGGL(permute_finish_kernel, dim3((unsigned)(nb < 4096 ? nb : 4096)), dim3(256), 0, s, ids,
                     P, E, offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}
