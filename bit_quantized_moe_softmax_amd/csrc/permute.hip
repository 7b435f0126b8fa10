// Permute: stable counting sort of the (token, slot) pairs by expert.
//
// Gives each expert a contiguous run of rows, the expert-major order in which the
// Flash-MoE runtime streams only the routed experts ("Hy4-preview Flash-MoE STQ1_0",
// expert-major sidecar).  One workgroup of 16 waves: LDS histogram, block scan, then
// chunks of 1024 pairs where each pair's rank among equal experts comes from wave
// ballots (same-expert lanes found bit by bit) plus per-wave counts in LDS -- the
// output order is fixed by the pair index, never by atomics.
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

}  // namespace

hipError_t moe_launch_permute(const int32_t* ids, int P, int E, int32_t* sorted_pair,
                              int32_t* offsets, int32_t* pair_pos, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kThreads), 0, s, ids, P, E, nbits,
                     sorted_pair, offsets, pair_pos);
  return hipGetLastError();
}
