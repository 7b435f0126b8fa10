// Pieces shared by the persistent grouped GEMMs of the prefill regime: buffer loads,
// an LDS-only barrier, and the job tables that split each expert's pairs into M blocks.
#pragma once

#include "moe_device.h"

namespace {

constexpr int kMB = 128;        // max pairs per M block
constexpr int kXcd = 8;

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past every record: loads read 0

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// voff: per-lane byte offset; soff: a wave-uniform byte offset kept in an SGPR
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Workgroup barrier that orders LDS only: __syncthreads() also fences global memory, which
// would wait for every weight load in flight at each K step.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct Job {
  int e, m0, nrows, ntile;
};

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int blocks_of(int cnt) { return (cnt + kMB - 1) / kMB; }

constexpr int kMaxE = 1024;

// Per-workgroup job tables in LDS, built once: the expert offsets, and nb[e] = M blocks of
// the experts before e (nb[E] = all blocks).
struct JobTable {
  int off[kMaxE + 1];
  int nb[kMaxE + 1];
};

// Wave 0 builds the tables (the caller synchronises before use).
__device__ void build_job_table(const int32_t* __restrict__ off, int E, JobTable& t, int lane) {
  int run = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const int o0 = e < E ? off[e] : 0, o1 = e < E ? off[e + 1] : 0;
    const int nb = e < E ? blocks_of(o1 - o0) : 0;
    const int incl = wave_incl_scan(nb, lane);
    if (e < E) {
      t.off[e] = o0;
      t.nb[e + 1] = run + incl;
    }
    run += __shfl(incl, 63, 64);
  }
  if (lane == 0) {
    t.off[E] = off[E];
    t.nb[0] = 0;
  }
}

// Job w (< all blocks x NT).  Expert e owns jobs nb[e] NT .. nb[e + 1] NT - 1, ordered by N
// tile, then M block: the blocks of one expert that read the same weight tile are
// neighbours, run together, and the second read of the tile hits L2.  The expert is found
// by binary search over nb (every thread, same result).
__device__ __forceinline__ Job decode_job(const JobTable& t, int E, int NT, long w) {
  Job jb;
  int lo = 0, hi = E;   // the largest e with nb[e] NT <= w (then nb[e + 1] NT > w)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((long)t.nb[mid] * NT <= w) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int nbs = t.nb[e + 1] - t.nb[e];
  const int local = (int)(w - (long)t.nb[e] * NT);
  jb.ntile = local / nbs;
  const int mb = local % nbs;
  const int c = t.off[e + 1] - t.off[e];
  const int r0 = (int)((long)c * mb / nbs), r1 = (int)((long)c * (mb + 1) / nbs);
  jb.e = e;
  jb.m0 = t.off[e] + r0;
  jb.nrows = r1 - r0;
  return jb;
}

}  // namespace
