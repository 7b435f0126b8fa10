// Prefill expert FFN on MXFP4 weights x MX FP8 activations: grouped GEMMs on the gfx950
// scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, A = E4M3, B = E2M1, one UE8M0 scale per
// lane per 32 K), with the SiLU * up epilogue and the FP8 re-quantisation of h fused.
//
// Format: "Hy4-preview-SF-WFP4AFP8" (siliconflow), Quant Diff table -- recipe
// weight_fp4_activation_fp8, group 32, ue8m0 / e4m3; routed experts FP4 E2M1 weights with
// FP8 E4M3 activations (g32).  Every routed linear takes E4M3 activations, so h is
// MX-quantised along I before the down projection.
//
// Work split.  The pairs of one expert (contiguous in sorted order) are cut into M blocks
// of at most 128 rows, evenly (150 pairs -> 75 + 75).  A job is (M block, N tile of 512
// weight rows): for gate/up 256 gate rows + the 256 up rows of the same h-columns, for down
// 512 output columns.  Jobs are numbered expert-major, then by N tile, then by M block, and
// the jobs of one XCD are one contiguous range (workgroup b runs on XCD b % 8): the blocks
// of an expert that read the same weight tile run side by side, and the N tiles that share
// an M block's activation rows run close together, behind one L2.  The kernel is
// persistent: one workgroup of eight waves per CU takes its XCD's jobs in turn, decoding
// each from job tables built once in LDS.
//
// Tiling.  The eight waves share the M block's activation rows, staged per K step (128) in
// LDS; each wave owns 64 weight rows and keeps their E2M1 codes in registers, loaded
// straight from HBM three K steps ahead: every weight byte is used by exactly one wave, so
// it never passes through LDS.  Per K step a wave issues (tiles of the block) x 4 MFMAs;
// the tile count is uniform over a job, and each count has its own straight-line copy of
// the K loop in which tile t + 1's A fragment is read before tile t's MFMAs.  With 128
// accumulators and no staging registers a wave fits 256 registers, two waves per SIMD.
//
// Weight layouts.  Row-major MXFP4 (codes [rows][K/2], scales [rows][K/32]) has each wave
// read 64 bytes from each of 16 rows K/2 bytes apart per K step and n-tile: half a cache
// line per row, the other half a step later, which scatters the weight stream over DRAM
// pages.  The tiled layout (moe_mxfp4_pack_tiles) stores the same bytes in the order the
// MFMA consumes them: per 16-row tile and K step one 1 KiB code block whose 16 bytes at
// 16 l are lane l's operand (row l % 16, K bytes 16 (l / 16) .. + 15 of the step), and one
// 64-byte scale block (4 bytes per row, byte g = scale of the step's K block g).  A wave
// then streams each of its tiles as one contiguous run of K/2 * 16 bytes.
//
// Operand layout of the scaled 16x16x128 MFMA (measured with an in-bounds probe on gfx950,
// K counted within the 128-wide step): lane l serves row/column l % 16 and lane group
// g = l / 16.  An E2M1 operand lane holds the 32 consecutive K = 32g .. 32g+31 (16 bytes,
// element 2i in the low nibble); an E4M3 operand lane holds K = 16g .. 16g+15 in bytes
// 0..15 and K = 64+16g .. 64+16g+15 in bytes 16..31.  The scale register of lane l is the
// UE8M0 scale of K block g (K = 32g .. 32g+31) of its row/column, whatever data the lane
// holds.  The MFMA sums its products at reduced precision: up to about 2^-16 of the sum of
// their magnitudes (median 2^-20) on K = 2048, where a sequential fp32 sum stays below
// 2^-24 (measured against exact sums on the GPU), far inside the 2e-3 output tolerance.
#include "moe_device.h"
#include "gemm_jobs.h"

#include <math.h>

namespace {

constexpr int kMT = kMB / 16;   // 16-row MFMA tiles per M block
constexpr int kNWave = 64;      // weight rows per wave
constexpr int kBK = 128;        // K per step

// Largest value over each 16-lane row of the wave (the 16 columns of one MFMA D row), by
// DPP within the row: swaps of neighbours and pairs, then the half-row and row mirrors.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lanes ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lanes ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

// ---------------------------------------------------------------------------------------
// Activation staging.  A K step's tile (128 rows x 128 E4M3 bytes) goes from memory straight
// into LDS (buffer loads with the LDS flag, 16 bytes per lane, whole 128-byte rows: 8 rows
// per load), without a register ring or LDS stores.  Row r's 16-byte chunk c lands at
// 128 r + 16 (c ^ (r % 8)), so a fragment read (lane l: row l % 16 of its tile, chunks
// l / 16 and 4 + l / 16) spreads over the LDS banks.  Wave w loads tile w and the scale
// words of rows 16 w .. 16 w + 15 (lanes repeat them so every lane's load is unconditional).
// Whole rows per load measured 3-4 % faster than 16 rows x 64 bytes in MFMA operand order.
//
// Three LDS buffers: step s computes from buffer s % 3 while the tiles of steps s + 1 and
// s + 2 are in flight, so a tile has two steps to arrive (the rows come from L2 or the
// Infinity Cache, about a step's time away).  The tile loads are written in inline asm, out
// of the compiler's sight: it treats every LDS-DMA load as a pending write to any LDS
// address and would wait for the newest one before each LDS read, which leaves one step of
// lead whatever the ring depth.  The waits are therefore explicit: vector memory loads
// complete in issue order, and after the tile of step s only the weight loads of step
// s - 1 and the tile of step s + 1 are issued, so step s waits for vmcnt (weight loads +
// tile loads per step) and then meets the other waves at a barrier (their parts of the
// tile), with an acquire fence on LDS only (a release fence would wait for every load in
// flight).  Loads past the last step repeat it, so these counts never change, and an opaque
// use at the end of each job keeps the compiler from dropping those repeated weight loads
// as dead.  The inline asm sets M0, which nothing else in these kernels uses.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS-DMA buffer loads: lane l's 16 (or 4) bytes at voff + soff land at LDS byte
// lds + 16 l (or 4 l).  lds is wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}

constexpr int kRingD = 3;       // K steps of tiles and of weight loads in flight per wave

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <bool GATEUP, bool TILED, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void mx_gemm_kernel(MxArgs p) {
  constexpr int TPW = kMT / NW;        // 16-row A tiles this wave loads
  constexpr int RPW = kMB / NW;        // A rows whose scale words this wave loads
  constexpr int NTW = NW * kNWave;     // weight rows per job
  constexpr int NDMA = 2 * TPW + 1;    // LDS-DMA loads per wave and step
  __shared__ __align__(16) uint8_t s_a[kRingD][kMB * kBK];   // [buf][row][chunk ^ row % 8] 16 B
  __shared__ __align__(16) uint32_t s_as[kRingD][NW][64];    // [buf][wave][lane]
  __shared__ int s_arow[kMB];
  __shared__ JobTable s_jt;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N;
  const int NT = GATEUP ? (N + NTW / 2 - 1) / (NTW / 2) : (N + NTW - 1) / NTW;

  if (wave == 0) build_job_table(p.offsets, p.E, s_jt, lane);
  __syncthreads();
  const long n_work = (long)s_jt.nb[p.E] * NT;
  const int x = blockIdx.x % kXcd, slot = blockIdx.x / kXcd, nslot = gridDim.x / kXcd;
  const long w_lo = n_work * x / kXcd, w_hi = n_work * (x + 1) / kXcd;
  for (long w = w_lo + slot; w < w_hi; w += nslot) {
  const Job jb = decode_job(s_jt, p.E, NT, w);
  const int nrows = jb.nrows;
  if (tid < kMB) {
    int src = -1;
    if (tid < nrows) {
      const int pos = jb.m0 + tid;
      src = GATEUP ? p.sorted_pair[pos] / p.k : pos;
    }
    s_arow[tid] = src;
  }
  __syncthreads();

  // ---- A: this wave loads tiles TPW wave .. TPW wave + TPW - 1 (8 rows of 128 bytes per
  // load) and the scale words of rows RPW wave .. RPW wave + RPW - 1
  const int g = lane >> 4, c16 = lane & 15;
  const rsrc_t ra_q = make_rsrc(p.aq, (uint32_t)((GATEUP ? p.T : p.P) * (size_t)K));
  const rsrc_t ra_s = make_rsrc(p.as, (uint32_t)((GATEUP ? p.T : p.P) * (size_t)(K / 32)));
  uint32_t voff[2 * TPW];   // load i: lane j takes row 8 i + j / 8, chunk (j % 8) ^ (j / 8)
#pragma unroll
  for (int i = 0; i < 2 * TPW; ++i) {
    const int src = s_arow[16 * TPW * wave + 8 * i + (lane >> 3)];
    voff[i] = src >= 0 ? (uint32_t)src * K + 16 * ((lane & 7) ^ (lane >> 3)) : kOOB;
  }
  const int ssrc = s_arow[RPW * wave + (lane % RPW)];
  const uint32_t vsoff = ssrc >= 0 ? (uint32_t)ssrc * (K / 32) : kOOB;
  auto dma_a = [&](int buf, int k0) {
    const uint32_t sq = (uint32_t)__builtin_amdgcn_readfirstlane(k0);
#pragma unroll
    for (int i = 0; i < 2 * TPW; ++i)
      dma16(ra_q, lds_addr(&s_a[buf][(16 * TPW * wave + 8 * i) * 128]), voff[i], sq);
    dma4(ra_s, lds_addr(&s_as[buf][wave][0]), vsoff, sq / 32);
  };

  // ---- this wave's weight rows: 4 n-tiles of 16 (gate/up: gate, gate, up, up)
  const int col0 = GATEUP ? jb.ntile * (NTW / 2) + 32 * wave
                          : jb.ntile * NTW + kNWave * wave;
  // (always true for gate/up, whose N is a multiple of the tile; kept a run-time test there
  // too: the branch keeps the compiler from scheduling the unrolled steps into each other,
  // which spilled)
  const bool wvalid = col0 < N;
  const size_t ebytes = (size_t)N * (K / 2), escales = (size_t)N * (K / 32);
  const rsrc_t rb0 = make_rsrc(p.wcodes0 + jb.e * ebytes, (uint32_t)ebytes);
  const rsrc_t rs0 = make_rsrc(p.wscales0 + jb.e * escales, (uint32_t)escales);
  const rsrc_t rb1 = GATEUP ? make_rsrc(p.wcodes1 + jb.e * ebytes, (uint32_t)ebytes) : rb0;
  const rsrc_t rs1 = GATEUP ? make_rsrc(p.wscales1 + jb.e * escales, (uint32_t)escales) : rs0;
  const uint32_t trow = (uint32_t)(wvalid ? col0 : 0);
  const uint32_t brow = trow + c16;
  // per-lane offsets of step 0 of the first tile; per step and n-tile the SGPR offset adds
  // the step (1 KiB tiled, 64 B row-major) and the n-tile's first row (16 rows in both)
  const uint32_t boff = TILED ? trow * (K / 2) + 16 * lane : brow * (K / 2) + 16 * g;
  const uint32_t bsoff = TILED ? trow * (K / 32) + 4 * c16 : brow * (K / 32);
  auto qrow = [](int q) { return GATEUP ? 16 * (q & 1) : 16 * q; };
  auto qoff = [&](int q, int k0) { return qrow(q) * (K / 2) + (TILED ? 8 * k0 : k0 / 2); };
  auto qsoff = [&](int q, int k0) { return qrow(q) * (K / 32) + (TILED ? k0 / 2 : k0 / 32); };
  constexpr int NBL = 8;   // weight loads per wave and step: 4 code pieces + 4 scale words

  uint4 rb[kRingD][4];
  uint32_t rbs[kRingD][4];
  auto load_b = [&](int slot, int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool hi = GATEUP && q >= 2;
      rb[slot][q] = bload16(hi ? rb1 : rb0, boff, qoff(q, k0));
      rbs[slot][q] = bload4(hi ? rs1 : rs0, bsoff, qsoff(q, k0));
    }
  };
  // the UE8M0 scale of n-tile q for this lane (row c16, K block g of the step)
  auto bscale = [&](int slot, int q) { return (int)((rbs[slot][q] >> (8 * g)) & 0xFF); };

  f32x4_t acc[kMT][4];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int mtiles = (nrows + 15) >> 4;

  auto compute = [&](int buf, int slot, auto mtc) {
    constexpr int MTC = decltype(mtc)::value;
    i32x8_t bop[4];
    int bsc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = rb[slot][q];
      bop[q] = (i32x8_t){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      bsc[q] = bscale(slot, q);
    }
    const uint8_t* sa = s_a[buf];
    auto afrag = [&](int mt, i32x8_t& aop, int& asc) {
      // row 16 mt + c16, K bytes 16 g and 64 + 16 g of the step (chunks g and 4 + g, stored
      // at chunk ^ (row % 8))
      const uint8_t* rp = sa + (16 * mt + c16) * 128;
      const uint4 v0 = *reinterpret_cast<const uint4*>(rp + 16 * (g ^ (c16 & 7)));
      const uint4 v1 = *reinterpret_cast<const uint4*>(rp + 16 * ((4 + g) ^ (c16 & 7)));
      aop = (i32x8_t){(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      const int arow = 16 * mt + c16;
      asc = (s_as[buf][arow / RPW][arow % RPW] >> (8 * g)) & 0xFF;
    };
    // MTC tiles, known at compile time: tile mt + 1's fragment read is issued before tile
    // mt's MFMAs, and no further ahead
    i32x8_t an;
    int ascn;
    afrag(0, an, ascn);
#pragma unroll
    for (int mt = 0; mt < MTC; ++mt) {
      const i32x8_t aop = an;
      const int asc = ascn;
      if (mt + 1 < MTC) afrag(mt + 1, an, ascn);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[mt][q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            aop, bop[q], acc[mt][q], 0 /*A: E4M3*/, 4 /*B: E2M1*/, 0, asc, 0, bsc[q]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nsteps = K / kBK;
  // Step s: wait for this wave's part of tile s, meet the other waves, compute from buffer
  // s % kRingD and weight slot s % kRingD, refill that slot with step s + kRingD, then load
  // tile s + 2 into buffer (s + 2) % kRingD (read last at step s - 1, before the barrier).
  auto step = [&](int s, auto slot_c, auto mtc) {
    constexpr int SLOT = decltype(slot_c)::value;
    if (s == 0) wait_vmcnt<NDMA>();   // behind tile 0: tile 1
    else wait_vmcnt<NBL + NDMA>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    __builtin_amdgcn_sched_barrier(0);
    if (wvalid) compute(SLOT, SLOT, mtc);
    __builtin_amdgcn_sched_barrier(0);
    load_b(SLOT, min(s + kRingD, nsteps - 1) * kBK);
    __builtin_amdgcn_sched_barrier(0);
    dma_a((SLOT + 2) % kRingD, min(s + 2, nsteps - 1) * kBK);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto kloop = [&](auto mtc) {
#pragma unroll
    for (int i = 0; i < kRingD; ++i) {
      load_b(i, min(i, nsteps - 1) * kBK);
      __builtin_amdgcn_sched_barrier(0);
    }
    dma_a(0, 0);
    dma_a(1, min(1, nsteps - 1) * kBK);
    __builtin_amdgcn_sched_barrier(0);
    int s = 0;
    for (; s + kRingD <= nsteps; s += kRingD)
      static_for<0, kRingD>([&](auto i) { step(s + i, i, mtc); });
    static_for<0, kRingD - 1>([&](auto i) { if (s + i < nsteps) step(s + i, i, mtc); });
  };
  // one straight-line copy of the K loop per tile count (the count is uniform over the
  // workgroup): a tile loop with a branch per tile keeps the compiler from reading the
  // fragments ahead and spills at 256 registers
  switch (mtiles) {
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 5: kloop(std::integral_constant<int, 5>{}); break;
    case 6: kloop(std::integral_constant<int, 6>{}); break;
    case 7: kloop(std::integral_constant<int, 7>{}); break;
    default: kloop(std::integral_constant<int, 8>{}); break;
  }
  if (wvalid) {
  if (GATEUP) {
    const int I = N;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt >= mtiles) continue;
      float hh[4][2];
      uint32_t am[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float gv = acc[mt][q][i], uv = acc[mt][q + 2][i];
          hh[i][q] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        }
        am[i] = row16_max(max(__float_as_uint(hh[i][0]) & 0x7FFFFFFFu,
                              __float_as_uint(hh[i][1]) & 0x7FFFFFFFu));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 16 * mt + 4 * g + i;
        const uint32_t amax = am[i];
        if (rl < nrows) {
          const int pos = jb.m0 + rl;
          uint8_t* hrow = p.hq + (size_t)pos * I + col0;
          if (amax == 0) {
            hrow[c16] = 0;
            hrow[c16 + 16] = 0;
            if (c16 == 0) p.hs[(size_t)pos * (I / 32) + col0 / 32] = 0;
          } else {
            const int X = moe_mx_exp(amax);
            const uint32_t q = moe_e4m3_pair_hw(hh[i][0], hh[i][1], X);
            hrow[c16] = (uint8_t)q;
            hrow[c16 + 16] = (uint8_t)(q >> 8);
            if (c16 == 0) p.hs[(size_t)pos * (I / 32) + col0 / 32] = (uint8_t)(X + 127);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt >= mtiles) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 16 * mt + 4 * g + i;
        if (rl < nrows) {
          float* yrow = p.y + (size_t)(jb.m0 + rl) * N + col0 + c16;
#pragma unroll
          for (int q = 0; q < 4; ++q) yrow[16 * q] = acc[mt][q][i];
        }
      }
    }
  }
  }   // wvalid
  // The waits of the K loop count every weight load, including those past the last step,
  // whose data no MFMA uses: this opaque use keeps the compiler from dropping them as dead
  // (it waits for them here, where the barrier below waits for every load anyway).
#pragma unroll
  for (int i = 0; i < kRingD; ++i) {
    uint32_t f = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) f ^= rb[i][q].x ^ rb[i][q].y ^ rb[i][q].z ^ rb[i][q].w ^ rbs[i][q];
    asm volatile("" ::"v"(f));
  }
  __syncthreads();   // s_arow and the LDS buffers are reused by the next job
  }   // jobs
}

// Grid: enough workgroups for the most jobs any routing of P pairs over E experts makes
// (sum over active experts of ceil(cnt / 128) <= min(P, E) + ceil(P / 128)), rounded up to
// a multiple of the XCD count so that every XCD's job range fits.
inline unsigned grid_for(const MxArgs& a, int NT, int per_cu = 1) {
  const long slots = (a.P < a.E ? a.P : a.E) + (a.P + kMB - 1) / kMB;
  const long work = slots * NT;
  const long most = kXcd * ((work + kXcd - 1) / kXcd);
  // persistent: per_cu workgroups per CU (as many as the kernel holds), in whole XCD groups
  static int n_cu[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (n_cu[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    n_cu[dev] = n;
  }
  const long per = kXcd * ((per_cu * n_cu[dev] + kXcd - 1) / kXcd);
  return (unsigned)(most < per ? most : per);
}

// Row-major MXFP4 -> tiled layout.  One thread per 16-byte lane operand: tile t, K step j,
// lane l read row 16 t + l % 16, bytes 64 j + 16 (l / 16) .. + 15; threads with l < 16 also
// move the row's 4 scale bytes of the step.
__global__ __launch_bounds__(256) void mx_pack_tiles_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            long rows, int K,
                                                            uint8_t* __restrict__ tcodes,
                                                            uint8_t* __restrict__ tscales) {
  const int steps = K / kBK;
  const long n = rows / 16 * steps * 64;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const long tj = i >> 6;
    const int j = (int)(tj % steps);
    const long t = tj / steps;
    const long row = 16 * t + (l & 15);
    const uint4 v = *reinterpret_cast<const uint4*>(codes + row * (K / 2) + 64 * j + 16 * (l >> 4));
    *reinterpret_cast<uint4*>(tcodes + 16 * i) = v;
    if (l < 16) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(scales + row * (K / 32) + 4 * j);
      *reinterpret_cast<uint32_t*>(tscales + 4 * (tj * 16 + l)) = w;
    }
  }
}

}  // namespace

constexpr int kNW = 8;   // waves per workgroup

template <bool GATEUP>
static void launch_mx(const MxArgs& a, hipStream_t s) {
  constexpr int NTW = kNW * kNWave;
  const int NT = GATEUP ? (a.N + NTW / 2 - 1) / (NTW / 2) : (a.N + NTW - 1) / NTW;
  const unsigned grid = grid_for(a, NT, 8 / kNW);
  if (a.tiled)
    hipLaunchKernelGGL((mx_gemm_kernel<GATEUP, true, kNW>), dim3(grid), dim3(64 * kNW), 0, s, a);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<GATEUP, false, kNW>), dim3(grid), dim3(64 * kNW), 0, s, a);
}

hipError_t moe_launch_mx_gateup(const MxArgs& a, hipStream_t s) {
  if (a.N % 128 || a.K % kBK) return hipErrorInvalidValue;
  launch_mx<true>(a, s);
  return hipGetLastError();
}

hipError_t moe_launch_mx_down(const MxArgs& a, hipStream_t s) {
  if (a.N % kNWave || a.K % kBK) return hipErrorInvalidValue;
  launch_mx<false>(a, s);
  return hipGetLastError();
}

hipError_t moe_launch_mxfp4_pack_tiles(const uint8_t* codes, const uint8_t* scales, long rows,
                                       int K, uint8_t* tcodes, uint8_t* tscales, hipStream_t s) {
  if (rows % 16 || K % kBK) return hipErrorInvalidValue;
  const long n = rows / 16 * (K / kBK) * 64;
  if (n == 0) return hipSuccess;
  const long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(mx_pack_tiles_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                     dim3(256), 0, s, codes, scales, rows, K, tcodes, tscales);
  return hipGetLastError();
}
