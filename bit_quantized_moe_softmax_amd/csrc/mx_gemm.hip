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
// of at most 128 rows, evenly (150 pairs -> 75 + 75).  A job is (M block, N tile of 256
// weight rows): for gate/up 128 gate rows + the 128 up rows of the same h-columns, for down
// 256 output columns.  Jobs are numbered expert-major, then by N tile, then by M block, and
// the jobs of one XCD are one contiguous range (workgroup b runs on XCD b % 8): the blocks
// of an expert that read the same weight tile run side by side, and the N tiles that share
// an M block's activation rows run close together, behind one L2.  The kernel is
// persistent: one workgroup per CU takes its XCD's jobs in turn, decoding each from job
// tables built once in LDS.
//
// Tiling.  Four waves share the M block's activation rows, staged per K step (128) in LDS
// (double-buffered, rows padded against bank conflicts).  Each wave owns 64 weight rows and
// keeps their E2M1 codes in registers, loaded straight from HBM four K steps ahead: every
// weight byte is used by exactly one wave, so it never passes through LDS.  Per K step a
// wave issues up to 8 x 4 MFMAs (16-row tiles past the block's last pair are skipped).
//
// Weight layouts.  Row-major MXFP4 (codes [rows][K/2], scales [rows][K/32]) has each wave
// read 64 bytes from each of 16 rows K/2 bytes apart per K step: half a cache line per row,
// the other half a step later, which scatters the weight stream over DRAM pages.  The tiled
// layout (moe_mxfp4_pack_tiles) stores the same bytes in the order the MFMA consumes them:
// per 16-row tile and K step one 1 KiB block whose 16 bytes at 16 l are lane l's operand
// (row l % 16, K bytes 16 (l / 16) .. + 15 of the step), and one 64-byte scale block (4 bytes
// per row, byte g = scale of the step's K block g).  A wave then streams each of its tiles
// as one contiguous run of K/2 * 16 bytes.
//
// Operand layout of the scaled 16x16x128 MFMA (measured with an in-bounds probe on gfx950,
// K counted within the 128-wide step): lane l serves row/column l % 16 and lane group
// g = l / 16.  An E2M1 operand lane holds the 32 consecutive K = 32g .. 32g+31 (16 bytes,
// element 2i in the low nibble); an E4M3 operand lane holds K = 16g .. 16g+15 in bytes
// 0..15 and K = 64+16g .. 64+16g+15 in bytes 16..31.  The scale register of lane l is the
// UE8M0 scale of K block g (K = 32g .. 32g+31) of its row/column, whatever data the lane
// holds.  The MFMA's internal dot products carry about 2^-14 relative error (probe), far
// inside the 2e-3 output tolerance.
#include "moe_device.h"
#include "gemm_jobs.h"

#include <math.h>

namespace {

constexpr int kMT = kMB / 16;   // 16-row MFMA tiles per M block
constexpr int kNWave = 64;      // weight rows per wave
constexpr int kNTile = 4 * kNWave;
constexpr int kBK = 128;        // K per step
constexpr int kAStride = 144;   // bytes per A row in LDS (128 + 16 pad)
constexpr int kRing = 4;       // K steps of loads in flight (register rings)

// Largest value over each 16-lane row of the wave (the 16 columns of one MFMA D row), by
// DPP within the row: swaps of neighbours and pairs, then the half-row and row mirrors.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lanes ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lanes ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

// Two values to E4M3 codes at MX exponent X (bytes 0 and 1 of the result) with the scaled
// hardware conversion, which divides by the scale 2^X and rounds to nearest even.  Inputs are
// clamped to +-448 2^X first: past it the conversion gives the NaN code where the MX rule
// saturates.  For every exponent the rule produces (-127 .. 119) and |v| < 2^(X+9) this
// equals moe_e4m3_code on each value (compared on the GPU over random values, rounding ties,
// tiny values, zeros and the saturating band).
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b, int X) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const float lim = ldexpf(448.0f, X);
  const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((v2s){0, 0}, fminf(fmaxf(a, -lim), lim),
                                                         fminf(fmaxf(b, -lim), lim), ldexpf(1.0f, X), false);
  return (uint16_t)r.x;
}

template <bool GATEUP, bool TILED>
__global__ __launch_bounds__(256, 1) void mx_gemm_kernel(MxArgs p) {
  __shared__ __align__(16) uint8_t s_a[2][kMB * kAStride];
  __shared__ uint32_t s_as[2][256];   // entries >= kMB are written, never read
  __shared__ int s_arow[kMB];
  __shared__ JobTable s_jt;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int K = p.K, N = p.N;
  const int NT = GATEUP ? N / (kNTile / 2) : (N + kNTile - 1) / kNTile;

  if (wave == 0) build_job_table(p.offsets, p.E, s_jt, lane);
  __syncthreads();
  // Persistent: the jobs of XCD x are one contiguous range, taken by its workgroups in turn,
  // so the N tiles that share an M block's activation rows run together behind one L2.
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

  // ---- A staging: thread covers 16-byte chunk (tid & 7) of rows (tid >> 3) + 32 i
  const int achunk = tid & 7;
  const rsrc_t ra_q = make_rsrc(p.aq, (uint32_t)((GATEUP ? p.T : p.P) * (size_t)K));
  const rsrc_t ra_s = make_rsrc(p.as, (uint32_t)((GATEUP ? p.T : p.P) * (size_t)(K / 32)));
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int src = s_arow[(tid >> 3) + 32 * i];
    aoff[i] = src >= 0 ? (uint32_t)src * K + 16 * achunk : kOOB;
  }
  const int srow = s_arow[tid & (kMB - 1)];   // threads >= kMB load a scale word they never store
  const uint32_t asoff = srow >= 0 ? (uint32_t)srow * (K / 32) : kOOB;

  // ---- this wave's weight rows: 4 n-tiles of 16 (gate/up: gate, gate, up, up)
  const int g = lane >> 4, c16 = lane & 15;
  const int col0 = GATEUP ? jb.ntile * (kNTile / 2) + 32 * wave   // first of 32 h-columns
                          : jb.ntile * kNTile + kNWave * wave;    // first of 64 output columns
  const bool wvalid = GATEUP || col0 < N;
  const size_t ebytes = (size_t)N * (K / 2), escales = (size_t)N * (K / 32);
  const rsrc_t rb0 = make_rsrc(p.wcodes0 + jb.e * ebytes, (uint32_t)ebytes);
  const rsrc_t rs0 = make_rsrc(p.wscales0 + jb.e * escales, (uint32_t)escales);
  const rsrc_t rb1 = GATEUP ? make_rsrc(p.wcodes1 + jb.e * ebytes, (uint32_t)ebytes) : rb0;
  const rsrc_t rs1 = GATEUP ? make_rsrc(p.wscales1 + jb.e * escales, (uint32_t)escales) : rs0;
  const uint32_t trow = (uint32_t)(wvalid ? col0 : 0);   // first row of the wave's first tile
  const uint32_t brow = trow + c16;
  // per-lane offsets of step 0 of the first tile; per step and tile the SGPR offset adds
  // koff(k0) and qrow(q) rows (a tile of 16 rows is 16 rows in both layouts)
  const uint32_t boff = TILED ? trow * (K / 2) + 16 * lane : brow * (K / 2) + 16 * g;
  const uint32_t bsoff = TILED ? trow * (K / 32) + 4 * c16 : brow * (K / 32);
  auto koff = [](int k0) { return TILED ? k0 * 8 : k0 / 2; };    // 1 KiB or 64 B per step
  auto ksoff = [](int k0) { return TILED ? k0 / 2 : k0 / 32; };  // 64 B or 4 B per step
  // n-tile q starts qrow(q) rows after the lane's first row
  auto qrow = [](int q) { return GATEUP ? 16 * (q & 1) : 16 * q; };

  // Register rings: A(s) is loaded kRing - 1 steps before it is stored to LDS (at the end of
  // step s - 1), B(s) kRing steps before step s uses it.  Slot of step s: s % kRing.
  uint4 ra[kRing][4];
  uint32_t ras[kRing];
  auto load_a = [&](int slot, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[slot][i] = bload16(ra_q, aoff[i], k0);
    ras[slot] = bload4(ra_s, asoff, k0 / 32);
  };
  auto store_a = [&](int slot, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&s_a[buf][((tid >> 3) + 32 * i) * kAStride + 16 * achunk]) = ra[slot][i];
    s_as[buf][tid] = ras[slot];   // unconditional: keeps the load from sinking into a branch
  };

  uint4 rb[kRing][4];
  uint32_t rbs[kRing][4];
  auto load_b = [&](int slot, int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool hi = GATEUP && q >= 2;
      rb[slot][q] = bload16(hi ? rb1 : rb0, boff, qrow(q) * (K / 2) + koff(k0));
      rbs[slot][q] = bload4(hi ? rs1 : rs0, bsoff, qrow(q) * (K / 32) + ksoff(k0));
    }
  };

  f32x4_t acc[kMT][4];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int mtiles = (nrows + 15) >> 4;

  auto compute = [&](int buf, int slot) {
    i32x8_t bop[4];
    int bsc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = rb[slot][q];
      bop[q] = (i32x8_t){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      bsc[q] = (rbs[slot][q] >> (8 * g)) & 0xFF;
    }
    const uint8_t* sa = s_a[buf];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt < mtiles) {
        const int arow = 16 * mt + c16;
        const uint4 v0 = *reinterpret_cast<const uint4*>(&sa[arow * kAStride + 16 * g]);
        const uint4 v1 = *reinterpret_cast<const uint4*>(&sa[arow * kAStride + 64 + 16 * g]);
        const i32x8_t aop = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                             (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        const int asc = (s_as[buf][arow] >> (8 * g)) & 0xFF;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[mt][q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              aop, bop[q], acc[mt][q], 0 /*A: E4M3*/, 4 /*B: E2M1*/, 0, asc, 0, bsc[q]);
      }
    }
  };

  // Step s: issue A(s + kRing - 1) (its slot held A(s - 1), stored to LDS a step ago), compute
  // from LDS buffer s & 1 and B slot s % kRing, refill that B slot with B(s + kRing), then
  // store A(s + 1) to the other LDS buffer.  Loads complete in issue order, so waiting for
  // A(s + 1) waits for nothing issued in the last kRing - 2 steps.  Past the last step the
  // loads repeat the last step's data, which keeps the code branch-free and the wait counts
  // exact.
  const int nsteps = K / kBK;
  auto step = [&](int s, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    constexpr int AN = (SLOT + kRing - 1) % kRing, A1 = (SLOT + 1) % kRing;
    load_a(AN, min(s + kRing - 1, nsteps - 1) * kBK);
    if (wvalid) compute(s & 1, SLOT);
    load_b(SLOT, min(s + kRing, nsteps - 1) * kBK);
    if (s + 1 < nsteps) store_a(A1, (s + 1) & 1);
    lds_barrier();
  };

#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    load_b(i, min(i, nsteps - 1) * kBK);
    if (i < kRing - 1) load_a(i, min(i, nsteps - 1) * kBK);
    // keep the issue order of the steady state, whose wait counts the loop relies on
    __builtin_amdgcn_sched_barrier(0);
  }
  store_a(0, 0);
  lds_barrier();
  // Whole groups of kRing steps first, with no branch between them: the compiler counts the
  // loads in flight along every path into a wait, and a path that skipped steps would make
  // it wait for loads issued one step earlier instead of kRing.
  int s = 0;
  for (; s + kRing <= nsteps; s += kRing) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
    step(s + 2, std::integral_constant<int, 2>{});
    step(s + 3, std::integral_constant<int, 3>{});
  }
  if (s < nsteps) step(s, std::integral_constant<int, 0>{});
  if (s + 1 < nsteps) step(s + 1, std::integral_constant<int, 1>{});
  if (s + 2 < nsteps) step(s + 2, std::integral_constant<int, 2>{});
  if (wvalid) {
  // ---- epilogue.  D element (4*(lane/16)+i, lane%16) of each 16x16 tile is acc[..][..][i].
  if (GATEUP) {
    const int I = N;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt >= mtiles) continue;
      // the four rows of this lane group first, so their reductions overlap
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
        const float h[2] = {hh[i][0], hh[i][1]};
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
            const uint32_t q = e4m3_pair(h[0], h[1], X);
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
  __syncthreads();   // s_arow and the LDS buffers are reused by the next job
  }   // jobs
}

// Grid: enough workgroups for the most jobs any routing of P pairs over E experts makes
// (sum over active experts of ceil(cnt / 128) <= min(P, E) + ceil(P / 128)), rounded up to
// a multiple of the XCD count so that every XCD's job range fits.
inline unsigned grid_for(const MxArgs& a, int NT) {
  const long slots = (a.P < a.E ? a.P : a.E) + (a.P + kMB - 1) / kMB;
  const long work = slots * NT;
  const long most = kXcd * ((work + kXcd - 1) / kXcd);
  // persistent: one workgroup per CU (the kernel holds one per CU), in whole XCD groups
  static int n_cu[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (n_cu[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    n_cu[dev] = n;
  }
  const long per = kXcd * ((n_cu[dev] + kXcd - 1) / kXcd);
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

hipError_t moe_launch_mx_gateup(const MxArgs& a, hipStream_t s) {
  if (a.N % (kNTile / 2) || a.K % kBK) return hipErrorInvalidValue;
  const int NT = a.N / (kNTile / 2);
  if (a.tiled)
    hipLaunchKernelGGL((mx_gemm_kernel<true, true>), dim3(grid_for(a, NT)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<true, false>), dim3(grid_for(a, NT)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t moe_launch_mx_down(const MxArgs& a, hipStream_t s) {
  if (a.N % kNWave || a.K % kBK) return hipErrorInvalidValue;
  const int NT = (a.N + kNTile - 1) / kNTile;
  if (a.tiled)
    hipLaunchKernelGGL((mx_gemm_kernel<false, true>), dim3(grid_for(a, NT)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<false, false>), dim3(grid_for(a, NT)), dim3(256), 0, s, a);
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
