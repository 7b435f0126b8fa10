// Prefill expert FFN on MXFP4 weights x MX FP8 activations: grouped GEMMs on the gfx950
// scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, A = E4M3, B = E2M1, one UE8M0 scale per
// lane per 32 K), with the SiLU * up epilogue and the FP8 re-quantisation of h fused.
//
// Format: "Hy4-preview-SF-WFP4AFP8" (siliconflow), Quant Diff table -- recipe
// weight_fp4_activation_fp8, group 32, ue8m0 / e4m3; routed experts FP4 E2M1 weights with
// FP8 E4M3 activations (g32).  Every routed linear takes E4M3 activations, so h is
// MX-quantised along I before the down projection.
//
// Tiling.  A workgroup (4 waves, 2 x 2) owns up to 128 routed pairs of one expert (the
// pairs are contiguous in sorted order; for gate/up their x rows are gathered by token)
// and 128 weight rows: for gate/up 64 gate + 64 up rows of the same 64 h-columns, for down
// 128 output columns.  Each K step (128) stages the A rows (E4M3, 16 KB) and the weight rows
// (E2M1, 8 KB) plus their scale bytes in LDS (double-buffered, rows padded against bank
// conflicts); each wave then issues 4 x 4 MFMAs from LDS.  16-row MFMA tiles past the
// expert's last pair are skipped.
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

#include <math.h>

namespace {

constexpr int kBM = 128;        // pairs per M block (a workgroup loops over its expert's blocks)
constexpr int kBN = 128;        // weight rows per workgroup
constexpr int kBK = 128;        // K per step
constexpr int kAStride = 144;   // bytes per A row in LDS (128 + 16 pad)
constexpr int kBStride = 80;    // bytes per B row in LDS (64 + 16 pad)

struct __align__(16) Stage {
  uint8_t a[kBM * kAStride];
  uint8_t b[kBN * kBStride];
  uint32_t as[kBM];
  uint32_t bs[kBN];
};


template <bool GATEUP>
__global__ __launch_bounds__(256) void mx_ffn_kernel(MxArgs p) {
  __shared__ Stage st[2];
  __shared__ int s_arow[kBM];     // A source row per local pair (-1: none)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = p.K, N = p.N;

  int start, cnt;
  const int e = moe_find_active_expert(p.offsets, p.E, blockIdx.y, start, cnt);
  if (e < 0) return;
  for (int m0 = blockIdx.z * kBM; m0 < cnt; m0 += kBM * gridDim.z) {
  const int nrows = min(kBM, cnt - m0);
  const int n0 = blockIdx.x * (GATEUP ? kBN / 2 : kBN);   // h-column base (gate/up) or out col

  if (tid < kBM) {
    int src = -1;
    if (tid < nrows) {
      const int pos = start + m0 + tid;
      src = GATEUP ? p.sorted_pair[pos] / p.k : pos;
    }
    s_arow[tid] = src;
  }
  __syncthreads();

  // ---- global -> register staging assignment
  const int ar = tid >> 1, ah = tid & 1;          // A: row, 64-byte half
  const int br = tid >> 1, bh = tid & 1;          // B: row, 32-byte half
  const int asrc = s_arow[ar];
  const uint8_t* aptr = asrc >= 0 ? p.aq + (size_t)asrc * K + 64 * ah : nullptr;
  const uint8_t* asptr = (tid < kBM && s_arow[tid] >= 0) ? p.as + (size_t)s_arow[tid] * (K / 32) : nullptr;
  int wrow;
  const uint8_t* bcodes;
  const uint8_t* bscales;
  if (GATEUP) {
    const bool up = br >= kBN / 2;
    wrow = n0 + (up ? br - kBN / 2 : br);
    bcodes = up ? p.wcodes1 : p.wcodes0;
    bscales = up ? p.wscales1 : p.wscales0;
  } else {
    wrow = n0 + br;
    bcodes = p.wcodes0;
    bscales = p.wscales0;
  }
  const uint8_t* bptr = bcodes + ((size_t)e * N + wrow) * (K / 2) + 32 * bh;
  const uint8_t* bsptr = nullptr;
  if (tid < kBN) {
    int r2 = tid, wr2;
    const uint8_t* bsc = p.wscales0;
    if (GATEUP) {
      const bool up = r2 >= kBN / 2;
      wr2 = n0 + (up ? r2 - kBN / 2 : r2);
      bsc = up ? p.wscales1 : p.wscales0;
    } else {
      wr2 = n0 + r2;
    }
    bsptr = bsc + ((size_t)e * N + wr2) * (K / 32);
  }

  uint4 ra[4], rb[2];
  uint32_t ras = 0, rbs = 0;
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = aptr ? *reinterpret_cast<const uint4*>(aptr + k0 + 16 * i) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) rb[i] = *reinterpret_cast<const uint4*>(bptr + k0 / 2 + 16 * i);
    if (tid < kBM) ras = asptr ? *reinterpret_cast<const uint32_t*>(asptr + k0 / 32) : 0u;
    if (tid < kBN) rbs = *reinterpret_cast<const uint32_t*>(bsptr + k0 / 32);
  };
  auto sstore = [&](Stage& s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&s.a[ar * kAStride + 64 * ah + 16 * i]) = ra[i];
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(&s.b[br * kBStride + 32 * bh + 16 * i]) = rb[i];
    if (tid < kBM) s.as[tid] = ras;
    if (tid < kBN) s.bs[tid] = rbs;
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4, c16 = lane & 15;
  // weight-row (within the B tile) of each of this wave's 4 n-tiles
  int nrow[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (GATEUP) nrow[nt] = (nt < 2 ? 0 : kBN / 2) + 32 * wn + 16 * (nt & 1) + c16;
    else nrow[nt] = 64 * wn + 16 * nt + c16;
  }
  int mtiles = 0;   // valid 16-row tiles of this wave
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    if (64 * wm + 16 * mt < nrows) mtiles = mt + 1;

  const int nsteps = K / kBK;
  gload(0);
  sstore(st[0]);
  __syncthreads();
  for (int ks = 0; ks < nsteps; ++ks) {
    Stage& cur = st[ks & 1];
    if (ks + 1 < nsteps) gload((ks + 1) * kBK);
    i32x8_t bop[4];
    int bsc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const uint4 v = *reinterpret_cast<const uint4*>(&cur.b[nrow[nt] * kBStride + 16 * g]);
      bop[nt] = (i32x8_t){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      bsc[nt] = (cur.bs[nrow[nt]] >> (8 * g)) & 0xFF;
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < mtiles) {
        const int arow = 64 * wm + 16 * mt + c16;
        const uint4 v0 = *reinterpret_cast<const uint4*>(&cur.a[arow * kAStride + 16 * g]);
        const uint4 v1 = *reinterpret_cast<const uint4*>(&cur.a[arow * kAStride + 64 + 16 * g]);
        const i32x8_t aop = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                             (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        const int asc = (cur.as[arow] >> (8 * g)) & 0xFF;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              aop, bop[nt], acc[mt][nt], 0 /*A: E4M3*/, 4 /*B: E2M1*/, 0, asc, 0, bsc[nt]);
      }
    }
    if (ks + 1 < nsteps) {
      sstore(st[(ks + 1) & 1]);
    }
    __syncthreads();
  }

  // ---- epilogue.  D element (4*(lane/16)+i, lane%16) of each 16x16 tile is acc[..][..][i].
  if (GATEUP) {
    const int I = N;
    const int hcol0 = n0 + 32 * wn;             // this wave's 32 h-columns = one MX group
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt >= mtiles) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 64 * wm + 16 * mt + 4 * g + i;
        float h[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float gv = acc[mt][q][i], uv = acc[mt][q + 2][i];
          h[q] = gv / (1.0f + expf(-gv)) * uv;
        }
        uint32_t amax = max(__float_as_uint(h[0]) & 0x7FFFFFFFu, __float_as_uint(h[1]) & 0x7FFFFFFFu);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o, 64));
        if (rl < nrows) {
          const int pos = start + m0 + rl;
          uint8_t* hrow = p.hq + (size_t)pos * I + hcol0;
          if (amax == 0) {
            hrow[c16] = 0;
            hrow[c16 + 16] = 0;
            if (c16 == 0) p.hs[(size_t)pos * (I / 32) + hcol0 / 32] = 0;
          } else {
            const int X = moe_mx_exp(amax);
            hrow[c16] = (uint8_t)moe_e4m3_from_f32(__float_as_uint(h[0]), X);
            hrow[c16 + 16] = (uint8_t)moe_e4m3_from_f32(__float_as_uint(h[1]), X);
            if (c16 == 0) p.hs[(size_t)pos * (I / 32) + hcol0 / 32] = (uint8_t)(X + 127);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt >= mtiles) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 64 * wm + 16 * mt + 4 * g + i;
        if (rl < nrows) {
          float* yrow = p.y + (size_t)(start + m0 + rl) * N + n0 + 64 * wn + c16;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) yrow[16 * nt] = acc[mt][nt][i];
        }
      }
    }
  }
  __syncthreads();   // the next M block reuses s_arow and the stages
  }
}

inline int expert_slots(const MxArgs& a) { return a.P < a.E ? a.P : a.E; }

}  // namespace

hipError_t moe_launch_mx_gateup(const MxArgs& a, hipStream_t s) {
  // N = I (h columns); each workgroup covers 64 h-columns (64 gate + 64 up rows)
  dim3 grid(a.N / (kBN / 2), expert_slots(a), 1);
  hipLaunchKernelGGL((mx_ffn_kernel<true>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t moe_launch_mx_down(const MxArgs& a, hipStream_t s) {
  dim3 grid(a.N / kBN, expert_slots(a), 1);
  hipLaunchKernelGGL((mx_ffn_kernel<false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
