// Decode-regime expert FFN on the bf16 MFMA: routed STQ1_0 experts (fused in-register
// decode) and the bf16 shared expert.
//
// SwiGLU expert MLP (gate_proj / up_proj / down_proj): h = silu(Wg a) * (Wu a),
// y = Wd h.  STQ1_0 ("Hy4-preview-GGUF" (AngelSlim) section 3, The format;
// "Hy4-preview Flash-MoE STQ1_0", How the STQ1_0 packing works): 256-weight blocks of
// 64 four-weight groups, one zero and three +-d per group, one fp16 d per block.
//
// Work decomposition.  A workgroup owns 16 output rows of one expert and a tile of
// tokens; its waves split the reduction (K) axis and meet in LDS at the end, in a
// fixed order, so results are deterministic.  Each MFMA step is
// v_mfma_f32_16x16x32_bf16: A = 16 weight rows x 32 K, B = 32 K x 16 token columns.
// The ternary weights are exact in bf16 (+-1, 0): a lane turns each 5-bit pattern into
// four bf16 values with one LDS lookup (32-entry table), and the block scale d is
// applied to the per-block fp32 partial sums.  x is bf16 already, so the gate/up
// products are exact and accumulate in fp32.  For the down projection the fp32 h is
// split into bf16 hi + lo (h - hi), two B columns per token, so h keeps ~16 bits.
//
// Lane layout of the 16x16x32 MFMA used here: A row = lane % 16, B column = lane % 16,
// both take 8 consecutive K-slots from slot 8 * (lane / 16); D element (4 * (lane/16) + i,
// lane % 16) sits in accumulator register i.  The K-slot -> K-index map is ours and is
// the same for A and B: for STQ1_0 lane group g covers groups 16g .. 16g+15 of the block
// (8 code bytes + 2 high-bit bytes it loads itself), step t takes groups 16g+2t, 16g+2t+1,
// so K = 256 b + 64 g + 8 t + s; for bf16 weights K = 256 b + 32 t + 8 g + s (64
// contiguous bytes of a row per step).
#include "moe_device.h"

#include <math.h>

namespace {

constexpr int kRows = 16;        // output rows per workgroup
constexpr int kMaxWaveBlocks = 16;

__device__ __forceinline__ uint32_t bf16_of_lane(uint32_t p, int j) {
  const int z = p >> 3;
  if (j == z) return 0u;
  const int i = j < z ? j : j - 1;
  return ((p >> i) & 1) ? 0xBF80u : 0x3F80u;   // -1.0 / +1.0
}

__device__ __forceinline__ void build_lut(uint2* lut) {
  const int t = threadIdx.x;
  if (t < 32) {
    uint2 v;
    v.x = bf16_of_lane(t, 0) | (bf16_of_lane(t, 1) << 16);
    v.y = bf16_of_lane(t, 2) | (bf16_of_lane(t, 3) << 16);
    lut[t] = v;
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A operand of STQ1_0 step t from this lane's 8 code bytes and 16 high bits.
__device__ __forceinline__ bf16x8_t stq_a(const uint2* lut, uint2 qs, uint32_t qh, int t) {
  const uint32_t byte = ((t < 4 ? qs.x : qs.y) >> (8 * (t & 3))) & 0xFFu;
  const uint32_t p0 = (byte & 15u) | (((qh >> (2 * t)) & 1u) << 4);
  const uint32_t p1 = (byte >> 4) | (((qh >> (2 * t + 1)) & 1u) << 4);
  const uint2 l0 = lut[p0];
  const uint2 l1 = lut[p1];
  return as_bf16x8(make_uint4(l0.x, l0.y, l1.x, l1.y));
}

// hi/lo bf16 split of 8 fp32 values: part 0 gives the RNE bf16, part 1 the bf16 of the rest.
__device__ __forceinline__ bf16x8_t split_bf16(const float4 a, const float4 b, int part) {
  float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t hi = f32_to_bf16_rne(v[i]);
    o[i] = part ? f32_to_bf16_rne(v[i] - bf16_to_f32(hi)) : hi;
  }
  return as_bf16x8(make_uint4(o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16),
                              o[6] | (o[7] << 16)));
}

// ------------------------------------------------------------------ gate/up (+ SiLU * up)
// grid: x = row tile (N/16), y = expert slot (routed) or 0, z = token tile of 16.
// out h [pos][N] fp32.
template <bool STQ, int KS>
__global__ __launch_bounds__(64 * KS) void gateup_kernel(FfnArgs a) {
  __shared__ uint2 s_lut[32];
  __shared__ __align__(16) float s_sc[KS][2][kMaxWaveBlocks][kRows];
  __shared__ __align__(16) float s_red[KS][2][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int N = a.N, K = a.K;
  int e = 0, start = 0, cnt = a.T;
  if (STQ) {
    e = moe_find_active_expert(a.offsets, a.E, blockIdx.y, start, cnt);
    if (e < 0) return;
  }
  const int j0 = blockIdx.z * 16;
  if (j0 >= cnt) return;
  const int ntok = min(16, cnt - j0);
  const int row0 = blockIdx.x * kRows;
  const int col = lane & 15, g = lane >> 4;
  const uint16_t* xrow = nullptr;
  if (col < ntok) {
    const int pos = start + j0 + col;
    const int tok = STQ ? a.sorted_pair[pos] / a.k : pos;
    xrow = static_cast<const uint16_t*>(a.act) + (size_t)tok * K;
  }
  const int nblk = K / 256;
  const int b0 = wave * nblk / KS, b1 = (wave + 1) * nblk / KS;
  if (STQ) {
    build_lut(s_lut);
    const uint16_t* sg = static_cast<const uint16_t*>(a.scales0);
    const uint16_t* su = static_cast<const uint16_t*>(a.scales1);
    for (int i = lane; i < (b1 - b0) * kRows; i += 64) {
      const int bl = i / kRows, r = i % kRows;
      const size_t idx = ((size_t)e * N + row0 + r) * nblk + b0 + bl;
      s_sc[wave][0][bl][r] = fp16_to_f32(sg[idx]);
      s_sc[wave][1][bl][r] = fp16_to_f32(su[idx]);
    }
  }
  __syncthreads();

  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  const int arow = row0 + (lane & 15);
  for (int b = b0; b < b1; ++b) {
    if (STQ) {
      const uint8_t* rg = static_cast<const uint8_t*>(a.codes0) + ((size_t)e * N + arow) * nblk * 40 + (size_t)b * 40;
      const uint8_t* ru = static_cast<const uint8_t*>(a.codes1) + ((size_t)e * N + arow) * nblk * 40 + (size_t)b * 40;
      const uint2 qsg = *reinterpret_cast<const uint2*>(rg + 8 * g);
      const uint32_t qhg = *reinterpret_cast<const uint16_t*>(rg + 32 + 2 * g);
      const uint2 qsu = *reinterpret_cast<const uint2*>(ru + 8 * g);
      const uint32_t qhu = *reinterpret_cast<const uint16_t*>(ru + 32 + 2 * g);
      f32x4_t bg = {0.f, 0.f, 0.f, 0.f}, bu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint4 xv = make_uint4(0, 0, 0, 0);
        if (xrow) xv = *reinterpret_cast<const uint4*>(xrow + 256 * b + 64 * g + 8 * t);
        const bf16x8_t bx = as_bf16x8(xv);
        bg = mfma16(stq_a(s_lut, qsg, qhg, t), bx, bg);
        bu = mfma16(stq_a(s_lut, qsu, qhu, t), bx, bu);
      }
      const float4 dg = *reinterpret_cast<const float4*>(&s_sc[wave][0][b - b0][4 * g]);
      const float4 du = *reinterpret_cast<const float4*>(&s_sc[wave][1][b - b0][4 * g]);
      accg[0] = fmaf(dg.x, bg[0], accg[0]); accg[1] = fmaf(dg.y, bg[1], accg[1]);
      accg[2] = fmaf(dg.z, bg[2], accg[2]); accg[3] = fmaf(dg.w, bg[3], accg[3]);
      accu[0] = fmaf(du.x, bu[0], accu[0]); accu[1] = fmaf(du.y, bu[1], accu[1]);
      accu[2] = fmaf(du.z, bu[2], accu[2]); accu[3] = fmaf(du.w, bu[3], accu[3]);
    } else {
      const uint16_t* rg = static_cast<const uint16_t*>(a.codes0) + (size_t)arow * K + 256 * b;
      const uint16_t* ru = static_cast<const uint16_t*>(a.codes1) + (size_t)arow * K + 256 * b;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint4 xv = make_uint4(0, 0, 0, 0);
        if (xrow) xv = *reinterpret_cast<const uint4*>(xrow + 256 * b + 32 * t + 8 * g);
        const bf16x8_t bx = as_bf16x8(xv);
        const bf16x8_t ag = as_bf16x8(*reinterpret_cast<const uint4*>(rg + 32 * t + 8 * g));
        const bf16x8_t au = as_bf16x8(*reinterpret_cast<const uint4*>(ru + 32 * t + 8 * g));
        accg = mfma16(ag, bx, accg);
        accu = mfma16(au, bx, accu);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s_red[wave][0][i][lane] = accg[i];
    s_red[wave][1][i][lane] = accu[i];
  }
  __syncthreads();
  if (wave != 0 || col >= ntok) return;
  float h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float gs = 0.f, us = 0.f;
    for (int w = 0; w < KS; ++w) {
      gs += s_red[w][0][i][lane];
      us += s_red[w][1][i][lane];
    }
    h[i] = gs / (1.0f + expf(-gs)) * us;
  }
  const int pos = start + j0 + col;
  *reinterpret_cast<float4*>(a.out + (size_t)pos * N + row0 + 4 * g) =
      make_float4(h[0], h[1], h[2], h[3]);
}

// ------------------------------------------------------------------ down projection
// grid: x = row tile (N/16), y = expert slot (routed) or 0, z = token tile of 8.
// act = h [pos][K] fp32; out y [pos][N] fp32.
template <bool STQ, int KS>
__global__ __launch_bounds__(64 * KS) void down_kernel(FfnArgs a) {
  __shared__ uint2 s_lut[32];
  __shared__ __align__(16) float s_sc[KS][kMaxWaveBlocks][kRows];
  __shared__ __align__(16) float s_red[KS][4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int N = a.N, K = a.K;
  int e = 0, start = 0, cnt = a.T;
  if (STQ) {
    e = moe_find_active_expert(a.offsets, a.E, blockIdx.y, start, cnt);
    if (e < 0) return;
  }
  const int j0 = blockIdx.z * 8;
  if (j0 >= cnt) return;
  const int ntok = min(8, cnt - j0);
  const int row0 = blockIdx.x * kRows;
  const int col = lane & 15, g = lane >> 4;
  const int tj = col >> 1, part = col & 1;
  const float* hrow = nullptr;
  if (tj < ntok) hrow = static_cast<const float*>(a.act) + (size_t)(start + j0 + tj) * K;
  const int nblk = K / 256;
  const int b0 = wave * nblk / KS, b1 = (wave + 1) * nblk / KS;
  if (STQ) {
    build_lut(s_lut);
    const uint16_t* sd = static_cast<const uint16_t*>(a.scales0);
    for (int i = lane; i < (b1 - b0) * kRows; i += 64) {
      const int bl = i / kRows, r = i % kRows;
      s_sc[wave][bl][r] = fp16_to_f32(sd[((size_t)e * N + row0 + r) * nblk + b0 + bl]);
    }
  }
  __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int arow = row0 + (lane & 15);
  for (int b = b0; b < b1; ++b) {
    if (STQ) {
      const uint8_t* rd = static_cast<const uint8_t*>(a.codes0) + ((size_t)e * N + arow) * nblk * 40 + (size_t)b * 40;
      const uint2 qs = *reinterpret_cast<const uint2*>(rd + 8 * g);
      const uint32_t qh = *reinterpret_cast<const uint16_t*>(rd + 32 + 2 * g);
      f32x4_t bacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        bf16x8_t bh = as_bf16x8(make_uint4(0, 0, 0, 0));
        if (hrow) {
          const float* hp = hrow + 256 * b + 64 * g + 8 * t;
          bh = split_bf16(*reinterpret_cast<const float4*>(hp), *reinterpret_cast<const float4*>(hp + 4), part);
        }
        bacc = mfma16(stq_a(s_lut, qs, qh, t), bh, bacc);
      }
      const float4 d = *reinterpret_cast<const float4*>(&s_sc[wave][b - b0][4 * g]);
      acc[0] = fmaf(d.x, bacc[0], acc[0]); acc[1] = fmaf(d.y, bacc[1], acc[1]);
      acc[2] = fmaf(d.z, bacc[2], acc[2]); acc[3] = fmaf(d.w, bacc[3], acc[3]);
    } else {
      const uint16_t* rd = static_cast<const uint16_t*>(a.codes0) + (size_t)arow * K + 256 * b;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        bf16x8_t bh = as_bf16x8(make_uint4(0, 0, 0, 0));
        if (hrow) {
          const float* hp = hrow + 256 * b + 32 * t + 8 * g;
          bh = split_bf16(*reinterpret_cast<const float4*>(hp), *reinterpret_cast<const float4*>(hp + 4), part);
        }
        acc = mfma16(as_bf16x8(*reinterpret_cast<const uint4*>(rd + 32 * t + 8 * g)), bh, acc);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave != 0) return;
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s = 0.f;
    for (int w = 0; w < KS; ++w) s += s_red[w][i][lane];
    y[i] = s;
  }
  // columns 2j (hi) and 2j+1 (lo) belong to the same token: add the partner lane's value
  float yo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) yo[i] = y[i] + __shfl_xor(y[i], 1, 64);
  if (part == 0 && tj < ntok) {
    const int pos = start + j0 + tj;
    *reinterpret_cast<float4*>(a.out + (size_t)pos * N + row0 + 4 * g) =
        make_float4(yo[0], yo[1], yo[2], yo[3]);
  }
}

// ------------------------------------------------------------------ generic STQ1_0 path
// Blocks may straddle rows (in % 256 != 0): one thread per (row, pair), weights decoded
// one at a time from the flattened block stream.  Slow; used for tiny shapes only.
__device__ __forceinline__ float stq_weight(const uint8_t* codes, const uint16_t* scales,
                                            size_t flat) {
  const size_t blk = flat >> 8;
  const int within = (int)(flat & 255);
  const int grp = within >> 2, ln = within & 3;
  const uint8_t* c = codes + blk * 40;
  const uint32_t nib = (c[grp >> 1] >> (4 * (grp & 1))) & 15u;
  const uint32_t hb = (c[32 + (grp >> 3)] >> (grp & 7)) & 1u;
  const uint32_t p = nib | (hb << 4);
  const int z = p >> 3;
  if (ln == z) return 0.f;
  const int i = ln < z ? ln : ln - 1;
  const float d = fp16_to_f32(scales[blk]);
  return ((p >> i) & 1) ? -d : d;
}

__global__ __launch_bounds__(256) void stq_generic_kernel(FfnArgs a, int down) {
  const int N = a.N, K = a.K;
  int start, cnt;
  const int e = moe_find_active_expert(a.offsets, a.E, blockIdx.y, start, cnt);
  if (e < 0) return;
  const int row = blockIdx.x * 256 + threadIdx.x;
  const int j = blockIdx.z;
  if (row >= N || j >= cnt) return;
  const int pos = start + j;
  const size_t mat = (size_t)N * K;
  const uint8_t* c0 = static_cast<const uint8_t*>(a.codes0) + (size_t)e * (mat / 256) * 40;
  const uint16_t* s0 = static_cast<const uint16_t*>(a.scales0) + (size_t)e * (mat / 256);
  if (down) {
    const float* hr = static_cast<const float*>(a.act) + (size_t)pos * K;
    float acc = 0.f;
    for (int c = 0; c < K; ++c) acc = fmaf(stq_weight(c0, s0, (size_t)row * K + c), hr[c], acc);
    a.out[(size_t)pos * N + row] = acc;
  } else {
    const uint8_t* c1 = static_cast<const uint8_t*>(a.codes1) + (size_t)e * (mat / 256) * 40;
    const uint16_t* s1 = static_cast<const uint16_t*>(a.scales1) + (size_t)e * (mat / 256);
    const uint16_t* xr = static_cast<const uint16_t*>(a.act) + (size_t)(a.sorted_pair[pos] / a.k) * K;
    float gs = 0.f, us = 0.f;
    for (int c = 0; c < K; ++c) {
      const float xv = bf16_to_f32(xr[c]);
      gs = fmaf(stq_weight(c0, s0, (size_t)row * K + c), xv, gs);
      us = fmaf(stq_weight(c1, s1, (size_t)row * K + c), xv, us);
    }
    a.out[(size_t)pos * N + row] = gs / (1.0f + expf(-gs)) * us;
  }
}

inline int expert_slots(const FfnArgs& a) { return a.P < a.E ? a.P : a.E; }

}  // namespace

hipError_t moe_launch_stq_gateup(const FfnArgs& a, hipStream_t s) {
  dim3 grid(a.N / kRows, expert_slots(a), (a.T + 15) / 16);
  hipLaunchKernelGGL((gateup_kernel<true, 4>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t moe_launch_stq_down(const FfnArgs& a, hipStream_t s) {
  dim3 grid(a.N / kRows, expert_slots(a), (a.T + 7) / 8);
  hipLaunchKernelGGL((down_kernel<true, 4>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t moe_launch_stq_generic(const FfnArgs& a, int down, hipStream_t s) {
  dim3 grid((a.N + 255) / 256, expert_slots(a), a.T);
  hipLaunchKernelGGL(stq_generic_kernel, grid, dim3(256), 0, s, a, down);
  return hipGetLastError();
}

hipError_t moe_launch_bf16_gateup(const FfnArgs& a, hipStream_t s) {
  dim3 grid(a.N / kRows, 1, (a.T + 15) / 16);
  hipLaunchKernelGGL((gateup_kernel<false, 8>), grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t moe_launch_bf16_down(const FfnArgs& a, hipStream_t s) {
  dim3 grid(a.N / kRows, 1, (a.T + 7) / 8);
  hipLaunchKernelGGL((down_kernel<false, 4>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}
