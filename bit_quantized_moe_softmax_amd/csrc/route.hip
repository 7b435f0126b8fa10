// Router: bf16 logits GEMV and the wave-level top-k with renormalised softmax weights.
//
// The router stays BF16 in the Hy4 checkpoints ("Hy4-preview-SF-WFP4AFP8", BF16 row of
// the Quant Diff table); each token keeps its 8 largest logits ("Hy4-preview Flash-MoE
// STQ1_0", Package details: 8 selected experts per token).  The routing function is
// not on the pages: softmax, top-k, renormalise over the selected k.
#include "moe_device.h"

#include <math.h>

namespace {

constexpr int kRouteTokTile = 8;   // tokens per wave in the logits GEMV

// One wave per expert row, up to kRouteTokTile tokens.  Each lane streams 8 bf16 of the
// router row per iteration (16-byte loads, coalesced over the wave) and reuses them for
// every token of the tile; the 64 lane partials are reduced with DPP/shuffles.
__global__ __launch_bounds__(256) void route_gemv_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wr,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits, int T,
                                                         int H, int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * kRouteTokTile;
  if (e >= E) return;
  const int nt = min(kRouteTokTile, T - t0);
  float acc[kRouteTokTile];
#pragma unroll
  for (int i = 0; i < kRouteTokTile; ++i) acc[i] = 0.f;
  const uint16_t* wrow = wr + (size_t)e * H;
  for (int c = lane * 8; c < H; c += 64 * 8) {
    const uint4 wv = *reinterpret_cast<const uint4*>(wrow + c);
    float wf[8];
    wf[0] = bf16_to_f32(wv.x & 0xFFFF); wf[1] = bf16_to_f32(wv.x >> 16);
    wf[2] = bf16_to_f32(wv.y & 0xFFFF); wf[3] = bf16_to_f32(wv.y >> 16);
    wf[4] = bf16_to_f32(wv.z & 0xFFFF); wf[5] = bf16_to_f32(wv.z >> 16);
    wf[6] = bf16_to_f32(wv.w & 0xFFFF); wf[7] = bf16_to_f32(wv.w >> 16);
#pragma unroll
    for (int i = 0; i < kRouteTokTile; ++i) {
      if (i < nt) {
        const uint4 xv = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + i) * H + c);
        float a = acc[i];
        a = fmaf(bf16_to_f32(xv.x & 0xFFFF), wf[0], a);
        a = fmaf(bf16_to_f32(xv.x >> 16), wf[1], a);
        a = fmaf(bf16_to_f32(xv.y & 0xFFFF), wf[2], a);
        a = fmaf(bf16_to_f32(xv.y >> 16), wf[3], a);
        a = fmaf(bf16_to_f32(xv.z & 0xFFFF), wf[4], a);
        a = fmaf(bf16_to_f32(xv.z >> 16), wf[5], a);
        a = fmaf(bf16_to_f32(xv.w & 0xFFFF), wf[6], a);
        a = fmaf(bf16_to_f32(xv.w >> 16), wf[7], a);
        acc[i] = a;
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int i = 0; i < kRouteTokTile; ++i) {
    if (i < nt) {
      const float v = wave_sum(acc[i]);
      if (lane == 0) logits[(size_t)(t0 + i) * E + e] = v + b;
    }
  }
}

constexpr int kMaxPerLane = 16;   // E <= 1024

// Order-preserving unsigned key of a logit: a larger value gives a larger key, -0 keys as
// +0, and every NaN takes the largest key (NaN ranks above every number, all NaNs equal),
// so the selection is a total order and every pick is a real expert index.
__device__ __forceinline__ uint32_t logit_key(float f) {
  if (f != f) return 0xFFFFFFFFu;
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave per token.  Lane l holds logits l, l+64, ...; k rounds of a wave arg-max over
// (key, -index) pick the slots in descending order, ties to the lower index.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits_out, int T,
                                                   int E, int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nper = (E + 63) >> 6;
  float v[kMaxPerLane];
  uint32_t key[kMaxPerLane];
  const float* row = logits + (size_t)t * E;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = i * 64 + lane;
    float val = 0.f;
    if (i < nper && e < E) {
      val = row[e];
      if (bias) val += bias[e];
      if (logits_out) logits_out[(size_t)t * E + e] = val;
    }
    v[i] = val;
    key[i] = logit_key(val);
  }
  // a lane slot is "live" when it maps to a real expert and has not been taken yet
  uint32_t live = 0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i)
    if (i < nper && i * 64 + lane < E) live |= 1u << i;
  float my_v = 0.f;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    // candidate = (key << 32) | (~index): the largest is the largest key, then the lowest
    // index; a lane with nothing live offers 0, below every real candidate
    uint64_t best = 0;
    float bv = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      if ((live >> i) & 1u) {
        const uint64_t c = ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(i * 64 + lane);
        if (c > best) { best = c; bv = v[i]; }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t ob = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), o, 64) << 32) |
                          (uint32_t)__shfl_xor((int)(uint32_t)best, o, 64);
      const float ov = __shfl_xor(bv, o, 64);
      if (ob > best) { best = ob; bv = ov; }
    }
    const int bi = (int)~(uint32_t)best;
    if ((bi & 63) == lane) live &= ~(1u << (bi >> 6));
    if (lane == j) { my_v = bv; my_i = bi; }
  }
  const float v0 = __shfl(my_v, 0, 64);
  const float ex = lane < k ? expf(my_v - v0) : 0.f;
  const float s = wave_sum(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_i;
    w[(size_t)t * k + lane] = ex / s;
  }
}

}  // namespace

hipError_t moe_launch_route_gemv(const uint16_t* x, const uint16_t* wr, const float* bias,
                                 float* logits, int T, int H, int E, hipStream_t s) {
  dim3 grid((E + 3) / 4, (T + kRouteTokTile - 1) / kRouteTokTile);
  hipLaunchKernelGGL(route_gemv_kernel, grid, dim3(256), 0, s, x, wr, bias, logits, T, H, E);
  return hipGetLastError();
}

hipError_t moe_launch_topk(const float* logits, const float* bias, float* logits_out, int T,
                           int E, int k, int32_t* ids, float* w, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, bias, logits_out,
                     T, E, k, ids, w);
  return hipGetLastError();
}
