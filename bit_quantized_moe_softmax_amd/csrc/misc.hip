// Combine, RMSNorm, STQ1_0 pack/decode, MXFP4 decode and MX activation quantisation.
#include "moe_device.h"

namespace {

// ---------------------------------------------------------------- combine
// out[t] = y_shared[t] + sum_j w[t][j] * y_pairs[pair_pos[t*k+j]] (+ residual[t]).
// The shared expert is ungated: the Flash-MoE package lists one shared expert per MoE
// block and no gate for it.  One thread per 4 consecutive hidden elements.  A pair with
// pair_pos -1 (not routed by moe_permute) contributes nothing.
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ y_pairs, const float* __restrict__ w,
    const int32_t* __restrict__ pair_pos, const float* __restrict__ y_shared,
    const float* residual, float* out, uint16_t* __restrict__ out_bf16, int H, int k) {
  const int t = blockIdx.x;   // tokens on x: the other grid dimensions stop at 65535
  const int h = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (h >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (y_shared) acc = *reinterpret_cast<const float4*>(y_shared + (size_t)t * H + h);
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const int pos = pair_pos[(size_t)t * k + j];
    if (pos < 0) continue;   // a pair moe_permute left unrouted adds nothing
    const float4 y = *reinterpret_cast<const float4*>(y_pairs + (size_t)pos * H + h);
    acc.x = fmaf(wj, y.x, acc.x);
    acc.y = fmaf(wj, y.y, acc.y);
    acc.z = fmaf(wj, y.z, acc.z);
    acc.w = fmaf(wj, y.w, acc.w);
  }
  if (residual) {
    const float4 r = *reinterpret_cast<const float4*>(residual + (size_t)t * H + h);
    acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
  }
  *reinterpret_cast<float4*>(out + (size_t)t * H + h) = acc;
  if (out_bf16) {
    uint2 b;
    b.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    b.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(out_bf16 + (size_t)t * H + h) = b;
  }
}

// ---------------------------------------------------------------- RMSNorm + bf16 cast
// One workgroup per row.  Rows of up to 8192 floats (H % 4 == 0): every thread loads its M
// float4 pieces (piece tid + 256 m) at once, keeps them in registers for the scaling, and the
// row is read once; other rows take the strided loop.
template <int M>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ r,
                                                      uint16_t* __restrict__ a, int H,
                                                      float eps) {
  __shared__ float s_part[4];
  const int t = blockIdx.x;
  const float* row = r + (size_t)t * H;
  float ss = 0.f;
  float4 v[M > 0 ? M : 1];
  if constexpr (M > 0) {
    const int n4 = H / 4;
    const float4* row4 = reinterpret_cast<const float4*>(row);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int i = threadIdx.x + 256 * m;
      v[m] = i < n4 ? row4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
      ss = fmaf(v[m].x, v[m].x, fmaf(v[m].y, v[m].y, fmaf(v[m].z, v[m].z, fmaf(v[m].w, v[m].w, ss))));
  } else {
    for (int i = threadIdx.x; i < H; i += 256) ss = fmaf(row[i], row[i], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  if constexpr (M > 0) {
    const int n4 = H / 4;
    uint2* a4 = reinterpret_cast<uint2*>(a + (size_t)t * H);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int i = threadIdx.x + 256 * m;
      if (i < n4)
        a4[i] = make_uint2(f32_to_bf16_rne(v[m].x * inv) | (f32_to_bf16_rne(v[m].y * inv) << 16),
                           f32_to_bf16_rne(v[m].z * inv) | (f32_to_bf16_rne(v[m].w * inv) << 16));
    }
  } else {
    for (int i = threadIdx.x; i < H; i += 256)
      a[(size_t)t * H + i] = (uint16_t)f32_to_bf16_rne(row[i] * inv);
  }
}

// ---------------------------------------------------------------- STQ1_0 pack / decode
// Pattern p = 8*z + s; byte i of the 32-byte nibble area = p[2i] & 15 | (p[2i+1] & 15) << 4;
// bytes 32..39 = little-endian word with bit g = p[g] >> 4.  One wave per block.
__global__ __launch_bounds__(256) void stq1_pack_kernel(const uint8_t* __restrict__ z,
                                                        const uint8_t* __restrict__ sg,
                                                        const uint16_t* __restrict__ d,
                                                        int64_t n_blocks,
                                                        uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= n_blocks) return;
  const int64_t g = b * 64 + lane;
  const uint32_t p = ((uint32_t)(z[g] & 3) << 3) | (sg[g] & 7);
  const uint64_t hi = __ballot((p >> 4) & 1);
  const uint32_t nib = p & 15;
  const uint32_t other = __shfl_xor(nib, 1, 64);
  uint8_t* blk = codes + b * 40;
  if ((lane & 1) == 0) blk[lane >> 1] = (uint8_t)(nib | (other << 4));
  if (lane < 8) blk[32 + lane] = (uint8_t)(hi >> (8 * lane));
  if (lane == 0) scales[b] = d[b];
}

// Lane j of pattern p (in units of d): the zero lane is z = p >> 3; the other lanes in
// ascending order take the sign bits 0, 1, 2 of s = p & 7 (1 = negative).
__device__ __forceinline__ float stq1_lane(uint32_t p, int j) {
  const int z = p >> 3;
  if (j == z) return 0.f;
  const int i = j < z ? j : j - 1;
  return ((p >> i) & 1) ? -1.f : 1.f;
}

__global__ __launch_bounds__(256) void stq1_dequant_kernel(const uint8_t* __restrict__ codes,
                                                           const uint16_t* __restrict__ scales,
                                                           int64_t n_blocks,
                                                           float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= n_blocks) return;
  const uint8_t* blk = codes + b * 40;
  const uint32_t nib = (blk[lane >> 1] >> ((lane & 1) * 4)) & 15;
  const uint32_t hb = (blk[32 + (lane >> 3)] >> (lane & 7)) & 1;
  const uint32_t p = nib | (hb << 4);
  const float dv = fp16_to_f32(scales[b]);
  float4 o;
  o.x = stq1_lane(p, 0) * dv;
  o.y = stq1_lane(p, 1) * dv;
  o.z = stq1_lane(p, 2) * dv;
  o.w = stq1_lane(p, 3) * dv;
  *reinterpret_cast<float4*>(out + b * 256 + lane * 4) = o;
}

// ---------------------------------------------------------------- MXFP4 decode
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t e = (c >> 1) & 3, m = c & 1;
  const float mag = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
  return (c & 8) ? -mag : mag;
}

__global__ __launch_bounds__(256) void mxfp4_dequant_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int64_t n_pairs, int K,
                                                            float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one code byte each
  if (i >= n_pairs) return;
  const int64_t row = i / (K / 2);
  const int64_t col = (i % (K / 2)) * 2;
  const uint8_t c = codes[i];
  const float sc = ldexpf(1.0f, (int)scales[row * (K / 32) + col / 32] - 127);
  out[row * K + col] = e2m1_to_f32(c & 15) * sc;
  out[row * K + col + 1] = e2m1_to_f32(c >> 4) * sc;
}

// Eight elements per lane (one 16-byte bf16 load or two fp32 loads); lanes 4q .. 4q + 3
// form a group (groups never straddle rows: K is a multiple of 32).  Lanes past the end
// load the last octet and store nothing (n8 is a multiple of 4, so groups stay whole).
__global__ __launch_bounds__(256) void mx_quant_kernel(int64_t n8, const uint16_t* xb,
                                                       const float* xf, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ sc) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t j = i < n8 ? i : n8 - 1;
  uint32_t bits[8];
  if (xb) {
    const uint4 v = reinterpret_cast<const uint4*>(xb)[j];
    bits[0] = v.x << 16; bits[1] = v.x & 0xFFFF0000u; bits[2] = v.y << 16; bits[3] = v.y & 0xFFFF0000u;
    bits[4] = v.z << 16; bits[5] = v.z & 0xFFFF0000u; bits[6] = v.w << 16; bits[7] = v.w & 0xFFFF0000u;
  } else {
    const uint4 v0 = reinterpret_cast<const uint4*>(xf)[2 * j];
    const uint4 v1 = reinterpret_cast<const uint4*>(xf)[2 * j + 1];
    bits[0] = v0.x; bits[1] = v0.y; bits[2] = v0.z; bits[3] = v0.w;
    bits[4] = v1.x; bits[5] = v1.y; bits[6] = v1.z; bits[7] = v1.w;
  }
  uint32_t codes[2];
  const uint32_t s = moe_mx_quant8(bits, codes);
  if (i < n8) {
    reinterpret_cast<uint2*>(q)[i] = make_uint2(codes[0], codes[1]);
    if ((i & 3) == 0) sc[i / 4] = (uint8_t)s;
  }
}

// The MX quantisation of fp32 rows with every E4M3 code from the scaled hardware conversion
// (moe_e4m3_pair_hw, the encoder of the MXFP4 gate/up epilogue) in place of moe_e4m3_code:
// the same group exponent and the same output layout as mx_quant_kernel.
__global__ __launch_bounds__(256) void mx_quant_hw_kernel(int64_t n8, const float* xf,
                                                          uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ sc) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t j = i < n8 ? i : n8 - 1;
  const uint4 v0 = reinterpret_cast<const uint4*>(xf)[2 * j];
  const uint4 v1 = reinterpret_cast<const uint4*>(xf)[2 * j + 1];
  const uint32_t bits[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t am = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) am = max(am, bits[e] & 0x7FFFFFFFu);
  am = max(am, (uint32_t)__shfl_xor((int)am, 1, 64));
  am = max(am, (uint32_t)__shfl_xor((int)am, 2, 64));
  uint32_t c[2] = {0u, 0u};
  const int X = am ? moe_mx_exp(am) : -127;
  if (am) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const float* f = reinterpret_cast<const float*>(bits + 4 * w);
      c[w] = moe_e4m3_pair_hw(f[0], f[1], X) | (moe_e4m3_pair_hw(f[2], f[3], X) << 16);
    }
  }
  if (i < n8) {
    reinterpret_cast<uint2*>(q)[i] = make_uint2(c[0], c[1]);
    if ((i & 3) == 0) sc[i / 4] = am ? (uint8_t)(X + 127) : (uint8_t)0;
  }
}

// The bf16 values of the MX E4M3 quantisation of rows (group 32 along K): the codes of
// moe_mx_quant8, decoded times 2^X by the gfx950 scaled conversion (E4M3 with 3 mantissa
// bits times a power of two is exact in bf16).  Eight elements per lane as mx_quant_kernel.
__global__ __launch_bounds__(256) void mx_roundtrip_kernel(int64_t n8, const uint16_t* xb,
                                                           const float* xf,
                                                           uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t j = i < n8 ? i : n8 - 1;
  uint32_t bits[8];
  if (xb) {
    const uint4 v = reinterpret_cast<const uint4*>(xb)[j];
    bits[0] = v.x << 16; bits[1] = v.x & 0xFFFF0000u; bits[2] = v.y << 16; bits[3] = v.y & 0xFFFF0000u;
    bits[4] = v.z << 16; bits[5] = v.z & 0xFFFF0000u; bits[6] = v.w << 16; bits[7] = v.w & 0xFFFF0000u;
  } else {
    const uint4 v0 = reinterpret_cast<const uint4*>(xf)[2 * j];
    const uint4 v1 = reinterpret_cast<const uint4*>(xf)[2 * j + 1];
    bits[0] = v0.x; bits[1] = v0.y; bits[2] = v0.z; bits[3] = v0.w;
    bits[4] = v1.x; bits[5] = v1.y; bits[6] = v1.z; bits[7] = v1.w;
  }
  uint32_t codes[2];
  const float sc = moe_ue8m0_scale(moe_mx_quant8(bits, codes));
  uint32_t o[4];
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    o[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[w], sc, false));
    o[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[w], sc, true));
  }
  if (i < n8) reinterpret_cast<uint4*>(out)[i] = make_uint4(o[0], o[1], o[2], o[3]);
}

// STQ1_0 encoders ("Hy4-preview-GGUF" (AngelSlim), section 3, Our encoder), one wave per
// 256-weight block of the flattened matrix, lane l = group l (weights 4l .. 4l+3).  Importance
// w of a weight: imatrix[flat index mod K], or 1.
//   method 0 (upstream): d = the block's largest magnitude; zero at the smallest |x| of each
//     group (the first lane on ties).
//   method 1 (weighted least squares): from the upstream zero placement, 3 rounds of
//     d = sum(w |x|) / sum(w) over the kept lanes (the LS scale with sel = sign(x)), then in
//     every group the zero at the smallest incremental cost w d (2 |x| - d) (= w (x^2 -
//     (|x| - d)^2)), and a final LS fit; a block whose kept lanes have no weight keeps
//     d = amax.
// Kept lanes take the sign of x (x = 0 counts as positive); d is rounded to fp16 (nearest
// even) once.  Sums are wave reductions in a fixed order.
__device__ __forceinline__ int argmin4(const float* c) {
  int z = 0;
  float m = c[0];
#pragma unroll
  for (int j = 1; j < 4; ++j)
    if (c[j] < m) { m = c[j]; z = j; }
  return z;
}

__global__ __launch_bounds__(256) void stq1_encode_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ imatrix,
                                                          int64_t n_blocks, int K, int method,
                                                          uint8_t* __restrict__ codes,
                                                          uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= n_blocks) return;   // whole waves
  const int64_t f0 = b * 256 + 4 * lane;
  const float4 xv = *reinterpret_cast<const float4*>(x + f0);
  const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
  float ax[4], w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ax[j] = fabsf(xs[j]);
    w[j] = imatrix ? imatrix[(f0 + j) % K] : 1.0f;
  }
  float amax = fmaxf(fmaxf(ax[0], ax[1]), fmaxf(ax[2], ax[3]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  int z = argmin4(ax);
  float d = amax;
  if (method == 1) {
    auto ls = [&]() {
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j != z) { num = fmaf(w[j], ax[j], num); den += w[j]; }
      num = wave_sum(num);
      den = wave_sum(den);
      return den > 0.f ? num / den : amax;
    };
    for (int r = 0; r < 3; ++r) {
      d = ls();
      float c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = w[j] * d * (2.0f * ax[j] - d);
      z = argmin4(c);
    }
    d = ls();
  }
  uint32_t sg = 0;
  int i = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (j != z) { sg |= (xs[j] < 0.f ? 1u : 0u) << i; ++i; }
  const uint32_t p = ((uint32_t)z << 3) | sg;
  const uint32_t pn = (uint32_t)__shfl_down((int)p, 1, 64);
  uint8_t* cb = codes + b * 40;
  if ((lane & 1) == 0) cb[lane >> 1] = (uint8_t)((p & 15u) | ((pn & 15u) << 4));
  const uint64_t hi = __ballot((p >> 4) & 1u);
  if (lane == 0) {
    reinterpret_cast<uint2*>(cb + 32)[0] = make_uint2((uint32_t)hi, (uint32_t)(hi >> 32));
    scales[b] = __builtin_bit_cast(uint16_t, (_Float16)d);
  }
}

}  // namespace

hipError_t moe_launch_combine(const float* y_pairs, const float* w, const int32_t* pair_pos,
                              const float* y_shared, const float* residual, float* out,
                              uint16_t* out_bf16, int T, int H, int k, hipStream_t s) {
  dim3 grid(T, (H / 4 + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, y_pairs, w, pair_pos, y_shared,
                     residual, out, out_bf16, H, k);
  return hipGetLastError();
}

hipError_t moe_launch_rmsnorm(const float* r, uint16_t* a, int T, int H, float eps,
                              hipStream_t s) {
  const bool vec = H % 4 == 0 && H <= 8192 && reinterpret_cast<uintptr_t>(r) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a) % 8 == 0;
  const int m = vec ? (H / 4 + 255) / 256 : 0;
  if (m == 0) hipLaunchKernelGGL(rmsnorm_kernel<0>, dim3(T), dim3(256), 0, s, r, a, H, eps);
  else if (m <= 2) hipLaunchKernelGGL(rmsnorm_kernel<2>, dim3(T), dim3(256), 0, s, r, a, H, eps);
  else if (m <= 4) hipLaunchKernelGGL(rmsnorm_kernel<4>, dim3(T), dim3(256), 0, s, r, a, H, eps);
  else if (m <= 6) hipLaunchKernelGGL(rmsnorm_kernel<6>, dim3(T), dim3(256), 0, s, r, a, H, eps);
  else hipLaunchKernelGGL(rmsnorm_kernel<8>, dim3(T), dim3(256), 0, s, r, a, H, eps);
  return hipGetLastError();
}

hipError_t moe_launch_stq1_pack(const uint8_t* z, const uint8_t* sg, const uint16_t* d,
                                int64_t n_blocks, uint8_t* codes, uint16_t* scales,
                                hipStream_t s) {
  hipLaunchKernelGGL(stq1_pack_kernel, dim3((unsigned)((n_blocks + 3) / 4)), dim3(256), 0, s, z,
                     sg, d, n_blocks, codes, scales);
  return hipGetLastError();
}

hipError_t moe_launch_stq1_dequant(const uint8_t* codes, const uint16_t* scales,
                                   int64_t n_blocks, float* out, hipStream_t s) {
  hipLaunchKernelGGL(stq1_dequant_kernel, dim3((unsigned)((n_blocks + 3) / 4)), dim3(256), 0, s,
                     codes, scales, n_blocks, out);
  return hipGetLastError();
}

hipError_t moe_launch_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                    int K, float* out, hipStream_t s) {
  const int64_t n = rows * (K / 2);
  hipLaunchKernelGGL(mxfp4_dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     codes, scales, n, K, out);
  return hipGetLastError();
}

hipError_t moe_launch_mx_quant(int64_t rows, int K, const uint16_t* xb, const float* xf,
                               uint8_t* q, uint8_t* sc, hipStream_t s) {
  const int64_t n8 = rows * K / 8;
  if (n8 == 0) return hipSuccess;
  if ((n8 + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_quant_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, n8,
                     xb, xf, q, sc);
  return hipGetLastError();
}

hipError_t moe_launch_mx_quant_hw(int64_t rows, int K, const float* xf, uint8_t* q, uint8_t* sc,
                                  hipStream_t s) {
  const int64_t n8 = rows * K / 8;
  if (n8 == 0) return hipSuccess;
  if ((n8 + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_quant_hw_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, n8,
                     xf, q, sc);
  return hipGetLastError();
}

hipError_t moe_launch_stq1_encode(const float* x, const float* imatrix, int64_t n_blocks, int K,
                                  int method, uint8_t* codes, uint16_t* scales, hipStream_t s) {
  if (n_blocks == 0) return hipSuccess;
  if ((n_blocks + 3) / 4 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stq1_encode_kernel, dim3((unsigned)((n_blocks + 3) / 4)), dim3(256), 0, s, x,
                     imatrix, n_blocks, K, method, codes, scales);
  return hipGetLastError();
}

hipError_t moe_launch_mx_roundtrip_bf16(int64_t rows, int K, const uint16_t* xb, const float* xf,
                                        uint16_t* out, hipStream_t s) {
  const int64_t n8 = rows * K / 8;
  if (n8 == 0) return hipSuccess;
  if ((n8 + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_roundtrip_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, n8,
                     xb, xf, out);
  return hipGetLastError();
}
