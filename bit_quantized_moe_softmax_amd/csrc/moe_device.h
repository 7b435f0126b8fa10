// Device-side helpers shared by the gfx950 kernels of libmoe_mi355x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "moe_mi355x.h"

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

#define MOE_WAVE 64

// ---------------------------------------------------------------- scalar formats
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round a finite fp32 to bf16 bits, nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float fp16_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;
}

// ---------------------------------------------------------------- E4M3 encoding
// Exact integer rounding of |v| / 2^X onto the E4M3 grid (3 mantissa bits, subnormal
// quantum 2^-9), ties to even, saturated to 448 (code 0x7E); sign from the input.
__device__ __forceinline__ uint32_t moe_e4m3_from_f32(uint32_t bits, int X) {
  const uint32_t sign = (bits >> 31) << 7;
  const uint32_t ev = (bits >> 23) & 0xFF;
  uint32_t M = bits & 0x7FFFFF;
  int E0;                                   // |v| = M * 2^E0
  if (ev == 0) {
    if (M == 0) return sign;
    E0 = -149;
  } else {
    M |= 0x800000;
    E0 = (int)ev - 150;
  }
  const int lg = (31 - __clz(M)) + E0 - X;  // floor(log2 |y|), y = v / 2^X
  const int qexp = lg - 3 > -9 ? lg - 3 : -9;
  const int sh = qexp - (E0 - X);           // y / 2^qexp = M / 2^sh
  uint32_t R;
  if (sh <= 0) {
    R = M << (-sh);                         // exact (only when y is a multiple of 2^qexp)
  } else if (sh > 25) {
    R = 0;
  } else {
    const uint32_t q = M >> sh;
    const uint32_t rem = M & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    R = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  }
  // value = R * 2^qexp with R <= 16
  uint32_t code;
  if (R == 0) {
    code = 0;
  } else if (qexp == -9 && R < 8) {
    code = R;                               // subnormal
  } else {
    int ef = qexp + 3 + 7;                  // exponent field for R in [8, 15]
    uint32_t m = R - 8;
    if (R == 16) { ef += 1; m = 0; }
    if (ef > 15 || (ef == 15 && m > 6)) code = 0x7E;   // saturate to 448
    else code = ((uint32_t)ef << 3) | m;
  }
  return sign | code;
}

// MX shared exponent of a group from the bits of its largest magnitude (> 0):
// X = floor(log2(amax)) - 8, clamped to [-127, 127]; the scale byte is X + 127.
__device__ __forceinline__ int moe_mx_exp(uint32_t amax_bits) {
  const uint32_t ea = amax_bits >> 23;
  const int lg = ea ? (int)ea - 127 : (31 - __clz(amax_bits & 0x7FFFFF)) - 149;
  const int X = lg - 8;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// The E4M3 code of v / 2^X by the rule of moe_e4m3_from_f32, branch-free: y = v 2^-X is
// exact wherever the code is not zero (a power-of-two scaling), the rounding quantum is
// 2^max(floor(log2|y|) - 3, -9), and rint() rounds the scaled magnitude to the nearest
// integer R (ties to even); R <= 16 picks the code.  Equal to moe_e4m3_from_f32 for every
// finite fp32 input with |v| < 2^(X + 9) (checked exhaustively on the CPU at nine X).
__device__ __forceinline__ uint32_t moe_e4m3_code(float v, int X) {
  const float y = ldexpf(v, -X);
  const uint32_t yb = __float_as_uint(y);
  const uint32_t sign = (yb >> 24) & 0x80u;
  const int e = (int)((yb >> 23) & 0xFFu) - 127;
  const int q = max(e - 3, -9);
  const uint32_t R = (uint32_t)rintf(ldexpf(fabsf(y), -q));
  const bool normal = q > -9 || R >= 8;
  const int ef = q + 10 + (int)(R >> 4);
  const uint32_t m = R == 16 ? 0u : R - 8;
  uint32_t code = normal ? (((uint32_t)ef << 3) | m) : R;
  code = (ef > 15 || (ef == 15 && m > 6)) ? 0x7Eu : code;
  return sign | code;
}

// Two values to E4M3 codes at MX exponent X (bytes 0 and 1 of the result) with the gfx950
// scaled hardware conversion, which divides by the scale 2^X and rounds to nearest even.
// Inputs are clamped to +-448 2^X first: past it the conversion gives the NaN code where the
// MX rule saturates.  Meant to equal moe_e4m3_code on each value for every exponent the MX
// rule produces (-127 .. 119) and |v| < 2^(X+9); moe_mx_quant_f32_hwcvt exposes it so that
// this can be checked against the integer rule on chosen values.
__device__ __forceinline__ uint32_t moe_e4m3_pair_hw(float a, float b, int X) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const float lim = ldexpf(448.0f, X);
  const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((v2s){0, 0}, fminf(fmaxf(a, -lim), lim),
                                                         fminf(fmaxf(b, -lim), lim), ldexpf(1.0f, X), false);
  return (uint16_t)r.x;
}

// Lane-parallel MX quantisation of 8 consecutive values per lane (fp32 bit patterns,
// finite): lanes 4q .. 4q + 3 of the wave hold the 32 values of one group.  Writes this
// lane's 8 E4M3 codes (element j in byte j % 4 of word j / 4) and returns the group's UE8M0
// scale byte (0 and zero codes for an all-zero group).  Every lane of the wave must call it
// (the group maximum is a cross-lane reduction).
__device__ __forceinline__ uint32_t moe_mx_quant8(const uint32_t* bits, uint32_t* codes) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = max(am, bits[i] & 0x7FFFFFFFu);
  am = max(am, (uint32_t)__shfl_xor((int)am, 1, 64));
  am = max(am, (uint32_t)__shfl_xor((int)am, 2, 64));
  if (am == 0) {
    codes[0] = codes[1] = 0;
    return 0;
  }
  const int X = moe_mx_exp(am);
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) c |= moe_e4m3_code(__uint_as_float(bits[4 * w + j]), X) << (8 * j);
    codes[w] = c;
  }
  return (uint32_t)(X + 127);
}

// 2^(byte - 127) as fp32 for a UE8M0 scale byte (byte 0: 2^-127, a subnormal).
__device__ __forceinline__ float moe_ue8m0_scale(uint32_t byte) {
  return byte ? __uint_as_float(byte << 23) : __uint_as_float(0x00400000u);
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

// The slot-th expert (in expert order) that has at least one routed pair, found by each
// wave on its own from the expert offsets (uniform across the wave).  Returns -1 when
// fewer experts are active.
__device__ __forceinline__ int moe_find_active_expert(const int32_t* __restrict__ off, int E,
                                                      int slot, int& start, int& cnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int run = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const int c = e < E ? off[e + 1] - off[e] : 0;
    const uint64_t m = __ballot(c > 0);
    const int n = __popcll(m);
    if (slot < run + n) {
      const int want = slot - run;
      const uint64_t mm = __ballot(c > 0 && __popcll(m & lt) == want);
      const int ee = base + __ffsll((unsigned long long)mm) - 1;
      start = off[ee];
      cnt = off[ee + 1] - start;
      return ee;
    }
    run += n;
  }
  return -1;
}

// ---------------------------------------------------------------- launch plumbing
#define MOE_HIP_TRY(expr)                                  \
  do {                                                     \
    hipError_t _e = (expr);                                \
    if (_e != hipSuccess) return _e;                       \
  } while (0)

// Host launchers implemented by the kernel translation units.
hipError_t moe_launch_route_gemv(const uint16_t* x, const uint16_t* wr, const float* bias,
                                 float* logits, int T, int H, int E, hipStream_t s);
hipError_t moe_launch_topk(const float* logits, const float* bias, float* logits_out, int T,
                           int E, int k, int32_t* ids, float* w, hipStream_t s);
hipError_t moe_launch_permute(const int32_t* ids, int P, int E, int32_t* sorted_pair,
                              int32_t* offsets, int32_t* pair_pos, hipStream_t s);
hipError_t moe_launch_combine(const float* y_pairs, const float* w, const int32_t* pair_pos,
                              const float* y_shared, const float* residual, float* out,
                              uint16_t* out_bf16, int T, int H, int k, hipStream_t s);
hipError_t moe_launch_rmsnorm(const float* r, uint16_t* a, int T, int H, float eps,
                              hipStream_t s);
hipError_t moe_launch_stq1_pack(const uint8_t* z, const uint8_t* sg, const uint16_t* d,
                                int64_t n_blocks, uint8_t* codes, uint16_t* scales,
                                hipStream_t s);
hipError_t moe_launch_stq1_encode(const float* x, const float* imatrix, int64_t n_blocks, int K,
                                  int method, uint8_t* codes, uint16_t* scales, hipStream_t s);
hipError_t moe_launch_stq1_dequant(const uint8_t* codes, const uint16_t* scales,
                                   int64_t n_blocks, float* out, hipStream_t s);
hipError_t moe_launch_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                    int K, float* out, hipStream_t s);
hipError_t moe_launch_mx_quant(int64_t rows, int K, const uint16_t* xb, const float* xf,
                               uint8_t* q, uint8_t* sc, hipStream_t s);
hipError_t moe_launch_mx_quant_hw(int64_t rows, int K, const float* xf, uint8_t* q, uint8_t* sc,
                                  hipStream_t s);

// Decode-regime FFN (routed STQ1_0 and shared bf16) on the bf16 MFMA.
// kind: 0 routed gate/up, 1 routed down, 2 shared gate/up, 3 shared down.
struct FfnArgs {
  const void* codes0;
  const void* scales0;
  const void* codes1;
  const void* scales1;
  const void* act;           // bf16 x [*, K] (gate/up) or fp32 h [*, K] (down)
  const int32_t* sorted_pair;
  const int32_t* offsets;
  float* out;
  int N, K, T, E, k, P;
};
hipError_t moe_launch_stq_gateup(const FfnArgs& a, hipStream_t s);
hipError_t moe_launch_stq_down(const FfnArgs& a, hipStream_t s);
hipError_t moe_launch_stq_generic(const FfnArgs& a, int down, hipStream_t s);
hipError_t moe_launch_bf16_gateup(const FfnArgs& a, hipStream_t s);
hipError_t moe_launch_bf16_down(const FfnArgs& a, hipStream_t s);

// Prefill MXFP4 x FP8 grouped GEMMs on the scaled MFMA.
struct MxArgs {
  const uint8_t* wcodes0; const uint8_t* wscales0;   // gate or down
  const uint8_t* wcodes1; const uint8_t* wscales1;   // up
  const uint8_t* aq; const uint8_t* as;              // activations E4M3 + UE8M0
  const int32_t* sorted_pair; const int32_t* offsets;
  uint8_t* hq; uint8_t* hs;                          // gate/up output (E4M3 h)
  float* y;                                          // down output
  int N, K, T, E, k, P;
  int tiled;                                         // weights in the tiled MXFP4 layout
};
hipError_t moe_launch_mx_gateup(const MxArgs& a, hipStream_t s);
hipError_t moe_launch_mxfp4_pack_tiles(const uint8_t* codes, const uint8_t* scales, long rows,
                                       int K, uint8_t* tcodes, uint8_t* tscales, hipStream_t s);

// Prefill grouped GEMMs on the 16-bit MFMA: routed STQ1_0 (fp16) and the bf16 shared expert.
struct G16Args {
  const void* w0; const void* w1;          // STQ1_0 codes or bf16 rows: gate (or down), up
  const uint16_t* s0; const uint16_t* s1;  // STQ1_0 fp16 block scales
  const uint16_t* a;                       // A rows [rows_a][Ka], fp16 (STQ1_0) or bf16
  const int32_t* aexp;                     // STQ1_0: row scale exponents (A = row * 2^aexp)
  const int32_t* sorted_pair;              // routed gate/up: A row of pos = sorted_pair[pos] / k
  const int32_t* offsets;                  // [E+1]; NULL: one expert owning all P rows
  float* out;                              // gate/up: h [P][N]; down: y [P][N]
  int N, K, Ka, rows_a, E, k, P;
};
hipError_t moe_launch_g16_stq_gateup(const G16Args& a, hipStream_t s);
hipError_t moe_launch_g16_stq_down(const G16Args& a, hipStream_t s);
hipError_t moe_launch_g16_bf16_gateup(const G16Args& a, hipStream_t s);
hipError_t moe_launch_g16_bf16_down(const G16Args& a, hipStream_t s);
hipError_t moe_launch_rowscale_f16(const uint16_t* in16, const float* in32, long rows, int C,
                                   int two, uint16_t* out, int32_t* sexp, hipStream_t s);
hipError_t moe_launch_split_bf16(const float* h, long rows, int C, uint16_t* out, hipStream_t s);
hipError_t moe_launch_g16_mx8_gateup(const G16Args& a, hipStream_t s);
hipError_t moe_launch_g16_mx8_down(const G16Args& a, hipStream_t s);
// Rows of bf16 (xb) or fp32 (xf) [rows][K] -> bf16 values of their MX E4M3 quantisation
// (group 32 along K), which bf16 holds exactly.
hipError_t moe_launch_mx_roundtrip_bf16(int64_t rows, int K, const uint16_t* xb, const float* xf,
                                        uint16_t* out, hipStream_t s);

// Compute units of the current device (cached per device).
inline int moe_cu_count() {
  static int n_cu[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (n_cu[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    n_cu[dev] = n;
  }
  return n_cu[dev];
}

// Opt-in kernel timing with HIP events recorded on the launch stream around single kernels.
enum {
  MOE_PROF_DECODE_K1 = 0, MOE_PROF_DECODE_K2 = 1, MOE_PROF_DECODE_K3 = 2, MOE_PROF_DECODE_K4 = 3,
  MOE_PROF_MX_QUANT = 4, MOE_PROF_MX_GATEUP = 5, MOE_PROF_MX_DOWN = 6,
  MOE_PROF_STQ_GATEUP = 7, MOE_PROF_STQ_DOWN = 8, MOE_PROF_SH_GATEUP = 9, MOE_PROF_SH_DOWN = 10,
  MOE_PROF_ACT_PREP = 11,
  MOE_PROF_SLOTS_INTERNAL = 16
};
bool moe_prof_on();
void moe_prof_begin(int slot, hipStream_t s);
void moe_prof_end(int slot, hipStream_t s);

// Fused decode layer (three kernels).
// Bytes of the static scratch array behind moe_layer_decode_noalloc (per device).
constexpr size_t kDecodeStaticScratchBytes = (size_t)8 << 20;
// This device's address of that array (looked up once per device), or nullptr on failure.
void* moe_decode_static_scratch();
// Enqueue a kernel that zeroes the fused decode workspace's header words (the router ticket).
hipError_t moe_clear_decode_header(void* ws, hipStream_t s);
bool moe_decode_shape_ok(int H, int I, int E);
bool moe_decode_mx_ok(int T, int I, int k);
size_t moe_decode_ws_layout(int T, int H, int I, int E, int k, int has_shared, size_t* offs);
hipError_t moe_launch_decode_fused(const moe_dims* d, const moe_experts* routed,
                                   const moe_experts* shared, const uint16_t* x,
                                   const uint16_t* wr, const float* bias, float* logits,
                                   int32_t* ids, float* w, int32_t* sorted_pair,
                                   int32_t* offsets, int32_t* pair_pos, float* y_pairs,
                                   float* y_shared, const float* residual, float* out,
                                   uint16_t* out_bf16, void* ws, hipStream_t s);
hipError_t moe_launch_mx_down(const MxArgs& a, hipStream_t s);
