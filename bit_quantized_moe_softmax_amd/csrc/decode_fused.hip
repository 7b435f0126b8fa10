// Fused decode-regime MoE layer: route -> permute -> expert FFN -> combine in three kernels.
//
// Same computation as the four separate entry points (router in BF16, top-k with
// renormalised softmax weights, stable permutation, SwiGLU experts on STQ1_0 weights,
// one bf16 shared expert, ungated combine); the kernel boundaries are chosen so that the
// work that does not depend on routing overlaps with the router:
//   K1  router GEMV (bf16 MFMA, K split over waves and workgroups) and, in the same grid,
//       the shared expert's gate/up; the last router workgroup to finish (atomic ticket)
//       sums the router partials in a fixed order, picks the top-k, sorts the pairs by
//       expert and writes the work list of active experts.
//   K2  routed gate/up + SiLU*up (STQ1_0, decoded in registers) and the shared expert's
//       down projection.
//   K3  routed down projection; the last workgroup to finish a 128-row slice of the
//       output (atomic counter per slice) combines that slice for every token.
// All sums run in a fixed order, so results do not depend on scheduling.  Counters live
// in the caller's workspace, must be zero before the first call, and are left zero.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16): A row = B column = lane % 16, lane group
// g = lane / 16 supplies K-slots 8g .. 8g+7; D(4g + i, lane % 16) sits in register i.
// K-slot -> K map: STQ1_0 K = 256 b + 64 g + 8 t + s (a lane decodes groups 16g+2t and
// 16g+2t+1 of block b at step t), bf16 weights K = 256 b + 32 t + 8 g + s.  h is stored
// as bf16 hi + bf16 lo (h - hi) so the down projection keeps ~16 bits of h: two MFMAs
// (A*hi + A*lo) into one accumulator.
#include "moe_device.h"

#include <math.h>

namespace {

constexpr int kNW = 8;             // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kMaxB = 8;           // blocks of 256 K per wave (H <= 16384)
constexpr int kRouterWgK = 2;      // router workgroups along K per expert tile
constexpr int kRouterChunks = kNW * kRouterWgK;
constexpr int kDownRows = 16 * kNW;  // output rows per down unit

struct DecodeArgs {
  int T, H, I, E, k;
  const uint8_t* gc; const uint16_t* gs;
  const uint8_t* uc; const uint16_t* us;
  const uint8_t* dc; const uint16_t* ds;
  const uint16_t* sg; const uint16_t* su; const uint16_t* sd;
  const uint16_t* x; const uint16_t* wr; const float* bias;
  float* logits; int32_t* ids; float* w; int32_t* sorted_pair; int32_t* offsets; int32_t* pair_pos;
  float* y_pairs; float* y_shared; const float* residual; float* out; uint16_t* out_bf16;
  int32_t* ctr; int32_t* wl; float* rpart;
  uint16_t* h_hi; uint16_t* h_lo; uint16_t* hs_hi; uint16_t* hs_lo;
  int n_router_wg, n_sgu_wg, n_gu_wg, n_sdn_wg, n_dn_wg;
};

// work list layout (int32): [0] active experts, [1] gate/up units, [2] down units,
// [3] (slot, token tile) units, then E expert ids, E starts, E counts, E+1 prefix of token tiles
__device__ __forceinline__ int* wl_e(int* wl) { return wl + 4; }
__device__ __forceinline__ int* wl_start(int* wl, int E) { return wl + 4 + E; }
__device__ __forceinline__ int* wl_cnt(int* wl, int E) { return wl + 4 + 2 * E; }
__device__ __forceinline__ int* wl_ttp(int* wl, int E) { return wl + 4 + 3 * E; }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_lane(uint32_t p, int j) {
  const int z = p >> 3;
  if (j == z) return 0u;
  const int i = j < z ? j : j - 1;
  return ((p >> i) & 1) ? 0xBF80u : 0x3F80u;
}

__device__ __forceinline__ void build_lut(uint2* lut) {
  const int t = threadIdx.x;
  if (t < 32) lut[t] = make_uint2(bf16_lane(t, 0) | (bf16_lane(t, 1) << 16),
                                  bf16_lane(t, 2) | (bf16_lane(t, 3) << 16));
}

__device__ __forceinline__ bf16x8_t stq_a(const uint2* lut, uint2 qs, uint32_t qh, int t) {
  const uint32_t byte = ((t < 4 ? qs.x : qs.y) >> (8 * (t & 3))) & 0xFFu;
  const uint32_t p0 = (byte & 15u) | (((qh >> (2 * t)) & 1u) << 4);
  const uint32_t p1 = (byte >> 4) | (((qh >> (2 * t + 1)) & 1u) << 4);
  const uint2 l0 = lut[p0];
  const uint2 l1 = lut[p1];
  return as_bf16x8(make_uint4(l0.x, l0.y, l1.x, l1.y));
}

__device__ __forceinline__ void store_h_split(uint16_t* hi, uint16_t* lo, size_t idx, const float h[4]) {
  uint32_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = f32_to_bf16_rne(h[i]);
    b[i] = f32_to_bf16_rne(h[i] - bf16_to_f32(a[i]));
  }
  *reinterpret_cast<uint2*>(hi + idx) = make_uint2(a[0] | (a[1] << 16), a[2] | (a[3] << 16));
  *reinterpret_cast<uint2*>(lo + idx) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
}

// ============================================================================ K1
// Router partial logits for one (expert tile, token tile, K half): wave w takes K chunk
// kw * 8 + w of 16; the 8 waves are summed in LDS in order; partial -> rpart[kw][t][e].
__device__ void router_unit(const DecodeArgs& a, int rw, float (*s_red)[4][64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_et = (a.E + 15) / 16;
  const int kw = rw % kRouterWgK;
  const int et = (rw / kRouterWgK) % n_et;
  const int tt = rw / (kRouterWgK * n_et);
  const int col = lane & 15, g = lane >> 4;
  const int e_row = et * 16 + col;                 // A row = expert
  const int tok = tt * 16 + col;                   // B column = token
  const int KC = a.H / kRouterChunks;              // multiple of 32
  const int k0 = (kw * kNW + wave) * KC;
  const uint16_t* arow = e_row < a.E ? a.wr + (size_t)e_row * a.H + k0 : nullptr;
  const uint16_t* brow = tok < a.T ? a.x + (size_t)tok * a.H + k0 : nullptr;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = KC / 32;
  for (int s0 = 0; s0 < nsteps; s0 += 4) {
    uint4 av[4], bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = s0 + j;
      av[j] = (arow && s < nsteps) ? *reinterpret_cast<const uint4*>(arow + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0);
      bv[j] = (brow && s < nsteps) ? *reinterpret_cast<const uint4*>(brow + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma16(as_bf16x8(av[j]), as_bf16x8(bv[j]), acc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
      for (int w = 0; w < kNW; ++w) v += s_red[w][i][lane];
      const int e = et * 16 + 4 * g + i;        // D row = expert
      if (e < a.E && tok < a.T) a.rpart[((size_t)kw * a.T + tok) * a.E + e] = v;
    }
  }
}

// Order-preserving unsigned key of a float (larger float -> larger key; -0 as +0).
__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of one token by one wave: k-th largest key by a 32-step bitwise search with
// ballots, then the selected slots ordered by (logit desc, expert asc) through LDS.
__device__ void wave_topk(const DecodeArgs& a, int t, float* s_v, int* s_i, int* s_ids) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  const int m = (E + 63) >> 6;
  float v[16];
  uint32_t key[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = i * 64 + lane;
    float val = -INFINITY;
    if (i < m && e < E) {
      val = a.bias ? a.bias[e] : 0.f;
      float s = 0.f;
      for (int kw = 0; kw < kRouterWgK; ++kw) s += a.rpart[((size_t)kw * a.T + t) * E + e];
      val = s + val;
      if (a.logits) a.logits[(size_t)t * E + e] = val;
    }
    v[i] = val;
    key[i] = (i < m && e < E) ? fkey(val) : 0u;
  }
  // k-th largest key
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < m) c += __popcll(__ballot(key[i] >= cand && (i * 64 + lane) < E));
    if (c >= k) thr = cand;
  }
  int greater = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (i < m) greater += __popcll(__ballot(key[i] > thr && (i * 64 + lane) < E));
  const int need_eq = k - greater;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int eq_before = 0, sel_before = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < m) {
      const bool valid = (i * 64 + lane) < E;
      const uint64_t eqm = __ballot(valid && key[i] == thr);
      const bool eq_sel = valid && key[i] == thr && (eq_before + __popcll(eqm & lt)) < need_eq;
      const bool sel = (valid && key[i] > thr) || eq_sel;
      const uint64_t selm = __ballot(sel);
      if (sel) {
        const int slot = sel_before + __popcll(selm & lt);
        s_v[slot] = v[i];
        s_i[slot] = i * 64 + lane;
      }
      eq_before += __popcll(eqm);
      sel_before += __popcll(selm);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
  if (lane < k) {
    const float mv = s_v[lane];
    const int mi = s_i[lane];
    int rank = 0;
    for (int j = 0; j < k; ++j) {
      const float ov = s_v[j];
      const int oi = s_i[j];
      rank += (ov > mv || (ov == mv && oi < mi)) ? 1 : 0;
    }
    float vmax = mv;
    for (int j = 0; j < k; ++j) vmax = fmaxf(vmax, s_v[j]);
    // softmax denominator, summed in the same (expert) order by every lane
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += expf(s_v[j] - vmax);
    a.ids[(size_t)t * k + rank] = mi;
    a.w[(size_t)t * k + rank] = expf(mv - vmax) / sum;
    s_ids[t * k + rank] = mi;
  }
  __builtin_amdgcn_wave_barrier();
}

// The last router workgroup: top-k of every token, stable permutation, work list.
__device__ void route_finalize(const DecodeArgs& a, int* s_ids, float (*s_v)[32], int (*s_i)[32],
                               int* s_cnt, int* s_base, uint8_t (*s_wc)[1024], int* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k, T = a.T, P = T * k;
  for (int t = wave; t < T; t += kNW) wave_topk(a, t, s_v[wave], s_i[wave], s_ids);
  for (int e = tid; e < E; e += kThreads) s_cnt[e] = 0;
  __syncthreads();
  for (int f = tid; f < P; f += kThreads) atomicAdd(&s_cnt[s_ids[f]], 1);
  __syncthreads();
  // exclusive scans over experts (E <= 1024: two values per thread at most)
  int* wl = a.wl;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  {
    // per expert: count, active flag, token tiles
    int c[2], act[2], tti[2];
    int loc_c = 0, loc_a = 0, loc_t = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid * 2 + q;
      c[q] = e < E ? s_cnt[e] : 0;
      act[q] = c[q] > 0;
      tti[q] = (c[q] + 15) / 16;
      loc_c += c[q]; loc_a += act[q]; loc_t += tti[q];
    }
    // wave inclusive scans of the three sums
    int ic = loc_c, ia = loc_a, it = loc_t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int yc = __shfl_up(ic, o, 64), ya = __shfl_up(ia, o, 64), yt = __shfl_up(it, o, 64);
      if (lane >= o) { ic += yc; ia += ya; it += yt; }
    }
    if (lane == 63) { s_wsum[wave * 3 + 0] = ic; s_wsum[wave * 3 + 1] = ia; s_wsum[wave * 3 + 2] = it; }
    __syncthreads();
    int bc = 0, ba = 0, bt = 0, tc = 0, ta = 0, ttot = 0;
    for (int w2 = 0; w2 < kNW; ++w2) {
      if (w2 < wave) { bc += s_wsum[w2 * 3]; ba += s_wsum[w2 * 3 + 1]; bt += s_wsum[w2 * 3 + 2]; }
      tc += s_wsum[w2 * 3]; ta += s_wsum[w2 * 3 + 1]; ttot += s_wsum[w2 * 3 + 2];
    }
    int ec = bc + ic - loc_c, ea = ba + ia - loc_a, et = bt + it - loc_t;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = tid * 2 + q;
      if (e < E) {
        s_base[e] = ec;
        a.offsets[e] = ec;
        if (act[q]) {
          wl_e(wl)[ea] = e;
          wl_start(wl, E)[ea] = ec;
          wl_cnt(wl, E)[ea] = c[q];
          wl_ttp(wl, E)[ea] = et;
        }
      }
      ec += c[q]; ea += act[q]; et += tti[q];
    }
    if (tid == 0) {
      a.offsets[E] = P;
      wl[0] = ta;
      wl[3] = ttot;
      wl[1] = ttot * (a.I / 16);
      wl[2] = ttot * (a.H / kDownRows);
      wl_ttp(wl, E)[ta] = ttot;
    }
  }
  __syncthreads();
  // stable scatter in chunks of kThreads pairs
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  for (int c0 = 0; c0 < P; c0 += kThreads) {
    for (int i = tid; i < kNW * E; i += kThreads) s_wc[i / E][i % E] = 0;
    __syncthreads();
    const int f = c0 + tid;
    const bool valid = f < P;
    const int e = valid ? s_ids[f] : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(valid && bit);
      peers &= bit ? ones : ~ones;
    }
    const int rank = __popcll(peers & lt);
    if (valid && rank == 0) s_wc[wave][e] = (uint8_t)__popcll(peers);
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int w2 = 0; w2 < wave; ++w2) pre += s_wc[w2][e];
      const int pos = s_base[e] + pre + rank;
      a.sorted_pair[pos] = f;
      a.pair_pos[f] = pos;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += kThreads) {
      int s = 0;
      for (int w2 = 0; w2 < kNW; ++w2) s += s_wc[w2][e2];
      s_base[e2] += s;
    }
    __syncthreads();
  }
}

// Shared expert gate/up (bf16): 16 rows of I, token tile of 16, K split over 8 waves.
__device__ void shared_gateup_unit(const DecodeArgs& a, int sw, float (*s_red)[2][4][64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_rt = a.I / 16;
  const int rt = sw % n_rt, tt = sw / n_rt;
  const int row0 = rt * 16;
  const int col = lane & 15, g = lane >> 4;
  const int tok = tt * 16 + col;
  const int H = a.H;
  const int nblk = H / 256;
  const int b0 = wave * nblk / kNW, b1 = (wave + 1) * nblk / kNW;
  const uint16_t* xr = tok < a.T ? a.x + (size_t)tok * H : nullptr;
  const uint16_t* rg = a.sg + (size_t)(row0 + col) * H;
  const uint16_t* ru = a.su + (size_t)(row0 + col) * H;
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  uint4 ng[8], nu[8], nx[8];
  auto load = [&](int b) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int off = 256 * b + 32 * t + 8 * g;
      ng[t] = *reinterpret_cast<const uint4*>(rg + off);
      nu[t] = *reinterpret_cast<const uint4*>(ru + off);
      nx[t] = xr ? *reinterpret_cast<const uint4*>(xr + off) : make_uint4(0, 0, 0, 0);
    }
  };
  if (b0 < b1) load(b0);
  for (int b = b0; b < b1; ++b) {
    uint4 cg[8], cu[8], cx[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) { cg[t] = ng[t]; cu[t] = nu[t]; cx[t] = nx[t]; }
    if (b + 1 < b1) load(b + 1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      accg = mfma16(as_bf16x8(cg[t]), as_bf16x8(cx[t]), accg);
      accu = mfma16(as_bf16x8(cu[t]), as_bf16x8(cx[t]), accu);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) { s_red[wave][0][i][lane] = accg[i]; s_red[wave][1][i][lane] = accu[i]; }
  __syncthreads();
  if (wave == 0 && tok < a.T) {
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float gs = 0.f, us = 0.f;
      for (int w = 0; w < kNW; ++w) { gs += s_red[w][0][i][lane]; us += s_red[w][1][i][lane]; }
      h[i] = gs / (1.0f + expf(-gs)) * us;
    }
    store_h_split(a.hs_hi, a.hs_lo, (size_t)tok * a.I + row0 + 4 * g, h);
  }
}

__global__ __launch_bounds__(kThreads) void k1_route_shared(DecodeArgs a) {
  __shared__ float s_red[kNW][2][4][64];
  __shared__ int s_last;
  __shared__ int s_ids[64 * 32];
  __shared__ float s_v[kNW][32];
  __shared__ int s_i[kNW][32];
  __shared__ int s_cnt[1024];
  __shared__ int s_base[1024];
  __shared__ uint8_t s_wc[kNW][1024];
  __shared__ int s_wsum[kNW * 3];
  if ((int)blockIdx.x >= a.n_router_wg) {
    shared_gateup_unit(a, blockIdx.x - a.n_router_wg, s_red);
    return;
  }
  router_unit(a, blockIdx.x, reinterpret_cast<float(*)[4][64]>(&s_red[0][0][0][0]));
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(&a.ctr[0], 1);
    s_last = (old == a.n_router_wg - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  route_finalize(a, s_ids, s_v, s_i, s_cnt, s_base, s_wc, s_wsum);
  if (threadIdx.x == 0) a.ctr[0] = 0;
}

// ============================================================================ K2
// Locate the (slot, token tile) of unit index ttg through the token-tile prefix.
__device__ __forceinline__ int find_slot(const int* ttp, int n_active, int ttg) {
  int lo = 0, hi = n_active;   // ttp[lo] <= ttg < ttp[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ttp[mid] <= ttg) lo = mid; else hi = mid;
  }
  return lo;
}

// Routed gate/up unit: expert e, 16 rows of I, 16 pairs; 8 waves split K.
__device__ void routed_gateup_unit(const DecodeArgs& a, int u, const uint2* s_lut,
                                   float (*s_sc)[2][kMaxB][16], float (*s_red)[2][4][64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int* wl = a.wl;
  const int E = a.E, I = a.I, H = a.H;
  const int n_rt = I / 16;
  const int ttg = u / n_rt, rt = u % n_rt;
  const int s = find_slot(wl_ttp(wl, E), wl[0], ttg);
  const int e = wl_e(wl)[s];
  const int start = wl_start(wl, E)[s];
  const int cnt = wl_cnt(wl, E)[s];
  const int j0 = (ttg - wl_ttp(wl, E)[s]) * 16;
  const int ntok = min(16, cnt - j0);
  const int row0 = rt * 16;
  const int col = lane & 15, g = lane >> 4;
  const int nblk = H / 256;
  const int b0 = wave * nblk / kNW, b1 = (wave + 1) * nblk / kNW;
  const int nb = b1 - b0;
  const uint16_t* xr = nullptr;
  if (col < ntok) xr = a.x + (size_t)(a.sorted_pair[start + j0 + col] / a.k) * H;
  // prefetch every code word of this wave's blocks
  const size_t rowbytes = (size_t)nblk * 40;
  const uint8_t* rg = a.gc + ((size_t)e * I + row0 + col) * rowbytes;
  const uint8_t* ru = a.uc + ((size_t)e * I + row0 + col) * rowbytes;
  uint2 qg[kMaxB], qu[kMaxB];
  uint32_t hg[kMaxB], hu[kMaxB];
#pragma unroll
  for (int j = 0; j < kMaxB; ++j) {
    if (j < nb) {
      const int b = b0 + j;
      qg[j] = *reinterpret_cast<const uint2*>(rg + b * 40 + 8 * g);
      hg[j] = *reinterpret_cast<const uint16_t*>(rg + b * 40 + 32 + 2 * g);
      qu[j] = *reinterpret_cast<const uint2*>(ru + b * 40 + 8 * g);
      hu[j] = *reinterpret_cast<const uint16_t*>(ru + b * 40 + 32 + 2 * g);
    }
  }
  // block scales of the 16 rows, wave-private LDS
  for (int i = lane; i < nb * 16; i += 64) {
    const int bl = i >> 4, r = i & 15;
    const size_t idx = ((size_t)e * I + row0 + r) * nblk + b0 + bl;
    s_sc[wave][0][bl][r] = fp16_to_f32(a.gs[idx]);
    s_sc[wave][1][bl][r] = fp16_to_f32(a.us[idx]);
  }
  uint4 nx[8];
  auto loadx = [&](int b) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      nx[t] = xr ? *reinterpret_cast<const uint4*>(xr + 256 * b + 64 * g + 8 * t) : make_uint4(0, 0, 0, 0);
  };
  if (nb > 0) loadx(b0);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kMaxB; ++j) {
    if (j < nb) {
      uint4 cx[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) cx[t] = nx[t];
      if (j + 1 < nb) loadx(b0 + j + 1);
      f32x4_t bg = {0.f, 0.f, 0.f, 0.f}, bu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8_t bx = as_bf16x8(cx[t]);
        bg = mfma16(stq_a(s_lut, qg[j], hg[j], t), bx, bg);
        bu = mfma16(stq_a(s_lut, qu[j], hu[j], t), bx, bu);
      }
      const float4 dg = *reinterpret_cast<const float4*>(&s_sc[wave][0][j][4 * g]);
      const float4 du = *reinterpret_cast<const float4*>(&s_sc[wave][1][j][4 * g]);
      accg[0] = fmaf(dg.x, bg[0], accg[0]); accg[1] = fmaf(dg.y, bg[1], accg[1]);
      accg[2] = fmaf(dg.z, bg[2], accg[2]); accg[3] = fmaf(dg.w, bg[3], accg[3]);
      accu[0] = fmaf(du.x, bu[0], accu[0]); accu[1] = fmaf(du.y, bu[1], accu[1]);
      accu[2] = fmaf(du.z, bu[2], accu[2]); accu[3] = fmaf(du.w, bu[3], accu[3]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) { s_red[wave][0][i][lane] = accg[i]; s_red[wave][1][i][lane] = accu[i]; }
  __syncthreads();
  if (wave == 0 && col < ntok) {
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float gs = 0.f, us = 0.f;
      for (int w = 0; w < kNW; ++w) { gs += s_red[w][0][i][lane]; us += s_red[w][1][i][lane]; }
      h[i] = gs / (1.0f + expf(-gs)) * us;
    }
    store_h_split(a.h_hi, a.h_lo, (size_t)(start + j0 + col) * I + row0 + 4 * g, h);
  }
  __syncthreads();   // s_red / s_sc are reused by the next unit
}

// Shared expert down (bf16): 16 rows of H, token tile of 16, K = I split over 8 waves.
__device__ void shared_down_unit(const DecodeArgs& a, int sd, float (*s_red)[2][4][64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_rt = a.H / 16;
  const int rt = sd % n_rt, tt = sd / n_rt;
  const int row0 = rt * 16;
  const int col = lane & 15, g = lane >> 4;
  const int tok = tt * 16 + col;
  const int I = a.I;
  const int nblk = I / 256;
  const int b0 = wave * nblk / kNW, b1 = (wave + 1) * nblk / kNW;
  const uint16_t* hh = tok < a.T ? a.hs_hi + (size_t)tok * I : nullptr;
  const uint16_t* hl = tok < a.T ? a.hs_lo + (size_t)tok * I : nullptr;
  const uint16_t* rd = a.sd + (size_t)(row0 + col) * I;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int b = b0; b < b1; ++b) {
    uint4 wv[8], bh[8], bl[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int off = 256 * b + 32 * t + 8 * g;
      wv[t] = *reinterpret_cast<const uint4*>(rd + off);
      bh[t] = hh ? *reinterpret_cast<const uint4*>(hh + off) : make_uint4(0, 0, 0, 0);
      bl[t] = hl ? *reinterpret_cast<const uint4*>(hl + off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc = mfma16(as_bf16x8(wv[t]), as_bf16x8(bh[t]), acc);
      acc = mfma16(as_bf16x8(wv[t]), as_bf16x8(bl[t]), acc);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[wave][0][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0 && tok < a.T) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
      for (int w = 0; w < kNW; ++w) v += s_red[w][0][i][lane];
      y[i] = v;
    }
    *reinterpret_cast<float4*>(a.y_shared + (size_t)tok * a.H + row0 + 4 * g) = make_float4(y[0], y[1], y[2], y[3]);
  }
}

__global__ __launch_bounds__(kThreads) void k2_gateup(DecodeArgs a) {
  __shared__ uint2 s_lut[32];
  __shared__ __align__(16) float s_sc[kNW][2][kMaxB][16];
  __shared__ __align__(16) float s_red[kNW][2][4][64];
  if ((int)blockIdx.x < a.n_sdn_wg) {
    shared_down_unit(a, blockIdx.x, s_red);
    return;
  }
  build_lut(s_lut);
  __syncthreads();
  const int n_units = a.wl[1];
  for (int u = blockIdx.x - a.n_sdn_wg; u < n_units; u += a.n_gu_wg)
    routed_gateup_unit(a, u, s_lut, s_sc, s_red);
}

// ============================================================================ K3
// Routed down unit: expert e, 128 rows of H (16 per wave, full K), 16 pairs.
__device__ void routed_down_unit(const DecodeArgs& a, int u, const uint2* s_lut,
                                 float (*s_scd)[kMaxB][16], int rt128, int ttg) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int* wl = a.wl;
  const int E = a.E, I = a.I, H = a.H;
  const int s = find_slot(wl_ttp(wl, E), wl[0], ttg);
  const int e = wl_e(wl)[s];
  const int start = wl_start(wl, E)[s];
  const int cnt = wl_cnt(wl, E)[s];
  const int j0 = (ttg - wl_ttp(wl, E)[s]) * 16;
  const int ntok = min(16, cnt - j0);
  const int row0 = rt128 * kDownRows + 16 * wave;
  const int col = lane & 15, g = lane >> 4;
  const int nblk = I / 256;                       // <= kMaxB
  const size_t rowbytes = (size_t)nblk * 40;
  const uint8_t* rd = a.dc + ((size_t)e * H + row0 + col) * rowbytes;
  uint2 q[kMaxB];
  uint32_t qh[kMaxB];
#pragma unroll
  for (int j = 0; j < kMaxB; ++j) {
    if (j < nblk) {
      q[j] = *reinterpret_cast<const uint2*>(rd + j * 40 + 8 * g);
      qh[j] = *reinterpret_cast<const uint16_t*>(rd + j * 40 + 32 + 2 * g);
    }
  }
  for (int i = lane; i < nblk * 16; i += 64) {
    const int bl = i >> 4, r = i & 15;
    s_scd[wave][bl][r] = fp16_to_f32(a.ds[((size_t)e * H + row0 + r) * nblk + bl]);
  }
  const uint16_t* hh = nullptr;
  const uint16_t* hl = nullptr;
  if (col < ntok) {
    hh = a.h_hi + (size_t)(start + j0 + col) * I;
    hl = a.h_lo + (size_t)(start + j0 + col) * I;
  }
  uint4 nh[8], nl[8];
  auto loadh = [&](int b) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int off = 256 * b + 64 * g + 8 * t;
      nh[t] = hh ? *reinterpret_cast<const uint4*>(hh + off) : make_uint4(0, 0, 0, 0);
      nl[t] = hl ? *reinterpret_cast<const uint4*>(hl + off) : make_uint4(0, 0, 0, 0);
    }
  };
  loadh(0);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kMaxB; ++j) {
    if (j < nblk) {
      uint4 ch[8], cl[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) { ch[t] = nh[t]; cl[t] = nl[t]; }
      if (j + 1 < nblk) loadh(j + 1);
      f32x4_t bacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8_t av = stq_a(s_lut, q[j], qh[j], t);
        bacc = mfma16(av, as_bf16x8(ch[t]), bacc);
        bacc = mfma16(av, as_bf16x8(cl[t]), bacc);
      }
      const float4 d = *reinterpret_cast<const float4*>(&s_scd[wave][j][4 * g]);
      acc[0] = fmaf(d.x, bacc[0], acc[0]); acc[1] = fmaf(d.y, bacc[1], acc[1]);
      acc[2] = fmaf(d.z, bacc[2], acc[2]); acc[3] = fmaf(d.w, bacc[3], acc[3]);
    }
  }
  if (col < ntok)
    *reinterpret_cast<float4*>(a.y_pairs + (size_t)(start + j0 + col) * H + row0 + 4 * g) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
}

// out[t][rows] = y_shared + sum_j w * y_pairs[pair_pos] (+ residual) for one 128-row slice.
__device__ void combine_slice(const DecodeArgs& a, int rt128) {
  const int H = a.H, k = a.k;
  const int r0 = rt128 * kDownRows;
  for (int idx = threadIdx.x; idx < a.T * (kDownRows / 4); idx += kThreads) {
    const int t = idx / (kDownRows / 4);
    const int h = r0 + (idx % (kDownRows / 4)) * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.y_shared) acc = *reinterpret_cast<const float4*>(a.y_shared + (size_t)t * H + h);
    for (int j = 0; j < k; ++j) {
      const float wj = a.w[(size_t)t * k + j];
      const int pos = a.pair_pos[(size_t)t * k + j];
      const float4 y = *reinterpret_cast<const float4*>(a.y_pairs + (size_t)pos * H + h);
      acc.x = fmaf(wj, y.x, acc.x); acc.y = fmaf(wj, y.y, acc.y);
      acc.z = fmaf(wj, y.z, acc.z); acc.w = fmaf(wj, y.w, acc.w);
    }
    if (a.residual) {
      const float4 r = *reinterpret_cast<const float4*>(a.residual + (size_t)t * H + h);
      acc.x += r.x; acc.y += r.y; acc.z += r.z; acc.w += r.w;
    }
    *reinterpret_cast<float4*>(a.out + (size_t)t * H + h) = acc;
    if (a.out_bf16) {
      uint2 b;
      b.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
      b.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
      *reinterpret_cast<uint2*>(a.out_bf16 + (size_t)t * H + h) = b;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k3_down_combine(DecodeArgs a) {
  __shared__ uint2 s_lut[32];
  __shared__ __align__(16) float s_scd[kNW][kMaxB][16];
  __shared__ int s_last;
  build_lut(s_lut);
  __syncthreads();
  const int n_units = a.wl[2];
  const int n_tt = a.wl[3];
  const int n_rt = a.H / kDownRows;
  for (int u = blockIdx.x; u < n_units; u += a.n_dn_wg) {
    const int ttg = u / n_rt, rt128 = u % n_rt;
    routed_down_unit(a, u, s_lut, s_scd, rt128, ttg);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int old = atomicAdd(&a.ctr[1 + rt128], 1);
      s_last = (old == n_tt - 1);
    }
    __syncthreads();
    if (s_last) {
      __threadfence();
      combine_slice(a, rt128);
      if (threadIdx.x == 0) a.ctr[1 + rt128] = 0;
    }
    __syncthreads();
  }
}

}  // namespace

// ---------------------------------------------------------------------------- host side
size_t moe_decode_ws_layout(int T, int H, int I, int E, int k, int has_shared, size_t* offs) {
  const size_t P = (size_t)T * k;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t cur = 0;
  offs[0] = cur; cur = al(cur + (1 + H / kDownRows + 1) * sizeof(int32_t));     // counters
  offs[1] = cur; cur = al(cur + (4 + 4 * (size_t)E + 1) * sizeof(int32_t));      // work list
  offs[2] = cur; cur = al(cur + (size_t)kRouterWgK * T * E * sizeof(float));    // router partials
  offs[3] = cur; cur = al(cur + P * I * 2);                                      // h hi
  offs[4] = cur; cur = al(cur + P * I * 2);                                      // h lo
  offs[5] = cur; cur = al(cur + (has_shared ? (size_t)T * I * 2 : 0));           // shared h hi
  offs[6] = cur; cur = al(cur + (has_shared ? (size_t)T * I * 2 : 0));           // shared h lo
  offs[7] = cur;
  return cur;
}

hipError_t moe_launch_decode_fused(const moe_dims* d, const moe_experts* routed,
                                   const moe_experts* shared, const uint16_t* x,
                                   const uint16_t* wr, const float* bias, float* logits,
                                   int32_t* ids, float* w, int32_t* sorted_pair,
                                   int32_t* offsets, int32_t* pair_pos, float* y_pairs,
                                   float* y_shared, const float* residual, float* out,
                                   uint16_t* out_bf16, void* ws, hipStream_t s) {
  DecodeArgs a{};
  a.T = d->T; a.H = d->H; a.I = d->I; a.E = d->E; a.k = d->k;
  a.gc = static_cast<const uint8_t*>(routed->gate.codes); a.gs = static_cast<const uint16_t*>(routed->gate.scales);
  a.uc = static_cast<const uint8_t*>(routed->up.codes);   a.us = static_cast<const uint16_t*>(routed->up.scales);
  a.dc = static_cast<const uint8_t*>(routed->down.codes); a.ds = static_cast<const uint16_t*>(routed->down.scales);
  if (shared) {
    a.sg = static_cast<const uint16_t*>(shared->gate.codes);
    a.su = static_cast<const uint16_t*>(shared->up.codes);
    a.sd = static_cast<const uint16_t*>(shared->down.codes);
  }
  a.x = x; a.wr = wr; a.bias = bias; a.logits = logits; a.ids = ids; a.w = w;
  a.sorted_pair = sorted_pair; a.offsets = offsets; a.pair_pos = pair_pos;
  a.y_pairs = y_pairs; a.y_shared = shared ? y_shared : nullptr; a.residual = residual;
  a.out = out; a.out_bf16 = out_bf16;
  size_t offs[8];
  moe_decode_ws_layout(a.T, a.H, a.I, a.E, a.k, shared != nullptr, offs);
  uint8_t* b = static_cast<uint8_t*>(ws);
  a.ctr = reinterpret_cast<int32_t*>(b + offs[0]);
  a.wl = reinterpret_cast<int32_t*>(b + offs[1]);
  a.rpart = reinterpret_cast<float*>(b + offs[2]);
  a.h_hi = reinterpret_cast<uint16_t*>(b + offs[3]);
  a.h_lo = reinterpret_cast<uint16_t*>(b + offs[4]);
  a.hs_hi = reinterpret_cast<uint16_t*>(b + offs[5]);
  a.hs_lo = reinterpret_cast<uint16_t*>(b + offs[6]);
  const int T = a.T, P = a.T * a.k;
  const int n_tt = (T + 15) / 16;
  const int max_slot_tiles = (P < a.E ? P : a.E) + (P + 15) / 16;
  a.n_router_wg = ((a.E + 15) / 16) * kRouterWgK * n_tt;
  a.n_sgu_wg = shared ? (a.I / 16) * n_tt : 0;
  a.n_sdn_wg = shared ? (a.H / 16) * n_tt : 0;
  const int cap = 4096;
  a.n_gu_wg = max_slot_tiles * (a.I / 16) < cap ? max_slot_tiles * (a.I / 16) : cap;
  a.n_dn_wg = max_slot_tiles * (a.H / kDownRows) < cap ? max_slot_tiles * (a.H / kDownRows) : cap;
  const bool prof = moe_prof_on();
  if (prof) moe_prof_begin(MOE_PROF_DECODE_K1, s);
  hipLaunchKernelGGL(k1_route_shared, dim3(a.n_router_wg + a.n_sgu_wg), dim3(kThreads), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K1, s); moe_prof_begin(MOE_PROF_DECODE_K2, s); }
  hipLaunchKernelGGL(k2_gateup, dim3(a.n_sdn_wg + a.n_gu_wg), dim3(kThreads), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K2, s); moe_prof_begin(MOE_PROF_DECODE_K3, s); }
  hipLaunchKernelGGL(k3_down_combine, dim3(a.n_dn_wg), dim3(kThreads), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) moe_prof_end(MOE_PROF_DECODE_K3, s);
  return hipSuccess;
}
