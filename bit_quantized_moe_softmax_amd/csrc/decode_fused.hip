// Fused decode-regime MoE layer: route -> permute -> expert FFN -> combine in three kernels.
//
// Same computation as the four separate entry points (router in BF16, top-k with
// renormalised softmax weights, stable permutation, SwiGLU experts on STQ1_0 weights,
// one bf16 shared expert, ungated combine).  Work that does not depend on routing runs
// beside the router:
//   K1  router logits (bf16 MFMA; a workgroup sums four K chunks of 16 experts in LDS and
//       writes one partial) beside the shared expert's gate/up + SiLU*up.  The last router
//       workgroup to finish (atomic ticket, one release fence per router workgroup) sums
//       the partials in a fixed order, picks the top-k, sorts the pairs by expert and writes
//       the unit table: (expert, first pair, pairs <= 16) with each pair's token and weight;
//   K2  routed gate/up + SiLU*up (STQ1_0 decoded in registers, bf16 MFMA) beside the shared
//       expert's down projection;
//   K3  routed down projection per 16-row slice of the output, every unit of the slice in
//       one workgroup (8 waves), weighted into per-wave LDS sums and combined with the
//       shared expert (and the residual) in a fixed order.
// Every sum runs in a fixed order, so results do not depend on scheduling.  The ticket
// counter lives in the workspace: zero before the first call, left zero by every call.
// The kernels are instantiated per (H/256, I/256) so every loop over K has a fixed trip
// count: a wave's loads are issued without branches and stay in flight together.  Rows a
// lane does not need (a token column past the unit's last pair) are read from a valid row
// and zeroed by a select rather than skipped.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16): A row = B column = lane % 16, lane group
// g = lane / 16 supplies K-slots 8g .. 8g+7; D(4g + i, lane % 16) sits in register i.
// K-slot -> K map: STQ1_0 K = 256 b + 64 g + 8 t + s (a lane decodes groups 16g+2t and
// 16g+2t+1 of block b at step t from the 8 code bytes and 16 high bits it loads);
// router K = k0 + 32 t + 8 g + s.  The routed h is stored as bf16 hi + bf16 lo (h - hi) so
// the down projection keeps ~16 bits of h with two MFMAs (A*hi + A*lo) into one sum.
// For up to four tokens the shared expert (plain bf16 GEMV, 75 MB of weights at Hy4
// shape) runs on the VALU with one wave per row and every load of the row in flight;
// beyond that it uses the MFMA with the K axis split over the workgroup's waves.
#include "moe_device.h"

#include <math.h>

namespace {

constexpr int kWG = 256;           // 4 waves
constexpr int kNW = 4;
constexpr int kRouterChunks = 16;  // router K chunks, 4 per workgroup
constexpr int kRouterParts = kRouterChunks / kNW;
constexpr int kSmallT = 4;         // shared expert on the VALU up to this many tokens
constexpr int kMaxT = 64;
constexpr int kMaxE = 256;
constexpr int kDnWaves = 8;        // waves of a routed-down workgroup

struct DecodeArgs {
  int T, E, k;
  const uint8_t* gc; const uint16_t* gs;
  const uint8_t* uc; const uint16_t* us;
  const uint8_t* dc; const uint16_t* ds;
  const uint16_t* sg; const uint16_t* su; const uint16_t* sd;
  const uint16_t* x; const uint16_t* wr; const float* bias;
  float* logits; int32_t* ids; float* w; int32_t* sorted_pair; int32_t* offsets; int32_t* pair_pos;
  float* y_pairs; float* y_shared; const float* residual; float* out; uint16_t* out_bf16;
  int32_t* wl;      // [0] active experts, [1] units
  int32_t* ctr;     // [0] router ticket (zero between calls)
  int4* ut;         // units: {expert, first sorted position, pairs (<= 16), 0}
  int32_t* utok;    // [unit][16] token of each pair of the unit
  float* uw;        // [unit][16] routing weight of each pair of the unit
  float* rpart;     // [kRouterParts][T][E]
  uint16_t* h_hi; uint16_t* h_lo;   // [P][I]
  float* hs;        // shared h [T][I]
  int n_router_wg, n_sgu_wg, n_gu_wg, n_sdn_wg;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint4 keep_if(bool ok, uint4 v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
// fp32 += a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float dot8(uint4 a, uint4 b, float c) {
  c = dot2(a.x, b.x, c);
  c = dot2(a.y, b.y, c);
  c = dot2(a.z, b.z, c);
  return dot2(a.w, b.w, c);
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

// The 8 A operands of one STQ1_0 block (8 code bytes + 16 high bits of this lane): all 16
// table reads are issued before any is used.
__device__ __forceinline__ void stq_block_a(const uint2* lut, uint2 qs, uint32_t qh, bf16x8_t* av) {
  uint2 l[16];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t byte = ((t < 4 ? qs.x : qs.y) >> (8 * (t & 3))) & 0xFFu;
    l[2 * t] = lut[(byte & 15u) | (((qh >> (2 * t)) & 1u) << 4)];
    l[2 * t + 1] = lut[(byte >> 4) | (((qh >> (2 * t + 1)) & 1u) << 4)];
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) av[t] = as_bf16x8(make_uint4(l[2 * t].x, l[2 * t].y, l[2 * t + 1].x, l[2 * t + 1].y));
}

__device__ __forceinline__ void wave_fence_lds() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

// ============================================================================ K1
// Router partial for one (16 experts, 16 tokens, quarter of K): wave w takes K chunk
// 4 q + w of 16 with every load up front; the four waves meet in LDS in order and wave 0
// writes rpart[q][t][e].
template <int HB>
__device__ void router_unit(const DecodeArgs& a, int rw, float (*s_red)[4][64]) {
  constexpr int H = HB * 256, KC = H / kRouterChunks, NS = KC / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_et = (a.E + 15) / 16;
  const int q = rw % kRouterParts;
  const int et = (rw / kRouterParts) % n_et;
  const int tt = rw / (kRouterParts * n_et);
  const int c = q * kNW + wave;
  const int col = lane & 15, g = lane >> 4;
  const bool e_ok = et * 16 + col < a.E;
  const bool t_ok = tt * 16 + col < a.T;
  const uint16_t* arow = a.wr + (size_t)(e_ok ? et * 16 + col : 0) * H + c * KC + 8 * g;
  const uint16_t* brow = a.x + (size_t)(t_ok ? tt * 16 + col : 0) * H + c * KC + 8 * g;
  uint4 av[NS], bv[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    av[j] = *reinterpret_cast<const uint4*>(arow + 32 * j);
    bv[j] = *reinterpret_cast<const uint4*>(brow + 32 * j);
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NS; ++j) acc = mfma16(as_bf16x8(keep_if(e_ok, av[j])), as_bf16x8(keep_if(t_ok, bv[j])), acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0 && t_ok) {
    const int tok = tt * 16 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = et * 16 + 4 * g + i;
      const float v = ((s_red[0][i][lane] + s_red[1][i][lane]) + s_red[2][i][lane]) + s_red[3][i][lane];
      if (e < a.E) a.rpart[((size_t)q * a.T + tok) * a.E + e] = v;
    }
  }
}

// Shared gate/up for up to kSmallT tokens: 2 rows per workgroup, wave = (row, gate|up);
// lane l reads the row at K = 8 l + 512 j, all loads of the row in flight at once.
template <int HB, int IB>
__device__ void shared_gateup_valu(const DecodeArgs& a, int sw, float (*s_gu)[2][kSmallT]) {
  constexpr int H = HB * 256, I = IB * 256, NJ = H / 512;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = wave >> 1, mat = wave & 1;
  const int row = sw * 2 + rl;
  const uint16_t* wrow = (mat ? a.su : a.sg) + (size_t)row * H + 8 * lane;
  uint4 wv[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) wv[j] = *reinterpret_cast<const uint4*>(wrow + 512 * j);
  float acc[kSmallT] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) {
    if (t < a.T) {
      const uint16_t* xr = a.x + (size_t)t * H + 8 * lane;
      uint4 xv[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) xv[j] = *reinterpret_cast<const uint4*>(xr + 512 * j);
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[t] = dot8(wv[j], xv[j], acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0) s_gu[rl][mat][t] = v;
  }
  __syncthreads();
  if (threadIdx.x < 2 * kSmallT) {
    const int r = threadIdx.x / kSmallT, t = threadIdx.x % kSmallT;
    if (t < a.T) {
      const float gv = s_gu[r][0][t], uv = s_gu[r][1][t];
      a.hs[(size_t)t * I + sw * 2 + r] = gv / (1.0f + expf(-gv)) * uv;
    }
  }
}

// Shared gate/up beyond kSmallT tokens: 16 rows x 16 tokens, the 4 waves split K.
template <int HB, int IB>
__device__ void shared_gateup_mfma(const DecodeArgs& a, int sw, float (*s_red)[2][4][64]) {
  constexpr int H = HB * 256, I = IB * 256, n_rt = I / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rt = sw % n_rt, tt = sw / n_rt;
  const int row0 = rt * 16;
  const int col = lane & 15, g = lane >> 4;
  const int tok = tt * 16 + col;
  const bool t_ok = tok < a.T;
  const int b0 = wave * HB / kNW, b1 = (wave + 1) * HB / kNW;
  const uint16_t* xr = a.x + (size_t)(t_ok ? tok : 0) * H;
  const uint16_t* rg = a.sg + (size_t)(row0 + col) * H;
  const uint16_t* ru = a.su + (size_t)(row0 + col) * H;
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  for (int b = b0; b < b1; ++b) {
    uint4 cg[8], cu[8], cx[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int off = 256 * b + 32 * t + 8 * g;
      cg[t] = *reinterpret_cast<const uint4*>(rg + off);
      cu[t] = *reinterpret_cast<const uint4*>(ru + off);
      cx[t] = *reinterpret_cast<const uint4*>(xr + off);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const bf16x8_t bx = as_bf16x8(keep_if(t_ok, cx[t]));
      accg = mfma16(as_bf16x8(cg[t]), bx, accg);
      accu = mfma16(as_bf16x8(cu[t]), bx, accu);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) { s_red[wave][0][i][lane] = accg[i]; s_red[wave][1][i][lane] = accu[i]; }
  __syncthreads();
  if (wave == 0 && t_ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float gs = 0.f, us = 0.f;
      for (int w = 0; w < kNW; ++w) { gs += s_red[w][0][i][lane]; us += s_red[w][1][i][lane]; }
      a.hs[(size_t)tok * I + row0 + 4 * g + i] = gs / (1.0f + expf(-gs)) * us;
    }
  }
}

// Order-preserving unsigned key of a float (larger float -> larger key; -0 as +0).
__device__ __forceinline__ uint32_t fkey(float f) {
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of one token by one wave (E <= 256: four logits per lane): the k-th largest key by a
// 32-step bitwise search with ballots, then the chosen slots ordered by (logit desc,
// expert asc) through LDS.
__device__ void wave_topk(const DecodeArgs& a, int t, float* s_v, int* s_i, int* s_ids) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  float part[4][kRouterParts];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = i * 64 + lane < E ? i * 64 + lane : 0;
#pragma unroll
    for (int c = 0; c < kRouterParts; ++c) part[i][c] = a.rpart[((size_t)c * a.T + t) * E + e];
  }
  float v[4];
  uint32_t key[4];
  bool valid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = i * 64 + lane;
    valid[i] = e < E;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kRouterParts; ++c) s += part[i][c];
    if (a.bias && valid[i]) s += a.bias[e];
    v[i] = s;
    if (valid[i]) a.logits[(size_t)t * E + e] = s;
    key[i] = valid[i] ? fkey(s) : 0u;
  }
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int c = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) c += __popcll(__ballot(valid[i] && key[i] >= cand));
    if (c >= k) thr = cand;
  }
  int greater = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) greater += __popcll(__ballot(valid[i] && key[i] > thr));
  const int need_eq = k - greater;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int eq_before = 0, sel_before = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool eq = valid[i] && key[i] == thr;
    const uint64_t eqm = __ballot(eq);
    const bool sel = (valid[i] && key[i] > thr) || (eq && (eq_before + __popcll(eqm & lt)) < need_eq);
    const uint64_t selm = __ballot(sel);
    if (sel) {
      const int slot = sel_before + __popcll(selm & lt);
      s_v[slot] = v[i];
      s_i[slot] = i * 64 + lane;
    }
    eq_before += __popcll(eqm);
    sel_before += __popcll(selm);
  }
  wave_fence_lds();
  if (lane < k) {
    const float mv = s_v[lane];
    const int mi = s_i[lane];
    int rank = 0;
    float vmax = mv;
    for (int j = 0; j < k; ++j) {
      const float ov = s_v[j];
      const int oi = s_i[j];
      rank += (ov > mv || (ov == mv && oi < mi)) ? 1 : 0;
      vmax = fmaxf(vmax, ov);
    }
    float sum = 0.f;   // the same (expert) order in every lane
    for (int j = 0; j < k; ++j) sum += expf(s_v[j] - vmax);
    a.ids[(size_t)t * k + rank] = mi;
    a.w[(size_t)t * k + rank] = expf(mv - vmax) / sum;
    s_ids[t * k + rank] = mi;
  }
  wave_fence_lds();
}


// Routing of all tokens by the last router workgroup (4 waves): top-k per token, stable
// permutation of the pairs by expert (E <= 256: one expert per thread), unit table.
__device__ void route_finalize(const DecodeArgs& a, int* s_ids, float (*s_v)[32], int (*s_i)[32],
                               int* s_cnt, int* s_base, uint8_t (*s_wc)[kMaxE], int* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k, T = a.T, P = T * k;
  for (int t = wave; t < T; t += kNW) wave_topk(a, t, s_v[wave], s_i[wave], s_ids);
  if (tid < E) s_cnt[tid] = 0;
  __syncthreads();
  for (int f = tid; f < P; f += kWG) atomicAdd(&s_cnt[s_ids[f]], 1);
  __syncthreads();
  const int c = tid < E ? s_cnt[tid] : 0;
  const int nt = (c + 15) / 16;
  int ic = c, iu = nt, ia = c > 0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int yc = __shfl_up(ic, o, 64), yu = __shfl_up(iu, o, 64), ya = __shfl_up(ia, o, 64);
    if (lane >= o) { ic += yc; iu += yu; ia += ya; }
  }
  if (lane == 63) { s_wsum[wave * 3] = ic; s_wsum[wave * 3 + 1] = iu; s_wsum[wave * 3 + 2] = ia; }
  __syncthreads();
  int bc = 0, bu = 0, tu = 0, ta = 0;
  for (int w2 = 0; w2 < kNW; ++w2) {
    if (w2 < wave) { bc += s_wsum[w2 * 3]; bu += s_wsum[w2 * 3 + 1]; }
    tu += s_wsum[w2 * 3 + 1]; ta += s_wsum[w2 * 3 + 2];
  }
  const int start = bc + ic - c;
  const int u0 = bu + iu - nt;
  if (tid < E) {
    s_base[tid] = start;
    a.offsets[tid] = start;
  }
  if (tid == 0) {
    a.offsets[E] = P;
    a.wl[0] = ta;
    a.wl[1] = tu;
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  for (int c0 = 0; c0 < P; c0 += kWG) {
    for (int i = tid; i < kNW * kMaxE; i += kWG) s_wc[i / kMaxE][i % kMaxE] = 0;
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
      s_ids[kMaxT * 32 + pos] = f;     // sorted order, for the unit table below
    }
    __syncthreads();
    if (tid < E) {
      int s = 0;
      for (int w2 = 0; w2 < kNW; ++w2) s += s_wc[w2][tid];
      s_base[tid] += s;
    }
    __syncthreads();
  }
  // unit table: unit u0 + q of expert tid covers sorted positions start + 16 q ..
  if (tid < E) {
    for (int q = 0; q < nt; ++q) {
      const int n = min(16, c - 16 * q);
      const int p0 = start + 16 * q;
      a.ut[u0 + q] = make_int4(tid, p0, n, 0);
      for (int j = 0; j < 16; ++j) {
        const int f = s_ids[kMaxT * 32 + p0 + (j < n ? j : 0)];
        a.utok[(u0 + q) * 16 + j] = f / k;
        a.uw[(u0 + q) * 16 + j] = j < n ? a.w[f] : 0.f;
      }
    }
  }
}

template <int HB, int IB>
__global__ __launch_bounds__(kWG) void k1_router_shared(DecodeArgs a) {
  __shared__ float s_red[kNW][2][4][64];
  __shared__ float s_gu[2][2][kSmallT];
  __shared__ int s_last;
  __shared__ int s_ids[2 * kMaxT * 32];
  __shared__ float s_v[kNW][32];
  __shared__ int s_i[kNW][32];
  __shared__ int s_cnt[kMaxE];
  __shared__ int s_base[kMaxE];
  __shared__ uint8_t s_wc[kNW][kMaxE];
  __shared__ int s_wsum[kNW * 3];
  const int b = blockIdx.x;
  if (b >= a.n_router_wg) {
    if (a.T <= kSmallT) shared_gateup_valu<HB, IB>(a, b - a.n_router_wg, s_gu);
    else shared_gateup_mfma<HB, IB>(a, b - a.n_router_wg, s_red);
    return;
  }
  router_unit<HB>(a, b, reinterpret_cast<float(*)[4][64]>(&s_red[0][0][0][0]));
  if (threadIdx.x < 64) {
    __threadfence();     // wave 0 wrote this workgroup's partial: publish it device-wide
    if (threadIdx.x == 0) s_last = atomicAdd(&a.ctr[0], 1) == a.n_router_wg - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  route_finalize(a, s_ids, s_v, s_i, s_cnt, s_base, s_wc, s_wsum);
  if (threadIdx.x == 0) a.ctr[0] = 0;
}

// ============================================================================ K2
// Routed gate/up unit: 16 rows of I for one unit (expert, <= 16 pairs); wave = (gate|up,
// K half), every code word of the wave's blocks loaded up front, x one block ahead.
template <int HB, int IB>
__device__ void routed_gateup_unit(const DecodeArgs& a, int u, const uint2* s_lut,
                                   float (*s_sc)[HB / 2][16], float (*s_red)[4][64]) {
  constexpr int H = HB * 256, I = IB * 256, n_rt = I / 16, NB = HB / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int un_i = u / n_rt;
  const int4 un = a.ut[un_i];
  const int rt = u % n_rt;
  const int e = un.x, pos0 = un.y, ntok = un.z;
  const int row0 = rt * 16;
  const int col = lane & 15, g = lane >> 4;
  const int tok = a.utok[un_i * 16 + col];
  const int mat = wave & 1, b0 = (wave >> 1) * NB;
  const uint8_t* codes = mat ? a.uc : a.gc;
  const uint16_t* scales = mat ? a.us : a.gs;
  const uint8_t* rp = codes + ((size_t)e * I + row0 + col) * HB * 40 + (size_t)b0 * 40;
  uint2 q[NB];
  uint32_t qh[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    q[j] = *reinterpret_cast<const uint2*>(rp + j * 40 + 8 * g);
    qh[j] = *reinterpret_cast<const uint16_t*>(rp + j * 40 + 32 + 2 * g);
  }
  for (int i = lane; i < NB * 16; i += 64) {
    const int bl = i >> 4, r = i & 15;
    s_sc[wave][bl][r] = fp16_to_f32(scales[((size_t)e * I + row0 + r) * HB + b0 + bl]);
  }
  const bool t_ok = col < ntok;
  const uint16_t* xr = a.x + (size_t)tok * H + 64 * g;
  uint4 nx[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) nx[t] = *reinterpret_cast<const uint4*>(xr + 256 * b0 + 8 * t);
  wave_fence_lds();
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    uint4 cx[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) cx[t] = nx[t];
    if (j + 1 < NB) {
#pragma unroll
      for (int t = 0; t < 8; ++t) nx[t] = *reinterpret_cast<const uint4*>(xr + 256 * (b0 + j + 1) + 8 * t);
    }
    bf16x8_t av[8];
    stq_block_a(s_lut, q[j], qh[j], av);
    f32x4_t bacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) bacc = mfma16(av[t], as_bf16x8(keep_if(t_ok, cx[t])), bacc);
    const float4 d = *reinterpret_cast<const float4*>(&s_sc[wave][j][4 * g]);
    acc[0] = fmaf(d.x, bacc[0], acc[0]); acc[1] = fmaf(d.y, bacc[1], acc[1]);
    acc[2] = fmaf(d.z, bacc[2], acc[2]); acc[3] = fmaf(d.w, bacc[3], acc[3]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0 && t_ok) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gs = s_red[0][i][lane] + s_red[2][i][lane];   // gate: K halves 0, 1
      const float us = s_red[1][i][lane] + s_red[3][i][lane];   // up
      const float h = gs / (1.0f + expf(-gs)) * us;
      hi[i] = f32_to_bf16_rne(h);
      lo[i] = f32_to_bf16_rne(h - bf16_to_f32(hi[i]));
    }
    const size_t idx = (size_t)(pos0 + col) * I + row0 + 4 * g;
    *reinterpret_cast<uint2*>(a.h_hi + idx) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
    *reinterpret_cast<uint2*>(a.h_lo + idx) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
  }
  __syncthreads();   // s_red / s_sc are reused by the next unit
}

// Shared down for up to kSmallT tokens: wave = 4 rows of H, lane l reads K = 8 l + 512 j
// (the last chunk is half-used when I is an odd multiple of 256).
template <int HB, int IB>
__device__ void shared_down_valu(const DecodeArgs& a, int sd) {
  constexpr int H = HB * 256, I = IB * 256, NJ = (IB + 1) / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = (sd * kNW + wave) * 4;
  const bool last_ok = (IB % 2 == 0) || lane < 32;
  const int lcol = (IB % 2 == 0 || lane < 32) ? lane : 0;
  uint4 wv[4][NJ];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int cl = j == NJ - 1 ? lcol : lane;
      wv[r][j] = *reinterpret_cast<const uint4*>(a.sd + (size_t)(row0 + r) * I + 8 * cl + 512 * j);
    }
  float acc[4][kSmallT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) acc[r][t] = 0.f;
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) {
    if (t < a.T) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int cl = j == NJ - 1 ? lcol : lane;
        const bool ok = j < NJ - 1 || last_ok;
        const float* hp = a.hs + (size_t)t * I + 8 * cl + 512 * j;
        float4 h0 = *reinterpret_cast<const float4*>(hp);
        float4 h1 = *reinterpret_cast<const float4*>(hp + 4);
        if (!ok) { h0 = make_float4(0.f, 0.f, 0.f, 0.f); h1 = h0; }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint4 wq = wv[r][j];
          float s = acc[r][t];
          s = fmaf(bf16_to_f32(wq.x & 0xFFFF), h0.x, s); s = fmaf(bf16_to_f32(wq.x >> 16), h0.y, s);
          s = fmaf(bf16_to_f32(wq.y & 0xFFFF), h0.z, s); s = fmaf(bf16_to_f32(wq.y >> 16), h0.w, s);
          s = fmaf(bf16_to_f32(wq.z & 0xFFFF), h1.x, s); s = fmaf(bf16_to_f32(wq.z >> 16), h1.y, s);
          s = fmaf(bf16_to_f32(wq.w & 0xFFFF), h1.z, s); s = fmaf(bf16_to_f32(wq.w >> 16), h1.w, s);
          acc[r][t] = s;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) {
      if (t < a.T) {
        const float v = wave_sum(acc[r][t]);
        if (lane == 0) a.y_shared[(size_t)t * H + row0 + r] = v;
      }
    }
}

// Shared down beyond kSmallT tokens: 16 rows x 16 tokens, the 4 waves split K = I; h is
// split into bf16 hi + lo on the fly.
template <int HB, int IB>
__device__ void shared_down_mfma(const DecodeArgs& a, int sd, float (*s_red)[4][64]) {
  constexpr int H = HB * 256, I = IB * 256, n_rt = H / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rt = sd % n_rt, tt = sd / n_rt;
  const int row0 = rt * 16;
  const int col = lane & 15, g = lane >> 4;
  const int tok = tt * 16 + col;
  const bool t_ok = tok < a.T;
  const int b0 = wave * IB / kNW, b1 = (wave + 1) * IB / kNW;
  const float* hr = a.hs + (size_t)(t_ok ? tok : 0) * I;
  const uint16_t* rd = a.sd + (size_t)(row0 + col) * I;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int b = b0; b < b1; ++b) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int off = 256 * b + 32 * t + 8 * g;
      const bf16x8_t av = as_bf16x8(*reinterpret_cast<const uint4*>(rd + off));
      const float4 h0 = *reinterpret_cast<const float4*>(hr + off);
      const float4 h1 = *reinterpret_cast<const float4*>(hr + off + 4);
      const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = t_ok ? hv[i] : 0.f;
        hi[i] = f32_to_bf16_rne(v);
        lo[i] = f32_to_bf16_rne(v - bf16_to_f32(hi[i]));
      }
      acc = mfma16(av, as_bf16x8(make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16))), acc);
      acc = mfma16(av, as_bf16x8(make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16))), acc);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0 && t_ok) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
      for (int w = 0; w < kNW; ++w) v += s_red[w][i][lane];
      y[i] = v;
    }
    *reinterpret_cast<float4*>(a.y_shared + (size_t)tok * H + row0 + 4 * g) = make_float4(y[0], y[1], y[2], y[3]);
  }
}

template <int HB, int IB>
__global__ __launch_bounds__(kWG) void k2_gateup(DecodeArgs a) {
  __shared__ uint2 s_lut[32];
  __shared__ __align__(16) float s_sc[kNW][HB / 2][16];
  __shared__ __align__(16) float s_red[kNW][4][64];
  const int b = blockIdx.x;
  if (b < a.n_sdn_wg) {
    if (a.T <= kSmallT) shared_down_valu<HB, IB>(a, b);
    else shared_down_mfma<HB, IB>(a, b, s_red);
    return;
  }
  build_lut(s_lut);
  __syncthreads();
  const int n_units = a.wl[1] * (IB * 256 / 16);
  for (int u = b - a.n_sdn_wg; u < n_units; u += a.n_gu_wg)
    routed_gateup_unit<HB, IB>(a, u, s_lut, s_sc, s_red);
}

// ============================================================================ K3
// One 16-row slice of the output: every unit (expert, <= 16 pairs) of the slice, spread
// over the 8 waves; each wave adds w * y into its own LDS sums; the slice is then
// out = y_shared + sum over waves in order (+ residual).
template <int HB, int IB>
__global__ __launch_bounds__(64 * kDnWaves) void k3_down_combine(DecodeArgs a) {
  constexpr int H = HB * 256, I = IB * 256;
  __shared__ uint2 s_lut[32];
  __shared__ __align__(16) float s_sc[kDnWaves][IB][16];
  __shared__ __align__(16) float s_acc[kDnWaves][kMaxT][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T;
  const int row0 = blockIdx.x * 16;
  const int col = lane & 15, g = lane >> 4;
  build_lut(s_lut);
  for (int i = threadIdx.x; i < kDnWaves * T * 16; i += 64 * kDnWaves)
    s_acc[i / (T * 16)][(i / 16) % T][i % 16] = 0.f;
  __syncthreads();
  const int n_units = a.wl[1];
  for (int uu = wave; uu < n_units; uu += kDnWaves) {
    const int4 un = a.ut[uu];
    const int e = un.x, pos0 = un.y, ntok = un.z;
    const int tok = a.utok[uu * 16 + col];
    const float wt = a.uw[uu * 16 + col];
    const uint8_t* rp = a.dc + ((size_t)e * H + row0 + col) * IB * 40;
    uint2 q[IB];
    uint32_t qh[IB];
#pragma unroll
    for (int j = 0; j < IB; ++j) {
      q[j] = *reinterpret_cast<const uint2*>(rp + j * 40 + 8 * g);
      qh[j] = *reinterpret_cast<const uint16_t*>(rp + j * 40 + 32 + 2 * g);
    }
    for (int i = lane; i < IB * 16; i += 64) {
      const int bl = i >> 4, r = i & 15;
      s_sc[wave][bl][r] = fp16_to_f32(a.ds[((size_t)e * H + row0 + r) * IB + bl]);
    }
    const bool t_ok = col < ntok;
    const size_t hoff = (size_t)(pos0 + (t_ok ? col : 0)) * I + 64 * g;
    const uint16_t* hh = a.h_hi + hoff;
    const uint16_t* hl = a.h_lo + hoff;
    uint4 nh[8], nl[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      nh[t] = *reinterpret_cast<const uint4*>(hh + 8 * t);
      nl[t] = *reinterpret_cast<const uint4*>(hl + 8 * t);
    }
    wave_fence_lds();
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < IB; ++j) {
      uint4 ch[8], cl[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) { ch[t] = nh[t]; cl[t] = nl[t]; }
      if (j + 1 < IB) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          nh[t] = *reinterpret_cast<const uint4*>(hh + 256 * (j + 1) + 8 * t);
          nl[t] = *reinterpret_cast<const uint4*>(hl + 256 * (j + 1) + 8 * t);
        }
      }
      bf16x8_t av[8];
      stq_block_a(s_lut, q[j], qh[j], av);
      f32x4_t bh = {0.f, 0.f, 0.f, 0.f}, bl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        bh = mfma16(av[t], as_bf16x8(keep_if(t_ok, ch[t])), bh);
        bl = mfma16(av[t], as_bf16x8(keep_if(t_ok, cl[t])), bl);
      }
      const float4 d = *reinterpret_cast<const float4*>(&s_sc[wave][j][4 * g]);
      acc[0] = fmaf(d.x, bh[0] + bl[0], acc[0]); acc[1] = fmaf(d.y, bh[1] + bl[1], acc[1]);
      acc[2] = fmaf(d.z, bh[2] + bl[2], acc[2]); acc[3] = fmaf(d.w, bh[3] + bl[3], acc[3]);
    }
    if (t_ok) {
      *reinterpret_cast<float4*>(a.y_pairs + (size_t)(pos0 + col) * H + row0 + 4 * g) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
      float* sa = &s_acc[wave][tok][4 * g];
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = fmaf(wt, acc[i], sa[i]);
    }
    wave_fence_lds();
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * 16; i += 64 * kDnWaves) {
    const int t = i >> 4, r = i & 15;
    float v = a.y_shared ? a.y_shared[(size_t)t * H + row0 + r] : 0.f;
    for (int w = 0; w < kDnWaves; ++w) v += s_acc[w][t][r];
    if (a.residual) v += a.residual[(size_t)t * H + row0 + r];
    a.out[(size_t)t * H + row0 + r] = v;
    if (a.out_bf16) a.out_bf16[(size_t)t * H + row0 + r] = (uint16_t)f32_to_bf16_rne(v);
  }
}

template <int HB, int IB>
hipError_t launch_all(DecodeArgs& a, hipStream_t s) {
  constexpr int H = HB * 256, I = IB * 256;
  const int T = a.T;
  const int n_tt = (T + 15) / 16;
  const int P = T * a.k;
  const int max_units = (P < a.E ? P : a.E) + (P + 15) / 16;
  a.n_router_wg = ((a.E + 15) / 16) * kRouterParts * n_tt;
  const bool small = T <= kSmallT;
  const bool shared = a.sg != nullptr;
  a.n_sgu_wg = shared ? (small ? I / 2 : (I / 16) * n_tt) : 0;
  a.n_sdn_wg = shared ? (small ? H / (4 * kNW) : (H / 16) * n_tt) : 0;
  const int cap = 8192;
  const int gu = max_units * (I / 16);
  a.n_gu_wg = gu < cap ? gu : cap;
  const bool prof = moe_prof_on();
  if (prof) moe_prof_begin(MOE_PROF_DECODE_K1, s);
  hipLaunchKernelGGL((k1_router_shared<HB, IB>), dim3(a.n_router_wg + a.n_sgu_wg), dim3(kWG), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K1, s); moe_prof_begin(MOE_PROF_DECODE_K2, s); }
  hipLaunchKernelGGL((k2_gateup<HB, IB>), dim3(a.n_sdn_wg + a.n_gu_wg), dim3(kWG), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K2, s); moe_prof_begin(MOE_PROF_DECODE_K3, s); }
  hipLaunchKernelGGL((k3_down_combine<HB, IB>), dim3(H / 16), dim3(64 * kDnWaves), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) moe_prof_end(MOE_PROF_DECODE_K3, s);
  return hipSuccess;
}

}  // namespace

// ---------------------------------------------------------------------------- host side
// Shapes with a compiled instantiation: (H, I) in units of 256.
bool moe_decode_shape_ok(int H, int I, int E) {
  if (E > kMaxE || H % 256 || I % 256) return false;
  const int hb = H / 256, ib = I / 256;
  return (hb == 2 && ib == 1) || (hb == 4 && ib == 2) || (hb == 8 && ib == 4) ||
         (hb == 16 && ib == 8) || (hb == 24 && ib == 8) || (hb == 32 && ib == 8);
}

size_t moe_decode_ws_layout(int T, int H, int I, int E, int k, int has_shared, size_t* offs) {
  const size_t P = (size_t)T * k;
  const size_t max_units = (size_t)(P < (size_t)E ? P : E) + (P + 15) / 16;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t cur = 0;
  offs[0] = cur; cur = al(cur + 8 * sizeof(int32_t));                              // work list + ticket
  offs[1] = cur; cur = al(cur + max_units * sizeof(int4));                          // unit table
  offs[2] = cur; cur = al(cur + max_units * 16 * sizeof(int32_t));                  // unit tokens
  offs[3] = cur; cur = al(cur + max_units * 16 * sizeof(float));                    // unit weights
  offs[4] = cur; cur = al(cur + (size_t)kRouterParts * T * E * sizeof(float));     // router partials
  offs[5] = cur; cur = al(cur + P * I * 2);                                          // h hi
  offs[6] = cur; cur = al(cur + P * I * 2);                                          // h lo
  offs[7] = cur; cur = al(cur + (has_shared ? (size_t)T * I * sizeof(float) : 0));   // shared h
  offs[8] = cur;
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
  a.T = d->T; a.E = d->E; a.k = d->k;
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
  size_t offs[9];
  moe_decode_ws_layout(d->T, d->H, d->I, d->E, d->k, shared != nullptr, offs);
  uint8_t* b = static_cast<uint8_t*>(ws);
  a.wl = reinterpret_cast<int32_t*>(b + offs[0]);
  a.ctr = a.wl + 4;
  a.ut = reinterpret_cast<int4*>(b + offs[1]);
  a.utok = reinterpret_cast<int32_t*>(b + offs[2]);
  a.uw = reinterpret_cast<float*>(b + offs[3]);
  a.rpart = reinterpret_cast<float*>(b + offs[4]);
  a.h_hi = reinterpret_cast<uint16_t*>(b + offs[5]);
  a.h_lo = reinterpret_cast<uint16_t*>(b + offs[6]);
  a.hs = reinterpret_cast<float*>(b + offs[7]);
  const int hb = d->H / 256, ib = d->I / 256;
  if (hb == 2 && ib == 1) return launch_all<2, 1>(a, s);
  if (hb == 4 && ib == 2) return launch_all<4, 2>(a, s);
  if (hb == 8 && ib == 4) return launch_all<8, 4>(a, s);
  if (hb == 16 && ib == 8) return launch_all<16, 8>(a, s);
  if (hb == 24 && ib == 8) return launch_all<24, 8>(a, s);
  if (hb == 32 && ib == 8) return launch_all<32, 8>(a, s);
  return hipErrorInvalidValue;
}
