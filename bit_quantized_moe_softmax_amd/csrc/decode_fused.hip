// Fused decode-regime MoE layer: route -> permute -> expert FFN -> combine in three or four
// kernels.
//
// Same computation as the four separate entry points (router in BF16, top-k with
// renormalised softmax weights, stable permutation, SwiGLU experts on STQ1_0 weights,
// one bf16 shared expert, ungated combine), split by what each step waits for.
// Up to kXT tokens:
//   K1  router partials (bf16 MFMA; a workgroup sums four K chunks of 16 experts in LDS
//       and writes one partial), beside the shared expert's gate/up (VALU dot products);
//   K2  every routed workgroup sums the partials and derives the whole routing in its own
//       LDS (top-k, stable pair order, units), so no workgroup waits on another; then the
//       routed gate/up (STQ1_0 decoded in registers, bf16 MFMA) with SiLU(gate) * up,
//       beside the shared down;
//   K3  one token: every routed down projection and the combine per 16-row slice of the
//       output, weighted into per-wave LDS sums, out = y_shared + sum over waves in a fixed
//       order (+ residual).  Two to four tokens (their h exceeds the LDS): the item-list
//       down kernel below, then the separate combine.
// Beyond kXT tokens (up to kMaxT):
//   K1  router partials per 16-token tile and two tickets (agent-scope atomics on counters
//       in the workspace): the last router workgroup of a tile picks that tile's top-k, the
//       last tile sorts all pairs and writes the work lists; the shared expert's gate/up
//       (bf16 MFMA, one weight read for every token tile) runs beside it;
//   K2  persistent workgroups, one per CU, over the list of routed gate/up items (half-unit
//       of <= 8 pairs x 128 rows of I), x rows staged per half-unit;
//   K3  persistent workgroups over the shared down items (16-token tile x 128 rows) and the
//       routed down items (unit of <= 16 pairs x 128 rows), h staged per unit; writes
//       y_pairs and y_shared;
//   K4  the combine (+ residual).
// Every sum runs in a fixed order, so results do not depend on scheduling.  The ticket
// counters live in the workspace: zero before the first call, left zero by every call.
//
// Memory-level order.  A wave's vector loads retire in issue order, so waiting for one
// load waits for every load issued before it.  The weight streams are therefore the only
// loads inside the main loops: activations (x, h) are staged into LDS once, from loads
// issued before the first weight load, and the loops read them with LDS instructions
// (a separate counter).  Weight code words run a fixed number of blocks ahead.
//
// MFMA roles (v_mfma_f32_16x16x32_bf16): the A operand carries activations (row = token
// slot = lane % 16), the B operand carries weights (column = weight row = lane % 16); lane
// group g = lane / 16 supplies K-slots 8g .. 8g+7 of both, and D(slot 4g + i, row) sits in
// register i of the lane that decoded that row, so one STQ1_0 block scale per lane and
// block applies to all four of its results.  K-slot -> K map inside a 256-weight block b at
// MFMA step t: K = 256 b + 64 g + 8 t + s, i.e. a lane decodes groups 16g+2t and 16g+2t+1
// from the 8 code bytes and 16 high bits it loads.  Lanes whose token slot lies past a
// unit's last pair skip their A reads (exec-masked LDS loads) and keep zeros: their D rows
// are never used.  (At one token this removes 15/16 of the A-operand LDS traffic but did not
// change the layer time: the gate/up stream is bound by its per-block dependency chain --
// code word, table offsets, table reads, MFMAs -- not by LDS bandwidth.)
// The routed h is kept as bf16 hi + bf16 lo (h - hi); in the down projection a pair takes
// two adjacent A rows (hi, lo) of one MFMA, so ~16 bits of h cost no extra MFMA and the
// pair's result is the sum of two D rows.  The shared h is kept the same way: up to kXT
// tokens it enters packed bf16 dot products, beyond that the MFMA as the routed h does.
// The kernels are instantiated per (H/256, I/256) so every loop over K has a fixed trip
// count and a wave's loads are issued without branches.  Up to kXT tokens every x row sits
// in LDS and the shared expert runs on the VALU (a plain bf16 GEMV: 75 MB of weights at
// Hy4 shape); beyond that the x rows of a half-unit and the h rows of a unit are staged
// in LDS per work item and the shared expert uses the MFMA.
#include "moe_device.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace {

constexpr int kWG = 256;           // 4 waves
constexpr int kNW = 4;
constexpr int kRouterChunks = 16;  // router K chunks, 4 per workgroup
constexpr int kRouterParts = kRouterChunks / kNW;
constexpr int kXT = 4;             // tokens whose activations are staged in LDS
constexpr int kMaxT = 64;
constexpr int kMaxE = 256;
constexpr int kDnWaves = 8;        // waves of a down/combine workgroup
constexpr int kHLdsPairs = 8;      // routed pairs (+ tokens) whose h fits the down kernel's LDS
constexpr int kMaxDevices = 64;
constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past every record: loads return 0
// Weight blocks a streaming wave keeps in flight.  HBM saturates at ~8 MB in flight across
// the chip; more only queues, and every load issued behind the queue (the activations a
// workgroup stages first, routing data) waits for it.  A few KB per wave x all resident
// waves keeps the queue short.
constexpr int kRing = 4;

struct DecodeArgs {
  int T, E, k;
  const uint8_t* gc; const uint16_t* gs;
  const uint8_t* uc; const uint16_t* us;
  const uint8_t* dc; const uint16_t* ds;
  const uint16_t* sg; const uint16_t* su; const uint16_t* sd;
  const uint16_t* x; const uint16_t* wr; const float* bias;
  float* logits; int32_t* ids; float* w; int32_t* sorted_pair; int32_t* offsets; int32_t* pair_pos;
  float* y_pairs; float* y_shared; const float* residual; float* out; uint16_t* out_bf16;
  int32_t* wl;      // [0] active experts, [1] units, [2] half-units
  int32_t* ctr;     // [0] router ticket (zero between calls)
  int4* ut;         // units: {expert, first sorted position, pairs (<= 16), 0}
  int32_t* utok;    // [unit][16] token of each pair of the unit
  float* uw;        // [unit][16] routing weight of each pair of the unit
  int4* hl;         // half-units: {expert, first sorted position, pairs (<= 8), index of
                    //  its first pair in utok / uw}
  int max_half;     // capacity of hl
  float* rpart;     // [kRouterParts][T][E]
  uint16_t* h_hi;   // [P][I] bf16, followed at h_lo_bytes by the lo half [P][I]
  uint32_t h_lo_bytes, h_bytes;
  uint16_t* hs;     // shared h [T][I] bf16 hi, then [T][I] bf16 lo
  int n_router_wg, n_sgu_wg, n_gu_wg;
  int n_xq_wg;      // MXFP4: x quantisation workgroups of the first kernel
  int h_lds;        // down kernel: all routed (and, without ysh_ready, shared) h staged in LDS
  int ysh_ready;    // y_shared was written by an earlier kernel: the down kernel adds it
  // MXFP4 routed experts: E4M3 x codes [T][H] then UE8M0 scales [T][H/32] (written by K1);
  // E4M3 h codes [P][I] then scales [P][I/32] (over the bf16 h region)
  uint8_t* xq;
  uint8_t* hq;
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes at voff + soff (soff: a wave-uniform constant, kept out of the VGPRs).
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Weight streams read in whole cache lines by one load are read once per call: non-temporal
// loads (cache policy nt) keep them from evicting what is reused from L2 -- activations,
// routing data, h, and the kernels' code.  Streams that touch a line through several loads
// (the STQ1_0 code words: a 40-byte block, a 160-byte run of a row, straddle lines) keep
// normal loads: an nt line may be gone before its next touch (measured: +13 % fetched).
constexpr int kNT = 2;
__device__ __forceinline__ uint4 bload16_nt(rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT));
}
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
__device__ __forceinline__ uint4 ntload16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}


__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// h as bf16 hi + bf16 lo (h - hi): ~16 significant bits in two bf16 operands.
__device__ __forceinline__ void store_hilo(uint16_t* hi_p, size_t lo_stride, float h) {
  const uint32_t hi = f32_to_bf16_rne(h);
  hi_p[0] = (uint16_t)hi;
  hi_p[lo_stride] = (uint16_t)f32_to_bf16_rne(h - bf16_to_f32(hi));
}

__device__ __forceinline__ uint32_t bf16_lane(uint32_t p, int j) {
  const int z = p >> 3;
  if (j == z) return 0u;
  const int i = j < z ? j : j - 1;
  return ((p >> i) & 1) ? 0xBF80u : 0x3F80u;
}

// 32-entry table: 5-bit STQ1_0 group pattern p -> its four weights in {-1, 0, +1} as bf16,
// 8 bytes per entry at byte 16 (p & 15) + 8 (p >> 4), i.e. words 4 (p & 15) + 2 (p >> 4)
// and the next (the two patterns that share a nibble sit side by side, so a nibble times 16
// and the high bit times 8 form the offset).  Splitting each entry into two 4-byte tables
// (conflict-free ds_read2_b32) measured slower.
__device__ __forceinline__ void build_lut(uint32_t* lut) {
  const int t = threadIdx.x;
  if (t < 32) {
    const int w = 4 * (t & 15) + 2 * (t >> 4);
    lut[w] = bf16_lane(t, 0) | (bf16_lane(t, 1) << 16);
    lut[w + 1] = bf16_lane(t, 2) | (bf16_lane(t, 3) << 16);
  }
}

// Table byte offsets of the 8 groups of one code word qw (4 bytes: group 2t is the low
// nibble of byte t, group 2t + 1 the high nibble) with their high bits hb (bits 2t and
// 2t + 1), four at a time: the nibbles x 16 by masks (the high nibbles are in place); the
// high bits moved to bit 3 of their bytes by one 24-bit multiply (bit 2i lands on bit
// 8i + 3; the stray products fall on bits that are masked off).  About 3 VALU instructions
// per lookup, all at full rate.
__device__ __forceinline__ void stq_word_offsets(uint32_t qw, uint32_t hb, uint32_t& alo, uint32_t& ahi) {
  const uint32_t lo8 = (qw << 4) & 0xF0F0F0F0u, hi8 = qw & 0xF0F0F0F0u;
  const uint32_t sl = __umul24(hb & 0x55u, 0x208208u) & 0x08080808u;
  const uint32_t sh = __umul24((hb >> 1) & 0x55u, 0x208208u) & 0x08080808u;
  alo = sl | lo8;
  ahi = sh | hi8;
}
__device__ __forceinline__ uint2 lut_at(const uint32_t* lut, uint32_t off) {
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(lut) + off);
}

// The 4 weight operands of one code word (its 8 groups): 8 table reads, all issued before
// any is used.
__device__ __forceinline__ void stq_word_w(const uint32_t* lut, uint32_t qw, uint32_t hb, bf16x8_t* wv) {
  uint32_t alo, ahi;
  stq_word_offsets(qw, hb, alo, ahi);
  uint2 l[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    l[2 * t] = lut_at(lut, (alo >> (8 * t)) & 0xFFu);
    l[2 * t + 1] = lut_at(lut, (ahi >> (8 * t)) & 0xFFu);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) wv[t] = as_bf16x8(make_uint4(l[2 * t].x, l[2 * t].y, l[2 * t + 1].x, l[2 * t + 1].y));
}

// The 8 weight operands of one STQ1_0 block (8 code bytes + 16 high bits of this lane).
__device__ __forceinline__ void stq_block_w(const uint32_t* lut, uint2 qs, uint32_t qh, bf16x8_t* wv) {
  stq_word_w(lut, qs.x, qh, wv);
  stq_word_w(lut, qs.y, qh >> 8, wv + 4);
}

// The 4 weight operands of half h of one STQ1_0 block (code bytes 4h .. 4h+3 of this lane
// and their 8 high bits).
__device__ __forceinline__ void stq_half_w(const uint32_t* lut, uint2 qs, uint32_t qh, int h, bf16x8_t* wv) {
  stq_word_w(lut, h ? qs.y : qs.x, qh >> (8 * h), wv);
}

// fp16 block scales of one row: words of two, in groups of 8 blocks (16 bytes, aligned
// when NB >= 8), fewer blocks in one smaller aligned load.
template <int NB>
__device__ __forceinline__ uint4 load_scale_group(const uint16_t* p, int grp) {
  if constexpr (NB == 1) {
    return make_uint4(*p, 0u, 0u, 0u);
  } else if constexpr (NB == 2) {
    return make_uint4(*reinterpret_cast<const uint32_t*>(p), 0u, 0u, 0u);
  } else if constexpr (NB == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_uint4(v.x, v.y, 0u, 0u);
  } else {
    static_assert(NB % 8 == 0, "block count");
    return reinterpret_cast<const uint4*>(p)[grp];
  }
}
__device__ __forceinline__ float scale_of(uint4 s, int j) {
  const int w = (j >> 1) & 3;
  const uint32_t v = w == 0 ? s.x : (w == 1 ? s.y : (w == 2 ? s.z : s.w));
  return fp16_to_f32((v >> (16 * (j & 1))) & 0xFFFFu);
}

// One wave's LDS writes made visible to its own later LDS reads: a workgroup-scope fence
// on the LDS address space only, so vector memory loads and stores stay in flight.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations, not for its
// vector memory loads still in flight (the weight stream keeps running across it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Pin a block's four accumulators in registers at this point (emits no instruction):
// sunk to the end of the unrolled loop, every block's partial sum would stay live.
__device__ __forceinline__ void pin4(f32x4_t& acc) {
  float a0 = acc[0], a1 = acc[1], a2 = acc[2], a3 = acc[3];
  asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
  acc[0] = a0; acc[1] = a1; acc[2] = a2; acc[3] = a3;
}

// Stream of one STQ1_0 row tile over NB blocks: 16 weight rows (this lane's row at rp, its
// scales at sp) against up to 16 activation rows.  issue() starts the code words of the
// first R blocks (672 bytes per block and wave) and the first scale group; the run
// functions decode block j while the code words of block j + R and the next scale group
// are in flight and return sum_b d_b * (A . W_b) in the D layout.
template <int NB, int RD = kRing>
struct StqStream {
  static constexpr int R = NB < RD ? NB : RD;
  uint2 q[R];
  uint32_t qh[R];
  uint4 sc, sc_next;
  const uint8_t* qp;
  const uint8_t* hp;
  const uint16_t* sp;

  __device__ __forceinline__ void issue(const uint8_t* rp, const uint16_t* sp_) {
    const int g = (threadIdx.x & 63) >> 4;
    qp = rp + 8 * g;
    hp = rp + 32 + 2 * g;
    sp = sp_;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      q[j] = *reinterpret_cast<const uint2*>(qp + j * 40);
      qh[j] = *reinterpret_cast<const uint16_t*>(hp + j * 40);
    }
    sc = load_scale_group<NB>(sp, 0);
    sc_next = sc;
  }

  __device__ __forceinline__ void next(int j, uint2& qj, uint32_t& qhj, float& d) {
    if (j % 8 == 0) {
      if (j > 0) sc = sc_next;
      if (j + 8 < NB) sc_next = load_scale_group<NB>(sp, j / 8 + 1);
    }
    qj = q[j % R];
    qhj = qh[j % R];
    if (j + R < NB) {
      q[j % R] = *reinterpret_cast<const uint2*>(qp + (j + R) * 40);
      qh[j % R] = *reinterpret_cast<const uint16_t*>(hp + (j + R) * 40);
    }
    d = scale_of(sc, j);
  }

  // A operands from LDS: row base `a_lds` (bf16 elements, this lane's token slot and K-slots
  // already applied), K stride 1; lanes with a_on false read nothing and feed zeros.
  // Software-pipelined by half blocks: the table reads of half h + 1 are in flight while the
  // 4 MFMAs of half h run, and the two halves of a block accumulate in separate registers
  // (two 4-deep MFMA chains).
  __device__ __forceinline__ f32x4_t run_lds(const uint32_t* lut, const uint16_t* a_lds, bool a_on = true) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint2 qj;
    uint32_t qhj;
    float d;
    next(0, qj, qhj, d);
    bf16x8_t wn[4];
    stq_half_w(lut, qj, qhj, 0, wn);
    f32x4_t b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0;
    uint4 av[4] = {};
#pragma unroll
    for (int hh = 0; hh < 2 * NB; ++hh) {
      const int j = hh >> 1, h = hh & 1;
      bf16x8_t wc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) wc[t] = wn[t];
      float dj = d;
      if (h == 0) {
        stq_half_w(lut, qj, qhj, 1, wn);
      } else if (j + 1 < NB) {
        next(j + 1, qj, qhj, d);
        stq_half_w(lut, qj, qhj, 0, wn);
      }
      if (a_on) {
#pragma unroll
        for (int t = 0; t < 4; ++t) av[t] = *reinterpret_cast<const uint4*>(a_lds + 256 * j + 8 * (4 * h + t));
      }
      f32x4_t& bh = h ? b1 : b0;
#pragma unroll
      for (int t = 0; t < 4; ++t) bh = mfma16(as_bf16x8(av[t]), wc[t], bh);
      if (h == 1) {
        acc[0] = fmaf(dj, b0[0] + b1[0], acc[0]); acc[1] = fmaf(dj, b0[1] + b1[1], acc[1]);
        acc[2] = fmaf(dj, b0[2] + b1[2], acc[2]); acc[3] = fmaf(dj, b0[3] + b1[3], acc[3]);
        pin4(acc);
        b0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
        b1 = b0;
      }
    }
    return acc;
  }
};

// The same stream with the code words staged through a per-wave LDS buffer.  A wave's 16
// weight rows are consecutive rows of one matrix, so chunk c (blocks CB c .. CB c + CB - 1
// of every row) is 16 runs of 40 CB contiguous bytes: fetched as 16-byte pieces (fully
// used cache lines, a quarter of the requests of per-lane 8- and 2-byte reads) DEPTH chunks
// ahead in registers, written to LDS when their turn comes, and read from there per block.
// (Four or six chunks ahead measured slower at one token: 55-56 us per layer against 48 us
// with two; the extra loads only lengthen the memory queue the routing and x loads wait in.)
// LDS rows are padded so the 16 lanes reading one column group hit distinct banks.
template <int NB, int DEPTH = 2>
struct StqStreamL {
  static constexpr int CB = NB % 4 == 0 ? 4 : 2;           // blocks per chunk (NB even)
  static constexpr int NC = NB / CB;                       // chunks
  static constexpr int D = DEPTH < NC ? DEPTH : NC;        // chunks in flight (register slots)
  static constexpr int RUN = 40 * CB;                      // bytes of one row in a chunk
  static constexpr int PPR = RUN / 16;                     // 16-byte pieces per row run
  static constexpr int NL = (16 * PPR + 63) / 64;          // loads per lane per chunk
  static constexpr int CROW = CB == 4 ? 176 : 112;         // padded LDS bytes per row
  static constexpr int BYTES = 16 * CROW;                  // LDS bytes per wave
  static_assert(NB % 2 == 0, "whole chunks");
  uint4 v[D][NL];
  uint4 sc, sc_next;
  rsrc_t tile;             // the wave's 16 rows (16 x 40 NB bytes)
  const uint16_t* sp;
  uint8_t* buf;            // this wave's LDS buffer

  // piece m of this lane: row and byte offset inside the row run (lanes past the last
  // piece reload piece 0 and store nothing)
  __device__ __forceinline__ static bool piece(int m, int& row, int& off) {
    const int pc = 64 * m + (threadIdx.x & 63);
    const bool ok = pc < 16 * PPR;
    const int pp = ok ? pc : 0;
    row = pp / PPR;
    off = 16 * (pp % PPR);
    return ok;
  }
  __device__ __forceinline__ void load_chunk(int slot, int c) {
#pragma unroll
    for (int m = 0; m < NL; ++m) {
      int row, off;
      piece(m, row, off);
      v[slot][m] = bload16(tile, (uint32_t)(row * 40 * NB + off), (uint32_t)(RUN * c));
    }
  }
  __device__ __forceinline__ void store_chunk(int slot) {
#pragma unroll
    for (int m = 0; m < NL; ++m) {
      int row, off;
      if (piece(m, row, off)) *reinterpret_cast<uint4*>(buf + row * CROW + off) = v[slot][m];
    }
  }

  __device__ __forceinline__ void issue(const uint8_t* tile_, const uint16_t* sp_, uint8_t* buf_) {
    tile = make_rsrc(tile_, 16 * 40 * NB);
    sp = sp_;
    buf = buf_;
#pragma unroll
    for (int c = 0; c < D; ++c) load_chunk(c, c);
    sc = load_scale_group<NB>(sp, 0);
    sc_next = sc;
    store_chunk(0);
    if (NC > D) load_chunk(0, D);
  }

  __device__ __forceinline__ void next(int j, uint2& qj, uint32_t& qhj, float& d) {
    if (j % 8 == 0) {
      if (j > 0) sc = sc_next;
      if (j + 8 < NB) sc_next = load_scale_group<NB>(sp, j / 8 + 1);
    }
    if (j % CB == 0 && j > 0) {
      const int c = j / CB;
      store_chunk(c % D);
      if (c + D < NC) load_chunk(c % D, c + D);
    }
    const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
    const uint8_t* bp = buf + col * CROW + 40 * (j % CB);
    qj = *reinterpret_cast<const uint2*>(bp + 8 * g);
    qhj = *reinterpret_cast<const uint16_t*>(bp + 32 + 2 * g);
    d = scale_of(sc, j);
  }

  // as StqStream::run_lds
  __device__ __forceinline__ f32x4_t run_lds(const uint32_t* lut, const uint16_t* a_lds, bool a_on = true) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint2 qj;
    uint32_t qhj;
    float d;
    next(0, qj, qhj, d);
    bf16x8_t wn[4];
    stq_half_w(lut, qj, qhj, 0, wn);
    f32x4_t b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0;
    uint4 av[4] = {};
#pragma unroll
    for (int hh = 0; hh < 2 * NB; ++hh) {
      const int j = hh >> 1, h = hh & 1;
      bf16x8_t wc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) wc[t] = wn[t];
      float dj = d;
      if (h == 0) {
        stq_half_w(lut, qj, qhj, 1, wn);
      } else if (j + 1 < NB) {
        next(j + 1, qj, qhj, d);
        stq_half_w(lut, qj, qhj, 0, wn);
      }
      if (a_on) {
#pragma unroll
        for (int t = 0; t < 4; ++t) av[t] = *reinterpret_cast<const uint4*>(a_lds + 256 * j + 8 * (4 * h + t));
      }
      f32x4_t& bh = h ? b1 : b0;
#pragma unroll
      for (int t = 0; t < 4; ++t) bh = mfma16(as_bf16x8(av[t]), wc[t], bh);
      if (h == 1) {
        acc[0] = fmaf(dj, b0[0] + b1[0], acc[0]); acc[1] = fmaf(dj, b0[1] + b1[1], acc[1]);
        acc[2] = fmaf(dj, b0[2] + b1[2], acc[2]); acc[3] = fmaf(dj, b0[3] + b1[3], acc[3]);
        pin4(acc);
        b0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
        b1 = b0;
      }
    }
    return acc;
  }
};

// Copy up to ROWS activation rows of K bf16 (row r from src_row(r)) into LDS rows of K
// through the whole workgroup: issue() loads ROWS rows into registers (rows past `rows`
// repeat the last one, so every load is unconditional), commit() writes them once they
// have arrived.  The LDS holds ROWS rows.
template <int K, int NTHR, int ROWS>
struct RowStage {
  static constexpr int PER = (K / 8 + NTHR - 1) / NTHR;   // uint4 per thread per row
  uint4 v[ROWS][PER];
  template <class F>
  __device__ __forceinline__ void issue(int rows, F src_row) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const uint4* p = reinterpret_cast<const uint4*>(src_row(r < rows ? r : rows - 1));
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        const int i = threadIdx.x + NTHR * m;
        v[r][m] = p[K / 8 % NTHR == 0 || i < K / 8 ? i : 0];
      }
    }
  }
  // Every one of the ROWS LDS rows is written (rows past `rows` get the repeated last row):
  // with no branch around the writes the loads stay where issue() put them instead of
  // being sunk to their first use.
  __device__ __forceinline__ void commit(int rows, uint16_t* lds) {
    (void)rows;
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
#pragma unroll
      for (int m = 0; m < PER; ++m) {
        const int i = threadIdx.x + NTHR * m;
        if (K / 8 % NTHR == 0 || i < K / 8) reinterpret_cast<uint4*>(lds + (size_t)r * K)[i] = v[r][m];
      }
    }
  }
};

// ============================================================================ K1
// Router partial for one (16 experts, 16 tokens, quarter of K): wave w takes K chunk
// 4 q + w of 16 with every load up front; the four waves meet in LDS in order and wave 0
// writes rpart[q][t][e].  Experts and tokens past the end read as zeros.
template <int HB>
__device__ __forceinline__ void router_unit(const DecodeArgs& a, int rw, float (*s_red)[4][64]) {
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
  const rsrc_t rw_r = make_rsrc(a.wr, (uint32_t)a.E * H * 2);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)a.T * H * 2);
  const uint32_t wo = e_ok ? 2u * ((uint32_t)(et * 16 + col) * H + c * KC + 8 * g) : kOOB;
  const uint32_t xo = t_ok ? 2u * ((uint32_t)(tt * 16 + col) * H + c * KC + 8 * g) : kOOB;
  uint4 av[NS], bv[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    av[j] = bload16_nt(rw_r, wo, 2 * 32 * j);
    bv[j] = bload16(rx, xo, 2 * 32 * j);
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NS; ++j) acc = mfma16(as_bf16x8(av[j]), as_bf16x8(bv[j]), acc);
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[wave][i][lane] = acc[i];
  __syncthreads();
  if (wave == 0 && t_ok) {
    const int tok = tt * 16 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = et * 16 + 4 * g + i;
      const float v = ((s_red[0][i][lane] + s_red[1][i][lane]) + s_red[2][i][lane]) + s_red[3][i][lane];
      // agent-coherent stores (written through past this XCD's L2): the workgroup that sums
      // the partials may run on another XCD, and a release would write back the whole L2
      if (e < a.E)
        __hip_atomic_store(&a.rpart[((size_t)q * a.T + tok) * a.E + e], v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Top-k of one token by one wave (E <= 256: four logits per lane), k rounds of: the
// largest remaining key (wave reduction), its lowest expert (ballots over the four slots),
// that key removed.  Slots come out ordered by (logit desc, expert asc).  The k experts and
// weights of token t land in slot order in ids_out / wbits_out (LDS); with `out` set,
// logits, ids and weights also go to the caller's arrays.
struct TopkIn {
  float part[4][kRouterParts];   // router partials of this lane's four experts
  float bias[4];
};
// Loads of wave_topk's inputs for token t, issued ahead of its use.
__device__ __forceinline__ void topk_load(const DecodeArgs& a, int t, TopkIn& in) {
  const int lane = threadIdx.x & 63;
  const int E = a.E;
  const rsrc_t rb = make_rsrc(a.bias, a.bias ? (uint32_t)E * 4 : 0u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = i * 64 + lane < E ? i * 64 + lane : 0;
#pragma unroll
    for (int c = 0; c < kRouterParts; ++c) in.part[i][c] = a.rpart[((size_t)c * a.T + t) * E + e];
    in.bias[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, i * 64 + lane < E ? 4u * (i * 64 + lane) : kOOB, 0, 0));
  }
}

// Order-preserving unsigned key of a float (larger float -> larger key, -0 as +0; every
// finite or infinite value maps above 0; every NaN takes the largest key, so NaN ranks
// above every number and all NaNs tie) and its inverse (a NaN key gives a NaN).
__device__ __forceinline__ uint32_t fkey(float f) {
  if (f != f) return 0xFFFFFFFFu;
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Largest value over the wave: within each row of 16 lanes by DPP (quad permutes, half and
// full row mirrors), then across the four rows through scalar reads.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lanes ^ 1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lanes ^ 2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Router logits of this lane's four experts: the partials summed in a fixed order, plus
// the bias.
struct TopkSum {
  float s[4];
};
__device__ __forceinline__ TopkSum topk_sums(const DecodeArgs& a, const TopkIn& in) {
  TopkSum r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kRouterParts; ++c) s += in.part[i][c];
    if (a.bias) s += in.bias[i];
    r.s[i] = s;
  }
  return r;
}

__device__ __forceinline__ void wave_topk(const DecodeArgs& a, int t, const TopkSum& ls, float* s_v, int* s_i,
                                          int* ids_out, int* wbits_out, bool out) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = i * 64 + lane;
    const float s = ls.s[i];
    if (out && e < E) a.logits[(size_t)t * E + e] = s;
    key[i] = e < E ? fkey(s) : 0u;
  }
  for (int r = 0; r < k; ++r) {
    const uint32_t lm = max(max(key[0], key[1]), max(key[2], key[3]));
    const uint32_t m = wave_max_u32(lm);
    int sel = -1;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      const uint64_t b = __ballot(key[i] == m);
      if (b) sel = i * 64 + __ffsll((unsigned long long)b) - 1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) key[i] = i * 64 + lane == sel ? 0u : key[i];
    if (lane == 0) {
      s_v[r] = fkey_value(m);
      s_i[r] = sel;
    }
  }
  wave_lds_sync();
  if (lane < k) {
    const float vmax = s_v[0];
    float sum = 0.f;   // the same (slot) order in every lane
    for (int j = 0; j < k; ++j) sum += expf(s_v[j] - vmax);
    const float wgt = expf(s_v[lane] - vmax) / sum;
    const int mi = s_i[lane];
    if (out) {
      a.ids[(size_t)t * k + lane] = mi;
      a.w[(size_t)t * k + lane] = wgt;
    }
    ids_out[t * k + lane] = mi;
    wbits_out[t * k + lane] = __float_as_int(wgt);
  }
  wave_lds_sync();
}

// Top-k of up to four tokens by one wave (token q valid for q < nq), the four selection
// chains interleaved round by round: each round's wave reduction and lane search is a
// chain of dependent DPP, readlane and scalar steps, and four independent chains keep the
// SIMD busy where one leaves it waiting.  Per token as wave_topk; token q's slots land in
// s_v[q] / s_i[q], its ids and weight bits at tq[q] k + slot of ids_out / wbits_out.
__device__ __forceinline__ void wave_topk4(const DecodeArgs& a, const int* tq, int nq, const TopkSum* ls,
                                           float (*s_v)[32], int (*s_i)[32], int* ids_out, int* wbits_out) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  uint32_t key[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) key[q][i] = i * 64 + lane < E ? fkey(ls[q].s[i]) : 0u;
  }
  for (int r = 0; r < k; ++r) {
    uint32_t m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = wave_max_u32(max(max(key[q][0], key[q][1]), max(key[q][2], key[q][3])));
    int sel[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sel[q] = -1;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        const uint64_t b = __ballot(key[q][i] == m[q]);
        if (b) sel[q] = i * 64 + __ffsll((unsigned long long)b) - 1;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) key[q][i] = i * 64 + lane == sel[q] ? 0u : key[q][i];
    }
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s_v[q][r] = fkey_value(m[q]);
        s_i[q][r] = sel[q];
      }
    }
  }
  wave_lds_sync();
  if (lane < k) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < nq) {
        const float vmax = s_v[q][0];
        float sum = 0.f;   // the same (slot) order in every lane
        for (int j = 0; j < k; ++j) sum += expf(s_v[q][j] - vmax);
        ids_out[tq[q] * k + lane] = s_i[q][lane];
        wbits_out[tq[q] * k + lane] = __float_as_int(expf(s_v[q][lane] - vmax) / sum);
      }
    }
  }
  wave_lds_sync();
}

template <int P0>
struct FinalizeLds {
  int ids[3 * P0];           // [0, P) expert of each pair; [P0, P0 + P) pairs in sorted order;
                             // [2 P0, 2 P0 + P) weight bits of each pair (P <= P0)
  float v[kNW][4][32];
  int i[kNW][4][32];
  int cnt[kMaxE];
  int base[kMaxE];
  int ebase[kMaxE];          // first sorted position of each expert
  int ubase[kMaxE];          // first unit of each expert
  uint8_t wc[kNW][kMaxE];
  int wsum[kNW * 4];
};

// Top-k of tokens t0 .. t1 - 1 (t1 - t0 <= 16: wave w takes t0 + w + 4 i, the four at once),
// every input load issued before the first selection; writes logits, ids and weights.
__device__ __forceinline__ void route_topk_tile(const DecodeArgs& a, int t0, int t1, float (*s_v)[32], int (*s_i)[32],
                                                int* ids_l, int* wb_l) {
  const int wave = threadIdx.x >> 6;
  TopkIn in[4];
  int tq[4], nq = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tq[i] = t0 + wave + kNW * i;
    nq += tq[i] < t1;
    topk_load(a, min(tq[i], t1 - 1), in[i]);
  }
  // Every sum before the first selection and every store after the last: a memory
  // operation in flight during the selection rounds (whose registers the rounds reuse)
  // makes each round wait for it.
  TopkSum ls[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ls[i] = topk_sums(a, in[i]);
  wave_topk4(a, tq, nq, ls, s_v, s_i, ids_l, wb_l);
  const int lane = threadIdx.x & 63, E = a.E, k = a.k;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = tq[i];
    if (t < t1) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q * 64 + lane < E) a.logits[(size_t)t * E + q * 64 + lane] = ls[i].s[q];
      if (lane < k) {
        // agent-coherent: the workgroup that permutes all pairs may run on another XCD
        __hip_atomic_store(&a.ids[(size_t)t * k + lane], ids_l[t * k + lane], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.w[(size_t)t * k + lane], __int_as_float(wb_l[t * k + lane]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Stable permutation of all pairs by expert (E <= 256: one expert per thread) and the work
// lists, from the ids and weights every tile's top-k wrote: units of <= 16 pairs of one
// expert (with each pair's token and weight) and half-units of <= QN.
// With `in_lds` the ids and weight bits are already in L.ids (one token tile: this workgroup
// selected them all) and are not read back.
template <int P0, int QN>
__device__ __forceinline__ void route_permute(const DecodeArgs& a, FinalizeLds<P0>& L, bool in_lds = false) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k, P = a.T * k;
  if (!in_lds) {
    for (int f = tid; f < P; f += kWG) {
      L.ids[f] = a.ids[f];
      L.ids[2 * P0 + f] = __float_as_int(a.w[f]);
    }
  }
  if (tid < E) L.cnt[tid] = 0;
  lds_barrier();
  for (int f = tid; f < P; f += kWG) atomicAdd(&L.cnt[L.ids[f]], 1);
  lds_barrier();
  const int c = tid < E ? L.cnt[tid] : 0;
  const int n16 = (c + 15) / 16, n8 = (c + QN - 1) / QN;
  int ic = c, iu = n16, ih = n8, ia = c > 0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int yc = __shfl_up(ic, o, 64), yu = __shfl_up(iu, o, 64);
    const int yh = __shfl_up(ih, o, 64), ya = __shfl_up(ia, o, 64);
    if (lane >= o) { ic += yc; iu += yu; ih += yh; ia += ya; }
  }
  if (lane == 63) {
    L.wsum[wave * 4] = ic; L.wsum[wave * 4 + 1] = iu; L.wsum[wave * 4 + 2] = ih; L.wsum[wave * 4 + 3] = ia;
  }
  lds_barrier();
  int bc = 0, bu = 0, bh = 0, tu = 0, th = 0, ta = 0;
  for (int w2 = 0; w2 < kNW; ++w2) {
    if (w2 < wave) { bc += L.wsum[w2 * 4]; bu += L.wsum[w2 * 4 + 1]; bh += L.wsum[w2 * 4 + 2]; }
    tu += L.wsum[w2 * 4 + 1]; th += L.wsum[w2 * 4 + 2]; ta += L.wsum[w2 * 4 + 3];
  }
  const int start = bc + ic - c;
  const int u0 = bu + iu - n16;
  const int h0 = bh + ih - n8;
  if (tid < E) {
    L.base[tid] = start;
    L.ebase[tid] = start;
    L.ubase[tid] = u0;
    a.offsets[tid] = start;
  }
  if (tid == 0) {
    a.offsets[E] = P;
    a.wl[0] = ta;
    a.wl[1] = tu;
    a.wl[2] = th;
  }
  lds_barrier();
  if (P <= kWG) {
    // one thread per pair: its rank among the earlier pairs of its expert
    if (tid < P) {
      const int e = L.ids[tid];
      int r = 0;
      for (int f = 0; f < tid; ++f) r += L.ids[f] == e;
      const int pos = L.base[e] + r;
      a.sorted_pair[pos] = tid;
      a.pair_pos[tid] = pos;
      L.ids[P0 + pos] = tid;
    }
  } else {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
    for (int c0 = 0; c0 < P; c0 += kWG) {
      for (int i = tid; i < kNW * kMaxE; i += kWG) L.wc[i / kMaxE][i % kMaxE] = 0;
      lds_barrier();
      const int f = c0 + tid;
      const bool valid = f < P;
      const int e = valid ? L.ids[f] : 0;
      uint64_t peers = __ballot(valid);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t ones = __ballot(valid && bit);
        peers &= bit ? ones : ~ones;
      }
      const int rank = __popcll(peers & lt);
      if (valid && rank == 0) L.wc[wave][e] = (uint8_t)__popcll(peers);
      lds_barrier();
      if (valid) {
        int pre = 0;
        for (int w2 = 0; w2 < wave; ++w2) pre += L.wc[w2][e];
        const int pos = L.base[e] + pre + rank;
        a.sorted_pair[pos] = f;
        a.pair_pos[f] = pos;
        L.ids[P0 + pos] = f;
      }
      lds_barrier();
      if (tid < E) {
        int s2 = 0;
        for (int w2 = 0; w2 < kNW; ++w2) s2 += L.wc[w2][tid];
        L.base[tid] += s2;
      }
      lds_barrier();
    }
  }
  lds_barrier();
  // work lists: units (expert, <= 16 pairs) and down entries (<= QN pairs); each pair writes
  // its own token / weight slot, slots past a unit's last pair are left as they are (the
  // readers clamp to the last pair)
  if (tid < E) {
    for (int q = 0; q < n16; ++q) a.ut[u0 + q] = make_int4(tid, start + 16 * q, min(16, c - 16 * q), 0);
    for (int r = 0; r < n8; ++r)
      a.hl[h0 + r] = make_int4(tid, start + QN * r, min(QN, c - QN * r), (u0 + QN * r / 16) * 16 + (QN * r) % 16);
  }
  for (int pos = tid; pos < P; pos += kWG) {
    const int f = L.ids[P0 + pos];
    const int e = L.ids[f];
    const int rel = pos - L.ebase[e];
    const int slot = (L.ubase[e] + rel / 16) * 16 + rel % 16;
    a.utok[slot] = f / k;
    a.uw[slot] = __int_as_float(L.ids[2 * P0 + f]);
  }
}

// Shared gate/up beyond kXT tokens, beside the routing chain of the first kernel: rows
// 16 rt .. 16 rt + 15 of the bf16 gate and up matrices (A) for up to MT token tiles (B = x
// columns), the 4 waves splitting K.  A block's weights are loaded once for all tiles and
// every tile's x operand of the block at once, while the next block's weights are in flight.
// Tiles tt0 .. tt0 + MT - 1: at four tiles two workgroups of two tiles share each row tile.
// The waves' partials meet in LDS in wave order, one tile at a time.
template <int HB, int IB, int MT>
__device__ __forceinline__ void shared_gateup_k1(const DecodeArgs& a, int rt, int tt0, float (*s_red)[2][4][64]) {
  constexpr int H = HB * 256, I = IB * 256, NBW = (HB + kNW - 1) / kNW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int T = a.T, n_tt = (T + 15) / 16;
  const int b0 = wave * HB / kNW, b1 = (wave + 1) * HB / kNW;
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)T * H * 2);
  const rsrc_t rg = make_rsrc(a.sg, (uint32_t)I * H * 2), ru = make_rsrc(a.su, (uint32_t)I * H * 2);
  const uint32_t wo = 2u * (uint32_t)(16 * rt + col) * H;
  auto load_w = [&](int m, uint4 (*w)[8]) {
    const int bk = b0 + m;
    const bool ok = bk < b1;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t off = 2u * (256 * bk + 64 * g + 8 * t);
      w[0][t] = bload16(rg, ok ? wo + off : kOOB);
      w[1][t] = bload16(ru, ok ? wo + off : kOOB);
    }
  };
  auto load_x = [&](int m, int tt, uint4* xv) {
    const int bk = b0 + m, tok = 16 * (tt0 + tt) + col;
    const bool ok = bk < b1 && tok < T;
#pragma unroll
    for (int t = 0; t < 8; ++t) xv[t] = bload16(rx, ok ? 2u * ((uint32_t)tok * H + 256 * bk + 64 * g + 8 * t) : kOOB);
  };
  f32x4_t acc[MT][2];
#pragma unroll
  for (int tt = 0; tt < MT; ++tt) { acc[tt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f}; acc[tt][1] = acc[tt][0]; }
  uint4 w[2][2][8];
  load_w(0, w[0]);
#pragma unroll
  for (int m = 0; m < NBW; ++m) {
    uint4 xv[MT][8];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) load_x(m, tt, xv[tt]);   // tiles past the last read zeros
    if (m + 1 < NBW) load_w(m + 1, w[(m + 1) & 1]);
    const int ws = m & 1;
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
      if (tt0 + tt < n_tt) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          acc[tt][0] = mfma16(as_bf16x8(w[ws][0][t]), as_bf16x8(xv[tt][t]), acc[tt][0]);
          acc[tt][1] = mfma16(as_bf16x8(w[ws][1][t]), as_bf16x8(xv[tt][t]), acc[tt][1]);
        }
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < MT; ++tt) {
    if (tt0 + tt < n_tt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) { s_red[wave][0][i][lane] = acc[tt][0][i]; s_red[wave][1][i][lane] = acc[tt][1][i]; }
      __syncthreads();
      const int tok = 16 * (tt0 + tt) + col;
      if (wave == 0 && tok < T) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float gs = 0.f, us = 0.f;
          for (int w2 = 0; w2 < kNW; ++w2) { gs += s_red[w2][0][i][lane]; us += s_red[w2][1][i][lane]; }
          store_hilo(a.hs + (size_t)tok * I + 16 * rt + 4 * g + i, (size_t)T * I, silu_mul(gs, us));
        }
      }
      __syncthreads();
    }
  }
}

template <int HB>
__device__ __forceinline__ void quant_x8(const DecodeArgs& a, int i);

// Beyond kXT tokens, first kernel: the shared expert's gate/up (workgroups n_router_wg ..)
// and, with MXFP4 routed experts, x -> E4M3 (the n_xq_wg workgroups after those) beside the
// routing -- router partials (per 16-token tile), then a chain of two tickets (relaxed
// agent-scope atomics on counters in the workspace, taken once the data they hand over,
// written with agent-coherent stores, has completed; the taker invalidates with an acquire
// fence): the last router workgroup of a token tile sums that tile's partials and picks its
// tokens' top-k (tiles in parallel); the last tile to finish sorts all pairs and writes the
// work lists, then leaves every counter at zero for the next call.  With one tile the first
// ticket's taker goes straight on to the permutation.
template <int HB, int IB, int MT, int P0, int QN>
// (the register budget of one wave per SIMD, which the shared gate/up's weight prefetch may
// use)
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(1, 1))) void k1_route(DecodeArgs a) {
  __shared__ __align__(16) float s_red[kNW][4][64];
  __shared__ int s_last;
  __shared__ FinalizeLds<P0> s_fin;
  const int b = blockIdx.x;
  if (b >= a.n_router_wg + a.n_sgu_wg) {
    quant_x8<HB>(a, (b - a.n_router_wg - a.n_sgu_wg) * kWG + (int)threadIdx.x);
    return;
  }
  if (b >= a.n_router_wg) {
    // four token tiles: two workgroups per 16 weight rows, each with two tiles (the pair runs
    // on one XCD, 128 workgroups apart, so the second weight read mostly hits L2)
    const int r = b - a.n_router_wg;
    if constexpr (MT == 4)
      shared_gateup_k1<HB, IB, 2>(a, r % (IB * 16), 2 * (r / (IB * 16)), reinterpret_cast<float(*)[2][4][64]>(s_fin.ids));
    else
      shared_gateup_k1<HB, IB, MT>(a, r, 0, reinterpret_cast<float(*)[2][4][64]>(s_fin.ids));
    return;
  }
  router_unit<HB>(a, b, s_red);
  const int per_tile = kRouterParts * ((a.E + 15) / 16);
  const int tt = b / per_tile, n_tt = (a.T + 15) / 16;
  // wave 0 wrote this workgroup's partial with agent-coherent stores: once they have
  // completed (vmcnt 0), its first lane takes the tile ticket with a relaxed atomic.  (An
  // acquire-release ticket would write back this XCD's whole L2 first, once per workgroup.)
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    s_last = __hip_atomic_fetch_add(&a.ctr[1 + tt], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == per_tile - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // every wave reads the tile's partials
  route_topk_tile(a, 16 * tt, min(16 * tt + 16, a.T), s_fin.v[threadIdx.x >> 6], s_fin.i[threadIdx.x >> 6],
                  s_fin.ids, s_fin.ids + 2 * P0);
  if (n_tt == 1) {
    // one token tile: this workgroup holds every pair's id and weight in LDS already, so the
    // second ticket (and its fences, an L2 write-back among them) has nothing to order
    __syncthreads();
    route_permute<P0, QN>(a, s_fin, true);
    if ((int)threadIdx.x <= n_tt) a.ctr[threadIdx.x] = 0;
    return;
  }
  // every wave's ids and weights (agent-coherent stores) complete before the relaxed ticket
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(&a.ctr[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_tt - 1;
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  route_permute<P0, QN>(a, s_fin);
  if ((int)threadIdx.x <= n_tt) a.ctr[threadIdx.x] = 0;
}

// ---------------------------------------------------------------------------- small T
constexpr int kMaxPL = kXT * 32;   // pairs of a small-T layer (k <= 32)

// Up to kXT tokens the first kernel only computes the router partials: every routed gate/up
// workgroup then derives the routing itself (below), so no workgroup waits on another.
// forward declaration (defined with the second kernel's pieces)
template <int HB, int IB, int XR, int NT>
__device__ __forceinline__ void shared_gateup_valu(const DecodeArgs& a, int sw, uint16_t* s_x);

// Up to kXT tokens, first kernel: everything that needs x alone -- the router partials
// (workgroups 0 .. n_router_wg - 1, dispatched first) and the shared expert's gate/up, whose
// 50 MB stream (Hy4) runs beside the router's short chain.
template <int HB, int IB, int XR>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4))) void k1s_router(DecodeArgs a) {
  extern __shared__ __align__(16) uint16_t s_x[];   // shared workgroups: XR bf16 x rows
  __shared__ __align__(16) float s_red[kNW][4][64];
  const int b = blockIdx.x;
  if (b < a.n_router_wg) {
    router_unit<HB>(a, b, s_red);
    return;
  }
  shared_gateup_valu<HB, IB, XR, kWG>(a, b - a.n_router_wg, s_x);
}

// Routing of up to kXT tokens inside one workgroup (LDS only): top-k per token (one wave per
// token), the stable order of the pairs by expert, and the units (one per selected expert:
// an expert holds at most kXT pairs).  With `out` the workgroup also writes the routing
// outputs and the down kernel's work lists.
struct SmallRoute {
  float v[kNW][32];
  int i[kNW][32];
  int ids[kMaxPL];      // expert of pair f = t k + j
  int wb[kMaxPL];       // routing weight bits of pair f
  int sorted[kMaxPL];   // pair at each sorted position
  int same[kMaxPL];     // rank of the pair at each position among its expert's pairs
  int4 ut[kMaxPL];      // units: {expert, first position, pairs, 0}
  int utok[kMaxPL];     // token of the pair at each position
  int wcnt[2];
  int n_units;
};

__device__ __forceinline__ void small_route_topk(const DecodeArgs& a, SmallRoute& R, const TopkSum& ls, bool out) {
  const int wave = threadIdx.x >> 6;
  if (wave < a.T) wave_topk(a, wave, ls, R.v[wave], R.i[wave], R.ids, R.wb, out);
}

__device__ __forceinline__ void small_route_units(const DecodeArgs& a, SmallRoute& R, bool out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.k, P = a.T * k, E = a.E;
  lds_barrier();
  if (tid < P) {
    const int e = R.ids[tid];
    int before = 0, same = 0;
    for (int f = 0; f < P; ++f) {
      const int ef = R.ids[f];
      before += ef < e;
      same += ef == e && f < tid;
    }
    const int pos = before + same;
    R.sorted[pos] = tid;
    R.same[pos] = same;
    R.utok[pos] = tid / k;
    if (out) {
      a.sorted_pair[pos] = tid;
      a.pair_pos[tid] = pos;
    }
  }
  if (out) {
    for (int e = tid; e <= E; e += (int)blockDim.x) {
      int before = 0;
      for (int f = 0; f < P; ++f) before += R.ids[f] < e;
      a.offsets[e] = before;
    }
  }
  lds_barrier();
  // a unit starts at every position whose pair is its expert's first (P <= 128: two waves)
  bool first = false;
  uint64_t m = 0;
  if (wave < 2) {
    first = tid < P && R.same[tid] == 0;
    m = __ballot(first);
    if (lane == 0) R.wcnt[wave] = __popcll(m);
  }
  lds_barrier();
  if (tid < P) {
    const uint64_t le = ~0ull >> (63 - lane);
    const int u = (wave ? R.wcnt[0] : 0) + __popcll(m & le) - 1;
    const int f = R.sorted[tid];
    const int e = R.ids[f];
    if (first) {
      int n = 0;
      for (int q = tid; q < P && R.ids[R.sorted[q]] == e; ++q) ++n;
      R.ut[u] = make_int4(e, tid, n, 0);
      if (out) {
        a.ut[u] = make_int4(e, tid, n, 0);
        a.hl[u] = make_int4(e, tid, n, 16 * u);
      }
    }
    if (out) {
      const int j = R.same[tid];
      a.utok[16 * u + j] = f / k;
      a.uw[16 * u + j] = __int_as_float(R.wb[f]);
    }
  }
  if (tid == 0) {
    const int nu = R.wcnt[0] + (P > 64 ? R.wcnt[1] : 0);
    R.n_units = nu;
    if (out) {
      a.wl[0] = nu;
      a.wl[1] = nu;
      a.wl[2] = nu;
    }
  }
  lds_barrier();
}

// ============================================================================ K2
// Shared gate/up for up to kXT tokens (x rows in LDS): wave = one row of I, gate and up,
// streamed in 16-byte chunks per lane (chunk c: K = 8 l + 512 c for lane l) with the next
// chunk of both matrices in flight while one is reduced.
template <int HB, int IB, int XR, int NT>
__device__ __forceinline__ void shared_gateup_valu(const DecodeArgs& a, int sw, uint16_t* s_x) {
  constexpr int H = HB * 256, I = IB * 256, NJ = H / 512, RS = NJ < 2 ? NJ : 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T;
  const int row = sw * (NT / 64) + wave;
  RowStage<H, NT, XR> xs;
  xs.issue(T, [&](int r) { return a.x + (size_t)r * H; });
  const uint16_t* gp = a.sg + (size_t)row * H + 8 * lane;
  const uint16_t* up = a.su + (size_t)row * H + 8 * lane;
  uint4 bg[RS], bu[RS];
#pragma unroll
  for (int c = 0; c < RS; ++c) {
    bg[c] = ntload16(gp + 512 * c);
    bu[c] = ntload16(up + 512 * c);
  }
  xs.commit(T, s_x);
  lds_barrier();
  static_assert(XR <= kXT, "staged rows");
  float ag[XR], au[XR];
#pragma unroll
  for (int t = 0; t < XR; ++t) { ag[t] = 0.f; au[t] = 0.f; }
#pragma unroll
  for (int c = 0; c < NJ; ++c) {
    const uint4 wg = bg[c % RS], wu = bu[c % RS];
    if (c + RS < NJ) {
      bg[c % RS] = ntload16(gp + 512 * (c + RS));
      bu[c % RS] = ntload16(up + 512 * (c + RS));
    }
#pragma unroll
    for (int t = 0; t < XR; ++t) {
      if (t < T) {
        const uint4 xv = *reinterpret_cast<const uint4*>(s_x + t * H + 8 * lane + 512 * c);
        ag[t] = dot8(wg, xv, ag[t]);
        au[t] = dot8(wu, xv, au[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < XR; ++t) {
    if (t < T) {
      const float gs = wave_sum(ag[t]), us = wave_sum(au[t]);
      if (lane == 0) store_hilo(a.hs + (size_t)t * I + row, (size_t)T * I, silu_mul(gs, us));
    }
  }
}

// ============================================================================ large T
// Beyond kXT tokens the routed projections run in persistent workgroups of 8 waves over a
// list of work items (gate/up: half-unit of <= 8 pairs; down: unit of <= 16 pairs; each
// with a slice of 128 weight rows, 16 per wave); each workgroup takes a contiguous range of
// the list, so its items mostly share a (half-)unit and the list is split evenly whatever
// the routing.
constexpr int kLW = 512;
constexpr int kLNW = kLW / 64;
constexpr int kSlice = 16 * kLNW;

// Work split of a persistent grid of G workgroups: workgroup b takes the heavy items
// b, b + G, b + 2 G, .. of n_heavy (each costing WH), then the contiguous range [i0, i1) of
// the n light items (each costing WL) that brings its share of the total cost closest to
// its even share (the ranges are monotone in b and cover every light item exactly once).
__device__ __forceinline__ void light_range(int b, int G, int n, int n_heavy, int WL, int WH, int& i0, int& i1) {
  const long C = (long)WL * n + (long)WH * n_heavy;
  const int full = n_heavy / G, rem = n_heavy % G;
  auto end = [&](int bb) {   // end of workgroup bb's light range
    if (bb < 0) return 0L;
    const long heavy = (long)WH * ((long)(bb + 1) * full + min(bb + 1, rem));
    const long e = (C * (bb + 1) / G - heavy) / WL;
    return e < 0 ? 0L : (e > n ? (long)n : e);
  };
  i0 = (int)end(b - 1);
  i1 = b == G - 1 ? n : (int)end(b);
}

// Large-T gate/up: the x rows of a half-unit (<= 8 tokens) in LDS, row r at byte r XROW
// (H bf16 + 16 bytes of padding, so the rows one MFMA operand read touches start in
// different banks); staged once per half-unit, every load issued before the first write.
template <int HB, int NTHR>
__device__ __forceinline__ void stage_x_large(const DecodeArgs& a, const int* toks, int n, uint8_t* s_x) {
  constexpr int H = HB * 256, XROW = 2 * H + 16, PR = H / 8, PER = (8 * PR + NTHR - 1) / NTHR;
  constexpr int PASS = PER < 12 ? PER : 12;
  const int tid = threadIdx.x;
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)a.T * H * 2);
#pragma unroll
  for (int m0 = 0; m0 < PER; m0 += PASS) {
    uint4 v[PASS];
#pragma unroll
    for (int m = 0; m < PASS; ++m) {
      const int idx = tid + NTHR * (m0 + m), r = idx / PR, pc = idx % PR;
      const bool ok = m0 + m < PER && r < n;
      v[m] = bload16(rx, ok ? 2u * (uint32_t)toks[ok ? r : 0] * H + 16u * pc : kOOB);
    }
#pragma unroll
    for (int m = 0; m < PASS; ++m) {
      const int idx = tid + NTHR * (m0 + m), r = idx / PR, pc = idx % PR;
      if (m0 + m < PER && r < 8) *reinterpret_cast<uint4*>(s_x + r * XROW + 16 * pc) = v[m];
    }
  }
}

// One item of the large-T gate/up: wave w multiplies the half-unit's staged x rows (A) with
// rows slice * 128 + 16 w .. + 15 of the expert's gate and up matrices (B, STQ1_0 code
// words staged through the wave's LDS buffers in whole 16-byte row runs, decoded through
// the table) over all of K, then writes h = SiLU(gate) * up as bf16 hi + lo.  No workgroup
// barrier inside: every wave streams on its own.
template <int HB, int IB, int NWV>
__device__ __forceinline__ void routed_gateup_large(const DecodeArgs& a, int e, int pos0, int ntok, int slice,
                                                    const uint32_t* s_lut, const uint8_t* s_x, uint8_t* s_cw) {
  constexpr int H = HB * 256, I = IB * 256, XROW = 2 * H + 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int row0 = slice * 16 * NWV + 16 * wave;
  const size_t wrow = (size_t)e * I + row0;   // the wave's first row
  StqStreamL<HB> sg, su;
  sg.issue(a.gc + wrow * HB * 40, a.gs + (wrow + col) * HB, s_cw + (2 * wave) * StqStreamL<HB>::BYTES);
  su.issue(a.uc + wrow * HB * 40, a.us + (wrow + col) * HB, s_cw + (2 * wave + 1) * StqStreamL<HB>::BYTES);
  const uint8_t* xa = s_x + col * XROW + 128 * g;   // this lane's A operand
  const bool a_on = col < ntok;   // token slots past the half-unit keep zeros, no LDS reads
  f32x4_t ag = {0.f, 0.f, 0.f, 0.f}, au = ag;
  uint4 av[8] = {};
#pragma unroll
  for (int j = 0; j < HB; ++j) {
    if (a_on) {
#pragma unroll
      for (int t = 0; t < 8; ++t) av[t] = *reinterpret_cast<const uint4*>(xa + 512 * j + 16 * t);
    }
    uint2 qg, qu;
    uint32_t hg, hu;
    float dg, du;
    sg.next(j, qg, hg, dg);
    su.next(j, qu, hu, du);
    bf16x8_t wg[8], wu[8];
    stq_block_w(s_lut, qg, hg, wg);
    stq_block_w(s_lut, qu, hu, wu);
    f32x4_t bg = {0.f, 0.f, 0.f, 0.f}, bu = bg;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      bg = mfma16(as_bf16x8(av[t]), wg[t], bg);
      bu = mfma16(as_bf16x8(av[t]), wu[t], bu);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) { ag[i] = fmaf(dg, bg[i], ag[i]); au[i] = fmaf(du, bu[i], au[i]); }
    pin4(ag);
    pin4(au);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = 4 * g + i;
    if (slot < ntok)
      store_hilo(a.h_hi + (size_t)(pos0 + slot) * I + row0 + col, a.h_lo_bytes / 2, silu_mul(ag[i], au[i]));
  }
}

// Waves of a large-T gate/up workgroup: 8, or 4 where 8 x rows and 8 waves' code staging
// would not fit the 160 KB of LDS (H above 6144).
__host__ __device__ constexpr int k2l_waves(int HB) { return HB > 24 ? 4 : 8; }
__host__ __device__ constexpr size_t k2l_lds_x(int HB) { return (size_t)8 * (2 * HB * 256 + 16); }

// Large T, second kernel: the routed gate/up items (half-unit, 16 rows per wave of I),
// persistent workgroups over contiguous ranges of the item list; x is restaged when the
// half-unit changes.
template <int HB, int IB>
__global__ __launch_bounds__(kLW) void k2l_gateup(DecodeArgs a) {
  constexpr int I = IB * 256, NWV = k2l_waves(HB), NS = I / (16 * NWV);
  static_assert(I % (16 * NWV) == 0, "slices");
  static_assert(k2l_lds_x(HB) + 2 * NWV * StqStreamL<HB>::BYTES + 256 <= 160 * 1024, "LDS");
  __shared__ uint32_t s_lut[64];                  // first: table offsets fit the offset field
  __shared__ __align__(16) uint8_t s_cw[2 * NWV * StqStreamL<HB>::BYTES];   // code staging
  extern __shared__ __align__(16) uint8_t s_xl[];  // 8 x rows
  build_lut(s_lut);
  int i0, i1;
  light_range(blockIdx.x, gridDim.x, a.wl[2] * NS, 0, 1, 1, i0, i1);
  int staged = -1;
  int4 hu = make_int4(0, 0, 0, 0);
  for (int i = i0; i < i1; ++i) {
    const int h = i / NS;
    if (h != staged) {
      hu = a.hl[h];
      __syncthreads();   // every wave is done with the previous rows
      stage_x_large<HB, 64 * NWV>(a, a.utok + hu.w, hu.z, s_xl);
      __syncthreads();
      staged = h;
    }
    routed_gateup_large<HB, IB, NWV>(a, hu.x, hu.y, hu.z, i % NS, s_lut, s_xl, s_cw);
  }
}

// Large-T down: the A operand of a unit (or of a 16-token tile of the shared expert) as two
// 16-row halves in LDS: pairs 8q .. 8q+7 in half q, pair p's bf16 hi row as A row
// 2 (p - 8q) and its lo row as 2 (p - 8q) + 1; rows of I bf16 + 16 bytes of padding.  Rows
// `first` .. `first` + n - 1 of the hi rows at byte 0 of rh (lo rows at lo_bytes); rows past
// n are zero.  All loads are issued before the first write.
template <int IB>
__device__ __forceinline__ void stage_h_large(rsrc_t rh, uint32_t lo_bytes, int first, int n, uint8_t* s_h) {
  constexpr int I = IB * 256, HROW = 2 * I + 16, PR = I / 8, PER = 2 * 16 * PR / kLW;
  constexpr int PASS = PER < 8 ? PER : 8;   // loads in flight per thread and pass
  static_assert((2 * 16 * PR) % kLW == 0 && PER % PASS == 0, "pieces");
  const int tid = threadIdx.x;
#pragma unroll
  for (int m0 = 0; m0 < PER; m0 += PASS) {
    uint4 v[PASS];
#pragma unroll
    for (int m = 0; m < PASS; ++m) {
      const int idx = tid + kLW * (m0 + m);
      const int q = idx / (16 * PR), r = (idx / PR) % 16, pc = idx % PR;
      const int p = 8 * q + (r >> 1);
      v[m] = bload16(rh, p < n ? (r & 1 ? lo_bytes : 0u) + 2u * (uint32_t)(first + p) * I + 16u * pc : kOOB);
    }
#pragma unroll
    for (int m = 0; m < PASS; ++m) {
      const int idx = tid + kLW * (m0 + m);
      const int q = idx / (16 * PR), r = (idx / PR) % 16, pc = idx % PR;
      *reinterpret_cast<uint4*>(s_h + (16 * q + r) * HROW + 16 * pc) = v[m];
    }
  }
}

// One shared-expert down item: tokens 16 tt .. 16 tt + 15 (staged A) times rows slice * 128 +
// 16 w .. + 15 of the bf16 down matrix (B, one block ahead in registers); writes y_shared.
template <int HB, int IB>
__device__ __forceinline__ void shared_down_item(const DecodeArgs& a, int tt, int slice, const uint8_t* s_h) {
  constexpr int H = HB * 256, I = IB * 256, HROW = 2 * I + 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int row = slice * kSlice + 16 * wave + col;
  const rsrc_t rw = make_rsrc(a.sd, (uint32_t)H * I * 2);
  const uint32_t wo = 2u * (uint32_t)row * I;
  uint4 w[2][8];
#pragma unroll
  for (int t = 0; t < 8; ++t) w[0][t] = bload16(rw, wo + 2u * (64 * g + 8 * t));
  const uint8_t* a0 = s_h + col * HROW + 128 * g;
  const uint8_t* a1 = a0 + 16 * HROW;
  f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    if (j + 1 < IB) {
#pragma unroll
      for (int t = 0; t < 8; ++t) w[(j + 1) & 1][t] = bload16(rw, wo + 2u * (256 * (j + 1) + 64 * g + 8 * t));
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(a0 + 512 * j + 16 * t);
      const uint4 x1 = *reinterpret_cast<const uint4*>(a1 + 512 * j + 16 * t);
      c0 = mfma16(as_bf16x8(x0), as_bf16x8(w[j & 1][t]), c0);
      c1 = mfma16(as_bf16x8(x1), as_bf16x8(w[j & 1][t]), c1);
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t0 = 16 * tt + 2 * g + m;
    if (t0 < a.T) a.y_shared[(size_t)t0 * H + row] = c0[2 * m] + c0[2 * m + 1];
    if (t0 + 8 < a.T) a.y_shared[(size_t)(t0 + 8) * H + row] = c1[2 * m] + c1[2 * m + 1];
  }
}

// The STQ1_0 down rows of one item in flight: all NB (<= 8) blocks of this lane's row (code
// words and high bits) and its scale group.  Loads of an absent item read as zeros.
template <int NB>
struct DownRing {
  uint2 q[NB];
  uint32_t qh[NB];
  uint4 sc;
  __device__ __forceinline__ void load_scales(rsrc_t rs, uint32_t so) {
    if constexpr (NB == 1) {
      sc = make_uint4(__builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0), 0u, 0u, 0u);
    } else if constexpr (NB == 2) {
      sc = make_uint4(__builtin_amdgcn_raw_buffer_load_b32(rs, so, 0, 0), 0u, 0u, 0u);
    } else if constexpr (NB == 4) {
      const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, so, 0, 0));
      sc = make_uint4(v.x, v.y, 0u, 0u);
    } else {
      static_assert(NB == 8, "one scale group");
      sc = bload16(rs, so);
    }
  }
  // block j of the row starting at byte `row` of the codes: this lane's 8 code bytes (group
  // g) and its 16 high bits
  __device__ __forceinline__ void load_block(rsrc_t rc, uint32_t row, int j) {
    const int g = (threadIdx.x & 63) >> 4;
    q[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, row + 8 * g, 40 * j, 0));
    qh[j] = __builtin_amdgcn_raw_buffer_load_b16(rc, row + 32 + 2 * g, 40 * j, 0);
  }
};

// One routed down item: the unit's staged h (A; NH halves) times rows r16 .. r16 + 15 of its
// expert's down matrix (B, from the ring; the next item's blocks are loaded as this item's
// are consumed, at code offset nco / scale offset nso); writes y_pairs.
template <int HB, int IB, int NH>
__device__ __forceinline__ void routed_down_item(const DecodeArgs& a, int pos0, int npairs, int r16,
                                                 DownRing<IB>& ring, rsrc_t rc, rsrc_t rs, uint32_t nco,
                                                 uint32_t nso, const uint32_t* s_lut, const uint8_t* s_h) {
  constexpr int H = HB * 256, I = IB * 256, HROW = 2 * I + 16;
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const uint4 sc = ring.sc;
  ring.load_scales(rs, nso);
  const uint8_t* a0 = s_h + col * HROW + 128 * g;
  f32x4_t acc[NH];
#pragma unroll
  for (int q = 0; q < NH; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const uint2 qj = ring.q[j];
    const uint32_t qhj = ring.qh[j];
    ring.load_block(rc, nco, j);
    bf16x8_t wv[8];
    stq_block_w(s_lut, qj, qhj, wv);
    // two MFMA chains per half (even and odd steps)
    f32x4_t b[2][NH];
#pragma unroll
    for (int q = 0; q < NH; ++q) { b[0][q] = f32x4_t{0.f, 0.f, 0.f, 0.f}; b[1][q] = b[0][q]; }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int q = 0; q < NH; ++q) {
        const uint4 x = *reinterpret_cast<const uint4*>(a0 + q * 16 * HROW + 512 * j + 16 * t);
        b[t & 1][q] = mfma16(as_bf16x8(x), wv[t], b[t & 1][q]);
      }
    }
    const float d = scale_of(sc, j);
#pragma unroll
    for (int q = 0; q < NH; ++q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[q][i] = fmaf(d, b[0][q][i] + b[1][q][i], acc[q][i]);
      pin4(acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < NH; ++q) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int p = 8 * q + 2 * g + m;
      if (p < npairs) a.y_pairs[(size_t)(pos0 + p) * H + r16 + col] = acc[q][2 * m] + acc[q][2 * m + 1];
    }
  }
}

// Large T, third kernel: the shared expert's down items (16-token tile, 128 rows: each
// weighs about 12 routed items -- bf16 against 42/256 bytes per weight -- so they are dealt
// round-robin, at most one or two per workgroup) and the routed down items (contiguous
// ranges), persistent workgroups.  A unit's (or tile's) h is staged once per change.
constexpr int kSharedItemWeight = 12;
template <int HB, int IB>
__global__ __launch_bounds__(kLW) void k3l_down(DecodeArgs a) {
  constexpr int H = HB * 256, I = IB * 256, NS = H / kSlice;
  static_assert(H % kSlice == 0, "slices");
  extern __shared__ __align__(16) uint8_t s_h[];   // 32 A rows of 2 I + 16 bytes
  __shared__ uint32_t s_lut[64];
  const int wave = threadIdx.x >> 6, col = threadIdx.x & 15;
  const int T = a.T;
  const int n_sh = a.sd && !a.ysh_ready ? ((T + 15) / 16) * NS : 0;
  const int n_units = a.wl[1];
  int i0, i1;
  light_range(blockIdx.x, gridDim.x, n_units * NS, n_sh, 1, kSharedItemWeight, i0, i1);
  build_lut(s_lut);
  if (n_sh) {
    const rsrc_t rhs = make_rsrc(a.hs, (uint32_t)T * I * 4);
    int staged = -1;
    for (int si = blockIdx.x; si < n_sh; si += gridDim.x) {
      const int tt = si / NS;
      if (tt != staged) {
        __syncthreads();   // every wave is done with the previous tile
        stage_h_large<IB>(rhs, (uint32_t)T * I * 2, 16 * tt, min(16, T - 16 * tt), s_h);
        __syncthreads();
        staged = tt;
      }
      shared_down_item<HB, IB>(a, tt, si % NS, s_h);
    }
  }
  int i = i0;
  if (i >= i1) return;
  const rsrc_t rh = make_rsrc(a.h_hi, a.h_bytes);
  const rsrc_t rc = make_rsrc(a.dc, (uint32_t)((size_t)a.E * H * IB * 40));
  const rsrc_t rs = make_rsrc(a.ds, (uint32_t)((size_t)a.E * H * IB * 2));
  auto code_off = [&](int e, int slice) {   // this lane's down row of expert e, item slice
    return (uint32_t)(((size_t)e * H + slice * kSlice + 16 * wave + col) * IB * 40);
  };
  auto scale_off = [&](int e, int slice) {
    return (uint32_t)(((size_t)e * H + slice * kSlice + 16 * wave + col) * IB * 2);
  };
  int u = i / NS;
  int4 un = a.ut[u];
  int4 un_next = a.ut[min(u + 1, n_units - 1)];
  DownRing<IB> ring;
  {
    const int sl = i % NS;
    const uint32_t co = code_off(un.x, sl);
#pragma unroll
    for (int j = 0; j < IB; ++j) ring.load_block(rc, co, j);
    ring.load_scales(rs, scale_off(un.x, sl));
  }
  // one unit's items at a time, the unit's half count fixed for the inner loop
  while (i < i1) {
    const int ui = i / NS;
    if (ui != u) {       // the next unit of the range
      u = ui;
      un = un_next;
      un_next = a.ut[min(u + 1, n_units - 1)];
    }
    __syncthreads();
    stage_h_large<IB>(rh, a.h_lo_bytes, un.y, un.z, s_h);
    __syncthreads();
    const int iend = min(i1, (u + 1) * NS);
    auto run = [&](auto nh_tag) {
      constexpr int NHC = decltype(nh_tag)::value;
      for (; i < iend; ++i) {
        const int slice = i % NS;
        uint32_t nco = kOOB, nso = kOOB;
        if (i + 1 < i1) {
          const bool same = slice + 1 < NS;
          const int e2 = same ? un.x : un_next.x;
          const int s2 = same ? slice + 1 : 0;
          nco = code_off(e2, s2);
          nso = scale_off(e2, s2);
        }
        routed_down_item<HB, IB, NHC>(a, un.y, un.z, slice * kSlice + 16 * wave, ring, rc, rs, nco, nso, s_lut, s_h);
      }
    };
    if (un.z > 8) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 1>{});
  }
}

// Shared down for up to kXT tokens: wave w takes NR consecutive rows from row0 + NR w,
// streamed in 16-byte chunks per lane (chunk j: K = 8 l + 512 j for lane l; the last chunk
// is half-used when I is an odd multiple of 256), R chunks in flight; h comes as bf16
// hi + lo rows from `hs` (LDS).  Writes y_shared and, with ACC, adds it into the wave's
// combine sums (a 16-row slice: row NR w + r of the slice).
// NR rows per wave; SR: row stride of the per-wave output sums in LDS.
template <int HB, int IB, int NR, bool ACC, int SR = 16>
struct SharedDown {
  static constexpr int H = HB * 256, I = IB * 256, NJ = (IB + 1) / 2, NI = NR * NJ, R = NI < 4 ? NI : 4;
  uint4 w[R];
  rsrc_t rsd;
  uint32_t rb;       // byte offset of this wave's first row
  int lcol;
  bool last_ok;

  __device__ __forceinline__ uint4 load(int it) const {
    const int j = it / NR, r = it % NR;
    const uint32_t cl = j == NJ - 1 ? lcol : (threadIdx.x & 63);
    return bload16_nt(rsd, rb + 2u * (r * I + 8 * cl), 2 * 512 * j);
  }
  __device__ __forceinline__ void issue(const DecodeArgs& a, int row0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    last_ok = (IB % 2 == 0) || lane < 32;
    lcol = last_ok ? lane : 0;
    rsd = make_rsrc(a.sd, a.sd ? (uint32_t)H * I * 2 : 0u);
    rb = 2u * (uint32_t)(row0 + NR * wave) * I;
#pragma unroll
    for (int it = 0; it < R; ++it) w[it] = load(it);
  }
  __device__ __forceinline__ void run(const DecodeArgs& a, int row0, const uint16_t* hs, float* s_acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int T = a.T;
    const size_t lo = (size_t)T * I;
    float acc[NR][kXT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < kXT; ++t) acc[r][t] = 0.f;
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const uint4 wv = w[it % R];
      if (it + R < NI) w[it % R] = load(it + R);
      const int j = it / NR, r = it % NR;
      const int cl = j == NJ - 1 ? lcol : lane;
#pragma unroll
      for (int t = 0; t < kXT; ++t) {
        if (t < T) {
          const uint16_t* hp = hs + (size_t)t * I + 8 * cl + 512 * j;
          uint4 hh = *reinterpret_cast<const uint4*>(hp);
          uint4 hl = *reinterpret_cast<const uint4*>(hp + lo);
          if (j == NJ - 1 && !last_ok) { hh = make_uint4(0u, 0u, 0u, 0u); hl = hh; }
          acc[r][t] = dot8(wv, hl, dot8(wv, hh, acc[r][t]));
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kXT; ++t) {
      if (t < T) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float v = wave_sum(acc[r][t]);
          if (lane == 0) {
            a.y_shared[(size_t)t * H + row0 + NR * wave + r] = v;
            if constexpr (ACC) s_acc[(wave * T + t) * SR + NR * wave + r] += v;
          }
        }
      }
    }
  }
};

// Shared down for up to kXT tokens in the second kernel (beside the routed gate/up): 16
// output rows per workgroup, 4 per wave; the shared h (bf16 hi rows, then lo rows, written by
// the first kernel) is loaded first, the rows' weight chunks next, and h lands in LDS before
// the stream is reduced.  Writes y_shared; the down kernel adds it into the combine.
template <int HB, int IB, int XR>
__device__ __forceinline__ void shared_down_small(const DecodeArgs& a, int sw, uint16_t* s_h) {
  constexpr int I = IB * 256;
  constexpr int PER = (XR * I / 4 + kWG - 1) / kWG;   // uint4 of h (hi + lo) per thread
  const int n16 = a.T * I / 4;
  const int row0 = sw * 16;
  const uint4* src = reinterpret_cast<const uint4*>(a.hs);
  uint4 v[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int i = threadIdx.x + kWG * m;
    v[m] = src[i < n16 ? i : 0];
  }
  SharedDown<HB, IB, 4, false> sdn;
  sdn.issue(a, row0);
  // branch-free: pieces past the end rewrite piece 0 with the value thread 0 writes there
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int i = threadIdx.x + kWG * m;
    reinterpret_cast<uint4*>(s_h)[i < n16 ? i : 0] = v[m];
  }
  lds_barrier();
  sdn.run(a, row0, s_h, nullptr);
}

// ============================================================================ K3
// Routed gate/up of one work item (unit, 32 rows of I) of a small-T layer, every token's x
// row already in LDS: wave = (16-row tile, gate|up) over all of K; the gate and up waves of
// a tile meet in LDS and the gate wave writes h = SiLU(gate) * up as bf16 hi + lo.
template <int HB, int IB>
__device__ __forceinline__ void routed_gateup_small(const DecodeArgs& a, int wi, const uint32_t* s_lut,
                                                    const uint16_t* s_x, float (*s_red)[2][4][64],
                                                    const SmallRoute& R, uint8_t* s_cw) {
  constexpr int H = HB * 256, I = IB * 256, NTP = I / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int un_i = wi / NTP, tp = wi % NTP;
  const int4 un = R.ut[un_i];
  const int e = un.x, pos0 = un.y, ntok = un.z;
  const int mat = wave & 1, tl = wave >> 1;
  const int row0 = (2 * tp + tl) * 16;
  const size_t wrow = (size_t)e * I + row0 + col;
  StqStreamL<HB> st;
  st.issue((mat ? a.uc : a.gc) + (wrow - col) * HB * 40, (mat ? a.us : a.gs) + wrow * HB,
           s_cw + wave * StqStreamL<HB>::BYTES);
  const int tok = R.utok[pos0 + (col < ntok ? col : ntok - 1)];
  const f32x4_t acc = st.run_lds(s_lut, s_x + tok * H + 64 * g, col < ntok);
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[tl][mat][i][lane] = acc[i];
  __syncthreads();
  if (mat == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 4 * g + i;
      if (slot < ntok)
        store_hilo(a.h_hi + (size_t)(pos0 + slot) * I + row0 + col, a.h_lo_bytes / 2,
                   silu_mul(s_red[tl][0][i][lane], s_red[tl][1][i][lane]));
    }
  }
  __syncthreads();   // s_red is reused by the next work item
}

template <int HB, int IB, int XR>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4))) void k2s_gateup(DecodeArgs a) {
  constexpr int H = HB * 256, I = IB * 256;
  static_assert(2 * I <= H, "the shared h (T rows of I fp32) fits the x staging (T rows of H bf16)");
  extern __shared__ __align__(16) uint16_t s_x[];   // XR x rows (bf16), or the shared h
  __shared__ uint32_t s_lut[64];
  __shared__ __align__(16) float s_red[2][2][4][64];
  __shared__ SmallRoute s_rt;
  __shared__ __align__(16) uint8_t s_cw[kNW * StqStreamL<HB>::BYTES];   // code staging
  const int b = blockIdx.x;
  const int T = a.T;
  if (b >= a.n_gu_wg) {
    shared_down_small<HB, IB, XR>(a, b - a.n_gu_wg, s_x);
    return;
  }
  {
    // The x rows and the router partials are loaded and used in one branch-free stretch
    // (every wave loads and sums some token's partials, only waves < T use them), so all of
    // these loads are in flight together: a partial load placed in a branch would be sunk to
    // its use and issued only after x had arrived.
    RowStage<H, kWG, XR> xs;
    xs.issue(T, [&](int r) { return a.x + (size_t)r * H; });
    TopkIn in;
    topk_load(a, min((int)(threadIdx.x >> 6), T - 1), in);
    build_lut(s_lut);
    xs.commit(T, s_x);
    const TopkSum ls = topk_sums(a, in);
    small_route_topk(a, s_rt, ls, b == 0);
    small_route_units(a, s_rt, b == 0);
    const int n_items = s_rt.n_units * (I / 32);
    for (int wi = b; wi < n_items; wi += a.n_gu_wg)
      routed_gateup_small<HB, IB>(a, wi, s_lut, s_x, s_red, s_rt, s_cw);
  }
}

// One token (its routed h fits the LDS), one RW-row slice of the output: every half-unit
// (expert, <= 8 pairs) spread over the 8 waves, each wave adding its results into its own
// LDS sums; out = y_shared (written by the second kernel) + sum over waves in order
// (+ residual).  All routed h is staged in LDS first (hi rows, then lo rows); a routed
// entry is RW / 16 work items, one per 16-row tile.
template <int HB, int IB, int RW = 16>
__global__ __launch_bounds__(64 * kDnWaves) void k3_down_combine(DecodeArgs a) {
  static_assert(RW % 16 == 0, "rows per workgroup");
  constexpr int NTL = RW / 16;
  constexpr int H = HB * 256, I = IB * 256;
  constexpr int kStage = 10;                 // uint4 per thread of staged h
  constexpr int kLoPad = 32;                 // lo rows start 64 bytes past the hi rows' end so a
                                             // pair's hi and lo reads fall in different banks
  extern __shared__ __align__(16) float s_dyn[];  // [kDnWaves][T][RW] sums, then staged h
  __shared__ uint32_t s_lut[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, P = T * a.k;
  const int row0 = blockIdx.x * RW;
  const int col = lane & 15, g = lane >> 4;
  float* s_acc = s_dyn;
  uint16_t* s_h = reinterpret_cast<uint16_t*>(s_dyn + kDnWaves * T * RW);
  // residual and y_shared of this slice (T * RW <= 1024 elements, two per thread), read up front
  const rsrc_t rres = make_rsrc(a.residual, a.residual ? (uint32_t)T * H * 4 : 0u);
  const rsrc_t rysh = make_rsrc(a.y_shared, a.y_shared ? (uint32_t)T * H * 4 : 0u);
  float rs[2], ys[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = tid + 64 * kDnWaves * m;
    const uint32_t o = i < T * RW ? 4u * ((uint32_t)(i / RW) * H + row0 + (i % RW)) : kOOB;
    rs[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rres, o, 0, 0));
    ys[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rysh, o, 0, 0));
  }
  // staged h, 16-byte pieces: routed hi rows, then routed lo rows (the workspace holds them
  // back to back, so the staging is one linear copy).  Branch-free: every piece is written
  // below, so the compiler keeps all loads in flight together (a load inside a conditional
  // write is sunk into it and waited for one at a time).  Pieces past the end reload and
  // rewrite piece 0, the same value thread 0 writes there.
  const int n_r0 = P * I / 8, n_all = 2 * n_r0;
  uint4 hv[kStage];
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.h_hi);
#pragma unroll
    for (int m = 0; m < kStage; ++m) {
      const int i = tid + 64 * kDnWaves * m;
      hv[m] = src[i < n_all ? i : 0];
    }
  }
  build_lut(s_lut);
  for (int i = tid; i < kDnWaves * T * RW; i += 64 * kDnWaves) s_acc[i] = 0.f;
  // the staged rows land before any weight load is issued: otherwise they would queue
  // behind every workgroup's weight stream
#pragma unroll
  for (int m = 0; m < kStage; ++m) {
    int i = tid + 64 * kDnWaves * m;
    i = i < n_all ? i : 0;
    reinterpret_cast<uint4*>(s_h + (i < n_r0 ? 0 : kLoPad))[i] = hv[m];
  }
  // keep the weight loads below: hoisted above these writes, one wave's weight stream
  // queued ahead of another wave's staging loads in the CU's in-order memory queue
  __builtin_amdgcn_sched_barrier(0);
  // first work item's code words, read beside the entry count (a wave without an item
  // streams some valid expert's rows, unused)
  const int n_ent = a.wl[2];
  StqStream<IB, 8> st;
  int it = wave;
  int4 hent = a.hl[it / NTL < a.max_half ? it / NTL : a.max_half - 1];
  {
    const int e0 = min(max(hent.x, 0), a.E - 1);
    const size_t wrow = (size_t)e0 * H + row0 + 16 * (it % NTL) + col;
    st.issue(a.dc + wrow * IB * 40, a.ds + wrow * IB);
  }
  lds_barrier();
  for (; it < n_ent * NTL; it += kDnWaves) {
    const int r16 = row0 + 16 * (it % NTL);   // first output row of this item's tile
    if (it != wave) {
      hent = a.hl[it / NTL];
      const size_t wrow = (size_t)hent.x * H + r16 + col;
      st.issue(a.dc + wrow * IB * 40, a.ds + wrow * IB);
    }
    const int pos0 = hent.y, nq = hent.z;
    {
      // entries of <= 8 pairs: A rows (pair, hi | lo); this lane's pairs are 2g, 2g+1
      const int sp2 = col >> 1;
      int tk[2];
      float wt[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int p = min(2 * g + m, nq - 1);
        tk[m] = a.utok[hent.w + p];
        wt[m] = a.uw[hent.w + p];
      }
      const int pr = pos0 + (sp2 < nq ? sp2 : 0);
      const f32x4_t acc = st.run_lds(s_lut, s_h + (col & 1) * (P * I + kLoPad) + pr * I + 64 * g, sp2 < nq);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int p = 2 * g + m;
        if (p < nq) {
          const float y = acc[2 * m] + acc[2 * m + 1];
          a.y_pairs[(size_t)(pos0 + p) * H + r16 + col] = y;
          float* sa = &s_acc[(wave * T + tk[m]) * RW + (r16 - row0) + col];
          *sa = fmaf(wt[m], y, *sa);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = tid + 64 * kDnWaves * m;
    if (i < T * RW) {
      const int t = i / RW, r = i % RW;
      float v = ys[m];   // y_shared (0 without a shared expert)
      for (int w = 0; w < kDnWaves; ++w) v += s_acc[(w * T + t) * RW + r];
      v += rs[m];
      const size_t o = (size_t)t * H + row0 + r;
      a.out[o] = v;
      if (a.out_bf16) a.out_bf16[o] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ============================================================================ MXFP4, small T
// Routed experts in MXFP4 (E2M1 weights with UE8M0 group-32 scales) take FP8 E4M3
// activations with group-32 scales ("Hy4-preview-SF-WFP4AFP8", Quant Diff table): x is
// quantised once (extra K1 workgroups), h in the gate/up epilogue (a workgroup owns 32
// consecutive h-columns, one group), and both projections run on the scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4: A = E4M3 activations from LDS (row = token or pair
// slot), B = E2M1 weight codes straight from memory (column = weight row), one scale byte
// per lane and operand.  Operand layout (as in the MXFP4 prefill GEMMs): lane l serves row /
// column l % 16; an E2M1 lane holds K = 32g .. 32g+31 of the 128-wide step (16 bytes), an
// E4M3 lane K = 16g .. 16g+15 and 64+16g .. 64+16g+15, and each lane's scale is that of K
// block g (K = 32g .. 32g+31) of its row.  The routing, the shared expert and the combine
// are the STQ1_0 path's.

// Stream of one MXFP4 16-row tile over NS K steps of 128, row-major (codes [rows][K/2],
// scales [rows][K/32]) or tiled (per tile and step a 1 KiB code block in lane order and a
// 64-byte scale block, 4 bytes per row).  RD steps of code words and scale words in flight.
template <int NS, bool TILED, int RD = kRing>
struct MxStream {
  static constexpr int R = NS < RD ? NS : RD;
  static constexpr int K = 128 * NS;
  uint4 q[R];
  uint32_t sw[R];
  rsrc_t rc, rs;
  uint32_t co, so;

  __device__ __forceinline__ void load(int j, int slot) {
    // tiled: each step is whole lines read once (non-temporal); row-major rows are read
    // half a line per step
    q[slot] = TILED ? bload16_nt(rc, co, 1024 * j) : bload16(rc, co, 64 * j);
    sw[slot] = __builtin_amdgcn_raw_buffer_load_b32(rs, so, TILED ? 64 * j : 4 * j, 0);
  }
  // codes / scales: one matrix of `rows` rows; trow: the tile's first row (a multiple of 16)
  __device__ __forceinline__ void issue(const uint8_t* codes, const uint8_t* scales, uint32_t rows,
                                        uint32_t trow) {
    const int lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
    rc = make_rsrc(codes, rows * (K / 2));
    rs = make_rsrc(scales, rows * (K / 32));
    co = TILED ? trow * (K / 2) + 16 * lane : (trow + c16) * (K / 2) + 16 * g;
    so = TILED ? trow * (K / 32) + 4 * c16 : (trow + c16) * (K / 32);
#pragma unroll
    for (int j = 0; j < R; ++j) load(j, j);
  }
  // sum over K of this lane's A row (E4M3 codes a_q, UE8M0 scales a_s, in LDS) times the tile;
  // lanes with a_on false read nothing and feed zero codes (their D rows are unused)
  __device__ __forceinline__ f32x4_t run_lds(const uint8_t* a_q, const uint8_t* a_s, bool a_on = true) {
    const int g = (threadIdx.x & 63) >> 4;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint4 v0 = {0u, 0u, 0u, 0u}, v1 = v0;
    int asc = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const uint4 w = q[j % R];
      const int bsc = (sw[j % R] >> (8 * g)) & 0xFF;
      if (j + R < NS) load(j + R, j % R);
      if (a_on) {
        v0 = *reinterpret_cast<const uint4*>(a_q + 128 * j + 16 * g);
        v1 = *reinterpret_cast<const uint4*>(a_q + 128 * j + 64 + 16 * g);
        asc = a_s[4 * j + g];
      }
      const i32x8_t aop = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                           (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      const i32x8_t bop = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc, 0 /*A: E4M3*/,
                                                             4 /*B: E2M1*/, 0, asc, 0, bsc);
    }
    return acc;
  }
};

// x -> E4M3 with group-32 scales, 8 elements (index i of T H / 8) per lane; the four lanes of
// a group meet by shuffles (T H / 8 is a multiple of 64, so waves past the end are whole).
template <int HB>
__device__ __forceinline__ void quant_x8(const DecodeArgs& a, int i) {
  constexpr int H = HB * 256;
  if (i >= a.T * H / 8) return;
  const uint4 v = reinterpret_cast<const uint4*>(a.x)[i];
  const uint32_t bits[8] = {v.x << 16, v.x & 0xFFFF0000u, v.y << 16, v.y & 0xFFFF0000u,
                            v.z << 16, v.z & 0xFFFF0000u, v.w << 16, v.w & 0xFFFF0000u};
  uint32_t codes[2];
  const uint32_t sc = moe_mx_quant8(bits, codes);
  reinterpret_cast<uint2*>(a.xq)[i] = make_uint2(codes[0], codes[1]);
  if ((i & 3) == 0) a.xq[(size_t)a.T * H + i / 4] = (uint8_t)sc;
}

// K1 for MXFP4: the router partials, and in the workgroups past them x -> E4M3 with group-32
// scales, 8 elements per lane.
template <int HB, int IB, int XR>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4))) void k1s_router_mx(DecodeArgs a) {
  constexpr int H = HB * 256;
  extern __shared__ __align__(16) uint16_t s_x[];   // shared workgroups: XR bf16 x rows
  __shared__ __align__(16) float s_red[kNW][4][64];
  const int b = blockIdx.x;
  if (b < a.n_router_wg) {
    router_unit<HB>(a, b, s_red);
    return;
  }
  if (b >= a.n_router_wg + a.n_xq_wg) {
    shared_gateup_valu<HB, IB, XR, kWG>(a, b - a.n_router_wg - a.n_xq_wg, s_x);
    return;
  }
  quant_x8<HB>(a, (b - a.n_router_wg) * kWG + (int)threadIdx.x);
}

// Routed gate/up of one work item (unit, 32 rows of I): wave = (16-row tile, gate|up); the
// four waves meet in LDS, then threads (slot, column) form h = SiLU(gate) * up for the
// item's 32 h-columns and quantise each slot's 32 values as one MX group.
template <int HB, int IB, bool TILED>
__device__ __forceinline__ void routed_gateup_mx(const DecodeArgs& a, int wi, const uint8_t* s_xq,
                                                 float (*s_red)[2][4][64], const SmallRoute& R) {
  constexpr int H = HB * 256, I = IB * 256, NTP = I / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int un_i = wi / NTP, tp = wi % NTP;
  const int4 un = R.ut[un_i];
  const int e = un.x, pos0 = un.y, ntok = un.z;
  const int mat = wave & 1, tl = wave >> 1;
  const int row0 = (2 * tp + tl) * 16;
  const size_t eb = (size_t)I * (H / 2), es = (size_t)I * (H / 32);
  MxStream<H / 128, TILED> st;
  st.issue((mat ? a.uc : a.gc) + e * eb,
           reinterpret_cast<const uint8_t*>(mat ? a.us : a.gs) + e * es, I, row0);
  const int tok = R.utok[pos0 + (col < ntok ? col : ntok - 1)];
  const f32x4_t acc = st.run_lds(s_xq + (size_t)tok * H, s_xq + (size_t)a.T * H + tok * (H / 32));
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[tl][mat][i][lane] = acc[i];
  __syncthreads();
  if (threadIdx.x < 128) {
    // thread (slot, c): h-column 32 tp + c of token slot `slot`; D(4g + i, r) of tile t2 is
    // register i of lane 16 g + r
    const int slot = threadIdx.x >> 5, c = threadIdx.x & 31;
    const int t2 = c >> 4, L = 16 * (slot >> 2) + (c & 15), i = slot & 3;
    const float h = silu_mul(s_red[t2][0][i][L], s_red[t2][1][i][L]);
    uint32_t am = __float_as_uint(h) & 0x7FFFFFFFu;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, o, 64));
    if (slot < ntok) {
      const size_t pos = pos0 + slot;
      uint32_t code = 0, sc = 0;
      if (am != 0) {
        const int X = moe_mx_exp(am);
        code = moe_e4m3_code(h, X);
        sc = (uint32_t)(X + 127);
      }
      a.hq[pos * I + 32 * tp + c] = (uint8_t)code;
      if (c == 0) a.hq[(size_t)a.T * a.k * I + pos * (I / 32) + tp] = (uint8_t)sc;
    }
  }
  __syncthreads();   // s_red is reused by the next work item
}

template <int HB, int IB, int XR, bool TILED>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4))) void k2s_gateup_mx(DecodeArgs a) {
  constexpr int H = HB * 256, I = IB * 256;
  extern __shared__ __align__(16) uint16_t s_x[];   // shared-down workgroups: the shared h;
                                                    // routed: E4M3 x rows, then their scales
  __shared__ __align__(16) float s_red[2][2][4][64];
  __shared__ SmallRoute s_rt;
  const int b = blockIdx.x;
  const int T = a.T;
  if (b >= a.n_gu_wg) {
    shared_down_small<HB, IB, XR>(a, b - a.n_gu_wg, s_x);
    return;
  }
  uint8_t* s_xq = reinterpret_cast<uint8_t*>(s_x);
  {
    // the x codes and scales (one linear run) and the router partials are loaded in one
    // branch-free stretch: pieces past the end reload and rewrite piece 0
    constexpr int PER = (XR * (H + H / 32) / 16 + kWG - 1) / kWG;
    const int n16 = T * (H + H / 32) / 16;
    const uint4* src = reinterpret_cast<const uint4*>(a.xq);
    uint4 v[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = threadIdx.x + kWG * m;
      v[m] = src[i < n16 ? i : 0];
    }
    TopkIn in;
    topk_load(a, min((int)(threadIdx.x >> 6), T - 1), in);
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int i = threadIdx.x + kWG * m;
      reinterpret_cast<uint4*>(s_xq)[i < n16 ? i : 0] = v[m];
    }
    const TopkSum ls = topk_sums(a, in);
    small_route_topk(a, s_rt, ls, b == 0);
    small_route_units(a, s_rt, b == 0);   // starts and ends with a barrier: s_xq is complete
    const int n_items = s_rt.n_units * (I / 32);
    for (int wi = b; wi < n_items; wi += a.n_gu_wg)
      routed_gateup_mx<HB, IB, TILED>(a, wi, s_xq, s_red, s_rt);
  }
}

// Down projections and combine for MXFP4 routed experts: as k3_down_combine with every
// pair's E4M3 h codes and scales staged in LDS; an entry's pairs are A rows 0 .. nq - 1.
template <int HB, int IB, bool TILED, bool YSH = false>
__global__ __launch_bounds__(64 * kDnWaves) void k3_down_combine_mx(DecodeArgs a) {
  constexpr int H = HB * 256, I = IB * 256;
  constexpr int kStage = 10;                 // uint4 per thread of staged h
  extern __shared__ __align__(16) float s_dyn[];  // [kDnWaves][T][16] sums, then h codes + scales
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, P = T * a.k;
  const int row0 = blockIdx.x * 16;
  const int col = lane & 15, g = lane >> 4;
  float* s_acc = s_dyn;
  uint8_t* s_h = reinterpret_cast<uint8_t*>(s_dyn + kDnWaves * T * 16);
  const rsrc_t rres = make_rsrc(a.residual, a.residual ? (uint32_t)T * H * 4 : 0u);
  const rsrc_t rysh = make_rsrc(a.y_shared, YSH && a.y_shared ? (uint32_t)T * H * 4 : 0u);
  float rs[2], ys[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = tid + 64 * kDnWaves * m;
    const uint32_t o = i < T * 16 ? 4u * ((uint32_t)(i >> 4) * H + row0 + (i & 15)) : kOOB;
    rs[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rres, o, 0, 0));
    ys[m] = YSH ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rysh, o, 0, 0)) : 0.f;
  }
  // staged h: P I code bytes then P I / 32 scale bytes, one linear copy (branch-free, as in
  // k3_down_combine); the last piece may run up to 15 bytes past the scales (inside the h
  // region of the workspace)
  const int n_all = (P * (I + I / 32) + 15) / 16;
  uint4 hv[kStage];
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.hq);
#pragma unroll
    for (int m = 0; m < kStage; ++m) {
      const int i = tid + 64 * kDnWaves * m;
      hv[m] = src[i < n_all ? i : 0];
    }
  }
  for (int i = tid; i < kDnWaves * T * 16; i += 64 * kDnWaves) s_acc[i] = 0.f;
#pragma unroll
  for (int m = 0; m < kStage; ++m) {
    int i = tid + 64 * kDnWaves * m;
    i = i < n_all ? i : 0;
    reinterpret_cast<uint4*>(s_h)[i] = hv[m];
  }
  __builtin_amdgcn_sched_barrier(0);
  SharedDown<HB, IB, 2, true> sdn;
  if constexpr (!YSH) sdn.issue(a, row0);
  const int n_ent = a.wl[2];
  const size_t eb = (size_t)H * (I / 2), es = (size_t)H * (I / 32);
  const uint8_t* dsc = reinterpret_cast<const uint8_t*>(a.ds);
  MxStream<I / 128, TILED> st;
  int hu = wave;
  int4 hent = a.hl[wave < a.max_half ? wave : a.max_half - 1];
  {
    const int e0 = min(max(hent.x, 0), a.E - 1);
    st.issue(a.dc + e0 * eb, dsc + e0 * es, H, row0);
  }
  lds_barrier();
  if (!YSH && a.sd) sdn.run(a, row0, a.hs, s_acc);
  for (; hu < n_ent; hu += kDnWaves) {
    if (hu != wave) {
      hent = a.hl[hu];
      st.issue(a.dc + hent.x * eb, dsc + hent.x * es, H, row0);
    }
    const int pos0 = hent.y, nq = hent.z;
    const int pr = pos0 + (col < nq ? col : 0);
    const f32x4_t acc = st.run_lds(s_h + (size_t)pr * I, s_h + (size_t)P * I + pr * (I / 32));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = 4 * g + i;
      if (p < nq) {
        const float y = acc[i];
        a.y_pairs[(size_t)(pos0 + p) * H + row0 + col] = y;
        const int tk = a.utok[hent.w + p];
        float* sa = &s_acc[(wave * T + tk) * 16 + col];
        *sa = fmaf(a.uw[hent.w + p], y, *sa);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = tid + 64 * kDnWaves * m;
    if (i < T * 16) {
      const int t = i >> 4, r = i & 15;
      float v = ys[m];   // y_shared (0 without a shared expert)
      for (int w = 0; w < kDnWaves; ++w) v += s_acc[(w * T + t) * 16 + r];
      v += rs[m];
      const size_t o = (size_t)t * H + row0 + r;
      a.out[o] = v;
      if (a.out_bf16) a.out_bf16[o] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------------------- MXFP4, large T
// Beyond kXT tokens with MXFP4 routed experts.  A unit's E4M3 x rows (<= 16; 6.2 KB each at
// Hy4 shape) fit the LDS together, so the gate/up items are (unit, 64 rows of I): 8 waves =
// 4 row tiles x (gate, up), every expert's gate/up weights read once per unit (no half-units).
// The down items are (unit, 128 rows of H) on the unit's staged E4M3 h; the shared expert's
// down items and the combine are the STQ1_0 path's.
constexpr int kMxGuRows = 64;
constexpr int kMxSharedItemWeight = 4;   // a bf16 shared down item against an MXFP4 one

// E4M3 x rows of a unit in LDS: row s (pair s, token toks[s]) at byte s XR (XR = H + 16: the
// 16 lanes of one operand read start in different banks), its scales at 16 XR + s SR (SR =
// H / 32 + 16).  Rows past n read zeros; every load is issued before the first write.
template <int HB>
__device__ __forceinline__ void stage_xq_large(const DecodeArgs& a, const int* toks, int n, uint8_t* s_x) {
  constexpr int H = HB * 256, XR = H + 16, SR = H / 32 + 16;
  constexpr int PC = H / 16, PS = H / 32 / 16;   // 16-byte pieces of a code row, of a scale row
  constexpr int NP = 16 * (PC + PS), PER = (NP + kLW - 1) / kLW;
  const int tid = threadIdx.x;
  const rsrc_t rx = make_rsrc(a.xq, (uint32_t)a.T * (H + H / 32));
  uint4 v[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = tid + kLW * m;
    const bool code = idx < 16 * PC;
    const int r = code ? idx / PC : (idx - 16 * PC) / PS;
    const int pc = code ? idx % PC : (idx - 16 * PC) % PS;
    const bool ok = idx < NP && r < n;
    const uint32_t tok = ok ? (uint32_t)toks[r] : 0u;
    const uint32_t o = code ? tok * H + 16u * pc : (uint32_t)a.T * H + tok * (H / 32) + 16u * pc;
    v[m] = bload16(rx, ok ? o : kOOB);
  }
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = tid + kLW * m;
    if (idx < NP) {
      const bool code = idx < 16 * PC;
      const int r = code ? idx / PC : (idx - 16 * PC) / PS;
      const int pc = code ? idx % PC : (idx - 16 * PC) % PS;
      *reinterpret_cast<uint4*>(s_x + (code ? r * XR : 16 * XR + r * SR) + 16 * pc) = v[m];
    }
  }
}

// One gate/up item: unit (expert e, first sorted position pos0, npairs) x rows 64 sl .. +63
// of I.  Wave w streams row tile w / 2 of gate (w even) or up (w odd) against the staged x
// rows; the waves meet in LDS, then threads (slot, column) form h = SiLU(gate) * up for the
// item's 64 h-columns and quantise each slot's two 32-column groups.
template <int HB, int IB, bool TILED>
__device__ __forceinline__ void routed_gateup_mx_large(const DecodeArgs& a, int e, int pos0, int npairs, int sl,
                                                       const uint8_t* s_x, float (*s_red)[2][4][64]) {
  constexpr int H = HB * 256, I = IB * 256, XR = H + 16, SR = H / 32 + 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15;
  const int tl = wave >> 1, mat = wave & 1;
  const size_t eb = (size_t)I * (H / 2), es = (size_t)I * (H / 32);
  MxStream<H / 128, TILED> st;
  st.issue((mat ? a.uc : a.gc) + e * eb, reinterpret_cast<const uint8_t*>(mat ? a.us : a.gs) + e * es, I,
           kMxGuRows * sl + 16 * tl);
  const f32x4_t acc = st.run_lds(s_x + col * XR, s_x + 16 * XR + col * SR, col < npairs);
#pragma unroll
  for (int i = 0; i < 4; ++i) s_red[tl][mat][i][lane] = acc[i];
  __syncthreads();
  const int slot = threadIdx.x >> 5, c = threadIdx.x & 31;   // 16 slots x 32 columns
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    // h-column 64 sl + 32 q + c of token slot `slot`: D(4 g + i, r) of tile t2 is register i
    // of lane 16 g + r
    const int cc = 32 * q + c, t2 = cc >> 4, L = 16 * (slot >> 2) + (cc & 15), i = slot & 3;
    const float h = silu_mul(s_red[t2][0][i][L], s_red[t2][1][i][L]);
    uint32_t am = __float_as_uint(h) & 0x7FFFFFFFu;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, o, 64));
    if (slot < npairs) {
      const size_t pos = pos0 + slot;
      uint32_t code = 0, sc = 0;
      if (am != 0) {
        const int X = moe_mx_exp(am);
        code = moe_e4m3_code(h, X);
        sc = (uint32_t)(X + 127);
      }
      a.hq[pos * I + kMxGuRows * sl + cc] = (uint8_t)code;
      if (c == 0) a.hq[(size_t)a.T * a.k * I + pos * (I / 32) + 2 * sl + q] = (uint8_t)sc;
    }
  }
  __syncthreads();   // s_red is reused by the next item
}

// Large T, MXFP4, second kernel: persistent workgroups over contiguous ranges of the gate/up
// items; x is restaged when the unit changes.
template <int HB, int IB, bool TILED>
__global__ __launch_bounds__(kLW) void k2l_gateup_mx(DecodeArgs a) {
  constexpr int I = IB * 256, NS = I / kMxGuRows;
  static_assert(I % kMxGuRows == 0, "slices");
  __shared__ __align__(16) float s_red[4][2][4][64];
  extern __shared__ __align__(16) uint8_t s_xm[];   // 16 E4M3 x rows, then their scales
  int i0, i1;
  light_range(blockIdx.x, gridDim.x, a.wl[1] * NS, 0, 1, 1, i0, i1);
  int staged = -1;
  int4 un = make_int4(0, 0, 0, 0);
  for (int i = i0; i < i1; ++i) {
    const int u = i / NS;
    if (u != staged) {
      un = a.ut[u];
      __syncthreads();   // every wave is done with the previous rows
      stage_xq_large<HB>(a, a.utok + 16 * u, un.z, s_xm);
      __syncthreads();
      staged = u;
    }
    routed_gateup_mx_large<HB, IB, TILED>(a, un.x, un.y, un.z, i % NS, s_xm, s_red);
  }
}

// E4M3 h rows of a unit in LDS: pair s's codes at byte s HR (HR = I + 16), its scales at
// 16 HR + s HS (HS = I / 32 + 16); rows past n read zeros.
template <int IB>
__device__ __forceinline__ void stage_hq_large(const DecodeArgs& a, int first, int n, uint8_t* s_h) {
  constexpr int I = IB * 256, HR = I + 16, HS = I / 32 + 16;
  constexpr int PC = I / 16, PS = (I / 32 + 15) / 16;
  constexpr int NP = 16 * (PC + PS), PER = (NP + kLW - 1) / kLW;
  const int tid = threadIdx.x;
  const uint32_t P = (uint32_t)a.T * a.k;
  const rsrc_t rh = make_rsrc(a.hq, P * (I + I / 32));
  uint4 v[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = tid + kLW * m;
    const bool code = idx < 16 * PC;
    const int r = code ? idx / PC : (idx - 16 * PC) / PS;
    const int pc = code ? idx % PC : (idx - 16 * PC) % PS;
    const bool ok = idx < NP && r < n;
    const uint32_t pos = (uint32_t)(first + r);
    const uint32_t o = code ? pos * I + 16u * pc : P * I + pos * (I / 32) + 16u * pc;
    v[m] = bload16(rh, ok ? o : kOOB);
  }
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int idx = tid + kLW * m;
    if (idx < NP) {
      const bool code = idx < 16 * PC;
      const int r = code ? idx / PC : (idx - 16 * PC) / PS;
      const int pc = code ? idx % PC : (idx - 16 * PC) % PS;
      *reinterpret_cast<uint4*>(s_h + (code ? r * HR : 16 * HR + r * HS) + 16 * pc) = v[m];
    }
  }
}

// Large T, MXFP4, third kernel: as k3l_down (the shared expert's down items dealt round-robin
// first, then contiguous ranges of routed items) with MXFP4 routed down items: unit x rows
// slice * 128 + 16 w .. + 15 of H per wave, the next item's first K steps in flight while an
// item runs.
template <int HB, int IB, bool TILED>
__global__ __launch_bounds__(kLW) void k3l_down_mx(DecodeArgs a) {
  constexpr int H = HB * 256, I = IB * 256, NS = H / kSlice, HR = I + 16, HS = I / 32 + 16;
  static_assert(H % kSlice == 0, "slices");
  extern __shared__ __align__(16) uint8_t s_h[];   // shared tiles: 32 bf16 A rows; routed: E4M3 h
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, g = lane >> 4;
  const int T = a.T;
  const int n_sh = a.sd ? ((T + 15) / 16) * NS : 0;
  const int n_units = a.wl[1];
  int i0, i1;
  light_range(blockIdx.x, gridDim.x, n_units * NS, n_sh, 1, kMxSharedItemWeight, i0, i1);
  if (n_sh) {
    const rsrc_t rhs = make_rsrc(a.hs, (uint32_t)T * I * 4);
    int staged = -1;
    for (int si = blockIdx.x; si < n_sh; si += gridDim.x) {
      const int tt = si / NS;
      if (tt != staged) {
        __syncthreads();   // every wave is done with the previous tile
        stage_h_large<IB>(rhs, (uint32_t)T * I * 2, 16 * tt, min(16, T - 16 * tt), s_h);
        __syncthreads();
        staged = tt;
      }
      shared_down_item<HB, IB>(a, tt, si % NS, s_h);
    }
  }
  int i = i0;
  if (i >= i1) return;
  const size_t eb = (size_t)H * (I / 2), es = (size_t)H * (I / 32);
  const uint8_t* dsc = reinterpret_cast<const uint8_t*>(a.ds);
  int u = -1;
  int4 un = make_int4(0, 0, 0, 0);
  MxStream<I / 128, TILED> st;
  {
    const int4 u0 = a.ut[i / NS];
    st.issue(a.dc + u0.x * eb, dsc + u0.x * es, H, (i % NS) * kSlice + 16 * wave);
  }
  for (; i < i1; ++i) {
    if (i / NS != u) {   // the next unit of the range
      u = i / NS;
      un = a.ut[u];
      __syncthreads();
      stage_hq_large<IB>(a, un.y, un.z, s_h);
      __syncthreads();
    }
    MxStream<I / 128, TILED> nx = st;
    if (i + 1 < i1) {
      const int4 un2 = (i + 1) / NS == u ? un : a.ut[(i + 1) / NS];
      nx.issue(a.dc + un2.x * eb, dsc + un2.x * es, H, ((i + 1) % NS) * kSlice + 16 * wave);
    }
    const f32x4_t acc = st.run_lds(s_h + col * HR, s_h + 16 * HR + col * HS, col < un.z);
    const int r16 = (i % NS) * kSlice + 16 * wave;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = 4 * g + j;
      if (p < un.z) a.y_pairs[(size_t)(un.y + p) * H + r16 + col] = acc[j];
    }
    st = nx;
  }
}

// Compute units of the current device (persistent grids: one workgroup per CU).
int device_cus() {
  static int cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int HB, int IB, int XR, bool TILED>
hipError_t launch_small_mx(DecodeArgs& a, hipStream_t s) {
  constexpr int H = HB * 256, I = IB * 256;
  const int T = a.T;
  const int P = T * a.k;
  const int max_units = P < a.E ? P : a.E;
  const bool shared = a.sg != nullptr;
  a.n_router_wg = ((a.E + 15) / 16) * kRouterParts;
  a.n_xq_wg = (T * H / 8 + kWG - 1) / kWG;
  a.n_sgu_wg = shared ? I / kNW : 0;          // first kernel: one shared row (gate, up) per wave
  const int n_sdn_wg = shared ? H / 16 : 0;   // second kernel: 16 shared down rows per workgroup
  a.n_gu_wg = max_units * (I / 32);
  a.h_lds = 0;
  a.ysh_ready = shared ? 1 : 0;
  const size_t lds1 = shared ? (size_t)XR * H * 2 : 0;
  size_t lds2 = ((size_t)XR * (H + H / 32) + 15) / 16 * 16;   // E4M3 x rows and scales
  if (shared && (size_t)XR * I * 4 > lds2) lds2 = (size_t)XR * I * 4;   // or the shared h
  const size_t lds3 = (size_t)kDnWaves * T * 16 * 4 + ((size_t)P * (I + I / 32) + 15) / 16 * 16;
  if (((size_t)P * (I + I / 32) + 15) / 16 > (size_t)10 * 64 * kDnWaves) return hipErrorInvalidValue;
  const bool prof = moe_prof_on();
  if (prof) moe_prof_begin(MOE_PROF_DECODE_K1, s);
  hipLaunchKernelGGL((k1s_router_mx<HB, IB, XR>), dim3(a.n_router_wg + a.n_xq_wg + a.n_sgu_wg), dim3(kWG),
                     lds1, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K1, s); moe_prof_begin(MOE_PROF_DECODE_K2, s); }
  hipLaunchKernelGGL((k2s_gateup_mx<HB, IB, XR, TILED>), dim3(a.n_gu_wg + n_sdn_wg), dim3(kWG), lds2, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K2, s); moe_prof_begin(MOE_PROF_DECODE_K3, s); }
  hipLaunchKernelGGL((k3_down_combine_mx<HB, IB, TILED, true>), dim3(H / 16), dim3(64 * kDnWaves), lds3, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) moe_prof_end(MOE_PROF_DECODE_K3, s);
  return hipSuccess;
}

// Large T, MXFP4: (1) router + routing (tickets) beside the shared gate/up and x -> E4M3;
// (2) routed gate/up items (h -> E4M3); (3) shared and routed down items; (4) combine.
template <int HB, int IB, bool TILED>
hipError_t launch_large_mx(DecodeArgs& a, hipStream_t s) {
  constexpr int H = HB * 256, I = IB * 256;
  const int T = a.T;
  const int n_tt = (T + 15) / 16;
  a.n_router_wg = ((a.E + 15) / 16) * kRouterParts * n_tt;
  a.n_sgu_wg = a.sg ? I / 16 * (n_tt > 2 ? 2 : 1) : 0;   // two per row tile at four tiles
  a.n_xq_wg = (T * H / 8 + kWG - 1) / kWG;
  a.h_lds = 0;
  a.ysh_ready = 0;
  const int cus = device_cus();
  const size_t lds2 = (size_t)16 * (H + 16) + (size_t)16 * (H / 32 + 16);
  size_t lds3 = (size_t)16 * (I + 16) + (size_t)16 * (I / 32 + 16);
  if (a.sd && (size_t)32 * (2 * I + 16) > lds3) lds3 = (size_t)32 * (2 * I + 16);
  const bool prof = moe_prof_on();
  if (prof) moe_prof_begin(MOE_PROF_DECODE_K1, s);
  const dim3 g1(a.n_router_wg + a.n_sgu_wg + a.n_xq_wg);
  if (n_tt == 1) hipLaunchKernelGGL((k1_route<HB, IB, 1, kMaxT * 32, 8>), g1, dim3(kWG), 0, s, a);
  else if (n_tt == 2) hipLaunchKernelGGL((k1_route<HB, IB, 2, kMaxT * 32, 8>), g1, dim3(kWG), 0, s, a);
  else hipLaunchKernelGGL((k1_route<HB, IB, kMaxT / 16, kMaxT * 32, 8>), g1, dim3(kWG), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K1, s); moe_prof_begin(MOE_PROF_DECODE_K2, s); }
  hipLaunchKernelGGL((k2l_gateup_mx<HB, IB, TILED>), dim3(cus), dim3(kLW), lds2, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K2, s); moe_prof_begin(MOE_PROF_DECODE_K3, s); }
  hipLaunchKernelGGL((k3l_down_mx<HB, IB, TILED>), dim3(cus), dim3(kLW), lds3, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K3, s); moe_prof_begin(MOE_PROF_DECODE_K4, s); }
  MOE_HIP_TRY(moe_launch_combine(a.y_pairs, a.w, a.pair_pos, a.y_shared, a.residual, a.out, a.out_bf16,
                                 T, H, a.k, s));
  if (prof) moe_prof_end(MOE_PROF_DECODE_K4, s);
  return hipSuccess;
}

template <int HB, int IB, bool TILED>
hipError_t launch_shape_mx(DecodeArgs& a, hipStream_t s) {
  if (a.T == 1) return launch_small_mx<HB, IB, 1, TILED>(a, s);
  if (a.T == 2) return launch_small_mx<HB, IB, 2, TILED>(a, s);
  if (a.T <= kXT) return launch_small_mx<HB, IB, kXT, TILED>(a, s);
  return launch_large_mx<HB, IB, TILED>(a, s);
}

// Small T, split by what each piece waits for: (1) router partials + shared gate/up (x
// only); (2) per-workgroup routing + routed gate/up, beside the shared down (shared h only);
// (3) routed down + combine (+ y_shared, + residual).
template <int HB, int IB, int XR>
hipError_t launch_small(DecodeArgs& a, hipStream_t s) {
  constexpr int H = HB * 256, I = IB * 256;
  const int T = a.T;
  const int P = T * a.k;
  const int max_units = P < a.E ? P : a.E;   // T <= 16: an expert's pairs fit one unit
  const bool shared = a.sg != nullptr;
  a.n_router_wg = ((a.E + 15) / 16) * kRouterParts;
  a.n_sgu_wg = shared ? I / kNW : 0;          // first kernel: one shared row (gate, up) per wave
  const int n_sdn_wg = shared ? H / 16 : 0;   // second kernel: 16 shared down rows per workgroup
  a.n_gu_wg = max_units * (I / 32);           // a unit's 32 rows of I per workgroup
  a.ysh_ready = shared ? 1 : 0;
  const int hbytes = P * I * 4;               // routed h, bf16 hi + lo
  a.h_lds = a.h_lo_bytes == (uint32_t)P * I * 2 && hbytes <= 10 * 64 * kDnWaves * 16 ? 1 : 0;
  const size_t lds1 = shared ? (size_t)XR * H * 2 : 0;
  const size_t lds2 = (size_t)XR * H * 2;     // x rows, or the shared h (T I 4 <= XR H 2)
  // output rows per down workgroup (each stages all of h): 32 halves the staging but
  // leaves 192 workgroups for 256 CUs, and K3 measured 21.5 us against 20.4 us with 16
  constexpr int RW = 16;
  const size_t lds3 = (size_t)kDnWaves * T * RW * 4 + (size_t)hbytes + 64;
  const bool prof = moe_prof_on();
  if (prof) moe_prof_begin(MOE_PROF_DECODE_K1, s);
  hipLaunchKernelGGL((k1s_router<HB, IB, XR>), dim3(a.n_router_wg + a.n_sgu_wg), dim3(kWG), lds1, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K1, s); moe_prof_begin(MOE_PROF_DECODE_K2, s); }
  hipLaunchKernelGGL((k2s_gateup<HB, IB, XR>), dim3(a.n_gu_wg + n_sdn_wg), dim3(kWG), lds2, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K2, s); moe_prof_begin(MOE_PROF_DECODE_K3, s); }
  if (a.h_lds) {
    hipLaunchKernelGGL((k3_down_combine<HB, IB, RW>), dim3(H / RW), dim3(64 * kDnWaves), lds3, s, a);
    MOE_HIP_TRY(hipGetLastError());
    if (prof) moe_prof_end(MOE_PROF_DECODE_K3, s);
    return hipSuccess;
  }
  // h beyond the LDS (more than one token at Hy4 shape): the item-list down kernel (the
  // shared down already ran), then the combine
  hipLaunchKernelGGL((k3l_down<HB, IB>), dim3(device_cus()), dim3(kLW), (size_t)32 * (2 * I + 16), s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K3, s); moe_prof_begin(MOE_PROF_DECODE_K4, s); }
  MOE_HIP_TRY(moe_launch_combine(a.y_pairs, a.w, a.pair_pos, a.y_shared, a.residual, a.out, a.out_bf16,
                                 T, H, a.k, s));
  if (prof) moe_prof_end(MOE_PROF_DECODE_K4, s);
  return hipSuccess;
}

// Large T: (1) router + routing (tickets) beside the shared gate/up; (2) routed gate/up
// items; (3) shared and routed down items; (4) combine (+ y_shared, + residual).
template <int HB, int IB>
hipError_t launch_large(DecodeArgs& a, hipStream_t s) {
  constexpr int I = IB * 256;
  const int T = a.T;
  const int n_tt = (T + 15) / 16;
  a.n_router_wg = ((a.E + 15) / 16) * kRouterParts * n_tt;
  a.n_sgu_wg = a.sg ? I / 16 * (n_tt > 2 ? 2 : 1) : 0;   // two per row tile at four tiles
  a.h_lds = 0;
  a.ysh_ready = 0;
  const int cus = device_cus();
  const size_t lds2 = k2l_lds_x(HB);
  const size_t lds3 = (size_t)32 * (2 * I + 16);
  const bool prof = moe_prof_on();
  if (prof) moe_prof_begin(MOE_PROF_DECODE_K1, s);
  const dim3 g1(a.n_router_wg + a.n_sgu_wg);
  if (n_tt == 1) hipLaunchKernelGGL((k1_route<HB, IB, 1, kMaxT * 32, 8>), g1, dim3(kWG), 0, s, a);
  else if (n_tt == 2) hipLaunchKernelGGL((k1_route<HB, IB, 2, kMaxT * 32, 8>), g1, dim3(kWG), 0, s, a);
  else hipLaunchKernelGGL((k1_route<HB, IB, kMaxT / 16, kMaxT * 32, 8>), g1, dim3(kWG), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K1, s); moe_prof_begin(MOE_PROF_DECODE_K2, s); }
  hipLaunchKernelGGL((k2l_gateup<HB, IB>), dim3(cus), dim3(64 * k2l_waves(HB)), lds2, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K2, s); moe_prof_begin(MOE_PROF_DECODE_K3, s); }
  hipLaunchKernelGGL((k3l_down<HB, IB>), dim3(cus), dim3(kLW), lds3, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K3, s); moe_prof_begin(MOE_PROF_DECODE_K4, s); }
  MOE_HIP_TRY(moe_launch_combine(a.y_pairs, a.w, a.pair_pos, a.y_shared, a.residual, a.out, a.out_bf16,
                                 T, HB * 256, a.k, s));
  if (prof) moe_prof_end(MOE_PROF_DECODE_K4, s);
  return hipSuccess;
}

template <int HB, int IB>
hipError_t launch_shape(DecodeArgs& a, hipStream_t s) {
  if (a.T == 1) return launch_small<HB, IB, 1>(a, s);
  if (a.T == 2) return launch_small<HB, IB, 2>(a, s);
  if (a.T <= kXT) return launch_small<HB, IB, kXT>(a, s);
  return launch_large<HB, IB>(a, s);
}

}  // namespace

// ---------------------------------------------------------------------------- static scratch
// The workspace of moe_layer_decode_noalloc, for callers that cannot allocate: one array per
// device, held by the loaded library until the process ends.  Host code never uses the
// symbol's name as an address: moe_decode_static_scratch() looks up each device's own
// address once (hipGetSymbolAddress, that device current) and keeps it.
static __device__ __align__(256) uint8_t scratch[kDecodeStaticScratchBytes];

namespace {

// Zero the workspace header (the work-list words with the router ticket): a kernel, not
// hipMemsetAsync, so a captured call replays it as a kernel node.
__global__ __launch_bounds__(64) void clear_words_kernel(uint32_t* p) {
  if (threadIdx.x < 16) p[threadIdx.x] = 0u;   // work lists and the ticket counters
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

void* moe_decode_static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

hipError_t moe_clear_decode_header(void* ws, hipStream_t s) {
  hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(64), 0, s, static_cast<uint32_t*>(ws));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- host side
// Shapes with a compiled instantiation: (H, I) in units of 256.
bool moe_decode_shape_ok(int H, int I, int E) {
  if (E > kMaxE || H % 256 || I % 256) return false;
  const int hb = H / 256, ib = I / 256;
  return (hb == 2 && ib == 1) || (hb == 4 && ib == 2) || (hb == 8 && ib == 4) ||
         (hb == 16 && ib == 8) || (hb == 24 && ib == 8) || (hb == 32 && ib == 8);
}

// MXFP4 routed experts: up to kXT tokens every pair's E4M3 h (codes and scales) must fit the
// down kernel's LDS staging; beyond, up to kMaxT tokens, h is staged per unit.
bool moe_decode_mx_ok(int T, int I, int k) {
  const long P = (long)T * k;
  if (T > kXT) return T <= kMaxT;
  return (P * (I + I / 32) + 15) / 16 <= 10L * 64 * kDnWaves;
}

size_t moe_decode_ws_layout(int T, int H, int I, int E, int k, int has_shared, size_t* offs) {
  const size_t P = (size_t)T * k;
  const size_t pe = P < (size_t)E ? P : (size_t)E;
  const size_t max_units = pe + (P + 15) / 16;
  const size_t max_half = pe + (P + 3) / 4;     // entries of <= 8 (or <= 4) pairs
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t cur = 0;
  offs[0] = cur; cur = al(cur + 16 * sizeof(int32_t));                             // work lists + ticket
  offs[1] = cur; cur = al(cur + max_units * sizeof(int4));                          // unit table
  offs[2] = cur; cur = al(cur + max_units * 16 * sizeof(int32_t));                  // unit tokens
  offs[3] = cur; cur = al(cur + max_units * 16 * sizeof(float));                    // unit weights
  offs[4] = cur; cur = al(cur + max_half * sizeof(int4));                           // half-units
  offs[5] = cur; cur = al(cur + (size_t)kRouterParts * T * E * sizeof(float));     // router partials
  offs[6] = cur; cur = al(cur + P * I * 2);                                          // h hi
  offs[7] = cur; cur = al(cur + P * I * 2);                                          // h lo
  offs[8] = cur; cur = al(cur + (has_shared ? (size_t)T * I * 4 : 0));              // shared h hi, lo
  offs[9] = cur; cur = al(cur + (size_t)T * (H + H / 32));                          // MXFP4: E4M3 x
  offs[10] = cur;
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
  size_t offs[16];
  moe_decode_ws_layout(d->T, d->H, d->I, d->E, d->k, shared != nullptr, offs);
  uint8_t* b = static_cast<uint8_t*>(ws);
  a.wl = reinterpret_cast<int32_t*>(b + offs[0]);
  a.ctr = a.wl + 4;
  a.ut = reinterpret_cast<int4*>(b + offs[1]);
  a.utok = reinterpret_cast<int32_t*>(b + offs[2]);
  a.uw = reinterpret_cast<float*>(b + offs[3]);
  a.hl = reinterpret_cast<int4*>(b + offs[4]);
  {
    const int P = d->T * d->k;
    a.max_half = (P < d->E ? P : d->E) + (P + 7) / 8;
  }
  a.rpart = reinterpret_cast<float*>(b + offs[5]);
  a.h_hi = reinterpret_cast<uint16_t*>(b + offs[6]);
  a.h_lo_bytes = (uint32_t)(offs[7] - offs[6]);
  a.h_bytes = (uint32_t)(offs[7] - offs[6] + (size_t)d->T * d->k * d->I * 2);
  a.hs = reinterpret_cast<uint16_t*>(b + offs[8]);
  a.xq = b + offs[9];
  a.hq = b + offs[6];
  const int hb = d->H / 256, ib = d->I / 256;
  if (routed->fmt == MOE_W_MXFP4 || routed->fmt == MOE_W_MXFP4_TILED) {
    const bool tl = routed->fmt == MOE_W_MXFP4_TILED;
#define MOE_MX_SHAPE(HB_, IB_)                                                          \
    if (hb == HB_ && ib == IB_)                                                         \
      return tl ? launch_shape_mx<HB_, IB_, true>(a, s) : launch_shape_mx<HB_, IB_, false>(a, s);
    MOE_MX_SHAPE(2, 1) MOE_MX_SHAPE(4, 2) MOE_MX_SHAPE(8, 4) MOE_MX_SHAPE(16, 8)
    MOE_MX_SHAPE(24, 8) MOE_MX_SHAPE(32, 8)
#undef MOE_MX_SHAPE
    return hipErrorInvalidValue;
  }
  if (hb == 2 && ib == 1) return launch_shape<2, 1>(a, s);
  if (hb == 4 && ib == 2) return launch_shape<4, 2>(a, s);
  if (hb == 8 && ib == 4) return launch_shape<8, 4>(a, s);
  if (hb == 16 && ib == 8) return launch_shape<16, 8>(a, s);
  if (hb == 24 && ib == 8) return launch_shape<24, 8>(a, s);
  if (hb == 32 && ib == 8) return launch_shape<32, 8>(a, s);
  return hipErrorInvalidValue;
}
