// Fused decode-regime MoE layer: route -> permute -> expert FFN -> combine in three kernels.
//
// Same computation as the four separate entry points (router in BF16, top-k with
// renormalised softmax weights, stable permutation, SwiGLU experts on STQ1_0 weights,
// one bf16 shared expert, ungated combine), split by what each step waits for:
//   K1  routing only: router logits (bf16 MFMA; a workgroup sums four K chunks of 16
//       experts in LDS and writes one partial); the last router workgroup to finish (atomic
//       ticket, one release fence per workgroup) sums the partials in a fixed order, picks
//       the top-k, sorts the pairs by expert and writes the work lists: units of <= 16
//       pairs of one expert (with each pair's token and weight) and half-units of <= 8.
//       Nothing else runs beside it, so its short chain of dependent loads never queues
//       behind bulk weight traffic;
//   K2  every gate/up projection: routed (STQ1_0 decoded in registers, bf16 MFMA) and the
//       shared expert's, each followed by SiLU(gate) * up;
//   K3  every down projection and the combine, per 16-row slice of the output: the shared
//       expert's rows and each half-unit's rows, weighted into per-wave LDS sums, then
//       out = shared + sum over waves in a fixed order (+ residual).
// Every sum runs in a fixed order, so results do not depend on scheduling.  The ticket
// counter lives in the workspace: zero before the first call, left zero by every call.
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
// from the 8 code bytes and 16 high bits it loads.  Token slots past a unit's last pair
// read some valid row; their D rows are never used.
// The routed h is kept as bf16 hi + bf16 lo (h - hi); in the down projection a pair takes
// two adjacent A rows (hi, lo) of one MFMA, so ~16 bits of h cost no extra MFMA and the
// pair's result is the sum of two D rows.  The shared h is kept the same way and enters
// packed bf16 dot products.
// The kernels are instantiated per (H/256, I/256) so every loop over K has a fixed trip
// count and a wave's loads are issued without branches.  Up to kXT tokens per unit (and
// for the shared expert) activations come from LDS and the shared expert runs on the VALU
// (a plain bf16 GEMV: 75 MB of weights at Hy4 shape); beyond that activations are read
// from memory block by block and the shared expert uses the MFMA.
#include "moe_device.h"

#include <math.h>

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
  int h_lds;        // down kernel: all routed and shared h staged in LDS
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

// 32-entry table: 5-bit STQ1_0 group pattern -> its four weights in {-1, 0, +1} as bf16.
__device__ __forceinline__ void build_lut(uint2* lut) {
  const int t = threadIdx.x;
  if (t < 32) lut[t] = make_uint2(bf16_lane(t, 0) | (bf16_lane(t, 1) << 16),
                                  bf16_lane(t, 2) | (bf16_lane(t, 3) << 16));
}

// The 8 weight operands of one STQ1_0 block (8 code bytes + 16 high bits of this lane):
// all 16 table reads are issued before any is used.
__device__ __forceinline__ void stq_block_w(const uint2* lut, uint2 qs, uint32_t qh, bf16x8_t* wv) {
  uint2 l[16];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t byte = ((t < 4 ? qs.x : qs.y) >> (8 * (t & 3))) & 0xFFu;
    l[2 * t] = lut[(byte & 15u) | (((qh >> (2 * t)) & 1u) << 4)];
    l[2 * t + 1] = lut[(byte >> 4) | (((qh >> (2 * t + 1)) & 1u) << 4)];
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) wv[t] = as_bf16x8(make_uint4(l[2 * t].x, l[2 * t].y, l[2 * t + 1].x, l[2 * t + 1].y));
}

// The 4 weight operands of half h of one STQ1_0 block (code bytes 4h .. 4h+3 of this lane
// and their 8 high bits): 8 table reads, all issued before any is used.
__device__ __forceinline__ void stq_half_w(const uint2* lut, uint2 qs, uint32_t qh, int h, bf16x8_t* wv) {
  const uint32_t w4 = h ? qs.y : qs.x;
  const uint32_t hb = qh >> (8 * h);
  uint2 l[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t byte = (w4 >> (8 * t)) & 0xFFu;
    l[2 * t] = lut[(byte & 15u) | (((hb >> (2 * t)) & 1u) << 4)];
    l[2 * t + 1] = lut[(byte >> 4) | (((hb >> (2 * t + 1)) & 1u) << 4)];
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) wv[t] = as_bf16x8(make_uint4(l[2 * t].x, l[2 * t].y, l[2 * t + 1].x, l[2 * t + 1].y));
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
  // already applied), K stride 1.  Software-pipelined by half blocks: the table reads of
  // half h + 1 are in flight while the 4 MFMAs of half h run, and the two halves of a block
  // accumulate in separate registers (two 4-deep MFMA chains).
  __device__ __forceinline__ f32x4_t run_lds(const uint2* lut, const uint16_t* a_lds) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint2 qj;
    uint32_t qhj;
    float d;
    next(0, qj, qhj, d);
    bf16x8_t wn[4];
    stq_half_w(lut, qj, qhj, 0, wn);
    f32x4_t b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0;
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
      uint4 av[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) av[t] = *reinterpret_cast<const uint4*>(a_lds + 256 * j + 8 * (4 * h + t));
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

  // A operands from memory through rsrc ra at byte offset aoff (+ 2 K); each operand is
  // reloaded for the next block as soon as its MFMA has been issued.
  __device__ __forceinline__ f32x4_t run_mem(const uint2* lut, rsrc_t ra, uint32_t aoff) {
    uint4 av[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) av[t] = bload16(ra, aoff, 2 * (8 * t));
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      uint2 qj;
      uint32_t qhj;
      float d;
      next(j, qj, qhj, d);
      bf16x8_t wv[8];
      stq_block_w(lut, qj, qhj, wv);
      f32x4_t bacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        bacc = mfma16(as_bf16x8(av[t]), wv[t], bacc);
        if (j + 1 < NB) av[t] = bload16(ra, aoff, 2 * (256 * (j + 1) + 8 * t));
      }
      acc[0] = fmaf(d, bacc[0], acc[0]); acc[1] = fmaf(d, bacc[1], acc[1]);
      acc[2] = fmaf(d, bacc[2], acc[2]); acc[3] = fmaf(d, bacc[3], acc[3]);
      pin4(acc);
    }
    return acc;
  }
};

// The same stream with the code words staged through a per-wave LDS buffer.  A wave's 16
// weight rows are consecutive rows of one matrix, so chunk c (blocks CB c .. CB c + CB - 1
// of every row) is 16 runs of 40 CB contiguous bytes: fetched as 16-byte pieces (fully
// used cache lines, a quarter of the requests of per-lane 8- and 2-byte reads) two chunks
// ahead in registers, written to LDS when their turn comes, and read from there per block.
// LDS rows are padded so the 16 lanes reading one column group hit distinct banks.
template <int NB>
struct StqStreamL {
  static constexpr int CB = NB % 4 == 0 ? 4 : 2;           // blocks per chunk (NB even)
  static constexpr int NC = NB / CB;                       // chunks
  static constexpr int RUN = 40 * CB;                      // bytes of one row in a chunk
  static constexpr int PPR = RUN / 16;                     // 16-byte pieces per row run
  static constexpr int NL = (16 * PPR + 63) / 64;          // loads per lane per chunk
  static constexpr int CROW = CB == 4 ? 176 : 112;         // padded LDS bytes per row
  static constexpr int BYTES = 16 * CROW;                  // LDS bytes per wave
  static_assert(NB % 2 == 0, "whole chunks");
  uint4 v[2][NL];
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
    load_chunk(0, 0);
    if (NC > 1) load_chunk(1, 1);
    sc = load_scale_group<NB>(sp, 0);
    sc_next = sc;
    store_chunk(0);
    if (NC > 2) load_chunk(0, 2);
  }

  __device__ __forceinline__ void next(int j, uint2& qj, uint32_t& qhj, float& d) {
    if (j % 8 == 0) {
      if (j > 0) sc = sc_next;
      if (j + 8 < NB) sc_next = load_scale_group<NB>(sp, j / 8 + 1);
    }
    if (j % CB == 0 && j > 0) {
      const int c = j / CB;
      store_chunk(c & 1);
      if (c + 2 < NC) load_chunk(c & 1, c + 2);
    }
    const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
    const uint8_t* bp = buf + col * CROW + 40 * (j % CB);
    qj = *reinterpret_cast<const uint2*>(bp + 8 * g);
    qhj = *reinterpret_cast<const uint16_t*>(bp + 32 + 2 * g);
    d = scale_of(sc, j);
  }

  // as StqStream::run_lds
  __device__ __forceinline__ f32x4_t run_lds(const uint2* lut, const uint16_t* a_lds) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint2 qj;
    uint32_t qhj;
    float d;
    next(0, qj, qhj, d);
    bf16x8_t wn[4];
    stq_half_w(lut, qj, qhj, 0, wn);
    f32x4_t b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0;
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
      uint4 av[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) av[t] = *reinterpret_cast<const uint4*>(a_lds + 256 * j + 8 * (4 * h + t));
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
      if (e < a.E) a.rpart[((size_t)q * a.T + tok) * a.E + e] = v;
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
// finite or infinite value maps above 0) and its inverse.
__device__ __forceinline__ uint32_t fkey(float f) {
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

template <int P0>
struct FinalizeLds {
  int ids[3 * P0];           // [0, P) expert of each pair; [P0, P0 + P) pairs in sorted order;
                             // [2 P0, 2 P0 + P) weight bits of each pair (P <= P0)
  float v[kNW][32];
  int i[kNW][32];
  int cnt[kMaxE];
  int base[kMaxE];
  int ebase[kMaxE];          // first sorted position of each expert
  int ubase[kMaxE];          // first unit of each expert
  uint8_t wc[kNW][kMaxE];
  int wsum[kNW * 4];
};

// Routing of all tokens by the last router workgroup (4 waves): top-k per token, stable
// permutation of the pairs by expert (E <= 256: one expert per thread), work lists.
template <int P0, int QN>
__device__ __forceinline__ void route_finalize(const DecodeArgs& a, FinalizeLds<P0>& L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k, T = a.T, P = T * k;
  for (int t = wave; t < T; t += kNW) {
    TopkIn in;
    topk_load(a, t, in);
    wave_topk(a, t, topk_sums(a, in), L.v[wave], L.i[wave], L.ids, L.ids + 2 * P0, true);
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

template <int HB, int P0, int QN>
__global__ __launch_bounds__(kWG) void k1_route(DecodeArgs a) {
  __shared__ __align__(16) float s_red[kNW][4][64];
  __shared__ int s_last;
  __shared__ FinalizeLds<P0> s_fin;
  router_unit<HB>(a, blockIdx.x, s_red);
  if (threadIdx.x < 64) {
    __threadfence();     // wave 0 wrote this workgroup's partial: publish it device-wide
    if (threadIdx.x == 0) s_last = atomicAdd(&a.ctr[0], 1) == a.n_router_wg - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  route_finalize<P0, QN>(a, s_fin);
  if (threadIdx.x == 0) a.ctr[0] = 0;
}

// ---------------------------------------------------------------------------- small T
constexpr int kMaxPL = kXT * 32;   // pairs of a small-T layer (k <= 32)

// Up to kXT tokens the first kernel only computes the router partials: every routed gate/up
// workgroup then derives the routing itself (below), so no workgroup waits on another.
template <int HB>
__global__ __launch_bounds__(kWG) void k1s_router(DecodeArgs a) {
  __shared__ __align__(16) float s_red[kNW][4][64];
  router_unit<HB>(a, blockIdx.x, s_red);
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
// Routed gate/up: a workgroup takes one unit (expert, <= 16 pairs) and 32 rows of I; wave
// = (16-row tile, gate|up) over all of K; the gate and up waves of a tile meet in LDS and
// the gate wave writes h = SiLU(gate) * up as bf16 hi + lo.  Units of up to kXT tokens read
// their x rows from LDS.
template <int HB, int IB, int XR, bool MEM>
__device__ __forceinline__ void routed_gateup(const DecodeArgs& a, int wi, const uint2* s_lut, uint16_t* s_x,
                              float (*s_red)[2][4][64]) {
  constexpr int H = HB * 256, I = IB * 256, NTP = I / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int un_i = wi / NTP, tp = wi % NTP;
  const int4 un = a.ut[un_i];
  const int e = un.x, pos0 = un.y, ntok = un.z;
  const int mat = wave & 1, tl = wave >> 1;
  const int row0 = (2 * tp + tl) * 16;
  const size_t wrow = (size_t)e * I + row0 + col;
  const uint8_t* rp = (mat ? a.uc : a.gc) + wrow * HB * 40;
  const uint16_t* sp = (mat ? a.us : a.gs) + wrow * HB;
  const int* toks = a.utok + un_i * 16;
  f32x4_t acc;
  if (!MEM || ntok <= XR) {
    RowStage<H, kWG, XR> xs;
    xs.issue(ntok, [&](int r) { return a.x + (size_t)toks[r] * H; });
    StqStream<HB> st;
    st.issue(rp, sp);
    xs.commit(ntok, s_x);
    lds_barrier();
    acc = st.run_lds(s_lut, s_x + (col < ntok ? col : 0) * H + 64 * g);
  } else if constexpr (MEM) {
    const rsrc_t rx = make_rsrc(a.x, (uint32_t)a.T * H * 2);
    const uint32_t xo = col < ntok ? 2u * ((uint32_t)toks[col] * H + 64 * g) : kOOB;
    StqStream<HB> st;
    st.issue(rp, sp);
    acc = st.run_mem(s_lut, rx, xo);
  }
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
  __syncthreads();   // s_red and the x rows are reused by the next work item
}

// Shared gate/up for up to kXT tokens (x rows in LDS): wave = one row of I, gate and up,
// streamed in 16-byte chunks per lane (chunk c: K = 8 l + 512 c for lane l) with the next
// chunk of both matrices in flight while one is reduced.
template <int HB, int IB, int XR, int NT = kWG>
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

// Shared gate/up beyond kXT tokens: 16 rows x 16 tokens, the 4 waves split K.
template <int HB, int IB>
__device__ __forceinline__ void shared_gateup_mfma(const DecodeArgs& a, int sw, float (*s_red)[2][4][64]) {
  constexpr int H = HB * 256, I = IB * 256, n_rt = I / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rt = sw % n_rt, tt = sw / n_rt;
  const int row0 = rt * 16;
  const int col = lane & 15, g = lane >> 4;
  const int tok = tt * 16 + col;
  const bool t_ok = tok < a.T;
  const int b0 = wave * HB / kNW, b1 = (wave + 1) * HB / kNW;
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)a.T * H * 2);
  const uint32_t xo = t_ok ? 2u * (uint32_t)tok * H : kOOB;
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
      cx[t] = bload16(rx, xo, 2 * off);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      accg = mfma16(as_bf16x8(cg[t]), as_bf16x8(cx[t]), accg);
      accu = mfma16(as_bf16x8(cu[t]), as_bf16x8(cx[t]), accu);
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
      store_hilo(a.hs + (size_t)tok * I + row0 + 4 * g + i, (size_t)a.T * I, silu_mul(gs, us));
    }
  }
}

// Large T, second kernel: routed gate/up (units of up to kXT tokens stage their x rows)
// beside the shared expert's gate/up on the MFMA.
template <int HB, int IB>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4))) void k2_gateup(DecodeArgs a) {
  constexpr int XR = kXT;
  extern __shared__ __align__(16) uint16_t s_x[];   // x rows: XR x H bf16
  __shared__ uint2 s_lut[32];
  __shared__ __align__(16) float s_red[2][2][4][64];
  const int b = blockIdx.x;
  if (b >= a.n_gu_wg) {
    shared_gateup_mfma<HB, IB>(a, b - a.n_gu_wg, reinterpret_cast<float(*)[2][4][64]>(&s_red[0][0][0][0]));
    return;
  }
  build_lut(s_lut);
  __syncthreads();
  const int n_items = a.wl[1] * (IB * 256 / 32);
  for (int wi = b; wi < n_items; wi += a.n_gu_wg)
    routed_gateup<HB, IB, XR, true>(a, wi, s_lut, s_x, s_red);
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

// ============================================================================ K3
// Routed gate/up of one work item (unit, 32 rows of I) of a small-T layer, every token's x
// row already in LDS; as routed_gateup otherwise.
template <int HB, int IB>
__device__ __forceinline__ void routed_gateup_small(const DecodeArgs& a, int wi, const uint2* s_lut,
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
  const f32x4_t acc = st.run_lds(s_lut, s_x + tok * H + 64 * g);
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
  extern __shared__ __align__(16) uint16_t s_x[];   // XR x rows (bf16)
  __shared__ uint2 s_lut[32];
  __shared__ __align__(16) float s_red[2][2][4][64];
  __shared__ SmallRoute s_rt;
  __shared__ __align__(16) uint8_t s_cw[kNW * StqStreamL<HB>::BYTES];   // code staging
  const int b = blockIdx.x;
  const int T = a.T;
  if (b >= a.n_gu_wg) {
    shared_gateup_valu<HB, IB, XR, kWG>(a, b - a.n_gu_wg, s_x);
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

// Shared down beyond kXT tokens: 16 rows x 16-token tiles; wave w takes K blocks w, w + 8,
// .. (A = h hi and lo rows, B = weights); the waves' partials meet in LDS (s_red) in order,
// wave 0 writes y_shared and adds it into its own sums.
template <int HB, int IB>
__device__ __forceinline__ void shared_down_mfma(const DecodeArgs& a, int row0, float* s_acc, float* s_red) {
  constexpr int H = HB * 256, I = IB * 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int T = a.T;
  const rsrc_t rh = make_rsrc(a.hs, (uint32_t)T * I * 4);
  const uint32_t lo = 2u * (uint32_t)T * I;
  const uint16_t* rd = a.sd + (size_t)(row0 + col) * I;
  for (int tt = 0; tt * 16 < T; ++tt) {
    const int tok = tt * 16 + col;
    const uint32_t ho = tok < T ? 2u * (uint32_t)tok * I : kOOB;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int b = wave; b < IB; b += kDnWaves) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int off = 256 * b + 32 * t + 8 * g;
        const bf16x8_t wv = as_bf16x8(*reinterpret_cast<const uint4*>(rd + off));
        acc = mfma16(as_bf16x8(bload16(rh, ho, 2 * off)), wv, acc);
        acc = mfma16(as_bf16x8(bload16(rh, ho + lo, 2 * off)), wv, acc);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[(wave * 4 + i) * 64 + lane] = acc[i];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tt * 16 + 4 * g + i;
        if (t < T) {
          float v = 0.f;
          for (int w = 0; w < kDnWaves; ++w) v += s_red[(w * 4 + i) * 64 + lane];
          a.y_shared[(size_t)t * H + row0 + col] = v;
          s_acc[t * 16 + col] += v;
        }
      }
    }
    __syncthreads();
  }
}

// One 16-row slice of the output: the shared expert's down projection (SDN: MFMA over
// 16-token tiles, large T; otherwise 2 rows per wave on the VALU) and every half-unit
// (expert, <= 8 pairs) spread over the 8 waves, each wave adding its results into its own
// LDS sums; out = sum over waves in order (+ residual).  HLDS: all h (few tokens) is staged
// in LDS first: routed hi rows, routed lo rows, shared hi rows, shared lo rows.
// RW output rows per workgroup (every workgroup stages all of h); a routed entry is RW / 16
// work items, one per 16-row tile.
template <int HB, int IB, bool SDN, bool HLDS, int RW = 16>
__global__ __launch_bounds__(64 * kDnWaves) void k3_down_combine(DecodeArgs a) {
  static_assert(RW % 16 == 0 && (!SDN || RW == 16), "rows per workgroup");
  constexpr int NTL = RW / 16;
  constexpr int H = HB * 256, I = IB * 256;
  constexpr int kStage = 10;                 // uint4 per thread when h is staged
  constexpr int kLoPad = 32;                 // lo rows start 64 bytes past the hi rows' end so a
                                             // pair's hi and lo reads fall in different banks
  extern __shared__ __align__(16) float s_dyn[];  // [kDnWaves][T][16] sums, then staged h
                                                  // or the shared partials [kDnWaves][4][64]
  __shared__ uint2 s_lut[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, P = T * a.k;
  const int row0 = blockIdx.x * RW;
  const int col = lane & 15, g = lane >> 4;
  float* s_acc = s_dyn;
  uint16_t* s_h = reinterpret_cast<uint16_t*>(s_dyn + kDnWaves * T * RW);
  // residual of this slice (T * RW <= 1024 elements, two per thread), read up front
  const rsrc_t rres = make_rsrc(a.residual, a.residual ? (uint32_t)T * H * 4 : 0u);
  float rs[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = tid + 64 * kDnWaves * m;
    const uint32_t o = i < T * RW ? 4u * ((uint32_t)(i / RW) * H + row0 + (i % RW)) : kOOB;
    rs[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rres, o, 0, 0));
  }
  // staged h, 16-byte pieces: routed hi rows, routed lo rows, shared h
  const int n_r0 = P * I / 8, n_r1 = P * I / 8;
  const int n_all = n_r0 + n_r1 + T * I / 4;
  // h_lds is set only when the workspace holds routed hi, routed lo and shared h back to
  // back, so the staging is one linear copy.  Branch-free: every piece is written below, so
  // the compiler keeps all loads in flight together (a load inside a conditional write is
  // sunk into it and waited for one at a time).  Pieces past the end reload and rewrite
  // piece 0, the same value thread 0 writes there.
  uint4 hv[kStage];
  if constexpr (HLDS) {
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
  if constexpr (HLDS) {
#pragma unroll
    for (int m = 0; m < kStage; ++m) {
      int i = tid + 64 * kDnWaves * m;
      i = i < n_all ? i : 0;
      reinterpret_cast<uint4*>(s_h + (i < n_r0 ? 0 : kLoPad))[i] = hv[m];
    }
    // keep the weight loads below: hoisted above these writes, one wave's weight stream
    // queued ahead of another wave's staging loads in the CU's in-order memory queue
    __builtin_amdgcn_sched_barrier(0);
  }
  // the shared rows' first weight chunks
  SharedDown<HB, IB, RW / 8, true, RW> sdn;
  if constexpr (!SDN) sdn.issue(a, row0);
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
  if (a.sd) {
    if constexpr (SDN) shared_down_mfma<HB, IB>(a, row0, s_acc, s_dyn + kDnWaves * T * 16);
    else if constexpr (HLDS) sdn.run(a, row0, s_h + 2 * P * I + kLoPad, s_acc);
    else sdn.run(a, row0, a.hs, s_acc);
  }
  const rsrc_t rh = make_rsrc(a.h_hi, a.h_bytes);
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
      f32x4_t acc;
      if constexpr (HLDS) {
        const int pr = pos0 + (sp2 < nq ? sp2 : 0);
        acc = st.run_lds(s_lut, s_h + (col & 1) * (P * I + kLoPad) + pr * I + 64 * g);
      } else {
        const uint32_t ho = sp2 < nq ? (col & 1 ? a.h_lo_bytes : 0u) + 2u * ((uint32_t)(pos0 + sp2) * I + 64 * g) : kOOB;
        acc = st.run_mem(s_lut, rh, ho);
      }
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
      float v = 0.f;
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
  // sum over K of this lane's A row (E4M3 codes a_q, UE8M0 scales a_s, in LDS) times the tile
  __device__ __forceinline__ f32x4_t run_lds(const uint8_t* a_q, const uint8_t* a_s) {
    const int g = (threadIdx.x & 63) >> 4;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const uint4 w = q[j % R];
      const int bsc = (sw[j % R] >> (8 * g)) & 0xFF;
      if (j + R < NS) load(j + R, j % R);
      const uint4 v0 = *reinterpret_cast<const uint4*>(a_q + 128 * j + 16 * g);
      const uint4 v1 = *reinterpret_cast<const uint4*>(a_q + 128 * j + 64 + 16 * g);
      const int asc = a_s[4 * j + g];
      const i32x8_t aop = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                           (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      const i32x8_t bop = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc, 0 /*A: E4M3*/,
                                                             4 /*B: E2M1*/, 0, asc, 0, bsc);
    }
    return acc;
  }
};

// K1 for MXFP4: the router partials, and in the workgroups past them x -> E4M3 with group-32
// scales, 8 elements per lane (T H / 8 is a multiple of 64, so waves past the end are whole).
template <int HB>
__global__ __launch_bounds__(kWG) void k1s_router_mx(DecodeArgs a) {
  constexpr int H = HB * 256;
  __shared__ __align__(16) float s_red[kNW][4][64];
  if ((int)blockIdx.x < a.n_router_wg) {
    router_unit<HB>(a, blockIdx.x, s_red);
    return;
  }
  const int i = ((int)blockIdx.x - a.n_router_wg) * kWG + (int)threadIdx.x;
  if (i >= a.T * H / 8) return;
  const uint4 v = reinterpret_cast<const uint4*>(a.x)[i];
  const uint32_t bits[8] = {v.x << 16, v.x & 0xFFFF0000u, v.y << 16, v.y & 0xFFFF0000u,
                            v.z << 16, v.z & 0xFFFF0000u, v.w << 16, v.w & 0xFFFF0000u};
  uint32_t codes[2];
  const uint32_t sc = moe_mx_quant8(bits, codes);
  reinterpret_cast<uint2*>(a.xq)[i] = make_uint2(codes[0], codes[1]);
  if ((i & 3) == 0) a.xq[(size_t)a.T * H + i / 4] = (uint8_t)sc;
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
  extern __shared__ __align__(16) uint16_t s_x[];   // shared workgroups: XR bf16 x rows;
                                                    // routed: E4M3 x rows, then their scales
  __shared__ __align__(16) float s_red[2][2][4][64];
  __shared__ SmallRoute s_rt;
  const int b = blockIdx.x;
  const int T = a.T;
  if (b >= a.n_gu_wg) {
    shared_gateup_valu<HB, IB, XR, kWG>(a, b - a.n_gu_wg, s_x);
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
template <int HB, int IB, bool TILED>
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
  float rs[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = tid + 64 * kDnWaves * m;
    const uint32_t o = i < T * 16 ? 4u * ((uint32_t)(i >> 4) * H + row0 + (i & 15)) : kOOB;
    rs[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rres, o, 0, 0));
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
  sdn.issue(a, row0);
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
  if (a.sd) sdn.run(a, row0, a.hs, s_acc);
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
      float v = 0.f;
      for (int w = 0; w < kDnWaves; ++w) v += s_acc[(w * T + t) * 16 + r];
      v += rs[m];
      const size_t o = (size_t)t * H + row0 + r;
      a.out[o] = v;
      if (a.out_bf16) a.out_bf16[o] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

template <int HB, int IB, int XR, bool TILED>
hipError_t launch_small_mx(DecodeArgs& a, hipStream_t s) {
  constexpr int H = HB * 256, I = IB * 256;
  const int T = a.T;
  const int P = T * a.k;
  const int max_units = P < a.E ? P : a.E;
  const bool shared = a.sg != nullptr;
  a.n_router_wg = ((a.E + 15) / 16) * kRouterParts;
  const int n_xq_wg = (T * H / 8 + kWG - 1) / kWG;
  a.n_sgu_wg = shared ? I / kNW : 0;
  a.n_gu_wg = max_units * (I / 32);
  a.h_lds = 0;
  const size_t lds2 = (size_t)XR * H * 2;
  const size_t lds3 = (size_t)kDnWaves * T * 16 * 4 + ((size_t)P * (I + I / 32) + 15) / 16 * 16;
  if (((size_t)P * (I + I / 32) + 15) / 16 > (size_t)10 * 64 * kDnWaves) return hipErrorInvalidValue;
  const bool prof = moe_prof_on();
  if (prof) moe_prof_begin(MOE_PROF_DECODE_K1, s);
  hipLaunchKernelGGL((k1s_router_mx<HB>), dim3(a.n_router_wg + n_xq_wg), dim3(kWG), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K1, s); moe_prof_begin(MOE_PROF_DECODE_K2, s); }
  hipLaunchKernelGGL((k2s_gateup_mx<HB, IB, XR, TILED>), dim3(a.n_gu_wg + a.n_sgu_wg), dim3(kWG), lds2, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K2, s); moe_prof_begin(MOE_PROF_DECODE_K3, s); }
  hipLaunchKernelGGL((k3_down_combine_mx<HB, IB, TILED>), dim3(H / 16), dim3(64 * kDnWaves), lds3, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) moe_prof_end(MOE_PROF_DECODE_K3, s);
  return hipSuccess;
}

template <int HB, int IB, bool TILED>
hipError_t launch_shape_mx(DecodeArgs& a, hipStream_t s) {
  if (a.T == 1) return launch_small_mx<HB, IB, 1, TILED>(a, s);
  if (a.T == 2) return launch_small_mx<HB, IB, 2, TILED>(a, s);
  if (a.T <= kXT) return launch_small_mx<HB, IB, kXT, TILED>(a, s);
  return hipErrorInvalidValue;
}

// Small T: router + routing; routed + shared gate/up; routed + shared down + combine.
template <int HB, int IB, int XR>
hipError_t launch_small(DecodeArgs& a, hipStream_t s) {
  constexpr int H = HB * 256, I = IB * 256;
  const int T = a.T;
  const int P = T * a.k;
  const int max_units = P < a.E ? P : a.E;   // T <= 16: an expert's pairs fit one unit
  const bool shared = a.sg != nullptr;
  a.n_router_wg = ((a.E + 15) / 16) * kRouterParts;
  a.n_sgu_wg = shared ? I / kNW : 0;          // one shared row (gate and up) per wave
  a.n_gu_wg = max_units * (I / 32);           // a unit's 32 rows of I per workgroup
  const int hbytes = (P + T) * I * 4;
  // LDS staging of h copies routed hi, routed lo and shared h as one run
  const bool h_run = a.h_lo_bytes == (uint32_t)P * I * 2 &&
                     (!shared || a.hs == a.h_hi + (size_t)2 * P * I);
  a.h_lds = h_run && hbytes <= 10 * 64 * kDnWaves * 16 ? 1 : 0;
  const size_t lds2 = (size_t)XR * H * 2;
  // output rows per down workgroup (each stages all of h): 32 halves the staging but
  // leaves 192 workgroups for 256 CUs, and K3 measured 21.5 us against 20.4 us with 16
  constexpr int RW = 16;
  const size_t lds3 = (size_t)kDnWaves * T * RW * 4 + (a.h_lds ? (size_t)hbytes + 64 : 0);
  const bool prof = moe_prof_on();
  if (prof) moe_prof_begin(MOE_PROF_DECODE_K1, s);
  hipLaunchKernelGGL((k1s_router<HB>), dim3(a.n_router_wg), dim3(kWG), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K1, s); moe_prof_begin(MOE_PROF_DECODE_K2, s); }
  hipLaunchKernelGGL((k2s_gateup<HB, IB, XR>), dim3(a.n_gu_wg + a.n_sgu_wg), dim3(kWG), lds2, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K2, s); moe_prof_begin(MOE_PROF_DECODE_K3, s); }
  if (a.h_lds) hipLaunchKernelGGL((k3_down_combine<HB, IB, false, true, RW>), dim3(H / RW), dim3(64 * kDnWaves), lds3, s, a);
  else hipLaunchKernelGGL((k3_down_combine<HB, IB, false, false, RW>), dim3(H / RW), dim3(64 * kDnWaves), lds3, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) moe_prof_end(MOE_PROF_DECODE_K3, s);
  return hipSuccess;
}

// Large T: router + routing (ticket), routed + shared gate/up, all down + combine.
template <int HB, int IB>
hipError_t launch_large(DecodeArgs& a, hipStream_t s) {
  constexpr int H = HB * 256, I = IB * 256;
  const int T = a.T;
  const int n_tt = (T + 15) / 16;
  const int P = T * a.k;
  const int max_units = (P < a.E ? P : a.E) + (P + 15) / 16;
  a.n_router_wg = ((a.E + 15) / 16) * kRouterParts * n_tt;
  const bool shared = a.sg != nullptr;
  a.n_sgu_wg = shared ? (I / 16) * n_tt : 0;
  const int cap = 8192;
  const int gu = max_units * (I / 32);
  a.n_gu_wg = gu < cap ? gu : cap;
  a.h_lds = 0;
  const size_t lds2 = (size_t)kXT * H * 2;
  const size_t lds3 = (size_t)kDnWaves * T * 16 * 4 + (size_t)kDnWaves * 4 * 64 * 4;
  const bool prof = moe_prof_on();
  if (prof) moe_prof_begin(MOE_PROF_DECODE_K1, s);
  hipLaunchKernelGGL((k1_route<HB, kMaxT * 32, 8>), dim3(a.n_router_wg), dim3(kWG), 0, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K1, s); moe_prof_begin(MOE_PROF_DECODE_K2, s); }
  hipLaunchKernelGGL((k2_gateup<HB, IB>), dim3(a.n_gu_wg + a.n_sgu_wg), dim3(kWG), lds2, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) { moe_prof_end(MOE_PROF_DECODE_K2, s); moe_prof_begin(MOE_PROF_DECODE_K3, s); }
  hipLaunchKernelGGL((k3_down_combine<HB, IB, true, false>), dim3(H / 16), dim3(64 * kDnWaves), lds3, s, a);
  MOE_HIP_TRY(hipGetLastError());
  if (prof) moe_prof_end(MOE_PROF_DECODE_K3, s);
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

// ---------------------------------------------------------------------------- host side
// Shapes with a compiled instantiation: (H, I) in units of 256.
bool moe_decode_shape_ok(int H, int I, int E) {
  if (E > kMaxE || H % 256 || I % 256) return false;
  const int hb = H / 256, ib = I / 256;
  return (hb == 2 && ib == 1) || (hb == 4 && ib == 2) || (hb == 8 && ib == 4) ||
         (hb == 16 && ib == 8) || (hb == 24 && ib == 8) || (hb == 32 && ib == 8);
}

// MXFP4 routed experts: up to kXT tokens, every pair's E4M3 h (codes and scales) fits the
// down kernel's LDS staging.
bool moe_decode_mx_ok(int T, int I, int k) {
  const long P = (long)T * k;
  return T <= kXT && (P * (I + I / 32) + 15) / 16 <= 10L * 64 * kDnWaves;
}

size_t moe_decode_ws_layout(int T, int H, int I, int E, int k, int has_shared, size_t* offs) {
  const size_t P = (size_t)T * k;
  const size_t pe = P < (size_t)E ? P : (size_t)E;
  const size_t max_units = pe + (P + 15) / 16;
  const size_t max_half = pe + (P + 3) / 4;     // entries of <= 8 (or <= 4) pairs
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t cur = 0;
  offs[0] = cur; cur = al(cur + 8 * sizeof(int32_t));                              // work list + ticket
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
