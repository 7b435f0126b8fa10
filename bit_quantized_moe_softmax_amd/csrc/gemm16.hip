// Prefill expert FFN on the 16-bit MFMA: routed STQ1_0 experts and the bf16 shared expert
// as persistent grouped GEMMs (v_mfma_f32_16x16x32_f16 / _bf16), SiLU * up fused into the
// gate/up epilogue.
//
// STQ1_0 ("Hy4-preview-GGUF" (AngelSlim) section 3, The format; "Hy4-preview Flash-MoE
// STQ1_0", How the STQ1_0 packing works): blocks of 256 weights along K, 64 groups of four,
// each group one zero and three +-d, one fp16 d per block.  Every weight is 0 or +-d with d
// an fp16 number, so fp16 holds it exactly: the B operand is decoded in registers (a
// 32-entry LDS table turns a 5-bit group pattern into four fp16 +-1 / 0, a packed fp16
// multiply applies d) and one fp32 accumulator covers the whole K axis.
//
// Activations.  The fp16 MFMA needs fp16 activations: each activation row is scaled by a
// power of two 2^s that puts its largest magnitude in [2^14, 2^15) and rounded to fp16
// (rowscale_f16_kernel); the epilogue scales the row back by 2^-s.  For bf16 x this is exact
// (8 significant bits fit in 11) except for elements under 2^-38 of the row maximum.  The
// fp32 h of the down projection is split the same way into fp16 hi + lo (the rounding
// error of hi), taken as two K halves against the same weight columns: about 22
// significant bits, where one fp16 term (11 bits) leaves output errors near 1e-3 of the row
// RMS.  The bf16 shared expert runs on the bf16 MFMA: x as it is for gate/up, and h split
// into bf16 hi + lo for the down projection, again as two K halves (16 bits of h).  An
// MXFP8 (W8A8 group 32) shared expert runs on the bf16 MFMA too: its E4M3 weights times
// their UE8M0 scale are exact in bf16 (decoded in registers by the gfx950 scaled
// conversion), and so are its activations, which are MX-quantised (x along H, h along I)
// into the bf16 values of their E4M3 codes before the GEMMs.
//
// Work split (as in the first MXFP4 prefill GEMMs): the pairs of one expert are cut evenly into M
// blocks of at most 128 rows; a job is (M block, N tile of 256 weight rows: 128 gate + the
// 128 up rows of the same h-columns, or 256 output columns); jobs are numbered expert-major,
// then N tile, then M block, each XCD takes one contiguous range, and one workgroup per CU
// walks it (two for a down projection with 64 or more pairs per expert).  Four waves share
// the M block's activation rows, staged per K step (64) in LDS (double-buffered); each wave
// owns 64 weight rows whose codes it loads from HBM into registers, so weights never pass
// through LDS.
//
// K order.  The MFMA lane l serves row / column l % 16 and takes 8 consecutive K-slots from
// slot 8 (l / 16) of the 32-wide step.  The slot -> K map is ours, the same for A and B:
//   STQ1_0: lane group g owns groups 16g .. 16g+15 of each block (8 code bytes + 16 high
//     bits, loaded once per block); K step j (0..3) of block b and sub-step t (0, 1) take
//     groups 16g + 4j + 2t, +1, i.e. K = 256 b + 64 g + 16 j + 8 t + (0..7).
//   bf16 and MXFP8: K step j, sub-step t: K = 64 j + 32 t + 8 g + (0..7).
// The A rows are staged in the same order, so each lane reads its A operand as one
// 16-byte LDS word.
#include "moe_device.h"
#include "gemm_jobs.h"

#include <math.h>

namespace {

constexpr int kMT = kMB / 16;   // 16-row MFMA tiles per M block
constexpr int kNWave = 64;      // weight rows per wave
constexpr int kNTile = 4 * kNWave;
constexpr int kBK = 64;         // K (16-bit elements) per step
constexpr int kAStride = 144;   // bytes per A row in LDS (128 + 16 pad)
constexpr int kRingB = 2;       // bf16 B: K steps of loads in flight
// Workgroups per CU (WGS): with full M blocks the down GEMMs run two per CU in 256
// registers per lane (one wave's LDS reads and barrier overlap another's MFMAs: -20 % time
// at 4096 tokens); with blocks of a few rows they run one, with deeper load rings (two were
// 55 % slower at 64 tokens).  The gate/up GEMMs need more registers (the SiLU epilogue, two
// weight families) and always run one.

enum { kSTQ = 0, kBF16 = 1, kMX8 = 2 };

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

// Table of the 32 STQ1_0 group patterns: four fp16 weights of +-1 or 0 (pattern bits 3-4 =
// position of the zero; bits 0-2 = signs of the other three in order, set = negative).
__device__ __forceinline__ uint32_t f16_of(uint32_t p, int j) {
  const int z = p >> 3;
  if (j == z) return 0u;
  const int i = j < z ? j : j - 1;
  return ((p >> i) & 1) ? 0xBC00u : 0x3C00u;
}

__device__ __forceinline__ void build_lut16(uint2* lut, int t) {
  if (t < 32)
    lut[t] = make_uint2(f16_of(t, 0) | (f16_of(t, 1) << 16), f16_of(t, 2) | (f16_of(t, 3) << 16));
}

// Job tables of one "expert" owning every row (the shared expert): offsets {0, P}.
__device__ void single_job_table(int P, JobTable& t, int lane) {
  if (lane == 0) {
    t.off[0] = 0;
    t.off[1] = P;
    t.nb[0] = 0;
    t.nb[1] = blocks_of(P);
  }
}

__device__ __forceinline__ f32x4_t mfma16(const uint4 a, const uint4 b, f32x4_t c, bool f16) {
  if (f16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Raw STQ1_0 data of one block for one lane and tile: 8 code bytes (16 groups, group 2i in
// the low nibble of byte i), 16 high bits, and the row's fp16 scale d.
struct StqRaw {
  uint32_t qs0, qs1, qh, d;
};

template <int WF, bool GATEUP, int WGS>
__global__ __launch_bounds__(256, WGS) void g16_kernel(G16Args p) {
  // A: K steps of loads in flight (fewer registers at two workgroups per CU)
  constexpr int kRing = WGS == 1 ? 4 : 2;
  __shared__ __align__(16) uint8_t s_a[2][kMB * kAStride];
  __shared__ int s_arow[kMB];
  __shared__ int s_aexp[kMB];
  __shared__ uint2 s_lut[32];
  __shared__ JobTable s_jt;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int K = p.K, N = p.N, Ka = p.Ka;
  const int NT = GATEUP ? N / (kNTile / 2) : (N + kNTile - 1) / kNTile;
  const int E = p.offsets ? p.E : 1;
  constexpr bool F16 = WF == kSTQ;

  if (wave == 0) {
    if (p.offsets) build_job_table(p.offsets, p.E, s_jt, lane);
    else single_job_table(p.P, s_jt, lane);
  }
  if (F16 && wave == 1) build_lut16(s_lut, lane);
  __syncthreads();
  const long n_work = (long)s_jt.nb[E] * NT;
  const int x = blockIdx.x % kXcd, slot = blockIdx.x / kXcd, nslot = gridDim.x / kXcd;
  const long w_lo = n_work * x / kXcd, w_hi = n_work * (x + 1) / kXcd;
  const rsrc_t ra = make_rsrc(p.a, (uint32_t)((size_t)p.rows_a * Ka * 2));
  const int achunk = tid & 7;
  // per-lane part of the A column of this thread's staging chunk (bytes)
  const uint32_t acol = F16 ? 2 * (64 * (achunk >> 1) + 8 * (achunk & 1)) : 16 * achunk;
  const int g = lane >> 4, c16 = lane & 15;
  const int nblk = K / 256;   // STQ1_0 blocks per weight row
  const int kw = K / kBK;     // weight K steps (the A row may hold two K halves)

  for (long w = w_lo + slot; w < w_hi; w += nslot) {
  const Job jb = decode_job(s_jt, E, NT, w);
  const int nrows = jb.nrows;
  if (tid < kMB) {
    int src = -1;
    if (tid < nrows) {
      const int pos = jb.m0 + tid;
      src = (GATEUP && p.sorted_pair) ? p.sorted_pair[pos] / p.k : pos;
    }
    s_arow[tid] = src;
    s_aexp[tid] = (F16 && src >= 0) ? p.aexp[src] : 0;
  }
  __syncthreads();

  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int src = s_arow[(tid >> 3) + 32 * i];
    aoff[i] = src >= 0 ? (uint32_t)src * (uint32_t)(Ka * 2) + acol : kOOB;
  }
  // uniform byte offset of K step s within an A row
  auto astep = [](int s) { return F16 ? 2 * (256 * (s >> 2) + 16 * (s & 3)) : 128 * s; };

  // this wave's weight rows: 4 tiles of 16 (gate/up: gate, gate, up, up)
  const int col0 = GATEUP ? jb.ntile * (kNTile / 2) + 32 * wave : jb.ntile * kNTile + kNWave * wave;
  const bool wvalid = GATEUP || col0 < N;
  const uint32_t trow = (uint32_t)(wvalid ? col0 : 0);
  auto qrow = [](int q) { return GATEUP ? 16 * (q & 1) : 16 * q; };

  // weight resources of the job's expert
  const size_t mat = (size_t)N * K;
  rsrc_t rw0, rw1, rd0, rd1;
  if (F16) {
    const size_t eb = mat / 256 * 40, es = mat / 256 * 2;
    rw0 = make_rsrc(static_cast<const uint8_t*>(p.w0) + jb.e * eb, (uint32_t)eb);
    rd0 = make_rsrc(reinterpret_cast<const uint8_t*>(p.s0) + jb.e * es, (uint32_t)es);
    rw1 = GATEUP ? make_rsrc(static_cast<const uint8_t*>(p.w1) + jb.e * eb, (uint32_t)eb) : rw0;
    rd1 = GATEUP ? make_rsrc(reinterpret_cast<const uint8_t*>(p.s1) + jb.e * es, (uint32_t)es) : rd0;
  } else if (WF == kBF16) {
    rw0 = make_rsrc(p.w0, (uint32_t)(mat * 2));
    rw1 = GATEUP ? make_rsrc(p.w1, (uint32_t)(mat * 2)) : rw0;
    rd0 = rd1 = rw0;
  } else {   // MXFP8: E4M3 codes [N][K], UE8M0 scales [N][K/32] (one expert)
    rw0 = make_rsrc(p.w0, (uint32_t)mat);
    rw1 = GATEUP ? make_rsrc(p.w1, (uint32_t)mat) : rw0;
    rd0 = make_rsrc(p.s0, (uint32_t)(mat / 32));
    rd1 = GATEUP ? make_rsrc(p.s1, (uint32_t)(mat / 32)) : rd0;
  }
  // per-lane byte offsets of the lane's row in tile 0; tile q adds qrow(q) rows
  const uint32_t brow = trow + c16;
  const uint32_t rstride = F16 ? (uint32_t)nblk * 40 : WF == kBF16 ? (uint32_t)K * 2 : (uint32_t)K;
  const uint32_t boff = F16 ? brow * rstride + 8 * g : WF == kBF16 ? brow * rstride + 16 * g
                                                                    : brow * rstride + 8 * g;
  const uint32_t bsoff = brow * (uint32_t)(K / 32);   // MXFP8 scale bytes
  const uint32_t bhoff = brow * rstride + 32 + 2 * g;
  const uint32_t bdoff = brow * (uint32_t)nblk * 2;

  // ---- A: register ring, stored to LDS one step ahead
  uint4 ra_[kRing][4];
  auto load_a = [&](int sl, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra_[sl][i] = bload16(ra, aoff[i], astep(s));
  };
  auto store_a = [&](int sl, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&s_a[buf][((tid >> 3) + 32 * i) * kAStride + 16 * achunk]) = ra_[sl][i];
  };

  // ---- B, STQ1_0: raw block data, one block ahead
  StqRaw cur[4], nxt[4];
  auto load_stq = [&](StqRaw* r, int b) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool hi = GATEUP && q >= 2;
      // the tile's row offset is wave-uniform: it goes in the scalar offset
      const uint32_t ro = qrow(q) * rstride;
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(hi ? rw1 : rw0, boff, ro + 40 * b, 0);
      r[q].qs0 = v[0];
      r[q].qs1 = v[1];
      r[q].qh = __builtin_amdgcn_raw_buffer_load_b16(hi ? rw1 : rw0, bhoff, ro + 40 * b, 0);
      r[q].d = __builtin_amdgcn_raw_buffer_load_b16(hi ? rd1 : rd0, bdoff, qrow(q) * nblk * 2 + 2 * b, 0);
    }
  };
  // B operand of tile q at K step j (0..3 within the block), sub-step t
  auto stq_b = [&](const StqRaw& r, int j, int t) -> uint4 {
    const int bi = 2 * j + t;                                   // code byte
    const uint32_t byte = ((bi < 4 ? r.qs0 : r.qs1) >> (8 * (bi & 3))) & 0xFFu;
    const uint32_t p0 = (byte & 15u) | (((r.qh >> (2 * bi)) & 1u) << 4);
    const uint32_t p1 = (byte >> 4) | (((r.qh >> (2 * bi + 1)) & 1u) << 4);
    const uint2 l0 = s_lut[p0], l1 = s_lut[p1];
    const f16x2_t dd = __builtin_bit_cast(f16x2_t, r.d | (r.d << 16));
    uint4 o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, l0.x) * dd);
    o.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, l0.y) * dd);
    o.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, l1.x) * dd);
    o.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, l1.y) * dd);
    return o;
  };

  // ---- B, bf16 or MXFP8: register ring of kRingB steps, 2 sub-steps x 4 tiles per step
  // (MXFP8: 8 code bytes and the scale byte of their 32-block per lane)
  uint4 rb[kRingB][2][4];
  auto load_bf = [&](int sl, int s) {
    const int ws = s % kw;   // weight K step (the two K halves of hi / lo share the weights)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool hi = GATEUP && q >= 2;
        if constexpr (WF == kBF16) {
          rb[sl][t][q] = bload16(hi ? rw1 : rw0, boff, qrow(q) * rstride + 128 * ws + 64 * t);
        } else {
          const auto c = __builtin_amdgcn_raw_buffer_load_b64(hi ? rw1 : rw0, boff,
                                                              qrow(q) * rstride + 64 * ws + 32 * t, 0);
          const uint32_t sb = __builtin_amdgcn_raw_buffer_load_b8(hi ? rd1 : rd0, bsoff,
                                                                  qrow(q) * (K / 32) + 2 * ws + t, 0);
          rb[sl][t][q] = make_uint4(c[0], c[1], sb, 0u);
        }
      }
  };
  // B operand from the ring entry: bf16 as loaded, MXFP8 decoded (8 codes times the scale)
  auto bf_b = [&](const uint4& r) -> uint4 {
    if constexpr (WF == kBF16) {
      return r;
    } else {
      const float sc = moe_ue8m0_scale(r.z);
      return make_uint4(
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, sc, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.x, sc, true)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, sc, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.y, sc, true)));
    }
  };

  f32x4_t acc[kMT][4];
#pragma unroll
  for (int i = 0; i < kMT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const int mtiles = (nrows + 15) >> 4;

  // MFMAs of one K step from LDS buffer `buf`: B operands from `bq(t, q)`.  A full M block
  // runs straight-line code that issues four A fragment reads before their MFMAs; a partial
  // one skips the tiles past its last row, reading each fragment just before its MFMAs.  The
  // two are separate copies of the whole K loop (chosen once per job), so each keeps its own
  // register pressure.
  auto main_loop = [&](auto full_c) {
  constexpr bool full = decltype(full_c)::value;
  auto compute = [&](int buf, auto&& bq) {
    const uint8_t* sa = s_a[buf];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint4 bop[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) bop[q] = bq(t, q);
      const int chunk = F16 ? 2 * g + t : 4 * t + g;
      if constexpr (full) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint4 av[kMT / 2];
#pragma unroll
          for (int i = 0; i < kMT / 2; ++i)
            av[i] = *reinterpret_cast<const uint4*>(&sa[(16 * (4 * hh + i) + c16) * kAStride + 16 * chunk]);
#pragma unroll
          for (int i = 0; i < kMT / 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[4 * hh + i][q] = mfma16(av[i], bop[q], acc[4 * hh + i][q], F16);
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          if (mt < mtiles) {
            const uint4 av = *reinterpret_cast<const uint4*>(&sa[(16 * mt + c16) * kAStride + 16 * chunk]);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[mt][q] = mfma16(av, bop[q], acc[mt][q], F16);
          }
        }
      }
    }
  };

  const int nsteps = Ka / kBK;
  // Step s: issue A(s + kRing - 1), compute step s, issue the next B loads, store A(s + 1)
  // to the other LDS buffer.  Past the last step the loads repeat the last step's data,
  // which keeps the code branch-free and the wait counts exact.
  auto step = [&](int s, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    constexpr int AN = (SLOT + kRing - 1) % kRing, A1 = (SLOT + 1) % kRing;
    load_a(AN, min(s + kRing - 1, nsteps - 1));
    if constexpr (F16) {
      if (SLOT == 0) load_stq(nxt, ((s >> 2) + 1) % nblk);   // the lo half reuses the blocks
      if (wvalid) compute(s & 1, [&](int t, int q) { return stq_b(cur[q], SLOT, t); });
      if (SLOT == 3) {
#pragma unroll
        for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
      }
    } else {
      constexpr int BS = SLOT % kRingB;
      if (wvalid) compute(s & 1, [&](int t, int q) { return bf_b(rb[BS][t][q]); });
      load_bf(BS, min(s + kRingB, nsteps - 1));
    }
    if (s + 1 < nsteps) store_a(A1, (s + 1) & 1);
    lds_barrier();
  };

  // prologue
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i) load_a(i, min(i, nsteps - 1));
  if constexpr (F16) {
    load_stq(cur, 0);
  } else {
#pragma unroll
    for (int i = 0; i < kRingB; ++i) load_bf(i, min(i, nsteps - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
  store_a(0, 0);
  lds_barrier();
  // whole groups of 4 steps (one STQ1_0 block): the caller guarantees nsteps % 4 == 0
  for (int s = 0; s < nsteps; s += 4) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
    step(s + 2, std::integral_constant<int, 2>{});
    step(s + 3, std::integral_constant<int, 3>{});
  }
  };   // main_loop
  // the shared expert's blocks split all tokens evenly (full at 128-token multiples): its
  // kernels keep only the straight-line loop
  if constexpr (!F16) main_loop(std::true_type{});
  else if (mtiles == kMT) main_loop(std::true_type{});
  else main_loop(std::false_type{});

  if (wvalid) {
    // D element (4 (lane / 16) + i, lane % 16) of each 16x16 tile is acc[..][..][i]
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt >= mtiles) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 16 * mt + 4 * g + i;
        if (rl >= nrows) continue;
        const int se = -s_aexp[rl];
        float* orow = p.out + (size_t)(jb.m0 + rl) * N + col0 + c16;
        if (GATEUP) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float gv = ldexpf(acc[mt][q][i], se), uv = ldexpf(acc[mt][q + 2][i], se);
            orow[16 * q] = gv / (1.0f + expf(-gv)) * uv;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) orow[16 * q] = ldexpf(acc[mt][q][i], se);
        }
      }
    }
  }
  __syncthreads();   // s_arow, s_aexp and the LDS buffers are reused by the next job
  }   // jobs
}

// Rows of bf16 (in16) or fp32 (in32) -> fp16 rows * 2^s with s = 14 - floor(log2 max|row|)
// (s = 0 for an all-zero row), rounded to nearest even.  With `two` the output row has 2C
// entries: hi = fp16(v 2^s), then lo = fp16(v 2^s - hi).  One workgroup per row.
__global__ __launch_bounds__(256) void rowscale_f16_kernel(const uint16_t* __restrict__ in16,
                                                           const float* __restrict__ in32, int C,
                                                           int two, uint16_t* __restrict__ out,
                                                           int32_t* __restrict__ sexp) {
  __shared__ uint32_t s_max[4];
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x;
  auto bits = [&](int c) -> uint32_t {
    return in16 ? (uint32_t)in16[row * C + c] << 16 : __float_as_uint(in32[row * C + c]);
  };
  uint32_t m = 0;
  for (int c = tid; c < C; c += 256) m = max(m, bits(c) & 0x7FFFFFFFu);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((tid & 63) == 0) s_max[tid >> 6] = m;
  __syncthreads();
  m = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  int s = 0;
  if (m != 0) {
    const int e = (m >> 23) ? (int)(m >> 23) - 127 : (31 - __clz(m)) - 149;
    s = 14 - e;
  }
  const size_t oc = two ? 2 * (size_t)C : (size_t)C;
  for (int c = tid; c < C; c += 256) {
    const float v = ldexpf(__uint_as_float(bits(c)), s);
    const _Float16 hi = (_Float16)v;
    out[row * oc + c] = __builtin_bit_cast(uint16_t, hi);
    if (two) out[row * oc + C + c] = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)hi));
  }
  if (tid == 0) sexp[row] = s;
}

// fp32 rows [R][C] -> bf16 rows [R][2C]: hi = RNE bf16 of h, then lo = RNE bf16 of h - hi.
__global__ __launch_bounds__(256) void split_bf16_kernel(const float* __restrict__ h, long R, int C,
                                                         uint16_t* __restrict__ out) {
  const long n = R * C;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const long r = i / C;
    const int c = (int)(i - r * C);
    const float v = h[i];
    const uint32_t hi = f32_to_bf16_rne(v);
    const uint32_t lo = f32_to_bf16_rne(v - bf16_to_f32(hi));
    out[r * 2 * C + c] = (uint16_t)hi;
    out[r * 2 * C + C + c] = (uint16_t)lo;
  }
}

inline unsigned grid_for(const G16Args& a, int NT, int per_cu) {
  const int E = a.offsets ? a.E : 1;
  const long slots = (a.P < E ? a.P : E) + (a.P + kMB - 1) / kMB;
  const long work = slots * NT;
  const long most = kXcd * ((work + kXcd - 1) / kXcd);
  const long per = per_cu * kXcd * ((moe_cu_count() + kXcd - 1) / kXcd);
  return (unsigned)(most < per ? most : per);
}

template <int WF, bool GATEUP>
hipError_t launch(const G16Args& a, hipStream_t s) {
  // two workgroups per CU where the pairs fill most M blocks (64 or more per expert)
  const int E = a.offsets ? a.E : 1;
  const bool two = !GATEUP && (long)a.P >= 64L * E;
  if (GATEUP ? a.N % (kNTile / 2) : a.N % 16) return hipErrorInvalidValue;
  if (a.K % (WF == kSTQ ? 256 : 4 * kBK) || a.Ka % (4 * kBK)) return hipErrorInvalidValue;
  if ((size_t)a.rows_a * a.Ka * 2 >= 0x80000000ull) return hipErrorInvalidValue;
  if ((size_t)a.N * a.K * 2 >= 0x80000000ull) return hipErrorInvalidValue;
  if (a.P == 0) return hipSuccess;
  const int NT = GATEUP ? a.N / (kNTile / 2) : (a.N + kNTile - 1) / kNTile;
  if constexpr (!GATEUP) {
    if (two) {
      hipLaunchKernelGGL((g16_kernel<WF, false, 2>), dim3(grid_for(a, NT, 2)), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((g16_kernel<WF, GATEUP, 1>), dim3(grid_for(a, NT, 1)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t moe_launch_g16_stq_gateup(const G16Args& a, hipStream_t s) { return launch<kSTQ, true>(a, s); }
hipError_t moe_launch_g16_stq_down(const G16Args& a, hipStream_t s) { return launch<kSTQ, false>(a, s); }
hipError_t moe_launch_g16_bf16_gateup(const G16Args& a, hipStream_t s) { return launch<kBF16, true>(a, s); }
hipError_t moe_launch_g16_bf16_down(const G16Args& a, hipStream_t s) { return launch<kBF16, false>(a, s); }
hipError_t moe_launch_g16_mx8_gateup(const G16Args& a, hipStream_t s) { return launch<kMX8, true>(a, s); }
hipError_t moe_launch_g16_mx8_down(const G16Args& a, hipStream_t s) { return launch<kMX8, false>(a, s); }

hipError_t moe_launch_rowscale_f16(const uint16_t* in16, const float* in32, long rows, int C,
                                   int two, uint16_t* out, int32_t* sexp, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (rows > 0x7FFFFFFFL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rowscale_f16_kernel, dim3((unsigned)rows), dim3(256), 0, s, in16, in32, C, two,
                     out, sexp);
  return hipGetLastError();
}

hipError_t moe_launch_split_bf16(const float* h, long rows, int C, uint16_t* out, hipStream_t s) {
  const long n = rows * C;
  if (n == 0) return hipSuccess;
  const long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(split_bf16_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0,
                     s, h, rows, C, out);
  return hipGetLastError();
}
