// C ABI of libmoe_mi355x: argument checks, workspace layout, kernel dispatch and the
// host-side path counters.  Every entry point only enqueues work on the caller's stream.
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "moe_device.h"

namespace {

std::atomic<uint64_t> g_counters[MOE_CNT_SLOTS];

inline void bump(int slot) { g_counters[slot].fetch_add(1, std::memory_order_relaxed); }

bool debug_sync() {
  static const bool on = [] {
    const char* v = std::getenv("MOE_MI355X_DEBUG_SYNC");
    return v && v[0] == '1';
  }();
  return on;
}

moe_status finish(hipError_t e, hipStream_t s) {
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (debug_sync()) {
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool dims_ok(const moe_dims* d) {
  if (!d) return false;
  if (d->T < 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->k <= 0) return false;
  if (d->E > 1024 || d->k > d->E || d->k > 32) return false;
  if (d->H % 32 || d->I % 32) return false;
  return true;
}

// Token counts from which moe_expert_ffn runs the tiled prefill GEMMs instead of the
// decode-shaped kernels: routed STQ1_0 experts, and the bf16 shared expert.
// MOE_MI355X_PREFILL_MIN_T overrides both (measurement).
int prefill_min_t(bool shared) {
  static const int over = [] {
    const char* v = std::getenv("MOE_MI355X_PREFILL_MIN_T");
    return v ? std::atoi(v) : -1;
  }();
  if (over >= 0) return over;
  // measured crossovers (Hy4 shapes): routed 1.72 vs 2.12 ms at 64 tokens, 2.50 vs 2.43 ms
  // at 128; shared 151 vs 241 us at 128 tokens, 294 vs about 230 us at 256
  return shared ? 256 : 128;
}

bool stq_gemm_ok(const moe_dims* d) {
  return d->T >= prefill_min_t(false) && d->H % 256 == 0 && d->I % 256 == 0;
}
bool shared_gemm_ok(const moe_dims* d) {
  return d->T >= prefill_min_t(true) && d->H % 256 == 0 && d->I % 256 == 0;
}

// Size limits of moe_expert_ffn.  The grouped GEMMs address each activation operand through
// a buffer resource with 32-bit offsets, and an offset of 2^31 or more marks an absent row,
// so every operand stays within 2^31 bytes: x and h, in the GEMM's input format, per family
// (routed STQ1_0: x fp16 [T][H], h fp16 hi | lo [P][2I]; routed MXFP4: x and h E4M3 [T][H],
// [P][I]; shared bf16 or MXFP8: x bf16 [T][H], h two bf16 [T][2I]).  The decode-shaped kernels
// put token tiles of 8 (the generic STQ1_0 one: single tokens) on a grid dimension that stops
// at 65535.
constexpr int64_t kMaxOperand = (int64_t)1 << 31;
constexpr int64_t kMaxGridYZ = 65535;
bool ffn_size_ok(const moe_dims* d, int fmt, const moe_experts* shared) {
  const int64_t T = d->T, H = d->H, I = d->I, P = T * d->k;
  if (fmt == MOE_W_STQ1_0) {
    if (stq_gemm_ok(d)) {
      if (T * H * 2 > kMaxOperand || P * I * 4 > kMaxOperand) return false;
    } else if (T > ((H % 256 || I % 256) ? kMaxGridYZ : 8 * kMaxGridYZ)) {
      return false;
    }
  } else if (T * H > kMaxOperand || P * I > kMaxOperand) {
    return false;
  }
  if (shared) {
    if (shared->fmt == MOE_W_MXFP8 || shared_gemm_ok(d)) {
      if (T * H * 2 > kMaxOperand || T * I * 4 > kMaxOperand) return false;
    } else if (T > 8 * kMaxGridYZ) {
      return false;
    }
  }
  return true;
}

// Workspace regions: 0 h routed f32, 1 h shared f32, 2 xq, 3 xs, 4 hq, 5 hs, 6 total;
// internal regions of the prefill GEMMs (ext): 0 x fp16 [T][H], 1 x row exponents [T],
// 2 h as fp16 hi | lo [P][2I], 3 h row exponents [P], 4 shared h as bf16 hi | lo [T][2I]
// (MXFP8 shared expert: the bf16 values of its E4M3 h [T][I]), 5 MXFP8 shared expert: the
// bf16 values of its E4M3 x [T][H].
void layout(const moe_dims* d, int fmt, int has_shared, size_t* offs, size_t* ext = nullptr) {
  const size_t T = d->T, H = d->H, I = d->I, P = (size_t)d->T * d->k;
  size_t e[6];
  for (int i = 0; i < 7; ++i) offs[i] = (size_t)-1;
  for (int i = 0; i < 6; ++i) e[i] = (size_t)-1;
  size_t cur = 0;
  if (fmt == MOE_W_STQ1_0) {
    offs[0] = cur;
    cur = align_up(cur + P * I * sizeof(float));
  }
  if (has_shared) {
    offs[1] = cur;
    cur = align_up(cur + T * I * sizeof(float));
  }
  if (fmt == MOE_W_MXFP4 || fmt == MOE_W_MXFP4_TILED) {
    offs[2] = cur; cur = align_up(cur + T * H);
    offs[3] = cur; cur = align_up(cur + T * (H / 32));
    offs[4] = cur; cur = align_up(cur + P * I);
    offs[5] = cur; cur = align_up(cur + P * (I / 32));
  }
  if (fmt == MOE_W_STQ1_0 && stq_gemm_ok(d)) {
    e[0] = cur; cur = align_up(cur + T * H * 2);
    e[1] = cur; cur = align_up(cur + T * 4);
    e[2] = cur; cur = align_up(cur + P * 2 * I * 2);
    e[3] = cur; cur = align_up(cur + P * 4);
  }
  if (has_shared) {   // (the shared expert's format is not known here: bf16 or MXFP8)
    e[4] = cur; cur = align_up(cur + T * 2 * I * 2);
    e[5] = cur; cur = align_up(cur + T * H * 2);
  }
  offs[6] = cur;
  if (ext)
    for (int i = 0; i < 6; ++i) ext[i] = e[i];
}

bool routed_fmt_ok(int fmt) {
  return fmt == MOE_W_STQ1_0 || fmt == MOE_W_MXFP4 || fmt == MOE_W_MXFP4_TILED;
}

bool mat_ok(const moe_mat& m, bool need_scales) { return m.codes && (!need_scales || m.scales); }

// ---- opt-in event profiler: per slot a pool of (begin, end) event pairs
constexpr int kProfPool = 8192;
struct ProfSlot {
  std::vector<hipEvent_t> ev;   // 2 * kProfPool
  int used = 0;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
ProfSlot g_prof[MOE_PROF_SLOTS_INTERNAL];

}  // namespace

bool moe_prof_on() { return g_prof_on.load(std::memory_order_relaxed); }

void moe_prof_begin(int slot, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfSlot& p = g_prof[slot];
  if (p.ev.empty() || p.used >= kProfPool) return;
  hipEventRecord(p.ev[2 * p.used], s);
}

void moe_prof_end(int slot, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfSlot& p = g_prof[slot];
  if (p.ev.empty() || p.used >= kProfPool) return;
  hipEventRecord(p.ev[2 * p.used + 1], s);
  ++p.used;
}

extern "C" {

moe_status moe_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on) {
    for (auto& p : g_prof) {
      if (p.ev.empty()) {
        p.ev.resize(2 * kProfPool);
        for (auto& e : p.ev)
          if (hipEventCreate(&e) != hipSuccess) return MOE_ERR_HIP;
      }
      p.used = 0;
    }
  }
  g_prof_on.store(on != 0);
  return MOE_OK;
}

moe_status moe_profile_read(double* avg_us, int64_t* count) {
  if (!avg_us || !count) return MOE_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (int i = 0; i < MOE_PROF_SLOTS_INTERNAL; ++i) {
    ProfSlot& p = g_prof[i];
    double tot = 0.0;
    for (int j = 0; j < p.used; ++j) {
      if (hipEventSynchronize(p.ev[2 * j + 1]) != hipSuccess) return MOE_ERR_HIP;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, p.ev[2 * j], p.ev[2 * j + 1]) != hipSuccess) return MOE_ERR_HIP;
      tot += ms;
    }
    count[i] = p.used;
    avg_us[i] = p.used ? tot * 1e3 / p.used : 0.0;
    p.used = 0;
  }
  return MOE_OK;
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or format";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* moe_version(void) { return "moe_mi355x 0.1 gfx950"; }

moe_status moe_get_counters(uint64_t* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < MOE_CNT_SLOTS; ++i) out[i] = g_counters[i].load(std::memory_order_relaxed);
  return MOE_OK;
}

moe_status moe_reset_counters(void) {
  for (int i = 0; i < MOE_CNT_SLOTS; ++i) g_counters[i].store(0, std::memory_order_relaxed);
  return MOE_OK;
}

moe_status moe_route(const moe_dims* d, const uint16_t* x_bf16, const uint16_t* wr_bf16,
                     const float* logit_bias, const float* logits_in, float* logits_out,
                     int32_t* topk_ids, float* topk_w, void* stream) {
  if (!dims_ok(d) || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!logits_in && (!x_bf16 || !wr_bf16 || !logits_out)) return MOE_ERR_INVALID_ARG;
  // the logits GEMV puts 8-token tiles on a grid dimension that stops at 65535
  if (!logits_in && d->T > 8 * kMaxGridYZ) return MOE_ERR_UNSUPPORTED;
  if (d->T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  if (!logits_in) {
    hipError_t e = moe_launch_route_gemv(x_bf16, wr_bf16, logit_bias, logits_out, d->T, d->H,
                                         d->E, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    bump(MOE_CNT_ROUTE_GEMV);
    e = moe_launch_topk(logits_out, nullptr, nullptr, d->T, d->E, d->k, topk_ids, topk_w, s);
    bump(MOE_CNT_ROUTE_TOPK);
    return finish(e, s);
  }
  hipError_t e = moe_launch_topk(logits_in, logit_bias, logits_out, d->T, d->E, d->k, topk_ids,
                                 topk_w, s);
  bump(MOE_CNT_ROUTE_TOPK);
  return finish(e, s);
}

moe_status moe_permute(const moe_dims* d, const int32_t* topk_ids, int32_t* sorted_pair,
                       int32_t* expert_offsets, int32_t* pair_pos, void* stream) {
  if (!dims_ok(d) || !topk_ids || !sorted_pair || !expert_offsets || !pair_pos)
    return MOE_ERR_INVALID_ARG;
  if ((int64_t)d->T * d->k > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  hipError_t e = moe_launch_permute(topk_ids, d->T * d->k, d->E, sorted_pair, expert_offsets,
                                    pair_pos, s);
  bump(MOE_CNT_PERMUTE);
  return finish(e, s);
}

moe_status moe_workspace_size(const moe_dims* d, int32_t routed_fmt, int32_t has_shared,
                              size_t* bytes) {
  if (!dims_ok(d) || !bytes) return MOE_ERR_INVALID_ARG;
  if (!routed_fmt_ok(routed_fmt)) return MOE_ERR_INVALID_ARG;
  size_t offs[7];
  layout(d, routed_fmt, has_shared, offs);
  *bytes = offs[6];
  return MOE_OK;
}

moe_status moe_workspace_offsets(const moe_dims* d, int32_t routed_fmt, int32_t has_shared,
                                 size_t* offs) {
  if (!dims_ok(d) || !offs) return MOE_ERR_INVALID_ARG;
  if (!routed_fmt_ok(routed_fmt)) return MOE_ERR_INVALID_ARG;
  layout(d, routed_fmt, has_shared, offs);
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_dims* d, const moe_experts* routed,
                          const moe_experts* shared, const uint16_t* x_bf16,
                          const int32_t* sorted_pair, const int32_t* expert_offsets,
                          float* y_pairs, float* y_shared, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!dims_ok(d) || !routed || !x_bf16 || !sorted_pair || !expert_offsets || !y_pairs)
    return MOE_ERR_INVALID_ARG;
  const int fmt = routed->fmt;
  if (!routed_fmt_ok(fmt)) return MOE_ERR_INVALID_ARG;
  if (!mat_ok(routed->gate, true) || !mat_ok(routed->up, true) || !mat_ok(routed->down, true))
    return MOE_ERR_INVALID_ARG;
  if (shared) {
    if ((shared->fmt != MOE_W_BF16 && shared->fmt != MOE_W_MXFP8) || !y_shared) return MOE_ERR_INVALID_ARG;
    const bool sc = shared->fmt == MOE_W_MXFP8;
    if (!mat_ok(shared->gate, sc) || !mat_ok(shared->up, sc) || !mat_ok(shared->down, sc))
      return MOE_ERR_INVALID_ARG;
    if (d->H % 256 || d->I % 256) return MOE_ERR_UNSUPPORTED;
  }
  if (!ffn_size_ok(d, fmt, shared)) return MOE_ERR_UNSUPPORTED;
  const int T = d->T, H = d->H, I = d->I, E = d->E, k = d->k;
  if (fmt == MOE_W_STQ1_0) {
    if (((int64_t)H * I) % 256) return MOE_ERR_UNSUPPORTED;
    if (H % 256 == 0 && H / 256 > 4 * 16) return MOE_ERR_UNSUPPORTED;
    if (I % 256 == 0 && I / 256 > 4 * 16) return MOE_ERR_UNSUPPORTED;
  } else {
    if (H % 128 || I % 128) return MOE_ERR_UNSUPPORTED;
  }
  size_t offs[7], ext[6];
  layout(d, fmt, shared != nullptr, offs, ext);
  if (!ws || ws_bytes < offs[6]) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const int P = T * k;

  const bool prof = moe_prof_on();
  if (fmt == MOE_W_STQ1_0 && ext[0] != (size_t)-1) {
    // prefill: x -> fp16 rows, grouped GEMMs on the fp16 MFMA, h -> fp16 hi | lo rows
    float* h = reinterpret_cast<float*>(wsb + offs[0]);
    uint16_t* x16 = reinterpret_cast<uint16_t*>(wsb + ext[0]);
    int32_t* xe = reinterpret_cast<int32_t*>(wsb + ext[1]);
    uint16_t* h16 = reinterpret_cast<uint16_t*>(wsb + ext[2]);
    int32_t* he = reinterpret_cast<int32_t*>(wsb + ext[3]);
    if (prof) moe_prof_begin(MOE_PROF_ACT_PREP, s);
    hipError_t e = moe_launch_rowscale_f16(x_bf16, nullptr, T, H, 0, x16, xe, s);
    if (prof) moe_prof_end(MOE_PROF_ACT_PREP, s);
    bump(MOE_CNT_ROWSCALE);
    if (e != hipSuccess) return MOE_ERR_HIP;
    G16Args a{};
    a.w0 = routed->gate.codes; a.s0 = static_cast<const uint16_t*>(routed->gate.scales);
    a.w1 = routed->up.codes;   a.s1 = static_cast<const uint16_t*>(routed->up.scales);
    a.a = x16; a.aexp = xe; a.sorted_pair = sorted_pair; a.offsets = expert_offsets; a.out = h;
    a.N = I; a.K = H; a.Ka = H; a.rows_a = T; a.E = E; a.k = k; a.P = P;
    if (prof) moe_prof_begin(MOE_PROF_STQ_GATEUP, s);
    e = moe_launch_g16_stq_gateup(a, s);
    if (prof) moe_prof_end(MOE_PROF_STQ_GATEUP, s);
    bump(MOE_CNT_STQ_GEMM);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (prof) moe_prof_begin(MOE_PROF_ACT_PREP, s);
    e = moe_launch_rowscale_f16(nullptr, h, P, I, 1, h16, he, s);
    if (prof) moe_prof_end(MOE_PROF_ACT_PREP, s);
    bump(MOE_CNT_ROWSCALE);
    if (e != hipSuccess) return MOE_ERR_HIP;
    G16Args b{};
    b.w0 = routed->down.codes; b.s0 = static_cast<const uint16_t*>(routed->down.scales);
    b.a = h16; b.aexp = he; b.sorted_pair = sorted_pair; b.offsets = expert_offsets; b.out = y_pairs;
    b.N = H; b.K = I; b.Ka = 2 * I; b.rows_a = P; b.E = E; b.k = k; b.P = P;
    if (prof) moe_prof_begin(MOE_PROF_STQ_DOWN, s);
    e = moe_launch_g16_stq_down(b, s);
    if (prof) moe_prof_end(MOE_PROF_STQ_DOWN, s);
    bump(MOE_CNT_STQ_GEMM);
    if (e != hipSuccess) return MOE_ERR_HIP;
  } else if (fmt == MOE_W_STQ1_0) {
    float* h = reinterpret_cast<float*>(wsb + offs[0]);
    FfnArgs a{};
    a.codes0 = routed->gate.codes; a.scales0 = routed->gate.scales;
    a.codes1 = routed->up.codes;   a.scales1 = routed->up.scales;
    a.act = x_bf16; a.sorted_pair = sorted_pair; a.offsets = expert_offsets; a.out = h;
    a.N = I; a.K = H; a.T = T; a.E = E; a.k = k; a.P = P;
    hipError_t e;
    if (H % 256 == 0) { e = moe_launch_stq_gateup(a, s); bump(MOE_CNT_STQ_GATEUP_MFMA); }
    else { e = moe_launch_stq_generic(a, 0, s); bump(MOE_CNT_STQ_GENERIC); }
    if (e != hipSuccess) return MOE_ERR_HIP;
    FfnArgs b{};
    b.codes0 = routed->down.codes; b.scales0 = routed->down.scales;
    b.act = h; b.sorted_pair = sorted_pair; b.offsets = expert_offsets; b.out = y_pairs;
    b.N = H; b.K = I; b.T = T; b.E = E; b.k = k; b.P = P;
    if (I % 256 == 0) { e = moe_launch_stq_down(b, s); bump(MOE_CNT_STQ_DOWN_MFMA); }
    else { e = moe_launch_stq_generic(b, 1, s); bump(MOE_CNT_STQ_GENERIC); }
    if (e != hipSuccess) return MOE_ERR_HIP;
  } else {
    uint8_t* xq = wsb + offs[2];
    uint8_t* xs = wsb + offs[3];
    uint8_t* hq = wsb + offs[4];
    uint8_t* hs = wsb + offs[5];
    if (prof) moe_prof_begin(MOE_PROF_MX_QUANT, s);
    hipError_t e = moe_launch_mx_quant(T, H, x_bf16, nullptr, xq, xs, s);
    if (prof) moe_prof_end(MOE_PROF_MX_QUANT, s);
    bump(MOE_CNT_MX_QUANT);
    if (e != hipSuccess) return MOE_ERR_HIP;
    MxArgs a{};
    a.wcodes0 = static_cast<const uint8_t*>(routed->gate.codes);
    a.wscales0 = static_cast<const uint8_t*>(routed->gate.scales);
    a.wcodes1 = static_cast<const uint8_t*>(routed->up.codes);
    a.wscales1 = static_cast<const uint8_t*>(routed->up.scales);
    a.aq = xq; a.as = xs; a.sorted_pair = sorted_pair; a.offsets = expert_offsets;
    a.hq = hq; a.hs = hs; a.N = I; a.K = H; a.T = T; a.E = E; a.k = k; a.P = P;
    a.tiled = fmt == MOE_W_MXFP4_TILED;
    if (prof) moe_prof_begin(MOE_PROF_MX_GATEUP, s);
    e = moe_launch_mx_gateup(a, s);
    if (prof) moe_prof_end(MOE_PROF_MX_GATEUP, s);
    bump(MOE_CNT_MX_GATEUP_MFMA);
    if (e != hipSuccess) return MOE_ERR_HIP;
    MxArgs b{};
    b.wcodes0 = static_cast<const uint8_t*>(routed->down.codes);
    b.wscales0 = static_cast<const uint8_t*>(routed->down.scales);
    b.aq = hq; b.as = hs; b.sorted_pair = sorted_pair; b.offsets = expert_offsets;
    b.y = y_pairs; b.N = H; b.K = I; b.T = T; b.E = E; b.k = k; b.P = P;
    b.tiled = fmt == MOE_W_MXFP4_TILED;
    if (prof) moe_prof_begin(MOE_PROF_MX_DOWN, s);
    e = moe_launch_mx_down(b, s);
    if (prof) moe_prof_end(MOE_PROF_MX_DOWN, s);
    bump(MOE_CNT_MX_DOWN_MFMA);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }

  if (shared && shared->fmt == MOE_W_MXFP8) {
    // W8A8: x and h through their MX E4M3 values (exact in bf16), grouped GEMMs on the bf16
    // MFMA with the E4M3 weights decoded in registers, at every token count
    float* hsh = reinterpret_cast<float*>(wsb + offs[1]);
    uint16_t* h2 = reinterpret_cast<uint16_t*>(wsb + ext[4]);
    uint16_t* xr = reinterpret_cast<uint16_t*>(wsb + ext[5]);
    if (prof) moe_prof_begin(MOE_PROF_ACT_PREP, s);
    hipError_t e = moe_launch_mx_roundtrip_bf16(T, H, x_bf16, nullptr, xr, s);
    if (prof) moe_prof_end(MOE_PROF_ACT_PREP, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    G16Args a{};
    a.w0 = shared->gate.codes; a.s0 = static_cast<const uint16_t*>(shared->gate.scales);
    a.w1 = shared->up.codes;   a.s1 = static_cast<const uint16_t*>(shared->up.scales);
    a.a = xr; a.out = hsh;
    a.N = I; a.K = H; a.Ka = H; a.rows_a = T; a.E = 1; a.k = 1; a.P = T;
    if (prof) moe_prof_begin(MOE_PROF_SH_GATEUP, s);
    e = moe_launch_g16_mx8_gateup(a, s);
    if (prof) moe_prof_end(MOE_PROF_SH_GATEUP, s);
    bump(MOE_CNT_MXFP8_SHARED);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (prof) moe_prof_begin(MOE_PROF_ACT_PREP, s);
    e = moe_launch_mx_roundtrip_bf16(T, I, nullptr, hsh, h2, s);
    if (prof) moe_prof_end(MOE_PROF_ACT_PREP, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    G16Args b{};
    b.w0 = shared->down.codes; b.s0 = static_cast<const uint16_t*>(shared->down.scales);
    b.a = h2; b.out = y_shared;
    b.N = H; b.K = I; b.Ka = I; b.rows_a = T; b.E = 1; b.k = 1; b.P = T;
    if (prof) moe_prof_begin(MOE_PROF_SH_DOWN, s);
    e = moe_launch_g16_mx8_down(b, s);
    if (prof) moe_prof_end(MOE_PROF_SH_DOWN, s);
    bump(MOE_CNT_MXFP8_SHARED);
    if (e != hipSuccess) return MOE_ERR_HIP;
  } else if (shared && shared_gemm_ok(d)) {
    // prefill: grouped GEMMs on the bf16 MFMA (one expert owning every token)
    float* hsh = reinterpret_cast<float*>(wsb + offs[1]);
    uint16_t* h2 = reinterpret_cast<uint16_t*>(wsb + ext[4]);
    G16Args a{};
    a.w0 = shared->gate.codes; a.w1 = shared->up.codes;
    a.a = x_bf16; a.out = hsh;
    a.N = I; a.K = H; a.Ka = H; a.rows_a = T; a.E = 1; a.k = 1; a.P = T;
    if (prof) moe_prof_begin(MOE_PROF_SH_GATEUP, s);
    hipError_t e = moe_launch_g16_bf16_gateup(a, s);
    if (prof) moe_prof_end(MOE_PROF_SH_GATEUP, s);
    bump(MOE_CNT_BF16_GEMM);
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (prof) moe_prof_begin(MOE_PROF_ACT_PREP, s);
    e = moe_launch_split_bf16(hsh, T, I, h2, s);
    if (prof) moe_prof_end(MOE_PROF_ACT_PREP, s);
    bump(MOE_CNT_ROWSCALE);
    if (e != hipSuccess) return MOE_ERR_HIP;
    G16Args b{};
    b.w0 = shared->down.codes; b.a = h2; b.out = y_shared;
    b.N = H; b.K = I; b.Ka = 2 * I; b.rows_a = T; b.E = 1; b.k = 1; b.P = T;
    if (prof) moe_prof_begin(MOE_PROF_SH_DOWN, s);
    e = moe_launch_g16_bf16_down(b, s);
    if (prof) moe_prof_end(MOE_PROF_SH_DOWN, s);
    bump(MOE_CNT_BF16_GEMM);
    if (e != hipSuccess) return MOE_ERR_HIP;
  } else if (shared) {
    float* hsh = reinterpret_cast<float*>(wsb + offs[1]);
    FfnArgs a{};
    a.codes0 = shared->gate.codes; a.codes1 = shared->up.codes;
    a.act = x_bf16; a.out = hsh; a.N = I; a.K = H; a.T = T; a.E = 1; a.k = 1; a.P = T;
    hipError_t e = moe_launch_bf16_gateup(a, s);
    bump(MOE_CNT_BF16_GATEUP);
    if (e != hipSuccess) return MOE_ERR_HIP;
    FfnArgs b{};
    b.codes0 = shared->down.codes; b.act = hsh; b.out = y_shared;
    b.N = H; b.K = I; b.T = T; b.E = 1; b.k = 1; b.P = T;
    e = moe_launch_bf16_down(b, s);
    bump(MOE_CNT_BF16_DOWN);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return finish(hipSuccess, s);
}

static bool decode_fused_ok(const moe_dims* d) {
  return d->T <= 64 && moe_decode_shape_ok(d->H, d->I, d->E);
}

moe_status moe_layer_decode_workspace_size(const moe_dims* d, int32_t has_shared, size_t* bytes) {
  if (!dims_ok(d) || !bytes) return MOE_ERR_INVALID_ARG;
  if (!decode_fused_ok(d)) return MOE_ERR_UNSUPPORTED;
  size_t offs[16];
  *bytes = moe_decode_ws_layout(d->T, d->H, d->I, d->E, d->k, has_shared != 0, offs);
  return MOE_OK;
}

moe_status moe_layer_decode_workspace_offsets(const moe_dims* d, int32_t has_shared, size_t* offs) {
  if (!dims_ok(d) || !offs) return MOE_ERR_INVALID_ARG;
  if (!decode_fused_ok(d)) return MOE_ERR_UNSUPPORTED;
  size_t o[16];
  moe_decode_ws_layout(d->T, d->H, d->I, d->E, d->k, has_shared != 0, o);
  for (int i = 0; i < 11; ++i) offs[i] = o[i];
  return MOE_OK;
}

// Argument checks of the fused decode (both entry points); MOE_OK when the call may proceed.
static moe_status decode_args_ok(const moe_dims* d, const moe_experts* routed,
                                 const moe_experts* shared, const uint16_t* x_bf16,
                                 const uint16_t* wr_bf16, const float* logits_out,
                                 const int32_t* topk_ids, const float* topk_w,
                                 const int32_t* sorted_pair, const int32_t* expert_offsets,
                                 const int32_t* pair_pos, const float* y_pairs, const float* y_shared,
                                 const float* out_f32) {
  if (!dims_ok(d) || !routed || !x_bf16 || !wr_bf16 || !logits_out || !topk_ids || !topk_w ||
      !sorted_pair || !expert_offsets || !pair_pos || !y_pairs || !out_f32)
    return MOE_ERR_INVALID_ARG;
  if (!routed_fmt_ok(routed->fmt)) return MOE_ERR_INVALID_ARG;   // as moe_expert_ffn
  const bool mx = routed->fmt == MOE_W_MXFP4 || routed->fmt == MOE_W_MXFP4_TILED;
  if (mx && !moe_decode_mx_ok(d->T, d->I, d->k)) return MOE_ERR_UNSUPPORTED;
  if (!mat_ok(routed->gate, true) || !mat_ok(routed->up, true) || !mat_ok(routed->down, true))
    return MOE_ERR_INVALID_ARG;
  if (shared) {
    if (shared->fmt == MOE_W_MXFP8) return MOE_ERR_UNSUPPORTED;   // four-call path only
    if (shared->fmt != MOE_W_BF16 || !y_shared) return MOE_ERR_INVALID_ARG;
    if (!mat_ok(shared->gate, false) || !mat_ok(shared->up, false) || !mat_ok(shared->down, false))
      return MOE_ERR_INVALID_ARG;
  }
  if (!decode_fused_ok(d)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_layer_decode_noalloc(const moe_dims* d, const moe_experts* routed,
                                    const moe_experts* shared, const uint16_t* x_bf16,
                                    const uint16_t* wr_bf16, const float* logit_bias,
                                    float* logits_out, int32_t* topk_ids, float* topk_w,
                                    int32_t* sorted_pair, int32_t* expert_offsets,
                                    int32_t* pair_pos, float* y_pairs, float* y_shared,
                                    const float* residual, float* out_f32, uint16_t* out_bf16,
                                    void* stream) {
  const moe_status st = decode_args_ok(d, routed, shared, x_bf16, wr_bf16, logits_out, topk_ids,
                                       topk_w, sorted_pair, expert_offsets, pair_pos, y_pairs,
                                       y_shared, out_f32);
  if (st != MOE_OK) return st;
  size_t offs[16];
  const size_t need = moe_decode_ws_layout(d->T, d->H, d->I, d->E, d->k, shared != nullptr, offs);
  if (need > kDecodeStaticScratchBytes) return MOE_ERR_UNSUPPORTED;
  if (d->T == 0) return MOE_OK;
  void* ws = moe_decode_static_scratch();
  if (!ws) return MOE_ERR_HIP;
  hipStream_t s = as_stream(stream);
  hipError_t e = moe_clear_decode_header(ws, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe_launch_decode_fused(d, routed, shared, x_bf16, wr_bf16, logit_bias, logits_out,
                              topk_ids, topk_w, sorted_pair, expert_offsets, pair_pos, y_pairs,
                              y_shared, residual, out_f32, out_bf16, ws, s);
  bump(MOE_CNT_DECODE_FUSED);
  return finish(e, s);
}

moe_status moe_layer_decode(const moe_dims* d, const moe_experts* routed,
                            const moe_experts* shared, const uint16_t* x_bf16,
                            const uint16_t* wr_bf16, const float* logit_bias, float* logits_out,
                            int32_t* topk_ids, float* topk_w, int32_t* sorted_pair,
                            int32_t* expert_offsets, int32_t* pair_pos, float* y_pairs,
                            float* y_shared, const float* residual, float* out_f32,
                            uint16_t* out_bf16, void* ws, size_t ws_bytes, void* stream) {
  const moe_status st = decode_args_ok(d, routed, shared, x_bf16, wr_bf16, logits_out, topk_ids,
                                       topk_w, sorted_pair, expert_offsets, pair_pos, y_pairs,
                                       y_shared, out_f32);
  if (st != MOE_OK) return st;
  size_t offs[16];
  const size_t need = moe_decode_ws_layout(d->T, d->H, d->I, d->E, d->k, shared != nullptr, offs);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (d->T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  hipError_t e = moe_launch_decode_fused(d, routed, shared, x_bf16, wr_bf16, logit_bias,
                                         logits_out, topk_ids, topk_w, sorted_pair,
                                         expert_offsets, pair_pos, y_pairs, y_shared, residual,
                                         out_f32, out_bf16, ws, s);
  bump(MOE_CNT_DECODE_FUSED);
  return finish(e, s);
}

moe_status moe_combine(const moe_dims* d, const float* y_pairs, const float* topk_w,
                       const int32_t* pair_pos, const float* y_shared, const float* residual,
                       float* out_f32, uint16_t* out_bf16, void* stream) {
  if (!dims_ok(d) || !y_pairs || !topk_w || !pair_pos || !out_f32) return MOE_ERR_INVALID_ARG;
  if (d->T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  hipError_t e = moe_launch_combine(y_pairs, topk_w, pair_pos, y_shared, residual, out_f32,
                                    out_bf16, d->T, d->H, d->k, s);
  bump(MOE_CNT_COMBINE);
  return finish(e, s);
}

moe_status moe_stq1_pack(const uint8_t* zpos, const uint8_t* signs, const uint16_t* d_f16,
                         int64_t n_blocks, uint8_t* codes, uint16_t* scales, void* stream) {
  if (n_blocks < 0 || (n_blocks > 0 && (!zpos || !signs || !d_f16 || !codes || !scales)))
    return MOE_ERR_INVALID_ARG;
  if (n_blocks == 0) return MOE_OK;
  if (n_blocks > (int64_t)4 * 0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  return finish(moe_launch_stq1_pack(zpos, signs, d_f16, n_blocks, codes, scales, s), s);
}

moe_status moe_stq1_dequant(const uint8_t* codes, const uint16_t* scales, int64_t n_blocks,
                            float* out, void* stream) {
  if (n_blocks < 0 || (n_blocks > 0 && (!codes || !scales || !out))) return MOE_ERR_INVALID_ARG;
  if (n_blocks == 0) return MOE_OK;
  if (n_blocks > (int64_t)4 * 0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  bump(MOE_CNT_DEQUANT);
  return finish(moe_launch_stq1_dequant(codes, scales, n_blocks, out, s), s);
}

moe_status moe_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int32_t K, float* out, void* stream) {
  if (rows < 0 || K <= 0 || K % 32 || (rows > 0 && (!codes || !scales || !out)))
    return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (rows * (K / 2) > (int64_t)256 * 0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  bump(MOE_CNT_DEQUANT);
  return finish(moe_launch_mxfp4_dequant(codes, scales, rows, K, out, s), s);
}

moe_status moe_mxfp4_pack_tiles(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                int32_t K, uint8_t* tcodes, uint8_t* tscales, void* stream) {
  if (rows < 0 || K <= 0 || rows % 16 || K % 128) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!codes || !scales || !tcodes || !tscales) return MOE_ERR_INVALID_ARG;
  if (((uintptr_t)codes | (uintptr_t)tcodes) % 16 || ((uintptr_t)scales | (uintptr_t)tscales) % 4)
    return MOE_ERR_INVALID_ARG;
  const uintptr_t nc = (uintptr_t)rows * (K / 2), ns = (uintptr_t)rows * (K / 32);
  auto overlap = [](const void* a, uintptr_t na, const void* b, uintptr_t nb) {
    return (uintptr_t)a < (uintptr_t)b + nb && (uintptr_t)b < (uintptr_t)a + na;
  };
  if (overlap(tcodes, nc, codes, nc) || overlap(tcodes, nc, scales, ns) ||
      overlap(tscales, ns, codes, nc) || overlap(tscales, ns, scales, ns))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = as_stream(stream);
  return finish(moe_launch_mxfp4_pack_tiles(codes, scales, rows, K, tcodes, tscales, s), s);
}

moe_status moe_stq1_encode(const float* x, const float* imatrix, int64_t n_weights, int32_t K,
                           int32_t method, uint8_t* codes, uint16_t* scales, void* stream) {
  if (n_weights < 0 || n_weights % 256 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (method != MOE_STQ1_ENC_UPSTREAM && method != MOE_STQ1_ENC_WLS) return MOE_ERR_INVALID_ARG;
  if (n_weights == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(codes) % 8 ||
      reinterpret_cast<uintptr_t>(scales) % 2)
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = as_stream(stream);
  return finish(moe_launch_stq1_encode(x, imatrix, n_weights / 256, K, method, codes, scales, s), s);
}

moe_status moe_mx_quant_act(int64_t rows, int32_t K, const uint16_t* x_bf16, const float* x_f32,
                            uint8_t* q, uint8_t* sc, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARG;
  if ((x_bf16 == nullptr) == (x_f32 == nullptr)) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!q || !sc)) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if ((rows * (int64_t)K / 8 + 255) / 256 > 0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;   // 8 elements per lane
  hipStream_t s = as_stream(stream);
  bump(MOE_CNT_MX_QUANT);
  return finish(moe_launch_mx_quant(rows, K, x_bf16, x_f32, q, sc, s), s);
}

moe_status moe_mx_quant_f32_hwcvt(int64_t rows, int32_t K, const float* x_f32, uint8_t* q,
                                  uint8_t* sc, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!x_f32 || !q || !sc)) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if ((rows * (int64_t)K / 8 + 255) / 256 > 0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  return finish(moe_launch_mx_quant_hw(rows, K, x_f32, q, sc, s), s);
}

moe_status moe_rmsnorm_bf16(int32_t T, int32_t H, float eps, const float* r, uint16_t* a,
                            void* stream) {
  if (T < 0 || H <= 0 || (T > 0 && (!r || !a)) || !(eps >= 0.f)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  hipStream_t s = as_stream(stream);
  bump(MOE_CNT_RMSNORM);
  return finish(moe_launch_rmsnorm(r, a, T, H, eps, s), s);
}

}  // extern "C"
