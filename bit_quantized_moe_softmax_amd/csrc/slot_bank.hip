// Expert slot bank: routed experts held in a fixed number of device slots, filled on demand
// from caller-owned host memory ("Hy4-preview Flash-MoE STQ1_0": the routed gate/up/down
// tensors live expert-major outside the dense model and are streamed into a slot bank as the
// router asks for them; 8 slots are the minimum for top-8, more slots cache more experts; a
// miss is read in bounded chunks, independent misses in parallel).  Here the source is pinned
// host memory (no file I/O) and the bank is HBM.
//
// Per step the host plans (moe_slot_bank_plan): the step's distinct experts that are resident
// are hits; each miss takes an empty slot, else the least recently used slot that no expert of
// this step holds (lowest slot on ties).  moe_slot_bank_fetch enqueues every planned copy not
// yet fetched (every family buffer of a missing expert, cut into io_split chunks) on the
// caller's stream, so a plan made twice, or a fetch that failed, loses no copy (a copy whose
// slot a later plan reuses is dropped).  moe_remap_ids turns the routed expert ids into slot
// ids on the device, so the unchanged permute / expert FFN / combine calls run on the S slots
// as S experts.
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "moe_device.h"

struct moe_slot_bank {
  int E = 0, S = 0, io_split = 1;
  uint64_t bytes[6] = {0, 0, 0, 0, 0, 0};   // per expert: gate codes, scales, up ..., down ...
  std::vector<int> slot_of;                  // [E] slot of each expert, -1 if not resident
  std::vector<int> expert_in;                // [S] expert in each slot, -1 if empty
  std::vector<uint64_t> last_use;            // [S] step of the last use
  std::vector<std::pair<int, int>> pending;  // (expert, slot) copies planned, not yet fetched
  uint64_t step = 0, hits = 0, misses = 0;
};

namespace {

__global__ __launch_bounds__(256) void remap_ids_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                        const int32_t* __restrict__ slot_of,
                                                        int32_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = slot_of[ids[i]];
}

inline const void* family_ptr(const moe_experts* m, int f) {
  const moe_mat& mm = f < 2 ? m->gate : (f < 4 ? m->up : m->down);
  return (f & 1) ? mm.scales : mm.codes;
}

}  // namespace

extern "C" {

moe_status moe_slot_bank_create(int32_t E, int32_t S, const uint64_t* bytes, int32_t io_split,
                                moe_slot_bank** out) {
  if (!out || !bytes || E <= 0 || E > 1024 || S <= 0 || S > E || io_split <= 0)
    return MOE_ERR_INVALID_ARG;
  moe_slot_bank* b = new (std::nothrow) moe_slot_bank();
  if (!b) return MOE_ERR_INVALID_ARG;
  b->E = E;
  b->S = S;
  b->io_split = io_split;
  std::memcpy(b->bytes, bytes, sizeof(b->bytes));
  b->slot_of.assign(E, -1);
  b->expert_in.assign(S, -1);
  b->last_use.assign(S, 0);
  *out = b;
  return MOE_OK;
}

moe_status moe_slot_bank_destroy(moe_slot_bank* b) {
  delete b;
  return MOE_OK;
}

moe_status moe_slot_bank_plan(moe_slot_bank* b, const int32_t* ids, int64_t n, int32_t* slot_of,
                              int32_t* n_copies) {
  if (!b || (n > 0 && !ids) || n < 0 || !slot_of || !n_copies) return MOE_ERR_INVALID_ARG;
  // the step's distinct experts, in order of first appearance
  std::vector<int> distinct;
  std::vector<char> seen(b->E, 0);
  for (int64_t i = 0; i < n; ++i) {
    const int e = ids[i];
    if (e < 0 || e >= b->E) return MOE_ERR_INVALID_ARG;
    if (!seen[e]) {
      seen[e] = 1;
      distinct.push_back(e);
    }
  }
  if ((int)distinct.size() > b->S) return MOE_ERR_UNSUPPORTED;   // more experts than slots
  const uint64_t misses0 = b->misses;
  ++b->step;
  for (int e : distinct)
    if (b->slot_of[e] >= 0) {
      b->last_use[b->slot_of[e]] = b->step;
      ++b->hits;
    }
  for (int e : distinct) {
    if (b->slot_of[e] >= 0) continue;
    int victim = -1;
    for (int s = 0; s < b->S && victim < 0; ++s)
      if (b->expert_in[s] < 0) victim = s;
    if (victim < 0)
      for (int s = 0; s < b->S; ++s)
        if (b->last_use[s] < b->step && (victim < 0 || b->last_use[s] < b->last_use[victim])) victim = s;
    // a victim always exists: at most S distinct experts use this step's slots
    if (b->expert_in[victim] >= 0) b->slot_of[b->expert_in[victim]] = -1;
    // a copy into this slot planned earlier and never fetched is superseded
    b->pending.erase(std::remove_if(b->pending.begin(), b->pending.end(),
                                    [victim](const std::pair<int, int>& c) { return c.second == victim; }),
                     b->pending.end());
    b->expert_in[victim] = e;
    b->slot_of[e] = victim;
    b->last_use[victim] = b->step;
    b->pending.emplace_back(e, victim);
    ++b->misses;
  }
  std::copy(b->slot_of.begin(), b->slot_of.end(), slot_of);
  *n_copies = (int32_t)(b->misses - misses0);
  return MOE_OK;
}

moe_status moe_slot_bank_fetch(moe_slot_bank* b, const moe_experts* host_src,
                               const moe_experts* dev_slots, void* stream) {
  if (!b || !host_src || !dev_slots) return MOE_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (const auto& c : b->pending) {
    for (int f = 0; f < 6; ++f) {
      const uint64_t nb = b->bytes[f];
      if (nb == 0) continue;
      const uint8_t* src = static_cast<const uint8_t*>(family_ptr(host_src, f));
      uint8_t* dst = static_cast<uint8_t*>(const_cast<void*>(family_ptr(dev_slots, f)));
      if (!src || !dst) return MOE_ERR_INVALID_ARG;
      src += (uint64_t)c.first * nb;
      dst += (uint64_t)c.second * nb;
      const uint64_t chunk = (nb + b->io_split - 1) / b->io_split;
      for (uint64_t o = 0; o < nb; o += chunk) {
        const uint64_t len = std::min(chunk, nb - o);
        if (hipMemcpyAsync(dst + o, src + o, len, hipMemcpyHostToDevice, s) != hipSuccess)
          return MOE_ERR_HIP;
      }
    }
  }
  b->pending.clear();
  return MOE_OK;
}

moe_status moe_slot_bank_stats(const moe_slot_bank* b, uint64_t* hits, uint64_t* misses) {
  if (!b || !hits || !misses) return MOE_ERR_INVALID_ARG;
  *hits = b->hits;
  *misses = b->misses;
  return MOE_OK;
}

moe_status moe_remap_ids(const int32_t* ids, int64_t n, const int32_t* slot_of, int32_t* out,
                         void* stream) {
  if (n < 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!ids || !slot_of || !out) return MOE_ERR_INVALID_ARG;
  if ((n + 255) / 256 > 0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(remap_ids_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids, n,
                     slot_of, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
