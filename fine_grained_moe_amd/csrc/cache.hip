// Expert streaming for the int4 top-1 serving path: a budgeted set of expert
// slots in HBM with least-recently-used replacement, filled from pinned host
// memory.  The article's opening section (proof-of-loop paragraph) has a
// token touch the always-resident shared expert plus a couple of small routed
// experts streamed from larger storage; its "Two embarrassing lessons"
// section warns that a warm cache can hide the miss cost.
//
// The runtime is host code: per step it reads the batch's loads (from
// moe_route), keeps the experts with a load resident, and for each miss
// evicts the slot used longest ago among those the batch does not need; then
// it fills the missed slots and rewrites the device slot table (expert ->
// slot) on the caller's stream.  When the runtime maps the pinned host copy
// at the same address on the device (unified addressing, checked once with
// hipPointerGetAttributes), one launch copies every missed expert's four int4
// arrays, reading host memory over PCIe; otherwise each array is a
// hipMemcpyAsync (measured on gfx950: four copies per expert cost ~47 us per
// miss, mostly per-copy overhead).  The slot table travels as kernel
// arguments.  The device buffers and the pinned host copy belong to the
// caller; the runtime allocates only its own host bookkeeping.
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "kernels.h"
#include "moe.h"

namespace {

struct SlotTable {
  int32_t s[64];
};

__global__ void set_slots_kernel(int32_t* __restrict__ dst, SlotTable t, int E) {
  const int e = threadIdx.x;
  if (e < E) dst[e] = t.s[e];
}

// One step's misses: expert e[m]'s four arrays (bytes[i] each, multiples of
// 16) from src[i] + e[m] * bytes[i] to dst[i] + slot[m] * bytes[i].  Grid y:
// the miss; the x blocks stride over its 16-byte units.
struct FillArgs {
  const char* src[4];
  char* dst[4];
  unsigned long long bytes[4];
  int n;
  int16_t e[64], slot[64];
};

__global__ __launch_bounds__(256) void fill_slots_kernel(FillArgs a) {
  const int m = blockIdx.y;
  if (m >= a.n) return;
  const unsigned long long units = (a.bytes[0] + a.bytes[1] + a.bytes[2] + a.bytes[3]) / 16;
  for (unsigned long long u = (unsigned long long)blockIdx.x * 256 + threadIdx.x; u < units;
       u += (unsigned long long)gridDim.x * 256) {
    unsigned long long off = u * 16;
    int i = 0;
    while (i < 3 && off >= a.bytes[i]) {
      off -= a.bytes[i];
      ++i;
    }
    const uint4 v = *reinterpret_cast<const uint4*>(a.src[i] + (unsigned long long)a.e[m] * a.bytes[i] + off);
    *reinterpret_cast<uint4*>(a.dst[i] + (unsigned long long)a.slot[m] * a.bytes[i] + off) = v;
  }
}

}  // namespace

struct moe_expert_cache {
  int E = 0, n_slots = 0;
  bool dry = false;
  bool zero_copy = false;                    // the host copy is readable by kernels at its own address
  size_t bytes[4] = {0, 0, 0, 0};            // per expert: q gate/up, scales, q down, scales
  const char* host[4] = {nullptr, nullptr, nullptr, nullptr};
  char* dev[4] = {nullptr, nullptr, nullptr, nullptr};
  int32_t* dev_slot = nullptr;
  std::vector<int> slot_of;                  // expert -> slot, -1 if not resident
  std::vector<int> expert_in;                // slot -> expert, -1 if free
  std::vector<long long> last_use;           // slot -> step of its last use
  long long step = 0;
  long long hits = 0, misses = 0;
};

extern "C" {

moe_status moe_cache_create(const moe_dims* dims, int32_t n_slots, const moe_weights* host, const moe_weights* dev,
                            int32_t* dev_slot, int32_t flags, moe_expert_cache** out) {
  if (!dims || !out) return MOE_E_ARG;
  *out = nullptr;
  const moe_dims& d = *dims;
  if (d.E < 1 || d.E > 64 || d.d < 128 || d.d % 128 || d.F < 128 || d.F % 128) return MOE_E_UNSUPPORTED;
  if (d.w_routed != MOE_INT4_G128) return MOE_E_UNSUPPORTED;
  if (n_slots < 1 || n_slots > d.E) return MOE_E_ARG;
  if (flags & ~(MOE_CACHE_DRY_RUN | MOE_CACHE_COPY_FILLS)) return MOE_E_ARG;
  const bool dry_run = (flags & MOE_CACHE_DRY_RUN) != 0;
  if (!dry_run) {
    if (!host || !dev || !dev_slot) return MOE_E_ARG;
    if (!host->w_gate_up || !host->s_gate_up || !host->w_down || !host->s_down || !dev->w_gate_up ||
        !dev->s_gate_up || !dev->w_down || !dev->s_down)
      return MOE_E_ARG;
  }
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache;
  if (!c) return MOE_E_ARG;
  c->E = d.E;
  c->n_slots = n_slots;
  c->dry = dry_run;
  const size_t D = d.d, F = d.F;
  c->bytes[0] = 2 * F * D / 2;               // [2F, d/2] packed
  c->bytes[1] = 2 * F * (D / 128) * 2;       // [2F, d/128] bf16
  c->bytes[2] = D * F / 2;                   // [d, F/2] packed
  c->bytes[3] = D * (F / 128) * 2;           // [d, F/128] bf16
  if (!c->dry) {
    const void* h[4] = {host->w_gate_up, host->s_gate_up, host->w_down, host->s_down};
    const void* v[4] = {dev->w_gate_up, dev->s_gate_up, dev->w_down, dev->s_down};
    for (int i = 0; i < 4; ++i) {
      c->host[i] = static_cast<const char*>(h[i]);
      c->dev[i] = static_cast<char*>(const_cast<void*>(v[i]));
    }
    c->dev_slot = dev_slot;
    c->zero_copy = (flags & MOE_CACHE_COPY_FILLS) == 0;
    for (int i = 0; i < 4 && c->zero_copy; ++i) {
      hipPointerAttribute_t at;
      memset(&at, 0, sizeof(at));
      if (hipPointerGetAttributes(&at, h[i]) != hipSuccess || at.type != hipMemoryTypeHost ||
          at.devicePointer != h[i])
        c->zero_copy = false;
    }
    (void)hipGetLastError();                 // a refused query leaves no error behind
  }
  c->slot_of.assign(d.E, -1);
  c->expert_in.assign(n_slots, -1);
  c->last_use.assign(n_slots, -1);
  *out = c;
  return MOE_OK;
}

moe_status moe_cache_prepare(moe_expert_cache* c, const int32_t* host_counts, void* stream, int32_t* misses) {
  if (!c || !host_counts) return MOE_E_ARG;
  int needed = 0;
  for (int e = 0; e < c->E; ++e) needed += host_counts[e] > 0;
  if (needed > c->n_slots) return MOE_E_UNSUPPORTED;       // the batch needs more experts than there are slots
  const long long now = ++c->step;
  // hits first, so no needed expert is evicted below
  for (int e = 0; e < c->E; ++e)
    if (host_counts[e] > 0 && c->slot_of[e] >= 0) {
      c->last_use[c->slot_of[e]] = now;
      ++c->hits;
    }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int step_misses = 0;
  FillArgs fa;
  memset(&fa, 0, sizeof(fa));
  for (int e = 0; e < c->E; ++e) {
    if (host_counts[e] <= 0 || c->slot_of[e] >= 0) continue;
    // a free slot (lowest index), else the least recently used slot that this
    // batch does not need (lowest index among equals)
    int victim = -1;
    for (int sl = 0; sl < c->n_slots && victim < 0; ++sl)
      if (c->expert_in[sl] < 0) victim = sl;
    if (victim < 0)
      for (int sl = 0; sl < c->n_slots; ++sl)
        if (c->last_use[sl] < now && (victim < 0 || c->last_use[sl] < c->last_use[victim])) victim = sl;
    if (victim < 0) return MOE_E_UNSUPPORTED;               // cannot happen: needed <= n_slots
    if (c->expert_in[victim] >= 0) c->slot_of[c->expert_in[victim]] = -1;
    c->slot_of[e] = victim;
    c->expert_in[victim] = e;
    c->last_use[victim] = now;
    ++c->misses;
    ++step_misses;
    if (c->dry) continue;
    if (c->zero_copy) {
      fa.e[fa.n] = (int16_t)e;
      fa.slot[fa.n] = (int16_t)victim;
      ++fa.n;
    } else {
      for (int i = 0; i < 4; ++i)
        if (hipMemcpyAsync(c->dev[i] + (size_t)victim * c->bytes[i], c->host[i] + (size_t)e * c->bytes[i],
                           c->bytes[i], hipMemcpyHostToDevice, s) != hipSuccess)
          return MOE_E_DEVICE;
    }
  }
  if (!c->dry && fa.n > 0) {
    for (int i = 0; i < 4; ++i) {
      fa.src[i] = c->host[i];
      fa.dst[i] = c->dev[i];
      fa.bytes[i] = c->bytes[i];
    }
    hipLaunchKernelGGL(fill_slots_kernel, dim3(64, (unsigned)fa.n), dim3(256), 0, s, fa);
    if (hipGetLastError() != hipSuccess) return MOE_E_DEVICE;
  }
  if (!c->dry) {
    SlotTable t;
    for (int e = 0; e < 64; ++e) t.s[e] = e < c->E ? c->slot_of[e] : -1;
    hipLaunchKernelGGL(set_slots_kernel, dim3(1), dim3(64), 0, s, c->dev_slot, t, c->E);
    if (hipGetLastError() != hipSuccess) return MOE_E_DEVICE;
  }
  if (misses) *misses = step_misses;
  return MOE_OK;
}

moe_status moe_cache_state(const moe_expert_cache* c, int32_t* slot_of, int64_t* hits_misses) {
  if (!c) return MOE_E_ARG;
  if (slot_of)
    for (int e = 0; e < c->E; ++e) slot_of[e] = c->slot_of[e];
  if (hits_misses) {
    hits_misses[0] = c->hits;
    hits_misses[1] = c->misses;
    hits_misses[2] = c->zero_copy ? 1 : 0;
  }
  return MOE_OK;
}

void moe_cache_destroy(moe_expert_cache* c) { delete c; }

}  // extern "C"
