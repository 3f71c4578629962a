// Two-part expert dispatch over a host-pinned record tier (host code only).
//
// The engine of the pages keeps every expert record in a store outside GPU
// memory and a fixed pool of device slots, LRU managed (gpu.rs module doc;
// Struct Gpu: res, the LRU expert pool).  Per layer (Struct Gpu
// service_block, the event / event_res field docs, experts_b):
//   1. the GPU runs the router, signals, and the CPU reads the union;
//   2. the CPU publishes the slot table with the resident records first
//      (entry 62: resident count, 63: union size);
//   3. the GPU runs part 0 (resident records + shared expert) while the CPU
//      reads the missing records into free slots;
//   4. the GPU runs part 1 (the fetched records) once they have landed.
// Here the store is pinned host memory (hipHostMalloc, read by the copy
// engine over PCIe), the signals are stream synchronisation and HIP events,
// and the GPU work is moe_route and moe_experts_part.  Two policies of the
// pages ride on it: the deadline cut of weak late records (Struct Gpu
// cut_w, wait_for_deadline) and the one-layer lookahead prefetch (Struct Gpu
// lookahead_layer, prefetch_async, lookahead_hit).
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "moe_internal.h"

extern "C" int moe_route(const float *x, int32_t nb, const moe_router *router, const moe_shared *shared,
                         moe_slots *slots, void *stream);
extern "C" int moe_experts_part(const float *x, int32_t nb, const moe_dims *dims, moe_slots *slots,
                                int32_t part, const moe_pool *pool, const moe_shared *shared, float *out,
                                void *stream);
extern "C" const char *moe_last_error(void);

struct moe_tier {
  moe_tier_config cfg;
  std::vector<int32_t> slot_of;     // [n_layers * E]: device slot of record (l, e), -1 if not resident
  std::vector<int64_t> owner;       // [n_slots]: record (l * E + e) in the slot, -1 if free
  std::vector<uint64_t> last_use;   // [n_slots]: LRU clock
  std::vector<uint8_t> dirty;       // [n_slots]: written by a copy the compute stream has not waited for
  std::vector<hipEvent_t> landed;   // [n_slots]: recorded after the slot's last copy
  uint64_t clock = 0;
  // pinned staging: routing results read back, tables published
  uint32_t *h_ids = nullptr;        // [64]
  float *h_wmap = nullptr;          // [4][64]
  uint64_t *h_tab = nullptr;        // [2][64] (part 0 table, part 1 republished table)
  float *h_wpub = nullptr;          // [2][4][64]
  uint32_t *h_idpub = nullptr;      // [64]
  uint32_t *h_la_ids = nullptr;     // [64] lookahead: predicted union of the next layer
  uint64_t *h_la_tab = nullptr;     // [64]
  hipEvent_t ev_route = nullptr, ev_part0 = nullptr, ev_t[4] = {};
  // lookahead: the experts predicted for the next layer by the previous call
  int pred_layer = -1;
  std::vector<int32_t> predicted;
};

namespace {

thread_local char g_tier_err[512] = "";

int tfail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_tier_err, sizeof g_tier_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return tfail(MOE_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCHK(call, what)                       \
  do {                                           \
    const hipError_t e_ = (call);                \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

uint64_t record_bytes_of(const moe_dims &d, uint64_t desc) {
  const int bits = moe::bits_of_tag(desc);
  return bits ? moe::record_layout(d.hidden, d.inter, bits).total : 0;
}

// A free slot, else the least recently used one whose record is not in
// `keep` (records this call needs resident); evicts its record.
int take_slot(moe_tier *t, const std::vector<int64_t> &keep) {
  int best = -1;
  for (int s = 0; s < t->cfg.n_slots; ++s) {
    if (t->owner[s] < 0) return s;
    if (std::find(keep.begin(), keep.end(), t->owner[s]) != keep.end()) continue;
    if (best < 0 || t->last_use[s] < t->last_use[best]) best = s;
  }
  if (best >= 0) t->slot_of[size_t(t->owner[best])] = -1;
  return best;
}

uint64_t slot_desc(const moe_tier *t, int slot, uint64_t host_desc) {
  return (t->cfg.slot_offset + uint64_t(slot) * t->cfg.slot_stride) | (host_desc & 3u);
}

// Copy record `rec` (l * E + e) from the host tier into `slot` on the copy
// stream and record the slot's landed event.
int fetch(moe_tier *t, int64_t rec, int slot, hipStream_t cs) {
  const uint64_t hd = t->cfg.host_desc[rec];
  const uint64_t bytes = record_bytes_of(t->cfg.dims, hd);
  const uint64_t src = hd & ~uint64_t(255);
  HIPCHK(hipMemcpyAsync(t->cfg.dev_pool + t->cfg.slot_offset + uint64_t(slot) * t->cfg.slot_stride,
                        t->cfg.host_tier + src, bytes, hipMemcpyHostToDevice, cs),
         "record copy");
  HIPCHK(hipEventRecord(t->landed[slot], cs), "landed event");
  t->owner[slot] = rec;
  t->slot_of[size_t(rec)] = slot;
  t->dirty[slot] = 1;
  return MOE_OK;
}

// The compute stream waits for the copies into these slots.
int wait_landed(moe_tier *t, const std::vector<int> &slots, hipStream_t s) {
  for (int sl : slots)
    if (t->dirty[sl]) {
      HIPCHK(hipStreamWaitEvent(s, t->landed[sl], 0), "wait for a copy");
      t->dirty[sl] = 0;
    }
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_tier_create(const moe_tier_config *cfg, moe_tier **out) {
  if (!cfg || !out) return tfail(MOE_EINVAL, "cfg or out is NULL");
  *out = nullptr;
  const moe_dims &d = cfg->dims;
  if (d.hidden < 256 || d.hidden % 256 || d.inter < 64 || d.inter % 64 || d.n_experts < 1 ||
      d.n_experts > 256 || d.top_k < 1 || d.top_k > 15 || d.top_k > d.n_experts)
    return tfail(MOE_EINVAL, "invalid dims");
  if (cfg->n_layers < 1) return tfail(MOE_EINVAL, "n_layers %d: must be >= 1", cfg->n_layers);
  if (!cfg->host_tier || !cfg->host_desc || !cfg->dev_pool) return tfail(MOE_EINVAL, "a tier pointer is NULL");
  if (cfg->slot_offset % 256 || cfg->slot_stride % 256 || reinterpret_cast<uintptr_t>(cfg->dev_pool) % 256)
    return tfail(MOE_EINVAL, "slot offset, stride and pool must be 256-byte aligned");
  if (cfg->slot_stride < moe::record_layout(d.hidden, d.inter, 4).total)
    return tfail(MOE_EINVAL, "slot stride %llu is below a 4-bit record", (unsigned long long)cfg->slot_stride);
  if (cfg->n_slots < d.top_k * MOE_MAX_NB)
    return tfail(MOE_EINVAL, "n_slots %d: must hold a whole union (k * MAX_NB = %d)", cfg->n_slots,
                 d.top_k * MOE_MAX_NB);
  if (cfg->slot_offset + uint64_t(cfg->n_slots) * cfg->slot_stride > cfg->dev_bytes)
    return tfail(MOE_EINVAL, "the slots run past the device pool");
  const size_t n_rec = size_t(cfg->n_layers) * d.n_experts;
  for (size_t r = 0; r < n_rec; ++r) {
    const uint64_t hd = cfg->host_desc[r];
    const uint64_t bytes = record_bytes_of(d, hd);
    if (!bytes || (hd & ~uint64_t(255)) + bytes > cfg->host_bytes)
      return tfail(MOE_EINVAL, "host record %zu: bad descriptor or outside the host tier", r);
  }
  moe_tier *t = new (std::nothrow) moe_tier();
  if (!t) return tfail(MOE_EINVAL, "out of host memory");
  t->cfg = *cfg;
  t->slot_of.assign(n_rec, -1);
  t->owner.assign(size_t(cfg->n_slots), -1);
  t->last_use.assign(size_t(cfg->n_slots), 0);
  t->dirty.assign(size_t(cfg->n_slots), 0);
  t->landed.assign(size_t(cfg->n_slots), nullptr);
  hipError_t e = hipSuccess;
  for (auto &ev : t->landed)
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&t->ev_route, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&t->ev_part0, hipEventDisableTiming);
  for (auto &ev : t->ev_t)
    if (e == hipSuccess) e = hipEventCreate(&ev);
  void *p = nullptr;
  const size_t staging = 64 * 4 + 4 * 64 * 4 + 2 * 64 * 8 + 2 * 4 * 64 * 4 + 64 * 4 + 64 * 4 + 64 * 8;
  if (e == hipSuccess) e = hipHostMalloc(&p, staging, hipHostMallocDefault);
  if (e != hipSuccess) {
    moe_tier_destroy(t);
    return hip_fail(e, "tier set-up");
  }
  uint8_t *b = static_cast<uint8_t *>(p);
  t->h_tab = reinterpret_cast<uint64_t *>(b);
  t->h_ids = reinterpret_cast<uint32_t *>(b + 2 * 64 * 8);
  t->h_wmap = reinterpret_cast<float *>(b + 2 * 64 * 8 + 64 * 4);
  t->h_wpub = t->h_wmap + 4 * 64;
  t->h_idpub = reinterpret_cast<uint32_t *>(t->h_wpub + 2 * 4 * 64);
  t->h_la_ids = t->h_idpub + 64;
  t->h_la_tab = reinterpret_cast<uint64_t *>(t->h_la_ids + 64);
  *out = t;
  return MOE_OK;
}

void moe_tier_destroy(moe_tier *t) {
  if (!t) return;
  for (auto &ev : t->landed)
    if (ev) (void)hipEventDestroy(ev);
  if (t->ev_route) (void)hipEventDestroy(t->ev_route);
  if (t->ev_part0) (void)hipEventDestroy(t->ev_part0);
  for (auto &ev : t->ev_t)
    if (ev) (void)hipEventDestroy(ev);
  if (t->h_tab) (void)hipHostFree(t->h_tab);
  delete t;
}

int moe_tier_warm(moe_tier *t, int32_t layer, const int32_t *experts, int32_t n, void *copy_stream) {
  if (!t) return tfail(MOE_EINVAL, "tier is NULL");
  const int E = t->cfg.dims.n_experts;
  if (layer < 0 || layer >= t->cfg.n_layers) return tfail(MOE_EINVAL, "layer %d out of range", layer);
  std::vector<int64_t> keep;
  for (int i = 0; i < n; ++i) {
    if (experts[i] < 0 || experts[i] >= E) return tfail(MOE_EINVAL, "expert %d out of range", experts[i]);
    const int64_t rec = int64_t(layer) * E + experts[i];
    if (t->slot_of[size_t(rec)] >= 0) continue;
    const int slot = take_slot(t, keep);
    if (slot < 0) return tfail(MOE_EINVAL, "no free slot");
    int rc = fetch(t, rec, slot, static_cast<hipStream_t>(copy_stream));
    if (rc) return rc;
    t->last_use[slot] = ++t->clock;
    keep.push_back(rec);
  }
  return MOE_OK;
}

int moe_tier_layer(moe_tier *t, int32_t layer, const float *x, int32_t nb, const moe_router *router,
                   moe_slots *slots, const moe_shared *shared, float *out, const moe_tier_policy *policy,
                   const moe_router *next_router, moe_slots *la_slots, moe_tier_stats *stats, void *stream,
                   void *copy_stream) {
  if (!t || !router || !slots || !shared || !stats) return tfail(MOE_EINVAL, "a required argument is NULL");
  if (layer < 0 || layer >= t->cfg.n_layers) return tfail(MOE_EINVAL, "layer %d out of range", layer);
  const moe_tier_policy pol = policy ? *policy : moe_tier_policy{};
  const bool lookahead = pol.lookahead && next_router && la_slots && layer + 1 < t->cfg.n_layers;
  const moe_dims &d = t->cfg.dims;
  if (std::memcmp(&router->dims, &d, sizeof d) != 0) return tfail(MOE_EINVAL, "router dims differ from the tier's");
  const int E = d.n_experts;
  hipStream_t s = static_cast<hipStream_t>(stream), cs = static_cast<hipStream_t>(copy_stream);
  *stats = moe_tier_stats{};
  const bool timing = pol.timing != 0;
  moe_pool pool{t->cfg.dev_pool, t->cfg.dev_bytes};

  // 1. router on the GPU; the CPU reads the union (the handshake)
  int rc = moe_route(x, nb, router, shared, slots, stream);
  if (rc) return tfail(rc, "route: %s", moe_last_error());
  HIPCHK(hipEventRecord(t->ev_route, s), "route event");
  HIPCHK(hipMemcpyAsync(t->h_ids, slots->ids, 64 * 4, hipMemcpyDeviceToHost, s), "ids read-back");
  HIPCHK(hipMemcpyAsync(t->h_wmap, slots->wmap, 4 * 64 * 4, hipMemcpyDeviceToHost, s), "wmap read-back");
  HIPCHK(hipMemcpyAsync(t->h_tab + 64, slots->tab, 64 * 8, hipMemcpyDeviceToHost, s), "tab read-back");
  HIPCHK(hipStreamSynchronize(s), "route wait");
  const int n_u = int(std::min<uint64_t>(t->h_tab[64 + MOE_UNION_ENTRY], MOE_RESIDENT_ENTRY));
  stats->n_union = n_u;
  // lookahead hits: experts of this layer that the previous call predicted
  if (t->pred_layer == layer) {
    stats->n_predicted = int32_t(t->predicted.size());
    for (int j = 0; j < n_u; ++j)
      if (std::find(t->predicted.begin(), t->predicted.end(), int32_t(t->h_ids[j])) != t->predicted.end())
        ++stats->n_hit;
  }

  // 2. residency: resident records first, then the misses (union order)
  std::vector<int> res, miss;   // union slot indices
  std::vector<int64_t> keep;
  for (int j = 0; j < n_u; ++j) {
    const int64_t rec = int64_t(layer) * E + t->h_ids[j];
    keep.push_back(rec);
    if (t->slot_of[size_t(rec)] >= 0) res.push_back(j);
    else miss.push_back(j);
  }
  // misses in order of their largest weight over the rows (strong first: the
  // copies land in that order, so a deadline cut drops the weakest)
  auto wmax = [&](int j) {
    float m = 0.0f;
    for (int b = 0; b < nb; ++b) m = std::max(m, t->h_wmap[b * 64 + j]);
    return m;
  };
  std::stable_sort(miss.begin(), miss.end(), [&](int a, int b) { return wmax(a) > wmax(b); });
  std::vector<int> order = res;
  order.insert(order.end(), miss.begin(), miss.end());
  std::vector<int> dev_slot(size_t(n_u), -1);
  std::vector<int> res_slots;
  for (int j : res) {
    const int sl = t->slot_of[size_t(int64_t(layer) * E + t->h_ids[j])];
    dev_slot[size_t(j)] = sl;
    t->last_use[sl] = ++t->clock;
    res_slots.push_back(sl);
  }
  for (int j : miss) {
    const int sl = take_slot(t, keep);
    if (sl < 0) return tfail(MOE_EINVAL, "no slot left for a missing record");
    dev_slot[size_t(j)] = sl;
    t->last_use[sl] = ++t->clock;
    t->owner[sl] = int64_t(layer) * E + t->h_ids[j];   // reserved (copied below)
    t->slot_of[size_t(t->owner[sl])] = sl;
  }
  // the published table: tab / wmap / ids in published order
  auto publish = [&](int which, const std::vector<int> &ord, int n_res) {
    uint64_t *tab = t->h_tab + 64 * which;
    float *w = t->h_wpub + 4 * 64 * which;
    std::memset(tab, 0, 64 * 8);
    std::memset(w, 0, 4 * 64 * 4);
    for (size_t q = 0; q < ord.size(); ++q) {
      const int j = ord[q];
      const int64_t rec = int64_t(layer) * E + t->h_ids[j];
      tab[q] = slot_desc(t, dev_slot[size_t(j)], t->cfg.host_desc[rec]);
      for (int b = 0; b < nb; ++b) w[b * 64 + q] = t->h_wmap[b * 64 + j];
      if (which == 0) t->h_idpub[q] = t->h_ids[j];
    }
    if (which == 0)
      for (size_t q = ord.size(); q < 64; ++q) t->h_idpub[q] = 0;
    tab[MOE_RESIDENT_ENTRY] = uint64_t(n_res);
    tab[MOE_UNION_ENTRY] = uint64_t(ord.size());
  };
  publish(0, order, int(res.size()));
  stats->n_resident = int32_t(res.size());
  stats->n_fetched = int32_t(miss.size());

  // 3. part 0 (resident records + shared expert) as published; the copies
  // of the misses run meanwhile (after the route: no kernel still reads a
  // victim slot then)
  HIPCHK(hipMemcpyAsync(slots->tab, t->h_tab, 64 * 8, hipMemcpyHostToDevice, s), "table publish");
  HIPCHK(hipMemcpyAsync(slots->wmap, t->h_wpub, 4 * 64 * 4, hipMemcpyHostToDevice, s), "wmap publish");
  HIPCHK(hipMemcpyAsync(slots->ids, t->h_idpub, 64 * 4, hipMemcpyHostToDevice, s), "ids publish");
  if ((rc = wait_landed(t, res_slots, s))) return rc;   // resident but still landing (prefetches)
  if (timing) HIPCHK(hipEventRecord(t->ev_t[0], s), "timing event");
  rc = moe_experts_part(x, nb, &d, slots, 0, &pool, shared, out, stream);
  if (rc) return tfail(rc, "part 0: %s", moe_last_error());
  if (timing) HIPCHK(hipEventRecord(t->ev_t[1], s), "timing event");
  HIPCHK(hipEventRecord(t->ev_part0, s), "part 0 event");
  if (!miss.empty()) {
    HIPCHK(hipStreamWaitEvent(cs, t->ev_route, 0), "copy stream wait");
    if (timing) HIPCHK(hipEventRecord(t->ev_t[2], cs), "timing event");
    for (int j : miss)
      if ((rc = fetch(t, int64_t(layer) * E + t->h_ids[j], dev_slot[size_t(j)], cs))) return rc;
    if (timing) HIPCHK(hipEventRecord(t->ev_t[3], cs), "timing event");
  }

  // the lookahead for the next layer: its router on this layer's input,
  // predicted records fetched into free or least recently used slots
  if (lookahead) {
    rc = moe_route(x, nb, next_router, shared, la_slots, stream);
    if (rc) return tfail(rc, "lookahead route: %s", moe_last_error());
    HIPCHK(hipMemcpyAsync(t->h_la_ids, la_slots->ids, 64 * 4, hipMemcpyDeviceToHost, s), "lookahead read-back");
    HIPCHK(hipMemcpyAsync(t->h_la_tab, la_slots->tab, 64 * 8, hipMemcpyDeviceToHost, s), "lookahead read-back");
  }

  // 4. the deadline (part 0 done): late weak records are cut
  std::vector<int> late = miss;
  if (pol.cut_w > 0.0f && !miss.empty()) {
    HIPCHK(hipEventSynchronize(t->ev_part0), "deadline wait");
    std::vector<int> kept;
    for (int j : miss) {
      const int sl = dev_slot[size_t(j)];
      const bool landed_now = !pol.deadline_now && hipEventQuery(t->landed[sl]) == hipSuccess;
      if (!landed_now && wmax(j) < pol.cut_w) {
        ++stats->n_cut;   // its copy completes in the background; the record stays resident
        continue;
      }
      kept.push_back(j);
    }
    late = kept;
    std::vector<int> ord2 = res;
    ord2.insert(ord2.end(), kept.begin(), kept.end());
    publish(1, ord2, int(res.size()));
    HIPCHK(hipMemcpyAsync(slots->tab, t->h_tab + 64, 64 * 8, hipMemcpyHostToDevice, s), "table republish");
    HIPCHK(hipMemcpyAsync(slots->wmap, t->h_wpub + 4 * 64, 4 * 64 * 4, hipMemcpyHostToDevice, s),
           "wmap republish");
  }
  // part 1: the fetched records, once landed
  if (!late.empty()) {
    std::vector<int> late_slots;
    for (int j : late) late_slots.push_back(dev_slot[size_t(j)]);
    if ((rc = wait_landed(t, late_slots, s))) return rc;
    rc = moe_experts_part(x, nb, &d, slots, 1, &pool, shared, out, stream);
    if (rc) return tfail(rc, "part 1: %s", moe_last_error());
  }
  if (timing) {
    HIPCHK(hipStreamSynchronize(s), "timing wait");
    float ms = 0.0f;
    HIPCHK(hipEventElapsedTime(&ms, t->ev_t[0], t->ev_t[1]), "timing");
    stats->part0_us = ms * 1e3f;
    if (!miss.empty()) {
      HIPCHK(hipStreamSynchronize(cs), "timing wait");
      HIPCHK(hipEventElapsedTime(&ms, t->ev_t[2], t->ev_t[3]), "timing");
      stats->fetch_us = ms * 1e3f;
    }
  }

  // the lookahead's predicted records: fetched after this layer's own copies
  if (lookahead) {
    HIPCHK(hipStreamSynchronize(s), "lookahead wait");
    const int n_p = int(std::min<uint64_t>(t->h_la_tab[MOE_UNION_ENTRY], MOE_RESIDENT_ENTRY));
    t->predicted.assign(t->h_la_ids, t->h_la_ids + n_p);
    t->pred_layer = layer + 1;
    std::vector<int64_t> keep_next;
    for (int j = 0; j < n_p; ++j) keep_next.push_back(int64_t(layer + 1) * E + t->h_la_ids[j]);
    keep_next.insert(keep_next.end(), keep.begin(), keep.end());
    for (int j = 0; j < n_p; ++j) {
      const int64_t rec = int64_t(layer + 1) * E + t->h_la_ids[j];
      if (t->slot_of[size_t(rec)] >= 0) continue;
      const int sl = take_slot(t, keep_next);
      if (sl < 0) break;
      if ((rc = fetch(t, rec, sl, cs))) return rc;
      t->last_use[sl] = ++t->clock;
      ++stats->n_prefetched;
    }
  } else {
    t->pred_layer = -1;
  }
  return MOE_OK;
}

int moe_tier_join(moe_tier *t, void *stream) {
  if (!t) return tfail(MOE_EINVAL, "tier is NULL");
  std::vector<int> all;
  for (int s = 0; s < t->cfg.n_slots; ++s) all.push_back(s);
  return wait_landed(t, all, static_cast<hipStream_t>(stream));
}

const char *moe_tier_last_error(void) { return g_tier_err; }

}  // extern "C"
