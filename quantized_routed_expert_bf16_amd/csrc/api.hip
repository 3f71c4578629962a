// C ABI of the MoE library: host-side validation, workspace layout, launches.
//
// The shape checks mirror load.rs load_bounded: hidden % 256 == 0, expert
// width a multiple of the 64-code group, k * MAX_NB below the 64-entry slot
// table; the row limits are gpu.rs MAX_NB (decode) and a 32-row prefill tile.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "moe_internal.h"

// The scratch of moe_layer_forward_noalloc: the decode kernel's exchange
// buffers (counters, epoch-tagged act values and slice partials, router
// logits) for callers that cannot allocate.  Each GPU the library runs on
// holds one copy until the process ends.  Host code never uses this name as
// an address: the device address of each GPU's copy comes from
// hipGetSymbolAddress (scratch_on_device below).
constexpr size_t kStaticScratchBytes = size_t(3) << 20;   // 3 MiB
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace moe {

static thread_local char g_err[512] = "";

static int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

static int ok() {
  g_err[0] = 0;
  return MOE_OK;
}

static bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

static bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

static int check_dims(const moe_dims *d) {
  if (!d) return fail(MOE_EINVAL, "dims is NULL");
  if (d->hidden < 256 || d->hidden > 4096 || d->hidden % 256)
    return fail(MOE_EINVAL, "hidden %d: must be a multiple of 256 in 256..4096", d->hidden);
  if (!pow2(d->inter) || d->inter < 64 || d->inter > 2048)
    return fail(MOE_EINVAL, "inter %d: expert width must be a power of two in 64..2048 "
                "(a multiple of the 64-code quantization group)", d->inter);
  if (d->n_experts < 1 || d->n_experts > kMaxExperts)
    return fail(MOE_EINVAL, "n_experts %d: must be in 1..%d", d->n_experts, kMaxExperts);
  if (d->top_k < 1 || d->top_k > kMaxTopK || d->top_k > d->n_experts)
    return fail(MOE_EINVAL, "top_k %d: must be in 1..%d and <= n_experts (slot table too narrow)",
                d->top_k, kMaxTopK);
  return MOE_OK;
}

#define REQ(p, a, name)                                                              \
  do {                                                                               \
    if (!(p)) return fail(MOE_EINVAL, "%s is NULL", name);                           \
    if (!aligned((p), (a))) return fail(MOE_EINVAL, "%s is not %d-byte aligned", name, int(a)); \
  } while (0)

WorkspaceLayout workspace_layout(int hidden, int inter, int n_experts, int top_k, int rows) {
  (void)n_experts;
  WorkspaceLayout w;
  size_t pos = 0;
  auto take = [&](size_t bytes) {
    const size_t at = pos;
    pos = align256(pos + bytes);
    return at;
  };
  const int pf_rows = rows > MOE_MAX_NB ? rows : MOE_MAX_NB;
  w.counters = take(kSyncWords * sizeof(uint32_t));
  w.act = take(size_t(kSlotStride) * kMaxNb * inter * sizeof(uint64_t));
  w.opart = take(size_t(kSlices) * kMaxNb * hidden * sizeof(uint64_t));
  w.slice_logits = take(size_t(kSlices) * kMaxNb * kMaxExperts * sizeof(double) +
                        size_t(kSlices) * kMaxNb * sizeof(float));
  w.pf_xf = take(size_t(4) * MOE_MAX_PREFILL_ROWS * hidden * sizeof(_Float16));
  w.pf_xg = take(size_t(MOE_MAX_PREFILL_ROWS) * (hidden / kGroup) * sizeof(float));
  w.pf_act_rows = pf_rows * (top_k + 1);
  w.pf_act = take(size_t(2) * w.pf_act_rows * inter * sizeof(_Float16));
  w.pf_asum = take(size_t(w.pf_act_rows) * (inter / 32) * sizeof(float));
  w.pf_y = take(size_t(pf_rows) * (top_k + 1) * hidden * sizeof(float));
  w.pf_meta = take(size_t(kJobInts) * (1 + 2 * kMaxExperts + 2) * sizeof(int32_t));
  w.total = pos;
  return w;
}

static int check_router(const moe_router *r) {
  if (!r) return fail(MOE_EINVAL, "router is NULL");
  int rc = check_dims(&r->dims);
  if (rc) return rc;
  REQ(r->weight, 16, "router.weight");
  REQ(r->rec, 8, "router.rec");
  return MOE_OK;
}

static int check_shared(const moe_shared *sh, const moe_dims &d, const moe_pool *pool) {
  if (!sh) return fail(MOE_EINVAL, "shared is NULL");
  REQ(sh->gate, 16, "shared.gate");
  if (pool) {
    if ((sh->rec & 255) != 0)
      return fail(MOE_EINVAL, "shared.rec: the shared expert must be a 4-bit record (tag 0) "
                  "at a 256-byte aligned offset");
    const uint64_t need = record_layout(d.hidden, d.inter, 4).total;
    if (sh->rec > pool->bytes || pool->bytes - sh->rec < need)
      return fail(MOE_EINVAL, "shared.rec: record at %llu (+%llu bytes) lies outside the %llu-byte pool",
                  (unsigned long long)sh->rec, (unsigned long long)need,
                  (unsigned long long)pool->bytes);
  }
  return MOE_OK;
}

static int check_pool(const moe_pool *p) {
  if (!p) return fail(MOE_EINVAL, "pool is NULL");
  REQ(p->base, 256, "pool.base");
  if (p->bytes == 0) return fail(MOE_EINVAL, "pool.bytes is 0");
  return MOE_OK;
}

static int check_ws(void *ws, size_t ws_bytes, const moe_dims &d, int rows) {
  if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_EINVAL, "workspace is not 256-byte aligned");
  const size_t need = workspace_layout(d.hidden, d.inter, d.n_experts, d.top_k, rows).total;
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return MOE_OK;
}

static thread_local hipEvent_t g_stage_ev[8] = {};
static thread_local int g_stage_n = 0;

static int launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MOE_ELAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

// Records the profiling event of stage i (if any) after that stage's launch.
static int stage_done(int i, hipStream_t s) {
  if (i < g_stage_n && g_stage_ev[i]) {
    const hipError_t e = hipEventRecord(g_stage_ev[i], s);
    if (e != hipSuccess) return fail(MOE_ELAUNCH, "stage event %d: %s", i, hipGetErrorString(e));
  }
  return MOE_OK;
}

static int check_slot_tables(const moe_slots *s) {
  if (!s) return fail(MOE_EINVAL, "slots is NULL");
  REQ(s->tab, 8, "slots.tab");
  REQ(s->wmap, 4, "slots.wmap");
  REQ(s->ids, 4, "slots.ids");
  REQ(s->topk_idx, 4, "slots.topk_idx");
  REQ(s->topk_w, 4, "slots.topk_w");
  REQ(s->logits, 8, "slots.logits");
  REQ(s->gamma, 4, "slots.gamma");
  return MOE_OK;
}

static int check_slots(const moe_slots *s, const moe_dims &d, int nb) {
  const int rc = check_slot_tables(s);
  if (rc) return rc;
  return check_ws(s->ws, s->ws_bytes, d, nb);
}

// Bytes of the decode sections at the head of the workspace (counters, act,
// slice partials, router logits): the prefill sections start after them.
static size_t decode_ws_bytes(const moe_dims &d, int nb) {
  return workspace_layout(d.hidden, d.inter, d.n_experts, d.top_k, nb).pf_xf;
}

// Checks shared by moe_layer_forward and moe_layer_forward_noalloc (all but
// the workspace).
static int check_forward(const float *x, int nb, const moe_router *router, const moe_slots *slots,
                         const moe_pool *pool, const moe_shared *shared, const float *out) {
  int rc = check_router(router);
  if (rc) return rc;
  const moe_dims &d = router->dims;
  if (nb < 1 || nb > MOE_MAX_NB) return fail(MOE_EINVAL, "nb %d: must be in 1..%d", nb, MOE_MAX_NB);
  REQ(x, 16, "x");
  REQ(out, 16, "out");
  if ((rc = check_pool(pool))) return rc;
  if ((rc = check_shared(shared, d, pool))) return rc;
  return check_slot_tables(slots);
}


// The decode launch description shared by moe_route (no pool, no output),
// moe_layer_forward and moe_layer_forward_noalloc (ws = the workspace or the
// static scratch); arguments were validated by the caller.
static LayerLaunch layer_launch(const float *x, int nb, const moe_router *router, const moe_slots *slots,
                                const moe_pool *pool, const moe_shared *shared, float *out, uint8_t *ws) {
  const moe_dims &d = router->dims;
  const WorkspaceLayout L = workspace_layout(d.hidden, d.inter, d.n_experts, d.top_k, nb);
  LayerLaunch l{};
  l.x = x;
  l.nb = nb;
  l.router = router->weight;
  l.gvec = shared->gate;
  l.rec = router->rec;
  l.pool = pool ? pool->base : nullptr;
  l.pool_bytes = pool ? pool->bytes : 0;
  l.shared_rec = shared->rec;
  l.hidden = d.hidden;
  l.inter = d.inter;
  l.n_experts = d.n_experts;
  l.top_k = d.top_k;
  l.logits = slots->logits;
  l.gamma = slots->gamma;
  l.topk_idx = slots->topk_idx;
  l.topk_w = slots->topk_w;
  l.tab = slots->tab;
  l.wmap = slots->wmap;
  l.ids = slots->ids;
  l.out = out;
  l.sync = reinterpret_cast<uint32_t *>(ws + L.counters);
  l.act = reinterpret_cast<uint64_t *>(ws + L.act);
  l.opart = reinterpret_cast<uint64_t *>(ws + L.opart);
  l.slice_logits = reinterpret_cast<double *>(ws + L.slice_logits);
  l.slice_gamma = reinterpret_cast<float *>(ws + L.slice_logits +
                                            size_t(kSlices) * kMaxNb * kMaxExperts * sizeof(double));
  return l;
}

// Device address of this GPU's copy of `scratch`, looked up (and the copy
// zero-filled on `s`) on the first call on each device.  Under a lock: the
// lookup and the fill happen once per device.
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static uint8_t *g_scratch_ptr[kMaxDevices] = {};

static int scratch_on_device(hipStream_t s, uint8_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ELAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EINVAL, "device %d: above %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ELAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    // counters start at zero and no act value carries an epoch tag yet
    e = launch_fill_zero(p, kStaticScratchBytes, s);
    if (e != hipSuccess) return fail(MOE_ELAUNCH, "scratch fill on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<uint8_t *>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// The copy of `scratch` on the current device, if a call has set it up.
static uint8_t *scratch_if_set_up() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[dev];
}

}  // namespace moe

using namespace moe;

extern "C" {

uint64_t moe_record_bytes(int32_t hidden, int32_t inter, int32_t bits) {
  if (bits != 4 && bits != 3 && bits != 2) return 0;
  moe_dims d{hidden, inter, 1, 1};
  if (check_dims(&d)) return 0;
  return record_layout(hidden, inter, bits).total;
}

size_t moe_workspace_bytes(const moe_dims *dims, int32_t max_rows) {
  if (check_dims(dims)) return 0;
  if (max_rows < 1 || max_rows > MOE_MAX_PREFILL_ROWS) return 0;
  return workspace_layout(dims->hidden, dims->inter, dims->n_experts, dims->top_k, max_rows).total;
}

int moe_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256) || ws_bytes % 256)
    return fail(MOE_EINVAL, "workspace must be 256-byte aligned with a size multiple of 256");
  const int rc = launched(launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)), "fill");
  return rc ? rc : ok();
}

int moe_route(const float *x, int32_t nb, const moe_router *router, const moe_shared *shared,
              moe_slots *slots, void *stream) {
  int rc = check_router(router);
  if (rc) return rc;
  const moe_dims &d = router->dims;
  if (nb < 1 || nb > MOE_MAX_NB) return fail(MOE_EINVAL, "nb %d: must be in 1..%d", nb, MOE_MAX_NB);
  REQ(x, 16, "x");
  if ((rc = check_shared(shared, d, nullptr))) return rc;
  if ((rc = check_slots(slots, d, nb))) return rc;
  const LayerLaunch l =
      layer_launch(x, nb, router, slots, nullptr, shared, nullptr, static_cast<uint8_t *>(slots->ws));
  rc = launched(launch_route_only(l, static_cast<hipStream_t>(stream)), "route");
  return rc ? rc : ok();
}

int moe_layer_forward(const float *x, int32_t nb, const moe_router *router, moe_slots *slots,
                      const moe_pool *pool, const moe_shared *shared, float *out, void *stream) {
  int rc = check_forward(x, nb, router, slots, pool, shared, out);
  if (rc) return rc;
  if ((rc = check_ws(slots->ws, slots->ws_bytes, router->dims, nb))) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const LayerLaunch l = layer_launch(x, nb, router, slots, pool, shared, out, static_cast<uint8_t *>(slots->ws));
  if ((rc = launched(launch_layer(l, s), "layer"))) return rc;
  if ((rc = stage_done(0, s))) return rc;
  return ok();
}

int moe_layer_forward_noalloc(const float *x, int32_t nb, const moe_router *router, moe_slots *slots,
                              const moe_pool *pool, const moe_shared *shared, float *out, void *stream) {
  int rc = check_forward(x, nb, router, slots, pool, shared, out);
  if (rc) return rc;
  if (slots->ws || slots->ws_bytes)
    return fail(MOE_EINVAL, "slots.ws must be NULL and slots.ws_bytes 0: moe_layer_forward_noalloc "
                "uses the library's static scratch");
  const size_t need = decode_ws_bytes(router->dims, nb);
  if (need > kStaticScratchBytes)
    return fail(MOE_EWORKSPACE, "these dims need %zu bytes of decode scratch, above the %zu-byte static "
                "scratch of moe_layer_forward_noalloc (use moe_layer_forward with a workspace)",
                need, kStaticScratchBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *ws = nullptr;
  if ((rc = scratch_on_device(s, &ws))) return rc;
  const LayerLaunch l = layer_launch(x, nb, router, slots, pool, shared, out, ws);
  if ((rc = launched(launch_layer(l, s), "layer"))) return rc;
  if ((rc = stage_done(0, s))) return rc;
  return ok();
}

int moe_prefill_forward(const float *x, int32_t t, const moe_router *router, moe_prefill_plan *plan,
                        const moe_pool *pool, const moe_shared *shared, float *out, void *stream) {
  int rc = check_router(router);
  if (rc) return rc;
  const moe_dims &d = router->dims;
  if (t < 1 || t > MOE_MAX_PREFILL_ROWS)
    return fail(MOE_EINVAL, "t %d: must be in 1..%d", t, MOE_MAX_PREFILL_ROWS);
  REQ(x, 16, "x");
  REQ(out, 16, "out");
  if ((rc = check_pool(pool))) return rc;
  if ((rc = check_shared(shared, d, pool))) return rc;
  if (!plan) return fail(MOE_EINVAL, "plan is NULL");
  REQ(plan->topk_idx, 4, "plan.topk_idx");
  REQ(plan->topk_w, 4, "plan.topk_w");
  REQ(plan->logits, 8, "plan.logits");
  REQ(plan->gamma, 4, "plan.gamma");
  REQ(plan->expert_ptr, 4, "plan.expert_ptr");
  REQ(plan->entry_row, 4, "plan.entry_row");
  REQ(plan->entry_rank, 4, "plan.entry_rank");
  if ((rc = check_ws(plan->ws, plan->ws_bytes, d, t))) return rc;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const WorkspaceLayout L = workspace_layout(d.hidden, d.inter, d.n_experts, d.top_k, t);
  uint8_t *ws = static_cast<uint8_t *>(plan->ws);
  PrefillArgs pa{};
  pa.pool = pool->base;
  pa.pool_bytes = pool->bytes;
  pa.x = x;
  pa.rec = router->rec;
  pa.shared_rec = shared->rec;
  pa.topk_idx = plan->topk_idx;
  pa.expert_ptr = plan->expert_ptr;
  pa.entry_row = plan->entry_row;
  pa.entry_rank = plan->entry_rank;
  pa.topk_w = plan->topk_w;
  pa.gamma = plan->gamma;
  pa.hidden = d.hidden;
  pa.inter = d.inter;
  pa.n_experts = d.n_experts;
  pa.top_k = d.top_k;
  pa.t = t;
  pa.xf = reinterpret_cast<_Float16 *>(ws + L.pf_xf);
  pa.xg = reinterpret_cast<float *>(ws + L.pf_xg);
  pa.act = reinterpret_cast<_Float16 *>(ws + L.pf_act);
  pa.asum = reinterpret_cast<float *>(ws + L.pf_asum);
  pa.act_rows = L.pf_act_rows;
  pa.y = reinterpret_cast<float *>(ws + L.pf_y);
  pa.meta = reinterpret_cast<int32_t *>(ws + L.pf_meta);
  pa.status = reinterpret_cast<uint32_t *>(ws + L.counters) + kSyncStatus;
  pa.out = out;
  rc = launched(launch_prefill(pa, router->weight, shared->gate, plan->logits, plan->gamma,
                               plan->topk_idx, s, g_stage_ev, g_stage_n),
                "prefill");
  return rc ? rc : ok();
}

int moe_experts_part(const float *x, int32_t nb, const moe_dims *dims, moe_slots *slots, int32_t part,
                     const moe_pool *pool, const moe_shared *shared, float *out, void *stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (nb < 1 || nb > MOE_MAX_NB) return fail(MOE_EINVAL, "nb %d: must be in 1..%d", nb, MOE_MAX_NB);
  if (part != 0 && part != 1) return fail(MOE_EINVAL, "part %d: must be 0 or 1", part);
  REQ(x, 16, "x");
  REQ(out, 16, "out");
  if ((rc = check_pool(pool))) return rc;
  if ((rc = check_shared(shared, *dims, pool))) return rc;
  if (!slots) return fail(MOE_EINVAL, "slots is NULL");
  REQ(slots->tab, 8, "slots.tab");
  REQ(slots->wmap, 4, "slots.wmap");
  REQ(slots->gamma, 4, "slots.gamma");
  if ((rc = check_ws(slots->ws, slots->ws_bytes, *dims, nb))) return rc;
  moe_router r{};
  r.dims = *dims;   // the router itself is not read: the table is published
  const LayerLaunch l = layer_launch(x, nb, &r, slots, pool, shared, out, static_cast<uint8_t *>(slots->ws));
  rc = launched(launch_layer(l, static_cast<hipStream_t>(stream), part), "experts part");
  return rc ? rc : ok();
}

int moe_repack(const uint8_t *src_pool, uint64_t src_bytes, const uint64_t *src_desc, uint8_t *dst_pool,
               uint64_t dst_bytes, const uint64_t *dst_desc, int32_t n_records, int32_t hidden, int32_t inter,
               uint32_t *status, void *stream) {
  moe_dims d{hidden, inter, 1, 1};
  int rc = check_dims(&d);
  if (rc) return rc;
  if (n_records < 0) return fail(MOE_EINVAL, "n_records %d: must be >= 0", n_records);
  if (n_records == 0) return ok();
  REQ(src_pool, 256, "src_pool");
  REQ(dst_pool, 256, "dst_pool");
  REQ(src_desc, 8, "src_desc");
  REQ(dst_desc, 8, "dst_desc");
  if (status && !aligned(status, 4)) return fail(MOE_EINVAL, "status is not 4-byte aligned");
  rc = launched(launch_repack(src_pool, src_bytes, src_desc, dst_pool, dst_bytes, dst_desc, n_records, hidden,
                              inter, status, static_cast<hipStream_t>(stream)),
                "repack");
  return rc ? rc : ok();
}

int moe_workspace_status(void *ws, size_t ws_bytes, void *stream) {
  if (!ws && ws_bytes == 0) {   // the static scratch of moe_layer_forward_noalloc on this device
    ws = scratch_if_set_up();
    if (!ws) return fail(MOE_EWORKSPACE, "no moe_layer_forward_noalloc call has run on this device");
    ws_bytes = kStaticScratchBytes;
  }
  if (!ws || ws_bytes < kSyncWords * sizeof(uint32_t)) return fail(MOE_EWORKSPACE, "workspace is NULL or too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t *word = static_cast<uint32_t *>(ws) + kSyncStatus;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, word, sizeof v, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  const uint32_t zero = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(word, &zero, sizeof zero, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(MOE_ELAUNCH, "status read failed: %s", hipGetErrorString(e));
  ok();
  return int(v & 0x7fffffff);
}

int moe_set_stage_events(void *const *events, int32_t n) {
  if (n < 0 || n > 8) return fail(MOE_EINVAL, "stage events: n %d must be in 0..8", n);
  if (n > 0 && !events) return fail(MOE_EINVAL, "stage events: events is NULL");
  for (int i = 0; i < 8; ++i) g_stage_ev[i] = i < n ? static_cast<hipEvent_t>(events[i]) : nullptr;
  g_stage_n = n;
  return ok();
}

const char *moe_last_error(void) { return g_err; }

}  // extern "C"
