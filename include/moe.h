/*
 * moe.h -- C ABI of the routed-expert MoE layer for MI355X (gfx950).
 *
 * One MoE FFN step of a quantized decode engine: a bf16 router matvec with
 * top-k softmax per row, the first-seen union of the rows' experts written to
 * a 64-entry slot table of record descriptors, per union expert an affine
 * low-bit gate/up matvec fused with silu(gate)*up, the down matvec, and a
 * routing-weighted combine with a sigmoid-gated shared expert.  The method is
 * the one the qwen4_exp GPU engine pages describe: "Struct Gpu" (methods
 * router_b, experts_b, prepare_expert_jobs, pf_experts, encode_block), the
 * gpu.rs source page (struct Q, struct Moe, MAX_NB, SLOT_STRIDE, union_of, the
 * slot_tab/wmap field docs) and the gpu/load.rs source page (load_bounded:
 * shape checks, Moe descriptors, low-bit store kinds).
 *
 * Conventions for every entry point
 *   - Data pointers marked "device" are HIP device memory owned by the caller;
 *     the library never allocates, frees or keeps them after the call returns.
 *   - Struct arguments are host memory, read during the call only.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns without synchronising.
 *   - Arguments are validated on the host before any HIP call.  A failed
 *     check returns MOE_EINVAL or MOE_EWORKSPACE and nothing is enqueued; a
 *     failed launch returns MOE_ELAUNCH.  moe_last_error() gives the text of
 *     the last failure on the calling thread.
 *   - Activations are row-major [rows][...] f32 (the pages' [nb][...] layout).
 *   - Results are deterministic: no floating-point atomics, fixed summation
 *     order; two identical calls give identical bits.
 *
 * Shapes (checks mirror load.rs load_bounded)
 *   hidden H      multiple of 256, 256..4096          (hidden % 256 == 0)
 *   inter  I      power of two, 64..2048              (multiple of the 64-code group)
 *   n_experts E   1..256
 *   top_k  k      1..15 and k <= E                    (k * MAX_NB < SLOT_STRIDE)
 *   nb            1..4 rows per decode step            (MAX_NB = 4)
 *   t             1..32 rows per prefill chunk
 *
 * Record layout (one expert = one record in the byte pool; each section
 * starts on a 256-byte boundary, in this order):
 *   GU codes  2I rows x H codes; row 2j = gate row j, row 2j+1 = up row j
 *   GU sb     2I rows x H/64 words: (scale, bias) bf16 pair per 64-code group
 *   D codes   group-major: I/64 column groups, each H rows, each row's 64
 *             codes of that group packed like a 64-code row
 *   D sb      group-major: I/64 column groups, each H words
 *   An sb word holds the bf16 bits of the scale in its low half and of the
 *   bias in its high half; w = q * scale + bias.
 *   Codes, packed into little-endian u32 words, first code in the lowest bits:
 *     4-bit: 8 per word;  2-bit: 16 per word;
 *     3-bit: a row is a 2-bit plane of (q & 3) (n/4 bytes) followed by a 1-bit
 *            plane of (q >> 2) (n/8 bytes); inside each 32-code block, the
 *            high bit of code i (m = i/16, k = (i/4)%4, p = i%4) is bit
 *            8k + 4m + p of the block's u32 word.
 *   Descriptor: u64 = byte offset of the record in the pool (multiple of 256)
 *   | tag, tag 0 = 4-bit, 1 = 3-bit, 2 = 2-bit (the load.rs low-bit kinds).
 *   Record bytes: 4-bit 1,769,472 / 3-bit 1,376,256 / 2-bit 983,040 at
 *   H = 2048, I = 512 (moe_record_bytes).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_NB 4         /* rows per decode step (gpu.rs MAX_NB) */
#define MOE_SLOT_STRIDE 64   /* slot table entries per layer (gpu.rs SLOT_STRIDE) */
#define MOE_RESIDENT_ENTRY 62
#define MOE_UNION_ENTRY 63
#define MOE_MAX_PREFILL_ROWS 32

enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,       /* bad shape, count, pointer or alignment */
    MOE_EWORKSPACE = -2,   /* workspace missing or too small */
    MOE_ELAUNCH = -3,      /* a kernel launch failed (HIP error text in moe_last_error) */
};

typedef struct moe_dims {
    int32_t hidden;      /* H */
    int32_t inter;       /* I, routed and shared expert width (load.rs requires equal) */
    int32_t n_experts;   /* E */
    int32_t top_k;       /* k */
} moe_dims;

/* One layer's router (gpu.rs Moe.router: the bf16 mlp.gate.weight) and the
 * descriptors of that layer's routed expert records. */
typedef struct moe_router {
    moe_dims dims;
    const uint16_t *weight;   /* device, bf16 [E][H], 16-byte aligned */
    const uint64_t *rec;      /* device, [E] record descriptors (u64) */
} moe_router;

/* The byte pool holding every record. */
typedef struct moe_pool {
    const uint8_t *base;      /* device, 256-byte aligned */
    uint64_t bytes;           /* size of the pool; records must lie inside */
} moe_pool;

/* The shared expert (load.rs Moe: shared_expert_gate.weight and the shared
 * gate/up/down projections); always 4-bit (the pages keep every dense
 * projection at 4 bits when routed experts go to 3 or 2). */
typedef struct moe_shared {
    const uint16_t *gate;     /* device, bf16 [H] sigmoid gate vector, 16-byte aligned */
    uint64_t rec;             /* descriptor of its 4-bit record, tag 0 */
} moe_shared;

/* Routing results of one decode step (device buffers, written by the call). */
typedef struct moe_slots {
    uint64_t *tab;        /* [64]: tab[j] = descriptor of union expert j for j < |U|,
                             0 for |U| <= j < 62, tab[62] = resident count (= |U|:
                             every record is in device memory), tab[63] = |U| */
    float    *wmap;       /* [4][64]: routing weight of union slot j in row b, else 0 */
    uint32_t *ids;        /* [64]: expert id of union slot j (first-seen order), else 0 */
    uint32_t *topk_idx;   /* [nb][k]: per row, experts by descending logit (ties: lower id) */
    float    *topk_w;     /* [nb][k]: softmax over the k selected logits */
    double   *logits;     /* [nb][E]: router logits, f64 accumulation */
    float    *gamma;      /* [nb]: shared-expert gate sigmoid(gvec . x) */
    void     *ws;         /* workspace, >= moe_workspace_bytes(dims, nb); must be
                             zero-filled once after allocation (moe_workspace_init);
                             every call leaves its counter words zero again */
    size_t    ws_bytes;
} moe_slots;

/* Routing results of one prefill chunk, rows grouped by expert (Struct Gpu,
 * prepare_expert_jobs): experts ascending, rows ascending inside an expert. */
typedef struct moe_prefill_plan {
    uint32_t *topk_idx;   /* [t][k] */
    float    *topk_w;     /* [t][k] */
    double   *logits;     /* [t][E] */
    float    *gamma;      /* [t] */
    int32_t  *expert_ptr; /* [E+1]: rows of expert e are entries ptr[e]..ptr[e+1]-1 */
    int32_t  *entry_row;  /* [t*k]: row of each entry */
    int32_t  *entry_rank; /* [t*k]: rank of the expert in that row's top-k */
    void     *ws;         /* workspace, >= moe_workspace_bytes(dims, t); zero-filled once */
    size_t    ws_bytes;
} moe_prefill_plan;

/* Bytes of one record of the given bit width (4, 3 or 2); 0 if invalid. */
uint64_t moe_record_bytes(int32_t hidden, int32_t inter, int32_t bits);

/* Workspace bytes for up to max_rows rows (1..4 decode, 1..32 prefill);
 * 0 if dims or max_rows are invalid.  The analog of the engine's expert
 * scratch, which the gpu/load.rs source page (load_bounded, the Scratch
 * buffers) sizes once for MAX_NB rows and k * MAX_NB + 1 union entries (the
 * routed union plus the shared expert): here the per-call exchange of the
 * decode kernel (counters, act values of up to 64 slots x 4 rows, per-slice
 * partial outputs, router logits) and the prefill buffers for max_rows rows
 * (MFMA-ordered x, act per (row, rank) entry, weighted outputs).  The
 * caller allocates it (device memory, 256-byte aligned) and keeps it for
 * the calls that use it; one workspace serves one stream at a time. */
size_t moe_workspace_bytes(const moe_dims *dims, int32_t max_rows);

/* Zero-fill a workspace on `stream` (a fill kernel, no memset node). */
int moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Router matvec (f64 accumulation), top-k softmax, union, slot table and
 * shared-gate value for nb rows of x (device f32 [nb][H], 16-byte aligned).
 * Struct Gpu router_b + the union publication of service_block, on device. */
int moe_route(const float *x, int32_t nb, const moe_router *router,
              const moe_shared *shared, moe_slots *slots, void *stream);

/* The whole layer for nb rows: moe_route, then every union expert and the
 * shared expert (gate/up + silu*up, down, weighted combine).  out: device f32
 * [nb][H], 16-byte aligned, overwritten (no residual).  Struct Gpu experts_b. */
int moe_layer_forward(const float *x, int32_t nb, const moe_router *router,
                      moe_slots *slots, const moe_pool *pool,
                      const moe_shared *shared, float *out, void *stream);

/* One part of the experts of a slot table the caller published (Struct Gpu
 * experts_b; the slot_tab field doc: entry 62 = resident count, 63 = union
 * size).  part 0 runs the union slots [0, tab[62]) -- the records resident
 * when the table was published -- plus the shared expert (weight gamma[b]),
 * and overwrites out; part 1 runs the slots [tab[62], tab[63]) -- the
 * records fetched meanwhile -- and adds them to out.  Between the two the
 * caller may fill the late records' pool bytes (for example copies from a
 * host tier ordered before part 1 on `stream`).
 *   slots->tab: device [64] descriptors as published (entries j < tab[63]
 *     name records in the pool; 0 <= tab[62] <= tab[63] <= 62, else the
 *     counts are clamped and status bit 0 is set); slots->wmap: device
 *     [4][64] per-row weights of the published slots; slots->gamma: device
 *     [nb] shared gate values (as moe_route writes them); slots->ws as for
 *     moe_layer_forward.  ids, topk_idx, topk_w and logits are not used.
 *   out: device f32 [nb][H]; x: device f32 [nb][H]; dims: host.
 * A record the table names that lies outside the pool is skipped (zero
 * contribution) and flags status bit 0. */
int moe_experts_part(const float *x, int32_t nb, const moe_dims *dims, moe_slots *slots,
                     int32_t part, const moe_pool *pool, const moe_shared *shared, float *out,
                     void *stream);

/* ------------------------------------------------------------------------
 * Two-part dispatch over a host-pinned record tier.  The pages' engine keeps
 * every expert record outside GPU memory and a fixed pool of device slots,
 * LRU managed (gpu.rs module doc; Struct Gpu: res, event, event_res,
 * service_block, experts_b).  Per layer: the GPU routes and the CPU reads
 * the union; the CPU publishes the slot table with the resident records
 * first (entry 62 = resident count, 63 = union size); part 0 (resident
 * records + shared expert) runs while the CPU copies the missing records
 * into free slots; part 1 runs once they have landed.  Here the store is
 * pinned host memory the caller fills, the copies run on a second stream,
 * and the GPU<->CPU signals are stream synchronisation and HIP events.
 * Two policies of the pages are options: the deadline cut of weak late
 * records (Struct Gpu cut_w, wait_for_deadline) and the one-layer
 * lookahead prefetch (Struct Gpu lookahead_layer, prefetch_async,
 * lookahead_hit).  The tier object is host memory plus a small pinned
 * staging area and one HIP event per slot, created by moe_tier_create and
 * released by moe_tier_destroy; device memory is the caller's.
 * ---------------------------------------------------------------------- */
typedef struct moe_tier moe_tier;

typedef struct moe_tier_config {
    moe_dims dims;
    int32_t n_layers;
    const uint8_t *host_tier;    /* pinned host memory (hipHostMalloc) holding every routed record */
    uint64_t host_bytes;
    const uint64_t *host_desc;   /* host [n_layers][E]: descriptor of record (layer, expert) in the
                                    host tier (offset | bits tag) */
    uint8_t *dev_pool;           /* device pool: the slot region, plus whatever else the caller keeps
                                    there (the shared experts' records) */
    uint64_t dev_bytes;
    uint64_t slot_offset;        /* byte offset of slot 0 in dev_pool (multiple of 256) */
    uint64_t slot_stride;        /* bytes per slot: >= a 4-bit record, multiple of 256 */
    int32_t n_slots;             /* >= k * MAX_NB, so that a whole union fits */
} moe_tier_config;

typedef struct moe_tier_policy {
    float cut_w;            /* > 0: at the deadline (part 0 done) a fetched record whose weight is
                               below cut_w in every row and whose copy has not landed is cut from
                               part 1 (its copy still completes); 0 = off */
    int32_t deadline_now;   /* 1: no fetched record counts as landed at the deadline (a
                               deterministic cut set, for tests and error studies) */
    int32_t lookahead;      /* 1: the next layer's router runs on this layer's input and the
                               records it predicts are fetched after this layer's copies */
    int32_t timing;         /* 1: fill part0_us and fetch_us (synchronises the streams) */
} moe_tier_policy;

typedef struct moe_tier_stats {
    int32_t n_union;        /* union size of this layer's step */
    int32_t n_resident;     /* records resident when the table was published (part 0) */
    int32_t n_fetched;      /* records copied from the host tier for part 1 */
    int32_t n_cut;          /* fetched records cut at the deadline */
    int32_t n_prefetched;   /* records fetched for the next layer by the lookahead */
    int32_t n_predicted;    /* experts the previous call predicted for this layer */
    int32_t n_hit;          /* of this layer's union, how many were predicted */
    float part0_us;         /* part 0 kernel time (timing = 1) */
    float fetch_us;         /* copy-stream time of this layer's fetches (timing = 1) */
} moe_tier_stats;

/* Validates the configuration (every host descriptor inside the host tier)
 * and creates the tier; the slots start empty.  MOE_EINVAL with a message
 * (moe_tier_last_error) on a bad configuration, MOE_ELAUNCH on a HIP error. */
int moe_tier_create(const moe_tier_config *cfg, moe_tier **out);
void moe_tier_destroy(moe_tier *t);

/* Copy the records of `experts` (n ids) of `layer` into free or least
 * recently used slots on copy_stream (warming the pool).  Call only while
 * no kernel reads the slots. */
int moe_tier_warm(moe_tier *t, int32_t layer, const int32_t *experts, int32_t n, void *copy_stream);

/* One MoE layer through the tier: moe_route on `stream` (router->rec may be
 * any device array of E descriptors: its slot table output is replaced),
 * the handshake, the published table in slots->tab / wmap / ids (resident
 * first), part 0, the copies on copy_stream, optionally the deadline cut
 * and the lookahead (next_router: the next layer's router; la_slots: its own
 * result buffers, which may share slots->ws), part 1.  out: device f32
 * [nb][H], overwritten.  Returns after part 1 is enqueued; the host blocks
 * on the route (and on part 0 when cut_w > 0, and on the lookahead route).
 * Errors are reported with moe_tier_last_error. */
int moe_tier_layer(moe_tier *t, int32_t layer, const float *x, int32_t nb, const moe_router *router,
                   moe_slots *slots, const moe_shared *shared, float *out,
                   const moe_tier_policy *policy, const moe_router *next_router,
                   moe_slots *la_slots, moe_tier_stats *stats, void *stream, void *copy_stream);

/* `stream` waits for every copy issued so far (cut or prefetched records). */
int moe_tier_join(moe_tier *t, void *stream);

/* Text of the last tier error on the calling thread. */
const char *moe_tier_last_error(void);

/* moe_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as moe_layer_forward,
 * except that slots->ws must be NULL and slots->ws_bytes 0: the decode
 * kernel's exchange buffers (counters, act values, slice partials, router
 * logits) live in the library's static scratch, 3 MiB of device memory per
 * GPU, held from the first call on that GPU until the process ends (its
 * first call zero-fills it on `stream` with a kernel).  The call allocates
 * nothing and calls no allocating routine.  Limit: the decode sections of
 * moe_workspace_bytes(dims, nb) must fit in 3 MiB (every width up to 512
 * with hidden up to 4096; width 1024 up to hidden 2048); larger dims return
 * MOE_EWORKSPACE before any HIP call.  Every call on one GPU shares that
 * GPU's scratch: calls that overlap in time on one GPU (other streams or
 * threads) race and give wrong results; serialise them.  The status word of
 * the scratch is read and cleared with moe_workspace_status(NULL, 0, stream)
 * on the same device. */
int moe_layer_forward_noalloc(const float *x, int32_t nb, const moe_router *router,
                              moe_slots *slots, const moe_pool *pool,
                              const moe_shared *shared, float *out, void *stream);

/* One prefill chunk of t rows (1..32): route every row, group rows by expert,
 * run each used expert on its rows with MFMA tiles (sub-jobs of at most 16
 * rows), the shared expert on all rows, and combine per row in a fixed order.
 * Struct Gpu prepare_expert_jobs / pf_experts.  out: device f32 [t][H]. */
int moe_prefill_forward(const float *x, int32_t t, const moe_router *router,
                        moe_prefill_plan *plan, const moe_pool *pool,
                        const moe_shared *shared, float *out, void *stream);

/* Low-bit store builder: the engine keeps a 3- or 2-bit copy of every
 * expert record, built once from the 4-bit source (gpu/load.rs source page,
 * load_bounded: the low-bit store and its smaller record stride; the pages
 * give no requantization rule).  For i < n_records, the 4-bit record at
 * src_desc[i] (tag 0) in the source pool is requantized into a record of
 * dst_desc[i]'s width (tag 1 = 3-bit, 2 = 2-bit) at its offset in the
 * destination pool.  Rule (min/max affine requantization of each 64-code
 * group of dequantised weights w = q s + b, exact in the code domain): with
 * q_lo and q_hi the group's codes of its smallest and largest weight and
 * d = |q_hi - q_lo|, the new code of a weight is round_half_up(|q - q_lo|
 * (2^bits - 1) / d), the new scale bf16(|s| d / (2^bits - 1)) and the new bias
 * bf16(b + s q_lo) (float32 operations, bf16 round to nearest even; codes 0
 * and scale 0 when d = 0).
 *   src_pool/dst_pool: device, 256-byte aligned, src_bytes/dst_bytes long
 *     (may be the same pool when the records do not overlap).
 *   src_desc/dst_desc: device arrays [n_records] of record descriptors.
 *   status: device u32 or NULL; bit 0 is OR-ed in when a descriptor pair is
 *     invalid (wrong tag, or a record outside its pool): that record is
 *     skipped, the others are written.
 * Validation of the shape and pointers happens on the host before any HIP
 * call; one kernel launch on `stream`. */
int moe_repack(const uint8_t *src_pool, uint64_t src_bytes, const uint64_t *src_desc,
               uint8_t *dst_pool, uint64_t dst_bytes, const uint64_t *dst_desc,
               int32_t n_records, int32_t hidden, int32_t inter, uint32_t *status,
               void *stream);

/* Status word kept in the workspace: bit 0 set when a kernel met a record
 * descriptor outside the pool or with tag 3 (that expert was skipped; its
 * contribution is zero); bit 2 set when the decode kernel's bounded wait for
 * another block ran out (its output is then not valid).  Synchronises
 * `stream`, reads the word and clears it; <0 on error.  ws = NULL with
 * ws_bytes = 0 reads the static scratch of moe_layer_forward_noalloc on the
 * current device (MOE_EWORKSPACE if no such call has run there). */
int moe_workspace_status(void *ws, size_t ws_bytes, void *stream);

/* Profiling hook (the analog of per-phase GPU timestamps): for the calling
 * thread, each call records events[i] (hipEvent_t, created by the caller) on
 * its stream.  moe_layer_forward runs one fused kernel and records events[0]
 * right after it.  moe_prefill_forward records events[0] after routing, top-k
 * and the expert grouping, events[1] after gate/up, events[2] after down and
 * events[3] after the per-row combine.  Entries may be NULL; n = 0 turns the
 * hook off.  No work is skipped.  At most 8 events. */
int moe_set_stage_events(void *const *events, int32_t n);

/* Text of the last non-zero return on the calling thread ("" if none): the
 * analog of the error messages of the shape checks in load_bounded (gpu/load.rs
 * source page, e.g. the check that k * MAX_NB entries leave room in the
 * 64-entry slot table) and of the HIP error of a failed launch.  The returned
 * string is owned by the library and valid until the thread's next call. */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
