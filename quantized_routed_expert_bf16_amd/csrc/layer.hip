// The whole decode MoE layer in one persistent launch (gfx950).
//
// What it computes is Struct Gpu router_b (a softmax over the router logits
// and a top-k selection, for nb rows) followed by experts_b (the routed
// experts of the union published in the slot table, plus the shared expert,
// summed per row), with the union and slot table of gpu.rs (union_of:
// first-seen order; slot_tab entry 62 = resident count, 63 = union size;
// wmap = per-row weight per slot) built on the device instead of by a host
// round trip.
//
// XCD-aware split.  The grid is 8 slices of blocks (block b belongs to slice
// b % 8, which the round-robin dispatcher places on XCD b % 8).  Slice x owns
// columns [x*W, (x+1)*W) of the expert width I (W = I / slices): the gate/up
// rows of those act values and the matching columns of every down matrix,
// for every slot of the union.  A slice therefore needs nothing from other
// slices until the very end:
//   1. every block stages the nb rows of x in LDS (plus per-32 sums of x);
//   2. router blocks, numbered across the slices, compute the E expert rows
//      and the shared gate vector (row E) with float64 accumulation, publish
//      the logits and bump a counter in every slice; meanwhile the other
//      blocks run the shared expert's gate/up units, which need no routing;
//   3. every block waits for its slice's router count, then selects each
//      row's top-k and builds the union itself (wave-parallel);
//   4. gate/up units (slot, 8 row pairs of the slice) write silu(g)*u tagged
//      with the call's epoch and bump the slice's gate/up counter; down
//      tiles (32 output rows) load their weights for all slots, wait for the
//      slice's gate/up count, and publish the slice's routing-weighted
//      partial rows (sum over slots in slot order, shared expert last);
//   5. the block of slice (tile mod slices) sums every slice's partial of a
//      tile in slice order into `out`, re-reading partials whose epoch tag
//      is not yet this call's;
//   6. the last block out publishes the epoch and resets the counters.
// Two to four rows at H = 2048 with 64 columns per slice run a second
// instantiation (kM) whose gate/up units and down tiles are MFMA
// contractions on exact f16 codes and f16 high/low halves of x and act; the
// others run the same steps on the VALU with in-register dequantisation.
// Cross-block data moves through device-coherent loads/stores (see
// device_common.h), so results do not depend on where blocks actually run;
// the slice-to-XCD placement only keeps the polling local.  Every wait is
// bounded: one that runs out sets the abort word and status bit 2, after
// which every wait falls through, so a launch cannot hang.
#include "device_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileRowPairs = 8;                      // gate/up unit: 8 row pairs
constexpr int kPairsPerWave = kTileRowPairs / kWaves;
constexpr int kRowsPerWave = 8;                       // down unit: 8 rows per wave
constexpr int kRowsPerTile = kRowsPerWave * kWaves;   // 32 rows per down tile
constexpr int kSlotBatch = 10;                        // slots per lane per down batch
constexpr int kStageCols = 256;                       // slot groups x slice width (= 8 x 32)
constexpr int kStagePad = 4;                          // floats after each staged (slot, row) run of W
// staged act floats per row of x: (slot groups x kSlotBatch) runs of W + pad, W >= 32
constexpr int kStageFloats = kStageCols * kSlotBatch + (kStageCols / kChunk) * kSlotBatch * kStagePad;
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kLateStageSleep = 20;   // s_sleep units (64 clocks each): ~0.5 us
// x in LDS is chunk-major with rows of n_chunks + kXPad float4s: the pad
// puts the 8 float4s of one chunk on different banks when they are written
constexpr int kXPad = 1;
__host__ __device__ constexpr int x_lds_floats(int nb, int hidden) { return nb * (hidden + 32 * kXPad); }

struct LayerArgs {
  LayerLaunch l;
  int n_slices;      // slices with work (<= 8)
  int W;             // columns of I per slice
  int ups;           // gate/up units per slot per slice
  int tiles;         // down tiles (of kRowsPerTile rows)
  int per_slice;     // blocks per slice (gridDim.x / 8)
  int route_blocks;  // router blocks in all (block g = lr * n_slices + x)
  uint32_t d_codes[3], d_sb[3];   // down section offsets in a record, per bits tag 0..2
  int part;          // -1: route and run every expert; 0 / 1: part of a published slot table
};

__device__ inline uint32_t *sw(const LayerArgs &a, int x, int field) {
  return a.l.sync + kSyncSliceStride * x + field;
}

__device__ inline void set_status(const LayerArgs &a, uint32_t bits) {
  __hip_atomic_fetch_or(a.l.sync + kSyncStatus, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait until *p >= target (thread 0 polls, then the block proceeds).
__device__ inline void wait_geq(const LayerArgs &a, const uint32_t *p, uint32_t target) {
  if (threadIdx.x == 0) {
    uint32_t it = 0;
    while (ld_dev(p) < target) {
      if ((++it & 63) == 0) {
        if (ld_dev(a.l.sync + kSyncAbort)) break;
        if (it > kSpinLimit) {
          st_dev(a.l.sync + kSyncAbort, 1u);
          set_status(a, 4u);
          break;
        }
      }
      __builtin_amdgcn_s_sleep(4);
    }
  }
  __syncthreads();
}

template <int NB>
struct Shared {
  float exq[64];
  int sel[NB][kMaxTopK];
  double selv[NB][kMaxTopK];
  float wsel[NB][kMaxTopK];
  int uid[kSlotStride];
  int first[NB > 1 ? kMaxExperts : 1];   // union: lowest (row, rank) entry per expert
  float wslot[NB][kSlotStride];   // routing weight per slot (index u: gamma)
  uint64_t desc[kSlotStride];     // descriptor per slot (index u: shared expert)
  const uint8_t *dcodes[kSlotStride];   // down codes of the slot's record (null: skip)
  const uint32_t *dsb[kSlotStride];     // down (scale, bias) words
  int dbits[kSlotStride];               // bit width (0: bad descriptor)
  float gam[NB];
  int u;
  int nsl;            // slots the down tiles take: u + 1 (the shared expert last), u in part 1
  uint32_t prev;
  uint32_t ep;        // this call's epoch
};

// ----------------------------------------------------------------- route
// A wave's first router row (or the shared-expert gate vector, row E), loaded
// into registers before the block stages x so that both loads overlap.
// x in LDS, chunk-major: the 4-float group q (0..7) of 32-input chunk c of
// row b is float4 number (8 b + q) n_chunks + c, so a wave whose lanes read
// chunks lane + 64 t touches consecutive float4s (no bank conflicts).
struct ChunkX {
  const float4 *p;
  int nch, c;
  __device__ float4 operator()(int b, int q) const { return p[(b * 8 + q) * (nch + kXPad) + c]; }
};

template <int CPL>
struct RouterRow {
  uint4 w[4 * CPL];   // lane's 32 bf16 of chunk lane + 64 (t / 4), 8 per uint4
};

template <int CPL>
__device__ __forceinline__ void router_prefetch(const LayerArgs &a, int g, RouterRow<CPL> &r) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.l.hidden, E = a.l.n_experts;
  const int e = g * kWaves + wave;
  if (e > E) return;
  const uint16_t *w = e < E ? a.l.router + size_t(e) * H : a.l.gvec;
#pragma unroll
  for (int t = 0; t < 4 * CPL; ++t) {
    const int c = lane + 64 * (t / 4);
    if (c < H / kChunk) r.w[t] = *reinterpret_cast<const uint4 *>(w + c * kChunk + 8 * (t % 4));
  }
}

// Router logits (float64 accumulation of the bf16 weights times x) of rows
// e = 4 g + wave, e += 4 G for router block g of G; row E is the shared
// expert's gate, stored as its sigmoid.  Lane l takes chunks l + 64 t.
template <int NB, int CPL>
__device__ __forceinline__ void router_rows(const LayerArgs &a, const float *xs, int g, const RouterRow<CPL> &first,
                            double *lg, float *gm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.l.hidden, E = a.l.n_experts, nch = H / kChunk;
  for (int e = g * kWaves + wave; e <= E; e += a.route_blocks * kWaves) {
    const uint16_t *w = e < E ? a.l.router + size_t(e) * H : a.l.gvec;
    const bool pre = e == g * kWaves + wave;
    double acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.0;
#pragma unroll
    for (int t = 0; t < 4 * CPL; ++t) {
      const int c = lane + 64 * (t / 4), j = t % 4;
      if (c >= nch) break;
      const uint4 wv = pre ? first.w[t] : *reinterpret_cast<const uint4 *>(w + c * kChunk + 8 * j);
      const float wf[8] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y),
                           bf16_lo(wv.z), bf16_hi(wv.z), bf16_lo(wv.w), bf16_hi(wv.w)};
      const ChunkX X{reinterpret_cast<const float4 *>(xs), nch, c};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 x0 = X(b, 2 * j), x1 = X(b, 2 * j + 1);
        const float xf[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[b] = fma(double(wf[q]), double(xf[q]), acc[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const double v = wave_sum_d(acc[b]);
      if (lane == 0) {
        if (e < E)
          st_dev(lg + b * kMaxExperts + e, v);
        else
          st_dev(gm + b, float(1.0 / (1.0 + exp(-v))));
      }
    }
  }
}

// Of the keys kk (0: not a candidate), the `need` largest in the order (key
// descending, lower index first): a most-significant-bit-first radix select
// with ballot counts finds the longest prefix T that at least `need` keys
// reach (stopping as soon as exactly `need` do); keys above T are taken and,
// of the keys equal to T, the lowest indices fill the remaining places.
template <typename K, int kJ>
__device__ __forceinline__ void radix_take(const K (&kk)[kJ], int need, bool (&take)[kJ]) {
  const int lane = threadIdx.x & 63;
  constexpr int kBits = 8 * sizeof(K);
  K T = 0;
  int cnt = kJ * 64;   // keys >= T (before the first step: every key)
  for (int bit = kBits - 1; bit >= 0 && cnt != need; --bit) {
    const K c = T | (K(1) << bit);
    int n = 0;
#pragma unroll
    for (int j = 0; j < kJ; ++j) n += __popcll(__ballot(kk[j] >= c));
    if (n >= need) {
      T = c;
      cnt = n;
    }
  }
  int left = need;   // places left for keys equal to T
#pragma unroll
  for (int j = 0; j < kJ; ++j) left -= __popcll(__ballot(kk[j] > T));
  const uint64_t below = (uint64_t(1) << lane) - 1;
  int eq_before = 0;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const bool eq = kk[j] == T && T != 0;
    const uint64_t eqm = __ballot(eq);
    take[j] = kk[j] > T || (eq && eq_before + __popcll(eqm & below) < left);
    eq_before += __popcll(eqm);
  }
}

// Top-k of the published logits (every block).  Wave b (b < NB) holds row
// b's logits in registers, expert lane + 64 j in register j.  The select runs
// on 32-bit order-preserving keys of the logits rounded to float32 (rounding
// never reverses an order, so a key above the float32 threshold T is in the
// top k and a key below it is not); only logits whose float32 rounding equals
// T are ranked again on their 64-bit keys of the float64 values, with ties
// to the lower expert id, which is the order (logit descending, id
// ascending).  In the common case T's group is exactly the places left and
// no 64-bit step runs.  The k selected entries are then ranked against each
// other in registers (the wave walks the selected lanes with readlane):
// s.sel[b][rank] and s.selv[b][rank] on return.
// kJ = 2 serves up to 128 experts, 4 up to 256.
template <int NB, int kJ>
__device__ __forceinline__ void select_row(const LayerArgs &a, Shared<NB> &s, const double *lg, const float *gm,
                           int b) {
  const int lane = threadIdx.x & 63;
  const int E = a.l.n_experts, k = a.l.top_k;
  double v[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j)   // clamped and unconditional: all loads in flight at once
    v[j] = ld_dev(lg + b * kMaxExperts + min(lane + 64 * j, E - 1));
  const float gam = ld_dev(gm + b);
  uint64_t kk[kJ];
  uint32_t k32[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    // + 0.0 folds -0 into +0 so that equal logits tie on the id alone;
    // padding keys are 0, below every logit's key and below every prefix
    // the select tries
    const bool in = lane + 64 * j < E;
    const double vv = v[j] + 0.0;
    kk[j] = in ? order_key(vv) : 0;
    k32[j] = in ? order_key32(float(vv)) : 0;
  }
  // float32 keys: T = the k-th largest key, gt keys above it, neq equal to it
  // two key bits per step: the three candidate prefixes are counted
  // independently, and the largest one that k keys reach is kept
  uint32_t T = 0;
  int cnt = kJ * 64;
  for (int bit = 30; bit >= 0 && cnt != k; bit -= 2) {
    const uint32_t c1 = T | (1u << bit), c2 = T | (2u << bit), c3 = T | (3u << bit);
    int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      n1 += __popcll(__ballot(k32[j] >= c1));
      n2 += __popcll(__ballot(k32[j] >= c2));
      n3 += __popcll(__ballot(k32[j] >= c3));
    }
    if (n3 >= k) {
      T = c3;
      cnt = n3;
    } else if (n2 >= k) {
      T = c2;
      cnt = n2;
    } else if (n1 >= k) {
      T = c1;
      cnt = n1;
    }
  }
  int gt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    gt += __popcll(__ballot(k32[j] > T));
    neq += __popcll(__ballot(k32[j] == T));
  }
  bool take[kJ];
  if (neq == k - gt) {   // T's group fills the places left exactly
#pragma unroll
    for (int j = 0; j < kJ; ++j) take[j] = k32[j] >= T;
  } else {               // equal in float32: the float64 values and ids decide
    uint64_t km[kJ];
    bool te[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) km[j] = k32[j] == T ? kk[j] : 0;
    radix_take<uint64_t, kJ>(km, k - gt, te);
#pragma unroll
    for (int j = 0; j < kJ; ++j) take[j] = k32[j] > T || te[j];
  }
  uint64_t tm[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) tm[j] = __ballot(take[j]);
  // rank the k selected entries against each other in registers: the
  // wave walks the selected lanes (uniform masks) and reads each entry's
  // key with readlane
  int rank[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) rank[j] = 0;
#pragma unroll
  for (int jq = 0; jq < kJ; ++jq) {
    for (uint64_t m = tm[jq]; m; m &= m - 1) {
      const int L = __builtin_ctzll(m);
      const uint64_t qk = readlane_u64(kk[jq], L);
      const int qi = L + 64 * jq;
#pragma unroll
      for (int j = 0; j < kJ; ++j) rank[j] += int(pair_before(qk, qi, kk[j], lane + 64 * j));
    }
  }
#pragma unroll
  for (int j = 0; j < kJ; ++j)
    if (take[j]) {
      s.sel[b][rank[j]] = lane + 64 * j;
      s.selv[b][rank[j]] = v[j] + 0.0;
    }
  if (lane == 0) s.gam[b] = gam;
  if (blockIdx.x == 0) {   // caller-visible logits (as published)
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      if (lane + 64 * j < E) a.l.logits[b * E + lane + 64 * j] = v[j];
  }
}

template <int NB>
__device__ __forceinline__ void route_select(const LayerArgs &a, Shared<NB> &s, const double *lg, const float *gm) {
  const int wave = threadIdx.x >> 6;
  if (wave < NB) {
    if (a.l.n_experts <= 128) select_row<NB, 2>(a, s, lg, gm, wave);
    else select_row<NB, kMaxExperts / 64>(a, s, lg, gm, wave);
  }
  __syncthreads();
}

// Softmax weights of each row's k selected logits, the first-seen union of
// the (row, rank) list and the per-slot record pointers used by the expert
// units (wave 0; every wave on return).  A row's k experts are distinct, so
// union slot s < k is always row 0's rank-s expert.
template <int NB>
__device__ __forceinline__ void route_union(const LayerArgs &a, Shared<NB> &s, const uint64_t *rec_lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k = a.l.top_k;
  if (wave == 0) {
    // lane l < NB k holds entry (row l / k, rank l % k)
    const int n = NB * k;
    const bool ent = lane < n;
    const int lb = ent ? lane / k : 0, lr = lane - lb * k;
    const int e_l = ent ? s.sel[lb][lr] : 0;
    const uint64_t d_l = ent ? rec_lds[e_l] : a.l.shared_rec;
    // (float32: the weights are float32 results, within a few ulp of the
    // float64 softmax)
    const float ex = ent ? expf(float(s.selv[lb][lr] - s.selv[lb][0])) : 0.0f;
    s.exq[lane] = ex;
    // first-seen union: fq = lowest entry with this lane's expert (an LDS
    // minimum per expert id; one wave, whose LDS operations run in order)
    int fq = lane;
    if constexpr (NB > 1) {
      if (ent) s.first[e_l] = 64;
      if (ent) atomicMin(&s.first[e_l], lane);
      if (ent) fq = s.first[e_l];
    }
    const bool first = ent && fq == lane;
    const uint64_t mask = __ballot(first);
    const int slot = __popcll(mask & ((uint64_t(1) << fq) - 1));
    const int u = __popcll(mask);
    __builtin_amdgcn_wave_barrier();
    // softmax of each row's k selected logits: with k = 8 a row's entries
    // are one group of 8 lanes (DPP sum), else summed in rank order
    float sum = 0.0f;
    if (k == 8) {
      sum = group8_sum(ex);
    } else {
#pragma unroll
      for (int r = 0; r < kMaxTopK; ++r) {   // every read issued at once; adding 0 past k
        const float e = s.exq[min(lb * k + r, 63)];
        sum += r < k ? e : 0.0f;
      }
    }
    const float w_l = ent ? ex / sum : 0.0f;
    if (ent) s.wsel[lb][lr] = w_l;
    if (lane == 0) {
      s.u = u;
      s.nsl = u + 1;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) s.wslot[b][lane] = lane == u ? s.gam[b] : 0.0f;
    __builtin_amdgcn_wave_barrier();
    if (ent) s.wslot[lb][slot] = w_l;
    // slot records: the first entry of each expert fills its slot, lane 63
    // (never an entry) the shared expert's slot u
    if (first || lane == 63) {
      const int js = first ? slot : u;
      if (first) s.uid[js] = e_l;
      s.desc[js] = d_l;
      const bool ok = record_ok(d_l, a.l.pool_bytes, a.l.hidden, a.l.inter);
      const int bt = ok ? bits_of_tag(d_l) : 0;
      const RecordLayout L = record_layout(a.l.hidden, a.l.inter, ok ? bt : 4);
      const uint8_t *rec = a.l.pool + (d_l & ~uint64_t(255));
      s.dbits[js] = bt;
      s.dcodes[js] = ok ? rec + L.d_codes : nullptr;
      s.dsb[js] = ok ? reinterpret_cast<const uint32_t *>(rec + L.d_sb) : nullptr;
    }
  }
  __syncthreads();
  const int u = s.u;
  if (blockIdx.x == 0) {   // caller-visible routing tables
    for (int j = threadIdx.x; j < kSlotStride; j += kThreads) {
      a.l.ids[j] = j < u ? uint32_t(s.uid[j]) : 0u;
      a.l.tab[j] = (j == MOE_RESIDENT_ENTRY || j == MOE_UNION_ENTRY) ? uint64_t(u)
                                                                    : (j < u ? s.desc[j] : 0);
      for (int b = 0; b < kMaxNb; ++b)
        a.l.wmap[b * kSlotStride + j] = (b < NB && j < u) ? s.wslot[b < NB ? b : 0][j] : 0.0f;
    }
    for (int p = threadIdx.x; p < NB * k; p += kThreads) {
      a.l.topk_idx[p] = uint32_t(s.sel[p / k][p % k]);
      a.l.topk_w[p] = s.wsel[p / k][p % k];
    }
    if (threadIdx.x < NB) a.l.gamma[threadIdx.x] = s.gam[threadIdx.x];
  }
}

// The slots of one part of a slot table published by the caller (Struct Gpu
// experts_b: part 0 runs the records resident when the table was published,
// entries [0, tab[62]), plus the shared expert; part 1 the records fetched
// meanwhile, entries [tab[62], tab[63])), with the per-row weights of wmap
// and the shared gate values in gamma.  Counts outside 0 <= tab[62] <=
// tab[63] <= 62 are clamped and flag status bit 0.
template <int NB>
__device__ __forceinline__ void table_slots(const LayerArgs &a, Shared<NB> &s) {
  const int j = threadIdx.x;
  const uint64_t r62 = a.l.tab[MOE_RESIDENT_ENTRY], r63 = a.l.tab[MOE_UNION_ENTRY];
  const int n_u = int(min(r63, uint64_t(MOE_RESIDENT_ENTRY)));
  const int n_res = int(min(r62, uint64_t(n_u)));
  const int begin = a.part == 0 ? 0 : n_res, end = a.part == 0 ? n_res : n_u;
  const int u = end - begin;
  const bool shared = a.part == 0;
  if (j == 0 && (r62 > r63 || r63 > uint64_t(MOE_RESIDENT_ENTRY))) set_status(a, 1u);
  if (j <= u && j < kSlotStride) {
    const uint64_t d = j < u ? a.l.tab[begin + j] : (shared ? a.l.shared_rec : 0);
    const bool ok = (j < u || shared) && record_ok(d, a.l.pool_bytes, a.l.hidden, a.l.inter);
    const int bt = ok ? bits_of_tag(d) : 0;
    const RecordLayout L = record_layout(a.l.hidden, a.l.inter, ok ? bt : 4);
    const uint8_t *rec = a.l.pool + (d & ~uint64_t(255));
    s.desc[j] = d;
    s.dbits[j] = bt;
    s.dcodes[j] = ok ? rec + L.d_codes : nullptr;
    s.dsb[j] = ok ? reinterpret_cast<const uint32_t *>(rec + L.d_sb) : nullptr;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      s.wslot[b][j] = j < u ? a.l.wmap[b * kSlotStride + begin + j] : (shared ? a.l.gamma[b] : 0.0f);
    if (j < u && !ok) set_status(a, 1u);
  }
  if (j == 0) {
    s.u = u;
    s.nsl = shared ? u + 1 : u;
  }
  __syncthreads();
}

template <int NB>
__device__ __forceinline__ void build_slots(const LayerArgs &a, Shared<NB> &s, const uint64_t *rec_lds) {
  if (a.part >= 0) table_slots<NB>(a, s);
  else route_union<NB>(a, s, rec_lds);
}

// ------------------------------------------------------------ gate / up
// 8 row pairs (gate j, up j) of one slot; each wave takes 2, a lane one
// 32-code chunk of the H inputs (CPL chunks when H > 2048).
// The lane's codes and (scale, bias) words of a unit's row pairs.
template <int CPL>
struct GuRegs {
  uint32_t w[kPairsPerWave][2][CPL][4];
  uint32_t s[kPairsPerWave][2][CPL];
};

template <int CPL, int BITS>
__device__ __forceinline__ void gate_up_load(const LayerArgs &a, const uint8_t *rec, int j0, GuRegs<CPL> &r) {
  const int lane = threadIdx.x & 63;
  const int H = a.l.hidden, I = a.l.inter;
  const RecordLayout L = record_layout(H, I, BITS);
  const int n_chunks = H / kChunk, gpr = H / kGroup;
  const uint8_t *codes = rec + L.gu_codes;
  const uint32_t *sb = reinterpret_cast<const uint32_t *>(rec + L.gu_sb);
#pragma unroll
  for (int p = 0; p < kPairsPerWave; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 2 * (j0 + p) + h;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {   // clamped, unconditional (lanes past H drop out later)
        const int chunk = min(lane + 64 * c, n_chunks - 1);
        load_chunk<BITS>(codes + size_t(row) * L.gu_row_bytes, H, chunk, r.w[p][h][c]);
        r.s[p][h][c] = sb[size_t(row) * gpr + chunk / 2];
      }
    }
}

// Loads for a record of any bit width (the tag is uniform).
template <int CPL>
__device__ __forceinline__ void gate_up_load_any(const LayerArgs &a, uint64_t desc, int j0, GuRegs<CPL> &r) {
  const uint8_t *rec = a.l.pool + (desc & ~uint64_t(255));
  switch (bits_of_tag(desc)) {
    case 4: gate_up_load<CPL, 4>(a, rec, j0, r); break;
    case 3: gate_up_load<CPL, 3>(a, rec, j0, r); break;
    default: gate_up_load<CPL, 2>(a, rec, j0, r); break;
  }
}

template <int NB, int CPL, int BITS>
__device__ __forceinline__ void gate_up_unit(const LayerArgs &a, const GuRegs<CPL> &r, int j0, int act_slot,
                             const float *xs, const float *xsum, uint32_t ep) {
  const int lane = threadIdx.x & 63;
  const int H = a.l.hidden, I = a.l.inter;
  const int n_chunks = H / kChunk;
  const auto &w = r.w;
  const auto &s = r.s;
  float v[kPairsPerWave][2][NB];
#pragma unroll
  for (int p = 0; p < kPairsPerWave; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int b = 0; b < NB; ++b) v[p][h][b] = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int chunk = min(lane + 64 * c, n_chunks - 1);
    const bool live = lane + 64 * c < n_chunks;
    const ChunkX X{reinterpret_cast<const float4 *>(xs), n_chunks, chunk};
    float xsm[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) xsm[b] = live ? xsum[b * n_chunks + chunk] : 0.0f;
    if constexpr (NB <= 2) {   // x of the chunk in registers, shared by the four rows
      float xr[NB][kChunk];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < kChunk / 4; ++q) {
          const float4 f = X(b, q);
          xr[b][4 * q] = f.x; xr[b][4 * q + 1] = f.y; xr[b][4 * q + 2] = f.z; xr[b][4 * q + 3] = f.w;
        }
#pragma unroll
      for (int p = 0; p < kPairsPerWave; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float P[NB];
          chunk_dot<BITS, NB>(w[p][h][c], RegX<NB>{xr}, P);
          const float sc = live ? sb_scale(s[p][h][c]) : 0.0f, bi = live ? sb_bias(s[p][h][c]) : 0.0f;
#pragma unroll
          for (int b = 0; b < NB; ++b) v[p][h][b] += fmaf(sc, P[b], bi * xsm[b]);
        }
    } else {   // more rows: each x float4 from LDS feeds the four rows at once
      constexpr int R = 2 * kPairsPerWave;
      uint32_t wr[R][4];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) wr[r][q] = w[r / 2][r % 2][c][q];
      float P[R][NB];
      chunk_dot_rows<BITS, NB, R>(wr, X, P);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float sc = live ? sb_scale(s[r / 2][r % 2][c]) : 0.0f;
        const float bi = live ? sb_bias(s[r / 2][r % 2][c]) : 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b) v[r / 2][r % 2][b] += fmaf(sc, P[r][b], bi * xsm[b]);
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kPairsPerWave; ++p) {
    float g = 0.0f, u = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float gs = wave_sum(v[p][0][b]), us = wave_sum(v[p][1][b]);
      if (lane == b) { g = gs; u = us; }
    }
    if (lane < NB) st_dev(a.l.act + (size_t(act_slot) * kMaxNb + lane) * I + j0 + p, tag_f32(ep, silu_mul(g, u)));
  }
}

// A gate/up unit publishes its act values tagged with the call's epoch and
// bumps the slice counter without waiting for the stores: the counter tells
// the down tiles when to look, the tags tell them what is current.
// First gate/up row pair of the wave in a unit.
__device__ __forceinline__ int gate_up_row0(const LayerArgs &a, int x, int unit) {
  return x * a.W + unit * kTileRowPairs + (threadIdx.x >> 6) * kPairsPerWave;
}

// kLoaded: `r` already holds the unit's weights.
template <int NB, int CPL, bool kLoaded = false>
__device__ __forceinline__ void run_gate_up(const LayerArgs &a, int x, uint64_t desc, int act_slot, int unit,
                            const float *xs, const float *xsum, uint32_t ep, GuRegs<CPL> &r) {
  const int lane = threadIdx.x & 63;
  const int j0 = gate_up_row0(a, x, unit);
  if (record_ok(desc, a.l.pool_bytes, a.l.hidden, a.l.inter)) {
    if constexpr (!kLoaded) gate_up_load_any<CPL>(a, desc, j0, r);
    switch (bits_of_tag(desc)) {
      case 4: gate_up_unit<NB, CPL, 4>(a, r, j0, act_slot, xs, xsum, ep); break;
      case 3: gate_up_unit<NB, CPL, 3>(a, r, j0, act_slot, xs, xsum, ep); break;
      default: gate_up_unit<NB, CPL, 2>(a, r, j0, act_slot, xs, xsum, ep); break;
    }
  } else {
    if (threadIdx.x == 0) set_status(a, 1u);
    if (lane < NB * kPairsPerWave)
      st_dev(a.l.act + (size_t(act_slot) * kMaxNb + lane / kPairsPerWave) * a.l.inter + j0 +
                 lane % kPairsPerWave, tag_f32(ep, 0.0f));
  }
  __syncthreads();   // every wave has issued its stores
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(sw(a, x, kSliceGu), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------- gate / up on MFMA
// With two or more rows the dequantised dot products dominate the VALU time
// of a gate/up unit (one FMA per code and row).  For 4-bit records (and
// H <= 2048) the unit runs on v_mfma_f32_16x16x32_f16 instead: A = the 16
// rows of the unit (8 gate/up pairs) as exact f16 integers, B = x split into
// f16 high and low halves (columns b and 4 + b for row b), one 64-code group
// (two MFMAs) per accumulator so that the group's scale and bias apply after
// the product: y += s * (q . x) + b * sum(x).  Wave w takes the unit's 16
// rows over groups [w G/4, (w+1) G/4); the waves' partial rows are summed in
// LDS.
//
// Operand order.  Lane l holds A row l % 16 and B column l % 16 at k-slot
// q = l / 16.  The four slot lanes of a row load 64 contiguous bytes, two
// groups, with one 16-byte load each (slots 0, 1: halves of the even group,
// slots 2, 3: of the odd one); swapping the upper two words between slots q
// and q ^ 2 leaves every lane two words (16 codes) of each group: slot q of
// group g holds codes base(g, q) + 8 st + (0..7) in step st, with base =
// 16 (2 (q & 1) + ((q >> 1) ^ (g & 1))).  A word is expanded as code pairs
// (0,4), (1,5), (2,6), (3,7).  The B fragments are staged once per block in
// the same order.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));


constexpr int kMfmaHidden = 64 * kChunk;               // the one H the MFMA units take (2048)
constexpr int kMG = kMfmaHidden / kGroup;               // groups per row (32)
constexpr int kMGw = kMG / kWaves;                      // groups per wave (8)

// x as MFMA B fragments: [group][step][slot][column 0..7] half8; and per
// group the sums of x in columns 0..NB-1 (0 elsewhere).

template <int NB>
__device__ __forceinline__ void stage_x_fragments(const LayerArgs &a, const float *xs, const float *xsum,
                                                  uint4 *xb, float *xg) {
  constexpr int nch = kMfmaHidden / kChunk;
  const ChunkX X0{reinterpret_cast<const float4 *>(xs), nch, 0};
  for (int i = threadIdx.x; i < kMG * 64; i += kThreads) {
    const int j = i & 7, q = (i >> 3) & 3, st = (i >> 5) & 1, g = i >> 6;
    const int b = j & 3, part = j >> 2;
    uint4 out = make_uint4(0, 0, 0, 0);
    if (b < NB) {
      // inputs k0 .. k0 + 7; the slot order alternates with the group's
      // parity
      const int k0 = kGroup * g + 16 * (2 * (q & 1) + ((q >> 1) ^ (g & 1))) + 8 * st;
      const ChunkX X{X0.p, nch, k0 / kChunk};
      const float4 f0 = X(b, (k0 % kChunk) / 4), f1 = X(b, (k0 % kChunk) / 4 + 1);
      const float f[8] = {f0.x, f1.x, f0.y, f1.y, f0.z, f1.z, f0.w, f1.w};   // codes 0,4,1,5,2,6,3,7
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        half2v v;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const _Float16 hi = _Float16(f[2 * e + t]);
          v[t] = part ? _Float16(f[2 * e + t] - float(hi)) : hi;
        }
        h[e] = __builtin_bit_cast(uint32_t, v);
      }
      out = make_uint4(h[0], h[1], h[2], h[3]);
    }
    xb[i] = out;
  }
  for (int i = threadIdx.x; i < kMG * 8; i += kThreads) {
    const int j = i & 7, g = i >> 3;
    xg[i] = j < NB ? xsum[j * nch + 2 * g] + xsum[j * nch + 2 * g + 1] : 0.0f;
  }
}

// One 4-bit code word as an A fragment: f16 pairs (0,4), (1,5), (2,6), (3,7).
// Nibbles at bits 0..3 of a half become 1024 + q and at bits 4..7 1024 + 16q
// (exponent bits OR-ed in); one packed f16 add or fma takes them to q exactly.
// The masks come in as register values: with a mask in a register the AND
// and the OR of a pair fuse into one v_and_or_b32 (a literal cannot be an
// operand of it).
struct NibbleMasks {
  uint32_t lo, hi, ex;   // 0x000F000F, 0x00F000F0, 0x64006400
};
__device__ __forceinline__ NibbleMasks nibble_masks() {
  NibbleMasks m{0x000F000Fu, 0x00F000F0u, 0x64006400u};
  asm volatile("" : "+v"(m.lo), "+v"(m.hi), "+v"(m.ex));
  return m;
}
__device__ __forceinline__ half8 word_to_a(uint32_t w, const NibbleMasks &m) {
  const half2v k1024 = {_Float16(-1024.0f), _Float16(-1024.0f)};
  const half2v s16 = {_Float16(0.0625f), _Float16(0.0625f)};
  const half2v k64 = {_Float16(-64.0f), _Float16(-64.0f)};
  const uint32_t t = w >> 8;
  const half2v p0 = __builtin_bit_cast(half2v, (w & m.lo) | m.ex) + k1024;
  const half2v p1 = __builtin_bit_cast(half2v, (w & m.hi) | m.ex) * s16 + k64;
  const half2v p2 = __builtin_bit_cast(half2v, (t & m.lo) | m.ex) + k1024;
  const half2v p3 = __builtin_bit_cast(half2v, (t & m.hi) | m.ex) * s16 + k64;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// A 2- or 3-bit code word (16 codes) as two A fragments in the same k
// order as word_to_a gives a 4-bit word's codes: step 0 holds codes 0..7 as
// pairs (0,4), (1,5), (2,6), (3,7), step 1 codes 8..15 likewise.  One byte
// permute puts byte 1 (codes 4..7) beside byte 0 in the other half word;
// field p of a byte, scaled by 4^p once in place, is undone by one packed
// f16 fma.  `hb`: the high bits of the word's codes, bit 8k + p for code
// 4k + p (3-bit only).
template <int BITS>
__device__ __forceinline__ void lowbit_to_a(uint32_t w, uint32_t hb, half8 &A0, half8 &A1) {
  const uint32_t wp = __builtin_amdgcn_perm(0u, w, 0x03010200u);
  const uint32_t hp = BITS == 3 ? __builtin_amdgcn_perm(0u, hb, 0x03010200u) : 0u;
  half8 A[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const uint32_t x = wp >> (8 * st), xh = hp >> (8 * st);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t v = (x & (0x00030003u << (2 * p))) | 0x64006400u;
      if constexpr (BITS == 3) v |= (xh & (0x00010001u << p)) << (p + 2);
      const float sc = 1.0f / float(1 << (2 * p));
      const half2v m = {_Float16(sc), _Float16(sc)}, o = {_Float16(-1024.0f * sc), _Float16(-1024.0f * sc)};
      const half2v h = __builtin_bit_cast(half2v, v) * m + o;
      A[st][2 * p] = h[0];
      A[st][2 * p + 1] = h[1];
    }
  }
  A0 = A[0];
  A1 = A[1];
}

// The lane's code words and (scale, bias) words of a unit: row l % 16 of
// the unit, slot l / 16, the wave's groups; (scale, bias) of that row for
// the wave's groups 2 (l / 16) and 2 (l / 16) + 1.
struct GuRegsM {
  uint4 c[kMGw / 2];
  uint2 s;
};

// 4-bit: c[gp] = the row's 16 bytes of group pair gp in the lane's slot.
// 2/3-bit: coalesced row pieces, rearranged through LDS by the unit:
// c[0], c[1] = low-plane bytes 16 (l % 8) .. + 15 (group l % 8 of the wave)
// of rows l / 8 and 8 + l / 8; c[2] = high-plane bytes 16 (l % 4) .. + 15
// (chunks 4 (l % 4) .. + 3 of the wave) of row l / 4.
template <int BITS>
__device__ __forceinline__ void gate_up_load_m(const LayerArgs &a, uint64_t desc, int x, int unit, GuRegsM &r) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RecordLayout L = record_layout(kMfmaHidden, a.l.inter, BITS);
  const uint8_t *rec = a.l.pool + (desc & ~uint64_t(255));
  const int r0 = 2 * (x * a.W + unit * kTileRowPairs);   // the unit's first of 16 rows
  const int q = lane >> 4, rr = r0 + (lane & 15);
  const uint8_t *codes = rec + L.gu_codes;
  if constexpr (BITS == 4) {
    const uint8_t *row = codes + size_t(rr) * L.gu_row_bytes + 32 * (wave * kMGw) + 16 * q;
#pragma unroll
    for (int gp = 0; gp < kMGw / 2; ++gp) r.c[gp] = *reinterpret_cast<const uint4 *>(row + 64 * gp);
  } else {
    const int lo = kMGw * kGroup / 4;   // low-plane bytes of the wave's groups per row (128)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      r.c[h] = *reinterpret_cast<const uint4 *>(codes + size_t(r0 + (lane >> 3) + 8 * h) * L.gu_row_bytes +
                                                lo * wave + 16 * (lane & 7));
    if constexpr (BITS == 3)
      r.c[2] = *reinterpret_cast<const uint4 *>(codes + size_t(r0 + (lane >> 2)) * L.gu_row_bytes +
                                                kMfmaHidden / 4 + (lo / 2) * wave + 16 * (lane & 3));
  }
  const uint32_t *sb = reinterpret_cast<const uint32_t *>(rec + L.gu_sb);
  r.s = *reinterpret_cast<const uint2 *>(sb + size_t(rr) * kMG + wave * kMGw + 2 * q);
}

__device__ __forceinline__ void gate_up_load_m_any(const LayerArgs &a, uint64_t desc, int x, int unit, GuRegsM &r) {
  switch (bits_of_tag(desc)) {
    case 4: gate_up_load_m<4>(a, desc, x, unit, r); break;
    case 3: gate_up_load_m<3>(a, desc, x, unit, r); break;
    default: gate_up_load_m<2>(a, desc, x, unit, r); break;
  }
}

// Per-wave LDS rows for 2/3-bit codes: [16 rows][kLbRow words]: 32 low-plane
// words (group-major, 4 per group), then 16 high-plane words (one per chunk).
constexpr int kLbRow = 52;
constexpr int kLbWave = 16 * kLbRow;

// `red` holds one 512-byte slice per wave: first the wave's (scale, bias)
// words [group][16 rows], then its partial rows [16 rows][8 columns].
template <int NB, int BITS>
__device__ __forceinline__ void gate_up_unit_m(const LayerArgs &a, const GuRegsM &r, int x, int unit, int act_slot,
                                               const uint4 *xb, const float *xg, float *red, uint32_t *stg,
                                               uint32_t ep) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int I = a.l.inter;
  const int q = lane >> 4, j = lane & 15;
  float *slice = red + wave * 128;
  uint32_t *sbl = reinterpret_cast<uint32_t *>(slice);
  sbl[2 * q * 16 + j] = r.s.x;
  sbl[(2 * q + 1) * 16 + j] = r.s.y;
  uint32_t *lb = stg + wave * kLbWave;
  if constexpr (BITS != 4) {   // the wave's rows into LDS, read back in slot order below
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<uint4 *>(lb + ((lane >> 3) + 8 * h) * kLbRow + 4 * (lane & 7)) = r.c[h];
    if constexpr (BITS == 3) *reinterpret_cast<uint4 *>(lb + (lane >> 2) * kLbRow + 32 + 4 * (lane & 3)) = r.c[2];
  }
  __builtin_amdgcn_wave_barrier();
  const int partner = (lane ^ 32) * 4;   // ds_bpermute address of slot q ^ 2
  const uint4 z = make_uint4(0, 0, 0, 0);
  uint32_t ex0 = 0, ex1 = 0;
  const NibbleMasks nm = nibble_masks();
  floatx4 tot = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int gi = 0; gi < kMGw; ++gi) {
    const int g = wave * kMGw + gi;
    // LDS operands first (columns 8..15 read columns 0..7 and are masked)
    const float xsg0 = xg[g * 8 + (j & 7)];
    const uint4 sv = *reinterpret_cast<const uint4 *>(sbl + gi * 16 + 4 * q);   // rows 4q .. 4q + 3
    const uint4 b0 = xb[((g * 2 + 0) * 4 + q) * 8 + (j & 7)];
    const uint4 b1 = xb[((g * 2 + 1) * 4 + q) * 8 + (j & 7)];
    half8 A0, A1;
    if constexpr (BITS == 4) {
      // the lane's two words of group g: its own lower pair for the group
      // its slot loaded, the partner slot's upper pair for the other one
      const uint4 v = r.c[gi / 2];
      const bool own = ((q >> 1) == (gi & 1));
      uint32_t w0 = v.x, w1 = v.y;
      if ((gi & 1) == 0) {   // one exchange serves both groups of the pair
        const uint32_t o0 = __builtin_amdgcn_ds_bpermute(partner, v.z);
        const uint32_t o1 = __builtin_amdgcn_ds_bpermute(partner, v.w);
        w0 = own ? v.x : o0;
        w1 = own ? v.y : o1;
        ex0 = o0;
        ex1 = o1;
      } else {
        w0 = own ? v.x : ex0;
        w1 = own ? v.y : ex1;
      }
      A0 = word_to_a(w0, nm);
      A1 = word_to_a(w1, nm);
    } else {
      // the slot's word of the group (codes 16 wq .. + 15) and, 3-bit, the
      // high bits of those codes: nibble wq % 2 of each byte of the high
      // word of chunk 2 gi + wq / 2
      const int wq = 2 * (q & 1) + ((q >> 1) ^ (gi & 1));
      const uint32_t *rowp = lb + (lane & 15) * kLbRow;
      const uint32_t w = rowp[4 * gi + wq];
      uint32_t hb = 0;
      if constexpr (BITS == 3) hb = (rowp[32 + 2 * gi + (wq >> 1)] >> (4 * (wq & 1))) & 0x0F0F0F0Fu;
      lowbit_to_a<BITS>(w, hb, A0, A1);
    }
    const half8 B0 = __builtin_bit_cast(half8, j < 8 ? b0 : z);
    const half8 B1 = __builtin_bit_cast(half8, j < 8 ? b1 : z);
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B1, acc, 0, 0, 0);
    const float xsg = j < 8 ? xsg0 : 0.0f;
    const uint32_t sw4[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] = fmaf(sb_scale(sw4[i]), acc[i], fmaf(sb_bias(sw4[i]), xsg, tot[i]));
  }
  // partial rows 4q + i, column j of this wave -> its slice; then row pairs
  __builtin_amdgcn_wave_barrier();
  if (j < 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) slice[(4 * q + i) * 8 + j] = tot[i];
  }
  __syncthreads();
  if (threadIdx.x < kTileRowPairs * NB) {
    const int p = threadIdx.x / NB, b = threadIdx.x % NB;
    float gs = 0.0f, us = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      gs += red[w * 128 + (2 * p) * 8 + b] + red[w * 128 + (2 * p) * 8 + 4 + b];
      us += red[w * 128 + (2 * p + 1) * 8 + b] + red[w * 128 + (2 * p + 1) * 8 + 4 + b];
    }
    const int j0 = x * a.W + unit * kTileRowPairs;
    st_dev(a.l.act + (size_t(act_slot) * kMaxNb + b) * I + j0 + p, tag_f32(ep, silu_mul(gs, us)));
  }
}

// The unit's act stores are issued by every wave: count it for the slice.
__device__ __forceinline__ void gate_up_signal(const LayerArgs &a, int x) {
  __syncthreads();   // every wave has issued its stores; red is free again
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(sw(a, x, kSliceGu), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NB, bool kLoaded = false>
__device__ __forceinline__ void run_gate_up_m(const LayerArgs &a, int x, uint64_t desc, int act_slot, int unit,
                                              const uint4 *xb, const float *xg, float *red, uint32_t *stg,
                                              uint32_t ep, GuRegsM &r) {
  if constexpr (!kLoaded) gate_up_load_m_any(a, desc, x, unit, r);
  switch (bits_of_tag(desc)) {
    case 4: gate_up_unit_m<NB, 4>(a, r, x, unit, act_slot, xb, xg, red, stg, ep); break;
    case 3: gate_up_unit_m<NB, 3>(a, r, x, unit, act_slot, xb, xg, red, stg, ep); break;
    default: gate_up_unit_m<NB, 2>(a, r, x, unit, act_slot, xb, xg, red, stg, ep); break;
  }
  gate_up_signal(a, x);
}

// A unit whose descriptor fails the record check: its act values are 0
// (status bit 0 tells the caller).
template <int NB>
__device__ __forceinline__ void gate_up_bad(const LayerArgs &a, int x, int act_slot, int unit, uint32_t ep) {
  const int lane = threadIdx.x & 63;
  const int j0 = gate_up_row0(a, x, unit);
  if (threadIdx.x == 0) set_status(a, 1u);
  if (lane < NB * kPairsPerWave)
    st_dev(a.l.act + (size_t(act_slot) * kMaxNb + lane / kPairsPerWave) * a.l.inter + j0 + lane % kPairsPerWave,
           tag_f32(ep, 0.0f));
  gate_up_signal(a, x);
}

// A gate/up unit on the kernel's path: kM kernels (two to four rows,
// H = 2048) run every unit on MFMA, the others on the VALU.
template <int NB, int CPL, bool kM>
__device__ __forceinline__ void gate_up_item(const LayerArgs &a, int x, uint64_t desc, int act_slot, int unit,
                                             const float *xs, const float *xsum, const uint4 *xb,
                                             const float *xg, float *red, uint32_t ep) {
  if constexpr (kM) {
    if (record_ok(desc, a.l.pool_bytes, a.l.hidden, a.l.inter)) {
      GuRegsM r;
      // x in f32 is dead once the B fragments are staged: its LDS takes the
      // 2/3-bit code rows
      run_gate_up_m<NB>(a, x, desc, act_slot, unit, xb, xg, red,
                        reinterpret_cast<uint32_t *>(const_cast<float *>(xs)), ep, r);
    } else {
      gate_up_bad<NB>(a, x, act_slot, unit, ep);
    }
  } else {
    GuRegs<CPL> r;
    run_gate_up<NB, CPL>(a, x, desc, act_slot, unit, xs, xsum, ep, r);
  }
}

// ----------------------------------------------------------------- exit
// Two-level exit count: a block counts itself out of its slice once it has
// made its last use of the counters (every block has read the call's epoch
// by then); the last block of a slice counts the slice out, and the last
// slice's block puts the counters back to zero and publishes the epoch.  A
// block whose last down tile it combines issues its slice-level count before
// the combine (which waits on epoch-tagged partials, not on counters) and
// reads the result after it: the count's round trip runs beside the combine.
__device__ __forceinline__ uint32_t exit_count_issue(const LayerArgs &a, int x) {
  __syncthreads();   // every thread is past its last counter use
  return threadIdx.x == 0 ? __hip_atomic_fetch_add(sw(a, x, kSliceExit), 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                          : 0u;
}
template <int NB>
__device__ __forceinline__ void exit_count_finish(const LayerArgs &a, Shared<NB> &sh, uint32_t prev) {
  if (threadIdx.x == 0) sh.prev = prev;
  __syncthreads();
  if (sh.prev == uint32_t(a.per_slice - 1)) {
    block_signal(a.l.sync + kSyncExit, 1u, &sh.prev);
    __syncthreads();
    if (sh.prev == uint32_t(kSlices - 1)) {   // every block has read the epoch: publish it
      for (int i = threadIdx.x; i < kSyncWords; i += kThreads)
        if (i != kSyncStatus) st_dev(a.l.sync + i, i == kSyncEpoch ? sh.ep : 0u);
    }
  }
}

// ----------------------------------------------------------------- down
// The block of slice tile % slices sums the tile's rows of every slice's
// partial in slice order (re-reading, boundedly, partials not yet of this
// call) into `out`.
template <int NB>
__device__ __forceinline__ void combine_tile(const LayerArgs &a, const Shared<NB> &sh, int x, int tile) {
  const int H = a.l.hidden;
  if (tile % a.n_slices == x) {   // this slice's block combines the tile's rows in slice order
    for (int i = threadIdx.x; i < kRowsPerTile * NB; i += kThreads) {
      const int b = i / kRowsPerTile, r = tile * kRowsPerTile + i % kRowsPerTile;
      uint64_t w[kSlices];
#pragma unroll
      for (int q = 0; q < kSlices; ++q)
        w[q] = q < a.n_slices ? ld_dev(a.l.opart + (size_t(q) * kMaxNb + b) * H + r) : 0;
      for (uint32_t it = 1;; ++it) {   // re-read the partials not yet of this call (bounded)
        bool all = true;
#pragma unroll
        for (int q = 0; q < kSlices; ++q) all &= q >= a.n_slices || uint32_t(w[q] >> 32) == sh.ep;
        if (all) break;
        // (no abort flag from here: the counters may already be reset for the
        // next call, which must not start aborted)
        if ((it & 63) == 0 && (ld_dev(a.l.sync + kSyncAbort) || it > kSpinLimit)) {
          set_status(a, 4u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int q = 0; q < kSlices; ++q)
          if (q < a.n_slices && uint32_t(w[q] >> 32) != sh.ep)
            w[q] = ld_dev(a.l.opart + (size_t(q) * kMaxNb + b) * H + r);
      }
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < kSlices; ++q)
        if (q < a.n_slices) v += __uint_as_float(uint32_t(w[q]));
      // part 1 adds to part 0's output (an earlier launch on the stream)
      a.l.out[size_t(b) * H + r] = a.part == 1 ? a.l.out[size_t(b) * H + r] + v : v;
    }
  }
  __syncthreads();
}


// A down tile: 32 output rows of the slice's columns, every slot.  Lane
// (row rw, chunk c, slot group g) of a wave handles row rw, 32-code chunk c
// of the slice, and slots g, g + SG, ...; weights for the lane's slots are
// loaded before the wait for the slice's gate/up units, the act chunks with
// device-coherent loads after it.
// The lane's down weights of one batch of slots (the batch starting at slot
// s0): code words and (scale, bias) words.  Addresses come from the pool
// argument and the host-computed section offsets (global loads, which LDS
// waits never wait for).
// Slots per lane per down batch: with one row the union has at most k + 1
// <= 16 slots, which four per lane cover at 64 columns per slice (and a
// shorter unrolled batch keeps the kernel's code small).
template <int NB>
constexpr int slot_batch() { return NB == 1 ? 4 : kSlotBatch; }

template <int NB>
struct DownRegs {
  uint32_t w[slot_batch<NB>()][4];
  uint32_t sbw[slot_batch<NB>()];
};

template <int NB>
__device__ __forceinline__ void down_load(const LayerArgs &a, const Shared<NB> &sh, int x, int tile, int s0,
                                          DownRegs<NB> &r) {
  constexpr int kSB = slot_batch<NB>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.l.hidden, W = a.W;
  const int cpr = W / kChunk, sg = 8 / cpr;
  const int idx = lane & 7;
  const int rw = lane >> 3, c = idx % cpr, g = idx / cpr;
  const int row = tile * kRowsPerTile + wave * kRowsPerWave + rw;
  const int col = x * W + c * kChunk;
  const int grp = col / kGroup, half = (col % kGroup) / kChunk;
  const int n_slots = sh.nsl;
  // section offsets read with constant indices (scalar loads of the kernel
  // arguments), then chosen per lane by the bits tag
  const uint32_t dc0 = a.d_codes[0], dc1 = a.d_codes[1], dc2 = a.d_codes[2];
  const uint32_t ds0 = a.d_sb[0], ds1 = a.d_sb[1], ds2 = a.d_sb[2];
#pragma unroll
  for (int m = 0; m < kSB; ++m) {
    const int slot = s0 + g + sg * m;
    r.w[m][0] = r.w[m][1] = r.w[m][2] = r.w[m][3] = 0;
    r.sbw[m] = 0;
    const int bt = slot < n_slots ? sh.dbits[slot] : 0;
    if (bt) {
      const uint64_t d = sh.desc[slot];
      const uint8_t *rec = a.l.pool + (d & ~uint64_t(255));
      const uint32_t dco = bt == 4 ? dc0 : (bt == 3 ? dc1 : dc2);
      const uint32_t dso = bt == 4 ? ds0 : (bt == 3 ? ds1 : ds2);
      const uint8_t *grow = rec + dco + (size_t(grp) * H + row) * (kGroup * bt / 8);
      if (__builtin_expect(bt == 4, 1)) load_chunk<4>(grow, kGroup, half, r.w[m]);
      else if (bt == 3) load_chunk<3>(grow, kGroup, half, r.w[m]);
      else load_chunk<2>(grow, kGroup, half, r.w[m]);
      r.sbw[m] = reinterpret_cast<const uint32_t *>(rec + dso)[size_t(grp) * H + row];
    }
  }
}

template <int NB>
__device__ __forceinline__ void publish_partial(const LayerArgs &a, Shared<NB> &sh, int x, int tile, float (&acc)[NB],
                                                bool last);

template <int NB>
__device__ __forceinline__ void run_down(const LayerArgs &a, Shared<NB> &sh, int x, int tile, float *act_lds,
                         float *asum_lds, bool last) {
  const int lane = threadIdx.x & 63;
  const int I = a.l.inter, W = a.W;
  const int cpr = W / kChunk;                 // chunks per row in the slice (1..8)
  const int sg = 8 / cpr;                     // slot groups per row
  const int idx = lane & 7;
  const int c = idx % cpr, g = idx / cpr;
  const int u = sh.u, n_slots = sh.nsl;
  constexpr int kSB = slot_batch<NB>();
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.0f;

  for (int s0 = 0; s0 < n_slots; s0 += sg * kSB) {
    // 1. this lane's weights for the batch
    DownRegs<NB> r;
    down_load<NB>(a, sh, x, tile, s0, r);
    uint32_t (&w)[kSB][4] = r.w;
    uint32_t (&sbw)[kSB] = r.sbw;
    // 2. the slice's act values must be complete
    if (s0 == 0) wait_geq(a, sw(a, x, kSliceGu), uint32_t(n_slots * a.ups));
    // 3. stage the batch's act chunks in LDS: one device-coherent 16-byte
    //    load per thread; 8 consecutive threads hold one 32-value chunk and
    //    form its sum with a DPP group-of-8 reduction
    const int nb_slots = min(n_slots - s0, sg * kSB);
    const int n_f4 = nb_slots * NB * (W / 4);
    __syncthreads();
    constexpr int kStIt = 4;   // loads in flight per thread
    for (int i0 = 0; i0 < n_f4; i0 += kStIt * kThreads) {
      uint64_t v[kStIt][4];
      uint32_t off[kStIt];
#pragma unroll
      for (int t = 0; t < kStIt; ++t) {   // unconditional loads keep v in registers
        const int i = min(i0 + t * kThreads + int(threadIdx.x), n_f4 - 1);
        const int q = i % (W / 4), b = (i / (W / 4)) % NB, sl = i / (W / 4) / NB;
        const int slot = s0 + sl;
        const int ps = slot < u ? slot : kSharedSlot;
        off[t] = uint32_t(((ps * kMaxNb + b) * I + x * W + 4 * q) * 8);
        ld_dev_u64x2(a.l.act, off[t], v[t][0], v[t][1]);
        ld_dev_u64x2(a.l.act, off[t] + 16, v[t][2], v[t][3]);
      }
      // values of an earlier call (the counter can run ahead of the stores)
      // are read again, boundedly
      for (uint32_t it = 1;; ++it) {
        bool stale = false;
#pragma unroll
        for (int t = 0; t < kStIt; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) stale |= uint32_t(v[t][e] >> 32) != sh.ep;
        if (!stale) break;
        if ((it & 63) == 0 && (ld_dev(a.l.sync + kSyncAbort) || it > kSpinLimit)) {
          st_dev(a.l.sync + kSyncAbort, 1u);
          set_status(a, 4u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int t = 0; t < kStIt; ++t) {
          ld_dev_u64x2(a.l.act, off[t], v[t][0], v[t][1]);
          ld_dev_u64x2(a.l.act, off[t] + 16, v[t][2], v[t][3]);
        }
      }
      float4 f[kStIt];
#pragma unroll
      for (int t = 0; t < kStIt; ++t)
        f[t] = i0 + t * kThreads + int(threadIdx.x) < n_f4
                   ? make_float4(__uint_as_float(uint32_t(v[t][0])), __uint_as_float(uint32_t(v[t][1])),
                                 __uint_as_float(uint32_t(v[t][2])), __uint_as_float(uint32_t(v[t][3])))
                   : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int t = 0; t < kStIt; ++t) {
        const int i = i0 + t * kThreads + threadIdx.x;
        if (i < n_f4) {
          const int q = i % (W / 4), b = (i / (W / 4)) % NB, sl = i / (W / 4) / NB;
          *reinterpret_cast<float4 *>(act_lds + (sl * NB + b) * (W + kStagePad) + 4 * q) = f[t];
        }
        const float cs = group8_sum((f[t].x + f[t].y) + (f[t].z + f[t].w));   // i = 8 chunk + (0..7)
        if (i < n_f4 && (i & 7) == 0) asum_lds[i >> 3] = cs;
      }
    }
    __syncthreads();
    // 4. accumulate the lane's slots
#pragma unroll
    for (int m = 0; m < kSB; ++m) {
      const int sl = g + sg * m;
      const int slot = s0 + sl;
      const int bt = slot < n_slots ? sh.dbits[slot] : 0;
      if (bt == 0) continue;
      float P[NB];
      // runs of W + 4 floats: the slot groups of a row read different banks
      const LdsX ax{act_lds + sl * NB * (W + kStagePad) + c * kChunk, W + kStagePad};
      if (__builtin_expect(bt == 4, 1)) chunk_dot<4, NB>(w[m], ax, P);
      else if (bt == 3) chunk_dot<3, NB>(w[m], ax, P);
      else chunk_dot<2, NB>(w[m], ax, P);
      const float sc = sb_scale(sbw[m]), bi = sb_bias(sbw[m]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = fmaf(sh.wslot[b][slot], fmaf(sc, P[b], bi * asum_lds[(sl * NB + b) * cpr + c]), acc[b]);
    }
  }
  publish_partial<NB>(a, sh, x, tile, acc, last);
}

// Sum the row's 8 lanes (chunks x slot groups) and publish the slice
// partial, tagged with this call's epoch: no wait and no counter, the
// combining block checks every partial's tag.  Then the tile's combine.
template <int NB>
__device__ __forceinline__ void publish_partial(const LayerArgs &a, Shared<NB> &sh, int x, int tile, float (&acc)[NB],
                                                bool last) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = group8_sum(acc[b]);
  const int H = a.l.hidden;
  const int row = tile * kRowsPerTile + (threadIdx.x >> 6) * kRowsPerWave + (lane >> 3);
  if ((threadIdx.x & 7) == 0)
#pragma unroll
    for (int b = 0; b < NB; ++b)
      st_dev(a.l.opart + (size_t(x) * kMaxNb + b) * H + row,
             (uint64_t(sh.ep) << 32) | __float_as_uint(acc[b]));

  const uint32_t prev = last ? exit_count_issue(a, x) : 0u;
  combine_tile<NB>(a, sh, x, tile);
  if (last) exit_count_finish<NB>(a, sh, prev);
}

// ------------------------------------------------------- down on MFMA
// In the MFMA kernels (W = 64: the slice's columns are one group of every
// down row) a down tile runs as MFMAs too.  A = 16 down rows x the slot's 64
// codes (the slot lane q holds codes 16q .. 16q + 15: step st takes codes
// 16q + 8st + (0,4,1,5,2,6,3,7), the order of the gate/up units), B = act
// of the slot as f16 high/low halves, staged per batch of slots straight
// into that fragment order.  Wave w takes row block w % 2 of the tile and
// the slots of parity w / 2; the two waves of a row block are summed in LDS.
constexpr int kDownSlots = 8;   // slots per wave per batch (2 kDownSlots per block)

template <int NB>
__device__ __forceinline__ void run_down_m(const LayerArgs &a, Shared<NB> &sh, int x, int tile, uint4 *frag,
                                           float *gsum, float *red, bool last) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.l.hidden, I = a.l.inter;
  const int q = lane >> 4, j = lane & 15;
  const int rb = wave & 1, par = wave >> 1;
  const int r0 = tile * kRowsPerTile + 16 * rb;   // the wave's 16 rows
  const int u = sh.u, n_slots = sh.nsl;
  floatx4 tot = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < n_slots; s0 += 2 * kDownSlots) {
    // 1. the lane's code words and the (scale, bias) words of its 4 output
    //    rows for the wave's slots of the batch
    uint2 cw[kDownSlots];
    uint4 sbv[kDownSlots];
#pragma unroll
    for (int m = 0; m < kDownSlots; ++m) {
      const int slot = s0 + par + 2 * m;
      const int bt = slot < n_slots ? sh.dbits[slot] : 0;
      cw[m] = make_uint2(0, 0);
      sbv[m] = make_uint4(0, 0, 0, 0);
      if (bt) {
        const uint8_t *grow = sh.dcodes[slot] + (size_t(x) * H + r0 + (lane & 15)) * (kGroup * bt / 8);
        if (bt == 4) {
          cw[m] = *reinterpret_cast<const uint2 *>(grow + 8 * q);
        } else {
          cw[m].x = *reinterpret_cast<const uint32_t *>(grow + 4 * q);
          if (bt == 3) cw[m].y = *reinterpret_cast<const uint32_t *>(grow + 16 + 4 * (q >> 1));
        }
        sbv[m] = *reinterpret_cast<const uint4 *>(sh.dsb[slot] + size_t(x) * H + r0 + 4 * q);
      }
    }
    // 2. the slice's act values must be complete
    if (s0 == 0) wait_geq(a, sw(a, x, kSliceGu), uint32_t(n_slots * a.ups));
    // 3. stage the batch's act as B fragments: item = (slot, row b, block
    //    of 8 columns); one device-coherent pass of 8 tagged values each,
    //    high and low halves in fragment order, and the slot's column sums
    const int nbs = min(n_slots - s0, 2 * kDownSlots);
    const int n_items = nbs * NB * 8;
    __syncthreads();
    for (int i0 = 0; i0 < n_items; i0 += kThreads) {   // every lane runs the DPP sum
      const int i = i0 + threadIdx.x;
      const int ic = min(i, n_items - 1);
      const int blk = ic & 7, b = (ic >> 3) % NB, sl = (ic >> 3) / NB;
      const int slot = s0 + sl;
      const int ps = slot < u ? slot : kSharedSlot;
      const uint32_t off = uint32_t(((ps * kMaxNb + b) * I + x * kGroup + 8 * blk) * 8);
      uint64_t v[8];
#pragma unroll
      for (int t = 0; t < 4; ++t) ld_dev_u64x2(a.l.act, off + 16 * t, v[2 * t], v[2 * t + 1]);
      for (uint32_t it = 1;; ++it) {   // values of an earlier call are read again (bounded)
        bool stale = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) stale |= uint32_t(v[e] >> 32) != sh.ep;
        if (!stale) break;
        if ((it & 63) == 0 && (ld_dev(a.l.sync + kSyncAbort) || it > kSpinLimit)) {
          st_dev(a.l.sync + kSyncAbort, 1u);
          set_status(a, 4u);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int t = 0; t < 4; ++t) ld_dev_u64x2(a.l.act, off + 16 * t, v[2 * t], v[2 * t + 1]);
      }
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = i < n_items ? __uint_as_float(uint32_t(v[e])) : 0.0f;
      half8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float fv = f[(e & 1) * 4 + (e >> 1)];   // element e holds column (0,4,1,5,2,6,3,7)[e]
        hi[e] = _Float16(fv);
        lo[e] = _Float16(fv - float(hi[e]));
      }
      if (i < n_items) {
        const int fi = ((sl * 2 + (blk & 1)) * 4 + (blk >> 1)) * 8 + b;
        frag[fi] = __builtin_bit_cast(uint4, hi);
        frag[fi + 4] = __builtin_bit_cast(uint4, lo);
      }
      const float cs = group8_sum(((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7])));
      if (i < n_items && blk == 0) gsum[sl * 4 + b] = cs;
    }
    __syncthreads();
    // 4. the wave's slots
    const NibbleMasks nm = nibble_masks();
#pragma unroll
    for (int m = 0; m < kDownSlots; ++m) {
      const int sl = par + 2 * m, slot = s0 + sl;
      const int bt = slot < n_slots ? sh.dbits[slot] : 0;
      if (bt == 0) continue;
      half8 A0, A1;
      if (bt == 4) {
        A0 = word_to_a(cw[m].x, nm);
        A1 = word_to_a(cw[m].y, nm);
      } else {
        // 3-bit: the high bits of the slot word's codes are nibble q % 2 of
        // each byte of its chunk's high word
        const uint32_t hb = bt == 3 ? (cw[m].y >> (4 * (q & 1))) & 0x0F0F0F0Fu : 0u;
        if (bt == 3) lowbit_to_a<3>(cw[m].x, hb, A0, A1);
        else lowbit_to_a<2>(cw[m].x, 0u, A0, A1);
      }
      const uint4 b0 = frag[((sl * 2 + 0) * 4 + q) * 8 + (j & 7)];
      const uint4 b1 = frag[((sl * 2 + 1) * 4 + q) * 8 + (j & 7)];
      // column j < 4: high half of row j (with the bias term); 4..7: low
      // half; 8..15 and rows past NB (never staged): nothing
      const bool live = j < 8 && (j & 3) < NB;
      const uint4 z = make_uint4(0, 0, 0, 0);
      floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, __builtin_bit_cast(half8, live ? b0 : z), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, __builtin_bit_cast(half8, live ? b1 : z), acc, 0, 0, 0);
      const float wsl = live ? sh.wslot[(j & 3) < NB ? (j & 3) : 0][slot] : 0.0f;
      const float gs = live && j < 4 ? gsum[sl * 4 + (j & 3)] : 0.0f;
      const uint32_t s4[4] = {sbv[m].x, sbv[m].y, sbv[m].z, sbv[m].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[i] = fmaf(wsl, fmaf(sb_scale(s4[i]), acc[i], sb_bias(s4[i]) * gs), tot[i]);
    }
  }
  // rows 4q + i, column j of the wave -> LDS; a row's value for row b of x
  // is the sum over both parity waves of columns b and 4 + b
  __syncthreads();
  if (j < 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 16 + 4 * q + i) * 8 + j] = tot[i];
  }
  __syncthreads();
  if (threadIdx.x < kRowsPerTile * NB) {
    const int rr = threadIdx.x % kRowsPerTile, b = threadIdx.x / kRowsPerTile;
    const int rbk = rr / 16, r = rr % 16;
    float v = 0.0f;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int w = rbk + 2 * pr;
      v += red[(w * 16 + r) * 8 + b] + red[(w * 16 + r) * 8 + 4 + b];
    }
    st_dev(a.l.opart + (size_t(x) * kMaxNb + b) * H + tile * kRowsPerTile + rr,
           (uint64_t(sh.ep) << 32) | __float_as_uint(v));
  }
  const uint32_t prev = last ? exit_count_issue(a, x) : 0u;
  combine_tile<NB>(a, sh, x, tile);
  if (last) exit_count_finish<NB>(a, sh, prev);
}

// The nb rows of x into LDS, chunk-major (ChunkX), and their per-32 sums.
// All of a thread's loads are in flight at once.
// An empty asm that takes every loaded value as a read-write register
// operand: all of the loads are issued before it and nothing that uses them
// moves above it (no memory clobber, so the values stay in registers).
__device__ __forceinline__ void pin_loaded(floatx4 (&v)[2]) { asm volatile("" : "+v"(v[0]), "+v"(v[1])); }
__device__ __forceinline__ void pin_loaded(floatx4 (&v)[4]) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}
__device__ __forceinline__ void pin_loaded(floatx4 (&v)[6]) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]));
}
__device__ __forceinline__ void pin_loaded(floatx4 (&v)[8]) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
               "+v"(v[7]));
}
__device__ __forceinline__ void pin_loaded(floatx4 (&v)[12]) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
               "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]));
}
__device__ __forceinline__ void pin_loaded(floatx4 (&v)[16]) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
               "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]),
               "+v"(v[14]), "+v"(v[15]));
}

// The descriptor table (rec_dst, when not null: rv per thread) and the call's
// epoch (ep_dst: the workspace's last epoch + 1, never 0) go to LDS together
// with x, under the same barrier.
template <int NB, int CPL>
__device__ __forceinline__ void stage_x(const LayerArgs &a, float *xs, float *xsum, uint64_t *rec_dst, uint64_t rv,
                                        uint32_t *ep_dst) {
  uint32_t ep_next = 0;
  const int H = a.l.hidden;
  {   // all of the thread's x loads in flight at once (H <= 2048 CPL)
    constexpr int kXIt = 2 * NB * CPL;
    floatx4 xv[kXIt];
#pragma unroll
    for (int t = 0; t < kXIt; ++t) {   // unconditional loads keep xv in registers
      const int i = min((threadIdx.x + t * kThreads) * 4, NB * H - 4);
      xv[t] = *reinterpret_cast<const floatx4 *>(a.l.x + i);
    }
    // the call's epoch, read by wave 0 (one device-coherent read per block)
    // while the x loads are in flight
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0) ep_next = ld_dev(a.l.sync + kSyncEpoch) + 1u;
    // every load ahead of the first write (left alone, the scheduler pairs
    // each load with its write: one round trip per load)
    pin_loaded(xv);
    const int nch = H / kChunk;
#pragma unroll
    for (int t = 0; t < kXIt; ++t) {   // float4 f of row b -> group f % 8 of chunk f / 8
      // unconditional writes (a guarded write lets the compiler sink its load
      // into the branch, one round trip per load): past the rows, into the
      // pad slot of the first LDS row, which is never read
      const int i = threadIdx.x + t * kThreads, rq = H / 4;
      const int b = int(i >= rq) + int(i >= 2 * rq) + int(i >= 3 * rq);   // row (nb <= 4), no division
      const int f = i - b * rq;
      const int at = i * 4 < NB * H ? (b * 8 + f % 8) * (nch + kXPad) + f / 8 : nch;
      reinterpret_cast<floatx4 *>(xs)[at] = xv[t];
    }
  }
  if (rec_dst && int(threadIdx.x) < a.l.n_experts) rec_dst[threadIdx.x] = rv;
  if (threadIdx.x == 0) *ep_dst = ep_next ? ep_next : 1u;
  __syncthreads();
  for (int i = threadIdx.x; i < NB * (H / kChunk); i += kThreads) {   // per-32 sums
    const int b = i / (H / kChunk), c = i - b * (H / kChunk);
    const ChunkX X{reinterpret_cast<const float4 *>(xs), H / kChunk, c};
    float sm = 0.0f;
#pragma unroll
    for (int q = 0; q < kChunk / 4; ++q) {
      const float4 f = X(b, q);
      sm += (f.x + f.y) + (f.z + f.w);
    }
    xsum[i] = sm;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- kernel
template <int NB, int CPL, bool kM>
__global__ __launch_bounds__(kThreads, 2) void layer_kernel(LayerArgs a) {
  extern __shared__ float4 dyn[];
  __shared__ Shared<NB> sh;
  __shared__ uint64_t rec_lds[kMaxExperts];
  const int H = a.l.hidden;
  // x and its sums live until the block's last gate/up unit; a block takes
  // its down tiles after all of its gate/up units, so the act staging of the
  // down tiles reuses that space.
  float *xs = reinterpret_cast<float *>(dyn);           // [NB][H]
  float *xsum = xs + x_lds_floats(NB, H);               // [NB][H/32]
  // MFMA gate/up operands after the sums: B fragments, group sums, the
  // waves' partial rows
  uint4 *xb = reinterpret_cast<uint4 *>(xsum + NB * (H / kChunk));
  float *xg = reinterpret_cast<float *>(xb) + (kM ? kMG * 256 : 0);
  float *red = xg + kMG * 8;
  float *act_lds = xs;                                  // [batch slots][NB][W + pad]
  float *asum_lds = act_lds + kStageFloats * NB;       // [batch slots][NB][W/32]

  const int x = blockIdx.x % kSlices, lr = blockIdx.x / kSlices;
  const int P = a.per_slice;
  bool counted = false;   // counted out of the slice with its last down tile
  // this call's epoch (tags the slice partials; never 0, the workspace's
  // initial tag) is read while x is staged (stage_x)


  if (x < a.n_slices) {
    // router blocks g < G are spread over the slices; R of them are in this
    // one (none for a part of a published table: route_blocks is 0)
    const bool tbl = a.part >= 0;
    const int g = lr * a.n_slices + x;
    const bool route = g < a.route_blocks;
    const int R = x < a.route_blocks ? (a.route_blocks - 1 - x) / a.n_slices + 1 : 0;
    RouterRow<CPL> rrow;
    if (route) router_prefetch<CPL>(a, g, rrow);
    // Blocks that neither compute router rows nor run a shared-expert unit
    // need x and the descriptors only after routing: they load them after a
    // short sleep, so that the router blocks' loads of the same lines do not
    // queue behind hundreds of identical requests.
    if (!tbl && !route && ((lr - R) % P + P) % P >= a.ups) __builtin_amdgcn_s_sleep(kLateStageSleep);
    // the descriptors go to LDS with x, so that no wait for them holds up
    // the x loads
    const uint64_t rv = tbl ? 0 : a.l.rec[min(int(threadIdx.x), a.l.n_experts - 1)];
    stage_x<NB, CPL>(a, xs, xsum, tbl ? nullptr : rec_lds, rv, &sh.ep);

    double *lg = a.l.slice_logits;
    float *gm = a.l.slice_gamma;
    if (route) {
      router_rows<NB, CPL>(a, xs, g, rrow, lg, gm);
      // every slice counts the router blocks (one counter per slice)
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x < a.n_slices)
        __hip_atomic_fetch_add(sw(a, threadIdx.x, kSliceRoute), 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if constexpr (kM) {   // after the router rows: they are on the routing path
      stage_x_fragments<NB>(a, xs, xsum, xb, xg);
      __syncthreads();
    }
    // the shared expert's gate/up units need no routing (part 1 has none)
    const int shared_units = a.part == 1 ? 0 : a.ups;
    for (int i = ((lr - R) % P + P) % P; i < shared_units; i += P)
      gate_up_item<NB, CPL, kM>(a, x, a.l.shared_rec, kSharedSlot, i, xs, xsum, xb, xg, red, sh.ep);

    if (!tbl) {
      wait_geq(a, sw(a, x, kSliceRoute), uint32_t(a.route_blocks));
      route_select<NB>(a, sh, lg, gm);
    }
    // the block's work items i0, i0 + P, ...: gate/up units first, then down
    // tiles (two loops, so neither carries the other's live values).  When
    // the first unit's slot is one of row 0's ranks its expert is known
    // already: its weights load while the union is built.
    int i = ((lr - R - a.ups) % P + P) % P;
    const int slot0 = i / a.ups;
    const bool early = !tbl && slot0 < a.l.top_k;
    uint64_t d0 = 0;
    if (early) d0 = rec_lds[sh.sel[0][slot0]];
    if constexpr (kM) {
      // the block's units i, i + P, ... < n_gu run as a pipeline: the next
      // unit's weights are in flight while the current one computes.  When
      // the first unit's slot is one of row 0's ranks (a 4-bit record: the
      // early loads stay out of the other widths' register budget) its
      // weights load while the union is built.
      GuRegsM cur, nxt;
      const bool em = early && bits_of_tag(d0) == 4 && record_ok(d0, a.l.pool_bytes, a.l.hidden, a.l.inter);
      if (em) gate_up_load_m<4>(a, d0, x, i - slot0 * a.ups, cur);
      asm volatile("" ::: "memory");   // the loads are issued here, not sunk to their use
      build_slots<NB>(a, sh, rec_lds);
      const int n_gu0 = sh.u * a.ups;
      auto load_unit = [&](int it, GuRegsM &r) {
        const int slot = it / a.ups;
        const uint64_t d = sh.desc[slot];
        if (record_ok(d, a.l.pool_bytes, a.l.hidden, a.l.inter)) gate_up_load_m_any(a, d, x, it - slot * a.ups, r);
      };
      if (!em && i < n_gu0) load_unit(i, cur);
      while (i < n_gu0) {
        const int nx = i + P;
        if (nx < n_gu0) load_unit(nx, nxt);
        asm volatile("" ::: "memory");
        const int slot = i / a.ups, unit = i - slot * a.ups;
        const uint64_t d = sh.desc[slot];
        uint32_t *stg = reinterpret_cast<uint32_t *>(xs);
        if (record_ok(d, a.l.pool_bytes, a.l.hidden, a.l.inter)) {
          switch (bits_of_tag(d)) {
            case 4: gate_up_unit_m<NB, 4>(a, cur, x, unit, slot, xb, xg, red, stg, sh.ep); break;
            case 3: gate_up_unit_m<NB, 3>(a, cur, x, unit, slot, xb, xg, red, stg, sh.ep); break;
            default: gate_up_unit_m<NB, 2>(a, cur, x, unit, slot, xb, xg, red, stg, sh.ep); break;
          }
          gate_up_signal(a, x);
        } else {
          gate_up_bad<NB>(a, x, slot, unit, sh.ep);
        }
        cur = nxt;
        i = nx;
      }
    } else {
      GuRegs<CPL> pre;
      if (early && record_ok(d0, a.l.pool_bytes, a.l.hidden, a.l.inter))
        gate_up_load_any<CPL>(a, d0, gate_up_row0(a, x, i - slot0 * a.ups), pre);
      asm volatile("" ::: "memory");   // the loads are issued here, not sunk to their use
      build_slots<NB>(a, sh, rec_lds);
      const int n_gu = sh.u * a.ups;
      if (early) {   // slot0 < k <= u: a gate/up unit
        run_gate_up<NB, CPL, true>(a, x, d0, slot0, i - slot0 * a.ups, xs, xsum, sh.ep, pre);
        i += P;
      }
      for (; i < n_gu; i += P) {
        const int slot = i / a.ups;
        gate_up_item<NB, CPL, kM>(a, x, sh.desc[slot], slot, i - slot * a.ups, xs, xsum, xb, xg, red, sh.ep);
      }
      for (; i < n_gu + a.tiles; i += P) {
        counted = true;
        run_down<NB>(a, sh, x, i - n_gu, act_lds, asum_lds, i + P >= n_gu + a.tiles);
      }
    }
    if constexpr (kM) {
      const int n_gu = sh.u * a.ups;
      for (; i < n_gu + a.tiles; i += P) {
        counted = true;
        run_down_m<NB>(a, sh, x, i - n_gu, xb, xg, red, i + P >= n_gu + a.tiles);
      }
    }
  } else if (threadIdx.x == 0) {
    // a block of a slice without columns (I < 8 * 32) still reads the call's
    // epoch: whichever block leaves last publishes its copy
    const uint32_t e = ld_dev(a.l.sync + kSyncEpoch) + 1u;
    sh.ep = e ? e : 1u;
  }

  // a block without down tiles counts itself out here (the others did
  // with their last tile)
  if (!counted) exit_count_finish<NB>(a, sh, exit_count_issue(a, x));
}

// moe_route: the routing steps of the layer kernel alone.  Every block is a
// router block (rows 4 g .. of router block g); block 0 then selects each
// row's top-k, builds the union and writes the caller's tables, exactly as
// block 0 of the layer kernel does.
template <int NB, int CPL>
__global__ __launch_bounds__(kThreads) void route_kernel(LayerArgs a) {
  extern __shared__ float4 dyn[];
  __shared__ Shared<NB> sh;
  __shared__ uint64_t rec_lds[kMaxExperts];
  const int H = a.l.hidden;
  float *xs = reinterpret_cast<float *>(dyn);           // [NB][H]
  float *xsum = xs + x_lds_floats(NB, H);               // [NB][H/32]

  const int g = blockIdx.x;
  RouterRow<CPL> rrow;
  router_prefetch<CPL>(a, g, rrow);
  const uint64_t rv = a.l.rec[min(int(threadIdx.x), a.l.n_experts - 1)];
  stage_x<NB, CPL>(a, xs, xsum, g == 0 ? rec_lds : nullptr, rv, &sh.ep);
  router_rows<NB, CPL>(a, xs, g, rrow, a.l.slice_logits, a.l.slice_gamma);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(sw(a, 0, kSliceRoute), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (g == 0) {
    wait_geq(a, sw(a, 0, kSliceRoute), uint32_t(gridDim.x));
    route_select<NB>(a, sh, a.l.slice_logits, a.l.slice_gamma);
    route_union<NB>(a, sh, rec_lds);
  }
  // the last block out publishes the epoch and resets the counters
  block_signal(a.l.sync + kSyncExit, 1u, &sh.prev);
  __syncthreads();
  if (sh.prev == gridDim.x - 1)
    for (int i = threadIdx.x; i < kSyncWords; i += kThreads)
      if (i != kSyncStatus) st_dev(a.l.sync + i, i == kSyncEpoch ? sh.ep : 0u);
}

size_t dyn_lds_bytes(int nb, int hidden, bool mfma) {
  // x and its per-32 sums (and with MFMA gate/up units the B
  // fragments, group sums and partial rows); or one batch of staged act
  // chunks and their sums
  const size_t xk = sizeof(float) * (size_t(x_lds_floats(nb, hidden)) + size_t(nb) * (hidden / kChunk)) +
                    (mfma ? size_t(kMG) * (1024 + 32) + sizeof(float) * kWaves * 128 : 0);
  const size_t st = sizeof(float) * (size_t(kStageFloats) * nb + size_t(8) * kSlotBatch * nb);
  return xk > st ? xk : st;
}

struct LaunchCache {
  int device = -1;
  int blocks_per_cu[kMaxNb + 1][3][2] = {};
  int cus = 0;
};
thread_local LaunchCache g_cache;

template <int NB, int CPL, bool kM>
hipError_t launch_nb(LayerArgs &a, hipStream_t s) {
  const size_t lds = dyn_lds_bytes(NB, a.l.hidden, kM);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (g_cache.device != dev) {
    g_cache = LaunchCache();
    g_cache.device = dev;
    e = hipDeviceGetAttribute(&g_cache.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  int &per_cu = g_cache.blocks_per_cu[NB][CPL][kM];
  if (per_cu == 0) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, layer_kernel<NB, CPL, kM>, kThreads,
                                                     dyn_lds_bytes(NB, CPL * 64 * kChunk, kM));
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    if (per_cu > 2) per_cu = 2;
  }
  const int grid = (per_cu * g_cache.cus) / kSlices * kSlices;
  a.per_slice = grid / kSlices;
  a.route_blocks = a.part >= 0 ? 0 : min(a.per_slice * a.n_slices, (a.l.n_experts + 1 + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((layer_kernel<NB, CPL, kM>), dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int NB, int CPL>
hipError_t launch_route_nb(LayerArgs &a, hipStream_t s) {
  const int H = a.l.hidden;
  const size_t lds = sizeof(float) * (size_t(x_lds_floats(NB, H)) + size_t(NB) * (H / kChunk));
  hipLaunchKernelGGL((route_kernel<NB, CPL>), dim3(a.route_blocks), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_only(const LayerLaunch &l, hipStream_t s) {
  LayerArgs a{};
  a.l = l;
  a.part = -1;
  a.n_slices = 1;
  a.route_blocks = (l.n_experts + 1 + kWaves - 1) / kWaves;
  a.per_slice = a.route_blocks;
  const bool two = l.hidden > 64 * kChunk;
  switch (l.nb) {
    case 1: return two ? launch_route_nb<1, 2>(a, s) : launch_route_nb<1, 1>(a, s);
    case 2: return two ? launch_route_nb<2, 2>(a, s) : launch_route_nb<2, 1>(a, s);
    case 3: return two ? launch_route_nb<3, 2>(a, s) : launch_route_nb<3, 1>(a, s);
    default: return two ? launch_route_nb<4, 2>(a, s) : launch_route_nb<4, 1>(a, s);
  }
}

hipError_t launch_layer(const LayerLaunch &l, hipStream_t s, int part) {
  LayerArgs a{};
  a.l = l;
  a.part = part;
  a.n_slices = min(kSlices, l.inter / kChunk);
  a.W = l.inter / a.n_slices;
  a.ups = a.W / kTileRowPairs;
  a.tiles = l.hidden / kRowsPerTile;
  if (a.tiles > kMaxDownTiles || a.W / kChunk > 8 || a.W % kTileRowPairs) return hipErrorInvalidValue;
  for (int tag = 0; tag < 3; ++tag) {
    const RecordLayout L = record_layout(l.hidden, l.inter, 4 - tag);
    a.d_codes[tag] = uint32_t(L.d_codes);
    a.d_sb[tag] = uint32_t(L.d_sb);
  }
  const bool two = l.hidden > 64 * kChunk;
  // two to four rows at H = 2048 and 64 columns per slice: gate/up units and
  // down tiles on MFMA
  const bool mfma = l.hidden == kMfmaHidden && a.W == kGroup;
  switch (l.nb) {
    case 1: return two ? launch_nb<1, 2, false>(a, s) : launch_nb<1, 1, false>(a, s);
    case 2: return two ? launch_nb<2, 2, false>(a, s) : mfma ? launch_nb<2, 1, true>(a, s) : launch_nb<2, 1, false>(a, s);
    case 3: return two ? launch_nb<3, 2, false>(a, s) : mfma ? launch_nb<3, 1, true>(a, s) : launch_nb<3, 1, false>(a, s);
    default: return two ? launch_nb<4, 2, false>(a, s) : mfma ? launch_nb<4, 1, true>(a, s) : launch_nb<4, 1, false>(a, s);
  }
}

}  // namespace moe
