// Internal declarations of the MoE HIP library (gfx950 only).
//
// Everything here belongs to the device path; the CPU oracle has its own
// record reader and arithmetic and shares none of this.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kGroup = 64;        // codes per (scale, bias) group along the input dim
constexpr int kChunk = 32;        // codes one lane handles per row step
constexpr int kSlotStride = MOE_SLOT_STRIDE;
constexpr int kMaxNb = MOE_MAX_NB;
constexpr int kSharedSlot = 63;   // act / partial index used for the shared expert
constexpr int kMaxExperts = 256;
constexpr int kJobInts = 4;   // prefill sub-job record (ints), after a header of the same size
constexpr int kMaxTopK = 15;

// ----------------------------------------------------------- record layout
__host__ __device__ inline uint64_t align256(uint64_t n) { return (n + 255) & ~uint64_t(255); }

struct RecordLayout {
  uint64_t gu_codes, gu_sb, d_codes, d_sb, total;
  uint32_t gu_row_bytes, d_row_bytes;
};

__host__ __device__ inline RecordLayout record_layout(int hidden, int inter, int bits) {
  RecordLayout r;
  r.gu_row_bytes = uint32_t(hidden) * bits / 8;
  r.d_row_bytes = uint32_t(inter) * bits / 8;
  r.gu_codes = 0;
  r.gu_sb = align256(uint64_t(2 * inter) * r.gu_row_bytes);
  r.d_codes = r.gu_sb + align256(uint64_t(2 * inter) * (hidden / kGroup) * 4);
  r.d_sb = r.d_codes + align256(uint64_t(hidden) * r.d_row_bytes);
  r.total = r.d_sb + align256(uint64_t(hidden) * (inter / kGroup) * 4);
  return r;
}

__host__ __device__ inline int bits_of_tag(uint64_t desc) {
  uint32_t t = uint32_t(desc & 3u);
  return t == 0 ? 4 : (t == 1 ? 3 : (t == 2 ? 2 : 0));
}

// ------------------------------------------------------------ arguments
// One decode layer launch (the fused persistent kernel of layer.hip).
struct LayerLaunch {
  const float *x;            // [nb][H]
  int nb;
  const uint16_t *router;    // [E][H] bf16
  const uint16_t *gvec;      // [H] bf16
  const uint64_t *rec;       // [E]
  const uint8_t *pool;
  uint64_t pool_bytes;
  uint64_t shared_rec;
  int hidden, inter, n_experts, top_k;
  double *logits;            // [nb][E]
  float *gamma;              // [nb]
  uint32_t *topk_idx;        // [nb][k]
  float *topk_w;             // [nb][k]
  uint64_t *tab;             // [64]
  float *wmap;               // [4][64]
  uint32_t *ids;             // [64]
  float *out;                // [nb][H]
  uint32_t *sync;            // 256 counter words (workspace head)
  uint64_t *act;             // [64][4][I]  epoch << 32 | f32 bits
  uint64_t *opart;           // [8][4][H]  per-slice partial outputs: epoch << 32 | f32 bits
  double *slice_logits;      // [8][4][256] per-slice router logits
  float *slice_gamma;        // [8][4]
};

// Workspace layout (decode and prefill share the head).
struct WorkspaceLayout {
  size_t counters;     // kSyncWords u32 counter / status words
  size_t act;          // decode: [64][4][I] epoch-tagged f32
  size_t opart;        // decode: [8][4][H] per-slice partial outputs (epoch-tagged f32)
  size_t slice_logits; // decode: [8][4][256] f64, [8][4] f32 gamma after it
  size_t pf_xf;        // prefill: [2 orders][hi, lo][32][H] f16 MFMA-ordered x
  size_t pf_xg;        // prefill: [32][H/64] f32 group sums of x
  size_t pf_act;       // prefill: [hi, lo][t*k + t][I] f16 MFMA-ordered act per entry
  int pf_act_rows;     // entries pf_act holds
  size_t pf_asum;      // prefill: [t*k + t][I/32] f32 sums of 32-column act blocks
  size_t pf_y;         // prefill: [t][k+1][H] f32 weighted outputs per (row, rank)
  size_t pf_meta;      // prefill: sub-job count, then one 32-byte record per sub-job
  size_t total;
};

WorkspaceLayout workspace_layout(int hidden, int inter, int n_experts, int top_k, int rows);

// Counter block at the workspace head: kSyncWords u32 words.  Words that
// many blocks poll sit on their own 128-byte lines.
constexpr int kSyncWords = 1024;
constexpr int kSlices = 8;                  // logical XCDs of the decode kernel
constexpr int kSyncSliceStride = 64;        // slice x owns words [64x, 64x + 64)
constexpr int kSliceRoute = 0;              //   router blocks of the slice arrived
constexpr int kSliceGu = 32;                //   gate/up units of the slice done
constexpr int kSliceExit = 48;              //   blocks of the slice that left
constexpr int kSyncStatus = 520;            // bit 0: bad descriptor skipped; bit 2: a wait ran out
constexpr int kSyncExit = 528;              // slices whose blocks all left
constexpr int kSyncAbort = 576;             // set when a wait ran out: all waits fall through
constexpr int kSyncEpoch = 608;             // decode: number of the last finished call (tags data)
constexpr int kMaxDownTiles = 256;

// ------------------------------------------------------------- launchers
hipError_t launch_route_only(const LayerLaunch &l, hipStream_t s);   // moe_route
// part -1: route and run the layer; 0 / 1: a part of the published slot table
hipError_t launch_layer(const LayerLaunch &l, hipStream_t s, int part = -1);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_repack(const uint8_t *src, uint64_t src_bytes, const uint64_t *src_desc, uint8_t *dst,
                         uint64_t dst_bytes, const uint64_t *dst_desc, int n, int hidden, int inter,
                         uint32_t *status, hipStream_t s);

struct PrefillArgs {
  const uint8_t *pool;
  uint64_t pool_bytes;
  const float *x;              // [t][H]
  const uint64_t *rec;         // [E]
  uint64_t shared_rec;
  const uint32_t *topk_idx;    // [t][k]
  int32_t *expert_ptr;         // [E+1]  (written by the gate/up pass)
  int32_t *entry_row;          // [t*k]
  int32_t *entry_rank;         // [t*k]
  float *topk_w;               // [t][k]
  const float *gamma;          // [t]
  int hidden, inter, n_experts, top_k, t;
  _Float16 *xf;                // [2 orders][hi, lo][32][H]: x split in f16 halves, MFMA order
  float *xg;                   // [32][H/64] group sums of x
  _Float16 *act;               // [hi, lo][act_rows][I]: silu(g)*u per entry, same split and order
  float *asum;                 // [act_rows][I/32] sums of act over 32-column blocks
  int act_rows;                // entries the act buffer holds (shared entries last)
  float *y;                    // [t][k+1][H] weighted output per (row, rank); rank k = shared
  int32_t *meta;               // [0] sub-job count; sub-job s at 4 + 4 s: expert (-1 = shared),
                               // first entry | rows << 16, descriptor (two words); written by
                               // the gate/up pass for the down pass
  uint32_t *status;
  float *out;                  // [t][H]
};
hipError_t launch_prefill(const PrefillArgs &a, const uint16_t *router, const uint16_t *gvec,
                          double *logits, float *gamma, uint32_t *topk_idx, hipStream_t s,
                          hipEvent_t *stage_ev, int n_ev);


}  // namespace moe
