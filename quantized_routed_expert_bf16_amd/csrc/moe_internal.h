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
struct RouteArgs {
  const float *x;          // [rows][H]
  const uint16_t *router;  // [E][H] bf16
  const uint16_t *gvec;    // [H] bf16
  const uint64_t *rec;     // [E]
  int hidden, n_experts, top_k, rows;
  double *logits;          // [rows][E]
  float *gamma;            // [rows]
  uint32_t *topk_idx;      // [rows][k]
  float *topk_w;           // [rows][k]
  // decode outputs (may be null for prefill)
  uint64_t *tab;           // [64]
  float *wmap;             // [4][64]
  uint32_t *ids;           // [64]
  // prefill outputs (may be null for decode)
  int32_t *expert_ptr;     // [E+1]
  int32_t *entry_row;      // [t*k]
  int32_t *entry_rank;     // [t*k]
  uint32_t *counter;       // one zero-initialised word, reset by the last block
};

struct ExpertArgs {
  const uint8_t *pool;
  uint64_t pool_bytes;
  const float *x;          // [nb][H]
  const uint64_t *tab;     // [64] slot table written by the route kernel
  const float *wmap;       // [4][64]
  const float *gamma;      // [nb]
  uint64_t shared_rec;
  int hidden, inter;
  float *act;              // [64][4][I]  silu(g)*u per slot and row
  float *ypart;            // [64][4][H]  weighted down output per slot and row
  uint32_t *tile_count;    // [H / rows-per-tile] zero-initialised counters
  uint32_t *status;        // bit 0: a descriptor was out of range
  float *out;              // [nb][H]
};

// Workspace layout (decode and prefill share the head).
struct WorkspaceLayout {
  size_t counters;     // 256 u32 counter / status words
  size_t act;          // decode: [64][4][I] f32
  size_t ypart;        // decode: [64][4][H] f32
  size_t pf_xh;        // prefill: [32][H] f16 activations
  size_t pf_act;       // prefill: [t*k + t][I] f16 activations per CSR entry
  size_t pf_y;         // prefill: [t][k+1][H] f32 weighted outputs per (row, rank)
  size_t total;
};

WorkspaceLayout workspace_layout(int hidden, int inter, int n_experts, int top_k, int rows);

// word indices inside the counter block
constexpr int kCounterRoute = 0;
constexpr int kCounterStatus = 1;
constexpr int kCounterTiles = 64;   // 64..255: per-tile counters of the down kernel
constexpr int kMaxTiles = 192;

// ------------------------------------------------------------- launchers
hipError_t launch_route(const RouteArgs &a, hipStream_t s);
hipError_t launch_prefill_route(const RouteArgs &a, hipStream_t s);
hipError_t launch_gate_up(const ExpertArgs &a, int nb, int max_slots, hipStream_t s);
hipError_t launch_down(const ExpertArgs &a, int nb, int max_slots, hipStream_t s);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);

struct PrefillArgs {
  const uint8_t *pool;
  uint64_t pool_bytes;
  const float *x;              // [t][H]
  const uint64_t *rec;         // [E]
  uint64_t shared_rec;
  const int32_t *expert_ptr;   // [E+1]
  const int32_t *entry_row;    // [t*k]
  const int32_t *entry_rank;   // [t*k]
  const float *topk_w;         // [t][k]
  const float *gamma;          // [t]
  int hidden, inter, n_experts, top_k, t;
  _Float16 *xh;                // [32][H]
  _Float16 *act;               // [(t*k + t)][I]
  float *y;                    // [t][k+1][H]
  uint32_t *status;
  float *out;                  // [t][H]
};
hipError_t launch_prefill_experts(const PrefillArgs &a, hipStream_t s);

}  // namespace moe
