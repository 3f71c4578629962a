// Prefill chunk of the MoE layer on MFMA (gfx950): t <= 32 rows, each
// routed independently, rows grouped by expert, every used expert run once
// over its rows as a small dense contraction.
//
// Struct Gpu prefill_chunk / pf_layer / pf_experts: the shared expert over
// all rows, then the routed experts one at a time with their rows gathered,
// computed and scatter-added; prepare_expert_jobs: rows grouped by expert in
// CSR row order; qmm_from / expert_qmm_from: the x rows padded to the token
// tile, with 3/2-bit records using their own unpacking.
//
// Kernels (one stream, in order):
//   P1 router logits (float64) of the t rows and, for the experts, an f16
//      hi/lo split of x plus per-64 group sums of x;
//   P2 per-row top-k and weights (one block a row, nothing across blocks);
//   P3 gate/up: every block first groups the rows by expert from the top-k
//      ids (experts ascending, rows ascending) and lists the sub-jobs (at
//      most 16 rows of one expert), longest first; one block also writes the
//      entry order and one record per sub-job (expert, entries, descriptor)
//      for P4; then per (used expert, 64 gate/up rows), MFMA 16x16x32 f16 tiles
//      of 16 rows x 16 tokens (1 or 2 token tiles for m <= 16 or <= 32);
//   P4 down: per (used expert, 64 output rows), same tiles, writes the
//      routing-weighted rows of every (row, rank) entry;
//   P5 combine: per row, ranks in order, shared expert last.
//
// Exactness of the contraction.  The A operand is the integer code itself
// (exact in f16: 1024 + q built with a bit trick, minus 1024); the B operand
// is x (or act) split into two f16 halves hi + lo whose sum carries ~22
// mantissa bits, one MFMA each, f32 accumulation.  Every MFMA covers 32
// codes of a single 64-code group, so a group's partial sum is scaled after
// the fact: y += s * sum(q x) + b * sum(x).  The result is as accurate as a
// float32 dot product; no weight or activation is rounded to f16 as a whole.
#include <type_traits>

#include "device_common.h"

namespace moe {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTok = MOE_MAX_PREFILL_ROWS;   // 32 token slots per expert

// MFMA operand order.  A lane feeds 16 codes of a 64-code group to two
// 16x16x32 steps; position p = 8 s + j of its 16 (step s, half j) holds code
// frag_code(order, p) of them.  Order 0 (4-bit records: nibble pairs q and
// q + 4 of a word) and order 1 (2/3-bit records: fields q and q + 8) follow
// from how the codes unpack into f16 pairs; x and act are stored in the same
// order so that a lane's B fragment is 16 contiguous bytes.
__host__ __device__ __forceinline__ constexpr int frag_code(int order, int p) {
  return order == 0 ? 8 * (p >> 3) + ((p & 7) >> 1) + 4 * (p & 1)
                    : 4 * (p >> 3) + ((p & 7) >> 1) + 8 * (p & 1);
}
__host__ __device__ __forceinline__ constexpr int frag_pos(int order, int c) {   // inverse of frag_code
  return order == 0 ? 8 * (c >> 3) + 2 * ((c & 7) & 3) + ((c & 7) >> 2)
                    : 8 * ((c & 7) >> 2) + 2 * (c & 3) + (c >> 3);
}
constexpr bool frag_maps_inverse() {
  for (int o = 0; o < 2; ++o)
    for (int p = 0; p < 16; ++p)
      if (frag_pos(o, frag_code(o, p)) != p) return false;
  return true;
}
static_assert(frag_maps_inverse(), "frag_pos must invert frag_code");

// ------------------------------------------------------------------ P1
constexpr int kRouteTok = 2;     // rows per router block
constexpr int kRouteSteps = 4;   // 512-input steps a lane has in flight (all of them at H = 2048)

__host__ __device__ inline int pf_router_blocks(int n_experts, int t) {
  return (n_experts + 1 + kWaves - 1) / kWaves * ((t + kRouteTok - 1) / kRouteTok);
}

// Blocks (rb, tg) below pf_router_blocks: router rows 4 rb + wave (row E =
// shared gate) for rows kRouteTok tg .. +kRouteTok, float64 accumulation.
// The blocks after them split x into f16 hi/lo halves and sum its 64-groups,
// at the same time.
__global__ __launch_bounds__(kThreads) void pf_router_kernel(PrefillArgs a, const uint16_t *router,
                                                             const uint16_t *gvec, double *logits,
                                                             float *gamma) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.hidden, E = a.n_experts, t = a.t;
  const int n_rb = (E + 1 + kWaves - 1) / kWaves;
  const int rb = blockIdx.x % n_rb, r0 = (blockIdx.x / n_rb) * kRouteTok;
  const int e = rb * kWaves + wave;
  if (e <= E && r0 < t) {
    const uint16_t *w = e < E ? router + size_t(e) * H : gvec;
    double acc[kRouteTok] = {};
    for (int i0 = lane * 8; i0 < H; i0 += 512 * kRouteSteps) {
      uint4 wv[kRouteSteps];
      float4 xv[kRouteSteps][kRouteTok][2];
#pragma unroll
      for (int u = 0; u < kRouteSteps; ++u) {
        const int i = min(i0 + 512 * u, H - 8);
        wv[u] = *reinterpret_cast<const uint4 *>(w + i);
#pragma unroll
        for (int b = 0; b < kRouteTok; ++b) {
          const float *xr = a.x + size_t(min(r0 + b, t - 1)) * H + i;
          xv[u][b][0] = *reinterpret_cast<const float4 *>(xr);
          xv[u][b][1] = *reinterpret_cast<const float4 *>(xr + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < kRouteSteps; ++u) {
        if (i0 + 512 * u >= H) break;
        const float wf[8] = {bf16_lo(wv[u].x), bf16_hi(wv[u].x), bf16_lo(wv[u].y), bf16_hi(wv[u].y),
                             bf16_lo(wv[u].z), bf16_hi(wv[u].z), bf16_lo(wv[u].w), bf16_hi(wv[u].w)};
#pragma unroll
        for (int b = 0; b < kRouteTok; ++b) {
          const float xf[8] = {xv[u][b][0].x, xv[u][b][0].y, xv[u][b][0].z, xv[u][b][0].w,
                               xv[u][b][1].x, xv[u][b][1].y, xv[u][b][1].z, xv[u][b][1].w};
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[b] = fma(double(wf[q]), double(xf[q]), acc[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kRouteTok; ++b) {
      const double v = wave_sum_d(acc[b]);
      if (lane == 0 && r0 + b < t) {
        if (e < E) logits[size_t(r0 + b) * E + e] = v;
        else gamma[r0 + b] = float(1.0 / (1.0 + exp(-v)));
      }
    }
  }
  // x -> f16 hi/lo halves in both MFMA code orders: one 16-code block a
  // thread (4-bit order at xf[0], 2/3-bit order at xf[1])
  const int first_split = pf_router_blocks(E, t);
  if (int(blockIdx.x) < first_split) return;
  const int n_split = int(gridDim.x) - first_split;
  for (int i0 = (int(blockIdx.x) - first_split) * kThreads; i0 < t * H / 16; i0 += n_split * kThreads) {
    // (t H / 16 is a multiple of 16, so whole 64-lane groups stay together)
    const int i = min(i0 + int(threadIdx.x), t * H / 16 - 1);
    const bool live = i0 + int(threadIdx.x) < t * H / 16;
    const int r = i / (H / 16), c = (i - r * (H / 16)) * 16;
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = *reinterpret_cast<const float4 *>(a.x + size_t(r) * H + c + 4 * q);
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
    {   // per-64 group sums of x: the 4 threads of a group combine over DPP
      float sm = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) sm += v[q];
      sm += dpp_f<kDppXor1>(sm);
      sm += dpp_f<kDppXor2>(sm);
      if (live && (i & 3) == 0) a.xg[size_t(r) * (H / kGroup) + c / kGroup] = sm;
    }
#pragma unroll
    for (int fam = 0; fam < 2; ++fam) {
      _Float16 hi[16], lo[16];
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const float x = v[frag_code(fam, p)];
        hi[p] = _Float16(x);
        lo[p] = _Float16(x - float(hi[p]));
      }
      if (live) {
        __builtin_memcpy(a.xf + (size_t(2 * fam) * kTok + r) * H + c, hi, 32);
        __builtin_memcpy(a.xf + (size_t(2 * fam + 1) * kTok + r) * H + c, lo, 32);
      }
    }
  }
}

// ------------------------------------------------------------------ P2
// One block a row: the row's top k (logit descending, id ascending) and
// their softmax weights.  The grouping of the rows by expert is rebuilt by
// every block of the gate/up pass from these ids (no cross-block step here).
__global__ __launch_bounds__(128) void pf_topk_kernel(PrefillArgs a, const double *logits, uint32_t *topk_idx) {
  __shared__ double lg[kMaxExperts];
  __shared__ uint32_t k32[kMaxExperts];
  __shared__ int sel[kMaxTopK];
  __shared__ double selv[kMaxTopK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = a.n_experts, k = a.top_k;
  const int r = blockIdx.x;
  const int Ep = (E + 7) & ~7;
  // logits (+ 0.0 folds -0 into +0, so equal values tie on the id alone) and
  // 32-bit order keys of them rounded to float32; padding keys are 0, below
  // every logit's key
  for (int e = threadIdx.x; e < Ep; e += 128) {
    const double v = e < E ? logits[size_t(r) * E + e] + 0.0 : -__builtin_inf();
    lg[e] = v;
    k32[e] = e < E ? order_key32(float(v)) : 0u;
  }
  if (threadIdx.x < kMaxTopK) sel[threadIdx.x] = 0;
  __syncthreads();
  // rank = entries ahead in (logit descending, id ascending).  Rounding to
  // float32 never reverses an order, so a larger key is a larger logit and
  // a smaller key a smaller one; only entries whose keys are equal are
  // compared again in float64, and only for an entry that can still place
  for (int e = threadIdx.x; e < E; e += 128) {
    const uint32_t ke = k32[e];
    const uint4 *kr = reinterpret_cast<const uint4 *>(k32);
    int gt = 0, eq = 0;
    for (int f4 = 0; f4 < Ep / 4; ++f4) {
      const uint4 o = kr[f4];
      gt += int(o.x > ke) + int(o.y > ke) + int(o.z > ke) + int(o.w > ke);
      eq += int(o.x == ke) + int(o.y == ke) + int(o.z == ke) + int(o.w == ke);
    }
    int rank = gt;
    if (gt < k && eq > 1) {   // float32 ties (the entry itself is one of them)
      const double v = lg[e];
      for (int f = 0; f < E; ++f)
        if (k32[f] == ke) rank += int(lg[f] > v) + (int(lg[f] == v) & int(f < e));
    }
    if (rank < k) { sel[rank] = e; selv[rank] = lg[e]; }
  }
  __syncthreads();
  if (wave == 0) {
    double ex = 0.0;
    if (lane < k) ex = exp(selv[lane] - selv[0]);
    const double sum = wave_sum_d(ex);
    if (lane < k) {
      st_dev(topk_idx + r * k + lane, uint32_t(sel[lane]));
      a.topk_w[r * k + lane] = float(ex / sum);
    }
  }
}

// --------------------------------------------------------- shared helpers
// The 16 codes a lane feeds to the two MFMA steps of one group, as exact f16
// values: A[s] holds 8 halfs.  Half j of step s is code off(s, j) of the
// lane's 16 (4-bit: 8s + j/2 + 4(j%2); 2/3-bit: 4s + j/2 + 8(j%2)); the
// B operand is staged in the same order.
__device__ inline uint32_t pair_to_f16(uint32_t v) {
  // v holds two small integers in bits [0,3) and [16,19): make them f16
  // (1024 + q via the exponent bits, then subtract 1024 exactly)
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  const half2v h = __builtin_bit_cast(half2v, v | 0x64006400u);
  const half2v one_k = {_Float16(1024.0f), _Float16(1024.0f)};
  return __builtin_bit_cast(uint32_t, h - one_k);
}

// The three masks of the 4-bit expansion, as values the compiler must keep
// in registers: a mask in a register lets the AND and the OR of a nibble
// pair fuse into one v_and_or_b32 (a literal cannot be an operand of it).
struct NibbleMasks {
  uint32_t lo, hi, ex;   // 0x000F000F, 0x00F000F0, 0x64006400
};
__device__ __forceinline__ NibbleMasks nibble_masks() {
  NibbleMasks m{0x000F000Fu, 0x00F000F0u, 0x64006400u};
  asm volatile("" : "+v"(m.lo), "+v"(m.hi), "+v"(m.ex));
  return m;
}

// One 4-bit code word as eight exact f16 values in the order (0, 4), (1, 5),
// (2, 6), (3, 7): nibbles at bits 0..3 of a half become 1024 + q and at bits
// 4..7 1024 + 16 q (exponent bits OR-ed in); one packed f16 add or fma takes
// them to q exactly.
__device__ __forceinline__ half8 word4_to_a(uint32_t w, const NibbleMasks &m) {
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
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

template <int BITS>
__device__ inline void codes_to_a(const uint32_t (&w)[3], half8 (&A)[2], int hshift) {
  uint32_t r[8];
  if constexpr (BITS == 4) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) r[4 * s + q] = pair_to_f16((w[s] >> (4 * q)) & 0x000F000Fu);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t v = (w[0] >> (2 * q)) & 0x00030003u;
      if constexpr (BITS == 3) {
        // high bits of codes q and q+8 sit at bits P and P+16 of the block's
        // high-plane word (P = 8(q/4) + 4*hshift + q%4)
        const int P = 8 * (q / 4) + 4 * hshift + (q % 4);
        v |= ((w[1] >> P) & 0x00010001u) << 2;
      }
      r[q] = pair_to_f16(v);
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    uint4 u = make_uint4(r[4 * s], r[4 * s + 1], r[4 * s + 2], r[4 * s + 3]);
    A[s] = __builtin_bit_cast(half8, u);
  }
}


// 16 codes of one lane for one 64-code group: codes [16g, 16g+16) of the
// group starting at code index `c0` of a packed row (`row` points at the row,
// `row_codes` codes long; for group-major down records the row is the
// 64-code group itself).
template <int BITS>
__device__ inline void load16(const uint8_t *row, int row_codes, int c0, uint32_t (&w)[3]) {
  if constexpr (BITS == 4) {
    const uint2 v = *reinterpret_cast<const uint2 *>(row + c0 / 2);
    w[0] = v.x; w[1] = v.y; w[2] = 0;
  } else if constexpr (BITS == 2) {
    w[0] = *reinterpret_cast<const uint32_t *>(row + c0 / 4);
    w[1] = 0; w[2] = 0;
  } else {
    w[0] = *reinterpret_cast<const uint32_t *>(row + c0 / 4);
    w[1] = *reinterpret_cast<const uint32_t *>(row + row_codes / 4 + (c0 / 32) * 4);
    w[2] = 0;
  }
}

// A sub-job: at most 16 rows of one expert (or of the shared expert).
struct Job {
  int e;        // expert id, or -1 for the shared expert
  int base;     // first entry index of its rows
  int m;        // rows (1..16)
  uint64_t desc;
  int lane_row;       // lane n < m: token row of slot n (set by the gate/up pass's grouping)
};

// Rows grouped by expert (experts ascending, rows ascending inside an
// expert) and the sub-jobs (at most 16 rows of one expert), longest first:
// the shared expert's, then those of experts with more than 8 rows, then
// the rest, experts ascending in each, so that the items with the most
// rounds issue their loads first.  Every gate/up block builds it in LDS from
// the top-k ids and the descriptors (one load each), so that no pass needs a
// cross-block step for it; one block writes the entry order (CSR) and the
// sub-job records for the down pass.
struct Grouping {
  uint32_t emask[kMaxExperts];   // rows that selected the expert (a row selects an expert once, t <= 32)
  int scan[kMaxExperts];         // exclusive scan of (rows << 20 | heavy << 10 | light) over experts
  uint64_t desc[kMaxExperts];
  int job[2 * kMaxExperts + 2];  // sub-job -> expert | (half << 16), or -1 - half for the shared expert
  int wsum[kWaves];
};

// position of the i-th (from 0) set bit of m (m has more than i)
__device__ inline int nth_set_bit(uint32_t m, int i) {
  int pos = 0;
#pragma unroll
  for (int s = 16; s >= 1; s >>= 1)
    if (__popc(m & ((1u << (pos + s)) - 1u)) <= i) pos += s;
  return pos;
}

// Builds the grouping; returns the sub-job count.  All threads call it.
__device__ inline int build_grouping(const PrefillArgs &a, Grouping &gr) {
  static_assert(kThreads == kMaxExperts, "one thread per expert");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.n_experts, k = a.top_k, t = a.t, nsel = t * k;   // nsel <= 2 kThreads
  const uint32_t s0 = a.topk_idx[min(tid, nsel - 1)], s1 = a.topk_idx[min(tid + kThreads, nsel - 1)];
  const uint64_t rv = a.rec[min(tid, E - 1)];
  gr.emask[tid] = 0u;
  __syncthreads();
  if (tid < nsel) atomicOr(&gr.emask[s0], 1u << (tid / k));
  if (tid + kThreads < nsel) atomicOr(&gr.emask[s1], 1u << ((tid + kThreads) / k));
  __syncthreads();
  // an expert with more than 8 rows is heavy (one sub-job, two above 16
  // rows), one with 1-8 rows light
  // The scan inside a wave is bit-sliced: each field is a sum of bits times
  // their weights, and a bit's prefix over the lanes is a ballot counted
  // below the lane (no lane exchanges).
  const int c = tid < E ? __popc(gr.emask[tid]) : 0;
  const int hv = c > 8 ? 1 + int(c > 16) : 0, lt = int(c > 0 && c <= 8);
  int wexcl = 0, wtot = 0;
  auto slice = [&](bool bit, int weight) {
    const uint64_t m = __ballot(bit);
    wexcl += weight * int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
    wtot += weight * __popcll(m);
  };
#pragma unroll
  for (int b = 0; b < 6; ++b) slice((c >> b) & 1, 1 << (20 + b));   // c <= 32
  slice(hv & 1, 1 << 10);
  slice(hv >> 1, 2 << 10);
  slice(lt, 1);
  if (lane == 0) gr.wsum[wave] = wtot;
  __syncthreads();
  int pre = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) pre += w < wave ? gr.wsum[w] : 0;
  const int total = (gr.wsum[0] + gr.wsum[1]) + (gr.wsum[2] + gr.wsum[3]);
  const int excl = wexcl + pre;
  const int n_shared = t > 16 ? 2 : 1, n_heavy = (total >> 10) & 1023;
  gr.scan[tid] = excl;
  gr.desc[tid] = rv;
  if (c > 0) {
    const int sj = c > 8 ? n_shared + ((excl >> 10) & 1023) : n_shared + n_heavy + (excl & 1023);
    gr.job[sj] = tid;
    if (c > 16) gr.job[sj + 1] = tid | (1 << 16);
  }
  if (tid < n_shared) gr.job[tid] = -1 - tid;
  __syncthreads();
  return n_shared + n_heavy + (total & 1023);
}

// Sub-job sj of the grouping; lane_row = the token row of slot lane & 15.
__device__ inline Job job_from(const PrefillArgs &a, const Grouping &gr, int sj) {
  const int n = threadIdx.x & 15;
  const int je = __builtin_amdgcn_readfirstlane(gr.job[sj]);
  Job j;
  if (je < 0) {
    const int h = -1 - je;
    j.e = -1;
    j.base = a.t * a.top_k + 16 * h;
    j.m = min(16, a.t - 16 * h);
    j.desc = a.shared_rec;
    j.lane_row = 16 * h + min(n, j.m - 1);
  } else {
    const int e = je & 0xffff, h = je >> 16;
    const uint32_t em = __builtin_amdgcn_readfirstlane(gr.emask[e]);
    j.e = e;
    j.base = (__builtin_amdgcn_readfirstlane(gr.scan[e]) >> 20) + 16 * h;
    j.m = min(16, __popc(em) - 16 * h);
    const uint64_t d = gr.desc[e];
    j.desc = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(d)))) |
             (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(d >> 32)))) << 32);
    j.lane_row = nth_set_bit(em, 16 * h + min(n, j.m - 1));
  }
  return j;
}

// The entry order (CSR: expert starts, each entry's row and rank) and the
// sub-job records of the down pass, from one block's grouping.
__device__ inline void write_grouping(const PrefillArgs &a, const Grouping &gr, int n_jobs) {
  const int tid = threadIdx.x;
  const int E = a.n_experts, k = a.top_k, t = a.t;
  for (int e = tid; e <= E; e += kThreads)
    a.expert_ptr[e] = e < E ? gr.scan[e] >> 20 : t * k;
  for (int p = tid; p < t * k; p += kThreads) {
    const int e = int(a.topk_idx[p]), r = p / k;
    const int pos = (gr.scan[e] >> 20) + __popc(gr.emask[e] & ((1u << r) - 1u));
    a.entry_row[pos] = r;
    a.entry_rank[pos] = p - r * k;
  }
  for (int sj = tid; sj < n_jobs; sj += kThreads) {
    const int je = gr.job[sj];
    int32_t *jr = a.meta + kJobInts * (1 + sj);
    int e, base, m;
    uint64_t d;
    if (je < 0) {
      e = -1;
      base = t * k + 16 * (-1 - je);
      m = min(16, t - 16 * (-1 - je));
      d = a.shared_rec;
    } else {
      e = je & 0xffff;
      base = (gr.scan[e] >> 20) + 16 * (je >> 16);
      m = min(16, __popc(gr.emask[e]) - 16 * (je >> 16));
      d = gr.desc[e];
    }
    jr[0] = e;
    jr[1] = base | (m << 16);
    jr[2] = int32_t(uint32_t(d));
    jr[3] = int32_t(uint32_t(d >> 32));
  }
  if (tid == 0) a.meta[0] = n_jobs;
}

// the record of sub-job sj (below the workspace's capacity of sub-jobs)
__device__ inline Job job_of(const PrefillArgs &a, int sj) {
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 r = *reinterpret_cast<const i32x4 *>(a.meta + kJobInts * (1 + sj));
  Job j;
  j.e = __builtin_amdgcn_readfirstlane(r[0]);
  const int bm = __builtin_amdgcn_readfirstlane(r[1]);
  j.base = bm & 0xffff;
  j.m = bm >> 16;
  j.desc = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(r[2]))) |
           (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(r[3]))) << 32);
  j.lane_row = -1;   // the down pass's B rows are the job's act rows
  return j;
}

// token row of a sub-job's n-th entry
__device__ inline int entry_token_row(const PrefillArgs &a, const Job &j, int n) {
  return j.e < 0 ? j.base - a.t * a.top_k + n : a.entry_row[j.base + n];
}

// ------------------------------------------------------- P3 / P4 tiles
// One work item: 64 output rows (16 per wave) of one sub-job (m <= 16 token
// rows, one 16-column MFMA tile), over K = n_groups 64-code groups.  The
// B rows (f16 hi and lo halves, already in MFMA order) and the B rows' group
// sums go straight from global memory into LDS (global_load_lds: lane i's 16
// or 4 bytes land at base + 16 i or 4 i), with the tile's (scale, bias)
// words (by DMA for group-major records, through registers for row-major
// ones), one round of groups at a time (gate/up: 32 groups for up to 4 rows,
// 16 for up to 8, 8 for up to 16; down: 8); the lane's codes for a batch of
// groups (32 for gate/up, 8 for down) load into registers at once.  The
// buffers are small enough for three (gate/up) or four (down) blocks per CU,
// whose load and compute phases interleave.  Token slots past the job's rows
// hold stale LDS contents: an MFMA output column depends on its own B column
// only, and those columns are never stored.
typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

constexpr int kCodeGroups = 32;                 // groups of codes held in registers (gate/up)
// B area of one round: 16 rows of 8 groups, 8 rows of 16 or 4 rows of 32
constexpr int kBufHalfs = 16 * (8 * kGroup + 8) > 8 * (16 * kGroup + 8) ? 16 * (8 * kGroup + 8)
                                                                       : 8 * (16 * kGroup + 8);
template <int SBG>   // rounds of up to SBG groups
struct TileBufT {
  __attribute__((aligned(16))) _Float16 bh[kBufHalfs];
  __attribute__((aligned(16))) _Float16 bl[kBufHalfs];
  __attribute__((aligned(16))) uint32_t sb[SBG * 64];   // [group][64 rows] (scale, bias) words
  float xs[8 * 16 * 2];                                 // [token][group][part] B group sums
};
typedef TileBufT<32> TileBuf;   // gate/up: rounds of up to 32 groups
typedef TileBufT<8> DownBuf;    // down: rounds of 8 groups (four blocks per CU)

// Where a work item's operands live.
struct TileSrc {
  __amdgpu_buffer_rsrc_t codes;   // A: the record's code section
  bool group_major;       // D layout [group][row][64 codes] (else [row][K codes])
  int row_bytes;          // bytes per packed row (row-major layout)
  int rows_total;         // rows of the matrix (group-major layout)
  const uint32_t *sb;     // (scale, bias) words
  __amdgpu_buffer_rsrc_t sbr;   // the same words as a bounded resource (row-major records)
  bool sb_group_major;    // [group][rows] (else [row][groups])
  int sb_stride;          // groups per row, or rows per group
  const _Float16 *bh, *bl;   // B rows (row stride = K halfs)
  const float *xsum;      // B group sums, `parts` per group (row stride = parts n_groups)
  int parts;
  int K;                  // codes per row = 64 n_groups
  int r0;                 // first of the tile's 64 rows
  int m;                  // token rows of the job (<= 16)
  int lane_brow;          // lane n < m: the B row of token slot n (other lanes: unused)
};

// A buffer resource built from wave-uniform parts (readfirstlane), so that
// the compiler keeps it in scalar registers wherever it is used.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint64_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v)), hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(uint32_t(bytes < 0x7fffffffu ? bytes : 0x7fffffffu));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((uint64_t(hi) << 32) | lo), (short)0, int(n),
                                           0x00020000);
}

// 16 codes of a lane for one group: the same words load16 reads, by offset.
template <int BITS>
__device__ __forceinline__ void load_codes(const TileSrc &src, int row, int grp, int g, uint32_t (&w)[3]) {
  uint32_t off, hi_off = 0;
  if (src.group_major) {
    const uint32_t base = (uint32_t(grp) * src.rows_total + row) * (kGroup * BITS / 8);
    off = base + 16 * g * BITS / 8;
    if constexpr (BITS == 3) { off = base + 16 * g / 4; hi_off = base + kGroup / 4 + (16 * g / 32) * 4; }
  } else {
    const uint32_t base = uint32_t(row) * src.row_bytes, c0 = grp * kGroup + 16 * g;
    off = base + c0 * (BITS == 4 ? 4 : 2) / 8;
    if constexpr (BITS == 3) hi_off = base + src.K / 4 + (c0 / 32) * 4;
  }
  w[2] = 0;
  if constexpr (BITS == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(src.codes, off, 0, 0);
    w[0] = v[0]; w[1] = v[1];
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(src.codes, off, 0, 0);
    w[1] = BITS == 3 ? __builtin_amdgcn_raw_buffer_load_b32(src.codes, hi_off, 0, 0) : 0u;
  }
}

// 4-bit row-major codes, two groups a load: lane (row, slot g) reads bytes
// 16 g .. 16 g + 15 of the 64 bytes of groups grp and grp + 1 (slots 0, 1:
// halves of grp, slots 2, 3: of grp + 1) into w0 (lower 8 bytes) and w1
// (upper 8).  Reads past a row's last group (an odd group count) stay inside
// the code section or are dropped by the resource's bound, and are never
// used.
__device__ __forceinline__ void load_codes_pair(const TileSrc &src, int row, int grp, int g, uint32_t (&w0)[3],
                                                uint32_t (&w1)[3]) {
  const uint32_t off = uint32_t(row) * src.row_bytes + uint32_t(grp) * (kGroup / 2) + 16 * g;
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(src.codes, off, 0, 0);
  w0[0] = v[0]; w0[1] = v[1]; w0[2] = 0;
  w1[0] = v[2]; w1[1] = v[3]; w1[2] = 0;
}

// LDS loads of groups [g0, g0 + gq) into `buf`; wave w takes every fourth.
template <int CG, bool SBDMA, class Buf>
__device__ __forceinline__ void chunk_dma(const TileSrc &src, Buf &buf, int g0, int gq, int n_groups) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kRow = CG * kGroup + 8;            // B row stride in LDS (halfs)
  constexpr int kSegs = CG * kGroup / 512;         // 1 KB segments per B row
  const int lane_brow = src.lane_brow;   // the B row of token slot n is lane n's
  // B rows: one load per (token row, hi/lo, segment)
  for (int q = wave; q < 2 * kSegs * src.m; q += kWaves) {
    const int n = q / (2 * kSegs), hl = (q / kSegs) & 1, seg = q % kSegs;
    const int k0 = seg * 512 + lane * 8;
    const int brow_n = __builtin_amdgcn_readlane(lane_brow, n);
    const _Float16 *row = (hl ? src.bl : src.bh) + size_t(brow_n) * src.K + g0 * kGroup;
    _Float16 *dst = (hl ? buf.bl : buf.bh) + n * kRow + seg * 512;
    if (k0 < gq * kGroup)
      __builtin_amdgcn_global_load_lds((gvoid *)(row + k0), (lvoid *)dst, 16, 0, 0);
  }
  // (scale, bias) words of group-major records: one load per group, lane =
  // tile row (row-major records load theirs through registers: sb_fetch)
#pragma unroll
  for (int i = 0; i < (SBDMA ? (CG + kWaves - 1) / kWaves : 0); ++i) {
    const int Q = wave + kWaves * i;
    if (Q < gq) {
      const int row = src.r0 + lane, grp = g0 + Q;
      const uint32_t *p = src.sb_group_major ? src.sb + size_t(grp) * src.sb_stride + row
                                             : src.sb + size_t(row) * src.sb_stride + grp;
      __builtin_amdgcn_global_load_lds((gvoid *)p, (lvoid *)(buf.sb + Q * 64), 4, 0, 0);
    }
  }
  // group sums: entry i = (token n, group Q, part h); at most 16 x 16 x 2
  // or 8 x 32 x 1 entries, 8 chunks of 64
  const int ents = src.m * CG * src.parts;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int q = wave + kWaves * c;
    const int i = q * 64 + lane, n = i / (CG * src.parts), Q = (i / src.parts) % CG, h = i % src.parts;
    const int brow_n = __builtin_amdgcn_ds_bpermute(min(n, 63) << 2, lane_brow);
    if (q * 64 < ents && i < ents && Q < gq) {
      const float *p = src.xsum + (size_t(brow_n) * n_groups + g0 + Q) * src.parts + h;
      __builtin_amdgcn_global_load_lds((gvoid *)p, (lvoid *)(buf.xs + q * 64), 4, 0, 0);
    }
  }
}

// (scale, bias) words of a round from a row-major record ([row][groups]):
// thread t takes tile row t / 4 and the quarter t % 4 of the round's CG
// groups, a run of CG / 4 contiguous words, so that a wave's loads cover
// whole rows (a load per group with lane = row touches 64 rows); the words
// go to LDS group-major, [group][64 rows], once the round has landed.  Runs
// past the section's end read 0 through the bounded resource, and groups
// past the round's are never read.
template <int CG>
struct SbRun {
  uint32_t v[CG / 4];
};

template <int CG>
__device__ __forceinline__ void sb_fetch(const TileSrc &src, int g0, SbRun<CG> &r) {
  static_assert(CG == 8 || CG == 16 || CG == 32, "runs of 2, 4 or 8 words");
  const int t = threadIdx.x;
  const uint32_t off = (uint32_t(src.r0 + t / 4) * src.sb_stride + g0 + (t % 4) * (CG / 4)) * 4;
#pragma unroll
  for (int h = 0; h < (CG / 4 + 3) / 4; ++h) {
    if constexpr (CG == 8) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(src.sbr, off, 0, 0);
      r.v[0] = v[0]; r.v[1] = v[1];
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(src.sbr, off + 16 * h, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) r.v[4 * h + j] = v[j];
    }
  }
}

template <int CG, class Buf>
__device__ __forceinline__ void sb_store(Buf &buf, const SbRun<CG> &r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < CG / 4; ++j) buf.sb[((t % 4) * (CG / 4) + j) * 64 + t / 4] = r.v[j];
}

// PAIR: the codes were loaded two groups a load (load_codes_pair).  One
// exchange of the upper two words with slot g ^ 2 (lane ^ 32) leaves every
// slot 16 codes of each group of the pair: slot g holds codes kb .. kb + 15
// of group Q with kb = 16 (2 (g & 1) + ((g >> 1) ^ (Q & 1))), its own lower
// words when (g >> 1) == (Q & 1) and the received ones otherwise; the B
// fragments are read at the same kb.
// Group Q of the round whose first group is batch group q0; on the paired
// path the even group of a pair receives both groups' exchanged words
// (ex0, ex1) for the odd one.
template <int BITS, int CG, int ROWS, int KCG, bool PAIR, class Buf>
__device__ __forceinline__ void group_mma(const TileSrc &src, const Buf &buf, const uint32_t (&w)[KCG][3],
                                          int q0, int Q, floatx4 &acc, const NibbleMasks &nm,
                                          uint32_t &ex0, uint32_t &ex1) {
  static_assert(!PAIR || (BITS == 4 && CG % 2 == 0), "paired loads: 4-bit codes, whole pairs a round");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // token slot of the lane's B column; when a round stages fewer than 16
  // rows, slots past them (past m) read the staged rows again (their
  // columns are unused)
  static_assert(ROWS == 4 || ROWS == 8 || ROWS == 16, "rounds stage 4, 8 or 16 token rows");
  const int g = lane >> 4, n = lane & (ROWS - 1);
  constexpr int kRow = CG * kGroup + 8;
  half8 A[2];
  int kb = 16 * g;   // first of the lane's 16 codes of group Q
  if constexpr (PAIR) {
    if ((Q & 1) == 0) {   // one exchange serves both groups of the pair
      const int partner = (lane ^ 32) * 4;   // ds_bpermute address of slot g ^ 2
      ex0 = __builtin_amdgcn_ds_bpermute(partner, w[q0 + Q + 1][0]);
      ex1 = __builtin_amdgcn_ds_bpermute(partner, w[q0 + Q + 1][1]);
    }
    const bool own = (g >> 1) == (Q & 1);
    A[0] = word4_to_a(own ? w[q0 + (Q & ~1)][0] : ex0, nm);
    A[1] = word4_to_a(own ? w[q0 + (Q & ~1)][1] : ex1, nm);
    kb = 16 * (2 * (g & 1) + ((g >> 1) ^ (Q & 1)));
  } else if constexpr (BITS == 4) {
    A[0] = word4_to_a(w[q0 + Q][0], nm);
    A[1] = word4_to_a(w[q0 + Q][1], nm);
  } else {
    codes_to_a<BITS>(w[q0 + Q], A, g & 1);
  }
  const uint4 sq = *static_cast<const uint4 *>(__builtin_assume_aligned(buf.sb + Q * 64 + wave * 16 + 4 * g, 16));
  const uint32_t sw4[4] = {sq.x, sq.y, sq.z, sq.w};
  floatx4 cgv = {0, 0, 0, 0};
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int at = n * kRow + Q * kGroup + kb + 8 * st;
    const half8 Bh = *static_cast<const half8 *>(__builtin_assume_aligned(buf.bh + at, 16));
    const half8 Bl = *static_cast<const half8 *>(__builtin_assume_aligned(buf.bl + at, 16));
    cgv = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[st], Bh, cgv, 0, 0, 0);
    cgv = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[st], Bl, cgv, 0, 0, 0);
  }
  const float *xp = buf.xs + (n * CG + Q) * src.parts;
  const float xs = src.parts == 2 ? xp[0] + xp[1] : xp[0];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = fmaf(sb_scale(sw4[q]), cgv[q], fmaf(sb_bias(sw4[q]), xs, acc[q]));
}

// The first gq groups of the round.
template <int BITS, int CG, int ROWS, int KCG, bool PAIR, class Buf>
__device__ __forceinline__ void chunk_mma(const TileSrc &src, const Buf &buf, const uint32_t (&w)[KCG][3],
                                          int q0, int gq, floatx4 &acc, const NibbleMasks &nm) {
  uint32_t ex0 = 0, ex1 = 0;
#pragma unroll
  for (int Q = 0; Q < CG; ++Q)
    if (Q < gq) group_mma<BITS, CG, ROWS, KCG, PAIR>(src, buf, w, q0, Q, acc, nm, ex0, ex1);
}

// s_waitcnt on the vector-memory count only: at most N loads of this wave
// still in flight (the expcnt and lgkmcnt fields at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_sched_barrier(0);   // no use of a pending load is scheduled above the wait
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __builtin_amdgcn_sched_barrier(0);
}

// A workgroup barrier with no memory fence: this wave's LDS operations have
// completed (lgkmcnt 0) and the empty asm statements keep the compiler from
// moving memory operations across it, but global loads in flight stay in
// flight (a fenced barrier waits for all of them).  LDS written by DMA loads
// is covered only by the waits the caller does before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// The rounds of a work item, with an early start: round 0's operands go to
// LDS first, then the codes of the batch's first PRE groups load in group
// order, and round 0 waits only for its operands (the codes are the loads
// issued after them, and the counter retires loads in issue order); its
// groups then consume the codes as they land, and on the paired path each
// computed pair of groups issues the loads of the next pair not yet in
// flight, so that a wave computes between its load issues instead of
// stalling on a full memory queue with every load of the item still to
// issue.  Later rounds load their operands after the previous round is
// computed.  Rounds: 32 groups of 4 rows, 16 of 8 or 8 of 16.
template <int BITS, int CG, int ROWS, int KCG, bool PAIR, bool SBROWS, int HEAD, int SBG, int PRE = KCG>
__device__ __forceinline__ void mfma_tile(const TileSrc &src, TileBufT<SBG> &buf, floatx4 &acc) {
  static_assert(ROWS * (CG * kGroup + 8) <= kBufHalfs, "round does not fit the B area");
  static_assert(CG <= SBG && CG <= KCG && ROWS * CG * 2 <= 8 * 16 * 2, "round does not fit the (scale, bias) or sum areas");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int arow = src.r0 + wave * 16 + (lane & 15), g = lane >> 4;
  const int n_groups = src.K / kGroup;
  // the codes of the batch's first HEAD groups load before round 0's
  // operands, the rest after them: the wait for the operands then allows
  // exactly the later codes in flight
  constexpr int kHead = HEAD;
  constexpr int kPre = PAIR ? PRE : KCG;   // groups whose codes load before round 0 computes
  constexpr int kLoadsAfter = PAIR ? (kPre - kHead) / 2 : (BITS == 3 ? 2 : 1) * (KCG - kHead);
  static_assert(!PAIR || (kHead % 2 == 0 && kPre % 2 == 0), "whole pairs before the operands");
  static_assert(kPre >= kHead && kPre <= KCG, "the first loads are a prefix of the batch");
  const NibbleMasks nm = nibble_masks();
  acc = floatx4{0, 0, 0, 0};
  for (int g0 = 0; g0 < n_groups; g0 += KCG) {
    const int nr = (min(KCG, n_groups - g0) + CG - 1) / CG;
    uint32_t w[KCG][3];
    auto load_groups = [&](auto qa, auto qb) {   // groups [qa, qb) of the batch
      if constexpr (PAIR) {
#pragma unroll
        for (int P = decltype(qa)::value / 2; P < decltype(qb)::value / 2; ++P)
          load_codes_pair(src, arow, min(g0 + 2 * P, (n_groups - 1) & ~1), g, w[2 * P], w[2 * P + 1]);
      } else {
#pragma unroll
        for (int Q = decltype(qa)::value; Q < decltype(qb)::value; ++Q)
          load_codes<BITS>(src, arow, min(g0 + Q, n_groups - 1), g, w[Q]);
      }
    };
    load_groups(std::integral_constant<int, 0>(), std::integral_constant<int, kHead>());
    asm volatile("" ::: "memory");   // round 0's operands are issued after the first codes
    chunk_dma<CG, !SBROWS>(src, buf, g0, min(CG, n_groups - g0), n_groups);
    SbRun<CG> sbw;
    if constexpr (SBROWS) sb_fetch<CG>(src, g0, sbw);
    asm volatile("" ::: "memory");   // ... and the remaining codes after them
    load_groups(std::integral_constant<int, kHead>(), std::integral_constant<int, kPre>());
    asm volatile("" ::: "memory");   // ... all before the wait
    wait_vm<(kLoadsAfter < 63 ? kLoadsAfter : 63)>();
    if constexpr (SBROWS) sb_store<CG>(buf, sbw);
    lds_barrier();
#pragma unroll
    for (int cs = 0; cs < KCG / CG; ++cs) {
      const int cb = g0 + cs * CG;
      if (cs < nr) {
        if (cs > 0) {
          lds_barrier();   // every wave is done with round cs - 1
          chunk_dma<CG, !SBROWS>(src, buf, cb, min(CG, n_groups - cb), n_groups);
          if constexpr (SBROWS) sb_fetch<CG>(src, cb, sbw);
          wait_vm<0>();
          if constexpr (SBROWS) sb_store<CG>(buf, sbw);
          lds_barrier();
        }
        if (kPre < KCG && cs == 0) {
          const int gq = min(CG, n_groups - cb);
          uint32_t ex0 = 0, ex1 = 0;
#pragma unroll
          for (int P = 0; P < CG / 2; ++P) {
            if (2 * P < gq) group_mma<BITS, CG, ROWS, KCG, PAIR>(src, buf, w, 0, 2 * P, acc, nm, ex0, ex1);
            if (2 * P + 1 < gq) group_mma<BITS, CG, ROWS, KCG, PAIR>(src, buf, w, 0, 2 * P + 1, acc, nm, ex0, ex1);
            if (kPre / 2 + P < KCG / 2) {
              asm volatile("" ::: "memory");   // issued after the pair's operand reads
              const int L = kPre / 2 + P;
              load_codes_pair(src, arow, min(g0 + 2 * L, (n_groups - 1) & ~1), g, w[2 * L], w[2 * L + 1]);
            }
          }
          // pairs still unissued go before the next round's operands
          load_groups(std::integral_constant<int, (kPre + CG < KCG ? kPre + CG : KCG)>(),
                      std::integral_constant<int, KCG>());
        } else {
          chunk_mma<BITS, CG, ROWS, KCG, PAIR>(src, buf, w, cs * CG, min(CG, n_groups - cb), acc, nm);
        }
      }
    }
    __syncthreads();   // the buffer is free for the next batch or work item
  }
}

constexpr int kPreGroups = 8;   // gate/up: groups whose codes load before round 0 computes

template <int BITS>
__device__ __forceinline__ void mfma_tile_any(const TileSrc &src, TileBuf &buf, floatx4 &acc) {
  // (4-bit records are row-major: their codes load two groups a load)
  constexpr bool kPair = BITS == 4;
  constexpr int kPre = kPair ? kPreGroups : kCodeGroups;
  if (src.m > 8) mfma_tile<BITS, 8, 16, kCodeGroups, kPair, true, 0, 32, kPre>(src, buf, acc);
  else if (src.m > 4) mfma_tile<BITS, 16, 8, kCodeGroups, kPair, true, 0, 32, kPre>(src, buf, acc);
  else mfma_tile<BITS, 32, 4, kCodeGroups, kPair, true, 0, 32, kPre>(src, buf, acc);
}

// down: 8 groups of codes in registers and rounds of 8 groups for any m
// (K = I is 8 groups at I = 512: one round, and a register budget and LDS
// area small enough for four blocks per CU); the first 4 groups' codes load
// before the round's operands (for gate/up that order measured slower)
template <int BITS>
__device__ __forceinline__ void mfma_tile_down(const TileSrc &src, DownBuf &buf, floatx4 &acc) {
  mfma_tile<BITS, 8, 16, 8, false, false, 4>(src, buf, acc);
}


// ------------------------------------------------------------------ P3
// gate/up: work item (job, 64 interleaved gate/up rows); act = silu(g) * u
// of the tile's 32 columns, stored as f16 hi/lo halves in the MFMA order of
// the job's record, plus the sum of the 32 values for the down pass's bias
// term.
__global__ __launch_bounds__(kThreads, 3) void pf_gate_up_kernel(PrefillArgs a) {
  __shared__ TileBuf buf;
  __shared__ Grouping gr;
  __shared__ float red[kWaves][16];
  const int H = a.hidden, I = a.inter;
  // grid: (tile, sub-job)
  const int tile = blockIdx.x;
  const int n_jobs = build_grouping(a, gr);
  if (blockIdx.x == 0 && blockIdx.y == 0) write_grouping(a, gr, n_jobs);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, nl = lane & 15;
  for (int sj = blockIdx.y; sj < n_jobs; sj += gridDim.y) {
    const Job j = job_from(a, gr, sj);
    const bool ok = record_ok(j.desc, a.pool_bytes, H, I);
    const int bits = ok ? bits_of_tag(j.desc) : 4, order = bits == 4 ? 0 : 1;
    floatx4 acc = {0, 0, 0, 0};
    if (ok) {
      const RecordLayout R = record_layout(H, I, bits);
      const uint8_t *rec = a.pool + (j.desc & ~uint64_t(255));
      TileSrc src;
      src.codes = rsrc(rec + R.gu_codes, R.gu_sb - R.gu_codes);
      src.group_major = false;
      src.row_bytes = R.gu_row_bytes;
      src.rows_total = 2 * I;
      src.sb = reinterpret_cast<const uint32_t *>(rec + R.gu_sb);
      src.sbr = rsrc(rec + R.gu_sb, R.d_codes - R.gu_sb);
      src.sb_group_major = false;
      src.sb_stride = H / kGroup;
      src.bh = a.xf + size_t(2 * order) * kTok * H;
      src.bl = a.xf + size_t(2 * order + 1) * kTok * H;
      src.xsum = a.xg;
      src.parts = 1;
      src.K = H;
      src.r0 = tile * 64;
      src.m = j.m;
      src.lane_brow = j.lane_row;
      switch (bits) {
        case 4: mfma_tile_any<4>(src, buf, acc); break;
        case 3: mfma_tile_any<3>(src, buf, acc); break;
        default: mfma_tile_any<2>(src, buf, acc); break;
      }
    } else if (threadIdx.x == 0) {
      __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // lane rows 4g + q: (gate, up) pairs q = (0, 1) and (2, 3); a bad record
    // leaves zeros so that the down pass stays finite
    const int p0 = (tile * 64 + wave * 16 + 4 * g) / 2;
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) v[h] = ok ? silu_mul(acc[2 * h], acc[2 * h + 1]) : 0.0f;
    if (nl < j.m) {
      _Float16 *dh = a.act + size_t(j.base + nl) * I;
      _Float16 *dl = a.act + (size_t(a.act_rows) + j.base + nl) * I;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = p0 + h;
        const int at = (col & ~15) + frag_pos(order, col & 15);
        const _Float16 hv = _Float16(v[h]);
        dh[at] = hv;
        dl[at] = _Float16(v[h] - float(hv));
      }
    }
    // the tile's 32 columns of token nl: 2 per lane, 4 lanes (g) per wave
    float sm = v[0] + v[1];
    sm += __shfl_xor(sm, 16);
    sm += __shfl_xor(sm, 32);
    if (g == 0) red[wave][nl] = sm;
    __syncthreads();
    if (int(threadIdx.x) < j.m)
      a.asum[size_t(j.base + threadIdx.x) * (I / 32) + tile] =
          (red[0][threadIdx.x] + red[1][threadIdx.x]) + (red[2][threadIdx.x] + red[3][threadIdx.x]);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ P4
// down: work item (job, 64 output rows); writes the routing-weighted rows of
// every (row, rank) entry of the job.
__global__ __launch_bounds__(kThreads) void pf_down_kernel(PrefillArgs a) {
  __shared__ DownBuf buf;
  const int H = a.hidden, I = a.inter;
  const int tile = blockIdx.x;   // grid: (tile, sub-job)
  const int n_jobs = a.meta[0];
  Job j = job_of(a, blockIdx.y);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, nl = lane & 15;
  for (int sj = blockIdx.y; sj < n_jobs; sj += gridDim.y) {
    if (sj != int(blockIdx.y)) j = job_of(a, sj);
    const bool ok = record_ok(j.desc, a.pool_bytes, H, I);
    floatx4 acc = {0, 0, 0, 0};
    if (ok) {
      const int bits = bits_of_tag(j.desc);
      const RecordLayout R = record_layout(H, I, bits);
      const uint8_t *rec = a.pool + (j.desc & ~uint64_t(255));
      TileSrc src;
      src.codes = rsrc(rec + R.d_codes, R.d_sb - R.d_codes);
      src.group_major = true;
      src.row_bytes = R.d_row_bytes;
      src.rows_total = H;
      src.sb = reinterpret_cast<const uint32_t *>(rec + R.d_sb);
      src.sb_group_major = true;
      src.sb_stride = H;
      src.bh = a.act;
      src.bl = a.act + size_t(a.act_rows) * I;
      src.xsum = a.asum;
      src.parts = 2;
      src.K = I;
      src.r0 = tile * 64;
      src.m = j.m;
      src.lane_brow = j.base + min(lane, j.m - 1);   // the job's act rows
      switch (bits) {
        case 4: mfma_tile_down<4>(src, buf, acc); break;
        case 3: mfma_tile_down<3>(src, buf, acc); break;
        default: mfma_tile_down<2>(src, buf, acc); break;
      }
    } else if (threadIdx.x == 0) {
      __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (nl < j.m) {
      int row, rank;
      float wgt;
      if (j.e < 0) {
        row = entry_token_row(a, j, nl);
        rank = a.top_k;
        wgt = a.gamma[row];
      } else {
        row = a.entry_row[j.base + nl];
        rank = a.entry_rank[j.base + nl];
        wgt = a.topk_w[row * a.top_k + rank];
      }
      float *dst = a.y + (size_t(row) * (a.top_k + 1) + rank) * H + tile * 64 + wave * 16 + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = ok ? wgt * acc[q] : 0.0f;
    }
  }
}

// ------------------------------------------------------------------ P5
// Four columns a thread, 64-thread blocks (the chunk's 256 KB of output
// spread over every CU); all k + 1 rank rows are loaded before the sum (the
// loads are unconditional, clamped to row k, so that none waits for the
// previous one), which then runs in rank order (shared expert last).
constexpr int kCombineThreads = 64;
__global__ __launch_bounds__(kCombineThreads) void pf_combine_kernel(PrefillArgs a) {
  const int H = a.hidden, k = a.top_k;
  for (int i = blockIdx.x * kCombineThreads + threadIdx.x; i < a.t * H / 4; i += gridDim.x * kCombineThreads) {
    const int r = 4 * i / H, h = 4 * i - r * H;
    const float *y = a.y + size_t(r) * (k + 1) * H + h;
    float4 yv[kMaxTopK + 1];
#pragma unroll
    for (int c = 0; c <= kMaxTopK; ++c) yv[c] = *reinterpret_cast<const float4 *>(y + size_t(min(c, k)) * H);
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int c = 0; c <= kMaxTopK; ++c) {
      const bool on = c <= k;
      v.x += on ? yv[c].x : 0.0f;
      v.y += on ? yv[c].y : 0.0f;
      v.z += on ? yv[c].z : 0.0f;
      v.w += on ? yv[c].w : 0.0f;
    }
    *reinterpret_cast<float4 *>(a.out + size_t(r) * H + h) = v;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, const uint16_t *router, const uint16_t *gvec,
                          double *logits, float *gamma, uint32_t *topk_idx, hipStream_t s,
                          hipEvent_t *stage_ev, int n_ev) {
  auto mark = [&](int i) -> hipError_t {
    if (i < n_ev && stage_ev[i]) return hipEventRecord(stage_ev[i], s);
    return hipSuccess;
  };
  hipError_t e;
  const int split_blocks = (a.t * a.hidden / 16 + kThreads - 1) / kThreads;
  const int route_blocks = pf_router_blocks(a.n_experts, a.t) + split_blocks;
  hipLaunchKernelGGL(pf_router_kernel, dim3(route_blocks), dim3(kThreads), 0, s, a, router, gvec,
                     logits, gamma);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(pf_topk_kernel, dim3(a.t), dim3(128), 0, s, a, logits, topk_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(0)) != hipSuccess) return e;
  const int max_jobs = min(a.n_experts, a.t * a.top_k) + 1;
  // (tile, sub-job) grids of at most 1024 blocks; sub-jobs past the count
  // exit at once, and those past the grid are taken in strides
  const int gu_tiles = 2 * a.inter / 64, d_tiles = a.hidden / 64;
  const dim3 gu_grid(gu_tiles, min(max_jobs, max(1, 1024 / gu_tiles)));
  hipLaunchKernelGGL(pf_gate_up_kernel, gu_grid, dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(1)) != hipSuccess) return e;
  const dim3 d_grid(d_tiles, min(max_jobs, max(1, 1024 / d_tiles)));
  hipLaunchKernelGGL(pf_down_kernel, d_grid, dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(2)) != hipSuccess) return e;
  const int c_grid = min((a.t * a.hidden / 4 + kCombineThreads - 1) / kCombineThreads, 4096);
  hipLaunchKernelGGL(pf_combine_kernel, dim3(c_grid), dim3(kCombineThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(3);
}

}  // namespace moe
