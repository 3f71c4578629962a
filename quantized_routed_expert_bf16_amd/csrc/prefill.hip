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
//   P2 per-row top-k and weights; the last block groups the rows by expert
//      (experts ascending, rows ascending) and lists the experts in use;
//   P3 gate/up: per (used expert, 64 gate/up rows), MFMA 16x16x32 f16 tiles
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
#include "device_common.h"

namespace moe {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTok = MOE_MAX_PREFILL_ROWS;   // 32 token slots per expert
constexpr int kSlab = 256;                   // gate/up K slab (4 groups)
constexpr int kBStride = kSlab + 8;          // halfs per token row in LDS (bank spread)

// ------------------------------------------------------------------ P1
constexpr int kRouteTok = 4;   // rows per router block

// Block (rb, tg): router rows 4 rb + wave (row E = shared gate) for rows
// kRouteTok tg .. +kRouteTok, float64 accumulation; then every block takes a
// share of the x -> f16 hi/lo split and the per-64 group sums.
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
    for (int i0 = lane * 8; i0 < H; i0 += 1024) {
      uint4 wv[2];
      float4 xv[2][kRouteTok][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {   // two 512-input steps in flight
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
      for (int u = 0; u < 2; ++u) {
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
  // x -> f16 hi/lo halves and per-64 group sums: 8 values a thread, the 8
  // threads of a group add their sums with a DPP reduction
  for (int i0 = blockIdx.x * kThreads; i0 < t * H / 8; i0 += gridDim.x * kThreads) {
    const int i = i0 + threadIdx.x;
    const bool live = i < t * H / 8;
    const int il = live ? i : 0;
    const float4 v0 = *reinterpret_cast<const float4 *>(a.x + size_t(il) * 8);
    const float4 v1 = *reinterpret_cast<const float4 *>(a.x + size_t(il) * 8 + 4);
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    _Float16 hi[8], lo[8];
    float sm = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      hi[q] = _Float16(v[q]);
      lo[q] = _Float16(v[q] - float(hi[q]));
      sm += v[q];
    }
    sm = group8_sum(sm);
    if (live) {
      const int r = il / (H / 8), c = (il - r * (H / 8)) * 8;
      __builtin_memcpy(a.xh + size_t(r) * H + c, hi, 16);
      __builtin_memcpy(a.xh + size_t(kTok + r) * H + c, lo, 16);
      if ((il & 7) == 0) a.xg[size_t(r) * (H / kGroup) + c / kGroup] = sm;
    }
  }
}

// ------------------------------------------------------------------ P2
__global__ __launch_bounds__(128) void pf_topk_kernel(PrefillArgs a, const double *logits,
                                                      uint32_t *topk_idx, uint32_t *counter,
                                                      int32_t *expert_ptr, int32_t *entry_row,
                                                      int32_t *entry_rank) {
  __shared__ double lg[kMaxExperts];
  __shared__ int sel[kMaxTopK];
  __shared__ double selv[kMaxTopK];
  __shared__ uint32_t prev;
  __shared__ int all_sel[kTok * kMaxTopK];
  __shared__ int cnt[kMaxExperts + 1];
  __shared__ uint32_t emask[kMaxExperts];
  __shared__ int wsum[2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = a.n_experts, k = a.top_k, t = a.t;
  const int r = blockIdx.x;
  const int Ep = (E + 7) & ~7;
  for (int e = threadIdx.x; e < Ep; e += 128) lg[e] = e < E ? logits[size_t(r) * E + e] : -__builtin_inf();
  if (threadIdx.x < kMaxTopK) sel[threadIdx.x] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 128) {
    const double v = lg[e];
    const double2 *row = reinterpret_cast<const double2 *>(lg);
    int rank = 0;
    for (int f2 = 0; f2 < Ep / 2; f2 += 4) {
      const double2 o0 = row[f2], o1 = row[f2 + 1], o2 = row[f2 + 2], o3 = row[f2 + 3];
      const int f = 2 * f2;
      rank += int(o0.x > v) + int(o0.y > v) + int(o1.x > v) + int(o1.y > v) +
              int(o2.x > v) + int(o2.y > v) + int(o3.x > v) + int(o3.y > v);
      rank += (int(o0.x == v) & int(f < e)) + (int(o0.y == v) & int(f + 1 < e)) +
              (int(o1.x == v) & int(f + 2 < e)) + (int(o1.y == v) & int(f + 3 < e)) +
              (int(o2.x == v) & int(f + 4 < e)) + (int(o2.y == v) & int(f + 5 < e)) +
              (int(o3.x == v) & int(f + 6 < e)) + (int(o3.y == v) & int(f + 7 < e));
    }
    if (rank < k) { sel[rank] = e; selv[rank] = v; }
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
  block_signal(counter, 1u, &prev);
  __syncthreads();
  if (prev != uint32_t(t - 1)) return;
  // last block: rows grouped by expert, experts ascending, rows ascending.
  // Each expert gets a mask of the rows that selected it (a row selects an
  // expert at most once, t <= 32); an entry's place is the expert's start
  // plus the rows below it in that mask.
  for (int p = threadIdx.x; p < t * k; p += 128) all_sel[p] = int(ld_dev(topk_idx + p));
  for (int e = threadIdx.x; e < kMaxExperts; e += 128) emask[e] = 0u;
  __syncthreads();
  for (int p = threadIdx.x; p < t * k; p += 128) atomicOr(&emask[all_sel[p]], 1u << (p / k));
  __syncthreads();
  // exclusive scan over experts of (rows << 16 | used), two experts a thread
  {
    const int e0 = 2 * threadIdx.x, e1 = e0 + 1;
    const int c0 = e0 < E ? __popc(emask[e0]) : 0, c1 = e1 < E ? __popc(emask[e1]) : 0;
    const int v0 = (c0 << 16) | int(c0 > 0), v1 = (c1 << 16) | int(c1 > 0);
    int incl = v0 + v1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    const int excl = incl - (v0 + v1) + (wave ? wsum[0] : 0);
    if (e0 < E) { cnt[e0] = excl; }
    if (e1 < E) { cnt[e1] = excl + v0; }
    if (threadIdx.x == 0) cnt[E] = wsum[0] + wsum[1];
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += 128) {
    const int v = cnt[e];
    expert_ptr[e] = v >> 16;
    if (e < E && emask[e]) a.meta[1 + (v & 0xffff)] = e;
  }
  if (threadIdx.x == 0) a.meta[0] = cnt[E] & 0xffff;
  for (int p = threadIdx.x; p < t * k; p += 128) {
    const int e = all_sel[p], r = p / k;
    const int pos = (cnt[e] >> 16) + __popc(emask[e] & ((1u << r) - 1u));
    entry_row[pos] = r;
    entry_rank[pos] = p - r * k;
  }
  if (threadIdx.x == 0) st_dev(counter, 0u);
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

__device__ inline int code_offset(int bits, int s, int j) {
  return bits == 4 ? 8 * s + j / 2 + 4 * (j % 2) : 4 * s + j / 2 + 8 * (j % 2);
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

struct Job {
  int e;        // expert id, or -1 for the shared expert
  int base;     // first entry index of its rows
  int m;        // rows
  uint64_t desc;
};

__device__ inline bool job_of(const PrefillArgs &a, int ui, Job &j) {
  const int n_used = a.meta[0];
  if (ui < n_used) {
    j.e = a.meta[1 + ui];
    j.base = a.expert_ptr[j.e];
    j.m = a.expert_ptr[j.e + 1] - j.base;
    j.desc = a.rec[j.e];
    return true;
  }
  if (ui == n_used) {
    j.e = -1;
    j.base = a.t * a.top_k;
    j.m = a.t;
    j.desc = a.shared_rec;
    return true;
  }
  return false;
}

__device__ inline int entry_token_row(const PrefillArgs &a, const Job &j, int n) {
  return j.e < 0 ? n : a.entry_row[j.base + n];
}

// ------------------------------------------------------------------ P3
template <int BITS>
__device__ void gate_up_tile(const PrefillArgs &a, const Job &j, int tile, _Float16 *bh, _Float16 *bl,
                             float *xg_lds, uint32_t *sb_lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.hidden, I = a.inter, groups = H / kGroup;
  const RecordLayout L = record_layout(H, I, BITS);
  const uint8_t *rec = a.pool + (j.desc & ~uint64_t(255));
  const int R0 = tile * 64 + wave * 16;            // first gate/up row of this wave
  const int arow = R0 + (lane & 15), g = lane >> 4;
  const uint8_t *codes = rec + L.gu_codes + size_t(arow) * L.gu_row_bytes;
  const uint32_t *sb = reinterpret_cast<const uint32_t *>(rec + L.gu_sb);
  const int nt = (j.m + 15) / 16;
  floatx4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};

  for (int slab = 0; slab < H / kSlab; ++slab) {
    __syncthreads();
    // stage x (hi, lo) of the tokens for this slab in MFMA B order, and the
    // group sums of x; padding tokens are zero
    for (int it = threadIdx.x; it < kTok * 16; it += kThreads) {
      const int n = it >> 4, Q = (it >> 2) & 3, gg = it & 3;
      const int k0 = slab * kSlab + 64 * Q + 16 * gg;
      _Float16 vh[16], vl[16];
      if (n < j.m) {
        const int row = entry_token_row(a, j, n);
        const uint4 *ph = reinterpret_cast<const uint4 *>(a.xh + size_t(row) * H + k0);
        const uint4 *pl = reinterpret_cast<const uint4 *>(a.xh + size_t(kTok + row) * H + k0);
        const uint4 h0 = ph[0], h1 = ph[1], l0 = pl[0], l1 = pl[1];
        __builtin_memcpy(vh, &h0, 16); __builtin_memcpy(vh + 8, &h1, 16);
        __builtin_memcpy(vl, &l0, 16); __builtin_memcpy(vl + 8, &l1, 16);
      } else {
        for (int q = 0; q < 16; ++q) vh[q] = vl[q] = _Float16(0.0f);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        _Float16 oh[8], ol[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int o = code_offset(BITS, s, jj);
          oh[jj] = vh[o];
          ol[jj] = vl[o];
        }
        const int at = n * kBStride + ((Q * 4 + gg) * 2 + s) * 8;
        __builtin_memcpy(bh + at, oh, 16);
        __builtin_memcpy(bl + at, ol, 16);
      }
    }
    for (int it = threadIdx.x; it < kTok * 4; it += kThreads) {
      const int n = it >> 2, Q = it & 3;
      xg_lds[it] = n < j.m ? a.xg[size_t(entry_token_row(a, j, n)) * groups + slab * 4 + Q] : 0.0f;
    }
    // (scale, bias) of the 16 rows x 4 groups of each wave, for the C layout
    {
      const int rr = R0 + (lane >> 2), Q = lane & 3;
      sb_lds[wave * 64 + lane] = sb[size_t(rr) * groups + slab * 4 + Q];
    }
    __syncthreads();
#pragma unroll
    for (int Q = 0; Q < 4; ++Q) {
      uint32_t w[3];
      load16<BITS>(codes, H, slab * kSlab + 64 * Q + 16 * g, w);
      half8 A[2];
      codes_to_a<BITS>(w, A, (g & 1));
      float sc[4], bi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t v = sb_lds[wave * 64 + (4 * g + q) * 4 + Q];
        sc[q] = sb_scale(v);
        bi[q] = sb_bias(v);
      }
      for (int tt = 0; tt < nt; ++tt) {
        floatx4 cg = {0, 0, 0, 0};
        const int n = tt * 16 + (lane & 15);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int at = n * kBStride + ((Q * 4 + g) * 2 + s) * 8;
          const half8 Bh = *reinterpret_cast<const half8 *>(bh + at);
          const half8 Bl = *reinterpret_cast<const half8 *>(bl + at);
          cg = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[s], Bh, cg, 0, 0, 0);
          cg = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[s], Bl, cg, 0, 0, 0);
        }
        const float xs = xg_lds[n * 4 + Q];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[tt][q] += fmaf(sc[q], cg[q], bi[q] * xs);
      }
    }
  }
  // rows 4g+q of the tile: (gate, up) pairs (q = 0,1) and (q = 2,3)
  for (int tt = 0; tt < nt; ++tt) {
    const int n = tt * 16 + (lane & 15);
    if (n >= j.m) continue;
    const int p0 = (R0 + 4 * g) / 2;
    float *dst = a.act + size_t(j.base + n) * I;
    dst[p0] = silu_mul(acc[tt][0], acc[tt][1]);
    dst[p0 + 1] = silu_mul(acc[tt][2], acc[tt][3]);
  }
}

__global__ __launch_bounds__(kThreads) void pf_gate_up_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 bh[kTok * kBStride];
  __shared__ __attribute__((aligned(16))) _Float16 bl[kTok * kBStride];
  __shared__ float xg_lds[kTok * 4];
  __shared__ uint32_t sb_lds[kWaves * 64];
  const int tiles = 2 * a.inter / 64;
  const int n_jobs = a.meta[0] + 1;
  for (int w = blockIdx.x; w < n_jobs * tiles; w += gridDim.x) {
    Job j;
    if (!job_of(a, w / tiles, j)) break;
    if (!record_ok(j.desc, a.pool_bytes, a.hidden, a.inter)) {
      if (threadIdx.x == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // zero this tile's act values so the down pass stays finite
      const int tile = w % tiles;
      for (int i = threadIdx.x; i < j.m * 32; i += kThreads)
        a.act[size_t(j.base + i / 32) * a.inter + tile * 32 + i % 32] = 0.0f;
      continue;
    }
    switch (bits_of_tag(j.desc)) {
      case 4: gate_up_tile<4>(a, j, w % tiles, bh, bl, xg_lds, sb_lds); break;
      case 3: gate_up_tile<3>(a, j, w % tiles, bh, bl, xg_lds, sb_lds); break;
      default: gate_up_tile<2>(a, j, w % tiles, bh, bl, xg_lds, sb_lds); break;
    }
  }
}

// ------------------------------------------------------------------ P4
constexpr int kActStride = 512 + 8;   // halfs per token row of one 512-wide K pass

template <int BITS>
__device__ void down_tile(const PrefillArgs &a, const Job &j, int tile, _Float16 *ah, _Float16 *al,
                          float *as_lds, float *sb_lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.hidden, I = a.inter, gpr = I / kGroup;
  const RecordLayout L = record_layout(H, I, BITS);
  const uint8_t *rec = a.pool + (j.desc & ~uint64_t(255));
  const uint32_t *sb = reinterpret_cast<const uint32_t *>(rec + L.d_sb);
  const int R0 = tile * 64 + wave * 16;            // first output row of this wave
  const int arow = R0 + (lane & 15), g = lane >> 4;
  const int nt = (j.m + 15) / 16;
  const int gb = kGroup * BITS / 8;                // bytes of one row's group
  floatx4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};

  for (int k0 = 0; k0 < I; k0 += 512) {            // K passes of up to 8 groups
    const int gq = min(8, (I - k0) / kGroup);
    __syncthreads();
    for (int it = threadIdx.x; it < kTok * gq * 4; it += kThreads) {
      const int n = it / (gq * 4), Q = (it >> 2) % gq, gg = it & 3;
      float v[16];
      if (n < j.m) {
        const float *src = a.act + size_t(j.base + n) * I + k0 + 64 * Q + 16 * gg;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 f = *reinterpret_cast<const float4 *>(src + 4 * q);
          v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
      } else {
        for (int q = 0; q < 16; ++q) v[q] = 0.0f;
      }
      float sm = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) sm += v[q];
      as_lds[it] = sm;                                      // [n][Q][gg] partial sums
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        _Float16 oh[8], ol[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float x = v[code_offset(BITS, s, jj)];
          oh[jj] = _Float16(x);
          ol[jj] = _Float16(x - float(oh[jj]));
        }
        const int at = n * kActStride + ((Q * 4 + gg) * 2 + s) * 8;
        __builtin_memcpy(ah + at, oh, 16);
        __builtin_memcpy(al + at, ol, 16);
      }
    }
    for (int it = threadIdx.x; it < 64 * gq; it += kThreads) {   // 64 rows x gq groups
      const int wv = it / (16 * gq), rr = (it / gq) % 16, Q = it % gq;
      const int row = tile * 64 + wv * 16 + rr;
      sb_lds[(wv * 16 + rr) * 8 + Q] = __uint_as_float(sb[size_t(k0 / kGroup + Q) * H + row]);
    }
    __syncthreads();
    for (int Q = 0; Q < gq; ++Q) {
      const int grp = k0 / kGroup + Q;
      uint32_t w[3];
      const uint8_t *grow = rec + L.d_codes + (size_t(grp) * H + arow) * gb;
      load16<BITS>(grow, kGroup, 16 * g, w);
      half8 A[2];
      codes_to_a<BITS>(w, A, (g & 1));
      float sc[4], bi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t v = __float_as_uint(sb_lds[(wave * 16 + 4 * g + q) * 8 + Q]);
        sc[q] = sb_scale(v);
        bi[q] = sb_bias(v);
      }
      for (int tt = 0; tt < nt; ++tt) {
        floatx4 cg = {0, 0, 0, 0};
        const int n = tt * 16 + (lane & 15);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int at = n * kActStride + ((Q * 4 + g) * 2 + s) * 8;
          const half8 Bh = *reinterpret_cast<const half8 *>(ah + at);
          const half8 Bl = *reinterpret_cast<const half8 *>(al + at);
          cg = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[s], Bh, cg, 0, 0, 0);
          cg = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[s], Bl, cg, 0, 0, 0);
        }
        const float* asn = as_lds + (n * gq + Q) * 4;
        const float xs = (asn[0] + asn[1]) + (asn[2] + asn[3]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[tt][q] += fmaf(sc[q], cg[q], bi[q] * xs);
      }
    }
  }
  (void)gpr;
  // routing-weighted output rows of every entry, one (row, rank) slot each
  for (int tt = 0; tt < nt; ++tt) {
    const int n = tt * 16 + (lane & 15);
    if (n >= j.m) continue;
    const int p = j.base + n;
    int row, rank;
    float wgt;
    if (j.e < 0) {
      row = n;
      rank = a.top_k;
      wgt = a.gamma[n];
    } else {
      row = a.entry_row[p];
      rank = a.entry_rank[p];
      wgt = a.topk_w[row * a.top_k + rank];
    }
    float *dst = a.y + (size_t(row) * (a.top_k + 1) + rank) * H + R0 + 4 * g;
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = wgt * acc[tt][q];
  }
}

__global__ __launch_bounds__(kThreads) void pf_down_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 ah[kTok * kActStride];
  __shared__ __attribute__((aligned(16))) _Float16 al[kTok * kActStride];
  __shared__ float as_lds[kTok * 8 * 4];
  __shared__ float sb_lds[64 * 8];
  const int tiles = a.hidden / 64;
  const int n_jobs = a.meta[0] + 1;
  for (int w = blockIdx.x; w < n_jobs * tiles; w += gridDim.x) {
    Job j;
    if (!job_of(a, w / tiles, j)) break;
    const int tile = w % tiles;
    if (!record_ok(j.desc, a.pool_bytes, a.hidden, a.inter)) {
      if (threadIdx.x == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = threadIdx.x; i < j.m * 64; i += kThreads) {
        const int n = i / 64, h = tile * 64 + i % 64;
        const int row = j.e < 0 ? n : a.entry_row[j.base + n];
        const int rank = j.e < 0 ? a.top_k : a.entry_rank[j.base + n];
        a.y[(size_t(row) * (a.top_k + 1) + rank) * a.hidden + h] = 0.0f;
      }
      continue;
    }
    switch (bits_of_tag(j.desc)) {
      case 4: down_tile<4>(a, j, tile, ah, al, as_lds, sb_lds); break;
      case 3: down_tile<3>(a, j, tile, ah, al, as_lds, sb_lds); break;
      default: down_tile<2>(a, j, tile, ah, al, as_lds, sb_lds); break;
    }
  }
}

// ------------------------------------------------------------------ P5
__global__ __launch_bounds__(kThreads) void pf_combine_kernel(PrefillArgs a) {
  const int H = a.hidden, k = a.top_k;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < a.t * H; i += gridDim.x * kThreads) {
    const int r = i / H, h = i - r * H;
    const float *y = a.y + size_t(r) * (k + 1) * H + h;
    float v = 0.0f;
    for (int c = 0; c < k; ++c) v += y[size_t(c) * H];
    v += y[size_t(k) * H];
    a.out[i] = v;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, const uint16_t *router, const uint16_t *gvec,
                          double *logits, float *gamma, uint32_t *topk_idx, uint32_t *counter,
                          int32_t *expert_ptr, int32_t *entry_row, int32_t *entry_rank,
                          hipStream_t s, hipEvent_t *stage_ev, int n_ev) {
  auto mark = [&](int i) -> hipError_t {
    if (i < n_ev && stage_ev[i]) return hipEventRecord(stage_ev[i], s);
    return hipSuccess;
  };
  hipError_t e;
  const int route_blocks = (a.n_experts + 1 + kWaves - 1) / kWaves * ((a.t + kRouteTok - 1) / kRouteTok);
  hipLaunchKernelGGL(pf_router_kernel, dim3(route_blocks), dim3(kThreads), 0, s, a, router, gvec,
                     logits, gamma);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(pf_topk_kernel, dim3(a.t), dim3(128), 0, s, a, logits, topk_idx, counter,
                     expert_ptr, entry_row, entry_rank);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(0)) != hipSuccess) return e;
  const int max_jobs = min(a.n_experts, a.t * a.top_k) + 1;
  const int gu_grid = min(max_jobs * (2 * a.inter / 64), 1024);
  hipLaunchKernelGGL(pf_gate_up_kernel, dim3(gu_grid), dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(1)) != hipSuccess) return e;
  const int d_grid = min(max_jobs * (a.hidden / 64), 1024);
  hipLaunchKernelGGL(pf_down_kernel, dim3(d_grid), dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(2)) != hipSuccess) return e;
  const int c_grid = min((a.t * a.hidden + kThreads - 1) / kThreads, 1024);
  hipLaunchKernelGGL(pf_combine_kernel, dim3(c_grid), dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(3);
}

}  // namespace moe
