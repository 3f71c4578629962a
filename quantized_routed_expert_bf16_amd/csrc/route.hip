// Router matvec, top-k softmax, union and slot table of one decode step
// (moe_route without the experts), for gfx950.
//
// Struct Gpu router_b: softmax over the router logits and top-k selection
// for nb rows; gpu.rs union_of: the distinct experts in the order they are
// first met; gpu.rs slot_tab / wmap field
// docs: 64 descriptors per layer, entry 62 = resident count, 63 = union size,
// per-row routing weight per slot.
//
// One launch does everything: every wave computes whole router rows (the E
// expert rows plus the shared-gate vector as row E) with float64 accumulation
// of exact bf16 x f32 products, then the last block to finish (a device-scope
// counter) ranks the logits and publishes the routing tables.  No host round
// trip and no second launch.
#include "device_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Logits of rows [row0, row0+NV) for router row `e` (e == E: shared gate).
template <int NV>
__device__ inline void router_rows(const RouteArgs &a, int e, int row0, int lane) {
  const uint16_t *w = (e < a.n_experts) ? a.router + size_t(e) * a.hidden : a.gvec;
  double acc[NV];
#pragma unroll
  for (int b = 0; b < NV; ++b) acc[b] = 0.0;
  // lane l takes 32-input chunks l, l + 64, ..., 8 inputs at a time: the
  // same order (and so the same float64 sums) as the fused layer kernel
  for (int t = 0; (lane + 64 * (t / 4)) * kChunk < a.hidden; ++t) {
    const int i0 = (lane + 64 * (t / 4)) * kChunk + 8 * (t % 4);
    const uint4 wv = *reinterpret_cast<const uint4 *>(w + i0);
    const float wf[8] = {bf16_lo(wv.x), bf16_hi(wv.x), bf16_lo(wv.y), bf16_hi(wv.y),
                         bf16_lo(wv.z), bf16_hi(wv.z), bf16_lo(wv.w), bf16_hi(wv.w)};
#pragma unroll
    for (int b = 0; b < NV; ++b) {
      const float4 *xp = reinterpret_cast<const float4 *>(a.x + size_t(row0 + b) * a.hidden + i0);
      const float4 x0 = xp[0], x1 = xp[1];
      const float xf[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[b] = fma(double(wf[t]), double(xf[t]), acc[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < NV; ++b) {
    const double s = wave_sum_d(acc[b]);
    if (lane == 0) {
      if (e < a.n_experts)
        st_dev(a.logits + size_t(row0 + b) * a.n_experts + e, s);
      else
        st_dev(a.gamma + row0 + b, float(1.0 / (1.0 + exp(-s))));
    }
  }
}

__device__ inline void router_matvec(const RouteArgs &a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_rows = a.n_experts + 1;
  for (int e = blockIdx.x * kWaves + wave; e < n_rows; e += gridDim.x * kWaves) {
    int r = 0;
    for (; r + 4 <= a.rows; r += 4) router_rows<4>(a, e, r, lane);
    switch (a.rows - r) {
      case 3: router_rows<3>(a, e, r, lane); break;
      case 2: router_rows<2>(a, e, r, lane); break;
      case 1: router_rows<1>(a, e, r, lane); break;
      default: break;
    }
  }
}

// Returns true in the one block that arrives last; it then reads the other
// blocks' logits with device-coherent loads.
__device__ inline bool arrive_last(uint32_t *counter) {
  __shared__ uint32_t prev;
  block_signal(counter, 1u, &prev);
  __syncthreads();
  return prev == gridDim.x - 1;
}

// Top-k of `rows` rows from logits in LDS: rank of expert e in row b is the
// number of experts ordered before it by (logit descending, id ascending).
__device__ inline void rank_topk(const double *lg, int rows, int E, int k, int *sel) {
  // every slot gets a valid id even if non-finite logits make ranks collide
  for (int p = threadIdx.x; p < rows * kMaxTopK; p += kThreads) sel[p] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < rows * E; p += kThreads) {
    const int b = p / E, e = p - b * E;
    const double v = lg[b * E + e];
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const double u = lg[b * E + f];
      rank += (u > v) || (u == v && f < e);
    }
    if (rank < k) sel[b * kMaxTopK + rank] = e;
  }
}

// Softmax over the selected logits of each row (float64), written to the
// caller's topk buffers and kept in LDS.
__device__ inline void topk_weights(const RouteArgs &a, const double *lg, const int *sel,
                                    float *wsel) {
  const int E = a.n_experts, k = a.top_k;
  for (int b = threadIdx.x; b < a.rows; b += kThreads) {
    const double m = lg[b * E + sel[b * kMaxTopK]];
    double sum = 0.0;
    for (int r = 0; r < k; ++r) sum += exp(lg[b * E + sel[b * kMaxTopK + r]] - m);
    for (int r = 0; r < k; ++r) {
      const int e = sel[b * kMaxTopK + r];
      const float w = float(exp(lg[b * E + e] - m) / sum);
      wsel[b * kMaxTopK + r] = w;
      a.topk_idx[b * k + r] = uint32_t(e);
      a.topk_w[b * k + r] = w;
    }
  }
}

__global__ __launch_bounds__(kThreads) void route_decode_kernel(RouteArgs a) {
  router_matvec(a);
  if (!arrive_last(a.counter)) return;

  __shared__ double lg[kMaxNb * kMaxExperts];
  __shared__ int sel[kMaxNb * kMaxTopK];
  __shared__ float wsel[kMaxNb * kMaxTopK];
  __shared__ int first[kMaxNb * kMaxTopK];
  __shared__ int uid[kSlotStride];
  const int E = a.n_experts, k = a.top_k, nb = a.rows;
  for (int p = threadIdx.x; p < nb * E; p += kThreads) lg[p] = ld_dev(a.logits + p);
  __syncthreads();
  rank_topk(lg, nb, E, k, sel);
  __syncthreads();
  topk_weights(a, lg, sel, wsel);

  // first-seen union over the row-major (row, rank) list
  const int n = nb * k;
  for (int p = threadIdx.x; p < n; p += kThreads) {
    const int e = sel[(p / k) * kMaxTopK + p % k];
    int f = 1;
    for (int q = 0; q < p; ++q) f &= (sel[(q / k) * kMaxTopK + q % k] != e);
    first[p] = f;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < n; p += kThreads) {
    if (!first[p]) continue;
    int slot = 0;
    for (int q = 0; q < p; ++q) slot += first[q];
    uid[slot] = sel[(p / k) * kMaxTopK + p % k];
  }
  __syncthreads();
  int u = 0;
  for (int q = 0; q < n; ++q) u += first[q];
  for (int j = threadIdx.x; j < kSlotStride; j += kThreads) {
    if (j < u) {
      a.ids[j] = uint32_t(uid[j]);
      a.tab[j] = a.rec[uid[j]];
    } else {
      a.ids[j] = 0;
      if (j < MOE_RESIDENT_ENTRY) a.tab[j] = 0;
    }
    if (j == MOE_RESIDENT_ENTRY || j == MOE_UNION_ENTRY) a.tab[j] = uint64_t(u);
    for (int b = 0; b < kMaxNb; ++b) {
      float w = 0.0f;
      if (b < nb && j < u)
        for (int r = 0; r < k; ++r)
          if (sel[b * kMaxTopK + r] == uid[j]) w = wsel[b * kMaxTopK + r];
      a.wmap[b * kSlotStride + j] = w;
    }
  }
  if (threadIdx.x == 0) st_dev(a.counter, 0u);
}

__global__ void fill_zero_kernel(uint4 *p, size_t n16) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n16;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

int route_blocks(int n_experts) { return (n_experts + 1 + kWaves - 1) / kWaves; }

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(route_decode_kernel, dim3(route_blocks(a.n_experts)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                     static_cast<uint4 *>(p), n16);
  return hipGetLastError();
}

}  // namespace moe
