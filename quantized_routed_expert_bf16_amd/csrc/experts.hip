// Decode expert kernels for gfx950: fused gate/up matvec + silu(gate)*up, and
// down matvec + routing-weighted combine with the sigmoid-gated shared expert.
//
// Struct Gpu experts_b: the routed experts of the union published in the slot
// table plus the shared expert, summed per row; gpu.rs struct Q: affine
// quantized projection with per-group scale and bias; load.rs load_bounded:
// 3/2-bit low-bit records with their own unpacking (kind per record).
//
// Both kernels are bandwidth kernels over packed codes.  A lane owns one
// 32-code chunk of a row (16 B of 4-bit codes, one 128-bit load; 12 B of 3-bit
// codes, 8 + 4 B; 8 B of 2-bit codes) and keeps the matching 32 activations of
// every row in registers for the whole kernel, so activations are read once
// per wave, not once per weight row.  Codes are expanded with one AND per four
// codes and a byte->float conversion per code; the group scale and bias are
// applied once per chunk (y = s * sum(q x) + b * sum(x)), with f32 FMAs.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTileRowPairs = 8;                  // gate/up row pairs per work unit
constexpr int kPairsPerWave = kTileRowPairs / kWaves;

__device__ inline float byte_f(uint32_t v, int k) { return float((v >> (8 * k)) & 0xffu); }
__device__ inline float sb_scale(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float sb_bias(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Codes of one 32-code chunk as loaded: 4-bit: w[0..3]; 2-bit: w[0..1];
// 3-bit: w[0..1] low plane, w[2] high plane.
template <int BITS>
__device__ inline void load_chunk(const uint8_t *row, int row_codes, int chunk, uint32_t (&w)[4]) {
  if constexpr (BITS == 4) {
    const uint4 v = *reinterpret_cast<const uint4 *>(row + chunk * 16);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2 *>(row + chunk * 8);
    w[0] = v.x; w[1] = v.y; w[2] = 0; w[3] = 0;
  } else {
    const uint2 v = *reinterpret_cast<const uint2 *>(row + chunk * 8);
    w[0] = v.x; w[1] = v.y;
    w[2] = *reinterpret_cast<const uint32_t *>(row + row_codes / 4 + chunk * 4);
    w[3] = 0;
  }
}

// P[b] = sum_t q_t * x[b][t] over the chunk's 32 codes.
template <int BITS, int NB>
__device__ inline void chunk_dot(const uint32_t (&w)[4], const float (&x)[NB][kChunk], float (&P)[NB]) {
  if constexpr (BITS == 4) {
    // low nibbles (even codes) and high nibbles (odd codes, x16) per byte
    float lo[NB], hi[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) lo[b] = hi[b] = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t l = w[m] & 0x0f0f0f0fu, h = w[m] & 0xf0f0f0f0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float cl = byte_f(l, k), ch = byte_f(h, k);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          lo[b] = fmaf(cl, x[b][8 * m + 2 * k], lo[b]);
          hi[b] = fmaf(ch, x[b][8 * m + 2 * k + 1], hi[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) P[b] = fmaf(hi[b], 0.0625f, lo[b]);
  } else {
    // 2-bit field p of each byte holds code 4k+p (x 4^p); 3-bit adds the
    // high bit from the high-plane byte k, bit 4m+p.
    float acc[4][NB];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[p][b] = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t l = w[m] & (0x03030303u << (2 * p));
        uint32_t h = 0;
        if constexpr (BITS == 3) h = w[2] & (0x01010101u << (4 * m + p));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float c = byte_f(l, k);
          if constexpr (BITS == 3) c = fmaf(byte_f(h, k), __builtin_ldexpf(1.0f, 2 + p - 4 * m), c);
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[p][b] = fmaf(c, x[b][16 * m + 4 * k + p], acc[p][b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
      P[b] = acc[0][b] + 0.25f * acc[1][b] + 0.0625f * acc[2][b] + 0.015625f * acc[3][b];
  }
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

template <int NB, int CPL>
__device__ inline void load_x(const float *x, int hidden, int lane, float (&xr)[CPL][NB][kChunk],
                              float (&xs)[CPL][NB]) {
  const int n_chunks = hidden / kChunk;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int chunk = lane + 64 * c;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < kChunk / 4; ++q) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (chunk < n_chunks)
          v = *reinterpret_cast<const float4 *>(x + size_t(b) * hidden + chunk * kChunk + 4 * q);
        xr[c][b][4 * q] = v.x; xr[c][b][4 * q + 1] = v.y;
        xr[c][b][4 * q + 2] = v.z; xr[c][b][4 * q + 3] = v.w;
        s += (v.x + v.y) + (v.z + v.w);
      }
      xs[c][b] = s;
    }
  }
}

__device__ inline bool record_ok(uint64_t desc, uint64_t pool_bytes, int hidden, int inter) {
  const int bits = bits_of_tag(desc);
  if (bits == 0) return false;
  const uint64_t off = desc & ~uint64_t(255);
  const RecordLayout L = record_layout(hidden, inter, bits);
  return off + L.total <= pool_bytes && off + L.total > off;
}

// ------------------------------------------------------------ gate / up
template <int NB, int CPL, int BITS>
__device__ inline void gate_up_pairs(const ExpertArgs &a, const uint8_t *rec, int j0, int act_slot,
                                     const float (&xr)[CPL][NB][kChunk], const float (&xs)[CPL][NB],
                                     int lane) {
  const int H = a.hidden, I = a.inter;
  const RecordLayout L = record_layout(H, I, BITS);
  const int n_chunks = H / kChunk, gpr = H / kGroup;
  const uint8_t *codes = rec + L.gu_codes;
  const uint32_t *sb = reinterpret_cast<const uint32_t *>(rec + L.gu_sb);

  uint32_t w[kPairsPerWave][2][CPL][4];
  uint32_t s[kPairsPerWave][2][CPL];
#pragma unroll
  for (int p = 0; p < kPairsPerWave; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 2 * (j0 + p) + h;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int chunk = lane + 64 * c;
        if (chunk < n_chunks) {
          load_chunk<BITS>(codes + size_t(row) * L.gu_row_bytes, H, chunk, w[p][h][c]);
          s[p][h][c] = sb[size_t(row) * gpr + chunk / 2];
        } else {
          w[p][h][c][0] = w[p][h][c][1] = w[p][h][c][2] = w[p][h][c][3] = 0;
          s[p][h][c] = 0;
        }
      }
    }
#pragma unroll
  for (int p = 0; p < kPairsPerWave; ++p) {
    float v[2][NB];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int b = 0; b < NB; ++b) v[h][b] = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        float P[NB];
        chunk_dot<BITS, NB>(w[p][h][c], xr[c], P);
        const float sc = sb_scale(s[p][h][c]), bi = sb_bias(s[p][h][c]);
#pragma unroll
        for (int b = 0; b < NB; ++b) v[h][b] += fmaf(sc, P[b], bi * xs[c][b]);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < NB; ++b) v[h][b] += __shfl_xor(v[h][b], off, 64);
    if (lane < NB) {
      float g = v[0][0], u = v[1][0];
#pragma unroll
      for (int b = 1; b < NB; ++b)
        if (lane == b) { g = v[0][b]; u = v[1][b]; }
      a.act[(size_t(act_slot) * kMaxNb + lane) * I + j0 + p] = silu_mul(g, u);
    }
  }
}

template <int NB, int CPL>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(ExpertArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float xr[CPL][NB][kChunk];
  float xs[CPL][NB];
  load_x<NB, CPL>(a.x, a.hidden, lane, xr, xs);

  const int u = int(a.tab[MOE_UNION_ENTRY]);
  const int units_per_slot = a.inter / kTileRowPairs;
  const int total = (u + 1) * units_per_slot;
  for (int unit = blockIdx.x; unit < total; unit += gridDim.x) {
    const int slot = unit / units_per_slot;
    const int tile = unit - slot * units_per_slot;
    const uint64_t desc = slot < u ? a.tab[slot] : a.shared_rec;
    const int act_slot = slot < u ? slot : kSharedSlot;
    const int j0 = tile * kTileRowPairs + wave * kPairsPerWave;
    if (!record_ok(desc, a.pool_bytes, a.hidden, a.inter)) {
      if (threadIdx.x == 0) atomicOr(a.status, 1u);
      if (lane < NB * kPairsPerWave)
        a.act[(size_t(act_slot) * kMaxNb + lane / kPairsPerWave) * a.inter + j0 + lane % kPairsPerWave] = 0.0f;
      continue;
    }
    const uint8_t *rec = a.pool + (desc & ~uint64_t(255));
    switch (bits_of_tag(desc)) {
      case 4: gate_up_pairs<NB, CPL, 4>(a, rec, j0, act_slot, xr, xs, lane); break;
      case 3: gate_up_pairs<NB, CPL, 3>(a, rec, j0, act_slot, xr, xs, lane); break;
      default: gate_up_pairs<NB, CPL, 2>(a, rec, j0, act_slot, xr, xs, lane); break;
    }
  }
}

// ------------------------------------------------------- down / combine
// One work unit = (tile of output rows, slot).  Each wave keeps the slot's
// 32-activation chunk per row in registers and streams its rows; the
// weighted row results go to ypart[slot]; the last unit of a tile to finish
// sums the slots of that tile in slot order (shared expert last) into out.
template <int NB, int BITS>
__device__ inline void down_rows(const ExpertArgs &a, const uint8_t *rec, int ps, int r0, int n_rows,
                                 int lpr, const float (&ar)[NB][kChunk], const float (&as)[NB],
                                 const float (&wv)[NB], int lane) {
  const int H = a.hidden, I = a.inter;
  const RecordLayout L = record_layout(H, I, BITS);
  const int gpr = I / kGroup;
  const int rps = 64 / lpr;
  const int cc = lane % lpr;
  const uint8_t *codes = rec + L.d_codes;
  const uint32_t *sb = reinterpret_cast<const uint32_t *>(rec + L.d_sb);
  constexpr int kUnroll = 2;
  for (int st = 0; st < n_rows; st += rps * kUnroll) {
    uint32_t w[kUnroll][4];
    uint32_t s[kUnroll];
    int rr[kUnroll];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      rr[q] = r0 + st + q * rps + lane / lpr;
      const bool ok = st + q * rps < n_rows;
      if (ok) {
        load_chunk<BITS>(codes + size_t(rr[q]) * L.d_row_bytes, I, cc, w[q]);
        s[q] = sb[size_t(rr[q]) * gpr + cc / 2];
      } else {
        w[q][0] = w[q][1] = w[q][2] = w[q][3] = 0;
        s[q] = 0;
      }
    }
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      if (st + q * rps >= n_rows) break;
      float P[NB], v[NB];
      chunk_dot<BITS, NB>(w[q], ar, P);
      const float sc = sb_scale(s[q]), bi = sb_bias(s[q]);
#pragma unroll
      for (int b = 0; b < NB; ++b) v[b] = fmaf(sc, P[b], bi * as[b]);
      for (int off = lpr / 2; off > 0; off >>= 1)
#pragma unroll
        for (int b = 0; b < NB; ++b) v[b] += __shfl_xor(v[b], off, 64);
      if (cc == 0)
#pragma unroll
        for (int b = 0; b < NB; ++b) a.ypart[(size_t(ps) * kMaxNb + b) * H + rr[q]] = wv[b] * v[b];
    }
  }
}

template <int NB>
__global__ __launch_bounds__(kThreads) void down_kernel(ExpertArgs a, int rows_per_tile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = a.hidden, I = a.inter;
  const int lpr = I / kChunk;
  const int u = int(a.tab[MOE_UNION_ENTRY]);
  const int n_slots = u + 1;
  const int n_tiles = H / rows_per_tile;
  const int rows_per_wave = rows_per_tile / kWaves;
  const int total = n_slots * n_tiles;
  __shared__ int last;
  for (int unit = blockIdx.x; unit < total; unit += gridDim.x) {
    const int slot = unit / n_tiles;
    const int tile = unit - slot * n_tiles;
    const uint64_t desc = slot < u ? a.tab[slot] : a.shared_rec;
    const int ps = slot < u ? slot : kSharedSlot;
    const int r0 = tile * rows_per_tile + wave * rows_per_wave;
    if (record_ok(desc, a.pool_bytes, H, I)) {
      float wv[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) wv[b] = slot < u ? a.wmap[b * kSlotStride + slot] : a.gamma[b];
      float ar[NB][kChunk], as[NB];
      const int cc = lane % lpr;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float *ap = a.act + (size_t(ps) * kMaxNb + b) * I + cc * kChunk;
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < kChunk / 4; ++q) {
          const float4 v = *reinterpret_cast<const float4 *>(ap + 4 * q);
          ar[b][4 * q] = v.x; ar[b][4 * q + 1] = v.y; ar[b][4 * q + 2] = v.z; ar[b][4 * q + 3] = v.w;
          s += (v.x + v.y) + (v.z + v.w);
        }
        as[b] = s;
      }
      const uint8_t *rec = a.pool + (desc & ~uint64_t(255));
      switch (bits_of_tag(desc)) {
        case 4: down_rows<NB, 4>(a, rec, ps, r0, rows_per_wave, lpr, ar, as, wv, lane); break;
        case 3: down_rows<NB, 3>(a, rec, ps, r0, rows_per_wave, lpr, ar, as, wv, lane); break;
        default: down_rows<NB, 2>(a, rec, ps, r0, rows_per_wave, lpr, ar, as, wv, lane); break;
      }
    } else {
      if (threadIdx.x == 0) atomicOr(a.status, 1u);
      for (int i = lane; i < rows_per_wave * NB; i += 64)
        a.ypart[(size_t(ps) * kMaxNb + i / rows_per_wave) * H + r0 + i % rows_per_wave] = 0.0f;
    }
    // arrive on the tile; the last arriving unit combines the tile
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(a.tile_count + tile, 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      last = (prev == uint32_t(n_slots - 1));
    }
    __syncthreads();
    if (last) {
      __threadfence();
      for (int i = threadIdx.x; i < rows_per_tile * NB; i += kThreads) {
        const int b = i / rows_per_tile;
        const int r = tile * rows_per_tile + i % rows_per_tile;
        float acc = 0.0f;
        for (int s = 0; s < u; ++s) acc += a.ypart[(size_t(s) * kMaxNb + b) * H + r];
        acc += a.ypart[(size_t(kSharedSlot) * kMaxNb + b) * H + r];
        a.out[size_t(b) * H + r] = acc;
      }
      if (threadIdx.x == 0)
        __hip_atomic_store(a.tile_count + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }
}

template <int NB>
hipError_t gate_up_nb(const ExpertArgs &a, int grid, hipStream_t s) {
  if (a.hidden > 64 * kChunk)
    hipLaunchKernelGGL((gate_up_kernel<NB, 2>), dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((gate_up_kernel<NB, 1>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int NB>
hipError_t down_nb(const ExpertArgs &a, int grid, int rows_per_tile, hipStream_t s) {
  hipLaunchKernelGGL((down_kernel<NB>), dim3(grid), dim3(kThreads), 0, s, a, rows_per_tile);
  return hipGetLastError();
}

int clamp_grid(long n) { return int(n < 1 ? 1 : (n > 2048 ? 2048 : n)); }

}  // namespace

int down_rows_per_tile(int inter) {
  const int rps = 64 / (inter / kChunk);
  const int rows = 4 * rps;
  return rows < 32 ? 32 : rows;
}

hipError_t launch_gate_up(const ExpertArgs &a, int nb, int max_slots, hipStream_t s) {
  const int grid = clamp_grid(long(max_slots) * (a.inter / kTileRowPairs));
  switch (nb) {
    case 1: return gate_up_nb<1>(a, grid, s);
    case 2: return gate_up_nb<2>(a, grid, s);
    case 3: return gate_up_nb<3>(a, grid, s);
    default: return gate_up_nb<4>(a, grid, s);
  }
}

hipError_t launch_down(const ExpertArgs &a, int nb, int max_slots, hipStream_t s) {
  const int rpt = down_rows_per_tile(a.inter);
  const int grid = clamp_grid(long(max_slots) * (a.hidden / rpt));
  switch (nb) {
    case 1: return down_nb<1>(a, grid, rpt, s);
    case 2: return down_nb<2>(a, grid, rpt, s);
    case 3: return down_nb<3>(a, grid, rpt, s);
    default: return down_nb<4>(a, grid, rpt, s);
  }
}

}  // namespace moe
