// Device-side helpers of the MoE kernels (gfx950): code unpacking and the
// per-chunk dot product, bf16 / (scale, bias) decoding, and the cross-block
// exchange primitives.
//
// Cross-block exchange.  Each XCD of the chip has its own L2, so a block on
// one XCD cannot read another XCD's ordinary stores through its L2.  A
// device-scope fence would write back and invalidate the whole L2 of every
// wave that executes it (tens of microseconds per layer when every wave does
// it), so the kernels never use one.  Instead, data that another block reads
// in the same launch is stored and loaded with device-coherent (sc1) memory
// operations, the writer waits for its stores to complete (s_waitcnt) before
// it bumps a device-coherent atomic counter, and the reader polls that
// counter before loading.  Data read only by later launches uses ordinary
// stores (kernel boundaries order them).
#pragma once

#include "moe_internal.h"

namespace moe {

// ------------------------------------------------------------ decoding
__device__ inline float byte_f(uint32_t v, int k) { return float((v >> (8 * k)) & 0xffu); }
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline float sb_scale(uint32_t w) { return bf16_lo(w); }
__device__ inline float sb_bias(uint32_t w) { return bf16_hi(w); }

__device__ inline bool record_ok(uint64_t desc, uint64_t pool_bytes, int hidden, int inter) {
  const int bits = bits_of_tag(desc);
  if (bits == 0) return false;
  const uint64_t off = desc & ~uint64_t(255);
  const RecordLayout L = record_layout(hidden, inter, bits);
  return off + L.total <= pool_bytes && off + L.total > off;
}

// Codes of one 32-code chunk of a packed row: 4-bit: w[0..3] (16 B);
// 2-bit: w[0..1] (8 B); 3-bit: w[0..1] low plane, w[2] high plane (8 + 4 B).
// Words a width does not use are left as they are (no decoder reads them).
template <int BITS>
__device__ inline void load_chunk(const uint8_t *row, int row_codes, int chunk, uint32_t (&w)[4]) {
  if constexpr (BITS == 4) {
    const uint4 v = *reinterpret_cast<const uint4 *>(row + chunk * 16);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2 *>(row + chunk * 8);
    w[0] = v.x; w[1] = v.y;
  } else {
    const uint2 v = *reinterpret_cast<const uint2 *>(row + chunk * 8);
    w[0] = v.x; w[1] = v.y;
    w[2] = *reinterpret_cast<const uint32_t *>(row + row_codes / 4 + chunk * 4);
  }
}

// P[b] = sum_t q_t * x(b, t) over one chunk's 32 codes, f32 FMAs.  Codes
// are expanded with one AND per four codes and a byte->float conversion per
// code (v_cvt_f32_ubyte); the power-of-two scale of each bit field is undone
// once per chunk.  `X` supplies the operand four values at a time:
// X(b, q) returns x(b, 4q .. 4q+3) as a float4, so the caller decides whether
// they live in registers or in LDS.
template <int BITS, int NB, typename XSrc>
__device__ inline void chunk_dot(const uint32_t (&w)[4], const XSrc &X, float (&P)[NB]) {
  if constexpr (BITS == 4) {
    // word m holds codes 8m..8m+7: low nibbles = even codes, high = odd (x16)
    float lo[NB], hi[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) lo[b] = hi[b] = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t l = w[m] & 0x0f0f0f0fu, h = w[m] & 0xf0f0f0f0u;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 x0 = X(b, 2 * m), x1 = X(b, 2 * m + 1);
        lo[b] = fmaf(byte_f(l, 0), x0.x, lo[b]);
        hi[b] = fmaf(byte_f(h, 0), x0.y, hi[b]);
        lo[b] = fmaf(byte_f(l, 1), x0.z, lo[b]);
        hi[b] = fmaf(byte_f(h, 1), x0.w, hi[b]);
        lo[b] = fmaf(byte_f(l, 2), x1.x, lo[b]);
        hi[b] = fmaf(byte_f(h, 2), x1.y, hi[b]);
        lo[b] = fmaf(byte_f(l, 3), x1.z, lo[b]);
        hi[b] = fmaf(byte_f(h, 3), x1.w, hi[b]);
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) P[b] = fmaf(hi[b], 0.0625f, lo[b]);
  } else {
    // 2-bit field p of byte k of word m holds code 16m+4k+p (x 4^p); 3-bit
    // adds the high bit from byte k, bit 4m+p, of the high-plane word.
    float acc[4][NB];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[p][b] = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float c[4][4];   // [p][k]
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t l = w[m] & (0x03030303u << (2 * p));
        uint32_t h = 0;
        if constexpr (BITS == 3) h = w[2] & (0x01010101u << (4 * m + p));
        // 2^(2+p-4m): scales the high-bit byte value 2^(4m+p) to 4 * 4^p
        const float hs = (m == 0) ? float(4 << p) : float(4 << p) / 16.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          c[p][k] = byte_f(l, k);
          if constexpr (BITS == 3) c[p][k] = fmaf(byte_f(h, k), hs, c[p][k]);
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 xv = X(b, 4 * m + k);     // codes 16m+4k .. 16m+4k+3 (p = 0..3)
          acc[0][b] = fmaf(c[0][k], xv.x, acc[0][b]);
          acc[1][b] = fmaf(c[1][k], xv.y, acc[1][b]);
          acc[2][b] = fmaf(c[2][k], xv.z, acc[2][b]);
          acc[3][b] = fmaf(c[3][k], xv.w, acc[3][b]);
        }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
      P[b] = acc[0][b] + 0.25f * acc[1][b] + 0.0625f * acc[2][b] + 0.015625f * acc[3][b];
  }
}

// chunk_dot for R rows that share the operand: each float4 of x is read once
// and applied to all R rows right away, so no row keeps x in registers.
template <int BITS, int NB, int R, typename XSrc>
__device__ inline void chunk_dot_rows(const uint32_t (&w)[R][4], const XSrc &X, float (&P)[R][NB]) {
  if constexpr (BITS == 4) {
    float lo[R][NB], hi[R][NB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) lo[r][b] = hi[r][b] = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float cl[R][4], ch[R][4];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t l = w[r][m] & 0x0f0f0f0fu, h = w[r][m] & 0xf0f0f0f0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) { cl[r][k] = byte_f(l, k); ch[r][k] = byte_f(h, k); }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4 x0 = X(b, 2 * m), x1 = X(b, 2 * m + 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          lo[r][b] = fmaf(cl[r][0], x0.x, lo[r][b]);
          hi[r][b] = fmaf(ch[r][0], x0.y, hi[r][b]);
          lo[r][b] = fmaf(cl[r][1], x0.z, lo[r][b]);
          hi[r][b] = fmaf(ch[r][1], x0.w, hi[r][b]);
          lo[r][b] = fmaf(cl[r][2], x1.x, lo[r][b]);
          hi[r][b] = fmaf(ch[r][2], x1.y, hi[r][b]);
          lo[r][b] = fmaf(cl[r][3], x1.z, lo[r][b]);
          hi[r][b] = fmaf(ch[r][3], x1.w, hi[r][b]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) P[r][b] = fmaf(hi[r][b], 0.0625f, lo[r][b]);
  } else {
    float acc[R][4][NB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][p][b] = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint32_t lm[R][4], hm[R][4];   // field p of every byte (low plane, high bit)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          lm[r][p] = w[r][m] & (0x03030303u << (2 * p));
          hm[r][p] = BITS == 3 ? w[r][2] & (0x01010101u << (4 * m + p)) : 0u;
        }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float c[R][4];   // [row][p]: codes 16m+4k+p
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            c[r][p] = byte_f(lm[r][p], k);
            if constexpr (BITS == 3) {
              const float hs = (m == 0) ? float(4 << p) : float(4 << p) / 16.0f;
              c[r][p] = fmaf(byte_f(hm[r][p], k), hs, c[r][p]);
            }
          }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float4 xv = X(b, 4 * m + k);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            acc[r][0][b] = fmaf(c[r][0], xv.x, acc[r][0][b]);
            acc[r][1][b] = fmaf(c[r][1], xv.y, acc[r][1][b]);
            acc[r][2][b] = fmaf(c[r][2], xv.z, acc[r][2][b]);
            acc[r][3][b] = fmaf(c[r][3], xv.w, acc[r][3][b]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        P[r][b] = acc[r][0][b] + 0.25f * acc[r][1][b] + 0.0625f * acc[r][2][b] + 0.015625f * acc[r][3][b];
  }
}

// Operand sources for chunk_dot.
template <int NB>
struct RegX {   // x[b][0..31] in registers
  const float (&x)[NB][kChunk];
  __device__ float4 operator()(int b, int q) const {
    return make_float4(x[b][4 * q], x[b][4 * q + 1], x[b][4 * q + 2], x[b][4 * q + 3]);
  }
};
struct LdsX {   // x(b, t) = p[b * stride + t], 16-byte aligned, in LDS
  const float *p;
  int stride;
  __device__ float4 operator()(int b, int q) const {
    return *reinterpret_cast<const float4 *>(p + b * stride + 4 * q);
  }
};

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ------------------------------------------------- wave reductions (DPP)
// Lane permutations inside 16-lane rows run on the DPP path (a few cycles)
// instead of the LDS crossbar (ds_bpermute); rows are combined with
// v_readlane, so the result is uniform across the wave.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each 16

template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ inline double dpp_d(double v) {
  const uint64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp(int(uint32_t(u)), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(int(uint32_t(u >> 32)), CTRL, 0xF, 0xF, true);
  return __longlong_as_double((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo));
}

// Sum over each group of 8 lanes (all lanes of the group get it).
__device__ inline float group8_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v;
}
// Sum over each 16-lane row.
__device__ inline float row16_sum(float v) {
  v = group8_sum(v);
  return v + dpp_f<kDppMirror>(v);
}
// Sum over the wave, uniform result.
__device__ inline float wave_sum(float v) {
  v = row16_sum(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}
__device__ inline double readlane_d(double v, int lane) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(u)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(u >> 32)), lane);
  return __longlong_as_double((uint64_t(hi) << 32) | lo);
}
// Order-preserving u64 key of a finite double (larger double <-> larger key).
__device__ inline uint64_t order_key(double v) {
  const uint64_t b = __double_as_longlong(v);
  return (b >> 63) ? ~b : (b | (uint64_t(1) << 63));
}
// Order-preserving u32 key of a float (larger float <-> larger key).
__device__ inline uint32_t order_key32(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b >> 31) ? ~b : (b | 0x80000000u);
}
template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp(int(uint32_t(v)), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(int(uint32_t(v >> 32)), CTRL, 0xF, 0xF, true);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}
__device__ inline uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane(int(uint32_t(v)), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(int(uint32_t(v >> 32)), lane);
  return (uint64_t(hi) << 32) | lo;
}
// (key, id) pairs ordered by key descending, then id ascending.
__device__ inline bool pair_before(uint64_t ka, int ia, uint64_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}
template <int CTRL>
__device__ inline void argmax_step(uint64_t &k, int &i) {
  const uint64_t ok = dpp_u64<CTRL>(k);
  const int oi = __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, true);
  if (pair_before(ok, oi, k, i)) { k = ok; i = oi; }
}
// Wave-wide best (key, id); the result is uniform.
__device__ inline void wave_argmax(uint64_t &k, int &i) {
  argmax_step<0xB1>(k, i);
  argmax_step<0x4E>(k, i);
  argmax_step<0x141>(k, i);
  argmax_step<0x140>(k, i);
  uint64_t bk = readlane_u64(k, 0);
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const uint64_t ck = readlane_u64(k, r);
    const int ci = __builtin_amdgcn_readlane(i, r);
    if (pair_before(ck, ci, bk, bi)) { bk = ck; bi = ci; }
  }
  k = bk;
  i = bi;
}

__device__ inline double wave_sum_d(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppMirror>(v);
  return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}

// ------------------------------------------------ cross-block exchange
template <typename T>
__device__ inline void st_dev(T *p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ inline T ld_dev(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 4 consecutive floats at byte offset `off` (16-byte aligned) from `base`,
// with one device-coherent load.  `base` must be the same in every lane: the
// buffer descriptor lives in scalar registers, and a per-lane base would make
// the compiler issue the load once per distinct lane value.
__device__ inline float4 ld_dev_f4(const float *base, uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, 0x7fffffff, 0x00020000);
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16));
}

// Two consecutive 64-bit words at byte offset `off` (16-byte aligned) from a
// lane-uniform `base`, with one device-coherent load; each word is read whole.
__device__ inline void ld_dev_u64x2(const uint64_t *base, uint32_t off, uint64_t &w0, uint64_t &w1) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t *>(base), (short)0, 0x7fffffff, 0x00020000);
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
  w0 = uint64_t(v[0]) | (uint64_t(v[1]) << 32);
  w1 = uint64_t(v[2]) | (uint64_t(v[3]) << 32);
}

__device__ inline uint64_t tag_f32(uint32_t epoch, float v) {
  return (uint64_t(epoch) << 32) | __float_as_uint(v);
}

// All of this block's prior stores are complete before thread 0 signals.
__device__ inline void block_signal(uint32_t *counter, uint32_t inc, uint32_t *prev_out = nullptr) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev_out) *prev_out = prev;
  }
}

}  // namespace moe
