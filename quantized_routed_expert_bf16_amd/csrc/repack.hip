// Low-bit store builder (gfx950): 4-bit expert records requantized to 3- or
// 2-bit records.
//
// The engine keeps a 3- or 2-bit copy of every expert, built once from the
// 4-bit source (gpu/load.rs source page, load_bounded: the low-bit store and
// its smaller record stride).  The pages give no requantization rule; the
// one implemented is min/max affine requantization of each 64-code group of
// dequantised weights w = q s + b.  The group's weights span [lo, hi], lo
// and hi at its extreme codes q_lo and q_hi (by the sign of s), and the new
// grid of 2^bits - 1 steps spans the same interval:
//   d = |q_hi - q_lo|,  q' = round_half_up(|q - q_lo| (2^bits - 1) / d),
//   s' = bf16(|s| d / (2^bits - 1)),  b' = bf16(b + s q_lo)
// (q' = 0 and s' = 0 when d = 0).  The codes are exact integer results; the
// scale and bias are float32 operations rounded to nearest even bf16.
//
// One thread takes one 64-code group: 32 bytes of codes and one (scale,
// bias) word in, 16 (2-bit) or 24 (3-bit) bytes and one word out.  A record
// has 3 I H / 64 groups (gate/up rows, then the group-major down section),
// a multiple of 256, so no block straddles two records.  The kernel is
// bound by HBM bandwidth.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRepackThreads = 256;

__device__ inline uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16) & 0xFFFFu;
}

__device__ inline bool desc_ok(uint64_t desc, uint64_t pool_bytes, int hidden, int inter, int want_bits) {
  const int bits = bits_of_tag(desc);
  if (bits != want_bits) return false;
  const uint64_t off = desc & ~uint64_t(255);
  const uint64_t total = record_layout(hidden, inter, bits).total;
  return off + total <= pool_bytes && off + total > off;
}

struct RepackArgs {
  const uint8_t *src;
  uint64_t src_bytes;
  const uint64_t *src_desc;
  uint8_t *dst;
  uint64_t dst_bytes;
  const uint64_t *dst_desc;
  int hidden, inter;
  int groups_per_record;   // 3 I H / 64
  int gu_groups;           // 2 I H / 64
  uint32_t *status;        // may be null
};

__global__ __launch_bounds__(kRepackThreads) void repack_kernel(RepackArgs a) {
  const int per_rec_blocks = a.groups_per_record / kRepackThreads;
  const int r = blockIdx.x / per_rec_blocks;
  const int gi = (blockIdx.x - r * per_rec_blocks) * kRepackThreads + threadIdx.x;
  const uint64_t sd = a.src_desc[r], dd = a.dst_desc[r];
  const int bits = bits_of_tag(dd);
  const int H = a.hidden, I = a.inter;
  if (!desc_ok(sd, a.src_bytes, H, I, 4) || (bits != 3 && bits != 2) ||
      !desc_ok(dd, a.dst_bytes, H, I, bits)) {
    if (threadIdx.x == 0 && gi == 0 && a.status)
      __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const RecordLayout L4 = record_layout(H, I, 4), Lb = record_layout(H, I, bits);
  const uint8_t *src = a.src + (sd & ~uint64_t(255));
  uint8_t *dst = a.dst + (dd & ~uint64_t(255));
  // source and destination of this group's codes and (scale, bias) word
  const uint8_t *cin;
  const uint32_t *sbin;
  uint8_t *cout_lo, *cout_hi;   // low plane (2 bits per code); 3-bit high plane
  uint32_t *sbout;
  if (gi < a.gu_groups) {
    const int gpr = H / kGroup;
    const int row = gi / gpr, grp = gi - row * gpr;
    cin = src + L4.gu_codes + size_t(row) * L4.gu_row_bytes + grp * 32;
    sbin = reinterpret_cast<const uint32_t *>(src + L4.gu_sb) + gi;
    uint8_t *orow = dst + Lb.gu_codes + size_t(row) * Lb.gu_row_bytes;
    cout_lo = orow + grp * 16;
    cout_hi = orow + H / 4 + grp * 8;
    sbout = reinterpret_cast<uint32_t *>(dst + Lb.gu_sb) + gi;
  } else {   // down: group-major, each (group, row) one 64-code row
    const int dg = gi - a.gu_groups;
    cin = src + L4.d_codes + size_t(dg) * 32;
    sbin = reinterpret_cast<const uint32_t *>(src + L4.d_sb) + dg;
    uint8_t *orow = dst + Lb.d_codes + size_t(dg) * (kGroup * bits / 8);
    cout_lo = orow;
    cout_hi = orow + 16;
    sbout = reinterpret_cast<uint32_t *>(dst + Lb.d_sb) + dg;
  }
  const uint4 c0 = reinterpret_cast<const uint4 *>(cin)[0];
  const uint4 c1 = reinterpret_cast<const uint4 *>(cin)[1];
  const uint32_t sbw = *sbin;
  const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  // extreme codes of the group
  int qmin = 15, qmax = 0;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int q = int((w[m] >> (4 * n)) & 15u);
      qmin = min(qmin, q);
      qmax = max(qmax, q);
    }
  const float s = __uint_as_float(sbw << 16), b = __uint_as_float(sbw & 0xFFFF0000u);
  const bool neg = s < 0.0f;
  const int q_lo = neg ? qmax : qmin;
  const int d = qmax - qmin;
  const int levels = (1 << bits) - 1;
  // q' = floor((2 k levels + d) / (2 d)), k = |q - q_lo|: a multiply-shift
  // by ceil(2^16 / (2 d)) is exact for these numerators (<= 225)
  const uint32_t magic = d ? (65536u + uint32_t(2 * d) - 1u) / uint32_t(2 * d) : 0u;
  uint32_t lo[4] = {0, 0, 0, 0}, hi[2] = {0, 0};
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int i = 8 * m + n;   // code index in the group
      const int q = int((w[m] >> (4 * n)) & 15u);
      const uint32_t k = uint32_t(q > q_lo ? q - q_lo : q_lo - q);
      const uint32_t code = d ? ((2u * k * uint32_t(levels) + uint32_t(d)) * magic) >> 16 : 0u;
      lo[i / 16] |= (code & 3u) << (2 * (i % 16));
      if (bits == 3) {
        const int j = i % 32;   // high bit of code j of a 32-code block
        hi[i / 32] |= (code >> 2) << (8 * ((j / 4) % 4) + 4 * (j / 16) + j % 4);
      }
    }
  // scale |s| d / levels (|s| d exact in float32), bias b + s q_lo (s q_lo exact)
  const float step = d ? (fabsf(s) * float(d)) / float(levels) : 0.0f;
  const float bias = b + s * float(q_lo);
  *reinterpret_cast<uint4 *>(cout_lo) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  if (bits == 3) *reinterpret_cast<uint2 *>(cout_hi) = make_uint2(hi[0], hi[1]);
  *sbout = bf16_rne(step) | (bf16_rne(bias) << 16);
}

}  // namespace

hipError_t launch_repack(const uint8_t *src, uint64_t src_bytes, const uint64_t *src_desc, uint8_t *dst,
                         uint64_t dst_bytes, const uint64_t *dst_desc, int n, int hidden, int inter,
                         uint32_t *status, hipStream_t s) {
  RepackArgs a{};
  a.src = src;
  a.src_bytes = src_bytes;
  a.src_desc = src_desc;
  a.dst = dst;
  a.dst_bytes = dst_bytes;
  a.dst_desc = dst_desc;
  a.hidden = hidden;
  a.inter = inter;
  a.gu_groups = 2 * inter * (hidden / kGroup);
  a.groups_per_record = 3 * inter * (hidden / kGroup);
  a.status = status;
  if (a.groups_per_record % kRepackThreads) return hipErrorInvalidValue;
  const uint64_t blocks = uint64_t(n) * (a.groups_per_record / kRepackThreads);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
  hipLaunchKernelGGL(repack_kernel, dim3(unsigned(blocks)), dim3(kRepackThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
