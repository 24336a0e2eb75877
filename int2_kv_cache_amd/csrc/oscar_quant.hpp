// oscar_quant.hpp -- the INT2 min-max quantizer of one 32-value range and the
// assembly of record code words from 16-code image words, shared by the
// cache kernels (append, prefill, stateless pack) and the fused decode step,
// so that every path turns the same fp16 values into the same bytes.
#pragma once
#include "oscar_device.hpp"

namespace oscar {

// INT2 min-max quantizer over 32 fp16-valued numbers: delta = (max - min)/3,
// zero = min, code = clamp(rint((x - zero)/delta), 0, 3) with ties to even,
// delta == 0 -> code 0 ([SUM] 前置知识 on per-channel quantization and
// 方法步骤详情 ②; [RN] §I).
// Range of 32 values: zero = min, delta = (max - min) / 3, both from the
// canonicalised (+0) extremes; 1/delta (0 when delta == 0).
struct Range {
  float zero, delta, rdelta;
  float c0;     // -zero * rdelta, rounded: the fast quotient is x * rdelta + c0
  float near;   // a fast quotient this close to a half integer is recomputed
  uint32_t zm;  // fp16 bits of min | max << 16 (both fp16 values)
};
// From the extremes (fp16 values as fp32): both canonicalised to +0 if
// zero, delta, 1/delta and the fast-quotient constants.  `wide` widens the
// near margin for inputs that are not yet the quantized values (the
// prefill's Value ranges, taken before the rounding to fp16).
__device__ __forceinline__ Range range_of(float mn, float mx, float wide) {
#pragma clang fp contract(off)
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  Range r;
  r.zero = mn;
  r.delta = __fdiv_rn(mx - mn, 3.0f);
  r.rdelta = r.delta > 0.0f ? __fdiv_rn(1.0f, r.delta) : 0.0f;
  r.c0 = -mn * r.rdelta;
  // q1 = fl(x * rdelta + c0) (one fma) against q = fl(fl(x - min) / delta):
  // rdelta and c0 carry relative errors below 2^-24 each, x * rdelta + c0 =
  // (x - min) / delta + e with |e| <= 2^-24 (|q| + |c0|) (1 + 2^-23), q1
  // adds one rounding (|q1| <= 3.5) and q two, so |q1 - q| <= 2^-24 (14 +
  // 1.01 |c0|).  Codes can differ only if a half integer lies within that
  // distance of q1.
  r.near = 0.5f - 0x1p-24f * (16.0f + 1.01f * fabsf(r.c0) + wide * r.rdelta);
  r.zm = static_cast<uint32_t>(f32_to_f16(mn)) | (static_cast<uint32_t>(f32_to_f16(mx)) << 16);
  return r;
}
__device__ __forceinline__ Range range32(const float* x) {
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  return range_of(mn, mx, 0.0f);
}

// The 32 codes of a range's own values, packed two bits each: channel or
// token i at bits 2 (i & 15) of w[i >> 4].  The fast quotient q1 = x *
// (1/delta) - min/delta (one fma) is close enough to the correctly rounded
// quotient of (x - min) by delta (bound at range32) that rint(q1) is the code
// unless q1 lies near a half integer.  Such values (exact ties among fp16
// inputs make them common enough that most waves hold one) are recomputed
// one at a time with the exact quotient: a wave-wide mask per value records
// which lanes need it, so a wave pays only for the values some lane needs.
// Codes accumulate eight at a time as sum c * 4^k in fp32 (exact: below
// 2^16); a recomputed code adds its difference.
// ROW: x holds a Value unit's unrounded inputs and r comes from range32_row;
// a value recomputed exactly is first rounded to its stored fp16 value, and
// a NaN input (it always counts as near) makes the call return false.
// xv(i): value i as fp32.
template <bool ROW = false, class XV>
__device__ __forceinline__ bool codes32_of(XV xv, const Range& r, uint32_t w[2]) {
#pragma clang fp contract(off)
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // near[i]: the lanes whose value i lies near a half integer (a wave-wide
  // mask, so that finding them later costs no vector instructions)
  uint64_t near[32], any = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float c = rintf(__builtin_fmaf(xv(i), r.rdelta, r.c0));
    const float d = fabsf(__builtin_fmaf(xv(i), r.rdelta, r.c0) - c);
    near[i] = __ballot(ROW ? !(d < r.near) : d >= r.near);
    any |= near[i];
    acc[i >> 3] = __builtin_fmaf(c, static_cast<float>(1u << (2 * (i & 7))), acc[i >> 3]);
  }
  bool ok = true;
  if (any) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (near[i]) {  // uniform: some lane needs value i; the wave recomputes it
        const float c = rintf(__builtin_fmaf(xv(i), r.rdelta, r.c0));
        const float xs = ROW ? f16_to_f32(f32_to_f16(xv(i))) : xv(i);
        if (ROW && xv(i) != xv(i)) ok = false;
        const float q = rintf(__fdiv_rn(xs - r.zero, r.delta));
        const float ce = r.delta > 0.0f ? fminf(fmaxf(q, 0.0f), 3.0f) : 0.0f;
        // the correction applies in the lanes of the mask only
        const float corr = __builtin_amdgcn_inverse_ballot_w64(near[i]) ? ce - c : 0.0f;
        acc[i >> 3] = __builtin_fmaf(corr, static_cast<float>(1u << (2 * (i & 7))), acc[i >> 3]);
      }
    }
  }
  w[0] = static_cast<uint32_t>(acc[0]) | (static_cast<uint32_t>(acc[1]) << 16);
  w[1] = static_cast<uint32_t>(acc[2]) | (static_cast<uint32_t>(acc[3]) << 16);
  return ok;
}
template <bool ROW = false>
__device__ __forceinline__ bool codes32(const float* x, const Range& r, uint32_t w[2]) {
  return codes32_of<ROW>([x](int i) { return x[i]; }, r, w);
}

// range32 and codes32 for values read one at a time (xv(i) may load from
// LDS each time): no value array and no per-value masks, a near value is
// corrected on the spot.  The same extremes in the same order, the same
// quotients and the same exact sums of c 4^k, hence the same bits; for rare
// paths inside kernels whose registers are spoken for.
template <class XV>
__device__ __forceinline__ Range range32_stream(XV xv) {
  float mn = xv(0), mx = mn;
#pragma unroll 1
  for (int i = 1; i < 32; ++i) {
    const float x = xv(i);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  return range_of(mn, mx, 0.0f);
}
template <class XV>
__device__ __forceinline__ void codes32_stream(XV xv, const Range& r, uint32_t w[2]) {
#pragma clang fp contract(off)
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll 1
    for (int i = 8 * k; i < 8 * k + 8; ++i) {
      const float x = xv(i);
      const float q1 = __builtin_fmaf(x, r.rdelta, r.c0);
      float c = rintf(q1);
      if (fabsf(q1 - c) >= r.near) {
        const float q = rintf(__fdiv_rn(x - r.zero, r.delta));
        c = r.delta > 0.0f ? fminf(fmaxf(q, 0.0f), 3.0f) : 0.0f;
      }
      acc[k] = __builtin_fmaf(c, static_cast<float>(1u << (2 * (i & 7))), acc[k]);
    }
  }
  w[0] = static_cast<uint32_t>(acc[0]) | (static_cast<uint32_t>(acc[1]) << 16);
  w[1] = static_cast<uint32_t>(acc[2]) | (static_cast<uint32_t>(acc[3]) << 16);
}

// Value image: per (head, group) a row of 32 tokens x 2 words (channels
// 0..15 and 16..31 of the group), padded to 80 words so that the four groups
// a wave reads fall in different banks.
constexpr int kVImgRow = 80;
// Key code word j of token t (channels 16 j .. 16 j + 15) from a head's Key
// image [2][128] (word s of channel c holds tokens 16 s .. 16 s + 15).
__device__ __forceinline__ uint32_t key_word(const uint32_t* img, int t, int j) {
  const uint4* src = reinterpret_cast<const uint4*>(img + (t >> 4) * kD + 16 * j);
  const int sh = 2 * (t & 15);
  uint32_t word = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w4 = src[q];
    const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) word |= ((ww[e] >> sh) & 3u) << (2 * e + 8 * q);
  }
  return word;
}
// Value code word (octet, m, group d): tokens 8 octet .. + 7 at channels
// 32 d + 16 e + m, e = 0, 1, from a head's Value image [4][kVImgRow].
__device__ __forceinline__ uint32_t value_word(const uint32_t* img, int oct, int m, int d) {
  const uint4* src = reinterpret_cast<const uint4*>(img + d * kVImgRow + 16 * oct);
  uint32_t word = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w4 = src[q];  // tokens 8 oct + 2q, + 2q + 1; words e = 0, 1
    const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int kk = 2 * q + (f >> 1), e = f & 1;
      const int sk = (kk & 4) | ((kk & 1) << 1) | ((kk >> 1) & 1);
      word |= ((ww[f] >> (2 * m)) & 3u) << (2 * (8 * e + sk));
    }
  }
  return word;
}

}  // namespace oscar
