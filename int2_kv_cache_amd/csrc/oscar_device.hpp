// oscar_device.hpp -- device helpers of the gfx950 OScaR kernels.
//
// Sources cited by tag:
//   [RN]  reading notes "OScaR: The Occam's Razor for Extreme KV Cache
//         Quantization in LLMs and Beyond" (yingwang.github.io paper-reads)
//   [SUM] structured summary "OScaR：面向大模型及多模态LLM极限KV缓存量化的奥卡姆剃刀"
//         (paper.rainbus.top)
//   [POP] popular-science article on OScaR (animattoys.com), sections 一 to 五
//
// Everything that decides a stored bit (rotation, norm, fp16 rounding, INT2
// codes) is written with contraction off and IEEE-rounded divide and sqrt,
// so it reproduces one fixed sequence of fp32 operations exactly.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

namespace oscar {

constexpr int kD = 128;       // head dim
constexpr int kG = 32;        // Key block (tokens)
constexpr int kR = 128;       // residual window (tokens)
constexpr int kVG = 32;       // Value group (channels)
constexpr int kRec = 3072;    // bytes per (physical block, KV head) record
constexpr int kRecKCodes = 0, kRecVCodes = 1024, kRecKDelta = 2048, kRecKZero = 2304,
              kRecVParam = 2560;

// fp32(1/sqrt(128)); the orthonormal Hadamard matrix has entries +-1/sqrt(d)
// ([RN] §II Step One: Canalized Rotation).
constexpr float kFhtScale = 0x1.6a09e6p-4f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
// fp32 -> fp16 bits of a stored value (a Value row entry, a token norm):
// clamped to the finite fp16 range first, so nothing stored is infinite; the
// max returns its other operand for a NaN, which is therefore stored as
// -65504.  (The pages only say FP16; saturation is this code's reading.)
__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
  return f32_to_f16(fminf(fmaxf(f, -65504.0f), 65504.0f));
}
__device__ __forceinline__ float in_to_f32(uint16_t x, int is_bf16) {
  return is_bf16 ? bf16_to_f32(x) : f16_to_f32(x);
}

// 128-point fast Hadamard transform of one vector spread over a full wave:
// lane l holds x[l] in `a` and x[l + 64] in `b`.  Butterflies with strides
// 1, 2, 4, 8, 16, 32 pair lane l with lane l ^ h; stride 64 pairs the two
// registers of one lane; then one multiply by 1/sqrt(128).  Same strides in
// the same order as the plain butterfly definition, so every fp32 rounding is
// the same: the upper element of each pair gets (lower - upper), the lower
// gets (lower + upper) ([SUM] 前置知识 on FHT; [POP] 二; [RN] §II Step One).
// All 64 lanes must be active.
// x of lane l ^ H (H a power of two below 64) without an LDS round trip:
// quad permutes for 1 and 2, the swizzle unit's xor mode for 4..16, the
// half-wave swap for 32.
template <int H>
__device__ __forceinline__ float lane_xor(float x) {
  const int xi = __builtin_bit_cast(int, x);
  if constexpr (H == 1) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  } else if constexpr (H == 2) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  } else if constexpr (H == 4 || H == 8 || H == 16) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(xi, 0x1F | (H << 10)));
  } else {
    static_assert(H == 32, "lane distance");
    // swaps the upper half of the first copy with the lower half of the
    // second: {lo, lo} and {hi, hi}
    const auto p = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? p[0] : p[1]);
  }
}

// Workgroup barrier that orders LDS accesses only: loads and stores to
// global memory in flight (prefetched inputs, results) stay in flight across
// it, where __syncthreads would wait for every one of them.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void fht128_wave(float& a, float& b) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  auto stage = [&](auto hc) {
    constexpr int h = decltype(hc)::value;
    const float pa = lane_xor<h>(a);
    const float pb = lane_xor<h>(b);
    const bool upper = (lane & h) != 0;
    a = upper ? (pa - a) : (a + pa);
    b = upper ? (pb - b) : (b + pb);
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
  stage(std::integral_constant<int, 16>{});
  stage(std::integral_constant<int, 32>{});
  const float lo = a + b, hi = a - b;
  a = lo * kFhtScale;
  b = hi * kFhtScale;
}

// Sum of squares of the wave's 128 values (layout of fht128_wave) by the
// pairwise tree: level s adds element i + s into element i.  Levels 1..32
// are lane butterflies (each lane of a pair ends with the same, commutative,
// sum), level 64 adds the two registers.  Every lane returns the sum.
__device__ __forceinline__ float wave_tree_sumsq(float a, float b) {
#pragma clang fp contract(off)
  float sa = a * a, sb = b * b;
  auto level = [&](auto sc) {
    constexpr int st = decltype(sc)::value;
    sa = sa + lane_xor<st>(sa);
    sb = sb + lane_xor<st>(sb);
  };
  level(std::integral_constant<int, 1>{});
  level(std::integral_constant<int, 2>{});
  level(std::integral_constant<int, 4>{});
  level(std::integral_constant<int, 8>{});
  level(std::integral_constant<int, 16>{});
  level(std::integral_constant<int, 32>{});
  return sa + sb;
}

// Pairwise tree over up to 16 per-head partial sums (zero-padded to 16; the
// extra levels only add +0, which leaves a sum of squares unchanged).
__device__ __forceinline__ float tree16(const float* part, int n) {
#pragma clang fp contract(off)
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = i < n ? part[i] : 0.0f;
#pragma unroll
  for (int s = 1; s < 16; s <<= 1)
#pragma unroll
    for (int i = 0; i + s < 16; i += 2 * s) v[i] = v[i] + v[i + s];
  return v[0];
}

// fp32 product rounded to fp32 and kept there.  Without the empty asm the
// backend may fuse a following fp16 conversion into one mixed-precision FMA
// that rounds only once, which differs from rounding to fp32 first.
__device__ __forceinline__ float mul_rn(float a, float b) {
  float p = a * b;
  asm volatile("" : "+v"(p));
  return p;
}

// Rotary position embedding of one channel pair (x_i, x_{i+64}) with the
// (cos, sin) of its position: a <- a c - b s, b <- b c + a s, each product
// rounded to fp32 (not fused), then one add -- the oracle's sequence.  RoPE
// sits right before the FHT; it is why that rotation runs online ([POP] 五).
__device__ __forceinline__ void rope_pair(float& a, float& b, float c, float s) {
#pragma clang fp contract(off)
  const float ac = mul_rn(a, c), bs = mul_rn(b, s), bc = mul_rn(b, c), as = mul_rn(a, s);
  a = ac - bs;
  b = bc + as;
}

// Correctly rounded fp32 square root for x >= 0.  v_sqrt_f32 is accurate to
// 1 ulp; the result is then fixed among its neighbours s-, s, s+.  With u the
// spacing of the neighbours, x - s*s+ and x - s-*s are integer multiples of u^2
// (x is a multiple of u^2 since x ~ s^2), so one fused multiply-add gives their
// exact sign: sqrt(x) lies above the midpoint of (s, s+) iff x - s*s+ > 0, and
// below the midpoint of (s-, s) iff x - s-*s <= 0.  Tiny inputs are scaled by
// 2^64 (and the root by 2^-32) to keep the residuals in the normal range.
__device__ __forceinline__ float sqrt_rn(float x) {
  if (!(x > 0.0f)) return x == 0.0f ? x : __builtin_nanf("");
  const bool tiny = x < 0x1p-64f;
  const float xs = tiny ? x * 0x1p64f : x;
  float s = __builtin_amdgcn_sqrtf(xs);
  const float sm = __uint_as_float(__float_as_uint(s) - 1u);
  const float sp = __uint_as_float(__float_as_uint(s) + 1u);
  if (__builtin_fmaf(-sm, s, xs) <= 0.0f)
    s = sm;
  else if (__builtin_fmaf(-s, sp, xs) > 0.0f)
    s = sp;
  return tiny ? s * 0x1p-32f : s;
}

// Omni-Token Scaling factors from a sum of squares: norm = sqrt(ss) and
// r = 1/norm, both correctly rounded fp32; ss == 0 gives r = 0 ([RN] §II
// Step Two; [POP] 三 on 1/sqrt(sum x^2)).
// With hw_rsq, r comes from the hardware reciprocal square root instead
// ([POP] 三: one rsqrt instruction rather than the norm and its reciprocal);
// the norm is the same correctly rounded root.
__device__ __forceinline__ void scale_from_ss(float ss, float& norm, float& r, bool hw_rsq = false) {
  norm = sqrt_rn(ss);
  if (hw_rsq)
    r = ss > 0.0f ? __builtin_amdgcn_rsqf(ss) : 0.0f;
  else
    r = ss > 0.0f ? __fdiv_rn(1.0f, norm) : 0.0f;
}

// Packed record layout (see include/oscar.h).
__device__ __forceinline__ int vcode_bitpos(int t, int c) {   // bit index in V codes
  const int slice = 16 * (t >> 3) + (c & 15), word = c >> 5, e = (c >> 4) & 1, k = t & 7;
  const int sk = (k & 4) | ((k & 1) << 1) | ((k >> 1) & 1);
  return 32 * (4 * slice + word) + 2 * (8 * e + sk);
}

}  // namespace oscar
