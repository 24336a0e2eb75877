// oscar_attn.hip -- split-K decode attention over the INT2 cache and the
// cross-split log-sum-exp reduce: oscar_decode_attn.
//
// [SUM] 方法步骤详情 ③: one kernel dequantizes, undoes the token scaling and
// computes attention; the substrate is split-K FlashDecoding ([SUM] 技术新颖性).
// [RN] End-to-End Flow: the rotated query meets the dequantized, inverse-scaled
// Keys in q.K^T; the dequantized Values are combined with the attention
// weights.  (Tags: oscar_device.hpp.)
//
// Work of one (sequence b, KV head h) is a list of units: the Q/32 quantized
// blocks, then ceil((n-Q)/32) chunks of the fp16 residual window.  Split s of
// S takes units [s*U/S, (s+1)*U/S) and writes a partial (m, l, o) per query
// head: m = running max of the scores in log2 units, l = sum of 2^(s2 - m),
// o = sum of 2^(s2 - m) v.  The reduce merges the S partials.
#include <math.h>

#include "oscar_device.hpp"
#include "oscar_host.hpp"
#include "oscar_quant.hpp"

namespace oscar {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128) score scale

struct AttnArgs {
  const uint8_t* pool;
  const uint16_t* pool_norm;
  const uint16_t* res_k;
  const uint16_t* res_v;
  const uint16_t* res_norm;
  const int32_t* block_table;
  const int32_t* seq_state;
  const void* q;
  int q_mode;  // 0 fp16, 1 bf16, 2 fp32 pre-rotated
  int hkv, hq, max_blocks, nphys, splits;
  int head_norm;  // 1: token norms per (token, KV head): [P][Hkv][32], [B][Hkv][128]
  int32_t* error_flag;
  float2* ws_ml;  // [B][Hq][S] (m, l)
  float* ws_o;    // [B][Hq][S][128]
  // arrival counters of the cross-split merge, one per (sequence, KV head)
  // at counter_slot(pair): zero before a launch, and zero again after it
  // (the merging workgroup resets its own)
  int32_t* counters;
  float* out;     // [B][Hq][128]
  float* lse;     // [B][Hq] or null
  int merge_in_kernel;  // 0: partials only, a separate launch merges them
  // null, or [rope_max_pos][64] (cos, sin): a raw (fp16 / bf16) query is
  // rotated by position n - 1, the step's own token, before its FHT
  const float* rope;
  int rope_max_pos;
  // Decode step (STEP kernels): each sequence's new token, appended by the
  // same launch (it writes the cache buffers above through the same pointers)
  const uint16_t* k_new;  // [B][Hkv][128], bf16 or fp16 (kv_bf16)
  const uint16_t* v_new;
  int kv_bf16;
  int flush_blocks;       // blocks quantized when the window is full: 1 or 4
  int hw_rsq;             // 1: Key scaling factor from the hardware rsqrt
  int32_t* append_sync;   // [B] arrival counters: zero before and after a launch
  // null, or the launch order of the sequences: for rank r, {b, n, Q, 0} of
  // the r-th longest sequence, taken before the launch (sched_kernel)
  const int32_t* sched;
};

// The counter of pair p (= b Hkv + h) in the 65536-int counter region:
// slot 32 (p mod 2048) + p / 2048, a one-to-one map that gives each of the
// first 2048 pairs a 128-byte line of its own.  Adjacent counters would put
// every KV head's arrivals (one device-scope atomic per split) on one line,
// where they serialize.
__device__ __forceinline__ int counter_slot(int pair) { return ((pair & 2047) << 5) | (pair >> 11); }

// A stored fp16 value from fp32, as the append stores Values and norms:
// clamped to +-65504 first, a NaN stored as -65504 (the clamp's result in
// IEEE max/min order).  Integer tests, so that the result does not depend on
// how this file's floating-point options treat NaN.
__device__ __forceinline__ uint16_t f16_sat_bits(float f) {
  if ((__float_as_uint(f) & 0x7fffffffu) > 0x7f800000u) return 0xFBFFu;
  return f32_to_f16(__builtin_amdgcn_fmed3f(f, -65504.0f, 65504.0f));
}

// The (cos, sin) of the decode query's position n - 1 for lane L (channel
// pair L, L + 64), or (1, 0) when no RoPE applies; a position past the
// table flags the call and leaves the query unrotated.
__device__ __forceinline__ float2 query_rope(const AttnArgs& A, int n, int L) {
  if (!A.rope || A.q_mode == 2 || n < 1) return make_float2(1.0f, 0.0f);
  if (n - 1 >= A.rope_max_pos) {
    if (L == 0) atomicOr(A.error_flag, static_cast<int32_t>(OSCAR_FLAG_POSITION));
    return make_float2(1.0f, 0.0f);
  }
  return reinterpret_cast<const float2*>(A.rope)[static_cast<size_t>(n - 1) * 64 + L];
}

// The 32 token norms of block p for KV head h, and window slot 0 of (b, h).
__device__ __forceinline__ const uint16_t* block_norms(const AttnArgs& A, int p, int h) {
  return A.pool_norm + (A.head_norm ? (static_cast<size_t>(p) * A.hkv + h) * 32 : static_cast<size_t>(p) * 32);
}
__device__ __forceinline__ const uint16_t* window_norms(const AttnArgs& A, int b, int h) {
  return A.res_norm + (A.head_norm ? (static_cast<size_t>(b) * A.hkv + h) * kR : static_cast<size_t>(b) * kR);
}

// Rotated query heads of KV head h into qs[GRP][128] (fp32): RoPE at the
// position of the step's own token (n - 1) if enabled, then the FHT.
template <int GRP>
__device__ __forceinline__ void load_rotated_q(const AttnArgs& A, int b, int h, int n, float* qs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const float2 cs = query_rope(A, n, lane);
  for (int i = wave; i < GRP; i += nw) {
    const size_t base = (static_cast<size_t>(b) * A.hq + h * GRP + i) * kD;
    float a, bb;
    if (A.q_mode == 2) {
      a = static_cast<const float*>(A.q)[base + lane];
      bb = static_cast<const float*>(A.q)[base + lane + 64];
    } else {
      const uint16_t* q16 = static_cast<const uint16_t*>(A.q);
      a = in_to_f32(q16[base + lane], A.q_mode);
      bb = in_to_f32(q16[base + lane + 64], A.q_mode);
      rope_pair(a, bb, cs.x, cs.y);
      fht128_wave(a, bb);
    }
    qs[i * kD + lane] = a;
    qs[i * kD + lane + 64] = bb;
  }
}

// ---------------------------------------------------------------- VALU
// grid (S, Hkv, B), 256 threads.  Every dot product on the vector ALUs.
template <int GRP>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs A) {
  constexpr int NO = (GRP * kD + 255) / 256;  // outputs per thread
  __shared__ float qs[GRP * kD];
  __shared__ float alpha[GRP][kD + 1];
  __shared__ float beta[GRP];
  __shared__ uint4 stage[(2 * 32 * kD * 2) / 16];  // record+norms, or ring K and V
  __shared__ float sc[GRP][33];
  __shared__ float resc[GRP];
  __shared__ float mrun[GRP], lrun[GRP];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int n = A.seq_state[2 * b], Q = A.seq_state[2 * b + 1];
  if (!(Q >= 0 && (Q & 31) == 0 && n >= Q && n - Q <= kR && Q / kG <= A.max_blocks)) {
    if (tid == 0 && s == 0) atomicOr(A.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    n = Q = 0;  // attend to nothing
  }
  const int nb = Q / kG, nr = (n - Q + kG - 1) / kG, U = nb + nr;
  const int u0 = static_cast<int>((static_cast<long long>(s) * U) / A.splits);
  const int u1 = static_cast<int>((static_cast<long long>(s + 1) * U) / A.splits);

  load_rotated_q<GRP>(A, b, h, n, qs);
  if (tid < GRP) {
    mrun[tid] = -INFINITY;
    lrun[tid] = 0.0f;
  }
  float o[NO];
#pragma unroll
  for (int k = 0; k < NO; ++k) o[k] = 0.0f;

  const uint32_t* st32 = reinterpret_cast<const uint32_t*>(stage);
  const uint16_t* st16 = reinterpret_cast<const uint16_t*>(stage);

  for (int u = u0; u < u1; ++u) {
    __syncthreads();  // readers of the previous unit are done
    const bool quant = u < nb;
    int t_valid = 32;
    if (quant) {
      int p = A.block_table[static_cast<size_t>(b) * A.max_blocks + u];
      if (p < 0 || p >= A.nphys) {
        if (tid == 0) atomicOr(A.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
        p = 0;  // read a valid record; the result is flagged as garbage
      }
      const uint4* rec = reinterpret_cast<const uint4*>(A.pool + (static_cast<size_t>(p) * A.hkv + h) * kRec);
      if (tid < 192) stage[tid] = rec[tid];
      else if (tid < 196) stage[tid] = reinterpret_cast<const uint4*>(block_norms(A, p, h))[tid - 192];
      __syncthreads();
      const uint16_t* dl = st16 + kRecKDelta / 2;
      const uint16_t* zr = st16 + kRecKZero / 2;
      for (int idx = tid; idx < GRP * kD; idx += 256) {
        const int i = idx >> 7, c = idx & 127;
        alpha[i][c] = qs[i * kD + c] * f16_to_f32(dl[c]);
      }
      for (int i = wave; i < GRP; i += 4) {
        float v = qs[i * kD + lane] * f16_to_f32(zr[lane]) + qs[i * kD + lane + 64] * f16_to_f32(zr[lane + 64]);
#pragma unroll
        for (int o2 = 32; o2 >= 1; o2 >>= 1) v += __shfl_xor(v, o2, 64);
        if (lane == 0) beta[i] = v;
      }
      __syncthreads();
      if (tid < 32 * GRP) {
        const int t = tid / GRP, i = tid % GRP;
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const uint32_t word = st32[8 * t + w];
#pragma unroll
          for (int m = 0; m < 16; ++m) acc += alpha[i][16 * w + m] * static_cast<float>((word >> (2 * m)) & 3u);
        }
        const float nt = f16_to_f32(st16[kRec / 2 + t]);
        sc[i][t] = nt * (acc + beta[i]) * (kInvSqrtD * kLog2e);
      }
    } else {
      // fp16 residual chunk: tokens Q + 32*(u-nb) + t.
      const int tb = Q + kG * (u - nb);
      t_valid = min(32, n - tb);
      const int s0 = tb % kR;
      const size_t bh = static_cast<size_t>(b) * A.hkv + h;
      // K rows: 32 slots x 256 B contiguous; V: 128 channels x 64 B.
      const uint4* kr = reinterpret_cast<const uint4*>(A.res_k + (bh * kR + s0) * kD);
      for (int i = tid; i < 512; i += 256) stage[i] = kr[i];
      for (int i = tid; i < 512; i += 256) {
        const int c = i >> 2, qd = i & 3;
        stage[512 + i] = reinterpret_cast<const uint4*>(A.res_v + (bh * kD + c) * kR + s0)[qd];
      }
      __syncthreads();
      if (tid < 32 * GRP) {
        const int t = tid / GRP, i = tid % GRP;
        float acc = 0.0f;
        for (int c = 0; c < kD; ++c) acc += qs[i * kD + c] * f16_to_f32(st16[t * kD + c]);
        const float nt = f16_to_f32(window_norms(A, b, h)[s0 + (t < t_valid ? t : 0)]);
        sc[i][t] = t < t_valid ? nt * acc * (kInvSqrtD * kLog2e) : -INFINITY;
      }
    }
    __syncthreads();
    // Online softmax per query head (wave i handles head i).
    for (int i = wave; i < GRP; i += 4) {
      const float sv = lane < 32 ? sc[i][lane] : -INFINITY;
      float mb = sv;
#pragma unroll
      for (int o2 = 32; o2 >= 1; o2 >>= 1) mb = fmaxf(mb, __shfl_xor(mb, o2, 64));
      const float mo = mrun[i];
      const float mn = fmaxf(mo, mb);
      const float p = (mn == -INFINITY || sv == -INFINITY) ? 0.0f : exp2f(sv - mn);
      float ps = p;
#pragma unroll
      for (int o2 = 32; o2 >= 1; o2 >>= 1) ps += __shfl_xor(ps, o2, 64);
      const float r = (mo == -INFINITY) ? 0.0f : exp2f(mo - mn);
      if (lane < 32) sc[i][lane] = p;
      if (lane == 0) {
        resc[i] = r;
        lrun[i] = lrun[i] * r + ps;
        mrun[i] = mn;
      }
    }
    __syncthreads();
    // P.V for this thread's outputs.
#pragma unroll
    for (int k = 0; k < NO; ++k) {
      const int idx = tid + 256 * k;
      if (idx < GRP * kD) {
        const int i = idx >> 7, c = idx & 127;
        float acc = o[k] * resc[i];
        if (quant) {
          const int g = c >> 5;
          for (int t = 0; t < 32; ++t) {
            const uint32_t pz = st32[kRecVParam / 4 + 32 * g + t];
            const float dv = f16_to_f32(static_cast<uint16_t>(pz & 0xffffu));
            const float zv = f16_to_f32(static_cast<uint16_t>(pz >> 16));
            const int bit = vcode_bitpos(t, c);
            const float code = static_cast<float>((st32[(kRecVCodes * 8 + bit) >> 5] >> (bit & 31)) & 3u);
            acc += sc[i][t] * (zv + dv * code);
          }
        } else {
          for (int t = 0; t < t_valid; ++t) acc += sc[i][t] * f16_to_f32(st16[32 * kD + c * 32 + t]);
        }
        o[k] = acc;
      }
    }
  }
  __syncthreads();
  const size_t pbase = (static_cast<size_t>(b) * A.hq + h * GRP) * A.splits;
  if (tid < GRP) A.ws_ml[pbase + static_cast<size_t>(tid) * A.splits + s] = make_float2(mrun[tid], lrun[tid]);
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int idx = tid + 256 * k;
    if (idx < GRP * kD) {
      const int i = idx >> 7, c = idx & 127;
      A.ws_o[(pbase + static_cast<size_t>(i) * A.splits + s) * kD + c] = o[k];
    }
  }
}

// ---------------------------------------------------------------- MFMA
// The GQA group's q.K^T and P.V products as v_mfma_f32_16x16x32_f16 tiles
// (gfx950: A 16x32, lane l holds row l%16, K elements 8*(l/16)..+7; B 32x16,
// lane l holds column l%16, K elements 8*(l/16)..+7; C 16x16, lane l holds
// column l%16, rows 4*(l/16)..+3).
//
// Key side, per 32-token block: S^T[token, col] = sum_k A[token, k] B[k, col]
//   A = INT2 codes as exact fp16 0..3: a packed word is split into its even
//       and odd 2-bit fields (one and, one shift+and), and each byte of those
//       converts to two fp16 codes with one fp4->fp16 instruction (the fields
//       are e2m1 values code/2, scaled by 2);
//   B = q'_h * delta in two fp16 parts: column h holds the high part, column
//       h + GRP the low part, so q' * delta enters to ~22 bits.
//   The score's zero-point term q'.z is a per-head scalar added afterwards.
// Value side: o^T[channel, col] += sum_t A[channel, t] B[t, col] with
//   A = V codes (fp16 0..3), B = p * delta_v (hi/lo columns); the zero points
//   add a per-(group, head) scalar Z += sum_t p * z_v.
// One MFMA step covers 8 consecutive channels (Key) or tokens (Value) in the
// slot order s = 0,2,1,3,4,6,5,7 that the even/odd split produces.
// Every per-block operand (B tiles, q'.z, probabilities) is computed once per
// wave, spread over its 64 lanes, and exchanged through the wave's LDS.  The
// next block's global data is loaded while the current one is processed.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

template <int BYTE>
__device__ __forceinline__ uint32_t fp4x2_to_f16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, BYTE));
}
// A operand of half H (positions 8H..8H+7) of a 16-code word, from its even
// (e) and odd (o) 2-bit fields: slot i holds position 8H + s(i).
template <int H>
__device__ __forceinline__ u32x4 code_tile(uint32_t e, uint32_t o) {
  return u32x4{fp4x2_to_f16x2<2 * H>(e), fp4x2_to_f16x2<2 * H>(o),
               fp4x2_to_f16x2<2 * H + 1>(e), fp4x2_to_f16x2<2 * H + 1>(o)};
}
__device__ __forceinline__ uint32_t even_fields(uint32_t w) { return w & 0x33333333u; }
__device__ __forceinline__ uint32_t odd_fields(uint32_t w) { return (w >> 2) & 0x33333333u; }
__device__ __forceinline__ constexpr int slot_pos(int i) {
  return (i & 4) | ((i & 1) << 1) | ((i >> 1) & 1);
}

// Cross-lane moves inside a row of 16 lanes (DPP): quad_perm [1,0,3,2] and
// [2,3,0,1] swap neighbours and pairs, row_half_mirror and row_mirror reverse
// 8 and 16 lanes, row_shl:n reads lane l + n.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  // bound_ctrl: a lane whose source is outside the row reads 0
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
constexpr int dpp_row_shl(int n) { return 0x100 + n; }

// max / sum over aligned groups of N lanes; every lane of a group gets the result
template <int N>
__device__ __forceinline__ float group_max(float v) {
  if (N >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if (N >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if (N >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  if (N >= 32) v = fmaxf(v, __shfl_xor(v, 16, 64));
  if (N >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if (N >= 2) v += dpp<kDppXor1>(v);
  if (N >= 4) v += dpp<kDppXor2>(v);
  if (N >= 8) v += dpp<kDppHalfMirror>(v);
  if (N >= 16) v += dpp<kDppMirror>(v);
  if (N >= 32) v += __shfl_xor(v, 16, 64);
  if (N >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// max / sum over the whole wave, the same value in every lane: rows of 16
// lanes reduce with cross-lane moves, then the four row results are read
// out and combined in row order (no LDS round trip)
__device__ __forceinline__ float row_value(float v, int row) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * row));
}
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  return fmaxf(fmaxf(row_value(v, 0), row_value(v, 1)), fmaxf(row_value(v, 2), row_value(v, 3)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  return ((row_value(v, 0) + row_value(v, 1)) + row_value(v, 2)) + row_value(v, 3);
}

// fp32 -> packed fp16 pair, rounding toward zero (hi/lo splits: the low part
// carries the remainder).
__device__ __forceinline__ uint32_t pk_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ float h_lo(uint32_t x) { return f16_to_f32(static_cast<uint16_t>(x)); }
__device__ __forceinline__ float h_hi(uint32_t x) { return f16_to_f32(static_cast<uint16_t>(x >> 16)); }

// Low parts of a hi/lo split: fp16(w0 - hi.lo) into the low half and
// fp16(w1 - hi.hi) into the high half, each from one fused mixed-precision
// multiply-add (w * 1 - hi, rounded once to fp16).
__device__ __forceinline__ uint32_t lo_pair(float w0, float w1, uint32_t hi) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%3 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %2, 1.0, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(r)
      : "v"(w0), "v"(w1), "v"(hi));
  return r;
}

__device__ __forceinline__ void split8(const float* w, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint32_t h = pk_rtz(w[2 * v], w[2 * v + 1]);
    hi[v] = h;
    lo[v] = lo_pair(w[2 * v], w[2 * v + 1], h);
  }
}

// hi/lo fp16 parts of the 8 products a[i] * b[i] (a fp32, b fp16):
// hi = fp16 of the fp32 product (toward zero), lo = fp16(a*b - hi).
__device__ __forceinline__ void split8_mul(const float* a, const _Float16* b, u32x4& hi,
                                           u32x4& lo) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float w0 = __builtin_fmaf(a[2 * v], static_cast<float>(b[2 * v]), 0.0f);
    const float w1 = __builtin_fmaf(a[2 * v + 1], static_cast<float>(b[2 * v + 1]), 0.0f);
    const uint32_t h = pk_rtz(w0, w1);
    hi[v] = h;
    lo[v] = lo_pair(w0, w1, h);
  }
}
__device__ __forceinline__ _Float16 hbits(uint32_t x, int hi) {
  return __builtin_bit_cast(_Float16, static_cast<uint16_t>(hi ? (x >> 16) : x));
}

// LDS operations of one wave execute in order, so lanes exchanging data
// through LDS only need the compiler to keep the accesses in program order.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// B tiles are stored with their 16-byte rows permuted (XOR swizzle) so that
// both the writers (lanes grouped by unit) and the readers (lane l reads row
// l) touch 8 different 16-byte bank groups in every group of 8 lanes.
__device__ __forceinline__ int bk_row(int x) { return x ^ (4 * ((x >> 4) & 1)); }
__device__ __forceinline__ int bv_row(int x) { return x ^ (2 * ((x >> 4) & 3)); }
// A B tile keeps only its NCOL used columns: row c + NCOL g4 holds column c
// of K step g4, and lane (col, g4) reads row (col % NCOL) + NCOL g4 (lanes of
// the unused columns read a duplicate).  Rows are permuted as above so that
// the writers' and readers' 16-byte accesses fall in distinct bank groups.
// With 8 used columns (4 query heads per KV head) the Key tiles' writers
// (units: heads, then channel groups) and the Value tiles' writers (units:
// token octets, then heads) both reach distinct 16-byte bank groups in every
// group of 8 lanes and of 16 lanes, and so do the readers, when bit 3 of the
// row flips bit 2 and bit 4 flips bits 1 and 2.
__device__ __forceinline__ int b8_row(int x) { return x ^ (4 * ((x >> 3) & 1)) ^ (6 * ((x >> 4) & 1)); }
template <int NCOL>
__device__ __forceinline__ int brow_k(int x) { return NCOL == 8 ? b8_row(x) : bk_row(x); }
template <int NCOL>
__device__ __forceinline__ int brow_v(int x) { return NCOL == 16 ? bv_row(x) : NCOL == 8 ? b8_row(x) : bk_row(x); }
constexpr int kRowPad = 36;  // score / probability rows: 32 floats + 4 of padding

// Global data one lane needs for one INT2 block.
// Unit assignments of one block's per-lane work (c = L + 64 r):
//   alpha unit c: head c % GRP, channel group (c / GRP) & 3, step c / (4 GRP);
//   W unit c:     token octet c & 3, head (c >> 2) % GRP, Value group
//                 c / (4 GRP);
//   softmax lane L: head L / LPH, tokens TPL * (L % LPH) .. +TPL-1, and the
//                 zero-point channels CPL * (L % LPH) .. +CPL-1 of q'.z.
template <int NR, int CPL>
struct UnitRegs {
  u32x2 kc[2];   // Key codes of tokens col, 16 + col: channels 32 g4 .. +31
  u32x4 vc;      // Value codes: slice L
  u32x4 dz[NR];  // delta of the alpha unit's 8 channels
  u32x4 vp[NR][2];  // (delta_v, z_v) of the W unit's 8 tokens
  u32x4 zz[(CPL + 7) / 8];  // zero points of the softmax lane's channels
  u32x2 nrm;     // token norms of the softmax lane
};

// Byte offsets of a lane's loads inside a record (and its norm row), fixed
// for the whole kernel: the record base is a wave-uniform (scalar) address.
template <int NR>
struct UnitOffs {
  uint32_t kc0, kc1, vc, dz[NR], vp[NR], zz, nrm;
};

// Buffer resource over one record (or one norm row): loads then take the
// scalar base and a 32-bit per-lane offset, with no per-load address math;
// an offset past num_bytes reads zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, num_bytes, 0x00020000);
}

// One LDS stage of the record pipeline: the record's 3072 bytes, then its
// norm row (64 bytes; the DMA writes 256, lanes past the row reading zero).
constexpr int kStage = kRec + 256;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct HBM -> LDS copy of one record and its norm row into a stage: lane l
// moves bytes 16 l .. 16 l + 15 of each kilobyte (no registers involved).
// Written as inline assembly so that the compiler does not track these LDS
// writes (its tracking waits for every copy in flight before any LDS access
// it cannot prove disjoint); the stage readers wait with vmcnt_le4 instead.
// M0 holds the stage's LDS address.  The copies are non-temporal (nt): each
// record is read once per call, and streaming it through the caches as
// normal lines would evict what the call does reuse (its partials, the state,
// the block table, its own code) -- measured 1.2 to 1.5 us less per call at
// batch 1.
// The Key codes (the record's first 1024 bytes: token t's 32 bytes are
// 16-byte chunks 2t and 2t + 1) are copied with chunk p at chunk p ^ bit 4
// of p, one of the copy's free lane-to-chunk choices: the 16 lanes that read
// 8 bytes of 16 different tokens' chunks then reach 16 different bank pairs.
// The map is its own inverse.
// (Used with 4 query heads per KV head, whose readers it was chosen for.)
__device__ __forceinline__ uint32_t kc_chunk(uint32_t p) { return p ^ ((p >> 4) & 1u); }
template <bool KC_SWZ>
__device__ __forceinline__ void dma_unit(__amdgpu_buffer_rsrc_t rec, __amdgpu_buffer_rsrc_t nrm,
                                         const uint8_t* st, int L) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)st));
  const uint32_t v0 = 16 * (KC_SWZ ? kc_chunk(L) : L), v1 = 16 * L + 1024, v2 = 16 * L + 2048, vn = 4 * L;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %5, 0 offen nt lds\n\t"
      "s_add_u32 m0, %0, 0x400\n\t"
      "buffer_load_dwordx4 %2, %5, 0 offen nt lds\n\t"
      "s_add_u32 m0, %0, 0x800\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen nt lds\n\t"
      "s_add_u32 m0, %0, 0xc00\n\t"
      "buffer_load_dword %4, %6, 0 offen nt lds"
      :
      : "s"(base), "v"(v0), "v"(v1), "v"(v2), "v"(vn), "s"(rec), "s"(nrm)
      : "memory", "m0", "scc");
}
// Wait until at most the 4 newest vector-memory loads are in flight: the
// copy of the next block (4 instructions) may still run, every older one
// (the block about to be read) has landed in LDS.
__device__ __forceinline__ void vmcnt_le4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }
__device__ __forceinline__ void vmcnt_0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The lane's operands of one block, from a stage.
template <class T>
__device__ __forceinline__ T lds_ld(const uint8_t* st, uint32_t off) {
  return *reinterpret_cast<const T*>(st + off);
}
// Key part (codes, steps, zero points, norms) and Value part (codes,
// steps and zero points) of a block: the Key part is dead once the block's
// softmax is done, the Value part once its P.V is issued, so the next block
// is read into the same registers in two halves.
template <int GRP, int NR, int TPL, int CPL>
__device__ __forceinline__ void read_kpart(UnitRegs<NR, CPL>& R, const UnitOffs<NR>& O,
                                           const uint8_t* st, int L) {
  constexpr int NCOMBO = 16 * GRP;
  R.kc[0] = lds_ld<u32x2>(st, O.kc0);
  R.kc[1] = lds_ld<u32x2>(st, O.kc1);
#pragma unroll
  for (int r = 0; r < NR; ++r)
    if (L + 64 * r < NCOMBO) R.dz[r] = lds_ld<u32x4>(st, O.dz[r]);
  if (CPL >= 8) {
#pragma unroll
    for (int j = 0; j < (CPL + 7) / 8; ++j) R.zz[j] = lds_ld<u32x4>(st, O.zz + 16 * j);
  } else {
    const u32x2 z2 = lds_ld<u32x2>(st, O.zz);
    R.zz[0] = u32x4{z2[0], z2[1], 0u, 0u};
  }
  if (TPL == 4)
    R.nrm = lds_ld<u32x2>(st, kRec + O.nrm);
  else if (TPL == 2)
    R.nrm[0] = lds_ld<uint32_t>(st, kRec + O.nrm);
  else
    R.nrm[0] = lds_ld<uint16_t>(st, kRec + O.nrm);
}
template <int GRP, int NR, int TPL, int CPL>
__device__ __forceinline__ void read_vpart(UnitRegs<NR, CPL>& R, const UnitOffs<NR>& O,
                                           const uint8_t* st, int L) {
  constexpr int NCOMBO = 16 * GRP;
  R.vc = lds_ld<u32x4>(st, O.vc);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (L + 64 * r < NCOMBO) {
      R.vp[r][0] = lds_ld<u32x4>(st, O.vp[r]);
      R.vp[r][1] = lds_ld<u32x4>(st, O.vp[r] + 16);
    }
  }
}

// Wait for the wave's outstanding LDS operations (lgkmcnt(0) on gfx9).
__device__ __forceinline__ void lds_wait() { __builtin_amdgcn_s_waitcnt(0xc07f); }

constexpr int kRingWeight = 3;

// Wave priority from its progress through a list of cnt blocks: a wave that
// is behind the others of its SIMD gets the issue slots first, so that the
// waves of a SIMD (which all hold about the same number of blocks) finish
// together instead of the oldest wave running ahead.
__device__ __forceinline__ void progress_prio(int k, int cnt) {
  const int k4 = 4 * k;
  if (k4 < cnt)
    __builtin_amdgcn_s_setprio(3);
  else if (k4 < 2 * cnt)
    __builtin_amdgcn_s_setprio(2);
  else if (k4 < 3 * cnt)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Agent-scope (whole device) relaxed atomic stores and loads of fp32: they
// go to the device's coherence point (global_store / global_load with sc1),
// so a workgroup on another XCD, whose L2 is a different cache, reads what
// they wrote without any cache write-back or invalidation.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroups of NW waves (NW = 12: one workgroup fills a CU with three waves
// per SIMD; NW = 4 or 6: three or two workgroups share a CU).  The grid is
// one-dimensional, B * Hkv * S workgroups, workgroup (b * Hkv + h) * S + s.
// The dispatcher deals consecutive workgroup ids round-robin to the eight
// XCDs, so consecutive splits of one (sequence, KV head) land on different
// XCDs and every XCD gets an even share of every sequence, ragged or not.
//
// PUB selects how a split's partial is published to the merging workgroup:
// 0 = ordinary stores with an agent-scope release (the arrival counter's
// read-modify-write) and acquire (a fence in the merging workgroup); 1 =
// agent-scope atomic stores and loads (coherent at the device level by
// themselves), each wave waiting for its stores to complete before the
// workgroup counts itself in.
template <int GRP, int NW, int PUB, int STEP>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3, 8)))
void attn_mfma_kernel(AttnArgs A) {
  static_assert(GRP == 1 || GRP == 2 || GRP == 4 || GRP == 8, "group size");
  static_assert(NW == 4 || NW == 6 || NW == 12, "waves per workgroup");
  constexpr int NT = 64 * NW;
  constexpr int NCOL = 2 * GRP;                 // used B columns (hi + lo)
  constexpr int TPL = GRP >= 2 ? GRP / 2 : 1;   // softmax tokens per lane
  constexpr int LPH = 32 / TPL;                 // softmax lanes per head
  constexpr int NCOMBO = 16 * GRP;              // alpha / W units per block
  constexpr int NR = (NCOMBO + 63) / 64;        // units per lane
  constexpr int CPL = kD / LPH;                 // q'.z channels per softmax lane
  constexpr float kScale = kInvSqrtD * kLog2e;
  // LDS, one array per use: the compiler tells distinct arrays apart from
  // the stages' DMA writes and waits for those only where a stage is read.
  __shared__ float qs[GRP * kD];                         // rotated query heads
  // per wave: one tile region, used in turn by a block's Key-side B tiles,
  // its combined scores and probabilities, and its Value-side B tiles (each
  // user's last reads precede the next user's writes in the wave's program
  // order, and a wave's LDS operations complete in order)
  constexpr int kTileBytes = 4 * 8 * GRP * 16;
  static_assert((NCOL + GRP) * kRowPad * 4 <= kTileBytes, "scores and probabilities fit a tile");
  __shared__ __attribute__((aligned(16))) uint8_t lds_tile[NW][kTileBytes];
  __shared__ float lds_fac[NW][GRP];                     // per wave: rescale factors
  __shared__ float lds_zs[NW][4][GRP];                   // per wave: Value zero-point sums
  __shared__ float lds_ml[2][NW][GRP];                   // per wave: final (m, l)
  // the two stages of each wave's record pipeline; after the loop they hold
  // the waves' partial outputs for the merge
  __shared__ __attribute__((aligned(16))) uint8_t stage0[NW][kStage];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[NW][kStage];
  __shared__ int lds_last;
  // decode step: the new token's per-head sums of squares, its rotated Key
  // row and stored Value row for this head; whether this workgroup appends
  __shared__ float step_part[STEP ? 16 : 1];
  __shared__ float step_y[STEP ? kD : 1];
  __shared__ uint16_t step_v[STEP ? kD : 2];
  __shared__ int lds_app;

  // The arguments (216 bytes: four 64-byte lines of the scalar cache) are
  // requested in one batch before anything else: the pointers of the first
  // loads (read here, before the state's load: read after it, the wait for
  // them would also wait for the state), the split and head counts, and one
  // field of every line besides, so that the set-up's later argument reads
  // hit the scalar cache instead of each waiting for a line of its own.
  const uint16_t* kn_arg = A.k_new;
  const uint16_t* vn_arg = A.v_new;
  const int32_t* st_arg = A.seq_state;
  const int32_t* sc_arg = A.sched;
  if constexpr (STEP != 0)
    asm volatile("" : "+s"(kn_arg), "+s"(vn_arg), "+s"(st_arg), "+s"(sc_arg)
                 : "s"(A.pool), "s"(A.splits), "s"(A.hkv), "s"(A.out));
  else
    asm volatile("" : "+s"(st_arg), "+s"(sc_arg) : "s"(A.pool), "s"(A.splits), "s"(A.hkv), "s"(A.out),
                 "s"(A.k_new));
  // workgroup (r Hkv + h) S + s: split s of KV head h of the sequence of
  // launch rank r (the sequence itself with no schedule)
  const int wid = static_cast<int>(blockIdx.x);
  const int rh = wid / A.splits, s = wid - rh * A.splits;
  const int rank = rh / A.hkv, h = rh - rank * A.hkv;
  // wave index as a wave-uniform (scalar) value: unit indices and record
  // addresses then stay in scalar registers
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), L = tid & 63;
  typedef u32x4 BTiles[4][8 * GRP];   // [K step][row]
  typedef float Rows[GRP][kRowPad];
  typedef float ScoreRows[NCOL][kRowPad];  // row h: hi part of head h, row h + GRP: lo part
  BTiles& Wbk = *reinterpret_cast<BTiles*>(lds_tile[wave]);
  BTiles& Wbv = *reinterpret_cast<BTiles*>(lds_tile[wave]);
  ScoreRows& Wsc = *reinterpret_cast<ScoreRows*>(lds_tile[wave]);
  Rows& Wpr = *reinterpret_cast<Rows*>(lds_tile[wave] + NCOL * kRowPad * 4);
  float (&Wfac)[GRP] = lds_fac[wave];
  float (&Wzs)[4][GRP] = lds_zs[wave];
  // set-up (loads, query rotation, the window chunk) runs at the highest
  // priority: the main loop lowers it as a wave progresses
  __builtin_amdgcn_s_setprio(3);
  // Decode step: the new token's Keys for the heads this wave rotates (wave,
  // wave + NW, ..) and this head's Value row (threads 0..127), requested
  // with the state in every workgroup (the one that appends is known only
  // from the state), so that their latency hides behind the state's
  constexpr int HPW = (16 + NW - 1) / NW;  // heads per wave (Hkv <= 16)
  uint16_t knx[HPW], kny[HPW];
  uint16_t vnew = 0;
#pragma unroll
  for (int j = 0; j < HPW; ++j) knx[j] = kny[j] = 0;
  typedef __attribute__((address_space(1))) const uint16_t* glb_u16_t;  // global loads
  const glb_u16_t kn_ptr = (glb_u16_t)(kn_arg), vn_ptr = (glb_u16_t)(vn_arg);
  auto issue_new = [&](int bb) {
    if constexpr (STEP != 0) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int hh = wave + NW * j;
        if (hh < A.hkv) {
          const size_t base = (static_cast<size_t>(bb) * A.hkv + hh) * kD;
          knx[j] = kn_ptr[base + L];
          kny[j] = kn_ptr[base + L + 64];
        }
      }
      if (tid < kD) vnew = vn_ptr[(static_cast<size_t>(bb) * A.hkv + h) * kD + tid];
    }
  };
  // {n, Q} by a scalar load (the index is uniform): with a schedule, the
  // sequence and its state as they were before the launch; else the state,
  // which nothing in the launch writes before every workgroup of the
  // sequence has read it.  The vector loads issued next do not wait
  // behind it (without a schedule: with a schedule they need b).
  typedef __attribute__((address_space(4))) const int32_t* cst_i32_t;
  int b, n, Q;
  if (sc_arg) {
    const cst_i32_t sc = (cst_i32_t)(sc_arg) + 4 * rank;
    b = sc[0];
    n = sc[1];
    Q = sc[2];
    issue_new(b);
  } else {
    const cst_i32_t st_cst = (cst_i32_t)(st_arg);
    b = rank;
    n = st_cst[2 * b];
    Q = st_cst[2 * b + 1];
    issue_new(b);
  }
  const int pair = b * A.hkv + h;
  const size_t bh = static_cast<size_t>(b) * A.hkv + h;
  auto load_new = [&](int hh, uint16_t& kx, uint16_t& ky) {
    const size_t base = (static_cast<size_t>(b) * A.hkv + hh) * kD;
    kx = A.k_new[base + L];
    ky = A.k_new[base + L + 64];
  };
  const bool state_good = Q >= 0 && (Q & 31) == 0 && n >= Q && n - Q <= kR && Q / kG <= A.max_blocks;
  if (!state_good) {
    if (tid == 0 && s == 0) atomicOr(A.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    n = Q = 0;
  }
  // Decode step: the append's own checks, the same in every workgroup of the
  // sequence.  When the append goes ahead, attention covers the state it
  // leaves -- n + 1 tokens, with the block(s) a full window flushes quantized
  // by this launch -- so the step equals an append followed by attention.
  const int n_old = n, Q_old = Q;
  bool app = false;
  if constexpr (STEP != 0) {
    if (state_good) {
      app = true;
      int32_t why = 0;
      if (A.rope && n >= A.rope_max_pos) {
        app = false;  // no (cos, sin) for position n
        why = OSCAR_FLAG_POSITION;
      } else if (n - Q == kR) {
        const int j0 = Q / kG;
        if (j0 + A.flush_blocks > A.max_blocks) {
          app = false;
          why = OSCAR_FLAG_CAPACITY;
        } else {
          for (int i = 0; i < A.flush_blocks; ++i) {
            const int pi = A.block_table[static_cast<size_t>(b) * A.max_blocks + j0 + i];
            if (pi < 0 || pi >= A.nphys) {
              app = false;
              why = OSCAR_FLAG_BADSTATE;
            }
          }
        }
      }
      if (!app && tid == 0 && s == 0 && h == 0) atomicOr(A.error_flag, why);
    }
    if (app) {
      if (n - Q == kR) Q += kG * A.flush_blocks;
      n += 1;
    }
    // the same in every lane: kept in scalar registers, so that the unit
    // bounds derived from them (and the main loop's branches) stay uniform
    n = __builtin_amdgcn_readfirstlane(n);
    Q = __builtin_amdgcn_readfirstlane(Q);
  }
  // Splits partition the units by weight: an INT2 block weighs 1, a window
  // chunk (16 KB of fp16 data against a 3 KB record) kRingWeight.
  const int nb = Q / kG, nr = (n - Q + kG - 1) / kG;
  const unsigned wt = nb + kRingWeight * nr, S_u = A.splits;
  auto unit_at = [&](unsigned w) {
    return w <= static_cast<unsigned>(nb) ? static_cast<int>(w)
                                          : nb + static_cast<int>((w - nb + kRingWeight - 1) / kRingWeight);
  };
  // floor(s wt / S) in 32-bit arithmetic: with wt = qw S + rw it is
  // s qw + floor(s rw / S), and s rw < S^2 <= 2^20
  const unsigned qw = wt / S_u, rw = wt - qw * S_u;
  const int u0 = unit_at(s * qw + s * rw / S_u), u1 = unit_at((s + 1) * qw + (s + 1) * rw / S_u);
  const int col = L & 15, g4 = L >> 4;
  const int sm_head = L / LPH, sm_t0 = TPL * (L % LPH), sm_c0 = CPL * (L % LPH);
  const bool sm_on = sm_head < GRP;
  const int krow = brow_k<NCOL>((col % NCOL) + NCOL * g4), vrow = brow_v<NCOL>((col % NCOL) + NCOL * g4);

  // The wave's units are u = first + NW k.  The first cnt are INT2 blocks;
  // at most one more (k = cnt) is a chunk of the fp16 window, since the
  // window spans at most 4 consecutive units and NW >= 4.
  const int first = u0 + wave;
  const int n_units = u1 > first ? (u1 - first + NW - 1) / NW : 0;
  const int cnt = nb > first ? min(n_units, (nb - first + NW - 1) / NW) : 0;
  const bool has_ring = n_units > cnt;
  // Decode step: this split's share of the blocks the append flushes
  // (units f0 .. f1 - 1, quantized here from the window before any record
  // copy), and whether its window chunk holds the new token (unit_new).
  const int f0 = app ? max(u0, Q_old / kG) : 0, f1 = app ? min(u1, nb) : 0;
  const bool wg_fresh = STEP != 0 && f1 > f0;
  const int unit_new = nb + (n_old - Q) / kG;
  const bool wg_new = STEP != 0 && app && unit_new >= u0 && unit_new < u1;
  const bool wave_new = wg_new && has_ring && first + NW * cnt == unit_new;

  // Physical block ids of the wave's INT2 blocks, 64 at a time: lane j holds
  // block k0 + j; a block is then taken out with readlane (no scalar memory
  // traffic inside the loop).  Invalid ids are flagged and replaced by 0.
  const int* tab = A.block_table + static_cast<size_t>(b) * A.max_blocks + first;
  auto load_ids = [&](int k0) {
    int id = 0;
    if (L < cnt - k0) id = tab[NW * (k0 + L)];
    const bool bad = static_cast<unsigned>(id) >= static_cast<unsigned>(A.nphys);
    if (__any(bad) && L == 0) atomicOr(A.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    return bad ? 0 : id;
  };
  // The query heads of this wave (wave, wave + NW) load first: their latency
  // overlaps the block-table read and the first record's.  They stay raw
  // bits (fp32, or the 16-bit value) until the record copies are issued: a
  // conversion here would wait for them before the block ids are requested.
  constexpr int QPW = (GRP + NW - 1) / NW;
  uint32_t qbx[QPW], qby[QPW];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int i = wave + NW * j;
    qbx[j] = qby[j] = 0u;
    if (i < GRP) {
      const size_t base = (static_cast<size_t>(b) * A.hq + h * GRP + i) * kD;
      if (A.q_mode == 2) {
        qbx[j] = static_cast<const uint32_t*>(A.q)[base + L];
        qby[j] = static_cast<const uint32_t*>(A.q)[base + L + 64];
      } else {
        const uint16_t* q16 = static_cast<const uint16_t*>(A.q);
        qbx[j] = q16[base + L];
        qby[j] = q16[base + L + 64];
      }
    }
  }
  // and their RoPE (cos, sin) at the step's own position, n - 1.  The load is
  // made in every case, from the state's first word when no RoPE applies:
  // with a branch around it, the path that sets (1, 0) instead would write
  // its registers while the load may still be in flight, and must first
  // wait for every earlier load.  A position past the table flags the call
  // and leaves the query unrotated.
  const bool q_rope = A.rope && A.q_mode != 2 && n >= 1;
  if (q_rope && n - 1 >= A.rope_max_pos && wave == 0 && L == 0)
    atomicOr(A.error_flag, static_cast<int32_t>(OSCAR_FLAG_POSITION));
  const bool q_rope_on = q_rope && n - 1 < A.rope_max_pos;
  const float2 qcs_ld = *(q_rope_on ? reinterpret_cast<const float2*>(A.rope) + static_cast<size_t>(n - 1) * 64 + L
                                    : reinterpret_cast<const float2*>(A.seq_state));

  UnitOffs<NR> off;
  constexpr bool kKcSwz = GRP == 4;  // Key codes copied with their chunks permuted
  if constexpr (kKcSwz) {
    off.kc0 = kRecKCodes + 16 * kc_chunk(2 * col + (g4 >> 1)) + 8 * (g4 & 1);
    off.kc1 = off.kc0 + 512;  // tokens 16 + col: the chunk map commutes with adding 32 chunks
  } else {
    off.kc0 = kRecKCodes + 32 * col + 8 * g4;
    off.kc1 = kRecKCodes + 32 * (16 + col) + 8 * g4;
  }
  off.vc = kRecVCodes + 16 * L;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int c = L + 64 * r;
    off.dz[r] = kRecKDelta + 2 * (32 * ((c / GRP) & 3) + 8 * ((c / (4 * GRP)) & 3));
    off.vp[r] = kRecVParam + 4 * (32 * ((c / (4 * GRP)) & 3) + 8 * (c & 3));
  }
  off.zz = kRecKZero + 2 * sm_c0;
  off.nrm = 2 * (sm_t0 & 31);
  auto unit_rec = [&](int p) {
    return rsrc(A.pool + (static_cast<size_t>(p) * A.hkv + h) * kRec, kRec);
  };
  auto unit_nrm = [&](int p) { return rsrc(block_norms(A, p, h), 64); };

  // The wave's chunk of the fp16 window (if any) is its first unit: its
  // loads go out before the records' copies, so that waiting for them does
  // not wait for the copies (vector loads complete in order).
  const int ring_tb = Q + kG * (first + NW * cnt - nb);
  const int ring_valid = has_ring ? min(32, n - ring_tb) : 0;
  u32x4 rk[2][4], rv[8];
  // the softmax lane's token norms of the chunk (tokens sm_t0 .. sm_t0 + TPL
  // - 1, consecutive and 4-byte aligned when TPL > 1), fp16 bits kept in
  // whole words until they are used
  constexpr int RNW = (TPL + 1) / 2;
  uint32_t rnw[RNW];
  auto load_ring = [&]() {
    const int slot0 = ring_tb % kR;  // a multiple of 32: the chunk is 32 consecutive slots
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        rk[tau][kk] = *reinterpret_cast<const u32x4*>(
            A.res_k + (bh * kR + slot0 + 16 * tau + col) * kD + 32 * g4 + 8 * kk);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      rv[ct] = *reinterpret_cast<const u32x4*>(A.res_v + (bh * kD + 16 * ct + col) * kR + slot0 + 8 * g4);
    const uint16_t* wn = window_norms(A, b, h) + slot0 + sm_t0;
    if constexpr (TPL == 1) {
      rnw[0] = wn[0];
    } else {
#pragma unroll
      for (int i = 0; i < RNW; ++i) rnw[i] = reinterpret_cast<const uint32_t*>(wn)[i];
    }
  };
  // (a workgroup that quantizes a flushed block first loads its window
  // chunks after that, so that their registers are free meanwhile)
  if (has_ring && !wg_fresh) load_ring();
  // the block ids, requested after every load that does not depend on them
  int idv = cnt > 0 ? load_ids(0) : 0;

  // Block j of the wave goes through stage j % 2.  Its DMA is issued two
  // blocks ahead (unconditionally: past the end it re-reads the last block)
  // so that two records are in flight while one is processed.
  uint8_t* st0 = stage0[wave];
  uint8_t* st1 = stage1[wave];
  auto dma_block = [&](int j, uint8_t* st) {
    if (j > 0 && (j & 63) == 0) idv = load_ids(j);
    const int p = __builtin_amdgcn_readlane(idv, j & 63);
    dma_unit<kKcSwz>(unit_rec(p), unit_nrm(p), st, L);
  };
  // Block 0's copy goes out now, block 1's after the query rotation (below):
  // every wave's first record then lands ahead of the second ones, instead of
  // the two fills sharing the bandwidth, and the loop starts sooner.
  if (!wg_fresh && cnt > 0) dma_block(0, st0);
  if constexpr (STEP != 0) {
    if (wg_fresh) {
      // The flushed block(s) of this split: head h's 32 window tokens of
      // each, quantized to the bytes the append writes (the streaming form
      // of its range and code functions), written to the pool, and then
      // copied like any record.  The
      // stages are free until the copies start: Key rows [32][128] and the
      // Key image in stage0, Value columns [128][32] and the Value image in
      // stage1.
      uint16_t* fk = reinterpret_cast<uint16_t*>(&stage0[0][0]);
      uint32_t* fimg_k = reinterpret_cast<uint32_t*>(&stage0[0][0] + 32 * kD * 2);
      uint16_t* fv = reinterpret_cast<uint16_t*>(&stage1[0][0]);
      uint32_t* fimg_v = reinterpret_cast<uint32_t*>(&stage1[0][0] + 32 * kD * 2);
      static_assert(32 * kD * 2 + 2 * kD * 4 <= 4 * kStage && 32 * kD * 2 + 4 * kVImgRow * 4 <= 4 * kStage,
                    "the flush staging fits the stages");
      for (int fu = f0; fu < f1; ++fu) {
        const int s0 = (Q_old + kG * (fu - Q_old / kG)) % kR;
        const int p = A.block_table[static_cast<size_t>(b) * A.max_blocks + fu];
        uint8_t* rec = const_cast<uint8_t*>(A.pool) + (static_cast<size_t>(p) * A.hkv + h) * kRec;
        for (int i = tid; i < 32 * kD / 8; i += NT) {
          reinterpret_cast<uint4*>(fk)[i] =
              reinterpret_cast<const uint4*>(A.res_k + (bh * kR + s0) * kD)[i];
          reinterpret_cast<uint4*>(fv)[i] = reinterpret_cast<const uint4*>(
              A.res_v + (bh * kD + (i >> 2)) * kR + s0)[i & 3];
        }
        // TOKEN scope: every head writes the same 32 norms
        if (tid < 32) {
          const uint16_t nv = window_norms(A, b, h)[s0 + tid];
          const_cast<uint16_t*>(A.pool_norm)[A.head_norm ? (static_cast<size_t>(p) * A.hkv + h) * 32 + tid
                                    : static_cast<size_t>(p) * 32 + tid] = nv;
        }
        __syncthreads();
        uint32_t cw[2];
        if (tid < kD) {
          // Key channel tid over the block's 32 window tokens
          auto xk = [&](int t) { return f16_to_f32(fk[t * kD + tid]); };
          const Range r = range32_stream(xk);
          reinterpret_cast<uint16_t*>(rec + kRecKDelta)[tid] = f32_to_f16(r.delta);
          reinterpret_cast<uint16_t*>(rec + kRecKZero)[tid] = static_cast<uint16_t>(r.zm);
          codes32_stream(xk, r, cw);
          fimg_k[tid] = cw[0];
          fimg_k[kD + tid] = cw[1];
        } else if (tid < 2 * kD) {
          // Value (token t, group g) over 32 channels
          const int u = tid - kD, t = u & 31, g = u >> 5;
          auto xv = [&](int i) { return f16_to_f32(fv[(32 * g + i) * 32 + t]); };
          const Range r = range32_stream(xv);
          reinterpret_cast<uint32_t*>(rec + kRecVParam)[32 * g + t] =
              static_cast<uint32_t>(f32_to_f16(r.delta)) | (r.zm << 16);
          codes32_stream(xv, r, cw);
          *reinterpret_cast<uint2*>(fimg_v + g * kVImgRow + 2 * t) = uint2{cw[0], cw[1]};
        }
        __syncthreads();
        for (int i = tid; i < 512; i += NT) {
          if (i < 256) {
            const int t = i >> 3, j = i & 7;  // Key word j of token t
            *reinterpret_cast<uint32_t*>(rec + kRecKCodes + 32 * t + 4 * j) = key_word(fimg_k, t, j);
          } else {
            const int w = i - 256, oct = (w >> 6) & 3, m = (w >> 2) & 15, d = w & 3;
            *reinterpret_cast<uint32_t*>(rec + kRecVCodes + 16 * (16 * oct + m) + 4 * d) =
                value_word(fimg_v, oct, m, d);
          }
        }
        __syncthreads();  // the next block reuses the staging
      }
      // the records are in memory (this workgroup's stores have completed)
      // before its copies of them start
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      __syncthreads();
      if (has_ring) load_ring();
      if (cnt > 0) dma_block(0, st0);
      if (cnt > 1) dma_block(1, st1);
    }
  }

#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int i = wave + NW * j;
    if (i < GRP) {
      float qx, qy;
      if (A.q_mode == 2) {
        qx = __uint_as_float(qbx[j]);
        qy = __uint_as_float(qby[j]);
      } else {
        qx = in_to_f32(static_cast<uint16_t>(qbx[j]), A.q_mode);
        qy = in_to_f32(static_cast<uint16_t>(qby[j]), A.q_mode);
        const float2 qcs = q_rope_on ? qcs_ld : make_float2(1.0f, 0.0f);
        rope_pair(qx, qy, qcs.x, qcs.y);
        fht128_wave(qx, qy);
      }
      // q' carries the score scale 1/sqrt(128) * log2(e): every score
      // comes out in the log2 domain of the softmax
      qs[i * kD + L] = qx * kScale;
      qs[i * kD + L + 64] = qy * kScale;
    }
  }
  // Decode step: the new token's rotated Key rows (every head: the TOKEN
  // norm spans them) and this head's stored Value row, for the wave whose
  // window chunk holds it -- the append's arithmetic, in the append's order.
  auto rotate_new = [&](uint16_t kx, uint16_t ky, float& ya, float& yb) {
    ya = in_to_f32(kx, A.kv_bf16);
    yb = in_to_f32(ky, A.kv_bf16);
    if (A.rope) {  // the new token sits at position n_old
      const float2 cs = reinterpret_cast<const float2*>(A.rope)[static_cast<size_t>(n_old) * 64 + L];
      rope_pair(ya, yb, cs.x, cs.y);
    }
    fht128_wave(ya, yb);
  };
  const bool flush_step = app && n_old - Q_old == kR;
  if constexpr (STEP != 0) {
    if (wg_new) {
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int hh = wave + NW * j;
        if (hh < A.hkv) {
          float ya, yb;
          rotate_new(knx[j], kny[j], ya, yb);
          const float ss = wave_tree_sumsq(ya, yb);
          if (L == 0) step_part[hh] = ss;
          if (hh == h) {
            step_y[L] = ya;
            step_y[L + 64] = yb;
          }
        }
      }
      if (tid < kD) step_v[tid] = f16_sat_bits(in_to_f32(vnew, A.kv_bf16));
    }
  }
  __syncthreads();
  // block 1's copy (a flushing workgroup issued both with its records)
  if (!wg_fresh && cnt > 1) dma_block(1, st1);
  if constexpr (STEP != 0) {
    if (wave_new) {
      // the token's Key row and norm as the append stores them, put in place
      // of what the window loads read at its slot
      const float ss = A.head_norm ? step_part[h] : tree16(step_part, A.hkv);
      float nrm, r;
      scale_from_ss(ss, nrm, r, A.hw_rsq != 0);
      const int tau = n_old - ring_tb;  // its place in the chunk
      if (col == (tau & 15)) {
        // lane (col, g4): token 16 tau' + col, channels 32 g4 + 8 kk + 0..7
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          u32x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = 32 * g4 + 8 * kk + 2 * i;
            w[i] = static_cast<uint32_t>(f32_to_f16(mul_rn(step_y[c], r))) |
                   (static_cast<uint32_t>(f32_to_f16(mul_rn(step_y[c + 1], r))) << 16);
          }
          if (tau < 16)
            rk[0][kk] = w;
          else
            rk[1][kk] = w;
        }
      }
      if (g4 == (tau >> 3)) {
        // lane (col, g4): channel 16 ct + col, tokens 8 g4 .. 8 g4 + 7
        const int e = tau & 7;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          const uint32_t hv = step_v[16 * ct + col];
#pragma unroll
          for (int wi = 0; wi < 4; ++wi)
            if ((e >> 1) == wi)
              rv[ct][wi] = (e & 1) ? ((rv[ct][wi] & 0xFFFFu) | (hv << 16)) : ((rv[ct][wi] & 0xFFFF0000u) | hv);
        }
      }
      const uint16_t nrm16 = f16_sat_bits(nrm);
#pragma unroll
      for (int j = 0; j < TPL; ++j)
        if (sm_t0 + j == tau) {
          uint32_t& w = rnw[j >> 1];
          w = TPL == 1 ? nrm16
              : (j & 1) ? ((w & 0xFFFFu) | (static_cast<uint32_t>(nrm16) << 16)) : ((w & 0xFFFF0000u) | nrm16);
        }
      // Without a flush no other wave reads the new token's slot in this
      // launch (the window holds at most 128 tokens, each slot in one chunk,
      // and this wave has read its chunk): it stores the append's window
      // row and column of this head, and the norm, now, so that they complete
      // during its main loop rather than at the end of the launch.
      if (!flush_step) {
        const int slot = n_old % kR;
        uint16_t* rkw = const_cast<uint16_t*>(A.res_k) + (bh * kR + slot) * kD;
        rkw[L] = f32_to_f16(mul_rn(step_y[L], r));
        rkw[L + 64] = f32_to_f16(mul_rn(step_y[L + 64], r));
        const_cast<uint16_t*>(A.res_v)[(bh * kD + L) * kR + slot] = step_v[L];
        const_cast<uint16_t*>(A.res_v)[(bh * kD + L + 64) * kR + slot] = step_v[L + 64];
        if (L == 0 && (A.head_norm || h == 0))
          const_cast<uint16_t*>(A.res_norm)[A.head_norm ? bh * kR + slot : static_cast<size_t>(b) * kR + slot] = nrm16;
      }
    }
  }
  float m_run = -INFINITY, l_part = 0.0f;
  float zacc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) zacc[r] = 0.0f;
  f32x4 o[8];  // set by the window chunk or zeroed before the INT2 blocks

  // Online softmax of one block's raw scores (Wsc) in the log2 domain; also
  // rescales the accumulators when a head's running maximum grows (nothing to
  // rescale in a wave's first block).  Every processed block has at least one
  // valid token, so m_new is finite.
  auto softmax_block = [&](const float* nt, float kp, int t_valid, bool first) {
    float sv[TPL];
    float bm = -INFINITY;
    if (sm_on) {
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const int t = sm_t0 + j;
        sv[j] = t < t_valid ? (Wsc[sm_head][t] + Wsc[sm_head + GRP][t] + kp) * nt[j] : -INFINITY;
        bm = fmaxf(bm, sv[j]);
      }
    }
    bm = group_max<LPH>(bm);
    const float m_new = fmaxf(m_run, bm);
    const bool grow = sm_on && m_new > m_run;
    float ps = 0.0f;
    if (sm_on) {
#pragma unroll
      for (int j = 0; j < TPL; ++j) {
        const float pj = __builtin_amdgcn_exp2f(sv[j] - m_new);  // -inf gives 0
        Wpr[sm_head][sm_t0 + j] = pj;
        ps = j == 0 ? pj : ps + pj;
      }
    }
    if (!first && __any(grow)) {
      // rare after the first blocks: rescale the heads whose maximum grew
      // (a wave's first block has m_run = -inf: factor 0 on zero sums)
      const float f = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // -inf gives 0
      l_part *= f;
      if (sm_on && (L % LPH) == 0) Wfac[sm_head] = f;
      lds_order();
      const float fo = col < NCOL ? Wfac[col % GRP] : 1.0f;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) o[ct] *= fo;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int c = L + 64 * r;
        if (c < NCOMBO) zacc[r] *= Wfac[(c >> 2) % GRP];
      }
    }
    l_part += ps;
    m_run = m_new;
    lds_order();
  };

  // the q.K^T tiles' score columns into Wsc as they are: the hi column of
  // head h into row h, its lo column into row h + GRP (the softmax adds the
  // two, which costs its lanes one LDS read instead of a cross-lane move and
  // an add per score here)
  auto store_scores = [&](const f32x4* cs) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
      if (col < NCOL) *reinterpret_cast<f32x4*>(&Wsc[col][16 * tau + 4 * g4]) = cs[tau];
    lds_order();
  };

  // P.V operands of one block from Wpr: W unit c -> group c / (4 GRP),
  // head (c >> 2) % GRP, token octet c & 3
  auto pv_tiles = [&](const UnitRegs<NR, CPL>* cur) {
    // every unit's probabilities are read before any B tile is written: the
    // tiles share their LDS region with Wpr
    f32x4 pq[NR][2];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int c = L + 64 * r;
      if (c < NCOMBO) {
        const int hh = (c >> 2) % GRP, g8 = c & 3;
        pq[r][0] = *reinterpret_cast<const f32x4*>(&Wpr[hh][8 * g8]);
        pq[r][1] = *reinterpret_cast<const f32x4*>(&Wpr[hh][8 * g8 + 4]);
      }
    }
    lds_order();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int c = L + 64 * r;
      if (c < NCOMBO) {
        const int gv = c / (4 * GRP), hh = (c >> 2) % GRP, g8 = c & 3;
        const f32x4 p0 = pq[r][0], p1 = pq[r][1];
        const float pv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        u32x4 hi, lo;
        if (cur) {
          _Float16 d8[8];
          // sum p * z_v with fused mixed-precision multiply-adds (the fp16
          // zero point enters the fma without a conversion of its own)
          float zsum = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t pz = cur->vp[r][k >> 2][k & 3];
            d8[k] = hbits(pz, 0);
            zsum = __builtin_fmaf(pv[k], static_cast<float>(hbits(pz, 1)), zsum);
          }
          zacc[r] += zsum;
          split8_mul(pv, d8, hi, lo);
        } else {
          split8(pv, hi, lo);
        }
        Wbv[gv][brow_v<NCOL>(hh + NCOL * g8)] = hi;
        Wbv[gv][brow_v<NCOL>(hh + GRP + NCOL * g8)] = lo;
      }
    }
    lds_order();
  };

#pragma unroll
  for (int ct = 0; ct < 8; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};


  // the INT2 blocks' per-lane query operands (filled after the window chunk)
  float qa[NR][8];
  float zq[CPL];

  // ---------------- quantized blocks, software-pipelined one block ahead
  auto process_int2 = [&](const UnitRegs<NR, CPL>& cur, auto&& after_qk, auto&& after_softmax) {
    // alpha units: q' * delta as hi/lo B tiles
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int c = L + 64 * r;
      if (c < NCOMBO) {
        const int hh = c % GRP, g = (c / GRP) & 3, kk = (c / (4 * GRP)) & 3;
        _Float16 d8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = slot_pos(i);
          d8[i] = hbits(cur.dz[r][j >> 1], j & 1);
        }
        u32x4 hi, lo;
        split8_mul(qa[r], d8, hi, lo);
        Wbk[kk][brow_k<NCOL>(hh + NCOL * g)] = hi;
        Wbk[kk][brow_k<NCOL>(hh + GRP + NCOL * g)] = lo;
      }
    }
    // q'.z of the softmax lane's head (one row of lanes), fused
    // mixed-precision multiply-adds as above
    float kz = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      kz = __builtin_fmaf(zq[j], static_cast<float>(hbits(cur.zz[j >> 3][(j & 7) >> 1], j & 1)), kz);
    kz = group_sum<LPH>(kz);
    lds_order();

    // q.K^T on the matrix cores
    f32x4 cs[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const uint32_t e0 = even_fields(cur.kc[tau][0]), o0 = odd_fields(cur.kc[tau][0]);
      const uint32_t e1 = even_fields(cur.kc[tau][1]), o1 = odd_fields(cur.kc[tau][1]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_f16(code_tile<0>(e0, o0), Wbk[0][krow], acc);
      acc = mfma_f16(code_tile<1>(e0, o0), Wbk[1][krow], acc);
      acc = mfma_f16(code_tile<0>(e1, o1), Wbk[2][krow], acc);
      acc = mfma_f16(code_tile<1>(e1, o1), Wbk[3][krow], acc);
      cs[tau] = acc;
    }
    after_qk();
    store_scores(cs);

    float nt[TPL];
#pragma unroll
    for (int j = 0; j < TPL; ++j)
      nt[j] = (j & 1) ? h_hi(cur.nrm[j >> 1]) : h_lo(cur.nrm[j >> 1]);
    softmax_block(nt, kz, 32, false);
    after_softmax();
    pv_tiles(&cur);

    // P.V on the matrix cores: tile ct = channels 16 ct .. 16 ct + 15
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t e = even_fields(cur.vc[d]), od = odd_fields(cur.vc[d]);
      const u32x4 bvd = Wbv[d][vrow];
      o[2 * d] = mfma_f16(code_tile<0>(e, od), bvd, o[2 * d]);
      o[2 * d + 1] = mfma_f16(code_tile<1>(e, od), bvd, o[2 * d + 1]);
    }
  };
  // ---------------- the fp16 window chunk, first (its loads were issued
  // before the records' copies; splits weigh a chunk as kRingWeight blocks)
  if (has_ring) {
    // q' hi/lo B tiles, channels 32 g4 + 8 kk + 0..7 in natural order
    u32x4 bq[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float x[8];
      const float* q = qs + (col % GRP) * kD + 32 * g4 + 8 * kk;
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = q[i];
      u32x4 hi, lo;
      split8(x, hi, lo);
      bq[kk] = col < GRP ? hi : lo;  // columns >= 2 GRP are unused
    }
    f32x4 cs[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma_f16(rk[tau][kk], bq[kk], acc);
      cs[tau] = acc;
    }
    store_scores(cs);
    // converted here, not where they were loaded: the empty statement keeps
    // the compiler from moving the conversion (and its wait) up there
#pragma unroll
    for (int i = 0; i < RNW; ++i) asm volatile("" : "+v"(rnw[i]));
    float rnt[TPL];
#pragma unroll
    for (int j = 0; j < TPL; ++j) rnt[j] = f16_to_f32(static_cast<uint16_t>(rnw[j >> 1] >> (16 * (j & 1))));
    softmax_block(rnt, 0.0f, ring_valid, true);
    pv_tiles(nullptr);
    const u32x4 b0 = Wbv[0][vrow];
    lds_order();  // the INT2 blocks write this tile region next
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) o[ct] = mfma_f16(rv[ct], b0, o[ct]);
  }

  // The INT2 blocks' query operands, read from LDS once the window chunk's
  // registers are dead.
  // Alpha unit c: head c % GRP, channels c0 .. c0+7 with
  // c0 = 32 ((c / GRP) & 3) + 8 (c / (4 GRP)); slot i holds channel c0 + s(i).
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int c = L + 64 * r;
    const int hh = c % GRP, c0 = 32 * ((c / GRP) & 3) + 8 * ((c / (4 * GRP)) & 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) qa[r][i] = qs[hh * kD + c0 + slot_pos(i)];
  }
  // the softmax lane's share of q'.z
#pragma unroll
  for (int j = 0; j < CPL; ++j) zq[j] = sm_on ? qs[sm_head * kD + sm_c0 + j] : 0.0f;

  // One register set: block k + 1 is read from its stage into it in two
  // halves while block k is processed (Key part after k's softmax, Value part
  // after k's P.V); block k's stage is refilled with block k + 2 once k's
  // Q.K^T has been issued.  Copies of blocks k + 1 and k + 2 are in flight
  // during most of block k.
  UnitRegs<NR, CPL> ru;
  // Block 0 has landed, and so has every load issued before the copies:
  // only block 1's four copies, the newest operations, may still run.  A
  // wait the compiler sees on every path into the loop, so that it keeps no
  // stale wait for earlier register loads inside the loop, where a full wait
  // would also stall on the copies in flight.
  if (cnt > 1)
    __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4)
  else
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  if (cnt > 0) {
    read_kpart<GRP, NR, TPL, CPL>(ru, off, st0, L);
    read_vpart<GRP, NR, TPL, CPL>(ru, off, st0, L);
  }
  auto step = [&](int k, uint8_t* stc, uint8_t* stn) {
    progress_prio(k, cnt);
    process_int2(
        ru,
        [&]() {
          if (k + 2 < cnt) {
            lds_wait();  // block k's stage has been read completely
            dma_block(k + 2, stc);
          }
        },
        [&]() {
          // block k + 1's copy has landed (k + 2's may still run); past the
          // last block nothing is read that is used
          if (k + 2 < cnt)
            vmcnt_le4();
          else
            vmcnt_0();
          read_kpart<GRP, NR, TPL, CPL>(ru, off, stn, L);
        });
    read_vpart<GRP, NR, TPL, CPL>(ru, off, stn, L);
  };
  for (int k = 0; k < cnt; k += 2) {
    step(k, st0, st1);
    if (k + 1 >= cnt) break;
    step(k + 1, st1, st0);
  }
  __builtin_amdgcn_s_setprio(0);

  // ---------------- this wave's partial: l, Z, o for each head
  const float lsum = group_sum<LPH>(l_part);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int c = L + 64 * r;
    const float z = group_sum<4>(zacc[r]);
    if (c < NCOMBO && (c & 3) == 0) Wzs[c / (4 * GRP)][(c >> 2) % GRP] = z;
  }
  lds_order();
  // (the four sums of the lane's head, read by every lane: col % GRP is a
  // head of the wave)
  float zs[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) zs[d] = Wzs[d][col % GRP];
  // (only the lanes of the hi columns, col < GRP, store: the zero-point sum
  // is chosen once per group of 32 channels, not per element)
#pragma unroll
  for (int d = 0; d < 4; ++d) zs[d] = col < GRP ? zs[d] : 0.0f;
  float ov[8][4];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ov[ct][j] = o[ct][j] + dpp<dpp_row_shl(GRP)>(o[ct][j]) + zs[ct >> 1];
  // the stages take the waves' partial outputs: head hh of wave w at
  // (hh < 4 ? stage0 : stage1)[w] + 512 (hh % 4) bytes, once every copy into
  // them has landed
  auto wo_at = [&](int w, int hh) {
    return reinterpret_cast<float*>((hh < 4 ? stage0[w] : stage1[w]) + 512 * (hh & 3));
  };
  // Decode step, in the workgroup that counted itself in last (every other
  // workgroup of the sequence has finished reading {n, Q} and the window):
  // on a flush step the new token's window rows and norm for every head
  // (their slot held a flushed token that others read), then the new state.
  auto append_tail = [&]() {
    if (flush_step) {
      const int slot = n_old % kR;
      float ya[HPW], yb[HPW];
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int hh = wave + NW * j;
        ya[j] = yb[j] = 0.0f;
        if (hh < A.hkv) {
          uint16_t kx, ky;
          load_new(hh, kx, ky);
          rotate_new(kx, ky, ya[j], yb[j]);
          const float ss = wave_tree_sumsq(ya[j], yb[j]);
          if (L == 0) step_part[hh] = ss;
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int hh = wave + NW * j;
        if (hh < A.hkv) {
          float nrm, r;
          scale_from_ss(A.head_norm ? step_part[hh] : tree16(step_part, A.hkv), nrm, r, A.hw_rsq != 0);
          uint16_t* rkw = const_cast<uint16_t*>(A.res_k) + ((static_cast<size_t>(b) * A.hkv + hh) * kR + slot) * kD;
          rkw[L] = f32_to_f16(mul_rn(ya[j], r));
          rkw[L + 64] = f32_to_f16(mul_rn(yb[j], r));
          if (L == 0 && (A.head_norm || hh == 0))
            const_cast<uint16_t*>(A.res_norm)[A.head_norm ? (static_cast<size_t>(b) * A.hkv + hh) * kR + slot
                                     : static_cast<size_t>(b) * kR + slot] = f16_sat_bits(nrm);
        }
      }
      // Value rows [B][Hkv][128][slots]; v_new [B][Hkv][128]
      for (int i = tid; i < A.hkv * kD; i += NT) {
        const size_t row = static_cast<size_t>(b) * A.hkv * kD + i;
        const_cast<uint16_t*>(A.res_v)[row * kR + slot] = f16_sat_bits(in_to_f32(A.v_new[row], A.kv_bf16));
      }
    }
    if (tid == 0) {
      const_cast<int32_t*>(A.seq_state)[2 * b] = n_old + 1;
      const_cast<int32_t*>(A.seq_state)[2 * b + 1] = Q;
      __hip_atomic_store(A.append_sync + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  // Decode step: this workgroup counts itself in (all of its reads are done)
  // and learns whether it is the sequence's last; where no merge counter is
  // taken below, on its own.
  auto count_in_alone = [&]() {
    if constexpr (STEP != 0) {
      // (lds_app is written in every case: LDS keeps an earlier launch's bytes)
      if (tid == 0)
        lds_app = app && __hip_atomic_fetch_add(A.append_sync + b, 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT) == A.hkv * A.splits - 1;
      __syncthreads();
    }
  };
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (sm_on && (L % LPH) == 0) {
    lds_ml[0][wave][sm_head] = m_run;
    lds_ml[1][wave][sm_head] = lsum;
  }
  if (col < GRP) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      *reinterpret_cast<f32x4*>(wo_at(wave, col) + 16 * ct + 4 * g4) =
          f32x4{ov[ct][0], ov[ct][1], ov[ct][2], ov[ct][3]};
  }
  __syncthreads();

  // ---------------- merge the NW waves into this split's partial
  const int S = A.splits;
  const size_t pbase = (static_cast<size_t>(b) * A.hq + h * GRP) * S;
  constexpr int NI = (GRP * kD + NT - 1) / NT;
  float Mi[NI], Li[NI], Oi[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int idx = tid + NT * i, hh = (idx >> 7) % GRP, c = idx & 127;
    // every operand is read before any is combined; a wave with no tokens
    // has m = -inf and weight 0.  Weights come from the hardware exp2 here
    // and in the cross-split merge: each is at most 1, and one below 2^-126
    // (a partial that small against the largest) may count as 0.
    float mw[NW], lw[NW], ow[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = lds_ml[0][w][hh];
      lw[w] = lds_ml[1][w][hh];
      ow[w] = wo_at(w, hh)[c];
    }
    float M = mw[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, mw[w]);
    float Lw = 0.0f, Ow = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = mw[w] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - M);
      Lw += sc * lw[w];
      Ow += sc * ow[w];
    }
    Mi[i] = M;
    Li[i] = Lw;
    Oi[i] = Ow;
  }
  // out = o / l, lse = (m + log2 l) ln 2 (scores are in log2 units); a
  // (sequence, head) with no tokens gets zeros and -inf
  auto finish = [&](int idx, float M, float Lw, float Ow) {
    const int hh = idx >> 7, c = idx & 127;
    const size_t row = static_cast<size_t>(b) * A.hq + h * GRP + hh;
    const bool empty = M == -INFINITY;
    A.out[row * kD + c] = empty ? 0.0f : Ow * (1.0f / Lw);
    if (c == 0 && A.lse) A.lse[row] = empty ? -INFINITY : (M + log2f(Lw)) * 0.6931471805599453f;
  };
  // the merge of the splits and the outputs; returns where this workgroup's
  // part ends
  auto merge_out = [&]() {
  if (S == 1) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (tid + NT * i < GRP * kD) finish(tid + NT * i, Mi[i], Li[i], Oi[i]);
    count_in_alone();
    return;
  }

  // ---------------- cross-split merge, in this launch: every split publishes
  // its partial and counts itself in; the last of the S to arrive merges
  // all S partials, in split order (the result does not depend on which
  // workgroup that is), and resets the counter for the next launch.
  float* ml = reinterpret_cast<float*>(A.ws_ml);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int idx = tid + NT * i, hh = idx >> 7, c = idx & 127;
    if (idx >= GRP * kD) break;
    const size_t part = pbase + static_cast<size_t>(hh) * S + s;
    if constexpr (PUB == 1) {
      store_dev(A.ws_o + part * kD + c, Oi[i]);
      if (c == 0) {
        store_dev(ml + 2 * part, Mi[i]);
        store_dev(ml + 2 * part + 1, Li[i]);
      }
    } else {
      A.ws_o[part * kD + c] = Oi[i];
      if (c == 0) A.ws_ml[part] = make_float2(Mi[i], Li[i]);
    }
  }
  if (!A.merge_in_kernel) {
    count_in_alone();
    return;
  }
  // every wave's stores have completed (reached the L2, or with PUB 1 the
  // device's coherence point) before the workgroup counts itself in
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __syncthreads();
  if (tid == 0) {
    int prev;
    if constexpr (PUB == 1)
      prev = __hip_atomic_fetch_add(A.counters + counter_slot(pair), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      prev = __hip_atomic_fetch_add(A.counters + counter_slot(pair), 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (STEP != 0) lds_app = 0;
    lds_last = prev == S - 1;
  }
  __syncthreads();
  // (PUB 0: the counter's acquire, on this workgroup's CU, precedes the
  // barrier that every thread passed before reading the partials)
  if (!lds_last) return;
  // Decode step: the last split of each (sequence, KV head) counts the head
  // in for the sequence once all S splits have read what they read (one
  // counter increment per head, not per split); the answer comes back
  // while the splits are merged.
  // It is issued by a wave that reads no partials when there is one (its
  // loads then need not wait for the counter's round trip: a wave's vector
  // memory results return in order).
  constexpr int kCountTid = NT > GRP * kD ? NT - 64 : 0;
  int pa = -1;
  if constexpr (STEP != 0)
    if (app && tid == kCountTid)
      pa = __hip_atomic_fetch_add(A.append_sync + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto counted = [&]() {
    if constexpr (STEP != 0)
      if (tid == kCountTid) lds_app = app && pa == A.hkv - 1;
  };
  if (S <= 32) {
    // Lane j < S of each wave reads split j's (m, l) of the wave's head and
    // every lane reads its channel of all S partial outputs, all at once; the
    // weights come from wave reductions (the same values in every lane) and
    // the outputs fold in split order, weight j read from lane j.
    const int lane = tid & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = tid + NT * i, hh = idx >> 7, c = idx & 127;
      if (idx >= GRP * kD) break;  // whole waves: GRP * 128 is a multiple of 64
      const size_t base = pbase + static_cast<size_t>(hh) * S;
      float mj = -INFINITY, lj = 0.0f, oc[32];
      if (lane < S) {
        mj = load_dev(ml + 2 * (base + lane));
        lj = load_dev(ml + 2 * (base + lane) + 1);
      }
      // all 32 loads issued back to back, with no branch between them: a
      // split index past S re-reads split S - 1, whose weight below is 0
      const float* const ob = A.ws_o + base * kD + c;
#pragma unroll
      for (int j = 0; j < 32; ++j) oc[j] = load_dev(ob + static_cast<size_t>(j < S ? j : S - 1) * kD);
      const float M = wave_max(mj);
      const float wj = mj == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mj - M);
      const float Lw = wave_sum(wj * lj);
      float Ow = 0.0f;
      // (no branch on S: weight j >= S is 0 and oc[j] a finite re-read, so
      // those terms add zero and leave Ow unchanged)
#pragma unroll
      for (int j = 0; j < 32; ++j)
        Ow += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), j)) * oc[j];
      finish(idx, M, Lw, Ow);
    }
    if (tid == 0) __hip_atomic_store(A.counters + counter_slot(pair), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    counted();
    return;
  }
  // more splits: a thread's partials are requested 16 at a time
  constexpr int kChunk = 16;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int idx = tid + NT * i, hh = idx >> 7, c = idx & 127;
    if (idx >= GRP * kD) break;
    const size_t base = pbase + static_cast<size_t>(hh) * S;
    float M = -INFINITY, Lw = 0.0f, Ow = 0.0f;
    for (int s0 = 0; s0 < S; s0 += kChunk) {
      float mc[kChunk], lc[kChunk], oc[kChunk];
      // the chunk's loads back to back, with no branch between them: a split
      // index past S re-reads split S - 1 and gets m = -inf (weight 0)
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const int sj = s0 + j;
        const size_t sc = static_cast<size_t>(sj < S ? sj : S - 1);
        if constexpr (PUB == 1) {
          mc[j] = load_dev(ml + 2 * (base + sc));
          lc[j] = load_dev(ml + 2 * (base + sc) + 1);
          oc[j] = load_dev(A.ws_o + (base + sc) * kD + c);
        } else {
          const float2 v = A.ws_ml[base + sc];
          mc[j] = v.x;
          lc[j] = v.y;
          oc[j] = A.ws_o[(base + sc) * kD + c];
        }
      }
#pragma unroll
      for (int j = 0; j < kChunk; ++j) mc[j] = s0 + j < S ? mc[j] : -INFINITY;
      float mb = M;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) mb = fmaxf(mb, mc[j]);
      if (mb == -INFINITY) continue;
      const float f = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - mb);
      Lw *= f;
      Ow *= f;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        const float w = mc[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mc[j] - mb);
        Lw += w * lc[j];
        Ow += w * oc[j];
      }
      M = mb;
    }
    finish(idx, M, Lw, Ow);
  }
  if (tid == 0) __hip_atomic_store(A.counters + counter_slot(pair), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  counted();
  };
  merge_out();
  if constexpr (STEP != 0) {
    // the sequence's last workgroup makes the append's remaining stores
    // (one place, after whatever merging this workgroup did)
    __syncthreads();
    if (lds_app) append_tail();
  }
}

// ---------------------------------------------------------------- reduce
// grid (Hq, B), 256 threads: merge the S partials of one query head.  Thread
// t takes channels 4*(t&31)..+3 of the splits s = t>>5 + 8j; it loads up to
// 16 of them at once and folds them into a running (max, sum, o) of its own;
// the 8 split lanes of a channel quad are then merged through LDS.
__global__ __launch_bounds__(256) void lse_reduce_kernel(const float2* __restrict__ ws_ml,
                                                         const float* __restrict__ ws_o, int hq,
                                                         int splits, float* __restrict__ out,
                                                         float* __restrict__ lse) {
  constexpr int kBatch = 16;
  __shared__ float4 red_o[8][32];
  __shared__ float red_m[8], red_l[8];
  const int i = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const size_t base = (static_cast<size_t>(b) * hq + i) * splits;
  const int cg = t & 31, sl = t >> 5;
  float m = -INFINITY, l = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = sl; s0 < splits; s0 += 8 * kBatch) {
    float2 ml[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int sj = s0 + 8 * j;
      if (sj < splits) {
        ml[j] = ws_ml[base + sj];
        v[j] = reinterpret_cast<const float4*>(ws_o + (base + sj) * kD)[cg];
      } else {
        ml[j] = make_float2(-INFINITY, 0.0f);
        v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float mb = m;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, ml[j].x);
    if (mb == -INFINITY) continue;
    const float f = exp2f(m - mb);  // m == -inf gives 0
    l *= f;
    acc.x *= f;
    acc.y *= f;
    acc.z *= f;
    acc.w *= f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float w = ml[j].x == -INFINITY ? 0.0f : exp2f(ml[j].x - mb);
      acc.x += w * v[j].x;
      acc.y += w * v[j].y;
      acc.z += w * v[j].z;
      acc.w += w * v[j].w;
      l += w * ml[j].y;
    }
    m = mb;
  }
  red_o[sl][cg] = acc;
  if (cg == 0) {
    red_m[sl] = m;
    red_l[sl] = l;
  }
  __syncthreads();
  if (t < 32) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) M = fmaxf(M, red_m[k]);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float Lt = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (red_m[k] == -INFINITY) continue;
        const float w = exp2f(red_m[k] - M);
        const float4 v = red_o[k][t];
        a.x += w * v.x;
        a.y += w * v.y;
        a.z += w * v.z;
        a.w += w * v.w;
        Lt += w * red_l[k];
      }
    }
    const bool empty = M == -INFINITY;
    const float inv = empty ? 0.0f : 1.0f / Lt;
    reinterpret_cast<float4*>(out + (static_cast<size_t>(b) * hq + i) * kD)[t] =
        make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    if (lse && t == 0)
      lse[static_cast<size_t>(b) * hq + i] = empty ? -INFINITY : (M + log2f(Lt)) * 0.6931471805599453f;
  }
}

// Build-time overrides of the launch shape, for A/B timing of alternatives
// (0 = chosen per call below).
#ifndef OSCAR_ATTN_NW
#define OSCAR_ATTN_NW 0
#endif
#ifndef OSCAR_ATTN_PUB
#define OSCAR_ATTN_PUB 1
#endif

// Launch shape of the matrix-core kernel: waves per workgroup and splits per
// (sequence, KV head).  The chip holds 256 CUs x 12 waves at three waves per
// SIMD.  Few (sequence, KV head) pairs: one 12-wave workgroup per CU, as
// many splits as fill all 256 CUs once (a CU left idle costs its share of the
// bandwidth), while every wave still gets a unit.  Many pairs: three 4-wave
// workgroups per CU, one round of them.  The launch order (longest sequence
// first, dealt round-robin over the CUs) already gives each CU a long, a
// middle and a short workgroup; a second round would only add a second
// round of set-up and merge per workgroup slot (ragged batch of 48 at 8K..32K:
// 180 us per step with two splits per pair against 183 us with four).
struct AttnShape {
  int nw, splits, merge_in_kernel;
};
#ifndef OSCAR_ATTN_MERGE_MANY
#define OSCAR_ATTN_MERGE_MANY 1   // merge in the kernel also with many pairs
#endif
AttnShape attn_shape(const oscar_cache_geom* g, int max_ctx, int num_splits) {
  const int units = (max_ctx + kG - 1) / kG + 1;
  const int pairs = g->batch * g->num_kv_heads;
  int nw = OSCAR_ATTN_NW ? OSCAR_ATTN_NW : (pairs >= 128 ? 4 : 12);
  int s = num_splits;
  if (!s) {
    s = (256 * (12 / nw) + pairs - 1) / pairs;
    const int cap = units / (nw == 12 ? nw : 4 * nw) > 1 ? units / (nw == 12 ? nw : 4 * nw) : 1;
    if (s > cap) s = cap;
    if (s > 1024) s = 1024;
    if (s < 1) s = 1;
  }
  return AttnShape{nw, s, (pairs >= 128 && !OSCAR_ATTN_MERGE_MANY) ? 0 : 1};
}
int auto_splits(const oscar_cache_geom* g, int max_ctx) { return attn_shape(g, max_ctx, 0).splits; }

// Workspace of the matrix-core path: the merge's arrival counters first, at
// a fixed place and size (one int32 per (sequence, KV head), for up to
// kMaxPairs pairs, at counter_slot), so that a workspace zero-filled once stays valid for any
// later call whatever its geometry or split count; then the partials in the
// layout the separate merge launch reads (workspace_bytes below).
constexpr int kMaxPairs = 65536;
constexpr size_t kCounterBytes = static_cast<size_t>(kMaxPairs) * sizeof(int32_t);

// Partials: ws_ml [B][Hq][S] float2, then (256-B aligned) ws_o [B][Hq][S][128],
// then (256-B aligned) the launch schedule, [B] x {b, n, Q, 0}.
static size_t round256(size_t x) { return (x + 255) / 256 * 256; }
size_t workspace_bytes(const oscar_cache_geom* g, int splits) {
  const size_t n = static_cast<size_t>(g->batch) * g->num_q_heads * splits;
  return round256(n * sizeof(float2)) + round256(n * kD * sizeof(float)) +
         round256(static_cast<size_t>(g->batch) * 4 * sizeof(int32_t));
}

// The launch schedule of a batch: the sequences longest first (ties in
// index order), each with the {n, Q} it has before the launch.  The GPU
// starts workgroups in launch order as slots free up, so with contexts of
// different lengths the long sequences' workgroups, started first, no
// longer end the launch alone.  The attention kernel reads every {n, Q} from
// here, so that its workgroups agree on the order even once a decode step's
// appends have rewritten some states.  One workgroup; B <= 1024.
constexpr int kSchedMax = 1024;
__global__ __launch_bounds__(kSchedMax) void sched_kernel(const int32_t* __restrict__ seq_state, int batch,
                                                         int32_t* __restrict__ sched) {
  __shared__ int len[kSchedMax];
  const int t = threadIdx.x;
  int n = 0, Q = 0;
  if (t < batch) {
    n = seq_state[2 * t];
    Q = seq_state[2 * t + 1];
    len[t] = n;
  }
  __syncthreads();
  if (t < batch) {
    int r = 0;
    for (int j = 0; j < batch; ++j) {
      const int m = len[j];
      r += (m > n || (m == n && j < t)) ? 1 : 0;
    }
    *reinterpret_cast<int4*>(sched + 4 * r) = make_int4(t, n, Q, 0);
  }
}
static size_t attn_workspace_bytes(const oscar_cache_geom* g, int splits) {
  return kCounterBytes + workspace_bytes(g, splits);
}

void launch_lse_reduce(const float2* ws_ml, const float* ws_o, int hq, int batch, int splits,
                       float* out, float* lse, hipStream_t st) {
  hipLaunchKernelGGL(lse_reduce_kernel, dim3(hq, batch), dim3(256), 0, st, ws_ml, ws_o, hq, splits,
                     out, lse);
}

template <int GRP, int STEP>
void launch_mfma(const AttnArgs& A, int nwg, int nw, hipStream_t st) {
  constexpr int P = OSCAR_ATTN_PUB;
  if (nw == 12)
    hipLaunchKernelGGL((attn_mfma_kernel<GRP, 12, P, STEP>), dim3(nwg), dim3(768), 0, st, A);
  else if (nw == 6)
    hipLaunchKernelGGL((attn_mfma_kernel<GRP, 6, P, STEP>), dim3(nwg), dim3(384), 0, st, A);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<GRP, 4, P, STEP>), dim3(nwg), dim3(256), 0, st, A);
}

}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_decode_workspace_bytes(const oscar_cache_geom* geom, int32_t max_ctx,
                                                     int32_t num_splits, int32_t* splits_out,
                                                     size_t* bytes) {
  oscar_status st = check_geom(geom);
  if (st != OSCAR_OK) return st;
  if (!bytes || max_ctx < 0 || num_splits < 0 || num_splits > 1024) return OSCAR_EINVAL;
  const int s = attn_shape(geom, max_ctx, num_splits).splits;
  if (splits_out) *splits_out = s;
  *bytes = attn_workspace_bytes(geom, s);
  return OSCAR_OK;
}

// One decode call: attention alone (step == null) or, with the new tokens,
// the fused decode step.
static oscar_status decode_call(const oscar_cache_geom* geom, const oscar_cache* cache,
                                const void* q, oscar_dtype q_dtype, float* out, float* lse,
                                void* workspace, size_t ws_bytes, int32_t num_splits,
                                int32_t max_ctx, oscar_attn_variant variant, void* stream,
                                const void* k_new, const void* v_new, oscar_dtype kv_dtype) {
  const bool step = k_new != nullptr;
  oscar_status st = check_cache(geom, cache);
  if (st != OSCAR_OK) return st;
  if (!q || !out || !workspace || max_ctx < 0 || num_splits < 0 || num_splits > 1024)
    return OSCAR_EINVAL;
  if (q_dtype != OSCAR_FP16 && q_dtype != OSCAR_BF16 && q_dtype != OSCAR_FP32) return OSCAR_EINVAL;
  if (!aligned(workspace, 256) || !aligned(q, 4) || !aligned(out, 16)) return OSCAR_EINVAL;
  if (variant != OSCAR_ATTN_AUTO && variant != OSCAR_ATTN_VALU && variant != OSCAR_ATTN_MFMA)
    return OSCAR_EINVAL;
  if (step && (!v_new || (kv_dtype != OSCAR_FP16 && kv_dtype != OSCAR_BF16))) return OSCAR_EINVAL;
  if (static_cast<long long>(geom->batch) * geom->num_kv_heads > kMaxPairs) return OSCAR_EINVAL;
  const AttnShape shape = attn_shape(geom, max_ctx, num_splits);
  const int S = shape.splits;
  if (ws_bytes < attn_workspace_bytes(geom, S)) return OSCAR_EWORKSPACE;
  st = check_device();
  if (st != OSCAR_OK) return st;
  if (step && variant == OSCAR_ATTN_VALU) {
    // the vector-ALU variant has no fused form: the append, then attention
    st = oscar_append_kv(geom, cache, k_new, v_new, kv_dtype, stream);
    if (st != OSCAR_OK) return st;
    return decode_call(geom, cache, q, q_dtype, out, lse, workspace, ws_bytes, num_splits, max_ctx,
                       variant, stream, nullptr, nullptr, kv_dtype);
  }
  AttnArgs A;
  A.pool = static_cast<const uint8_t*>(cache->pool);
  A.pool_norm = static_cast<const uint16_t*>(cache->pool_norm);
  A.res_k = static_cast<const uint16_t*>(cache->res_k);
  A.res_v = static_cast<const uint16_t*>(cache->res_v);
  A.res_norm = static_cast<const uint16_t*>(cache->res_norm);
  A.head_norm = geom->norm_scope == OSCAR_NORM_HEAD ? 1 : 0;
  A.block_table = cache->block_table;
  A.seq_state = cache->seq_state;
  A.q = q;
  A.q_mode = q_dtype == OSCAR_FP32 ? 2 : (q_dtype == OSCAR_BF16 ? 1 : 0);
  A.hkv = geom->num_kv_heads;
  A.hq = geom->num_q_heads;
  A.max_blocks = geom->max_blocks_per_seq;
  A.nphys = geom->num_physical_blocks;
  A.error_flag = cache->error_flag;
  A.splits = S;
  const size_t npart = static_cast<size_t>(geom->batch) * geom->num_q_heads * S;
  char* part_base = static_cast<char*>(workspace) + kCounterBytes;
  A.counters = static_cast<int32_t*>(workspace);
  A.ws_ml = reinterpret_cast<float2*>(part_base);
  A.ws_o = reinterpret_cast<float*>(part_base + ((npart * sizeof(float2) + 255) / 256) * 256);
  A.out = out;
  A.lse = lse;
  A.rope = geom->rope_max_pos > 0 ? cache->rope : nullptr;
  A.rope_max_pos = geom->rope_max_pos;
  A.k_new = static_cast<const uint16_t*>(k_new);
  A.v_new = static_cast<const uint16_t*>(v_new);
  A.kv_bf16 = kv_dtype == OSCAR_BF16 ? 1 : 0;
  A.flush_blocks = geom->flush_tokens == 128 ? 4 : 1;
  A.hw_rsq = geom->key_scale == OSCAR_SCALE_HW_RSQ ? 1 : 0;
  A.append_sync = cache->append_sync;
  A.sched = nullptr;
  hipStream_t hs = as_stream(stream);
  const int grp = geom->num_q_heads / geom->num_kv_heads;
  if (variant == OSCAR_ATTN_VALU) {
    // the vector-ALU kernel writes partials; a second launch merges them
    const dim3 grid(S, geom->num_kv_heads, geom->batch);
    switch (grp) {
      case 1: hipLaunchKernelGGL(attn_valu_kernel<1>, grid, dim3(256), 0, hs, A); break;
      case 2: hipLaunchKernelGGL(attn_valu_kernel<2>, grid, dim3(256), 0, hs, A); break;
      case 4: hipLaunchKernelGGL(attn_valu_kernel<4>, grid, dim3(256), 0, hs, A); break;
      default: hipLaunchKernelGGL(attn_valu_kernel<8>, grid, dim3(256), 0, hs, A); break;
    }
    st = launch_status();
    if (st != OSCAR_OK) return st;
    launch_lse_reduce(A.ws_ml, A.ws_o, geom->num_q_heads, geom->batch, S, out, lse, hs);
    return launch_status();
  }
  // the matrix-core kernel; with few (sequence, KV head) pairs it merges
  // the splits itself (one launch), with many the separate merge launch
  // spreads the merging over the chip
  A.merge_in_kernel = shape.merge_in_kernel;
  const int nwg = geom->batch * geom->num_kv_heads * S;
  if (geom->batch >= 2 && geom->batch <= kSchedMax) {
    int32_t* sched = reinterpret_cast<int32_t*>(
        part_base + round256(npart * sizeof(float2)) + round256(npart * kD * sizeof(float)));
    // one thread per sequence, in whole waves (one wave up to 64 sequences)
    const int threads = (geom->batch + 63) / 64 * 64;
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(threads), 0, hs, cache->seq_state, geom->batch, sched);
    st = launch_status();
    if (st != OSCAR_OK) return st;
    A.sched = sched;
  }
  if (step) {
    switch (grp) {
      case 1: launch_mfma<1, 1>(A, nwg, shape.nw, hs); break;
      case 2: launch_mfma<2, 1>(A, nwg, shape.nw, hs); break;
      case 4: launch_mfma<4, 1>(A, nwg, shape.nw, hs); break;
      default: launch_mfma<8, 1>(A, nwg, shape.nw, hs); break;
    }
  } else {
    switch (grp) {
      case 1: launch_mfma<1, 0>(A, nwg, shape.nw, hs); break;
      case 2: launch_mfma<2, 0>(A, nwg, shape.nw, hs); break;
      case 4: launch_mfma<4, 0>(A, nwg, shape.nw, hs); break;
      default: launch_mfma<8, 0>(A, nwg, shape.nw, hs); break;
    }
  }
  st = launch_status();
  if (st != OSCAR_OK || A.merge_in_kernel || S == 1) return st;
  launch_lse_reduce(A.ws_ml, A.ws_o, geom->num_q_heads, geom->batch, S, out, lse, hs);
  return launch_status();
}

extern "C" oscar_status oscar_decode_attn(const oscar_cache_geom* geom, const oscar_cache* cache,
                                          const void* q, oscar_dtype q_dtype, float* out,
                                          float* lse, void* workspace, size_t ws_bytes,
                                          int32_t num_splits, int32_t max_ctx,
                                          oscar_attn_variant variant, void* stream) {
  return decode_call(geom, cache, q, q_dtype, out, lse, workspace, ws_bytes, num_splits, max_ctx,
                     variant, stream, nullptr, nullptr, OSCAR_FP16);
}

extern "C" oscar_status oscar_decode_step(const oscar_cache_geom* geom, const oscar_cache* cache,
                                          const void* k_new, const void* v_new,
                                          oscar_dtype kv_dtype, const void* q,
                                          oscar_dtype q_dtype, float* out, float* lse,
                                          void* workspace, size_t ws_bytes, int32_t num_splits,
                                          int32_t max_ctx, oscar_attn_variant variant,
                                          void* stream) {
  if (!k_new) return OSCAR_EINVAL;
  return decode_call(geom, cache, q, q_dtype, out, lse, workspace, ws_bytes, num_splits, max_ctx,
                     variant, stream, k_new, v_new, kv_dtype);
}
