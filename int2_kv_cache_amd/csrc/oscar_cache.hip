// oscar_cache.hip -- INT2 quantization and the residual window:
// oscar_quant_pack, oscar_append_kv, oscar_prefill_quantize.
//
// [SUM] 方法步骤详情 ②: one kernel quantizes Keys and Values together; Keys per
// channel over blocks of G=32 tokens, Values per token.  [POP] 三: the newest
// tokens stay in an fp16 residual cache of 128 tokens and are quantized in
// batch.  [RN] End-to-End Flow: prefill Keys go through FHT, per-token scaling
// and per-channel INT2 before entering the cache.  (Tags: oscar_device.hpp.)
#include "oscar_device.hpp"
#include "oscar_host.hpp"
#include "oscar_quant.hpp"

namespace oscar {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> two fp16, round to nearest even, packed a | b << 16 (one
// v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){a, b}, half2_t));
}

// Range of 32 fp16 values held as 16 packed pairs: two values per
// instruction, in fp16 (the extremes are exact there).
__device__ __forceinline__ Range range32_pk(const half2_t* xp) {
  half2_t mn = xp[0], mx = xp[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    mn = __builtin_elementwise_minimum(mn, xp[i]);
    mx = __builtin_elementwise_maximum(mx, xp[i]);
  }
  return range_of(static_cast<float>(__builtin_elementwise_minimum(mn.x, mn.y)),
                  static_cast<float>(__builtin_elementwise_maximum(mx.x, mx.y)), 0.0f);
}

// Range of a Value unit from its 32 inputs as fp32 (bf16 or fp16 values,
// exact), before their rounding to the stored fp16 values.  That rounding
// (clamp to +-65504, then round to nearest even) is monotone, so the stored
// extremes are the rounded input extremes: only those two are converted.
// Below 2^-14 the rounding moves a value by at most 2^-25 (fp16's subnormal
// spacing is 2^-24; bf16 values from 2^-14 to 65504 are fp16 values
// already), so the fast quotient of an unrounded input lies within a further
// 2^-25 rdelta of the stored value's, and the near margin widens by that.
// Returns false when an input is NaN or beyond +-65504 (the min / max
// propagate NaN): such a unit takes the plain path on its stored values.
__device__ __forceinline__ bool range32_row(const float* x, Range& r) {
#pragma clang fp contract(off)
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) {
    mn = __builtin_elementwise_minimum(mn, x[i]);
    mx = __builtin_elementwise_maximum(mx, x[i]);
  }
  if (!(mn >= -65504.0f && mx <= 65504.0f)) return false;
  r = range_of(f16_to_f32(f32_to_f16(mn)), f16_to_f32(f32_to_f16(mx)), 0.51f);
  return true;
}

// Prefill: the heads' Value images one after another, 4 words apart beyond
// their 4 rows, so that a wave's image writes (all heads, four groups, two
// tokens) spread over the banks.
constexpr int kVImgHead = 4 * kVImgRow + 4;

// Transpose of a 16 x 16 matrix of 2-bit fields: on return r[f] field i is
// what r[i] field f was (field i of a word at bits 2i).  Recursive block
// swap: at block size s the fields of rows r (bit s of r clear) whose index
// has bit s set trade places with the fields of row r + s whose index has it
// clear, two bitfield inserts per pair of rows.
__device__ __forceinline__ void transpose16x2(uint32_t* r) {
  constexpr uint32_t kMask[4] = {0x33333333u, 0x0F0F0F0Fu, 0x00FF00FFu, 0x0000FFFFu};
#pragma unroll
  for (int k = 3; k >= 0; --k) {
    const int s = 1 << k, sh = 2 * s;
    const uint32_t m = kMask[k];  // fields whose index has bit s clear
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & s) continue;
      const uint32_t a = r[i], b = r[i + s];
      r[i] = (a & m) | ((b << sh) & ~m);
      r[i + s] = ((a >> sh) & m) | (b & ~m);
    }
  }
}

// ---------------------------------------------------------------- quant_pack
// grid (n_blocks, Hkv), 256 threads: one (block, KV head) record.  Thread
// tg < 128 takes Key channel tg over the 32 tokens, thread tg >= 128 the
// Value (token, group) unit tg - 128; each computes its range and its 32
// codes into the LDS images, then every thread assembles two code words.
__global__ __launch_bounds__(256) void quant_pack_kernel(const uint16_t* __restrict__ khat,
                                                         const uint16_t* __restrict__ knorm,
                                                         const uint16_t* __restrict__ v16,
                                                         int hkv, int head_norm,
                                                         uint8_t* __restrict__ rec_out,
                                                         uint16_t* __restrict__ norm_out) {
  __shared__ __attribute__((aligned(16))) uint32_t img_k[2 * kD];
  __shared__ __attribute__((aligned(16))) uint32_t img_v[4 * kVImgRow];
  const int j = blockIdx.x, h = blockIdx.y, tg = threadIdx.x;
  const size_t row = static_cast<size_t>(hkv) * kD;
  uint8_t* rec = rec_out + (static_cast<size_t>(j) * hkv + h) * kRec;
  float x[32];
  uint32_t w[2];
  if (tg < 128) {
    const uint16_t* kb = khat + static_cast<size_t>(32 * j) * row + static_cast<size_t>(h) * kD + tg;
#pragma unroll
    for (int t = 0; t < 32; ++t) x[t] = f16_to_f32(kb[t * row]);
    const Range r = range32(x);
    reinterpret_cast<uint16_t*>(rec + kRecKDelta)[tg] = f32_to_f16(r.delta);
    reinterpret_cast<uint16_t*>(rec + kRecKZero)[tg] = static_cast<uint16_t>(r.zm);
    codes32(x, r, w);
    img_k[tg] = w[0];
    img_k[kD + tg] = w[1];
  } else {
    const int u = tg - 128, t = u >> 2, g = u & 3;
    const uint4* src = reinterpret_cast<const uint4*>(v16 + static_cast<size_t>(32 * j + t) * row +
                                                      static_cast<size_t>(h) * kD + 32 * g);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w8 = src[q];
      const uint32_t ww[4] = {w8.x, w8.y, w8.z, w8.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * q + e] = f16_to_f32(static_cast<uint16_t>(ww[e >> 1] >> (16 * (e & 1))));
    }
    const Range r = range32(x);
    reinterpret_cast<uint32_t*>(rec + kRecVParam)[32 * g + t] =
        static_cast<uint32_t>(f32_to_f16(r.delta)) | (r.zm << 16);
    codes32(x, r, w);
    *reinterpret_cast<uint2*>(img_v + g * kVImgRow + 2 * t) = uint2{w[0], w[1]};
  }
  __syncthreads();
  {
    const int t = tg >> 3, jw = tg & 7;  // Key word jw of token t
    *reinterpret_cast<uint32_t*>(rec + kRecKCodes + 32 * t + 4 * jw) = key_word(img_k, t, jw);
    const int oct = (tg >> 6) & 3, m = (tg >> 2) & 15, d = tg & 3;
    *reinterpret_cast<uint32_t*>(rec + kRecVCodes + 16 * (16 * oct + m) + 4 * d) =
        value_word(img_v, oct, m, d);
  }
  // norms: TOKEN knorm [T] -> [n_blocks][32]; HEAD knorm [T][Hkv] -> [n_blocks][Hkv][32]
  if (tg < 32) {
    if (head_norm)
      norm_out[(static_cast<size_t>(j) * hkv + h) * 32 + tg] = knorm[static_cast<size_t>(32 * j + tg) * hkv + h];
    else if (h == 0)
      norm_out[static_cast<size_t>(j) * 32 + tg] = knorm[32 * j + tg];
  }
}

// Quad cross-lane read (lanes 4m..4m+3 exchange): xor 1 or xor 2.
template <int X>
__device__ __forceinline__ float quad_xor(float x) {
  constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), ctrl, 0xF, 0xF, true));
}

// RoPE of the 128-vector a lane quad holds (lane tq: elements 32 tq ..
// 32 tq + 31) at position pos: element j of lane tq pairs with element j of
// lane tq ^ 2 (channels i and i + 64).  Four elements at a time: both lanes
// of a pair read each other's elements of the chunk before either
// overwrites them.  An invalid lane (no token) uses (1, 0).
__device__ __forceinline__ void rope_quad(float* x, int tq, const float* rope, int pos,
                                          bool valid) {
  const float2* cs = reinterpret_cast<const float2*>(rope) +
                     static_cast<size_t>(valid ? pos : 0) * 64 + 32 * (tq & 1);
  const bool lower = tq < 2;
#pragma unroll
  for (int j0 = 0; j0 < 32; j0 += 4) {
    float mate[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mate[j] = quad_xor<2>(x[j0 + j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float2 r = valid ? cs[j0 + j] : make_float2(1.0f, 0.0f);
      float lo = lower ? x[j0 + j] : mate[j], hi = lower ? mate[j] : x[j0 + j];
      rope_pair(lo, hi, r.x, r.y);
      x[j0 + j] = lower ? lo : hi;
    }
  }
}

// FHT of the 128-vector a lane quad holds, then x 1/sqrt(128): butterflies
// with strides 1..16 in registers, strides 32 and 64 across the quad (the
// partner is lane tq ^ 1, then tq ^ 2; the upper lane of a pair takes
// partner - own as one exactly rounded fma with -1) -- the oracle's stages
// in the oracle's order.  Returns the vector's sum of squares by the same
// pairwise tree (strides 1..16 in registers, 32 and 64 across the quad), the
// same value in all four lanes.
__device__ __forceinline__ float fht_quad(float* x, int tq) {
#pragma clang fp contract(off)
#pragma unroll
  for (int hs = 1; hs < 32; hs <<= 1)
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if ((j & hs) == 0) {
        const float a = x[j], b = x[j + hs];
        x[j] = a + b;
        x[j + hs] = a - b;
      }
  const float sg1 = (tq & 1) ? -1.0f : 1.0f, sg2 = (tq & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = __builtin_fmaf(sg1, x[j], quad_xor<1>(x[j]));
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = __builtin_fmaf(sg2, x[j], quad_xor<2>(x[j]));
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = x[j] * kFhtScale;
  // levels 1, 2, 4 within each run of 8 (the same additions as level by
  // level over all 32), then levels 8 and 16
  float s8[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float sq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sq[j] = x[8 * c + j] * x[8 * c + j];
#pragma unroll
    for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
      for (int j = 0; j < 8; j += 2 * hs) sq[j] = sq[j] + sq[j + hs];
    s8[c] = sq[0];
  }
  s8[0] = s8[0] + s8[1];
  s8[2] = s8[2] + s8[3];
  float ssum = s8[0] + s8[2];
  ssum = ssum + quad_xor<1>(ssum);
  ssum = ssum + quad_xor<2>(ssum);
  return ssum;
}

// ---------------------------------------------------------------- append
struct CacheArgs {
  uint8_t* pool;
  uint16_t* pool_norm;
  uint16_t* res_k;
  uint16_t* res_v;
  uint16_t* res_norm;
  const int32_t* block_table;
  int32_t* seq_state;
  int32_t* error_flag;
  int32_t* append_sync;  // [B] arrival counters of the append's workgroups
  int hkv;
  int max_blocks;
  int nphys;
  int head_norm;    // 1: a norm per (token, KV head) ([P][Hkv][32], [B][Hkv][128])
  int flush_blocks;  // blocks quantized when the window is full: 1 or 4
  int hw_rsq;        // 1: scaling factor from the hardware rsqrt
  const float* rope;  // null, or [rope_max_pos][64] (cos, sin) of each position
  int rope_max_pos;
};
// Token norm slots: TOKEN scope [P][32] and [B][128]; HEAD scope [P][Hkv][32]
// and [B][Hkv][128].
__device__ __forceinline__ size_t pool_norm_at(const CacheArgs& ca, int p, int h, int t) {
  return ca.head_norm ? (static_cast<size_t>(p) * ca.hkv + h) * 32 + t : static_cast<size_t>(p) * 32 + t;
}
__device__ __forceinline__ size_t res_norm_at(const CacheArgs& ca, int b, int h, int slot) {
  return ca.head_norm ? (static_cast<size_t>(b) * ca.hkv + h) * kR + slot : static_cast<size_t>(b) * kR + slot;
}

// {n, Q} as the kernels leave it: 0 <= Q, Q % 32 == 0, 0 <= n - Q <= 128,
// Q / 32 <= max_blocks.
__device__ __forceinline__ bool state_ok(int n, int Q, int max_blocks) {
  return Q >= 0 && (Q & 31) == 0 && n >= Q && n - Q <= kR && Q / kG <= max_blocks;
}

// grid B * Hkv: workgroup b * Hkv + h appends head h of sequence b's new
// token (and, when the window is full, quantizes head h's share of the
// flushed block); 512 threads, so that each of up to 8 heads of the new
// token rotates in a wave of its own (two per wave for 9..16 heads).  Every workgroup of a sequence reads {n, Q}
// first and counts itself in (append_sync[b]) once it knows the append goes
// ahead; the last to count itself in writes the new state at its end and
// resets the counter, so no workgroup can see a half-updated state.  The
// barriers order LDS only, so the counter's round trip overlaps the work.  In TOKEN scope every workgroup rotates all heads of the new token
// (2 KB) so that it has the norm over all heads without talking to the
// others; the same tree order as a single workgroup gives the same bits.
__global__ __launch_bounds__(512) void append_kernel(CacheArgs ca, const uint16_t* __restrict__ k_new,
                                                     const uint16_t* __restrict__ v_new,
                                                     int is_bf16) {
  __shared__ __attribute__((aligned(16))) uint32_t img_k[2 * kD];
  __shared__ __attribute__((aligned(16))) uint32_t img_v[4 * kVImgRow];
  // a flushed block of head h: its 32 Key rows [slot][channel] and its Value
  // columns [channel][slot], copied from the window with one 16-byte load per
  // thread each
  __shared__ __attribute__((aligned(16))) uint16_t fk[32 * kD];
  __shared__ __attribute__((aligned(16))) uint16_t fv[kD * 32];
  __shared__ float part[16];
  const int hkv = ca.hkv;
  const int b = blockIdx.x / hkv, h = blockIdx.x - b * hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // the new token's inputs do not depend on the state: load them first
  // (wave w holds heads w and w + 8)
  uint16_t kin[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hh = wave + 8 * j;
    kin[j][0] = kin[j][1] = 0;
    if (hh < hkv) {
      const size_t base = (static_cast<size_t>(b) * hkv + hh) * kD;
      kin[j][0] = k_new[base + lane];
      kin[j][1] = k_new[base + lane + 64];
    }
  }
  uint16_t vin = 0;
  if (tid < kD) vin = v_new[(static_cast<size_t>(b) * hkv + h) * kD + tid];
  int32_t* st = ca.seq_state + 2 * b;
  const int n = st[0];
  int Q = st[1];
  if (!state_ok(n, Q, ca.max_blocks)) {
    if (tid == 0 && h == 0) atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    return;
  }
  if (ca.rope && n >= ca.rope_max_pos) {  // no (cos, sin) for position n
    if (tid == 0 && h == 0) atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_POSITION));
    return;
  }
  const size_t bh = static_cast<size_t>(b) * hkv + h;
  const bool flush = n - Q == kR;
  if (flush) {
    const int nfb = ca.flush_blocks, j0 = Q / kG;
    if (j0 + nfb > ca.max_blocks) {
      if (tid == 0 && h == 0) atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_CAPACITY));
      return;
    }
    for (int i = 0; i < nfb; ++i) {
      const int pi = ca.block_table[static_cast<size_t>(b) * ca.max_blocks + j0 + i];
      if (pi < 0 || pi >= ca.nphys) {
        if (tid == 0 && h == 0) atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
        return;
      }
    }
  }
  // The append will happen (every check above is the same for all of the
  // sequence's workgroups): count this workgroup in now, while its work
  // proceeds.  The counter only orders the reads of {n, Q} -- each
  // workgroup has read them by now -- before the last arrival's write of
  // the new state, which later launches read.
  int prev = 0;
  if (tid == 0)
    prev = __hip_atomic_fetch_add(ca.append_sync + b, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  if (flush) {
    const int nfb = ca.flush_blocks, j0 = Q / kG;
    for (int fi = 0; fi < nfb; ++fi) {
      const int p = ca.block_table[static_cast<size_t>(b) * ca.max_blocks + j0 + fi];
      const int s0 = (Q + kG * fi) % kR;
      if (tid < 32 && (ca.head_norm || h == 0))
        ca.pool_norm[pool_norm_at(ca, p, h, tid)] = ca.res_norm[res_norm_at(ca, b, h, s0 + tid)];
      uint8_t* rec = ca.pool + (static_cast<size_t>(p) * hkv + h) * kRec;
      // Key rows of slots s0 .. s0 + 31 (contiguous), Value slots s0 .. s0 + 31
      // of each channel (64 contiguous bytes per channel)
      reinterpret_cast<uint4*>(fk)[tid] =
          reinterpret_cast<const uint4*>(ca.res_k + (bh * kR + s0) * kD)[tid];
      reinterpret_cast<uint4*>(fv)[tid] = reinterpret_cast<const uint4*>(
          ca.res_v + (bh * kD + (tid >> 2)) * kR + s0)[tid & 3];
      barrier_lds();
      float x[32];
      uint32_t cw[2];
      if (tid < kD) {
        // Key channel tid over the block's 32 window tokens
#pragma unroll
        for (int t = 0; t < 32; ++t) x[t] = f16_to_f32(fk[t * kD + tid]);
        const Range r = range32(x);
        reinterpret_cast<uint16_t*>(rec + kRecKDelta)[tid] = f32_to_f16(r.delta);
        reinterpret_cast<uint16_t*>(rec + kRecKZero)[tid] = static_cast<uint16_t>(r.zm);
        codes32(x, r, cw);
        img_k[tid] = cw[0];
        img_k[kD + tid] = cw[1];
      } else if (tid < 2 * kD) {
        // Value (token t, group g) over 32 channels; slot fastest across lanes
        const int u = tid - kD, t = u & 31, g = u >> 5;
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = f16_to_f32(fv[(32 * g + i) * 32 + t]);
        const Range r = range32(x);
        reinterpret_cast<uint32_t*>(rec + kRecVParam)[32 * g + t] =
            static_cast<uint32_t>(f32_to_f16(r.delta)) | (r.zm << 16);
        codes32(x, r, cw);
        *reinterpret_cast<uint2*>(img_v + g * kVImgRow + 2 * t) = uint2{cw[0], cw[1]};
      }
      barrier_lds();
      if (tid < 256) {
        const int t = tid >> 3, j = tid & 7;  // Key word j of token t
        *reinterpret_cast<uint32_t*>(rec + kRecKCodes + 32 * t + 4 * j) = key_word(img_k, t, j);
      } else {
        const int w = tid - 256, oct = (w >> 6) & 3, m = (w >> 2) & 15, d = w & 3;
        *reinterpret_cast<uint32_t*>(rec + kRecVCodes + 16 * (16 * oct + m) + 4 * d) =
            value_word(img_v, oct, m, d);
      }
      barrier_lds();  // the next block reuses the images
    }
    Q += kG * nfb;
  }

  // Rotate + scale the new token; head h goes to slot n % 128.
  const int slot = n % kR;
  float a[2], bb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hh = wave + 8 * j;
    a[j] = bb[j] = 0.0f;
    if (hh < hkv) {
      a[j] = in_to_f32(kin[j][0], is_bf16);
      bb[j] = in_to_f32(kin[j][1], is_bf16);
      if (ca.rope) {  // the new token sits at position n
        const float2 cs = reinterpret_cast<const float2*>(ca.rope)[static_cast<size_t>(n) * 64 + lane];
        rope_pair(a[j], bb[j], cs.x, cs.y);
      }
      fht128_wave(a[j], bb[j]);
      const float hs = wave_tree_sumsq(a[j], bb[j]);
      if (lane == 0) part[hh] = hs;
    }
  }
  barrier_lds();
  if (wave == (h & 7)) {
    // head h's rotated values: register set h / 8 of this wave
    const float ya = h >= 8 ? a[1] : a[0], yb = h >= 8 ? bb[1] : bb[0];
    float nrm, r;
    // TOKEN: the tree over all heads; HEAD: the head's own (within-head) tree
    scale_from_ss(ca.head_norm ? part[h] : tree16(part, hkv), nrm, r, ca.hw_rsq != 0);
    uint16_t* rk = ca.res_k + (bh * kR + slot) * kD;
    rk[lane] = f32_to_f16(mul_rn(ya, r));
    rk[lane + 64] = f32_to_f16(mul_rn(yb, r));
    if (lane == 0 && (ca.head_norm || h == 0)) ca.res_norm[res_norm_at(ca, b, h, slot)] = f32_to_f16_sat(nrm);
  }
  if (tid < kD) ca.res_v[(bh * kD + tid) * kR + slot] = f32_to_f16_sat(in_to_f32(vin, is_bf16));
  // the last of the sequence's workgroups to count itself in writes the new
  // state and resets the counter
  if (tid == 0 && prev == hkv - 1) {
    st[0] = n + 1;
    st[1] = Q;
    __hip_atomic_store(ca.append_sync + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- prefill
// grid nb + nr, NT threads: workgroup j < nb turns tokens 32j..32j+31 (all
// KV heads) into block j; workgroup nb + c writes window chunk c (tokens
// Q + 32c ..) without quantizing.  The last workgroup to finish (arrival
// counter append_sync[seq]) writes {n, Q}.  Barriers order LDS only, so the
// Value loads issued before the Key ranges stay in flight across them.
//
// Rotation: four lanes per (token, head) vector, lane tq holding elements
// 32 tq .. 32 tq + 31; butterflies with strides 1..16 are in registers,
// strides 32 and 64 exchange within the lane quad -- the oracle's stages in
// the oracle's order.  The sum of squares follows the same tree (strides
// 1..16 in registers, 32 and 64 across the quad, then over the heads).
// Quantization without atomics: the thread that takes a range (Key: head,
// channel over the 32 tokens; Value: token, head, 32-channel group) holds its
// 32 values and computes their codes at once, into an LDS image of 32-bit
// words of 16 codes; whole code words of the record are then assembled from
// that image (Key: one word = 16 channels of one token; Value: one word = 8
// tokens x 2 channels).
// Dynamic LDS: k_hat [Hkv][32][128] fp16, the 16-byte chunks of token t's
// row permuted by chunk ^ (t & 3) so that a wave's chunk writes (four lanes
// per row, 16 consecutive rows) fall in distinct banks; channel c of token t
// sits at element c ^ 8 (t & 3).  (The Value image reuses it once the
// Key ranges are done), then the Key image [Hkv][2][128] words (the rotation
// phase borrows it for the per-head sums and per-token factors).
size_t prefill_lds_bytes(int hkv) {
  return static_cast<size_t>(hkv) * (32 * kD * 2 + 2 * kD * 4);
}


// NT threads: 512 for Hkv <= 8 (two workgroups share a CU, so that one's
// loads overlap the other's arithmetic), 1024 above.  Four waves per SIMD
// either way (at most 128 registers).
// BF16: the input type (bf16 or fp16) as a compile-time choice; ROPE: the
// Keys are rotated by position before the FHT (ca.rope non-null).
template <int NT, int BF16, int ROPE>
__device__ __forceinline__ void prefill_unit(const CacheArgs& ca, int seq,
                                             const uint16_t* __restrict__ k,
                                             const uint16_t* __restrict__ v, int n_tokens,
                                             int Qn) {
  constexpr int is_bf16 = BF16;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  const int hkv = ca.hkv;
  uint16_t* khs = reinterpret_cast<uint16_t*>(dyn);                      // [hkv][32][128]
  uint32_t* img_v = reinterpret_cast<uint32_t*>(dyn);                    // [hkv][kVImgHead]
  uint8_t* prm = dyn + static_cast<size_t>(32) * hkv * kD * 2;
  uint32_t* img_k = reinterpret_cast<uint32_t*>(prm);                    // [hkv][2][128]
  float* part = reinterpret_cast<float*>(prm);                          // rotation phase: [32][hkv]
  float* tok_r = part + 32 * hkv;                          // [32] or [32][hkv] (HEAD)

  const int nb = Qn / kG;
  const bool ring = static_cast<int>(blockIdx.x) >= nb;
  const int t0 = ring ? Qn + 32 * (blockIdx.x - nb) : 32 * blockIdx.x;
  const int tid = threadIdx.x;
  const size_t row = static_cast<size_t>(hkv) * kD;
  const int p = ring ? 0 : ca.block_table[static_cast<size_t>(seq) * ca.max_blocks + blockIdx.x];
  if (p < 0 || p >= ca.nphys) {
    if (threadIdx.x == 0) atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    return;
  }
  auto rec_of = [&](int h) { return ca.pool + (static_cast<size_t>(p) * hkv + h) * kRec; };

  // ---- rotation and sums of squares (32 Hkv vectors, four lanes each: one
  // or two rounds of NT threads).  Vector (head h, token t) is 32 h + t.
  const int nvec = 32 * hkv;
  float y[2][32];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int task = rr * NT + tid;
    const int vtx = task >> 2, tq = task & 3;
    if (rr * NT >= nvec * 4) break;  // uniform
    const int t = vtx & 31, h = vtx >> 5;
    const bool valid = vtx < nvec && t0 + t < n_tokens;
    float* x = y[rr];
    if (valid) {
      const uint16_t* src = k + static_cast<size_t>(t0 + t) * row + h * kD + 32 * tq;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 w = reinterpret_cast<const uint4*>(src)[q];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * q + 2 * e] = in_to_f32(static_cast<uint16_t>(ww[e]), is_bf16);
          x[8 * q + 2 * e + 1] = in_to_f32(static_cast<uint16_t>(ww[e] >> 16), is_bf16);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) x[j] = 0.0f;
    }
    if constexpr (ROPE != 0) rope_quad(x, tq, ca.rope, t0 + t, valid);
    const float ssum = fht_quad(x, tq);
    if (tq == 0 && vtx < nvec) part[t * hkv + h] = ssum;
  }
  barrier_lds();
  // one factor per token (TOKEN: tree over the heads) or per (token, head)
  // (HEAD: the head's own tree); NT >= 32 * 16
  if (tid < 32 * (ca.head_norm ? hkv : 1)) {
    const int tl = ca.head_norm ? tid / hkv : tid, h = ca.head_norm ? tid % hkv : 0;
    float nrm, r;
    scale_from_ss(ca.head_norm ? part[tid] : tree16(part + tid * hkv, hkv), nrm, r, ca.hw_rsq != 0);
    tok_r[tid] = r;
    const int t = t0 + tl;
    if (t < n_tokens) {
      if (ring)
        ca.res_norm[res_norm_at(ca, seq, h, t % kR)] = f32_to_f16_sat(nrm);
      else
        ca.pool_norm[pool_norm_at(ca, p, h, tl)] = f32_to_f16_sat(nrm);
    }
  }
  barrier_lds();
  // ---- scaled Keys (and, for a window chunk, fp16 Values) to LDS or the ring
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int task = rr * NT + tid;
    const int vtx = task >> 2, tq = task & 3;
    if (rr * NT >= nvec * 4) break;
    const int t = vtx & 31, h = vtx >> 5;
    if (vtx < nvec && t0 + t < n_tokens) {
      const float r = tok_r[ca.head_norm ? t * hkv + h : t];
      uint32_t kw[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) kw[e] = f32x2_to_f16x2(mul_rn(y[rr][2 * e], r), mul_rn(y[rr][2 * e + 1], r));
      uint4* dst;
      if (ring) {
        const int slot = (t0 + t) % kR;
        const size_t bh = static_cast<size_t>(seq) * hkv + h;
        dst = reinterpret_cast<uint4*>(ca.res_k + (bh * kR + slot) * kD + 32 * tq);
        const uint16_t* vs = v + static_cast<size_t>(t0 + t) * row + h * kD + 32 * tq;
        uint16_t* rv = ca.res_v + bh * kD * kR + slot;
#pragma unroll
        for (int j = 0; j < 32; ++j)
          rv[static_cast<size_t>(32 * tq + j) * kR] = f32_to_f16_sat(in_to_f32(vs[j], is_bf16));
      } else {
        dst = reinterpret_cast<uint4*>(khs + (h * 32 + t) * kD + 32 * tq);
      }
      const int sw = ring ? 0 : (t & 3);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q ^ sw] = uint4{kw[4 * q], kw[4 * q + 1], kw[4 * q + 2], kw[4 * q + 3]};
    }
  }
  if (ring) return;
  barrier_lds();

  // ---- Key ranges and codes: unit (head, channel) over the 32 tokens
  for (int u = tid; u < hkv * kD; u += NT) {
    const int h = u >> 7, c = u & 127;
    const _Float16* kh = reinterpret_cast<const _Float16*>(khs) + h * 32 * kD;
    const _Float16* kc[4] = {kh + c, kh + (c ^ 8), kh + (c ^ 16), kh + (c ^ 24)};  // by t & 3
    half2_t xp[16];  // tokens 2i, 2i + 1
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xp[i].x = kc[(2 * i) & 3][(2 * i) * kD];
      xp[i].y = kc[(2 * i + 1) & 3][(2 * i + 1) * kD];
    }
    const Range r = range32_pk(xp);
    uint8_t* rec = rec_of(h);
    reinterpret_cast<uint16_t*>(rec + kRecKDelta)[c] = f32_to_f16(r.delta);
    reinterpret_cast<uint16_t*>(rec + kRecKZero)[c] = static_cast<uint16_t>(r.zm);
    uint32_t w[2];
    codes32_of([&xp](int i) { return static_cast<float>(i & 1 ? xp[i >> 1].y : xp[i >> 1].x); }, r, w);
    img_k[(2 * h) * kD + c] = w[0];      // tokens 0..15
    img_k[(2 * h + 1) * kD + c] = w[1];  // tokens 16..31
  }
  barrier_lds();  // k_hat is dead: its space takes the Value image

  // ---- Value ranges and codes: unit (token, head, group) over 32 channels
  // (at most two per thread: 32 Hkv 4 units over NT threads).  A unit's
  // inputs are requested just before it is processed.
  static_assert(32 * 16 * 4 <= 2 * 1024 && 32 * 8 * 4 <= 2 * 512, "two Value units per thread");
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = tid + NT * i;
    if (u >= 32 * hkv * 4) break;
    const int t = u / (hkv * 4), h = (u >> 2) % hkv, g = u & 3;
    const uint4* src = reinterpret_cast<const uint4*>(v + static_cast<size_t>(t0 + t) * row + h * kD + 32 * g);
    uint4 vraw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) vraw[q] = src[q];
    float x[32];  // the inputs as fp32 (exact)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w8 = vraw[q];
      const uint32_t ww[4] = {w8.x, w8.y, w8.z, w8.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[8 * q + e] = in_to_f32(static_cast<uint16_t>(ww[e >> 1] >> (16 * (e & 1))), is_bf16);
    }
    Range r;
    uint32_t w[2];
    const bool fast = range32_row(x, r) && codes32<true>(x, r, w);
    if (__ballot(!fast)) {  // uniform: a NaN or out-of-range input in some lane
      if (!fast) {
#pragma unroll
        for (int j = 0; j < 32; ++j) x[j] = f16_to_f32(f32_to_f16_sat(x[j]));
        r = range32(x);
        codes32(x, r, w);
      }
    }
    reinterpret_cast<uint32_t*>(rec_of(h) + kRecVParam)[32 * g + t] =
        static_cast<uint32_t>(f32_to_f16(r.delta)) | (r.zm << 16);
    *reinterpret_cast<uint2*>(img_v + h * kVImgHead + g * kVImgRow + 2 * t) = uint2{w[0], w[1]};
  }
  barrier_lds();

  // ---- code words, sixteen per thread by one 16 x 16 transpose of 2-bit
  // fields.  Key word (head, token t, j): channels 16 j .. 16 j + 15 of token
  // t, i.e. field (t & 15) of the image words of those 16 channels (token
  // half t >> 4).  Value word (head, octet, m, group d): field m of the
  // image words (w_e of token 8 octet + kk) for the 8 tokens and e = 0, 1,
  // at field 8 e + s(kk) (s: the record's token order within an octet).
  if (tid < hkv * 32) {
    uint32_t r[16];
    if (tid < hkv * 16) {
      const int h = tid >> 4, half = (tid >> 3) & 1, j = tid & 7;
      const uint4* src = reinterpret_cast<const uint4*>(img_k + (2 * h + half) * kD + 16 * j);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 w4 = src[q];
        r[4 * q] = w4.x;
        r[4 * q + 1] = w4.y;
        r[4 * q + 2] = w4.z;
        r[4 * q + 3] = w4.w;
      }
      transpose16x2(r);
      uint8_t* dst = rec_of(h) + kRecKCodes + 32 * (16 * half) + 4 * j;
#pragma unroll
      for (int f = 0; f < 16; ++f) *reinterpret_cast<uint32_t*>(dst + 32 * f) = r[f];
    } else {
      const int w = tid - hkv * 16, h = w >> 4, d = (w >> 2) & 3, oct = w & 3;
      const uint4* src = reinterpret_cast<const uint4*>(img_v + h * kVImgHead + d * kVImgRow + 16 * oct);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 w4 = src[q];  // tokens 2q, 2q + 1 of the octet, words e = 0, 1
        const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int kk = 2 * q + (f >> 1), e = f & 1;
          const int sk = (kk & 4) | ((kk & 1) << 1) | ((kk >> 1) & 1);
          r[8 * e + sk] = ww[f];
        }
      }
      transpose16x2(r);
      uint8_t* dst = rec_of(h) + kRecVCodes + 16 * (16 * oct) + 4 * d;
#pragma unroll
      for (int m = 0; m < 16; ++m) *reinterpret_cast<uint32_t*>(dst + 16 * m) = r[m];
    }
  }
}

template <int NT, int BF16, int ROPE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8)))
void prefill_kernel(CacheArgs ca, int seq, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, int n_tokens, int Qn) {
  // every workgroup reads {n} before any of them arrives below
  const bool nonempty = ca.seq_state[2 * seq] != 0;
  if (!nonempty)
    prefill_unit<NT, BF16, ROPE>(ca, seq, k, v, n_tokens, Qn);
  else if (blockIdx.x == 0 && threadIdx.x == 0)
    atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_NONEMPTY));
  // the last workgroup to finish writes {n, Q} (not if the sequence was not
  // empty) and leaves the arrival counter zero.  Every wave has used its
  // read of {n} (a branch) before the barrier, so no read can see the new
  // state; the writes need no ordering within the launch (they are read by
  // later launches), hence a relaxed counter and no cache write-back.
  barrier_lds();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(ca.append_sync + seq, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    if (old == static_cast<int>(gridDim.x) - 1) {
      __hip_atomic_store(ca.append_sync + seq, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!nonempty) {
        ca.seq_state[2 * seq] = n_tokens;
        ca.seq_state[2 * seq + 1] = Qn;
      }
    }
  }
}

CacheArgs make_args(const oscar_cache_geom* g, const oscar_cache* c) {
  CacheArgs a;
  a.pool = static_cast<uint8_t*>(c->pool);
  a.pool_norm = static_cast<uint16_t*>(c->pool_norm);
  a.res_k = static_cast<uint16_t*>(c->res_k);
  a.res_v = static_cast<uint16_t*>(c->res_v);
  a.res_norm = static_cast<uint16_t*>(c->res_norm);
  a.block_table = c->block_table;
  a.seq_state = c->seq_state;
  a.error_flag = c->error_flag;
  a.append_sync = c->append_sync;
  a.hkv = g->num_kv_heads;
  a.max_blocks = g->max_blocks_per_seq;
  a.nphys = g->num_physical_blocks;
  a.head_norm = g->norm_scope == OSCAR_NORM_HEAD ? 1 : 0;
  a.flush_blocks = g->flush_tokens == 128 ? 4 : 1;
  a.hw_rsq = g->key_scale == OSCAR_SCALE_HW_RSQ ? 1 : 0;
  a.rope = g->rope_max_pos > 0 ? c->rope : nullptr;
  a.rope_max_pos = g->rope_max_pos;
  return a;
}

}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_quant_pack(const void* khat16, const void* knorm16, const void* v16,
                                         int32_t n_blocks, int32_t n_kv_heads,
                                         oscar_norm_scope norm_scope, void* rec_out,
                                         void* norm_out, void* stream) {
  if (!khat16 || !knorm16 || !v16 || !rec_out || !norm_out) return OSCAR_EINVAL;
  if (n_blocks < 0 || n_kv_heads < 1 || n_kv_heads > 16) return OSCAR_EINVAL;
  if (norm_scope != OSCAR_NORM_TOKEN && norm_scope != OSCAR_NORM_HEAD) return OSCAR_EINVAL;
  if (!aligned(rec_out, 16) || !aligned(v16, 16)) return OSCAR_EINVAL;
  oscar_status st = check_device();
  if (st != OSCAR_OK) return st;
  if (n_blocks == 0) return OSCAR_OK;
  hipLaunchKernelGGL(quant_pack_kernel, dim3(n_blocks, n_kv_heads), dim3(256), 0,
                     as_stream(stream), static_cast<const uint16_t*>(khat16),
                     static_cast<const uint16_t*>(knorm16), static_cast<const uint16_t*>(v16),
                     static_cast<int>(n_kv_heads), norm_scope == OSCAR_NORM_HEAD ? 1 : 0,
                     static_cast<uint8_t*>(rec_out), static_cast<uint16_t*>(norm_out));
  return launch_status();
}

extern "C" oscar_status oscar_append_kv(const oscar_cache_geom* geom, const oscar_cache* cache,
                                        const void* k_new, const void* v_new, oscar_dtype dtype,
                                        void* stream) {
  oscar_status st = check_cache(geom, cache);
  if (st != OSCAR_OK) return st;
  if (!k_new || !v_new) return OSCAR_EINVAL;
  if (dtype != OSCAR_FP16 && dtype != OSCAR_BF16) return OSCAR_EINVAL;
  st = check_device();
  if (st != OSCAR_OK) return st;
  hipLaunchKernelGGL(append_kernel, dim3(geom->batch * geom->num_kv_heads), dim3(512), 0,
                     as_stream(stream),
                     make_args(geom, cache), static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), dtype == OSCAR_BF16 ? 1 : 0);
  return launch_status();
}

extern "C" oscar_status oscar_prefill_quantize(const oscar_cache_geom* geom,
                                               const oscar_cache* cache, int32_t seq,
                                               const void* k, const void* v, int32_t n_tokens,
                                               oscar_dtype dtype, void* stream) {
  oscar_status st = check_cache(geom, cache);
  if (st != OSCAR_OK) return st;
  if (!k || !v || n_tokens < 0 || seq < 0 || seq >= geom->batch) return OSCAR_EINVAL;
  if (!aligned(k, 16) || !aligned(v, 16)) return OSCAR_EINVAL;
  if (dtype != OSCAR_FP16 && dtype != OSCAR_BF16) return OSCAR_EINVAL;
  // The state n appends would leave: Q(n) = 32 * ceil(max(0, n - 128) / 32)
  // with one-block flushes, 128 * floor((n - 1) / 128) (n > 128) with
  // 128-token flushes.
  const int Qb = geom->flush_tokens == 128 ? (n_tokens > kR ? 4 * ((n_tokens - 1) / kR) : 0)
                                           : ((n_tokens > kR ? n_tokens - kR : 0) + 31) / 32;
  if (Qb > geom->max_blocks_per_seq) return OSCAR_EINVAL;
  // positions 0 .. n_tokens - 1 must all have a (cos, sin) row
  if (geom->rope_max_pos > 0 && n_tokens > geom->rope_max_pos) return OSCAR_EINVAL;
  st = check_device();
  if (st != OSCAR_OK) return st;
  if (n_tokens == 0) return OSCAR_OK;
  const int Q = 32 * Qb;
  const int nr = (n_tokens - Q + 31) / 32;
  const size_t lds = prefill_lds_bytes(geom->num_kv_heads);
  auto launch = [&](auto kernel, int nt) {
    if (lds > 64 * 1024)
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    hipLaunchKernelGGL(kernel, dim3(Qb + nr), dim3(nt), lds, as_stream(stream),
                       make_args(geom, cache), static_cast<int>(seq),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                       static_cast<int>(n_tokens), Q);
  };
  const bool bf16 = dtype == OSCAR_BF16, rope = geom->rope_max_pos > 0;
  if (geom->num_kv_heads <= 8) {
    if (rope)
      bf16 ? launch(&prefill_kernel<512, 1, 1>, 512) : launch(&prefill_kernel<512, 0, 1>, 512);
    else
      bf16 ? launch(&prefill_kernel<512, 1, 0>, 512) : launch(&prefill_kernel<512, 0, 0>, 512);
  } else {
    if (rope)
      bf16 ? launch(&prefill_kernel<1024, 1, 1>, 1024) : launch(&prefill_kernel<1024, 0, 1>, 1024);
    else
      bf16 ? launch(&prefill_kernel<1024, 1, 0>, 1024) : launch(&prefill_kernel<1024, 0, 0>, 1024);
  }
  return launch_status();
}
