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

namespace oscar {

// Record quantization by one group of 256 threads.  Thread tg < 128 takes
// Key channel tg (32 tokens); thread tg >= 128 takes Value (token, group)
// unit tg - 128.  Codes are OR-ed into the LDS image `img` (512 words: Key
// codes then Value codes), steps and zero points go straight to `rec`.
template <class KGet, class VGet>
__device__ __forceinline__ void quant_record_units(int tg, KGet kget, VGet vget, uint32_t* img,
                                                   uint8_t* rec) {
  float x[32];
  float d, z;
  if (tg < 128) {
    const int c = tg;
#pragma unroll
    for (int t = 0; t < 32; ++t) x[t] = f16_to_f32(kget(t, c));
    const uint64_t codes = quant32(x, d, z);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int bit = kcode_bitpos(t, c);
      atomicOr(&img[bit >> 5], static_cast<uint32_t>((codes >> (2 * t)) & 3u) << (bit & 31));
    }
    reinterpret_cast<uint16_t*>(rec + kRecKDelta)[c] = f32_to_f16(d);
    reinterpret_cast<uint16_t*>(rec + kRecKZero)[c] = f32_to_f16(z);
  } else {
    const int u = tg - 128, t = u >> 2, g = u & 3;
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = f16_to_f32(vget(t, 32 * g + i));
    const uint64_t codes = quant32(x, d, z);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int bit = vcode_bitpos(t, 32 * g + i);
      atomicOr(&img[256 + (bit >> 5)], static_cast<uint32_t>((codes >> (2 * i)) & 3u) << (bit & 31));
    }
    reinterpret_cast<uint32_t*>(rec + kRecVParam)[32 * g + t] =
        static_cast<uint32_t>(f32_to_f16(d)) | (static_cast<uint32_t>(f32_to_f16(z)) << 16);
  }
}

__device__ __forceinline__ void copy_codes_out(int tg, const uint32_t* img, uint8_t* rec) {
  if (tg < 128)
    reinterpret_cast<uint4*>(rec)[tg] = reinterpret_cast<const uint4*>(img)[tg];
}

// ---------------------------------------------------------------- quant_pack
// grid (n_blocks, Hkv), 256 threads.
__global__ __launch_bounds__(256) void quant_pack_kernel(const uint16_t* __restrict__ khat,
                                                         const uint16_t* __restrict__ knorm,
                                                         const uint16_t* __restrict__ v16,
                                                         int hkv, uint8_t* __restrict__ rec_out,
                                                         uint16_t* __restrict__ norm_out) {
  __shared__ uint32_t img[512];
  const int j = blockIdx.x, h = blockIdx.y, tg = threadIdx.x;
  for (int i = tg; i < 512; i += 256) img[i] = 0;
  __syncthreads();
  const size_t row = static_cast<size_t>(hkv) * kD;
  const uint16_t* kb = khat + static_cast<size_t>(32 * j) * row + static_cast<size_t>(h) * kD;
  const uint16_t* vb = v16 + static_cast<size_t>(32 * j) * row + static_cast<size_t>(h) * kD;
  uint8_t* rec = rec_out + (static_cast<size_t>(j) * hkv + h) * kRec;
  quant_record_units(
      tg, [&](int t, int c) { return kb[t * row + c]; },
      [&](int t, int c) { return vb[t * row + c]; }, img, rec);
  __syncthreads();
  copy_codes_out(tg, img, rec);
  if (h == 0 && tg < 32) norm_out[static_cast<size_t>(j) * 32 + tg] = knorm[32 * j + tg];
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
  int hkv;
  int max_blocks;
  int nphys;
};

// {n, Q} as the kernels leave it: 0 <= Q, Q % 32 == 0, 0 <= n - Q <= 128,
// Q / 32 <= max_blocks.
__device__ __forceinline__ bool state_ok(int n, int Q, int max_blocks) {
  return Q >= 0 && (Q & 31) == 0 && n >= Q && n - Q <= kR && Q / kG <= max_blocks;
}

// grid B, block max(256, 64*Hkv) rounded up to a multiple of 256.
__global__ __launch_bounds__(1024) void append_kernel(CacheArgs ca, const uint16_t* __restrict__ k_new,
                                                      const uint16_t* __restrict__ v_new,
                                                      int is_bf16) {
  __shared__ uint32_t img[4][512];
  __shared__ float part[16];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int grp = tid >> 8, tg = tid & 255, ngrp = blockDim.x >> 8;
  const int hkv = ca.hkv;
  int32_t* st = ca.seq_state + 2 * b;
  const int n = st[0];
  int Q = st[1];
  if (!state_ok(n, Q, ca.max_blocks)) {
    if (tid == 0) atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    return;
  }

  if (n - Q == kR) {
    // The window is full: its 32 oldest tokens become block Q/32.
    const int j = Q / kG;
    if (j >= ca.max_blocks) {
      if (tid == 0) atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_CAPACITY));
      return;
    }
    const int p = ca.block_table[static_cast<size_t>(b) * ca.max_blocks + j];
    if (p < 0 || p >= ca.nphys) {
      if (tid == 0) atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
      return;
    }
    const int s0 = Q % kR;
    if (tid < 32) ca.pool_norm[static_cast<size_t>(p) * 32 + tid] = ca.res_norm[b * kR + s0 + tid];
    for (int h0 = 0; h0 < hkv; h0 += ngrp) {
      const int h = h0 + grp;
      for (int i = tg; i < 512; i += 256) img[grp][i] = 0;
      __syncthreads();
      uint8_t* rec = ca.pool + (static_cast<size_t>(p) * hkv + h) * kRec;
      if (h < hkv) {
        const uint16_t* rk = ca.res_k + ((static_cast<size_t>(b) * hkv + h) * kR + s0) * kD;
        const uint16_t* rv = ca.res_v + (static_cast<size_t>(b) * hkv + h) * kD * kR + s0;
        quant_record_units(
            tg, [&](int t, int c) { return rk[t * kD + c]; },
            [&](int t, int c) { return rv[c * kR + t]; }, img[grp], rec);
      }
      __syncthreads();
      if (h < hkv) copy_codes_out(tg, img[grp], rec);
      __syncthreads();
    }
    Q += kG;
  }

  // Rotate + scale the new token; store it in slot n % 128.
  const int slot = n % kR;
  const int h = tid >> 6, lane = tid & 63;
  float a = 0.0f, bb = 0.0f;
  if (h < hkv) {
    const size_t base = (static_cast<size_t>(b) * hkv + h) * kD;
    a = in_to_f32(k_new[base + lane], is_bf16);
    bb = in_to_f32(k_new[base + lane + 64], is_bf16);
    fht128_wave(a, bb);
    const float hs = wave_tree_sumsq(a, bb);
    if (lane == 0) part[h] = hs;
  }
  __syncthreads();
  if (h < hkv) {
    float nrm, r;
    scale_from_ss(tree16(part, hkv), nrm, r);
    const size_t bh = static_cast<size_t>(b) * hkv + h;
    uint16_t* rk = ca.res_k + (bh * kR + slot) * kD;
    rk[lane] = f32_to_f16(mul_rn(a, r));
    rk[lane + 64] = f32_to_f16(mul_rn(bb, r));
    const size_t base = bh * kD;
    uint16_t* rv = ca.res_v + bh * kD * kR + slot;
    rv[static_cast<size_t>(lane) * kR] = f32_to_f16(in_to_f32(v_new[base + lane], is_bf16));
    rv[static_cast<size_t>(lane + 64) * kR] = f32_to_f16(in_to_f32(v_new[base + lane + 64], is_bf16));
    if (h == 0 && lane == 0) ca.res_norm[b * kR + slot] = f32_to_f16(nrm);
  }
  if (tid == 0) {
    st[0] = n + 1;
    st[1] = Q;
  }
}

// ---------------------------------------------------------------- prefill
// Lane-parallel INT2 quantizer: the 32 values of a group sit one per lane in
// a 32-lane half-wave.  Same arithmetic as quant32 (min and max do not depend
// on the order once a zero is canonicalised to +0).
__device__ __forceinline__ int quant_lane32(float x, float& d, float& z) {
#pragma clang fp contract(off)
  float mn = x, mx = x;
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, s, 64));
    mx = fmaxf(mx, __shfl_xor(mx, s, 64));
  }
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  d = __fdiv_rn(mx - mn, 3.0f);
  z = mn;
  int q = 0;
  if (d > 0.0f) {
    const float r = rintf(__fdiv_rn(x - mn, d));
    q = r < 0.0f ? 0 : (r > 3.0f ? 3 : static_cast<int>(r));
  }
  return q;
}

// grid nb + nr: block j < nb quantizes tokens 32j..32j+31 (all KV heads);
// block nb + c writes ring chunk c (tokens Q + 32c ..) without quantizing.
// 256 threads.  Dynamic LDS: k_hat [32][Hkv][128] fp16 + images [Hkv][512].
__global__ __launch_bounds__(256) void prefill_kernel(CacheArgs ca, int seq,
                                                      const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v,
                                                      int n_tokens, int Qn, int is_bf16) {
  extern __shared__ uint32_t dyn[];
  const int hkv = ca.hkv;
  uint16_t* khs = reinterpret_cast<uint16_t*>(dyn);         // [32][hkv][128]
  uint32_t* imgs = dyn + 32 * hkv * kD / 2;                   // [hkv][512]
  __shared__ float nrm_s[32];
  if (ca.seq_state[2 * seq] != 0) {
    if (blockIdx.x == 0 && threadIdx.x == 0)
      atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_NONEMPTY));
    return;
  }
  const int nb = Qn / kG;
  const bool ring = static_cast<int>(blockIdx.x) >= nb;
  const int t0 = ring ? Qn + 32 * (blockIdx.x - nb) : 32 * blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const size_t row = static_cast<size_t>(hkv) * kD;
  const int p = ring ? 0 : ca.block_table[static_cast<size_t>(seq) * ca.max_blocks + blockIdx.x];
  if (p < 0 || p >= ca.nphys) {
    if (threadIdx.x == 0) atomicOr(ca.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    return;
  }

  if (!ring) {
    for (int i = tid; i < hkv * 512; i += 256) imgs[i] = 0;
    __syncthreads();
  }
  // Token phase: wave w takes tokens w, w+4, ...: rotate + scale every head
  // of the token, then (quantized blocks) Value quantization per token.
  for (int tt = wave; tt < 32; tt += 4) {
    const int t = t0 + tt;
    if (t >= n_tokens) break;  // ring chunk tail; uniform per wave
    float ya[16], yb[16];
    float part[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      part[h] = 0.0f;
      if (h < hkv) {
        const size_t base = static_cast<size_t>(t) * row + h * kD;
        float a = in_to_f32(k[base + lane], is_bf16);
        float b = in_to_f32(k[base + lane + 64], is_bf16);
        fht128_wave(a, b);
        part[h] = wave_tree_sumsq(a, b);
        ya[h] = a;
        yb[h] = b;
      }
    }
    float nrm, r;
    scale_from_ss(tree16(part, hkv), nrm, r);
    const int slot = t % kR;
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      if (h < hkv) {
        const uint16_t ka = f32_to_f16(mul_rn(ya[h], r)), kb = f32_to_f16(mul_rn(yb[h], r));
        const size_t base = static_cast<size_t>(t) * row + h * kD;
        const uint16_t va = f32_to_f16(in_to_f32(v[base + lane], is_bf16));
        const uint16_t vb = f32_to_f16(in_to_f32(v[base + lane + 64], is_bf16));
        if (ring) {
          const size_t bh = static_cast<size_t>(seq) * hkv + h;
          uint16_t* rk = ca.res_k + (bh * kR + slot) * kD;
          rk[lane] = ka;
          rk[lane + 64] = kb;
          uint16_t* rv = ca.res_v + bh * kD * kR + slot;
          rv[static_cast<size_t>(lane) * kR] = va;
          rv[static_cast<size_t>(lane + 64) * kR] = vb;
        } else {
          khs[(tt * hkv + h) * kD + lane] = ka;
          khs[(tt * hkv + h) * kD + lane + 64] = kb;
          // Value groups: lanes 0..31 / 32..63 of register a are groups 0 / 1,
          // of register b groups 2 / 3.
          float da, za, db, zb;
          const int qa = quant_lane32(f16_to_f32(va), da, za);
          const int qb = quant_lane32(f16_to_f32(vb), db, zb);
          uint32_t* img = imgs + h * 512 + 256;
          const int bita = vcode_bitpos(tt, lane), bitb = vcode_bitpos(tt, lane + 64);
          atomicOr(&img[bita >> 5], static_cast<uint32_t>(qa) << (bita & 31));
          atomicOr(&img[bitb >> 5], static_cast<uint32_t>(qb) << (bitb & 31));
          uint8_t* rec = ca.pool + (static_cast<size_t>(p) * hkv + h) * kRec;
          uint32_t* vp = reinterpret_cast<uint32_t*>(rec + kRecVParam);
          if ((lane & 31) == 0) {
            const int g = lane >> 5;
            vp[32 * g + tt] = static_cast<uint32_t>(f32_to_f16(da)) |
                             (static_cast<uint32_t>(f32_to_f16(za)) << 16);
            vp[32 * (2 + g) + tt] = static_cast<uint32_t>(f32_to_f16(db)) |
                                 (static_cast<uint32_t>(f32_to_f16(zb)) << 16);
          }
        }
      }
    }
    if (lane == 0) {
      if (ring)
        ca.res_norm[seq * kR + slot] = f32_to_f16(nrm);
      else
        nrm_s[tt] = nrm;
    }
  }
  if (ring) return;
  __syncthreads();
  if (tid < 32) ca.pool_norm[static_cast<size_t>(p) * 32 + tid] = f32_to_f16(nrm_s[tid]);
  // Key quantization: per (head, channel) over the block's 32 tokens.
  for (int u = tid; u < hkv * kD; u += 256) {
    const int h = u >> 7, c = u & 127;
    float x[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) x[t] = f16_to_f32(khs[(t * hkv + h) * kD + c]);
    float d, z;
    const uint64_t codes = quant32(x, d, z);
    uint32_t* img = imgs + h * 512;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int bit = kcode_bitpos(t, c);
      atomicOr(&img[bit >> 5], static_cast<uint32_t>((codes >> (2 * t)) & 3u) << (bit & 31));
    }
    uint8_t* rec = ca.pool + (static_cast<size_t>(p) * hkv + h) * kRec;
    reinterpret_cast<uint16_t*>(rec + kRecKDelta)[c] = f32_to_f16(d);
    reinterpret_cast<uint16_t*>(rec + kRecKZero)[c] = f32_to_f16(z);
  }
  __syncthreads();
  for (int i = tid; i < hkv * 128; i += 256) {
    const int h = i >> 7, q = i & 127;
    uint8_t* rec = ca.pool + (static_cast<size_t>(p) * hkv + h) * kRec;
    reinterpret_cast<uint4*>(rec)[q] = reinterpret_cast<const uint4*>(imgs + h * 512)[q];
  }
}

__global__ void prefill_finish_kernel(int32_t* seq_state, int seq, int n_tokens, int Qn) {
  if (threadIdx.x == 0 && seq_state[2 * seq] == 0) {
    seq_state[2 * seq] = n_tokens;
    seq_state[2 * seq + 1] = Qn;
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
  a.hkv = g->num_kv_heads;
  a.max_blocks = g->max_blocks_per_seq;
  a.nphys = g->num_physical_blocks;
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
  if (norm_scope == OSCAR_NORM_HEAD) return OSCAR_EUNSUPPORTED;
  if (norm_scope != OSCAR_NORM_TOKEN) return OSCAR_EINVAL;
  if (!aligned(rec_out, 16)) return OSCAR_EINVAL;
  oscar_status st = check_device();
  if (st != OSCAR_OK) return st;
  if (n_blocks == 0) return OSCAR_OK;
  hipLaunchKernelGGL(quant_pack_kernel, dim3(n_blocks, n_kv_heads), dim3(256), 0,
                     as_stream(stream), static_cast<const uint16_t*>(khat16),
                     static_cast<const uint16_t*>(knorm16), static_cast<const uint16_t*>(v16),
                     static_cast<int>(n_kv_heads), static_cast<uint8_t*>(rec_out),
                     static_cast<uint16_t*>(norm_out));
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
  const int threads = ((64 * geom->num_kv_heads + 255) / 256) * 256;
  hipLaunchKernelGGL(append_kernel, dim3(geom->batch), dim3(threads), 0, as_stream(stream),
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
  if (dtype != OSCAR_FP16 && dtype != OSCAR_BF16) return OSCAR_EINVAL;
  // Q(n) = 32 * ceil(max(0, n - 128) / 32): the state n appends would leave.
  const int Qb = ((n_tokens > kR ? n_tokens - kR : 0) + 31) / 32;
  if (Qb > geom->max_blocks_per_seq) return OSCAR_EINVAL;
  st = check_device();
  if (st != OSCAR_OK) return st;
  if (n_tokens == 0) return OSCAR_OK;
  const int Q = 32 * Qb;
  const int nr = (n_tokens - Q + 31) / 32;
  const size_t lds = static_cast<size_t>(32) * geom->num_kv_heads * kD * sizeof(uint16_t) +
                     static_cast<size_t>(geom->num_kv_heads) * 512 * sizeof(uint32_t);
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  hipLaunchKernelGGL(prefill_kernel, dim3(Qb + nr), dim3(256), lds, as_stream(stream),
                     make_args(geom, cache), static_cast<int>(seq),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<int>(n_tokens), Q, dtype == OSCAR_BF16 ? 1 : 0);
  st = launch_status();
  if (st != OSCAR_OK) return st;
  hipLaunchKernelGGL(prefill_finish_kernel, dim3(1), dim3(64), 0, as_stream(stream),
                     cache->seq_state, static_cast<int>(seq), static_cast<int>(n_tokens), Q);
  return launch_status();
}
