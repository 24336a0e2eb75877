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
  int32_t* error_flag;
  float2* ws_ml;  // [B][Hq][S] (m, l)
  float* ws_o;    // [B][Hq][S][128]
};

// Rotated query heads of KV head h into qs[GRP][128] (fp32).
template <int GRP>
__device__ __forceinline__ void load_rotated_q(const AttnArgs& A, int b, int h, float* qs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
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

  load_rotated_q<GRP>(A, b, h, qs);
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
      else if (tid < 196) stage[tid] = reinterpret_cast<const uint4*>(A.pool_norm + static_cast<size_t>(p) * 32)[tid - 192];
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
        const float nt = f16_to_f32(A.res_norm[static_cast<size_t>(b) * kR + s0 + (t < t_valid ? t : 0)]);
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
            const uint32_t pz = st32[kRecVParam / 4 + 4 * t + g];
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

// ---------------------------------------------------------------- reduce
// grid (Hq, B), 128 threads: merge the S partials of one query head.
__global__ __launch_bounds__(128) void lse_reduce_kernel(const float2* __restrict__ ws_ml,
                                                         const float* __restrict__ ws_o, int hq,
                                                         int splits, float* __restrict__ out,
                                                         float* __restrict__ lse) {
  const int i = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const size_t base = (static_cast<size_t>(b) * hq + i) * splits;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ws_ml[base + s].x);
  float L = 0.0f, acc = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float2 ml = ws_ml[base + s];
      if (ml.x == -INFINITY) continue;
      const float w = exp2f(ml.x - M);
      L += w * ml.y;
      acc += w * ws_o[(base + s) * kD + c];
    }
  }
  out[(static_cast<size_t>(b) * hq + i) * kD + c] = M == -INFINITY ? 0.0f : acc / L;
  if (lse && c == 0)
    lse[static_cast<size_t>(b) * hq + i] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * 0.6931471805599453f;
}

int auto_splits(const oscar_cache_geom* g, int max_ctx) {
  const int units = (max_ctx + kG - 1) / kG + 1;
  const int pairs = g->batch * g->num_kv_heads;
  int s = (2048 + pairs - 1) / pairs;
  const int cap = units / 8 > 1 ? units / 8 : 1;
  if (s > cap) s = cap;
  if (s > 1024) s = 1024;
  return s < 1 ? 1 : s;
}

size_t workspace_bytes(const oscar_cache_geom* g, int splits) {
  const size_t n = static_cast<size_t>(g->batch) * g->num_q_heads * splits;
  return n * sizeof(float2) + n * kD * sizeof(float) + 256;
}

template <int GRP>
void launch_valu(const AttnArgs& A, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL(attn_valu_kernel<GRP>, grid, dim3(256), 0, st, A);
}

}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_decode_workspace_bytes(const oscar_cache_geom* geom, int32_t max_ctx,
                                                     int32_t num_splits, int32_t* splits_out,
                                                     size_t* bytes) {
  oscar_status st = check_geom(geom);
  if (st != OSCAR_OK) return st;
  if (!bytes || max_ctx < 0 || num_splits < 0 || num_splits > 1024) return OSCAR_EINVAL;
  const int s = num_splits ? num_splits : auto_splits(geom, max_ctx);
  if (splits_out) *splits_out = s;
  *bytes = workspace_bytes(geom, s);
  return OSCAR_OK;
}

extern "C" oscar_status oscar_decode_attn(const oscar_cache_geom* geom, const oscar_cache* cache,
                                          const void* q, oscar_dtype q_dtype, float* out,
                                          float* lse, void* workspace, size_t ws_bytes,
                                          int32_t num_splits, int32_t max_ctx,
                                          oscar_attn_variant variant, void* stream) {
  oscar_status st = check_cache(geom, cache);
  if (st != OSCAR_OK) return st;
  if (!q || !out || !workspace || max_ctx < 0 || num_splits < 0 || num_splits > 1024)
    return OSCAR_EINVAL;
  if (q_dtype != OSCAR_FP16 && q_dtype != OSCAR_BF16 && q_dtype != OSCAR_FP32) return OSCAR_EINVAL;
  if (!aligned(workspace, 256) || !aligned(q, 4) || !aligned(out, 16)) return OSCAR_EINVAL;
  if (variant != OSCAR_ATTN_AUTO && variant != OSCAR_ATTN_VALU && variant != OSCAR_ATTN_MFMA)
    return OSCAR_EINVAL;
  const int S = num_splits ? num_splits : auto_splits(geom, max_ctx);
  if (ws_bytes < workspace_bytes(geom, S)) return OSCAR_EWORKSPACE;
  st = check_device();
  if (st != OSCAR_OK) return st;

  AttnArgs A;
  A.pool = static_cast<const uint8_t*>(cache->pool);
  A.pool_norm = static_cast<const uint16_t*>(cache->pool_norm);
  A.res_k = static_cast<const uint16_t*>(cache->res_k);
  A.res_v = static_cast<const uint16_t*>(cache->res_v);
  A.res_norm = static_cast<const uint16_t*>(cache->res_norm);
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
  A.ws_ml = static_cast<float2*>(workspace);
  A.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    ((npart * sizeof(float2) + 255) / 256) * 256);
  const dim3 grid(S, geom->num_kv_heads, geom->batch);
  hipStream_t hs = as_stream(stream);
  const int grp = geom->num_q_heads / geom->num_kv_heads;
  (void)variant;
  switch (grp) {
    case 1: launch_valu<1>(A, grid, hs); break;
    case 2: launch_valu<2>(A, grid, hs); break;
    case 4: launch_valu<4>(A, grid, hs); break;
    default: launch_valu<8>(A, grid, hs); break;
  }
  st = launch_status();
  if (st != OSCAR_OK) return st;
  hipLaunchKernelGGL(lse_reduce_kernel, dim3(geom->num_q_heads, geom->batch), dim3(128), 0, hs,
                     A.ws_ml, A.ws_o, geom->num_q_heads, S, out, lse);
  return launch_status();
}
