// oscar_dense.hip -- the BF16 baseline: split-K decode attention over an
// unquantized, paged bf16 KV cache (oscar_dense_write_kv,
// oscar_dense_workspace_bytes, oscar_dense_decode_attn).
//
// The pages measure the INT2 kernel against BF16 FlashDecoding-v2 on the same
// model ([SUM] 实验结果 and 论文图表: decode speed-up over BF16 at 128K
// context; [POP] 四: memory and throughput at batch 48).  This is that
// baseline written for the same GPU and harness: no rotation, no scaling, no
// quantization; softmax(q K^T / sqrt(128)) V with the contiguous GQA mapping,
// partials merged by the same log-sum-exp reduce as the INT2 path.
//
// Cache layout, per (physical block p, KV head h), 32 tokens:
//   k_pool [P][Hkv][32 tokens][128] bf16  (a token's Key is one 256-B row)
//   v_pool [P][Hkv][128 ch][32 tokens] bf16 (a channel's 32 values are one
//                                            64-B row, so the P.V operand of
//                                            8 consecutive tokens is 16 B)
#include <math.h>

#include "oscar_host.hpp"

namespace oscar {
namespace {

constexpr int kD = 128, kG = 32;
constexpr float kScale = 0.08838834764831845f * 1.4426950408889634f;  // 1/sqrt(128) * log2(e)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16 (gfx950): A 16x32, lane l holds row l%16, K
// elements 8*(l/16)..+7; B 32x16, lane l holds column l%16, K elements
// 8*(l/16)..+7; C 16x16, lane l holds column l%16, rows 4*(l/16)..+3.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

struct DenseArgs {
  const uint16_t* kp;
  const uint16_t* vp;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const uint16_t* q;
  int hkv, hq, max_blocks, nphys, splits;
  int32_t* error_flag;
  float2* ws_ml;  // [B][Hq][S] (m, l), m in log2 units
  float* ws_o;    // [B][Hq][S][128]
};

// grid (S, Hkv, B), 256 threads.  Split s takes blocks [s*nb/S, (s+1)*nb/S)
// of its (sequence, KV head); wave w of the split takes every fourth block
// from the split's block w.  Per 32-token block and wave:
//   q.K^T: 2 row tiles (16 tokens) x 4 K steps (32 channels); B = the GQA
//          group's query heads in columns 0..GRP-1 (bf16 inputs, exact);
//   softmax in the log2 domain, lane (col, g4) owning head col % GRP and
//          tokens 8*g4..8*g4+7; the running maximum and sum of a head are
//          the same in all its lanes;
//   P.V:   8 row tiles (16 channels) x 1 K step (32 tokens); B = p split
//          into bf16 high (column h) and low (column h + GRP) parts, so p
//          enters to ~16 bits.
// The next block's 16 KB are loaded into registers while one is processed.
template <int GRP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8)))
void dense_attn_kernel(DenseArgs A) {
  static_assert(GRP == 1 || GRP == 2 || GRP == 4 || GRP == 8, "group size");
  __shared__ float lds_s[4][GRP][kG];            // per wave: one block's scores
  __shared__ float lds_o[4][2 * GRP][kD];        // per wave: hi and lo columns of o
  __shared__ float lds_ml[2][4][GRP];            // per wave: (m, l) per head

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), L = tid & 63;
  const int col = L & 15, g4 = L >> 4, hh = col % GRP;

  int n = A.ctx_lens[b];
  if (n < 0 || n > A.max_blocks * kG) {
    if (tid == 0 && s == 0) atomicOr(A.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    n = 0;
  }
  const int nb = (n + kG - 1) / kG;
  const int u0 = static_cast<int>((static_cast<long long>(s) * nb) / A.splits);
  const int u1 = static_cast<int>((static_cast<long long>(s + 1) * nb) / A.splits);
  const int first = u0 + wave;
  const int cnt = u1 > first ? (u1 - first + 3) / 4 : 0;

  // query B tile: column col < GRP holds head h*GRP + col; K step kk covers
  // channels 32 kk .. 32 kk + 31, lane group g4 channels 32 kk + 8 g4 .. +7
  u32x4 bq[4];
  {
    const uint16_t* qh = A.q + (static_cast<size_t>(b) * A.hq + h * GRP + hh) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qh + 32 * kk + 8 * g4);
      bq[kk] = col < GRP ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // physical block ids of the wave's blocks, 64 at a time (lane j: block j)
  const int32_t* tab = A.block_table + static_cast<size_t>(b) * A.max_blocks + first;
  auto load_ids = [&](int k0) {
    int id = 0;
    if (L < cnt - k0) id = tab[4 * (k0 + L)];
    const bool bad = static_cast<unsigned>(id) >= static_cast<unsigned>(A.nphys);
    if (__any(bad) && L == 0) atomicOr(A.error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    return bad ? 0 : id;
  };
  int idv = cnt > 0 ? load_ids(0) : 0;

  auto load_block = [&](int j, u32x4 (&rk)[2][4], u32x4 (&rv)[8]) {
    if (j > 0 && (j & 63) == 0) idv = load_ids(j);
    const int p = __builtin_amdgcn_readlane(idv, j & 63);
    const size_t ph = static_cast<size_t>(p) * A.hkv + h;
    const uint16_t* kb = A.kp + ph * (kG * kD);
    const uint16_t* vb = A.vp + ph * (kD * kG);
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        rk[tau][kk] = *reinterpret_cast<const u32x4*>(kb + (16 * tau + col) * kD + 32 * kk + 8 * g4);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      rv[ct] = *reinterpret_cast<const u32x4*>(vb + (16 * ct + col) * kG + 8 * g4);
  };

  f32x4 o[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.0f;

  auto process = [&](int j, const u32x4 (&rk)[2][4], const u32x4 (&rv)[8]) {
    const int t_valid = min(kG, n - kG * (first + 4 * j));
    f32x4 cs[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma_bf16(rk[tau][kk], bq[kk], acc);
      cs[tau] = acc;
    }
    // scores to the wave's LDS rows, read back in the P.V operand's layout
    if (col < GRP) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
        *reinterpret_cast<f32x4*>(&lds_s[wave][col][16 * tau + 4 * g4]) = cs[tau] * kScale;
    }
    asm volatile("" ::: "memory");  // a wave's LDS accesses complete in order
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(&lds_s[wave][hh][8 * g4]);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(&lds_s[wave][hh][8 * g4 + 4]);
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (8 * g4 + i >= t_valid) sv[i] = -INFINITY;
      bm = fmaxf(bm, sv[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float m_new = fmaxf(m_run, bm);  // finite: the block has a valid token
    const float f = __builtin_amdgcn_exp2f(m_run - m_new);  // -inf gives 0
    float ps = 0.0f;
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sv[i] - m_new), p1 = __builtin_amdgcn_exp2f(sv[i + 1] - m_new);
      ps += p0 + p1;
      const uint32_t h0 = bf16_rne(p0), h1 = bf16_rne(p1);
      const uint32_t l0 = bf16_rne(p0 - __uint_as_float(h0 << 16));
      const uint32_t l1 = bf16_rne(p1 - __uint_as_float(h1 << 16));
      hw[i / 2] = h0 | (h1 << 16);
      lw[i / 2] = l0 | (l1 << 16);
    }
    l_part = l_part * f + ps;
    m_run = m_new;
    const u32x4 bp = col < GRP ? u32x4{hw[0], hw[1], hw[2], hw[3]}
                     : col < 2 * GRP ? u32x4{lw[0], lw[1], lw[2], lw[3]}
                                     : u32x4{0u, 0u, 0u, 0u};
    if (t_valid == kG) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) o[ct] = mfma_bf16(rv[ct], bp, o[ct] * f);
    } else {
      // a partial last block: the rows past the sequence are whatever the
      // pool holds (possibly NaN patterns), so their Values are zeroed too
      u32x4 keep;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        keep[e] = (8 * g4 + 2 * e < t_valid ? 0xffffu : 0u) | (8 * g4 + 2 * e + 1 < t_valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) o[ct] = mfma_bf16(rv[ct] & keep, bp, o[ct] * f);
    }
  };

  u32x4 ka[2][4], va[8], kb2[2][4], vb2[8];
  if (cnt > 0) load_block(0, ka, va);
  for (int j = 0; j < cnt; j += 2) {
    if (j + 1 < cnt) load_block(j + 1, kb2, vb2);
    process(j, ka, va);
    if (j + 1 >= cnt) break;
    if (j + 2 < cnt) load_block(j + 2, ka, va);
    process(j + 1, kb2, vb2);
  }

  // this wave's partial: l summed over the head's 4 lane groups; o as hi and
  // lo columns in LDS
  float lsum = l_part + __shfl_xor(l_part, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (col < GRP && g4 == 0) {
    lds_ml[0][wave][col] = m_run;
    lds_ml[1][wave][col] = lsum;
  }
  if (col < 2 * GRP) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      *reinterpret_cast<f32x4*>(&lds_o[wave][col][16 * ct + 4 * g4]) = o[ct];
  }
  __syncthreads();

  // merge the 4 waves into this split's partial
  const size_t pbase = (static_cast<size_t>(b) * A.hq + h * GRP) * A.splits;
  for (int idx = tid; idx < GRP * kD; idx += 256) {
    const int i = idx >> 7, c = idx & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, lds_ml[0][w][i]);
    float Lw = 0.0f, Ow = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = lds_ml[0][w][i];
      const float sc = mw == -INFINITY ? 0.0f : exp2f(mw - M);
      Lw += sc * lds_ml[1][w][i];
      Ow += sc * (lds_o[w][i][c] + lds_o[w][i + GRP][c]);
    }
    const size_t part = pbase + static_cast<size_t>(i) * A.splits + s;
    A.ws_o[part * kD + c] = Ow;
    if (c == 0) A.ws_ml[part] = make_float2(M, Lw);
  }
}

// grid (ceil(n_tokens * Hkv * 16 / 256)), 256 threads: thread -> (token i,
// KV head, 8-channel chunk c8) of the input; writes the Key's 16 B and the 8
// Value elements of the cache rows of token start + i.
__global__ __launch_bounds__(256) void dense_write_kernel(uint16_t* __restrict__ kp, uint16_t* __restrict__ vp,
                                                          const int32_t* __restrict__ block_table,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, int seq,
                                                          int start, int n_tokens, int hkv,
                                                          int max_blocks, int nphys,
                                                          int32_t* error_flag) {
  const long long gid = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= static_cast<long long>(n_tokens) * hkv * 16) return;
  const int c8 = static_cast<int>(gid & 15);
  const int hh = static_cast<int>((gid >> 4) % hkv);
  const int i = static_cast<int>((gid >> 4) / hkv);
  const int t = start + i, blk = t / kG, tt = t % kG;
  if (blk >= max_blocks) {
    atomicOr(error_flag, static_cast<int32_t>(OSCAR_FLAG_CAPACITY));
    return;
  }
  const int p = block_table[static_cast<size_t>(seq) * max_blocks + blk];
  if (static_cast<unsigned>(p) >= static_cast<unsigned>(nphys)) {
    atomicOr(error_flag, static_cast<int32_t>(OSCAR_FLAG_BADSTATE));
    return;
  }
  const size_t src = (static_cast<size_t>(i) * hkv + hh) * kD + 8 * c8;
  const size_t ph = static_cast<size_t>(p) * hkv + hh;
  *reinterpret_cast<u32x4*>(kp + (ph * kG + tt) * kD + 8 * c8) = *reinterpret_cast<const u32x4*>(k + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(v + src);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    vp[(ph * kD + 8 * c8 + e) * kG + tt] = static_cast<uint16_t>(vv[e / 2] >> (16 * (e & 1)));
}

// Two rounds of workgroups at two per CU on 256 CUs, at least 8 blocks each.
int dense_auto_splits(const oscar_cache_geom* g, int max_ctx) {
  const int blocks = (max_ctx + kG - 1) / kG;
  const int pairs = g->batch * g->num_kv_heads;
  int s = (1024 + pairs - 1) / pairs;
  const int cap = blocks / 8 > 1 ? blocks / 8 : 1;
  if (s > cap) s = cap;
  if (s > 1024) s = 1024;
  return s < 1 ? 1 : s;
}

template <int GRP>
void launch_dense(const DenseArgs& A, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL(dense_attn_kernel<GRP>, grid, dim3(256), 0, st, A);
}

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_dense_write_kv(const oscar_cache_geom* geom, void* k_pool, void* v_pool,
                                             const int32_t* block_table, int32_t seq, int32_t start,
                                             const void* k, const void* v, int32_t n_tokens,
                                             int32_t* error_flag, void* stream) {
  oscar_status st = check_geom(geom);
  if (st != OSCAR_OK) return st;
  if (!k_pool || !v_pool || !block_table || !error_flag || seq < 0 || seq >= geom->batch ||
      start < 0 || n_tokens < 0)
    return OSCAR_EINVAL;
  if (n_tokens > 0 && (!k || !v || !aligned(k, 16) || !aligned(v, 16))) return OSCAR_EINVAL;
  if (!aligned(k_pool, 256) || !aligned(v_pool, 256) || !aligned(block_table, 4) ||
      !aligned(error_flag, 4))
    return OSCAR_EINVAL;
  if (static_cast<long long>(start) + n_tokens > static_cast<long long>(geom->max_blocks_per_seq) * kG)
    return OSCAR_EINVAL;
  st = check_device();
  if (st != OSCAR_OK) return st;
  if (n_tokens == 0) return OSCAR_OK;
  const long long threads = static_cast<long long>(n_tokens) * geom->num_kv_heads * 16;
  const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
  hipLaunchKernelGGL(dense_write_kernel, dim3(blocks), dim3(256), 0, as_stream(stream),
                     static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), block_table,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), seq, start,
                     n_tokens, geom->num_kv_heads, geom->max_blocks_per_seq,
                     geom->num_physical_blocks, error_flag);
  return launch_status();
}

extern "C" oscar_status oscar_dense_workspace_bytes(const oscar_cache_geom* geom, int32_t max_ctx,
                                                    int32_t num_splits, int32_t* splits_out,
                                                    size_t* bytes) {
  oscar_status st = check_geom(geom);
  if (st != OSCAR_OK) return st;
  if (!bytes || max_ctx < 0 || num_splits < 0 || num_splits > 1024) return OSCAR_EINVAL;
  const int s = num_splits ? num_splits : dense_auto_splits(geom, max_ctx);
  if (splits_out) *splits_out = s;
  *bytes = workspace_bytes(geom, s);
  return OSCAR_OK;
}

extern "C" oscar_status oscar_dense_decode_attn(const oscar_cache_geom* geom, const void* k_pool,
                                                const void* v_pool, const int32_t* block_table,
                                                const int32_t* ctx_lens, const void* q, float* out,
                                                float* lse, void* workspace, size_t ws_bytes,
                                                int32_t num_splits, int32_t max_ctx,
                                                int32_t* error_flag, void* stream) {
  oscar_status st = check_geom(geom);
  if (st != OSCAR_OK) return st;
  if (!k_pool || !v_pool || !block_table || !ctx_lens || !q || !out || !workspace || !error_flag ||
      max_ctx < 0 || num_splits < 0 || num_splits > 1024)
    return OSCAR_EINVAL;
  if (!aligned(k_pool, 256) || !aligned(v_pool, 256) || !aligned(block_table, 4) ||
      !aligned(ctx_lens, 4) || !aligned(q, 16) || !aligned(out, 16) || !aligned(workspace, 256) ||
      !aligned(error_flag, 4))
    return OSCAR_EINVAL;
  const int S = num_splits ? num_splits : dense_auto_splits(geom, max_ctx);
  if (ws_bytes < workspace_bytes(geom, S)) return OSCAR_EWORKSPACE;
  st = check_device();
  if (st != OSCAR_OK) return st;

  DenseArgs A;
  A.kp = static_cast<const uint16_t*>(k_pool);
  A.vp = static_cast<const uint16_t*>(v_pool);
  A.block_table = block_table;
  A.ctx_lens = ctx_lens;
  A.q = static_cast<const uint16_t*>(q);
  A.hkv = geom->num_kv_heads;
  A.hq = geom->num_q_heads;
  A.max_blocks = geom->max_blocks_per_seq;
  A.nphys = geom->num_physical_blocks;
  A.splits = S;
  A.error_flag = error_flag;
  const size_t npart = static_cast<size_t>(geom->batch) * geom->num_q_heads * S;
  A.ws_ml = static_cast<float2*>(workspace);
  A.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    ((npart * sizeof(float2) + 255) / 256) * 256);
  const dim3 grid(S, geom->num_kv_heads, geom->batch);
  hipStream_t hs = as_stream(stream);
  switch (geom->num_q_heads / geom->num_kv_heads) {
    case 1: launch_dense<1>(A, grid, hs); break;
    case 2: launch_dense<2>(A, grid, hs); break;
    case 4: launch_dense<4>(A, grid, hs); break;
    default: launch_dense<8>(A, grid, hs); break;
  }
  st = launch_status();
  if (st != OSCAR_OK) return st;
  launch_lse_reduce(A.ws_ml, A.ws_o, geom->num_q_heads, geom->batch, S, out, lse, hs);
  return launch_status();
}
