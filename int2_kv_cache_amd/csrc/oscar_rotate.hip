// oscar_rotate.hip -- Canalized Rotation (online FHT) and Omni-Token Scaling
// on a batch of tokens: oscar_rotate_scale.
//
// [SUM] 方法步骤详情 (1) and (2): the query gets an online FHT; each Key gets an
// online FHT, then is divided by its L2 norm, which is stored.  [RN] §II Step
// Two: the norm is taken over all heads of the token.  (Tags: see
// oscar_device.hpp.)
#include "oscar_device.hpp"
#include "oscar_host.hpp"

namespace oscar {

// One wave per 128-vector; four vectors per 256-thread block.
__global__ __launch_bounds__(256) void rotate_query_kernel(const uint16_t* __restrict__ x,
                                                           int is_bf16, int n_vec,
                                                           float* __restrict__ out) {
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= n_vec) return;  // uniform per wave
  const int lane = threadIdx.x & 63;
  const size_t base = static_cast<size_t>(v) * kD;
  float a = in_to_f32(x[base + lane], is_bf16);
  float b = in_to_f32(x[base + lane + 64], is_bf16);
  fht128_wave(a, b);
  out[base + lane] = a;
  out[base + lane + 64] = b;
}

// Lane quad exchange (lanes 4m..4m+3): the value of lane l ^ X, X = 1 or 2.
template <int X>
__device__ __forceinline__ float quad_partner(float x) {
  constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), ctrl, 0xF, 0xF, true));
}

// Four lanes per (token, head) vector, 32 consecutive elements each; a
// 256-thread block takes floor(64 / n_heads) tokens.  Butterfly strides 1..16
// run in registers, strides 32 and 64 across the lane quad (the upper lane of
// a pair takes partner - own as one exactly rounded fma with -1), then one
// multiply by 1/sqrt(128): the same fp32 operations, in the same order, as
// the plain butterfly.  The sum of squares follows the same pairwise tree:
// levels 1..16 in registers, 32 and 64 across the quad, then over the heads
// (TOKEN scope) from LDS.
__global__ __launch_bounds__(256) void rotate_scale_key_kernel(
    const uint16_t* __restrict__ x, int is_bf16, int n_tokens, int n_heads, int head_scope,
    int hw_rsq, uint16_t* __restrict__ khat, uint16_t* __restrict__ norm) {
#pragma clang fp contract(off)
  __shared__ float part[64][16];  // [token in block][head]
  const int tpb = 64 / n_heads;
  const int tid = threadIdx.x, tq = tid & 3, vec = tid >> 2;
  const int tl = vec / n_heads, h = vec % n_heads;
  const int t = blockIdx.x * tpb + tl;
  const bool active = tl < tpb && t < n_tokens;
  float y[32];
  const size_t off = (static_cast<size_t>(t) * n_heads + h) * kD + 32 * tq;
  if (active) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = reinterpret_cast<const uint4*>(x + off)[q];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y[8 * q + 2 * e] = in_to_f32(static_cast<uint16_t>(ww[e]), is_bf16);
        y[8 * q + 2 * e + 1] = in_to_f32(static_cast<uint16_t>(ww[e] >> 16), is_bf16);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = 0.0f;
  }
#pragma unroll
  for (int hs = 1; hs < 32; hs <<= 1)
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if ((j & hs) == 0) {
        const float a = y[j], b = y[j + hs];
        y[j] = a + b;
        y[j + hs] = a - b;
      }
  const float sg1 = (tq & 1) ? -1.0f : 1.0f, sg2 = (tq & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) y[j] = __builtin_fmaf(sg1, y[j], quad_partner<1>(y[j]));
#pragma unroll
  for (int j = 0; j < 32; ++j) y[j] = __builtin_fmaf(sg2, y[j], quad_partner<2>(y[j]));
#pragma unroll
  for (int j = 0; j < 32; ++j) y[j] = y[j] * kFhtScale;
  float sq[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) sq[j] = y[j] * y[j];
#pragma unroll
  for (int hs = 1; hs < 32; hs <<= 1)
#pragma unroll
    for (int j = 0; j < 32; j += 2 * hs) sq[j] = sq[j] + sq[j + hs];
  float ss = sq[0];
  ss = ss + quad_partner<1>(ss);
  ss = ss + quad_partner<2>(ss);
  if (!head_scope) {
    if (active && tq == 0) part[tl][h] = ss;
    __syncthreads();
    if (active) ss = tree16(part[tl], n_heads);
  }
  if (!active) return;
  float nrm, r;
  scale_from_ss(ss, nrm, r, hw_rsq != 0);
  uint32_t kw[16];
#pragma unroll
  for (int e = 0; e < 16; ++e)
    kw[e] = static_cast<uint32_t>(f32_to_f16(mul_rn(y[2 * e], r))) |
            (static_cast<uint32_t>(f32_to_f16(mul_rn(y[2 * e + 1], r))) << 16);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    reinterpret_cast<uint4*>(khat + off)[q] = uint4{kw[4 * q], kw[4 * q + 1], kw[4 * q + 2], kw[4 * q + 3]};
  if (tq == 0) {
    if (head_scope)
      norm[static_cast<size_t>(t) * n_heads + h] = f32_to_f16_sat(nrm);
    else if (h == 0)
      norm[t] = f32_to_f16_sat(nrm);
  }
}

// Offline absorption of the Value rotation into the projection weights
// (reading notes §II Step One, query-side symmetric processing; summary
// 方法步骤详情 (3)): storing V' = H V per KV head means W_v' = H W_v, and
// the attention output, then in the rotated basis, is turned back by
// W_o' = W_o H.  Both are the plain fp32 FHT (strides 1..64, then x
// 1/sqrt(128)) of 128-element vectors of the weight matrix.

// axis 1: vectors along a row; with cols % 128 == 0 they are the consecutive
// 128-element runs of the row-major matrix.  One wave per vector.
__global__ __launch_bounds__(256) void absorb_rows_kernel(const float* __restrict__ w,
                                                          long long n_vec, float* out) {
  const long long v = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (v >= n_vec) return;  // uniform per wave
  const int lane = threadIdx.x & 63;
  const size_t base = static_cast<size_t>(v) * kD;
  float a = w[base + lane];
  float b = w[base + lane + 64];
  fht128_wave(a, b);
  out[base + lane] = a;
  out[base + lane + 64] = b;
}

// axis 0: vectors down a column, 128 rows apart from one 128-row block.  One
// thread per (row block, column): neighbouring threads read neighbouring
// columns, so every row access of a wave is one contiguous run.
__global__ __launch_bounds__(256) void absorb_cols_kernel(const float* __restrict__ w,
                                                          long long cols, long long n_thr,
                                                          float* out) {
#pragma clang fp contract(off)
  const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n_thr) return;
  const long long blk = t / cols, j = t % cols;
  const size_t base = static_cast<size_t>(blk) * kD * cols + j;
  float x[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) x[i] = w[base + static_cast<size_t>(i) * cols];
#pragma unroll
  for (int hs = 1; hs < kD; hs <<= 1)
#pragma unroll
    for (int i = 0; i < kD; ++i)
      if ((i & hs) == 0) {
        const float a = x[i], b = x[i + hs];
        x[i] = a + b;
        x[i + hs] = a - b;
      }
#pragma unroll
  for (int i = 0; i < kD; ++i) out[base + static_cast<size_t>(i) * cols] = x[i] * kFhtScale;
}

}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_absorb_value_rotation(const float* w, float* out, int64_t rows,
                                                    int64_t cols, int32_t axis, void* stream) {
  if (!w || !out || rows < 0 || cols < 0 || (axis != 0 && axis != 1)) return OSCAR_EINVAL;
  if ((axis == 0 ? rows : cols) % kD != 0) return OSCAR_EINVAL;
  if (rows != 0 && cols > (1LL << 62) / rows) return OSCAR_EINVAL;
  const long long total = static_cast<long long>(rows) * cols;
  const long long blocks = axis == 1 ? (total / kD + 3) / 4 : (total / kD + 255) / 256;
  if (blocks > 0x7fffffffLL) return OSCAR_EINVAL;
  oscar_status st = check_device();
  if (st != OSCAR_OK) return st;
  if (total == 0) return OSCAR_OK;
  if (axis == 1)
    hipLaunchKernelGGL(absorb_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       as_stream(stream), w, total / kD, out);
  else
    hipLaunchKernelGGL(absorb_cols_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       as_stream(stream), w, static_cast<long long>(cols), total / kD, out);
  return launch_status();
}

extern "C" oscar_status oscar_rotate_scale(const void* x, oscar_dtype dtype, int32_t n_tokens,
                                           int32_t n_heads, oscar_rot_mode mode,
                                           oscar_norm_scope norm_scope, float* q_out,
                                           void* khat_out, void* norm_out, void* stream) {
  if (!x || n_tokens < 0 || n_heads < 1) return OSCAR_EINVAL;
  if (mode != OSCAR_ROT_QUERY && n_heads > 16) return OSCAR_EINVAL;
  if (static_cast<long long>(n_tokens) * n_heads > (1LL << 30)) return OSCAR_EINVAL;
  if (dtype != OSCAR_FP16 && dtype != OSCAR_BF16) return OSCAR_EINVAL;
  if (norm_scope != OSCAR_NORM_TOKEN && norm_scope != OSCAR_NORM_HEAD) return OSCAR_EINVAL;
  if (mode == OSCAR_ROT_QUERY) {
    if (!q_out) return OSCAR_EINVAL;
  } else if (mode == OSCAR_ROT_KEY || mode == OSCAR_ROT_KEY_HW_RSQ) {
    if (!khat_out || !norm_out || !aligned(x, 16) || !aligned(khat_out, 16)) return OSCAR_EINVAL;
  } else {
    return OSCAR_EINVAL;
  }
  oscar_status st = check_device();
  if (st != OSCAR_OK) return st;
  if (n_tokens == 0) return OSCAR_OK;
  const int is_bf16 = dtype == OSCAR_BF16;
  if (mode == OSCAR_ROT_QUERY) {
    const long long n_vec = static_cast<long long>(n_tokens) * n_heads;
    const unsigned grid = static_cast<unsigned>((n_vec + 3) / 4);
    hipLaunchKernelGGL(rotate_query_kernel, dim3(grid), dim3(256), 0, as_stream(stream),
                       static_cast<const uint16_t*>(x), is_bf16, static_cast<int>(n_vec), q_out);
  } else {
    const int tpb = 64 / n_heads;
    const unsigned grid = static_cast<unsigned>((static_cast<long long>(n_tokens) + tpb - 1) / tpb);
    hipLaunchKernelGGL(rotate_scale_key_kernel, dim3(grid), dim3(256), 0, as_stream(stream),
                       static_cast<const uint16_t*>(x), is_bf16, n_tokens, n_heads,
                       norm_scope == OSCAR_NORM_HEAD ? 1 : 0, mode == OSCAR_ROT_KEY_HW_RSQ ? 1 : 0,
                       static_cast<uint16_t*>(khat_out), static_cast<uint16_t*>(norm_out));
  }
  return launch_status();
}
