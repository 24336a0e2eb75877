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

// One wave per token, all of its heads in registers (lane l holds elements l
// and l + 64 of every head), four tokens per 256-thread block.  The heads'
// butterflies are independent, so a wave keeps up to 2 * n_heads loads and
// stores in flight; the sums of squares are the same per-head trees as in
// the oracle, then the tree over the heads (TOKEN scope) in registers.
template <int MAXH>
__global__ __launch_bounds__(256) void rotate_scale_key_kernel(
    const uint16_t* __restrict__ x, int is_bf16, int n_tokens, int n_heads, int head_scope,
    int hw_rsq, uint16_t* __restrict__ khat, uint16_t* __restrict__ norm) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= n_tokens) return;  // uniform per wave
  const size_t base = static_cast<size_t>(t) * n_heads * kD;
  float a[MAXH], b[MAXH], hs[MAXH];
#pragma unroll
  for (int h = 0; h < MAXH; ++h) {
    if (h < n_heads) {
      a[h] = in_to_f32(x[base + h * kD + lane], is_bf16);
      b[h] = in_to_f32(x[base + h * kD + lane + 64], is_bf16);
    }
  }
#pragma unroll
  for (int h = 0; h < MAXH; ++h) {
    if (h < n_heads) {
      fht128_wave(a[h], b[h]);
      hs[h] = wave_tree_sumsq(a[h], b[h]);
    } else {
      hs[h] = 0.0f;
    }
  }
  const float ss_tok = head_scope ? 0.0f : tree16(hs, n_heads);
#pragma unroll
  for (int h = 0; h < MAXH; ++h) {
    if (h < n_heads) {
      float nrm, r;
      scale_from_ss(head_scope ? hs[h] : ss_tok, nrm, r, hw_rsq != 0);
      khat[base + h * kD + lane] = f32_to_f16(mul_rn(a[h], r));
      khat[base + h * kD + lane + 64] = f32_to_f16(mul_rn(b[h], r));
      if (lane == 0) {
        if (head_scope)
          norm[static_cast<size_t>(t) * n_heads + h] = f32_to_f16(nrm);
        else if (h == 0)
          norm[t] = f32_to_f16(nrm);
      }
    }
  }
}

}  // namespace oscar

using namespace oscar;

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
    if (!khat_out || !norm_out) return OSCAR_EINVAL;
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
    const unsigned grid = static_cast<unsigned>((static_cast<long long>(n_tokens) + 3) / 4);
    const int hs = norm_scope == OSCAR_NORM_HEAD ? 1 : 0, hw = mode == OSCAR_ROT_KEY_HW_RSQ ? 1 : 0;
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    uint16_t* kh = static_cast<uint16_t*>(khat_out);
    uint16_t* nm = static_cast<uint16_t*>(norm_out);
    if (n_heads <= 8)
      hipLaunchKernelGGL(rotate_scale_key_kernel<8>, dim3(grid), dim3(256), 0, as_stream(stream), xs,
                         is_bf16, n_tokens, n_heads, hs, hw, kh, nm);
    else
      hipLaunchKernelGGL(rotate_scale_key_kernel<16>, dim3(grid), dim3(256), 0, as_stream(stream), xs,
                         is_bf16, n_tokens, n_heads, hs, hw, kh, nm);
  }
  return launch_status();
}
