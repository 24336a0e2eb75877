// oscar_abi.hip -- C-ABI bookkeeping: status strings, device check, geometry
// validation and the cache layout query.
#include "oscar_host.hpp"

namespace oscar {

// The library holds gfx950 code objects only; the runtime finds a kernel of
// ours for the current device exactly when that device is gfx950.  (Asking
// the runtime about a kernel is independent of the hipDeviceProp_t layout,
// which differs between HIP runtime versions.)
__global__ void device_probe_kernel() {}

oscar_status check_device() {
  static int cached[64];  // 0 unknown, 1 supported, 2 not
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return OSCAR_EUNSUPPORTED;
  if (cached[dev] == 0) {
    hipFuncAttributes attr;
    const hipError_t e =
        hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&device_probe_kernel));
    cached[dev] = e == hipSuccess ? 1 : 2;
    if (e != hipSuccess) (void)hipGetLastError();  // clear the sticky error
  }
  return cached[dev] == 1 ? OSCAR_OK : OSCAR_EUNSUPPORTED;
}

oscar_status check_geom(const oscar_cache_geom* g) {
  if (!g) return OSCAR_EINVAL;
  if (g->head_dim != OSCAR_HEAD_DIM || g->block_tokens != OSCAR_BLOCK_TOKENS ||
      g->residual_tokens != OSCAR_RESIDUAL_TOKENS || g->v_group != OSCAR_V_GROUP)
    return OSCAR_EINVAL;
  if (g->batch < 1 || g->num_kv_heads < 1 || g->num_kv_heads > 16) return OSCAR_EINVAL;
  if (g->num_q_heads < g->num_kv_heads || g->num_q_heads % g->num_kv_heads) return OSCAR_EINVAL;
  const int grp = g->num_q_heads / g->num_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8) return OSCAR_EINVAL;
  if (g->max_blocks_per_seq < 1 || g->num_physical_blocks < 1) return OSCAR_EINVAL;
  if (g->norm_scope != OSCAR_NORM_TOKEN && g->norm_scope != OSCAR_NORM_HEAD) return OSCAR_EINVAL;
  if (g->flush_tokens != 0 && g->flush_tokens != 32 && g->flush_tokens != 128) return OSCAR_EINVAL;
  if (g->key_scale != OSCAR_SCALE_IEEE && g->key_scale != OSCAR_SCALE_HW_RSQ) return OSCAR_EINVAL;
  if (g->rope_max_pos < 0) return OSCAR_EINVAL;
  return OSCAR_OK;
}

oscar_status check_cache(const oscar_cache_geom* g, const oscar_cache* c) {
  oscar_status st = check_geom(g);
  if (st != OSCAR_OK) return st;
  if (!c || !c->pool || !c->pool_norm || !c->res_k || !c->res_v || !c->res_norm ||
      !c->block_table || !c->seq_state || !c->error_flag || !c->append_sync)
    return OSCAR_EINVAL;
  if (!aligned(c->pool, 256) || !aligned(c->pool_norm, 16) || !aligned(c->res_k, 16) ||
      !aligned(c->res_v, 16) || !aligned(c->res_norm, 16) || !aligned(c->block_table, 4) ||
      !aligned(c->seq_state, 8) || !aligned(c->error_flag, 4) || !aligned(c->append_sync, 4))
    return OSCAR_EINVAL;
  if (g->rope_max_pos > 0 && (!c->rope || !aligned(c->rope, 8))) return OSCAR_EINVAL;
  return OSCAR_OK;
}

}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_cache_layout(const oscar_cache_geom* g, oscar_cache_sizes* out) {
  if (!out) return OSCAR_EINVAL;
  oscar_status st = check_geom(g);
  if (st != OSCAR_OK) return st;
  const size_t B = g->batch, H = g->num_kv_heads, P = g->num_physical_blocks;
  out->pool = P * H * OSCAR_RECORD_BYTES;
  const size_t NH = g->norm_scope == OSCAR_NORM_HEAD ? H : 1;  // norms per token
  out->pool_norm = P * NH * 32 * sizeof(uint16_t);
  out->res_k = B * H * 128 * 128 * sizeof(uint16_t);
  out->res_v = B * H * 128 * 128 * sizeof(uint16_t);
  out->res_norm = B * NH * 128 * sizeof(uint16_t);
  out->block_table = B * static_cast<size_t>(g->max_blocks_per_seq) * sizeof(int32_t);
  out->seq_state = B * 2 * sizeof(int32_t);
  out->error_flag = sizeof(int32_t);
  out->append_sync = B * sizeof(int32_t);
  return OSCAR_OK;
}

extern "C" const char* oscar_status_str(oscar_status s) {
  switch (s) {
    case OSCAR_OK: return "ok";
    case OSCAR_EINVAL: return "invalid argument";
    case OSCAR_EUNSUPPORTED: return "unsupported device or option";
    case OSCAR_ELAUNCH: return "kernel launch failed";
    case OSCAR_EWORKSPACE: return "workspace too small";
  }
  return "unknown status";
}
