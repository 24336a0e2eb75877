// oscar_host.hpp -- host-side helpers shared by the C-ABI launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oscar.h"

namespace oscar {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// The current device must be gfx950.  The answer is cached per device.
oscar_status check_device();

// hipGetLastError after a launch -> ELAUNCH.
inline oscar_status launch_status() {
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_ELAUNCH;
}

// Geometry accepted by the kernels: d = 128, Hq % Hkv == 0, group of 1, 2,
// 4 or 8 query heads per KV head, 1..16 KV heads, TOKEN norm scope.
oscar_status check_geom(const oscar_cache_geom* g);
oscar_status check_cache(const oscar_cache_geom* g, const oscar_cache* c);

// Split-K partials of decode attention, shared by the INT2 and bf16 paths:
// ws_ml [B][Hq][S] (m, l) with m in log2 units, ws_o [B][Hq][S][128]; the
// workspace holds both (ws_o from the first 256-B boundary after ws_ml).
size_t workspace_bytes(const oscar_cache_geom* g, int splits);
// Merge the S partials of every (sequence, query head) into out [B][Hq][128]
// and, if lse is not NULL, lse [B][Hq] (natural log).
void launch_lse_reduce(const float2* ws_ml, const float* ws_o, int hq, int batch, int splits,
                       float* out, float* lse, hipStream_t st);

}  // namespace oscar
