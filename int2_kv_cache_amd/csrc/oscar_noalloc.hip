// oscar_noalloc.hip -- oscar_decode_attn_noalloc: decode attention for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The workspace of oscar_decode_attn comes from a file-scope device array
// instead of an argument: one copy per GPU, OSCAR_STATIC_WORKSPACE_BYTES
// long, held until the process ends.  Its first 256 KiB are the arrival
// counters of the cross-split merge, which must start at zero: the first
// call on a device clears them with a fill kernel on the call's stream, and
// every call leaves them zero again.  The partials after them are rewritten
// by every call.  All calls on one GPU share its copy, so calls that overlap
// in time on one GPU (different streams) race.
#include <mutex>

#include "oscar_host.hpp"

static __device__ __align__(256) unsigned char scratch[OSCAR_STATIC_WORKSPACE_BYTES];

namespace oscar {

// The merge's counter region at the start of every decode workspace.
constexpr size_t kNoallocCounterBytes = 65536 * 4;
static_assert(kNoallocCounterBytes <= OSCAR_STATIC_WORKSPACE_BYTES, "counter region");

__global__ __launch_bounds__(256) void clear_words_kernel(uint4* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = uint4{0u, 0u, 0u, 0u};
}

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  void* ptr = nullptr;   // this device's copy of `scratch`
  bool cleared = false;  // its counter clear has been enqueued
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

}  // namespace

// The device address of the current GPU's copy of `scratch`, looked up once
// per device with that device current, and kept.  In host code the array's
// name is a host-side stand-in, not a device address: only this pointer is
// ever passed on.  The first call on a device also enqueues the clear of the
// counter region on `st`, ahead of the attention that follows on it.
static void* scratch_ptr(hipStream_t st, oscar_status* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = OSCAR_EUNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& d = g_dev[dev];
  if (!d.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();  // clear the sticky error
      *status = OSCAR_ELAUNCH;
      return nullptr;
    }
    d.ptr = p;
  }
  if (!d.cleared) {
    const int words = static_cast<int>(kNoallocCounterBytes / 16);
    hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st,
                       static_cast<uint4*>(d.ptr), words);
    if (launch_status() != OSCAR_OK) {
      *status = OSCAR_ELAUNCH;
      return nullptr;
    }
    d.cleared = true;
  }
  *status = OSCAR_OK;
  return d.ptr;
}

}  // namespace oscar

using namespace oscar;

extern "C" oscar_status oscar_decode_attn_noalloc(const oscar_cache_geom* geom,
                                                  const oscar_cache* cache, const void* q,
                                                  oscar_dtype q_dtype, float* out, float* lse,
                                                  int32_t num_splits, int32_t max_ctx,
                                                  oscar_attn_variant variant, void* stream) {
  // the workspace this call needs, by oscar_decode_attn's own rule
  size_t need = 0;
  oscar_status st = oscar_decode_workspace_bytes(geom, max_ctx, num_splits, nullptr, &need);
  if (st != OSCAR_OK) return st;
  if (need > OSCAR_STATIC_WORKSPACE_BYTES) return OSCAR_EWORKSPACE;
  st = check_device();
  if (st != OSCAR_OK) return st;
  void* ws = scratch_ptr(as_stream(stream), &st);
  if (!ws) return st;
  return oscar_decode_attn(geom, cache, q, q_dtype, out, lse, ws, OSCAR_STATIC_WORKSPACE_BYTES,
                           num_splits, max_ctx, variant, stream);
}
