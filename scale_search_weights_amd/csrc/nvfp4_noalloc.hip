// Allocation-free block Hessian: nvfp4_block_hessian with its workspace (the per-chunk
// partial sums and the per-group item offsets) in a file-scope device array instead of a
// caller buffer, for callers that cannot allocate (code under HIP graph capture, tight
// loops, harnesses that forbid hipMalloc).
//
// The array is NVFP4_STATIC_SCRATCH_BYTES long and exists once per device the library runs
// on, for the life of the process. In host code its name is only a stand-in: the device
// address comes from hipGetSymbolAddress, looked up once per device on the first call made
// with that device current, and is what the kernels receive. Every call on a device shares
// the array and it keeps the previous call's contents; the block-Hessian kernels write every
// partial sum and offset they later read, so nothing needs clearing. Calls that overlap on
// one device (two streams at once) race on the array.
#include <mutex>

#include "nvfp4_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[NVFP4_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null until set)

// The current device's address of the scratch array, or null if it cannot be found.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int nvfp4_block_hessian_noalloc(const void *x, int dtype, int64_t tokens, int64_t cols,
                                int64_t groups, const int32_t *group_offsets,
                                const int32_t *token_ids, int64_t n_ids, float *H, int accumulate,
                                void *stream) {
  bool empty = false;
  const int rc = nvfp4::check_block_hessian(x, dtype, tokens, cols, groups, group_offsets,
                                            token_ids, n_ids, H, &empty);
  if (rc != NVFP4_OK || empty) return rc;
  if (nvfp4_block_hessian_workspace_size(tokens, cols, groups, n_ids) >
      (size_t)NVFP4_STATIC_SCRATCH_BYTES)
    return NVFP4_ERR_WORKSPACE;
  void *ws = scratch_on_current_device();
  if (!ws) return NVFP4_ERR_HIP;
  return nvfp4::run_block_hessian(x, dtype, tokens, cols, groups, group_offsets, token_ids,
                                  n_ids, H, accumulate, ws, stream);
}

}  // extern "C"
