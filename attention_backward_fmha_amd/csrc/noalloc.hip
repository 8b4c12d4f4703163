// noalloc.hip -- fmha_bwd_run_noalloc: prepare + run with a workspace the library owns, for
// callers that cannot allocate device memory.
//
// The workspace is a file-scope device array (one copy per GPU, held until the process ends).
// Its device address is looked up once per device with hipGetSymbolAddress while that device
// is current, and only that address is handed to the kernels: in host code the array's name
// is a host-side stand-in, not a device address.
#include <hip/hip_runtime.h>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>

#include "fmha_bwd.h"

static __device__ __align__(256) unsigned char scratch[FMHA_BWD_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};

int report(int status, const char* msg) {
  const char* e = getenv("FMHA_BWD_LOG");
  if (status != FMHA_OK && e && e[0] == '1') fprintf(stderr, "[fmha_bwd] run_noalloc: %s\n", msg);
  return status;
}

// The current device's copy of the scratch array (set up on the first call on that device).
int scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return report(FMHA_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return report(FMHA_ERR_UNSUPPORTED, "device ordinal out of range");
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return report(FMHA_ERR_HIP, e != hipSuccess ? hipGetErrorString(e) : "null scratch address");
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return FMHA_OK;
}

}  // namespace

extern "C" {

int fmha_bwd_run_noalloc(const fmha_bwd_args* args, void* stream) {
  size_t need = 0;
  int st = fmha_bwd_workspace_size(args, &need);
  if (st != FMHA_OK) return st;
  if (need > (size_t)FMHA_BWD_NOALLOC_MAX_BYTES)
    return report(FMHA_ERR_WORKSPACE_TOO_SMALL,
                  "these arguments need more workspace than the library's static scratch "
                  "(FMHA_BWD_NOALLOC_MAX_BYTES); use fmha_bwd_run with a caller workspace");
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != FMHA_OK) return st;
  st = fmha_bwd_prepare_workspace(args, ws, (size_t)FMHA_BWD_NOALLOC_MAX_BYTES, stream);
  if (st != FMHA_OK) return st;
  return fmha_bwd_run(args, ws, (size_t)FMHA_BWD_NOALLOC_MAX_BYTES, stream);
}

}  // extern "C"
