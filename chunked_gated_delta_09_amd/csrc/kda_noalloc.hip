// kda_chunk_bwd_noalloc: the chunkwise backward with its workspace in a device array of the
// library itself, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array below is file-scope device memory: each GPU the library runs on holds one copy
// of KDA_NOALLOC_MAX_WORKSPACE bytes from module load until the process ends. Its name is a
// host-side stand-in in host code, not a device address; the device address of the current
// GPU's copy comes from hipGetSymbolAddress, looked up once per device on that device's
// first call, with the device current, and kept per device. Only that address is passed on.
// Every call on one GPU shares that GPU's copy (the last call's contents stay in it):
// calls that overlap on one GPU race. The backward needs no initialised workspace, so
// nothing is cleared.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kda.h"
#include "kda_launch.h"

#define KDA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = KDA_NOALLOC_MAX_WORKSPACE;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (nullptr and a message on error).
void* scratch_for_current_device(kda_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof(msg), "kda_chunk_bwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    *st = kda::set_error(KDA_EHIP, msg);
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = kda::set_error(KDA_EUNSUPPORTED, "kda_chunk_bwd_noalloc: device index beyond the supported 64");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      char msg[256];
      snprintf(msg, sizeof(msg), "kda_chunk_bwd_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
      *st = kda::set_error(KDA_EHIP, msg);
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

KDA_EXPORT kda_status kda_chunk_bwd_noalloc(const kda_dims* dims, const void* q, const void* k, const void* v,
                                            const float* g, const float* beta, const void* states, const void* inv,
                                            const void* dO, const void* dS_final, void* dq, void* dk, void* dv,
                                            float* dg, float* dbeta, float* dh0, void* stream) {
  size_t need = 0;
  kda_status st = kda::bwd_plan(dims, &need);
  if (st != KDA_OK) return st;
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "kda_chunk_bwd_noalloc: this call needs %zu workspace bytes, more than the %zu of the "
             "library's static scratch; use kda_chunk_bwd with a caller workspace",
             need, kScratchBytes);
    return kda::set_error(KDA_EINVAL, msg);
  }
  void* ws = scratch_for_current_device(&st);
  if (ws == nullptr) return st;
  return kda_chunk_bwd(dims, q, k, v, g, beta, states, inv, dO, dS_final, dq, dk, dv, dg, dbeta, dh0, ws,
                       kScratchBytes, stream);
}
