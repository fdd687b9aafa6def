// sd_decode_step_noalloc: the decode step with its scratch space in a static
// device array instead of a caller workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid allocation).  The kernels and the work are those of
// sd_decode_step; only where the scratch lives differs.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>

#include "sd.h"

namespace {

// The most scratch one call may use: every decode-step configuration of
// the benchmark fits (the largest, 128K tokens in token unit, needs about
// 28 MiB).  Each device the library runs on holds its own copy of the array
// until the process ends.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;

// In host code `scratch` names a host-side stand-in, not device memory: only
// the address hipGetSymbolAddress returns for the current device is passed
// to kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];

thread_local char g_msg[256] = "";

// Device address of this device's scratch array, looked up once per device
// with that device current; NULL (and the HIP error in msg) on failure.
void* device_scratch(int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    std::snprintf(g_msg, sizeof g_msg, "no usable current device (%s)",
                  e != hipSuccess ? hipGetErrorString(e) : "device index out of range");
    return nullptr;
  }
  *dev_out = dev;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    std::snprintf(g_msg, sizeof g_msg, "hipGetSymbolAddress of the static scratch failed: %s",
                  hipGetErrorString(e));
    return nullptr;
  }
  g_scratch[dev].store(p, std::memory_order_release);  // every thread finds the same address
  return p;
}

}  // namespace

extern "C" {

// Defined in abi.cpp: records a message for sd_last_error().
sd_status sdkv_fail_noalloc(sd_status st, const char* msg);

SD_API sd_status sd_decode_step_noalloc(const sd_shape* shape, const void* q, const void* k_pages,
                                        const void* v_pages, const void* page_bounds,
                                        const int32_t* block_table, const int32_t* seq_lens,
                                        int32_t unit, double r_kv, float* out, float* lse,
                                        int32_t* sel_idx, int32_t* sel_count, void* stream) {
  size_t need = 0;
  sd_status st = sd_workspace_bytes(shape, unit, r_kv, &need);
  if (st != SD_OK) return st;  // message already set
  if (need > kScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof msg,
                  "this shape needs %zu bytes of scratch, more than the %zu of the static "
                  "scratch; use sd_decode_step with a workspace",
                  need, kScratchBytes);
    return sdkv_fail_noalloc(SD_E_WORKSPACE, msg);
  }
  int dev = -1;
  void* ws = device_scratch(&dev);
  if (!ws) return sdkv_fail_noalloc(SD_E_DEVICE, g_msg);
  return sd_decode_step(shape, q, k_pages, v_pages, page_bounds, block_table, seq_lens, unit,
                        r_kv, out, lse, sel_idx, sel_count, ws, kScratchBytes, stream);
}

}  // extern "C"
