// moe_forward for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the same launches as
// moe_forward, with the workspace taken from a fixed device array that the
// library owns instead of a caller buffer.
//
// `scratch` lives in the code object, so each GPU the library runs on holds
// its own copy from module load until the process ends. In host code the
// array's name is only a host-side stand-in; its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and
// only that address is ever handed to kernels.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "moe_mi355x.h"

namespace {

constexpr size_t kScratchBytes = (size_t)MOE_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
thread_local char g_msg[160] = "";

// the device address of this device's scratch, looked up on its first use
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(g_msg, sizeof g_msg, "hipGetDevice: %s", hipGetErrorString(e));
    return MOE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(g_msg, sizeof g_msg, "device %d beyond the %d the scratch table holds", dev,
             kMaxDevices);
    return MOE_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(g_msg, sizeof g_msg, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
               hipGetErrorString(e));
      return MOE_ERR_HIP;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_no_workspace(const moe_layer* layer, const void* x_bf16,
                             const float* logits, long T, long ld_logits, float* out,
                             int* topk_ids, float* topk_w, float* sink_w, int* err_word,
                             void* stream) {
  g_msg[0] = '\0';
  if (!layer) return MOE_ERR_NULL;
  if (T < 0) return MOE_ERR_SHAPE;
  const size_t need = moe_workspace_size(layer, T);
  if (need == 0) return MOE_ERR_SHAPE;      // the layer descriptor is invalid
  if (need > kScratchBytes) {
    snprintf(g_msg, sizeof g_msg,
             "this layer at T = %ld needs %zu workspace bytes; the static scratch "
             "holds %zu",
             T, need, kScratchBytes);
    return MOE_ERR_SCRATCH;
  }
  void* ws = nullptr;
  int st = scratch_ptr(&ws);
  if (st) return st;
  // every byte moe_forward reads from its workspace is written earlier in
  // the same call, so nothing in the scratch has to start at zero
  return moe_forward(layer, x_bf16, logits, T, ld_logits, out, topk_ids, topk_w, sink_w,
                     err_word, ws, kScratchBytes, stream);
}

const char* moe_scratch_error(void) { return g_msg; }

}  // extern "C"
