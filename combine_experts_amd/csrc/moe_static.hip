// moe_layer_static: moe_layer on a library-owned scratch array instead of a
// caller workspace, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The call allocates nothing: its intermediates live in the
// file-scope `scratch` array below, of which every GPU the library runs on
// holds its own copy until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress, and
// only that address is ever passed to kernels.  Calls on one GPU share that
// GPU's array and keep the last call's contents; the routing counters at its
// start must be zero when a call begins, which the combine of every call
// restores for its own config's experts, and which a small fill kernel
// establishes on a device's first call, after a call that returned an error,
// and before a call whose config has more experts than the last one's.  Calls
// that overlap on one GPU (different streams or threads) race on the array.
#include <mutex>

#include "moe_kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void zero_counts_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

struct DeviceScratch {
  void* ptr = nullptr;  // device address of this GPU's copy of scratch
  // leading int32 words of scratch known to be zero: the routing counters
  // of the last call that succeeded (its combine zeroed them); the words
  // after them belong to whatever that call's layout put there
  int zero_words = 0;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

}  // namespace

extern "C" {

size_t moe_layer_static_max_bytes(void) { return kScratchBytes; }

moe_status moe_layer_static(const moe_config* cfg, int32_t T, const void* x, const float* logits,
                            const float* bias, const moe_weights* w, void* y, void* stream) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_workspace_size(cfg, T);
  if (need == 0) return cfg == nullptr ? MOE_ERR_INVALID_ARG : moe_layer(cfg, T, x, logits, bias, w, y, nullptr, 0, stream);
  if (need > kScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  if (T == 0) return moe_layer(cfg, T, x, logits, bias, w, y, nullptr, 0, stream);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& d = g_dev[dev];
  if (!d.ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    d.ptr = p;
    d.zero_words = 0;
  }
  // the counters sit at offset 0 of the workspace layout, one int per
  // expert; a config with more experts than the last call's also needs the
  // words after those zeroed
  const int E = cfg->num_experts;
  if (d.zero_words < E) {
    hipLaunchKernelGGL(zero_counts_kernel, dim3((E + 255) / 256), dim3(256), 0, s, static_cast<int*>(d.ptr), E);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  }
  const moe_status st = moe_layer(cfg, T, x, logits, bias, w, y, d.ptr, kScratchBytes, stream);
  // success: this call's combine zeroed its E counters and its layout
  // overwrote the words after them; failure: the counters may be non-zero
  d.zero_words = st == MOE_OK ? E : 0;
  return st;
}

}  // extern "C"
