// Allocation-free Hybrid Latent Attention decode, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): hla_decode_windowed with its workspace
// (query-map output, split and window partials, fused-path tickets) in a
// file-scope device array instead of a caller-provided buffer.
//
// Each GPU holds its own copy of `scratch` until the process ends.  Its
// device address is looked up once per device, with that device current, and
// kept; host code uses that address, never the array's name (a host-side
// stand-in).  Every call on one GPU shares the array: calls that overlap on
// one GPU (different streams, or threads without ordering) race.  Nothing in
// it must start at zero: the decode kernels overwrite every workspace element
// they read, and the fused path clears its tickets with a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lla.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;
static_assert(kScratchBytes == LLA_NOALLOC_SCRATCH_BYTES, "header and array disagree");

__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, 0 until looked up

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" lla_status hla_decode_windowed_noalloc(const lla_set_desc* desc, const lla_store* store,
                                                  int32_t batch, const lla_decode_args* args,
                                                  lla_stream_t stream) {
  if (!args) return LLA_ERR_INVALID_ARGUMENT;
  if (args->workspace || args->workspace_bytes) return LLA_ERR_INVALID_ARGUMENT;
  // argument checks only: without a workspace the regular entry point checks
  // every argument, then returns WORKSPACE_TOO_SMALL before it enqueues anything
  const lla_status checked = hla_decode_windowed(desc, store, batch, args, stream);
  if (checked != LLA_ERR_WORKSPACE_TOO_SMALL) return checked;
  const size_t need =
      lla_decode_workspace_bytes(desc, batch, args->max_pos_hint, args->window, args->splits);
  if (need > kScratchBytes) return LLA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return LLA_ERR_HIP;
  lla_decode_args a = *args;
  a.workspace = ws;
  a.workspace_bytes = kScratchBytes;
  return hla_decode_windowed(desc, store, batch, &a, stream);
}
