// Greedy verification that allocates nothing and takes no workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The verification's partial argmax keys live in `scratch`, a file-scope
// device array of kScratchBytes that each GPU holds for the life of the
// process.  Its device address is looked up once per device, with that device
// current, on the first call there, and kept in g_scratch; kernels receive
// that address, never the array's host-side name.  Every call on one GPU
// shares the array: calls that overlap on a GPU (different streams, no
// ordering) race on it.  Each call writes every key it reads, so nothing in
// the array needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/longspark.h"
#include "common.hpp"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(512) << 10;              // 512 KiB
constexpr int64_t kScratchKeys = int64_t(kScratchBytes / sizeof(uint64_t));
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// the current device's copy of `scratch`, looked up on its first use there
ls_status device_scratch(uint64_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return LS_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = static_cast<uint64_t*>(g_scratch[dev]);
  return LS_OK;
}

}  // namespace

extern "C" {

ls_status ls_verify_greedy_noalloc(const ls_dims* dims, const void* logits, const int32_t* draft,
                                   int32_t* target_tok, int32_t* tau, ls_stream stream) {
  const ls_status st = ls::check_dims(dims);
  if (st != LS_OK) return st;
  if (!logits || !draft || !target_tok || !tau) return LS_ERR_NULL;
  // the partial keys must fit the static array (checked before any HIP call)
  if (int64_t(dims->C) * (dims->B + 1) * ls::verify_splits(*dims) > kScratchKeys)
    return LS_ERR_SCRATCH;
  uint64_t* keys = nullptr;
  const ls_status sp = device_scratch(&keys);
  if (sp != LS_OK) return sp;
  return ls::launch_verify_into(*dims, logits, draft, target_tok, tau, keys,
                                static_cast<hipStream_t>(stream));
}

}  // extern "C"
