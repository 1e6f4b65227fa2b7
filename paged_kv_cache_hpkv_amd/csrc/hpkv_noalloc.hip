// Scratch of the no-allocation decode (hpkv_paged_attention_decode_noalloc):
// the split-context workspace (partials and dispatch order) in a fixed
// file-scope device array instead of caller memory, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array is part of the library's code object, so every GPU the library
// runs on holds its own copy, at its own address, until the process ends. Its
// device address is looked up once per device, with that device current, on
// the entry point's first call there; kernels only ever receive that address
// (the array's name in host code is a host-side stand-in, not a device
// pointer). Nothing in the workspace needs to start at zero: the ordering
// pass writes the order list and the partition pass writes every partial
// before the reduce reads it.

#include <mutex>

#include "hpkv_internal.h"

namespace hpkv {
namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace hpkv
