// Device scratch of aut_encode_noalloc: the forward's workspace (plan tables,
// conv-stem batch buffers, residual stream, layer activations) in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate device memory.  Each GPU the library runs on holds its own copy
// from module load until the process ends; its host-side name is only a
// handle, so the device address is looked up once per device and kept.
#include <mutex>
#include <vector>

#include "aut_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)256 << 20;  // 256 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device id, null until looked up

}  // namespace

namespace aut {

size_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_ptr(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace aut
