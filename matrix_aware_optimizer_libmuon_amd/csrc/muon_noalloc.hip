// Fixed device scratch of muon_step_noalloc, for callers that cannot
// allocate: one file-scope array per device holds the descriptor table and
// every intermediate (X, A, C) that muon_step keeps in the caller's
// workspace.  The array's host-side name is not a device address: host code
// uses only the address hipGetSymbolAddress returns for the current device.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "muon.h"
#include "muon_internal.h"

namespace muon {

static __device__ __align__(256) unsigned char scratch[MUON_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> address of its scratch array
}  // namespace

// Address of `scratch` on device `dev` (which must be current), resolved on
// the first call for that device and kept.
int noalloc_scratch(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return static_cast<int>(hipSuccess);
}

// The descriptor table travels in kernel arguments: each launch carries up to
// kPutWords 32-bit words by value and one workgroup stores them at dst.  No
// host staging buffer, no copy engine, nothing to allocate.
constexpr int kPutWords = 960;
struct PutChunk {
  uint32_t n;
  uint32_t w[kPutWords];
};

__global__ __launch_bounds__(256) void k_put_words(uint32_t* __restrict__ dst, PutChunk c) {
  for (uint32_t k = threadIdx.x; k < c.n; k += 256) dst[k] = c.w[k];
}

int put_bytes(void* dst, const void* src, size_t bytes, void* stream) {
  // the table is a multiple of 256 bytes; a ragged tail is zero-padded
  const unsigned char* s = static_cast<const unsigned char*>(src);
  uint32_t* d = static_cast<uint32_t*>(dst);
  for (size_t off = 0; off < bytes; off += 4 * static_cast<size_t>(kPutWords)) {
    PutChunk c;
    const size_t take = bytes - off < 4 * static_cast<size_t>(kPutWords) ? bytes - off
                                                                          : 4 * static_cast<size_t>(kPutWords);
    c.n = static_cast<uint32_t>((take + 3) / 4);
    c.w[c.n - 1] = 0;
    __builtin_memcpy(c.w, s + off, take);
    hipLaunchKernelGGL(k_put_words, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream),
                       d + off / 4, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
  }
  return static_cast<int>(hipSuccess);
}

}  // namespace muon
