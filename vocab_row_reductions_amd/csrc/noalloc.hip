// noalloc.hip -- vsel_topk_noalloc: the fused top-k with its scratch in a
// fixed device array instead of a caller workspace, for callers that cannot
// allocate device memory.
//
// `scratch` is one file-scope device array per GPU (each device that loads the
// library holds its own copy until the process ends).  Host code never uses
// the array's name as an address: on a device's first call the address comes
// from hipGetSymbolAddress, with that device current, and is kept per device.
// The first kTicketBytes hold the per-row ticket counters, which must be zero
// before a call; the kernels leave them at zero again, so they are cleared by
// a small fill kernel on a device's first call (and again after a call whose
// launch failed).  Every call on a device shares its array: calls that overlap
// on one GPU (two streams, or a graph replay beside an eager call) race.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/vsel.h"
#include "internal.hpp"

namespace {

constexpr size_t kTicketBytes = 65536;  // tickets of up to VSEL_NOALLOC_MAX_ROWS rows
static_assert(kTicketBytes == 4 * (size_t)VSEL_NOALLOC_MAX_ROWS, "one uint32 ticket per row");
static_assert(VSEL_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch is a whole number of 256-byte blocks");

static __device__ __align__(256) unsigned char scratch[VSEL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];      // the device's address of `scratch`
bool g_clear[kMaxDevices];     // tickets known to be zero (cleared, or left so by the kernels)

__global__ void __launch_bounds__(256) clear_words(uint32_t* p, uint32_t n) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

extern "C" vsel_status vsel_topk_noalloc(const void* logits, int dtype, int64_t rows, int64_t vocab, int64_t ld,
                                         int32_t k, float* out_vals, uint32_t* out_ids, uint32_t* out_argmax,
                                         float* out_lse, void* stream) {
  if (rows < 1 || rows > VSEL_NOALLOC_MAX_ROWS) return VSEL_EINVAL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VSEL_EDEVICE;
  hipStream_t s = (hipStream_t)stream;
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return VSEL_EDEVICE;
      g_ptr[dev] = p;
      g_clear[dev] = false;
    }
    base = g_ptr[dev];
    if (!g_clear[dev]) {
      const uint32_t n = (uint32_t)(kTicketBytes / 4);
      hipLaunchKernelGGL(clear_words, dim3((n + 255) / 256), dim3(256), 0, s, static_cast<uint32_t*>(base), n);
      if (hipGetLastError() != hipSuccess) return VSEL_EDEVICE;
      g_clear[dev] = true;
    }
  }
  const int st = vsel::topk_entry(logits, dtype, rows, vocab, ld, k, out_vals, out_ids, out_argmax, out_lse, base,
                                  VSEL_NOALLOC_SCRATCH_BYTES, stream, true);
  if (st == VSEL_EDEVICE) {
    std::lock_guard<std::mutex> lock(g_mu);
    g_clear[dev] = false;
  }
  return (vsel_status)st;
}
