// Static device scratch for knapspec_solve_static: the library's per-solve device buffers
// (DP states, activation rows, GEMM and attention partial results, decisions, row maps) carved
// from one file-scope __device__ array instead of a workspace allocation, for callers that
// cannot allocate device memory.  Each GPU the library runs on holds its own copy of the array
// until the process ends.  Host code never passes the array's name to a kernel: its host-side
// symbol is only a handle, and the device address comes from hipGetSymbolAddress, taken once
// per device (with that device current) at set-up and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace ks {

namespace {

static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

}  // namespace

hipError_t resolve_static_scratch(int device) {
  if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[device]) return hipSuccess;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  g_ptr[device] = p;
  return hipSuccess;
}

void* static_scratch(int device) {
  if (device < 0 || device >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_ptr[device];
}

}  // namespace ks
