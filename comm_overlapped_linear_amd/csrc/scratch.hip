// Static device scratch of the allocation-free all-gather entry point, and
// the gate words of the carried in-kernel gates.
//
// The receive slots of tpgemm_stage_ag_noalloc live in a file-scope device
// array, so that call needs no caller workspace and allocates nothing. Each
// GPU the library runs on holds its own copy of the array (kStaticScratchBytes)
// until the process ends. In host code the array's name is only a host-side
// stand-in: its device address on the current GPU comes from
// hipGetSymbolAddress, resolved once per device and kept; kernels and copies
// only ever receive that address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

static __device__ __align__(256) uint8_t scratch[tpg::kStaticScratchBytes];
// Gate words of the carried in-kernel gates (zero at load; see gemm.h).
static __device__ __align__(256) unsigned long long gate_word[tpg::kGateWords];

namespace tpg {

namespace {
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device (nullptr: not resolved)
void* g_words[kMaxDevices] = {};     // device address of `gate_word` per device
}

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

hipError_t gate_words(unsigned long long** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (g_words[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(gate_word));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_words[dev] = p;
  }
  *ptr = static_cast<unsigned long long*>(g_words[dev]);
  return hipSuccess;
}

}  // namespace tpg
