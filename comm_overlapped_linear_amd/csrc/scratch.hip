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
// Words of the cross-stream dependencies of eager calls (see gemm.h).
static __device__ __align__(256) unsigned long long sync_word[tpg::kSyncWords];

namespace tpg {

namespace {
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device (nullptr: not resolved)
void* g_words[kMaxDevices] = {};     // device address of `gate_word` per device
void* g_sync[kMaxDevices] = {};      // device address of `sync_word` per device

// Device address of a static array on the current device, resolved once.
hipError_t resolve(const void* symbol, void** cache, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (cache[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, symbol);
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    cache[dev] = p;
  }
  *ptr = cache[dev];
  return hipSuccess;
}
}

hipError_t static_scratch(void** ptr) { return resolve(HIP_SYMBOL(scratch), g_scratch, ptr); }

hipError_t gate_words(unsigned long long** ptr) {
  return resolve(HIP_SYMBOL(gate_word), g_words, reinterpret_cast<void**>(ptr));
}

hipError_t sync_words(unsigned long long** ptr) {
  return resolve(HIP_SYMBOL(sync_word), g_sync, reinterpret_cast<void**>(ptr));
}

}  // namespace tpg
