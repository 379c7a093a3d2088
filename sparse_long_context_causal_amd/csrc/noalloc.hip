// Allocation-free form of sparse_attn_windowed (declared in include/amtk.h).
//
// The windowed gather needs scratch beside its inputs and outputs: the start
// of every key window in every row's support and, when the caller passes no
// lse_sparse, the running log-sum-exp the windows merge through. Here that
// scratch is a file-scope device array, so a call allocates nothing and needs
// no workspace argument. Each GPU the library runs on holds its own copy of
// the array until the process ends.
//
// The array's name is only a host-side stand-in for the device symbol: host
// code never passes it to a kernel. At the first call on a device (with that
// device current) hipGetSymbolAddress resolves that device's copy; the
// address is kept per device and is what the kernels receive.
//
// The windowed kernels write every scratch word they later read (window 0
// writes every row's output and LSE, the window-start kernel every start of
// every row), so nothing needs clearing between calls. Calls that overlap on
// one GPU share its array and race.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "amtk.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = AMTK_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (resolved once per device), or null
// with *err set when the runtime refuses.
void* device_scratch(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int sparse_attn_windowed_static(const amtk_attn_desc* a, int32_t key_block, int32_t max_units,
                                const void* q, const void* k, const void* v, const int32_t* idx,
                                const int32_t* count, float* o, float* lse_sparse,
                                void* stream) {
  // the same checks as sparse_attn_windowed, on the host, before any HIP call
  amtk::LayerShape s;
  int rc = amtk::validate_attn(a, &s);
  if (rc) return rc;
  if (max_units < 1) return AMTK_E_INVALID;
  if (key_block != 1 && key_block != 64) return AMTK_E_UNSUPPORTED;
  if (!amtk::sparse_shape_supported(s)) return AMTK_E_UNSUPPORTED;
  if (!q || !k || !v || !idx || !count || !o) return AMTK_E_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(idx, 4) ||
      !aligned(count, 4) || !aligned(o, 16) || (lse_sparse && !aligned(lse_sparse, 4)))
    return AMTK_E_INVALID;
  if (amtk::sparse_windowed_scratch_bytes(s) > kScratchBytes) return AMTK_E_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ptr = device_scratch(&e);
  if (!ptr) return amtk::record_hip_error(e);
  e = amtk::launch_sparse_attn_windowed(s, key_block, max_units, q, k, v, idx, count, o,
                                        lse_sparse, ptr, kScratchBytes,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? AMTK_OK : amtk::record_hip_error(e);
}

}  // extern "C"
#pragma GCC visibility pop
