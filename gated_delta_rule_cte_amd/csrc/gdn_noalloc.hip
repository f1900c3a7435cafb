// gdn_cte_noalloc: gdn_cte with its workspace in a fixed, library-owned
// device array, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU that loads the
// library holds its own copy, at its own address, until the process ends.
// Host code never uses the array's name as an address (on the host it is
// only a stand-in); the per-device address comes from hipGetSymbolAddress,
// looked up once per device with that device current, and is what the
// kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
std::vector<void*> g_ptr;  // per device: the scratch address (nullptr = not looked up yet)

}  // namespace

extern "C" int gdn_cte_noalloc(const void* query, const void* key, const void* value, const float* g_log,
                               const float* beta, float scale, float* recurrent_state, int has_initial_state,
                               void* out, int B, int Hk, int Hv, int S, int Dk, int Dv, int dtype, int algorithm,
                               void* stream) {
  const size_t need = gdn_cte_workspace_size(B, Hk, Hv, S, Dk, Dv, dtype);
  // every argument check of gdn_cte, before any HIP call: with no workspace a
  // valid call stops at the workspace check (and an empty one succeeds)
  int r = gdn_cte(query, key, value, g_log, beta, scale, recurrent_state, has_initial_state, out, B, Hk, Hv, S,
                  Dk, Dv, dtype, algorithm, nullptr, 0, stream);
  if (r != GDN_ERR_WORKSPACE) return r;
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
    return gdn::set_error(GDN_ERR_WORKSPACE,
                          "this call needs %zu bytes of scratch; gdn_cte_noalloc holds %zu (use gdn_cte with a "
                          "caller-owned workspace, or fewer tokens or heads per call)",
                          need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return gdn::set_error(GDN_ERR_DEVICE, "no HIP device is available");
  }
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if ((int)g_ptr.size() <= dev) g_ptr.resize(dev + 1, nullptr);
    if (!g_ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return gdn::set_error(GDN_ERR_DEVICE, "device %d: the scratch array's address is unavailable (not a gfx950?)",
                              dev);
      }
      g_ptr[dev] = p;
    }
    ptr = g_ptr[dev];
  }
  return gdn_cte(query, key, value, g_log, beta, scale, recurrent_state, has_initial_state, out, B, Hk, Hv, S, Dk,
                 Dv, dtype, algorithm, ptr, (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream);
}
