// Allocation-free MLP chain entry point: chain_mlp_ex with the workspace in
// a file-scope device array instead of a caller buffer or the library's
// hipMalloc'd one, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops).
//
// The array (kNoAllocScratchBytes) holds the workspace layout of any call
// that fits: the control block and the fixed flag regions, then the call's
// split partials and its intermediate Z.  Each device gets its own copy when
// the library's code object is loaded there, and keeps it until the process
// ends.  Host code never uses the array's name as an address: the first call
// on a device looks up that device's copy with hipGetSymbolAddress (with the
// device current) and every launch, fill and copy uses that pointer.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "internal.h"
#include "runtime_internal.h"

namespace tls {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// First use on device `dev` (current): the array's address on this device,
// and the control block and flag regions cleared by a fill kernel on the
// call's stream (a kernel, so a captured call records no memset node).
chain_status scratch_for_device(int dev, hipStream_t stream, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return CHAIN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e != hipSuccess ? e : hipErrorUnknown);
    chain_status st = fill_u32(p, 0u, kFixedBytes, stream);
    if (st != CHAIN_OK) return st;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CHAIN_OK;
}

}  // namespace
}  // namespace tls

using namespace tls;

extern "C" {

chain_status chain_mlp_noalloc(const chain_mlp_args* a) {
  if (!a) return CHAIN_EINVAL;
  if (a->workspace) return CHAIN_EINVAL;  // the scratch array is the workspace
  // An order table would be copied from the host (a synchronous copy): only
  // the orders without one (the default, and row-major unseeded) are taken.
  if (a->order_seed != 0 ||
      (a->order != CHAIN_ORDER_XCD && a->order != CHAIN_ORDER_ROW_MAJOR))
    return CHAIN_EUNSUPPORTED;
  // The same argument checks as chain_mlp_ex, then the call's exact need.
  size_t need = 0;
  chain_status st = mlp_workspace_need(a, &need);
  if (st != CHAIN_OK) return st;
  if (need > kNoAllocScratchBytes) return CHAIN_ESCRATCH;
  int dev = 0;
  if ((st = current_device(&dev)) != CHAIN_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_for_device(dev, (hipStream_t)a->stream, &ws)) != CHAIN_OK) return st;
  chain_mlp_args b;
  std::memcpy(&b, a, sizeof(b));
  b.workspace = ws;
  b.workspace_bytes = kNoAllocScratchBytes;
  return chain_mlp_ex(&b);
}

chain_status chain_noalloc_status(void* stream) {
  int dev = 0;
  chain_status st = current_device(&dev);
  if (st != CHAIN_OK) return st;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_noalloc_mu);
    if (dev >= 0 && dev < kMaxDevices) ws = g_scratch_ptr[dev];
  }
  return read_status(ws, (hipStream_t)stream);
}

}  // extern "C"
