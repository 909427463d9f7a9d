// The one-call routed layer without a caller-provided workspace, for callers
// that cannot allocate device memory (code under HIP graph capture that must
// not allocate, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace of w4a16_moe_routed_forward (alignment histograms and buffers,
// h rows, per-slot fp32 down outputs, the tiled stages' scratch) lives in a
// file-scope device array of a fixed size. Each GPU the library runs on holds
// its own copy of the array, at its own address, from the first call on that
// GPU until the process ends. In host code the array's name is only a host-side
// stand-in: the device address of the current GPU's copy is looked up once per
// device with hipGetSymbolAddress and kept, and only that address is handed to
// the kernels. Nothing in the routed path needs this memory to start at zero
// (every buffer is written before it is read), so it is never cleared.
//
// Every call on one GPU shares that GPU's array and it keeps the last call's
// contents: calls that overlap on one GPU (two streams, or two host threads
// whose work is in flight at once) race on it.
#include <mutex>

#include "internal.h"
#include "w4a16_moe.h"

namespace {

__device__ __align__(256) uint8_t scratch[W4A16_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of the current GPU's copy of `scratch` (looked up once per
// device, with that device current).
hipError_t scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_ptr[dev];
  return g_err[dev];
}

}  // namespace

extern "C" {

int w4a16_moe_routed_forward_noalloc(const w4a16_moe_shape* shape, const uint16_t* x, int32_t T, int32_t topk,
                                     int32_t num_experts_global, const int32_t* topk_ids, const float* topk_weights,
                                     const void* w13_packed, const void* w2_packed, uint16_t* out, void* stream) {
  const size_t need = w4a16_moe_routed_workspace_bytes(shape, T, topk, num_experts_global);
  if (need == 0) {
    // invalid arguments: the routed entry point names the error without touching memory
    return w4a16_moe_routed_forward(shape, x, T, topk, num_experts_global, topk_ids, topk_weights, w13_packed,
                                    w2_packed, out, nullptr, 0, stream);
  }
  if (need > (size_t)W4A16_NOALLOC_SCRATCH_BYTES) return W4A16_ERR_NOALLOC_LIMIT;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess || ws == nullptr) return W4A16_ERR_HIP;
  return w4a16_moe_routed_forward(shape, x, T, topk, num_experts_global, topk_ids, topk_weights, w13_packed,
                                  w2_packed, out, ws, W4A16_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
