// Decode without allocation (gfx950): qmoe_decode_layer on a workspace that the
// library holds itself, for callers that cannot call hipMalloc (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
#include <hip/hip_runtime.h>

#include <mutex>

#include "qmoe_host.h"
#include "qmoe_internal.h"

using namespace qmoe;

// The workspace of qmoe_decode_layer_noalloc: a fixed device array, one copy
// per GPU, held until the process ends. Host code never uses the array's name
// as an address: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept in g_scratch_ptr.
namespace {

constexpr size_t kNoallocScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) QMOE_FAIL(QMOE_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) QMOE_FAIL(QMOE_E_HIP, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      QMOE_FAIL(QMOE_E_HIP, "hipGetSymbolAddress of the decode scratch failed on device %d: %s", dev,
                hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QMOE_OK;
}

}  // namespace

extern "C" size_t qmoe_decode_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

extern "C" int qmoe_decode_layer_noalloc(const qmoe_layer* L, const float* x, int32_t q, float* out, void* stream) {
  clear_error();
  if (q < 1 || q > 4) QMOE_FAIL(QMOE_E_SHAPE, "q=%d outside 1..4", q);
  qmoe_ws_layout lay;
  int st = qmoe_workspace_layout(L, q, &lay);
  if (st) return st;
  if (lay.total > kNoallocScratchBytes)
    QMOE_FAIL(QMOE_E_WORKSPACE, "decode of this layer at q=%d needs %zu bytes of workspace, more than the %zu-byte "
              "built-in scratch (use qmoe_decode_layer with a caller workspace)", q, lay.total, kNoallocScratchBytes);
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  // the decode kernels write every workspace region before they read it, so the
  // previous call's contents need no clearing
  return qmoe_decode_layer(L, x, q, out, ws, kNoallocScratchBytes, stream);
}
