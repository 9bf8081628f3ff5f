// Prefill layer entry point (grouped expert GEMMs) — see qmoe_prefill_layer in include/qmoe.h.
#include <hip/hip_runtime.h>

#include "qmoe_device.h"
#include "qmoe_host.h"
#include "qmoe_internal.h"

using namespace qmoe;

extern "C" int qmoe_prefill_layer(const qmoe_layer* L, const float* x, int32_t ntok, float* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  clear_error();
  if (ntok < 0) QMOE_FAIL(QMOE_E_SHAPE, "ntok=%d", ntok);
  WsPtrs w;
  int st = ws_ptrs(L, ntok > 0 ? ntok : 1, ws, ws_bytes, &w);
  if (st) return st;
  (void)x; (void)out; (void)stream;
  QMOE_FAIL(QMOE_E_INVAL, "prefill not built yet");
}
