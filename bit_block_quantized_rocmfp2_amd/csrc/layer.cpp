// Layer descriptor validation and workspace layout (host, no device access).
//
// Validation classes follow lucebox.com "Lucebox × Geometric: DeepSeek V4 Flash
// 0731 reaches 32.7 tok/s on AMD Strix Halo", section "Lucebox Engine
// integration with Geometric": codebooks that are missing, truncated or
// mismatched are refused before any work starts; soothill.io "DeepSeek V4 Flash
// 0731 on evox3" (introduction) shows why an unsupported rotation must be
// refused at load rather than mid-run.
#include "qmoe_internal.h"

using namespace qmoe;

namespace {

constexpr int kMaxExperts = 512;
constexpr int kMaxHidden = 8192;
constexpr int kMaxTopk = 8;
constexpr size_t kAlign = 256;

int check_tensor(const char* name, int fmt, int64_t rows, int64_t k, int64_t E,
                 const void* w, size_t w_bytes, const int8_t* cb, size_t cb_bytes) {
  FormatInfo fi;
  if (!format_info(fmt, &fi)) QMOE_FAIL(QMOE_E_FORMAT, "%s: unknown format %d", name, fmt);
  if (k % 32) QMOE_FAIL(QMOE_E_SHAPE, "%s: K=%lld not a multiple of 32", name, (long long)k);
  const size_t row_bytes = (size_t)(k / 32) * fi.block_bytes;
  if (row_bytes % 16)
    QMOE_FAIL(QMOE_E_SHAPE, "%s: row of %zu bytes is not a multiple of 16 (K must be a multiple of %d for this format)",
              name, row_bytes, fmt == QMOE_FP4 ? 512 : 256);
  if (!w) QMOE_FAIL(QMOE_E_INVAL, "%s: missing weights (NULL)", name);
  if (reinterpret_cast<uintptr_t>(w) % 16) QMOE_FAIL(QMOE_E_INVAL, "%s: weights not 16-byte aligned", name);
  const size_t need = (size_t)E * rows * row_bytes;
  if (w_bytes < need) QMOE_FAIL(QMOE_E_SIZE, "%s: %zu weight bytes < %zu required", name, w_bytes, need);
  if (!cb) QMOE_FAIL(QMOE_E_CODEBOOK, "%s: missing codebook (NULL)", name);
  // the kernels read each expert's 4, 8 or 16 entries as whole dwords
  if (reinterpret_cast<uintptr_t>(cb) % 4) QMOE_FAIL(QMOE_E_INVAL, "%s: codebook not 4-byte aligned", name);
  const size_t cb_need = (size_t)E << fi.bits;
  if (cb_bytes < cb_need)
    QMOE_FAIL(QMOE_E_CODEBOOK, "%s: truncated codebook: %zu bytes < %lld experts x %d entries", name, cb_bytes,
              (long long)E, 1 << fi.bits);
  if (cb_bytes > cb_need)
    QMOE_FAIL(QMOE_E_CODEBOOK, "%s: mismatched codebook: %zu bytes != %lld experts x %d entries for format FP%d",
              name, cb_bytes, (long long)E, 1 << fi.bits, fmt);
  return QMOE_OK;
}

}  // namespace

extern "C" int qmoe_layer_check(const qmoe_layer* L) {
  clear_error();
  if (!L) QMOE_FAIL(QMOE_E_INVAL, "NULL layer descriptor");
  if (L->hidden <= 0 || L->inter <= 0) QMOE_FAIL(QMOE_E_SHAPE, "hidden=%d inter=%d must be positive", L->hidden, L->inter);
  if (L->n_experts < 1 || L->n_experts > kMaxExperts)
    QMOE_FAIL(QMOE_E_SHAPE, "n_experts=%d outside 1..%d", L->n_experts, kMaxExperts);
  if (L->topk < 1 || L->topk > kMaxTopk || L->topk > L->n_experts)
    QMOE_FAIL(QMOE_E_SHAPE, "topk=%d outside 1..min(n_experts, %d)", L->topk, kMaxTopk);
  if (L->rot_gateup != 0 && L->rot_gateup != 1) QMOE_FAIL(QMOE_E_FORMAT, "rot_gateup=%d unsupported (0 or 1)", L->rot_gateup);
  if (L->rot_down != 0 && L->rot_down != 1) QMOE_FAIL(QMOE_E_FORMAT, "rot_down=%d unsupported (0 or 1)", L->rot_down);
  if (L->fmt_gate != L->fmt_up)
    QMOE_FAIL(QMOE_E_FORMAT, "gate format FP%d differs from up format FP%d (must match)", L->fmt_gate, L->fmt_up);
  if (L->hidden % 32 || L->inter % 32) QMOE_FAIL(QMOE_E_SHAPE, "hidden=%d / inter=%d not multiples of 32", L->hidden, L->inter);
  if (L->hidden > kMaxHidden) QMOE_FAIL(QMOE_E_SHAPE, "hidden=%d exceeds %d", L->hidden, kMaxHidden);
  if (!L->w_router) QMOE_FAIL(QMOE_E_INVAL, "router: missing weights (NULL)");
  // router rows are read in 16-byte pieces (64 B per 32-block), the bias as fp64
  if (reinterpret_cast<uintptr_t>(L->w_router) % 16) QMOE_FAIL(QMOE_E_INVAL, "router: weights not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(L->router_bias) % 8) QMOE_FAIL(QMOE_E_INVAL, "router: bias not 8-byte aligned");
  const size_t rneed = (size_t)L->n_experts * L->hidden * 2;
  if (L->w_router_bytes < rneed) QMOE_FAIL(QMOE_E_SIZE, "router: %zu bytes < %zu required", L->w_router_bytes, rneed);
  int st;
  if ((st = check_tensor("gate", L->fmt_gate, L->inter, L->hidden, L->n_experts, L->gate, L->gate_bytes, L->cb_gate,
                         L->cb_gate_bytes)))
    return st;
  if ((st = check_tensor("up", L->fmt_up, L->inter, L->hidden, L->n_experts, L->up, L->up_bytes, L->cb_up,
                         L->cb_up_bytes)))
    return st;
  if ((st = check_tensor("down", L->fmt_down, L->hidden, L->inter, L->n_experts, L->down, L->down_bytes, L->cb_down,
                         L->cb_down_bytes)))
    return st;
  return QMOE_OK;
}

extern "C" int qmoe_workspace_layout(const qmoe_layer* L, int32_t max_tokens, qmoe_ws_layout* o) {
  int st = qmoe_layer_check(L);
  if (st) return st;
  if (!o) QMOE_FAIL(QMOE_E_INVAL, "NULL layout pointer");
  if (max_tokens < 1) QMOE_FAIL(QMOE_E_SHAPE, "max_tokens=%d must be >= 1", max_tokens);
  const size_t T = (size_t)max_tokens, H = L->hidden, I = L->inter, E = L->n_experts, K = L->topk;
  const size_t slots = T * K > 128 ? T * K : 128;   // decode uses slot = u*4 + t, u < 32
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = round_up(off + bytes, kAlign);
    return at;
  };
  o->xq = take(T * H);
  o->dx = take(T * (H / 32) * 4);
  o->idx = take(T * K * 4);
  o->gw = take(T * K * 4);
  o->logits = take(T * E * 8);
  o->plan = take(4096);
  o->hq = take(slots * I);
  o->dh = take(slots * (I / 32) * 4);
  // counts[E], offsets[E+1], cursor[E], pairs[T*K], tile list (2 int32 per tile),
  // small-expert count and list[E]
  o->group = take(4 * (3 * E + 1) + 4 * T * K + 8 * (T * K + E) + 4 * (E + 1) + 4096);
  o->ypair = take(T * K * H * 4);
  o->total = off;
  return QMOE_OK;
}

extern "C" size_t qmoe_workspace_bytes(const qmoe_layer* L, int32_t max_tokens) {
  qmoe_ws_layout o;
  return qmoe_workspace_layout(L, max_tokens, &o) == QMOE_OK ? o.total : 0;
}

extern "C" size_t qmoe_matvec_workspace_bytes(int64_t k, int32_t ncols) {
  if (k <= 0 || k % 32 || ncols < 1 || ncols > 4) return 0;
  return round_up((size_t)ncols * k, kAlign) + round_up((size_t)ncols * (k / 32) * 4, kAlign);
}
