// Host-side helpers shared by the HIP translation units of libqmoe.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "qmoe_internal.h"

namespace qmoe {

// Decode plan (int32 words in the `plan` region): [0] U distinct experts,
// [1..32] expert ids ascending, [33..64] column masks, fp32 weights from word
// 128: w[u][t] for u < 32, t < 4.
constexpr int kPlanMax = 32;
constexpr int kPlanIdOff = 1;
constexpr int kPlanMaskOff = 1 + kPlanMax;
constexpr int kPlanWOff = 128;

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_check(const char* what);

inline int ilog2(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) ++l;
  return l;
}

// Lanes per row for a row of nb blocks processed nbl at a time: the largest power
// of two <= nb/nbl, at most 64 and at least 1.
inline int lanes_per_row(int nb, int nbl) {
  int chunks = (nb + nbl - 1) / nbl;
  int l = 1;
  while (l * 2 <= chunks && l < 64) l *= 2;
  return l;
}

struct WsPtrs {
  int8_t* xq;
  float* dx;
  int32_t* idx;
  float* gw;
  double* logits;
  int32_t* plan;
  int8_t* hq;
  float* dh;
  uint8_t* group;
  float* ypair;
  // region sizes in bytes (up to the next region), for the debug bounds checks
  size_t n_xq, n_dx, n_idx, n_gw, n_logits, n_plan, n_hq, n_dh, n_group, n_ypair;
};

int ws_ptrs(const qmoe_layer* L, int32_t ntok, void* ws, size_t ws_bytes, WsPtrs* p);

// Opt-in kernel timing (qmoe_timing_enable / qmoe_timing_read): when enabled,
// returns a pair of events from a pool, filed under `name`; otherwise nulls.
void timing_slot(const char* name, hipEvent_t* start, hipEvent_t* stop);

// Launches `kernel` on `s`. With timing enabled the start and stop events ride
// in the kernel's own dispatch (hipExtLaunchKernel), so their elapsed time is
// the kernel's execution without the gaps around it.
template <typename... Args, typename F = void (*)(Args...)>
void launch_kernel(const char* name, F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  timing_slot(name, &a, &b);
  if (a)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, a, b, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// Number of compute units of the current device, cached.
int device_cu_count();

// Host checks of one packed matrix and its codebook (format, shape, NULL,
// alignment, size); fills *fi.
int check_matrix(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes, const int8_t* cb, FormatInfo* fi);

// Prefill experts routed by 1 .. small_pairs pairs (at most kPrefillSmallPairs;
// the grouping lists them: nsmall[0] experts in small[]) go through the decode
// path's matvec arithmetic instead of a mostly empty MFMA tile
// (qmoe_decode.hip): gate/up, SwiGLU and requantization into the hq / dh rows
// of their sorted pair positions, then down into the ypair rows of their pair
// indices, times the pair's routing weight.
constexpr int kPrefillSmallPairs = 4;
struct PrefillSmall {
  const qmoe_layer* L;
  const int8_t* xq;        // every token's quantized activations [ntok][hidden]
  const float* dx;         // and their block scales [ntok][hidden / 32]
  const int32_t* counts;   // pairs per expert
  const int32_t* offsets;  // first sorted position per expert
  const int32_t* pairs;    // pair indices t * K + s by sorted position
  const int32_t* nsmall;   // number of listed experts (device)
  const int32_t* small;    // their ids, ascending
  const float* gw;         // routing weight per pair index
  int8_t* hq;              // [npairs][inter] by sorted position
  float* dh;               // [npairs][inter / 32]
  float* ypair;            // [npairs][hidden] by pair index
};
int launch_prefill_small(const PrefillSmall& p, hipStream_t s);

// Launch helpers shared by the entry points (qmoe_kernels.hip).
int launch_quant(const float* x, int64_t nblocks, int rot, int8_t* xq, float* dx, hipStream_t s);
int launch_route(const qmoe_layer* L, const float* x, int32_t ntok, double* logits, int32_t* idx, float* gw,
                 hipStream_t s);

}  // namespace qmoe
