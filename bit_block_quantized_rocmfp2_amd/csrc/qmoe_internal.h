// Internal helpers shared by the host translation units of libqmoe.
#pragma once
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdarg>

#include "qmoe.h"

namespace qmoe {

// Thread-local error detail (qmoe_last_error).
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

// Per-format geometry of a 32-weight block (ROCmFP2 / FP3 / FP4).
struct FormatInfo {
  int bits;          // code width
  int lo_bytes;      // 2-bit plane (FP2, FP3 low bits) or nibble plane (FP4)
  int hi_bytes;      // FP3 bit-2 plane
  int scale_bytes;   // fp16 = 2, E8M0 = 1
  int block_bytes;   // 10 / 14 / 17
};

inline bool format_info(int fmt, FormatInfo* fi) {
  switch (fmt) {
    case QMOE_FP2: *fi = {2, 8, 0, 2, 10}; return true;
    case QMOE_FP3: *fi = {3, 8, 4, 2, 14}; return true;
    case QMOE_FP4: *fi = {4, 16, 0, 1, 17}; return true;
    default: return false;
  }
}

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace qmoe

#define QMOE_FAIL(code, ...)       \
  do {                             \
    ::qmoe::set_error(__VA_ARGS__); \
    return (code);                 \
  } while (0)

// Debug builds (-DQMOE_DEBUG_BOUNDS, libqmoe_debug.so): before each launch the
// host checks that the extents its kernels address, worked out from their own
// index formulas, fit the buffers and that the grids cover the rows; a failed
// check returns QMOE_E_INVAL naming the extent, and nothing is launched.
// Release builds compile the checks out.
#ifdef QMOE_DEBUG_BOUNDS
#define QMOE_BOUNDS(cond, what)                                                             \
  do {                                                                                      \
    if (!(cond)) QMOE_FAIL(QMOE_E_INVAL, "bounds check failed: %s (%s)", what, #cond);      \
  } while (0)
#else
#define QMOE_BOUNDS(cond, what) \
  do {                          \
    (void)sizeof((cond));       \
  } while (0)
#endif
