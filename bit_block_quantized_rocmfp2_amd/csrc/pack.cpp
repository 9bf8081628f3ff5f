// Host-side packing of ROCmFPX blocks and descriptor validation (CPU only).
//
// Block geometry: lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
// AMD Ryzen AI MAX+ 395", section "ROCmFPX: fitting 284B weights into 128 GB"
// (32 weights per block; FP2 10 B, FP3 3.50 bpw = 14 B, FP4 4.25 bpw = 17 B).
// Bit positions (this library's layout, see include/qmoe.h):
//   2-bit plane: weight j -> byte 4*(j>>4) + (j&3), shift 2*((j>>2)&3)
//   FP3 bit 2  : weight j -> byte j&3 of the 4-byte plane, shift j>>2
//   FP4 nibble : weight j -> byte 4*(j>>3) + (j&3), shift 4*((j>>2)&1)
// so that, read as 32-bit words, one shift-and-mask yields the 4 selectors of
// weights 4g..4g+3 for one byte permute and one 4-way int8 dot product.
#include <cstring>
#include <string>

#include "qmoe_internal.h"

namespace qmoe {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}
void clear_error() { g_err[0] = 0; }

}  // namespace qmoe

using namespace qmoe;

extern "C" const char* qmoe_last_error(void) { return g_err; }

extern "C" const char* qmoe_strerror(int s) {
  switch (s) {
    case QMOE_OK: return "ok";
    case QMOE_E_INVAL: return "invalid argument";
    case QMOE_E_SHAPE: return "invalid shape";
    case QMOE_E_FORMAT: return "unsupported format or rotation";
    case QMOE_E_CODEBOOK: return "missing, truncated or mismatched codebook";
    case QMOE_E_SCALE: return "invalid scale";
    case QMOE_E_WORKSPACE: return "workspace missing or too small";
    case QMOE_E_HIP: return "HIP runtime error";
    case QMOE_E_SIZE: return "weight buffer too small";
    default: return "unknown status";
  }
}

extern "C" int qmoe_version(void) { return 100; }

extern "C" size_t qmoe_block_bytes(int fmt) {
  FormatInfo fi;
  return format_info(fmt, &fi) ? (size_t)fi.block_bytes : 0;
}

extern "C" size_t qmoe_packed_bytes(int fmt, int64_t rows, int64_t k) {
  FormatInfo fi;
  if (!format_info(fmt, &fi) || rows < 0 || k < 0 || k % 32) return 0;
  return (size_t)rows * (size_t)(k / 32) * (size_t)fi.block_bytes;
}

static inline void lo_pos(int fmt, int j, int* byte, int* shift) {
  if (fmt == QMOE_FP4) {
    *byte = 4 * (j >> 3) + (j & 3);
    *shift = 4 * ((j >> 2) & 1);
  } else {
    *byte = 4 * (j >> 4) + (j & 3);
    *shift = 2 * ((j >> 2) & 3);
  }
}

static int check_geometry(int fmt, int64_t rows, int64_t k, FormatInfo* fi) {
  if (!format_info(fmt, fi)) QMOE_FAIL(QMOE_E_FORMAT, "unknown format %d", fmt);
  if (rows < 0 || k < 0) QMOE_FAIL(QMOE_E_SHAPE, "negative shape rows=%lld k=%lld", (long long)rows, (long long)k);
  if (k % 32) QMOE_FAIL(QMOE_E_SHAPE, "k=%lld is not a multiple of 32", (long long)k);
  return QMOE_OK;
}

extern "C" int qmoe_pack(int fmt, int64_t rows, int64_t k, const uint8_t* codes,
                         const void* scales, void* out, size_t out_bytes) {
  clear_error();
  FormatInfo fi;
  int st = check_geometry(fmt, rows, k, &fi);
  if (st) return st;
  const int64_t nb = k / 32;
  const size_t need = (size_t)rows * nb * fi.block_bytes;
  if ((rows * k > 0) && (!codes || !scales || !out)) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (out_bytes < need) QMOE_FAIL(QMOE_E_SIZE, "out_bytes %zu < %zu", out_bytes, need);
  const uint8_t maxc = (uint8_t)((1u << fi.bits) - 1);
  const size_t row_bytes = (size_t)nb * fi.block_bytes;
  uint8_t* o = static_cast<uint8_t*>(out);
  for (int64_t r = 0; r < rows; ++r) {
    uint8_t* row = o + (size_t)r * row_bytes;
    std::memset(row, 0, row_bytes);
    uint8_t* lo = row;
    uint8_t* hi = row + nb * fi.lo_bytes;
    uint8_t* sc = hi + nb * fi.hi_bytes;
    for (int64_t b = 0; b < nb; ++b) {
      const uint8_t* c = codes + r * k + b * 32;
      for (int j = 0; j < 32; ++j) {
        const uint8_t v = c[j];
        if (v > maxc) QMOE_FAIL(QMOE_E_INVAL, "code %u out of range at row %lld col %lld", v, (long long)r, (long long)(b * 32 + j));
        int byte, shift;
        lo_pos(fmt, j, &byte, &shift);
        const uint8_t lv = (fmt == QMOE_FP4) ? v : (uint8_t)(v & 3);
        lo[b * fi.lo_bytes + byte] |= (uint8_t)(lv << shift);
        if (fmt == QMOE_FP3) hi[b * 4 + (j & 3)] |= (uint8_t)(((v >> 2) & 1) << (j >> 2));
      }
      if (fmt == QMOE_FP4) {
        const uint8_t e = static_cast<const uint8_t*>(scales)[r * nb + b];
        if (e == 0xFF) QMOE_FAIL(QMOE_E_SCALE, "E8M0 scale 0xFF at row %lld block %lld", (long long)r, (long long)b);
        sc[b] = e;
      } else {
        const uint16_t h = static_cast<const uint16_t*>(scales)[r * nb + b];
        if ((h & 0x7C00) == 0x7C00) QMOE_FAIL(QMOE_E_SCALE, "non-finite fp16 scale 0x%04x at row %lld block %lld", h, (long long)r, (long long)b);
        sc[2 * b] = (uint8_t)(h & 0xFF);
        sc[2 * b + 1] = (uint8_t)(h >> 8);
      }
    }
  }
  return QMOE_OK;
}

extern "C" int qmoe_unpack(int fmt, int64_t rows, int64_t k, const void* packed,
                           size_t packed_bytes, uint8_t* codes, void* scales) {
  clear_error();
  FormatInfo fi;
  int st = check_geometry(fmt, rows, k, &fi);
  if (st) return st;
  const int64_t nb = k / 32;
  const size_t row_bytes = (size_t)nb * fi.block_bytes;
  if ((rows * k > 0) && (!codes || !scales || !packed)) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (packed_bytes < (size_t)rows * row_bytes) QMOE_FAIL(QMOE_E_SIZE, "packed_bytes %zu too small", packed_bytes);
  const uint8_t* p = static_cast<const uint8_t*>(packed);
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* row = p + (size_t)r * row_bytes;
    const uint8_t* lo = row;
    const uint8_t* hi = row + nb * fi.lo_bytes;
    const uint8_t* sc = hi + nb * fi.hi_bytes;
    for (int64_t b = 0; b < nb; ++b) {
      for (int j = 0; j < 32; ++j) {
        int byte, shift;
        lo_pos(fmt, j, &byte, &shift);
        uint8_t v = (uint8_t)((lo[b * fi.lo_bytes + byte] >> shift) & (fmt == QMOE_FP4 ? 0xF : 0x3));
        if (fmt == QMOE_FP3) v |= (uint8_t)(((hi[b * 4 + (j & 3)] >> (j >> 2)) & 1) << 2);
        codes[r * k + b * 32 + j] = v;
      }
      if (fmt == QMOE_FP4)
        static_cast<uint8_t*>(scales)[r * nb + b] = sc[b];
      else
        static_cast<uint16_t*>(scales)[r * nb + b] = (uint16_t)(sc[2 * b] | (sc[2 * b + 1] << 8));
    }
  }
  return QMOE_OK;
}
