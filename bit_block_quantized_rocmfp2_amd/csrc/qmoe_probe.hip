// Measurement probes (gfx950): the denominators the layer kernels are put
// against. None of them is a step of the layer.
//
//   k_probe_read   a read-only HBM stream: each workgroup reads one contiguous
//                  share of the buffer with 16-byte loads, four in flight per
//                  lane, and folds the words into a checksum (so no load is
//                  dead). Timed over a buffer much larger than the 256 MB last-
//                  level cache it gives the sustained read rate; one launch on
//                  a cold buffer of B bytes gives the fixed cost of a streaming
//                  launch plus B over that rate.
//   k_probe_mfma   int8 matrix-core throughput alone: four independent
//                  accumulation chains of one MFMA form per wave, operands in
//                  registers.
//   k_probe_valu   the vector-ALU rate of the prefill GEMMs' per-block epilogue
//                  (int32 -> fp32 convert, fused multiply-add), 16 independent
//                  values per lane.
//
// The pages measure decode as bound by memory traffic (lucebox.com, "DeepSeek
// V4 Flash: 284B model, up to 32 tok/s on AMD Ryzen AI MAX+ 395", section
// "ROCmFPX: fitting 284B weights into 128 GB") and report kernel measurements
// apart from end-to-end figures (lucebox.com, "Lucebox × Geometric: DeepSeek V4
// Flash 0731 reaches 32.7 tok/s on AMD Strix Halo", section "Lucebox Engine
// integration with Geometric"); these probes give the same split on MI355X.
#include <hip/hip_runtime.h>

#include "qmoe_device.h"
#include "qmoe_host.h"
#include "qmoe_internal.h"

using namespace qk;
using namespace qmoe;

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;
constexpr int kReadUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const u32x4* __restrict__ buf, size_t n16,
                                                             uint32_t* __restrict__ sink) {
  __shared__ uint32_t s_x[kProbeThreads / 64];
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  uint32_t x = 0;
  for (size_t i0 = beg + threadIdx.x; i0 < end; i0 += (size_t)kProbeThreads * kReadUnroll) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) {
      const size_t i = i0 + (size_t)k * kProbeThreads;
      v[k] = buf[i < end ? i : i0];   // i0 < end: every load stays inside the share
    }
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m);
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_x[0] ^ s_x[1] ^ s_x[2] ^ s_x[3];
}

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma(int iters, uint32_t* __restrict__ sink) {
  const int gid = blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t total = 0;
  if constexpr (KIND == 0) {
    const long a = (long)(0x0102030405060708ll * (gid + 1)), b = (long)(0x1112131415161718ll ^ gid);
    v4i c[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) total += (uint32_t)(c[j][0] + c[j][1] + c[j][2] + c[j][3]);
  } else {
    const v4i a = {gid, gid * 3, gid ^ 0x55, gid + 7}, b = {gid * 5, ~gid, gid ^ 0x33, gid - 9};
    v16i c[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) total += (uint32_t)c[j][r];
  }
  sink[gid] = total;
}

__global__ __launch_bounds__(kProbeThreads) void k_probe_valu(int iters, uint32_t* __restrict__ sink) {
  const int gid = blockIdx.x * kProbeThreads + threadIdx.x;
  int p[16];
  float s[16], acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    p[i] = gid * 17 + i * 1021;
    s[i] = 1.0f / (float)(i + 3);
    acc[i] = 0.0f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // the empty statement marks p[i] as rewritten, so the convert stays in the
      // loop, as it would for a fresh MFMA result (it emits no instruction)
      asm volatile("" : "+v"(p[i]));
      acc[i] = fmaf((float)p[i], s[i], acc[i]);
    }
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) t += acc[i];
  sink[gid] = __float_as_uint(t);
}

int probe_grid(int32_t grid) { return grid > 0 ? grid : 4 * device_cu_count(); }

}  // namespace

extern "C" int qmoe_probe_read(const void* buf, size_t bytes, int32_t grid, uint32_t* sink, void* stream) {
  clear_error();
  if (!buf || !sink) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(buf) || bytes % 16) QMOE_FAIL(QMOE_E_INVAL, "buffer not 16-byte aligned or bytes %% 16 != 0");
  if (grid < 0) QMOE_FAIL(QMOE_E_SHAPE, "grid=%d", grid);
  if (bytes == 0) return QMOE_OK;
  const int g = probe_grid(grid);
  launch_kernel("probe_read", k_probe_read, dim3(g), dim3(kProbeThreads), as_stream(stream),
                static_cast<const u32x4*>(buf), bytes / 16, sink);
  return launch_check("probe_read");
}

extern "C" int qmoe_probe_mfma(int32_t kind, int32_t iters, int32_t grid, uint32_t* sink, void* stream) {
  clear_error();
  if (!sink) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (kind != 0 && kind != 1) QMOE_FAIL(QMOE_E_INVAL, "kind=%d (0 or 1)", kind);
  if (iters < 1 || grid < 0) QMOE_FAIL(QMOE_E_SHAPE, "iters=%d grid=%d", iters, grid);
  const int g = probe_grid(grid);
  if (kind == 0)
    launch_kernel("probe_mfma", k_probe_mfma<0>, dim3(g), dim3(kProbeThreads), as_stream(stream), (int)iters, sink);
  else
    launch_kernel("probe_mfma", k_probe_mfma<1>, dim3(g), dim3(kProbeThreads), as_stream(stream), (int)iters, sink);
  return launch_check("probe_mfma");
}

extern "C" int qmoe_probe_valu(int32_t iters, int32_t grid, uint32_t* sink, void* stream) {
  clear_error();
  if (!sink) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (iters < 1 || grid < 0) QMOE_FAIL(QMOE_E_SHAPE, "iters=%d grid=%d", iters, grid);
  launch_kernel("probe_valu", k_probe_valu, dim3(probe_grid(grid)), dim3(kProbeThreads), as_stream(stream),
                (int)iters, sink);
  return launch_check("probe_valu");
}
