// HIP kernels (gfx950, wave64) and launch entry points of libqmoe.
//
// Page citations:
//   [Strix-284B] lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
//     AMD Ryzen AI MAX+ 395": section "ROCmFPX: fitting 284B weights into 128 GB"
//     (packed blocks read directly, codebooks expanded in registers by byte
//     permutes, integer dot products; decode is memory-traffic bound) and
//     section "Decode: up to 32 tok/s" (q = 4 verification columns, each packed
//     weight decoded once for all columns; dedicated top-k routing kernels).
//   [0731-Strix] lucebox.com, "Lucebox × Geometric: DeepSeek V4 Flash 0731
//     reaches 32.7 tok/s on AMD Strix Halo": sections "How the model fits on AMD
//     Strix Halo" (gate/up 2.5 bpw, down 3.5 bpw, per-expert codebooks),
//     "Run with Lucebox Engine" (256 experts, 6 routed) and "Lucebox Engine
//     integration with Geometric" (sync-free MoE decode path).
//   [evox3] soothill.io, "DeepSeek V4 Flash 0731 on evox3", table "The
//     optimization ladder" (shared H32 input; layer-major prefill batching).
//
// Decode data flow (no host synchronisation anywhere):
//   k_quant_act    x fp32 -> xq int8 + dx fp32 per 32-block (shared by all experts)
//   k_router       fp64 logits in a fixed order (one wave per expert)
//   k_topk         top-k, softmax, and the decode plan: the union of the experts
//                  chosen by the q tokens, ascending, with a column mask each
//   k_gateup       per (expert, 32 rows): gate and up rows streamed once, each
//                  block expanded once for every column routed to the expert,
//                  SwiGLU, requantization of the 32-row block (+ optional H32)
//   k_down         per row group: every selected expert's down row, combined in
//                  ascending expert id with the routing weights
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "qmoe_device.h"
#include "qmoe_internal.h"

using namespace qk;
using qmoe::FormatInfo;
using qmoe::format_info;
using qmoe::clear_error;
using qmoe::round_up;

namespace {

constexpr int kPlanMax = 32;          // max distinct experts in one decode call (4 x 8)
// plan words: [0] U, [1..32] expert ids, [33..64] column masks, floats at word 128: w[32][4]
constexpr int kPlanMaskOff = 1 + kPlanMax;
constexpr int kPlanWOff = 128;

// ------------------------------------------------------------ activation quantization
__global__ __launch_bounds__(256) void k_quant_act(const float* __restrict__ x, int64_t nblocks, int rot,
                                                   int8_t* __restrict__ xq, float* __restrict__ dx) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  const float4* src = reinterpret_cast<const float4*>(x + b * 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 f = src[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  uint32_t q[8];
  float d;
  quant_block32(v, rot, q, &d);
  uint4* dst = reinterpret_cast<uint4*>(xq + b * 32);
  dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
  dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
  dx[b] = d;
}

// ------------------------------------------------------------ router logits
// One wave per (expert, group of up to TT tokens). Lane l holds blocks l + 64c.
// Per block: sequential fp64 sum of the 32 exact products; then the stride-
// halving tree: in-lane stages (stride >= 64 blocks) then xor-butterfly stages
// 32..1 across lanes (lane j + lane j^m equals s_j + s_{j+m} for j < m).
constexpr int kRouterMaxC = 8;   // hidden <= 32 * 64 * 8 = 16384

template <int TT>
__global__ __launch_bounds__(256) void k_router(const uint16_t* __restrict__ W, const float* __restrict__ x, int ntok,
                                                int E, int H, const double* __restrict__ bias,
                                                double* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  const int t0 = blockIdx.y * TT;
  const int nb = H >> 5;
  int P2 = 1;
  while (P2 < nb) P2 <<= 1;
  const int C = P2 > 64 ? P2 / 64 : 1;
  double s[TT][kRouterMaxC];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int c = 0; c < kRouterMaxC; ++c) s[t][c] = 0.0;
#pragma unroll
  for (int c = 0; c < kRouterMaxC; ++c) {
    const int b = lane + 64 * c;
    if (c < C && b < nb) {
      const uint4* wp = reinterpret_cast<const uint4*>(W + (size_t)e * H + (size_t)b * 32);
      uint32_t wv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 u = wp[i];
        wv[4 * i] = u.x; wv[4 * i + 1] = u.y; wv[4 * i + 2] = u.z; wv[4 * i + 3] = u.w;
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (t0 + t < ntok) {
          const float4* xp = reinterpret_cast<const float4*>(x + (size_t)(t0 + t) * H + (size_t)b * 32);
          double acc = 0.0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float4 f = xp[i];
            const float xs[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int j = 4 * i + k;
              const uint32_t hb = (j & 1) ? (wv[j >> 1] >> 16) : (wv[j >> 1] & 0xFFFFu);
              // the product of an fp16 and an fp32 is exact in fp64: fma == mul + add
              acc = fma((double)half_bits_to_float(hb), (double)xs[k], acc);
            }
          }
          s[t][c] = acc;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
#pragma unroll
    for (int n = kRouterMaxC / 2; n >= 1; n >>= 1)
      if (n < C)
#pragma unroll
        for (int c = 0; c < n; ++c) s[t][c] = s[t][c] + s[t][c + n];
    double v = s[t][0];
    for (int m = 32; m >= 1; m >>= 1)
      if (m < P2) v = v + __shfl_xor(v, m);
    if (lane == 0 && t0 + t < ntok) logits[(size_t)(t0 + t) * E + e] = bias ? v + bias[e] : v;
  }
}

// ------------------------------------------------------------ top-k (+ decode plan)
// One wave per token. Ties go to the lower id. Output ids ascending; softmax over
// the selected logits in fp64 (sum in ascending id order).
__device__ __forceinline__ bool better(double av, int ai, double bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

constexpr int kTopkMaxPerLane = 16;   // E <= 1024

__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int ntok, int E, int K,
                                              int32_t* __restrict__ idx, float* __restrict__ gw,
                                              int32_t* __restrict__ plan) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  __shared__ int s_ids[4][8];
  __shared__ float s_w[4][8];
  if (t < ntok) {
    const double* row = logits + (size_t)t * E;
    double v[kTopkMaxPerLane];
#pragma unroll
    for (int j = 0; j < kTopkMaxPerLane; ++j) {
      const int e = lane + 64 * j;
      v[j] = (e < E) ? row[e] : -INFINITY;
    }
    uint32_t taken = 0;
    int sel[8];
    for (int k = 0; k < K; ++k) {
      double bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < kTopkMaxPerLane; ++j) {
        const int e = lane + 64 * j;
        if (e < E && !(taken >> j & 1) && better(v[j], e, bv, bi)) {
          bv = v[j];
          bi = e;
        }
      }
      for (int m = 32; m >= 1; m >>= 1) {
        const double ov = __shfl_xor(bv, m);
        const int oi = __shfl_xor(bi, m);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      sel[k] = bi;
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
    // ascending ids (K <= 8)
    for (int a = 1; a < K; ++a) {
      const int key = sel[a];
      int b = a - 1;
      while (b >= 0 && sel[b] > key) {
        sel[b + 1] = sel[b];
        --b;
      }
      sel[b + 1] = key;
    }
    if (lane == 0) {
      double m = -INFINITY;
      for (int k = 0; k < K; ++k) m = fmax(m, row[sel[k]]);
      double ex[8], S = 0.0;
      for (int k = 0; k < K; ++k) {
        ex[k] = exp(row[sel[k]] - m);
        S = S + ex[k];
      }
      for (int k = 0; k < K; ++k) {
        const float g = (float)(ex[k] / S);
        idx[(size_t)t * K + k] = sel[k];
        gw[(size_t)t * K + k] = g;
        if (wave < 4) {
          s_ids[wave][k] = sel[k];
          s_w[wave][k] = g;
        }
      }
    }
  }
  if (plan == nullptr) return;
  // Decode plan (launched as one workgroup with ntok <= 4): union of the chosen
  // experts in ascending id, a column mask and the routing weight per column.
  __syncthreads();
  if (threadIdx.x == 0) {
    int U = 0;
    int ids[kPlanMax];
    uint32_t mask[kPlanMax];
    float w[kPlanMax][4];
    for (int tt = 0; tt < ntok; ++tt)
      for (int k = 0; k < K; ++k) {
        const int e = s_ids[tt][k];
        int u = 0;
        while (u < U && ids[u] != e) ++u;
        if (u == U) {
          ids[U] = e;
          mask[U] = 0;
          for (int c = 0; c < 4; ++c) w[U][c] = 0.0f;
          ++U;
        }
        mask[u] |= 1u << tt;
        w[u][tt] = s_w[tt][k];
      }
    // sort by expert id (stable insertion sort; U <= 32)
    for (int a = 1; a < U; ++a) {
      int b = a - 1;
      const int ke = ids[a];
      const uint32_t km = mask[a];
      float kw[4] = {w[a][0], w[a][1], w[a][2], w[a][3]};
      while (b >= 0 && ids[b] > ke) {
        ids[b + 1] = ids[b];
        mask[b + 1] = mask[b];
        for (int c = 0; c < 4; ++c) w[b + 1][c] = w[b][c];
        --b;
      }
      ids[b + 1] = ke;
      mask[b + 1] = km;
      for (int c = 0; c < 4; ++c) w[b + 1][c] = kw[c];
    }
    plan[0] = U;
    float* pw = reinterpret_cast<float*>(plan + kPlanWOff);
    for (int u = 0; u < kPlanMax; ++u) {
      plan[1 + u] = u < U ? ids[u] : -1;
      plan[kPlanMaskOff + u] = u < U ? (int)mask[u] : 0;
      for (int c = 0; c < 4; ++c) pw[4 * u + c] = u < U ? w[u][c] : 0.0f;
    }
  }
}

// ------------------------------------------------------------ decode: gate/up + SwiGLU + requant
// Workgroup = 4 waves = 32 consecutive rows of one selected expert (one block of
// the down projection's input); each wave owns 8 rows of both gate and up.
// Lanes cover NBL consecutive blocks each; the token activations for the lane's
// blocks stay in registers across the wave's rows.
constexpr int kGU_RowsPerWave = 8;

template <int FMT, int Q>
__global__ __launch_bounds__(256) void k_gateup(const uint8_t* __restrict__ gate, const uint8_t* __restrict__ up,
                                                size_t expert_stride, size_t row_bytes, int nb,
                                                const int8_t* __restrict__ cb_gate, const int8_t* __restrict__ cb_up,
                                                const int8_t* __restrict__ xq, const float* __restrict__ dx,
                                                const int32_t* __restrict__ plan, int rot_down, int inter,
                                                int8_t* __restrict__ hq, float* __restrict__ dh) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  const int u = blockIdx.y;
  const int U = plan[0];
  if (u >= U) return;
  const int e = plan[1 + u];
  const uint32_t mask = (uint32_t)plan[kPlanMaskOff + u];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = blockIdx.x * 32 + wave * kGU_RowsPerWave;
  const uint8_t* gbase = gate + (size_t)e * expert_stride;
  const uint8_t* ubase = up + (size_t)e * expert_stride;
  uint32_t cbg[4], cbu[4];
  load_codebook<FMT>(cb_gate + ((size_t)e << FMT), cbg);
  load_codebook<FMT>(cb_up + ((size_t)e << FMT), cbu);

  float ag[kGU_RowsPerWave][Q], au[kGU_RowsPerWave][Q];
#pragma unroll
  for (int r = 0; r < kGU_RowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < Q; ++t) ag[r][t] = au[r][t] = 0.0f;

  for (int c0 = 0; c0 < nb; c0 += 64 * NBL) {
    const int b = c0 + lane * NBL;
    if (b < nb) {
      Acts<NBL> act[Q];
#pragma unroll
      for (int t = 0; t < Q; ++t)
        if (mask >> t & 1) act[t].load(xq + (size_t)t * nb * 32, dx + (size_t)t * nb, b);
#pragma unroll
      for (int r = 0; r < kGU_RowsPerWave; ++r) {
        Blocks<FMT, NBL> bg, bu;
        bg.load(gbase + (size_t)(row0 + r) * row_bytes, nb, b);
        bu.load(ubase + (size_t)(row0 + r) * row_bytes, nb, b);
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
          uint32_t wg[8], wu[8];
          bg.expand(i, cbg, wg);
          bu.expand(i, cbu, wu);
#pragma unroll
          for (int t = 0; t < Q; ++t) {
            if (mask >> t & 1) {
              const int pg = block_dot(wg, act[t].q[i]);
              const int pu = block_dot(wu, act[t].q[i]);
              ag[r][t] = fmaf((float)pg, bg.s[i] * act[t].d[i], ag[r][t]);
              au[r][t] = fmaf((float)pu, bu.s[i] * act[t].d[i], au[r][t]);
            }
          }
        }
      }
    }
  }
  __shared__ float a_lds[4][32];
#pragma unroll
  for (int r = 0; r < kGU_RowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      if (mask >> t & 1) {
        const float g = group_sum(ag[r][t], 64);
        const float uu = group_sum(au[r][t], 64);
        if (lane == 0) a_lds[t][wave * kGU_RowsPerWave + r] = g / (1.0f + expf(-g)) * uu;
      }
    }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < Q && (mask >> t & 1)) {
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = a_lds[t][j];
    uint32_t q[8];
    float d;
    quant_block32(v, rot_down, q, &d);
    const size_t slot = (size_t)u * 4 + t;
    uint4* dst = reinterpret_cast<uint4*>(hq + slot * inter + (size_t)blockIdx.x * 32);
    dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
    dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
    dh[slot * (inter / 32) + blockIdx.x] = d;
  }
}

// ------------------------------------------------------------ decode: down + combine
// Each wave handles 64/LPR rows at once (LPR lanes per row, NBL blocks per lane)
// for every selected expert, accumulating g_e * y_e per lane in ascending expert
// order, then one group reduction per (row, column).
template <int FMT, int Q>
__global__ __launch_bounds__(256) void k_down(const uint8_t* __restrict__ down, size_t expert_stride,
                                              size_t row_bytes, int nb, int lpr_log2,
                                              const int8_t* __restrict__ cb_down, const int8_t* __restrict__ hq,
                                              const float* __restrict__ dh, const int32_t* __restrict__ plan,
                                              int hidden, int inter, float* __restrict__ out) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  const int lpr = 1 << lpr_log2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int rows_per_wave = 64 >> lpr_log2;
  const int row = (blockIdx.x * 4 + wave) * rows_per_wave + sub;
  const bool row_ok = row < hidden;
  const int U = plan[0];
  const float* pw = reinterpret_cast<const float*>(plan + kPlanWOff);
  float acc[Q];
#pragma unroll
  for (int t = 0; t < Q; ++t) acc[t] = 0.0f;
  for (int u = 0; u < U; ++u) {
    const int e = plan[1 + u];
    const uint32_t mask = (uint32_t)plan[kPlanMaskOff + u];
    uint32_t cb[4];
    load_codebook<FMT>(cb_down + ((size_t)e << FMT), cb);
    const uint8_t* rowp = down + (size_t)e * expert_stride + (size_t)row * row_bytes;
    float accu[Q];
#pragma unroll
    for (int t = 0; t < Q; ++t) accu[t] = 0.0f;
    for (int c0 = 0; c0 < nb; c0 += lpr * NBL) {
      const int b = c0 + sl * NBL;
      if (row_ok && b < nb) {
        Blocks<FMT, NBL> bl;
        bl.load(rowp, nb, b);
        Acts<NBL> act[Q];
#pragma unroll
        for (int t = 0; t < Q; ++t)
          if (mask >> t & 1) {
            const size_t slot = (size_t)u * 4 + t;
            act[t].load(hq + slot * inter, dh + slot * (inter / 32), b);
          }
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
          uint32_t w[8];
          bl.expand(i, cb, w);
#pragma unroll
          for (int t = 0; t < Q; ++t)
            if (mask >> t & 1) {
              const int p = block_dot(w, act[t].q[i]);
              accu[t] = fmaf((float)p, bl.s[i] * act[t].d[i], accu[t]);
            }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < Q; ++t)
      if (mask >> t & 1) acc[t] = fmaf(pw[4 * u + t], accu[t], acc[t]);
  }
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    const float v = group_sum(acc[t], lpr);
    if (sl == 0 && row_ok) out[(size_t)t * hidden + row] = v;
  }
}

// ------------------------------------------------------------ dense matvec (1..4 columns)
template <int FMT, int Q>
__global__ __launch_bounds__(256) void k_matvec(const uint8_t* __restrict__ W, int64_t rows, size_t row_bytes, int nb,
                                                int lpr_log2, const int8_t* __restrict__ cbp,
                                                const int8_t* __restrict__ xq, const float* __restrict__ dx,
                                                float* __restrict__ y) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  const int lpr = 1 << lpr_log2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int rows_per_wave = 64 >> lpr_log2;
  const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * rows_per_wave + sub;
  const bool row_ok = row < rows;
  uint32_t cb[4];
  load_codebook<FMT>(cbp, cb);
  float acc[Q];
#pragma unroll
  for (int t = 0; t < Q; ++t) acc[t] = 0.0f;
  const uint8_t* rowp = W + (size_t)row * row_bytes;
  for (int c0 = 0; c0 < nb; c0 += lpr * NBL) {
    const int b = c0 + sl * NBL;
    if (row_ok && b < nb) {
      Blocks<FMT, NBL> bl;
      bl.load(rowp, nb, b);
      Acts<NBL> act[Q];
#pragma unroll
      for (int t = 0; t < Q; ++t) act[t].load(xq + (size_t)t * nb * 32, dx + (size_t)t * nb, b);
#pragma unroll
      for (int i = 0; i < NBL; ++i) {
        uint32_t w[8];
        bl.expand(i, cb, w);
#pragma unroll
        for (int t = 0; t < Q; ++t) {
          const int p = block_dot(w, act[t].q[i]);
          acc[t] = fmaf((float)p, bl.s[i] * act[t].d[i], acc[t]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    const float v = group_sum(acc[t], lpr);
    if (sl == 0 && row_ok) y[(size_t)t * rows + row] = v;
  }
}

// ------------------------------------------------------------ per-block integer sums (test entry)
template <int FMT>
__global__ __launch_bounds__(256) void k_block_dots(const uint8_t* __restrict__ W, int64_t rows, size_t row_bytes,
                                                    int nb, const int8_t* __restrict__ cbp,
                                                    const int8_t* __restrict__ xq, int32_t* __restrict__ P) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * nb) return;
  const int64_t r = i / nb;
  const int b = (int)(i % nb);
  uint32_t cb[4];
  load_codebook<FMT>(cbp, cb);
  Blocks<FMT, 1> bl;
  bl.load(W + (size_t)r * row_bytes, nb, b);
  const uint4* p = reinterpret_cast<const uint4*>(xq + (size_t)b * 32);
  uint4 a = p[0], c = p[1];
  const uint32_t x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  uint32_t w[8];
  bl.expand(0, cb, w);
  P[i] = block_dot(w, x);
}

}  // namespace

// ============================================================ host side

namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int launch_check(const char* what) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) QMOE_FAIL(QMOE_E_HIP, "%s: %s", what, hipGetErrorString(err));
  return QMOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ilog2(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) ++l;
  return l;
}

// lanes per row for a row of nb blocks processed NBL at a time: the largest power
// of two <= nb/NBL, at most 64 and at least 1.
int lanes_per_row(int nb, int nbl) {
  int chunks = (nb + nbl - 1) / nbl;
  int l = 1;
  while (l * 2 <= chunks && l < 64) l *= 2;
  return l;
}

int launch_quant(const float* x, int64_t nblocks, int rot, int8_t* xq, float* dx, hipStream_t s) {
  if (nblocks == 0) return QMOE_OK;
  const int threads = 256;
  const unsigned grid = (unsigned)((nblocks + threads - 1) / threads);
  hipLaunchKernelGGL(k_quant_act, dim3(grid), dim3(threads), 0, s, x, nblocks, rot, xq, dx);
  return launch_check("quant_act");
}

template <int FMT, int Q>
void launch_matvec_t(const uint8_t* W, int64_t rows, size_t row_bytes, int nb, int lpr_log2, const int8_t* cb,
                     const int8_t* xq, const float* dx, float* y, hipStream_t s) {
  const int rows_per_wg = 4 * (64 >> lpr_log2);
  const unsigned grid = (unsigned)((rows + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((k_matvec<FMT, Q>), dim3(grid), dim3(256), 0, s, W, rows, row_bytes, nb, lpr_log2, cb, xq, dx, y);
}

template <int FMT>
void launch_matvec_f(int q, const uint8_t* W, int64_t rows, size_t row_bytes, int nb, int lpr_log2,
                     const int8_t* cb, const int8_t* xq, const float* dx, float* y, hipStream_t s) {
  switch (q) {
    case 1: launch_matvec_t<FMT, 1>(W, rows, row_bytes, nb, lpr_log2, cb, xq, dx, y, s); break;
    case 2: launch_matvec_t<FMT, 2>(W, rows, row_bytes, nb, lpr_log2, cb, xq, dx, y, s); break;
    case 3: launch_matvec_t<FMT, 3>(W, rows, row_bytes, nb, lpr_log2, cb, xq, dx, y, s); break;
    default: launch_matvec_t<FMT, 4>(W, rows, row_bytes, nb, lpr_log2, cb, xq, dx, y, s); break;
  }
}

int check_matrix(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes, const int8_t* cb, FormatInfo* fi) {
  if (!format_info(fmt, fi)) QMOE_FAIL(QMOE_E_FORMAT, "unknown format %d", fmt);
  if (rows < 0 || k <= 0 || k % 32) QMOE_FAIL(QMOE_E_SHAPE, "rows=%lld k=%lld (k must be a positive multiple of 32)",
                                            (long long)rows, (long long)k);
  const size_t row_bytes = (size_t)(k / 32) * fi->block_bytes;
  if (row_bytes % 16)
    QMOE_FAIL(QMOE_E_SHAPE, "row of %zu bytes not a multiple of 16 (k must be a multiple of %d for FP%d)", row_bytes,
              fmt == 4 ? 512 : 256, fmt);
  if (k / 32 > 0x7FFFFFFF) QMOE_FAIL(QMOE_E_SHAPE, "k too large");
  if (!w) QMOE_FAIL(QMOE_E_INVAL, "missing weights (NULL)");
  if (!aligned16(w)) QMOE_FAIL(QMOE_E_INVAL, "weights not 16-byte aligned");
  if (w_bytes < (size_t)rows * row_bytes) QMOE_FAIL(QMOE_E_SIZE, "%zu weight bytes < %zu", w_bytes, (size_t)rows * row_bytes);
  if (!cb) QMOE_FAIL(QMOE_E_CODEBOOK, "missing codebook (NULL)");
  if (reinterpret_cast<uintptr_t>(cb) & 3) QMOE_FAIL(QMOE_E_INVAL, "codebook not 4-byte aligned");
  return QMOE_OK;
}

struct WsPtrs {
  uint32_t* ctrl;
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
};

int ws_ptrs(const qmoe_layer* L, int32_t ntok, void* ws, size_t ws_bytes, WsPtrs* p) {
  qmoe_ws_layout lay;
  int st = qmoe_workspace_layout(L, ntok, &lay);
  if (st) return st;
  if (!ws) QMOE_FAIL(QMOE_E_WORKSPACE, "missing workspace (NULL)");
  if (!aligned16(ws)) QMOE_FAIL(QMOE_E_WORKSPACE, "workspace not 16-byte aligned");
  if (ws_bytes < lay.total) QMOE_FAIL(QMOE_E_WORKSPACE, "workspace %zu bytes < %zu required for %d tokens", ws_bytes,
                                      lay.total, ntok);
  uint8_t* b = static_cast<uint8_t*>(ws);
  p->ctrl = reinterpret_cast<uint32_t*>(b + lay.ctrl);
  p->xq = reinterpret_cast<int8_t*>(b + lay.xq);
  p->dx = reinterpret_cast<float*>(b + lay.dx);
  p->idx = reinterpret_cast<int32_t*>(b + lay.idx);
  p->gw = reinterpret_cast<float*>(b + lay.gw);
  p->logits = reinterpret_cast<double*>(b + lay.logits);
  p->plan = reinterpret_cast<int32_t*>(b + lay.plan);
  p->hq = reinterpret_cast<int8_t*>(b + lay.hq);
  p->dh = reinterpret_cast<float*>(b + lay.dh);
  p->group = b + lay.group;
  p->ypair = reinterpret_cast<float*>(b + lay.ypair);
  return QMOE_OK;
}

int launch_router(const qmoe_layer* L, const float* x, int32_t ntok, double* logits, hipStream_t s) {
  if (L->hidden > 32 * 64 * kRouterMaxC) QMOE_FAIL(QMOE_E_SHAPE, "hidden=%d exceeds router limit %d", L->hidden, 32 * 64 * kRouterMaxC);
  dim3 grid((L->n_experts + 3) / 4, (ntok + 3) / 4);
  hipLaunchKernelGGL(k_router<4>, grid, dim3(256), 0, s, L->w_router, x, ntok, L->n_experts, L->hidden,
                     L->router_bias, logits);
  return launch_check("router");
}

int launch_topk(const qmoe_layer* L, const double* logits, int32_t ntok, int32_t* idx, float* gw, int32_t* plan,
                hipStream_t s) {
  dim3 grid((ntok + 3) / 4);
  hipLaunchKernelGGL(k_topk, grid, dim3(256), 0, s, logits, ntok, L->n_experts, L->topk, idx, gw, plan);
  return launch_check("topk");
}

template <int FMT, int Q>
void launch_gateup_t(const qmoe_layer* L, const WsPtrs& w, int U_max, hipStream_t s) {
  const int nb = L->hidden / 32;
  const size_t row_bytes = (size_t)nb * Fmt<FMT>::kBlockBytes;
  const size_t stride = row_bytes * L->inter;
  dim3 grid(L->inter / 32, U_max);
  hipLaunchKernelGGL((k_gateup<FMT, Q>), grid, dim3(256), 0, s, static_cast<const uint8_t*>(L->gate),
                     static_cast<const uint8_t*>(L->up), stride, row_bytes, nb, L->cb_gate, L->cb_up, w.xq, w.dx,
                     w.plan, L->rot_down, L->inter, w.hq, w.dh);
}

template <int FMT, int Q>
void launch_down_t(const qmoe_layer* L, const WsPtrs& w, float* out, hipStream_t s) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  const int nb = L->inter / 32;
  const size_t row_bytes = (size_t)nb * Fmt<FMT>::kBlockBytes;
  const size_t stride = row_bytes * L->hidden;
  const int lpr = lanes_per_row(nb, NBL);
  const int lg = ilog2(lpr);
  const int rows_per_wg = 4 * (64 >> lg);
  dim3 grid((L->hidden + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((k_down<FMT, Q>), grid, dim3(256), 0, s, static_cast<const uint8_t*>(L->down), stride, row_bytes,
                     nb, lg, L->cb_down, w.hq, w.dh, w.plan, L->hidden, L->inter, out);
}

template <int Q>
int launch_decode_experts(const qmoe_layer* L, const WsPtrs& w, float* out, hipStream_t s) {
  const int U_max = std::min(Q * L->topk, L->n_experts);
  switch (L->fmt_gate) {
    case 2: launch_gateup_t<2, Q>(L, w, U_max, s); break;
    case 3: launch_gateup_t<3, Q>(L, w, U_max, s); break;
    default: launch_gateup_t<4, Q>(L, w, U_max, s); break;
  }
  int st = launch_check("gateup");
  if (st) return st;
  switch (L->fmt_down) {
    case 2: launch_down_t<2, Q>(L, w, out, s); break;
    case 3: launch_down_t<3, Q>(L, w, out, s); break;
    default: launch_down_t<4, Q>(L, w, out, s); break;
  }
  return launch_check("down");
}

}  // namespace

extern "C" int qmoe_quant_act(const float* x, int64_t n_vec, int64_t k, int32_t rot, int8_t* xq, float* dx,
                              void* stream) {
  clear_error();
  if (rot != 0 && rot != 1) QMOE_FAIL(QMOE_E_FORMAT, "rot=%d unsupported (0 or 1)", rot);
  if (n_vec < 0 || k <= 0 || k % 32) QMOE_FAIL(QMOE_E_SHAPE, "n_vec=%lld k=%lld", (long long)n_vec, (long long)k);
  if (n_vec == 0) return QMOE_OK;
  if (!x || !xq || !dx) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(x) || !aligned16(xq) || (reinterpret_cast<uintptr_t>(dx) & 3))
    QMOE_FAIL(QMOE_E_INVAL, "x and xq must be 16-byte aligned, dx 4-byte aligned");
  return launch_quant(x, n_vec * (k / 32), rot, xq, dx, as_stream(stream));
}

extern "C" int qmoe_block_dots(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes, const int8_t* cb,
                               const int8_t* xq, int32_t* P, void* stream) {
  clear_error();
  FormatInfo fi;
  int st = check_matrix(fmt, rows, k, w, w_bytes, cb, &fi);
  if (st) return st;
  if (rows == 0) return QMOE_OK;
  if (!xq || !P) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(xq)) QMOE_FAIL(QMOE_E_INVAL, "xq not 16-byte aligned");
  const int nb = (int)(k / 32);
  const size_t row_bytes = (size_t)nb * fi.block_bytes;
  const int64_t n = rows * nb;
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipStream_t s = as_stream(stream);
  const uint8_t* W = static_cast<const uint8_t*>(w);
  switch (fmt) {
    case 2: hipLaunchKernelGGL(k_block_dots<2>, dim3(grid), dim3(256), 0, s, W, rows, row_bytes, nb, cb, xq, P); break;
    case 3: hipLaunchKernelGGL(k_block_dots<3>, dim3(grid), dim3(256), 0, s, W, rows, row_bytes, nb, cb, xq, P); break;
    default: hipLaunchKernelGGL(k_block_dots<4>, dim3(grid), dim3(256), 0, s, W, rows, row_bytes, nb, cb, xq, P); break;
  }
  return launch_check("block_dots");
}

extern "C" int qmoe_matvec(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes, const int8_t* cb,
                           int32_t rot, const float* x, int32_t ncols, float* y, void* ws, size_t ws_bytes,
                           void* stream) {
  clear_error();
  FormatInfo fi;
  int st = check_matrix(fmt, rows, k, w, w_bytes, cb, &fi);
  if (st) return st;
  if (rot != 0 && rot != 1) QMOE_FAIL(QMOE_E_FORMAT, "rot=%d unsupported (0 or 1)", rot);
  if (ncols < 1 || ncols > 4) QMOE_FAIL(QMOE_E_SHAPE, "ncols=%d outside 1..4", ncols);
  if (!x || !y) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(x)) QMOE_FAIL(QMOE_E_INVAL, "x not 16-byte aligned");
  const size_t need = qmoe_matvec_workspace_bytes(k, ncols);
  if (!ws) QMOE_FAIL(QMOE_E_WORKSPACE, "missing workspace (NULL)");
  if (!aligned16(ws)) QMOE_FAIL(QMOE_E_WORKSPACE, "workspace not 16-byte aligned");
  if (ws_bytes < need) QMOE_FAIL(QMOE_E_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if (rows == 0) return QMOE_OK;
  int8_t* xq = static_cast<int8_t*>(ws);
  float* dx = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + round_up((size_t)ncols * k, 256));
  hipStream_t s = as_stream(stream);
  const int nb = (int)(k / 32);
  if ((st = launch_quant(x, (int64_t)ncols * nb, rot, xq, dx, s))) return st;
  const int nbl = fmt == 4 ? 1 : 2;
  const int lg = ilog2(lanes_per_row(nb, nbl));
  const size_t row_bytes = (size_t)nb * fi.block_bytes;
  const uint8_t* W = static_cast<const uint8_t*>(w);
  switch (fmt) {
    case 2: launch_matvec_f<2>(ncols, W, rows, row_bytes, nb, lg, cb, xq, dx, y, s); break;
    case 3: launch_matvec_f<3>(ncols, W, rows, row_bytes, nb, lg, cb, xq, dx, y, s); break;
    default: launch_matvec_f<4>(ncols, W, rows, row_bytes, nb, lg, cb, xq, dx, y, s); break;
  }
  return launch_check("matvec");
}

extern "C" int qmoe_route(const qmoe_layer* L, const float* x, int32_t ntok, int32_t* idx, float* gate_w, void* ws,
                          size_t ws_bytes, void* stream) {
  clear_error();
  if (ntok < 0) QMOE_FAIL(QMOE_E_SHAPE, "ntok=%d", ntok);
  WsPtrs w;
  int st = ws_ptrs(L, ntok > 0 ? ntok : 1, ws, ws_bytes, &w);
  if (st) return st;
  if (ntok == 0) return QMOE_OK;
  if (!x || !idx || !gate_w) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(x)) QMOE_FAIL(QMOE_E_INVAL, "x not 16-byte aligned");
  hipStream_t s = as_stream(stream);
  if ((st = launch_router(L, x, ntok, w.logits, s))) return st;
  return launch_topk(L, w.logits, ntok, idx, gate_w, nullptr, s);
}

extern "C" int qmoe_decode_layer(const qmoe_layer* L, const float* x, int32_t q, float* out, void* ws,
                                 size_t ws_bytes, void* stream) {
  clear_error();
  if (q < 1 || q > 4) QMOE_FAIL(QMOE_E_SHAPE, "q=%d outside 1..4", q);
  WsPtrs w;
  int st = ws_ptrs(L, q, ws, ws_bytes, &w);
  if (st) return st;
  if (!x || !out) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(x)) QMOE_FAIL(QMOE_E_INVAL, "x not 16-byte aligned");
  hipStream_t s = as_stream(stream);
  if ((st = launch_quant(x, (int64_t)q * (L->hidden / 32), L->rot_gateup, w.xq, w.dx, s))) return st;
  if ((st = launch_router(L, x, q, w.logits, s))) return st;
  // one workgroup: top-k for the q tokens, then the expert union plan
  hipLaunchKernelGGL(k_topk, dim3(1), dim3(256), 0, s, w.logits, q, L->n_experts, L->topk, w.idx, w.gw, w.plan);
  if ((st = launch_check("topk+plan"))) return st;
  switch (q) {
    case 1: return launch_decode_experts<1>(L, w, out, s);
    case 2: return launch_decode_experts<2>(L, w, out, s);
    case 3: return launch_decode_experts<3>(L, w, out, s);
    default: return launch_decode_experts<4>(L, w, out, s);
  }
}

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
