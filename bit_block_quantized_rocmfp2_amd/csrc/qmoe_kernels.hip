// Generic HIP kernels (gfx950, wave64) of libqmoe and their entry points:
// activation quantization, router + top-k, dense matvec, per-block dots; plus
// the shared host helpers (workspace carving, launch checks, kernel timing).
//
// Page citations:
//   [Strix-284B] lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
//     AMD Ryzen AI MAX+ 395": section "ROCmFPX: fitting 284B weights into 128 GB"
//     (packed blocks read directly; codebooks expanded in registers by byte
//     permutes feeding integer dot products; decode bound by memory traffic),
//     section "Decode: up to 32 tok/s" (q <= 4 columns, each packed weight
//     expanded once for every column; dedicated top-k routing kernels).
//   [0731-Strix] lucebox.com, "Lucebox × Geometric: DeepSeek V4 Flash 0731
//     reaches 32.7 tok/s on AMD Strix Halo", section "Run with Lucebox Engine"
//     (256 experts, 6 routed).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "qmoe_device.h"
#include "qmoe_host.h"
#include "qmoe_internal.h"

using namespace qk;
using namespace qmoe;

namespace {

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
// One wave per (expert, group of 4 tokens).
__global__ __launch_bounds__(256) void k_router(const uint16_t* __restrict__ W, const float* __restrict__ x, int ntok,
                                                int E, int H, const double* __restrict__ bias,
                                                double* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  const int t0 = blockIdx.y * 4;
  double lg[4];
  router_wave<4>(W, x, ntok, H, bias, e, t0, lane, lg);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (lane == 0 && t0 + t < ntok) logits[(size_t)(t0 + t) * E + e] = lg[t];
}

// ------------------------------------------------------------ router, many tokens
// A workgroup computes a 32-expert x 32-token tile of logits on the fp64 matrix
// cores, each logit in the same fixed order as the wave router: per 32-block a
// sequential fp64 sum of the exact fp16 x fp32 products, then the stride-halving
// tree over the (zero-padded) power-of-two block count. Wave w owns the 16 x 16
// subtile of experts 16 (w & 1).. and tokens 16 (w >> 1)... One
// v_mfma_f64_16x16x4f64 adds its four products to the accumulator one after the
// other in K order, each step rounded as a fused multiply-add (measured on the
// GPU on operands whose sum depends on the order; the tiled-logits parity tests
// hold every logit to the oracle's sequential order bit for bit), and operand
// lane l holds row (or column) l % 16 at K = l / 16; so a block is 8
// instructions, step s taking K = 4s + l / 16, from +0. Result register r of
// lane l is expert 4r + l / 16, token l % 16 of the subtile. The tree is
// evaluated depth first: its leaves are visited in bit-reversed order and
// partial sums are kept per level like the digits of a binary counter (level k
// holds a sum of 2^k leaves). Two leaves' MFMA chains run interleaved
// (independent sums; 0.60 -> 0.43 ms for 8192 tokens x 256 experts); four
// at once measured the same and needed more registers. Operands are staged in LDS as fp32, 4 leaves at a
// time (the fp16 weights widened exactly once per workgroup), and widened to
// fp64 at each use: exact, so the products are those of an all-fp64 evaluation.
typedef double v4d __attribute__((ext_vector_type(4)));
constexpr int kRtE = 32, kRtT = 32, kRtLeaves = 4;
constexpr int kRtStride = 36;   // floats per LDS row: a read's 16 rows x 4 K lanes fall in distinct banks
constexpr int kRtLevels = 9;    // up to 256 blocks (hidden <= 8192)

__device__ __forceinline__ int bit_reverse(int v, int bits) {
  return (int)(__builtin_bitreverse32((uint32_t)v) >> (32 - bits));
}

__global__ __launch_bounds__(256) void k_router_tiles(const uint16_t* __restrict__ W, const float* __restrict__ x,
                                                      int ntok, int E, int H, const double* __restrict__ bias,
                                                      double* __restrict__ logits) {
  __shared__ float s_w[kRtLeaves][kRtE][kRtStride];
  __shared__ float s_x[kRtLeaves][kRtT][kRtStride];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e_base = blockIdx.x * kRtE, t_base = blockIdx.y * kRtT;
  const int we = 16 * (wave & 1), wt = 16 * (wave >> 1);   // the wave's subtile
  const int row = lane & 15, kg = lane >> 4;                // operand row / column, K lane group
  const int nb = H >> 5;
  int L = 0;
  while ((1 << L) < nb) ++L;
  const int P2 = 1 << L;
  // loader mapping: row r (expert or token) = tid >> 3, 16 consecutive values of
  // one of the chunk's 4 leaves: leaf (tid >> 1) & 3, half tid & 1
  const int lr = tid >> 3, lk = (tid >> 1) & 3, lh = tid & 1;
  const int le = min(e_base + lr, E - 1), lt = min(t_base + lr, ntok - 1);
  double lvl[4][kRtLevels];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int k = 0; k < kRtLevels; ++k) lvl[c][k] = 0.0;
  for (int i0 = 0; i0 < P2; i0 += kRtLeaves) {
    {
      const int b = bit_reverse(i0 + lk, L);
      float wv[16];
      float4 xv[4];
      if (b < nb) {
        const u32x4* wp = reinterpret_cast<const u32x4*>(W + (size_t)le * H + (size_t)b * 32 + 16 * lh);
        const u32x4 u0 = wp[0], u1 = wp[1];
        const uint32_t hw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) wv[j] = half_bits_to_float((hw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
        const float4* xp = reinterpret_cast<const float4*>(x + (size_t)lt * H + (size_t)b * 32 + 16 * lh);
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = xp[j];
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) wv[j] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
      __syncthreads();   // the previous chunk's reads are done
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<float4*>(&s_w[lk][lr][16 * lh + 4 * j]) =
            make_float4(wv[4 * j], wv[4 * j + 1], wv[4 * j + 2], wv[4 * j + 3]);
        *reinterpret_cast<float4*>(&s_x[lk][lr][16 * lh + 4 * j]) = xv[j];
      }
      __syncthreads();
    }
    // two leaves at a time: their MFMA chains are independent (each is its own
    // block's sequential sum), so they are interleaved to keep the matrix unit
    // busy; the leaves are then pushed in order
    auto push = [&](int i, const v4d& acc) {   // carry through the occupied levels (bits of i), left + right
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        double carry = acc[c];
        bool open = true;
#pragma unroll
        for (int lv = 0; lv < kRtLevels; ++lv) {
          if (open) {
            if ((i >> lv) & 1) {
              carry = lvl[c][lv] + carry;
            } else {
              lvl[c][lv] = carry;
              open = false;
            }
          }
        }
      }
    };
#pragma unroll 1
    for (int k = 0; k < kRtLeaves; k += 2) {
      const int i = i0 + k;   // depth-first leaf index (uniform)
      const bool v0 = bit_reverse(i, L) < nb, v1 = bit_reverse(i + 1, L) < nb;   // padding leaves are +0
      v4d acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
      if (v0 && v1) {
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const double a0 = s_w[k][we + row][4 * st + kg], b0 = s_x[k][wt + row][4 * st + kg];
          const double a1 = s_w[k + 1][we + row][4 * st + kg], b1 = s_x[k + 1][wt + row][4 * st + kg];
          acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc1, 0, 0, 0);
        }
      } else {
        if (v0)
#pragma unroll
          for (int st = 0; st < 8; ++st) {
            const double a0 = s_w[k][we + row][4 * st + kg], b0 = s_x[k][wt + row][4 * st + kg];
            acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc0, 0, 0, 0);
          }
        if (v1)
#pragma unroll
          for (int st = 0; st < 8; ++st) {
            const double a1 = s_w[k + 1][we + row][4 * st + kg], b1 = s_x[k + 1][wt + row][4 * st + kg];
            acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc1, 0, 0, 0);
          }
      }
      push(i, acc0);
      push(i + 1, acc1);
    }
  }
  // after P2 = 2^L leaves the whole tree sits at level L
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = e_base + we + 4 * c + kg, t = t_base + wt + row;
    double v = lvl[c][0];
#pragma unroll
    for (int lv = 1; lv < kRtLevels; ++lv)
      if (lv == L) v = lvl[c][lv];
    if (e < E && t < ntok) logits[(size_t)t * E + e] = bias ? v + bias[e] : v;
  }
}

// ------------------------------------------------------------ top-k, one wave per token
__global__ __launch_bounds__(256) void k_topk(const double* __restrict__ logits, int ntok, int E, int K,
                                              int32_t* __restrict__ idx, float* __restrict__ gw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= ntok) return;
  TopkPick p;
  const uint64_t first = topk_select(logits + (size_t)t * E, E, K, lane, p);
  const float g = topk_softmax(p, first, K, lane);
  if (lane < K) {
    idx[(size_t)t * K + p.rank] = p.id;
    gw[(size_t)t * K + p.rank] = g;
  }
}

// ------------------------------------------------------------ dense matvec (1..4 columns)
// Each wave handles 64/LPR rows at once (LPR lanes per row, NBL blocks per lane),
// R times: the R row groups of a wave use the same lanes for the same blocks,
// so each activation load serves R rows (with one row per wave and long rows,
// the activations read from L2 otherwise outweigh the weights several times
// at four columns). Each row's lane mapping and accumulation order do not
// depend on R.
template <int FMT, int Q, int UF, int R = 1>
__device__ __forceinline__ void matvec_body(const uint8_t* __restrict__ W, int64_t rows, size_t row_bytes, int nb,
                                            int lpr_log2, const int8_t* __restrict__ cbp,
                                            const int8_t* __restrict__ xq, const float* __restrict__ dx,
                                            float* __restrict__ y) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  const int lpr = 1 << lpr_log2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int rows_per_wave = 64 >> lpr_log2;
  int64_t row[R];
  bool row_ok[R];
  const uint8_t* rowp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row[r] = (((int64_t)blockIdx.x * 4 + wave) * R + r) * rows_per_wave + sub;
    row_ok[r] = row[r] < rows;
    rowp[r] = W + (size_t)(row_ok[r] ? row[r] : rows - 1) * row_bytes;
  }
  uint32_t cb[4];
  load_codebook<FMT>(cbp, cb);
  float acc[R][Q];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < Q; ++t) acc[r][t] = 0.0f;
  // UF chunks of the row (lpr * NBL blocks each) per step: the loads of all UF
  // chunks are issued (clamped into range) before any is used, so a wave makes
  // one memory round trip per UF chunks; the products are taken chunk by chunk
  // in ascending order, as a one-chunk loop would (UF = 1 when a row is one chunk)
  for (int c0 = 0; c0 < nb; c0 += UF * lpr * NBL) {
    Blocks<FMT, NBL> bl[UF][R];
    Acts<NBL> act[UF][Q];
#pragma unroll
    for (int u = 0; u < UF; ++u) {
      const int bc = min(c0 + u * lpr * NBL + sl * NBL, nb - NBL);
#pragma unroll
      for (int r = 0; r < R; ++r) bl[u][r].load(rowp[r], nb, bc);
#pragma unroll
      for (int t = 0; t < Q; ++t) act[u][t].load(xq + (size_t)t * nb * 32, dx + (size_t)t * nb, bc);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < UF; ++u) {
      const int b = c0 + u * lpr * NBL + sl * NBL;
      if (b < nb) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (row_ok[r]) {
#pragma unroll
            for (int i = 0; i < NBL; ++i) {
              uint32_t w[8];
              bl[u][r].expand(i, cb, w);
              const float s = bl[u][r].scale(i);
#pragma unroll
              for (int t = 0; t < Q; ++t) {
                const int p = block_dot(w, act[u][t].q[i]);
                acc[r][t] = fmaf((float)p, s * act[u][t].d[i], acc[r][t]);
              }
            }
          }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const float v = group_sum(acc[r][t], lpr);
      if (sl == 0 && row_ok[r]) y[(size_t)t * rows + row[r]] = v;
    }
}

template <int FMT, int Q, int UF, int R>
__global__ __launch_bounds__(256) void k_matvec(const uint8_t* __restrict__ W, int64_t rows, size_t row_bytes, int nb,
                                                int lpr_log2, const int8_t* __restrict__ cbp,
                                                const int8_t* __restrict__ xq, const float* __restrict__ dx,
                                                float* __restrict__ y) {
  matvec_body<FMT, Q, UF, R>(W, rows, row_bytes, nb, lpr_log2, cbp, xq, dx, y);
}

// The same matvec with the activation quantization in the launch, when the
// columns hold at most kFqMaxBlocks blocks in all: every workgroup quantizes
// them itself (32 lanes per block, two blocks per wave pass, the same IEEE
// operations as k_quant_act) into LDS, with all of a wave's loads in flight at
// once, which costs less than the separate launch it replaces; workgroup 0 also
// writes the int8 values and scales to xq_out / dx_out, as the two-launch form
// leaves them. With more blocks (four columns of 2048 values: 256) the
// redundant quantization costs more than the launch.
constexpr int kFqMaxBlocks = 64;
constexpr int kFqBatch = kFqMaxBlocks / 8;   // passes of the workgroup

template <int FMT, int Q, int UF>
__global__ __launch_bounds__(256) void k_matvec_fq(const uint8_t* __restrict__ W, int64_t rows, size_t row_bytes,
                                                   int nb, int lpr_log2, const int8_t* __restrict__ cbp,
                                                   const float* __restrict__ x, int rot, int8_t* __restrict__ xq_out,
                                                   float* __restrict__ dx_out, float* __restrict__ y) {
  __shared__ __align__(16) int8_t s_xq[kFqMaxBlocks * 32];
  __shared__ float s_dx[kFqMaxBlocks];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31;
  const int nblk = Q * nb;             // <= kFqMaxBlocks
  const int npass = (nblk + 7) / 8;   // 8 blocks per pass of the workgroup, <= kFqBatch
  const bool writer = blockIdx.x == 0;
  for (int p0 = 0; p0 < npass; p0 += kFqBatch) {
    float v[kFqBatch];
#pragma unroll
    for (int k = 0; k < kFqBatch; ++k) {
      const int i = min(((p0 + k) * 4 + wave) * 2 + (lane >> 5), nblk - 1);
      v[k] = x[(size_t)i * 32 + j];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kFqBatch; ++k) {
      if (p0 + k >= npass) break;   // wave-uniform
      const int i = ((p0 + k) * 4 + wave) * 2 + (lane >> 5);
      float d;
      const uint32_t packed = quant_block32_lanes(v[k], rot, &d);
      if (i < nblk) {
        if ((j & 3) == 0) {
          *reinterpret_cast<uint32_t*>(&s_xq[i * 32 + j]) = packed;
          if (writer) *reinterpret_cast<uint32_t*>(xq_out + (size_t)i * 32 + j) = packed;
        }
        if (j == 0) {
          s_dx[i] = d;
          if (writer) dx_out[i] = d;
        }
      }
    }
  }
  __syncthreads();
  matvec_body<FMT, Q, UF>(W, rows, row_bytes, nb, lpr_log2, cbp, s_xq, s_dx, y);
}

// ------------------------------------------------------------ expand-then-multiply (comparison path)
// The unfused form of k_matvec, kept to measure what fusion saves ([0731-Strix]
// section "Lucebox Engine integration with Geometric": the fused 3.5-bit
// matvec against the expand-then-multiply fallback). k_expand writes every
// block as 32 int8 weights C[code] and an fp32 scale; k_matvec_x multiplies the
// expanded matrix with k_matvec's lane mapping and accumulation order, so the
// outputs are identical bit for bit and only the bytes moved differ
// (1 + 1/8 B per weight read, plus the expansion's own pass, against 0.31 to
// 0.53 B).
template <int FMT>
__global__ __launch_bounds__(256) void k_expand(const uint8_t* __restrict__ W, int64_t rows, size_t row_bytes, int nb,
                                                const int8_t* __restrict__ cbp, int8_t* __restrict__ w8,
                                                float* __restrict__ s32) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * nb) return;
  const int64_t r = i / nb;
  const int b = (int)(i % nb);
  uint32_t cb[4];
  load_codebook<FMT>(cbp, cb);
  Blocks<FMT, 1> bl;
  bl.load(W + (size_t)r * row_bytes, nb, b);
  uint32_t w[8];
  bl.expand(0, cb, w);
  u32x4* dst = reinterpret_cast<u32x4*>(w8 + (size_t)i * 32);
  dst[0] = u32x4{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  s32[i] = bl.scale(0);
}

template <int NBL, int Q>
__global__ __launch_bounds__(256) void k_matvec_x(const int8_t* __restrict__ w8, const float* __restrict__ s32,
                                                  int64_t rows, int nb, int lpr_log2, const int8_t* __restrict__ xq,
                                                  const float* __restrict__ dx, float* __restrict__ y) {
  const int lpr = 1 << lpr_log2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int rows_per_wave = 64 >> lpr_log2;
  const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * rows_per_wave + sub;
  const bool row_ok = row < rows;
  float acc[Q];
#pragma unroll
  for (int t = 0; t < Q; ++t) acc[t] = 0.0f;
  const int8_t* roww = w8 + (size_t)row * nb * 32;
  const float* rows32 = s32 + (size_t)row * nb;
  for (int c0 = 0; c0 < nb; c0 += lpr * NBL) {
    const int b = c0 + sl * NBL;
    if (row_ok && b < nb) {
      uint32_t w[NBL][8];
      float sc[NBL];
#pragma unroll
      for (int i = 0; i < NBL; ++i) {
        const u32x4* p = reinterpret_cast<const u32x4*>(roww + (size_t)(b + i) * 32);
        const u32x4 a = p[0], c = p[1];
        w[i][0] = a.x; w[i][1] = a.y; w[i][2] = a.z; w[i][3] = a.w;
        w[i][4] = c.x; w[i][5] = c.y; w[i][6] = c.z; w[i][7] = c.w;
        sc[i] = rows32[b + i];
      }
      Acts<NBL> act[Q];
#pragma unroll
      for (int t = 0; t < Q; ++t) act[t].load(xq + (size_t)t * nb * 32, dx + (size_t)t * nb, b);
#pragma unroll
      for (int i = 0; i < NBL; ++i)
#pragma unroll
        for (int t = 0; t < Q; ++t) {
          const int p = block_dot(w[i], act[t].q[i]);
          acc[t] = fmaf((float)p, sc[i] * act[t].d[i], acc[t]);
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
  const u32x4* p = reinterpret_cast<const u32x4*>(xq + (size_t)b * 32);
  const u32x4 a = p[0], c = p[1];
  const uint32_t x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  uint32_t w[8];
  bl.expand(0, cb, w);
  P[i] = block_dot(w, x);
}

// ------------------------------------------------------------ timing pool
struct TimingPool {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> start, stop;
  std::vector<std::string> name;
  size_t used = 0;
};
TimingPool g_timing;

}  // namespace

// ============================================================ shared host helpers

namespace qmoe {

int launch_check(const char* what) {
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) QMOE_FAIL(QMOE_E_HIP, "%s: %s", what, hipGetErrorString(err));
  return QMOE_OK;
}

void timing_slot(const char* nm, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (!g_timing.on) return;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  if (g_timing.used == g_timing.start.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return;
    g_timing.start.push_back(a);
    g_timing.stop.push_back(b);
    g_timing.name.emplace_back();
  }
  const size_t slot = g_timing.used++;
  g_timing.name[slot] = nm;
  *start = g_timing.start[slot];
  *stop = g_timing.stop[slot];
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int ws_ptrs(const qmoe_layer* L, int32_t ntok, void* ws, size_t ws_bytes, WsPtrs* p) {
  qmoe_ws_layout lay;
  int st = qmoe_workspace_layout(L, ntok, &lay);
  if (st) return st;
  if (!ws) QMOE_FAIL(QMOE_E_WORKSPACE, "missing workspace (NULL)");
  if (!aligned16(ws)) QMOE_FAIL(QMOE_E_WORKSPACE, "workspace not 16-byte aligned");
  if (ws_bytes < lay.total)
    QMOE_FAIL(QMOE_E_WORKSPACE, "workspace %zu bytes < %zu required for %d tokens", ws_bytes, lay.total, ntok);
  uint8_t* b = static_cast<uint8_t*>(ws);
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
  p->n_xq = lay.dx - lay.xq;
  p->n_dx = lay.idx - lay.dx;
  p->n_idx = lay.gw - lay.idx;
  p->n_gw = lay.logits - lay.gw;
  p->n_logits = lay.plan - lay.logits;
  p->n_plan = lay.hq - lay.plan;
  p->n_hq = lay.dh - lay.hq;
  p->n_dh = lay.group - lay.dh;
  p->n_group = lay.ypair - lay.group;
  p->n_ypair = lay.total - lay.ypair;
  return QMOE_OK;
}

int launch_quant(const float* x, int64_t nblocks, int rot, int8_t* xq, float* dx, hipStream_t s) {
  if (nblocks == 0) return QMOE_OK;
  const int threads = 256;
  const unsigned grid = (unsigned)((nblocks + threads - 1) / threads);
  launch_kernel("quant_act", k_quant_act, dim3(grid), dim3(threads), s, x, nblocks, rot, xq, dx);
  return launch_check("quant_act");
}

int launch_route(const qmoe_layer* L, const float* x, int32_t ntok, double* logits, int32_t* idx, float* gw,
                 hipStream_t s) {
  if (L->hidden > 32 * 64 * kRouterMaxC)
    QMOE_FAIL(QMOE_E_SHAPE, "hidden=%d exceeds router limit %d", L->hidden, 32 * 64 * kRouterMaxC);
  if (ntok >= kRtT / 2) {   // many tokens: 32 x 32 logit tiles (same order, same bits)
    dim3 grid((L->n_experts + kRtE - 1) / kRtE, (ntok + kRtT - 1) / kRtT);
    launch_kernel("router", k_router_tiles, grid, dim3(256), s, L->w_router, x, ntok, L->n_experts, L->hidden,
                  L->router_bias, logits);
  } else {
    dim3 grid((L->n_experts + 3) / 4, (ntok + 3) / 4);
    launch_kernel("router", k_router, grid, dim3(256), s, L->w_router, x, ntok, L->n_experts, L->hidden,
                  L->router_bias, logits);
  }
  int st = launch_check("router");
  if (st) return st;
  {
    dim3 grid((ntok + 3) / 4);
    launch_kernel("topk", k_topk, grid, dim3(256), s, logits, ntok, L->n_experts, L->topk, idx, gw);
  }
  return launch_check("topk");
}

}  // namespace qmoe

namespace {

template <int FMT, int Q>
void launch_matvec_t(const uint8_t* W, int64_t rows, size_t row_bytes, int nb, int lpr_log2, const int8_t* cb,
                     const int8_t* xq, const float* dx, float* y, hipStream_t s) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  const int chunks = (nb + (NBL << lpr_log2) - 1) / (NBL << lpr_log2);
  // three or four columns over rows of several chunks (one row per wave): two
  // rows per wave share the activation loads (with one or two columns the
  // halved workgroup count cost more than the shared loads saved)
  const int R = (Q >= 3 && chunks > 1 && lpr_log2 == 6) ? 2 : 1;
  const int rows_per_wg = 4 * R * (64 >> lpr_log2);
  const unsigned grid = (unsigned)((rows + rows_per_wg - 1) / rows_per_wg);
  if (chunks == 1)
    launch_kernel("matvec", k_matvec<FMT, Q, 1, 1>, dim3(grid), dim3(256), s, W, rows, row_bytes, nb, lpr_log2, cb,
                  xq, dx, y);
  else if (R == 2)
    launch_kernel("matvec", k_matvec<FMT, Q, 2, (Q >= 3) ? 2 : 1>, dim3(grid), dim3(256), s, W, rows, row_bytes, nb,
                  lpr_log2, cb, xq, dx, y);
  else
    launch_kernel("matvec", k_matvec<FMT, Q, (Q <= 2) ? 4 : 2, 1>, dim3(grid), dim3(256), s, W, rows, row_bytes, nb,
                  lpr_log2, cb, xq, dx, y);
}

template <int FMT, int Q>
void launch_matvec_fq_t(const uint8_t* W, int64_t rows, size_t row_bytes, int nb, int lpr_log2, const int8_t* cb,
                        const float* x, int rot, int8_t* xq, float* dx, float* y, hipStream_t s) {
  const int rows_per_wg = 4 * (64 >> lpr_log2);
  const unsigned grid = (unsigned)((rows + rows_per_wg - 1) / rows_per_wg);
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  const int chunks = (nb + (NBL << lpr_log2) - 1) / (NBL << lpr_log2);
  if (chunks == 1)
    launch_kernel("matvec_fq", k_matvec_fq<FMT, Q, 1>, dim3(grid), dim3(256), s, W, rows, row_bytes, nb, lpr_log2,
                  cb, x, rot, xq, dx, y);
  else
    launch_kernel("matvec_fq", k_matvec_fq<FMT, Q, (Q <= 2) ? 4 : 2>, dim3(grid), dim3(256), s, W, rows, row_bytes,
                  nb, lpr_log2, cb, x, rot, xq, dx, y);
}

template <int FMT>
void launch_matvec_fq_f(int q, const uint8_t* W, int64_t rows, size_t row_bytes, int nb, int lpr_log2,
                        const int8_t* cb, const float* x, int rot, int8_t* xq, float* dx, float* y, hipStream_t s) {
  switch (q) {
    case 1: launch_matvec_fq_t<FMT, 1>(W, rows, row_bytes, nb, lpr_log2, cb, x, rot, xq, dx, y, s); break;
    case 2: launch_matvec_fq_t<FMT, 2>(W, rows, row_bytes, nb, lpr_log2, cb, x, rot, xq, dx, y, s); break;
    case 3: launch_matvec_fq_t<FMT, 3>(W, rows, row_bytes, nb, lpr_log2, cb, x, rot, xq, dx, y, s); break;
    default: launch_matvec_fq_t<FMT, 4>(W, rows, row_bytes, nb, lpr_log2, cb, x, rot, xq, dx, y, s); break;
  }
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

}  // namespace

namespace qmoe {

int check_matrix(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes, const int8_t* cb, FormatInfo* fi) {
  if (!format_info(fmt, fi)) QMOE_FAIL(QMOE_E_FORMAT, "unknown format %d", fmt);
  if (rows < 0 || k <= 0 || k % 32)
    QMOE_FAIL(QMOE_E_SHAPE, "rows=%lld k=%lld (k must be a positive multiple of 32)", (long long)rows, (long long)k);
  const size_t row_bytes = (size_t)(k / 32) * fi->block_bytes;
  if (row_bytes % 16)
    QMOE_FAIL(QMOE_E_SHAPE, "row of %zu bytes not a multiple of 16 (k must be a multiple of %d for FP%d)", row_bytes,
              fmt == 4 ? 512 : 256, fmt);
  if (k / 32 > 0x7FFFFFFF) QMOE_FAIL(QMOE_E_SHAPE, "k too large");
  if (!w) QMOE_FAIL(QMOE_E_INVAL, "missing weights (NULL)");
  if (!aligned16(w)) QMOE_FAIL(QMOE_E_INVAL, "weights not 16-byte aligned");
  if (w_bytes < (size_t)rows * row_bytes)
    QMOE_FAIL(QMOE_E_SIZE, "%zu weight bytes < %zu", w_bytes, (size_t)rows * row_bytes);
  if (!cb) QMOE_FAIL(QMOE_E_CODEBOOK, "missing codebook (NULL)");
  if (reinterpret_cast<uintptr_t>(cb) & 3) QMOE_FAIL(QMOE_E_INVAL, "codebook not 4-byte aligned");
  return QMOE_OK;
}

}  // namespace qmoe

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
  const int nbl = fmt == 4 ? 1 : 2;
  const int lg = ilog2(lanes_per_row(nb, nbl));
  const size_t row_bytes = (size_t)nb * fi.block_bytes;
  const uint8_t* W = static_cast<const uint8_t*>(w);
  {
    const size_t rows_per_wg = 4 * (64 >> lg);
    QMOE_BOUNDS((size_t)ncols * k <= round_up((size_t)ncols * k, 256) &&
                    round_up((size_t)ncols * k, 256) + (size_t)ncols * nb * 4 <= ws_bytes,
                "matvec: quantized columns and scales inside the workspace");
    QMOE_BOUNDS(((size_t)rows + rows_per_wg - 1) / rows_per_wg * rows_per_wg >= (size_t)rows,
                "matvec: grid covers the rows");
    QMOE_BOUNDS(lg >= 0 && lg <= 6 && (nbl << lg) <= nb, "matvec: lanes per row within the row's blocks");
  }
  if ((int64_t)ncols * nb <= kFqMaxBlocks) {   // one launch: quantization inside the matvec
    switch (fmt) {
      case 2: launch_matvec_fq_f<2>(ncols, W, rows, row_bytes, nb, lg, cb, x, rot, xq, dx, y, s); break;
      case 3: launch_matvec_fq_f<3>(ncols, W, rows, row_bytes, nb, lg, cb, x, rot, xq, dx, y, s); break;
      default: launch_matvec_fq_f<4>(ncols, W, rows, row_bytes, nb, lg, cb, x, rot, xq, dx, y, s); break;
    }
    return launch_check("matvec_fq");
  }
  if ((st = launch_quant(x, (int64_t)ncols * nb, rot, xq, dx, s))) return st;
  switch (fmt) {
    case 2: launch_matvec_f<2>(ncols, W, rows, row_bytes, nb, lg, cb, xq, dx, y, s); break;
    case 3: launch_matvec_f<3>(ncols, W, rows, row_bytes, nb, lg, cb, xq, dx, y, s); break;
    default: launch_matvec_f<4>(ncols, W, rows, row_bytes, nb, lg, cb, xq, dx, y, s); break;
  }
  return launch_check("matvec");
}

extern "C" size_t qmoe_matvec_expanded_workspace_bytes(int64_t rows, int64_t k, int32_t ncols) {
  const size_t base = qmoe_matvec_workspace_bytes(k, ncols);
  if (!base || rows < 0) return 0;
  return base + round_up((size_t)rows * k, 256) + round_up((size_t)rows * (k / 32) * 4, 256);
}

template <int NBL>
void launch_matvec_x(int q, const int8_t* w8, const float* s32, int64_t rows, int nb, int lg, const int8_t* xq,
                     const float* dx, float* y, hipStream_t s) {
  const int rows_per_wg = 4 * (64 >> lg);
  const dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  switch (q) {
    case 1: launch_kernel("matvec_x", k_matvec_x<NBL, 1>, grid, dim3(256), s, w8, s32, rows, nb, lg, xq, dx, y); break;
    case 2: launch_kernel("matvec_x", k_matvec_x<NBL, 2>, grid, dim3(256), s, w8, s32, rows, nb, lg, xq, dx, y); break;
    case 3: launch_kernel("matvec_x", k_matvec_x<NBL, 3>, grid, dim3(256), s, w8, s32, rows, nb, lg, xq, dx, y); break;
    default: launch_kernel("matvec_x", k_matvec_x<NBL, 4>, grid, dim3(256), s, w8, s32, rows, nb, lg, xq, dx, y);
  }
}

extern "C" int qmoe_matvec_expanded(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes, const int8_t* cb,
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
  const size_t need = qmoe_matvec_expanded_workspace_bytes(rows, k, ncols);
  if (!ws) QMOE_FAIL(QMOE_E_WORKSPACE, "missing workspace (NULL)");
  if (!aligned16(ws)) QMOE_FAIL(QMOE_E_WORKSPACE, "workspace not 16-byte aligned");
  if (ws_bytes < need) QMOE_FAIL(QMOE_E_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if (rows == 0) return QMOE_OK;
  uint8_t* base = static_cast<uint8_t*>(ws);
  int8_t* xq = reinterpret_cast<int8_t*>(base);
  float* dx = reinterpret_cast<float*>(base + round_up((size_t)ncols * k, 256));
  const size_t mv = qmoe_matvec_workspace_bytes(k, ncols);
  int8_t* w8 = reinterpret_cast<int8_t*>(base + mv);
  float* s32 = reinterpret_cast<float*>(base + mv + round_up((size_t)rows * k, 256));
  hipStream_t s = as_stream(stream);
  const int nb = (int)(k / 32);
  if ((st = launch_quant(x, (int64_t)ncols * nb, rot, xq, dx, s))) return st;
  const size_t row_bytes = (size_t)nb * fi.block_bytes;
  const uint8_t* W = static_cast<const uint8_t*>(w);
  const unsigned eg = (unsigned)((rows * nb + 255) / 256);
  switch (fmt) {
    case 2: launch_kernel("expand", k_expand<2>, dim3(eg), dim3(256), s, W, rows, row_bytes, nb, cb, w8, s32); break;
    case 3: launch_kernel("expand", k_expand<3>, dim3(eg), dim3(256), s, W, rows, row_bytes, nb, cb, w8, s32); break;
    default: launch_kernel("expand", k_expand<4>, dim3(eg), dim3(256), s, W, rows, row_bytes, nb, cb, w8, s32); break;
  }
  if ((st = launch_check("expand"))) return st;
  const int nbl = fmt == 4 ? 1 : 2;
  const int lg = ilog2(lanes_per_row(nb, nbl));
  if (nbl == 2)
    launch_matvec_x<2>(ncols, w8, s32, rows, nb, lg, xq, dx, y, s);
  else
    launch_matvec_x<1>(ncols, w8, s32, rows, nb, lg, xq, dx, y, s);
  return launch_check("matvec_x");
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
  return launch_route(L, x, ntok, w.logits, idx, gate_w, as_stream(stream));
}

extern "C" int qmoe_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.on = on != 0;
  g_timing.used = 0;
  return QMOE_OK;
}

extern "C" int qmoe_timing_read(const char* name, double* total_ms, int* count) {
  clear_error();
  if (!name || !total_ms || !count) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  double tot = 0.0;
  int n = 0;
  for (size_t i = 0; i < g_timing.used; ++i) {
    if (g_timing.name[i] != name) continue;
    if (hipEventSynchronize(g_timing.stop[i]) != hipSuccess) QMOE_FAIL(QMOE_E_HIP, "event synchronize failed");
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, g_timing.start[i], g_timing.stop[i]) != hipSuccess)
      QMOE_FAIL(QMOE_E_HIP, "event elapsed time failed");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *count = n;
  return QMOE_OK;
}
