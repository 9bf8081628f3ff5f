// Several packed matrix-vector products in two launches (gfx950): the dense
// projections of one decode step, for example a 4-bit 4096 x 16384 matrix and a
// 3-bit 4096 x 2048 one with H32 on its input, instead of one launch per
// matrix plus one per long input's quantization.
//
// Page citations:
//   [Strix-284B] lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
//     AMD Ryzen AI MAX+ 395", section "ROCmFPX: fitting 284B weights into 128 GB"
//     (decode reads the packed blocks directly and is bound by memory traffic)
//     and section "Decode: up to 32 tok/s" (the dense 4-bit weights of a step,
//     decoded once for all of its columns).
//   [evox3] soothill.io, "DeepSeek V4 Flash 0731 on evox3", table "The
//     optimization ladder" (the fused H32 matrix-vector path).
//
//   k_group_fq     (one or two columns, inputs of at most 512 blocks) one
//                  launch: every workgroup quantizes its matrix's input into
//                  LDS, then multiplies its rows
//   k_group_quant  otherwise, every input of every matrix, one 32-block per
//                  half-wave (the same IEEE operations as qmoe_quant_act), into
//                  the workspace, then
//   k_group_mvl    every matrix's rows in one grid when each input (all
//                  columns) holds at most 2048 blocks: each workgroup serves
//                  one matrix and first copies its quantized input into LDS;
//                  each wave takes one row unit (the rows that one wave
//                  covers, 64 / lanes-per-row of them) at a time, in the lane
//                  mapping and accumulation order of qmoe_matvec, so every
//                  output equals qmoe_matvec's bit for bit (every form);
//   k_group_mv     the same with the input read from the workspace, for
//                  longer inputs.
// Each launch costs a fixed ~3 us on MI355X. (A one-launch form with a grid
// barrier between the quantization and the products was measured slower: its
// products cannot start before the barrier, so they no longer overlap the
// weight stream.)
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qmoe_device.h"
#include "qmoe_host.h"
#include "qmoe_internal.h"

using namespace qk;
using namespace qmoe;

namespace {

constexpr int kGroupMax = 4;      // matrices per call
constexpr int kGroupThreads = 256;

template <int FMT>
constexpr int group_nbl() { return FMT == 4 ? 1 : 2; }
[[maybe_unused]] inline int group_nbl_rt(int fmt) { return fmt == 4 ? 1 : 2; }   // (used by the debug build's checks)

struct GroupItem {
  const uint8_t* w;
  const int8_t* cb;
  const float* x;
  float* y;
  int8_t* xq;        // quantized input [Q][nb][32] (workspace)
  float* dx;         // its block scales [Q][nb]
  int64_t rows;
  size_t row_bytes;
  int nb, lpr_log2, fmt, rot;
  int units;         // row units of 64 >> lpr_log2 rows
  int wg0, nwg;      // the item's workgroups of k_group_mv: wg0 .. wg0 + nwg - 1
  int blk0;          // first block of this item in the quantization order
};

struct GroupArgs {
  GroupItem it[kGroupMax];
  int n;
  int nblk;          // blocks to quantize, all items
};

// Half-wave h of the grid quantizes block h of the concatenated inputs.
__global__ __launch_bounds__(kGroupThreads) void k_group_quant(GroupArgs g) {
  const int lane = threadIdx.x & 63, j = lane & 31;
  const int B = (blockIdx.x * (kGroupThreads / 64) + (threadIdx.x >> 6)) * 2 + (lane >> 5);
  int i = 0;
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k < g.n && B >= g.it[k].blk0) i = k;
  const GroupItem& it = g.it[i];
  const int local = min(B, g.nblk - 1) - it.blk0;   // column local / nb, block local % nb
  const float v = it.x[(size_t)(local / it.nb) * it.nb * 32 + (size_t)(local % it.nb) * 32 + j];
  float d;
  const uint32_t packed = quant_block32_lanes(v, it.rot, &d);
  if (B < g.nblk) {
    if ((j & 3) == 0) *reinterpret_cast<uint32_t*>(it.xq + (size_t)local * 32 + j) = packed;
    if (j == 0) it.dx[local] = d;
  }
}

// Row units lw, lw + W, ... of one matrix (W: its waves; WPG waves per
// workgroup). The row's chunks are taken UF at a time (all their loads issued
// before the first product), UF as qmoe_matvec picks it: 4 with one or two
// columns, 2 with more. xq / dx: the quantized input, [Q][nb][32] and [Q][nb],
// in the workspace or in LDS.
template <int FMT, int Q, int WPG, int UF = (Q <= 2) ? 4 : 2>
__device__ __forceinline__ void group_wave(const GroupItem& it, int lw, const int8_t* xq, const float* dx) {
  constexpr int NBL = group_nbl<FMT>();
  const int lane = threadIdx.x & 63;
  const int lpr_log2 = it.lpr_log2, lpr = 1 << lpr_log2;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int rpw = 64 >> lpr_log2;
  const int nb = it.nb, W = it.nwg * WPG;
  uint32_t cb[4];
  load_codebook<FMT>(it.cb, cb);
  for (int u = lw; u < it.units; u += W) {
    const int64_t row = (int64_t)u * rpw + sub;
    const bool ok = row < it.rows;
    const uint8_t* rp = it.w + (size_t)(ok ? row : it.rows - 1) * it.row_bytes;
    float acc[Q];
#pragma unroll
    for (int t = 0; t < Q; ++t) acc[t] = 0.0f;
    for (int c0 = 0; c0 < nb; c0 += UF * lpr * NBL) {
      Blocks<FMT, NBL> bl[UF];
      Acts<NBL> act[UF][Q];
#pragma unroll
      for (int c = 0; c < UF; ++c) {
        const int bc = min(c0 + c * lpr * NBL + sl * NBL, nb - NBL);   // clamped into the row
        bl[c].load(rp, nb, bc);
#pragma unroll
        for (int t = 0; t < Q; ++t) act[c][t].load(xq + (size_t)t * nb * 32, dx + (size_t)t * nb, bc);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < UF; ++c) {
        const int b = c0 + c * lpr * NBL + sl * NBL;
        if (ok && b < nb) {
#pragma unroll
          for (int i = 0; i < NBL; ++i) {
            uint32_t w[8];
            bl[c].expand(i, cb, w);
            const float s = bl[c].scale(i);
#pragma unroll
            for (int t = 0; t < Q; ++t) {
              const int p = block_dot(w, act[c][t].q[i]);
              acc[t] = fmaf((float)p, s * act[c][t].d[i], acc[t]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const float v = group_sum(acc[t], lpr);
      if (sl == 0 && ok) it.y[(size_t)t * it.rows + row] = v;
    }
  }
}

// group_wave with the quantized input in LDS: the weights of UF chunks are
// requested first, as there, but each block's activations are read from LDS
// just before its products instead of being held in registers for the whole
// step (LDS answers within the step; the registers go to the weights). The
// products and additions are group_wave's, in its order.
template <int FMT, int Q, int WPG, int UF>
__device__ __forceinline__ void group_wave_lds(const GroupItem& it, int lw, const int8_t* xq, const float* dx) {
  constexpr int NBL = group_nbl<FMT>();
  const int lane = threadIdx.x & 63;
  const int lpr_log2 = it.lpr_log2, lpr = 1 << lpr_log2;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int rpw = 64 >> lpr_log2;
  const int nb = it.nb, W = it.nwg * WPG;
  uint32_t cb[4];
  load_codebook<FMT>(it.cb, cb);
  for (int u = lw; u < it.units; u += W) {
    const int64_t row = (int64_t)u * rpw + sub;
    const bool ok = row < it.rows;
    const uint8_t* rp = it.w + (size_t)(ok ? row : it.rows - 1) * it.row_bytes;
    float acc[Q];
#pragma unroll
    for (int t = 0; t < Q; ++t) acc[t] = 0.0f;
    for (int c0 = 0; c0 < nb; c0 += UF * lpr * NBL) {
      Blocks<FMT, NBL> bl[UF];
#pragma unroll
      for (int c = 0; c < UF; ++c) bl[c].load(rp, nb, min(c0 + c * lpr * NBL + sl * NBL, nb - NBL));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < UF; ++c) {
        const int b = c0 + c * lpr * NBL + sl * NBL;
        if (ok && b < nb) {
#pragma unroll
          for (int i = 0; i < NBL; ++i) {
            Acts<1> act[Q];
#pragma unroll
            for (int t = 0; t < Q; ++t) act[t].load(xq + (size_t)t * nb * 32, dx + (size_t)t * nb, b + i);
            uint32_t w[8];
            bl[c].expand(i, cb, w);
            const float s = bl[c].scale(i);
#pragma unroll
            for (int t = 0; t < Q; ++t) {
              const int p = block_dot(w, act[t].q[0]);
              acc[t] = fmaf((float)p, s * act[t].d[0], acc[t]);
            }
            // one block's activations in registers at a time
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const float v = group_sum(acc[t], lpr);
      if (sl == 0 && ok) it.y[(size_t)t * it.rows + row] = v;
    }
  }
}

template <int Q>
__global__ __launch_bounds__(kGroupThreads) void k_group_mv(GroupArgs g) {
  int i = 0;
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k < g.n && (int)blockIdx.x >= g.it[k].wg0) i = k;
  const GroupItem& it = g.it[i];
  const int lw = ((int)blockIdx.x - it.wg0) * (kGroupThreads / 64) + (threadIdx.x >> 6);
  constexpr int WPG = kGroupThreads / 64;
  switch (it.fmt) {   // uniform over the workgroup
    case 2: group_wave<2, Q, WPG>(it, lw, it.xq, it.dx); break;
    case 3: group_wave<3, Q, WPG>(it, lw, it.xq, it.dx); break;
    default: group_wave<4, Q, WPG>(it, lw, it.xq, it.dx); break;
  }
}

// One-launch form, for one or two columns when every item's input holds at
// most kFqMaxBlocks blocks (all columns): each workgroup first quantizes its
// item's whole input into LDS, one block per thread with all 32 values in the
// thread's registers (quant_block32: the same IEEE operations as
// k_group_quant's half-waves, so the same bytes and scales), then, after one
// barrier, runs the item's row units through group_wave from LDS. The item's
// first workgroup also writes the quantized input to the workspace, as the
// two-launch form does. Workgroups of 8 waves keep the redundant quantization
// to one block per thread for a 16384-wide input, and at one column the
// kernel fits three of them per compute unit. (Requesting each wave's first
// row of weights before the quantization, so that the stream starts earlier,
// measured slower: 13.8 against 12.7 us for the dense 4-bit 16384 + 3-bit 2048
// pair; workgroups of 4 waves doubled the redundant quantization: 15.8 us.)
constexpr int kFqThreads = 512;
constexpr int kFqMaxBlocks = 512;
constexpr int kFqUF = 2;   // chunks per step (the per-lane block order does not depend on it)

template <int Q>
__global__ __launch_bounds__(kFqThreads, Q == 1 ? 6 : 4) void k_group_fq(GroupArgs g) {
  __shared__ u32x4 s_xq[2 * kFqMaxBlocks];
  __shared__ float s_dx[kFqMaxBlocks];
  int i = 0;
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k < g.n && (int)blockIdx.x >= g.it[k].wg0) i = k;
  const GroupItem& it = g.it[i];
  const int tid = threadIdx.x;
  const bool first = (int)blockIdx.x == it.wg0;
  // the item's input, one block per thread per pass (column B / nb, block B % nb)
  for (int B = tid; B < Q * it.nb; B += kFqThreads) {
    const float4* src = reinterpret_cast<const float4*>(it.x + (size_t)B * 32);
    float v[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 f = src[k];
      v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
    }
    uint32_t q[8];
    float d;
    quant_block32(v, it.rot, q, &d);
    const u32x4 lo = {q[0], q[1], q[2], q[3]}, hi = {q[4], q[5], q[6], q[7]};
    s_xq[2 * B] = lo;
    s_xq[2 * B + 1] = hi;
    s_dx[B] = d;
    if (first) {
      reinterpret_cast<u32x4*>(it.xq)[2 * B] = lo;
      reinterpret_cast<u32x4*>(it.xq)[2 * B + 1] = hi;
      it.dx[B] = d;
    }
  }
  __syncthreads();
  constexpr int WPG = kFqThreads / 64;
  const int lw = ((int)blockIdx.x - it.wg0) * WPG + (tid >> 6);
  const int8_t* xq = reinterpret_cast<const int8_t*>(s_xq);
  switch (it.fmt) {   // uniform over the workgroup
    case 2: group_wave<2, Q, WPG, kFqUF>(it, lw, xq, s_dx); break;
    case 3: group_wave<3, Q, WPG, kFqUF>(it, lw, xq, s_dx); break;
    default: group_wave<4, Q, WPG, kFqUF>(it, lw, xq, s_dx); break;
  }
}

// Two-launch form with the quantized inputs in LDS, when every item's input
// (all columns) holds at most kMvlMaxBlocks blocks: k_group_mv's row units, but
// each workgroup first copies its item's quantized input and scales from the
// workspace into LDS (all of a thread's loads issued before its stores), so
// that the rows read the activations from LDS instead of from the caches: at
// four columns a 16384-wide row re-reads 64 KB of them against its 8.5 KB of
// weights. The rows' order of operations is group_wave's, so the outputs are
// k_group_mv's bit for bit. (Dense 4-bit 4096 x 16384 + 3-bit 4096 x 2048 at
// four columns: 23.6 -> 16.9 us per step against k_group_mv. Requesting each
// wave's first weights before the copy, with the copy as direct global-to-LDS
// loads, measured slower at four columns: 17.5 us.)
constexpr int kMvlMaxBlocks = 2048;   // 64 KB of int8 blocks + 8 KB of scales: two workgroups per CU
template <int Q> constexpr int mvl_uf() { return Q <= 2 ? 4 : 2; }   // chunks per step

template <int Q>
__global__ __launch_bounds__(kFqThreads, 4) void k_group_mvl(GroupArgs g) {
  __shared__ u32x4 s_xq[2 * kMvlMaxBlocks];
  __shared__ float s_dx[kMvlMaxBlocks];
  int i = 0;
#pragma unroll
  for (int k = 1; k < kGroupMax; ++k)
    if (k < g.n && (int)blockIdx.x >= g.it[k].wg0) i = k;
  const GroupItem& it = g.it[i];
  const int tid = threadIdx.x;
  constexpr int NX = 2 * kMvlMaxBlocks / kFqThreads, ND = kMvlMaxBlocks / kFqThreads;
  const int nx = 2 * Q * it.nb, nd = Q * it.nb;
  const u32x4* gx = reinterpret_cast<const u32x4*>(it.xq);
  u32x4 xv[NX];
  float dv[ND];
#pragma unroll
  for (int k = 0; k < NX; ++k) xv[k] = gx[min(tid + k * kFqThreads, nx - 1)];
#pragma unroll
  for (int k = 0; k < ND; ++k) dv[k] = it.dx[min(tid + k * kFqThreads, nd - 1)];
#pragma unroll
  for (int k = 0; k < NX; ++k)
    if (tid + k * kFqThreads < nx) s_xq[tid + k * kFqThreads] = xv[k];
#pragma unroll
  for (int k = 0; k < ND; ++k)
    if (tid + k * kFqThreads < nd) s_dx[tid + k * kFqThreads] = dv[k];
  __syncthreads();
  constexpr int WPG = kFqThreads / 64;
  const int lw = ((int)blockIdx.x - it.wg0) * WPG + (tid >> 6);
  const int8_t* xq = reinterpret_cast<const int8_t*>(s_xq);
  switch (it.fmt) {   // uniform over the workgroup
    case 2: group_wave_lds<2, Q, WPG, mvl_uf<Q>()>(it, lw, xq, s_dx); break;
    case 3: group_wave_lds<3, Q, WPG, mvl_uf<Q>()>(it, lw, xq, s_dx); break;
    default: group_wave_lds<4, Q, WPG, mvl_uf<Q>()>(it, lw, xq, s_dx); break;
  }
}

template <int Q>
int launch_group(GroupArgs& g, hipStream_t s) {
  bool fq = Q <= 2;   // (three or four columns do not fit the one-launch form's registers)
  bool mvl = true;
  for (int i = 0; i < g.n; ++i) {
    fq = fq && Q * g.it[i].nb <= kFqMaxBlocks;
    mvl = mvl && Q * g.it[i].nb <= kMvlMaxBlocks;
  }
  const int wpg = (fq || mvl ? kFqThreads : kGroupThreads) / 64;
  int grid = 0;
  for (int i = 0; i < g.n; ++i) {   // one row unit per wave
    g.it[i].nwg = (g.it[i].units + wpg - 1) / wpg;
    g.it[i].wg0 = grid;
    grid += g.it[i].nwg;
    // every row unit has a wave; the quantized input fits its workspace region
    QMOE_BOUNDS((int64_t)g.it[i].nwg * wpg >= g.it[i].units &&
                    (int64_t)g.it[i].units * (64 >> g.it[i].lpr_log2) >= g.it[i].rows,
                "matvec group: grid covers the rows");
    QMOE_BOUNDS(g.it[i].lpr_log2 >= 0 && g.it[i].lpr_log2 <= 6 &&
                    (group_nbl_rt(g.it[i].fmt) << g.it[i].lpr_log2) <= g.it[i].nb,
                "matvec group: lanes per row within the row");
  }
  if constexpr (Q <= 2) {
    if (fq) {
      launch_kernel("group_fq", k_group_fq<Q>, dim3(grid), dim3(kFqThreads), s, g);
      return launch_check("group_fq");
    }
  }
  constexpr int qwpg = kGroupThreads / 64;   // k_group_quant: two blocks per wave
  const int qgrid = (g.nblk + 2 * qwpg - 1) / (2 * qwpg);
  launch_kernel("group_quant", k_group_quant, dim3(qgrid), dim3(kGroupThreads), s, g);
  int st = launch_check("group_quant");
  if (st) return st;
  if (mvl) {
    launch_kernel("group_mvl", k_group_mvl<Q>, dim3(grid), dim3(kFqThreads), s, g);
    return launch_check("group_mvl");
  }
  launch_kernel("group_mv", k_group_mv<Q>, dim3(grid), dim3(kGroupThreads), s, g);
  return launch_check("group_mv");
}

size_t group_ws_bytes(const qmoe_matvec_item* m, int32_t n, int32_t ncols) {
  size_t t = 0;
  for (int i = 0; i < n; ++i) {
    t += round_up((size_t)ncols * (size_t)m[i].k, 256);
    t += round_up((size_t)ncols * (size_t)(m[i].k / 32) * 4, 256);
  }
  return t;
}

}  // namespace

extern "C" size_t qmoe_matvec_group_workspace_bytes(const qmoe_matvec_item* m, int32_t n, int32_t ncols) {
  if (!m || n < 1 || n > kGroupMax || ncols < 1 || ncols > 4) return 0;
  for (int i = 0; i < n; ++i)
    if (m[i].k <= 0 || m[i].k % 32) return 0;
  return group_ws_bytes(m, n, ncols);
}

extern "C" int qmoe_matvec_group(const qmoe_matvec_item* m, int32_t n, int32_t ncols, void* ws, size_t ws_bytes,
                                 void* stream) {
  clear_error();
  if (!m) QMOE_FAIL(QMOE_E_INVAL, "NULL item list");
  if (n < 1 || n > kGroupMax) QMOE_FAIL(QMOE_E_SHAPE, "n=%d outside 1..%d", n, kGroupMax);
  if (ncols < 1 || ncols > 4) QMOE_FAIL(QMOE_E_SHAPE, "ncols=%d outside 1..4", ncols);
  GroupArgs g{};
  g.n = n;
  int64_t nblk = 0, wgs = 0;
  for (int i = 0; i < n; ++i) {
    FormatInfo fi;
    int st = check_matrix(m[i].fmt, m[i].rows, m[i].k, m[i].w, m[i].w_bytes, m[i].cb, &fi);
    if (st) return st;
    if (m[i].rot != 0 && m[i].rot != 1) QMOE_FAIL(QMOE_E_FORMAT, "item %d: rot=%d unsupported (0 or 1)", i, m[i].rot);
    if (!m[i].x || !m[i].y) QMOE_FAIL(QMOE_E_INVAL, "item %d: NULL x or y", i);
    if (!aligned16(m[i].x)) QMOE_FAIL(QMOE_E_INVAL, "item %d: x not 16-byte aligned", i);
    if (m[i].rows < 1 || m[i].rows > (int64_t)1 << 31)
      QMOE_FAIL(QMOE_E_SHAPE, "item %d: rows=%lld outside 1..2^31", i, (long long)m[i].rows);
    const int nb = (int)(m[i].k / 32);
    const int nbl = m[i].fmt == QMOE_FP4 ? 1 : 2;
    const int lpr = lanes_per_row(nb, nbl);
    GroupItem& it = g.it[i];
    it.w = static_cast<const uint8_t*>(m[i].w);
    it.cb = m[i].cb;
    it.x = m[i].x;
    it.y = m[i].y;
    it.rows = m[i].rows;
    it.row_bytes = (size_t)nb * fi.block_bytes;
    it.nb = nb;
    it.lpr_log2 = ilog2(lpr);
    it.fmt = m[i].fmt;
    it.rot = m[i].rot;
    const int rpw = 64 / lpr;
    it.units = (int)((m[i].rows + rpw - 1) / rpw);
    it.blk0 = (int)nblk;
    nblk += (int64_t)ncols * nb;
    wgs += (it.units + 3) / 4;
  }
  if (nblk > (int64_t)1 << 30 || wgs > 0x7FFFFFFF)
    QMOE_FAIL(QMOE_E_SHAPE, "too many input blocks (%lld) or workgroups (%lld)", (long long)nblk, (long long)wgs);
  g.nblk = (int)nblk;
  const size_t need = group_ws_bytes(m, n, ncols);
  if (!ws) QMOE_FAIL(QMOE_E_WORKSPACE, "missing workspace (NULL)");
  if (!aligned16(ws)) QMOE_FAIL(QMOE_E_WORKSPACE, "workspace not 16-byte aligned");
  if (ws_bytes < need) QMOE_FAIL(QMOE_E_WORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  uint8_t* p = static_cast<uint8_t*>(ws);
  for (int i = 0; i < n; ++i) {
    g.it[i].xq = reinterpret_cast<int8_t*>(p);
    p += round_up((size_t)ncols * (size_t)m[i].k, 256);
    g.it[i].dx = reinterpret_cast<float*>(p);
    p += round_up((size_t)ncols * (size_t)(m[i].k / 32) * 4, 256);
  }
  hipStream_t s = as_stream(stream);
  switch (ncols) {
    case 1: return launch_group<1>(g, s);
    case 2: return launch_group<2>(g, s);
    case 3: return launch_group<3>(g, s);
    default: return launch_group<4>(g, s);
  }
}
