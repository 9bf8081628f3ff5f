// Prefill layer (gfx950): ntok tokens through the top-k SwiGLU MoE layer with
// the (token, expert) pairs grouped by expert and each expert's tile of tokens
// multiplied on the int8 matrix cores.
//
// Page citations:
//   [evox3] soothill.io, "DeepSeek V4 Flash 0731 on evox3", table "The
//     optimization ladder": prefill gains come from batching the tokens of a
//     layer together (layer-major prefill) and from a multi-token H32 path.
//   [Strix-284B] lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
//     AMD Ryzen AI MAX+ 395", section "ROCmFPX: fitting 284B weights into 128 GB"
//     (codebook expansion by byte permutes feeding integer dot products) and
//     section "Sparse prefill: roughly 250 tok/s" (work batched layer by layer,
//     which changes the floating-point reduction order).
//
// Launch sequence (one stream, no host synchronisation):
//   quant_act   int8 per 32-block of every token (+ H32), shared by all experts
//   router/topk fp64 logits, top-k, softmax (the decode router's kernels)
//   k_count     one workgroup per expert: number of pairs routed to it (16-byte reads)
//   k_scan      expert offsets and the tile list (expert, first pair) of 64-pair tiles
//   k_scatter   one workgroup per expert: its pairs (t*K + s) in ascending order
//   k_gateup    per (tile, 64 rows): int8 MFMA 16x16x32 per 32-block, so every
//               MFMA result is one block's exact int32 sum; fp32 scale epilogue
//               (weight scale x activation scale) per block; SwiGLU; the 64 x 64
//               result is requantized per (pair, 32-row block) (+ H32) into hq
//   k_down      per (tile, 64 rows): the same on the down weights and hq; the
//               routing weight is applied and each pair's row stored in ypair
//   k_combine   out[t] = sum over slots s = 0..K-1 (ascending expert id) of
//               ypair[t][s]: a fixed order, so results are bit-reproducible.
// The per-pair results do not depend on a pair's position inside a tile (MFMA
// columns are independent), so the grouping affects speed only.
#include <hip/hip_runtime.h>

#include "qmoe_device.h"
#include "qmoe_host.h"
#include "qmoe_internal.h"

using namespace qk;
using namespace qmoe;

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTileN = 64;   // pairs (tokens) per tile
constexpr int kTileM = 64;   // weight rows per workgroup
constexpr int kKB = 8;       // 32-blocks per LDS stage (K = 256)

// Group region (int32 words): counts[E], offsets[E+1], ntiles at 2E+1 (one word
// of the cursor area), pairs[T*K] from word 3E+1, tiles (expert, first) after.
struct GroupPtrs {
  int32_t* counts;
  int32_t* offsets;
  int32_t* ntiles;
  int32_t* pairs;
  int32_t* tiles;
};

GroupPtrs group_ptrs(uint8_t* g, int E, int npairs) {
  int32_t* w = reinterpret_cast<int32_t*>(g);
  GroupPtrs p;
  p.counts = w;
  p.offsets = w + E;
  p.ntiles = w + 2 * E + 1;
  p.pairs = w + 3 * E + 1;
  p.tiles = w + 3 * E + 1 + npairs;
  return p;
}

// Upper bound on the number of 64-pair tiles: sum_e ceil(c_e / 64) <= npairs/64 + E.
int max_tiles(int npairs, int E) { return (npairs + kTileN - 1) / kTileN + E; }

// ------------------------------------------------------------ grouping
__device__ __forceinline__ int block_sum_256(int v, int* s_red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  const int r = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  __syncthreads();
  return r;
}

// Pair ids are read 16 bytes per lane (when idx is 16-byte aligned, as the
// workspace places it), kCountBatch pieces per lane in flight at once.
constexpr int kCountBatch = 8;

__global__ __launch_bounds__(256) void k_count(const int32_t* __restrict__ idx, int npairs, int32_t* counts) {
  __shared__ int s_red[4];
  const int e = blockIdx.x;
  const uint32_t ue = (uint32_t)e;
  int c = 0;
  const int n4 = ((reinterpret_cast<uintptr_t>(idx) & 15u) == 0) ? npairs / 4 : 0;
  const u32x4* v4 = reinterpret_cast<const u32x4*>(idx);
  for (int q0 = threadIdx.x; q0 < n4; q0 += 256 * kCountBatch) {
    u32x4 v[kCountBatch];
#pragma unroll
    for (int k = 0; k < kCountBatch; ++k) v[k] = v4[min(q0 + 256 * k, n4 - 1)];
    // an empty asm taking every piece keeps all the loads ahead of their uses
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]));
#pragma unroll
    for (int k = 0; k < kCountBatch; ++k) {
      const int n = (v[k].x == ue) + (v[k].y == ue) + (v[k].z == ue) + (v[k].w == ue);
      c += (q0 + 256 * k < n4) ? n : 0;
    }
  }
  for (int p = 4 * n4 + threadIdx.x; p < npairs; p += 256) c += (idx[p] == e) ? 1 : 0;
  c = block_sum_256(c, s_red);
  if (threadIdx.x == 0) counts[e] = c;
}

// One workgroup of 512 threads (E <= 512): exclusive scans of the counts and of
// the per-expert tile counts, then the tile list.
__global__ __launch_bounds__(512) void k_scan(const int32_t* __restrict__ counts, int E, int npairs,
                                              int32_t* offsets, int32_t* ntiles, int32_t* tiles) {
  __shared__ int s_c[512], s_t[512];
  const int e = threadIdx.x;
  const int c = (e < E) ? counts[e] : 0;
  const int t = (c + kTileN - 1) / kTileN;
  s_c[e] = c;
  s_t[e] = t;
  __syncthreads();
  for (int o = 1; o < 512; o <<= 1) {   // inclusive Hillis-Steele scan
    const int vc = (e >= o) ? s_c[e - o] : 0, vt = (e >= o) ? s_t[e - o] : 0;
    __syncthreads();
    s_c[e] += vc;
    s_t[e] += vt;
    __syncthreads();
  }
  const int off = s_c[e] - c, toff = s_t[e] - t;
  if (e < E) offsets[e] = off;
  if (e == 0) {
    offsets[E] = npairs;
    *ntiles = s_t[511];
  }
  for (int i = 0; i < t; ++i) {
    tiles[2 * (toff + i)] = e;
    tiles[2 * (toff + i) + 1] = i * kTileN;
  }
}

// Workgroup e writes the pairs routed to expert e in ascending order. With a
// 16-byte aligned idx, each pass covers 1024 pairs: lane tid holds pairs
// 4q..4q+3 (q = pass base + tid), and a workgroup-wide exclusive scan of the
// lanes' match counts, in lane order, places them; the last npairs % 4 pairs
// (and an unaligned idx) take passes of 256 pairs with one pair per lane.
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ idx, int npairs,
                                                 const int32_t* __restrict__ offsets, int32_t* pairs) {
  __shared__ int s_w[4];
  const int e = blockIdx.x;
  const uint32_t ue = (uint32_t)e;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int pos = offsets[e];
  const int n4 = ((reinterpret_cast<uintptr_t>(idx) & 15u) == 0) ? npairs / 4 : 0;
  const u32x4* v4 = reinterpret_cast<const u32x4*>(idx);
  for (int q0 = 0; q0 < n4; q0 += 256) {
    const int q = q0 + (int)threadIdx.x;
    const u32x4 v = v4[min(q, n4 - 1)];
    const bool ok = q < n4;
    const bool m0 = ok && v.x == ue, m1 = ok && v.y == ue, m2 = ok && v.z == ue, m3 = ok && v.w == ue;
    const int cnt = (int)m0 + (int)m1 + (int)m2 + (int)m3;
    int incl = cnt;   // inclusive scan over the wave's lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) before += (w < wave) ? s_w[w] : 0;
    const int total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    int at = pos + before + incl - cnt;
    if (m0) pairs[at++] = 4 * q;
    if (m1) pairs[at++] = 4 * q + 1;
    if (m2) pairs[at++] = 4 * q + 2;
    if (m3) pairs[at] = 4 * q + 3;
    pos += total;
    __syncthreads();
  }
  for (int p0 = 4 * n4; p0 < npairs; p0 += 256) {
    const int p = p0 + threadIdx.x;
    const bool m = p < npairs && idx[p] == e;
    const uint64_t b = __ballot(m);
    if (lane == 0) s_w[wave] = __popcll(b);
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) before += (w < wave) ? s_w[w] : 0;
    const int total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    if (m) pairs[pos + before + __popcll(b & ((1ull << lane) - 1ull))] = p;
    pos += total;
    __syncthreads();
  }
}

// ------------------------------------------------------------ MFMA tiles
// One 32-block of a weight row, as the A operand of v_mfma_i32_16x16x32_i8: lane
// l holds row l % 16 and the 8 weights 8q..8q+7 (q = l / 16), i.e. expanded
// dwords 2q and 2q+1 of the block (see Blocks::expand for the layout facts).
template <int FMT>
__device__ __forceinline__ long expand_a(const uint32_t* lo, uint32_t hi, int q, const uint32_t cb[4]) {
  uint32_t a0, a1;
  if constexpr (FMT == 2 || FMT == 3) {
    const uint32_t w = lo[q >> 1];
    const int k0 = (2 * q) & 3;
    uint32_t s0 = (w >> (2 * k0)) & 0x03030303u, s1 = (w >> (2 * k0 + 2)) & 0x03030303u;
    if constexpr (FMT == 3) {
      s0 |= ((hi >> (2 * q)) & 0x01010101u) << 2;
      s1 |= ((hi >> (2 * q + 1)) & 0x01010101u) << 2;
    }
    a0 = perm(cb[1], cb[0], s0);
    a1 = perm(cb[1], cb[0], s1);
  } else {
    const uint32_t w = lo[q];
    uint32_t r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t sel = (w >> (4 * h)) & 0x0F0F0F0Fu;
      const uint32_t s7 = sel & 0x07070707u;
      const uint32_t x = perm(cb[1], cb[0], s7);
      const uint32_t y = perm(cb[3], cb[2], s7);
      const uint32_t m = ((sel >> 3) & 0x01010101u) * 0xFFu;
      r[h] = (y & m) | (x & ~m);
    }
    a0 = r[0];
    a1 = r[1];
  }
  return (long)(((uint64_t)a1 << 32) | a0);
}

// LDS for one stage of a 64-row weight tile (up to two matrices) and a 64-pair
// activation tile. Row strides are padded by 4 dwords (16-byte aligned rows).
template <int FMT, int NMAT>
struct StageLds {
  static constexpr int LW = Fmt<FMT>::kLoWords;
  static constexpr int WS = kKB * LW + 4;    // code words per row
  static constexpr int HS = kKB + 4;         // high-plane words per row
  static constexpr int XS = kKB * 8 + 4;     // activation words per pair
  uint32_t w[NMAT][kTileM][WS];
  uint32_t h[NMAT][Fmt<FMT>::kHi ? kTileM : 1][HS];
  float s[NMAT][kKB][kTileM];                // weight scales, block-major
  uint32_t x[kTileN][XS];
  float dx[kKB][kTileN];                     // activation scales, block-major
};

// Loads stage `st` of NMAT weight matrices (rows row0.. of the row-planar
// tensors `wm[]`) and of the activation rows `arow[j]` into registers, then
// stores them to LDS. Thread layout: 256 threads; each weight row's KB blocks of
// code bytes (KB*LW*4 bytes) are read as 16-byte pieces.
template <int FMT, int NMAT, bool SCALES = true>
struct StageLoader {
  static constexpr int LW = Fmt<FMT>::kLoWords;
  static constexpr int CW = kKB * LW / 4;            // u32x4 per row of code words (4 or 8)
  static constexpr int NCODE = NMAT * kTileM * CW / 256;   // u32x4 per thread (1..4)
  u32x4 code[NCODE];
  u32x4 hiw;      // FP3 high planes: 8 words (2 x 16 B) per row, one piece per thread
  u32x4 sc;       // scales of one row: fp16 8 x 2 B, or E8M0 8 x 1 B (low half)
  u32x4 act[4];   // 64 pairs x 256 B: the 64-byte quarter (tid & 3) of pair tid >> 2
  u32x4 adx;      // 64 pairs x 32 B of activation scales: half (tid & 1) of pair tid >> 1

  // arow: int8 activation row of pair tid >> 2; adrow: scale row of pair tid >> 1
  // w0, w1: the weight matrices (w1 is used when NMAT == 2)
  // (SCALES = false: the weight and activation scales are neither loaded nor
  // stored, and adrow is not read)
  __device__ __forceinline__ void load(const uint8_t* w0, const uint8_t* w1, size_t row_bytes, int nb, int row0,
                                       int b0, const int8_t* arow, const float* adrow) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NCODE; ++i) {
      const int id = tid + 256 * i;                 // 0 .. NMAT*64*CW-1
      const int m = id / (kTileM * CW), rem = id % (kTileM * CW);
      const int r = rem / CW, c = rem % CW;
      const uint8_t* wb = (NMAT == 2 && m == 1) ? w1 : w0;
      code[i] = reinterpret_cast<const u32x4*>(wb + (size_t)(row0 + r) * row_bytes + (size_t)b0 * LW * 4)[c];
    }
    // Every thread issues every load (indices wrapped into range); only the LDS
    // stores are restricted, so no value is defined conditionally.
    if constexpr (Fmt<FMT>::kHi) {
      // high planes: 8 words = 32 B per row -> 2 u32x4 per row; NMAT*128 pieces
      const int id = tid % (NMAT * 128);
      const int m = id / 128, r = (id % 128) >> 1, c = id & 1;
      const uint8_t* hp = ((NMAT == 2 && m == 1) ? w1 : w0) + (size_t)(row0 + r) * row_bytes + (size_t)nb * LW * 4 +
                          (size_t)b0 * 4;
      hiw = reinterpret_cast<const u32x4*>(hp)[c];
    }
    if constexpr (SCALES) {
      const size_t sc_off = (size_t)nb * (LW * 4 + 4 * Fmt<FMT>::kHi);
      const int id = tid % (NMAT * kTileM);
      const int m = id / kTileM, r = id % kTileM;
      const uint8_t* sp = ((NMAT == 2 && m == 1) ? w1 : w0) + (size_t)(row0 + r) * row_bytes + sc_off +
                          (size_t)b0 * Fmt<FMT>::kScaleBytes;
      if constexpr (Fmt<FMT>::kScaleBytes == 2) {
        sc = *reinterpret_cast<const u32x4*>(sp);
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(sp);
        sc = u32x4{v.x, v.y, 0u, 0u};
      }
    }
    {
      const int c = tid & 3;   // 64-byte quarter c of the pair's 256 bytes
      const u32x4* src = reinterpret_cast<const u32x4*>(arow + (size_t)b0 * 32) + 4 * c;
#pragma unroll
      for (int i = 0; i < 4; ++i) act[i] = src[i];
      if constexpr (SCALES) adx = reinterpret_cast<const u32x4*>(adrow + b0)[tid & 1];
    }
  }

  __device__ __forceinline__ void store(StageLds<FMT, NMAT>& S) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NCODE; ++i) {
      const int id = tid + 256 * i;
      const int m = id / (kTileM * CW), rem = id % (kTileM * CW);
      const int r = rem / CW, c = rem % CW;
      *reinterpret_cast<u32x4*>(&S.w[m][r][4 * c]) = code[i];
    }
    if constexpr (Fmt<FMT>::kHi) {
      if (tid < NMAT * 128) {
        const int m = tid / 128, r = (tid % 128) >> 1, c = tid & 1;
        *reinterpret_cast<u32x4*>(&S.h[m][r][4 * c]) = hiw;
      }
    }
    if (SCALES && tid < NMAT * kTileM) {
      const int m = tid / kTileM, r = tid % kTileM;
      const uint32_t v[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
      for (int b = 0; b < kKB; ++b) {
        float f;
        if constexpr (Fmt<FMT>::kScaleBytes == 2)
          f = half_bits_to_float((v[b >> 1] >> (16 * (b & 1))) & 0xFFFFu);
        else
          f = e8m0_to_float((v[b >> 2] >> (8 * (b & 3))) & 0xFFu);
        S.s[m][b][r] = f;
      }
    }
    {
      const int j = tid >> 2, c = tid & 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&S.x[j][16 * c + 4 * i]) = act[i];
      if (SCALES && tid < 2 * kTileN) {
        const int jj = tid >> 1, cc = tid & 1;
        S.dx[4 * cc + 0][jj] = __uint_as_float(adx.x);
        S.dx[4 * cc + 1][jj] = __uint_as_float(adx.y);
        S.dx[4 * cc + 2][jj] = __uint_as_float(adx.z);
        S.dx[4 * cc + 3][jj] = __uint_as_float(adx.w);
      }
    }
  }
};

// The int8 products of one stage: wave w owns rows 16w..16w+15 of each matrix
// and the tile's pairs as up to four 16-column MFMA tiles (nn of them hold
// pairs). Per 32-block b, hook(b) runs once, then for each subtile n < nn and
// matrix m one v_mfma_i32_16x16x32_i8 gives the block's exact int32 sums and
// use(b, m, n, P) consumes them: P[r] in lane l is row 16w + 4q + r, column
// 16n + l % 16 (q = l / 16). Both the GEMMs and the block-sum test entry point
// go through this function.
template <int FMT, int NMAT, typename Hook, typename Use>
__device__ __forceinline__ void stage_int8(const StageLds<FMT, NMAT>& S, const uint32_t cb[NMAT][4], int nn,
                                           Hook&& hook, Use&& use) {
  constexpr int LW = Fmt<FMT>::kLoWords;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i16 = lane & 15, q = lane >> 4;
  const int ra = 16 * wave + i16;          // A-operand row of this lane
#pragma unroll 2
  for (int b = 0; b < kKB; ++b) {
    long A[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
      A[m] = expand_a<FMT>(&S.w[m][ra][b * LW], Fmt<FMT>::kHi ? S.h[m][Fmt<FMT>::kHi ? ra : 0][b] : 0u, q, cb[m]);
    hook(b);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if (n < nn) {   // 16-column subtiles beyond the tile's pairs are skipped (uniform)
        const int col = 16 * n + i16;
        const long B = *reinterpret_cast<const long*>(&S.x[col][b * 8 + 2 * q]);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) use(b, m, n, __builtin_amdgcn_mfma_i32_16x16x32_i8(A[m], B, v4i{0, 0, 0, 0}, 0, 0, 0));
      }
    }
  }
}

// Multiply one stage into fp32 accumulators: acc[m][n][r] (row 16w + 4q + r,
// column 16n + l % 16) += float(P) x (weight scale x activation scale).
// The scale products of one block form a 64-column x 16-row outer product per
// matrix; one fp32 4-block MFMA (K = 1, one rounding per product, as a plain
// fp32 multiply) leaves product (16n + l % 16, row 16w + 4q + r) in register
// 4n + r of lane l, the same place as the int32 result it scales, which takes
// the multiply off the vector ALU: per element and block only the convert and
// the fused multiply-add remain.
template <int FMT, int NMAT>
__device__ __forceinline__ void stage_mma(const StageLds<FMT, NMAT>& S, const uint32_t cb[NMAT][4],
                                          float acc[NMAT][4][4], int nn) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ra = 16 * wave + (lane & 15);
  v16f p[NMAT];
  stage_int8<FMT, NMAT>(
      S, cb, nn,
      [&](int b) {
        const float dl = S.dx[b][lane];    // activation scale of column `lane`
#pragma unroll
        for (int m = 0; m < NMAT; ++m) p[m] = __builtin_amdgcn_mfma_f32_16x16x1f32(S.s[m][b][ra], dl, v16f{}, 0, 0, 0);
      },
      [&](int, int m, int n, const v4i& P) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[m][n][r] = fmaf((float)P[r], p[m][4 * n + r], acc[m][n][r]);
      });
}

struct PrefillArgs {
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  const int8_t* cb_gate;
  const int8_t* cb_up;
  const int8_t* cb_down;
  const int8_t* xq;
  const float* dx;
  const float* gw;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* ntiles;
  const int32_t* pairs;
  const int32_t* tiles;
  int8_t* hq;
  float* dh;
  float* ypair;
  size_t gu_row_bytes, gu_stride, dn_row_bytes, dn_stride;
  int hidden, inter, K, rot_down;
  int nb_h, nb_i;
};

// Tile header shared by both GEMM kernels.
struct TileInfo {
  int e, first, cnt, pbase;
};

// Grid: x = 64-row weight tile, y = pair tile. Workgroups are dispatched in x-
// fastest order and spread over the 8 XCDs by id modulo 8: all row tiles of one
// pair tile run close together (its activations are fetched once per XCD), and
// when the row-tile count is a multiple of 8 (32 and 64 for inter 2048 and
// hidden 4096) each row tile's weights stay on one XCD for every pair tile.
__device__ __forceinline__ bool tile_info(const PrefillArgs& a, TileInfo& t) {
  if ((int)blockIdx.y >= *a.ntiles) return false;
  t.e = a.tiles[2 * blockIdx.y];
  t.first = a.tiles[2 * blockIdx.y + 1];
  t.cnt = min(kTileN, a.counts[t.e] - t.first);
  t.pbase = a.offsets[t.e] + t.first;
  return true;
}

// ------------------------------------------------------------ k_gateup
template <int FMT>
__global__ __launch_bounds__(256) void k_gateup(PrefillArgs a) {
  TileInfo T;
  if (!tile_info(a, T)) return;
  __shared__ StageLds<FMT, 2> S;
  __shared__ int s_pair[kTileN];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = blockIdx.x * kTileM;
  const int nn = (T.cnt + 15) >> 4;   // 16-column subtiles holding pairs
  if (tid < kTileN) s_pair[tid] = a.pairs[T.pbase + min(tid, T.cnt - 1)];   // padding repeats a valid pair
  __syncthreads();
  // the token rows this thread loads (pair tid >> 2 for bytes, tid >> 1 for scales)
  const int8_t* arow = a.xq + (size_t)(s_pair[tid >> 2] / a.K) * a.hidden;
  const float* adrow = a.dx + (size_t)(s_pair[(tid >> 1) & (kTileN - 1)] / a.K) * a.nb_h;
  const uint8_t* wg = a.gate + (size_t)T.e * a.gu_stride;
  const uint8_t* wu = a.up + (size_t)T.e * a.gu_stride;
  uint32_t cb[2][4];
  load_codebook<FMT>(a.cb_gate + ((size_t)T.e << FMT), cb[0]);
  load_codebook<FMT>(a.cb_up + ((size_t)T.e << FMT), cb[1]);
  float acc[2][4][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][n][r] = 0.0f;
  // two weight matrices leave no registers for a prefetch at four waves per SIMD:
  // each stage is loaded, stored to LDS and multiplied (other workgroups overlap)
  const int nst = a.nb_h / kKB;
  for (int st = 0; st < nst; ++st) {
    {
      StageLoader<FMT, 2> L;
      L.load(wg, wu, a.gu_row_bytes, a.nb_h, row0, st * kKB, arow, adrow);
      __syncthreads();               // the previous stage's LDS reads are done
      L.store(S);
    }
    __syncthreads();
    stage_mma<FMT, 2>(S, cb, acc, nn);
  }
  // SwiGLU into LDS as [pair][row] (reusing the activation stage buffer), then
  // requantize each (pair, 32-row block).
  __syncthreads();
  float* sa = reinterpret_cast<float*>(&S.x[0][0]);   // 64 x 68 floats fit in x (64 x 68 words)
  constexpr int AS = StageLds<FMT, 2>::XS;
  {
    const int i16 = lane & 15, q = lane >> 4;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      float4 v;
      float* pv = reinterpret_cast<float*>(&v);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float g = acc[0][n][r], u = acc[1][n][r];
        pv[r] = g / (1.0f + expf(-g)) * u;
      }
      *reinterpret_cast<float4*>(&sa[(16 * n + i16) * AS + 16 * wave + 4 * q]) = v;
    }
  }
  __syncthreads();
  for (int pass = 0; pass < 2 * kTileN / 8; ++pass) {
    const int bi = pass * 8 + wave * 2 + (lane >> 5);
    const int j = bi >> 1, blk = bi & 1, jj = lane & 31;
    float d;
    const uint32_t w = quant_block32_lanes(sa[j * AS + 32 * blk + jj], a.rot_down, &d);
    if (j < T.cnt) {
      const size_t p = (size_t)(T.pbase + j);
      if ((jj & 3) == 0) reinterpret_cast<uint32_t*>(a.hq + p * a.inter + row0 + 32 * blk)[jj >> 2] = w;
      if (jj == 0) a.dh[p * a.nb_i + (row0 >> 5) + blk] = d;
    }
  }
}

// ------------------------------------------------------------ k_down
// A workgroup covers 128 rows as two 64-row halves multiplied like the gate and
// up matrices of k_gateup, so each activation operand read from LDS feeds twice
// the MFMAs.
template <int FMT>
__global__ __launch_bounds__(256) void k_down(PrefillArgs a) {
  TileInfo T;
  if (!tile_info(a, T)) return;
  __shared__ StageLds<FMT, 2> S;
  __shared__ int s_pair[kTileN];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = blockIdx.x * 2 * kTileM;
  const int nn = (T.cnt + 15) >> 4;
  if (tid < kTileN) s_pair[tid] = a.pairs[T.pbase + min(tid, T.cnt - 1)];
  __syncthreads();
  // hq / dh rows are indexed by the pair's sorted position (padding repeats the last)
  const int8_t* arow = a.hq + (size_t)(T.pbase + min(tid >> 2, T.cnt - 1)) * a.inter;
  const float* adrow = a.dh + (size_t)(T.pbase + min((tid >> 1) & (kTileN - 1), T.cnt - 1)) * a.nb_i;
  const uint8_t* wd = a.down + (size_t)T.e * a.dn_stride;
  const uint8_t* wd_hi = wd + (size_t)kTileM * a.dn_row_bytes;   // the second 64-row half
  uint32_t cb[2][4];
  load_codebook<FMT>(a.cb_down + ((size_t)T.e << FMT), cb[0]);
#pragma unroll
  for (int i = 0; i < 4; ++i) cb[1][i] = cb[0][i];
  float acc[2][4][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][n][r] = 0.0f;
  const int nst = a.nb_i / kKB;
  for (int st = 0; st < nst; ++st) {
    {
      StageLoader<FMT, 2> L;
      L.load(wd, wd_hi, a.dn_row_bytes, a.nb_i, row0, st * kKB, arow, adrow);
      __syncthreads();
      L.store(S);
    }
    __syncthreads();
    stage_mma<FMT, 2>(S, cb, acc, nn);
  }
  const int i16 = lane & 15, q = lane >> 4;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int j = 16 * n + i16;
    if (j < T.cnt) {
      const int pair = s_pair[j];
      const float g = a.gw[pair];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float4 v = make_float4(acc[m][n][0] * g, acc[m][n][1] * g, acc[m][n][2] * g, acc[m][n][3] * g);
        *reinterpret_cast<float4*>(a.ypair + (size_t)pair * a.hidden + row0 + kTileM * m + 16 * wave + 4 * q) = v;
      }
    }
  }
}

// ------------------------------------------------------------ k_combine
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ ypair, int ntok, int K, int hidden,
                                                 float* __restrict__ out) {
  const size_t n4 = (size_t)ntok * hidden / 4;
  const int h4 = hidden / 4;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t t = i / h4, c = i % h4;
    const float4* src = reinterpret_cast<const float4*>(ypair + t * K * hidden) + c;
    float4 s = src[0];
    for (int k = 1; k < K; ++k) {
      const float4 v = src[(size_t)k * h4];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    reinterpret_cast<float4*>(out)[i] = s;
  }
}

template <int FG, int FD>
int launch_gemms(const PrefillArgs& a, int tiles_max, int ntok, float* out, hipStream_t s) {
  {
    launch_kernel("gateup_mfma", k_gateup<FG>, dim3(a.inter / kTileM, tiles_max), dim3(256), s, a);
  }
  int st = launch_check("gateup_mfma");
  if (st) return st;
  {
    launch_kernel("down_mfma", k_down<FD>, dim3(a.hidden / (2 * kTileM), tiles_max), dim3(256), s, a);
  }
  if ((st = launch_check("down_mfma"))) return st;
  {
    const size_t n4 = (size_t)ntok * a.hidden / 4;
    const unsigned grid = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
    launch_kernel("combine", k_combine, dim3(grid), dim3(256), s, a.ypair, ntok, a.K, a.hidden, out);
  }
  return launch_check("combine");
}

// ------------------------------------------------------------ raw block sums (test entry point)
// One workgroup per 64 rows x 64 columns: the prefill stage loader and
// stage_int8 with NMAT = 1, writing every int32 MFMA result to
// P[col][row][block] instead of scaling it. Columns past ncols repeat the last
// column in LDS and are not stored.
template <int FMT>
__global__ __launch_bounds__(256) void k_block_dots_mfma(const uint8_t* __restrict__ w, size_t row_bytes, int nb,
                                                         const uint32_t* __restrict__ cbw, const int8_t* __restrict__ xq,
                                                         int ncols, int32_t* __restrict__ P) {
  __shared__ StageLds<FMT, 1> S;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = blockIdx.x * kTileM, col0 = blockIdx.y * kTileN;
  const int cnt = min(kTileN, ncols - col0);
  const int nn = (cnt + 15) >> 4;
  const int8_t* arow = xq + (size_t)min(col0 + (tid >> 2), ncols - 1) * ((size_t)nb * 32);
  uint32_t cb[1][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) cb[0][i] = (i < Fmt<FMT>::kCbWords) ? cbw[i] : 0u;
  const int i16 = lane & 15, q = lane >> 4;
  for (int st = 0; st < nb / kKB; ++st) {
    {
      StageLoader<FMT, 1, false> L;
      L.load(w, w, row_bytes, nb, row0, st * kKB, arow, nullptr);
      __syncthreads();
      L.store(S);
    }
    __syncthreads();
    stage_int8<FMT, 1>(
        S, cb, nn, [](int) {},
        [&](int b, int, int n, const v4i& R) {
          const int col = col0 + 16 * n + i16;
          if (16 * n + i16 < cnt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = row0 + 16 * wave + 4 * q + r;
              P[((size_t)col * gridDim.x * kTileM + row) * nb + st * kKB + b] = R[r];
            }
          }
        });
  }
}

template <int FG>
int launch_gemms_g(const PrefillArgs& a, int fd, int tiles_max, int ntok, float* out, hipStream_t s) {
  if (fd == 2) return launch_gemms<FG, 2>(a, tiles_max, ntok, out, s);
  if (fd == 3) return launch_gemms<FG, 3>(a, tiles_max, ntok, out, s);
  return launch_gemms<FG, 4>(a, tiles_max, ntok, out, s);
}

}  // namespace

extern "C" int qmoe_block_dots_mfma(int fmt, int64_t rows, int64_t k, const void* w, size_t w_bytes,
                                    const int8_t* cb, const int8_t* xq, int32_t ncols, int32_t* P, void* stream) {
  clear_error();
  FormatInfo fi;
  int st = check_matrix(fmt, rows, k, w, w_bytes, cb, &fi);
  if (st) return st;
  if (ncols < 1 || ncols > kTileN) QMOE_FAIL(QMOE_E_SHAPE, "ncols=%d outside 1..%d", ncols, kTileN);
  if (rows % kTileM || k % (32 * kKB))
    QMOE_FAIL(QMOE_E_SHAPE, "rows=%lld must be a multiple of %d and k=%lld of %d", (long long)rows, kTileM,
              (long long)k, 32 * kKB);
  if (rows == 0) return QMOE_OK;
  if ((rows / kTileM) > 0x7FFFFFFF || (size_t)ncols * rows * (k / 32) > ((size_t)1 << 40))
    QMOE_FAIL(QMOE_E_SHAPE, "rows=%lld too large", (long long)rows);
  if (!xq || !P) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(xq) || (reinterpret_cast<uintptr_t>(P) & 3)) QMOE_FAIL(QMOE_E_INVAL, "xq not 16-byte / P not 4-byte aligned");
  const int nb = (int)(k / 32);
  const size_t row_bytes = (size_t)nb * fi.block_bytes;
  const dim3 grid((unsigned)(rows / kTileM), 1);
  hipStream_t s = as_stream(stream);
  const uint8_t* W = static_cast<const uint8_t*>(w);
  const uint32_t* cbw = reinterpret_cast<const uint32_t*>(cb);
  switch (fmt) {
    case 2: launch_kernel("block_dots_mfma", k_block_dots_mfma<2>, grid, dim3(256), s, W, row_bytes, nb, cbw, xq, (int)ncols, P); break;
    case 3: launch_kernel("block_dots_mfma", k_block_dots_mfma<3>, grid, dim3(256), s, W, row_bytes, nb, cbw, xq, (int)ncols, P); break;
    default: launch_kernel("block_dots_mfma", k_block_dots_mfma<4>, grid, dim3(256), s, W, row_bytes, nb, cbw, xq, (int)ncols, P); break;
  }
  return launch_check("block_dots_mfma");
}

extern "C" int qmoe_prefill_layer(const qmoe_layer* L, const float* x, int32_t ntok, float* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  clear_error();
  if (ntok < 0) QMOE_FAIL(QMOE_E_SHAPE, "ntok=%d must be >= 0", ntok);
  WsPtrs w;
  int st = ws_ptrs(L, ntok > 0 ? ntok : 1, ws, ws_bytes, &w);
  if (st) return st;
  if (ntok == 0) return QMOE_OK;
  if (!x || !out) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(x) || !aligned16(out)) QMOE_FAIL(QMOE_E_INVAL, "x / out not 16-byte aligned");
  // tile shapes: rows in 64s, K in stages of 8 blocks (guaranteed by the 16-byte row rule)
  if (L->inter % kTileM || L->hidden % (2 * kTileM) || (L->hidden / 32) % kKB || (L->inter / 32) % kKB)
    QMOE_FAIL(QMOE_E_SHAPE, "prefill needs hidden and inter multiples of 256 (hidden=%d inter=%d)", L->hidden,
              L->inter);
  hipStream_t s = as_stream(stream);
  const int E = L->n_experts, K = L->topk;
  const int npairs = ntok * K;
  if ((st = launch_quant(x, (int64_t)ntok * (L->hidden / 32), L->rot_gateup, w.xq, w.dx, s))) return st;
  if ((st = launch_route(L, x, ntok, w.logits, w.idx, w.gw, s))) return st;
  GroupPtrs g = group_ptrs(w.group, E, npairs);
  {
    launch_kernel("group_count", k_count, dim3(E), dim3(256), s, (const int32_t*)w.idx, npairs, g.counts);
    launch_kernel("group_scan", k_scan, dim3(1), dim3(512), s, (const int32_t*)g.counts, E, npairs, g.offsets, g.ntiles,
                  g.tiles);
    launch_kernel("group_scatter", k_scatter, dim3(E), dim3(256), s, (const int32_t*)w.idx, npairs,
                  (const int32_t*)g.offsets, g.pairs);
  }
  if ((st = launch_check("group"))) return st;
  FormatInfo fg, fd;
  format_info(L->fmt_gate, &fg);
  format_info(L->fmt_down, &fd);
  PrefillArgs a{};
  a.gate = static_cast<const uint8_t*>(L->gate);
  a.up = static_cast<const uint8_t*>(L->up);
  a.down = static_cast<const uint8_t*>(L->down);
  a.cb_gate = L->cb_gate;
  a.cb_up = L->cb_up;
  a.cb_down = L->cb_down;
  a.xq = w.xq;
  a.dx = w.dx;
  a.gw = w.gw;
  a.counts = g.counts;
  a.offsets = g.offsets;
  a.ntiles = g.ntiles;
  a.pairs = g.pairs;
  a.tiles = g.tiles;
  a.hq = w.hq;
  a.dh = w.dh;
  a.ypair = w.ypair;
  a.hidden = L->hidden;
  a.inter = L->inter;
  a.K = K;
  a.rot_down = L->rot_down;
  a.nb_h = L->hidden / 32;
  a.nb_i = L->inter / 32;
  a.gu_row_bytes = (size_t)a.nb_h * fg.block_bytes;
  a.gu_stride = a.gu_row_bytes * L->inter;
  a.dn_row_bytes = (size_t)a.nb_i * fd.block_bytes;
  a.dn_stride = a.dn_row_bytes * L->hidden;
  const int tiles_max = max_tiles(npairs, E);
  switch (L->fmt_gate) {
    case 2: return launch_gemms_g<2>(a, L->fmt_down, tiles_max, ntok, out, s);
    case 3: return launch_gemms_g<3>(a, L->fmt_down, tiles_max, ntok, out, s);
    default: return launch_gemms_g<4>(a, L->fmt_down, tiles_max, ntok, out, s);
  }
}
