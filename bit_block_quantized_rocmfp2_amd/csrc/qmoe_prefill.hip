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
//   k_scan      expert offsets; the tile list (expert, first pair) of 64-pair
//               tiles of the experts with more than small_pairs pairs, and the
//               list of the experts with 1 .. small_pairs pairs (small_pairs: an
//               argument of qmoe_prefill_layer_ex, 0 .. 4)
//   k_scatter   one workgroup per expert: its pairs (t*K + s) in ascending order
//   k_gateup    per (tile, 128 rows): int8 MFMA 32x32x32 per 32-block, so every
//               MFMA result is one block's exact int32 sums; fp32 scale epilogue
//               (weight scale x activation scale) per block; SwiGLU; the 128 x 64
//               result is requantized per (pair, 32-row block) (+ H32) into hq
//   k_down      per (tile, 128 rows): the same on the down weights and hq; the
//               routing weight is applied and each pair's row stored in ypair
//   small path  the listed experts' pairs through the q <= 4 matvec arithmetic
//               (sdot4 on byte-permuted codes, qmoe_decode.hip): a tile of one to
//               four pairs would be mostly padding on the matrix cores
//   k_combine   out[t] = sum over slots s = 0..K-1 (ascending expert id) of
//               ypair[t][s]: a fixed order, so results are bit-reproducible.
// The per-pair results do not depend on a pair's position inside a tile (MFMA
// columns are independent), so the grouping within a path affects speed only.
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
constexpr int kTileM = 128;  // weight rows per matrix and workgroup (4 waves x 32)
constexpr int kKB = 8;       // 32-blocks per LDS stage (K = 256)

// Group region (int32 words): counts[E], offsets[E+1], ntiles at 2E+1 (one word
// of the cursor area), pairs[T*K] from word 3E+1, tiles (expert, first) after
// (room for T*K + E of them), then nsmall and the small-expert list [E].
struct GroupPtrs {
  int32_t* counts;
  int32_t* offsets;
  int32_t* ntiles;
  int32_t* pairs;
  int32_t* tiles;
  int32_t* nsmall;
  int32_t* small;
};

GroupPtrs group_ptrs(uint8_t* g, int E, int npairs) {
  int32_t* w = reinterpret_cast<int32_t*>(g);
  GroupPtrs p;
  p.counts = w;
  p.offsets = w + E;
  p.ntiles = w + 2 * E + 1;
  p.pairs = w + 3 * E + 1;
  p.tiles = w + 3 * E + 1 + npairs;
  p.nsmall = p.tiles + 2 * (npairs + E);
  p.small = p.nsmall + 1;
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

// One workgroup of 512 threads (E <= 512): exclusive scans of the counts, of
// the per-expert tile counts (experts with more than small_max pairs) and of
// the small-expert flags (1 .. small_max pairs), then the tile list and the
// small list.
__global__ __launch_bounds__(512) void k_scan(const int32_t* __restrict__ counts, int E, int npairs, int small_max,
                                              int32_t* offsets, int32_t* ntiles, int32_t* tiles, int32_t* nsmall,
                                              int32_t* small) {
  __shared__ int s_c[512], s_t[512], s_s[512];
  const int e = threadIdx.x;
  const int c = (e < E) ? counts[e] : 0;
  const int sm = (c >= 1 && c <= small_max) ? 1 : 0;
  const int t = sm ? 0 : (c + kTileN - 1) / kTileN;
  s_c[e] = c;
  s_t[e] = t;
  s_s[e] = sm;
  __syncthreads();
  for (int o = 1; o < 512; o <<= 1) {   // inclusive Hillis-Steele scan
    const int vc = (e >= o) ? s_c[e - o] : 0, vt = (e >= o) ? s_t[e - o] : 0, vs = (e >= o) ? s_s[e - o] : 0;
    __syncthreads();
    s_c[e] += vc;
    s_t[e] += vt;
    s_s[e] += vs;
    __syncthreads();
  }
  const int off = s_c[e] - c, toff = s_t[e] - t;
  if (e < E) offsets[e] = off;
  if (e == 0) {
    offsets[E] = npairs;
    *ntiles = s_t[511];
    *nsmall = s_s[511];
  }
  for (int i = 0; i < t; ++i) {
    tiles[2 * (toff + i)] = e;
    tiles[2 * (toff + i) + 1] = i * kTileN;
  }
  if (sm) small[s_s[e] - 1] = e;
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
// Per 32-block, one v_mfma_i32_32x32x32_i8 gives the exact int32 sums of a
// 32-row x 32-column tile (one block per instruction, the gfx950 full-rate
// form), and one v_mfma_f32_32x32x8bf16_1k forms the 32 x 32 scale products
// s_w(row) x d_x(column) in the same register layout from exact bf16 parts:
// s_w (an fp16 value, or a power of two) = s_hi + s_lo, d_x (fp32) = d_hi +
// d_mid + d_lo, every part exact in bf16 and every part product exact in fp32,
// so the K = 6 sum is the fp32 product up to the final roundings. Per element
// and block the vector ALU then does one convert and one fused multiply-add.
// Lane layouts (checked on the GPU): operand lane l holds row (or column) l % 32
// and the 16 bytes of K half l / 32; result register r of lane l is row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
typedef int v16i __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

// Weights 16h..16h+15 of one block of a row (h = K half), expanded through the
// codebook: dword k = weights 16h+4k..+3 (layout facts as in Blocks::expand).
// lo: the block's code words, hi: its FP3 bit-2 plane.
template <int FMT>
__device__ __forceinline__ v4i expand_a32(const uint32_t* lo, uint32_t hi, int h, const uint32_t cb[4]) {
  v4i a;
  if constexpr (FMT == 2 || FMT == 3) {
    const uint32_t w = lo[0];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t sel = (w >> (2 * k)) & 0x03030303u;
      if constexpr (FMT == 3) sel |= ((hi >> (4 * h + k)) & 0x01010101u) << 2;
      a[k] = (int)perm(cb[1], cb[0], sel);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t sel = (lo[k >> 1] >> (4 * (k & 1))) & 0x0F0F0F0Fu;
      const uint32_t s7 = sel & 0x07070707u;
      const uint32_t x = perm(cb[1], cb[0], s7);
      const uint32_t y = perm(cb[3], cb[2], s7);
      const uint32_t m = ((sel >> 3) & 0x01010101u) * 0xFFu;
      a[k] = (int)((y & m) | (x & ~m));
    }
  }
  return a;
}

// Exact bf16 parts (bits in the low 16 of each result word) by truncation: a
// value with at most 11 significant bits (fp16, or a power of two) is hi + lo;
// an fp32 value is hi + mid + lo (each difference is exact in fp32).
__device__ __forceinline__ void bf16_split2(float v, uint32_t& hi, uint32_t& lo) {
#pragma clang fp contract(off)
  const uint32_t hb = __float_as_uint(v) & 0xFFFF0000u;
  const float r = v - __uint_as_float(hb);
  hi = hb >> 16;
  lo = __float_as_uint(r) >> 16;
}
__device__ __forceinline__ void bf16_split3(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
#pragma clang fp contract(off)
  const uint32_t hb = __float_as_uint(v) & 0xFFFF0000u;
  const float r1 = v - __uint_as_float(hb);
  const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(mb);
  hi = hb >> 16;
  mid = mb >> 16;
  lo = __float_as_uint(r2) >> 16;
}

// LDS of one stage: NMAT matrices of 128 rows x 8 blocks and 64 columns x 8
// blocks of activations. Code words and FP3 planes are stored block-major with
// rows innermost, so the 32 rows an operand read touches are consecutive
// words. (An XOR swizzle of the row index that takes the transposed stores and
// the two K halves of a read to distinct banks measured no faster.) Scales are
// stored as their bf16 parts; the bf16 MFMA operands hold 4 bf16 per lane,
// K = 4 (l / 32) + j.
//  * Two matrices (kWideD): laid out so that the operands are plain loads: the
//    weight side is (s_hi, s_lo, s_hi, s_lo) in both halves (one word s_hi |
//    s_lo << 16, used twice), the activation side (d_hi, d_hi, d_mid, d_mid) in
//    half 0 and (d_lo, d_lo, 0, 0) in half 1.
//  * One matrix: the activation side is one (d_hi | d_mid << 16, d_lo) pair
//    per column, half its size (the down GEMM then fits four workgroups per
//    compute unit), and a lane builds its operands with byte permutes: half 0 =
//    (s_hi, s_hi, s_hi, s_lo) x (d_hi, d_mid, d_lo, d_hi), half 1 = (s_lo,
//    s_lo, 0, 0) x (d_mid, d_lo, 0, 0).
// Either way the K = 8 sum holds the six part products (s_hi + s_lo)(d_hi +
// d_mid + d_lo).
template <int FMT, int NMAT>
struct StageLds {
  static constexpr bool kWideD = NMAT == 2;
  static constexpr int LW = Fmt<FMT>::kLoWords;
  static constexpr int XS = kKB * 8 + 4;     // activation words per column (16-byte pieces, spread over banks)
  uint32_t w[NMAT][kKB][LW][kTileM];
  uint32_t h[NMAT][kKB][Fmt<FMT>::kHi ? kTileM : 1];
  uint32_t s[NMAT][kKB][kTileM];           // weight-scale bf16 parts per (block, row)
  uint32_t x[kTileN][XS];
  // activation-scale words per (block, K half, column), the halves 32 banks apart
  u32x2 d[kKB][kWideD ? 2 : 1][kWideD ? kTileN + 16 : kTileN];
};

// One-matrix operand builders (see StageLds).
__device__ __forceinline__ v4s scale_operand_w(uint32_t sp, int kh) {
  const uint32_t w0 = perm(sp, sp, kh ? 0x03020302u : 0x01000100u);   // (s_hi, s_hi) or (s_lo, s_lo)
  return __builtin_bit_cast(v4s, u32x2{w0, kh ? 0u : sp});             // (.., s_hi, s_lo) or (.., 0, 0)
}
__device__ __forceinline__ v4s scale_operand_a(u32x2 dp, int kh) {
  // half 0: (d_hi, d_mid | d_lo, d_hi); half 1: (d_mid, d_lo | 0, 0)
  const uint32_t w0 = kh ? perm(dp.x, dp.y, 0x01000706u) : dp.x;
  const uint32_t w1 = kh ? 0u : perm(dp.x, dp.y, 0x05040100u);
  return __builtin_bit_cast(v4s, u32x2{w0, w1});
}

// Loads stage `st` of NMAT weight matrices (rows row0.. of the row-planar
// tensors w0, w1) and of the activation rows (arow: int8 row of column tid >> 2,
// adrow: scale row of column (tid >> 1) & 63) into registers; store() writes
// them to LDS. 256 threads; every thread issues every load (indices wrapped into
// range), so no loaded value is defined conditionally.
template <int FMT, int NMAT, bool SCALES = true>
struct StageLoader {
  static constexpr int LW = Fmt<FMT>::kLoWords;
  static constexpr int CW = kKB * LW / 4;            // u32x4 per row of code words (4 or 8)
  static constexpr int NCODE = NMAT * kTileM * CW / 256;   // u32x4 per thread (1..4)
  static constexpr int NHI = (NMAT * 2 * kTileM + 255) / 256;  // FP3 high-plane pieces per thread
  u32x4 code[NCODE];
  u32x4 hiw[NHI]; // FP3 high planes: 8 words (2 x 16 B) per row
  u32x4 sc;       // scales of one row: fp16 8 x 2 B, or E8M0 8 x 1 B (low half)
  u32x4 act[4];   // 64 columns x 256 B: the 64-byte quarter (tid & 3) of column tid >> 2
  u32x4 adx;      // 64 columns x 32 B of activation scales: half (tid & 1) of column (tid >> 1) & 63

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
    if constexpr (Fmt<FMT>::kHi) {
      // high planes: 8 words = 32 B per row -> 2 u32x4 per row; NMAT*2*kTileM pieces
#pragma unroll
      for (int i = 0; i < NHI; ++i) {
        const int id = (tid + 256 * i) % (NMAT * 2 * kTileM);
        const int m = id / (2 * kTileM), r = (id % (2 * kTileM)) >> 1, c = id & 1;
        const uint8_t* hp = ((NMAT == 2 && m == 1) ? w1 : w0) + (size_t)(row0 + r) * row_bytes +
                            (size_t)nb * LW * 4 + (size_t)b0 * 4;
        hiw[i] = reinterpret_cast<const u32x4*>(hp)[c];
      }
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
      const int c = tid & 3;   // 64-byte quarter c of the column's 256 bytes
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
      const uint32_t v[4] = {code[i].x, code[i].y, code[i].z, code[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int q = 4 * c + k;                    // word q of the row's stage: block q / LW, word q % LW
        S.w[m][q / LW][q % LW][r] = v[k];
      }
    }
    if constexpr (Fmt<FMT>::kHi) {
#pragma unroll
      for (int i = 0; i < NHI; ++i) {
        const int id = tid + 256 * i;
        if (id < NMAT * 2 * kTileM) {
          const int m = id / (2 * kTileM), r = (id % (2 * kTileM)) >> 1, c = id & 1;
          const uint32_t v[4] = {hiw[i].x, hiw[i].y, hiw[i].z, hiw[i].w};
#pragma unroll
          for (int k = 0; k < 4; ++k) S.h[m][4 * c + k][r] = v[k];
        }
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
        uint32_t hi, lo;
        bf16_split2(f, hi, lo);
        S.s[m][b][r] = hi | (lo << 16);
      }
    }
    {
      const int j = tid >> 2, c = tid & 3;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&S.x[j][16 * c + 4 * i]) = act[i];
      if (SCALES && tid < 2 * kTileN) {
        const int jj = tid >> 1, cc = tid & 1;
        const uint32_t v[4] = {adx.x, adx.y, adx.z, adx.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t hi, mid, lo;
          bf16_split3(__uint_as_float(v[k]), hi, mid, lo);
          if constexpr (StageLds<FMT, NMAT>::kWideD) {
            S.d[4 * cc + k][0][jj] = u32x2{hi * 0x10001u, mid * 0x10001u};
            S.d[4 * cc + k][1][jj] = u32x2{lo * 0x10001u, 0u};
          } else {
            S.d[4 * cc + k][0][jj] = u32x2{hi | (mid << 16), lo};
          }
        }
      }
    }
  }
};

// The int8 products of one stage: wave w owns rows 32w .. 32w+31 of each
// matrix and the tile's columns as two 32-column subtiles (the second skipped
// when it holds no column of the tile: ncol columns hold pairs), so one
// expanded A operand feeds both. Per 32-block b, hook(b) runs once, then for
// each matrix m and subtile n one v_mfma_i32_32x32x32_i8 gives the block's
// exact int32 sums and use(b, m, n, P) consumes them (layout above). Both the
// GEMMs and the block-sum test entry point go through this function.
template <int FMT, int NMAT, int NN, typename Hook, typename Use>
__device__ __forceinline__ void stage_int8_nn(const StageLds<FMT, NMAT>& S, const uint32_t cb[NMAT][4], Hook& hook,
                                              Use& use) {
  constexpr int LW = Fmt<FMT>::kLoWords;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kh = lane >> 5;
  const int ra = 32 * wave + (lane & 31);   // A-operand row of this lane
#pragma unroll 1
  for (int b = 0; b < kKB; ++b) {
    v4i B[NN];
#pragma unroll
    for (int n = 0; n < NN; ++n) B[n] = *reinterpret_cast<const v4i*>(&S.x[32 * n + (lane & 31)][b * 8 + 4 * kh]);
    hook(b, NN);
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      uint32_t lo[2];
      if constexpr (LW == 2) {
        lo[0] = S.w[m][b][kh][ra];
        lo[1] = 0u;
      } else {
        lo[0] = S.w[m][b][2 * kh][ra];
        lo[1] = S.w[m][b][2 * kh + 1][ra];
      }
      const uint32_t hi = Fmt<FMT>::kHi ? S.h[m][b][Fmt<FMT>::kHi ? ra : 0] : 0u;
      const v4i A = expand_a32<FMT>(lo, hi, kh, cb[m]);
#pragma unroll
      for (int n = 0; n < NN; ++n) use(b, m, n, __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B[n], v16i{}, 0, 0, 0));
    }
  }
}

// Dispatches on the number of column subtiles that hold pairs (uniform), so
// each block's products are straight-line code.
template <int FMT, int NMAT, typename Hook, typename Use>
__device__ __forceinline__ void stage_int8(const StageLds<FMT, NMAT>& S, const uint32_t cb[NMAT][4], int ncol,
                                           Hook&& hook, Use&& use) {
  if (ncol > 32)
    stage_int8_nn<FMT, NMAT, 2>(S, cb, hook, use);
  else
    stage_int8_nn<FMT, NMAT, 1>(S, cb, hook, use);
}

// Multiply one stage into fp32 accumulators: acc[m][n][r] (row 32w + 8 (r / 4)
// + 4 (l / 32) + r % 4, column 32n + l % 32) += float(P) x (weight scale x
// activation scale), each 32 x 32 tile of scale products formed by the bf16
// MFMA right where it is consumed (its operands are read once per block). NN:
// the column subtiles that hold pairs (the caller picks it once per tile, so the
// accumulators are not copied between two loop forms every stage).
template <int FMT, int NMAT, int NN>
__device__ __forceinline__ void stage_mma(const StageLds<FMT, NMAT>& S, const uint32_t cb[NMAT][4],
                                          float acc[NMAT][2][16]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kh = lane >> 5;
  const int ra = 32 * wave + (lane & 31);
  v4s sop[NMAT], dop[2];
  auto hook = [&](int b, int nn) {
        if constexpr (StageLds<FMT, NMAT>::kWideD) {
#pragma unroll
          for (int n = 0; n < 2; ++n)
            if (n < nn) dop[n] = __builtin_bit_cast(v4s, S.d[b][kh][32 * n + (lane & 31)]);
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            const uint32_t sp = S.s[m][b][ra];
            sop[m] = __builtin_bit_cast(v4s, u32x2{sp, sp});
          }
        } else {
#pragma unroll
          for (int n = 0; n < 2; ++n)
            if (n < nn) dop[n] = scale_operand_a(S.d[b][0][32 * n + (lane & 31)], kh);
#pragma unroll
          for (int m = 0; m < NMAT; ++m) sop[m] = scale_operand_w(S.s[m][b][ra], kh);
        }
      };
  auto use = [&](int, int m, int n, const v16i& P) {
        const v16f pr = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(sop[m], dop[n], v16f{}, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][n][r] = fmaf((float)P[r], pr[r], acc[m][n][r]);
      };
  stage_int8_nn<FMT, NMAT, NN>(S, cb, hook, use);
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

// Stage loop shared by the GEMMs: each stage is loaded, stored to LDS and
// multiplied; the other workgroups of the compute unit overlap one another's
// loads. (Requesting stage st + 1 into registers during the products of stage st
// was measured slower: the registers it holds cost occupancy.)
template <int FMT, int NMAT, typename Load, typename Mul>
__device__ __forceinline__ void stage_loop(StageLds<FMT, NMAT>& S, int nst, Load&& load, Mul&& mul) {
  for (int st = 0; st < nst; ++st) {
    StageLoader<FMT, NMAT> L;
    load(L, st);
    __syncthreads();               // the previous stage's LDS reads are done
    L.store(S);
    __syncthreads();
    mul();
  }
}

// The stage loop of one tile with the subtile count fixed for the whole loop.
template <int FMT, int NMAT, typename Load>
__device__ __forceinline__ void tile_mma(StageLds<FMT, NMAT>& S, const uint32_t cb[NMAT][4], float acc[NMAT][2][16],
                                         int ncol, int nst, Load&& load) {
  if (ncol > 32)
    stage_loop<FMT, NMAT>(S, nst, load, [&]() { stage_mma<FMT, NMAT, 2>(S, cb, acc); });
  else
    stage_loop<FMT, NMAT>(S, nst, load, [&]() { stage_mma<FMT, NMAT, 1>(S, cb, acc); });
}

// ------------------------------------------------------------ k_gateup
// A workgroup multiplies 128 rows of gate and of up with one tile of up to 64
// pairs; wave w owns rows 32w..32w+31 of both matrices and all the tile's
// columns, so SwiGLU pairs gate and up element by element in registers.
template <int FMT>
struct GateupLds {
  union {
    StageLds<FMT, 2> stage;
    float sa[kTileN][kTileM + 4];      // SwiGLU values [pair][row] for the requantization
  };
  int pair[kTileN];
};

template <int FMT>
__global__ __launch_bounds__(256, FMT == 2 ? 3 : 2) void k_gateup(PrefillArgs a) {
  TileInfo T;
  if (!tile_info(a, T)) return;
  __shared__ GateupLds<FMT> G;
  StageLds<FMT, 2>& S = G.stage;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = blockIdx.x * kTileM;
  if (tid < kTileN) G.pair[tid] = a.pairs[T.pbase + min(tid, T.cnt - 1)];   // padding repeats a valid pair
  __syncthreads();
  // the token rows this thread loads (column tid >> 2 for bytes, (tid >> 1) & 63 for scales)
  const int8_t* arow = a.xq + (size_t)(G.pair[tid >> 2] / a.K) * a.hidden;
  const float* adrow = a.dx + (size_t)(G.pair[(tid >> 1) & (kTileN - 1)] / a.K) * a.nb_h;
  const uint8_t* wg = a.gate + (size_t)T.e * a.gu_stride;
  const uint8_t* wu = a.up + (size_t)T.e * a.gu_stride;
  uint32_t cb[2][4];
  load_codebook<FMT>(a.cb_gate + ((size_t)T.e << FMT), cb[0]);
  load_codebook<FMT>(a.cb_up + ((size_t)T.e << FMT), cb[1]);
  float acc[2][2][16];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
  tile_mma<FMT, 2>(S, cb, acc, T.cnt, a.nb_h / kKB, [&](StageLoader<FMT, 2>& L, int st) {
    L.load(wg, wu, a.gu_row_bytes, a.nb_h, row0, st * kKB, arow, adrow);
  });
  // SwiGLU into LDS as [pair][row], then requantize each (pair, 32-row block)
  __syncthreads();
#pragma unroll
  for (int n = 0; n < 2; ++n)
    if (32 * n < T.cnt) {
      const int col = 32 * n + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v;
        float* pv = reinterpret_cast<float*>(&v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = acc[0][n][4 * q + i], u = acc[1][n][4 * q + i];
          pv[i] = g / (1.0f + expf(-g)) * u;
        }
        *reinterpret_cast<float4*>(&G.sa[col][32 * wave + 8 * q + 4 * (lane >> 5)]) = v;
      }
    }
  __syncthreads();
  constexpr int RB = kTileM / 32;   // 32-row blocks per tile
  for (int pass = 0; pass < RB * kTileN / 8; ++pass) {
    const int bi = pass * 8 + wave * 2 + (lane >> 5);
    const int j = bi / RB, blk = bi % RB, jj = lane & 31;
    float d;
    const uint32_t w = quant_block32_lanes(G.sa[j][32 * blk + jj], a.rot_down, &d);
    if (j < T.cnt) {
      const size_t p = (size_t)(T.pbase + j);
      if ((jj & 3) == 0) reinterpret_cast<uint32_t*>(a.hq + p * a.inter + row0 + 32 * blk)[jj >> 2] = w;
      if (jj == 0) a.dh[p * a.nb_i + (row0 >> 5) + blk] = d;
    }
  }
}

// ------------------------------------------------------------ k_down
// A workgroup covers 128 rows of one expert's down matrix and one tile of up to
// 64 pairs (its hq rows), wave w rows 32w..32w+31; the routing weight is applied
// and each pair's rows are stored in ypair.
template <int FMT>
__global__ __launch_bounds__(256, FMT == 4 ? 3 : 4) void k_down(PrefillArgs a) {
  TileInfo T;
  if (!tile_info(a, T)) return;
  __shared__ StageLds<FMT, 1> S;
  __shared__ int s_pair[kTileN];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row0 = blockIdx.x * kTileM;
  if (tid < kTileN) s_pair[tid] = a.pairs[T.pbase + min(tid, T.cnt - 1)];
  __syncthreads();
  // hq / dh rows are indexed by the pair's sorted position (padding repeats the last)
  const int8_t* arow = a.hq + (size_t)(T.pbase + min(tid >> 2, T.cnt - 1)) * a.inter;
  const float* adrow = a.dh + (size_t)(T.pbase + min((tid >> 1) & (kTileN - 1), T.cnt - 1)) * a.nb_i;
  const uint8_t* wd = a.down + (size_t)T.e * a.dn_stride;
  uint32_t cb[1][4];
  load_codebook<FMT>(a.cb_down + ((size_t)T.e << FMT), cb[0]);
  float acc[1][2][16];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][n][r] = 0.0f;
  tile_mma<FMT, 1>(S, cb, acc, T.cnt, a.nb_i / kKB, [&](StageLoader<FMT, 1>& L, int st) {
    L.load(wd, wd, a.dn_row_bytes, a.nb_i, row0, st * kKB, arow, adrow);
  });
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int j = 32 * n + (lane & 31);
    if (j < T.cnt) {
      const int pair = s_pair[j];
      const float g = a.gw[pair];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = make_float4(acc[0][n][4 * q] * g, acc[0][n][4 * q + 1] * g, acc[0][n][4 * q + 2] * g,
                                     acc[0][n][4 * q + 3] * g);
        *reinterpret_cast<float4*>(a.ypair + (size_t)pair * a.hidden + row0 + 32 * wave + 8 * q + 4 * (lane >> 5)) = v;
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
int launch_gemms(const PrefillArgs& a, const PrefillSmall& sp, int tiles_max, int ntok, float* out, hipStream_t s) {
  {
    launch_kernel("gateup_mfma", k_gateup<FG>, dim3(a.inter / kTileM, tiles_max), dim3(256), s, a);
  }
  int st = launch_check("gateup_mfma");
  if (st) return st;
  {
    launch_kernel("down_mfma", k_down<FD>, dim3(a.hidden / kTileM, tiles_max), dim3(256), s, a);
  }
  if ((st = launch_check("down_mfma"))) return st;
  if ((st = launch_prefill_small(sp, s))) return st;
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
  const int8_t* arow = xq + (size_t)min(col0 + (tid >> 2), ncols - 1) * ((size_t)nb * 32);
  uint32_t cb[1][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) cb[0][i] = (i < Fmt<FMT>::kCbWords) ? cbw[i] : 0u;
  for (int st = 0; st < nb / kKB; ++st) {
    {
      StageLoader<FMT, 1, false> L;
      L.load(w, w, row_bytes, nb, row0, st * kKB, arow, nullptr);
      __syncthreads();
      L.store(S);
    }
    __syncthreads();
    stage_int8<FMT, 1>(
        S, cb, cnt, [](int, int) {},
        [&](int b, int, int n, const v16i& R) {
          const int c = 32 * n + (lane & 31);
          if (c < cnt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = row0 + 32 * wave + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
              P[((size_t)(col0 + c) * gridDim.x * kTileM + row) * nb + st * kKB + b] = R[r];
            }
          }
        });
  }
}

template <int FG>
int launch_gemms_g(const PrefillArgs& a, const PrefillSmall& sp, int fd, int tiles_max, int ntok, float* out,
                   hipStream_t s) {
  if (fd == 2) return launch_gemms<FG, 2>(a, sp, tiles_max, ntok, out, s);
  if (fd == 3) return launch_gemms<FG, 3>(a, sp, tiles_max, ntok, out, s);
  return launch_gemms<FG, 4>(a, sp, tiles_max, ntok, out, s);
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
  return qmoe_prefill_layer_ex(L, x, ntok, out, ws, ws_bytes, QMOE_PREFILL_SMALL_DEFAULT, stream);
}

extern "C" int qmoe_prefill_layer_ex(const qmoe_layer* L, const float* x, int32_t ntok, float* out, void* ws,
                                     size_t ws_bytes, int32_t small_pairs, void* stream) {
  clear_error();
  if (ntok < 0) QMOE_FAIL(QMOE_E_SHAPE, "ntok=%d must be >= 0", ntok);
  if (small_pairs < 0 || small_pairs > kPrefillSmallPairs)
    QMOE_FAIL(QMOE_E_INVAL, "small_pairs=%d outside 0..%d", small_pairs, kPrefillSmallPairs);
  WsPtrs w;
  int st = ws_ptrs(L, ntok > 0 ? ntok : 1, ws, ws_bytes, &w);
  if (st) return st;
  if (ntok == 0) return QMOE_OK;
  if (!x || !out) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(x) || !aligned16(out)) QMOE_FAIL(QMOE_E_INVAL, "x / out not 16-byte aligned");
  // tile shapes: rows in 128s, K in stages of 8 blocks (256 weights)
  if (L->inter % kTileM || L->hidden % kTileM || (L->hidden / 32) % kKB || (L->inter / 32) % kKB)
    QMOE_FAIL(QMOE_E_SHAPE, "prefill needs hidden and inter multiples of 256 (hidden=%d inter=%d)", L->hidden,
              L->inter);
  hipStream_t s = as_stream(stream);
  const int E = L->n_experts, K = L->topk;
  const int npairs = ntok * K;
  {   // the extents the prefill kernels address
    const size_t np = (size_t)npairs, I = L->inter, H = L->hidden;
    const size_t group_words = 3 * (size_t)E + 1 + np + 2 * (np + E) + 1 + E;
    QMOE_BOUNDS((size_t)ntok * H <= w.n_xq && (size_t)ntok * (H / 32) * 4 <= w.n_dx, "prefill: quantized tokens");
    QMOE_BOUNDS((size_t)ntok * E * 8 <= w.n_logits, "prefill: logits");
    QMOE_BOUNDS(np * 4 <= w.n_idx && np * 4 <= w.n_gw, "prefill: routing ids and weights");
    QMOE_BOUNDS(group_words * 4 <= w.n_group, "prefill: group region (counts, offsets, pairs, tiles, small list)");
    QMOE_BOUNDS((size_t)max_tiles(npairs, E) <= np + E, "prefill: tile list inside its room");
    QMOE_BOUNDS(np * I <= w.n_hq && np * (I / 32) * 4 <= w.n_dh, "prefill: requantized intermediate rows");
    QMOE_BOUNDS(np * H * 4 <= w.n_ypair, "prefill: per-pair output rows");
    QMOE_BOUNDS(I % kTileM == 0 && H % kTileM == 0, "prefill: GEMM row tiles cover the rows exactly");
  }
  if ((st = launch_quant(x, (int64_t)ntok * (L->hidden / 32), L->rot_gateup, w.xq, w.dx, s))) return st;
  if ((st = launch_route(L, x, ntok, w.logits, w.idx, w.gw, s))) return st;
  GroupPtrs g = group_ptrs(w.group, E, npairs);
  {
    launch_kernel("group_count", k_count, dim3(E), dim3(256), s, (const int32_t*)w.idx, npairs, g.counts);
    launch_kernel("group_scan", k_scan, dim3(1), dim3(512), s, (const int32_t*)g.counts, E, npairs,
                  (int)small_pairs, g.offsets, g.ntiles, g.tiles, g.nsmall, g.small);
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
  PrefillSmall sp{};
  sp.L = L;
  sp.xq = w.xq;
  sp.dx = w.dx;
  sp.counts = g.counts;
  sp.offsets = g.offsets;
  sp.pairs = g.pairs;
  sp.nsmall = g.nsmall;
  sp.small = g.small;
  sp.gw = w.gw;
  sp.hq = w.hq;
  sp.dh = w.dh;
  sp.ypair = w.ypair;
  const int tiles_max = max_tiles(npairs, E);
  switch (L->fmt_gate) {
    case 2: return launch_gemms_g<2>(a, sp, L->fmt_down, tiles_max, ntok, out, s);
    case 3: return launch_gemms_g<3>(a, sp, L->fmt_down, tiles_max, ntok, out, s);
    default: return launch_gemms_g<4>(a, sp, L->fmt_down, tiles_max, ntok, out, s);
  }
}
