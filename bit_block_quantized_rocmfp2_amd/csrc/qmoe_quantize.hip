// Weight quantizer (gfx950): fp32 matrices -> ROCmFPX blocks, with one int8
// codebook per matrix fitted on the device.
//
// Page citations:
//   [0731-Strix] lucebox.com, "Lucebox × Geometric: DeepSeek V4 Flash 0731
//     reaches 32.7 tok/s on AMD Strix Halo", section "How the model fits on AMD
//     Strix Halo": the expert weights carry learned codebooks, one per expert.
//   [Strix-284B] lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
//     AMD Ryzen AI MAX+ 395", section "ROCmFPX: fitting 284B weights into 128
//     GB": 32-weight blocks of codes plus a small scale.
// The pages print no fitting procedure. This library's reading: an absmax scale
// per block, Lloyd's algorithm (1-D k-means) on the scale-normalized weights of
// one matrix in integer units of 1/256, then the nearest codebook entry of each
// weight; every step after the normalization is integer arithmetic, so the
// codebook does not depend on the order of any reduction.
//
//   k_qz_norm    8 lanes per block, 4 weights per lane (16-byte loads): amax
//                by DPP exchanges, the block's stored scale and divisor, the
//                int16 normalized values v; workgroup 0 also writes the
//                starting centroids.
//   k_qz_assign  one Lloyd assignment pass: G workgroups per matrix stream its
//                v, each lane keeps per-entry sums and counts in LDS slots of
//                its own (no contention; with 4 or 8 sorted entries, in registers
//                as sums above each threshold, from packed int16 arithmetic),
//                and each workgroup writes its integer partial sums; no
//                global atomics.
//   k_qz_update  one workgroup per matrix: adds the G partials of each entry
//                (exact integers) and moves the centroid to the mean rounded
//                half up (floor division); an entry with no members keeps its
//                value.
//   k_qz_pack    one thread per block: the int8 codebook from the centroids,
//                the nearest entry of each weight, packed into the row-planar
//                layout with the block's scale; the first block of each matrix
//                also writes the codebook.
#include <hip/hip_runtime.h>

#include "qmoe_device.h"
#include "qmoe_host.h"
#include "qmoe_internal.h"

using namespace qk;
using namespace qmoe;

namespace {

constexpr int kQzMaxEntries = 16;   // 2^bits, bits <= 4
constexpr int kQzGroups = 256;      // assignment workgroups per matrix
constexpr int kQzMaxIters = 64;

// Workspace regions (256-byte aligned).
struct QzWs {
  int16_t* v;          // [n][rows][k] normalized values
  uint16_t* sc;        // [n][rows][k/32] stored scales (fp16 bits or E8M0)
  long long* c;        // [n][16] centroids, units of 1/256
  long long* part;     // [n][G][16][2] partial sums and counts
};

inline size_t qz_align(size_t v) { return (v + 255) / 256 * 256; }

size_t qz_layout(int32_t n, int64_t rows, int64_t k, QzWs* w, uint8_t* base) {
  const size_t nw = (size_t)n * rows * k, nb = nw / 32;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = qz_align(off + bytes);
    return base ? base + at : nullptr;
  };
  uint8_t* pv = take(nw * 2);
  uint8_t* ps = take(nb * 2);
  uint8_t* pc = take((size_t)n * kQzMaxEntries * 8);
  uint8_t* pp = take((size_t)n * kQzGroups * kQzMaxEntries * 2 * 8);
  if (w) {
    w->v = reinterpret_cast<int16_t*>(pv);
    w->sc = reinterpret_cast<uint16_t*>(ps);
    w->c = reinterpret_cast<long long*>(pc);
    w->part = reinterpret_cast<long long*>(pp);
  }
  return off;
}

// Least k with 2^k >= t for a positive finite fp32 t, from its bits.
__device__ __forceinline__ int ceil_log2_f32(float t) {
  const uint32_t b = __float_as_uint(t);
  const uint32_t ex = (b >> 23) & 0xFFu, man = b & 0x7FFFFFu;
  if (ex == 0) return (man <= 1u ? 0 : 32 - __clz(man - 1u)) - 149;   // t = man * 2^-149
  return (int)ex - 127 + (man ? 1 : 0);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Q1, Q2: thread g handles weights 4g..4g+3 of the flattened [n][rows][k]
// (one 16-byte load); the 8 lanes of each aligned group of 8 hold one block.
// All lanes take part in the exchanges.
template <int FMT>
__global__ __launch_bounds__(256) void k_qz_norm(const float* __restrict__ w, size_t nw, int n, int16_t* __restrict__ v,
                                                 uint16_t* __restrict__ sc, long long* __restrict__ c) {
#pragma clang fp contract(off)
  const size_t g = (size_t)blockIdx.x * 256 + threadIdx.x;
  const bool ok = 4 * g < nw;
  const f32x4 x = ok ? reinterpret_cast<const f32x4*>(w)[g] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
  m = fmaxf(m, xchg32<1>(m));
  m = fmaxf(m, xchg32<2>(m));
  m = fmaxf(m, xchg32<4>(m));
  const float t = m / 127.0f;
  uint32_t stored;
  float d;
  if constexpr (FMT == 4) {
    const int e = (t > 0.0f) ? min(max(127 + ceil_log2_f32(t), 1), 254) : 0;
    stored = (uint32_t)e;
    d = __uint_as_float((uint32_t)max(e, 1) << 23);   // 2^(e - 127), a normal fp32
  } else {
    stored = (t >= 65520.0f) ? 0x7BFFu : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)t);
    d = half_bits_to_float(stored);
  }
  const bool live = m > 0.0f && d > 0.0f;
  const float xs[4] = {x.x, x.y, x.z, x.w};
  uint32_t q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int qi = 0;
    if (live) qi = (int)fminf(fmaxf(rintf((xs[i] / d) * 256.0f), -32767.0f), 32767.0f);
    q[i] = (uint32_t)qi & 0xFFFFu;
  }
  if (ok) {
    reinterpret_cast<u32x2*>(v)[g] = u32x2{q[0] | (q[1] << 16), q[2] | (q[3] << 16)};
    if ((threadIdx.x & 7) == 0) sc[g >> 3] = (uint16_t)stored;
  }
  if (blockIdx.x == 0 && threadIdx.x < n * kQzMaxEntries && threadIdx.x < 256) {
    // starting centroids: midpoints of 2^bits equal cells over [-127, 127]
    const int i = threadIdx.x % kQzMaxEntries;
    constexpr int NC = 1 << FMT;
    c[threadIdx.x] = (i < NC) ? (long long)(32512 * (2 * i + 1) / NC - 32512) : 0;
  }
}

// For n > 16 matrices the starting centroids of the rest are written here.
__global__ __launch_bounds__(256) void k_qz_init(long long* __restrict__ c, int n, int nc) {
  const int g = blockIdx.x * 256 + threadIdx.x;
  if (g < n * kQzMaxEntries) {
    const int i = g % kQzMaxEntries;
    c[g] = (i < nc) ? (long long)(32512 * (2 * i + 1) / nc - 32512) : 0;
  }
}

// Index of the nearest of NC centroids (ties to the lower index).
template <int NC>
__device__ __forceinline__ int qz_nearest(int x, const int (&cc)[NC]) {
  int best = 0, bd = abs(x - cc[0]);
#pragma unroll
  for (int i = 1; i < NC; ++i) {
    const int di = abs(x - cc[i]);
    if (di < bd) {
      bd = di;
      best = i;
    }
  }
  return best;
}

// Nearest of NC strictly increasing centroids, from their pairwise sums
// mid[i] = c_i + c_{i+1}: c_{i+1} is strictly nearer than c_i exactly when
// 2x > mid[i], and the mids increase, so the indicators read 1..1 0..0 and their
// count is the lowest index of the nearest centroid (ties stay low), the same
// as qz_nearest.
template <int NC>
__device__ __forceinline__ int qz_nearest_sorted(int x, const int (&mid)[NC - 1]) {
  int a = 0;
#pragma unroll
  for (int i = 0; i < NC - 1; ++i) a += (2 * x > mid[i]) ? 1 : 0;
  return a;
}

template <int NC, bool SORTED>
__device__ __forceinline__ void qz_assign_loop(const u32x4* __restrict__ src, size_t npieces, size_t first,
                                               size_t stride, const int (&cc)[NC], const int (&mid)[NC - 1],
                                               int (&s_sum)[NC][256], int (&s_cnt)[NC][256]) {
  const int tid = threadIdx.x;
  for (size_t p = first; p < npieces; p += stride) {
    const u32x4 r = src[p];
    const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const int x = (int)(int16_t)(wd[h >> 1] >> (16 * (h & 1)));
      const int a = SORTED ? qz_nearest_sorted<NC>(x, mid) : qz_nearest<NC>(x, cc);
      // LDS adds without a returned value: no read-modify-write chain between
      // the values (the slots are this thread's own, in distinct banks per lane)
      atomicAdd(&s_sum[a][tid], x);
      atomicAdd(&s_cnt[a][tid], 1);
    }
  }
}

typedef short qz_i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short qz_u16x2 __attribute__((ext_vector_type(2)));

// The sorted rule without per-value slots: a value x goes above threshold i
// (entry index > i) exactly when 2x > mid[i], i.e. x > h[i] = floor(mid[i] / 2)
// for integer x. Per pair of int16 values (one dword) and threshold: the
// saturating packed difference h - x is negative exactly when x > h, so its
// sign bit is the 0/1 indicator of each half; two integer dot products add the
// indicated values and the indicators. The thread ends with, per threshold,
// the sum and count of its values above it, plus the sum of all its values;
// the per-entry sums and counts are the differences of consecutive ones (exact
// integer arithmetic, the same totals as one slot per entry).
template <int NC>
__device__ __forceinline__ void qz_assign_sorted_pairs(const u32x4* __restrict__ src, size_t npieces, size_t first,
                                                       size_t stride, const int (&mid)[NC - 1],
                                                       int (&s_sum)[NC][256], int (&s_cnt)[NC][256]) {
  const int tid = threadIdx.x;
  qz_i16x2 h[NC - 1];
#pragma unroll
  for (int i = 0; i < NC - 1; ++i) {
    const short hi = (short)(mid[i] >> 1);   // floor division by 2; |mid| <= 65534
    h[i] = qz_i16x2{hi, hi};
  }
  const qz_i16x2 one = {1, 1};
  int above_sum[NC - 1], above_cnt[NC - 1], total = 0, n = 0;
#pragma unroll
  for (int i = 0; i < NC - 1; ++i) above_sum[i] = above_cnt[i] = 0;
  // four pieces in flight per lane: every load is issued (index clamped into
  // range) before any is used; pieces past the end are loaded but not counted
  constexpr int PF = 4;
  for (size_t p0 = first; p0 < npieces; p0 += PF * stride) {
    u32x4 r[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) r[k] = src[min(p0 + k * stride, npieces - 1)];
    // an empty asm that takes every loaded piece keeps the compiler from sinking
    // the later loads into the branches that use them (one round trip each)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"v"(r[0]), "v"(r[1]), "v"(r[2]), "v"(r[3]));
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      if (p0 + k * stride >= npieces) break;
      const uint32_t wd[4] = {r[k].x, r[k].y, r[k].z, r[k].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const qz_i16x2 x = __builtin_bit_cast(qz_i16x2, wd[d]);
        total = __builtin_amdgcn_sdot2(x, one, total, false);
#pragma unroll
        for (int i = 0; i < NC - 1; ++i) {
          const qz_i16x2 nd = __builtin_elementwise_sub_sat(h[i], x);
          const qz_u16x2 ind = __builtin_bit_cast(qz_u16x2, nd) >> (qz_u16x2){15, 15};
          above_sum[i] = __builtin_amdgcn_sdot2(x, __builtin_bit_cast(qz_i16x2, ind), above_sum[i], false);
          above_cnt[i] = __builtin_amdgcn_sdot2(__builtin_bit_cast(qz_i16x2, ind), one, above_cnt[i], false);
        }
      }
      n += 8;
    }
  }
  s_sum[0][tid] = total - above_sum[0];
  s_cnt[0][tid] = n - above_cnt[0];
#pragma unroll
  for (int i = 1; i < NC - 1; ++i) {
    s_sum[i][tid] = above_sum[i - 1] - above_sum[i];
    s_cnt[i][tid] = above_cnt[i - 1] - above_cnt[i];
  }
  s_sum[NC - 1][tid] = above_sum[NC - 2];
  s_cnt[NC - 1][tid] = above_cnt[NC - 2];
}

// Q3, assignment: grid (G, n). Lane slots s_sum/s_cnt[entry][thread] hold this
// thread's sums (at most 8 * 32767 per piece, so int32 is exact per slot up to
// 2^31 / 32767 = 65538 values per thread) and counts. Lloyd's iterations keep
// the centroids in order; the pairwise-sum shortcut is taken when they are
// strictly increasing (checked per workgroup), the full scan otherwise.
template <int NC>
__global__ __launch_bounds__(256) void k_qz_assign(const int16_t* __restrict__ v, size_t per_mat,
                                                   const long long* __restrict__ c, long long* __restrict__ part) {
  __shared__ int s_sum[NC][256];
  __shared__ int s_cnt[NC][256];
  const int tid = threadIdx.x, m = blockIdx.y, G = gridDim.x;
  int cc[NC], mid[NC - 1];
  bool inc = true;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    cc[i] = (int)c[(size_t)m * kQzMaxEntries + i];
    s_sum[i][tid] = 0;
    s_cnt[i][tid] = 0;
  }
#pragma unroll
  for (int i = 0; i < NC - 1; ++i) {
    mid[i] = cc[i] + cc[i + 1];
    inc = inc && cc[i] < cc[i + 1];
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(v + (size_t)m * per_mat);
  const size_t npieces = per_mat / 8;   // 8 values per 16-byte piece
  const size_t first = (size_t)blockIdx.x * 256 + tid, stride = (size_t)G * 256;
  if (inc && NC <= 8)
    qz_assign_sorted_pairs<NC>(src, npieces, first, stride, mid, s_sum, s_cnt);
  else if (inc)
    qz_assign_loop<NC, true>(src, npieces, first, stride, cc, mid, s_sum, s_cnt);
  else
    qz_assign_loop<NC, false>(src, npieces, first, stride, cc, mid, s_sum, s_cnt);
  __syncthreads();
  // per entry: the workgroup's sum and count, then its partial slot
  if (tid < NC) {
    long long S = 0, N = 0;
    for (int j = 0; j < 256; ++j) {
      S += s_sum[tid][j];
      N += s_cnt[tid][j];
    }
    long long* dst = part + (((size_t)m * kQzGroups + blockIdx.x) * kQzMaxEntries + tid) * 2;
    dst[0] = S;
    dst[1] = N;
  }
}

// Q3, update: one workgroup per matrix; 16 threads per entry each add every
// 16th partial (all loads in flight at once), then one thread per entry adds
// the 16 sub-sums in order.
__global__ __launch_bounds__(256) void k_qz_update(long long* __restrict__ c, const long long* __restrict__ part, int G,
                                                   int nc) {
  __shared__ long long sS[kQzMaxEntries][16], sN[kQzMaxEntries][16];
  const int m = blockIdx.x, i = threadIdx.x >> 4, j = threadIdx.x & 15;
  long long S = 0, N = 0;
  if (i < nc) {
#pragma unroll 16
    for (int g = j; g < G; g += 16) {
      const long long* p = part + (((size_t)m * kQzGroups + g) * kQzMaxEntries + i) * 2;
      S += p[0];
      N += p[1];
    }
  }
  sS[i][j] = S;
  sN[i][j] = N;
  __syncthreads();
  if (j == 0 && i < nc) {
    S = 0;
    N = 0;
    for (int r = 0; r < 16; ++r) {
      S += sS[i][r];
      N += sN[i][r];
    }
    if (N > 0) {
      const long long num = 2 * S + N, den = 2 * N;
      long long q = num / den;                       // truncates toward zero
      if (num % den != 0 && num < 0) q -= 1;          // floor
      c[(size_t)m * kQzMaxEntries + i] = q;
    }
  }
}

// Q4..Q6: one thread per block of 32 weights.
template <int FMT>
__global__ __launch_bounds__(256) void k_qz_pack(const int16_t* __restrict__ v, const uint16_t* __restrict__ sc,
                                                 const long long* __restrict__ c, uint8_t* __restrict__ out,
                                                 int8_t* __restrict__ cb, int rows, int nb, size_t row_bytes,
                                                 size_t nblocks) {
  constexpr int NC = 1 << FMT;
  const size_t blk = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= nblocks) return;
  const size_t per_mat = (size_t)rows * nb;
  const int m = (int)(blk / per_mat);
  const size_t rb = blk - (size_t)m * per_mat;
  const int r = (int)(rb / nb), b = (int)(rb - (size_t)r * nb);
  int C[NC], cc[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const long long ci = c[(size_t)m * kQzMaxEntries + i];
    C[i] = (int)min(max((ci + 128) >> 8, -127LL), 127LL);   // arithmetic shift = floor division by 256
    cc[i] = 256 * C[i];
  }
  if (rb == 0) {
#pragma unroll
    for (int i = 0; i < NC; ++i) cb[(size_t)m * NC + i] = (int8_t)C[i];
  }
  // with strictly increasing int8 entries the nearest one is the count of
  // pairwise sums below 2x (qz_nearest_sorted, the same index as the scan);
  // entries that rounded to equal values take the full scan (ties go low)
  int mid[NC - 1];
  bool inc = true;
#pragma unroll
  for (int i = 0; i < NC - 1; ++i) {
    mid[i] = cc[i] + cc[i + 1];
    inc = inc && cc[i] < cc[i + 1];
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(v + blk * 32);
  u32x4 pc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) pc[q] = src[q];
  uint32_t code[32];
  if (inc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wd[4] = {pc[q].x, pc[q].y, pc[q].z, pc[q].w};
#pragma unroll
      for (int h = 0; h < 8; ++h)
        code[8 * q + h] = (uint32_t)qz_nearest_sorted<NC>((int)(int16_t)(wd[h >> 1] >> (16 * (h & 1))), mid);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t wd[4] = {pc[q].x, pc[q].y, pc[q].z, pc[q].w};
#pragma unroll
      for (int h = 0; h < 8; ++h)
        code[8 * q + h] = (uint32_t)qz_nearest<NC>((int)(int16_t)(wd[h >> 1] >> (16 * (h & 1))), cc);
    }
  }
  uint8_t* row = out + (size_t)m * rows * row_bytes + (size_t)r * row_bytes;
  if constexpr (FMT == 2 || FMT == 3) {
    // 2-bit plane: code j (low two bits) at byte 4(j >> 4) + (j & 3), bit 2((j >> 2) & 3)
    uint32_t lo[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) lo[j >> 4] |= (code[j] & 3u) << (8 * (j & 3) + 2 * ((j >> 2) & 3));
    *reinterpret_cast<u32x2*>(row + (size_t)b * 8) = u32x2{lo[0], lo[1]};
    size_t after = (size_t)nb * 8;
    if constexpr (FMT == 3) {
      // bit 2 of code j at byte (j & 3), bit (j >> 2) of the 4-byte plane
      uint32_t hi = 0u;
#pragma unroll
      for (int j = 0; j < 32; ++j) hi |= ((code[j] >> 2) & 1u) << (8 * (j & 3) + (j >> 2));
      *reinterpret_cast<uint32_t*>(row + after + (size_t)b * 4) = hi;
      after += (size_t)nb * 4;
    }
    *reinterpret_cast<uint16_t*>(row + after + (size_t)b * 2) = sc[blk];
  } else {
    // nibble plane: code j at byte 4(j >> 3) + (j & 3), bit 4((j >> 2) & 1)
    uint32_t lo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) lo[j >> 3] |= code[j] << (8 * (j & 3) + 4 * ((j >> 2) & 1));
    *reinterpret_cast<u32x4*>(row + (size_t)b * 16) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    row[(size_t)nb * 16 + b] = (uint8_t)sc[blk];
  }
}

template <int FMT>
int launch_quantize(int32_t n, int64_t rows, int64_t k, const float* w, int32_t iters, uint8_t* out, int8_t* cb,
                    const QzWs& ws, hipStream_t s) {
  constexpr int NC = 1 << FMT;
  const size_t nw = (size_t)n * rows * k, nb_total = nw / 32;
  launch_kernel("qz_norm", k_qz_norm<FMT>, dim3((unsigned)((nw / 4 + 255) / 256)), dim3(256), s, w, nw, n, ws.v,
                ws.sc, ws.c);
  if (n * kQzMaxEntries > 256)
    launch_kernel("qz_init", k_qz_init, dim3((unsigned)((n * kQzMaxEntries + 255) / 256)), dim3(256), s, ws.c, n, NC);
  int st = launch_check("qz_norm");
  if (st) return st;
  const size_t per_mat = (size_t)rows * k;
  for (int it = 0; it < iters; ++it) {
    launch_kernel("qz_assign", k_qz_assign<NC>, dim3(kQzGroups, n), dim3(256), s, (const int16_t*)ws.v, per_mat,
                  (const long long*)ws.c, ws.part);
    launch_kernel("qz_update", k_qz_update, dim3(n), dim3(256), s, ws.c, (const long long*)ws.part, kQzGroups, NC);
    if ((st = launch_check("qz_lloyd"))) return st;
  }
  const size_t row_bytes = (size_t)(k / 32) * (FMT == 2 ? 10 : FMT == 3 ? 14 : 17);
  launch_kernel("qz_pack", k_qz_pack<FMT>, dim3((unsigned)((nb_total + 255) / 256)), dim3(256), s,
                (const int16_t*)ws.v, (const uint16_t*)ws.sc, (const long long*)ws.c, out, cb, (int)rows,
                (int)(k / 32), row_bytes, nb_total);
  return launch_check("qz_pack");
}

}  // namespace

extern "C" size_t qmoe_quantize_workspace_bytes(int32_t n, int64_t rows, int64_t k) {
  if (n < 1 || rows < 1 || k < 32 || k % 32) return 0;
  return qz_layout(n, rows, k, nullptr, nullptr);
}

extern "C" int qmoe_quantize(qmoe_format f, int32_t n, int64_t rows, int64_t k, const float* w, int32_t iters,
                             void* out, size_t out_bytes, int8_t* cb, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  FormatInfo fi;
  if (!format_info(f, &fi)) QMOE_FAIL(QMOE_E_FORMAT, "quantize: unknown format %d", (int)f);
  if (n < 1 || rows < 1 || k < 32) QMOE_FAIL(QMOE_E_SHAPE, "quantize: n=%d rows=%lld k=%lld must be positive (k >= 32)",
                                             n, (long long)rows, (long long)k);
  if (k % 32) QMOE_FAIL(QMOE_E_SHAPE, "quantize: k=%lld not a multiple of 32", (long long)k);
  const size_t row_bytes = (size_t)(k / 32) * fi.block_bytes;
  if (row_bytes % 16)
    QMOE_FAIL(QMOE_E_SHAPE, "quantize: row of %zu bytes is not a multiple of 16 (k must be a multiple of %d)", row_bytes,
              f == QMOE_FP4 ? 512 : 256);
  const size_t nw = (size_t)n * rows * k;
  if (nw > ((size_t)1 << 34)) QMOE_FAIL(QMOE_E_SHAPE, "quantize: %zu weights exceed 2^34", nw);
  if (n > 65535) QMOE_FAIL(QMOE_E_SHAPE, "quantize: n=%d matrices exceed 65535 (one grid row each)", n);
  if (iters < 0 || iters > kQzMaxIters) QMOE_FAIL(QMOE_E_SHAPE, "quantize: iters=%d outside 0..%d", iters, kQzMaxIters);
  if (!w || !out || !cb || !ws) QMOE_FAIL(QMOE_E_INVAL, "quantize: NULL pointer");
  if (!aligned16(w) || !aligned16(out)) QMOE_FAIL(QMOE_E_INVAL, "quantize: w and out must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(ws) % 256) QMOE_FAIL(QMOE_E_WORKSPACE, "quantize: workspace not 256-byte aligned");
  if (out_bytes < (size_t)n * rows * row_bytes)
    QMOE_FAIL(QMOE_E_SIZE, "quantize: out holds %zu bytes < %zu required", out_bytes, (size_t)n * rows * row_bytes);
  const size_t need = qz_layout(n, rows, k, nullptr, nullptr);
  if (ws_bytes < need) QMOE_FAIL(QMOE_E_WORKSPACE, "quantize: workspace of %zu bytes < %zu required", ws_bytes, need);
  // per-thread LDS slots of the assignment pass hold int32 sums of at most
  // ceil(pieces / (G * 256)) * 8 values of magnitude <= 32767
  const size_t per_thread = ((size_t)rows * k / 8 + (size_t)kQzGroups * 256 - 1) / ((size_t)kQzGroups * 256) * 8;
  if (per_thread > 65536) QMOE_FAIL(QMOE_E_SHAPE, "quantize: %lld x %lld matrices exceed the per-pass limit",
                                    (long long)rows, (long long)k);
  QzWs p;
  qz_layout(n, rows, k, &p, static_cast<uint8_t*>(ws));
  hipStream_t s = as_stream(stream);
  uint8_t* o = static_cast<uint8_t*>(out);
  switch (f) {
    case QMOE_FP2: return launch_quantize<2>(n, rows, k, w, iters, o, cb, p, s);
    case QMOE_FP3: return launch_quantize<3>(n, rows, k, w, iters, o, cb, p, s);
    default: return launch_quantize<4>(n, rows, k, w, iters, o, cb, p, s);
  }
}
