// Device building blocks for ROCmFPX block-quantized kernels on gfx950 (wave64).
//
// Page citations:
//   [Strix-284B] lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
//   AMD Ryzen AI MAX+ 395", section "ROCmFPX: fitting 284B weights into 128 GB":
//   32-weight blocks of low-bit codes and a small scale, read directly from
//   memory; the small codebook is expanded in registers with byte-permute
//   instructions and fed to integer dot products without a separate gather.
//   [evox3] soothill.io, "DeepSeek V4 Flash 0731 on evox3", table "The
//   optimization ladder": H32 rotation of the expert input, shared across experts.
//
// Layout facts used here (the library's format, also stated in include/qmoe.h):
//   - 2-bit plane word m of a block: (W_m >> 2k) & 0x03030303 = selectors of
//     weights 16m+4k+0..3, i.e. of activation dword 4m+k.
//   - FP3 bit-2 plane word H: (H >> g) & 0x01010101 = bit 2 of weights 4g+0..3.
//   - FP4 nibble word w: (W_w >> 4h) & 0x0F0F0F0F = codes of weights 8w+4h+0..3,
//     i.e. of activation dword 2w+h.
//   - Row-planar rows: code planes of all blocks, FP3 high planes, scales.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

constexpr int kWave = 64;

// Native vector types for wide loads: unlike HIP's uint4 / uint2 classes they stay
// in registers when held across loops and barriers.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  // v_perm_b32: result byte i = byte sel_i of the 8-byte value {hi, lo} (lo = bytes 0..3)
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);   // int8 x int8, int32 accumulate
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// E8M0: 2^(e-127). e >= 1 is a normal fp32 with exponent field e; e = 0 is the
// subnormal 2^-127 (mantissa bit 22).
__device__ __forceinline__ float e8m0_to_float(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00200000u);
}

template <int FMT> struct Fmt;
template <> struct Fmt<2> { static constexpr int kLoWords = 2, kHi = 0, kScaleBytes = 2, kBlockBytes = 10, kCbWords = 1; };
template <> struct Fmt<3> { static constexpr int kLoWords = 2, kHi = 1, kScaleBytes = 2, kBlockBytes = 14, kCbWords = 2; };
template <> struct Fmt<4> { static constexpr int kLoWords = 4, kHi = 0, kScaleBytes = 1, kBlockBytes = 17, kCbWords = 4; };

// Codebook of 2^bits int8 entries held as 1, 2 or 4 dwords.
template <int FMT>
__device__ __forceinline__ void load_codebook(const int8_t* cb, uint32_t w[4]) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(cb);
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (i < Fmt<FMT>::kCbWords) ? p[i] : 0u;
}

// NBL consecutive blocks of one row, starting at block b (row-planar layout).
// load() only issues the loads (raw scale bits are kept), so that a caller can
// put the loads of many rows in flight before touching any of them.
template <int FMT, int NBL>
struct Blocks {
  uint32_t lo[NBL][Fmt<FMT>::kLoWords];
  uint32_t hi[NBL];
  uint32_t sraw;   // NBL fp16 scales (2 bytes each) or NBL E8M0 bytes

  __device__ __forceinline__ void load(const uint8_t* row, int nb, int b) {
    constexpr int LW = Fmt<FMT>::kLoWords;
    const uint8_t* codes = row + (size_t)b * LW * 4;
    if constexpr (LW * NBL == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(codes);
      uint32_t t[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < NBL; ++i)
#pragma unroll
        for (int w = 0; w < LW; ++w) lo[i][w] = t[i * LW + w];
    } else if constexpr (LW * NBL == 2) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(codes);
      lo[0][0] = v.x;
      lo[0][1] = v.y;
    } else {  // FP4, NBL = 2: 32 bytes
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(codes);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(codes + 16);
      lo[0][0] = v0.x; lo[0][1] = v0.y; lo[0][2] = v0.z; lo[0][3] = v0.w;
      lo[NBL - 1][0] = v1.x; lo[NBL - 1][1] = v1.y; lo[NBL - 1][2] = v1.z; lo[NBL - 1][3] = v1.w;
    }
    const uint8_t* after_lo = row + (size_t)nb * LW * 4;
    if constexpr (Fmt<FMT>::kHi) {
      if constexpr (NBL == 2) {
        const u32x2 h = *reinterpret_cast<const u32x2*>(after_lo + (size_t)b * 4);
        hi[0] = h.x;
        hi[NBL - 1] = h.y;
      } else {
        hi[0] = *reinterpret_cast<const uint32_t*>(after_lo + (size_t)b * 4);
      }
    }
    const uint8_t* sc = after_lo + (size_t)nb * 4 * Fmt<FMT>::kHi;
    if constexpr (Fmt<FMT>::kScaleBytes == 2) {
      if constexpr (NBL == 2)
        sraw = *reinterpret_cast<const uint32_t*>(sc + (size_t)b * 2);
      else
        sraw = *reinterpret_cast<const uint16_t*>(sc + (size_t)b * 2);
    } else {
      if constexpr (NBL == 2)
        sraw = *reinterpret_cast<const uint16_t*>(sc + b);
      else
        sraw = sc[b];
    }
  }

  __device__ __forceinline__ float scale(int i) const {
    if constexpr (Fmt<FMT>::kScaleBytes == 2)
      return half_bits_to_float((sraw >> (16 * i)) & 0xFFFFu);
    else
      return e8m0_to_float((sraw >> (8 * i)) & 0xFFu);
  }

  // Expand block i into 8 dwords of int8 weights; out[g] covers weights 4g..4g+3.
  __device__ __forceinline__ void expand(int i, const uint32_t cb[4], uint32_t out[8]) const {
    if constexpr (FMT == 2) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int k = 0; k < 4; ++k) out[4 * m + k] = perm(cb[0], cb[0], (lo[i][m] >> (2 * k)) & 0x03030303u);
    } else if constexpr (FMT == 3) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int g = 4 * m + k;
          const uint32_t sel = ((lo[i][m] >> (2 * k)) & 0x03030303u) | (((hi[i] >> g) & 0x01010101u) << 2);
          out[g] = perm(cb[1], cb[0], sel);
        }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t sel = (lo[i][w] >> (4 * h)) & 0x0F0F0F0Fu;
          const uint32_t s7 = sel & 0x07070707u;
          const uint32_t a = perm(cb[1], cb[0], s7);           // entries 0..7
          const uint32_t c = perm(cb[3], cb[2], s7);           // entries 8..15
          const uint32_t m = ((sel >> 3) & 0x01010101u) * 0xFFu;
          out[2 * w + h] = (c & m) | (a & ~m);
        }
    }
  }
};

// int8 activations of NBL consecutive blocks.
template <int NBL>
struct Acts {
  uint32_t q[NBL][8];
  float d[NBL];
  __device__ __forceinline__ void load(const int8_t* xq, const float* dx, int b) {
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
      const u32x4* p = reinterpret_cast<const u32x4*>(xq + (size_t)(b + i) * 32);
      const u32x4 a = p[0], c = p[1];
      q[i][0] = a.x; q[i][1] = a.y; q[i][2] = a.z; q[i][3] = a.w;
      q[i][4] = c.x; q[i][5] = c.y; q[i][6] = c.z; q[i][7] = c.w;
      d[i] = dx[b + i];
    }
  }
};

__device__ __forceinline__ int block_dot(const uint32_t w[8], const uint32_t x[8]) {
  int acc = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) acc = dot4(w[g], x[g], acc);
  return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over groups of `lpr` adjacent lanes (lpr a power of two <= 64); every lane
// of a group gets the group's sum. Exchanges inside 16-lane rows use DPP (lane
// ^ 1, lane ^ 2, then the half-row and row mirrors, which pair lanes whose
// partial sums are already uniform over the smaller group), the rest use
// ds_bpermute. The addition order is fixed, so results are deterministic.
__device__ __forceinline__ float group_sum(float v, int lpr) {
  if (lpr >= 2) v += dpp_f32<0xB1>(v);     // quad_perm [1,0,3,2]
  if (lpr >= 4) v += dpp_f32<0x4E>(v);     // quad_perm [2,3,0,1]
  if (lpr >= 8) v += dpp_f32<0x141>(v);    // row_half_mirror
  if (lpr >= 16) v += dpp_f32<0x140>(v);   // row_mirror
  if (lpr >= 32) v += __shfl_xor(v, 16);
  if (lpr >= 64) v += __shfl_xor(v, 32);
  return v;
}

// ---------------------------------------------------------------------------
// int8 quantization of one 32-element activation block, bit-exact with the
// CPU checker: optional H32 (butterflies h = 1,2,4,8,16, then * fp32 nearest
// 1/sqrt(32)), amax, d = amax/127 (a zero or subnormal d stores the block as
// d = 0, q = 0), id = 1/d, q = clamp(rint(v*id), -127, 127). IEEE binary32, no
// contraction.
__device__ __forceinline__ void quant_block32(float v[32], int rot, uint32_t q[8], float* d_out) {
#pragma clang fp contract(off)
  if (rot) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1)
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (!(j & h)) {
          const float a = v[j], b = v[j + h];
          v[j] = a + b;
          v[j + h] = a - b;
        }
    const float c = __uint_as_float(0x3E3504F3u);
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = v[j] * c;
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  // a zero or subnormal scale (1/d would overflow) stores the block as zero
  const float d0 = amax / 127.0f;
  const bool normal = d0 >= __uint_as_float(0x00800000u);   // 2^-126
  const float d = normal ? d0 : 0.0f;
  const float id = normal ? 1.0f / d0 : 0.0f;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float r = rintf(v[4 * g + i] * id);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      w |= ((uint32_t)(int)r & 0xFFu) << (8 * i);
    }
    q[g] = w;
  }
  *d_out = d;
}


// Exchange with lane ^ H inside each group of 32 lanes: DPP quad permutes for
// H = 1, 2, ds_swizzle in bitmask mode (and 0x1F, xor H) for H = 4, 8, 16.
template <int H>
__device__ __forceinline__ float xchg32(float v) {
  const int b = __float_as_int(v);
  int o;
  if constexpr (H == 1) o = __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, true);
  else if constexpr (H == 2) o = __builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, true);
  else o = __builtin_amdgcn_ds_swizzle(b, 0x1F | (H << 10));
  return __int_as_float(o);
}

template <int H>
__device__ __forceinline__ float fwht_step(float v, int j) {
#pragma clang fp contract(off)
  const float o = xchg32<H>(v);
  return (j & H) ? o - v : v + o;   // (a, b) -> (a + b, a - b), a the lower index
}

// The same quantization with the 32 values of a block spread over 32 lanes:
// lane j = lane & 31 of each half-wave holds value j (both halves may hold
// different blocks). The butterflies, the amax and the rounding are the same
// IEEE operations as in quant_block32, so both give identical bytes and scales.
// All 64 lanes must be active. Returns, in lanes with j % 4 == 0, the packed
// bytes j..j+3; *d_out is the block scale in every lane of the half.
__device__ __forceinline__ uint32_t quant_block32_lanes(float v, int rot, float* d_out) {
#pragma clang fp contract(off)
  const int j = (int)(threadIdx.x & 31);
  if (rot) {
    v = fwht_step<1>(v, j);
    v = fwht_step<2>(v, j);
    v = fwht_step<4>(v, j);
    v = fwht_step<8>(v, j);
    v = fwht_step<16>(v, j);
    v = v * __uint_as_float(0x3E3504F3u);
  }
  float m = fabsf(v);
  m = fmaxf(m, xchg32<1>(m));
  m = fmaxf(m, xchg32<2>(m));
  m = fmaxf(m, xchg32<4>(m));
  m = fmaxf(m, xchg32<8>(m));
  m = fmaxf(m, xchg32<16>(m));
  const float amax = fmaxf(0.0f, m);
  const float d0 = amax / 127.0f;
  const bool normal = d0 >= __uint_as_float(0x00800000u);   // 2^-126
  const float id = normal ? 1.0f / d0 : 0.0f;
  float r = rintf(v * id);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  const uint32_t b = (uint32_t)(int)r & 0xFFu;
  // gather bytes j..j+3 into lane j (j % 4 == 0): quad_perm [1,1,3,3], then [2,2,2,2]
  const uint32_t x1 = b | ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)b, 0xF5, 0xF, 0xF, true) << 8);
  const uint32_t x2 = x1 | ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)x1, 0xAA, 0xF, 0xF, true) << 16);
  *d_out = normal ? d0 : 0.0f;
  return x2;
}

// ---------------------------------------------------------------------------
// Router: one wave computes the fp64 logits of expert e for tokens t0..t0+TT-1.
// Lane l holds blocks l + 64c. Per block: sequential fp64 sum of the 32 exact
// products (fp16 x fp32 is exact in fp64, so fma == mul + add); then the
// stride-halving tree: in-lane stages (strides >= 64 blocks) followed by
// xor-butterfly stages m = 32..1 across lanes, each only when m < P2 (lane j +
// lane j^m equals s_j + s_{j+m} for j < m). Routing: 256 experts, 6 routed
// (lucebox.com, "Lucebox × Geometric: DeepSeek V4 Flash 0731 reaches 32.7
// tok/s on AMD Strix Halo", section "Run with Lucebox Engine").
constexpr int kRouterMaxC = 4;   // blocks per lane: hidden <= 32 * 64 * 4 = 8192

// Sequential fp64 sum of the 32 exact products of block b of expert e's fp16
// router row and the token x (0 for padding blocks b >= nb).
__device__ __forceinline__ double router_block_sum(const uint16_t* __restrict__ W, const float* __restrict__ x,
                                                   int H, int e, int b, int nb) {
  if (b >= nb) return 0.0;
  const u32x4* wp = reinterpret_cast<const u32x4*>(W + (size_t)e * H + (size_t)b * 32);
  const u32x4* xp = reinterpret_cast<const u32x4*>(x + (size_t)b * 32);
  u32x4 wr[4], xr[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) wr[i] = wp[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) xr[i] = xp[i];
  // the weights and all 32 activations arrive in one memory round trip before
  // the first product: the empty statement takes every loaded piece as an
  // input (left to itself the compiler sank the last pieces between the
  // products of this dependent chain, a second round trip on the router's
  // critical path)
  asm volatile("" ::"v"(wr[0]), "v"(wr[1]), "v"(wr[2]), "v"(wr[3]), "v"(xr[0]), "v"(xr[1]), "v"(xr[2]),
               "v"(xr[3]), "v"(xr[4]), "v"(xr[5]), "v"(xr[6]), "v"(xr[7]));
  uint32_t wv[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wv[4 * i] = wr[i].x; wv[4 * i + 1] = wr[i].y; wv[4 * i + 2] = wr[i].z; wv[4 * i + 3] = wr[i].w;
  }
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float xs[4] = {__uint_as_float(xr[i].x), __uint_as_float(xr[i].y), __uint_as_float(xr[i].z),
                         __uint_as_float(xr[i].w)};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = 4 * i + k;
      const uint32_t hb = (j & 1) ? (wv[j >> 1] >> 16) : (wv[j >> 1] & 0xFFFFu);
      acc = fma((double)half_bits_to_float(hb), (double)xs[k], acc);
    }
  }
  return acc;
}

// On return every lane holds the logits of tokens t0..t0+TT-1 in out[] (bias
// included; entries for tokens >= ntok are undefined).
template <int TT>
__device__ __forceinline__ void router_wave(const uint16_t* __restrict__ W, const float* __restrict__ x, int ntok,
                                            int H, const double* __restrict__ bias, int e, int t0, int lane,
                                            double out[TT]) {
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
      const u32x4* wp = reinterpret_cast<const u32x4*>(W + (size_t)e * H + (size_t)b * 32);
      uint32_t wv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 u = wp[i];
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
    out[t] = bias ? v + bias[e] : v;
  }
}

// ---------------------------------------------------------------------------
// Top-k of one token's E logits (one wave, K <= 8, E <= 512). Equal logits go
// to the lower id. Logits are compared as order-preserving 64-bit keys (-0.0
// folded into +0.0 so that equal values tie). Each lane sorts its keys once; a
// selection round reduces only the 32-bit high words of the lanes' heads across
// the wave (DPP exchanges inside 16-lane rows, then row broadcasts); the low
// words and ids are compared only when several heads share the largest high
// word.

__device__ __forceinline__ uint64_t f64_order_key(double v) {
  if (v == 0.0) v = 0.0;   // -0.0 -> +0.0
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ double f64_from_order_key(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k ^ 0x8000000000000000ull) : ~k;
  return __longlong_as_double((long long)b);
}

// Wave-wide maximum of a uint32 (uniform result): four DPP exchanges give every
// lane its 16-lane row's maximum, then the four row maxima are combined.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, true));
  // row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2 and 3: the
  // last lane holds the wave's maximum (one readlane instead of four)
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(v, 63);
}

// Top-k of one row of E fp64 logits (E <= 512, K <= 8) by one wave; lane l holds
// logits l, l+64, ... as order keys and first sorts them (descending key, then
// ascending id: the oracle's pick order, ties to the lower id). Each of the K
// rounds then looks only at the lanes' heads: the largest high word among them;
// when exactly one head carries it, that head is the maximum. Otherwise the
// heads sharing the high word are compared on the low word, and among equal
// keys the lowest id wins. The winning lane advances to its next key. Lane
// k < K ends with the k-th pick: its id, its key and its rank among the picks in
// ascending id order (lanes >= K: id 0x7FFFFFFF, key 0, rank 8). Returns the key
// of the first pick, the largest logit. The row is read with plain loads: it
// must have been written by an earlier launch.
struct TopkPick {
  int id;
  uint64_t key;
  int rank;
};

// (key, id) ordered for picking: a before b when a.key > b.key, or the keys are
// equal and a.id < b.id.
__device__ __forceinline__ void topk_cas(uint64_t& ka, int& ia, uint64_t& kb, int& ib) {
  const bool swap = kb > ka || (kb == ka && ib < ia);
  const uint64_t k = swap ? kb : ka;
  const int i = swap ? ib : ia;
  kb = swap ? ka : kb;
  ib = swap ? ia : ib;
  ka = k;
  ia = i;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, v, 0xB1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, v, 0x4E, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, v, 0x141, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, v, 0x140, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(v, 63);
}

// NS = slots per lane (E <= 64 * NS); keys of ids >= E are 0 and never win.
template <int NS>
__device__ __forceinline__ uint64_t topk_select_ns(const double* __restrict__ row, int E, int K, int lane,
                                                   TopkPick& p) {
  uint64_t key[NS];
  int id[NS];
  // every slot's load is issued (index clamped) before any is used, and every
  // key is formed before the bound is applied by a select: one memory round
  // trip for the row (a load whose value is used only under e < E is sunk into
  // that branch and waits there on its own)
  double lg[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) lg[j] = row[min(lane + 64 * j, E - 1)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int e = lane + 64 * j;
    const uint64_t k = f64_order_key(lg[j]);
    key[j] = (e < E) ? k : 0ull;   // key 0: no candidate (no real logit maps to 0)
    id[j] = e;
  }
  // sort the lane's slots into pick order (odd-even transposition: NS rounds)
#pragma unroll
  for (int r = 0; r < NS; ++r)
#pragma unroll
    for (int j = r & 1; j + 1 < NS; j += 2) topk_cas(key[j], id[j], key[j + 1], id[j + 1]);
  p.id = 0x7FFFFFFF;
  p.key = 0;
  uint64_t first = 0;
  int ptr = 0;   // the lane's next unpicked slot (NS: none left)
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k >= K) break;
    uint64_t hk = 0;
    int hi_d = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (j == ptr) {
        hk = key[j];
        hi_d = id[j];
      }
    const uint32_t hh = (uint32_t)(hk >> 32), hl = (uint32_t)hk;
    const uint32_t gh = wave_max_u32(hh);
    const uint64_t b = __ballot(hh == gh);
    int L;
    uint32_t gl;
    if (__popcll(b) == 1) {   // one head carries the largest high word
      L = (int)__builtin_ctzll(b);
      gl = (uint32_t)__builtin_amdgcn_readlane(hl, L);
    } else {
      gl = wave_max_u32(hh == gh ? hl : 0u);
      const uint64_t b2 = __ballot(hh == gh && hl == gl);
      if (__popcll(b2) == 1) {
        L = (int)__builtin_ctzll(b2);
      } else {   // equal keys: the lowest id
        const uint32_t mid = wave_min_u32((hh == gh && hl == gl) ? (uint32_t)hi_d : 0xFFFFFFFFu);
        L = (int)__builtin_ctzll(__ballot((hh == gh && hl == gl) && (uint32_t)hi_d == mid));
      }
    }
    // the ballots above hold at least one lane by construction; the clamp keeps
    // an id that addresses expert tensors inside [0, E) regardless
    const int pick = min(max(__builtin_amdgcn_readlane(hi_d, L), 0), E - 1);
    const uint64_t gk = ((uint64_t)gh << 32) | gl;
    if (k == 0) first = gk;
    if (lane == k) {
      p.id = pick;
      p.key = gk;
    }
    if (lane == L) ++ptr;
  }
  // rank in ascending id order: the number of picks with a smaller id
  int r = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < K) r += (__builtin_amdgcn_readlane(p.id, j) < p.id) ? 1 : 0;
  p.rank = (lane < K) ? r : 8;
  return first;
}

__device__ __forceinline__ uint64_t topk_select(const double* __restrict__ row, int E, int K, int lane, TopkPick& p) {
  if (E <= 64) return topk_select_ns<1>(row, E, K, lane, p);
  if (E <= 256) return topk_select_ns<4>(row, E, K, lane, p);
  return topk_select_ns<8>(row, E, K, lane, p);
}

// Lane holding the pick of ascending-id rank r (wave-uniform r < K).
__device__ __forceinline__ int topk_lane_of_rank(const TopkPick& p, int r) {
  return (int)__builtin_ctzll(__ballot(p.rank == r));
}

// Routing weight of the pick held by lane k < K: softmax over the selected
// logits, shifted by their maximum (key `first`), summed in ascending id order,
// all in fp64 and rounded to fp32 once. Lanes >= K return 0.
__device__ __forceinline__ float topk_softmax(const TopkPick& p, uint64_t first, int K, int lane) {
  const double m = f64_from_order_key(first);
  const double ex = (lane < K) ? exp(f64_from_order_key(p.key) - m) : 0.0;
  const uint64_t exb = (uint64_t)__double_as_longlong(ex);
  double S = 0.0;
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < K) {
      const int l = topk_lane_of_rank(p, r);
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)exb, l);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(exb >> 32), l);
      S = S + __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    }
  return (lane < K) ? (float)(ex / S) : 0.0f;
}

}  // namespace qk
