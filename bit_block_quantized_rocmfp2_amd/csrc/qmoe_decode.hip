// Decode layer (gfx950): the top-k SwiGLU MoE layer for q = 1..4 tokens in three
// stream-ordered launches, with no host synchronisation.
//
// Page citations:
//   [Strix-284B] lucebox.com, "DeepSeek V4 Flash: 284B model, up to 32 tok/s on
//     AMD Ryzen AI MAX+ 395": section "ROCmFPX: fitting 284B weights into 128 GB"
//     (decode streams the active expert weights, so it is bound by memory
//     traffic; packed blocks are expanded in registers and fed to integer dot
//     products) and section "Decode: up to 32 tok/s" (q = 4 verification
//     columns; each packed weight is decoded once and applied to all columns;
//     dedicated top-k routing kernels).
//   [0731-Strix] lucebox.com, "Lucebox × Geometric: DeepSeek V4 Flash 0731
//     reaches 32.7 tok/s on AMD Strix Halo", section "Lucebox Engine integration
//     with Geometric" (a sync-free MoE decode path) and section "How the model
//     fits on AMD Strix Halo" (gate/up 2.5 bpw, down 3.5 bpw, per-expert
//     codebooks).
//
//   k_route    one workgroup per expert, two waves per token: fp64 logits;
//              further workgroups of the same launch quantize the tokens to
//              int8 blocks, alongside the logits.
//   k_gateup   the gate/up launch. Every workgroup first selects the top-k of
//              each token from the logits and builds the plan itself (the union
//              of the chosen experts in ascending id, a column mask and the
//              routing weights per expert), so no workgroup waits for another;
//              the first workgroup also writes the routing and the plan out.
//              Then the gate and up rows of its items (32 rows of one planned
//              expert) are streamed once, all loads of a wave issued before the
//              first use, each block expanded once for every column routed to
//              the expert; SwiGLU, then requantization of the 32-row block
//              (+ H32) for the down projection. One token: k_gateup1, one
//              workgroup per item. Several tokens: one workgroup per CU walks
//              the items (k_gateupq2 with the tokens' blocks in LDS when a row
//              fits one pass of the lanes, k_gateupq otherwise); k_gateupq2
//              splits the last round's items by columns and requests each next
//              item's weights before the current item's epilogue.
//   k_down     one workgroup per group of rows: the plan is read in one round
//              trip, the rows of every planned expert are loaded together, per
//              column contributions are accumulated per lane in ascending
//              expert id with the routing weights, and reduced once. k_down1
//              (one token) and k_downq (several) copy the routed activations
//              to LDS once per workgroup; k_down serves the other shapes.
//   k_gateupm, k_downm  the same layer with the expert products on the int8
//              matrix cores (v_mfma_i32_4x4x4_16b_i8, the tokens as its four
//              columns), behind qmoe_decode_layer_mfma.
// Kernel boundaries make each launch's results visible to the next across the
// 8 XCDs (separate L2 caches); no workgroup waits for another inside a launch.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "qmoe_device.h"
#include "qmoe_host.h"
#include "qmoe_internal.h"

using namespace qk;
using namespace qmoe;

namespace {

struct DecodeArgs {
  const uint16_t* w_router;
  const double* bias;
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  const int8_t* cb_gate;
  const int8_t* cb_up;
  const int8_t* cb_down;
  const float* x;
  float* out;
  int8_t* xq;
  float* dx;
  double* logits;
  int32_t* idx;
  float* gw;
  int32_t* plan;
  int8_t* hq;
  float* dh;
  size_t gu_row_bytes, gu_stride, dn_row_bytes, dn_stride;
  int hidden, inter, E, K, q, rot_gateup, rot_down;
  int nb_h, nb_i;
  int dn_lpr_log2;
  int quant_per_wg;
};

// ------------------------------------------------------------ k_route
// One workgroup per expert, two waves per token. The logit is the R6 tree over
// the row's blocks: lane l holds blocks l + 64c (c < C = P2 / 64), the in-lane
// levels add s[c] + s[c + n] for n = C/2 .. 1, then xor butterflies over the
// lanes. With C >= 2 the two waves of a token take c = h and h + 2 (h = wave
// parity): the in-lane level n = 2 stays in a lane, the level n = 1 (s[0] + s[1])
// is added across the waves through LDS in the same order, and wave h = 0 runs
// the butterflies. Each wave issues half the fp64 work of a one-wave router.
// With C = 1 (hidden <= 2048) the first wave does all of it.
template <int Q>
__global__ __launch_bounds__(128 * Q) void k_route(DecodeArgs a) {
  __shared__ double s_half[Q][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = w >> 1, h = w & 1;
  const int e = blockIdx.x;
  if (e >= a.E) {
    // workgroups past the experts quantize the tokens, quant_per_wg blocks
    // each, two per wave pass (one per half-wave), alongside the logits rather
    // than after them
    const int nblk = a.q * a.nb_h, qi = e - a.E;
    const int b_end = min((qi + 1) * a.quant_per_wg, nblk);
    for (int b0 = qi * a.quant_per_wg + 2 * w; b0 < b_end; b0 += 4 * Q) {
      const int b = b0 + (lane >> 5), j = lane & 31;
      const bool ok = b < b_end;
      const float v = ok ? a.x[(size_t)b * 32 + j] : 0.0f;
      float d;
      const uint32_t qw = quant_block32_lanes(v, a.rot_gateup, &d);
      if (ok) {
        if ((j & 3) == 0) reinterpret_cast<uint32_t*>(a.xq + (size_t)b * 32)[j >> 2] = qw;
        if (j == 0) a.dx[b] = d;
      }
    }
    return;
  }
  const int H = a.hidden, nb = a.nb_h;
  int P2 = 1;
  while (P2 < nb) P2 <<= 1;
  const int C = P2 > 64 ? P2 / 64 : 1;
  const float* xt = a.x + (size_t)t * H;
  if (C >= 2) {
    double v = router_block_sum(a.w_router, xt, H, e, lane + 64 * h, nb);
    if (C == 4) v = v + router_block_sum(a.w_router, xt, H, e, lane + 64 * (h + 2), nb);
    if (h == 1) s_half[t][lane] = v;
    __syncthreads();
    if (h == 0) {
      v = v + s_half[t][lane];
      for (int m = 32; m >= 1; m >>= 1) v = v + __shfl_xor(v, m);
      if (lane == 0) a.logits[(size_t)t * a.E + e] = a.bias ? v + a.bias[e] : v;
    }
  } else if (h == 0) {
    double lg[1];
    router_wave<1>(a.w_router, xt, 1, H, a.bias, e, 0, lane, lg);
    if (lane == 0) a.logits[(size_t)t * a.E + e] = lg[0];
  }
}

// ------------------------------------------------------------ top-k and plan (per workgroup)
struct PlanLds {
  uint32_t bits[4][16];   // per token: bitmap of its selected experts (E <= 512)
  int ids[4][8];          // plan writer only: selected ids of token t, ascending
  float w[4][8];          // plan writer only: their routing weights
  int e;                  // one token: the expert of this workgroup's plan slot
  int uid[kPlanMax];      // plan slot s -> its expert (the s-th distinct id, ascending)
  uint32_t umask[kPlanMax];  // its column mask
  int U;                  // plan size
};

// Workgroup barrier that orders LDS accesses only: this wave's LDS operations
// complete before it, and vector-memory loads in flight stay in flight across
// it. (__syncthreads also waits for those.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Every workgroup selects the experts itself. With one token wave 0 runs the
// top-k and passes the expert of slot u (the plan is the K ids ascending with
// column mask 1) to the other waves through LDS, and lists the plan in P.uid,
// P.umask, P.U. With q > 1 tokens, waves t < q
// select token t and set its experts in an LDS bitmap; after one barrier wave 0
// lists the union of the bitmaps in LDS: plan slot s holds the s-th set bit,
// i.e. the distinct ids in ascending order, and its column mask is that bit
// across the tokens (P.uid, P.umask, P.U, read by every item of the
// workgroup). Returns the expert of plan slot u (-1 if u is beyond the plan)
// and its column mask. `write` (one workgroup) also computes the routing
// weights and stores the routing (idx, gw) and the plan (size, ids, masks,
// weights per column).
struct NoListingWork {
  __device__ void operator()() const {}
};
template <int Q, typename ListingWork = NoListingWork>
__device__ __forceinline__ int topk_and_plan(const DecodeArgs& a, PlanLds& P, int u, bool write, uint32_t& mask,
                                             int* U_out = nullptr, ListingWork&& while_listing = ListingWork()) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  TopkPick p;
  if constexpr (Q == 1) {
    if (wave == 0) {
      const uint64_t first = topk_select(a.logits, a.E, a.K, lane, p);
      const int eu = (u < a.K) ? __builtin_amdgcn_readlane(p.id, topk_lane_of_rank(p, u)) : -1;
      if (lane == 0) {
        P.e = eu;
        P.U = a.K;
      }
      if (lane < a.K) {   // the plan list (slot = rank in ascending id), as for q > 1
        P.uid[p.rank] = p.id;
        P.umask[p.rank] = 1u;
      }
      if (write) {
        const float g = topk_softmax(p, first, a.K, lane);
        if (lane < a.K) {
          a.idx[p.rank] = p.id;
          a.gw[p.rank] = g;
          a.plan[kPlanIdOff + p.rank] = p.id;
          a.plan[kPlanMaskOff + p.rank] = 1;
          reinterpret_cast<float4*>(a.plan + kPlanWOff)[p.rank] = make_float4(g, 0.0f, 0.0f, 0.0f);
        }
        if (lane == 0) a.plan[0] = a.K;
      }
    }
    __syncthreads();
    mask = 1u;
    if (U_out) *U_out = a.K;
    return P.e;
  } else {
    // (the barriers order LDS only: other waves' loads stay in flight across them)
    if (tid < 64) (&P.bits[0][0])[tid] = 0u;
    lds_barrier();
    if (wave < a.q) {
      const uint64_t first = topk_select(a.logits + (size_t)wave * a.E, a.E, a.K, lane, p);
      if (lane < a.K) atomicOr(&P.bits[wave][p.id >> 5], 1u << (p.id & 31));
      if (write) {
        const float g = topk_softmax(p, first, a.K, lane);
        if (lane < a.K) {
          P.ids[wave][p.rank] = p.id;
          P.w[wave][p.rank] = g;
          a.idx[wave * a.K + p.rank] = p.id;
          a.gw[wave * a.K + p.rank] = g;
        }
      }
    }
    lds_barrier();
    // wave 0 lists the plan once for the workgroup: lane l holds bits
    // 8l .. 8l + 7 of every token's bitmap (E <= 512) and of their union; the
    // slot of its first expert is the number of set bits of the lanes below
    // (eight ballots), and it lists its experts in ascending id order, so slot
    // s holds the s-th distinct id and its column mask (the items then read
    // their slot from LDS)
    if (wave == 0) {
      const int wi = lane >> 2, sh = (lane & 3) * 8;
      uint32_t tb[Q];
      uint32_t ub = 0;
#pragma unroll
      for (int t = 0; t < Q; ++t) {
        tb[t] = (t < a.q) ? (P.bits[t][wi] >> sh) & 0xFFu : 0u;
        ub |= tb[t];
      }
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      int s = 0, Ucount = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint64_t bj = __ballot((ub >> j) & 1u);
        s += __popcll(bj & lt);
        Ucount += __popcll(bj);
      }
      for (uint32_t x = ub; x != 0u; x &= x - 1u, ++s) {
        const int j = (int)__builtin_ctz(x), es = 8 * lane + j;
        uint32_t ms = 0;
        float4 ws = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int t = 0; t < Q; ++t)
          if ((tb[t] >> j) & 1u) {
            ms |= 1u << t;
            if (write) {
              float wt = 0.0f;
#pragma unroll
              for (int k = 0; k < 8; ++k)
                if (k < a.K && P.ids[t][k] == es) wt = P.w[t][k];
              if (t == 0) ws.x = wt;
              if (t == 1) ws.y = wt;
              if (t == 2) ws.z = wt;
              if (t == 3) ws.w = wt;
            }
          }
        P.uid[s] = es;   // (s < Ucount <= q * K <= kPlanMax)
        P.umask[s] = ms;
        if (write) {
          a.plan[kPlanIdOff + s] = es;
          a.plan[kPlanMaskOff + s] = (int)ms;
          reinterpret_cast<float4*>(a.plan + kPlanWOff)[s] = ws;
        }
      }
      if (lane >= Ucount && lane < kPlanMax) {   // the unused slots
        P.uid[lane] = -1;
        P.umask[lane] = 0u;
        if (write) {
          a.plan[kPlanIdOff + lane] = -1;
          a.plan[kPlanMaskOff + lane] = 0;
          reinterpret_cast<float4*>(a.plan + kPlanWOff)[lane] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
      }
      if (lane == 0) {
        P.U = Ucount;
        if (write) a.plan[0] = Ucount;
      }
    } else {
      while_listing();   // the other waves' LDS work, ordered by the barrier below
    }
    lds_barrier();
    const int U = P.U;
    if (U_out) *U_out = U;
    const int e = (u < U) ? P.uid[u] : -1;
    mask = (u < U) ? P.umask[u] : 0u;
    return e;
  }
}

// ------------------------------------------------------------ wave sums of many values
// Value of lane l ^ M (all 64 lanes active): DPP quad permutes for M = 1, 2, a
// row rotation by 8 (lane ^ 8 inside a 16-lane row) for M = 8, ds_swizzle for
// M = 4 and 16, a permute across the halves for M = 32.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (M == 1 || M == 2) return xchg32<M>(v);
  else if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  else if constexpr (M == 4 || M == 16) return xchg32<M>(v);
  else return __shfl_xor(v, 32);
}

// One transposing step at stride M: lane l holds values a (lower) and b (upper)
// and returns a(l) + a(l ^ M) if lane & M is clear, b(l) + b(l ^ M) if it is set.
// For M = 32 and 16 this is one v_permlane32_swap / v_permlane16_swap, which
// exchanges the upper lanes (odd 16-lane rows) of its first operand with the
// lower lanes (even rows) of its second, so each lane then holds its own and
// its partner's copy of the half it keeps.
template <int M>
__device__ __forceinline__ float tstep(float a, float b, bool hi) {
  if constexpr (M == 32 || M == 16) {
    const auto r = (M == 32) ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                             : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const float keep = hi ? b : a, send = hi ? a : b;
    return keep + lane_xor<M>(send);
  }
}

// Sums N values per lane (N a power of two) over the wave by a transposing
// butterfly: at stride M = 32, 16, ... while a lane holds more than one value,
// it keeps half of them (the upper half when lane & M is set) and adds the
// partner's copy of that half; once one value remains, plain butterflies finish.
// Every value is summed in pairs at strides 32, 16, 8, 4, 2, 1 (the same tree
// for any N, and IEEE addition is commutative, so the order of the two
// operands does not matter). On return v[0] is the sum of value k, with k built
// from the lane bits of the transposing strides (the same k for equal N).
template <int N, int M>
__device__ __forceinline__ void wave_tsum(float* v, int lane, int& k) {
  if constexpr (M >= 1) {
    if constexpr (N > 1) {
      constexpr int H = N / 2;
      const bool hi = (lane & M) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) v[i] = tstep<M>(v[i], v[i + H], hi);
      if (hi) k += H;
      wave_tsum<H, M / 2>(v, lane, k);
    } else {
      v[0] = v[0] + lane_xor<M>(v[0]);
      wave_tsum<1, M / 2>(v, lane, k);
    }
  }
}

constexpr int pow2_at_least(int n) { return n <= 1 ? 1 : 2 * pow2_at_least((n + 1) / 2); }
constexpr int log2_exact(int n) { return n <= 1 ? 0 : 1 + log2_exact(n / 2); }

// ------------------------------------------------------------ k_gateup
// 8 waves; wave w owns rows 4w..4w+3 of both gate and up of the workgroup's 32
// rows. Lanes cover NBL consecutive blocks each.
// One item: rows rb*32 .. rb*32+31 of expert e's gate and up for plan slot u.

// SwiGLU of the wave's RPW gate and up rows (per-lane partial sums ag / au for
// each of the Q columns) into s_a[t][rowoff + r] for the routed columns t: the
// RPW * Q sums over the wave by transposing butterflies with one lane mapping
// (lane l ends with the gate and up sums of value k = r * Q + t), and the first
// lane of each group forms its SwiGLU (all values in one pass of the wave).
template <int Q, int RPW>
__device__ __forceinline__ void gateup_wave_swiglu(uint32_t mask, const float (&ag)[RPW][Q], const float (&au)[RPW][Q],
                                                   float (&s_a)[4][32], int rowoff) {
  const int lane = threadIdx.x & 63;
  constexpr int NV = RPW * Q, NP = pow2_at_least(NV);
  float g[NP], uu[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    g[i] = (i < NV) ? ag[i / Q][i % Q] : 0.0f;
    uu[i] = (i < NV) ? au[i / Q][i % Q] : 0.0f;
  }
  int kg = 0, ku = 0;
  wave_tsum<NP, 32>(g, lane, kg);
  wave_tsum<NP, 32>(uu, lane, ku);
  constexpr int GROUP = 64 >> log2_exact(NP);   // lanes holding the same value
  if ((lane & (GROUP - 1)) == 0 && kg < NV) {
    const int r = kg / Q, t = kg % Q;
    if (mask >> t & 1) s_a[t][rowoff + r] = g[0] / (1.0f + expf(-g[0])) * uu[0];
  }
}

// Requantization (+ H32) of the 32 SwiGLU values s_a[t][0..31] of each routed
// column t of slot u, row block rb, into hq / dh: half-wave h of wave w takes
// column 2w + h.
template <int Q>
__device__ __forceinline__ void requant_item(const DecodeArgs& a, uint32_t mask, int u, int rb,
                                             const float (&s_a)[4][32]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < (Q + 1) / 2) {
    const int t = 2 * wave + (lane >> 5), j = lane & 31;
    const bool act = t < Q && (mask >> t & 1);
    float d;
    const uint32_t w = quant_block32_lanes(act ? s_a[t][j] : 0.0f, a.rot_down, &d);
    if (act) {
      const size_t slot = (size_t)u * 4 + t;
      if ((j & 3) == 0) reinterpret_cast<uint32_t*>(a.hq + slot * a.inter + (size_t)rb * 32)[j >> 2] = w;
      if (j == 0) a.dh[slot * a.nb_i + rb] = d;
    }
  }
}

// SwiGLU of the workgroup's 32 rows (wave w holds rows RPW*w .. RPW*w + RPW-1 as
// per-lane partial sums) and requantization of the 32-row block (+ H32) for each
// routed column of slot u.
template <int Q, int RPW>
__device__ __forceinline__ void gateup_epilogue(const DecodeArgs& a, uint32_t mask, int u, int rb,
                                                const float (&ag)[RPW][Q], const float (&au)[RPW][Q],
                                                float (&s_a)[4][32]) {
  const int wave = threadIdx.x >> 6;
  gateup_wave_swiglu<Q, RPW>(mask, ag, au, s_a, wave * RPW);
  __syncthreads();
  requant_item<Q>(a, mask, u, rb, s_a);
}

// The gate and up rows row0 .. row0+RPW-1 of expert e against the routed
// columns (column t: quantized row xcol[t], scales dcol[t]): per-lane partial
// sums over the lane's blocks (NBL consecutive blocks per lane and pass).
template <int FMT, int Q, int RPW>
__device__ __forceinline__ void gateup_stream(const DecodeArgs& a, int e, uint32_t mask, int row0,
                                              const int8_t* const (&xcol)[Q], const float* const (&dcol)[Q],
                                              float (&ag)[RPW][Q], float (&au)[RPW][Q]) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  const int lane = threadIdx.x & 63;
  const uint8_t* gbase = a.gate + (size_t)e * a.gu_stride;
  const uint8_t* ubase = a.up + (size_t)e * a.gu_stride;
  uint32_t cbg[4], cbu[4];
  load_codebook<FMT>(a.cb_gate + ((size_t)e << FMT), cbg);
  load_codebook<FMT>(a.cb_up + ((size_t)e << FMT), cbu);
  const int nb = a.nb_h;
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int t = 0; t < Q; ++t) ag[r][t] = au[r][t] = 0.0f;
  for (int c0 = 0; c0 < nb; c0 += 64 * NBL) {
    const int b = c0 + lane * NBL;
    if (b < nb) {
      // the activations (cache-resident) are requested first, so the rows can be
      // used in load order while later rows are still in flight
      Acts<NBL> act[Q];
#pragma unroll
      for (int t = 0; t < Q; ++t)
        if (mask >> t & 1) act[t].load(xcol[t], dcol[t], b);
      Blocks<FMT, NBL> bg[RPW], bu[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        bg[r].load(gbase + (size_t)(row0 + r) * a.gu_row_bytes, nb, b);
        bu[r].load(ubase + (size_t)(row0 + r) * a.gu_row_bytes, nb, b);
      }
      // keep every load above this point: one memory round trip per wave (left
      // to itself the scheduler sinks the scale loads below the first products)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
          uint32_t wg[8], wu[8];
          bg[r].expand(i, cbg, wg);
          bu[r].expand(i, cbu, wu);
          const float sg = bg[r].scale(i), su = bu[r].scale(i);
#pragma unroll
          for (int t = 0; t < Q; ++t)
            if (mask >> t & 1) {
              const int pg = block_dot(wg, act[t].q[i]);
              const int pu = block_dot(wu, act[t].q[i]);
              ag[r][t] = fmaf((float)pg, sg * act[t].d[i], ag[r][t]);
              au[r][t] = fmaf((float)pu, su * act[t].d[i], au[r][t]);
            }
        }
    }
  }
}

template <int FMT, int Q>
__device__ __forceinline__ void gateup_item(const DecodeArgs& a, int e, uint32_t mask, int u, int rb,
                                            float (&s_a)[4][32]) {
  constexpr int RPW = 4;
  const int wave = threadIdx.x >> 6;
  float ag[RPW][Q], au[RPW][Q];
  const int8_t* xcol[Q];
  const float* dcol[Q];
#pragma unroll
  for (int t = 0; t < Q; ++t) {   // the decode tokens' rows are consecutive
    xcol[t] = a.xq + (size_t)t * a.nb_h * 32;
    dcol[t] = a.dx + (size_t)t * a.nb_h;
  }
  gateup_stream<FMT, Q, RPW>(a, e, mask, rb * 32 + wave * RPW, xcol, dcol, ag, au);
  gateup_epilogue<Q, RPW>(a, mask, u, rb, ag, au, s_a);
}

// One token: one workgroup per (plan slot, 32 rows), two workgroups per CU.
template <int FMT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_gateup1(DecodeArgs a) {
  __shared__ float s_a[4][32];
  __shared__ PlanLds P;
  uint32_t mask;
  const int u = blockIdx.y;
  const int e = topk_and_plan<1>(a, P, u, blockIdx.x == 0 && blockIdx.y == 0, mask);
  if (e < 0) return;
  gateup_item<FMT, 1>(a, e, mask, u, blockIdx.x, s_a);
}

// Two to four tokens: the kernel needs more registers, so one workgroup fits per
// CU; a grid of one workgroup per CU selects once and walks the (slot, 32-row)
// items with a stride, instead of paying the selection per item in several
// passes of workgroups.
template <int FMT, int Q>
__global__ __launch_bounds__(512) void k_gateupq(DecodeArgs a) {
  __shared__ float s_a[4][32];
  __shared__ PlanLds P;
  uint32_t mask;
  int U;
  topk_and_plan<Q>(a, P, 0, blockIdx.x == 0, mask, &U);
  const int nrb = a.inter / 32;
  for (int it = blockIdx.x; it < U * nrb; it += gridDim.x) {
    const int u = it / nrb;
    const int e = P.uid[u];
    mask = P.umask[u];
    gateup_item<FMT, Q>(a, e, mask, u, it % nrb, s_a);
    __syncthreads();   // s_a is reused by the next item
  }
}

// Two to four tokens and one pass over the blocks: 1024-thread workgroups (16
// waves of two gate and two up rows each) walk the same items with the tokens'
// int8 blocks and scales copied to LDS once. That leaves ~90 registers per lane,
// so four waves per SIMD issue the vector instructions (k_gateupq, at 223
// registers, runs two). The LDS copy puts piece g (16 bytes) of a token row at
// (g % CPL) * 64 + g / CPL and the scale of block k at (k % NBL) * 64 + k / NBL,
// so that the 64 lanes of a read touch consecutive addresses. The per-lane
// accumulation order is that of gateup_item.
template <int FMT, int Q>
__global__ __launch_bounds__(1024) void k_gateupq2(DecodeArgs a) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  constexpr int RPW = 2;
  constexpr int CPL = 2 * NBL;
  __shared__ float s_a2[2][4][32];   // SwiGLU rows of alternate items (see the item loop)
  __shared__ PlanLds P;
  __shared__ u32x4 s_xq[Q * 256];   // per token: 64 lanes x CPL pieces
  __shared__ float s_dx[Q * 128];   // per token: 64 lanes x NBL scales
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nb = a.nb_h;
  // The waves that do not select (wave >= Q) request the tokens' int8 blocks
  // and scales before the selection, so those loads complete while waves
  // 0 .. q-1 select (the selection's barriers order LDS only); the pieces are
  // stored to LDS afterwards. Every load of a copying thread is issued (index
  // clamped).
  constexpr int NCP = 1024 - 64 * Q;                     // copying threads
  constexpr int NXP = (Q * 256 + NCP - 1) / NCP;          // 16-byte pieces per copying thread
  constexpr int NDP = (Q * 128 + NCP - 1) / NCP;          // scales per copying thread
  const int ct = tid - 64 * Q;
  const int npx = Q * nb * 2, npd = Q * nb;
  u32x4 xv[NXP];
  float dv[NDP];
  if (ct >= 0) {   // (uniform per wave: the selecting waves issue nothing before their logits)
#pragma unroll
    for (int k = 0; k < NXP; ++k) xv[k] = reinterpret_cast<const u32x4*>(a.xq)[min(ct + NCP * k, npx - 1)];
#pragma unroll
    for (int k = 0; k < NDP; ++k) dv[k] = a.dx[min(ct + NCP * k, npd - 1)];
  }
  uint32_t mask0;
  int U;
  // the copying waves store the tokens to LDS while wave 0 lists the plan; the
  // selection's last barrier makes them visible to every wave
  auto store_tokens = [&]() {
    if (ct >= 0) {
#pragma unroll
      for (int k = 0; k < NXP; ++k) {
        const int i = ct + NCP * k;
        if (i < npx) {
          const int t = i / (nb * 2), g = i % (nb * 2);
          s_xq[t * 256 + (g % CPL) * 64 + g / CPL] = xv[k];
        }
      }
#pragma unroll
      for (int k = 0; k < NDP; ++k) {
        const int i = ct + NCP * k;
        if (i < npd) {
          const int t = i / nb, kk = i % nb;
          s_dx[t * 128 + (kk % NBL) * 64 + kk / NBL] = dv[k];
        }
      }
    }
  };
  topk_and_plan<Q>(a, P, 0, blockIdx.x == 0, mask0, &U, store_tokens);
  const int nrb = a.inter / 32;
  const int b = lane * NBL;
  const bool ok = b < nb;
  const int bc = min(b, nb - NBL);
  // Work units: the items of the full rounds whole, then the last round's items
  // split by columns (each column's products, SwiGLU and requantization are
  // independent), with the fewest columns per unit that leave every workgroup at
  // most one unit, so that the last round does not keep a few workgroups busy
  // with whole items while the rest wait.
  const int NI = U * nrb, G = (int)gridDim.x;
  const int full = NI - NI % G;
  const int L = NI - full;
  const int S = (L * Q <= G) ? 1 : (L * ((Q + 1) / 2) <= G) ? 2 : Q;   // columns per last-round unit
  const int CG = (Q + S - 1) / S;                                        // column groups per item
  const int nunits = full + L * CG;
  // the first non-empty unit at or after w (stride G), with its slot, row block
  // and column mask; nunits when none is left
  auto find_unit = [&](int w, int& u, int& rb, uint32_t& mask) -> int {
    for (; w < nunits; w += G) {
      int it;
      uint32_t cmask;
      if (w < full) {
        it = w;
        cmask = 0xFu;
      } else {
        const int j = w - full;
        it = full + j / CG;
        cmask = ((1u << S) - 1u) << (S * (j % CG));
      }
      u = it / nrb;
      rb = it % nrb;
      mask = P.umask[u] & cmask;
      if (mask != 0u) return w;
    }
    return nunits;
  };
  Blocks<FMT, NBL> bg[RPW], bu[RPW];
  uint32_t cbg[4], cbu[4];
  // the wave's gate and up rows of a unit, every load issued (index clamped)
  auto load_unit = [&](int u, int rb) {
    const int e = P.uid[u];
    const int row0 = rb * 32 + wave * RPW;
    const uint8_t* gbase = a.gate + (size_t)e * a.gu_stride;
    const uint8_t* ubase = a.up + (size_t)e * a.gu_stride;
    load_codebook<FMT>(a.cb_gate + ((size_t)e << FMT), cbg);
    load_codebook<FMT>(a.cb_up + ((size_t)e << FMT), cbu);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      bg[r].load(gbase + (size_t)(row0 + r) * a.gu_row_bytes, nb, bc);
      bu[r].load(ubase + (size_t)(row0 + r) * a.gu_row_bytes, nb, bc);
    }
  };
  int u = 0, rb = 0;
  uint32_t mask = 0u;
  int w = find_unit((int)blockIdx.x, u, rb, mask);
  if (w < nunits) load_unit(u, rb);
  int k = 0;   // units processed by this workgroup (alternate SwiGLU buffers)
  while (w < nunits) {
    __builtin_amdgcn_sched_barrier(0);
    float ag[RPW][Q], au[RPW][Q];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int t = 0; t < Q; ++t) ag[r][t] = au[r][t] = 0.0f;
    if (ok) {
#pragma unroll
      for (int i = 0; i < NBL; ++i) {
        uint32_t wg[RPW][8], wu[RPW][8];
        float sg[RPW], su[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          bg[r].expand(i, cbg, wg[r]);
          bu[r].expand(i, cbu, wu[r]);
          sg[r] = bg[r].scale(i);
          su[r] = bu[r].scale(i);
        }
#pragma unroll
        for (int t = 0; t < Q; ++t)
          if (mask >> t & 1) {
            const u32x4 x0 = s_xq[t * 256 + (2 * i) * 64 + lane], x1 = s_xq[t * 256 + (2 * i + 1) * 64 + lane];
            const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const float dxt = s_dx[t * 128 + i * 64 + lane];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
              const int pg = block_dot(wg[r], xw);
              const int pu = block_dot(wu[r], xw);
              ag[r][t] = fmaf((float)pg, sg[r] * dxt, ag[r][t]);
              au[r][t] = fmaf((float)pu, su[r] * dxt, au[r][t]);
            }
          }
      }
    }
    // the next unit's weights are requested before this unit's epilogue, so that
    // they stream during the SwiGLU, its barrier and the requantization (the
    // last unit requests its own rows again: no branch around the loads)
    int u2 = u, rb2 = rb;
    uint32_t mask2 = 0u;
    const int w2 = find_unit(w + G, u2, rb2, mask2);
    load_unit(w2 < nunits ? u2 : u, w2 < nunits ? rb2 : rb);
    // alternate units use alternate SwiGLU buffers, so no barrier is needed after
    // the requantization: the next unit's SwiGLU writes the other buffer, and the
    // unit after it passes the next unit's barrier, which the requantizing waves
    // reach only after finishing (q=4 42.35 -> 42.05 us in an interleaved
    // comparison, same bits)
    gateup_epilogue<Q, RPW>(a, mask, u, rb, ag, au, s_a2[k & 1]);
    ++k;
    w = w2;
    u = u2;
    rb = rb2;
    mask = mask2;
  }
}

// ------------------------------------------------------------ k_down
// Each wave handles 64/LPR rows (LPR lanes per row, NBL blocks per lane); the
// row chunks of UB planned experts are loaded together before any is used.
template <int FMT, int Q>
__global__ __launch_bounds__(256) void k_down(DecodeArgs a) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  constexpr int UB = (Q == 1) ? 6 : ((Q == 2) ? 4 : 3);
  const int lpr_log2 = a.dn_lpr_log2;
  const int lpr = 1 << lpr_log2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int row = (blockIdx.x * 4 + wave) * (64 >> lpr_log2) + sub;
  const bool row_ok = row < a.hidden;
  // the plan (256 words: size, ids, masks, weights), read in one round trip
  static_assert(kPlanWOff + 4 * kPlanMax == 256, "plan fits one load per thread");
  __shared__ int s_plan[kPlanWOff + 4 * kPlanMax];
  s_plan[threadIdx.x] = a.plan[threadIdx.x];
  __syncthreads();
  const int U = s_plan[0];
  const float* pw = reinterpret_cast<const float*>(s_plan + kPlanWOff);
  const int nb = a.nb_i;
  float acc[Q];
#pragma unroll
  for (int t = 0; t < Q; ++t) acc[t] = 0.0f;
  for (int c0 = 0; c0 < nb; c0 += lpr * NBL) {
    const int b = c0 + sl * NBL;
    const bool ok = row_ok && b < nb;
    for (int u0 = 0; u0 < U; u0 += UB) {
      Blocks<FMT, NBL> bl[UB];
      int ej[UB];
#pragma unroll
      for (int j = 0; j < UB; ++j) {
        ej[j] = (u0 + j < U) ? s_plan[kPlanIdOff + u0 + j] : 0;
        if (ok && u0 + j < U) bl[j].load(a.down + (size_t)ej[j] * a.dn_stride + (size_t)row * a.dn_row_bytes, nb, b);
      }
#pragma unroll
      for (int j = 0; j < UB; ++j) {
        const int u = u0 + j;
        if (u < U) {
          const uint32_t mask = (uint32_t)s_plan[kPlanMaskOff + u];
          uint32_t cb[4];
          load_codebook<FMT>(a.cb_down + ((size_t)ej[j] << FMT), cb);
          if (ok) {
#pragma unroll
            for (int t = 0; t < Q; ++t)
              if (mask >> t & 1) {
                const float wgt = pw[4 * u + t];
                const size_t slot = (size_t)u * 4 + t;
                Acts<NBL> act;
                act.load(a.hq + slot * a.inter, a.dh + slot * nb, b);
#pragma unroll
                for (int i = 0; i < NBL; ++i) {
                  uint32_t w[8];
                  bl[j].expand(i, cb, w);
                  const int p = block_dot(w, act.q[i]);
                  acc[t] = fmaf((float)p, bl[j].scale(i) * act.d[i] * wgt, acc[t]);
                }
              }
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    const float v = group_sum(acc[t], lpr);
    if (sl == 0 && row_ok) a.out[(size_t)t * a.hidden + row] = v;
  }
}

// Two to four tokens, when one pass covers the blocks and the routed
// (expert, token) slots' activations fit 48 KB: the workgroup lists the slots of
// the plan, requests their activations (16-byte pieces into registers, copied to
// LDS) and then the weight blocks of up to 12 experts, all in one round trip;
// each expert's products wait only for that expert's blocks, so the arithmetic
// of the first experts overlaps the arrival of the rest. (Direct global -> LDS
// loads of the activations save registers, but the compiler does not track
// them, so the kernel had to wait for every load before the first product.)
// Each block is expanded once and applied to every routed column. k_down instead loads each lane's own copy of every slot's activations
// after that expert's weights. The per-lane accumulation order is that of k_down
// (experts ascending, then columns, then the lane's blocks).
constexpr int kDownqActPieces = 48 * 1024 / 16;   // 16-byte pieces of staged activations
constexpr int kDownqMaxSlots = 32;
// 8 waves per workgroup: one copy of the routed activations serves 8 waves'
// rows (with 4 waves, the copies of all workgroups, re-read from the shared
// cache levels, added 0.8x the weight bytes to the traffic of the launch)
constexpr int kDownqThreads = 512;
template <int FMT, int Q>
__global__ __launch_bounds__(kDownqThreads) void k_downq(DecodeArgs a) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  constexpr int UB = 12;
  constexpr int CPL = 2 * NBL;   // 16-byte activation pieces per lane and slot
  const int lpr_log2 = a.dn_lpr_log2;
  const int lpr = 1 << lpr_log2;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int row = (blockIdx.x * (kDownqThreads / 64) + wave) * (64 >> lpr_log2) + sub;
  __shared__ int s_plan[kPlanWOff + 4 * kPlanMax];
  __shared__ int s_slot[kDownqMaxSlots];      // compact slot c -> u * 4 + t
  __shared__ int s_cidx[4 * kPlanMax];        // u * 4 + t -> compact slot
  __shared__ int s_nslot;
  __shared__ u32x4 s_act[kDownqActPieces];
  __shared__ u32x4 s_dh[kDownqMaxSlots * 16];
  static_assert(kPlanWOff + 4 * kPlanMax == 256, "plan fits one load per thread of the first 256");
  if (tid < 256) s_plan[tid] = a.plan[tid];
  __syncthreads();
  const int U = s_plan[0];
  const float* pw = reinterpret_cast<const float*>(s_plan + kPlanWOff);
  const int nb = a.nb_i;
  if (wave == 0) {
    // lane u < U: its routed columns; exclusive prefix of the counts by ballots
    const uint32_t m = (lane < U) ? ((uint32_t)s_plan[kPlanMaskOff + lane] & ((1u << Q) - 1u)) : 0u;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0, total = 0;
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const uint64_t bt = __ballot((m >> t) & 1u);
      base += __popcll(bt & lt);
      total += __popcll(bt);
    }
    int c = base;
#pragma unroll
    for (int t = 0; t < Q; ++t)
      if ((m >> t) & 1u) {
        s_slot[c] = lane * 4 + t;
        s_cidx[lane * 4 + t] = c;
        ++c;
      }
    if (lane == 0) s_nslot = total;
  }
  __syncthreads();
  const int nslot = s_nslot;
  const int b = sl * NBL;
  const bool ok = row < a.hidden && b < nb;
  const int rowc = min(row, a.hidden - 1), bc = min(b, nb - NBL);
  // activations of the listed slots, requested first into registers (so that
  // the compiler's waits before the LDS stores cover these loads only): LDS
  // piece (within slot c) m * lpr + l holds piece l * CPL + m of the slot's
  // row, so that each read of the lanes of one row touches consecutive pieces.
  // Every load is issued (index clamped); only the stores are restricted.
  const int pps = nb * 2;   // pieces per slot (= lpr * CPL)
  const int nq = nslot * pps;
  const int nd = nslot * (nb / 4);   // 16-byte pieces of scales (4 per piece)
  constexpr int AP = kDownqActPieces / kDownqThreads;
  constexpr int DP = (kDownqMaxSlots * 16 + kDownqThreads - 1) / kDownqThreads;
  u32x4 av[AP], dv[DP];
#pragma unroll
  for (int k = 0; k < AP; ++k) {
    const int P = min(tid + kDownqThreads * k, nq - 1);
    const int c = P / pps, within = P % pps;
    const int g = (within % lpr) * CPL + within / lpr;
    av[k] = *reinterpret_cast<const u32x4*>(a.hq + (size_t)s_slot[c] * a.inter + (size_t)g * 16);
  }
#pragma unroll
  for (int k = 0; k < DP; ++k) {
    const int P = min(tid + kDownqThreads * k, nd - 1);
    const int c = P / (nb / 4), within = P % (nb / 4);
    dv[k] = *reinterpret_cast<const u32x4*>(a.dh + (size_t)s_slot[c] * nb + (size_t)within * 4);
  }
  // weights of the first group of experts (unconditional, clamped loads), all
  // requested before any is used; each expert's products below wait for its
  // own blocks only, so the arithmetic overlaps the rest of the stream
  int ej[UB];
  uint32_t cb[UB][4];
  Blocks<FMT, NBL> bl[UB];
#pragma unroll
  for (int j = 0; j < UB; ++j) {
    ej[j] = (j < U) ? s_plan[kPlanIdOff + j] : 0;
    load_codebook<FMT>(a.cb_down + ((size_t)ej[j] << FMT), cb[j]);
    bl[j].load(a.down + (size_t)ej[j] * a.dn_stride + (size_t)rowc * a.dn_row_bytes, nb, bc);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < AP; ++k)
    if (tid + kDownqThreads * k < nq) s_act[tid + kDownqThreads * k] = av[k];
#pragma unroll
  for (int k = 0; k < DP; ++k)
    if (tid + kDownqThreads * k < nd) s_dh[tid + kDownqThreads * k] = dv[k];
  __syncthreads();
  const float* dh = reinterpret_cast<const float*>(s_dh);
  float acc[Q];
#pragma unroll
  for (int t = 0; t < Q; ++t) acc[t] = 0.0f;
  for (int u0 = 0; u0 < U; u0 += UB) {
    if (u0 > 0) {   // further groups (more than UB planned experts)
#pragma unroll
      for (int j = 0; j < UB; ++j) {
        ej[j] = (u0 + j < U) ? s_plan[kPlanIdOff + u0 + j] : 0;
        load_codebook<FMT>(a.cb_down + ((size_t)ej[j] << FMT), cb[j]);
        bl[j].load(a.down + (size_t)ej[j] * a.dn_stride + (size_t)rowc * a.dn_row_bytes, nb, bc);
      }
    }
#pragma unroll
    for (int j = 0; j < UB; ++j) {
      const int u = u0 + j;
      if (ok && u < U) {
        const uint32_t mask = (uint32_t)s_plan[kPlanMaskOff + u];
        uint32_t w[NBL][8];
#pragma unroll
        for (int i = 0; i < NBL; ++i) bl[j].expand(i, cb[j], w[i]);
#pragma unroll
        for (int t = 0; t < Q; ++t)
          if (mask >> t & 1) {
            const float wgt = pw[4 * u + t];
            const int c = s_cidx[u * 4 + t];
#pragma unroll
            for (int i = 0; i < NBL; ++i) {
              const u32x4 x0 = s_act[c * pps + (2 * i) * lpr + sl];
              const u32x4 x1 = s_act[c * pps + (2 * i + 1) * lpr + sl];
              const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
              const int p = block_dot(w[i], xw);
              acc[t] = fmaf((float)p, bl[j].scale(i) * dh[c * nb + b + i] * wgt, acc[t]);
            }
          }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    const float v = group_sum(acc[t], lpr);
    if (sl == 0 && row < a.hidden) a.out[(size_t)t * a.hidden + row] = v;
  }
}

// One token, at most six planned experts, one pass over the blocks and at most
// 16 KB of activations (the common shape; the host sends other shapes to
// k_down). The workgroup copies the activations of the planned experts to LDS
// with one 16-byte load per thread and piece (every lane of k_down loads its own
// copy, 8x the bytes through the vector cache per CU), and requests all weight
// blocks of the lane behind them, before any is used. The accumulation order is
// that of k_down.
constexpr int kDown1MaxU = 6;
constexpr int kDown1ActBytes = 16384;
template <int FMT>
__global__ __launch_bounds__(256) void k_down1(DecodeArgs a) {
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  constexpr int UB = kDown1MaxU;
  const int lpr_log2 = a.dn_lpr_log2;
  const int lpr = 1 << lpr_log2;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int row = (blockIdx.x * 4 + wave) * (64 >> lpr_log2) + sub;
  __shared__ int s_plan[kPlanWOff + 4 * kPlanMax];
  __shared__ u32x4 s_hq[kDown1ActBytes / 16];
  __shared__ u32x4 s_dh[256];   // >= kDown1ActBytes / 32 / 4, one piece per thread
  s_plan[tid] = a.plan[tid];
  __syncthreads();
  const int U = s_plan[0];
  const float* pw = reinterpret_cast<const float*>(s_plan + kPlanWOff);
  const int nb = a.nb_i;
  // activations of slots (u, token 0) = 4u: U rows of inter bytes and nb scales
  const int nq = U * a.inter / 16, nd = U * nb / 4;
  // every thread issues every load (indices clamped into range; only the LDS
  // stores below are restricted), so no loaded value is defined conditionally
  u32x4 hv[4], dv;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = min(tid + 256 * k, nq - 1);
    const int u = (16 * i) / a.inter, off = (16 * i) % a.inter;
    hv[k] = *reinterpret_cast<const u32x4*>(a.hq + (size_t)u * 4 * a.inter + off);
  }
  {
    const int i = min(tid, nd - 1);
    const int u = (4 * i) / nb, off = (4 * i) % nb;
    dv = *reinterpret_cast<const u32x4*>(a.dh + (size_t)u * 4 * nb + off);
  }
  const int b = sl * NBL;
  const bool ok = row < a.hidden && b < nb;
  // weight loads are unconditional too (row and block clamped, idle slots read
  // expert 0): a load inside a branch makes the wait before the LDS stores
  // below count as if it had not been issued
  const int rowc = min(row, a.hidden - 1), bc = min(b, nb - NBL);
  int ej[UB];
  uint32_t cb[UB][4];
  Blocks<FMT, NBL> bl[UB];
#pragma unroll
  for (int j = 0; j < UB; ++j) {
    ej[j] = (j < U) ? s_plan[kPlanIdOff + j] : 0;
    load_codebook<FMT>(a.cb_down + ((size_t)ej[j] << FMT), cb[j]);
  }
#pragma unroll
  for (int j = 0; j < UB; ++j)
    bl[j].load(a.down + (size_t)ej[j] * a.dn_stride + (size_t)rowc * a.dn_row_bytes, nb, bc);
  __builtin_amdgcn_sched_barrier(0);
  // pieces beyond nq / nd land in LDS slots that are never read
#pragma unroll
  for (int k = 0; k < 4; ++k) s_hq[tid + 256 * k] = hv[k];
  s_dh[tid] = dv;
  __syncthreads();
  const int8_t* hq = reinterpret_cast<const int8_t*>(s_hq);
  const float* dh = reinterpret_cast<const float*>(s_dh);
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < UB; ++j)
    if (ok && j < U) {
      const float wgt = pw[4 * j];
      Acts<NBL> act;
      act.load(hq + (size_t)j * a.inter, dh + (size_t)j * nb, b);
#pragma unroll
      for (int i = 0; i < NBL; ++i) {
        uint32_t w[8];
        bl[j].expand(i, cb[j], w);
        const int p = block_dot(w, act.q[i]);
        acc = fmaf((float)p, bl[j].scale(i) * act.d[i] * wgt, acc);
      }
    }
  const float v = group_sum(acc, lpr);
  if (sl == 0 && row < a.hidden) a.out[row] = v;
}

template <int FG, int FD, int Q>
int launch_decode_t(const DecodeArgs& a, int U_max, hipStream_t s) {
  {
    // E logit workgroups, then the token-quantization workgroups
    const int nq = (a.q * a.nb_h + a.quant_per_wg - 1) / a.quant_per_wg;
    launch_kernel("route", k_route<Q>, dim3(a.E + nq), dim3(128 * Q), s, a);
  }
  int st = launch_check("route");
  if (st) return st;
  {
    if constexpr (Q == 1)
      launch_kernel("gateup", k_gateup1<FG>, dim3(a.inter / 32, U_max), dim3(512), s, a);
    else
      if (a.nb_h <= 64 * ((FG == 4) ? 1 : 2))
        launch_kernel("gateup", k_gateupq2<FG, Q>, dim3(device_cu_count()), dim3(1024), s, a);
      else
        launch_kernel("gateup", k_gateupq<FG, Q>, dim3(device_cu_count()), dim3(512), s, a);
  }
  if ((st = launch_check("gateup"))) return st;
  const int rows_per_wg = 4 * (64 >> a.dn_lpr_log2);
  {
    const dim3 grid((a.hidden + rows_per_wg - 1) / rows_per_wg);
    constexpr int NBL = (FD == 4) ? 1 : 2;
    if (Q == 1 && U_max <= kDown1MaxU && a.nb_i <= (NBL << a.dn_lpr_log2) && a.nb_i % 4 == 0 &&
        U_max * a.inter <= kDown1ActBytes)
      launch_kernel("down", k_down1<FD>, grid, dim3(256), s, a);
    else if (Q > 1 && a.nb_i == (NBL << a.dn_lpr_log2) && a.nb_i % 4 == 0 && Q * a.K <= kDownqMaxSlots &&
             Q * a.K * a.inter <= kDownqActPieces * 16) {
      const int rq = (kDownqThreads / 64) * (64 >> a.dn_lpr_log2);   // rows per workgroup
      QMOE_BOUNDS(rq > 0 && (int64_t)((a.hidden + rq - 1) / rq) * rq >= a.hidden, "decode: down grid covers the rows");
      launch_kernel("down", k_downq<FD, Q>, dim3((a.hidden + rq - 1) / rq), dim3(kDownqThreads), s, a);
    }
    else
      launch_kernel("down", k_down<FD, Q>, grid, dim3(256), s, a);
  }
  return launch_check("down");
}

template <int Q>
int launch_decode_q(const DecodeArgs& a, int U_max, int fg, int fd, hipStream_t s) {
  if (fg == 2 && fd == 3) return launch_decode_t<2, 3, Q>(a, U_max, s);
  if (fg == 2 && fd == 2) return launch_decode_t<2, 2, Q>(a, U_max, s);
  if (fg == 2 && fd == 4) return launch_decode_t<2, 4, Q>(a, U_max, s);
  if (fg == 3 && fd == 3) return launch_decode_t<3, 3, Q>(a, U_max, s);
  if (fg == 3 && fd == 2) return launch_decode_t<3, 2, Q>(a, U_max, s);
  if (fg == 3 && fd == 4) return launch_decode_t<3, 4, Q>(a, U_max, s);
  if (fg == 4 && fd == 3) return launch_decode_t<4, 3, Q>(a, U_max, s);
  if (fg == 4 && fd == 2) return launch_decode_t<4, 2, Q>(a, U_max, s);
  return launch_decode_t<4, 4, Q>(a, U_max, s);
}

// ------------------------------------------------------------ decode on the matrix cores
// The same layer with the expert products on v_mfma_i32_4x4x4_16b_i8, which
// computes 16 independent 4 x 4 x 4 int8 products per instruction. Its 4 rows
// are 4 weight rows (2 gate + 2 up rows, or 4 down rows), its 4 columns the
// q <= 4 tokens (a column is zero past q and for a token not routed to the
// expert), and its 16 blocks 16 consecutive 32-weight blocks of those rows;
// 8 instructions (K = 4 each) give the exact int32 sum of every (row, token,
// block). Lane l = 4b + i supplies row i's weights of block b (expanded by byte
// permutes as for sdot4) and token i's activations of block b, and receives
// the sums of rows 0..3 of block b for token i. It adds float(P) * (s_w * d_x)
// per row in block order, and the 16 lanes of each token are then summed by
// xor butterflies over lane bits 2..5. That order is its own (results within
// the oracle's tolerance, not the bits of qmoe_decode_layer) and the same for
// every q, so column t of q tokens equals a one-token call bit for bit.
// ([Strix-284B] decode section: each block decoded once for the q = 4
// verification columns; here the q columns are the MFMA's N dimension.)
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kMxMaxNbH = 256;    // gate/up rows of at most 8192 weights
constexpr int kMxGroups = 8;      // 16-block groups per pass of a gate/up row
constexpr int kMxMaxNbI = 64;     // down rows of at most 2048 weights: one group per wave
constexpr int kMxUB = 12;         // down: experts whose weights are requested together
constexpr int kDownmActBytes = 64 * 1024;

// Exact int32 sums of one block for the lane's row and token (see above).
__device__ __forceinline__ v4i mfma4_block(const uint32_t w[8], const uint32_t x[8]) {
  v4i c = {0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < 8; ++k) c = __builtin_amdgcn_mfma_i32_4x4x4i8((int)w[k], (int)x[k], c, 0, 0, 0);
  return c;
}

// acc[r] += float(P[r]) * (s_w(row r) * f) for the 4 rows of the lane's block:
// the scales of rows 0..3 come from lanes 4b + 0..3 of the quad (DPP broadcasts).
__device__ __forceinline__ void mfma4_accumulate(const v4i& P, float sw, float f, float (&acc)[4]) {
  const float s0 = dpp_f32<0x00>(sw), s1 = dpp_f32<0x55>(sw), s2 = dpp_f32<0xAA>(sw), s3 = dpp_f32<0xFF>(sw);
  acc[0] = fmaf((float)P[0], s0 * f, acc[0]);
  acc[1] = fmaf((float)P[1], s1 * f, acc[1]);
  acc[2] = fmaf((float)P[2], s2 * f, acc[2]);
  acc[3] = fmaf((float)P[3], s3 * f, acc[3]);
}

// Sum over the 16 lanes that share lane & 3 (all 64 lanes active).
__device__ __forceinline__ float sum_lane_bits2to5(float v) {
  v = v + xchg32<4>(v);
  v = v + xchg32<8>(v);
  v = v + xchg32<16>(v);
  return v + __shfl_xor(v, 32);
}

// Gate/up: one workgroup of 16 waves per CU walks the (slot, 32-row) items as
// k_gateupq2 does; wave w takes gate rows 2w, 2w + 1 and up rows 2w, 2w + 1 of
// the item as MFMA rows 0..3. The tokens' int8 rows and scales are copied to
// LDS once (by the waves that do not select, during the selection), each row
// padded by one 16-byte piece so that the 4 tokens of a read fall in distinct
// banks.
template <int FMT, int Q>
__global__ __launch_bounds__(1024) void k_gateupm(DecodeArgs a) {
  constexpr int XT = 2 * kMxMaxNbH + 1;   // 16-byte pieces per token row in LDS
  constexpr int DT = kMxMaxNbH + 1;
  __shared__ float s_a[4][32];
  __shared__ PlanLds P;
  __shared__ u32x4 s_xq[Q * XT];
  __shared__ float s_dx[Q * DT];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nb = a.nb_h;
  constexpr int NCP = 1024 - 64 * Q;                              // copying threads
  constexpr int NXP = (Q * 2 * kMxMaxNbH + NCP - 1) / NCP;        // 16-byte pieces per copying thread
  constexpr int NDP = (Q * kMxMaxNbH + NCP - 1) / NCP;            // scales per copying thread
  const int ct = tid - 64 * Q;
  const int npx = Q * nb * 2, npd = Q * nb;
  u32x4 xv[NXP];
  float dv[NDP];
  if (ct >= 0) {   // (uniform per wave)
#pragma unroll
    for (int k = 0; k < NXP; ++k) xv[k] = reinterpret_cast<const u32x4*>(a.xq)[min(ct + NCP * k, npx - 1)];
#pragma unroll
    for (int k = 0; k < NDP; ++k) dv[k] = a.dx[min(ct + NCP * k, npd - 1)];
  }
  uint32_t mask0;
  int U;
  topk_and_plan<Q>(a, P, 0, blockIdx.x == 0, mask0, &U);
  if (ct >= 0) {
#pragma unroll
    for (int k = 0; k < NXP; ++k) {
      const int i = ct + NCP * k;
      if (i < npx) s_xq[(i / (nb * 2)) * XT + i % (nb * 2)] = xv[k];
    }
#pragma unroll
    for (int k = 0; k < NDP; ++k) {
      const int i = ct + NCP * k;
      if (i < npd) s_dx[(i / nb) * DT + i % nb] = dv[k];
    }
  }
  __syncthreads();
  const int i4 = lane & 3, b = lane >> 2;
  const int tq = min(i4, Q - 1);   // the lane's token column (read in range; zeroed when not live)
  const int nrb = a.inter / 32;
  const int G = nb >> 4;
  const bool is_up = i4 >= 2;
  for (int it = blockIdx.x; it < U * nrb; it += gridDim.x) {
    const int u = it / nrb, rb = it % nrb;
    const uint32_t mask = P.umask[u];
    const int e = min(max(P.uid[u], 0), a.E - 1);   // (a plan id is in range; the clamp keeps any address so)
    const bool live = i4 < Q && ((mask >> i4) & 1u);
    const int row = rb * 32 + 2 * wave + (i4 & 1);
    const uint8_t* rp = (is_up ? a.up : a.gate) + (size_t)e * a.gu_stride + (size_t)row * a.gu_row_bytes;
    uint32_t cb[4];
    load_codebook<FMT>((is_up ? a.cb_up : a.cb_gate) + ((size_t)e << FMT), cb);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int g0 = 0; g0 < G; g0 += kMxGroups) {
      // every block load of the pass is requested (index clamped) before any is used
      Blocks<FMT, 1> bl[kMxGroups];
#pragma unroll
      for (int k = 0; k < kMxGroups; ++k) bl[k].load(rp, nb, min(16 * (g0 + k) + b, nb - 1));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kMxGroups; ++k)
        if (g0 + k < G) {   // uniform
          const int blk = 16 * (g0 + k) + b;
          uint32_t w[8];
          bl[k].expand(0, cb, w);
          const u32x4 x0 = s_xq[tq * XT + 2 * blk], x1 = s_xq[tq * XT + 2 * blk + 1];
          const uint32_t xr[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          uint32_t xw[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) xw[j] = live ? xr[j] : 0u;
          mfma4_accumulate(mfma4_block(w, xw), bl[k].scale(0), s_dx[tq * DT + blk], acc);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = sum_lane_bits2to5(acc[r]);
    // lane t < Q holds the gate (acc[0], acc[1]) and up (acc[2], acc[3]) sums of
    // rows 2w, 2w + 1 for token t
    if (lane < Q && ((mask >> lane) & 1u)) {
#pragma unroll
      for (int r = 0; r < 2; ++r) s_a[lane][2 * wave + r] = acc[r] / (1.0f + expf(-acc[r])) * acc[2 + r];
    }
    __syncthreads();
    requant_item<Q>(a, mask, u, rb, s_a);
    __syncthreads();   // s_a is reused by the next item
  }
}

// Down: one workgroup of 16 waves per 16 rows: wave w takes rows 4 (w % 4) ..
// + 3 as MFMA rows and the blocks of K quarter w / 4 (one 16-block group for
// inter 2048), for every planned expert in ascending id; the four quarters'
// sums meet in LDS in quarter order. The routed slots' activations are copied
// to LDS once per workgroup, each slot row padded by one 16-byte piece.
template <int FMT, int Q>
__global__ __launch_bounds__(1024) void k_downm(DecodeArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rq = wave & 3, kq = wave >> 2;
  const int nb = a.nb_i;
  const int SS = 2 * nb + 1;   // 16-byte pieces per slot row in LDS
  constexpr int DS = kMxMaxNbI + 1;
  __shared__ int s_plan[kPlanWOff + 4 * kPlanMax];
  __shared__ int s_slot[kDownqMaxSlots];
  __shared__ int s_cidx[4 * kPlanMax];
  __shared__ int s_nslot;
  __shared__ u32x4 s_act[kDownmActBytes / 16];
  __shared__ float s_dh[kDownqMaxSlots * DS];
  __shared__ float s_part[4][4][4][4];   // [K quarter][row quad][token][row]
  static_assert(kPlanWOff + 4 * kPlanMax == 256, "plan fits one load per thread of the first 256");
  if (tid < 256) s_plan[tid] = a.plan[tid];
  __syncthreads();
  const int U = s_plan[0];
  const float* pw = reinterpret_cast<const float*>(s_plan + kPlanWOff);
  if (wave == 0) {
    // lane u < U: its routed columns; compact slots by ballots (as k_downq)
    const uint32_t m = (lane < U) ? ((uint32_t)s_plan[kPlanMaskOff + lane] & ((1u << Q) - 1u)) : 0u;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0, total = 0;
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const uint64_t bt = __ballot((m >> t) & 1u);
      base += __popcll(bt & lt);
      total += __popcll(bt);
    }
    int c = base;
#pragma unroll
    for (int t = 0; t < Q; ++t)
      if ((m >> t) & 1u) {
        s_slot[c] = lane * 4 + t;
        s_cidx[lane * 4 + t] = c;
        ++c;
      }
    if (lane == 0) s_nslot = total;
  }
  __syncthreads();
  const int nslot = s_nslot;
  // activations of the listed slots into registers (indices clamped), then the
  // first experts' weights, then the LDS stores
  constexpr int AP = kDownmActBytes / 16 / 1024;
  const int pps = nb * 2, nq = nslot * pps, nd = nslot * (nb / 4);
  u32x4 av[AP], dv;
#pragma unroll
  for (int k = 0; k < AP; ++k) {
    const int i = min(tid + 1024 * k, nq - 1);
    av[k] = *reinterpret_cast<const u32x4*>(a.hq + (size_t)s_slot[i / pps] * a.inter + (size_t)(i % pps) * 16);
  }
  {
    const int i = min(tid, nd - 1);
    dv = *reinterpret_cast<const u32x4*>(a.dh + (size_t)s_slot[i / (nb / 4)] * nb + (size_t)(i % (nb / 4)) * 4);
  }
  const int i4 = lane & 3, b = lane >> 2;
  const int row = blockIdx.x * 16 + 4 * rq + i4;           // the lane's weight row
  const int rowc = min(row, a.hidden - 1);
  const bool has_group = 16 * kq < nb;                      // (uniform) this quarter holds a group
  const int blk = min(16 * kq + b, nb - 1);
  int ej[kMxUB];
  uint32_t cb[kMxUB][4];
  Blocks<FMT, 1> bl[kMxUB];
#pragma unroll
  for (int j = 0; j < kMxUB; ++j) {
    ej[j] = (j < U) ? min(max(s_plan[kPlanIdOff + j], 0), a.E - 1) : 0;
    load_codebook<FMT>(a.cb_down + ((size_t)ej[j] << FMT), cb[j]);
    bl[j].load(a.down + (size_t)ej[j] * a.dn_stride + (size_t)rowc * a.dn_row_bytes, nb, blk);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < AP; ++k) {
    const int i = tid + 1024 * k;
    if (i < nq) s_act[(i / pps) * SS + i % pps] = av[k];
  }
  if (tid < nd) {
    const int c = tid / (nb / 4), o = (tid % (nb / 4)) * 4;
    s_dh[c * DS + o] = __uint_as_float(dv.x);
    s_dh[c * DS + o + 1] = __uint_as_float(dv.y);
    s_dh[c * DS + o + 2] = __uint_as_float(dv.z);
    s_dh[c * DS + o + 3] = __uint_as_float(dv.w);
  }
  __syncthreads();
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int u0 = 0; u0 < U; u0 += kMxUB) {
    if (u0 > 0) {   // further experts (more than kMxUB planned)
#pragma unroll
      for (int j = 0; j < kMxUB; ++j) {
        ej[j] = (u0 + j < U) ? min(max(s_plan[kPlanIdOff + u0 + j], 0), a.E - 1) : 0;
        load_codebook<FMT>(a.cb_down + ((size_t)ej[j] << FMT), cb[j]);
        bl[j].load(a.down + (size_t)ej[j] * a.dn_stride + (size_t)rowc * a.dn_row_bytes, nb, blk);
      }
    }
#pragma unroll
    for (int j = 0; j < kMxUB; ++j) {
      const int u = u0 + j;
      if (has_group && u < U) {   // uniform
        const uint32_t mask = (uint32_t)s_plan[kPlanMaskOff + u];
        const bool live = i4 < Q && ((mask >> i4) & 1u);
        const int c = live ? s_cidx[u * 4 + i4] : 0;
        uint32_t w[8];
        bl[j].expand(0, cb[j], w);
        const u32x4 x0 = s_act[c * SS + 2 * blk], x1 = s_act[c * SS + 2 * blk + 1];
        const uint32_t xr[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        uint32_t xw[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) xw[k] = live ? xr[k] : 0u;
        const float wgt = live ? pw[4 * u + i4] : 0.0f;
        const v4i P4 = mfma4_block(w, xw);
        // (s_w * d_h) * routing weight, as k_downq
        const float sw = bl[j].scale(0), dht = s_dh[c * DS + blk];
        const float s0 = dpp_f32<0x00>(sw), s1 = dpp_f32<0x55>(sw), s2 = dpp_f32<0xAA>(sw), s3 = dpp_f32<0xFF>(sw);
        acc[0] = fmaf((float)P4[0], s0 * dht * wgt, acc[0]);
        acc[1] = fmaf((float)P4[1], s1 * dht * wgt, acc[1]);
        acc[2] = fmaf((float)P4[2], s2 * dht * wgt, acc[2]);
        acc[3] = fmaf((float)P4[3], s3 * dht * wgt, acc[3]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = sum_lane_bits2to5(acc[r]);
  if (lane < 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s_part[kq][rq][lane][r] = acc[r];
  }
  __syncthreads();
  if (tid < 64) {
    const int q4 = tid >> 4, t = (tid >> 2) & 3, r = tid & 3;
    const float v = ((s_part[0][q4][t][r] + s_part[1][q4][t][r]) + s_part[2][q4][t][r]) + s_part[3][q4][t][r];
    const int orow = blockIdx.x * 16 + 4 * q4 + r;
    if (t < Q && orow < a.hidden) a.out[(size_t)t * a.hidden + orow] = v;
  }
}

template <int FG, int FD, int Q>
int launch_decode_mfma_t(const DecodeArgs& a, hipStream_t s) {
  {
    const int nq = (a.q * a.nb_h + a.quant_per_wg - 1) / a.quant_per_wg;
    launch_kernel("route", k_route<Q>, dim3(a.E + nq), dim3(128 * Q), s, a);
  }
  int st = launch_check("route");
  if (st) return st;
  launch_kernel("gateup_mx", k_gateupm<FG, Q>, dim3(device_cu_count()), dim3(1024), s, a);
  if ((st = launch_check("gateup_mx"))) return st;
  launch_kernel("down_mx", k_downm<FD, Q>, dim3((a.hidden + 15) / 16), dim3(1024), s, a);
  return launch_check("down_mx");
}

template <int Q>
int launch_decode_mfma_q(const DecodeArgs& a, int fg, int fd, hipStream_t s) {
  if (fg == 2 && fd == 3) return launch_decode_mfma_t<2, 3, Q>(a, s);
  if (fg == 2 && fd == 2) return launch_decode_mfma_t<2, 2, Q>(a, s);
  if (fg == 2 && fd == 4) return launch_decode_mfma_t<2, 4, Q>(a, s);
  if (fg == 3 && fd == 3) return launch_decode_mfma_t<3, 3, Q>(a, s);
  if (fg == 3 && fd == 2) return launch_decode_mfma_t<3, 2, Q>(a, s);
  if (fg == 3 && fd == 4) return launch_decode_mfma_t<3, 4, Q>(a, s);
  if (fg == 4 && fd == 3) return launch_decode_mfma_t<4, 3, Q>(a, s);
  if (fg == 4 && fd == 2) return launch_decode_mfma_t<4, 2, Q>(a, s);
  return launch_decode_mfma_t<4, 4, Q>(a, s);
}

// ------------------------------------------------------------ prefill: experts with few pairs
// Experts that 1 .. kPrefillSmallPairs pairs of a prefill batch route to would
// fill an MFMA tile with padding; their pairs take the q <= 4 matvec arithmetic
// instead: each weight block is loaded and expanded once and dotted (sdot4)
// with every pair of the expert. Workgroup (x, y) serves listed expert y (those
// beyond the device-side count return at once); its pairs are the columns.
struct SmallArgs {
  DecodeArgs d;   // weights, codebooks, shapes, rot_down, dn_lpr_log2
  PrefillSmall p;
};

// 32 rows of gate and up per pass (8 waves x 4 rows, as gateup_item),
// kSmallGateupPasses passes per workgroup.
constexpr int kSmallGateupPasses = 2;
template <int FMT>
__global__ __launch_bounds__(512) void k_pf_gateup_small(SmallArgs sa) {
  constexpr int Q = kPrefillSmallPairs, RPW = 4;
  if ((int)blockIdx.y >= *sa.p.nsmall) return;
  const DecodeArgs& a = sa.d;
  const int e = sa.p.small[blockIdx.y];
  const int cnt = sa.p.counts[e], pbase = sa.p.offsets[e];
  const uint32_t mask = (1u << cnt) - 1u;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ float s_a[4][32];
  const int8_t* xcol[Q];
  const float* dcol[Q];
#pragma unroll
  for (int t = 0; t < Q; ++t) {   // unused columns repeat the last pair's row (masked out)
    const int tok = sa.p.pairs[pbase + min(t, cnt - 1)] / a.K;
    xcol[t] = sa.p.xq + (size_t)tok * a.nb_h * 32;
    dcol[t] = sa.p.dx + (size_t)tok * a.nb_h;
  }
  for (int pass = 0; pass < kSmallGateupPasses; ++pass) {
    const int rb = blockIdx.x * kSmallGateupPasses + pass;
    if (rb * 32 >= a.inter) break;   // uniform
    float ag[RPW][Q], au[RPW][Q];
    gateup_stream<FMT, Q, RPW>(a, e, mask, rb * 32 + wave * RPW, xcol, dcol, ag, au);
    gateup_wave_swiglu<Q, RPW>(mask, ag, au, s_a, wave * RPW);
    __syncthreads();
    // requantize the 32-row block of each pair: half-wave h of wave w takes column 2w + h
    if (wave < Q / 2) {
      const int t = 2 * wave + (lane >> 5), j = lane & 31;
      const bool act = t < cnt;
      float d;
      const uint32_t w = quant_block32_lanes(act ? s_a[t][j] : 0.0f, a.rot_down, &d);
      if (act) {
        const size_t pos = (size_t)(pbase + t);
        if ((j & 3) == 0) reinterpret_cast<uint32_t*>(sa.p.hq + pos * a.inter + (size_t)rb * 32)[j >> 2] = w;
        if (j == 0) sa.p.dh[pos * a.nb_i + rb] = d;
      }
    }
    __syncthreads();   // s_a is rewritten by the next pass
  }
}

// Down rows as k_down (lanes per row 2^dn_lpr_log2, NBL blocks per lane and
// pass), kSmallDownPasses row groups per workgroup; each block expanded once for
// all the expert's pairs.
constexpr int kSmallDownPasses = 8;
template <int FMT>
__global__ __launch_bounds__(256) void k_pf_down_small(SmallArgs sa) {
  constexpr int Q = kPrefillSmallPairs;
  constexpr int NBL = (FMT == 4) ? 1 : 2;
  if ((int)blockIdx.y >= *sa.p.nsmall) return;
  const DecodeArgs& a = sa.d;
  const int e = sa.p.small[blockIdx.y];
  const int cnt = sa.p.counts[e], pbase = sa.p.offsets[e];
  const int lpr_log2 = a.dn_lpr_log2, lpr = 1 << lpr_log2;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane >> lpr_log2, sl = lane & (lpr - 1);
  const int nb = a.nb_i;
  uint32_t cb[4];
  load_codebook<FMT>(a.cb_down + ((size_t)e << FMT), cb);
  // The expert's pairs' activations of the lane's blocks are the same for every
  // pass (row group), so they are loaded once per chunk, and every pass's weight
  // blocks are requested before any is used; each (row, pair) accumulates in
  // the same order as a pass-by-pass walk.
  constexpr int NP = kSmallDownPasses;
  float acc[NP][Q];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps)
#pragma unroll
    for (int t = 0; t < Q; ++t) acc[ps][t] = 0.0f;
  for (int c0 = 0; c0 < nb; c0 += lpr * NBL) {
    const int b = c0 + sl * NBL;
    const int bcl = min(b, nb - NBL);
    Acts<NBL> act[Q];
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const int pt = pbase + min(t, cnt - 1);   // (clamped: pairs past cnt are not used)
      act[t].load(sa.p.hq + (size_t)pt * a.inter, sa.p.dh + (size_t)pt * nb, bcl);
    }
    Blocks<FMT, NBL> bl[NP];
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
      const int row = ((blockIdx.x * NP + ps) * 4 + wave) * (64 >> lpr_log2) + sub;
      bl[ps].load(a.down + (size_t)e * a.dn_stride + (size_t)min(row, a.hidden - 1) * a.dn_row_bytes, nb, bcl);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
      const int row = ((blockIdx.x * NP + ps) * 4 + wave) * (64 >> lpr_log2) + sub;
      if (row < a.hidden && b < nb) {
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
          uint32_t w[8];
          bl[ps].expand(i, cb, w);
          const float sw = bl[ps].scale(i);
#pragma unroll
          for (int t = 0; t < Q; ++t)
            if (t < cnt) acc[ps][t] = fmaf((float)block_dot(w, act[t].q[i]), sw * act[t].d[i], acc[ps][t]);
        }
      }
    }
  }
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int row = ((blockIdx.x * NP + ps) * 4 + wave) * (64 >> lpr_log2) + sub;
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      const float v = group_sum(acc[ps][t], lpr);
      if (t < cnt && sl == 0 && row < a.hidden) {
        const int pair = sa.p.pairs[pbase + t];
        sa.p.ypair[(size_t)pair * a.hidden + row] = v * sa.p.gw[pair];
      }
    }
  }
}

template <int FG, int FD>
int launch_small_t(const SmallArgs& sa, hipStream_t s) {
  const DecodeArgs& a = sa.d;
  QMOE_BOUNDS((a.inter / 32 + kSmallGateupPasses - 1) / kSmallGateupPasses * kSmallGateupPasses * 32 >= a.inter,
              "prefill small path: gate/up grid covers the rows");
  QMOE_BOUNDS(a.dn_lpr_log2 >= 0 && a.dn_lpr_log2 <= 6, "prefill small path: down lanes per row");
  const int rb = a.inter / 32;
  launch_kernel("gateup_small", k_pf_gateup_small<FG>,
                dim3((rb + kSmallGateupPasses - 1) / kSmallGateupPasses, a.E), dim3(512), s, sa);
  int st = launch_check("gateup_small");
  if (st) return st;
  const int rows_per_wg = 4 * (64 >> a.dn_lpr_log2) * kSmallDownPasses;
  launch_kernel("down_small", k_pf_down_small<FD>, dim3((a.hidden + rows_per_wg - 1) / rows_per_wg, a.E), dim3(256),
                s, sa);
  return launch_check("down_small");
}

}  // namespace

namespace qmoe {

int launch_prefill_small(const PrefillSmall& p, hipStream_t s) {
  const qmoe_layer* L = p.L;
  FormatInfo fg, fd;
  format_info(L->fmt_gate, &fg);
  format_info(L->fmt_down, &fd);
  SmallArgs sa{};
  DecodeArgs& a = sa.d;
  a.gate = static_cast<const uint8_t*>(L->gate);
  a.up = static_cast<const uint8_t*>(L->up);
  a.down = static_cast<const uint8_t*>(L->down);
  a.cb_gate = L->cb_gate;
  a.cb_up = L->cb_up;
  a.cb_down = L->cb_down;
  a.hidden = L->hidden;
  a.inter = L->inter;
  a.E = L->n_experts;
  a.K = L->topk;
  a.rot_down = L->rot_down;
  a.nb_h = L->hidden / 32;
  a.nb_i = L->inter / 32;
  a.gu_row_bytes = (size_t)a.nb_h * fg.block_bytes;
  a.gu_stride = a.gu_row_bytes * L->inter;
  a.dn_row_bytes = (size_t)a.nb_i * fd.block_bytes;
  a.dn_stride = a.dn_row_bytes * L->hidden;
  a.dn_lpr_log2 = ilog2(lanes_per_row(a.nb_i, L->fmt_down == QMOE_FP4 ? 1 : 2));
  sa.p = p;
  const int g = L->fmt_gate, d = L->fmt_down;
  if (g == 2 && d == 3) return launch_small_t<2, 3>(sa, s);
  if (g == 2 && d == 2) return launch_small_t<2, 2>(sa, s);
  if (g == 2 && d == 4) return launch_small_t<2, 4>(sa, s);
  if (g == 3 && d == 3) return launch_small_t<3, 3>(sa, s);
  if (g == 3 && d == 2) return launch_small_t<3, 2>(sa, s);
  if (g == 3 && d == 4) return launch_small_t<3, 4>(sa, s);
  if (g == 4 && d == 3) return launch_small_t<4, 3>(sa, s);
  if (g == 4 && d == 2) return launch_small_t<4, 2>(sa, s);
  return launch_small_t<4, 4>(sa, s);
}

}  // namespace qmoe

namespace {

// Checks the arguments of a decode call and fills the kernels' argument block.
int decode_setup(const qmoe_layer* L, const float* x, int32_t q, float* out, void* ws, size_t ws_bytes,
                 DecodeArgs& a, int& U_max) {
  if (q < 1 || q > 4) QMOE_FAIL(QMOE_E_SHAPE, "q=%d outside 1..4", q);
  WsPtrs w;
  int st = ws_ptrs(L, q, ws, ws_bytes, &w);
  if (st) return st;
  if (!x || !out) QMOE_FAIL(QMOE_E_INVAL, "NULL pointer");
  if (!aligned16(x)) QMOE_FAIL(QMOE_E_INVAL, "x not 16-byte aligned");
  FormatInfo fg, fd;
  format_info(L->fmt_gate, &fg);
  format_info(L->fmt_down, &fd);
  a = DecodeArgs{};
  a.w_router = L->w_router;
  a.bias = L->router_bias;
  a.gate = static_cast<const uint8_t*>(L->gate);
  a.up = static_cast<const uint8_t*>(L->up);
  a.down = static_cast<const uint8_t*>(L->down);
  a.cb_gate = L->cb_gate;
  a.cb_up = L->cb_up;
  a.cb_down = L->cb_down;
  a.x = x;
  a.out = out;
  a.xq = w.xq;
  a.dx = w.dx;
  a.logits = w.logits;
  a.idx = w.idx;
  a.gw = w.gw;
  a.plan = w.plan;
  a.hq = w.hq;
  a.dh = w.dh;
  a.hidden = L->hidden;
  a.inter = L->inter;
  a.E = L->n_experts;
  a.K = L->topk;
  a.q = q;
  a.rot_gateup = L->rot_gateup;
  a.rot_down = L->rot_down;
  a.nb_h = L->hidden / 32;
  a.nb_i = L->inter / 32;
  a.gu_row_bytes = (size_t)a.nb_h * fg.block_bytes;
  a.gu_stride = a.gu_row_bytes * L->inter;
  a.dn_row_bytes = (size_t)a.nb_i * fd.block_bytes;
  a.dn_stride = a.dn_row_bytes * L->hidden;
  a.dn_lpr_log2 = ilog2(lanes_per_row(a.nb_i, L->fmt_down == QMOE_FP4 ? 1 : 2));
  a.quant_per_wg = 4 * q;   // blocks per token-quantization workgroup: one pass of its half-waves
  U_max = std::min(q * L->topk, L->n_experts);
  {   // the extents the decode kernels address (slot = 4 u + t for plan slot u, column t)
    const size_t maxslot = (size_t)(U_max - 1) * 4 + (q - 1);
    QMOE_BOUNDS((size_t)q * a.hidden <= w.n_xq && (size_t)q * a.nb_h * 4 <= w.n_dx, "decode: quantized tokens");
    QMOE_BOUNDS((size_t)q * a.E * 8 <= w.n_logits, "decode: logits");
    QMOE_BOUNDS((size_t)q * a.K * 4 <= w.n_idx && (size_t)q * a.K * 4 <= w.n_gw, "decode: routing ids and weights");
    QMOE_BOUNDS(U_max <= kPlanMax && (size_t)(kPlanWOff + 4 * kPlanMax) * 4 <= w.n_plan, "decode: plan");
    QMOE_BOUNDS((maxslot + 1) * a.inter <= w.n_hq && (maxslot + 1) * a.nb_i * 4 <= w.n_dh,
                "decode: requantized intermediate rows");
    QMOE_BOUNDS(a.inter % 32 == 0 && 4 * (64 >> a.dn_lpr_log2) > 0, "decode: gate/up row blocks, down rows per group");
  }
  return QMOE_OK;
}

}  // namespace

extern "C" int qmoe_decode_layer(const qmoe_layer* L, const float* x, int32_t q, float* out, void* ws,
                                 size_t ws_bytes, void* stream) {
  clear_error();
  DecodeArgs a;
  int U_max = 0;
  int st = decode_setup(L, x, q, out, ws, ws_bytes, a, U_max);
  if (st) return st;
  hipStream_t s = as_stream(stream);
  switch (q) {
    case 1: return launch_decode_q<1>(a, U_max, L->fmt_gate, L->fmt_down, s);
    case 2: return launch_decode_q<2>(a, U_max, L->fmt_gate, L->fmt_down, s);
    case 3: return launch_decode_q<3>(a, U_max, L->fmt_gate, L->fmt_down, s);
    default: return launch_decode_q<4>(a, U_max, L->fmt_gate, L->fmt_down, s);
  }
}

extern "C" int qmoe_decode_layer_mfma(const qmoe_layer* L, const float* x, int32_t q, float* out, void* ws,
                                      size_t ws_bytes, void* stream) {
  clear_error();
  DecodeArgs a;
  int U_max = 0;
  int st = decode_setup(L, x, q, out, ws, ws_bytes, a, U_max);
  if (st) return st;
  if (a.nb_h % 16 != 0 || a.nb_h > kMxMaxNbH)
    QMOE_FAIL(QMOE_E_SHAPE, "matrix-core decode: hidden=%d must be a multiple of 512 and at most %d", a.hidden,
              32 * kMxMaxNbH);
  if (a.nb_i % 16 != 0 || a.nb_i > kMxMaxNbI)
    QMOE_FAIL(QMOE_E_SHAPE, "matrix-core decode: inter=%d must be a multiple of 512 and at most %d", a.inter,
              32 * kMxMaxNbI);
  if (q * a.K > kDownqMaxSlots || (int64_t)q * a.K * (2 * a.nb_i + 1) * 16 > kDownmActBytes)
    QMOE_FAIL(QMOE_E_SHAPE, "matrix-core decode: q * topk = %d routed slots of %d blocks exceed the down "
              "kernel's LDS", q * a.K, a.nb_i);
  QMOE_BOUNDS((int64_t)((a.hidden + 15) / 16) * 16 >= a.hidden && a.inter % 32 == 0,
              "matrix-core decode: down grid covers the rows, gate/up items of 32 rows");
  hipStream_t s = as_stream(stream);
  switch (q) {
    case 1: return launch_decode_mfma_q<1>(a, L->fmt_gate, L->fmt_down, s);
    case 2: return launch_decode_mfma_q<2>(a, L->fmt_gate, L->fmt_down, s);
    case 3: return launch_decode_mfma_q<3>(a, L->fmt_gate, L->fmt_down, s);
    default: return launch_decode_mfma_q<4>(a, L->fmt_gate, L->fmt_down, s);
  }
}
