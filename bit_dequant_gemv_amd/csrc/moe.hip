// Sparse-MoE expert decode: router, top-k, grouped gate_up + SwiGLU,
// grouped down + router-weighted combine (+ RMSNorm residual stack).
//
// Per layer the pages run a router and then the chosen experts one after
// another, two small GEMVs each, one submission per GEMV ("Sovereign
// gpt-oss-20B (MXFP4) on Apple Silicon", section 3: "4 sequential experts x
// 2 small-block GEMVs", dispatch-bound); running the active experts together
// is named there as the untried lever (section 5), and the TinyTitan tracker
// moves a layer's experts into one submission (entry D114).  Here a layer is
// two kernels on the per-token path (three for steps of M > 1), each over
// ALL chosen experts of the layer:
//   route  : the router GEMV (one router row per wavefront) and the input's
//            sum of squares, as one slice of router partial sums; it runs
//            for steps of M > 1 (where it also forms the layer input from
//            the previous layer's per-pick down outputs), and on the
//            per-token path only with BDG_MOE_ROUTE_KERNEL or the fused
//            per-layer kernel;
//   gate_up: adds the router slices (or, in a layer whose router no down
//            kernel carries, computes the router rows itself: SelfRoute),
//            applies the RMSNorm scale and bias, and every wavefront
//            computes the top-k + softmax itself; it issues the loads of
//            all its (g, u) row pairs at once, then stages x and runs the
//            grouped dequant-GEMV of all k experts with the SwiGLU epilogue
//            h = silu(g) * u;
//   down   : one block per row block, waves split over the chosen experts:
//            grouped dequant-GEMV over h, then the router-weighted combine
//            and the residual add in LDS, in a fixed expert order; in a
//            stack it also writes the next layer's router slice for its
//            rows, which saves that layer's route kernel.
// A whole token is one captured HIP graph (the per-token setup amortised as
// in the host-sync page, section 3).
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <type_traits>

#include "bdg_host.hpp"
#include "bdg_moe.hpp"
#include "bdg_moe_down.hpp"
#include "bdg_moe_layer.hpp"
#include "bdg_moe_mfma.hpp"

namespace bdg {

// ---------------------------------------------------------------- route

// The route kernel writes slice 0 of the router partial sums (see
// bdg_moe.hpp) for the layer input, and for grouped steps forms that input.

struct RouteParams {
  int M, H, E;
  int compute_logits;
  const void* x_in;   // [M][H] layer input: caller x (bf16/f32) at layer 0, else the residual buffer
  int x_bf16;
  float* x_copy;      // [M][H] fp32 copy of x_in written by block 0 (layer 0), or NULL
  float* resid_trace; // [M][H] or NULL, written by block 0
  float* part;        // [M][E + 1][pstride]: slice 0 written
  int pstride;
  // combine (grouped path): the layer input is (x_in when combine_residual,
  // else 0) + sum_j wts[t][j] * dout[t*K + j], j in order
  const float* dout;  // [M * K][H] previous layer's down output per pick, or NULL
  const float* wts;   // [M][K]
  int K;
  int combine_residual;
  LayerDev L;         // this layer's weights (a kernel argument: no dependent table load)
  // the matrix-core path's operands (written by block 0, or NULL): the layer
  // input times its RMSNorm factor (1 without norm or logits) as bf16 parts
  uint16_t* xh;       // [M][H] hi = bf16(v)
  uint16_t* xl;       // [M][H] lo = bf16(v - hi)
  int norm;
  float eps;
  unsigned* seq;      // or NULL: the token sequence number, advanced by block (0, 0)
};

// One router row per wavefront; block b handles rows 4b .. 4b+3 of token t.
// Used when the layer input has to be formed first (the combine of a grouped
// step) or when no logits are wanted (only the fp32 copy of x): the input is
// built once per block in LDS and shared by the block's four rows.
__global__ void __launch_bounds__(kThreads) moe_route_kernel(RouteParams p) {
  extern __shared__ float lds[];
  float* xs = lds;               // [H]
  const int t = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  const int e = blockIdx.x * kWaves + wave;
  const bool row_ok = p.compute_logits && e < p.E;
  const LayerDev& L = p.L;

  // the router row first: its loads do not depend on x
  // in-bounds clamped addresses, loads issued unconditionally; entries past
  // the row end (h >= H) are never used
  const int ec = e < p.E ? e : p.E - 1;
  float4 wv[kRouteMaxF4];
#pragma unroll
  for (int i = 0; i < kRouteMaxF4; ++i) {
    const int h = (i * kWave + lane) * 4;
    wv[i] = ldg_f4(L.w_r + (int64_t)ec * p.H + (h < p.H ? h : p.H - 4));
  }
  const int64_t xoff = (int64_t)t * p.H;
  constexpr int NX = kRouteMaxF4 * kWave / kThreads;   // float4 of x per thread (H <= 4096)
  float4 xv4[NX];
  uint2 xb[NX];
  if (p.x_bf16) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int h = (i * kThreads + threadIdx.x) * 4;
      xb[i] = ldg_u64(reinterpret_cast<const uint16_t*>(p.x_in) + xoff + (h < p.H ? h : p.H - 4));
    }
#pragma unroll
    for (int i = 0; i < NX; ++i)
      xv4[i] = make_float4(bf16_to_f32((uint16_t)(xb[i].x & 0xFFFFu)), bf16_to_f32((uint16_t)(xb[i].x >> 16)),
                           bf16_to_f32((uint16_t)(xb[i].y & 0xFFFFu)), bf16_to_f32((uint16_t)(xb[i].y >> 16)));
  } else {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int h = (i * kThreads + threadIdx.x) * 4;
      xv4[i] = ldg_f4(reinterpret_cast<const float*>(p.x_in) + xoff + (h < p.H ? h : p.H - 4));
    }
  }
  if (p.dout) {
    if (!p.combine_residual) {
#pragma unroll
      for (int i = 0; i < NX; ++i) xv4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int j = 0; j < p.K; ++j) {
      const float wj = p.wts[t * p.K + j];
      const float* dj = p.dout + ((int64_t)t * p.K + j) * p.H;
      float4 d[NX];
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const int h = (i * kThreads + threadIdx.x) * 4;
        d[i] = ldg_f4(dj + (h < p.H ? h : p.H - 4));
      }
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        xv4[i].x = __builtin_fmaf(wj, d[i].x, xv4[i].x);
        xv4[i].y = __builtin_fmaf(wj, d[i].y, xv4[i].y);
        xv4[i].z = __builtin_fmaf(wj, d[i].z, xv4[i].z);
        xv4[i].w = __builtin_fmaf(wj, d[i].w, xv4[i].w);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int h = (i * kThreads + threadIdx.x) * 4;
    if (h < p.H) {
      const float4 v = xv4[i];
      *reinterpret_cast<float4*>(xs + h) = v;
      if (blockIdx.x == 0) {
        if (p.x_copy) *reinterpret_cast<float4*>(p.x_copy + xoff + h) = v;
        if (p.resid_trace) *reinterpret_cast<float4*>(p.resid_trace + xoff + h) = v;
      }
    }
  }
  __syncthreads();
  if (p.compute_logits && blockIdx.x == 0 && wave == 0) {
    // sum of squares in the lane order of moe_route_direct_kernel (same value)
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kRouteMaxF4; ++i) {
      const int h = (i * kWave + lane) * 4;
      if (h < p.H) {
        const float4 v = *reinterpret_cast<const float4*>(xs + h);
        ss = __builtin_fmaf(v.x, v.x, ss);
        ss = __builtin_fmaf(v.y, v.y, ss);
        ss = __builtin_fmaf(v.z, v.z, ss);
        ss = __builtin_fmaf(v.w, v.w, ss);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) p.part[((int64_t)t * (p.E + 1) + p.E) * p.pstride] = ss;
    // the RMSNorm factor as the gate_up kernels compute it from this sum
    if (lane == 0) xs[p.H] = (p.norm ? 1.0f / sqrtf(ss / (float)p.H + p.eps) : 1.0f);
  }
  if (p.xh && blockIdx.x == 0) {   // block-uniform
    __syncthreads();
    const float r = p.compute_logits ? xs[p.H] : 1.0f;
    for (int h = threadIdx.x * 4; h < p.H; h += kThreads * 4) {
      const float4 v = *reinterpret_cast<const float4*>(xs + h);
      const float vv[4] = {v.x * r, v.y * r, v.z * r, v.w * r};
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = f32_to_bf16_rne(vv[i]);
        lo[i] = f32_to_bf16_rne(vv[i] - bf16_to_f32(hi[i]));
      }
      *reinterpret_cast<uint2*>(p.xh + xoff + h) = make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
      *reinterpret_cast<uint2*>(p.xl + xoff + h) = make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
    }
  }
  if (!row_ok) return;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kRouteMaxF4; ++i) {
    const int h = (i * kWave + lane) * 4;
    if (h < p.H) {
      const float4 xv = *reinterpret_cast<const float4*>(xs + h);
      acc = __builtin_fmaf(wv[i].x, xv.x, acc);
      acc = __builtin_fmaf(wv[i].y, xv.y, acc);
      acc = __builtin_fmaf(wv[i].z, xv.z, acc);
      acc = __builtin_fmaf(wv[i].w, xv.w, acc);
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) p.part[((int64_t)t * (p.E + 1) + e) * p.pstride] = acc;
}

// The same for the plain case (no combine): one wavefront per router row,
// one block per row (grid (E, M)), x read straight into registers in the
// row's lane layout (float4 i of lane l covers x[4(64i + l) .. +3]), so there
// is no LDS staging and no barrier.  The wave of row 0 also writes the sum of
// squares and, when asked, the fp32 copy and trace of x.  NF float4 per lane
// cover H <= 256 NF.
template <int NF>
__global__ void __launch_bounds__(kWave) moe_route_direct_kernel(RouteParams p) {
  const int e = blockIdx.x;
  const int t = blockIdx.y;
  const int lane = threadIdx.x;
  const float* wr = p.L.w_r + (int64_t)e * p.H;
  const int64_t xoff = (int64_t)t * p.H;
  float4 wv[NF], xv[NF];
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int h = (i * kWave + lane) * 4;
    wv[i] = ldg_f4(wr + (h < p.H ? h : p.H - 4));
  }
  if (p.x_bf16) {
    uint2 xb[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int h = (i * kWave + lane) * 4;
      xb[i] = ldg_u64(reinterpret_cast<const uint16_t*>(p.x_in) + xoff + (h < p.H ? h : p.H - 4));
    }
#pragma unroll
    for (int i = 0; i < NF; ++i)
      xv[i] = make_float4(bf16_to_f32((uint16_t)(xb[i].x & 0xFFFFu)), bf16_to_f32((uint16_t)(xb[i].x >> 16)),
                          bf16_to_f32((uint16_t)(xb[i].y & 0xFFFFu)), bf16_to_f32((uint16_t)(xb[i].y >> 16)));
  } else {
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int h = (i * kWave + lane) * 4;
      xv[i] = ldg_f4(reinterpret_cast<const float*>(p.x_in) + xoff + (h < p.H ? h : p.H - 4));
    }
  }
  float acc, ss;
  router_lane_sums<NF>(wv, xv, p.H, lane, acc, ss);
  acc = wave_sum(acc);
  float* prow = p.part + (int64_t)t * (p.E + 1) * p.pstride;
  if (lane == 0) prow[(int64_t)e * p.pstride] = acc;
  // a stack whose later layers route themselves: this launch starts a new
  // token (its sequence number tags those layers' router sums)
  if (p.seq && e == 0 && t == 0 && lane == 0)
    __hip_atomic_fetch_add(p.seq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (e == 0) {
    ss = wave_sum(ss);
    if (lane == 0) prow[(int64_t)p.E * p.pstride] = ss;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int h = (i * kWave + lane) * 4;
      if (h < p.H) {
        if (p.x_copy) *reinterpret_cast<float4*>(p.x_copy + xoff + h) = xv[i];
        if (p.resid_trace) *reinterpret_cast<float4*>(p.resid_trace + xoff + h) = xv[i];
      }
    }
  }
}

// ---------------------------------------------------------------- gate_up + SwiGLU

struct GateUpParams {
  int M, H, I, E, K;
  RouteSrc rt;                // routing inputs (partial router sums, or the caller's routing)
  int32_t* idx_out;           // [M][K] routing buffer, written by block 0
  float* w_out;
  int32_t* topk_trace;        // [M][K] or NULL
  float* wts_trace;
  const float* x;             // [M][H] layer input: fp32, or the caller's bf16 bits (SR == 2)
  LayerDev L;                 // this layer's weights
  QGeom g;                    // reduction over H
  float* h_out;               // [M][K][I]
  SelfRoute sr;               // self-routing launches (SR != 0): router rows, tags, the wait
};

// Wave gw of token t owns the (expert slot, row pair) range
// [P*gw/GW, P*(gw+1)/GW) of the P = K*I pairs; the grid makes it <= NP.
// Lanes 0..31 compute the gate row i, lanes 32..63 the up row I+i.
// SR != 0: the launch computes the layer's router itself (see SelfRoute):
// wave w of block b < sr.blocks takes router row 4b + w of token t, and wave
// 0 of every block waits for the token's tagged logits; the routing rule and
// its arithmetic are the route kernel's, so the selection is bit for bit the
// same.  SR == 2: the input is the caller's bf16 x (the first layer), widened
// exactly to fp32 as the route kernel's copy of it would be.
template <int FMT, int S, int NP, int V, int SR>
__global__ void __launch_bounds__(kThreads) moe_gateup_kernel(GateUpParams p) {
  constexpr bool kSR = SR != 0;
  constexpr bool kXBF = SR == 2;
  constexpr int L = 32;
  extern __shared__ float lds[];
  float* xs = lds;                                          // [(chunks + 1) * kXStride], chunk `chunks` zero
  float* red = xs + (p.g.chunks + 1) * kXStride;            // [kWaves]
  float* psum = red + kWaves;                               // [E << log2T]
  const int t = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  const int li = lane % L;
  const bool is_up = lane >= L;
  const LayerDev& Ld = p.L;

  // load order: routing inputs, then x (independent of the routing), then
  // the expert weights - the in-order wait for each stays short
  RouteState<V> rs;
  constexpr int RNF = kSR ? kSelfRouteNF : 1;
  float4 rw[RNF], rx[RNF];
  uint2 rxb[kXBF ? RNF : 1];   // bf16 input: the raw words, widened where they are used
  unsigned tag = 0;
  int re = 0;
  bool router_wave = false;
  if constexpr (kSR) {
    // the router rows this wave computes come first: the wait below
    // depends on them
    tag = __hip_atomic_load(p.sr.seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + p.sr.tag_add;
    re = blockIdx.x * kWaves + wave;
    router_wave = (int)blockIdx.x < p.sr.blocks && re < p.E;
    if (router_wave) {
      const float* wr = Ld.w_r + (int64_t)re * p.H;
#pragma unroll
      for (int i = 0; i < RNF; ++i) {
        const int h = (i * kWave + lane) * 4;
        rw[i] = ldg_f4(wr + (h < p.H ? h : p.H - 4));
      }
      if constexpr (kXBF) {
        const uint16_t* xb = reinterpret_cast<const uint16_t*>(p.x) + (int64_t)t * p.H;
#pragma unroll
        for (int i = 0; i < RNF; ++i) {
          const int h = (i * kWave + lane) * 4;
          rxb[i] = ldg_u64(xb + (h < p.H ? h : p.H - 4));
        }
      } else {
        const float* xr = p.x + (int64_t)t * p.H;
#pragma unroll
        for (int i = 0; i < RNF; ++i) {
          const int h = (i * kWave + lane) * 4;
          rx[i] = ldg_f4(xr + (h < p.H ? h : p.H - 4));
        }
      }
    }
    rs.ssq = 0.f;
    rs.my_e = 0;
    rs.my_w = 0.f;
    rs.r = 1.f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = lane + kWave * i;
      rs.bias[i] = p.rt.b_r ? p.rt.b_r[e < p.E ? e : p.E - 1] : 0.f;
    }
  } else {
    route_issue<V, kThreads>(rs, p.rt, t, lane);
  }
  constexpr int NX = kRouteMaxF4 * kWave / kThreads;   // H <= 4096
  std::conditional_t<kXBF, StageBF16<NX>, StageF32<NX>> xstage;
  if constexpr (kXBF)
    xstage.load(reinterpret_cast<const uint16_t*>(p.x) + (int64_t)t * p.H, p.H, threadIdx.x, kThreads);
  else
    xstage.load(p.x + (int64_t)t * p.H, p.H, threadIdx.x, kThreads);

  // this wave's pair range (independent of the routing: computed while the
  // routing inputs are in flight)
  const int P = p.K * p.I;
  const int GW = gridDim.x * kWaves;
  const int gw = blockIdx.x * kWaves + wave;
  const int q0 = (int)((int64_t)P * gw / GW);
  const int q1 = (int)((int64_t)P * (gw + 1) / GW);
  const int nq = q1 - q0;                 // <= NP pairs for this wave
  // (slot, row) of q0; later pairs step the row and wrap to the next slot
  const int j0 = q0 / p.I;
  const int row0 = q0 - j0 * p.I;

  float poison = 0.f;   // 1 after a self-routing wait gave up: h is NaN
  if constexpr (kSR) {
    if (router_wave) {
      if constexpr (kXBF) {
#pragma unroll
        for (int i = 0; i < RNF; ++i)
          rx[i] = make_float4(bf16_to_f32((uint16_t)(rxb[i].x & 0xFFFFu)), bf16_to_f32((uint16_t)(rxb[i].x >> 16)),
                              bf16_to_f32((uint16_t)(rxb[i].y & 0xFFFFu)), bf16_to_f32((uint16_t)(rxb[i].y >> 16)));
      }
      float acc, ss;
      router_lane_sums<RNF>(rw, rx, p.H, lane, acc, ss);
      acc = wave_sum(acc);
      unsigned long long* lrow = p.sr.log + (int64_t)t * (p.E + 1);
      if (lane == 0) __hip_atomic_store(lrow + re, tagged(tag, acc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (re == 0) {
        ss = wave_sum(ss);
        if (lane == 0) __hip_atomic_store(lrow + p.E, tagged(tag, ss), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the layer input's trace and (first layer) its fp32 copy
#pragma unroll
        for (int i = 0; i < RNF; ++i) {
          const int h = (i * kWave + lane) * 4;
          if (h < p.H) {
            if (p.sr.resid_trace) *reinterpret_cast<float4*>(p.sr.resid_trace + (int64_t)t * p.H + h) = rx[i];
            if (p.sr.x_copy) *reinterpret_cast<float4*>(p.sr.x_copy + (int64_t)t * p.H + h) = rx[i];
          }
        }
      }
    }
    if (wave == 0) self_route_wait<V>(p.sr, t, p.E, tag, lane, psum, red);
    block_sync_lds();
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = lane + kWave * i;
      rs.lg[i] = psum[e < p.E ? e : p.E - 1];
    }
    rs.ssq = red[0];
    poison = red[1];
  }
  route_finish<V, kThreads>(rs, p.rt, t, lane, wave, red, psum);
  const int my_e = rs.my_e;
  const float my_w = rs.my_w;
  const float mult = rs.r;
  if (blockIdx.x == 0 && wave == 0 && lane < p.K) {
    p.idx_out[t * p.K + lane] = my_e;
    p.w_out[t * p.K + lane] = my_w;
    if (p.topk_trace) p.topk_trace[t * p.K + lane] = my_e;
    if (p.wts_trace) p.wts_trace[t * p.K + lane] = my_w;
  }

  // every slot loads (a wave short of NP pairs repeats its last pair and
  // stores nothing for the repeats): no branch around the loads
  GroupLoad<FMT, S> ld[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int ii = i < nq ? i : (nq > 0 ? nq - 1 : 0);
    int row = row0 + ii;
    int j = j0;
    while (row >= p.I) {                  // NP <= I: at most one wrap in practice
      row -= p.I;
      ++j;
    }
    if (j >= p.K) j = p.K - 1;
    const int e = __builtin_amdgcn_readlane(my_e, j);
    load_row<FMT, L, S>(ld[i], expert_gu(Ld, e), p.g, is_up ? p.I + row : row, true, li);
  }

  xstage.store(xs, p.H, p.H, 0, mult, threadIdx.x, kThreads);
  xs[p.g.chunks * kXStride + (threadIdx.x & (kChunkElems - 1))] = 0.f;   // the zero chunk (no branch)
  block_sync_lds();   // weights still in flight: each pair's dot waits for its own rows only
  XRegs<FMT, L, S> xr;
  xr.load_zpad(xs, p.g.chunks, li);

  // pair i: lanes 0..31 hold the gate row's dot g_i, lanes 32..63 the up
  // row's u_i; lane i gathers (g_i, u_i) and SwiGLU runs once per wave
  float g_sel = 0.f, u_sel = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const float d = row_dot<FMT, L, S>(ld[i], xr);
    const float gv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), kRowSumLane<L>));
    const float uv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), L + kRowSumLane<L>));
    if (lane == i) {
      g_sel = gv;
      u_sel = uv;
    }
  }
  if (lane < nq) {
    float hv = g_sel / (1.0f + expf(-g_sel)) * u_sel;
    if constexpr (kSR) hv = poison != 0.f ? __uint_as_float(0x7FC00000u) : hv;
    p.h_out[(int64_t)t * P + q0 + lane] = hv;
  }
}

// ---------------------------------------------------------------- grouped path (M > 1)
//
// With several tokens per step, tokens share experts (the 120B small-M
// workload reads ~36 distinct experts for 64 picks at M = 16).  The grouped
// path reads each chosen (layer, expert) matrix once per step: every gate_up
// block routes all M tokens and builds the same deterministic list of
// "chunks" - one expert and up to kGroupTT of its picks (token, slot) - then
// the blocks share the (chunk, row block) items of the layer; the weights of
// an item are loaded once and applied to all of its picks (MXFP4: in one
// pass, each code chunk decoded once for every pick; int4: one pick per
// pass).  The
// down kernel does the same over the chunk table gate_up wrote, and writes one
// output row per pick; the weighted combine with the residual then happens
// in the next layer's route kernel (or a final combine kernel), in slot
// order, with the same arithmetic as the per-token down kernel.

constexpr int kGroupTT = 2;           // picks per chunk

// f(std::integral_constant<int, n>{}) for a runtime n in [1, N]: one
// unrolled instantiation per count.
template <int N, class F>
__device__ __forceinline__ void with_count(int n, F&& f) {
  if constexpr (N > 1) {
    if (n == N) {
      f(std::integral_constant<int, N>{});
      return;
    }
    with_count<N - 1>(n, f);
  } else {
    f(std::integral_constant<int, 1>{});
  }
}

// (g, u) row pairs per wave in the grouped gate_up, and down rows per wave:
// as many as fit 256 VGPRs with the loaded rows held across a chunk's picks.
__host__ __device__ constexpr int gu_group_np(int fmt, int S) {
  return fmt == 0 ? (S <= 3 ? 6 : 4) : (S <= 2 ? 6 : 4);
}
__host__ __device__ constexpr int dn_group_nr(int fmt, int L, int S) {
  return (kWave / L <= 2 && (fmt == 0 || L * S < 96)) ? 4 : 2;
}
constexpr int kChunkInts = 2 + kGroupTT;
using GroupLds = GroupLdsT<kGroupTT>;

struct GroupParams {
  int M, H, I, E, K;
  int routed;                 // 1: routing given in idx_in / w_in
  const float* part;          // [M][E + 1][pstride] router sums, one slice (route kernel)
  int pstride;
  int norm;
  float eps;
  const int32_t* idx_in;
  const float* w_in;
  int32_t* idx_out;           // [M][K]
  float* w_out;
  int32_t* topk_trace;        // [M][K] or NULL
  float* wts_trace;
  const float* x;             // [M][H] layer input (fp32)
  LayerDev L;
  QGeom g;                    // reduction over H
  float* h_out;               // [M * K][I], row p = t*K + j
  int32_t* chunks_out;        // chunk table for the down kernel, written by block 0
  int bpc;                    // row blocks per chunk (a multiple of 8)
};

__host__ __device__ constexpr size_t group_lds_floats() { return (sizeof(GroupLds) + 15) / 16 * 4; }

// Persistent grid: block b takes items b, b + G, ... of the chunks x row
// blocks of the layer (a row block = kWaves * NP (g, u) row pairs).  Items of
// one row block in consecutive chunks are bpc apart, bpc % 8 == 0, so with
// G % 8 == 0 they run on one XCD (blocks are dealt to the 8 XCDs in turn)
// and share its L2 when a hot expert spans several chunks.
template <int FMT, int S, int NP, int V>
__global__ void __launch_bounds__(kThreads, 2) moe_gu_group_kernel(GroupParams p) {
  constexpr int L = 32;
  constexpr bool kMulti = FMT == kMXFP4;                // all picks per pass (int4: one pick per pass)
  constexpr int NX = S;                                 // H <= 32 * L * S: float4 of x per thread
  extern __shared__ float lds[];
  GroupLds& gl = *reinterpret_cast<GroupLds*>(lds);
  float* xs = lds + group_lds_floats();                 // [kGroupTT][(chunks + 1) * kXStride]
  const int xstride = (p.g.chunks + 1) * kXStride;      // each input: chunks, then a zero chunk
  // the zero chunks (staging never writes them; the first item's barrier
  // orders these stores before any read); no branch
  xs[min((int)(threadIdx.x / kChunkElems), kGroupTT - 1) * xstride + p.g.chunks * kXStride +
     (threadIdx.x & (kChunkElems - 1))] = 0.f;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  const int li = lane % L;
  const bool is_up = lane >= L;
  const LayerDev& Ld = p.L;
  const int P = p.M * p.K;

  // routing of every token of the step and the chunk table (block 0 writes
  // it for the down kernel)
  group_route<V, kGroupTT>(gl, p, lane, wave, kWaves);
  if (blockIdx.x == 0) write_chunk_table(gl, p.chunks_out, kThreads);

  const int nitems = gl.n * p.bpc;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int c = item / p.bpc;
    const int r0 = (item - c * p.bpc) * (kWaves * NP);
    if (r0 >= p.I) continue;                              // block-uniform
    const int e = gl.ce[c];
    const int nt = __builtin_amdgcn_readfirstlane(gl.cn[c]);   // block-uniform: one path per chunk
    // the picks' inputs first, then the expert weights (vmcnt retires in order)
    StageF32<NX> xst[kGroupTT];
#pragma unroll
    for (int k = 0; k < kGroupTT; ++k)
      if (k < nt) xst[k].load(p.x + (int64_t)(gl.cpk[c][k] / p.K) * p.H, p.H, threadIdx.x, kThreads);
    const int rw = r0 + wave * NP;                        // this wave's first pair
    const QMat wm = expert_gu(Ld, e);
    GroupLoad<FMT, S> ld[NP];
    if constexpr (kMulti) {
#pragma unroll
      for (int i = 0; i < NP; ++i) ld[i].ok = ld[i].zhi = 0;
#pragma unroll
      for (int s = 0; s < S; ++s)                         // slot-major, the order rows_dot_multi takes them
#pragma unroll
        for (int i = 0; i < NP; ++i)
          load_row_slot<FMT, L, S>(ld[i], wm, p.g, is_up ? p.I + rw + i : rw + i, rw + i < p.I, li, s);
    } else {
#pragma unroll
      for (int i = 0; i < NP; ++i)
        load_row<FMT, L, S>(ld[i], wm, p.g, is_up ? p.I + rw + i : rw + i, rw + i < p.I, li);
    }
    block_sync_lds();                                     // the previous item's x reads are done
#pragma unroll
    for (int k = 0; k < kGroupTT; ++k)
      if (k < nt) xst[k].store(xs + k * xstride, p.H, p.H, 0, gl.rt[gl.cpk[c][k] / p.K], threadIdx.x, kThreads);
    block_sync_lds();                                     // weights still in flight
    const int nq = min(max(p.I - rw, 0), NP);
    // (g, u) of pair i to lane i, SwiGLU there, h of pick k stored
    auto finish = [&](const float (&d)[NP], int k) {
      float g_sel = 0.f, u_sel = 0.f;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const float gv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d[i]), kRowSumLane<L>));
        const float uv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d[i]), L + kRowSumLane<L>));
        if (lane == i) {
          g_sel = gv;
          u_sel = uv;
        }
      }
      if (lane < nq)
        p.h_out[(int64_t)gl.cpk[c][k] * p.I + rw + lane] = g_sel / (1.0f + expf(-g_sel)) * u_sel;
    };
    if constexpr (kMulti) {
      // every pick of the chunk in one pass: each code chunk decoded once
      with_count<kGroupTT>(nt, [&](auto ntc) {
        constexpr int NT = decltype(ntc)::value;
        float d[NP][NT];
        rows_dot_multi<FMT, L, S, NP, NT>(ld, xs, xstride, p.g.chunks, li, d);
#pragma unroll
        for (int k = 0; k < NT; ++k) {
          float dk[NP];
#pragma unroll
          for (int i = 0; i < NP; ++i) dk[i] = d[i][k];
          finish(dk, k);
        }
      });
    } else {
#pragma unroll 1
      for (int k = 0; k < nt; ++k) {
        XRegs<FMT, L, S> xr;
        xr.load_zpad(xs + k * xstride, p.g.chunks, li);
        float d[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          pin_regs(ld[i]);
          d[i] = row_dot<FMT, L, S>(ld[i], xr);
        }
        finish(d, k);
      }
    }
  }
}

struct DnGroupParams {
  int H, I, E;
  const int32_t* chunks;      // chunk table written by the gate_up kernel
  const float* h;             // [M * K][I]
  float* dout;                // [M * K][H] down output per pick
  LayerDev L;
  QGeom g;                    // reduction over I
  int nrb;                    // row blocks per chunk (a multiple of 8)
};

// Persistent grid over (chunk, row block) items; a row block is
// kWaves * NR * (64 / L) rows of the expert's down matrix, its weights loaded
// once per item and applied to every pick of the chunk.
template <int FMT, int L, int S, int NR>
__global__ void __launch_bounds__(kThreads, 2) moe_dn_group_kernel(DnGroupParams p) {
  constexpr int RPW = kWave / L;
  constexpr bool kMulti = FMT == kMXFP4;                // all picks per pass (int4: one pick per pass)
  constexpr int NH = (L * S + 31) / 32;                // I <= 32 * L * S: float4 of h per thread
  extern __shared__ float lds[];
  int* tab = reinterpret_cast<int*>(lds);               // [1 + kGroupMaxPicks * kChunkInts]
  float* hs = lds + (1 + kGroupMaxPicks * kChunkInts + 3) / 4 * 4;   // [kGroupTT][(chunks + 1) * kXStride]
  const int hstride = (p.g.chunks + 1) * kXStride;      // each input: chunks, then a zero chunk
  hs[min((int)(threadIdx.x / kChunkElems), kGroupTT - 1) * hstride + p.g.chunks * kXStride +
     (threadIdx.x & (kChunkElems - 1))] = 0.f;           // the zero chunks (no branch)
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  const int li = lane % L;
  const int rr = lane / L;
  const int B = NR * RPW * kWaves;
  const LayerDev& Ld = p.L;

  const int n = p.chunks[0];
  for (int i = threadIdx.x; i < n * kChunkInts; i += kThreads) tab[1 + i] = p.chunks[1 + i];
  __syncthreads();

  const int nitems = n * p.nrb;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int c = item / p.nrb;
    const int r0 = (item - c * p.nrb) * B;
    if (r0 >= p.H) continue;                              // block-uniform
    const int* ch = tab + 1 + c * kChunkInts;
    const int e = clamp_expert(ch[0], p.E);
    const int nt = __builtin_amdgcn_readfirstlane(ch[1]);      // block-uniform: one path per chunk
    StageF32<NH> hst[kGroupTT];
#pragma unroll
    for (int k = 0; k < kGroupTT; ++k)
      if (k < nt) hst[k].load(p.h + (int64_t)ch[2 + k] * p.I, p.I, threadIdx.x, kThreads);
    GroupLoad<FMT, S> ld[NR];
    const QMat m = expert_dn(Ld, e);
    if constexpr (kMulti) {
#pragma unroll
      for (int i = 0; i < NR; ++i) ld[i].ok = ld[i].zhi = 0;
#pragma unroll
      for (int s = 0; s < S; ++s)                         // slot-major, the order rows_dot_multi takes them
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const int row = r0 + (i * kWaves + wave) * RPW + rr;
          load_row_slot<FMT, L, S>(ld[i], m, p.g, row, row < p.H, li, s);
        }
    } else {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int row = r0 + (i * kWaves + wave) * RPW + rr;
        load_row<FMT, L, S>(ld[i], m, p.g, row, row < p.H, li);
      }
    }
    block_sync_lds();                                     // the previous item's h reads are done
#pragma unroll
    for (int k = 0; k < kGroupTT; ++k)
      if (k < nt) hst[k].store(hs + k * hstride, p.I, p.I, 0, 1.0f, threadIdx.x, kThreads);
    block_sync_lds();                                     // weights still in flight
    auto store = [&](int i, int k, float d) {
      const int row = r0 + (i * kWaves + wave) * RPW + rr;
      if (li == kRowSumLane<L> && row < p.H) p.dout[(int64_t)ch[2 + k] * p.H + row] = d;
    };
    if constexpr (kMulti) {
      // every pick of the chunk in one pass: each code chunk decoded once
      with_count<kGroupTT>(nt, [&](auto ntc) {
        constexpr int NT = decltype(ntc)::value;
        float d[NR][NT];
        rows_dot_multi<FMT, L, S, NR, NT>(ld, hs, hstride, p.g.chunks, li, d);
#pragma unroll
        for (int k = 0; k < NT; ++k)
#pragma unroll
          for (int i = 0; i < NR; ++i) store(i, k, d[i][k]);
      });
    } else {
#pragma unroll 1
      for (int k = 0; k < nt; ++k) {
        XRegs<FMT, L, S> xr;
        xr.load_zpad(hs + k * hstride, p.g.chunks, li);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          pin_regs(ld[i]);
          store(i, k, row_dot<FMT, L, S>(ld[i], xr));
        }
      }
    }
  }
}

// y[t] = (x[t] +) sum_j w[t][j] * dout[t*K + j], j in order (the last layer
// of a grouped step; earlier layers combine inside the next route kernel).
__global__ void __launch_bounds__(kThreads)
moe_combine_kernel(const float* __restrict__ x_prev, int residual, const float* __restrict__ dout,
                   const float* __restrict__ w, int H, int K, float* __restrict__ y) {
  const int t = blockIdx.y;
  const int h = (blockIdx.x * kThreads + threadIdx.x) * 4;
  if (h >= H) return;
  float4 v = residual ? ldg_f4(x_prev + (int64_t)t * H + h) : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < K; ++j) {
    const float wj = w[t * K + j];
    const float4 d = ldg_f4(dout + ((int64_t)t * K + j) * H + h);
    v.x = __builtin_fmaf(wj, d.x, v.x);
    v.y = __builtin_fmaf(wj, d.y, v.y);
    v.z = __builtin_fmaf(wj, d.z, v.z);
    v.w = __builtin_fmaf(wj, d.w, v.w);
  }
  *reinterpret_cast<float4*>(y + (int64_t)t * H + h) = v;
}

// ---------------------------------------------------------------- plan

struct GraphKey {
  const void* x;
  int x_dtype;
  int m;
  float* y;
  int32_t* topk_trace;
  float* wts_trace;
  float* resid_trace;
  bool operator==(const GraphKey& o) const {
    return x == o.x && x_dtype == o.x_dtype && m == o.m && y == o.y && topk_trace == o.topk_trace &&
           wts_trace == o.wts_trace && resid_trace == o.resid_trace;
  }
};

constexpr int kGraphCache = 8;

struct GraphEntry {
  bool used = false;
  uint64_t stamp = 0;
  GraphKey key{};
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipEvent_t done = nullptr;   // recorded after each launch of exec, on the launching stream
};

}  // namespace bdg

struct bdg_plan {
  bdg_moe_desc d;
  int gu_S, dn_L, dn_S, dn_NR, topk_V;
  bdg::QGeom gu_geom, dn_geom;
  // device memory
  void* dev_base;
  bdg::LayerDev* hl;        // host copy of each layer's weight pointers (passed by value to the kernels)
  float* resid[2];
  float* part;              // [M][E + 1][pstride] router partial sums (column E: sums of squares)
  int pstride;
  int dn_blocks;            // down row blocks per token
  int fuse_route;           // layers >= 1 route from the previous down kernel's partial sums
  int log2T;
  const float** wr;         // host copy of each layer's router pointer
  // grouped path (steps of M > 1 tokens)
  int group_ok;             // the geometry fits the grouped kernels
  int g_grid_gu, g_grid_dn; // persistent grid sizes
  int g_bpc, g_nrb, g_dn_NR;
  float* dout;              // [max_m * K][H] down output per pick
  int32_t* chunks;          // chunk table
  // fused per-layer kernel (steps of one token)
  int fused_ok;
  bdg::LayerConfig fused_cfg;
  int fused_nblk, fused_B, fused_dn_blocks;
  size_t fused_lds;
  float* hbuf;              // [K * I] h exchanged between the fused kernel's blocks
  unsigned* bar;            // grid barrier words (arrivals, generation), zero at create
  unsigned* fault;          // fault word (moe_plan_check)
  int wait_polls;
  // self-routing gate_up for layers that need their own router (per-token kernels):
  // the first layer (self_route0), later layers without router sums from a down kernel
  int self_route, self_route0;
  int sr_blocks;            // gate_up blocks per token that compute router rows
  unsigned* seq;            // token sequence number (advanced once per token: see SelfRoute)
  unsigned long long* sr_log;   // [L][max_m][E + 1] tagged router sums
  // grouped products on the matrix cores (BDG_MOE_MFMA, steps of m > 1)
  int mfma;
  int mfma_grid_gu, mfma_grid_dn;
  uint16_t* xh;             // [max_m][H] bf16 hi/lo parts of the normalized layer input
  uint16_t* xl;
  uint16_t* h_hi;           // [max_m * K][I] bf16 hi/lo parts of h
  uint16_t* h_lo;
  uint16_t* zeros;          // [max(H, I)] zero bf16
  int32_t* mfma_table;      // chunk table (all picks of an expert per chunk)
  uint64_t* tl_stamps;      // timeline mode: [L][nblk][kLayerStamps] (lazily allocated)
  int tl_active;            // set only inside moe_expert_decode_timeline
  int32_t* idx;
  float* w;
  float* h;
  hipStream_t cap_stream;
  hipEvent_t* prof_ev;      // timing events for moe_expert_decode_profiled (lazily created)
  int* prof_kind;
  int prof_cap;
  bdg::GraphEntry graphs[bdg::kGraphCache];
  uint64_t clock;
};

namespace bdg {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- launches

// Optional per-kernel timing: every launch takes the next start/stop event
// pair (recorded by the runtime at kernel start and end) and notes its kind.
enum KernelKind { kRoute = 0, kGateUp = 1, kDown = 2, kCombine = 3, kLayer = 4, kKinds = 5 };

struct Prof {
  hipEvent_t* ev;     // 2 * cap events
  int* kind;          // cap kinds
  int cap;
  int used;
};

// A timed kernel is launched with a start and a stop event that take the
// dispatch's own start and end times (the times a kernel trace records for
// the same dispatch); separate event records on the stream would add their
// own gaps to every duration.
#define BDG_LAUNCH(PROF, KIND, KERNEL, GRID, BLOCK, LDS, STREAM, ...)                               \
  do {                                                                                              \
    if (PROF) {                                                                                     \
      if ((PROF)->used >= (PROF)->cap) return BDG_E_UNSUPPORTED;                                    \
      const int slot_ = (PROF)->used++;                                                             \
      (PROF)->kind[slot_] = (KIND);                                                                 \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, (PROF)->ev[2 * slot_],                 \
                            (PROF)->ev[2 * slot_ + 1], 0, __VA_ARGS__);                             \
    } else {                                                                                        \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, __VA_ARGS__);                            \
    }                                                                                               \
  } while (0)

// layer input: the caller's x at layer 0, else the residual buffer written
// by the previous layer's down kernel.
// combine != 0 (grouped path, layer >= 1): the layer input is formed here
// from the previous layer's input and per-pick down outputs.
static int launch_route(const bdg_plan* p, int layer, const void* x, int x_dtype, int m,
                        float* resid_trace, int compute_logits, hipStream_t s, Prof* prof, int combine = 0,
                        int mfma_ops = 0) {
  RouteParams rp{};
  rp.M = m;
  rp.H = p->d.hidden;
  rp.E = p->d.n_experts;
  rp.compute_logits = compute_logits;
  if (layer == 0) {
    rp.x_in = x;
    rp.x_bf16 = x_dtype == BDG_BF16 ? 1 : 0;
    rp.x_copy = p->resid[0];
  } else if (combine) {
    rp.x_in = p->resid[(layer - 1) & 1];
    rp.x_bf16 = 0;
    rp.x_copy = p->resid[layer & 1];
    rp.dout = p->dout;
    rp.wts = p->w;
    rp.K = p->d.top_k;
    rp.combine_residual = (p->d.flags & BDG_MOE_STACK) ? 1 : 0;
  } else {
    rp.x_in = p->resid[layer & 1];
    rp.x_bf16 = 0;
    rp.x_copy = nullptr;
  }
  rp.resid_trace = resid_trace;
  rp.part = p->part;
  rp.pstride = p->pstride;
  rp.L = p->hl[layer];
  if (layer == 0 && p->self_route) rp.seq = p->seq;   // a new token for the self-routing layers
  if (mfma_ops) {
    // the matrix-core path's bf16 hi/lo operands of the (normalized) input
    rp.xh = p->xh;
    rp.xl = p->xl;
    rp.norm = (p->d.flags & BDG_MOE_STACK) ? 1 : 0;
    rp.eps = p->d.norm_eps;
  }
  if (compute_logits && !rp.dout && !rp.xh) {
    // one wave per router row, no LDS
    const int nf = (rp.H + 255) / 256;
    const dim3 grid((unsigned)rp.E, (unsigned)m);
#define BDG_RD_CASE(NN)                                                                          \
    if (nf <= NN) {                                                                              \
      BDG_LAUNCH(prof, kRoute, moe_route_direct_kernel<NN>, grid, dim3(kWave), 0, s, rp);        \
      return launch_status();                                                                    \
    }
    BDG_RD_CASE(2) BDG_RD_CASE(4) BDG_RD_CASE(8) BDG_RD_CASE(12) BDG_RD_CASE(16)
#undef BDG_RD_CASE
  }
  const int nblk = compute_logits ? (rp.E + kWaves - 1) / kWaves : 1;
  const size_t lds = (size_t)(rp.H + kWaves) * sizeof(float);
  BDG_LAUNCH(prof, kRoute, moe_route_kernel, dim3(nblk, m), dim3(kThreads), lds, s, rp);
  return launch_status();
}

// Where a kernel that selects its own experts finds the routing of `layer`.
static RouteSrc route_src(const bdg_plan* p, int layer, int routed, int nparts, const int32_t* idx_in,
                          const float* w_in, int use_norm) {
  RouteSrc r{};
  r.routed = routed;
  r.idx_in = idx_in;
  r.w_in = w_in;
  r.part = p->part;
  r.nparts = nparts;
  r.pstride = p->pstride;
  r.log2T = p->log2T;
  r.norm = use_norm;
  r.eps = p->d.norm_eps;
  r.E = p->d.n_experts;
  r.K = p->d.top_k;
  r.H = p->d.hidden;
  r.b_r = p->hl[layer].b_r;
  return r;
}

// sr: a self-routing launch (the layer's router computed inside it), or NULL;
// x_in: the caller's input (the first layer of a self-routing launch, fp32 or
// bf16 bits), else the plan's residual buffer
static int launch_gateup(const bdg_plan* p, int layer, int m, int routed, int nparts, const int32_t* idx_in,
                         const float* w_in, int32_t* topk_trace, float* wts_trace, int use_norm,
                         hipStream_t s, Prof* prof, const SelfRoute* sr = nullptr, const void* x_in = nullptr,
                         int x_bf16 = 0) {
  GateUpParams gp{};
  gp.M = m;
  gp.H = p->d.hidden;
  gp.I = p->d.inter;
  gp.E = p->d.n_experts;
  gp.K = p->d.top_k;
  gp.rt = route_src(p, layer, routed, nparts, idx_in, w_in, use_norm);
  gp.idx_out = p->idx;
  gp.w_out = p->w;
  gp.topk_trace = topk_trace;
  gp.wts_trace = wts_trace;
  gp.x = p->resid[layer & 1];
  gp.L = p->hl[layer];
  gp.g = p->gu_geom;
  gp.h_out = p->h;
  const int64_t pairs = (int64_t)gp.K * gp.I;
  const int64_t per_block = (int64_t)kWaves * kGuPairsPerWave;
  int64_t blocks = (pairs + per_block - 1) / per_block;
  if (blocks > 65535) return BDG_E_UNSUPPORTED;
  const int E = gp.E;
  const size_t psum = (size_t)E << p->log2T;
  const size_t lds = ((size_t)(gp.g.chunks + 1) * kXStride + kWaves + psum) * sizeof(float);
  dim3 grid((unsigned)blocks, m);
  const int fmt = p->d.fmt, V = p->topk_V;
  // 0: routing from router sums; 1: self-routing; 2: self-routing on the caller's bf16 input
  int srk = 0;
  if (sr) {
    // every router row needs a wave of the launch's first blocks
    if (routed || nparts != 1 || p->d.hidden > kSelfRouteNF * 256 || V > 4 ||
        (int64_t)sr->blocks * kWaves < E || sr->blocks > blocks)
      return BDG_E_UNSUPPORTED;
    gp.sr = *sr;
    srk = x_in && x_bf16 ? 2 : 1;
  } else if (x_in) {
    return BDG_E_INVALID;
  }
  if (x_in) gp.x = static_cast<const float*>(x_in);   // bf16 bits when srk == 2
#define BDG_GU_CASE(F, SS, VV, SR)                                                                            \
  if (fmt == F && p->gu_S == SS && V == VV && srk == SR) {                                                    \
    BDG_LAUNCH(prof, kGateUp, (moe_gateup_kernel<F, SS, kGuPairsPerWave, VV, SR>), grid, dim3(kThreads), lds, \
               s, gp);                                                                                        \
    return launch_status();                                                                                   \
  }
#define BDG_GU_V(F, SS)                                                                                        \
  BDG_GU_CASE(F, SS, 1, 0) BDG_GU_CASE(F, SS, 2, 0) BDG_GU_CASE(F, SS, 4, 0) BDG_GU_CASE(F, SS, 16, 0)        \
  BDG_GU_CASE(F, SS, 1, 1) BDG_GU_CASE(F, SS, 2, 1) BDG_GU_CASE(F, SS, 4, 1)                                  \
  BDG_GU_CASE(F, SS, 1, 2) BDG_GU_CASE(F, SS, 2, 2) BDG_GU_CASE(F, SS, 4, 2)
  BDG_GU_V(kMXFP4, 1) BDG_GU_V(kMXFP4, 2) BDG_GU_V(kMXFP4, 3) BDG_GU_V(kMXFP4, 4)
  BDG_GU_V(kINT4G, 1) BDG_GU_V(kINT4G, 2) BDG_GU_V(kINT4G, 3) BDG_GU_V(kINT4G, 4)
#undef BDG_GU_V
#undef BDG_GU_CASE
  return BDG_E_UNSUPPORTED;
}

// h float4 staged per thread by a down block: a group of kg experts' inputs
// (kg * I floats) over 8 waves, in one batch.
static int down_stage_f4(int K, int I) {
  const int kg = K < kDownWaves ? K : kDownWaves;
  return (kg * I + kDownWaves * kWave * 4 - 1) / (kDownWaves * kWave * 4);
}

// The combine / residual / next-layer router outputs of `layer`'s down product.
static DownOut down_out(const bdg_plan* p, int layer, int residual, float* x_out, float* y_out, float* trace_out,
                        int route_next) {
  DownOut o{};
  o.H = p->d.hidden;
  o.E = p->d.n_experts;
  o.K = p->d.top_k;
  o.residual = residual;
  o.x_prev = p->resid[layer & 1];
  o.w = p->w;
  o.x_out = x_out;
  o.y_out = y_out;
  o.trace_out = trace_out;
  o.route_next = route_next;
  o.wr_next = route_next ? p->wr[layer + 1] : nullptr;
  o.part_out = p->part;
  o.pstride = p->pstride;
  return o;
}

// seq_bump: the token sequence number to advance (after a self-routing first layer), or NULL
static int launch_down(const bdg_plan* p, int layer, int m, int residual, float* x_out, float* y_out,
                       float* trace_out, int route_next, hipStream_t s, Prof* prof, unsigned* seq_bump = nullptr) {
  DownParams dp{};
  dp.seq_bump = seq_bump;
  dp.M = m;
  dp.H = p->d.hidden;
  dp.I = p->d.inter;
  dp.E = p->d.n_experts;
  dp.K = p->d.top_k;
  dp.idx = p->idx;
  dp.h = p->h;
  dp.o = down_out(p, layer, residual, x_out, y_out, trace_out, route_next);
  dp.L = p->hl[layer];
  dp.g = p->dn_geom;
  const int rpw = kWave / p->dn_L;
  const int kg = dp.K < kDownWaves ? dp.K : kDownWaves;
  const int wpe = kDownWaves / kg;
  const int B = p->dn_NR * rpw * wpe;
  const size_t lds = ((size_t)kg * (dp.g.chunks + 1) * kXStride + (size_t)dp.K * B) * sizeof(float);
  dim3 grid((unsigned)((dp.H + B - 1) / B), m);
  const int hv = down_stage_f4(dp.K, dp.I);
  const int HV = hv <= 2 ? 2 : hv <= 4 ? 4 : hv <= 6 ? 6 : hv <= 8 ? 8 : 12;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (prof) {
    if (prof->used >= prof->cap) return BDG_E_UNSUPPORTED;
    const int slot = prof->used++;
    prof->kind[slot] = kDown;
    e0 = prof->ev[2 * slot];
    e1 = prof->ev[2 * slot + 1];
  }
  return launch_down_kernel(dp, p->d.fmt, p->dn_L, p->dn_S, p->dn_NR, HV, grid, lds, s, e0, e1);
}

static int launch_gu_group(const bdg_plan* p, int layer, int m, int routed, const int32_t* idx_in,
                           const float* w_in, int32_t* topk_trace, float* wts_trace, int use_norm, hipStream_t s,
                           Prof* prof) {
  GroupParams gp{};
  gp.M = m;
  gp.H = p->d.hidden;
  gp.I = p->d.inter;
  gp.E = p->d.n_experts;
  gp.K = p->d.top_k;
  gp.routed = routed;
  gp.part = p->part;
  gp.pstride = p->pstride;
  gp.norm = use_norm;
  gp.eps = p->d.norm_eps;
  gp.idx_in = idx_in;
  gp.w_in = w_in;
  gp.idx_out = p->idx;
  gp.w_out = p->w;
  gp.topk_trace = topk_trace;
  gp.wts_trace = wts_trace;
  gp.x = p->resid[layer & 1];
  gp.L = p->hl[layer];
  gp.g = p->gu_geom;
  gp.h_out = p->h;
  gp.chunks_out = p->chunks;
  gp.bpc = p->g_bpc;
  const size_t lds = (group_lds_floats() + (size_t)kGroupTT * (gp.g.chunks + 1) * kXStride) * sizeof(float);
  const dim3 grid((unsigned)p->g_grid_gu);
  const int fmt = p->d.fmt, V = p->topk_V;
#define BDG_GG_CASE(F, SS, VV)                                                                            \
  if (fmt == F && p->gu_S == SS && V == VV) {                                                             \
    BDG_LAUNCH(prof, kGateUp, (moe_gu_group_kernel<F, SS, gu_group_np(F, SS), VV>), grid, dim3(kThreads), \
               lds, s, gp);                                                                               \
    return launch_status();                                                                               \
  }
#define BDG_GG_V(F, SS) BDG_GG_CASE(F, SS, 1) BDG_GG_CASE(F, SS, 2) BDG_GG_CASE(F, SS, 4) BDG_GG_CASE(F, SS, 16)
  // shapes whose rows, held across a chunk's picks, fit 256 VGPRs (group_ok)
  BDG_GG_V(kMXFP4, 1) BDG_GG_V(kMXFP4, 2) BDG_GG_V(kMXFP4, 3)
  BDG_GG_V(kINT4G, 1) BDG_GG_V(kINT4G, 2)
#undef BDG_GG_V
#undef BDG_GG_CASE
  return BDG_E_UNSUPPORTED;
}

static int launch_dn_group(const bdg_plan* p, int layer, hipStream_t s, Prof* prof) {
  DnGroupParams dp{};
  dp.H = p->d.hidden;
  dp.I = p->d.inter;
  dp.E = p->d.n_experts;
  dp.chunks = p->chunks;
  dp.h = p->h;
  dp.dout = p->dout;
  dp.L = p->hl[layer];
  dp.g = p->dn_geom;
  dp.nrb = p->g_nrb;
  const size_t lds =
      ((size_t)(1 + kGroupMaxPicks * kChunkInts + 3) / 4 * 4 + (size_t)kGroupTT * (dp.g.chunks + 1) * kXStride) *
      sizeof(float);
  const dim3 grid((unsigned)p->g_grid_dn);
  const int fmt = p->d.fmt;
#define BDG_DG_CASE(F, LL, SS)                                                                            \
  if (fmt == F && p->dn_L == LL && p->dn_S == SS) {                                                      \
    BDG_LAUNCH(prof, kDown, (moe_dn_group_kernel<F, LL, SS, dn_group_nr(F, LL, SS)>), grid, dim3(kThreads), \
               lds, s, dp);                                                                               \
    return launch_status();                                                                               \
  }
  // the (L, S) pairs pick_lanes gives for I <= 4096
#define BDG_DG_ALL(F)                                                                              \
  BDG_DG_CASE(F, 8, 1) BDG_DG_CASE(F, 8, 2) BDG_DG_CASE(F, 8, 3) BDG_DG_CASE(F, 16, 2)             \
  BDG_DG_CASE(F, 16, 3) BDG_DG_CASE(F, 32, 2) BDG_DG_CASE(F, 32, 3) BDG_DG_CASE(F, 64, 2)
  BDG_DG_ALL(kMXFP4)
  BDG_DG_ALL(kINT4G)
#undef BDG_DG_ALL
#undef BDG_DG_CASE
  return BDG_E_UNSUPPORTED;
}

static int launch_combine(const bdg_plan* p, int m, const float* x_prev, int residual, float* y, hipStream_t s,
                          Prof* prof) {
  const int H = p->d.hidden;
  const dim3 grid((unsigned)((H / 4 + kThreads - 1) / kThreads), (unsigned)m);
  BDG_LAUNCH(prof, kCombine, moe_combine_kernel, grid, dim3(kThreads), 0, s, x_prev, residual, p->dout, p->w, H,
             p->d.top_k, y);
  return launch_status();
}

// The fused per-layer kernel of a one-token step: routing from `nparts`
// router slices, gate_up + SwiGLU, down + combine, and the outputs of
// launch_down.
static int launch_layer(const bdg_plan* p, int layer, int nparts, int32_t* topk_trace, float* wts_trace, int use_norm,
                        int residual, float* x_out, float* y_out, float* trace_out, int route_next, hipStream_t s,
                        Prof* prof) {
  LayerParams lp{};
  lp.H = p->d.hidden;
  lp.I = p->d.inter;
  lp.E = p->d.n_experts;
  lp.K = p->d.top_k;
  lp.rt = route_src(p, layer, 0, nparts, nullptr, nullptr, use_norm);
  lp.idx_out = p->idx;
  lp.w_out = p->w;
  lp.topk_trace = topk_trace;
  lp.wts_trace = wts_trace;
  lp.x = p->resid[layer & 1];
  lp.L = p->hl[layer];
  lp.g_gu = p->gu_geom;
  lp.g_dn = p->dn_geom;
  lp.hbuf = p->hbuf;
  lp.bar = p->bar;
  lp.fault = p->fault;
  lp.wait_polls = p->wait_polls;
  lp.dn_blocks = p->fused_dn_blocks;
  lp.B = p->fused_B;
  lp.o = down_out(p, layer, residual, x_out, y_out, trace_out, route_next);
  lp.stamps = p->tl_active ? p->tl_stamps + (size_t)layer * p->fused_nblk * kLayerStamps : nullptr;
  if (prof) {
    // dispatch events, as BDG_LAUNCH takes them
    if (prof->used >= prof->cap) return BDG_E_UNSUPPORTED;
    const int slot = prof->used++;
    prof->kind[slot] = kLayer;
    return launch_layer_fused(p->fused_cfg, lp, p->fused_nblk, p->fused_lds, s, prof->ev[2 * slot],
                              prof->ev[2 * slot + 1]);
  }
  return launch_layer_fused(p->fused_cfg, lp, p->fused_nblk, p->fused_lds, s);
}

static MfmaParams mfma_params(const bdg_plan* p, int layer, int m, int routed, const int32_t* idx_in,
                               const float* w_in, int32_t* topk_trace, float* wts_trace, int use_norm) {
  MfmaParams mp{};
  mp.M = m;
  mp.H = p->d.hidden;
  mp.I = p->d.inter;
  mp.E = p->d.n_experts;
  mp.K = p->d.top_k;
  mp.routed = routed;
  mp.idx_in = idx_in;
  mp.w_in = w_in;
  mp.part = p->part;
  mp.pstride = p->pstride;
  mp.norm = use_norm;
  mp.eps = p->d.norm_eps;
  mp.idx_out = p->idx;
  mp.w_out = p->w;
  mp.topk_trace = topk_trace;
  mp.wts_trace = wts_trace;
  mp.L = p->hl[layer];
  mp.xh = p->xh;
  mp.xl = p->xl;
  mp.hh = p->h_hi;
  mp.hl = p->h_lo;
  mp.zeros = p->zeros;
  mp.table = p->mfma_table;
  mp.dout = p->dout;
  return mp;
}

// The matrix-core grouped gate_up and down of one layer, timed as BDG_LAUNCH times.
static int launch_mfma_pair(const bdg_plan* p, const MfmaParams& mp, hipStream_t s, Prof* prof) {
  for (int which = 0; which < 2; ++which) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (prof) {
      if (prof->used >= prof->cap) return BDG_E_UNSUPPORTED;
      const int slot = prof->used++;
      prof->kind[slot] = which == 0 ? kGateUp : kDown;
      e0 = prof->ev[2 * slot];
      e1 = prof->ev[2 * slot + 1];
    }
    const int st = which == 0 ? launch_gu_mfma(mp, p->topk_V, p->mfma_grid_gu, s, e0, e1)
                              : launch_dn_mfma(mp, p->mfma_grid_dn, s, e0, e1);
    if (st) return st;
  }
  return BDG_OK;
}

// A grouped step (M > 1): per layer route (forming the layer input from the
// previous layer's per-pick outputs), grouped gate_up, grouped down; a final
// combine writes y.
static int enqueue_decode_grouped(const bdg_plan* p, const GraphKey& k, hipStream_t s, Prof* prof) {
  const int L = p->d.n_layers;
  const int K = p->d.top_k;
  const int H = p->d.hidden;
  const int stack = (p->d.flags & BDG_MOE_STACK) ? 1 : 0;
  for (int l = 0; l < L; ++l) {
    int st = launch_route(p, l, k.x, k.x_dtype, k.m, k.resid_trace ? k.resid_trace + (int64_t)l * k.m * H : nullptr,
                          1, s, prof, /*combine=*/l > 0, /*mfma_ops=*/p->mfma);
    if (st) return st;
    if (p->mfma) {
      st = launch_mfma_pair(p, mfma_params(p, l, k.m, 0, nullptr, nullptr,
                                           k.topk_trace ? k.topk_trace + (int64_t)l * k.m * K : nullptr,
                                           k.wts_trace ? k.wts_trace + (int64_t)l * k.m * K : nullptr, stack),
                            s, prof);
      if (st) return st;
      continue;
    }
    st = launch_gu_group(p, l, k.m, 0, nullptr, nullptr,
                         k.topk_trace ? k.topk_trace + (int64_t)l * k.m * K : nullptr,
                         k.wts_trace ? k.wts_trace + (int64_t)l * k.m * K : nullptr, stack, s, prof);
    if (st) return st;
    st = launch_dn_group(p, l, s, prof);
    if (st) return st;
  }
  return launch_combine(p, k.m, p->resid[(L - 1) & 1], stack, k.y, s, prof);
}

// The whole per-token path, enqueued on s.
static int enqueue_decode(const bdg_plan* p, const GraphKey& k, hipStream_t s, Prof* prof = nullptr) {
  if (k.m > 1 && p->group_ok) return enqueue_decode_grouped(p, k, s, prof);
  const int L = p->d.n_layers;
  const int K = p->d.top_k;
  const int H = p->d.hidden;
  const int stack = (p->d.flags & BDG_MOE_STACK) ? 1 : 0;
  auto trace = [&](int l) { return k.resid_trace ? k.resid_trace + (int64_t)l * k.m * H : nullptr; };
  for (int l = 0; l < L; ++l) {
    // layer l's router sums: the route kernel, the previous down kernel, or
    // (self-routing) the gate_up launch itself
    const bool fused = p->fuse_route && l > 0;
    const bool one_kernel = k.m == 1 && p->fused_ok;
    const bool self0 = l == 0 && p->self_route0 && !one_kernel;
    const bool self = self0 || (p->self_route && l > 0 && !fused && !one_kernel);
    int st = BDG_OK;
    if (!fused && !self) {
      st = launch_route(p, l, k.x, k.x_dtype, k.m, trace(l), 1, s, prof);
      if (st) return st;
    }
    if (one_kernel) {
      const bool last = l + 1 == L;
      const bool feed = !last && p->fuse_route;
      st = launch_layer(p, l, fused ? p->dn_blocks : 1, k.topk_trace ? k.topk_trace + (int64_t)l * K : nullptr,
                        k.wts_trace ? k.wts_trace + (int64_t)l * K : nullptr, stack, stack,
                        last ? nullptr : p->resid[(l + 1) & 1], last ? k.y : nullptr, feed ? trace(l + 1) : nullptr,
                        feed ? 1 : 0, s, prof);
      if (st) return st;
      continue;
    }
    SelfRoute sr{};
    if (self) {
      sr.log = p->sr_log + (size_t)l * p->d.max_m * (p->d.n_experts + 1);
      sr.seq = p->seq;
      sr.tag_add = self0 ? 1u : 0u;   // the first layer's down kernel advances the number
      sr.blocks = p->sr_blocks;
      sr.polls = p->wait_polls;
      sr.fault = p->fault;
      sr.resid_trace = trace(l);
      sr.x_copy = self0 ? p->resid[0] : nullptr;
    }
    st = launch_gateup(p, l, k.m, 0, fused ? p->dn_blocks : 1, nullptr, nullptr,
                       k.topk_trace ? k.topk_trace + (int64_t)l * k.m * K : nullptr,
                       k.wts_trace ? k.wts_trace + (int64_t)l * k.m * K : nullptr, stack, s, prof,
                       self ? &sr : nullptr, self0 ? k.x : nullptr, k.x_dtype == BDG_BF16 ? 1 : 0);
    if (st) return st;
    const bool last = l + 1 == L;
    const bool feed = !last && p->fuse_route;
    st = launch_down(p, l, k.m, stack, last ? nullptr : p->resid[(l + 1) & 1], last ? k.y : nullptr,
                     feed ? trace(l + 1) : nullptr, feed ? 1 : 0, s, prof, self0 ? p->seq : nullptr);
    if (st) return st;
  }
  return BDG_OK;
}

// Destroy a cached graph once its last launch has finished, on whichever
// stream that launch was queued.
static void drop_graph(GraphEntry& g) {
  if (g.done) {
    (void)hipEventSynchronize(g.done);
    (void)hipEventDestroy(g.done);
  }
  if (g.exec) (void)hipGraphExecDestroy(g.exec);
  if (g.graph) (void)hipGraphDestroy(g.graph);
  g = GraphEntry{};
}

static int check_layer(const bdg_moe_desc* d, const bdg_layer_desc& L) {
  if (!L.w_router) return BDG_E_INVALID;
  if ((reinterpret_cast<uintptr_t>(L.w_router) & 15u) != 0) return BDG_E_ALIGN;
  const bdg_qmat* mats[2] = {&L.gate_up, &L.down};
  for (int i = 0; i < 2; ++i) {
    int st = check_qmat(mats[i], true);
    if (st) return st;
    if (mats[i]->fmt != d->fmt || mats[i]->group != d->group) return BDG_E_INVALID;
  }
  if (L.gate_up.n != 2LL * d->inter || L.gate_up.k != d->hidden) return BDG_E_INVALID;
  if (L.down.n != d->hidden || L.down.k != d->inter) return BDG_E_INVALID;
  if (d->n_experts > 1) {
    for (int i = 0; i < 2; ++i) {
      if (mats[i]->expert_stride_codes == 0 || mats[i]->expert_stride_scales == 0) return BDG_E_INVALID;
      if (mats[i]->fmt == BDG_FMT_INT4G && mats[i]->expert_stride_zeros == 0) return BDG_E_INVALID;
    }
  }
  return BDG_OK;
}

}  // namespace bdg

using namespace bdg;

extern "C" int moe_plan_create(const bdg_moe_desc* d, bdg_plan** out) {
  if (!d || !out) return BDG_E_INVALID;
  *out = nullptr;
  if (d->n_layers < 1 || d->hidden <= 0 || d->inter <= 0 || d->n_experts < 1 || d->top_k < 1 ||
      d->top_k > d->n_experts || !d->layers || d->max_m < 1)
    return BDG_E_INVALID;
  if (d->fmt != BDG_FMT_MXFP4 && d->fmt != BDG_FMT_INT4G) return BDG_E_INVALID;
  if ((d->hidden % 32) || (d->inter % 32)) return BDG_E_INVALID;
  if ((d->flags & ~(BDG_MOE_STACK | BDG_MOE_NO_GRAPH | BDG_MOE_ROUTE_EVERY_LAYER | BDG_MOE_PER_TOKEN |
                    BDG_MOE_FUSED_LAYER | BDG_MOE_MFMA | BDG_MOE_ROUTE_KERNEL)) != 0)
    return BDG_E_INVALID;
  if ((d->flags & BDG_MOE_STACK) && !(d->norm_eps >= 0.f)) return BDG_E_INVALID;
  if (d->top_k > BDG_MAX_TOPK || d->n_experts > BDG_MAX_EXPERTS || d->max_m > BDG_MAX_M)
    return BDG_E_UNSUPPORTED;
  if (d->hidden > 4096 || d->inter > BDG_MAX_K) return BDG_E_UNSUPPORTED;
  if (d->fmt == BDG_FMT_INT4G && ((d->hidden % d->group) || (d->inter % d->group))) return BDG_E_INVALID;
  for (int l = 0; l < d->n_layers; ++l) {
    int st = check_layer(d, d->layers[l]);
    if (st) return st;
  }
  bdg_plan* p = new (std::nothrow) bdg_plan();
  if (!p) return BDG_E_NOMEM;
  p->d = *d;
  p->d.layers = nullptr;
  const int hc = d->hidden / 32, ic = d->inter / 32;
  p->gu_S = (hc + 31) / 32;
  p->topk_V = d->n_experts <= 64 ? 1 : d->n_experts <= 128 ? 2 : d->n_experts <= 256 ? 4 : 16;
  if (!pick_lanes(ic, &p->dn_L, &p->dn_S)) {
    delete p;
    return BDG_E_UNSUPPORTED;
  }
  if (down_stage_f4(d->top_k, d->inter) > 12) {   // h staging must fit one batch
    delete p;
    return BDG_E_UNSUPPORTED;
  }
  {
    // rows per down block: keep about 300+ blocks at M = 1, up to 4 row groups per wave
    const int rpw = kWave / p->dn_L;
    const int kg = d->top_k < kDownWaves ? d->top_k : kDownWaves;
    const int wpe = kDownWaves / kg;
    // the kernel is latency-bound: size the grid to one resident round of
    // about one 8-wave block per CU
    int nr = (d->hidden + 256 * rpw * wpe - 1) / (256 * rpw * wpe);
    if (nr < 1) nr = 1;
    if (nr > 4) nr = 4;
    p->dn_NR = nr;
    const int B = p->dn_NR * rpw * wpe;
    p->dn_blocks = (d->hidden + B - 1) / B;
    // a layer routes from the previous down kernel's partial sums when the
    // sums are small enough for every gate_up block to add them up (more
    // than 64 experts route inside their gate_up launch instead: fusing them
    // needed fewer, taller down blocks and measured slower on the 128-expert
    // int4 stack)
    p->fuse_route = (d->flags & BDG_MOE_STACK) && d->n_layers > 1 && B <= kWave &&
                    p->dn_blocks <= 4 * kThreads && d->n_experts <= kDownWaves * kDnRouterPerWave &&
                    !(d->flags & BDG_MOE_ROUTE_EVERY_LAYER);
    int lt = 0;
    while (lt < 6 && (d->n_experts << (lt + 1)) <= kThreads) ++lt;
    p->log2T = lt;
    // gate_up loads 4 * T * kPartF4 slices per expert row up front, without
    // bounds checks: rows are at least that long, zero past the slices
    p->pstride = ((p->fuse_route ? p->dn_blocks : 1) + 3) & ~3;
    if (p->fuse_route) p->pstride = std::max(p->pstride, 4 * (1 << lt) * kPartF4);
  }
  {
    // grouped path: persistent grids sized to the device, items padded so a
    // row block's items in consecutive chunks are a multiple of 8 apart
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    const int hc32 = d->hidden / 32, ic32 = d->inter / 32;
    const size_t lds_gu = (group_lds_floats() + (size_t)kGroupTT * (hc32 + 1) * kXStride) * sizeof(float);
    const size_t lds_dn = ((size_t)(1 + kGroupMaxPicks * kChunkInts + 3) / 4 * 4 + (size_t)kGroupTT * (ic32 + 1) * kXStride) *
                          sizeof(float);
    const size_t lds_cu = 160 * 1024;
    const int bg = (int)std::min<size_t>(2, lds_cu / lds_gu), bd = (int)std::min<size_t>(2, lds_cu / lds_dn);
    p->g_grid_gu = (cus * (bg < 1 ? 1 : bg) + 7) / 8 * 8;
    p->g_grid_dn = (cus * (bd < 1 ? 1 : bd) + 7) / 8 * 8;
    const int np = gu_group_np(d->fmt == BDG_FMT_MXFP4 ? 0 : 1, p->gu_S);
    p->g_bpc = ((d->inter + kWaves * np - 1) / (kWaves * np) + 7) / 8 * 8;
    const int rpw = kWave / p->dn_L;
    p->g_dn_NR = dn_group_nr(d->fmt == BDG_FMT_MXFP4 ? 0 : 1, p->dn_L, p->dn_S);
    const int B = p->g_dn_NR * rpw * kWaves;
    p->g_nrb = ((d->hidden + B - 1) / B + 7) / 8 * 8;
    p->group_ok = d->max_m * d->top_k <= kGroupMaxPicks && d->inter <= 4096 && p->dn_L * p->dn_S <= 128 &&
                  p->gu_S <= (d->fmt == BDG_FMT_MXFP4 ? 3 : 2) &&
                  lds_gu <= 64 * 1024 &&
                  lds_dn <= 64 * 1024 && !(d->flags & BDG_MOE_PER_TOKEN);
    // grouped products on the matrix cores: MXFP4 (hidden and inter are
    // multiples of 32: whole 16-row tile pairs and MX blocks), grids of
    // every block the kernels keep resident
    p->mfma = 0;
    if ((d->flags & BDG_MOE_MFMA) && p->group_ok && d->fmt == BDG_FMT_MXFP4 && d->max_m <= 16) {
      int bg = 0, bd = 0;
      const void* fg = mfma_gu_kernel(p->topk_V);
      if (fg && hipOccupancyMaxActiveBlocksPerMultiprocessor(&bg, fg, 256, 0) == hipSuccess &&
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&bd, mfma_dn_kernel(), 256, 0) == hipSuccess && bg > 0 &&
          bd > 0) {
        p->mfma = 1;
        p->mfma_grid_gu = cus * bg;
        p->mfma_grid_dn = cus * bd;
      }
      (void)hipGetLastError();
    }
  }
  auto geom = [&](int k) {
    QGeom g;
    g.k = k;
    g.chunks = k / 32;
    g.group = d->group;
    g.groups = k / d->group;
    g.zrow = (g.groups + 1) / 2;
    return g;
  };
  p->gu_geom = geom(d->hidden);
  p->dn_geom = geom(d->inter);
  p->wait_polls = d->wait_polls == 0 ? (1 << 20) : (d->wait_polls < 0 ? 0 : d->wait_polls);
  {
    // self-routing gate_up (layers >= 1 that would otherwise launch the
    // route kernel): every router row needs one wave of the launch's first
    // blocks, and a row of x fits kSelfRouteNF float4 per lane
    p->self_route = 0;
    p->self_route0 = 0;
    p->sr_blocks = (d->n_experts + kWaves - 1) / kWaves;
    const int64_t gu_blocks =
        ((int64_t)d->top_k * d->inter + kWaves * kGuPairsPerWave - 1) / (kWaves * kGuPairsPerWave);
    const bool fits = !(d->flags & BDG_MOE_ROUTE_KERNEL) && d->hidden <= kSelfRouteNF * 256 && p->topk_V <= 4 &&
                      p->sr_blocks <= gu_blocks;
    p->self_route0 = fits ? 1 : 0;
    p->self_route = fits && d->n_layers > 1 && !p->fuse_route ? 1 : 0;
  }
  {
    // fused per-layer kernel for one-token steps (BDG_MOE_FUSED_LAYER): one
    // block of 8 waves per CU, all blocks resident (the grid waits on
    // itself); block b < dn_blocks owns B down rows of every chosen expert.
    // Shapes without a compiled variant, or whose grid would not be
    // resident, keep two kernels.
    int dev = 0, cus = 0;
    p->fused_ok = 0;
    const int K = d->top_k;
    const int rpw = kWave / p->dn_L;
    if ((d->flags & BDG_MOE_FUSED_LAYER) && K <= 8 && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) {
      const int nblk = cus;
      int B = rpw;
      while ((d->hidden + B - 1) / B > nblk) B += rpw;
      const int groups = K * (B / rpw);
      const int ng = (groups + layer_dn_load_waves() - 1) / layer_dn_load_waves();
      const int64_t pairs = (int64_t)K * d->inter;
      const int np = (int)((pairs + (int64_t)nblk * 8 - 1) / ((int64_t)nblk * 8));
      const int64_t nh = (pairs + layer_threads() - 1) / layer_threads();
      const int nhl = nh <= 12 ? 12 : nh <= 24 ? 24 : 0;
      LayerConfig c{d->fmt == BDG_FMT_MXFP4 ? (int)kMXFP4 : (int)kINT4G, p->gu_S, np, p->topk_V, p->dn_L, p->dn_S,
                    ng, nhl};
      LayerShape sh{p->gu_geom, p->dn_geom, K, d->n_experts, p->log2T, B};
      const int lds = layer_fused_lds_bytes(sh, np, ng, p->dn_S);
      const void* fn = layer_fused_kernel(c);
      const int dn_blocks = (d->hidden + B - 1) / B;
      // the epilogue's router slices must match what the next layer adds up
      const bool slices_match = !p->fuse_route || dn_blocks == p->dn_blocks;
      int per_cu = 0;
      if (fn && B <= kWave && nhl > 0 && slices_match && lds <= 160 * 1024) {
        (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, layer_threads(), (size_t)lds) != hipSuccess)
          per_cu = 0;
        (void)hipGetLastError();
      }
      if (per_cu >= 1) {
        p->fused_ok = 1;
        p->fused_cfg = c;
        p->fused_nblk = nblk;
        p->fused_B = B;
        p->fused_dn_blocks = dn_blocks;
        p->fused_lds = (size_t)lds;
      }
    }
  }
  // device memory: layer table + workspace
  const int M = d->max_m, H = d->hidden, I = d->inter, E = d->n_experts, K = d->top_k;
  size_t off = 0;
  const size_t o_res0 = off; off = align256(off + sizeof(float) * M * H);
  const size_t o_res1 = off; off = align256(off + sizeof(float) * M * H);
  const size_t o_part = off; off = align256(off + sizeof(float) * (size_t)M * (E + 1) * p->pstride);
  const size_t o_idx = off; off = align256(off + sizeof(int32_t) * M * K);
  const size_t o_w = off; off = align256(off + sizeof(float) * M * K);
  const size_t o_h = off; off = align256(off + sizeof(float) * (size_t)M * K * I);
  const size_t o_dout = off; off = align256(off + sizeof(float) * (size_t)M * K * H);
  const size_t o_chunks = off; off = align256(off + sizeof(int32_t) * (1 + kGroupMaxPicks * kChunkInts));
  const size_t o_hbuf = off; off = align256(off + sizeof(float) * (size_t)K * I);
  const size_t o_bar = off; off = align256(off + sizeof(unsigned) * 64);
  const size_t o_fault = off; off = align256(off + sizeof(unsigned) * 64);
  const size_t o_seq = off; off = align256(off + sizeof(unsigned) * 64);
  const size_t o_srlog = off;
  off = align256(off + sizeof(unsigned long long) *
                      (p->self_route || p->self_route0 ? (size_t)d->n_layers * M * (E + 1) : 1));
  const size_t o_xh = off; off = align256(off + sizeof(uint16_t) * (size_t)M * H);
  const size_t o_xl = off; off = align256(off + sizeof(uint16_t) * (size_t)M * H);
  const size_t o_hh = off; off = align256(off + sizeof(uint16_t) * (size_t)M * K * I);
  const size_t o_hlo = off; off = align256(off + sizeof(uint16_t) * (size_t)M * K * I);
  const size_t o_zero = off; off = align256(off + sizeof(uint16_t) * (size_t)std::max(H, I));
  const size_t o_mtab = off; off = align256(off + sizeof(int32_t) * (1 + kGroupMaxPicks * kMfmaChunkInts));
  if (hipMalloc(&p->dev_base, off) != hipSuccess) {
    delete p;
    return BDG_E_NOMEM;
  }
  char* base = static_cast<char*>(p->dev_base);
  p->resid[0] = reinterpret_cast<float*>(base + o_res0);
  p->resid[1] = reinterpret_cast<float*>(base + o_res1);
  p->part = reinterpret_cast<float*>(base + o_part);
  p->idx = reinterpret_cast<int32_t*>(base + o_idx);
  p->w = reinterpret_cast<float*>(base + o_w);
  p->h = reinterpret_cast<float*>(base + o_h);
  p->dout = reinterpret_cast<float*>(base + o_dout);
  p->chunks = reinterpret_cast<int32_t*>(base + o_chunks);
  p->hbuf = reinterpret_cast<float*>(base + o_hbuf);
  p->bar = reinterpret_cast<unsigned*>(base + o_bar);
  p->fault = reinterpret_cast<unsigned*>(base + o_fault);
  p->seq = reinterpret_cast<unsigned*>(base + o_seq);
  p->sr_log = reinterpret_cast<unsigned long long*>(base + o_srlog);
  p->xh = reinterpret_cast<uint16_t*>(base + o_xh);
  p->xl = reinterpret_cast<uint16_t*>(base + o_xl);
  p->h_hi = reinterpret_cast<uint16_t*>(base + o_hh);
  p->h_lo = reinterpret_cast<uint16_t*>(base + o_hlo);
  p->zeros = reinterpret_cast<uint16_t*>(base + o_zero);
  p->mfma_table = reinterpret_cast<int32_t*>(base + o_mtab);
  // router partial sums: zero once, so slots past the slices read as 0
  if (hipMemset(p->part, 0, sizeof(float) * (size_t)M * (E + 1) * p->pstride) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(p->dev_base);
    delete p;
    return BDG_E_HIP;
  }
  LayerDev* host = new (std::nothrow) LayerDev[d->n_layers];
  p->wr = new (std::nothrow) const float*[d->n_layers];
  if (!host || !p->wr) {
    delete[] host;
    delete[] p->wr;
    (void)hipFree(p->dev_base);
    delete p;
    return BDG_E_NOMEM;
  }
  for (int l = 0; l < d->n_layers; ++l) {
    const bdg_layer_desc& S = d->layers[l];
    p->wr[l] = S.w_router;
    LayerDev& D = host[l];
    D.w_r = S.w_router;
    D.b_r = S.b_router;
    D.gu_codes = static_cast<const uint8_t*>(S.gate_up.codes);
    D.gu_scales = static_cast<const uint8_t*>(S.gate_up.scales);
    D.gu_zeros = static_cast<const uint8_t*>(S.gate_up.zeros);
    D.gu_sc = S.gate_up.expert_stride_codes;
    D.gu_ss = S.gate_up.expert_stride_scales;
    D.gu_sz = S.gate_up.expert_stride_zeros;
    D.dn_codes = static_cast<const uint8_t*>(S.down.codes);
    D.dn_scales = static_cast<const uint8_t*>(S.down.scales);
    D.dn_zeros = static_cast<const uint8_t*>(S.down.zeros);
    D.dn_sc = S.down.expert_stride_codes;
    D.dn_ss = S.down.expert_stride_scales;
    D.dn_sz = S.down.expert_stride_zeros;
  }
  p->hl = host;
  hipError_t e2 = hipMemset(base + o_res0, 0, off - o_res0);
  if (e2 == hipSuccess) e2 = hipDeviceSynchronize();   // zeroed before any stream uses it
  hipError_t e3 = hipStreamCreateWithFlags(&p->cap_stream, hipStreamNonBlocking);
  if (e2 != hipSuccess || e3 != hipSuccess) {
    if (e3 == hipSuccess) (void)hipStreamDestroy(p->cap_stream);
    (void)hipFree(p->dev_base);
    delete[] p->wr;
    delete[] p->hl;
    delete p;
    return BDG_E_HIP;
  }
  p->clock = 0;
  *out = p;
  return BDG_OK;
}

extern "C" int moe_plan_destroy(bdg_plan* p) {
  if (!p) return BDG_OK;
  (void)hipStreamSynchronize(p->cap_stream);
  (void)hipDeviceSynchronize();
  for (int i = 0; i < kGraphCache; ++i) drop_graph(p->graphs[i]);
  (void)hipStreamDestroy(p->cap_stream);
  if (p->prof_ev) {
    for (int i = 0; i < 2 * p->prof_cap; ++i) (void)hipEventDestroy(p->prof_ev[i]);
    delete[] p->prof_ev;
    delete[] p->prof_kind;
  }
  if (p->tl_stamps) (void)hipFree(p->tl_stamps);
  (void)hipFree(p->dev_base);
  delete[] p->wr;
  delete[] p->hl;
  delete p;
  return BDG_OK;
}

extern "C" int64_t moe_expert_decode_timeline(bdg_plan* p, const void* x, int32_t x_dtype, float* y,
                                              uint64_t* stamps, int64_t max_stamps, void* stream) {
  if (!p || !x || !y || !stamps) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if (!aligned16(x) || !aligned16(y)) return BDG_E_ALIGN;
  if (!p->fused_ok) return BDG_E_UNSUPPORTED;
  const int64_t n = (int64_t)p->d.n_layers * p->fused_nblk * kLayerStamps;
  if (max_stamps < n) return BDG_E_INVALID;
  if (!p->tl_stamps && hipMalloc(&p->tl_stamps, n * sizeof(uint64_t)) != hipSuccess) {
    p->tl_stamps = nullptr;
    return BDG_E_NOMEM;
  }
  hipStream_t s = as_stream(stream);
  if (hipMemsetAsync(p->tl_stamps, 0, n * sizeof(uint64_t), s) != hipSuccess) return BDG_E_HIP;
  GraphKey key{x, x_dtype, 1, y, nullptr, nullptr, nullptr};
  p->tl_active = 1;
  const int st = enqueue_decode(p, key, s);
  p->tl_active = 0;
  if (st) return st;
  if (hipMemcpyAsync(stamps, p->tl_stamps, n * sizeof(uint64_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return BDG_E_HIP;
  return n;
}

extern "C" int moe_expert_decode_profiled(bdg_plan* p, const void* x, int32_t x_dtype, int32_t m, float* y,
                                          double* kernel_ms, int64_t* kernel_count, void* stream) {
  if (!p || !x || !y || !kernel_ms || !kernel_count || m < 1) return BDG_E_INVALID;
  if (m > p->d.max_m) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if (!aligned16(x) || !aligned16(y)) return BDG_E_ALIGN;
  const int need = 3 * p->d.n_layers + 1;   // at most route + gate_up + down per layer, + combine
  if (!p->prof_ev) {
    p->prof_ev = new (std::nothrow) hipEvent_t[2 * need];
    p->prof_kind = new (std::nothrow) int[need];
    if (!p->prof_ev || !p->prof_kind) return BDG_E_NOMEM;
    for (int i = 0; i < 2 * need; ++i)
      if (hipEventCreate(&p->prof_ev[i]) != hipSuccess) return BDG_E_HIP;
    p->prof_cap = need;
  }
  Prof prof{p->prof_ev, p->prof_kind, p->prof_cap, 0};
  GraphKey key{x, x_dtype, m, y, nullptr, nullptr, nullptr};
  hipStream_t s = as_stream(stream);
  int st = enqueue_decode(p, key, s, &prof);
  if (st) return st;
  if (hipEventSynchronize(p->prof_ev[2 * prof.used - 1]) != hipSuccess) return BDG_E_HIP;
  for (int i = 0; i < prof.used; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p->prof_ev[2 * i], p->prof_ev[2 * i + 1]) != hipSuccess) return BDG_E_HIP;
    kernel_ms[p->prof_kind[i]] += ms;
    kernel_count[p->prof_kind[i]] += 1;
  }
  return BDG_OK;
}

extern "C" int moe_plan_check(bdg_plan* p, void* stream) {
  if (!p) return BDG_E_INVALID;
  hipStream_t s = as_stream(stream);
  unsigned v = 0;
  if (hipMemcpyAsync(&v, p->fault, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return BDG_E_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return BDG_E_HIP;
  if (v == 0) return BDG_OK;
  const unsigned zero = 0;
  if (hipMemcpyAsync(p->fault, &zero, sizeof(zero), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return BDG_E_HIP;
  return BDG_E_WAIT;
}

extern "C" int moe_expert_decode(bdg_plan* p, const void* x, int32_t x_dtype, int32_t m, float* y,
                                 int32_t* topk_trace, float* wts_trace, float* resid_trace, void* stream) {
  if (!p || !x || !y || m < 1) return BDG_E_INVALID;
  if (m > p->d.max_m) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if (!aligned16(x) || !aligned16(y) || (resid_trace && !aligned16(resid_trace))) return BDG_E_ALIGN;
  GraphKey key{x, x_dtype, m, y, topk_trace, wts_trace, resid_trace};
  hipStream_t s = as_stream(stream);
  if (p->d.flags & BDG_MOE_NO_GRAPH) return enqueue_decode(p, key, s);
  GraphEntry* hit = nullptr;
  for (int i = 0; i < kGraphCache; ++i)
    if (p->graphs[i].used && p->graphs[i].key == key) hit = &p->graphs[i];
  if (!hit) {
    GraphEntry* slot = &p->graphs[0];
    for (int i = 0; i < kGraphCache; ++i) {
      if (!p->graphs[i].used) { slot = &p->graphs[i]; break; }
      if (p->graphs[i].stamp < slot->stamp) slot = &p->graphs[i];
    }
    if (slot->used) drop_graph(*slot);   // waits for that graph's last launch only
    if (hipStreamBeginCapture(p->cap_stream, hipStreamCaptureModeRelaxed) != hipSuccess) return BDG_E_HIP;
    int st = enqueue_decode(p, key, p->cap_stream);
    hipGraph_t graph = nullptr;
    hipError_t ee = hipStreamEndCapture(p->cap_stream, &graph);
    if (st || ee != hipSuccess || !graph) {
      if (graph) (void)hipGraphDestroy(graph);
      return st ? st : BDG_E_HIP;
    }
    hipGraphExec_t exec = nullptr;
    if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
      (void)hipGraphDestroy(graph);
      return BDG_E_HIP;
    }
    hipEvent_t done = nullptr;
    if (hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess) {
      (void)hipGraphExecDestroy(exec);
      (void)hipGraphDestroy(graph);
      return BDG_E_HIP;
    }
    slot->used = true;
    slot->key = key;
    slot->graph = graph;
    slot->exec = exec;
    slot->done = done;
    hit = slot;
  }
  hit->stamp = ++p->clock;
  if (hipGraphLaunch(hit->exec, s) != hipSuccess) return BDG_E_HIP;
  return hip_status(hipEventRecord(hit->done, s));
}

extern "C" int moe_experts_routed(bdg_plan* p, int32_t layer, const void* x, int32_t x_dtype, int32_t m,
                                  const int32_t* idx, const float* wts, float* y, void* stream) {
  if (!p || !x || !idx || !wts || !y || m < 1) return BDG_E_INVALID;
  if (m > p->d.max_m || layer < 0 || layer >= p->d.n_layers) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if (!aligned16(x)) return BDG_E_ALIGN;
  hipStream_t s = as_stream(stream);
  // x -> the plan's fp32 input buffer of `layer` (no norm, no logits)
  RouteParams rp{};
  rp.M = m;
  rp.H = p->d.hidden;
  rp.E = p->d.n_experts;
  rp.compute_logits = 0;
  rp.x_in = x;
  rp.x_bf16 = x_dtype == BDG_BF16 ? 1 : 0;
  rp.x_copy = p->resid[layer & 1];
  rp.part = p->part;
  rp.pstride = p->pstride;
  rp.L = p->hl[layer];
  const bool mfma = m > 1 && p->mfma;
  if (mfma) {   // also the bf16 operand parts of x (factor 1) for the matrix cores
    rp.xh = p->xh;
    rp.xl = p->xl;
  }
  hipLaunchKernelGGL(moe_route_kernel, dim3(1, m), dim3(kThreads), (size_t)(rp.H + kWaves) * sizeof(float), s,
                     rp);
  int st = launch_status();
  if (st) return st;
  // gate_up runs on the raw x (no norm), routing from the caller
  if (mfma) {
    st = launch_mfma_pair(p, mfma_params(p, layer, m, 1, idx, wts, nullptr, nullptr, 0), s, nullptr);
    if (st) return st;
    return launch_combine(p, m, p->resid[layer & 1], 0, y, s, nullptr);
  }
  if (m > 1 && p->group_ok) {
    st = launch_gu_group(p, layer, m, 1, idx, wts, nullptr, nullptr, 0, s, nullptr);
    if (st) return st;
    st = launch_dn_group(p, layer, s, nullptr);
    if (st) return st;
    return launch_combine(p, m, p->resid[layer & 1], 0, y, s, nullptr);
  }
  st = launch_gateup(p, layer, m, 1, 1, idx, wts, nullptr, nullptr, 0, s, nullptr);
  if (st) return st;
  return launch_down(p, layer, m, 0, nullptr, y, nullptr, 0, s, nullptr);
}
