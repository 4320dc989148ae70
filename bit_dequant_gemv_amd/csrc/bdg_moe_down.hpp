// The per-token down kernel (steps of M = 1, and per-token steps of M > 1):
// grouped down dequant-GEMV over h, router-weighted combine, residual, and
// in a stack the next layer's router partial sums.  Its many shape variants
// compile in a unit of their own (moe_down.hip), beside the rest of the
// decode path.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "bdg_host.hpp"
#include "bdg_moe.hpp"

namespace bdg {

struct DownParams {
  int M, H, I, E, K;
  const int32_t* idx;         // [M][K] routing buffer
  const float* h;             // [M][K][I]
  DownOut o;                  // combine, residual, outputs, next layer's router slice
  LayerDev L;                 // this layer's weights
  QGeom g;                    // reduction over I
  unsigned* seq_bump;         // or NULL: the token sequence number, advanced by block (0, 0)
};

// Block (rb, t) of 8 waves: WPE = 8 / K waves per chosen expert (1 when
// K >= 8; experts then go in groups of 8).  Wave w works on expert slot
// j = jg + w % K' and row groups (w / K'), (w / K') + WPE, ... of the block's
// B = NR * RPW * WPE rows.  The h_j of a group are staged into LDS by the whole
// block (loads issued before the expert weights' loads), the partial rows
// meet in LDS and are combined in slot order with the residual.
template <int FMT, int L, int S, int NR, int HV, int RW>
__global__ void __launch_bounds__(kDownWaves * kWave) moe_down_kernel(DownParams p) {
  constexpr int RPW = kWave / L;
  extern __shared__ float lds[];
  const int kg = p.K < kDownWaves ? p.K : kDownWaves;      // experts per group
  const int wpe = kDownWaves / kg;                          // waves per expert
  const int B = NR * RPW * wpe;
  const int stride = (p.g.chunks + 1) * kXStride;          // per expert: chunks of h, then a zero chunk
  float* dpart = lds + kg * stride;                         // [K][B]
  const int t = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  const int li = lane % L;
  const int rr = lane / L;
  const int r0 = blockIdx.x * B;
  const int jw = wave % kg;                                 // expert within the group
  const int sub = wave / kg;                                // row-group phase (sub < wpe, or idle)
  const bool wave_on = sub < wpe;
  const LayerDev& Ld = p.L;

  // One group of kg experts: h vectors staged through LDS, the expert rows'
  // dot products into dpart.  hstage holds the group's h loads, issued by the
  // caller before anything else it needs later.
  auto group = [&](int jg, int e, StageF32<HV>& hstage) {
    const int nj = min(kg, p.K - jg);
    const bool active = wave_on && jw < nj;
    const int nh = nj * p.I;
    GroupLoad<FMT, S> ld[NR];
    const QMat m = expert_dn(Ld, e);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int row = r0 + (i * wpe + sub) * RPW + rr;
      load_row<FMT, L, S>(ld[i], m, p.g, row, active && row < p.H, li);
    }
    hstage.store(lds, nh, p.I, stride, 1.0f, threadIdx.x, blockDim.x);
    block_sync_lds();   // weights still in flight
    if (active) {
      XRegs<FMT, L, S> xr;
      xr.load_zpad(lds + jw * stride, p.g.chunks, li);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const float d = row_dot<FMT, L, S>(ld[i], xr);
        const int b = (i * wpe + sub) * RPW + rr;
        if (li == kRowSumLane<L> && b < B) dpart[(jg + jw) * B + b] = d;
      }
    }
    block_sync_lds();
  };

  // loads, in the order their data is needed (vmcnt retires in order): the
  // first group's expert id and h vectors, the epilogue operands (router
  // weights of the next layer, residual row, combine weights: all in bounds,
  // issued unconditionally so the compiler's wait counts stay exact), then
  // the expert weights.  The first group is outside the loop so no loop
  // back edge makes the compiler wait for everything before the weights.
  const int e0 = clamp_expert(p.idx[t * p.K + (jw < p.K ? jw : p.K - 1)], p.E);
  StageF32<HV> h0;
  h0.load(p.h + (int64_t)t * p.K * p.I, min(kg, p.K) * p.I, threadIdx.x, blockDim.x);
  __builtin_amdgcn_sched_barrier(0);   // keep the issue order: the scheduler would sink loads
  DownEpiIn<RW> epi;
  down_epilogue_load(epi, p.o, t, r0, B, lane, wave);
  epi.wk = p.o.w[t * p.K + (lane < p.K ? lane : p.K - 1)];
  __builtin_amdgcn_sched_barrier(0);
  // the zero chunk after each expert's h (h staging never writes it); no
  // branch: threads past the kg chunks repeat the last one's stores
  {
    const int zr = min((int)(threadIdx.x / kChunkElems), kg - 1);
    lds[zr * stride + p.g.chunks * kXStride + (threadIdx.x & (kChunkElems - 1))] = 0.f;
  }
  group(0, e0, h0);
  for (int jg = kg; jg < p.K; jg += kg) {   // K > 8 only
    const int jn = jg + (jw < p.K - jg ? jw : p.K - jg - 1);
    const int e = clamp_expert(p.idx[t * p.K + jn], p.E);
    StageF32<HV> hs;
    hs.load(p.h + ((int64_t)t * p.K + jg) * p.I, min(kg, p.K - jg) * p.I, threadIdx.x, blockDim.x);
    group(jg, e, hs);
  }

  // after a self-routing first layer: the next token's tags differ from
  // this one's (issued after every load of the block, so no wait covers it)
  if (p.seq_bump && blockIdx.x == 0 && t == 0 && threadIdx.x == 0)
    __hip_atomic_fetch_add(p.seq_bump, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (B <= kWave) {
    down_epilogue(p.o, epi, dpart, t, blockIdx.x, r0, B, lane, wave);
    return;
  }
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int row = r0 + b;
    if (row >= p.H) continue;
    float v = p.o.residual ? p.o.x_prev[(int64_t)t * p.H + row] : 0.f;
    for (int j = 0; j < p.K; ++j) v = __builtin_fmaf(p.o.w[t * p.K + j], dpart[j * B + b], v);
    if (p.o.x_out) p.o.x_out[(int64_t)t * p.H + row] = v;
    if (p.o.y_out) p.o.y_out[(int64_t)t * p.H + row] = v;
    if (p.o.trace_out) p.o.trace_out[(int64_t)t * p.H + row] = v;
  }
}


// Launch the variant (FMT, L, S, NR, HV) of moe_down_kernel with RW router
// rows per wave; BDG_E_UNSUPPORTED when it was not compiled.
template <int RW>
int launch_down_variant(const DownParams& dp, int fmt, int L, int S, int NR, int HV, dim3 grid, size_t lds,
                        hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
#define BDG_DN_CASE(F, LL, SS, NN, HH)                                                                 \
  if (fmt == F && L == LL && S == SS && NR == NN && HV == HH) {                                       \
    if (ev_start)                                                                                      \
      hipExtLaunchKernelGGL((moe_down_kernel<F, LL, SS, NN, HH, RW>), grid, dim3(kDownWaves * kWave), \
                            lds, s, ev_start, ev_stop, 0, dp);                                         \
    else                                                                                               \
      hipLaunchKernelGGL((moe_down_kernel<F, LL, SS, NN, HH, RW>), grid, dim3(kDownWaves * kWave),    \
                         lds, s, dp);                                                                  \
    return launch_status();                                                                            \
  }
#define BDG_DN_HV(F, LL, SS, NN) \
  BDG_DN_CASE(F, LL, SS, NN, 2) BDG_DN_CASE(F, LL, SS, NN, 4) BDG_DN_CASE(F, LL, SS, NN, 6) \
  BDG_DN_CASE(F, LL, SS, NN, 8) BDG_DN_CASE(F, LL, SS, NN, 12)
#define BDG_DN_NR(F, LL, SS) \
  BDG_DN_HV(F, LL, SS, 1) BDG_DN_HV(F, LL, SS, 2) BDG_DN_HV(F, LL, SS, 3) BDG_DN_HV(F, LL, SS, 4)
#define BDG_DN_ALL(F)                                                             \
  BDG_DN_NR(F, 8, 1) BDG_DN_NR(F, 8, 2) BDG_DN_NR(F, 8, 3) BDG_DN_NR(F, 16, 2)   \
  BDG_DN_NR(F, 16, 3) BDG_DN_NR(F, 32, 2) BDG_DN_NR(F, 32, 3) BDG_DN_NR(F, 64, 2) \
  BDG_DN_NR(F, 64, 3) BDG_DN_NR(F, 64, 4)
  BDG_DN_ALL(kMXFP4)
  BDG_DN_ALL(kINT4G)
#undef BDG_DN_ALL
#undef BDG_DN_NR
#undef BDG_DN_HV
#undef BDG_DN_CASE
  return BDG_E_UNSUPPORTED;
}

// The compiled family (kDnRouterPerWave router rows per wave).
int launch_down_kernel(const DownParams& dp, int fmt, int L, int S, int NR, int HV, dim3 grid, size_t lds,
                       hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace bdg
