// One MoE layer of a single-token decode step in one kernel: routing,
// grouped gate_up + SwiGLU, grouped down + combine (+ residual and the next
// layer's router partial sums).
//
// The pages run each chosen expert's two GEMVs one after another ("Sovereign
// gpt-oss-20B (MXFP4) on Apple Silicon", section 3: dispatch/latency-bound)
// and leave running the active experts together untried (section 5); the
// TinyTitan tracker puts a layer's experts into one submission (entry D114).
// On the two-kernel path (moe.hip) a layer's down weights are read only once
// its gate_up kernel has finished, and each of the two kernels pays a launch
// and the latency of its first loads.  Here the down weights' addresses are
// known as soon as the block has selected the experts, so the block streams
// its share of them straight into LDS (global_load_lds, no registers) right
// behind its gate_up weights; HBM stays busy through the gate_up arithmetic
// and through the one exchange the layer needs, h.
//
// Block (512 threads, 8 waves) b of a grid of nblk co-resident blocks:
//   1. routing: adds the router partial sums, RMSNorm scale, bias, top-k
//      (every wave, as the gate_up kernel does);
//   2. gate_up: wave gw = 8b + w owns pairs [P gw / GW, P (gw+1) / GW) of the
//      P = K*I (g, u) row pairs; their weights load into registers;
//   3. waves 0..6 of blocks b < dn_blocks issue the codes of the block's down
//      rows (B rows of each chosen expert) into LDS, one 1 KB slab per
//      (row group, slot);
//   4. gate_up arithmetic and SwiGLU; the block's h values meet in LDS;
//   5. wave 7 (which issued no down loads, so waiting for its stores does not
//      wait for the down stream: vmcnt retires in order) writes them to
//      memory with device-coherent stores and arrives at a grid barrier;
//   6. every block reads the whole h (device-coherent loads) into LDS, the
//      waves that loaded down codes take their scales and compute their
//      rows from LDS, and the rows are combined as in the down kernel.
// The barrier is a counter and a generation word updated with device-scope
// relaxed atomics, the data ordered by waiting for the stores before the
// arrival; its wait is bounded (a wait that gives up sets the plan's fault
// word and makes the block's outputs NaN), so every wave exits.
//
// Measured on MI355X this path is slower than the two kernels, and it is
// opt-in (BDG_MOE_FUSED_LAYER) for A/B measurement: a wave's loads retire
// in order and the compiler waits for every load issued before a direct-to-
// LDS load before it uses any of them, so the gate_up arithmetic cannot run
// ahead of the down stream; and the grid barrier plus the h exchange cost
// about what the kernel boundary they replace costs.
#include <algorithm>

#include "bdg_host.hpp"
#include "bdg_moe.hpp"
#include "bdg_moe_layer.hpp"

namespace bdg {

constexpr int kLayerWaves = 8;
constexpr int kLayerThreads = kLayerWaves * kWave;
constexpr int kHWriter = kLayerWaves - 1;     // writes the block's h; loads no down weights
constexpr int kDnLoadWaves = kLayerWaves - 1;  // waves that load and compute down rows
constexpr int kSlabFloats = kWave * 4;         // one 16-byte chunk per lane: 1 KB

#define BDG_LDS_AS __attribute__((address_space(3)))

// Issue a row's code chunks straight into LDS: slot s of lane `lane` lands at
// slab + s * kSlabFloats + lane * 4 (the load unit writes 16 bytes per lane,
// lane-contiguous).  Clamped like load_row: every global address in bounds.
template <int L, int S>
__device__ __forceinline__ void issue_codes_lds(float* slab, const QMat& m, const QGeom& g, int64_t row, bool row_ok,
                                                int li) {
  const uint32_t r = row_ok ? (uint32_t)row : 0u;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = li + L * s;
    const uint32_t cc = (uint32_t)(c < g.chunks ? c : g.chunks - 1);
    const uint8_t* src = m.codes + (r * (uint32_t)g.chunks + cc) * 16u;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const BDG_GLOBAL void*>(reinterpret_cast<uintptr_t>(src)),
                                     (BDG_LDS_AS void*)(slab + s * kSlabFloats), 16, 0, 0);
  }
}

// The scales (and int4 zero points) of a row whose codes issue_codes_lds
// loaded, into ld (codes left untouched), with load_row's clamping.
template <int FMT, int L, int S>
__device__ __forceinline__ void load_row_scales(GroupLoad<FMT, S>& ld, const QMat& m, const QGeom& g, int64_t row,
                                                bool row_ok, int li) {
  const uint32_t r = row_ok ? (uint32_t)row : 0u;
  ld.ok = 0;
  ld.zhi = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = li + L * s;
    const bool ok = row_ok && c < g.chunks;
    const uint32_t cc = (uint32_t)(c < g.chunks ? c : g.chunks - 1);
    ld.ok |= (ok ? 1u : 0u) << s;
    if constexpr (FMT == kMXFP4) {
      ld.sc[s] = ldg_u8(m.scales + (r * (uint32_t)g.chunks + cc));
      ld.zn[s] = 0;
    } else {
      const uint32_t gi = (cc * kChunkElems) / (uint32_t)g.group;
      ld.sc[s] = ldg_u16(m.scales + (r * (uint32_t)g.groups + gi) * 2u);
      ld.zn[s] = ldg_u8(m.zeros + (r * (uint32_t)g.zrow + (gi >> 1)));
      ld.zhi |= (gi & 1u) << s;
    }
  }
}

// Grid barrier of one lane per block: arrive, then wait (at most `polls`
// polls) for the generation word to move on.  Returns false when the wait
// gave up.  The caller has waited for its stores to complete (they were
// device-coherent), so every block that sees the new generation sees them.
__device__ __forceinline__ bool grid_barrier_lane(unsigned* bar, unsigned nblk, int polls) {
  unsigned* count = bar;
  unsigned* gen = bar + 32;   // its own 128-byte line
  const unsigned g0 = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);   // g0 read before this block arrives
  const unsigned t = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (t == nblk - 1) {
    __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __hip_atomic_fetch_add(gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  for (int i = 0; i < polls; ++i) {
    if (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != g0) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Timeline mode: lane 0 of `wave` stamps the 100 MHz clock for phase `ph`
// (a uniform branch on a kernel argument when off).
__device__ __forceinline__ void stamp(const LayerParams& p, int wave, int want_wave, int ph) {
  if (p.stamps && wave == want_wave && (threadIdx.x & (kWave - 1)) == 0)
    p.stamps[blockIdx.x * kLayerStamps + ph] = __builtin_amdgcn_s_memrealtime();
}

// FMT: weight format; SG: gate_up slots; NP: (g, u) pairs per wave; V: top-k
// values per lane; LD / SD: down lanes per row / slots; NG: down row groups
// per loading wave; NHL: h values per thread in the exchange.
template <int FMT, int SG, int NP, int V, int LD, int SD, int NG, int NHL>
__global__ void __launch_bounds__(kLayerThreads) moe_layer_kernel(LayerParams p) {
  constexpr int LG = 32;                                    // gate_up lanes per row
  constexpr int RPW = kWave / LD;                           // down rows per row group
  extern __shared__ float lds[];
  const int gchunks = p.g_gu.chunks, dchunks = p.g_dn.chunks;
  float* slabs = lds;                                       // [kDnLoadWaves][NG][SD][kSlabFloats]
  float* xs = slabs + kDnLoadWaves * NG * SD * kSlabFloats; // x chunks (gate_up), later h chunks (down)
  const int hstride = (dchunks + 1) * kXStride;             // per expert: h chunks, then a zero chunk
  const int a_floats = max((gchunks + 1) * kXStride, p.K * hstride);
  float* red = xs + a_floats;                               // [kLayerWaves]
  float* psum = red + kLayerWaves;                          // [E << log2T]
  float* hblk = psum + (p.E << p.rt.log2T);                 // [kLayerWaves][NP]
  float* dpart = hblk + kLayerWaves * NP;                   // [K][B]
  int* flag = reinterpret_cast<int*>(dpart + p.K * p.B);    // [1]: the barrier wait gave up

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  const int lg = lane % LG;
  const bool is_up = lane >= LG;
  const LayerDev& Ld = p.L;

  stamp(p, wave, kHWriter, kStStart);
  // 1. routing inputs, then x (independent of the routing)
  RouteState<V> rs;
  route_issue<V, kLayerThreads>(rs, p.rt, 0, lane);
  constexpr int NX = kRouteMaxF4 * kWave / kLayerThreads;   // H <= 4096
  StageF32<NX> xstage;
  xstage.load(p.x, p.H, threadIdx.x, kLayerThreads);

  // this wave's pair range (independent of the routing)
  const int P = p.K * p.I;
  const int GW = gridDim.x * kLayerWaves;
  const int gw = blockIdx.x * kLayerWaves + wave;
  const int q0 = (int)((int64_t)P * gw / GW);
  const int nq = (int)((int64_t)P * (gw + 1) / GW) - q0;   // <= NP
  const int j0 = q0 / p.I;
  const int row0 = q0 - j0 * p.I;

  route_finish<V, kLayerThreads>(rs, p.rt, 0, lane, wave, red, psum);
  const int my_e = rs.my_e;
  const float my_w = rs.my_w;
  stamp(p, wave, kHWriter, kStRouted);
  if (blockIdx.x == 0 && wave == 0 && lane < p.K) {
    p.idx_out[lane] = my_e;
    p.w_out[lane] = my_w;
    if (p.topk_trace) p.topk_trace[lane] = my_e;
    if (p.wts_trace) p.wts_trace[lane] = my_w;
  }

  // 2. gate_up weights into registers (a wave short of NP pairs repeats its
  // last pair and stores nothing for the repeats)
  GroupLoad<FMT, SG> ld[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int ii = i < nq ? i : (nq > 0 ? nq - 1 : 0);
    int row = row0 + ii;
    int j = j0;
    while (row >= p.I) {
      row -= p.I;
      ++j;
    }
    if (j >= p.K) j = p.K - 1;
    const int e = __builtin_amdgcn_readlane(my_e, j);
    load_row<FMT, LG, SG>(ld[i], expert_gu(Ld, e), p.g_gu, is_up ? p.I + row : row, true, lg);
  }

  stamp(p, wave, kHWriter, kStGuIssued);
  // 3. this block's down codes into LDS.  Row group g < G = K * (B / RPW)
  // covers rows r0 + (g % gpe) * RPW + rr of expert slot g / gpe; loading
  // wave w takes groups w, w + 7, ...
  const bool dn_block = (int)blockIdx.x < p.dn_blocks;
  const int r0 = blockIdx.x * p.B;
  const int gpe = p.B / RPW;
  const int G = p.K * gpe;
  const int ld_dn = lane % LD;
  const int rr = lane / LD;
  const bool dn_wave = dn_block && wave < kDnLoadWaves;
  if (dn_wave) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int g = wave + kDnLoadWaves * i;
      const bool gok = g < G;
      const int gc = gok ? g : 0;
      const int j = gc / gpe;
      const int row = r0 + (gc - j * gpe) * RPW + rr;
      const int e = __builtin_amdgcn_readlane(my_e, j);
      issue_codes_lds<LD, SD>(slabs + (wave * NG + i) * SD * kSlabFloats, expert_dn(Ld, e), p.g_dn, row,
                              gok && row < p.H, ld_dn);
    }
  }

  stamp(p, wave, 0, kStDnIssued);
  // 4. gate_up arithmetic
  xstage.store(xs, p.H, p.H, 0, rs.r, threadIdx.x, kLayerThreads);
  xs[gchunks * kXStride + (threadIdx.x & (kChunkElems - 1))] = 0.f;   // the zero chunk (no branch)
  __syncthreads();
  {
    XRegs<FMT, LG, SG> xr;
    xr.load_zpad(xs, gchunks, lg);
    float g_sel = 0.f, u_sel = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const float d = row_dot<FMT, LG, SG>(ld[i], xr);
      const float gv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), kRowSumLane<LG>));
      const float uv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), LG + kRowSumLane<LG>));
      if (lane == i) {
        g_sel = gv;
        u_sel = uv;
      }
    }
    if (lane < NP) hblk[wave * NP + lane] = g_sel / (1.0f + expf(-g_sel)) * u_sel;
  }
  // the down rows' scales: their wait overlaps the exchange below
  GroupLoad<FMT, SD> dl[NG];
  if (dn_wave) {
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int g = wave + kDnLoadWaves * i;
      const bool gok = g < G;
      const int gc = gok ? g : 0;
      const int j = gc / gpe;
      const int row = r0 + (gc - j * gpe) * RPW + rr;
      const int e = __builtin_amdgcn_readlane(my_e, j);
      load_row_scales<FMT, LD, SD>(dl[i], expert_dn(Ld, e), p.g_dn, row, gok && row < p.H, ld_dn);
    }
  }
  block_sync_lds();   // every wave's h in hblk; every wave done with xs
  stamp(p, wave, kHWriter, kStGuDone);

  // 5. the block's h to memory (device-coherent stores), then the barrier
  if (wave == kHWriter) {
    const int gw0 = blockIdx.x * kLayerWaves;
    for (int idx = lane; idx < kLayerWaves * NP; idx += kWave) {
      const int w = idx / NP, i = idx - w * NP;
      const int qa = (int)((int64_t)P * (gw0 + w) / GW);
      const int na = (int)((int64_t)P * (gw0 + w + 1) / GW) - qa;
      if (i < na) __hip_atomic_store(p.hbuf + qa + i, hblk[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);   // the stores are complete before this block arrives
    stamp(p, wave, kHWriter, kStHStored);
    int ok = 1;
    if (lane == 0) ok = grid_barrier_lane(p.bar, gridDim.x, p.wait_polls) ? 1 : 0;
    if (lane == 0) {
      flag[0] = ok ? 0 : 1;
      if (!ok) __hip_atomic_store(p.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  block_sync_lds();
  stamp(p, wave, kHWriter, kStBarrier);
  if (!dn_block) return;

  // 6. the whole h (device-coherent loads: other blocks wrote it) into the
  // LDS chunk layout, one region per expert slot, then the epilogue operands
  const int KI = p.K * p.I;
  float hv[NHL];
#pragma unroll
  for (int n = 0; n < NHL; ++n) {
    const int idx = min((int)threadIdx.x + kLayerThreads * n, KI - 1);
    hv[n] = __hip_atomic_load(p.hbuf + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  DownEpiIn<kDnRouterPerWave> epi;
  down_epilogue_load(epi, p.o, 0, r0, p.B, lane, wave);
  epi.wk = my_w;
  const float poison = flag[0] ? __uint_as_float(0x7FC00000u) : 0.f;   // NaN after a failed wait
#pragma unroll
  for (int n = 0; n < NHL; ++n) {
    const int idx = (int)threadIdx.x + kLayerThreads * n;
    if (idx < KI) {
      const int j = idx / p.I, k = idx - j * p.I;
      xs[j * hstride + (k >> 5) * kXStride + (k & 31)] = hv[n] + poison;
    }
  }
  for (int z = threadIdx.x; z < p.K * kChunkElems; z += kLayerThreads)   // each expert's zero chunk
    xs[(z >> 5) * hstride + dchunks * kXStride + (z & 31)] = 0.f;
  __syncthreads();
  stamp(p, wave, 0, kStHStaged);

  // down rows from LDS
  if (dn_wave) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's LDS loads have landed
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int g = wave + kDnLoadWaves * i;
      if (g < G) {                   // wave-uniform
        const int j = g / gpe;
        const float* slab = slabs + (wave * NG + i) * SD * kSlabFloats;
#pragma unroll
        for (int s = 0; s < SD; ++s) dl[i].q[s] = *reinterpret_cast<const uint4*>(slab + s * kSlabFloats + lane * 4);
        XRegs<FMT, LD, SD> hr;
        hr.load_zpad(xs + j * hstride, dchunks, ld_dn);
        const float d = row_dot<FMT, LD, SD>(dl[i], hr);
        const int b = (g - j * gpe) * RPW + rr;
        if (ld_dn == kRowSumLane<LD>) dpart[j * p.B + b] = d;
      }
    }
  }
  __syncthreads();
  stamp(p, wave, 0, kStDnDone);
  down_epilogue(p.o, epi, dpart, 0, blockIdx.x, r0, p.B, lane, wave);
  stamp(p, wave, 0, kStEnd);
}

// ---------------------------------------------------------------- host side

int layer_fused_lds_bytes(const LayerShape& s, int np, int ng, int sd) {
  const int a = std::max((s.g_gu.chunks + 1) * kXStride, s.K * (s.g_dn.chunks + 1) * kXStride);
  const size_t floats = (size_t)kDnLoadWaves * ng * sd * kSlabFloats + a + kLayerWaves + ((size_t)s.E << s.log2T) +
                        (size_t)kLayerWaves * np + (size_t)s.K * s.B + 4;
  return (int)(floats * sizeof(float));
}

template <int FMT, int SG, int NP, int V, int LD, int SD, int NG, int NHL>
static const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&moe_layer_kernel<FMT, SG, NP, V, LD, SD, NG, NHL>);
}

// The instantiations the plan can pick: gpt-oss shapes (MXFP4, K = 2880:
// SG = 3, LD = 32, SD = 3) and the 30B int4 shape (int4, H = 2048, I = 768:
// SG = 2, LD = 8, SD = 3), with the pair, group and exchange counts their
// grids give; other shapes stay on the two-kernel path.
#define BDG_LAYER_VARIANTS(X)                   \
  X(kMXFP4, 3, 6, 1, 32, 3, 4, 24)              \
  X(kMXFP4, 3, 6, 2, 32, 3, 4, 24)              \
  X(kINT4G, 2, 3, 2, 8, 3, 2, 12)               \
  X(kINT4G, 2, 3, 1, 8, 3, 2, 12)

const void* layer_fused_kernel(const LayerConfig& c) {
#define BDG_PICK(F, SG_, NP_, V_, LD_, SD_, NG_, NHL_)                                                      \
  if (c.fmt == F && c.sg == SG_ && c.np == NP_ && c.v == V_ && c.ld == LD_ && c.sd == SD_ && c.ng == NG_ && \
      c.nhl == NHL_)                                                                                         \
    return kernel_ptr<F, SG_, NP_, V_, LD_, SD_, NG_, NHL_>();
  BDG_LAYER_VARIANTS(BDG_PICK)
#undef BDG_PICK
  return nullptr;
}

int launch_layer_fused(const LayerConfig& c, const LayerParams& lp, int nblk, size_t lds, hipStream_t s,
                       hipEvent_t ev_start, hipEvent_t ev_stop) {
#define BDG_LAUNCH_ONE(F, SG_, NP_, V_, LD_, SD_, NG_, NHL_)                                                \
  if (c.fmt == F && c.sg == SG_ && c.np == NP_ && c.v == V_ && c.ld == LD_ && c.sd == SD_ && c.ng == NG_ && \
      c.nhl == NHL_) {                                                                                       \
    hipExtLaunchKernelGGL((moe_layer_kernel<F, SG_, NP_, V_, LD_, SD_, NG_, NHL_>), dim3(nblk),             \
                          dim3(kLayerThreads), lds, s, ev_start, ev_stop, 0, lp);                            \
    return launch_status();                                                                                  \
  }
  BDG_LAYER_VARIANTS(BDG_LAUNCH_ONE)
#undef BDG_LAUNCH_ONE
  return BDG_E_UNSUPPORTED;
}

int layer_threads() { return kLayerThreads; }
int layer_dn_load_waves() { return kDnLoadWaves; }

}  // namespace bdg
