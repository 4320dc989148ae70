// Sparse-MoE expert decode: router, top-k, grouped gate_up + SwiGLU,
// grouped down, router-weighted combine (+ RMSNorm residual stack).
//
// Per layer the pages run a router and then the chosen experts one after
// another, two small GEMVs each, one submission per GEMV ("Sovereign
// gpt-oss-20B (MXFP4) on Apple Silicon", section 3: "4 sequential experts x
// 2 small-block GEMVs", dispatch-bound); running the active experts together
// is named there as the untried lever (section 5), and the TinyTitan tracker
// moves a layer's experts into one submission (entry D114).  Here each layer
// is three kernels, each over ALL chosen experts of the layer:
//   route  : combine of the previous layer + residual, RMSNorm, router GEMV
//   gate_up: top-k + softmax (every block, from the logits), then the
//            grouped gate_up dequant-GEMV of all k experts with the SwiGLU
//            epilogue h = silu(g) * u
//   down   : grouped down dequant-GEMV of all k experts -> d_j
// and the combine y = x + sum_j w_j d_j is folded into the next layer's
// route kernel (or a final finish kernel).  A whole token is one captured
// HIP graph (per-token setup amortised as in the host-sync page, section 3).
#include <stdlib.h>
#include <string.h>

#include <hip/hip_ext.h>

#include <new>

#include "bdg_gemv.hpp"
#include "bdg_host.hpp"

namespace bdg {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRouteRowsPerBlock = 8;

// Weight addresses of one layer, kept in a device table by the plan.
struct LayerDev {
  const float* w_r;
  const float* b_r;
  const uint8_t* gu_codes;
  const uint8_t* gu_scales;
  const uint8_t* gu_zeros;
  int64_t gu_sc, gu_ss, gu_sz;
  const uint8_t* dn_codes;
  const uint8_t* dn_scales;
  const uint8_t* dn_zeros;
  int64_t dn_sc, dn_ss, dn_sz;
};

__device__ __forceinline__ QMat expert_gu(const LayerDev& L, int e) {
  return QMat{L.gu_codes + (int64_t)e * L.gu_sc, L.gu_scales + (int64_t)e * L.gu_ss,
              L.gu_zeros ? L.gu_zeros + (int64_t)e * L.gu_sz : nullptr};
}
__device__ __forceinline__ QMat expert_dn(const LayerDev& L, int e) {
  return QMat{L.dn_codes + (int64_t)e * L.dn_sc, L.dn_scales + (int64_t)e * L.dn_ss,
              L.dn_zeros ? L.dn_zeros + (int64_t)e * L.dn_sz : nullptr};
}

// x_new = (residual ? x_prev : 0) + sum_j w_j d_j, in fixed j order.  Used by
// both the route kernel (next layer's input) and the finish kernel (output),
// so the two agree bit for bit.
__device__ __forceinline__ float combine_elem(const float* __restrict__ x_prev, const float* __restrict__ d,
                                              const float* __restrict__ w, int K, int H, int t, int h,
                                              int residual) {
  float v = residual ? x_prev[(int64_t)t * H + h] : 0.f;
  for (int j = 0; j < K; ++j) v = __builtin_fmaf(w[t * K + j], d[((int64_t)t * K + j) * H + h], v);
  return v;
}

// ---------------------------------------------------------------- top-k

__device__ __forceinline__ bool better(float a, int ea, float b, int eb) {
  return a > b || (a == b && ea < eb);
}

// One wavefront: the K largest of row[0..E) (descending, ties -> lower index)
// and softmax weights over them.  Lane j < K writes pick j to out_idx/out_w.
__device__ void wave_topk(const float* __restrict__ row, int E, int K, int* out_idx, float* out_w) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int V = BDG_MAX_EXPERTS / kWave;
  float v[V];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < E ? row[e] : -INFINITY;
    if (e >= E) taken |= 1u << i;
  }
  float my_l = 0.f;
  int my_e = 0;
  for (int j = 0; j < K; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = lane + kWave * i;
      if (!((taken >> i) & 1u) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) {
      const float ov = __shfl_xor(bv, msk);
      const int oe = __shfl_xor(be, msk);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if (be >= E) be = E - 1;   // only when every remaining logit is NaN
    if (lane == (be & (kWave - 1))) taken |= 1u << (be / kWave);
    if (lane == j) {
      my_l = bv;
      my_e = be;
    }
  }
  const float l0 = __shfl(my_l, 0);
  const float ex = lane < K ? expf(my_l - l0) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < K) {
    out_idx[lane] = my_e;
    out_w[lane] = ex / sum;
  }
}

// ---------------------------------------------------------------- route

struct RouteParams {
  int M, H, E, K;
  int combine;        // 0: x_new = x_in; 1: x_new = combine(x_prev, d_prev, w_prev)
  int residual;       // combine adds x_prev
  int norm;           // RMSNorm before routing / experts
  float eps;
  int compute_logits;
  const void* x_in;
  int x_bf16;
  const float* x_prev;
  const float* d_prev;
  const float* w_prev;
  float* x_out;        // [M][H], written by block 0
  float* resid_trace;  // [M][H] or NULL, written by block 0
  float* r_out;        // [M], written by block 0
  float* logits;       // [M][E]
  const LayerDev* layers;
  int layer;
};

__global__ void __launch_bounds__(kThreads) moe_route_kernel(RouteParams p) {
  extern __shared__ float lds[];
  float* xs = lds;               // [H]
  float* red = lds + p.H;        // [kWaves]
  const int t = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  float ss = 0.f;
  for (int h = threadIdx.x; h < p.H; h += kThreads) {
    float v;
    if (p.combine) {
      v = combine_elem(p.x_prev, p.d_prev, p.w_prev, p.K, p.H, t, h, p.residual);
    } else {
      v = p.x_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(p.x_in)[(int64_t)t * p.H + h])
                   : reinterpret_cast<const float*>(p.x_in)[(int64_t)t * p.H + h];
    }
    xs[h] = v;
    ss = __builtin_fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float r = 1.f;
  if (p.norm) {
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    r = 1.0f / sqrtf(tot / (float)p.H + p.eps);
  }
  if (blockIdx.x == 0) {
    for (int h = threadIdx.x; h < p.H; h += kThreads) {
      p.x_out[(int64_t)t * p.H + h] = xs[h];
      if (p.resid_trace) p.resid_trace[(int64_t)t * p.H + h] = xs[h];
    }
    if (threadIdx.x == 0) p.r_out[t] = r;
  }
  if (!p.compute_logits) return;
  const LayerDev L = p.layers[p.layer];
  const int e0 = blockIdx.x * kRouteRowsPerBlock;
  for (int e = e0 + wave; e < e0 + kRouteRowsPerBlock && e < p.E; e += kWaves) {
    const float* wr = L.w_r + (int64_t)e * p.H;
    float acc = 0.f;
    for (int h = lane * 4; h < p.H; h += kWave * 4) {
      const float4 wv = *reinterpret_cast<const float4*>(wr + h);
      acc = __builtin_fmaf(wv.x, xs[h] * r, acc);
      acc = __builtin_fmaf(wv.y, xs[h + 1] * r, acc);
      acc = __builtin_fmaf(wv.z, xs[h + 2] * r, acc);
      acc = __builtin_fmaf(wv.w, xs[h + 3] * r, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) p.logits[(int64_t)t * p.E + e] = acc + (L.b_r ? L.b_r[e] : 0.f);
  }
}

// ---------------------------------------------------------------- gate_up + SwiGLU

struct GateUpParams {
  int M, H, I, E, K;
  int routed;                 // 1: routing given in idx_in / w_in
  const float* logits;        // [M][E]
  const int32_t* idx_in;
  const float* w_in;
  int32_t* idx_out;           // [M][K] routing buffer, written by block 0
  float* w_out;
  int32_t* topk_trace;        // [M][K] or NULL
  float* wts_trace;
  const float* x;             // [M][H] layer input (fp32)
  const float* r;             // [M] norm scale or NULL
  const LayerDev* layers;
  int layer;
  QGeom g;                    // reduction over H
  float* h_out;               // [M][K][I]
};

template <int FMT, int S>
__global__ void __launch_bounds__(kThreads) moe_gateup_kernel(GateUpParams p) {
  constexpr int L = 32;       // a wave-iteration is one (g, u) row pair
  extern __shared__ float lds[];
  float* xs = lds;                                          // [chunks * kXStride]
  int* s_idx = reinterpret_cast<int*>(lds + p.g.chunks * kXStride);
  float* s_w = reinterpret_cast<float*>(s_idx + BDG_MAX_TOPK);
  const int t = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int li = lane % L;
  const bool is_up = lane >= L;

  if (wave == 0) {
    if (p.routed) {
      if (lane < p.K) {
        int e = p.idx_in[t * p.K + lane];
        e = e < 0 ? 0 : (e >= p.E ? p.E - 1 : e);
        s_idx[lane] = e;
        s_w[lane] = p.w_in[t * p.K + lane];
      }
    } else {
      wave_topk(p.logits + (int64_t)t * p.E, p.E, p.K, s_idx, s_w);
    }
  }
  const float mult = p.r ? p.r[t] : 1.0f;
  stage_x(xs, p.x, 0, (int64_t)t * p.H, p.H, mult);
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x < p.K) {
    p.idx_out[t * p.K + threadIdx.x] = s_idx[threadIdx.x];
    p.w_out[t * p.K + threadIdx.x] = s_w[threadIdx.x];
    if (p.topk_trace) p.topk_trace[t * p.K + threadIdx.x] = s_idx[threadIdx.x];
    if (p.wts_trace) p.wts_trace[t * p.K + threadIdx.x] = s_w[threadIdx.x];
  }
  XRegs<FMT, L, S> xr;
  xr.load(xs, p.g.chunks, li);
  const LayerDev Ld = p.layers[p.layer];

  const int64_t P = (int64_t)p.K * p.I;
  const int64_t p0 = P * blockIdx.x / gridDim.x;
  const int64_t p1 = P * (blockIdx.x + 1) / gridDim.x;
  float* ht = p.h_out + (int64_t)t * p.K * p.I;

  auto load_pair = [&](GroupLoad<FMT, S>& ld, int64_t pi) {
    const int j = (int)(pi / p.I);
    const int i = (int)(pi - (int64_t)j * p.I);
    const QMat m = expert_gu(Ld, s_idx[j]);
    load_row<FMT, L, S>(ld, m, p.g, is_up ? (int64_t)p.I + i : (int64_t)i, true, li);
  };
  auto finish_pair = [&](const GroupLoad<FMT, S>& ld, int64_t pi) {
    const float d = row_dot<FMT, L, S>(ld, xr);
    const float gv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), 0));
    const float uv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), L));
    if (lane == 0) ht[pi] = gv / (1.0f + expf(-gv)) * uv;
  };

  GroupLoad<FMT, S> a, b;
  int64_t pa = p0 + wave;
  if (pa < p1) load_pair(a, pa);
  while (pa < p1) {
    const int64_t pb = pa + kWaves;
    if (pb < p1) load_pair(b, pb);
    finish_pair(a, pa);
    if (pb >= p1) break;
    const int64_t pc = pb + kWaves;
    if (pc < p1) load_pair(a, pc);
    finish_pair(b, pb);
    pa = pc;
  }
}

// ---------------------------------------------------------------- down

struct DownParams {
  int M, H, I, E, K;
  const int32_t* idx;         // [M][K] routing buffer
  const float* h;             // [M][K][I]
  const LayerDev* layers;
  int layer;
  QGeom g;                    // reduction over I
  int rows_per_block;
  int blocks_per_expert;
  float* d_out;               // [M][K][H]
};

template <int FMT, int L, int S>
__global__ void __launch_bounds__(kThreads) moe_down_kernel(DownParams p) {
  constexpr int RPW = kWave / L;
  extern __shared__ float lds[];
  const int t = blockIdx.y;
  const int j = blockIdx.x / p.blocks_per_expert;
  const int rb = blockIdx.x - j * p.blocks_per_expert;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int li = lane % L;
  const int rr = lane / L;

  int e = p.idx[t * p.K + j];
  e = e < 0 ? 0 : (e >= p.E ? p.E - 1 : e);
  stage_x(lds, p.h, 0, ((int64_t)t * p.K + j) * p.I, p.I, 1.0f);
  __syncthreads();
  XRegs<FMT, L, S> xr;
  xr.load(lds, p.g.chunks, li);
  const LayerDev Ld = p.layers[p.layer];
  const QMat m = expert_dn(Ld, e);

  const int r0 = rb * p.rows_per_block;
  const int r1 = min(p.H, r0 + p.rows_per_block);
  const int ng = (r1 - r0 + RPW - 1) / RPW;
  float* dt = p.d_out + ((int64_t)t * p.K + j) * p.H;

  GroupLoad<FMT, S> a, b;
  int ga = wave;
  if (ga < ng) {
    const int row = r0 + ga * RPW + rr;
    load_row<FMT, L, S>(a, m, p.g, row, row < r1, li);
  }
  while (ga < ng) {
    const int gb = ga + kWaves;
    if (gb < ng) {
      const int row = r0 + gb * RPW + rr;
      load_row<FMT, L, S>(b, m, p.g, row, row < r1, li);
    }
    {
      const int row = r0 + ga * RPW + rr;
      const float d = row_dot<FMT, L, S>(a, xr);
      if (li == 0 && row < r1) dt[row] = d;
    }
    if (gb >= ng) break;
    const int gc = gb + kWaves;
    if (gc < ng) {
      const int row = r0 + gc * RPW + rr;
      load_row<FMT, L, S>(a, m, p.g, row, row < r1, li);
    }
    {
      const int row = r0 + gb * RPW + rr;
      const float d = row_dot<FMT, L, S>(b, xr);
      if (li == 0 && row < r1) dt[row] = d;
    }
    ga = gc;
  }
}

// ---------------------------------------------------------------- finish

struct FinishParams {
  int M, H, K, residual;
  const float* x_prev;
  const float* d;
  const float* w;
  float* y;
};

__global__ void __launch_bounds__(kThreads) moe_finish_kernel(FinishParams p) {
  const int t = blockIdx.y;
  const int h = blockIdx.x * kThreads + threadIdx.x;
  if (h >= p.H) return;
  p.y[(int64_t)t * p.H + h] = combine_elem(p.x_prev, p.d, p.w, p.K, p.H, t, h, p.residual);
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
};

}  // namespace bdg

struct bdg_plan {
  bdg_moe_desc d;
  int gu_L, gu_S, dn_L, dn_S;
  bdg::QGeom gu_geom, dn_geom;
  int gu_ppw;       // gate_up pairs per wave (grid sizing)
  int dn_it;        // down row groups per wave
  // device memory
  void* dev_base;
  bdg::LayerDev* layers;
  float* resid[2];
  float* r;
  float* logits;
  int32_t* idx;
  float* w;
  float* h;
  float* dout;
  hipStream_t cap_stream;
  hipEvent_t* prof_ev;      // timing events for moe_expert_decode_profiled (lazily created)
  int* prof_kind;
  int prof_cap;
  bdg::GraphEntry graphs[bdg::kGraphCache];
  uint64_t clock;
};

namespace bdg {

static int env_int(const char* name, int dflt, int lo, int hi) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  int x = atoi(v);
  if (x < lo) x = lo;
  if (x > hi) x = hi;
  return x;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- launches of one layer / the finish step

// Optional per-kernel timing: every launch takes the next start/stop event
// pair (recorded by the runtime at kernel start and end) and notes its kind.
enum KernelKind { kRoute = 0, kGateUp = 1, kDown = 2, kFinish = 3, kKinds = 4 };

struct Prof {
  hipEvent_t* ev;     // 2 * cap events
  int* kind;          // cap kinds
  int cap;
  int used;
};

#define BDG_LAUNCH(PROF, KIND, KERNEL, GRID, BLOCK, LDS, STREAM, ...)                          \
  do {                                                                                         \
    if (PROF) {                                                                                \
      if ((PROF)->used >= (PROF)->cap) return BDG_E_UNSUPPORTED;                               \
      const int slot_ = (PROF)->used++;                                                        \
      (PROF)->kind[slot_] = (KIND);                                                            \
      hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, (PROF)->ev[2 * slot_],            \
                            (PROF)->ev[2 * slot_ + 1], 0, __VA_ARGS__);                         \
    } else {                                                                                   \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, __VA_ARGS__);                       \
    }                                                                                          \
  } while (0)

static int launch_route(const bdg_plan* p, int layer, const void* x, int x_dtype, int m,
                        float* resid_trace, int compute_logits, hipStream_t s, Prof* prof) {
  RouteParams rp{};
  rp.M = m;
  rp.H = p->d.hidden;
  rp.E = p->d.n_experts;
  rp.K = p->d.top_k;
  const bool stack = (p->d.flags & BDG_MOE_STACK) != 0;
  rp.combine = layer > 0 ? 1 : 0;
  rp.residual = stack ? 1 : 0;
  rp.norm = stack ? 1 : 0;
  rp.eps = p->d.norm_eps;
  rp.compute_logits = compute_logits;
  rp.x_in = x;
  rp.x_bf16 = x_dtype == BDG_BF16 ? 1 : 0;
  rp.x_prev = p->resid[(layer + 1) & 1];
  rp.d_prev = p->dout;
  rp.w_prev = p->w;
  rp.x_out = p->resid[layer & 1];
  rp.resid_trace = resid_trace;
  rp.r_out = p->r;
  rp.logits = p->logits;
  rp.layers = p->layers;
  rp.layer = layer;
  const int nblk = compute_logits ? (rp.E + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock : 1;
  const size_t lds = (size_t)(rp.H + kWaves) * sizeof(float);
  BDG_LAUNCH(prof, kRoute, moe_route_kernel, dim3(nblk, m), dim3(kThreads), lds, s, rp);
  return launch_status();
}

static int launch_gateup(const bdg_plan* p, int layer, int m, int routed, const int32_t* idx_in,
                         const float* w_in, int32_t* topk_trace, float* wts_trace, int use_norm,
                         hipStream_t s, Prof* prof) {
  GateUpParams gp{};
  gp.M = m;
  gp.H = p->d.hidden;
  gp.I = p->d.inter;
  gp.E = p->d.n_experts;
  gp.K = p->d.top_k;
  gp.routed = routed;
  gp.logits = p->logits;
  gp.idx_in = idx_in;
  gp.w_in = w_in;
  gp.idx_out = p->idx;
  gp.w_out = p->w;
  gp.topk_trace = topk_trace;
  gp.wts_trace = wts_trace;
  gp.x = p->resid[layer & 1];
  gp.r = use_norm ? p->r : nullptr;
  gp.layers = p->layers;
  gp.layer = layer;
  gp.g = p->gu_geom;
  gp.h_out = p->h;
  const int64_t pairs = (int64_t)gp.K * gp.I;
  int64_t blocks = (pairs + (int64_t)kWaves * p->gu_ppw - 1) / ((int64_t)kWaves * p->gu_ppw);
  if (blocks < 1) blocks = 1;
  if (blocks > 65535) blocks = 65535;
  const size_t lds = (size_t)gp.g.chunks * kXStride * sizeof(float) + 2 * BDG_MAX_TOPK * sizeof(float);
  dim3 grid((unsigned)blocks, m);
  const int fmt = p->d.fmt;
#define BDG_GU_CASE(F, SS)                                                                    \
  if (fmt == F && p->gu_S == SS) {                                                            \
    BDG_LAUNCH(prof, kGateUp, (moe_gateup_kernel<F, SS>), grid, dim3(kThreads), lds, s, gp);  \
    return launch_status();                                                                   \
  }
  BDG_GU_CASE(kMXFP4, 1) BDG_GU_CASE(kMXFP4, 2) BDG_GU_CASE(kMXFP4, 3) BDG_GU_CASE(kMXFP4, 4)
  BDG_GU_CASE(kINT4G, 1) BDG_GU_CASE(kINT4G, 2) BDG_GU_CASE(kINT4G, 3) BDG_GU_CASE(kINT4G, 4)
#undef BDG_GU_CASE
  return BDG_E_UNSUPPORTED;
}

static int launch_down(const bdg_plan* p, int layer, int m, hipStream_t s, Prof* prof) {
  DownParams dp{};
  dp.M = m;
  dp.H = p->d.hidden;
  dp.I = p->d.inter;
  dp.E = p->d.n_experts;
  dp.K = p->d.top_k;
  dp.idx = p->idx;
  dp.h = p->h;
  dp.layers = p->layers;
  dp.layer = layer;
  dp.g = p->dn_geom;
  const int rpw = kWave / p->dn_L;
  dp.rows_per_block = kWaves * rpw * p->dn_it;
  dp.blocks_per_expert = (dp.H + dp.rows_per_block - 1) / dp.rows_per_block;
  dp.d_out = p->dout;
  const size_t lds = (size_t)dp.g.chunks * kXStride * sizeof(float);
  dim3 grid((unsigned)(dp.blocks_per_expert * dp.K), m);
  const int fmt = p->d.fmt;
#define BDG_DN_CASE(F, LL, SS)                                                                \
  if (fmt == F && p->dn_L == LL && p->dn_S == SS) {                                           \
    BDG_LAUNCH(prof, kDown, (moe_down_kernel<F, LL, SS>), grid, dim3(kThreads), lds, s, dp);  \
    return launch_status();                                                                   \
  }
  BDG_DN_CASE(kMXFP4, 8, 1) BDG_DN_CASE(kMXFP4, 8, 2) BDG_DN_CASE(kMXFP4, 8, 3)
  BDG_DN_CASE(kMXFP4, 16, 2) BDG_DN_CASE(kMXFP4, 16, 3)
  BDG_DN_CASE(kMXFP4, 32, 2) BDG_DN_CASE(kMXFP4, 32, 3)
  BDG_DN_CASE(kMXFP4, 64, 2) BDG_DN_CASE(kMXFP4, 64, 3) BDG_DN_CASE(kMXFP4, 64, 4)
  BDG_DN_CASE(kINT4G, 8, 1) BDG_DN_CASE(kINT4G, 8, 2) BDG_DN_CASE(kINT4G, 8, 3)
  BDG_DN_CASE(kINT4G, 16, 2) BDG_DN_CASE(kINT4G, 16, 3)
  BDG_DN_CASE(kINT4G, 32, 2) BDG_DN_CASE(kINT4G, 32, 3)
  BDG_DN_CASE(kINT4G, 64, 2) BDG_DN_CASE(kINT4G, 64, 3) BDG_DN_CASE(kINT4G, 64, 4)
#undef BDG_DN_CASE
  return BDG_E_UNSUPPORTED;
}

static int launch_finish(const bdg_plan* p, int last_layer, int m, int residual, float* y, hipStream_t s,
                         Prof* prof) {
  FinishParams fp{};
  fp.M = m;
  fp.H = p->d.hidden;
  fp.K = p->d.top_k;
  fp.residual = residual;
  fp.x_prev = p->resid[last_layer & 1];
  fp.d = p->dout;
  fp.w = p->w;
  fp.y = y;
  BDG_LAUNCH(prof, kFinish, moe_finish_kernel, dim3((fp.H + kThreads - 1) / kThreads, m), dim3(kThreads), 0, s,
             fp);
  return launch_status();
}

// The whole per-token path, enqueued on s.
static int enqueue_decode(const bdg_plan* p, const GraphKey& k, hipStream_t s, Prof* prof = nullptr) {
  const int L = p->d.n_layers;
  const int K = p->d.top_k;
  const int H = p->d.hidden;
  const bool stack = (p->d.flags & BDG_MOE_STACK) != 0;
  for (int l = 0; l < L; ++l) {
    int st = launch_route(p, l, k.x, k.x_dtype, k.m,
                          k.resid_trace ? k.resid_trace + (int64_t)l * k.m * H : nullptr, 1, s, prof);
    if (st) return st;
    st = launch_gateup(p, l, k.m, 0, nullptr, nullptr,
                       k.topk_trace ? k.topk_trace + (int64_t)l * k.m * K : nullptr,
                       k.wts_trace ? k.wts_trace + (int64_t)l * k.m * K : nullptr, stack ? 1 : 0, s,
                       prof);
    if (st) return st;
    st = launch_down(p, l, k.m, s, prof);
    if (st) return st;
  }
  return launch_finish(p, L - 1, k.m, stack ? 1 : 0, k.y, s, prof);
}

static void drop_graph(GraphEntry& g) {
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
  if (d->n_experts > 1 && (L.gate_up.expert_stride_codes == 0 || L.down.expert_stride_codes == 0))
    return BDG_E_INVALID;
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
  if ((d->hidden % 4) != 0) return BDG_E_INVALID;
  if ((d->flags & ~(BDG_MOE_STACK | BDG_MOE_NO_GRAPH)) != 0) return BDG_E_INVALID;
  if ((d->flags & BDG_MOE_STACK) && !(d->norm_eps >= 0.f)) return BDG_E_INVALID;
  if (d->top_k > BDG_MAX_TOPK || d->n_experts > BDG_MAX_EXPERTS || d->max_m > BDG_MAX_M)
    return BDG_E_UNSUPPORTED;
  if (d->hidden > 4096 || d->inter > BDG_MAX_K) return BDG_E_UNSUPPORTED;
  for (int l = 0; l < d->n_layers; ++l) {
    int st = check_layer(d, d->layers[l]);
    if (st) return st;
  }
  bdg_plan* p = new (std::nothrow) bdg_plan();
  if (!p) return BDG_E_NOMEM;
  p->d = *d;
  p->d.layers = nullptr;
  const int hc = d->hidden / 32, ic = d->inter / 32;
  p->gu_L = 32;
  p->gu_S = (hc + 31) / 32;
  if (!pick_lanes(ic, &p->dn_L, &p->dn_S)) {
    delete p;
    return BDG_E_UNSUPPORTED;
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
  if (d->fmt == BDG_FMT_INT4G && ((d->hidden % d->group) || (d->inter % d->group))) {
    delete p;
    return BDG_E_INVALID;
  }
  p->gu_geom = geom(d->hidden);
  p->dn_geom = geom(d->inter);
  p->gu_ppw = env_int("BDG_GU_PPW", 6, 1, 64);
  {
    const int rpw = kWave / p->dn_L;
    const int64_t groups = (int64_t)d->top_k * ((d->hidden + rpw - 1) / rpw);
    int it = (int)(groups / 1536);
    if (it < 1) it = 1;
    if (it > 8) it = 8;
    p->dn_it = env_int("BDG_DN_IT", it, 1, 64);
  }
  // device memory: layer table + workspace
  const int M = d->max_m, H = d->hidden, I = d->inter, E = d->n_experts, K = d->top_k;
  size_t off = 0;
  const size_t o_layers = off; off = align256(off + sizeof(LayerDev) * d->n_layers);
  const size_t o_res0 = off; off = align256(off + sizeof(float) * M * H);
  const size_t o_res1 = off; off = align256(off + sizeof(float) * M * H);
  const size_t o_r = off; off = align256(off + sizeof(float) * M);
  const size_t o_log = off; off = align256(off + sizeof(float) * M * E);
  const size_t o_idx = off; off = align256(off + sizeof(int32_t) * M * K);
  const size_t o_w = off; off = align256(off + sizeof(float) * M * K);
  const size_t o_h = off; off = align256(off + sizeof(float) * (size_t)M * K * I);
  const size_t o_d = off; off = align256(off + sizeof(float) * (size_t)M * K * H);
  if (hipMalloc(&p->dev_base, off) != hipSuccess) {
    delete p;
    return BDG_E_NOMEM;
  }
  char* base = static_cast<char*>(p->dev_base);
  p->layers = reinterpret_cast<LayerDev*>(base + o_layers);
  p->resid[0] = reinterpret_cast<float*>(base + o_res0);
  p->resid[1] = reinterpret_cast<float*>(base + o_res1);
  p->r = reinterpret_cast<float*>(base + o_r);
  p->logits = reinterpret_cast<float*>(base + o_log);
  p->idx = reinterpret_cast<int32_t*>(base + o_idx);
  p->w = reinterpret_cast<float*>(base + o_w);
  p->h = reinterpret_cast<float*>(base + o_h);
  p->dout = reinterpret_cast<float*>(base + o_d);
  LayerDev* host = new (std::nothrow) LayerDev[d->n_layers];
  if (!host) {
    (void)hipFree(p->dev_base);
    delete p;
    return BDG_E_NOMEM;
  }
  for (int l = 0; l < d->n_layers; ++l) {
    const bdg_layer_desc& S = d->layers[l];
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
  hipError_t e1 = hipMemcpy(p->layers, host, sizeof(LayerDev) * d->n_layers, hipMemcpyHostToDevice);
  delete[] host;
  hipError_t e2 = hipMemset(base + o_res0, 0, off - o_res0);
  hipError_t e3 = hipStreamCreateWithFlags(&p->cap_stream, hipStreamNonBlocking);
  if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess) {
    if (e3 == hipSuccess) (void)hipStreamDestroy(p->cap_stream);
    (void)hipFree(p->dev_base);
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
  for (int i = 0; i < kGraphCache; ++i) drop_graph(p->graphs[i]);
  (void)hipDeviceSynchronize();
  (void)hipStreamDestroy(p->cap_stream);
  if (p->prof_ev) {
    for (int i = 0; i < 2 * p->prof_cap; ++i) (void)hipEventDestroy(p->prof_ev[i]);
    delete[] p->prof_ev;
    delete[] p->prof_kind;
  }
  (void)hipFree(p->dev_base);
  delete p;
  return BDG_OK;
}

extern "C" int moe_expert_decode_profiled(bdg_plan* p, const void* x, int32_t x_dtype, int32_t m, float* y,
                                          double* kernel_ms, int64_t* kernel_count, void* stream) {
  if (!p || !x || !y || !kernel_ms || !kernel_count || m < 1) return BDG_E_INVALID;
  if (m > p->d.max_m) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  const int need = 3 * p->d.n_layers + 1;
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

extern "C" int moe_expert_decode(bdg_plan* p, const void* x, int32_t x_dtype, int32_t m, float* y,
                                 int32_t* topk_trace, float* wts_trace, float* resid_trace, void* stream) {
  if (!p || !x || !y || m < 1) return BDG_E_INVALID;
  if (m > p->d.max_m) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
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
    if (slot->used) {
      // the evicted graph may still be queued: let it finish before destroying
      (void)hipStreamSynchronize(s);
      drop_graph(*slot);
    }
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
    slot->used = true;
    slot->key = key;
    slot->graph = graph;
    slot->exec = exec;
    hit = slot;
  }
  hit->stamp = ++p->clock;
  return hip_status(hipGraphLaunch(hit->exec, s));
}

extern "C" int moe_experts_routed(bdg_plan* p, int32_t layer, const void* x, int32_t x_dtype, int32_t m,
                                  const int32_t* idx, const float* wts, float* y, void* stream) {
  if (!p || !x || !idx || !wts || !y || m < 1) return BDG_E_INVALID;
  if (m > p->d.max_m || layer < 0 || layer >= p->d.n_layers) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  hipStream_t s = as_stream(stream);
  // x -> the plan's fp32 input buffer of `layer` (no norm, no logits)
  RouteParams rp{};
  rp.M = m;
  rp.H = p->d.hidden;
  rp.E = p->d.n_experts;
  rp.K = p->d.top_k;
  rp.combine = 0;
  rp.residual = 0;
  rp.norm = 0;
  rp.eps = 0.f;
  rp.compute_logits = 0;
  rp.x_in = x;
  rp.x_bf16 = x_dtype == BDG_BF16 ? 1 : 0;
  rp.x_out = p->resid[layer & 1];
  rp.r_out = p->r;
  rp.logits = p->logits;
  rp.layers = p->layers;
  rp.layer = layer;
  hipLaunchKernelGGL(moe_route_kernel, dim3(1, m), dim3(kThreads), (size_t)(rp.H + kWaves) * sizeof(float), s,
                     rp);
  int st = launch_status();
  if (st) return st;
  // gate_up runs on the raw x (no norm), routing from the caller
  st = launch_gateup(p, layer, m, 1, idx, wts, nullptr, nullptr, 0, s, nullptr);
  if (st) return st;
  st = launch_down(p, layer, m, s, nullptr);
  if (st) return st;
  return launch_finish(p, layer, m, 0, y, s, nullptr);
}

// ---------------------------------------------------------------- standalone router

namespace bdg {

// One block per token: (optional RMSNorm of) x into LDS, all E router rows
// one wave at a time, then top-k + softmax by wave 0.  The decode plan uses
// the split route / gate_up kernels instead; this entry point serves callers
// that need only the routing.
__global__ void __launch_bounds__(kThreads)
router_topk_kernel(const void* __restrict__ x, int x_bf16, const float* __restrict__ w_r,
                   const float* __restrict__ b_r, int H, int E, int K, int norm, float eps,
                   int32_t* __restrict__ idx, float* __restrict__ wts, float* __restrict__ logits) {
  extern __shared__ float lds[];
  float* xs = lds;             // [H]
  float* lg = lds + H;         // [E]
  float* red = lg + E;         // [kWaves]
  __shared__ int s_idx[BDG_MAX_TOPK];
  __shared__ float s_w[BDG_MAX_TOPK];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float ss = 0.f;
  for (int h = threadIdx.x; h < H; h += kThreads) {
    const float v = x_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[(int64_t)t * H + h])
                           : reinterpret_cast<const float*>(x)[(int64_t)t * H + h];
    xs[h] = v;
    ss = __builtin_fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float r = 1.f;
  if (norm) r = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)H + eps);
  for (int e = wave; e < E; e += kWaves) {
    const float* wr = w_r + (int64_t)e * H;
    float acc = 0.f;
    for (int h = lane * 4; h < H; h += kWave * 4) {
      const float4 wv = *reinterpret_cast<const float4*>(wr + h);
      acc = __builtin_fmaf(wv.x, xs[h] * r, acc);
      acc = __builtin_fmaf(wv.y, xs[h + 1] * r, acc);
      acc = __builtin_fmaf(wv.z, xs[h + 2] * r, acc);
      acc = __builtin_fmaf(wv.w, xs[h + 3] * r, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) lg[e] = acc + (b_r ? b_r[e] : 0.f);
  }
  __syncthreads();
  if (wave == 0) wave_topk(lg, E, K, s_idx, s_w);
  __syncthreads();
  if (threadIdx.x < K) {
    idx[t * K + threadIdx.x] = s_idx[threadIdx.x];
    wts[t * K + threadIdx.x] = s_w[threadIdx.x];
  }
  if (logits)
    for (int e = threadIdx.x; e < E; e += kThreads) logits[(int64_t)t * E + e] = lg[e];
}

}  // namespace bdg

extern "C" int moe_router_topk(const void* x, int32_t x_dtype, const float* w_r, const float* b_r,
                               int32_t m, int32_t h, int32_t e, int32_t topk, int32_t flags,
                               float norm_eps, int32_t* idx, float* wts, float* logits, void* stream) {
  if (!x || !w_r || !idx || !wts || m < 1 || h < 1 || e < 1 || topk < 1 || topk > e) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if ((flags & ~BDG_ROUTER_RMSNORM) != 0 || (h % 4) != 0) return BDG_E_INVALID;
  if ((flags & BDG_ROUTER_RMSNORM) && !(norm_eps >= 0.f)) return BDG_E_INVALID;
  if ((reinterpret_cast<uintptr_t>(w_r) & 15u) != 0) return BDG_E_ALIGN;
  if (e > BDG_MAX_EXPERTS || topk > BDG_MAX_TOPK || h > 16384) return BDG_E_UNSUPPORTED;
  const size_t lds = (size_t)(h + e + kWaves) * sizeof(float);
  hipLaunchKernelGGL(router_topk_kernel, dim3(m), dim3(kThreads), lds, as_stream(stream), x,
                     x_dtype == BDG_BF16 ? 1 : 0, w_r, b_r, h, e, topk,
                     (flags & BDG_ROUTER_RMSNORM) ? 1 : 0, norm_eps, idx, wts, logits);
  return launch_status();
}
