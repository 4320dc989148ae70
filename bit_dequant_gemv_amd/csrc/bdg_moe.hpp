// Pieces shared by the MoE decode kernels (moe.hip: the router, gate_up and
// down kernels and the grouped kernels; moe_layer.hip: the fused per-layer
// kernel): per-layer weight addresses, expert views, and the routing
// prologue in which a kernel selects its own experts from router sums.
#pragma once

#include "bdg_gemv.hpp"
#include "bdg_topk.hpp"

namespace bdg {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kDownWaves = 8;        // waves per down block
constexpr int kGuPairsPerWave = 6;   // gate_up: (g, u) row pairs in flight per wave
constexpr int kRouteMaxF4 = 16;      // router row float4 per lane (H <= 4096)
constexpr int kPartF4 = 8;           // float4 of router partial sums per thread issued up front
constexpr int kDnRouterPerWave = 8;  // next-layer router rows per down wave (E <= 64)

// Weight addresses of one layer.  The plan keeps one per layer on the host
// and passes it by value to each kernel launch (a kernel argument, so the
// first weight load does not wait for a dependent table load).
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

__device__ __forceinline__ int uniform_wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// ---------------------------------------------------------------- routing prologue
//
// Router dot products travel between kernels as partial sums:
// part[t][e][k], k < nparts (row stride pstride), holds the sum over one
// slice of the hidden dimension of w_r[e][h] * x[h] for the layer input x,
// before the RMSNorm scale and the bias.  The route kernel writes one slice
// (the whole of x); a down kernel that feeds the next layer writes one slice
// per row block.  Column E holds the matching slices of the sum of squares
// of x.  A kernel that selects its own experts adds the slices in a fixed
// order, scales by the RMSNorm factor, adds the bias and takes the top-k.
// (RMSNorm is a per-token scale, so w_r . (x * r) = r * (w_r . x).)

struct RouteSrc {
  int routed;                 // 1: routing given in idx_in / w_in
  const int32_t* idx_in;      // [M][K]
  const float* w_in;
  const float* part;          // [M][E + 1][pstride] router partial sums
  int nparts, pstride;
  int log2T;                  // 2^log2T threads add up one expert's slices
  int norm;                   // RMSNorm scale on x (and on the router input)
  float eps;
  int E, K, H;
  const float* b_r;           // [E] or NULL
};

template <int V>
struct RouteState {
  float4 pv[kPartF4];
  float lg[V], bias[V];
  float ssq;
  int my_e;                   // lane j < K: pick j (expert, weight)
  float my_w;
  float r;                    // RMSNorm factor of the layer input (1 without norm)
};

// Issue the loads of token t's routing inputs (call first: vmcnt retires in
// order, so anything issued later does not delay their wait).  NT threads.
template <int V, int NT>
__device__ __forceinline__ void route_issue(RouteState<V>& rs, const RouteSrc& p, int t, int lane) {
  const int lt = p.log2T;
  const int T = 1 << lt;
  const int sub = threadIdx.x & (T - 1);
  const int n4 = (p.nparts + 3) >> 2;                      // float4 per expert row of slices
  const int64_t pbase = (int64_t)t * (p.E + 1) * p.pstride;
  const bool slices = !p.routed && p.nparts > 1;
  rs.ssq = 0.f;
  rs.my_e = 0;
  rs.my_w = 0.f;
  rs.r = 1.f;
  if (p.routed) {
    rs.my_e = clamp_expert(p.idx_in[t * p.K + (lane < p.K ? lane : 0)], p.E);
    rs.my_w = p.w_in[t * p.K + (lane < p.K ? lane : 0)];
    return;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane + kWave * i;
    rs.bias[i] = p.b_r ? p.b_r[e < p.E ? e : p.E - 1] : 0.f;
  }
  if (slices) {
    const int c = threadIdx.x >> lt;
    const float* row = p.part + pbase + (int64_t)(c < p.E ? c : p.E - 1) * p.pstride;
    // rows are zero past the nparts slices up to pstride >= 4 * T * kPartF4
    // (the plan zeroes the buffer once; no kernel writes there)
#pragma unroll
    for (int i = 0; i < kPartF4; ++i) rs.pv[i] = ldg_f4(row + 4 * (sub + (i << lt)));
    // sum-of-squares slices (column E): one float4 per thread, n4 <= kThreads
    const int k4 = threadIdx.x;
    const float4 q = k4 < n4 ? ldg_f4(p.part + pbase + (int64_t)p.E * p.pstride + 4 * k4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    const int k = 4 * k4;
    rs.ssq = k < p.nparts ? q.x : 0.f;
    rs.ssq += k + 1 < p.nparts ? q.y : 0.f;
    rs.ssq += k + 2 < p.nparts ? q.z : 0.f;
    rs.ssq += k + 3 < p.nparts ? q.w : 0.f;
  } else {
    // one slice (the route kernel's): each wave reads its values directly
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = lane + kWave * i;
      rs.lg[i] = p.part[pbase + (int64_t)(e < p.E ? e : p.E - 1) * p.pstride];
    }
    rs.ssq = p.part[pbase + (int64_t)p.E * p.pstride];
  }
}

// Add the slices in a fixed order, apply the RMSNorm factor and bias, and
// select: every wave ends with the token's top-k in its lanes 0..K-1.  All
// NT threads of the block call it (a barrier inside when slices are summed).
// red: NT / 64 floats of LDS; psum: E << log2T floats of LDS.
template <int V, int NT>
__device__ __forceinline__ void route_finish(RouteState<V>& rs, const RouteSrc& p, int t, int lane, int wave,
                                             float* red, float* psum) {
  if (p.routed) {
    if (lane >= p.K) {
      rs.my_e = 0;
      rs.my_w = 0.f;
    }
    return;
  }
  const int lt = p.log2T;
  const int T = 1 << lt;
  const int sub = threadIdx.x & (T - 1);
  const int n4 = (p.nparts + 3) >> 2;
  const int64_t pbase = (int64_t)t * (p.E + 1) * p.pstride;
  float ssq = rs.ssq;
  if (p.nparts > 1) {
    // slices of expert c: thread sub adds slices 4*(sub + i*T) .. +3, in order
    for (int c0 = 0; c0 < p.E; c0 += NT >> lt) {
      const int c = c0 + (threadIdx.x >> lt);
      const float* row = p.part + pbase + (int64_t)(c < p.E ? c : p.E - 1) * p.pstride;
      float a = 0.f;
      int k4 = sub;
      if (c0 == 0) {
#pragma unroll
        for (int i = 0; i < kPartF4; ++i, k4 += T) {
          a += rs.pv[i].x;
          a += rs.pv[i].y;
          a += rs.pv[i].z;
          a += rs.pv[i].w;
        }
      }
      for (; k4 < n4; k4 += T) {   // beyond the slices loaded up front
        const float4 v = ldg_f4(row + 4 * k4);
        const int k = 4 * k4;
        a += v.x;
        a += k + 1 < p.nparts ? v.y : 0.f;
        a += k + 2 < p.nparts ? v.z : 0.f;
        a += k + 3 < p.nparts ? v.w : 0.f;
      }
      if (c < p.E) psum[(c << lt) + sub] = a;
    }
    {
      const float ss = wave_sum(ssq);
      if (lane == 0) red[wave] = ss;
    }
    __syncthreads();
    // the sum-of-squares slices sit in threads 0..255 (waves 0..3)
    if (p.norm) ssq = (red[0] + red[1]) + (red[2] + red[3]);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = lane + kWave * i;
      const float* ps = psum + ((e < p.E ? e : p.E - 1) << lt);
      float a = 0.f;
      for (int q = 0; q < T; ++q) a += ps[q];
      rs.lg[i] = a;
    }
  }
  float r = 1.0f;
  if (p.norm) r = 1.0f / sqrtf(ssq / (float)p.H + p.eps);
#pragma unroll
  for (int i = 0; i < V; ++i) rs.lg[i] = r * rs.lg[i] + rs.bias[i];
  topk_rank<V>(rs.lg, p.E, p.K, rs.my_e, rs.my_w);
  rs.r = r;
  if (lane >= p.K) {
    rs.my_e = 0;
    rs.my_w = 0.f;
  }
}

// ---------------------------------------------------------------- router rows
//
// One router row against the layer input: lane l holds float4 i = elements
// 4 (64 i + l) .. +3 of the row and of x (elements past H are skipped), and
// adds w . x and x . x in that order.  The route kernel and a gate_up launch
// that routes itself both call this, so their logits agree bit for bit.
template <int NF>
__device__ __forceinline__ void router_lane_sums(const float4 (&wv)[NF], const float4 (&xv)[NF], int H, int lane,
                                                 float& acc, float& ss) {
  acc = 0.f;
  ss = 0.f;
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int h = (i * kWave + lane) * 4;
    if (h < H) {
      acc = __builtin_fmaf(wv[i].x, xv[i].x, acc);
      acc = __builtin_fmaf(wv[i].y, xv[i].y, acc);
      acc = __builtin_fmaf(wv[i].z, xv[i].z, acc);
      acc = __builtin_fmaf(wv[i].w, xv[i].w, acc);
      ss = __builtin_fmaf(xv[i].x, xv[i].x, ss);
      ss = __builtin_fmaf(xv[i].y, xv[i].y, ss);
      ss = __builtin_fmaf(xv[i].z, xv[i].z, ss);
      ss = __builtin_fmaf(xv[i].w, xv[i].w, ss);
    }
  }
}

// Self-routing gate_up (a layer whose router would otherwise have a kernel
// of its own: the first layer, and later layers the previous down kernel
// cannot hand router sums to): the launch's first blocks compute the router
// rows, one per wave, and publish each sum as one 64-bit word (tag << 32 |
// float bits) with a device-coherent store; every block then waits until all
// E logits and the sum of squares carry this token's tag.  The tag is the
// token's sequence number, advanced once per token (by the first layer's
// route kernel, or, when the first layer routes itself, by its down kernel,
// the first layer tagging with the number plus one), so words left by an
// earlier token never match.  No counter and no block waits on a block
// dispatched after it (router blocks have the lowest indices of their
// token), and the wait is bounded.
constexpr int kSelfRouteNF = 12;     // router row float4 per lane (H <= 3072)

struct SelfRoute {
  unsigned long long* log;   // [M][E + 1]: tagged logits, slot E the sum of squares
  const unsigned* seq;       // the token's sequence number (tag = *seq + tag_add)
  unsigned tag_add;          // 1 in the first layer (the number is advanced after it), else 0
  int blocks;                // blocks (per token) that compute router rows
  int polls;                 // bound of the wait, in polls (0: give up at once)
  unsigned* fault;           // set when a wait gives up
  float* resid_trace;        // [M][H] or NULL: the layer input, written by router row 0
  float* x_copy;             // [M][H] or NULL: its fp32 copy (the first layer), written by router row 0
};

__device__ __forceinline__ unsigned long long tagged(unsigned tag, float v) {
  return ((unsigned long long)tag << 32) | __float_as_uint(v);
}

// Wave 0 of a block: wait for token t's E tagged logits and sum of squares,
// then leave them in lds_lg[0 .. E) and lds_misc[0] (lds_misc[1] = 1 when the
// wait gave up: logits 0, the caller poisons its outputs).
template <int V>
__device__ __forceinline__ void self_route_wait(const SelfRoute& sr, int t, int E, unsigned tag, int lane,
                                                float* lds_lg, float* lds_misc) {
  const unsigned long long* row = sr.log + (int64_t)t * (E + 1);
  float lg[V];
  float ss = 0.f;
  bool ok = false;
#pragma unroll
  for (int i = 0; i < V; ++i) lg[i] = 0.f;
  int it = 0;
  // first the sum of squares alone: one line per poll (reading every
  // logit's line on each poll from every block crowded those lines and
  // slowed the launch by about a microsecond); the router rows finish
  // together, so this mostly waits for all of them
  for (; it < sr.polls; ++it) {
    const unsigned long long s = __hip_atomic_load(row + E, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((unsigned)(s >> 32) == tag) break;
    __builtin_amdgcn_s_sleep(1);
  }
  for (; it < sr.polls; ++it) {
    bool mine = true;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int e = lane + kWave * i;
      const unsigned long long v =
          __hip_atomic_load(row + (e < E ? e : E - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lg[i] = __uint_as_float((unsigned)v);
      mine = mine && (unsigned)(v >> 32) == tag;
    }
    const unsigned long long s = __hip_atomic_load(row + E, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ss = __uint_as_float((unsigned)s);
    mine = mine && (unsigned)(s >> 32) == tag;
    if (__builtin_amdgcn_ballot_w64(!mine) == 0) {
      ok = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!ok) {
#pragma unroll
    for (int i = 0; i < V; ++i) lg[i] = 0.f;
    ss = 0.f;
    if (lane == 0) __hip_atomic_store(sr.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane + kWave * i;
    if (e < E) lds_lg[e] = lg[i];
  }
  if (lane == 0) {
    lds_misc[0] = ss;
    lds_misc[1] = ok ? 0.f : 1.f;
  }
}

// ---------------------------------------------------------------- down epilogue
//
// A block of 8 waves that owns output rows [r0, r0 + B), B <= 64, with the
// expert rows' dot products in dpart[j][b] (LDS): every wave forms row
// r0 + lane = (x_prev +) sum_j w_j dpart[j][lane], j in slot order, and wave
// 0 stores it; with route_next, wave w also reduces the rows against router
// rows w, w + 8, ... of the next layer and writes slice `slice` of its
// router partial sums (and of the sum of squares, column E).

struct DownOut {
  int H, E, K;
  int residual;               // add x_prev
  const float* x_prev;        // [M][H] layer input (residual)
  const float* w;             // [M][K] routing weights
  float* x_out;               // [M][H] next layer's input, or NULL
  float* y_out;               // [M][H] caller output, or NULL
  float* trace_out;           // [M][H] copy of x_out (next layer's input trace), or NULL
  int route_next;             // then E <= kDownWaves * RW (the epilogue's router rows per wave)
  const float* wr_next;       // [E][H]
  float* part_out;            // [M][E + 1][pstride]
  int pstride;
};

// The epilogue's router and residual operands for this lane (all in
// bounds and unconditional, so the compiler's wait counts stay exact): idle
// lanes past the block's rows repeat its last row.
template <int RW>
struct DownEpiIn {
  float wr[RW];                 // wr[i] = w_r'[wave + 8i][orow]
  float xp;                     // x_prev[orow]
  float wk;                     // routing weight of slot `lane` (lane < K), set by the caller
};

template <int RW>
__device__ __forceinline__ void down_epilogue_load(DownEpiIn<RW>& in, const DownOut& o, int t, int r0, int B, int lane,
                                                   int wave) {
  const int orow = min(r0 + min(lane, B - 1), o.H - 1);
  const float* wsrc = o.route_next ? o.wr_next : o.x_prev;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int er = wave + kDownWaves * i;
    in.wr[i] = wsrc[(int64_t)(o.route_next ? (er < o.E ? er : o.E - 1) : 0) * o.H + orow];
  }
  in.xp = o.x_prev[(int64_t)t * o.H + orow];
}

template <int RW>
__device__ __forceinline__ void down_epilogue(const DownOut& o, const DownEpiIn<RW>& in, const float* dpart, int t,
                                              int slice, int r0, int B, int lane, int wave) {
  const int row = r0 + lane;
  const bool ok = lane < B && row < o.H;
  float v = o.residual ? in.xp : 0.f;
  for (int j = 0; j < o.K; ++j)
    v = __builtin_fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(in.wk), j)),
                       dpart[j * B + (ok ? lane : 0)], v);
  v = ok ? v : 0.f;
  if (wave == 0 && ok) {
    if (o.x_out) o.x_out[(int64_t)t * o.H + row] = v;
    if (o.y_out) o.y_out[(int64_t)t * o.H + row] = v;
    if (o.trace_out) o.trace_out[(int64_t)t * o.H + row] = v;
  }
  if (!o.route_next) return;
  // all router rows of the wave (and the rows' sum of squares, column E)
  // reduced together, one butterfly step at a time
  constexpr int NA = RW + 1;
  float a[NA];
#pragma unroll
  for (int i = 0; i < RW; ++i) a[i] = ok ? in.wr[i] * v : 0.f;
  a[RW] = v * v;
#pragma unroll
  for (int i = 0; i < NA; ++i) a[i] += dpp_quad_xor1(a[i]);
#pragma unroll
  for (int i = 0; i < NA; ++i) a[i] += dpp_quad_xor2(a[i]);
#pragma unroll
  for (int i = 0; i < NA; ++i) a[i] += dpp_f32<0x141, 0xF>(a[i]);   // row_half_mirror
#pragma unroll
  for (int i = 0; i < NA; ++i) a[i] += dpp_f32<0x140, 0xF>(a[i]);   // row_mirror
#pragma unroll
  for (int i = 0; i < NA; ++i) a[i] = add_pair16(a[i]);
#pragma unroll
  for (int i = 0; i < NA; ++i) a[i] = add_pair32(a[i]);
  if (lane == 0) {
    float* out = o.part_out + (int64_t)t * (o.E + 1) * o.pstride + slice;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int er = wave + kDownWaves * i;
      if (er < o.E) out[(int64_t)er * o.pstride] = a[i];
    }
    if (wave == 0) out[(int64_t)o.E * o.pstride] = a[RW];
  }
}

// ---------------------------------------------------------------- expert grouping (steps of M > 1)
//
// Every block of a grouped kernel routes all M tokens of the step and builds
// the same deterministic table of "chunks": the distinct chosen experts in
// ascending order, each with its picks (p = t*K + j) in pick order, TT picks
// per chunk (an expert with more picks spans several chunks).

constexpr int kGroupMaxPicks = 128;   // M * K bound of the grouped path

template <int TT>
struct GroupLdsT {
  int sel_e[kGroupMaxPicks];          // pick p = t*K + j -> expert
  float rt[BDG_MAX_M];                // RMSNorm scale per token
  unsigned used[BDG_MAX_EXPERTS / 32];
  int ppc[BDG_MAX_EXPERTS / 32 + 1];  // prefix popcounts of used[]
  int cnt[kGroupMaxPicks];            // picks per distinct expert (by rank)
  int cbase[kGroupMaxPicks + 1];      // first chunk of each distinct expert
  int n;                              // chunks
  int ce[kGroupMaxPicks];             // expert of chunk c
  int cn[kGroupMaxPicks];             // picks in chunk c
  int cpk[kGroupMaxPicks][TT];        // the picks of chunk c
};

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_scan_incl(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// Chunks of the P picks in g.sel_e.  The block's threads all call it; the
// result does not depend on thread timing (the only atomics are an OR and a
// count).  P <= kGroupMaxPicks, blockDim >= kGroupMaxPicks.
static_assert(BDG_MAX_EXPERTS / 32 <= kWave, "build_groups scans the used-expert words in one wave");
template <int TT>
__device__ void build_groups(GroupLdsT<TT>& g, int P, int E) {
  const int tid = threadIdx.x;
  const int nw = (E + 31) >> 5;
  if (tid < nw) g.used[tid] = 0u;
  if (tid < P) g.cnt[tid] = 0;
  __syncthreads();
  if (tid < P) atomicOr(&g.used[g.sel_e[tid] >> 5], 1u << (g.sel_e[tid] & 31));
  __syncthreads();
  if (tid < kWave) {
    const int pc = wave_scan_incl(tid < nw ? __popc(g.used[tid]) : 0);
    if (tid < nw) g.ppc[tid + 1] = pc;
    if (tid == 0) g.ppc[0] = 0;
  }
  __syncthreads();
  int my_u = 0, my_pos = 0;
  if (tid < P) {
    const int e = g.sel_e[tid];
    my_u = g.ppc[e >> 5] + __popc(g.used[e >> 5] & ((1u << (e & 31)) - 1u));
    for (int q = 0; q < tid; ++q) my_pos += g.sel_e[q] == e ? 1 : 0;
    atomicAdd(&g.cnt[my_u], 1);
  }
  __syncthreads();
  if (tid < kWave) {
    const int U = g.ppc[nw];
    const int a = tid < U ? (g.cnt[tid] + TT - 1) / TT : 0;
    const int b = tid + kWave < U ? (g.cnt[tid + kWave] + TT - 1) / TT : 0;
    const int sa = wave_scan_incl(a);
    const int sb = wave_scan_incl(b);
    const int tot_a = __shfl(sa, kWave - 1);
    g.cbase[tid] = sa - a;
    g.cbase[tid + kWave] = tot_a + sb - b;
    if (tid == kWave - 1) g.n = tot_a + sb;
  }
  __syncthreads();
  if (tid < P) {
    const int c = g.cbase[my_u] + my_pos / TT;
    const int k = my_pos % TT;
    g.cpk[c][k] = tid;
    if (k == 0) {
      g.ce[c] = g.sel_e[tid];
      g.cn[c] = min(TT, g.cnt[my_u] - my_pos);
    }
  }
  __syncthreads();
}

// Routing of every token of the step (a share of the tokens per wave, NW
// waves), then the chunk table; block 0 also writes the routing outputs.
// GP: a parameter block with M, H, E, K, routed, idx_in, w_in, part, pstride,
// norm, eps, idx_out, w_out, topk_trace, wts_trace and L (LayerDev).
template <int V, int TT, class GP>
__device__ void group_route(GroupLdsT<TT>& gl, const GP& p, int lane, int wave, int NW) {
  for (int t = wave; t < p.M; t += NW) {
    int my_e = 0;
    float my_w = 0.f, r = 1.f;
    if (p.routed) {
      my_e = clamp_expert(p.idx_in[t * p.K + (lane < p.K ? lane : 0)], p.E);
      my_w = p.w_in[t * p.K + (lane < p.K ? lane : 0)];
    } else {
      const int64_t pb = (int64_t)t * (p.E + 1) * p.pstride;
      float lg[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int e = lane + kWave * i;
        const int ec = e < p.E ? e : p.E - 1;
        lg[i] = p.part[pb + (int64_t)ec * p.pstride];
      }
      const float ssq = p.part[pb + (int64_t)p.E * p.pstride];
      if (p.norm) r = 1.0f / sqrtf(ssq / (float)p.H + p.eps);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int e = lane + kWave * i;
        lg[i] = r * lg[i] + (p.L.b_r ? p.L.b_r[e < p.E ? e : p.E - 1] : 0.f);
      }
      topk_rank<V>(lg, p.E, p.K, my_e, my_w);
    }
    if (lane < p.K) {
      gl.sel_e[t * p.K + lane] = my_e;
      if (blockIdx.x == 0) {
        p.idx_out[t * p.K + lane] = my_e;
        p.w_out[t * p.K + lane] = my_w;
        if (p.topk_trace) p.topk_trace[t * p.K + lane] = my_e;
        if (p.wts_trace) p.wts_trace[t * p.K + lane] = my_w;
      }
    }
    if (lane == 0) gl.rt[t] = r;
  }
  __syncthreads();
  build_groups<TT>(gl, p.M * p.K, p.E);
}

// The chunk table as the down kernels read it: [0] = chunks, then per chunk
// (expert, picks, pick 0 .. pick TT-1).
template <int TT>
__device__ void write_chunk_table(const GroupLdsT<TT>& gl, int32_t* out, int nthreads) {
  if (threadIdx.x == 0) out[0] = gl.n;
  for (int c = threadIdx.x; c < gl.n; c += nthreads) {
    int32_t* o = out + 1 + c * (2 + TT);
    o[0] = gl.ce[c];
    o[1] = gl.cn[c];
#pragma unroll
    for (int k = 0; k < TT; ++k) o[2 + k] = k < gl.cn[c] ? gl.cpk[c][k] : 0;
  }
}

}  // namespace bdg
