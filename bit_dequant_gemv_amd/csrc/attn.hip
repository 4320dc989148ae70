// Decode attention of a gpt-oss layer on gfx950: YaRN rotary embedding, the
// KV-cache append, learned per-head attention sinks and full or
// sliding-window causal attention with grouped KV heads.  The gpt-oss page
// ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon") names the sink kernel as
// one of its two new kernels (section 1), the 128-token window and the YaRN
// frequencies and attention scaling (section 3); the formulas are the
// published YaRN method and a softmax in which each query head's sink is one
// more logit with a zero value.
//
// Two launches per layer (one when a single block holds every cached key of
// a token), no block waiting on or signalling another.
// attn_split_kernel (flash-decoding) covers the keys already in the cache:
// block (split, kv head, token) takes a run of the token's window for the
// kGqa query heads that share the KV head, rotating their queries itself;
// each wave walks its keys in sub-chunks with its own running maximum.  A
// lane owns 8 of the 64 dimensions of one key (8 lanes per key, 8 keys per
// wave per pass): key and value loads are 1 KB contiguous per wave, the 8
// rotated queries stay in 64 registers, one transposing butterfly over the
// 8 lanes leaves lane (key, h) with head h's score, and the weighted values
// accumulate in the same lanes; the block writes (max, sum, weighted values)
// per head.  attn_merge_kernel, one wave per (kv head, pair of query heads,
// token), adds the keys of the call itself (rotated from their projections),
// merges the splits and the sink, and appends the token's key and value to
// the cache; with a single block the split kernel does this itself.
// Cross-half exchanges use gfx950's permlane swaps and DPP, not the LDS
// crossbar.
#include <math.h>

#include <mutex>

#include "bdg_device.hpp"
#include "bdg_host.hpp"

namespace bdg {

constexpr int kSplitWaves = 8;                 // waves of a split block (one of several per KV head)
constexpr int kFusedWaves = 4;                 // waves of a block that takes every cached key
constexpr int kGqa = 8;                        // query heads per KV head
constexpr int kHeadThreads = kGqa * 32;        // threads of the (head, 2 dimensions) phases
constexpr int kHd = 64;                        // head dimension
constexpr int kMaxSplits = 64;                 // blocks per (token, kv head) at most
constexpr int kTargetBlocks = 256;             // split-kernel blocks a call aims for
constexpr int kFuseKeys = 256;                 // cached keys one fused block takes
constexpr int kPartStride = kHd + 2;           // floats per head of a split: max, sum, o[64]
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- rotary table

struct RopeArgs {
  double theta, factor, beta_fast, beta_slow;
  int orig_ctx, truncate;
};

// YaRN inverse frequency of rotary pair i (float64): the base frequency
// theta^(-2i/d), and between the indices where a dimension turns beta_fast
// and beta_slow times over the original context a linear fade from it to
// the interpolated theta_i / s.
__device__ double yarn_inv_freq(int i, int d, const RopeArgs& r) {
  const double base_freq = pow(r.theta, -2.0 * (double)i / (double)d);
  if (r.factor <= 1.0) return base_freq;
  const double two_pi = 2.0 * M_PI;
  double lo = (double)d * log((double)r.orig_ctx / (r.beta_fast * two_pi)) / (2.0 * log(r.theta));
  double hi = (double)d * log((double)r.orig_ctx / (r.beta_slow * two_pi)) / (2.0 * log(r.theta));
  if (r.truncate) {
    lo = floor(lo);
    hi = ceil(hi);
  }
  lo = fmax(lo, 0.0);
  hi = fmin(hi, (double)(d - 1));
  if (lo == hi) hi += 0.001;
  const double ramp = fmin(fmax(((double)i - lo) / (hi - lo), 0.0), 1.0);
  const double keep = 1.0 - ramp;
  return (base_freq / r.factor) * (1.0 - keep) + base_freq * keep;
}

// table [n_pos][d]: cos(p f_i) a in column i, sin(p f_i) a in column d/2 + i,
// f_i and a rounded to fp32 first, the angle exact in float64, each entry
// rounded once to fp32.  One thread per (position, pair).
__global__ void __launch_bounds__(256)
attn_rope_table_kernel(RopeArgs r, int d, int64_t n_pos, float* __restrict__ table, float* __restrict__ inv_out,
                       float* __restrict__ scale_out) {
  const int half = d / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_pos * half) return;
  const int64_t p = idx / half;
  const int i = (int)(idx % half);
  const float f = (float)yarn_inv_freq(i, d, r);
  const float a = (float)(r.factor > 1.0 ? 0.1 * log(r.factor) + 1.0 : 1.0);
  double sn, cs;
  sincos((double)p * (double)f, &sn, &cs);
  table[p * d + i] = (float)(cs * (double)a);
  table[p * d + half + i] = (float)(sn * (double)a);
  if (p == 0 && inv_out) inv_out[i] = f;
  if (idx == 0 && scale_out) *scale_out = a;
}

// ---------------------------------------------------------------- rotation

// x1 c - x2 s and x2 c + x1 s with every product and the sum rounded on its
// own (no fused multiply-add): the cache entries are a rounding decision
// taken in exactly this arithmetic.
__device__ __forceinline__ float rot_first(float x1, float x2, float c, float s) {
#pragma clang fp contract(off)
  return x1 * c - x2 * s;
}
__device__ __forceinline__ float rot_second(float x1, float x2, float c, float s) {
#pragma clang fp contract(off)
  return x2 * c + x1 * s;
}

// ---------------------------------------------------------------- cache values

template <typename T>
struct Cache;

template <>
struct Cache<uint16_t> {        // bf16 cache: 8 values in one 16-byte load
  static constexpr int kU = 1;
  __device__ static float round(float x) { return __uint_as_float((uint32_t)f32_to_bf16_rne(x) << 16); }
  __device__ static void unpack(const uint4* u, float (&v)[8]) {
    const uint32_t w[4] = {u[0].x, u[0].y, u[0].z, u[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

template <>
struct Cache<float> {           // fp32 cache: 8 values in two 16-byte loads
  static constexpr int kU = 2;
  __device__ static float round(float x) { return x; }
  __device__ static void unpack(const uint4* u, float (&v)[8]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      v[4 * j] = __uint_as_float(u[j].x);
      v[4 * j + 1] = __uint_as_float(u[j].y);
      v[4 * j + 2] = __uint_as_float(u[j].z);
      v[4 * j + 3] = __uint_as_float(u[j].w);
    }
  }
};

// ---------------------------------------------------------------- attention over the cache

struct AttnArgs {
  const float* q;        // [m][hq][64] projections of the new tokens
  const float* k;        // [m][hkv][64]
  const float* v;        // [m][hkv][64]
  void* kc;              // [hkv][cap][64] cache
  void* vc;
  const float* tab;      // rotary table [rows][64]
  const float* sinks;    // [hq] or null
  float* o;              // [m][hq][64]
  float* part;           // split partials [m][hkv][n_split][kGqa][kPartStride] (workspace)
  int64_t cap, pos0;
  int hkv, window, n_split;
  int keys_per_block;    // a multiple of the sub-chunk
  float qscale;          // score scale times log2(e)
};

// first key position of token t's window
__device__ __forceinline__ int64_t window_lo(const AttnArgs& g, int64_t pt) {
  return g.window > 0 ? (pt - g.window + 1 > 0 ? pt - g.window + 1 : 0) : 0;
}

// Query head that lane db of a key group holds at position j of its score
// accumulators.  head_transpose_sum exchanges with lanes db ^ 7, db ^ 2 and
// db ^ 1 in turn; in this order each step's kept heads are the first half of
// the lane's positions and its partner sends the same heads from the second
// half, so the exchange needs no per-lane selects.
__device__ __forceinline__ int head_at(int db, int j) { return db ^ (j & 3) ^ ((j & 4) ? 7 : 0); }

// The block's 8 per-head scores of key group `a`: lane (a, db) holds the
// partial dot products d[j] of head head_at(db, j) over its 8 dimensions;
// three exchange steps (mirror within 8 lanes, then xor 2, xor 1 within 4)
// halve the heads a lane keeps and add the partner's share, ending with lane
// db holding head db's full sum.  Fixed order: deterministic.
__device__ __forceinline__ float head_transpose_sum(const float (&d)[kGqa]) {
  float k4[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) k4[c] = d[c] + dpp_f32<0x141, 0xF>(d[4 + c]);   // row_half_mirror: lane i <-> 7 - i
  float k2[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) k2[c] = k4[c] + dpp_quad_xor2(k4[2 + c]);
  return k2[0] + dpp_quad_xor1(k2[1]);
}

// a value and its partner's at lane ^ 16 / lane ^ 32 (gfx950 permlane swaps
// of a register with itself: the two results hold the pair in either order)
__device__ __forceinline__ void pair16(float x, float& u, float& v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  u = __uint_as_float(r[0]);
  v = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float x, float& u, float& v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  u = __uint_as_float(r[0]);
  v = __uint_as_float(r[1]);
}

// max / sum over the 8 key groups of a wave (lanes with equal lane & 7)
__device__ __forceinline__ float groups_max(float x) {
  float u, v;
  x = fmaxf(x, dpp_f32<0x128, 0xF>(x));                 // row_ror:8 = lane ^ 8
  pair16(x, u, v);
  x = fmaxf(u, v);
  pair32(x, u, v);
  return fmaxf(u, v);
}
__device__ __forceinline__ float groups_sum(float x) {
  float u, v;
  x += dpp_f32<0x128, 0xF>(x);
  pair16(x, u, v);
  x = u + v;
  pair32(x, u, v);
  return u + v;
}

// sum over each half-wave (32 lanes), every lane receiving its half's sum
__device__ __forceinline__ float half_sum(float x) {
  x += dpp_quad_xor1(x);
  x += dpp_quad_xor2(x);
  x += dpp_f32<0x141, 0xF>(x);                          // row_half_mirror: the other quad of 8
  x += dpp_f32<0x140, 0xF>(x);                          // row_mirror: the other 8 of 16
  float u, v;
  pair16(x, u, v);
  return u + v;
}

// maximum over each half-wave (32 lanes), every lane receiving its half's
__device__ __forceinline__ float half_max(float x) {
  x = fmaxf(x, dpp_quad_xor1(x));
  x = fmaxf(x, dpp_quad_xor2(x));
  x = fmaxf(x, dpp_f32<0x141, 0xF>(x));
  x = fmaxf(x, dpp_f32<0x140, 0xF>(x));
  float u, v;
  pair16(x, u, v);
  return fmaxf(u, v);
}

// value of lane (lane & ~7) | H, i.e. lane H of this lane's group of 8
template <int H>
__device__ __forceinline__ float bcast8(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (H << 5) | 0x18));
}

// value of lane W of this lane's group of 32
template <int W>
__device__ __forceinline__ float bcast32(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), W << 5));
}

__device__ __forceinline__ float lane_value(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// 2^x by the hardware exponential alone (v_exp_f32, 1 ulp).  The library
// exp2f adds a rescaling for results below 2^-126; every exponential here is
// a softmax weight relative to a running maximum (at most 1, and the maximum
// itself weighs 1), so such results are far below the sum's resolution.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(x - m) with an empty maximum (m = -inf) giving 0 rather than NaN
__device__ __forceinline__ float exp2_rel(float x, float m) { return m == -INFINITY ? 0.f : exp2_hw(x - m); }

// Sum over the 8 key groups of a wave of the 64 weighted-value accumulators
// acc[h][i] of lane (a, db), transposing as it halves: lane ^ 32, then ^ 16
// (gfx950's permlane32 / permlane16 swaps: each exchanges the half of one
// register that the partner keeps with the half of the other it sends, so
// the two results add to the kept sum), then ^ 8 (DPP).  Lanes keep 4, 2,
// then 1 head: lane (a, db) ends with head a's sums of dimensions 8 db ..
// 8 db + 7.  Fixed order: deterministic.
__device__ __forceinline__ float swap_sum32(float keep_lo, float keep_hi) {
  // lanes 0..31 keep keep_lo's head, lanes 32..63 keep_hi's
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(keep_lo), __float_as_uint(keep_hi), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float keep_even, float keep_odd) {
  // even 16-lane rows keep keep_even's head, odd rows keep_odd's
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(keep_even), __float_as_uint(keep_odd), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void group_transpose_sum(float (&acc)[kGqa][8], int a, float (&out)[8]) {
  const bool b0 = (a & 1) != 0;
  float s4[4][8];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) s4[c][i] = swap_sum32(acc[c][i], acc[4 + c][i]);
  float s2[2][8];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) s2[c][i] = swap_sum16(s4[c][i], s4[2 + c][i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float keep = b0 ? s2[1][i] : s2[0][i];
    const float send = b0 ? s2[0][i] : s2[1][i];
    out[i] = keep + dpp_f32<0x128, 0xF>(send);
  }
}

template <typename T, int NW>
struct AttnTile {
  using C = Cache<T>;
  static constexpr int kPasses = 4 / C::kU;                  // passes per sub-chunk
  static constexpr int kPass = NW * 8;                       // keys per block per pass (8 per wave)
  static constexpr int kSub = kPass * kPasses;               // keys per block per sub-chunk
};

// Keys of this block's sub-chunk starting at `sub`: pass p gives wave w the
// 8 keys sub + (4p + w) 8 + 0..7; passes wholly past the block's keys are
// skipped, and keys past its end repeat its last key (discarded later).
template <typename T, int NW, bool kKeys = true, bool kVals = true>
__device__ __forceinline__ void load_sub(const T* kc, const T* vc, int64_t row0, int sub, int nk, int w, int a,
                                         int db, uint4 (&kraw)[AttnTile<T, NW>::kPasses][Cache<T>::kU],
                                         uint4 (&vraw)[AttnTile<T, NW>::kPasses][Cache<T>::kU]) {
  constexpr int kPasses = AttnTile<T, NW>::kPasses, kU = Cache<T>::kU, kPass = AttnTile<T, NW>::kPass;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    if (sub + p * kPass >= nk) break;
    const int jl = sub + (p * NW + w) * 8 + a;
    const int jc = jl < nk ? jl : nk - 1;
    const int64_t off = (row0 + jc) * kHd + db * 8;
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      if constexpr (kKeys) kraw[p][i] = ldg_u128(kc + off + i * (8 / kU));
      if constexpr (kVals) vraw[p][i] = ldg_u128(vc + off + i * (8 / kU));
    }
  }
}

// Thread (head oh, dimensions e = 2 od, 2 od + 1) of a block: what it needs
// of the query and of the call's first key in the token's window, loaded up
// front (own pair, rotation partner pair e ^ 32, table rows).
struct NewKeyIn {
  float2 qx, qy, c, s;          // query own / partner pair, table row of the token
  float2 kx, ky, v, cj, sj;     // first key of the call in the window: own / partner, value, its table row
};

__device__ __forceinline__ float2 ld2(const float* p) { return *reinterpret_cast<const float2*>(p); }

__device__ __forceinline__ NewKeyIn load_new_in(const AttnArgs& g, int kvh, int t, int oh, int od) {
  NewKeyIn in;
  const int e = 2 * od, ti = e & 31;
  const int64_t pt = g.pos0 + t;
  const int64_t lo = window_lo(g, pt);
  const int64_t j0 = lo > g.pos0 ? lo : g.pos0;
  const float* qh = g.q + ((int64_t)t * g.hkv * kGqa + kvh * kGqa + oh) * kHd;
  in.qx = ld2(qh + e);
  in.qy = ld2(qh + (e ^ 32));
  in.c = ld2(g.tab + pt * kHd + ti);
  in.s = ld2(g.tab + pt * kHd + 32 + ti);
  const int64_t k0 = ((j0 - g.pos0) * g.hkv + kvh) * kHd;
  in.kx = ld2(g.k + k0 + e);
  in.ky = ld2(g.k + k0 + (e ^ 32));
  in.v = ld2(g.v + k0 + e);
  in.cj = ld2(g.tab + j0 * kHd + ti);
  in.sj = ld2(g.tab + j0 * kHd + 32 + ti);
  return in;
}

// rotation of an own / partner pair (dimensions below 32 are the first half)
__device__ __forceinline__ float2 rot_pair(float2 own, float2 par, float2 c, float2 s, bool first) {
  return first ? make_float2(rot_first(own.x, par.x, c.x, s.x), rot_first(own.y, par.y, c.y, s.y))
               : make_float2(rot_second(par.x, own.x, c.x, s.x), rot_second(par.y, own.y, c.y, s.y));
}

template <typename T>
__device__ __forceinline__ void merge_heads(const AttnArgs& g, int kvh, int t, int oh, int od, const NewKeyIn& in,
                                            const float* pb, int n_split, float* wls, float bm, float bl, float o0,
                                            float o1);


template <typename T, bool kFused>
__global__ void __launch_bounds__(kFused ? kFusedWaves * kWave : kSplitWaves * kWave)
attn_split_kernel(AttnArgs g) {
  constexpr int NW = kFused ? kFusedWaves : kSplitWaves;
  using C = Cache<T>;
  constexpr int kPasses = AttnTile<T, NW>::kPasses;
  constexpr int kSub = AttnTile<T, NW>::kSub;
  constexpr int kPass = AttnTile<T, NW>::kPass;
  __shared__ float wo[NW][kGqa][kHd];
  __shared__ float wm[NW][kGqa], wl[NW][kGqa];
  __shared__ float qlds[kGqa][kHd];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int a = lane >> 3, db = lane & 7;
  const int t = blockIdx.z, kvh = blockIdx.y, split = blockIdx.x;
  const int hq = g.hkv * kGqa;
  const int64_t pt = g.pos0 + t;
  const int64_t jb = window_lo(g, pt) + (int64_t)split * g.keys_per_block;
  const int64_t je = jb + g.keys_per_block < g.pos0 ? jb + g.keys_per_block : g.pos0;   // cached keys only
  const int nk = je > jb ? (int)(je - jb) : 0;
  const T* kc = reinterpret_cast<const T*>(g.kc);
  const T* vc = reinterpret_cast<const T*>(g.vc);
  const int64_t row0 = (int64_t)kvh * g.cap + jb;             // cache row of key jb

  // the query's rotation inputs first, so rotating them (below) waits only
  // for these and overlaps the cache loads: thread (head, pair i) takes
  // dimensions i and i + 32 of one of the 8 query heads of this KV head
  const int qh_i = (tid >> 5) & (kGqa - 1), q_i = tid & 31;
  const float* qh = g.q + ((int64_t)t * hq + kvh * kGqa + qh_i) * kHd;
  const float* tr = g.tab + pt * kHd;
  const float qx1 = qh[q_i], qx2 = qh[q_i + 32], qc = tr[q_i], qsn = tr[32 + q_i];
  __builtin_amdgcn_sched_barrier(0);
  uint4 kraw[kPasses][C::kU], vraw[kPasses][C::kU];
  if (nk > 0) load_sub<T, NW>(kc, vc, row0, 0, nk, w, a, db, kraw, vraw);
  NewKeyIn nin;
  if constexpr (kFused) nin = load_new_in(g, kvh, t, (tid >> 5) & (kGqa - 1), tid & 31);
  __builtin_amdgcn_sched_barrier(0);

  // rotated and scaled by qscale into LDS; lane (a, db) then keeps dimensions
  // 8 db .. of every head in registers, head head_at(db, j) at position j
  if (tid < kHeadThreads) {
    qlds[qh_i][q_i] = rot_first(qx1, qx2, qc, qsn) * g.qscale;
    qlds[qh_i][q_i + 32] = rot_second(qx1, qx2, qc, qsn) * g.qscale;
  }
  __syncthreads();
  float qs[kGqa][8];
#pragma unroll
  for (int j = 0; j < kGqa; ++j) {
    const int h = head_at(db, j);
    const float4 lo4 = *reinterpret_cast<const float4*>(&qlds[h][db * 8]);
    const float4 hi4 = *reinterpret_cast<const float4*>(&qlds[h][db * 8 + 4]);
    qs[j][0] = lo4.x; qs[j][1] = lo4.y; qs[j][2] = lo4.z; qs[j][3] = lo4.w;
    qs[j][4] = hi4.x; qs[j][5] = hi4.y; qs[j][6] = hi4.z; qs[j][7] = hi4.w;
  }

  float m_mine = -INFINITY; // running maximum of head db (equal in the lanes of equal db)
  float acc[kGqa][8];       // weighted values: head h, dimensions 8 db ..
  float lsum = 0.f;         // this lane's share of head db's weight sum
#pragma unroll
  for (int h = 0; h < kGqa; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;

  for (int sub = 0; sub < nk; sub += kSub) {
    float s[kPasses];
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      s[p] = -INFINITY;
      if (sub + p * kPass >= nk) break;
      const int jl = sub + (p * NW + w) * 8 + a;
      float kf[8];
      C::unpack(kraw[p], kf);
      float d[kGqa];
#pragma unroll
      for (int j = 0; j < kGqa; ++j) {
        float x = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) x += qs[j][i] * kf[i];
        d[j] = x;
      }
      const float sc = head_transpose_sum(d);
      s[p] = jl < nk ? sc : -INFINITY;
      mx = fmaxf(mx, s[p]);
    }
    // the next sub-chunk's keys load during this one's softmax and value sums
    const bool more = sub + kSub < nk;
    if (more) load_sub<T, NW, true, false>(kc, vc, row0, sub + kSub, nk, w, a, db, kraw, vraw);
    // new running maximum of head db (the group maximum is head db's in
    // every lane of equal db)
    mx = groups_max(mx);
    const float m_new = fmaxf(m_mine, mx);
    if (sub > 0) {
      // rescale what earlier sub-chunks gathered (before the first there is
      // nothing: the factor would be 0 on zero sums); lane h holds head h's
      // factor
      const float f_mine = exp2_rel(m_mine, m_new);
      lsum *= f_mine;
#pragma unroll
      for (int h = 0; h < kGqa; ++h) {
        const float fac = lane_value(f_mine, h);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] *= fac;
      }
    }
    m_mine = m_new;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      if (sub + p * kPass >= nk) break;
      const float e = exp2_rel(s[p], m_mine);              // weight of (head db, key a)
      lsum += e;
      float vf[8];
      C::unpack(vraw[p], vf);
      const float e8[kGqa] = {bcast8<0>(e), bcast8<1>(e), bcast8<2>(e), bcast8<3>(e),
                              bcast8<4>(e), bcast8<5>(e), bcast8<6>(e), bcast8<7>(e)};
#pragma unroll
      for (int h = 0; h < kGqa; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] += e8[h] * vf[i];
    }
    // and its values during the next one's scores
    if (more) load_sub<T, NW, false, true>(kc, vc, row0, sub + kSub, nk, w, a, db, kraw, vraw);
  }

  // wave results: weight sums per head, weighted values of head a
  lsum = groups_sum(lsum);
  float o8[8];
  group_transpose_sum(acc, a, o8);
  if (a == 0) {
    wm[w][db] = m_mine;
    wl[w][db] = lsum;
  }
  *reinterpret_cast<float4*>(&wo[w][a][db * 8]) = make_float4(o8[0], o8[1], o8[2], o8[3]);
  *reinterpret_cast<float4*>(&wo[w][a][db * 8 + 4]) = make_float4(o8[4], o8[5], o8[6], o8[7]);
  __syncthreads();

  // block partial: thread (head oh, dimensions 2 od, 2 od + 1)
  if (tid >= kHeadThreads) return;
  const int oh = tid >> 5, od = tid & 31;
  float bm = wm[0][oh];
#pragma unroll
  for (int ww = 1; ww < NW; ++ww) bm = fmaxf(bm, wm[ww][oh]);
  // thread od < NW weighs wave od; the head's 32 threads share the factors
  const float f_own = exp2_rel(wm[od < NW ? od : 0][oh], bm);
  const float fw[8] = {bcast32<0>(f_own), bcast32<1>(f_own), bcast32<2>(f_own), bcast32<3>(f_own),
                       bcast32<4 % NW>(f_own), bcast32<5 % NW>(f_own), bcast32<6 % NW>(f_own),
                       bcast32<7 % NW>(f_own)};
  float bl = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const float f = fw[ww];
    bl += f * wl[ww][oh];
    o0 += f * wo[ww][oh][2 * od];
    o1 += f * wo[ww][oh][2 * od + 1];
  }
  if constexpr (kFused) {                    // one block holds every cached key: merge here
    merge_heads<T>(g, kvh, t, oh, od, nin, nullptr, 0, nullptr, bm, bl, o0, o1);
  } else {
    float* pp = g.part + ((((int64_t)t * g.hkv + kvh) * g.n_split + split) * kGqa + oh) * kPartStride;
    if (od == 0) *reinterpret_cast<float2*>(pp) = make_float2(bm, bl);
    *reinterpret_cast<float2*>(pp + 2 + 2 * od) = make_float2(o0, o1);
  }
}

// ---------------------------------------------------------------- merge, new keys, append

// The softmax of one (token, query head) over the cached-key splits, the
// keys of this call and the sink, by thread (oh, od) for dimensions 2 od and
// 2 od + 1.  Splits come from `pb` ([n_split][kGqa][kPartStride], global) or,
// with pb null, as the single partial (bm, bl, o0, o1) in registers.  With
// pb, the caller is one wave holding two heads (lanes 0-31, 32-63) and `wls`
// is its LDS row of 64 floats: lane od loads the (max, sum) of split od of a
// chunk, weighs that split against the half-wave's maximum, and the
// half-wave reads the 32 weights back from LDS; a chunk costs 33 global
// loads per lane (a wave keeps at most 63 in flight) and one exponential.  The
// call's keys are rotated from their projections in the cache's rounding and
// scored with a sum over the head's 32 threads; threads of head 0 append the
// token's own key and value to the cache.
template <typename T>
__device__ __forceinline__ void merge_heads(const AttnArgs& g, int kvh, int t, int oh, int od, const NewKeyIn& in,
                                            const float* pb, int n_split, float* wls, float bm, float bl, float o0,
                                            float o1) {
  using C = Cache<T>;
  const int e = 2 * od, ti = e & 31;
  const bool first = e < 32;
  const int hq = g.hkv * kGqa;
  const int64_t pt = g.pos0 + t;
  const int64_t lo = window_lo(g, pt);
  const int64_t j0 = lo > g.pos0 ? lo : g.pos0;

  // running softmax state: max, weight sum, weighted values
  float M = -INFINITY, L = 0.f, A0 = 0.f, A1 = 0.f;
  if (pb == nullptr) {
    M = bm; L = bl; A0 = o0; A1 = o1;
  } else {
    constexpr int kChunk = 32;
    const int half = threadIdx.x & 32;
    for (int c0 = 0; c0 < n_split; c0 += kChunk) {
      // splits past the end read the chunk's first split and weigh nothing
      const int so = c0 + od < n_split ? c0 + od : c0;
      const float2 ml_own = ld2(pb + ((int64_t)so * kGqa + oh) * kPartStride);
      float2 ov[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int sp = c0 + u < n_split ? c0 + u : c0;
        ov[u] = ld2(pb + ((int64_t)sp * kGqa + oh) * kPartStride + 2 + e);
      }
      // the chunk's maximum over the half-wave (repeated splits change no
      // maximum), then lane od weighs split od alone
      const float cm = fmaxf(M, half_max(ml_own.x));
      const float f = exp2_rel(M, cm);
      const float w_own = c0 + od < n_split ? exp2_rel(ml_own.x, cm) : 0.f;
      L = L * f + half_sum(w_own * ml_own.y);
      wls[threadIdx.x] = w_own;
      __syncthreads();
      float wgt[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) wgt[u] = wls[half + u];
      __syncthreads();                         // the next chunk rewrites wls
      A0 *= f; A1 *= f;
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        A0 += wgt[u] * ov[u].x;
        A1 += wgt[u] * ov[u].y;
      }
      M = cm;
    }
  }

  // the call's keys in the window
  const float2 qr = rot_pair(in.qx, in.qy, in.c, in.s, first);
  const float q0 = qr.x * g.qscale, q1 = qr.y * g.qscale;
  for (int64_t j = j0; j <= pt; ++j) {
    float2 kx = in.kx, ky = in.ky, vv = in.v, cj = in.cj, sj = in.sj;
    if (j > j0) {
      const int64_t ki = ((j - g.pos0) * g.hkv + kvh) * kHd;
      kx = ld2(g.k + ki + e);
      ky = ld2(g.k + ki + (e ^ 32));
      vv = ld2(g.v + ki + e);
      cj = ld2(g.tab + j * kHd + ti);
      sj = ld2(g.tab + j * kHd + 32 + ti);
    }
    const float2 kr = rot_pair(kx, ky, cj, sj, first);
    const float k0 = C::round(kr.x), k1 = C::round(kr.y);
    const float v0 = C::round(vv.x), v1 = C::round(vv.y);
    if (j == pt && oh == 0) {                // the token's own key and value into the cache
      const int64_t ci = ((int64_t)kvh * g.cap + pt) * kHd + e;
      if constexpr (sizeof(T) == 2) {
        const uint32_t kb = (uint32_t)f32_to_bf16_rne(k0) | ((uint32_t)f32_to_bf16_rne(k1) << 16);
        const uint32_t vb = (uint32_t)f32_to_bf16_rne(v0) | ((uint32_t)f32_to_bf16_rne(v1) << 16);
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(g.kc) + ci) = kb;
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(g.vc) + ci) = vb;
      } else {
        *reinterpret_cast<float2*>(reinterpret_cast<float*>(g.kc) + ci) = make_float2(k0, k1);
        *reinterpret_cast<float2*>(reinterpret_cast<float*>(g.vc) + ci) = make_float2(v0, v1);
      }
    }
    const float sc = half_sum(q0 * k0 + q1 * k1);
    const float m2 = fmaxf(M, sc);
    const float f = exp2_rel(M, m2), ew = exp2_hw(sc - m2);
    L = L * f + ew;
    A0 = A0 * f + ew * v0;
    A1 = A1 * f + ew * v1;
    M = m2;
  }

  // the sink: one more logit with a zero value
  const int qh = kvh * kGqa + oh;
  if (g.sinks) {
    const float sk = g.sinks[qh] * kLog2e;
    const float m2 = fmaxf(M, sk);
    const float f = exp2_rel(M, m2);
    L = L * f + exp2_hw(sk - m2);
    A0 *= f;
    A1 *= f;
  }
  const float inv = 1.f / L;
  *reinterpret_cast<float2*>(g.o + ((int64_t)t * hq + qh) * kHd + e) = make_float2(A0 * inv, A1 * inv);
}

// One wave per (kv head, pair of query heads, token): 32 threads per head,
// so the partials of a KV head are read by four CUs rather than one.
template <typename T>
__global__ void __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_merge_kernel(AttnArgs g) {
  const int kvh = blockIdx.x >> 2, t = blockIdx.y;
  const int oh = (blockIdx.x & 3) * 2 + (threadIdx.x >> 5), od = threadIdx.x & 31;
  __shared__ float wls[kWave];
  const NewKeyIn in = load_new_in(g, kvh, t, oh, od);
  merge_heads<T>(g, kvh, t, oh, od, in, g.part + ((int64_t)t * g.hkv + kvh) * g.n_split * kGqa * kPartStride,
                 g.n_split, wls, 0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------- host side

// Keys per block: whole passes of 32 keys.  Up to kFuseKeys cached keys go
// to one block (the fused single launch); longer ranges are split to fill
// the chip (about kTargetBlocks blocks over all tokens and KV heads), at most
// kMaxSplits per token and KV head.
inline int64_t attn_keys_per_block(int64_t keys, int hkv, int m) {
  if (keys <= kFuseKeys) return (keys + kFusedWaves * 8 - 1) / (kFusedWaves * 8) * (kFusedWaves * 8);
  int64_t splits = kTargetBlocks / ((int64_t)hkv * m);
  splits = splits < 1 ? 1 : splits > kMaxSplits ? kMaxSplits : splits;
  const int64_t per = (keys + splits - 1) / splits;
  return (per + kSplitWaves * 8 - 1) / (kSplitWaves * 8) * (kSplitWaves * 8);
}

inline int64_t attn_ws_bytes(int hkv, int m, int64_t max_keys) {
  return (int64_t)m * hkv * kMaxSplits * kGqa * kPartStride * 4;
}

}  // namespace bdg

using namespace bdg;

extern "C" int attn_rope_table(const bdg_rope* rope, int32_t head_dim, int64_t n_pos, float* table,
                               float* inv_freq, float* attn_scale, void* stream) {
  if (!rope || !table || head_dim < 2 || (head_dim % 2) != 0 || n_pos < 1) return BDG_E_INVALID;
  if (!(rope->theta > 1.0) || !(rope->factor > 0.0) || rope->orig_ctx < 1 || !(rope->beta_fast > 0.0) ||
      !(rope->beta_slow > 0.0) || (rope->truncate != 0 && rope->truncate != 1))
    return BDG_E_INVALID;
  if (head_dim > 1024 || n_pos > (int64_t)1 << 31) return BDG_E_UNSUPPORTED;
  const RopeArgs r{rope->theta, rope->factor, rope->beta_fast, rope->beta_slow, rope->orig_ctx, rope->truncate};
  const int64_t n = n_pos * (head_dim / 2);
  hipLaunchKernelGGL(attn_rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, as_stream(stream), r,
                     head_dim, n_pos, table, inv_freq, attn_scale);
  return launch_status();
}

constexpr int kAttnMaxM = 64;

extern "C" int64_t attn_decode_workspace(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t m,
                                         int64_t max_keys) {
  if (n_kv_heads < 1 || n_kv_heads > 65535 || n_heads != n_kv_heads * kGqa || head_dim != kHd || m < 1 ||
      m > kAttnMaxM || max_keys < 1)
    return -1;
  return attn_ws_bytes(n_kv_heads, m, max_keys);
}

// The attention step over a workspace the caller (attn_decode) or the
// library's static scratch (attn_decode_noalloc) provides.
static int attn_decode_impl(const float* q, const float* k, const float* v, void* k_cache, void* v_cache,
                            int32_t cache_dtype, int64_t cache_cap, int32_t n_heads, int32_t n_kv_heads,
                            int32_t head_dim, int32_t m, int64_t pos0, const float* rope_table, int64_t table_rows,
                            float sm_scale, const float* sinks, int32_t window, float* o, void* workspace,
                            int64_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !k_cache || !v_cache || !rope_table || !o || !workspace) return BDG_E_INVALID;
  if (cache_dtype != BDG_F32 && cache_dtype != BDG_BF16) return BDG_E_INVALID;
  if (m < 1 || n_kv_heads < 1 || n_heads < 1 || pos0 < 0 || window < 0 || !(sm_scale > 0.f)) return BDG_E_INVALID;
  if (pos0 + m > cache_cap || pos0 + m > table_rows) return BDG_E_INVALID;
  if (n_heads != n_kv_heads * kGqa || head_dim != kHd) return BDG_E_UNSUPPORTED;
  if (m > kAttnMaxM || n_kv_heads > 65535) return BDG_E_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(rope_table) || !aligned16(o) || !aligned16(workspace))
    return BDG_E_ALIGN;
  if (workspace_bytes < attn_ws_bytes(n_kv_heads, m, pos0 + m)) return BDG_E_INVALID;
  // cached keys the first token attends: the longest run over the tokens
  const int64_t lo0 = window > 0 && pos0 - window + 1 > 0 ? pos0 - window + 1 : 0;
  const int64_t old_keys = pos0 - lo0;
  const int64_t kpb = old_keys > 0 ? attn_keys_per_block(old_keys, n_kv_heads, m) : kFusedWaves * 8;
  const int64_t n_split = old_keys > 0 ? (old_keys + kpb - 1) / kpb : 0;
  if (kpb > ((int64_t)1 << 30)) return BDG_E_UNSUPPORTED;
  AttnArgs g{};
  g.q = q; g.k = k; g.v = v; g.kc = k_cache; g.vc = v_cache; g.tab = rope_table; g.sinks = sinks; g.o = o;
  g.part = reinterpret_cast<float*>(workspace);
  g.cap = cache_cap; g.pos0 = pos0; g.hkv = n_kv_heads; g.window = window; g.n_split = (int)n_split;
  g.keys_per_block = (int)kpb;
  g.qscale = sm_scale * kLog2e;
  const dim3 grid((unsigned)n_split, (unsigned)n_kv_heads, (unsigned)m);
  const dim3 grid_m((unsigned)n_kv_heads * (kGqa / 2), (unsigned)m);
  // one block per (token, kv head) covers the cached keys: a single fused launch
  if (cache_dtype == BDG_BF16) {
    if (n_split == 1) {
      hipLaunchKernelGGL((attn_split_kernel<uint16_t, true>), grid, dim3(kFusedWaves * kWave), 0, as_stream(stream), g);
    } else {
      if (n_split > 0)
        hipLaunchKernelGGL((attn_split_kernel<uint16_t, false>), grid, dim3(kSplitWaves * kWave), 0, as_stream(stream), g);
      hipLaunchKernelGGL(attn_merge_kernel<uint16_t>, grid_m, dim3(kWave), 0, as_stream(stream), g);
    }
  } else {
    if (n_split == 1) {
      hipLaunchKernelGGL((attn_split_kernel<float, true>), grid, dim3(kFusedWaves * kWave), 0, as_stream(stream), g);
    } else {
      if (n_split > 0)
        hipLaunchKernelGGL((attn_split_kernel<float, false>), grid, dim3(kSplitWaves * kWave), 0, as_stream(stream), g);
      hipLaunchKernelGGL(attn_merge_kernel<float>, grid_m, dim3(kWave), 0, as_stream(stream), g);
    }
  }
  return launch_status();
}

extern "C" int attn_decode(const float* q, const float* k, const float* v, void* k_cache, void* v_cache,
                           int32_t cache_dtype, int64_t cache_cap, int32_t n_heads, int32_t n_kv_heads,
                           int32_t head_dim, int32_t m, int64_t pos0, const float* rope_table, int64_t table_rows,
                           float sm_scale, const float* sinks, int32_t window, float* o, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  return attn_decode_impl(q, k, v, k_cache, v_cache, cache_dtype, cache_cap, n_heads, n_kv_heads, head_dim, m,
                          pos0, rope_table, table_rows, sm_scale, sinks, window, o, workspace, workspace_bytes,
                          stream);
}

// ---------------------------------------------------------------- allocation-free variant

// The split partials of attn_decode_noalloc live in this device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): it uses the device address hipGetSymbolAddress returns for the
// current device, looked up once per device at that device's first call.
static __device__ __align__(256) unsigned char scratch[BDG_ATTN_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, or null

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BDG_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BDG_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return BDG_E_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return BDG_OK;
}
}  // namespace

extern "C" int attn_decode_noalloc(const float* q, const float* k, const float* v, void* k_cache, void* v_cache,
                                   int32_t cache_dtype, int64_t cache_cap, int32_t n_heads, int32_t n_kv_heads,
                                   int32_t head_dim, int32_t m, int64_t pos0, const float* rope_table,
                                   int64_t table_rows, float sm_scale, const float* sinks, int32_t window, float* o,
                                   void* stream) {
  const int64_t need = attn_decode_workspace(n_heads, n_kv_heads, head_dim, m, pos0 + m);
  if (need > (int64_t)BDG_ATTN_SCRATCH_BYTES) return BDG_E_TOO_LARGE;   // (need < 0: impl reports it)
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != BDG_OK) return st;
  return attn_decode_impl(q, k, v, k_cache, v_cache, cache_dtype, cache_cap, n_heads, n_kv_heads, head_dim, m, pos0,
                          rope_table, table_rows, sm_scale, sinks, window, o, ws, BDG_ATTN_SCRATCH_BYTES, stream);
}
