// Decode attention of a gpt-oss layer on gfx950: YaRN rotary embedding, the
// KV-cache append, learned per-head attention sinks and full or
// sliding-window causal attention with grouped KV heads, in one launch per
// layer.  The gpt-oss page ("Sovereign gpt-oss-20B (MXFP4) on Apple
// Silicon") names the sink kernel as one of its two new kernels (section 1),
// the 128-token window and the YaRN frequencies and attention scaling
// (section 3); the formulas are the published YaRN method and a softmax in
// which each query head's sink is one more logit with a zero value.
//
// Work split (flash-decoding): block (split, kv head, token) takes up to
// kKeys keys of the token's window for the kGqa query heads that share the
// KV head.  A lane owns 8 of the 64 dimensions of one key (8 lanes per key,
// 8 keys per wave per pass): the key loads are 1 KB contiguous per wave, the
// rotated queries of the 8 heads stay in 64 registers, and one transposing
// butterfly over the 8 lanes leaves lane (key, h) with head h's score.
// Values go to LDS as fp32; the weighted sum runs with lane (head, 8 dims).
// Each block writes (max, sum, weighted values) per head; the last block of
// a (token, kv head) to finish - found with one atomic counter - merges the
// splits with the sink.  No block waits on another.
#include <math.h>

#include "bdg_device.hpp"
#include "bdg_host.hpp"

namespace bdg {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kGqa = 8;                        // query heads per KV head
constexpr int kHd = 64;                        // head dimension
constexpr int kKeys = 128;                     // keys per block
constexpr int kKeysPerWave = kKeys / kAttnWaves;
constexpr int kPasses = kKeysPerWave / 8;      // 8 keys per wave per pass
constexpr int kPartStride = kHd + 2;           // floats per head of a split: max, sum, o[64]
constexpr float kLog2e = 1.4426950408889634f;

static_assert(kKeys % (8 * kAttnWaves) == 0, "keys per block");

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

__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = ldg_f4(p), b = ldg_f4(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Dimensions 8 db .. 8 db + 7 of a head vector x [64] rotated at the table
// row `tr` [64]: pair i of the first half is (i, i + 32).
__device__ __forceinline__ void rotate8(const float* x, const float* tr, int db, float (&out)[8]) {
  float own[8], par[8], c[8], s[8];
  ld8(x + db * 8, own);
  ld8(x + (db ^ 4) * 8, par);
  ld8(tr + (db & 3) * 8, c);
  ld8(tr + 32 + (db & 3) * 8, s);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    out[i] = db < 4 ? rot_first(own[i], par[i], c[i], s[i]) : rot_second(par[i], own[i], c[i], s[i]);
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
  __device__ static void store8(uint16_t* p, const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_rne(v[2 * i]) | ((uint32_t)f32_to_bf16_rne(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
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
  __device__ static void store8(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// ---------------------------------------------------------------- attention

struct AttnArgs {
  const float* q;        // [m][hq][64] projections of the new tokens
  const float* k;        // [m][hkv][64]
  const float* v;        // [m][hkv][64]
  void* kc;              // [hkv][cap][64] cache
  void* vc;
  const float* tab;      // rotary table [rows][64]
  const float* sinks;    // [hq] or null
  float* o;              // [m][hq][64]
  float* part;           // split partials [m][hkv][n_split][kGqa][kPartStride]
  int32_t* counters;     // [m][hkv], zero between calls
  int64_t cap, pos0;
  int hkv, window;
  float qscale;          // score scale times log2(e)
};

// The block's 8 per-head scores of key group `a`: lane (a, db) holds the
// partial dot products acc[h] over its 8 dimensions; three exchange steps
// (mirror within 8 lanes, then xor 2, xor 1 within 4) halve the heads a
// lane keeps and add the partner's share, ending with lane db holding head
// db's full sum.  Fixed order: deterministic.
__device__ __forceinline__ float head_transpose_sum(const float (&acc)[kGqa], int db) {
  const bool up4 = db >= 4, b1 = (db & 2) != 0, b0 = (db & 1) != 0;
  float k4[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float keep = up4 ? acc[4 + c] : acc[c];
    const float send = up4 ? acc[c] : acc[4 + c];
    k4[c] = keep + dpp_f32<0x141, 0xF>(send);          // row_half_mirror: lane i <-> 7 - i
  }
  float k2[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float keep = b1 ? k4[2 + c] : k4[c];
    const float send = b1 ? k4[c] : k4[2 + c];
    k2[c] = keep + dpp_quad_xor2(send);
  }
  const float keep = b0 ? k2[1] : k2[0];
  const float send = b0 ? k2[0] : k2[1];
  return keep + dpp_quad_xor1(send);
}

// max / sum over the 8 key groups of a wave (lanes with equal lane & 7)
__device__ __forceinline__ float groups_max(float x) {
  x = fmaxf(x, dpp_f32<0x128, 0xF>(x));                 // row_ror:8 = lane ^ 8
  x = fmaxf(x, swz_xor<16>(x));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float groups_sum(float x) {
  x += dpp_f32<0x128, 0xF>(x);
  x += swz_xor<16>(x);
  return x + __shfl_xor(x, 32);
}

template <typename T>
__global__ void __launch_bounds__(kAttnThreads)
attn_decode_kernel(AttnArgs g) {
  using C = Cache<T>;
  constexpr int kUnitsPerKey = kHd * (int)sizeof(T) / 16;     // 16-byte units of a value row
  constexpr int kValsPerUnit = 16 / (int)sizeof(T);
  constexpr int kVUnits = kKeys * kUnitsPerKey / kAttnThreads; // value units per thread
  __shared__ float vs[kKeys][kHd];
  __shared__ float ps[kKeys][kGqa];
  __shared__ float ow[kAttnWaves][kGqa][kHd];
  __shared__ float red_m[kAttnWaves][kGqa], red_l[kAttnWaves][kGqa];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int a = lane >> 3, db = lane & 7;
  const int t = blockIdx.z, kvh = blockIdx.y, split = blockIdx.x, n_split = gridDim.x;
  const int hq = g.hkv * kGqa;
  const int64_t pt = g.pos0 + t;
  const int64_t lo = g.window > 0 ? (pt - g.window + 1 > 0 ? pt - g.window + 1 : 0) : 0;
  const int64_t jb = lo + (int64_t)split * kKeys;
  const int64_t je = jb + kKeys < pt + 1 ? jb + kKeys : pt + 1;
  const int nk = je > jb ? (int)(je - jb) : 0;
  const T* kc = reinterpret_cast<const T*>(g.kc);
  const T* vc = reinterpret_cast<const T*>(g.vc);
  const int64_t row0 = (int64_t)kvh * g.cap + jb;             // cache row of key jb

  // this thread's share of the block result: head oh, dimensions 2 od, 2 od + 1
  const int oh = tid >> 5, od = tid & 31;
  float blk_m = -INFINITY, blk_l = 0.f, o0 = 0.f, o1 = 0.f;

  if (nk > 0) {
    // value rows and this lane's key rows, all loads issued up front (rows
    // past the block's keys repeat its last key and are discarded)
    uint4 vraw[kVUnits];
#pragma unroll
    for (int r = 0; r < kVUnits; ++r) {
      const int u = tid + r * kAttnThreads;
      const int jl = u / kUnitsPerKey, part = u % kUnitsPerKey;
      const int jc = jl < nk ? jl : nk - 1;
      vraw[r] = ldg_u128(vc + (row0 + jc) * kHd + part * kValsPerUnit);
    }
    uint4 kraw[kPasses][C::kU];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int jl = w * kKeysPerWave + p * 8 + a;
      const int jc = jl < nk ? jl : nk - 1;
#pragma unroll
      for (int i = 0; i < C::kU; ++i) kraw[p][i] = ldg_u128(kc + (row0 + jc) * kHd + db * 8 + i * (8 / C::kU));
    }

    // the 8 query heads of this KV head, rotated, scaled by qscale
    float qs[kGqa][8];
    const float* tr = g.tab + pt * kHd;
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      float r8[8];
      rotate8(g.q + ((int64_t)t * hq + kvh * kGqa + h) * kHd, tr, db, r8);
#pragma unroll
      for (int i = 0; i < 8; ++i) qs[h][i] = r8[i] * g.qscale;
    }

    // scores
    float sc[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int jl = w * kKeysPerWave + p * 8 + a;
      const int64_t j = jb + jl;
      float kf[8];
      C::unpack(kraw[p], kf);
      if (jl < nk && j >= g.pos0) {        // a key of this call: rotate its projection
        float r8[8];
        rotate8(g.k + ((j - g.pos0) * g.hkv + kvh) * kHd, g.tab + j * kHd, db, r8);
#pragma unroll
        for (int i = 0; i < 8; ++i) kf[i] = C::round(r8[i]);
      }
      float acc[kGqa];
#pragma unroll
      for (int h = 0; h < kGqa; ++h) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s += qs[h][i] * kf[i];
        acc[h] = s;
      }
      const float s = head_transpose_sum(acc, db);
      sc[p] = jl < nk ? s : -INFINITY;
    }

    // per-head maximum over the block
    float mx = sc[0];
#pragma unroll
    for (int p = 1; p < kPasses; ++p) mx = fmaxf(mx, sc[p]);
    mx = groups_max(mx);
    if (a == 0) red_m[w][db] = mx;
    __syncthreads();
    const float mh = fmaxf(fmaxf(red_m[0][db], red_m[1][db]), fmaxf(red_m[2][db], red_m[3][db]));
    float ls = 0.f;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const float e = exp2f(sc[p] - mh);
      ps[w * kKeysPerWave + p * 8 + a][db] = e;
      ls += e;
    }
    ls = groups_sum(ls);
    if (a == 0) red_l[w][db] = ls;

    // values to LDS as fp32 (keys of this call from their projections)
#pragma unroll
    for (int r = 0; r < kVUnits; ++r) {
      const int u = tid + r * kAttnThreads;
      const int jl = u / kUnitsPerKey, part = u % kUnitsPerKey;
      const int64_t j = jb + jl;
      float vals[kValsPerUnit];
      if constexpr (kValsPerUnit == 8) {
        float v8[8];
        C::unpack(&vraw[r], v8);
#pragma unroll
        for (int i = 0; i < 8; ++i) vals[i] = v8[i];
      } else {
        vals[0] = __uint_as_float(vraw[r].x);
        vals[1] = __uint_as_float(vraw[r].y);
        vals[2] = __uint_as_float(vraw[r].z);
        vals[3] = __uint_as_float(vraw[r].w);
      }
      if (jl < nk && j >= g.pos0) {
        const float* src = g.v + ((j - g.pos0) * g.hkv + kvh) * kHd + part * kValsPerUnit;
#pragma unroll
        for (int i = 0; i < kValsPerUnit; ++i) vals[i] = C::round(src[i]);
      }
#pragma unroll
      for (int i = 0; i < kValsPerUnit; ++i) vs[jl][part * kValsPerUnit + i] = jl < nk ? vals[i] : 0.f;
    }

    // the block that holds the token's own position appends its key and value
    if (pt < je && w == 0 && a == 0) {
      float r8[8], v8[8];
      rotate8(g.k + ((int64_t)t * g.hkv + kvh) * kHd, tr, db, r8);
      ld8(g.v + ((int64_t)t * g.hkv + kvh) * kHd + db * 8, v8);
      C::store8(reinterpret_cast<T*>(g.kc) + ((int64_t)kvh * g.cap + pt) * kHd + db * 8, r8);
      C::store8(reinterpret_cast<T*>(g.vc) + ((int64_t)kvh * g.cap + pt) * kHd + db * 8, v8);
    }
    __syncthreads();

    // weighted values: lane (head a, dimensions 8 db ..), this wave's keys
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int kk = 0; kk < kKeysPerWave; ++kk) {
      const int jl = w * kKeysPerWave + kk;
      const float pw = ps[jl][a];
      const float4 va = *reinterpret_cast<const float4*>(&vs[jl][db * 8]);
      const float4 vb = *reinterpret_cast<const float4*>(&vs[jl][db * 8 + 4]);
      acc[0] += pw * va.x; acc[1] += pw * va.y; acc[2] += pw * va.z; acc[3] += pw * va.w;
      acc[4] += pw * vb.x; acc[5] += pw * vb.y; acc[6] += pw * vb.z; acc[7] += pw * vb.w;
    }
    *reinterpret_cast<float4*>(&ow[w][a][db * 8]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(&ow[w][a][db * 8 + 4]) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    __syncthreads();
    blk_m = fmaxf(fmaxf(red_m[0][oh], red_m[1][oh]), fmaxf(red_m[2][oh], red_m[3][oh]));
    blk_l = (red_l[0][oh] + red_l[1][oh]) + (red_l[2][oh] + red_l[3][oh]);
    o0 = (ow[0][oh][2 * od] + ow[1][oh][2 * od]) + (ow[2][oh][2 * od] + ow[3][oh][2 * od]);
    o1 = (ow[0][oh][2 * od + 1] + ow[1][oh][2 * od + 1]) + (ow[2][oh][2 * od + 1] + ow[3][oh][2 * od + 1]);
  }

  const int qh = kvh * kGqa + oh;
  const float sink = g.sinks ? g.sinks[qh] * kLog2e : -INFINITY;
  float* out = g.o + ((int64_t)t * hq + qh) * kHd + 2 * od;
  if (n_split == 1) {
    const float mx = fmaxf(blk_m, sink);
    const float f = exp2f(blk_m - mx);
    const float den = blk_l * f + exp2f(sink - mx);
    out[0] = o0 * f / den;
    out[1] = o1 * f / den;
    return;
  }

  // split partial, then the last block of this (token, kv head) merges
  const int64_t grp = (int64_t)t * g.hkv + kvh;
  float* pp = g.part + ((grp * n_split + split) * kGqa + oh) * kPartStride;
  if (od == 0) {
    pp[0] = blk_m;
    pp[1] = blk_l;
  }
  pp[2 + 2 * od] = o0;
  pp[3 + 2 * od] = o1;
  __threadfence();
  __syncthreads();
  if (tid == 0) last_flag = atomicAdd(&g.counters[grp], 1) == n_split - 1;
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float* pb = g.part + (grp * n_split * kGqa + oh) * kPartStride;
  constexpr int64_t kSplitStride = (int64_t)kGqa * kPartStride;
  float mx = sink;
  for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, pb[s * kSplitStride]);
  float den = exp2f(sink - mx), n0 = 0.f, n1 = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float* ps_ = pb + s * kSplitStride;
    const float f = exp2f(ps_[0] - mx);
    den += f * ps_[1];
    n0 += f * ps_[2 + 2 * od];
    n1 += f * ps_[3 + 2 * od];
  }
  out[0] = n0 / den;
  out[1] = n1 / den;
  if (tid == 0) g.counters[grp] = 0;
}

// ---------------------------------------------------------------- host side

inline int64_t attn_splits(int64_t max_keys) { return (max_keys + kKeys - 1) / kKeys; }

inline int64_t round256(int64_t b) { return (b + 255) & ~(int64_t)255; }

// Workspace: counters [kAttnMaxM][hkv] int32 at a fixed place (so one
// workspace serves calls of any m and key count up to its size, every call
// leaving the counters it used at zero), then the split partials.
constexpr int kAttnMaxM = 64;

inline int64_t attn_counter_bytes(int hkv) { return round256((int64_t)kAttnMaxM * hkv * 4); }

inline int64_t attn_ws_bytes(int hkv, int m, int64_t max_keys) {
  const int64_t n_split = attn_splits(max_keys);
  if (n_split <= 1) return 0;
  return attn_counter_bytes(hkv) + (int64_t)m * hkv * n_split * kGqa * kPartStride * 4;
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

extern "C" int64_t attn_decode_workspace(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t m,
                                         int64_t max_keys) {
  if (n_kv_heads < 1 || n_kv_heads > 65535 || n_heads != n_kv_heads * kGqa || head_dim != kHd || m < 1 ||
      m > kAttnMaxM || max_keys < 1)
    return -1;
  return attn_ws_bytes(n_kv_heads, m, max_keys);
}

extern "C" int attn_decode(const float* q, const float* k, const float* v, void* k_cache, void* v_cache,
                           int32_t cache_dtype, int64_t cache_cap, int32_t n_heads, int32_t n_kv_heads,
                           int32_t head_dim, int32_t m, int64_t pos0, const float* rope_table, int64_t table_rows,
                           float sm_scale, const float* sinks, int32_t window, float* o, void* workspace,
                           int64_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !k_cache || !v_cache || !rope_table || !o) return BDG_E_INVALID;
  if (cache_dtype != BDG_F32 && cache_dtype != BDG_BF16) return BDG_E_INVALID;
  if (m < 1 || n_kv_heads < 1 || n_heads < 1 || pos0 < 0 || window < 0 || !(sm_scale > 0.f)) return BDG_E_INVALID;
  if (pos0 + m > cache_cap || pos0 + m > table_rows) return BDG_E_INVALID;
  if (n_heads != n_kv_heads * kGqa || head_dim != kHd) return BDG_E_UNSUPPORTED;
  if (m > kAttnMaxM || n_kv_heads > 65535) return BDG_E_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(rope_table) || !aligned16(o))
    return BDG_E_ALIGN;
  const int64_t last = pos0 + m;                                   // keys of the last token
  const int64_t max_keys = window > 0 && window < last ? window : last;
  const int64_t n_split = attn_splits(max_keys);
  if (n_split > 65535) return BDG_E_UNSUPPORTED;
  AttnArgs g{};
  g.q = q; g.k = k; g.v = v; g.kc = k_cache; g.vc = v_cache; g.tab = rope_table; g.sinks = sinks; g.o = o;
  g.cap = cache_cap; g.pos0 = pos0; g.hkv = n_kv_heads; g.window = window;
  g.qscale = sm_scale * kLog2e;
  if (n_split > 1) {
    const int64_t need = attn_ws_bytes(n_kv_heads, m, max_keys);
    if (!workspace || workspace_bytes < need) return BDG_E_INVALID;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return BDG_E_ALIGN;
    g.counters = reinterpret_cast<int32_t*>(workspace);
    g.part = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + attn_counter_bytes(n_kv_heads));
  }
  const dim3 grid((unsigned)n_split, (unsigned)n_kv_heads, (unsigned)m);
  if (cache_dtype == BDG_BF16)
    hipLaunchKernelGGL(attn_decode_kernel<uint16_t>, grid, dim3(kAttnThreads), 0, as_stream(stream), g);
  else
    hipLaunchKernelGGL(attn_decode_kernel<float>, grid, dim3(kAttnThreads), 0, as_stream(stream), g);
  return launch_status();
}
