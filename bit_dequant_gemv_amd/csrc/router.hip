// Standalone router: router GEMV + top-k + softmax for callers that need
// only the routing (moe_router_topk), e.g. a prefill over many tokens.
#include "bdg_device.hpp"
#include "bdg_host.hpp"
#include "bdg_topk.hpp"

namespace bdg {

constexpr int kRouterThreads = 256;
constexpr int kRouterWaves = kRouterThreads / kWave;

// One block per T tokens (the launch uses T = 1): (optional RMSNorm of)
// their x into LDS, all E router rows one wave at a time - each row chunk
// loaded once and applied to the T tokens, every token's sum in the same
// order for any T - then top-k + softmax, one wave per token.  The decode
// plan uses the split route / gate_up kernels instead; this entry point
// serves callers that need only the routing (e.g. a prefill).
template <int T, int V>
__global__ void __launch_bounds__(kRouterThreads)
router_topk_kernel(const void* __restrict__ x, int x_bf16, const float* __restrict__ w_r,
                   const float* __restrict__ b_r, int M, int H, int E, int K, int norm, float eps,
                   int32_t* __restrict__ idx, float* __restrict__ wts, float* __restrict__ logits) {
  extern __shared__ float lds[];
  float* xs = lds;             // [T][H]
  float* lg = lds + T * H;     // [T][E]
  float* red = lg + T * E;     // [T][kRouterWaves]
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float r[T];
  // stage the T inputs: 4 consecutive elements per thread per load, all of a
  // 4096-wide chunk's loads for the T tokens issued before the LDS stores
  constexpr int kXF4 = 4;         // float4 groups per thread per token per chunk
  float ss[T];
#pragma unroll
  for (int i = 0; i < T; ++i) ss[i] = 0.f;
  for (int h0 = 0; h0 < H; h0 += kRouterThreads * 4 * kXF4) {
    float4 v[T][kXF4];
#pragma unroll
    for (int i = 0; i < T; ++i) {
      int t = blockIdx.x * T + i;
      t = t < M ? t : M - 1;                     // a tail block repeats the last token (not stored)
#pragma unroll
      for (int c = 0; c < kXF4; ++c) {
        int h = h0 + (c * kRouterThreads + threadIdx.x) * 4;
        h = h < H ? h : H - 4;                   // in bounds; unused past H
        if (x_bf16) {
          const uint2 b = ldg_u64(reinterpret_cast<const uint16_t*>(x) + (int64_t)t * H + h);
          v[i][c] = make_float4(bf16_to_f32((uint16_t)(b.x & 0xFFFFu)), bf16_to_f32((uint16_t)(b.x >> 16)),
                                bf16_to_f32((uint16_t)(b.y & 0xFFFFu)), bf16_to_f32((uint16_t)(b.y >> 16)));
        } else {
          v[i][c] = ldg_f4(reinterpret_cast<const float*>(x) + (int64_t)t * H + h);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {
#pragma unroll
      for (int c = 0; c < kXF4; ++c) {
        const int h = h0 + (c * kRouterThreads + threadIdx.x) * 4;
        if (h < H) {
          *reinterpret_cast<float4*>(xs + i * H + h) = v[i][c];
          ss[i] = __builtin_fmaf(v[i][c].x, v[i][c].x, ss[i]);
          ss[i] = __builtin_fmaf(v[i][c].y, v[i][c].y, ss[i]);
          ss[i] = __builtin_fmaf(v[i][c].z, v[i][c].z, ss[i]);
          ss[i] = __builtin_fmaf(v[i][c].w, v[i][c].w, ss[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const float w = wave_sum(ss[i]);
    if (lane == 0) red[i * kRouterWaves + wave] = w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const float* rd = red + i * kRouterWaves;
    r[i] = norm ? 1.0f / sqrtf(((rd[0] + rd[1]) + (rd[2] + rd[3])) / (float)H + eps) : 1.f;
  }
  constexpr int kRowF4 = 16;      // float4 of a router row per lane loaded at once
  for (int e = wave; e < E; e += kRouterWaves) {
    const float* wr = w_r + (int64_t)e * H;
    float acc[T];
#pragma unroll
    for (int i = 0; i < T; ++i) acc[i] = 0.f;
    // lane l adds h = 4l, 4l + 256, ... in ascending order; the row's loads
    // of a 4096-wide chunk are issued together (clamped in bounds), so a row
    // costs one round trip per chunk rather than one per 256 elements
    for (int h0 = 0; h0 < H; h0 += kWave * 4 * kRowF4) {
      float4 wv[kRowF4];
#pragma unroll
      for (int c = 0; c < kRowF4; ++c) {
        const int h = h0 + (c * kWave + lane) * 4;
        wv[c] = *reinterpret_cast<const float4*>(wr + (h < H ? h : H - 4));
      }
#pragma unroll
      for (int c = 0; c < kRowF4; ++c) {
        const int h = h0 + (c * kWave + lane) * 4;
        if (h < H) {
#pragma unroll
          for (int i = 0; i < T; ++i) {
            const float* xi = xs + i * H;
            acc[i] = __builtin_fmaf(wv[c].x, xi[h] * r[i], acc[i]);
            acc[i] = __builtin_fmaf(wv[c].y, xi[h + 1] * r[i], acc[i]);
            acc[i] = __builtin_fmaf(wv[c].z, xi[h + 2] * r[i], acc[i]);
            acc[i] = __builtin_fmaf(wv[c].w, xi[h + 3] * r[i], acc[i]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const float a = wave_sum(acc[i]);
      if (lane == 0) lg[i * E + e] = a + (b_r ? b_r[e] : 0.f);
    }
  }
  __syncthreads();
  // top-k + softmax: wave i takes token i (T <= waves); V values per lane
  // cover E <= 64 V
  for (int i = wave; i < T; i += kRouterWaves) {
    const int t = blockIdx.x * T + i;
    if (t < M) {                                 // wave-uniform
      int my_e;
      float my_w;
      wave_topk<V>(lg + i * E, E, K, my_e, my_w);
      if (lane < K) {
        idx[t * K + lane] = my_e;
        wts[t * K + lane] = my_w;
      }
    }
  }
  if (logits) {
    for (int i = 0; i < T; ++i) {
      const int t = blockIdx.x * T + i;
      if (t >= M) break;                         // block-uniform
      for (int e = threadIdx.x; e < E; e += kRouterThreads) logits[(int64_t)t * E + e] = lg[i * E + e];
    }
  }
}

// Many tokens per block, the per-token arithmetic of router_topk_kernel
// unchanged (so results equal it bit for bit, and equal for any tile):
// 512 threads, TT tokens; wave w sums experts w + 8 j (j < EW) for all TT
// tokens at once, lane l over h = 4 l + 256 c in ascending c, so each router
// row is read once per block instead of once per token.  The RMSNorm scale
// comes from the first 256 threads with router_topk_kernel's partition and
// order; the top-k is the same wave_topk, a wave per token.  BF: bf16 x
// (a template parameter: a branch on it around each load would make every
// load wait for the previous one).
constexpr int kTileThreads = 512;
constexpr int kTileWaves = kTileThreads / kWave;

template <int TT, int EW, int V, int BF>
__global__ void __launch_bounds__(kTileThreads)
router_tile_kernel(const void* __restrict__ x, const float* __restrict__ w_r,
                   const float* __restrict__ b_r, int M, int H, int E, int K, int norm, float eps,
                   int32_t* __restrict__ idx, float* __restrict__ wts, float* __restrict__ logits) {
  __shared__ float lg[TT * kTileWaves * EW];        // [TT][E] (E <= 8 EW)
  __shared__ float red[TT * kRouterWaves];
  __shared__ float rs[TT];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * TT;
  auto x4 = [&](int t, int h) -> float4 {           // token t (clamped), elements h .. h + 3 (clamped)
    t = t < M ? t : M - 1;
    h = h < H ? h : H - 4;
    if constexpr (BF != 0) {
      const uint2 b = ldg_u64(reinterpret_cast<const uint16_t*>(x) + (int64_t)t * H + h);
      return make_float4(bf16_to_f32((uint16_t)(b.x & 0xFFFFu)), bf16_to_f32((uint16_t)(b.x >> 16)),
                         bf16_to_f32((uint16_t)(b.y & 0xFFFFu)), bf16_to_f32((uint16_t)(b.y >> 16)));
    } else {
      return ldg_f4(reinterpret_cast<const float*>(x) + (int64_t)t * H + h);
    }
  };
  if (norm) {
    // sum of squares as router_topk_kernel's 256 threads take it
    // (loads of 4 tokens issued together, clamped in bounds, then the FMAs
    // in that kernel's order)
    if (threadIdx.x < kRouterThreads) {               // waves 0-3: wave-uniform
      constexpr int kXF4 = 4;
      constexpr int kG = TT < 4 ? TT : 4;
      for (int i0 = 0; i0 < TT; i0 += kG) {
        float ss[kG];
#pragma unroll
        for (int g = 0; g < kG; ++g) ss[g] = 0.f;
        for (int h0 = 0; h0 < H; h0 += kRouterThreads * 4 * kXF4) {
          float4 v[kG][kXF4];
#pragma unroll
          for (int g = 0; g < kG; ++g)
#pragma unroll
            for (int c = 0; c < kXF4; ++c) v[g][c] = x4(t0 + i0 + g, h0 + (c * kRouterThreads + threadIdx.x) * 4);
#pragma unroll
          for (int g = 0; g < kG; ++g) {
#pragma unroll
            for (int c = 0; c < kXF4; ++c) {
              if (h0 + (c * kRouterThreads + threadIdx.x) * 4 < H) {
                ss[g] = __builtin_fmaf(v[g][c].x, v[g][c].x, ss[g]);
                ss[g] = __builtin_fmaf(v[g][c].y, v[g][c].y, ss[g]);
                ss[g] = __builtin_fmaf(v[g][c].z, v[g][c].z, ss[g]);
                ss[g] = __builtin_fmaf(v[g][c].w, v[g][c].w, ss[g]);
              }
            }
          }
        }
#pragma unroll
        for (int g = 0; g < kG; ++g) {
          const float w = wave_sum(ss[g]);
          if (lane == 0) red[(i0 + g) * kRouterWaves + wave] = w;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < TT) {
      const float* rd = red + threadIdx.x * kRouterWaves;
      rs[threadIdx.x] = 1.0f / sqrtf(((rd[0] + rd[1]) + (rd[2] + rd[3])) / (float)H + eps);
    }
  } else if (threadIdx.x < TT) {
    rs[threadIdx.x] = 1.f;
  }
  __syncthreads();
  float r[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) r[i] = rs[i];
  float acc[TT][EW];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < EW; ++j) acc[i][j] = 0.f;
  for (int h0 = 0; h0 < H; h0 += 4 * kWave) {
    const int h = h0 + 4 * lane;
    float4 wv[EW];
#pragma unroll
    for (int j = 0; j < EW; ++j) {
      int e = wave + kTileWaves * j;
      e = e < E ? e : E - 1;                         // in bounds; unused past E
      wv[j] = *reinterpret_cast<const float4*>(w_r + (int64_t)e * H + (h < H ? h : H - 4));
    }
    float4 xv[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) xv[i] = x4(t0 + i, h);
    if (h < H) {
#pragma unroll
      for (int i = 0; i < TT; ++i) {
#pragma unroll
        for (int j = 0; j < EW; ++j) {
          acc[i][j] = __builtin_fmaf(wv[j].x, xv[i].x * r[i], acc[i][j]);
          acc[i][j] = __builtin_fmaf(wv[j].y, xv[i].y * r[i], acc[i][j]);
          acc[i][j] = __builtin_fmaf(wv[j].z, xv[i].z * r[i], acc[i][j]);
          acc[i][j] = __builtin_fmaf(wv[j].w, xv[i].w * r[i], acc[i][j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < EW; ++j) {
    const int e = wave + kTileWaves * j;
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const float a = wave_sum(acc[i][j]);
      if (lane == 0 && e < E) lg[i * E + e] = a + (b_r ? b_r[e] : 0.f);
    }
  }
  __syncthreads();
  for (int i = wave; i < TT; i += kTileWaves) {
    const int t = t0 + i;
    if (t < M) {                                     // wave-uniform
      int my_e;
      float my_w;
      wave_topk<V>(lg + i * E, E, K, my_e, my_w);
      if (lane < K) {
        idx[t * K + lane] = my_e;
        wts[t * K + lane] = my_w;
      }
    }
  }
  if (logits) {
    for (int q = threadIdx.x; q < TT * E; q += kTileThreads) {
      const int t = t0 + q / E;
      if (t < M) logits[(int64_t)t * E + q % E] = lg[q];
    }
  }
}

}  // namespace bdg

using namespace bdg;

extern "C" int moe_router_topk(const void* x, int32_t x_dtype, const float* w_r, const float* b_r,
                               int32_t m, int32_t h, int32_t e, int32_t topk, int32_t flags,
                               float norm_eps, int32_t* idx, float* wts, float* logits, void* stream) {
  if (!x || !w_r || !idx || !wts || m < 1 || h < 1 || e < 1 || topk < 1 || topk > e) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if ((flags & ~BDG_ROUTER_RMSNORM) != 0 || (h % 4) != 0) return BDG_E_INVALID;
  if ((flags & BDG_ROUTER_RMSNORM) && !(norm_eps >= 0.f)) return BDG_E_INVALID;
  if ((reinterpret_cast<uintptr_t>(w_r) & 15u) != 0 || !aligned16(x)) return BDG_E_ALIGN;
  if (e > BDG_MAX_EXPERTS || topk > BDG_MAX_TOPK || h > 16384) return BDG_E_UNSUPPORTED;
  const int bf = x_dtype == BDG_BF16 ? 1 : 0, nrm = (flags & BDG_ROUTER_RMSNORM) ? 1 : 0;
  // up to 32 experts: the tiled kernel, each router row read once per block
  // of TT tokens (TT = 16 once that still fills 256 blocks, else fewer)
  if (e <= 32) {
    const int TT = m >= 16 * 256 ? 16 : m >= 4 * 256 ? 4 : 1;
#define BDG_RT_TILE(TTT, BFF)                                                                        \
  if (TT == TTT && bf == BFF) {                                                                      \
    hipLaunchKernelGGL((router_tile_kernel<TTT, 4, 1, BFF>), dim3((unsigned)((m + TTT - 1) / TTT)),   \
                       dim3(kTileThreads), 0, as_stream(stream), x, w_r, b_r, m, h, e, topk, nrm, norm_eps, \
                       idx, wts, logits);                                                            \
    return launch_status();                                                                          \
  }
    BDG_RT_TILE(16, 0) BDG_RT_TILE(4, 0) BDG_RT_TILE(1, 0) BDG_RT_TILE(16, 1) BDG_RT_TILE(4, 1) BDG_RT_TILE(1, 1)
#undef BDG_RT_TILE
  }
  // more experts: one token per block
  const int T = 1;
  const size_t lds = (size_t)T * (h + e + kRouterWaves) * sizeof(float);
  const dim3 grid((unsigned)((m + T - 1) / T));
  const int V = e <= 64 ? 1 : e <= 128 ? 2 : e <= 256 ? 4 : BDG_MAX_EXPERTS / kWave;
#define BDG_RT_CASE(TT, VV)                                                                                  \
  if (T == TT && V == VV) {                                                                                  \
    hipLaunchKernelGGL((router_topk_kernel<TT, VV>), grid, dim3(kRouterThreads), lds, as_stream(stream), x, bf, \
                       w_r, b_r, m, h, e, topk, nrm, norm_eps, idx, wts, logits);                            \
    return launch_status();                                                                                  \
  }
  BDG_RT_CASE(1, 1) BDG_RT_CASE(1, 2) BDG_RT_CASE(1, 4) BDG_RT_CASE(1, 16)
#undef BDG_RT_CASE
  return BDG_E_UNSUPPORTED;
}
