// Standalone router: router GEMV + top-k + softmax for callers that need
// only the routing (moe_router_topk), e.g. a prefill over many tokens.
#include "bdg_device.hpp"
#include "bdg_host.hpp"
#include "bdg_topk.hpp"

namespace bdg {

constexpr int kRouterThreads = 256;
constexpr int kRouterWaves = kRouterThreads / kWave;

// One block per T tokens: (optional RMSNorm of) their x into LDS, all E
// router rows one wave at a time - each row chunk loaded once and applied to
// the T tokens, every token's sum in the same order as with T = 1 - then
// top-k + softmax by wave 0.  The decode plan uses the split route / gate_up
// kernels instead; this entry point serves callers that need only the
// routing (T > 1 for many tokens at once, e.g. a prefill).
template <int T>
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
#pragma unroll
  for (int i = 0; i < T; ++i) {
    int t = blockIdx.x * T + i;
    t = t < M ? t : M - 1;                       // a tail block repeats the last token (not stored)
    float ss = 0.f;
    for (int h = threadIdx.x; h < H; h += kRouterThreads) {
      const float v = x_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[(int64_t)t * H + h])
                             : reinterpret_cast<const float*>(x)[(int64_t)t * H + h];
      xs[i * H + h] = v;
      ss = __builtin_fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[i * kRouterWaves + wave] = ss;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < T; ++i) {
    const float* rd = red + i * kRouterWaves;
    r[i] = norm ? 1.0f / sqrtf(((rd[0] + rd[1]) + (rd[2] + rd[3])) / (float)H + eps) : 1.f;
  }
  for (int e = wave; e < E; e += kRouterWaves) {
    const float* wr = w_r + (int64_t)e * H;
    float acc[T];
#pragma unroll
    for (int i = 0; i < T; ++i) acc[i] = 0.f;
    for (int h = lane * 4; h < H; h += kWave * 4) {
      const float4 wv = *reinterpret_cast<const float4*>(wr + h);
#pragma unroll
      for (int i = 0; i < T; ++i) {
        const float* xi = xs + i * H;
        acc[i] = __builtin_fmaf(wv.x, xi[h] * r[i], acc[i]);
        acc[i] = __builtin_fmaf(wv.y, xi[h + 1] * r[i], acc[i]);
        acc[i] = __builtin_fmaf(wv.z, xi[h + 2] * r[i], acc[i]);
        acc[i] = __builtin_fmaf(wv.w, xi[h + 3] * r[i], acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < T; ++i) {
      const float a = wave_sum(acc[i]);
      if (lane == 0) lg[i * E + e] = a + (b_r ? b_r[e] : 0.f);
    }
  }
  __syncthreads();
  for (int i = 0; i < T; ++i) {
    const int t = blockIdx.x * T + i;
    if (t >= M) break;                           // block-uniform
    if (wave == 0) {
      int my_e;
      float my_w;
      wave_topk<BDG_MAX_EXPERTS / kWave>(lg + i * E, E, K, my_e, my_w);
      if (lane < K) {
        idx[t * K + lane] = my_e;
        wts[t * K + lane] = my_w;
      }
    }
    if (logits)
      for (int e = threadIdx.x; e < E; e += kRouterThreads) logits[(int64_t)t * E + e] = lg[i * E + e];
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
  if ((reinterpret_cast<uintptr_t>(w_r) & 15u) != 0) return BDG_E_ALIGN;
  if (e > BDG_MAX_EXPERTS || topk > BDG_MAX_TOPK || h > 16384) return BDG_E_UNSUPPORTED;
  // four tokens per block when there are many and their inputs fit 64 KB of LDS
  const int T = (m >= 64 && (size_t)4 * (h + e + kRouterWaves) * sizeof(float) <= 65536) ? 4 : 1;
  const size_t lds = (size_t)T * (h + e + kRouterWaves) * sizeof(float);
  const dim3 grid((unsigned)((m + T - 1) / T));
  const int bf = x_dtype == BDG_BF16 ? 1 : 0, nrm = (flags & BDG_ROUTER_RMSNORM) ? 1 : 0;
  if (T == 4)
    hipLaunchKernelGGL(router_topk_kernel<4>, grid, dim3(kRouterThreads), lds, as_stream(stream), x, bf, w_r, b_r, m, h,
                       e, topk, nrm, norm_eps, idx, wts, logits);
  else
    hipLaunchKernelGGL(router_topk_kernel<1>, grid, dim3(kRouterThreads), lds, as_stream(stream), x, bf, w_r, b_r, m, h,
                       e, topk, nrm, norm_eps, idx, wts, logits);
  return launch_status();
}
