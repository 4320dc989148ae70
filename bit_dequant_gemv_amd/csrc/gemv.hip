// qgemv: fused dequant-GEMV y = W x over a packed MXFP4 / int4 matrix (the
// MXFP4 dequant-GEMV of "Sovereign gpt-oss-20B (MXFP4) on Apple Silicon",
// sections 1 and 4: 16-byte coalesced code loads, on-chip dequantisation).
#include "bdg_gemv.hpp"
#include "bdg_host.hpp"

namespace bdg {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

// grid = (blocks per token, m).  Wave gw of a token owns row groups
// [gw * NP, gw * NP + NP) (a row group = 64 / L rows).  Every load a wave needs
// is issued up front and branch-free: x first (its loads do not depend on
// anything), then all NP row groups; x is stored to LDS only after the
// weights are in flight, so the weight stream starts at once.
template <int FMT, int L, int S, int NP>
__global__ void __launch_bounds__(kGemvThreads)
qgemv_kernel(QMat w, QGeom g, int64_t n_rows, const void* __restrict__ x, int x_bf16,
             float* __restrict__ y) {
  extern __shared__ float lds_x[];
  constexpr int RPW = kWave / L;
  constexpr int NX = (L * S + 31) / 32;                 // float4 of x per thread (k <= 32 * L * S)
  const int t = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int li = lane % L;
  const int rr = lane / L;

  StageF32<NX> xf;
  uint2 xb[NX];
  if (x_bf16) {
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(x) + (int64_t)t * g.k;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int idx = (i * kGemvThreads + threadIdx.x) * 4;
      xb[i] = ldg_u64(xs + (idx < g.k ? idx : g.k - 4));
    }
  } else {
    xf.load(reinterpret_cast<const float*>(x) + (int64_t)t * g.k, g.k, threadIdx.x, kGemvThreads);
  }
  const int64_t gw = (int64_t)blockIdx.x * kGemvWaves + wave;
  GroupLoad<FMT, S> ld[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int64_t row = (gw * NP + i) * RPW + rr;
    load_row<FMT, L, S>(ld[i], w, g, row < n_rows ? row : 0, row < n_rows, li);
  }
  if (x_bf16) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int idx = (i * kGemvThreads + threadIdx.x) * 4;
      if (idx < g.k)
        *reinterpret_cast<float4*>(lds_x + (idx >> 5) * kXStride + (idx & 31)) =
            make_float4(bf16_to_f32((uint16_t)(xb[i].x & 0xFFFFu)), bf16_to_f32((uint16_t)(xb[i].x >> 16)),
                        bf16_to_f32((uint16_t)(xb[i].y & 0xFFFFu)), bf16_to_f32((uint16_t)(xb[i].y >> 16)));
    }
  } else {
    xf.store(lds_x, g.k, g.k, 0, 1.0f, threadIdx.x, kGemvThreads);
  }
  lds_x[g.chunks * kXStride + (threadIdx.x & (kChunkElems - 1))] = 0.f;   // the zero chunk after x (no branch)
  block_sync_lds();   // weights still in flight: each row group waits for its own rows only
  XRegs<FMT, L, S> xr;
  xr.load_zpad(lds_x, g.chunks, li);
  float* yt = y + (int64_t)t * n_rows;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int64_t row = (gw * NP + i) * RPW + rr;
    const float d = row_dot<FMT, L, S>(ld[i], xr);
    if (li == kRowSumLane<L> && row < n_rows) yt[row] = d;
  }
}

template <int FMT>
static int launch_qgemv(const QMat& w, const QGeom& g, int64_t n, const void* x, int x_bf16, int m,
                        float* y, hipStream_t s) {
  int L = 0, S = 0;
  if (!pick_lanes(g.chunks, &L, &S)) return BDG_E_UNSUPPORTED;
  const int rpw = kWave / L;
  const int64_t n_groups = (n + rpw - 1) / rpw;
  // one row group per wave while that keeps the grid within a few waves per
  // CU; long matrices take four per wave (fewer, fuller waves)
  const int np = n_groups <= 8192 ? 1 : 4;
  int64_t blocks = (n_groups + (int64_t)np * kGemvWaves - 1) / ((int64_t)np * kGemvWaves);
  if (blocks < 1) blocks = 1;
  if (blocks > 2147483647LL) return BDG_E_UNSUPPORTED;
  const size_t lds = (size_t)(g.chunks + 1) * kXStride * sizeof(float);   // x chunks and one zero chunk
  dim3 grid((unsigned)blocks, (unsigned)m);
#define BDG_GEMV_CASE(LL, SS, NN)                                                                       \
  if (L == LL && S == SS && np == NN) {                                                                 \
    hipLaunchKernelGGL((qgemv_kernel<FMT, LL, SS, NN>), grid, dim3(kGemvThreads), lds, s, w, g, n, x,   \
                       x_bf16, y);                                                                      \
    return launch_status();                                                                             \
  }
#define BDG_GEMV_NP(LL, SS) BDG_GEMV_CASE(LL, SS, 1) BDG_GEMV_CASE(LL, SS, 4)
  BDG_GEMV_NP(8, 1) BDG_GEMV_NP(8, 2) BDG_GEMV_NP(8, 3)
  BDG_GEMV_NP(16, 2) BDG_GEMV_NP(16, 3)
  BDG_GEMV_NP(32, 2) BDG_GEMV_NP(32, 3)
  BDG_GEMV_NP(64, 2) BDG_GEMV_NP(64, 3) BDG_GEMV_NP(64, 4)
#undef BDG_GEMV_NP
#undef BDG_GEMV_CASE
  return BDG_E_UNSUPPORTED;
}

}  // namespace bdg

using namespace bdg;

extern "C" int qgemv(const bdg_qmat* w, const void* x, int32_t x_dtype, int32_t m, float* y,
                     void* stream) {
  int st = check_qmat(w, false);
  if (st != BDG_OK) return st;
  if (!x || !y || m < 1) return BDG_E_INVALID;
  if (m > BDG_MAX_M) return BDG_E_UNSUPPORTED;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if (!aligned16(x)) return BDG_E_ALIGN;
  QMat qm{static_cast<const uint8_t*>(w->codes), static_cast<const uint8_t*>(w->scales),
          static_cast<const uint8_t*>(w->zeros)};
  QGeom g;
  g.k = (int)w->k;
  g.chunks = (int)(w->k / 32);
  g.group = w->group;
  g.groups = (int)(w->k / w->group);
  g.zrow = (g.groups + 1) / 2;
  const int bf = x_dtype == BDG_BF16 ? 1 : 0;
  hipStream_t s = as_stream(stream);
  if (w->fmt == BDG_FMT_MXFP4) return launch_qgemv<kMXFP4>(qm, g, w->n, x, bf, m, y, s);
  return launch_qgemv<kINT4G>(qm, g, w->n, x, bf, m, y, s);
}
