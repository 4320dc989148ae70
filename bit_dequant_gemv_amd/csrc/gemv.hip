// qgemv: fused dequant-GEMV y = W x over a packed MXFP4 / int4 matrix (the
// MXFP4 dequant-GEMV of "Sovereign gpt-oss-20B (MXFP4) on Apple Silicon",
// sections 1 and 4: 16-byte coalesced code loads, on-chip dequantisation).
#include "bdg_gemv.hpp"
#include "bdg_host.hpp"

namespace bdg {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

// grid = (blocks per token, m).  Block b owns row groups [g0, g1); its waves
// take them round-robin, two groups in flight per wave.
template <int FMT, int L, int S>
__global__ void __launch_bounds__(kGemvThreads)
qgemv_kernel(QMat w, QGeom g, int64_t n_rows, const void* __restrict__ x, int x_bf16,
             float* __restrict__ y) {
  extern __shared__ float lds_x[];
  constexpr int RPW = kWave / L;
  const int t = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int li = lane % L;
  const int rr = lane / L;

  if (x_bf16)
    stage_bf16<4>(lds_x, reinterpret_cast<const uint16_t*>(x) + (int64_t)t * g.k, g.k, threadIdx.x, kGemvThreads);
  else
    stage_f32<4>(lds_x, reinterpret_cast<const float*>(x) + (int64_t)t * g.k, g.k, g.k, 0, 1.0f, threadIdx.x,
                 kGemvThreads);
  __syncthreads();
  XRegs<FMT, L, S> xr;
  xr.load(lds_x, g.chunks, li);

  const int64_t n_groups = (n_rows + RPW - 1) / RPW;
  const int64_t g0 = n_groups * blockIdx.x / gridDim.x;
  const int64_t g1 = n_groups * (blockIdx.x + 1) / gridDim.x;
  float* yt = y + (int64_t)t * n_rows;

  GroupLoad<FMT, S> a, b;
  int64_t ga = g0 + wave;
  if (ga < g1) {
    const int64_t row = ga * RPW + rr;
    load_row<FMT, L, S>(a, w, g, row, row < n_rows, li);
  }
  while (ga < g1) {
    const int64_t gb = ga + kGemvWaves;
    if (gb < g1) {
      const int64_t row = gb * RPW + rr;
      load_row<FMT, L, S>(b, w, g, row, row < n_rows, li);
    }
    {
      const int64_t row = ga * RPW + rr;
      const float d = row_dot<FMT, L, S>(a, xr);
      if (li == 0 && row < n_rows) yt[row] = d;
    }
    if (gb >= g1) break;
    const int64_t gc = gb + kGemvWaves;
    if (gc < g1) {
      const int64_t row = gc * RPW + rr;
      load_row<FMT, L, S>(a, w, g, row, row < n_rows, li);
    }
    {
      const int64_t row = gb * RPW + rr;
      const float d = row_dot<FMT, L, S>(b, xr);
      if (li == 0 && row < n_rows) yt[row] = d;
    }
    ga = gc;
  }
}

template <int FMT>
static int launch_qgemv(const QMat& w, const QGeom& g, int64_t n, const void* x, int x_bf16, int m,
                        float* y, hipStream_t s) {
  int L = 0, S = 0;
  if (!pick_lanes(g.chunks, &L, &S)) return BDG_E_UNSUPPORTED;
  const int rpw = kWave / L;
  const int64_t n_groups = (n + rpw - 1) / rpw;
  // about two row groups per wave, at least one block per 64 row groups
  int64_t blocks = (n_groups + 2 * kGemvWaves - 1) / (2 * kGemvWaves);
  if (blocks < 1) blocks = 1;
  if (blocks > 65535) blocks = 65535;
  const size_t lds = (size_t)g.chunks * kXStride * sizeof(float);
  dim3 grid((unsigned)blocks, (unsigned)m);
#define BDG_GEMV_CASE(LL, SS)                                                                      \
  if (L == LL && S == SS) {                                                                        \
    hipLaunchKernelGGL((qgemv_kernel<FMT, LL, SS>), grid, dim3(kGemvThreads), lds, s, w, g, n, x, \
                       x_bf16, y);                                                                 \
    return launch_status();                                                                        \
  }
  BDG_GEMV_CASE(8, 1) BDG_GEMV_CASE(8, 2) BDG_GEMV_CASE(8, 3)
  BDG_GEMV_CASE(16, 2) BDG_GEMV_CASE(16, 3)
  BDG_GEMV_CASE(32, 2) BDG_GEMV_CASE(32, 3)
  BDG_GEMV_CASE(64, 2) BDG_GEMV_CASE(64, 3) BDG_GEMV_CASE(64, 4)
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
