// Large-M product of MXFP4 weights with MXFP8 activations on gfx950's
// MX-scaled matrix cores.
//
// At M = 1 the expert path is a bandwidth-bound GEMV; grouping the active
// experts into a GEMM is the lever the gpt-oss page names and leaves untried
// ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon", section 5), and the q4
// page puts fp8 / grouped-expert GEMM beyond its single-stream floor
// ("Amortizing the per-token host-sync setup tax ...", section 5).  With many
// tokens per weight byte (prefill) the product becomes a dense contraction,
// so it runs on V_MFMA_SCALE_F32_32X32X64_F8F6F4: A = 32 weight rows x 64 K
// in FP4 E2M1, B = 64 K x 32 tokens in FP8 E4M3, one E8M0 scale per operand
// row and 32-element K block, fp32 accumulation.  The MXFP4 weights are
// multiplied as stored (PLAIN layout, no repacking); the activations are
// first quantized to MXFP8 (OCP MX v1.0 conversion) by mxfp8_quant_kernel.
//
// Operand lane layout of the instruction, as measured on the device (one
// wavefront, lane l, j = l % 32, h = l / 32):
//   A (FP4, 4 VGPRs): row j, K elements 32h .. 32h+31 in nibble order (low
//     nibble first) - exactly 16 consecutive bytes of a PLAIN code row; the
//     lane's scale byte is the E8M0 of that 32-element block.
//   B (FP8, 8 VGPRs): column j; bytes 0..15 are K 16h .. 16h+15, bytes
//     16..31 are K 32+16h .. 32+16h+15; the lane's scale byte is the E8M0 of
//     K block h (K 0..31 or 32..63) of column j.
//   D (16 fp32): register r holds row 8(r/4) + 4h + (r%4), column j.
// The instruction adds its 64 products at reduced internal precision
// (measured: up to ~1e-4 of the sum of |products| per instruction), so the
// product is compared with the oracle under a tolerance relative to
// sum |W| |xq|, not bit for bit.
#include "bdg_device.hpp"
#include "bdg_host.hpp"

namespace bdg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kQuantThreads = 256;

// fp32 -> FP8 E4M3 code: round to nearest, ties to even, saturating at 448.
// Sign kept (so -0.0 and negative values that round to 0 give 0x80).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t c;
  if (a >= 0x43E00000u) {                   // |v| >= 448
    c = 0x7Eu;
  } else if (a >= 0x3C800000u) {            // 2^-6 <= |v| < 448: normal
    // keep 3 mantissa bits: round the 20 dropped bits half to even, then
    // rebias the exponent from 127 to 7 (a carry moves to the next binade)
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    c = r - (120u << 3);
    if (c > 0x7Eu) c = 0x7Eu;
  } else {                                  // subnormal: multiples of 2^-9
    c = (uint32_t)rintf(__uint_as_float(a) * 512.0f);   // exact scaling; 8 = smallest normal
  }
  return s | c;
}

// One 32-element block per 8 threads, 4 elements per thread.
__global__ void __launch_bounds__(kQuantThreads)
mxfp8_quant_kernel(const void* __restrict__ x, int x_bf16, int64_t n_elems, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ scales) {
  const int64_t e0 = ((int64_t)blockIdx.x * kQuantThreads + threadIdx.x) * 4;
  const bool ok = e0 < n_elems;
  const int64_t ec = ok ? e0 : n_elems - 4;   // in bounds; results unused
  float v[4];
  if (x_bf16) {
    const uint2 b = ldg_u64(reinterpret_cast<const uint16_t*>(x) + ec);
    v[0] = bf16_to_f32((uint16_t)(b.x & 0xFFFFu));
    v[1] = bf16_to_f32((uint16_t)(b.x >> 16));
    v[2] = bf16_to_f32((uint16_t)(b.y & 0xFFFFu));
    v[3] = bf16_to_f32((uint16_t)(b.y >> 16));
  } else {
    const float4 f = ldg_f4(reinterpret_cast<const float*>(x) + ec);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
  // block maximum of |v| as bits (non-negative floats order as integers);
  // any NaN or infinity makes the block non-finite
  uint32_t amax = 0, bad = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;
    bad |= a >= 0x7F800000u ? 1u : 0u;
    amax = max(amax, a);
  }
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, d));
    bad |= (uint32_t)__shfl_xor((int)bad, d);
  }
  // X = floor(log2 amax) - 8, clamped to >= -127 (amax = 0 or subnormal)
  const int eb = (int)(amax >> 23);            // biased exponent of amax
  int X = amax == 0 ? -127 : eb - 127 - 8;
  X = X < -127 ? -127 : X;
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X, X in [-127, 119]
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) word |= (bad ? 0x7Fu : f32_to_e4m3(v[i] * inv)) << (8 * i);
  if (ok) {
    *reinterpret_cast<uint32_t*>(codes + e0) = word;
    if ((threadIdx.x & 7) == 0) scales[e0 >> 5] = (uint8_t)(bad ? 255 : X + 127);
  }
}

constexpr int kGemmWaves = 4;
constexpr int kTileN = 64;       // weight rows per wave (two 32-row MFMA tiles)
constexpr int kTileM = 64;       // tokens per wave (two 32-column MFMA tiles)

// Operands of one 64-deep K step for one wave: two A tiles, two B tiles.
struct MxStep {
  v8i a[2];
  v8i b[2];
  int sa[2], sb[2];
};

// Loads of K step k0 (all addresses clamped in bounds, no branches).  kb_ok:
// the second 32-block of the step exists (false only for the last step of a
// K that is an odd number of 32-blocks; the missing half is then zeroed).
__device__ __forceinline__ void mx_load(MxStep& st, const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                                        const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                        int64_t n0, int64_t m0, int64_t N, int64_t M, int K, int k0, int lane) {
  const int j = lane & 31, h = lane >> 5;
  const int kblocks = K >> 5;
  const int kb = (k0 >> 5) + h;
  const bool second = (k0 >> 5) + 1 < kblocks;       // step holds two 32-blocks
  const int kbc = kb < kblocks ? kb : kblocks - 1;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int64_t row = n0 + 32 * t + j;
    row = row < N ? row : N - 1;
    const uint4 q = ldg_u128(wc + row * (K >> 1) + (int64_t)kbc * 16);
    const bool zero = h == 1 && !second;
    st.a[t][0] = zero ? 0 : (int)q.x;
    st.a[t][1] = zero ? 0 : (int)q.y;
    st.a[t][2] = zero ? 0 : (int)q.z;
    st.a[t][3] = zero ? 0 : (int)q.w;
    st.a[t][4] = st.a[t][5] = st.a[t][6] = st.a[t][7] = 0;
    st.sa[t] = (int)ldg_u8(ws + row * kblocks + kbc);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int64_t tok = m0 + 32 * t + j;
    tok = tok < M ? tok : M - 1;
    const uint8_t* base = xc + tok * K + k0;
    const uint4 lo = ldg_u128(base + 16 * h);
    const uint4 hi = ldg_u128(base + (second ? 32 : 0) + 16 * h);
    st.b[t][0] = (int)lo.x;
    st.b[t][1] = (int)lo.y;
    st.b[t][2] = (int)lo.z;
    st.b[t][3] = (int)lo.w;
    st.b[t][4] = second ? (int)hi.x : 0;
    st.b[t][5] = second ? (int)hi.y : 0;
    st.b[t][6] = second ? (int)hi.z : 0;
    st.b[t][7] = second ? (int)hi.w : 0;
    st.sb[t] = (int)ldg_u8(xs + tok * kblocks + kbc);
  }
}

// y[m][n] = sum_k W[n][k] * xq[m][k].  Block = 4 waves over a 128 x 128
// (rows x tokens) tile, wave w takes the 64 x 64 quarter (w & 1, w >> 1).
// The next K step's operands are loaded before the current step's four
// MFMAs issue.
__global__ void __launch_bounds__(kGemmWaves * 64)
mx_gemm_kernel(const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws, const uint8_t* __restrict__ xc,
               const uint8_t* __restrict__ xs, int64_t N, int64_t M, int K, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t n0 = (int64_t)blockIdx.x * (2 * kTileN) + (wave & 1) * kTileN;
  const int64_t m0 = (int64_t)blockIdx.y * (2 * kTileM) + (wave >> 1) * kTileM;
  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  MxStep cur, nxt;
  mx_load(cur, wc, ws, xc, xs, n0, m0, N, M, K, 0, lane);
  for (int k0 = 0; k0 < K; k0 += 64) {
    const int kn = k0 + 64 < K ? k0 + 64 : k0;   // the last step reloads itself (in bounds, unused)
    mx_load(nxt, wc, ws, xc, xs, n0, m0, N, M, K, kn, lane);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.a[a], cur.b[b], acc[a][b], 4, 0, 0,
                                                                     cur.sa[a], 0, cur.sb[b]);
    cur = nxt;
  }

  const int j = lane & 31, h = lane >> 5;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t tok = m0 + 32 * b + j;
    if (tok >= M) continue;
    float* yrow = y + tok * N;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t row = n0 + 32 * a + 8 * g + 4 * h;
        const float4 v = make_float4(acc[a][b][4 * g + 0], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                                     acc[a][b][4 * g + 3]);
        if (row + 3 < N && (N & 3) == 0) {
          *reinterpret_cast<float4*>(yrow + row) = v;
        } else {
          if (row + 0 < N) yrow[row + 0] = v.x;
          if (row + 1 < N) yrow[row + 1] = v.y;
          if (row + 2 < N) yrow[row + 2] = v.z;
          if (row + 3 < N) yrow[row + 3] = v.w;
        }
      }
    }
  }
}

}  // namespace bdg

using namespace bdg;

extern "C" int mxfp8_quantize(const void* x, int32_t x_dtype, int64_t m, int64_t k, uint8_t* codes,
                              uint8_t* scales, void* stream) {
  if (!x || !codes || !scales || m < 1 || k < 32 || (k % 32) != 0) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(codes) & 3u) != 0) return BDG_E_ALIGN;
  const int64_t n = m * k;
  const int64_t blocks = (n / 4 + kQuantThreads - 1) / kQuantThreads;
  if (blocks > 2147483647LL) return BDG_E_UNSUPPORTED;
  hipLaunchKernelGGL(mxfp8_quant_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, as_stream(stream), x,
                     x_dtype == BDG_BF16 ? 1 : 0, n, codes, scales);
  return launch_status();
}

extern "C" int mx_gemm(const bdg_qmat* w, const uint8_t* x_codes, const uint8_t* x_scales, int64_t m, float* y,
                       void* stream) {
  int st = check_qmat(w, false);
  if (st != BDG_OK) return st;
  if (w->fmt != BDG_FMT_MXFP4) return BDG_E_INVALID;
  if (!x_codes || !x_scales || !y || m < 1) return BDG_E_INVALID;
  if (!aligned16(x_codes)) return BDG_E_ALIGN;
  if (w->k > (int64_t)1 << 20 || w->n * (w->k / 2) >= ((int64_t)1 << 40)) return BDG_E_UNSUPPORTED;
  const int64_t gx = (w->n + 2 * kTileN - 1) / (2 * kTileN);
  const int64_t gy = (m + 2 * kTileM - 1) / (2 * kTileM);
  if (gx > 2147483647LL || gy > 65535) return BDG_E_UNSUPPORTED;
  hipLaunchKernelGGL(mx_gemm_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kGemmWaves * 64), 0,
                     as_stream(stream), static_cast<const uint8_t*>(w->codes),
                     static_cast<const uint8_t*>(w->scales), x_codes, x_scales, w->n, m, (int)w->k, y);
  return launch_status();
}
