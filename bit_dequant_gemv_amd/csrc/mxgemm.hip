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

constexpr int kGemmThreads = 256;   // 4 waves
constexpr int kBN = 256;            // weight rows per block (128 per wave)
constexpr int kBM = 128;            // tokens per block (64 per wave)
constexpr int kBK = 128;            // K per stage: two 64-deep MFMA steps, four 32-blocks

// LDS of one block: two stages of the A (weight) and B (activation) tiles,
// each stored piece-major - piece q = 16 bytes of a row - so that a half-wave
// reads 32 consecutive 16-byte slots.  Slots are XOR-swizzled (row ^ 4q for
// A, token ^ 2q for B, both inside aligned groups of 16) so that the 16
// lanes of a store pass - 4 pieces x 4 rows of A, 8 pieces x 2 tokens of B -
// also land in 16 different slots.
struct MxLds {
  uint4 a[2][4][kBN];               // [stage][piece: 32-block of the stage][row]       32 KB
  uint4 b[2][8][kBM];               // [stage][piece: 16 K of the stage][token]          32 KB
  uint8_t sa[2][4][kBN];            // [stage][32-block][row] E8M0
  uint8_t sb[2][4][kBM];            // [stage][32-block][token] E8M0
};

// One stage's global loads for this thread.  All addresses are clamped in
// bounds and nothing reads the loaded registers until the stage is stored to
// LDS (a select on a loaded value would make the wave wait for it at once);
// `valid` marks which pieces lie inside K, the others are stored as zeros.
struct MxStage {
  uint4 a[4], b[4];
  uint32_t sa[4], sb[4];            // scale bytes of the 4 32-blocks (sb: threads < kBM)
  uint32_t valid;                   // bit i: a[i] inside K; bit 4 + i: b[i] inside K
};

__device__ __forceinline__ void mx_stage_load(MxStage& st, const uint8_t* __restrict__ wc,
                                              const uint8_t* __restrict__ ws, const uint8_t* __restrict__ xc,
                                              const uint8_t* __restrict__ xs, int64_t n0, int64_t m0, int64_t N,
                                              int64_t M, int K, int k0, int tid) {
  const int kblocks = K >> 5;
  const int kb0 = k0 >> 5;
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // A: uint4 u = 256 i + tid of the stage: row u / 4, piece q = u % 4 (4 lanes per row)
    const int u = i * kGemmThreads + tid;
    int64_t row = n0 + (u >> 2);
    row = row < N ? row : N - 1;
    const int kb = kb0 + (u & 3);
    const int kbc = kb < kblocks ? kb : kblocks - 1;
    st.a[i] = ldg_u128(wc + row * (K >> 1) + (int64_t)kbc * 16);
    valid |= (kb < kblocks ? 1u : 0u) << i;
    // B: token u / 8, piece p = u % 8 (16 fp8 values, K k0 + 16 p ..)
    int64_t tok = m0 + (u >> 3);
    tok = tok < M ? tok : M - 1;
    const int kp = k0 + 16 * (u & 7);
    const int kpc = kp < K ? kp : K - 16;
    st.b[i] = ldg_u128(xc + tok * K + kpc);
    valid |= (kp < K ? 1u : 0u) << (4 + i);
  }
  st.valid = valid;
  int64_t row = n0 + tid;
  row = row < N ? row : N - 1;
  int64_t tok = m0 + (tid & (kBM - 1));
  tok = tok < M ? tok : M - 1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int kb = kb0 + q;
    const int kbc = kb < kblocks ? kb : kblocks - 1;
    st.sa[q] = ldg_u8(ws + row * kblocks + kbc);
    st.sb[q] = ldg_u8(xs + tok * kblocks + kbc);
  }
}

__device__ __forceinline__ void mx_stage_store(MxLds& l, int buf, const MxStage& st, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = i * kGemmThreads + tid;
    // component-wise selects (a select of whole structs can become a select
    // of their addresses, which moves the stage to scratch memory)
    const bool oka = (st.valid >> i) & 1u, okb = (st.valid >> (4 + i)) & 1u;
    l.a[buf][u & 3][(u >> 2) ^ (4 * (u & 3))] = make_uint4(oka ? st.a[i].x : 0u, oka ? st.a[i].y : 0u, oka ? st.a[i].z : 0u,
                                         oka ? st.a[i].w : 0u);
    l.b[buf][u & 7][(u >> 3) ^ (2 * (u & 7))] = make_uint4(okb ? st.b[i].x : 0u, okb ? st.b[i].y : 0u, okb ? st.b[i].z : 0u,
                                         okb ? st.b[i].w : 0u);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) l.sa[buf][q][tid] = (uint8_t)st.sa[q];
  if (tid < kBM) {
#pragma unroll
    for (int q = 0; q < 4; ++q) l.sb[buf][q][tid] = (uint8_t)st.sb[q];
  }
}

// Tile t of the gx x gy block tiles (gx over weight rows, gy over tokens):
// tiles are dealt to the 8 XCDs in contiguous chunks (block b runs on XCD
// b % 8), and inside a chunk 32 consecutive tiles form a 4 x 8 patch of
// (row tiles x token tiles), so the blocks one XCD runs at a time share
// their weight and activation tiles in that XCD's L2.
__device__ __forceinline__ bool mx_tile_of_block(int b, int gx, int gy, int* x, int* y) {
  const int T = gx * gy;
  const int per = (T + 7) / 8;
  const int t = (b & 7) * per + (b >> 3);
  if (t >= T) return false;
  constexpr int GX = 4;
  const int g = t / (GX * gy);                // group of GX row tiles
  const int gw = min(GX, gx - g * GX);        // its width (the last group may be narrower)
  const int r = t - g * GX * gy;
  *x = g * GX + r % gw;
  *y = r / gw;
  return true;
}

// y[m][n] = sum_k W[n][k] * xq[m][k].  Block = 4 waves over 256 weight rows
// x 128 tokens; wave w takes rows 128 (w & 1) + [0, 128) (four 32-row MFMA
// tiles) and tokens 64 (w >> 1) + [0, 64) (two 32-token tiles): 8 MFMAs per
// 64-deep step, operands read from LDS.  Global loads run two stages ahead
// of the MFMAs (two register sets), the LDS holds two stages.
__global__ void __launch_bounds__(kGemmThreads, 1)
mx_gemm_kernel(const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws, const uint8_t* __restrict__ xc,
               const uint8_t* __restrict__ xs, int64_t N, int64_t M, int K, int gx, int gy,
               float* __restrict__ y) {
  __shared__ MxLds l;
  int tx, ty;
  if (!mx_tile_of_block(blockIdx.x, gx, gy, &tx, &ty)) return;   // block-uniform
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int64_t n0 = (int64_t)tx * kBN;
  const int64_t m0 = (int64_t)ty * kBM;
  const int wr = (wave & 1) * 128;                 // the wave's first row in the block tile
  const int wt = (wave >> 1) * 64;                 // the wave's first token in the block tile
  v16f acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // both 64-deep steps' operands are read from LDS before the first MFMA
  // issues, so the reads of the second step overlap the first step's MFMAs
  auto compute = [&](int buf) {
    v8i A[2][4], B[2][2];
    int sa[2][4], sb[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int pa = 2 * ks + h;                  // A piece (32-block of the stage)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int r = wr + 32 * a + j;
        const uint4 q = l.a[buf][pa][r ^ (4 * pa)];
        A[ks][a][0] = (int)q.x;
        A[ks][a][1] = (int)q.y;
        A[ks][a][2] = (int)q.z;
        A[ks][a][3] = (int)q.w;
        A[ks][a][4] = A[ks][a][5] = A[ks][a][6] = A[ks][a][7] = 0;
        sa[ks][a] = l.sa[buf][pa][r];
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int t = wt + 32 * b + j;
        const int plo = 4 * ks + h, phi = 4 * ks + 2 + h;
        const uint4 lo = l.b[buf][plo][t ^ (2 * plo)];
        const uint4 hi = l.b[buf][phi][t ^ (2 * phi)];
        B[ks][b][0] = (int)lo.x;
        B[ks][b][1] = (int)lo.y;
        B[ks][b][2] = (int)lo.z;
        B[ks][b][3] = (int)lo.w;
        B[ks][b][4] = (int)hi.x;
        B[ks][b][5] = (int)hi.y;
        B[ks][b][6] = (int)hi.z;
        B[ks][b][7] = (int)hi.w;
        sb[ks][b] = l.sb[buf][2 * ks + h][t];
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[ks][a], B[ks][b], acc[a][b], 4, 0, 0,
                                                                       sa[ks][a], 0, sb[ks][b]);
  };

  // stage s: operands in LDS buffer s & 1; the register set that held it
  // takes the loads of stage s + 2 while the MFMAs run, the other set (stage
  // s + 1) goes to the other buffer afterwards.  The stage count is padded to
  // even: stages past K load clamped addresses and store zeros, so every
  // load and store is unconditional.
  const int stages = (K + kBK - 1) / kBK;
  const int padded = (stages + 1) & ~1;
  MxStage s0, s1;
  mx_stage_load(s0, wc, ws, xc, xs, n0, m0, N, M, K, 0, tid);
  mx_stage_load(s1, wc, ws, xc, xs, n0, m0, N, M, K, kBK, tid);
  mx_stage_store(l, 0, s0, tid);
  __syncthreads();
  for (int s = 0; s < padded; s += 2) {
    mx_stage_load(s0, wc, ws, xc, xs, n0, m0, N, M, K, (s + 2) * kBK, tid);
    compute(0);
    mx_stage_store(l, 1, s1, tid);
    __syncthreads();
    mx_stage_load(s1, wc, ws, xc, xs, n0, m0, N, M, K, (s + 3) * kBK, tid);
    compute(1);
    mx_stage_store(l, 0, s0, tid);
    __syncthreads();
  }

#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t tok = m0 + wt + 32 * b + j;
    if (tok >= M) continue;
    float* yrow = y + tok * N;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t row = n0 + wr + 32 * a + 8 * g + 4 * h;
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
  const int64_t gx = (w->n + kBN - 1) / kBN;
  const int64_t gy = (m + kBM - 1) / kBM;
  if (gx * gy + 8 > 2147483647LL) return BDG_E_UNSUPPORTED;
  const int64_t blocks = (gx * gy + 7) / 8 * 8;     // whole chunks for the 8 XCDs
  hipLaunchKernelGGL(mx_gemm_kernel, dim3((unsigned)blocks), dim3(kGemmThreads), 0, as_stream(stream),
                     static_cast<const uint8_t*>(w->codes), static_cast<const uint8_t*>(w->scales), x_codes,
                     x_scales, w->n, m, (int)w->k, (int)gx, (int)gy, y);
  return launch_status();
}
