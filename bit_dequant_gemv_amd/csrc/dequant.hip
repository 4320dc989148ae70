// Standalone dequantisation: the exact weight values every fused kernel
// multiplies with.  The gpt-oss page checks its MXFP4 reader bit-exact
// (max_abs 0.0, "Sovereign gpt-oss-20B (MXFP4) on Apple Silicon", section 3);
// tracker entry D108 states the fused int4 kernel equals dequantisation
// followed by an ordered matmul.  These kernels are that dequantisation.
#include "bdg_device.hpp"
#include "bdg_host.hpp"

namespace bdg {

// One thread per 16-byte chunk: 32 codes of one row and their scale.
__global__ void __launch_bounds__(256)
mxfp4_dequant_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                     int64_t n_chunks, int chunks_per_row, void* __restrict__ out, int bf16_out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_chunks) return;
  const uint4 q = reinterpret_cast<const uint4*>(codes)[t];
  const float s = e8m0_to_f32(scales[t]);    // chunk t of row r is block t of the flat scale array
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float v[32];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int nib = 0; nib < 8; ++nib) v[8 * d + nib] = e2m1_to_f32((w[d] >> (4 * nib)) & 15u) * s;
  if (!bf16_out) {
    float4* o = reinterpret_cast<float4*>(out) + t * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  } else {
    // bf16 through gfx950's scaled FP4 -> bf16 conversion, the instruction
    // the matrix-core decode path uses: E2M1 times 2^(e-127) is exact in
    // bf16 (subnormals included), so this is the fp32 value above rounded
    // to nearest even (+-inf where that overflows, NaN for e = 255)
    uint4* o = reinterpret_cast<uint4*>(out) + t * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], s, 0));
      const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], s, 1));
      const uint32_t p2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], s, 2));
      const uint32_t p3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], s, 3));
      o[i] = make_uint4(p0, p1, p2, p3);
    }
  }
  (void)chunks_per_row;
}

__global__ void __launch_bounds__(256)
int4g_dequant_kernel(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                     const uint8_t* __restrict__ zeros, int64_t n_chunks, int chunks_per_row,
                     int groups, int zrow, int chunks_per_group, float* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n_chunks) return;
  const int64_t row = t / chunks_per_row;
  const int c = (int)(t - row * chunks_per_row);
  const int g = c / chunks_per_group;
  const uint4 q = reinterpret_cast<const uint4*>(codes)[t];
  const float s = f16_bits_to_f32(scales[row * groups + g]);
  const uint32_t zb = zeros[row * zrow + (g >> 1)];
  const int z = (int)((g & 1) ? (zb >> 4) : (zb & 15u));
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float4* o = reinterpret_cast<float4*>(out) + t * 8;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    float v[8];
#pragma unroll
    for (int nib = 0; nib < 8; ++nib) v[nib] = (float)((int)((w[d] >> (4 * nib)) & 15u) - z) * s;
    o[2 * d] = make_float4(v[0], v[1], v[2], v[3]);
    o[2 * d + 1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

}  // namespace bdg

using namespace bdg;

extern "C" int mxfp4_dequant(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                             void* out, int32_t out_dtype, void* stream) {
  if (!codes || !scales || !out || n < 0 || k < 0 || (k % 32) != 0) return BDG_E_INVALID;
  if (out_dtype != BDG_F32 && out_dtype != BDG_BF16) return BDG_E_INVALID;
  if (!aligned16(codes) || !aligned16(out)) return BDG_E_ALIGN;
  const int64_t n_chunks = n * (k / 32);
  if (n_chunks == 0) return BDG_OK;
  const int64_t blocks = (n_chunks + 255) / 256;
  if (blocks > 0x7FFFFFFF) return BDG_E_UNSUPPORTED;
  hipLaunchKernelGGL(mxfp4_dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     codes, scales, n_chunks, (int)(k / 32), out, out_dtype == BDG_BF16 ? 1 : 0);
  return launch_status();
}

extern "C" int int4g_dequant(const uint8_t* codes, const uint16_t* scales_f16, const uint8_t* zeros,
                             int64_t n, int64_t k, int32_t group, float* out, void* stream) {
  if (!codes || !scales_f16 || !zeros || !out || n < 0 || k < 0) return BDG_E_INVALID;
  if (group <= 0 || (group % 32) != 0 || (k % group) != 0) return BDG_E_INVALID;
  if (!aligned16(codes) || !aligned16(out)) return BDG_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(scales_f16) & 1u) != 0) return BDG_E_ALIGN;
  const int64_t n_chunks = n * (k / 32);
  if (n_chunks == 0) return BDG_OK;
  const int64_t blocks = (n_chunks + 255) / 256;
  if (blocks > 0x7FFFFFFF) return BDG_E_UNSUPPORTED;
  const int groups = (int)(k / group);
  hipLaunchKernelGGL(int4g_dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                     codes, scales_f16, zeros, n_chunks, (int)(k / 32), groups, (groups + 1) / 2,
                     group / 32, out);
  return launch_status();
}
