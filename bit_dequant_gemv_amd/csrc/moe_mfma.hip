// Grouped expert products of a step of M > 1 tokens on the matrix cores.
//
// The pages leave the grouped-expert GEMM over the active experts untried
// ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon", section 5).  At the
// small M of a decode step most chosen experts serve one or two tokens, and
// the grouped VALU kernels (moe.hip) decode every weight once per pick; at
// M = 16 their waves keep the vector unit about 80% busy.  Here each
// distinct expert of a layer is one chunk holding all its picks (t <= 16),
// and its products run on v_mfma_f32_32x32x16_bf16 with:
//   * weights decoded once per element to bf16 with the E8M0 block scale
//     applied in the conversion (v_cvt_scalef32_pk_bf16_fp4: E2M1 times
//     2^(e-127) is exact in bf16, subnormals included, +-inf exactly where
//     the fp32 product overflows, NaN for e = 255);
//   * activations as two bf16 parts, hi = bf16(v) and lo = bf16(v - hi), so
//     hi + lo carries v to about 2^-17 relative and every product is exact
//     in the fp32 accumulator (the decode path's fp32 accuracy, not bf16's);
//   * the weight rows as the instruction's columns: D[token row][weight row],
//     token rows 0..15 = the picks' hi parts, 16..31 = their lo parts, so a
//     lane's 16 results all belong to one weight row and y = D[r] + D[r + 8].
// MFMA operand layout (measured on the device with one-hot operands): lane l
// supplies row (A) / column (B) l % 32 and K positions 8 (l / 32) + i; D
// register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column
// l % 32.  Lanes 0..31 take MX block 2s of a super-step s, lanes 32..63
// block 2s + 1, so one 16-byte code chunk feeds a lane for 4 instructions.
//
// A wave takes (chunk, 32-row tile) items: gate_up tiles pair gate rows
// i0..i0+31 with up rows I+i0..I+i0+31 so h = silu(g) u forms lane-locally
// and is written as its bf16 hi/lo parts; down tiles write one fp32 output
// row block per pick, combined later in slot order as on the VALU path.
#include "bdg_host.hpp"
#include "bdg_moe.hpp"
#include "bdg_moe_mfma.hpp"

namespace bdg {

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16_v __attribute__((ext_vector_type(16)));

constexpr int kMfmaThreads = 256;
constexpr int kMfmaWaves = kMfmaThreads / kWave;
using MfmaGroupLds = GroupLdsT<kMfmaTT>;

// 16 bytes of E2M1 codes (32 elements, one MX block) to 4 MFMA B operands of
// 8 bf16, the block scale applied in the conversion.
__device__ __forceinline__ void fp4_chunk_to_bf16(const uint4 q, float scale, bf16x8_v (&b)[4]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const bf16x2_v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], scale, 0);
    const bf16x2_v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], scale, 1);
    const bf16x2_v p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], scale, 2);
    const bf16x2_v p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], scale, 3);
    b[d] = bf16x8_v{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
}

__device__ __forceinline__ bf16x8_v as_bf16x8(const uint4 v) { return __builtin_bit_cast(bf16x8_v, v); }

// E8M0 byte -> fp32 scale 2^(e-127) (e = 0: the subnormal 2^-127; 255: NaN).
__device__ __forceinline__ float e8m0_scale(uint32_t e) { return e8m0_to_f32(e); }

__device__ __forceinline__ uint16_t bf16_bits(float v) { return f32_to_bf16_rne(v); }

// The operand row of token row `ar` of an item: the hi or lo part of the
// pick's activation (or the zero row when the chunk has fewer picks).
__device__ __forceinline__ const uint16_t* operand_row(const int* picks, int nt, int ar, const uint16_t* hi,
                                                       const uint16_t* lo, const uint16_t* zeros, int64_t stride,
                                                       int pick_div) {
  const int slot = ar & 15;
  if (slot >= nt) return zeros;
  const int src = picks[slot] / pick_div;
  return (ar >= 16 ? lo : hi) + (int64_t)src * stride;
}

// Token row of D register r (r < 8) for lane half h.
__device__ __forceinline__ int d_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// One tile: acc[T] += D over a K of `kblocks` MX blocks, for T weight tiles
// sharing the activation operand.  Row r of tile T reads codes/scales at
// crow[T] / srow[T] (the lane's weight row); the activation row is arow.
template <int T>
__device__ __forceinline__ void mfma_tile(f32x16_v (&acc)[T], const uint8_t* const (&crow)[T],
                                          const uint8_t* const (&srow)[T], const uint16_t* arow, int kblocks,
                                          int h) {
  const int nsuper = kblocks >> 1;
  // loads of super-step s: this lane's block 2s + h
  uint4 q[T], qn[T];
  uint32_t sc[T], scn[T];
  uint4 a[4], an[4];
  auto load = [&](int s, uint4 (&qq)[T], uint32_t (&ss)[T], uint4 (&aa)[4]) {
    const int bk = 2 * s + h;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      qq[t] = ldg_u128(crow[t] + (uint32_t)bk * 16u);
      ss[t] = ldg_u8(srow[t] + bk);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) aa[i] = ldg_u128(arow + bk * 32 + 8 * i);
  };
  load(0, q, sc, a);
  for (int s = 0; s < nsuper; ++s) {
    const int sn = s + 1 < nsuper ? s + 1 : s;   // the last step reloads itself (in bounds, unused)
    load(sn, qn, scn, an);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      bf16x8_v b[4];
      fp4_chunk_to_bf16(q[t], e8m0_scale(sc[t]), b);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), b[i], acc[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      q[t] = qn[t];
      sc[t] = scn[t];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = an[i];
  }
}

// ---------------------------------------------------------------- gate_up

template <int V>
__global__ void __launch_bounds__(kMfmaThreads) moe_gu_mfma_kernel(MfmaParams p) {
  __shared__ MfmaGroupLds gl;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  group_route<V, kMfmaTT>(gl, p, lane, wave, kMfmaWaves);
  if (blockIdx.x == 0) write_chunk_table(gl, p.table, kMfmaThreads);

  const int h = lane >> 5;
  const int wr = lane & 31;
  const int kb = p.H / 32;
  const int tiles = p.I / kMfmaRows;
  const int nitems = gl.n * tiles;
  const int GW = gridDim.x * kMfmaWaves;
  for (int item = blockIdx.x * kMfmaWaves + wave; item < nitems; item += GW) {
    const int c = item / tiles;
    const int i0 = (item - c * tiles) * kMfmaRows;
    const int e = gl.ce[c];
    const int nt = gl.cn[c];
    const QMat m = expert_gu(p.L, e);
    const uint32_t grow = (uint32_t)(i0 + wr), urow = (uint32_t)(p.I + i0 + wr);
    const uint8_t* const crow[2] = {m.codes + grow * (uint32_t)kb * 16u, m.codes + urow * (uint32_t)kb * 16u};
    const uint8_t* const srow[2] = {m.scales + grow * (uint32_t)kb, m.scales + urow * (uint32_t)kb};
    const uint16_t* arow = operand_row(gl.cpk[c], nt, lane & 31, p.xh, p.xl, p.zeros, p.H, p.K);
    f32x16_v acc[2] = {};
    mfma_tile<2>(acc, crow, srow, arow, kb, h);
    // h = silu(g) u for each pick of the chunk, as bf16 hi/lo parts
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int slot = d_row(r, h);
      if (slot < nt) {
        const float g = acc[0][r] + acc[0][r + 8];
        const float u = acc[1][r] + acc[1][r + 8];
        const float hv = g / (1.0f + expf(-g)) * u;
        const uint16_t hi = bf16_bits(hv);
        const uint16_t lo = bf16_bits(hv - bf16_to_f32(hi));
        const int64_t o = (int64_t)gl.cpk[c][slot] * p.I + i0 + wr;
        p.hh[o] = hi;
        p.hl[o] = lo;
      }
    }
  }
}

// ---------------------------------------------------------------- down

__global__ void __launch_bounds__(kMfmaThreads) moe_dn_mfma_kernel(MfmaParams p) {
  __shared__ int tab[1 + kGroupMaxPicks * kMfmaChunkInts];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  const int n = p.table[0];
  for (int i = threadIdx.x; i < n * kMfmaChunkInts; i += kMfmaThreads) tab[1 + i] = p.table[1 + i];
  __syncthreads();

  const int h = lane >> 5;
  const int wr = lane & 31;
  const int kb = p.I / 32;
  const int tiles = p.H / kMfmaRows;
  const int nitems = n * tiles;
  const int GW = gridDim.x * kMfmaWaves;
  for (int item = blockIdx.x * kMfmaWaves + wave; item < nitems; item += GW) {
    const int c = item / tiles;
    const int r0 = (item - c * tiles) * kMfmaRows;
    const int* ch = tab + 1 + c * kMfmaChunkInts;
    const int e = clamp_expert(ch[0], p.E);
    const int nt = ch[1];
    const QMat m = expert_dn(p.L, e);
    const uint32_t row = (uint32_t)(r0 + wr);
    const uint8_t* const crow[1] = {m.codes + row * (uint32_t)kb * 16u};
    const uint8_t* const srow[1] = {m.scales + row * (uint32_t)kb};
    const uint16_t* arow = operand_row(ch + 2, nt, lane & 31, p.hh, p.hl, p.zeros, p.I, 1);
    f32x16_v acc[1] = {};
    mfma_tile<1>(acc, crow, srow, arow, kb, h);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int slot = d_row(r, h);
      if (slot < nt) p.dout[(int64_t)ch[2 + slot] * p.H + r0 + wr] = acc[0][r] + acc[0][r + 8];
    }
  }
}

// ---------------------------------------------------------------- host side

size_t mfma_gu_lds_bytes() { return sizeof(MfmaGroupLds); }
size_t mfma_dn_lds_bytes() { return sizeof(int) * (1 + kGroupMaxPicks * kMfmaChunkInts); }

const void* mfma_gu_kernel(int V) {
  switch (V) {
    case 1: return reinterpret_cast<const void*>(&moe_gu_mfma_kernel<1>);
    case 2: return reinterpret_cast<const void*>(&moe_gu_mfma_kernel<2>);
    case 4: return reinterpret_cast<const void*>(&moe_gu_mfma_kernel<4>);
    case 16: return reinterpret_cast<const void*>(&moe_gu_mfma_kernel<16>);
    default: return nullptr;
  }
}
const void* mfma_dn_kernel() { return reinterpret_cast<const void*>(&moe_dn_mfma_kernel); }

int launch_gu_mfma(const MfmaParams& p, int V, int nblk, hipStream_t s) {
  switch (V) {
    case 1: hipLaunchKernelGGL(moe_gu_mfma_kernel<1>, dim3(nblk), dim3(kMfmaThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL(moe_gu_mfma_kernel<2>, dim3(nblk), dim3(kMfmaThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL(moe_gu_mfma_kernel<4>, dim3(nblk), dim3(kMfmaThreads), 0, s, p); break;
    case 16: hipLaunchKernelGGL(moe_gu_mfma_kernel<16>, dim3(nblk), dim3(kMfmaThreads), 0, s, p); break;
    default: return BDG_E_UNSUPPORTED;
  }
  return launch_status();
}

int launch_dn_mfma(const MfmaParams& p, int nblk, hipStream_t s) {
  hipLaunchKernelGGL(moe_dn_mfma_kernel, dim3(nblk), dim3(kMfmaThreads), 0, s, p);
  return launch_status();
}

}  // namespace bdg
