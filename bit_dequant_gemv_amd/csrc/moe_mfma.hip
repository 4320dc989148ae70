// Grouped expert products of a step of M > 1 tokens on the matrix cores.
//
// The pages leave the grouped-expert GEMM over the active experts untried
// ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon", section 5).  At the
// small M of a decode step most chosen experts serve one or two tokens, and
// the grouped VALU kernels (moe.hip) decode every weight once per pick; at
// M = 16 their waves keep the vector unit about 80% busy.  Here each
// distinct expert of a layer is one or more chunks of up to 8 picks, and its
// products run on v_mfma_f32_16x16x32_bf16 with:
//   * weights decoded once per element to bf16 with the E8M0 block scale
//     applied in the conversion (v_cvt_scalef32_pk_bf16_fp4: E2M1 times
//     2^(e-127) is exact in bf16, subnormals included, +-inf exactly where
//     the fp32 product overflows, NaN for e = 255);
//   * activations as two bf16 parts, hi = bf16(v) and lo = bf16(v - hi), so
//     hi + lo carries v to about 2^-17 relative and every product is exact
//     in the fp32 accumulator (the decode path's fp32 accuracy, not bf16's);
//   * the weight rows as the instruction's 16 columns and the picks' parts
//     as its 16 rows: token row 2s is pick slot s's hi part, 2s + 1 its lo
//     part, so lane (n, q) ends with rows 4q .. 4q+3 of weight row n, i.e.
//     slots 2q and 2q + 1, and y = D[2s] + D[2s + 1] lane-locally.
// Operand layout: lane l supplies row (A) / column (B) l % 16 and one group
// of 8 K positions per lane quarter q = l / 16 (A and B alike, so any
// assignment of K to (q, element) that both sides share is correct); D
// register r of lane l holds row 4 (l / 16) + r, column l % 16.  Quarter q
// of a K group takes MX block 4g + q whole: its 16 code bytes are one load
// and feed the 4 instructions of the group (bytes 4j .. 4j+3 in
// instruction j), so one load instruction reads 64 contiguous bytes of each
// of 16 weight rows and the next group the rest of the 128-byte line.
//
// A block (4 waves) takes (chunk, tile pair) items: gate_up pairs gate rows
// i0..i0+15 with up rows I+i0.. so h = silu(g) u forms lane-locally and is
// written as its bf16 hi/lo parts; down pairs two 16-row tiles of the
// output.  The 4 waves split the K groups of an item, keep 3 groups in
// flight each, and add their partial tiles in LDS in wave order (a fixed
// order: results do not depend on timing).
#include "bdg_host.hpp"
#include "bdg_moe.hpp"
#include "bdg_moe_mfma.hpp"

namespace bdg {

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

constexpr int kMfmaThreads = 256;
constexpr int kMfmaWaves = kMfmaThreads / kWave;
constexpr int kMfmaDepth = 3;               // K groups in flight per wave
using MfmaGroupLds = GroupLdsT<kMfmaTT>;

// 16 bytes of E2M1 codes (32 elements, one MX block) to 4 MFMA B operands of
// 8 bf16 (elements 8j .. 8j+7 in operand j), the block scale applied in the
// conversion.
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

// The operand row of token row `ar` (0..15) of an item: the hi (even rows)
// or lo (odd rows) part of pick slot ar / 2's activation, or the zero row
// when the chunk has fewer picks.
__device__ __forceinline__ const uint16_t* operand_row(const int* picks, int nt, int ar, const uint16_t* hi,
                                                       const uint16_t* lo, const uint16_t* zeros, int64_t stride,
                                                       int pick_div) {
  const int slot = ar >> 1;
  if (slot >= nt) return zeros;
  const int src = picks[slot] / pick_div;
  return ((ar & 1) ? lo : hi) + (int64_t)src * stride;
}

// One K group of one lane: the codes and scale of block b of its two weight
// rows, and elements 32b .. 32b+31 of its token row.
struct MfmaStage {
  uint4 q[2];
  uint32_t sc[2];
  uint4 a[4];
};

__device__ __forceinline__ void stage_load(MfmaStage& st, const uint8_t* const (&crow)[2],
                                           const uint8_t* const (&srow)[2], const uint16_t* arow, int b) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    st.q[t] = ldg_u128(crow[t] + (uint32_t)b * 16u);
    st.sc[t] = ldg_u8(srow[t] + b);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) st.a[j] = ldg_u128(arow + b * 32 + 8 * j);
}

// acc[t] += the group's products; an invalid group (past the row's blocks,
// or past this wave's share) adds exact zeros (zero codes, unit scale).  Both
// tiles are converted first and their products alternate, so no product
// waits on the one issued just before it.
__device__ __forceinline__ void stage_mma(f32x4_v (&acc)[2], const MfmaStage& st, bool valid) {
  bf16x8_v b[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint4 q = valid ? st.q[t] : make_uint4(0u, 0u, 0u, 0u);
    fp4_chunk_to_bf16(q, valid ? e8m0_to_f32(st.sc[t]) : 1.0f, b[t]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(st.a[j]), b[t][j], acc[t], 0, 0, 0);
}

// The 4 waves' partial tiles of an item meet here; wave 0 adds them in wave
// order.  Double-buffered by item parity, so one barrier per item suffices.
struct MfmaRed {
  float v[2][kMfmaWaves][8][kWave];
};

// Operand addresses of one item for one lane: its two weight rows' codes and
// scales, and its token row.
struct MfmaRows {
  const uint8_t* crow[2];
  const uint8_t* srow[2];
  const uint16_t* arow;
};

// A block's items (first, first + stride, ... < nitems) streamed by its 4
// waves: wave w takes K groups [g0, g1) of every item (4 MX blocks each, kb
// per row; lane quarter q takes block 4g + q), one step per group, and its
// loads run kMfmaDepth steps ahead across item boundaries, so the next
// item's first groups are in flight while an item finishes.  rows(item)
// gives an item's operand addresses; finish(item, j, y) runs in wave 0 with
// the item's summed tile (y[0..3]: first weight row, token rows 4q..4q+3;
// y[4..7]: second weight row), j the block-local item index.
template <class RowsF, class FinishF>
__device__ __forceinline__ void mfma_stream(MfmaRed& red, int first, int stride, int nitems, int kb, int wave,
                                            int lane, RowsF rows, FinishF finish) {
  const int q = lane >> 4;
  const int ngr = (kb + 3) >> 2;
  const int g0 = ngr * wave / kMfmaWaves, g1 = ngr * (wave + 1) / kMfmaWaves;
  const int n = g1 - g0;
  const int ns = n > 0 ? n : 1;              // steps per item (a wave without groups still meets each barrier)
  const int nj = first < nitems ? (nitems - first + stride - 1) / stride : 0;
  const int total = nj * ns;

  // load side: (item, step) of the next stage to fill, and its item's rows;
  // stages past the last step (the prologue of a block with few steps)
  // reload the last item's rows, in bounds and never used
  int ld_j = 0, ld_i = 0;
  MfmaRows lr = rows(first < nitems ? first : 0);
  auto load_next = [&](MfmaStage& st) {
    if (ld_i == 0 && ld_j > 0 && ld_j < nj) lr = rows(first + ld_j * stride);   // LDS reads only
    const int b = min(4 * (g0 + min(ld_i, ns - 1)) + q, kb - 1);
    stage_load(st, lr.crow, lr.srow, lr.arow, b);
    if (++ld_i == ns) {
      ld_i = 0;
      ++ld_j;
    }
  };
  MfmaStage st[kMfmaDepth];
#pragma unroll
  for (int d = 0; d < kMfmaDepth; ++d) load_next(st[d]);

  // Every stage is reloaded unconditionally (the last kMfmaDepth loads of a
  // wave fetch in-bounds rows nobody uses): with a load skipped on some path
  // the compiler could not count the loads still in flight at the loop's
  // join and would wait for all of them before the first product.
  f32x4_v acc[2] = {f32x4_v{0.f, 0.f, 0.f, 0.f}, f32x4_v{0.f, 0.f, 0.f, 0.f}};
  int cp_j = 0, cp_i = 0;
  for (int t0 = 0; t0 < total; t0 += kMfmaDepth) {
#pragma unroll
    for (int d = 0; d < kMfmaDepth; ++d) {
      const bool live = t0 + d < total;
      stage_mma(acc, st[d], live && cp_i < n && 4 * (g0 + cp_i) + q < kb);
      load_next(st[d]);
      if (live) {
        if (++cp_i == ns) {
          const int buf = cp_j & 1;
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int k = 0; k < 4; ++k) red.v[buf][wave][4 * t + k][lane] = acc[t][k];
          acc[0] = f32x4_v{0.f, 0.f, 0.f, 0.f};
          acc[1] = f32x4_v{0.f, 0.f, 0.f, 0.f};
          block_sync_lds();
          if (wave == 0) {
            float y[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              float sum = red.v[buf][0][k][lane];
#pragma unroll
              for (int w = 1; w < kMfmaWaves; ++w) sum += red.v[buf][w][k][lane];
              y[k] = sum;
            }
            finish(first + cp_j * stride, cp_j, y);
          }
          cp_i = 0;
          ++cp_j;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- gate_up

template <int V>
__global__ void __launch_bounds__(kMfmaThreads) moe_gu_mfma_kernel(MfmaParams p) {
  __shared__ MfmaGroupLds gl;
  __shared__ MfmaRed red;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  group_route<V, kMfmaTT>(gl, p, lane, wave, kMfmaWaves);
  if (blockIdx.x == 0) write_chunk_table(gl, p.table, kMfmaThreads);

  const int n = lane & 15;
  const int q = lane >> 4;
  const int kb = p.H / 32;
  const int tiles = p.I / kMfmaRows;
  auto rows = [&](int item) {
    const int c = item / tiles;
    const int i0 = (item - c * tiles) * kMfmaRows;
    const QMat m = expert_gu(p.L, gl.ce[c]);
    const uint32_t grow = (uint32_t)(i0 + n), urow = (uint32_t)(p.I + i0 + n);
    MfmaRows r;
    r.crow[0] = m.codes + grow * (uint32_t)kb * 16u;
    r.crow[1] = m.codes + urow * (uint32_t)kb * 16u;
    r.srow[0] = m.scales + grow * (uint32_t)kb;
    r.srow[1] = m.scales + urow * (uint32_t)kb;
    r.arow = operand_row(gl.cpk[c], gl.cn[c], n, p.xh, p.xl, p.zeros, p.H, p.K);
    return r;
  };
  // lane (n, q): slots 2q and 2q + 1 of gate row i0 + n (y[0..3]) and of up row I + i0 + n (y[4..7])
  auto finish = [&](int item, int, const float (&y)[8]) {
    const int c = item / tiles;
    const int i0 = (item - c * tiles) * kMfmaRows;
    const int nt = gl.cn[c];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int slot = 2 * q + h;
      if (slot < nt) {
        const float g = y[2 * h] + y[2 * h + 1];
        const float u = y[4 + 2 * h] + y[4 + 2 * h + 1];
        const float hv = g / (1.0f + expf(-g)) * u;
        const uint16_t hi = f32_to_bf16_rne(hv);
        const uint16_t lo = f32_to_bf16_rne(hv - bf16_to_f32(hi));
        const int64_t o = (int64_t)gl.cpk[c][slot] * p.I + i0 + n;
        p.hh[o] = hi;
        p.hl[o] = lo;
      }
    }
  };
  mfma_stream(red, blockIdx.x, gridDim.x, gl.n * tiles, kb, wave, lane, rows, finish);
}

// ---------------------------------------------------------------- down

__global__ void __launch_bounds__(kMfmaThreads) moe_dn_mfma_kernel(MfmaParams p) {
  __shared__ int tab[1 + kGroupMaxPicks * kMfmaChunkInts];
  __shared__ MfmaRed red;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_wave_id();
  const int nch = p.table[0];
  for (int i = threadIdx.x; i < nch * kMfmaChunkInts; i += kMfmaThreads) tab[1 + i] = p.table[1 + i];
  __syncthreads();

  const int n = lane & 15;
  const int q = lane >> 4;
  const int kb = p.I / 32;
  const int tiles = p.H / (2 * kMfmaRows);
  auto rows = [&](int item) {
    const int c = item / tiles;
    const int r0 = (item - c * tiles) * 2 * kMfmaRows;
    const int* ch = tab + 1 + c * kMfmaChunkInts;
    const QMat m = expert_dn(p.L, clamp_expert(ch[0], p.E));
    const uint32_t ra = (uint32_t)(r0 + n), rb = (uint32_t)(r0 + kMfmaRows + n);
    MfmaRows r;
    r.crow[0] = m.codes + ra * (uint32_t)kb * 16u;
    r.crow[1] = m.codes + rb * (uint32_t)kb * 16u;
    r.srow[0] = m.scales + ra * (uint32_t)kb;
    r.srow[1] = m.scales + rb * (uint32_t)kb;
    r.arow = operand_row(ch + 2, ch[1], n, p.hh, p.hl, p.zeros, p.I, 1);
    return r;
  };
  auto finish = [&](int item, int, const float (&y)[8]) {
    const int c = item / tiles;
    const int r0 = (item - c * tiles) * 2 * kMfmaRows;
    const int* ch = tab + 1 + c * kMfmaChunkInts;
    const int nt = ch[1];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int slot = 2 * q + h;
      if (slot < nt) {
        float* out = p.dout + (int64_t)ch[2 + slot] * p.H;
        out[r0 + n] = y[2 * h] + y[2 * h + 1];
        out[r0 + kMfmaRows + n] = y[4 + 2 * h] + y[4 + 2 * h + 1];
      }
    }
  };
  mfma_stream(red, blockIdx.x, gridDim.x, nch * tiles, kb, wave, lane, rows, finish);
}

// ---------------------------------------------------------------- host side

size_t mfma_gu_lds_bytes() { return sizeof(MfmaGroupLds) + sizeof(MfmaRed); }
size_t mfma_dn_lds_bytes() { return sizeof(int) * (1 + kGroupMaxPicks * kMfmaChunkInts) + sizeof(MfmaRed); }

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

int launch_gu_mfma(const MfmaParams& p, int V, int nblk, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
#define BDG_GU_MFMA(VV)                                                                                         \
  case VV:                                                                                                       \
    hipExtLaunchKernelGGL(moe_gu_mfma_kernel<VV>, dim3(nblk), dim3(kMfmaThreads), 0, s, ev_start, ev_stop, 0, p); \
    break;
  switch (V) {
    BDG_GU_MFMA(1) BDG_GU_MFMA(2) BDG_GU_MFMA(4) BDG_GU_MFMA(16)
    default: return BDG_E_UNSUPPORTED;
  }
#undef BDG_GU_MFMA
  return launch_status();
}

int launch_dn_mfma(const MfmaParams& p, int nblk, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  hipExtLaunchKernelGGL(moe_dn_mfma_kernel, dim3(nblk), dim3(kMfmaThreads), 0, s, ev_start, ev_stop, 0, p);
  return launch_status();
}

}  // namespace bdg
