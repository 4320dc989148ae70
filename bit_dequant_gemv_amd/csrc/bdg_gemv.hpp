// Row-group dequant-GEMV engine shared by qgemv and the MoE expert kernels.
//
// A wavefront computes dot products of RPW = 64/L rows at once: L lanes per
// row, lane li of a row handles the 16-byte code chunks c = li, li + L, ...,
// li + (S-1)L (S "slots").  Each chunk is one MX block (32 codes + 1 E8M0
// byte) or half an int4 group.  The matching x values of a lane's chunks sit
// in VGPRs for the whole task (32 per slot), staged once through LDS, so the
// hot loop is: 16-byte code load -> on-chip decode -> fp32 FMA -> block scale.
// The L partial sums of a row are combined by a fixed DPP/swizzle butterfly,
// so results are deterministic.  This replaces the pages' cooperative
// multi-SIMD-group GEMV ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon",
// section 4: the same math with the cross-block fp32 sum re-associated) with
// a wave64 layout: for K = 2880 (90 chunks) L = 32, S = 3 keeps 94% of lanes
// busy and a row pair per wave-iteration.
#pragma once

#include "bdg_device.hpp"

namespace bdg {

// Geometry of one packed matrix family (all experts of one projection).
struct QGeom {
  int k;          // reduction length
  int chunks;     // k / 32
  int group;      // int4 group size (elements)
  int groups;     // k / group
  int zrow;       // zero-point bytes per row
};

template <int FMT, int S>
struct GroupLoad {
  uint4 q[S];
  uint32_t sc[S];
  uint32_t zn[S];
};

// Load the slots of one row for this lane.  row_ok false -> zeros.
template <int FMT, int L, int S>
__device__ __forceinline__ void load_row(GroupLoad<FMT, S>& ld, const QMat& m, const QGeom& g,
                                         int64_t row, bool row_ok, int li) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = li + L * s;
    const bool ok = row_ok && c < g.chunks;
    if (ok) {
      const uint8_t* p = m.codes + row * (int64_t)(g.chunks * 16) + (int64_t)c * 16;
      ld.q[s] = *reinterpret_cast<const uint4*>(p);
      if constexpr (FMT == kMXFP4) {
        ld.sc[s] = m.scales[row * (int64_t)g.chunks + c];
        ld.zn[s] = 0;
      } else {
        const int gi = (c * kChunkElems) / g.group;
        ld.sc[s] = reinterpret_cast<const uint16_t*>(m.scales)[row * (int64_t)g.groups + gi];
        const uint32_t zb = m.zeros[row * (int64_t)g.zrow + (gi >> 1)];
        ld.zn[s] = (gi & 1) ? (zb >> 4) : (zb & 15u);
      }
    } else {
      ld.q[s] = make_uint4(0u, 0u, 0u, 0u);
      ld.sc[s] = 0u;
      ld.zn[s] = 0u;
    }
  }
}

// The x values of a lane's slots, from the LDS chunk layout (chunk c at
// floats [c*kXStride, c*kXStride+32)).  Chunks past the end read as 0.
template <int FMT, int L, int S>
struct XRegs {
  float v[S][kChunkElems];
  float sum[S];   // int4: sum of the chunk's x values (zero-point fold)

  __device__ __forceinline__ void load(const float* __restrict__ lds_x, int chunks, int li) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = li + L * s;
      if (c < chunks) {
        const float4* src = reinterpret_cast<const float4*>(lds_x + c * kXStride);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 t = src[q];
          v[s][4 * q + 0] = t.x;
          v[s][4 * q + 1] = t.y;
          v[s][4 * q + 2] = t.z;
          v[s][4 * q + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < kChunkElems; ++q) v[s][q] = 0.f;
      }
      if constexpr (FMT == kINT4G) {
        float a = 0.f;
#pragma unroll
        for (int q = 0; q < kChunkElems; ++q) a += v[s][q];
        sum[s] = a;
      } else {
        sum[s] = 0.f;
      }
    }
  }
};

// Lane-partial dot of the loaded row against x, summed over the L lanes of
// the row (every lane of the row group receives the row's dot product).
template <int FMT, int L, int S>
__device__ __forceinline__ float row_dot(const GroupLoad<FMT, S>& ld, const XRegs<FMT, L, S>& xr) {
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) acc += chunk_contrib<FMT>(ld.q[s], ld.sc[s], ld.zn[s], xr.v[s], xr.sum[s]);
  return group_sum<L>(acc);
}

// Stage x (fp32 or bf16, times an optional scalar) into the LDS chunk layout.
__device__ __forceinline__ void stage_x(float* __restrict__ lds_x, const void* x, int x_is_bf16,
                                        int64_t offset, int k, float mult) {
  for (int i = threadIdx.x; i < k; i += blockDim.x) {
    float v = x_is_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[offset + i])
                        : reinterpret_cast<const float*>(x)[offset + i];
    lds_x[(i >> 5) * kXStride + (i & 31)] = v * mult;
  }
}

}  // namespace bdg
