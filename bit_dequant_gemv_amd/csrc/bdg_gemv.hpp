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

// The scaling step of chunk_contrib alone, applied to a chunk's unscaled dot
// product (the same operations, so the same result).
template <int FMT>
__device__ __forceinline__ float chunk_finish(float dot, uint32_t scale_raw, uint32_t zero_nib, float xsum) {
  if constexpr (FMT == kMXFP4) {
    // block sum * 2^(e-127); e = 255 is NaN
    const float r = __builtin_amdgcn_ldexpf(dot, (int)scale_raw - 127);
    return scale_raw == 255u ? __uint_as_float(0x7FC00000u) : r;
  } else {
    const float s = f16_bits_to_f32((uint16_t)scale_raw);
    const float part = dot - (float)zero_nib * xsum;
    return part * s;
  }
}

// Unscaled dot products of one code chunk with NT inputs at once: each code
// pair is decoded once and used by every input.  Per input the two chains
// and the order of their FMAs are those of fp4_chunk_dot / u4_chunk_dot, so
// out[t] equals the single-input result bit for bit.
template <int FMT, int NT>
__device__ __forceinline__ void chunk_dot_multi(const uint4 q, const float (&x)[NT][kChunkElems], float (&out)[NT]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a0[NT], a1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) a0[t] = a1[t] = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f32x2 e0, e1, e2, e3;   // elements (8d, 8d+1), (8d+2, 8d+3), (8d+4, 8d+5), (8d+6, 8d+7)
    if constexpr (FMT == kMXFP4) {
      e0 = fp4_pair<0>(w[d]);
      e1 = fp4_pair<1>(w[d]);
      e2 = fp4_pair<2>(w[d]);
      e3 = fp4_pair<3>(w[d]);
    } else {
      const uint32_t lo = w[d] & 0x0F0F0F0Fu;
      const uint32_t hi = (w[d] >> 4) & 0x0F0F0F0Fu;
      const f32x2 e02 = u4_pair<false>(lo), e46 = u4_pair<true>(lo);
      const f32x2 e13 = u4_pair<false>(hi), e57 = u4_pair<true>(hi);
      e0 = f32x2{e02.x, e13.x};
      e1 = f32x2{e02.y, e13.y};
      e2 = f32x2{e46.x, e57.x};
      e3 = f32x2{e46.y, e57.y};
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      a0[t] = __builtin_fmaf(e0.x, x[t][8 * d + 0], a0[t]);
      a1[t] = __builtin_fmaf(e0.y, x[t][8 * d + 1], a1[t]);
      a0[t] = __builtin_fmaf(e1.x, x[t][8 * d + 2], a0[t]);
      a1[t] = __builtin_fmaf(e1.y, x[t][8 * d + 3], a1[t]);
      a0[t] = __builtin_fmaf(e2.x, x[t][8 * d + 4], a0[t]);
      a1[t] = __builtin_fmaf(e2.y, x[t][8 * d + 5], a1[t]);
      a0[t] = __builtin_fmaf(e3.x, x[t][8 * d + 6], a0[t]);
      a1[t] = __builtin_fmaf(e3.y, x[t][8 * d + 7], a1[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) out[t] = a0[t] + a1[t];
}

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
  uint32_t zn[S];   // int4: the byte holding the zero point
  uint32_t ok;      // bit s: slot s holds a real chunk of a real row
  uint32_t zhi;     // bit s: int4 zero point in the high nibble
};

// Load the slots of one row for this lane.  Branch-free: a row past the end
// (row_ok false) reads row 0 and a chunk past the end reads the row's last
// chunk, so every load is in bounds and issued unconditionally; row_dot gives
// such slots a neutral scale and their x registers are zero, so they add 0,
// and results of rows past the end are never stored.
// One slot of load_row (ld.ok and ld.zhi cleared beforehand).
template <int FMT, int L, int S>
__device__ __forceinline__ void load_row_slot(GroupLoad<FMT, S>& ld, const QMat& m, const QGeom& g,
                                              int64_t row, bool row_ok, int li, int s) {
  // offsets inside one matrix fit 32 bits (check_qmat rejects n * k / 2 >= 2^32)
  const uint32_t r = row_ok ? (uint32_t)row : 0u;
  const int c = li + L * s;
  const bool ok = row_ok && c < g.chunks;
  const uint32_t cc = (uint32_t)(c < g.chunks ? c : g.chunks - 1);
  ld.ok |= (ok ? 1u : 0u) << s;
  ld.q[s] = ldg_u128(m.codes + (r * (uint32_t)g.chunks + cc) * 16u);
  if constexpr (FMT == kMXFP4) {
    ld.sc[s] = ldg_u8(m.scales + (r * (uint32_t)g.chunks + cc));   // one 32-bit offset: scalar-base load
    ld.zn[s] = 0;
  } else {
    const uint32_t gi = (cc * kChunkElems) / (uint32_t)g.group;
    ld.sc[s] = ldg_u16(m.scales + (r * (uint32_t)g.groups + gi) * 2u);
    ld.zn[s] = ldg_u8(m.zeros + (r * (uint32_t)g.zrow + (gi >> 1)));
    ld.zhi |= (gi & 1u) << s;
  }
}

template <int FMT, int L, int S>
__device__ __forceinline__ void load_row(GroupLoad<FMT, S>& ld, const QMat& m, const QGeom& g,
                                         int64_t row, bool row_ok, int li) {
  ld.ok = 0;
  ld.zhi = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) load_row_slot<FMT, L, S>(ld, m, g, row, row_ok, li, s);
}

// Mark a loaded row's registers as rewritten (an empty asm, no instruction):
// when one row load serves several inputs in a loop, this keeps the compiler
// from hoisting the decode of all rows out of the loop (which would hold
// every decoded weight in registers at once).
template <int FMT, int S>
__device__ __forceinline__ void pin_regs(GroupLoad<FMT, S>& ld) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    asm volatile("" : "+v"(ld.q[s].x), "+v"(ld.q[s].y), "+v"(ld.q[s].z), "+v"(ld.q[s].w), "+v"(ld.sc[s]));
    if constexpr (FMT == kINT4G) asm volatile("" : "+v"(ld.zn[s]));
  }
}

// The x values of a lane's slots, from the LDS chunk layout (chunk c at
// floats [c*kXStride, c*kXStride+32)).  Chunks past the end read as 0.
template <int FMT, int L, int S>
struct XRegs {
  float v[S][kChunkElems];
  float sum[S];   // int4: sum of the chunk's x values (zero-point fold)

  // Branch-free: a slot past the row end reads the last chunk and zeroes it,
  // so no load is inside a branch (a branch here makes the compiler wait for
  // every outstanding weight load).
  __device__ __forceinline__ void load(const float* __restrict__ lds_x, int chunks, int li) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = li + L * s;
      const bool ok = c < chunks;
      const float4* src = reinterpret_cast<const float4*>(lds_x + (ok ? c : chunks - 1) * kXStride);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 t = src[q];
        v[s][4 * q + 0] = ok ? t.x : 0.f;
        v[s][4 * q + 1] = ok ? t.y : 0.f;
        v[s][4 * q + 2] = ok ? t.z : 0.f;
        v[s][4 * q + 3] = ok ? t.w : 0.f;
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

  // The same where the LDS region holds one more chunk, all zeros, at index
  // `chunks`: a slot past the row end reads that chunk, so no value needs a
  // select (one index clamp per slot instead of 32 selects).
  __device__ __forceinline__ void load_zpad(const float* __restrict__ lds_x, int chunks, int li) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = li + L * s;
      const float4* src = reinterpret_cast<const float4*>(lds_x + (c < chunks ? c : chunks) * kXStride);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 t = src[q];
        v[s][4 * q + 0] = t.x;
        v[s][4 * q + 1] = t.y;
        v[s][4 * q + 2] = t.z;
        v[s][4 * q + 3] = t.w;
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
// the row; the row's dot product is valid in the group's last lane
// (li == L - 1, see kRowSumLane).
template <int FMT, int L, int S>
__device__ __forceinline__ float row_dot(const GroupLoad<FMT, S>& ld, const XRegs<FMT, L, S>& xr) {
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool ok = (ld.ok >> s) & 1u;
    // neutral scale for padding slots (fp16 0x3C00 = 1.0: an infinite scale
    // times their zero sum would be NaN).  MXFP4 needs none: a padding slot
    // repeats the row's last chunk against zero x, so it adds 0, or NaN only
    // where that chunk's own scale (E8M0 255) already makes the row NaN.
    const uint32_t sc = FMT == kMXFP4 ? ld.sc[s] : (ok ? ld.sc[s] : 0x3C00u);
    const uint32_t z = (ld.zn[s] >> (((ld.zhi >> s) & 1u) * 4u)) & 15u;
    acc += chunk_contrib<FMT>(ld.q[s], sc, z, xr.v[s], xr.sum[s]);
  }
  return group_sum_last<L>(acc);
}

// row_dot of NR loaded rows against NT inputs staged in LDS (input t at
// lds_x + t * xstride in the chunk layout, with a zero chunk at index
// `chunks`), taken slot by slot: a slot's x values of the NT inputs are read
// into registers once and each code chunk is decoded once for all of them.
// Each row's slots are added in row_dot's order with row_dot's per-chunk
// arithmetic and butterfly, so out[i][t] equals row_dot(ld[i], x_t) bit for
// bit.  Rows whose loads were issued slot-major (every row's slot 0 first)
// are consumed in that order, so the first slot's math waits only for the
// first slot's loads.
template <int FMT, int L, int S, int NR, int NT>
__device__ __forceinline__ void rows_dot_multi(const GroupLoad<FMT, S> (&ld)[NR], const float* __restrict__ lds_x,
                                               int xstride, int chunks, int li, float (&out)[NR][NT]) {
  float acc[NR][NT];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    // one slot at a time: the scheduler would otherwise read every slot's x
    // values up front and hold S times the registers
    __builtin_amdgcn_sched_barrier(0);
    const int c = li + L * s;
    const int cc = c < chunks ? c : chunks;
    float xv[NT][kChunkElems];
    float xsum[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float4* src = reinterpret_cast<const float4*>(lds_x + t * xstride + cc * kXStride);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = src[q];
        xv[t][4 * q + 0] = v.x;
        xv[t][4 * q + 1] = v.y;
        xv[t][4 * q + 2] = v.z;
        xv[t][4 * q + 3] = v.w;
      }
      xsum[t] = 0.f;
      if constexpr (FMT == kINT4G) {
#pragma unroll
        for (int q = 0; q < kChunkElems; ++q) xsum[t] += xv[t][q];
      }
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const bool ok = (ld[i].ok >> s) & 1u;
      const uint32_t sc = FMT == kMXFP4 ? ld[i].sc[s] : (ok ? ld[i].sc[s] : 0x3C00u);
      const uint32_t z = (ld[i].zn[s] >> (((ld[i].zhi >> s) & 1u) * 4u)) & 15u;
      // an empty asm per input count: where one kernel takes several
      // counts on branches of its own, the decodes of the branches are no
      // longer identical, so the compiler cannot hoist all of them above the
      // branch (holding every decoded weight of the rows in registers)
      uint4 q = ld[i].q[s];
      asm volatile("; rows_dot_multi, %4 inputs" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w) : "i"(NT));
      float dot[NT];
      chunk_dot_multi<FMT, NT>(q, xv, dot);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[i][t] += chunk_finish<FMT>(dot[t], sc, z, xsum[t]);
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) out[i][t] = group_sum_last<L>(acc[i][t]);
}

// Lane (within its L-lane group) that holds row_dot's result.
template <int L>
constexpr int kRowSumLane = L - 1;

// Stage n fp32 values (times `mult`) from global memory into the LDS chunk
// layout.  Values are split into `per`-long vectors placed `region` floats
// apart in LDS (several expert inputs at once); per % 32 == 0.  NV float4
// loads per thread are issued before any LDS store, so a block pays the
// memory latency once per NV * nthreads * 4 values, not once per value.
template <int NV>
__device__ __forceinline__ void stage_f32(float* __restrict__ lds_x, const float* __restrict__ src, int n,
                                          int per, int region, float mult, int tid, int nthreads) {
  for (int base = 0; base < n; base += NV * nthreads * 4) {
    float4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = base + (i * nthreads + tid) * 4;
      v[i] = ldg_f4(src + (idx < n ? idx : n - 4));   // in bounds; unused past n
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = base + (i * nthreads + tid) * 4;
      if (idx < n) {
        const int rgn = idx / per;
        const int w = idx - rgn * per;
        float4 o = v[i];
        o.x *= mult;
        o.y *= mult;
        o.z *= mult;
        o.w *= mult;
        *reinterpret_cast<float4*>(lds_x + rgn * region + (w >> 5) * kXStride + (w & 31)) = o;
      }
    }
  }
}

// Two-phase staging for n <= NV * nthreads * 4 values: load() issues all the
// global loads (call it before anything whose data should arrive later, so
// the in-order vmcnt wait for these loads does not also wait for that), and
// store() writes them into the LDS chunk layout as stage_f32 does.
template <int NV>
struct StageF32 {
  float4 v[NV];

  __device__ __forceinline__ void load(const float* __restrict__ src, int n, int tid, int nthreads) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = (i * nthreads + tid) * 4;
      v[i] = ldg_f4(src + (idx < n ? idx : n - 4));   // in bounds; unused past n
    }
  }

  __device__ __forceinline__ void store(float* __restrict__ lds_x, int n, int per, int region, float mult, int tid,
                                        int nthreads) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = (i * nthreads + tid) * 4;
      if (idx < n) {
        const int rgn = idx / per;
        const int w = idx - rgn * per;
        float4 o = v[i];
        o.x *= mult;
        o.y *= mult;
        o.z *= mult;
        o.w *= mult;
        *reinterpret_cast<float4*>(lds_x + rgn * region + (w >> 5) * kXStride + (w & 31)) = o;
      }
    }
  }
};

// StageF32 for a bf16 source: the loads keep the raw 8-byte words, store()
// widens them (exactly) to fp32 and writes them as StageF32::store does.
template <int NV>
struct StageBF16 {
  uint2 v[NV];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int n, int tid, int nthreads) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = (i * nthreads + tid) * 4;
      v[i] = ldg_u64(src + (idx < n ? idx : n - 4));   // in bounds; unused past n
    }
  }

  __device__ __forceinline__ void store(float* __restrict__ lds_x, int n, int per, int region, float mult, int tid,
                                        int nthreads) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = (i * nthreads + tid) * 4;
      if (idx < n) {
        const int rgn = idx / per;
        const int w = idx - rgn * per;
        float4 o = make_float4(bf16_to_f32((uint16_t)(v[i].x & 0xFFFFu)), bf16_to_f32((uint16_t)(v[i].x >> 16)),
                               bf16_to_f32((uint16_t)(v[i].y & 0xFFFFu)), bf16_to_f32((uint16_t)(v[i].y >> 16)));
        o.x *= mult;
        o.y *= mult;
        o.z *= mult;
        o.w *= mult;
        *reinterpret_cast<float4*>(lds_x + rgn * region + (w >> 5) * kXStride + (w & 31)) = o;
      }
    }
  }
};

// The same for a bf16 source (4 values per 8-byte load), one region.
template <int NV>
__device__ __forceinline__ void stage_bf16(float* __restrict__ lds_x, const uint16_t* __restrict__ src, int n,
                                           int tid, int nthreads) {
  for (int base = 0; base < n; base += NV * nthreads * 4) {
    uint2 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = base + (i * nthreads + tid) * 4;
      v[i] = ldg_u64(src + (idx < n ? idx : n - 4));   // in bounds; unused past n
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = base + (i * nthreads + tid) * 4;
      if (idx < n) {
        const float4 o = make_float4(bf16_to_f32((uint16_t)(v[i].x & 0xFFFFu)), bf16_to_f32((uint16_t)(v[i].x >> 16)),
                                     bf16_to_f32((uint16_t)(v[i].y & 0xFFFFu)), bf16_to_f32((uint16_t)(v[i].y >> 16)));
        *reinterpret_cast<float4*>(lds_x + (idx >> 5) * kXStride + (idx & 31)) = o;
      }
    }
  }
}

}  // namespace bdg
