// Wavefront top-k + softmax over router logits, shared by the decode
// kernels (every gate_up wave selects its own experts) and the standalone
// router.  Selection: the k largest logits in descending order, ties to the
// lower expert index; weights: softmax over the chosen k (the GPU top-k of
// the host-sync page, section 3).
#pragma once

#include "bdg_device.hpp"

namespace bdg {

// Order-preserving unsigned key of a float: larger float <-> larger key.
// -0.0 is folded onto +0.0 (they compare equal as floats) and NaN onto -inf.
__device__ __forceinline__ uint32_t topk_key(float x) {
  if (x != x) x = -INFINITY;
  x = x + 0.0f;
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Maximum of a per-lane unsigned value over the wavefront (uniform result):
// a prefix maximum by DPP row shifts 1, 2, 4, 8 (lane 15 of each row then
// holds the row's maximum), the GFX9 row broadcasts carry it across rows to
// lane 63, one readlane.  Lanes without a DPP source read 0, the neutral value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0x111, 0xF>(v));   // row_shr:1
  v = max(v, dpp_u32<0x112, 0xF>(v));   // row_shr:2
  v = max(v, dpp_u32<0x114, 0xF>(v));   // row_shr:4
  v = max(v, dpp_u32<0x118, 0xF>(v));   // row_shr:8
  v = max(v, dpp_u32<0x142, 0xA>(v));   // row_bcast:15 into rows 1, 3
  v = max(v, dpp_u32<0x143, 0xC>(v));   // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

// One wavefront: the K largest of row[0..E) in descending order, ties to the
// lower index, and softmax weights over them.  Each of the K rounds takes the
// wave maximum of the untaken keys, then the lowest expert index holding it
// (a ballot per value slot, lowest slot first), and retires that one entry.
// NaN ranks as -inf.  Lane j < K receives pick j in (out_e, out_w); other
// lanes get (0, 0).  V = values per lane (E <= 64V); expert e sits in lane
// e % 64, slot e / 64.
template <int V>
__device__ __forceinline__ void topk_load(const float* row, int E, float (&v)[V]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane + kWave * i;
    v[i] = row[e < E ? e : E - 1];   // in bounds; lanes past E are masked in topk_rank
  }
}

template <int V>
__device__ __forceinline__ void topk_rank(float (&v)[V], int E, int K, int& out_e, float& out_w) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t key[V];
#pragma unroll
  for (int i = 0; i < V; ++i) key[i] = (lane + kWave * i < E) ? topk_key(v[i]) : 0u;   // 0 = retired / absent
  int my_e = 0;
  float my_l = 0.f;
  float l0 = 0.f;
  for (int j = 0; j < K; ++j) {
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < V; ++i) m = max(m, key[i]);
    const uint32_t best = wave_max_u32(m);
    int pick = E - 1;
    bool found = false;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(key[i] == best);
      if (!found && hit != 0) {
        pick = kWave * i + (int)__builtin_ctzll(hit);
        found = true;
      }
    }
    // the winner's value: floats ordered like their keys, so read it back from the key
    const uint32_t kb = (best & 0x80000000u) ? (best & 0x7FFFFFFFu) : ~best;
    const float val = best == 0u ? -INFINITY : __uint_as_float(kb);
    if (j == 0) l0 = val;
    if (lane == j) {
      my_e = pick;
      my_l = val;
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (lane + kWave * i == pick) key[i] = 0u;
  }
  const float ex = lane < K ? expf(my_l - l0) : 0.f;
  const float sum = wave_sum(ex);
  out_e = lane < K ? my_e : 0;
  out_w = lane < K ? ex / sum : 0.f;
}

template <int V>
__device__ __forceinline__ void wave_topk(const float* row, int E, int K, int& out_e, float& out_w) {
  float v[V];
  topk_load<V>(row, E, v);
  topk_rank<V>(v, E, K, out_e, out_w);
}

}  // namespace bdg
