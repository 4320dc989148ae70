// The grouped expert products of steps of M > 1 tokens on the matrix cores
// (moe_mfma.hip) as the plan (moe.hip) sees them.
#pragma once

#include <hip/hip_runtime.h>

#include "bdg_moe.hpp"

namespace bdg {

constexpr int kMfmaTT = 8;                  // picks per chunk (16 token rows: hi and lo part of each)
constexpr int kMfmaChunkInts = 2 + kMfmaTT;
constexpr int kMfmaRows = 16;               // weight rows per matrix-core tile

struct MfmaParams {
  // routing (gate_up kernel), as group_route reads it
  int M, H, I, E, K;
  int routed;
  const int32_t* idx_in;
  const float* w_in;
  const float* part;          // [M][E + 1][pstride] router sums, one slice (route kernel)
  int pstride;
  int norm;
  float eps;
  int32_t* idx_out;           // [M][K]
  float* w_out;
  int32_t* topk_trace;        // [M][K] or NULL
  float* wts_trace;
  LayerDev L;
  // operands
  const uint16_t* xh;         // [M][H] bf16 high part of the layer input (x times the RMSNorm factor)
  const uint16_t* xl;         // [M][H] bf16 low part: x r - xh
  uint16_t* hh;               // [M * K][I] bf16 high part of h, row = pick t*K + j
  uint16_t* hl;               // [M * K][I] bf16 low part
  const uint16_t* zeros;      // >= max(H, I) zero bf16: the operand rows of absent picks
  int32_t* table;             // chunk table: gate_up writes it, down reads it
  float* dout;                // [M * K][H] down output per pick
};

// ev_start / ev_stop (or null): events that take the dispatch's own start and
// end times.
int launch_gu_mfma(const MfmaParams& p, int V, int nblk, hipStream_t s, hipEvent_t ev_start = nullptr,
                   hipEvent_t ev_stop = nullptr);
int launch_dn_mfma(const MfmaParams& p, int nblk, hipStream_t s, hipEvent_t ev_start = nullptr,
                   hipEvent_t ev_stop = nullptr);
size_t mfma_gu_lds_bytes();
size_t mfma_dn_lds_bytes();
const void* mfma_gu_kernel(int V);
const void* mfma_dn_kernel();

}  // namespace bdg
