// The fused per-layer decode kernel (moe_layer.hip) as the plan (moe.hip)
// sees it: its parameters, its compile-time variant, and its launcher.
#pragma once

#include <hip/hip_runtime.h>

#include "bdg_moe.hpp"

namespace bdg {

struct LayerParams {
  int H, I, E, K;
  RouteSrc rt;                // routing inputs of the layer
  int32_t* idx_out;           // [K] routing buffer, written by block 0
  float* w_out;
  int32_t* topk_trace;        // [K] or NULL
  float* wts_trace;
  const float* x;             // [H] layer input (fp32)
  LayerDev L;
  QGeom g_gu, g_dn;           // reductions over H (gate_up) and I (down)
  float* hbuf;                // [K * I] h, exchanged between blocks through memory
  unsigned* bar;              // grid barrier: [0] arrivals, [32] generation
  unsigned* fault;            // set to 1 when a bounded wait gives up
  int wait_polls;             // polls before a wait gives up
  int dn_blocks;              // blocks [0, dn_blocks) own B down rows each
  int B;
  DownOut o;                  // combine, residual, outputs, next layer's router slice
  uint64_t* stamps;           // NULL, or [gridDim][kLayerStamps] 100 MHz clock stamps (timeline)
};

// Phase stamps of the fused kernel's timeline mode (moe_expert_decode_timeline),
// taken by lane 0 of the wave named, per block.
enum LayerStamp {
  kStStart = 0,        // wave 7: first instruction
  kStRouted = 1,       // wave 7: experts selected
  kStGuIssued = 2,     // wave 7: gate_up loads issued
  kStDnIssued = 3,     // wave 0: down codes issued into LDS
  kStGuDone = 4,       // wave 7: every wave's h in LDS
  kStHStored = 5,      // wave 7: h stores complete (arrival)
  kStBarrier = 6,      // wave 7: barrier passed
  kStHStaged = 7,      // wave 0: whole h in LDS
  kStDnDone = 8,       // wave 0: down rows computed
  kStEnd = 9,          // wave 0: epilogue done
  kLayerStamps = 16
};

// Shape facts that size the kernel's LDS.
struct LayerShape {
  QGeom g_gu, g_dn;
  int K, E, log2T, B;
};

// Compile-time variant: weight format, gate_up slots, pairs per wave, top-k
// values per lane, down lanes / slots per row, down row groups per loading
// wave, h values per thread in the exchange.
struct LayerConfig {
  int fmt, sg, np, v, ld, sd, ng, nhl;
};

int layer_fused_lds_bytes(const LayerShape& s, int np, int ng, int sd);
const void* layer_fused_kernel(const LayerConfig& c);   // NULL: no such variant
// ev_start / ev_stop (or null): events that take the dispatch's own start and
// end times.
int launch_layer_fused(const LayerConfig& c, const LayerParams& lp, int nblk, size_t lds, hipStream_t s,
                       hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
int layer_threads();
int layer_dn_load_waves();

}  // namespace bdg
