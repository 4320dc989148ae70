// Host-side helpers of libbdg: argument checks and launch error mapping.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bdg.h"

namespace bdg {

inline int hip_status(hipError_t e) { return e == hipSuccess ? BDG_OK : BDG_E_HIP; }

inline int launch_status() { return hip_status(hipGetLastError()); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Shape/format checks shared by every entry point that reads a bdg_qmat.
inline int check_qmat(const bdg_qmat* w, bool need_expert_strides) {
  if (!w || !w->codes || !w->scales) return BDG_E_INVALID;
  if (w->n <= 0 || w->k <= 0 || (w->k % 32) != 0) return BDG_E_INVALID;
  if (w->k > BDG_MAX_K) return BDG_E_UNSUPPORTED;
  if (w->fmt == BDG_FMT_MXFP4) {
    if (w->group != 32) return BDG_E_INVALID;
  } else if (w->fmt == BDG_FMT_INT4G) {
    if (w->group <= 0 || (w->group % 32) != 0 || (w->k % w->group) != 0) return BDG_E_INVALID;
    if (!w->zeros) return BDG_E_INVALID;
    if ((reinterpret_cast<uintptr_t>(w->scales) & 1u) != 0) return BDG_E_ALIGN;
  } else {
    return BDG_E_INVALID;
  }
  if (!aligned16(w->codes)) return BDG_E_ALIGN;
  // the kernels address one matrix (one expert) with 32-bit byte offsets
  if (w->n > (int64_t)0xFFFFFFFF / (w->k / 2)) return BDG_E_UNSUPPORTED;
  if (need_expert_strides) {
    if (w->expert_stride_codes < 0 || (w->expert_stride_codes & 15) != 0) return BDG_E_ALIGN;
    if (w->expert_stride_scales < 0 || w->expert_stride_zeros < 0) return BDG_E_INVALID;
    if (w->fmt == BDG_FMT_INT4G && (w->expert_stride_scales & 1) != 0) return BDG_E_ALIGN;
  }
  return BDG_OK;
}

// Lanes per row L and slots per lane S for a row of `chunks` 16-byte chunks:
// the smallest L in {8, 16, 32, 64} with S = ceil(chunks / L) <= 3, else
// L = 64 with S <= 4.  Returns false if no variant covers the row.
inline bool pick_lanes(int chunks, int* L, int* S) {
  const int ls[4] = {8, 16, 32, 64};
  for (int i = 0; i < 4; ++i) {
    const int s = (chunks + ls[i] - 1) / ls[i];
    if (s <= 3) { *L = ls[i]; *S = s; return true; }
  }
  const int s = (chunks + 63) / 64;
  if (s <= 4) { *L = 64; *S = s; return true; }
  return false;
}

}  // namespace bdg
