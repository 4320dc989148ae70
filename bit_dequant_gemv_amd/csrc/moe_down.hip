// The per-token down kernel's shape variants (up to 64 experts: 8 router
// rows of the next layer per wave).
#include "bdg_moe_down.hpp"

namespace bdg {

int launch_down_kernel(const DownParams& dp, int fmt, int L, int S, int NR, int HV, dim3 grid, size_t lds,
                       hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  return launch_down_variant<kDnRouterPerWave>(dp, fmt, L, S, NR, HV, grid, lds, s, ev_start, ev_stop);
}

}  // namespace bdg
