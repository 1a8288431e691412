// Expert kernels for NVFP4 routed weights (shared expert: NVFP4, BF16).
#include "grouped.hpp"

namespace moe {

hipError_t launch_experts_nvfp4(const ExpertArgs& gu, int gu_grid, size_t gu_lds,
                             const ExpertArgs& dn, int dn_grid, size_t dn_lds, int sf,
                             hipStream_t s) {
  if (sf == W_NVFP4) return launch_experts_t<W_NVFP4, W_NVFP4>(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, s);
  if (sf == W_BF16) return launch_experts_t<W_NVFP4, W_BF16>(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
