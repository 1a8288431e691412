// Expert kernels for BF16 routed weights (shared expert: BF16).
#include "grouped.hpp"

namespace moe {

hipError_t launch_experts_bf16(const ExpertArgs& gu, int gu_grid, size_t gu_lds,
                             const ExpertArgs& dn, int dn_grid, size_t dn_lds, int sf,
                             hipStream_t s) {
  if (sf == W_BF16) return launch_experts_t<W_BF16, W_BF16>(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
