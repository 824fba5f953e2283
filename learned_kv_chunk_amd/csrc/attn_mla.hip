// attn_mla.hip -- absorbed multi-head latent attention variant (placeholder
// until the matrix-core kernel lands; shapes route to other kernels).
#include "lsa_internal.hpp"

namespace lsa {

bool mla_attn_supported(const lsa_shape&) { return false; }

hipError_t launch_attn_mla(const lsa_shape&, const AttnArgs&, int64_t, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace lsa
