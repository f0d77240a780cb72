// Batched (B > 1) union product on the matrix cores: placeholder until the
// MFMA kernel lands.
#include "internal.h"

namespace sl {

hipError_t launch_union_product(const sl_linear*, const UnionPlan&, const void*, int, bool, void*, sl_dtype,
                                hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace sl
