// Causal MLA verify: the class of page sizes that are not a power of two
// (3 tokens or more; kernel in mla_verify_impl.h, dispatch in mla_verify.hip).
#include "mla_verify_impl.h"

namespace pd {

template hipError_t launch_mla_class<0>(const MlaArgs&, int, hipStream_t);

}  // namespace pd
