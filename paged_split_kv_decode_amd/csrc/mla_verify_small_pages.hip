// Causal MLA verify: the page classes of 1, 2, 4 and 8 tokens per page
// (kernel in mla_verify_impl.h, dispatch in mla_verify.hip).
#include "mla_verify_impl.h"

namespace pd {

template hipError_t launch_mla_class<1>(const MlaArgs&, int, hipStream_t);
template hipError_t launch_mla_class<2>(const MlaArgs&, int, hipStream_t);
template hipError_t launch_mla_class<4>(const MlaArgs&, int, hipStream_t);
template hipError_t launch_mla_class<8>(const MlaArgs&, int, hipStream_t);

}  // namespace pd
