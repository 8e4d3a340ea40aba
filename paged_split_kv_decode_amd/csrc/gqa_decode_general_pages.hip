// Paged GQA split-KV decode: the class of page sizes that are not a power of
// two (3 tokens or more; kernel in gqa_decode_impl.h, dispatch in
// gqa_decode.hip).
#include "gqa_decode_impl.h"

namespace pd {

template hipError_t launch_gqa_class<0, false>(const GqaArgs&, bool, int, hipStream_t);

}  // namespace pd
