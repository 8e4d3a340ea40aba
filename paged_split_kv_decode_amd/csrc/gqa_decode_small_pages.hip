// Paged GQA split-KV decode: the page classes of 1, 2, 4 and 8 tokens per
// page (kernel in gqa_decode_impl.h, dispatch in gqa_decode.hip).
#include "gqa_decode_impl.h"

namespace pd {

template hipError_t launch_gqa_class<1, false>(const GqaArgs&, bool, int, hipStream_t);
template hipError_t launch_gqa_class<2, false>(const GqaArgs&, bool, int, hipStream_t);
template hipError_t launch_gqa_class<4, false>(const GqaArgs&, bool, int, hipStream_t);
template hipError_t launch_gqa_class<8, false>(const GqaArgs&, bool, int, hipStream_t);

}  // namespace pd
