// Paged GQA decode and verify with the fused append: the page classes of 1,
// 2, 4 and 8 tokens per page (kernel in gqa_decode_impl.h, dispatch in
// gqa_decode.hip).
#include "gqa_decode_impl.h"

namespace pd {

template hipError_t launch_gqa_class<1, true>(const GqaArgs&, bool, int, hipStream_t);
template hipError_t launch_gqa_class<2, true>(const GqaArgs&, bool, int, hipStream_t);
template hipError_t launch_gqa_class<4, true>(const GqaArgs&, bool, int, hipStream_t);
template hipError_t launch_gqa_class<8, true>(const GqaArgs&, bool, int, hipStream_t);

}  // namespace pd
