// Paged GQA decode and verify with the fused append: the classes of 16-token
// pages, of power-of-two pages of 32 tokens or more and of every other page
// size (kernel in gqa_decode_impl.h, dispatch in gqa_decode.hip).
#include "gqa_decode_impl.h"

namespace pd {

template hipError_t launch_gqa_class<0, true>(const GqaArgs&, bool, int, hipStream_t);
template hipError_t launch_gqa_class<16, true>(const GqaArgs&, bool, int, hipStream_t);
template hipError_t launch_gqa_class<32, true>(const GqaArgs&, bool, int, hipStream_t);

}  // namespace pd
