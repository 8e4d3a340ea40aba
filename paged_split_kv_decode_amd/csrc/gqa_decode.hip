// Paged GQA split-KV decode: launch dispatch over the page classes, and the
// classes of 16-token pages and of power-of-two pages of 32 tokens or more.
// The kernel itself is in gqa_decode_impl.h; the classes of smaller pages are
// instantiated in gqa_decode_small_pages.hip, the class of every other page
// size in gqa_decode_general_pages.hip, the kernels with the fused append in
// gqa_append.hip and gqa_append_small_pages.hip.
#include "gqa_decode_impl.h"

namespace pd {

// instantiated in gqa_decode_small_pages.hip and gqa_decode_general_pages.hip
extern template hipError_t launch_gqa_class<0, false>(const GqaArgs&, bool, int, hipStream_t);
extern template hipError_t launch_gqa_class<1, false>(const GqaArgs&, bool, int, hipStream_t);
extern template hipError_t launch_gqa_class<2, false>(const GqaArgs&, bool, int, hipStream_t);
extern template hipError_t launch_gqa_class<4, false>(const GqaArgs&, bool, int, hipStream_t);
extern template hipError_t launch_gqa_class<8, false>(const GqaArgs&, bool, int, hipStream_t);

#define PD_APPEND_CLASS(P) \
  extern template hipError_t launch_gqa_class<P, true>(const GqaArgs&, bool, int, hipStream_t);
PD_APPEND_CLASS(0)
PD_APPEND_CLASS(1)
PD_APPEND_CLASS(2)
PD_APPEND_CLASS(4)
PD_APPEND_CLASS(8)
PD_APPEND_CLASS(16)
PD_APPEND_CLASS(32)
#undef PD_APPEND_CLASS

template hipError_t launch_gqa_class<16, false>(const GqaArgs&, bool, int, hipStream_t);
template hipError_t launch_gqa_class<32, false>(const GqaArgs&, bool, int, hipStream_t);

// Workgroups per launch: one per compute unit (a workgroup takes 160 KB of
// LDS, so one fits a CU).  Queried once per device.
static int grid_size() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

template <bool AP>
static hipError_t launch_classes(const GqaArgs& a, bool verify, int n, hipStream_t stream) {
  if ((a.P & (a.P - 1)) != 0) return a.P >= 3 ? launch_gqa_class<0, AP>(a, verify, n, stream)
                                               : hipErrorInvalidValue;
  if ((1 << a.p_shift) != a.P) return hipErrorInvalidValue;
  switch (a.P) {
    case 1: return launch_gqa_class<1, AP>(a, verify, n, stream);
    case 2: return launch_gqa_class<2, AP>(a, verify, n, stream);
    case 4: return launch_gqa_class<4, AP>(a, verify, n, stream);
    case 8: return launch_gqa_class<8, AP>(a, verify, n, stream);
    case 16: return launch_gqa_class<16, AP>(a, verify, n, stream);
    default: return launch_gqa_class<32, AP>(a, verify, n, stream);
  }
}

hipError_t launch_gqa_decode(const GqaArgs& a, hipStream_t stream) {
  const int n = grid_size();
  if (n <= 0) return hipErrorInvalidDevice;
  // the verify instantiations also take decode with more than 16 heads per kv head
  // (a slice of longer verify rows is verify whatever its length)
  const bool verify = a.qlen > 1 || a.q_req_rows > 1 || a.real_lens != nullptr ||
                      a.cu_q != nullptr || a.G > 16;
  if (a.P <= 0) return hipErrorInvalidValue;
  return a.kn != nullptr ? launch_classes<true>(a, verify, n, stream)
                         : launch_classes<false>(a, verify, n, stream);
}

}  // namespace pd
