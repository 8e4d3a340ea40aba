// Causal MLA verify: launch dispatch over the page classes, and the class of
// power-of-two pages of 16 tokens or more.  The kernel is in mla_verify_impl.h;
// the classes of smaller pages are instantiated in mla_verify_small_pages.hip,
// the class of every other page size in mla_verify_general_pages.hip.
#include "mla_verify_impl.h"

namespace pd {

// instantiated in mla_verify_small_pages.hip and mla_verify_general_pages.hip
extern template hipError_t launch_mla_class<0>(const MlaArgs&, int, hipStream_t);
extern template hipError_t launch_mla_class<1>(const MlaArgs&, int, hipStream_t);
extern template hipError_t launch_mla_class<2>(const MlaArgs&, int, hipStream_t);
extern template hipError_t launch_mla_class<4>(const MlaArgs&, int, hipStream_t);
extern template hipError_t launch_mla_class<8>(const MlaArgs&, int, hipStream_t);

template hipError_t launch_mla_class<16>(const MlaArgs&, int, hipStream_t);

// Workgroups per launch: one per compute unit.  Queried once per device.
static int mla_grid_size() {
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

hipError_t launch_mla_verify(const MlaArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  const int n = mla_grid_size();
  if (n <= 0) return hipErrorInvalidDevice;
  if (a.P <= 0) return hipErrorInvalidValue;
  if ((a.P & (a.P - 1)) != 0) return a.P >= 3 ? launch_mla_class<0>(a, n, stream) : hipErrorInvalidValue;
  if ((1 << a.p_shift) != a.P) return hipErrorInvalidValue;
  switch (a.P) {
    case 1: return launch_mla_class<1>(a, n, stream);
    case 2: return launch_mla_class<2>(a, n, stream);
    case 4: return launch_mla_class<4>(a, n, stream);
    case 8: return launch_mla_class<8>(a, n, stream);
    default: return launch_mla_class<16>(a, n, stream);
  }
}

}  // namespace pd
