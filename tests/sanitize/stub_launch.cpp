// Stand-ins for the kernel launchers, for a CPU build of the C ABI's host
// half under AddressSanitizer / UndefinedBehaviorSanitizer: each records
// the arguments of its last call instead of launching anything.
#include "../../paged_split_kv_decode_amd/csrc/kernels.h"

#include "stub_launch.h"

namespace pd_stub {
Record g_rec;
}  // namespace pd_stub

namespace pd {

hipError_t launch_gqa_decode(const GqaArgs& a, hipStream_t) {
  auto& r = pd_stub::g_rec;
  r.gqa = a;
  int* sl = r.gqa_slice[r.n_gqa % 16];
  sl[0] = a.qlen;
  sl[1] = a.t_off;
  sl[2] = a.len_sub;
  sl[3] = a.q_req_rows;
  ++r.n_gqa;
  return hipSuccess;
}

hipError_t launch_mla_verify(const MlaArgs& a, hipStream_t) {
  pd_stub::g_rec.mla = a;
  ++pd_stub::g_rec.n_mla;
  return hipSuccess;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t) {
  pd_stub::g_rec.merge = a;
  ++pd_stub::g_rec.n_merge;
  return hipSuccess;
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t) {
  pd_stub::g_rec.append = a;
  ++pd_stub::g_rec.n_append;
  return hipSuccess;
}

}  // namespace pd
