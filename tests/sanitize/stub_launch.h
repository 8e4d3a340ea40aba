// Launch records of the stand-in kernel launchers (stub_launch.cpp).
#pragma once

#include "../../paged_split_kv_decode_amd/csrc/kernels.h"

namespace pd_stub {

struct Record {
  pd::GqaArgs gqa{};
  pd::MlaArgs mla{};
  pd::MergeArgs merge{};
  pd::AppendArgs append{};
  int n_gqa = 0, n_mla = 0, n_merge = 0, n_append = 0;
  // (qlen, t_off, len_sub, q_req_rows) of GQA launches n_gqa - 1 ... (mod 16)
  int gqa_slice[16][4] = {};
};

extern Record g_rec;

}  // namespace pd_stub
