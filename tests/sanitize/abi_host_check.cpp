// Host half of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Calls every entry point of include/paged_decode.h with fake, never
// dereferenced device addresses: refused calls must return the documented
// status before any HIP call; accepted calls reach the stand-in launchers
// (stub_launch.cpp), whose recorded arguments are checked.  Sizes at the
// edges of the int32 / int64 ranges exercise the overflow guards, where the
// sanitizers would report any signed overflow or out-of-bounds access in
// the host code.  Prints "N checks passed" and exits 0, or lists failures.
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "../../include/paged_decode.h"
#include "stub_launch.h"

namespace {

int g_checks = 0, g_failures = 0;

void expect(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    ++g_failures;
    std::fprintf(stderr, "FAIL line %d: %s\n", line, what);
  }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

void* const kFake = reinterpret_cast<void*>(uintptr_t{0x100000});
float* const kFakeF = reinterpret_cast<float*>(uintptr_t{0x100000});
const int32_t* const kFakeI = reinterpret_cast<const int32_t*>(uintptr_t{0x100000});

// paged_verify_gqa arguments with defaults of a valid decode call.
struct Gqa {
  const void* q = kFake;
  int64_t q_sr = 64 * 128, q_sh = 128;
  const void* kv = kFake;
  int32_t dtype = PD_KV_BF16;
  const float* ks = nullptr;
  const float* vs = nullptr;
  int32_t per_head = 0;
  int64_t kv_sp = 8 * 16 * 256, kv_sh = 16 * 256;
  int32_t num_pages = 10;
  const int32_t* bt = kFakeI;
  int64_t bt_sb = 4;
  int32_t max_blocks = 4;
  const int32_t* sl = kFakeI;
  const int32_t* real = nullptr;
  int32_t qlen = 1;
  const float* sinks = nullptr;
  int32_t window = 0;
  float scale = 0.088f;
  int32_t B = 2, Hq = 64, Hkv = 8, D = 128, P = 16, S = 1;
  float* ws = nullptr;
  size_t wsb = 0;
  void* out = kFake;
  int64_t o_sr = 64 * 128, o_sh = 128;
  float* lse = nullptr;
  int64_t lse_sr = 64;

  int verify() const {
    return paged_verify_gqa(q, q_sr, q_sh, kv, dtype, ks, vs, per_head, kv_sp, kv_sh, num_pages,
                            bt, bt_sb, max_blocks, sl, real, qlen, sinks, window, scale, B, Hq,
                            Hkv, D, P, S, ws, wsb, out, o_sr, o_sh, lse, lse_sr, nullptr);
  }
  int decode() const {
    return paged_decode_gqa(q, q_sr, q_sh, kv, kv_sp, kv_sh, num_pages, bt, bt_sb, max_blocks, sl,
                            sinks, window, scale, B, Hq, Hkv, D, P, S, ws, wsb, out, o_sr, o_sh,
                            lse, lse_sr, nullptr);
  }
  int varlen(const int32_t* cu, int32_t total_rows) const {
    return paged_verify_gqa_varlen(q, q_sr, q_sh, kv, dtype, ks, vs, per_head, kv_sp, kv_sh,
                                   num_pages, bt, bt_sb, max_blocks, sl, real, cu, qlen,
                                   total_rows, sinks, window, scale, B, Hq, Hkv, D, P, S, ws, wsb,
                                   out, o_sr, o_sh, lse, lse_sr, nullptr);
  }
  int partials(const int32_t* cu, int32_t total_rows) const {
    return paged_verify_gqa_partials(q, q_sr, q_sh, kv, dtype, ks, vs, per_head, kv_sp, kv_sh,
                                     num_pages, bt, bt_sb, max_blocks, sl, real, cu, qlen,
                                     total_rows, window, scale, B, Hq, Hkv, D, P, S, ws, wsb,
                                     nullptr);
  }
  int append(const void* kn, int64_t kn_sr, int64_t kn_sh, const void* vn, int64_t vn_sr,
             int64_t vn_sh) const {
    return paged_verify_gqa_append(q, q_sr, q_sh, const_cast<void*>(kv), dtype, ks, vs, per_head,
                                   kv_sp, kv_sh, num_pages, bt, bt_sb, max_blocks, sl, real, qlen,
                                   kn, kn_sr, kn_sh, vn, vn_sr, vn_sh, sinks, window, scale, B, Hq,
                                   Hkv, D, P, S, ws, wsb, out, o_sr, o_sh, lse, lse_sr, nullptr);
  }
  int noalloc() const {
    return paged_verify_gqa_noalloc(q, q_sr, q_sh, kv, dtype, ks, vs, per_head, kv_sp, kv_sh,
                                    num_pages, bt, bt_sb, max_blocks, sl, real, qlen, sinks,
                                    window, scale, B, Hq, Hkv, D, P, S, out, o_sr, o_sh, lse,
                                    lse_sr, nullptr);
  }
};

struct Mla {
  const void* q = kFake;
  int64_t q_sr = 128 * 576, q_sh = 576;
  const void* kv = kFake;
  int32_t dtype = PD_KV_BF16;
  int64_t kv_sp = 16 * 576, kv_st = 576;
  int32_t num_pages = 10;
  const float* ks = nullptr;
  const int32_t* bt = kFakeI;
  int64_t bt_sb = 4;
  int32_t max_blocks = 4;
  const int32_t* sl = kFakeI;
  const int32_t* real = nullptr;
  int32_t qlen = 4;
  float scale = 0.072f;
  int32_t B = 2, H = 128, Lk = 576, Lv = 512, P = 16, S = 1;
  float* ws = nullptr;
  size_t wsb = 0;
  void* out = kFake;
  int64_t o_sr = 128 * 512, o_sh = 512;
  float* lse = nullptr;
  int64_t lse_sr = 128;

  int call() const {
    return paged_verify_mla(q, q_sr, q_sh, kv, dtype, kv_sp, kv_st, num_pages, ks, bt, bt_sb,
                            max_blocks, sl, real, qlen, scale, B, H, Lk, Lv, P, S, ws, wsb, out,
                            o_sr, o_sh, lse, lse_sr, nullptr);
  }
  int partials() const {
    return paged_verify_mla_partials(q, q_sr, q_sh, kv, dtype, kv_sp, kv_st, num_pages, ks, bt,
                                     bt_sb, max_blocks, sl, real, qlen, scale, B, H, Lk, Lv, P, S,
                                     ws, wsb, nullptr);
  }
};

void check_split_caps() {
  // the page's rule, hand-evaluated values
  EXPECT(pd_split_rule(70, 3, 1, 1, 1, 256, 1.f, 64, 8, 0) == 2);
  EXPECT(pd_split_rule(100000, 300, 1, 1, 1, 256, 1.f, 64, 8, 0) == 4);
  EXPECT(pd_split_rule(16384, 4, 4, 128, 64, 256, 1.f, 64, 16, 0) == 8);
  // the tuned policies at the configurations' sizes
  EXPECT(pd_gqa_split_cap(64, 8, 8192, 0, 256) == 8);
  EXPECT(pd_gqa_split_cap(64, 8, 32768, 128, 256) == 1);
  EXPECT(pd_gqa_split_cap(256, 8, 131072, 0, 256) == 64);
  EXPECT(pd_mla_split_cap(32, 4, 128, 16384, 256) == 8);
  // extreme sizes: a cap in range, no overflow in the cost arithmetic
  const int32_t big = INT32_MAX;
  const int32_t c1 = pd_split_rule(big, big, big, big, 1, 256, 1.f, 1, 64, 1);
  EXPECT(c1 >= 1 && c1 <= 64);
  const int32_t c2 = pd_gqa_split_cap(big, 65535, big, big, 256);
  EXPECT(c2 >= 1 && c2 <= 64);
  const int32_t c3 = pd_mla_split_cap(big, big, big, big, 256);
  EXPECT(c3 >= 1 && c3 <= 16);
  EXPECT(pd_split_rule(0, 0, 1, 1, 1, 256, 1.f, 0, 1, 0) == 1);
  // refusals before any device query
  EXPECT(pd_split_rule(-1, 1, 1, 1, 1, 256, 1.f, 64, 8, 0) == PD_ERR_INVALID);
  EXPECT(pd_split_rule(10, 1, 1, 1, 1, 256, NAN, 64, 8, 0) == PD_ERR_INVALID);
  EXPECT(pd_gqa_split_cap(-1, 8, 10, 0, 256) == PD_ERR_INVALID);
  EXPECT(pd_mla_split_cap(1, 0, 8, 10, 256) == PD_ERR_INVALID);
  EXPECT(num_kv_splits_cap(10, 1, 1, 12, 8, 128, 0, -1) == PD_ERR_INVALID);
  EXPECT(num_kv_splits_cap(10, 1, 1, 8, 8, 64, 0, -1) == PD_ERR_UNSUPPORTED);
  // a device query: a cap when a device is present, PD_ERR_HIP when not
  const int32_t c4 = num_kv_splits_cap(8192, 64, 1, 64, 8, 128, 0, -1);
  EXPECT(c4 == PD_ERR_HIP || (c4 >= 1 && c4 <= 64));
  EXPECT(pd_workspace_bytes(big, big, big, big) > 0);   // size_t arithmetic, no overflow trap
  EXPECT(pd_workspace_bytes(64, 64, 1, 128) == 0);
}

void check_gqa() {
  auto& r = pd_stub::g_rec;
  Gqa g;
  int n = r.n_gqa;
  EXPECT(g.decode() == PD_OK && r.n_gqa == n + 1);
  EXPECT(r.gqa.G == 8 && r.gqa.P == 16 && r.gqa.p_shift == 4 && r.gqa.S == 1 && r.gqa.qlen == 1);
  EXPECT(std::fabs(r.gqa.scale_log2 - 0.088f * 1.44269504f) < 1e-6f);
  EXPECT(r.gqa.q_sb == 64 * 128 && r.gqa.kv_sp == 8 * 16 * 256 && r.gqa.total_rows == 2);
  // splits: kernel and merge
  Gqa s = g;
  s.S = 4;
  s.ws = kFakeF;
  s.wsb = pd_workspace_bytes(2, 64, 4, 128);
  const int nm = r.n_merge;
  EXPECT(s.decode() == PD_OK && r.n_merge == nm + 1);
  EXPECT(r.merge.S == 4 && r.merge.rows == 2 && r.merge.H == 64 && r.merge.Dv == 128);
  s.wsb -= 4;
  EXPECT(s.decode() == PD_ERR_WORKSPACE);
  // any page size
  Gqa p = g;
  p.P = 12;
  EXPECT(p.decode() == PD_OK && r.gqa.P == 12 && r.gqa.p_shift == 0);
  p.P = 65536;
  p.max_blocks = 4;
  EXPECT(p.decode() == PD_OK && r.gqa.p_shift == 16);
  p.P = 65537;
  EXPECT(p.decode() == PD_ERR_UNSUPPORTED);
  p.P = 0;
  EXPECT(p.decode() == PD_ERR_INVALID);
  // columns: qlen * G up to 64 in one launch
  Gqa v = g;
  v.qlen = 8;
  v.q_sr = 64 * 128;
  n = r.n_gqa;
  EXPECT(v.verify() == PD_OK && r.gqa.qlen == 8 && r.gqa.total_rows == 16 && r.n_gqa == n + 1 &&
         r.gqa.q_req_rows == 8 && r.gqa.t_off == 0 && r.gqa.len_sub == 0);
  // longer rows: equal slices of whole tokens in token order, each with the
  // tokens after it taken off the causal limit (G = 8: 8 tokens per launch)
  v.qlen = 9;
  n = r.n_gqa;
  EXPECT(v.verify() == PD_OK && r.n_gqa == n + 2);
  {
    const int* s0 = r.gqa_slice[n % 16];
    const int* s1 = r.gqa_slice[(n + 1) % 16];
    EXPECT(s0[0] == 5 && s0[1] == 0 && s0[2] == 4 && s0[3] == 9);
    EXPECT(s1[0] == 4 && s1[1] == 5 && s1[2] == 0 && s1[3] == 9);
  }
  v.qlen = 20;
  v.S = 4;
  v.ws = kFakeF;
  v.wsb = pd_workspace_bytes(2 * 20, 64, 4, 128);
  n = r.n_gqa;
  int nm3 = r.n_merge;
  EXPECT(v.verify() == PD_OK && r.n_gqa == n + 3 && r.n_merge == nm3 + 1 && r.merge.rows == 40);
  {
    int t = 0;
    for (int i = 0; i < 3; ++i) {
      const int* si = r.gqa_slice[(n + i) % 16];
      EXPECT(si[0] == (i < 2 ? 7 : 6) && si[1] == t && si[2] == 20 - t - si[0] && si[3] == 20);
      t += si[0];
    }
    EXPECT(t == 20);
  }
  // G = 64: one token per launch
  Gqa w = g;
  w.Hq = 8 * 64;
  w.qlen = 3;
  w.q_sr = 8 * 64 * 128;
  w.o_sr = 8 * 64 * 128;
  n = r.n_gqa;
  EXPECT(w.verify() == PD_OK && r.n_gqa == n + 3 && r.gqa.qlen == 1 && r.gqa.t_off == 2 &&
         r.gqa.len_sub == 0);
  // variable rows are never sliced
  v = g;
  v.qlen = 9;
  EXPECT(v.varlen(kFakeI, 18) == PD_ERR_UNSUPPORTED);
  Gqa h = g;
  h.Hq = 8 * 64;
  EXPECT(h.decode() == PD_OK && r.gqa.G == 64);
  h.Hq = 8 * 65;
  EXPECT(h.decode() == PD_ERR_UNSUPPORTED);
  // refusals
  Gqa b = g;
  b.q = nullptr;
  EXPECT(b.decode() == PD_ERR_INVALID);
  b = g;
  b.Hq = 60;
  EXPECT(b.decode() == PD_ERR_INVALID);
  b = g;
  b.scale = -1.f;
  EXPECT(b.decode() == PD_ERR_INVALID);
  b.scale = INFINITY;
  EXPECT(b.decode() == PD_ERR_INVALID);
  b = g;
  b.q = static_cast<const char*>(kFake) + 8;
  EXPECT(b.decode() == PD_ERR_ALIGN);
  b = g;
  b.dtype = 7;
  EXPECT(b.verify() == PD_ERR_INVALID);
  b = g;
  b.dtype = PD_KV_FP8_E4M3FN;
  b.kv_sh = 16 * 256 + 8;
  EXPECT(b.verify() == PD_ERR_ALIGN);
  // int32 / int64 edges: strides and table capacity that do not fit the kernel
  b = g;
  b.q_sr = int64_t{1} << 31;
  EXPECT(b.decode() == PD_ERR_UNSUPPORTED);
  b = g;
  b.kv_sp = INT64_MAX - 7;
  EXPECT(b.decode() == PD_ERR_UNSUPPORTED);
  b = g;
  b.max_blocks = INT32_MAX;
  b.P = 65536;
  EXPECT(b.decode() == PD_ERR_UNSUPPORTED);
  b = g;
  b.B = 65535;
  b.Hkv = 8;
  b.max_blocks = 1 << 20;
  b.P = 512;
  EXPECT(b.decode() == PD_ERR_UNSUPPORTED);
  b = g;
  b.qlen = 2;
  b.q_sr = INT32_MAX - 7;
  EXPECT(b.verify() == PD_ERR_UNSUPPORTED);
  // an empty batch enqueues nothing
  n = r.n_gqa;
  b = g;
  b.B = 0;
  b.q = nullptr;
  b.kv = nullptr;
  EXPECT(b.decode() == PD_OK && r.n_gqa == n);
  // variable query length
  EXPECT(g.varlen(nullptr, 3) == PD_ERR_INVALID);
  EXPECT(g.varlen(kFakeI, -1) == PD_ERR_INVALID);
  n = r.n_gqa;
  EXPECT(g.varlen(kFakeI, 0) == PD_OK && r.n_gqa == n);
  EXPECT(g.varlen(kFakeI, 3) == PD_OK && r.gqa.cu_q == kFakeI && r.gqa.total_rows == 3);
  // partials only
  Gqa pp = g;
  pp.S = 3;
  pp.ws = kFakeF;
  pp.wsb = pd_workspace_bytes(2, 64, 3, 128);
  n = r.n_gqa;
  const int nm2 = r.n_merge;
  EXPECT(pp.partials(nullptr, 0) == PD_OK && r.n_gqa == n + 1 && r.n_merge == nm2);
  EXPECT(r.gqa.partials == 1);
  pp.S = 1;
  pp.wsb = 2 * 64 * 129 * 4 - 4;
  EXPECT(pp.partials(nullptr, 0) == PD_ERR_WORKSPACE);
  // allocation-free entry: checks first; then a HIP lookup (no device: an error)
  Gqa na = g;
  na.Hq = 60;
  EXPECT(na.noalloc() == PD_ERR_INVALID);
  na = g;
  na.B = 64;
  na.qlen = 2;
  na.S = 16;
  EXPECT(na.noalloc() == PD_ERR_WORKSPACE);
  na = g;
  na.S = 2;
  const int st = na.noalloc();
  EXPECT(st == PD_OK || st == PD_ERR_HIP);

  // fused append: the sources reach the launch as byte addresses and strides
  const char* kn = static_cast<const char*>(kFake);
  int n_app = r.n_gqa;
  EXPECT(g.append(kn, 8 * 128, 128, kn + 4096, 8 * 128, 128) == PD_OK && r.n_gqa == n_app + 1);
  EXPECT(r.gqa.kn == kn && r.gqa.vn == kn + 4096 && r.gqa.kn_srow == 8 * 128 * 2 &&
         r.gqa.kn_sh == 128 * 2 && r.gqa.vn_srow == 8 * 128 * 2 && r.gqa.vn_sh == 128 * 2);
  EXPECT(g.append(nullptr, 8 * 128, 128, kn, 8 * 128, 128) == PD_ERR_INVALID);
  EXPECT(g.append(kn + 8, 8 * 128, 128, kn, 8 * 128, 128) == PD_ERR_ALIGN);
  EXPECT(g.append(kn, (int64_t)INT32_MAX - 7, 128, kn, 8 * 128, 128) == PD_OK);
  EXPECT(g.append(kn, (int64_t)INT32_MAX + 1, 128, kn, 8 * 128, 128) == PD_ERR_UNSUPPORTED);
  // the plain calls launch with no append source
  EXPECT(g.verify() == PD_OK && r.gqa.kn == nullptr);
}

void check_mla() {
  auto& r = pd_stub::g_rec;
  Mla m;
  int n = r.n_mla;
  EXPECT(m.call() == PD_OK && r.n_mla == n + 1);
  EXPECT(r.mla.H == 128 && r.mla.qlen == 4 && r.mla.p_shift == 4 && r.mla.kv_fp8 == 0);
  Mla s = m;
  s.S = 3;
  s.ws = kFakeF;
  s.wsb = pd_workspace_bytes(8, 128, 3, 512);
  const int nm = r.n_merge;
  EXPECT(s.call() == PD_OK && r.n_merge == nm + 1 && r.merge.Dv == 512 && r.merge.rows == 8);
  s.wsb -= 4;
  EXPECT(s.call() == PD_ERR_WORKSPACE);
  Mla p = m;
  p.P = 24;
  EXPECT(p.call() == PD_OK && r.mla.P == 24 && r.mla.p_shift == 0);
  p = m;
  p.H = 7;
  p.qlen = 1;
  EXPECT(p.call() == PD_OK && r.mla.H == 7);
  p = m;
  p.Lk = 512;
  EXPECT(p.call() == PD_ERR_UNSUPPORTED);
  p = m;
  p.dtype = PD_KV_FP8_E4M3FN;
  p.kv_st = 576 + 8;
  EXPECT(p.call() == PD_ERR_ALIGN);
  p = m;
  p.qlen = 0;
  EXPECT(p.call() == PD_ERR_INVALID);
  p = m;
  p.max_blocks = INT32_MAX;
  EXPECT(p.call() == PD_ERR_UNSUPPORTED);
  p = m;
  p.B = INT32_MAX;
  p.qlen = 2;
  EXPECT(p.call() == PD_ERR_UNSUPPORTED);
  Mla pp = m;
  pp.ws = kFakeF;
  pp.wsb = 8 * 128 * 513 * 4;
  EXPECT(pp.partials() == PD_OK && r.mla.partials == 1);
}

void check_merge_and_append() {
  auto& r = pd_stub::g_rec;
  int n = r.n_merge;
  EXPECT(merge_splits(kFakeF, 4, 8, 2, 128, nullptr, kFake, 1024, 128, nullptr, 8, nullptr) ==
             PD_OK &&
         r.n_merge == n + 1);
  EXPECT(merge_splits(kFakeF, 4, 8, 2, 96, nullptr, kFake, 1024, 128, nullptr, 8, nullptr) ==
         PD_ERR_UNSUPPORTED);
  EXPECT(merge_splits(nullptr, 4, 8, 2, 128, nullptr, kFake, 1024, 128, nullptr, 8, nullptr) ==
         PD_ERR_INVALID);
  EXPECT(merge_splits(kFakeF, 4, 8, 2, 128, nullptr, static_cast<char*>(kFake) + 2, 1024, 128,
                      nullptr, 8, nullptr) == PD_ERR_ALIGN);
  n = r.n_merge;
  EXPECT(merge_splits(kFakeF, 0, 8, 2, 128, nullptr, kFake, 1024, 128, nullptr, 8, nullptr) ==
             PD_OK &&
         r.n_merge == n);
  n = r.n_append;
  EXPECT(paged_kv_append(kFake, 8 * 128, 128, 128, kFake, 8 * 128, 128, 128, 2, kFake,
                         8 * 16 * 256, 16 * 256, 256, 10, kFakeI, 4, 4, kFakeI, 1, 2, 8, 16,
                         nullptr) == PD_OK &&
         r.n_append == n + 1);
  EXPECT(r.append.c0 == 16 && r.append.c1 == 16 && r.append.c_st == 512);
  EXPECT(paged_kv_append(kFake, 8 * 128, 128, 128, kFake, 8 * 128, 128, 128, 3, kFake,
                         8 * 16 * 256, 16 * 256, 256, 10, kFakeI, 4, 4, kFakeI, 1, 2, 8, 16,
                         nullptr) == PD_ERR_INVALID);
  EXPECT(paged_kv_append(kFake, 8 * 128, 128, 200, kFake, 8 * 128, 128, 128, 2, kFake,
                         8 * 16 * 256, 16 * 256, 256, 10, kFakeI, 4, 4, kFakeI, 1, 2, 8, 16,
                         nullptr) == PD_ERR_INVALID);
  EXPECT(paged_kv_append(kFake, 8 * 128, 128, 128, kFake, 8 * 128, 128, 128, 2,
                         static_cast<char*>(kFake) + 4, 8 * 16 * 256, 16 * 256, 256, 10, kFakeI,
                         4, 4, kFakeI, 1, 2, 8, 16, nullptr) == PD_ERR_ALIGN);
  EXPECT(pd_stream_read_probe(nullptr, 1 << 20, reinterpret_cast<uint32_t*>(kFake), 4,
                              nullptr) == PD_ERR_INVALID);
  EXPECT(pd_stream_read_probe(static_cast<char*>(kFake) + 4, 1 << 20,
                              reinterpret_cast<uint32_t*>(kFake), 4,
                              nullptr) == PD_ERR_ALIGN);
  for (int s = -6; s <= 1; ++s) EXPECT(pd_status_string(s) != nullptr);
}

}  // namespace

int main() {
  check_split_caps();
  check_gqa();
  check_mla();
  check_merge_and_append();
  if (g_failures) {
    std::fprintf(stderr, "%d of %d checks failed\n", g_failures, g_checks);
    return 1;
  }
  std::printf("%d checks passed\n", g_checks);
  return 0;
}
