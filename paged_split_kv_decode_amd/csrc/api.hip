// C ABI of the library: argument checks (host only, before any HIP call),
// the static split cap, workspace sizing and dispatch to the kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/paged_decode.h"
#include "kernels.h"

namespace {

constexpr float kLog2eHost = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Page sizes with a kernel: every size from 1 to 65536 tokens.
constexpr int32_t kMaxPageSize = 1 << 16;
bool page_ok(int32_t p) { return p >= 1 && p <= kMaxPageSize; }
// log2 of a power-of-two page size, else 0 (the general page classes divide)
int32_t page_shift(int32_t p) { return (p & (p - 1)) == 0 ? __builtin_ctz((unsigned)p) : 0; }

constexpr int32_t kGqaHeadDim = 128;
constexpr int32_t kMlaHeadDimK = 576;

// Split policy the kernels are tuned for: the arguments this library passes
// to pd_split_rule.  GQA: one program per (request, kv head), one decode
// workgroup per CU; MLA: one program per (request, 128-row block).
struct SplitPolicy {
  int32_t block_h;
  float occupancy;
  int32_t min_work;       // keys per split before a request uses fewer splits
  int32_t max_splits;
  int32_t balance_chunk;  // skew bound: pieces of the longest request may be this short
};
constexpr SplitPolicy kGqaPolicy{1, 1.0f, 256, 64, 1024};
constexpr SplitPolicy kMlaPolicy{128, 1.0f, 128, 16, 2048};

// Compute units of a device (< 0: the current one), queried once per device;
// 0 if the query fails.
int32_t device_cus(int32_t device) {
  static int32_t cached[64] = {0};
  int dev = device;
  if (dev < 0 && hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// Split partials of the allocation-free entry point (paged_verify_gqa_noalloc):
// one array per GPU the library runs on, held until the process ends.
constexpr size_t kScratchBytes = size_t{64} << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// Device address of this GPU's scratch array, looked up once per device with
// the device current (host code never uses the array's own name: on the host
// it is a stand-in, not a device address).  nullptr if the lookup fails.
float* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev] = p;
  }
  return static_cast<float*>(ptrs[dev]);
}

}  // namespace

extern "C" {

const char* pd_status_string(int status) {
  switch (status) {
    case PD_OK: return "ok";
    case PD_ERR_INVALID: return "invalid argument";
    case PD_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case PD_ERR_UNSUPPORTED: return "unsupported size";
    case PD_ERR_WORKSPACE: return "workspace missing or too small";
    case PD_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t pd_split_rule(int32_t max_seq_len, int32_t batch, int32_t qlen, int32_t num_heads,
                      int32_t block_h, int32_t num_cus, float occupancy,
                      int32_t min_work_per_split, int32_t max_splits, int32_t balance_chunk) {
  if (max_seq_len < 0 || batch < 0 || qlen < 1 || num_heads < 1 || block_h < 1 ||
      !(occupancy > 0.f) || max_splits < 1)
    return PD_ERR_INVALID;
  if (num_cus <= 0) {
    num_cus = device_cus(-1);
    if (num_cus <= 0) return PD_ERR_HIP;
  }
  // 128-bit integers: the products below stay exact for any int32 sizes
  typedef __int128 i128;
  auto cdiv128 = [](i128 x, i128 y) { return (x + y - 1) / y; };
  const i128 row_blocks = cdiv128((i128)qlen * num_heads, block_h);
  const i128 per_split = (i128)(batch > 1 ? batch : 1) * row_blocks;
  const i128 ideal =
      cdiv128(max_seq_len > 1 ? max_seq_len : 1, min_work_per_split > 1 ? min_work_per_split : 1);
  // resident programs; the float product is clamped before its conversion
  const double slots_d = (double)occupancy * (double)num_cus;
  const i128 slots = slots_d >= 4.0e18 ? (i128)4000000000000000000LL
                                       : slots_d < 1.0 ? (i128)1 : (i128)(int64_t)slots_d;
  i128 n;
  if (per_split <= slots) {
    n = slots / per_split;
  } else {
    const i128 top = ideal < max_splits ? ideal : (i128)max_splits;
    const int64_t hi = top > 1 ? (int64_t)top : 1;
    double best = 1e300;
    for (int64_t k = 1; k <= hi; ++k) {
      const double cost = (double)cdiv128(k * per_split, slots) / (double)k;
      if (cost < best) best = cost;
    }
    n = hi;
    for (int64_t k = 1; k <= hi; ++k) {
      const double cost = (double)cdiv128(k * per_split, slots) / (double)k;
      if (cost <= best * 1.05) {
        n = k;
        break;
      }
    }
  }
  i128 cap = n;
  if (ideal < cap) cap = ideal;
  if (2 * (i128)num_cus < cap) cap = 2 * (i128)num_cus;
  if (cap < 1) cap = 1;
  if (balance_chunk > 0) {
    i128 bal = cdiv128(max_seq_len > 1 ? max_seq_len : 1, balance_chunk);
    if (bal > max_splits) bal = max_splits;
    if (bal > ideal) bal = ideal;
    if (bal > cap) cap = bal;
  }
  return (int32_t)(cap < INT32_MAX ? cap : (i128)INT32_MAX);
}

int32_t pd_gqa_split_cap(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                         int32_t window, int32_t num_cus) {
  if (batch < 0 || num_kv_heads < 1 || max_seq_len < 0) return PD_ERR_INVALID;
  const int32_t cus = num_cus > 0 ? num_cus : device_cus(-1);
  if (cus <= 0) return PD_ERR_HIP;
  // keys one (request, kv head) can attend: the window bounds them
  const int32_t keys = window > 0 && window < max_seq_len ? window : max_seq_len;
  return pd_split_rule(keys, batch, 1, num_kv_heads, 1, cus, kGqaPolicy.occupancy,
                       kGqaPolicy.min_work, kGqaPolicy.max_splits, kGqaPolicy.balance_chunk);
}

int32_t pd_mla_split_cap(int32_t batch, int32_t qlen, int32_t num_heads, int32_t max_seq_len,
                         int32_t num_cus) {
  if (batch < 0 || qlen < 1 || num_heads < 1 || max_seq_len < 0) return PD_ERR_INVALID;
  const int32_t cus = num_cus > 0 ? num_cus : device_cus(-1);
  if (cus <= 0) return PD_ERR_HIP;
  return pd_split_rule(max_seq_len, batch, qlen, num_heads, kMlaPolicy.block_h, cus,
                       kMlaPolicy.occupancy, kMlaPolicy.min_work, kMlaPolicy.max_splits,
                       kMlaPolicy.balance_chunk);
}

int32_t num_kv_splits_cap(int32_t max_seq_len, int32_t batch, int32_t qlen,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_k,
                          int32_t max_splits, int32_t device) {
  if (max_seq_len < 0 || batch < 0 || qlen < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0)
    return PD_ERR_INVALID;
  const bool mla = head_dim_k == kMlaHeadDimK && num_kv_heads == 1;
  if (!mla && head_dim_k != kGqaHeadDim) return PD_ERR_UNSUPPORTED;
  const SplitPolicy& pol = mla ? kMlaPolicy : kGqaPolicy;
  const int32_t cus = device_cus(device);
  if (cus <= 0) return PD_ERR_HIP;
  const int32_t top = max_splits > 0 && max_splits < pol.max_splits ? max_splits : pol.max_splits;
  if (mla)
    return pd_split_rule(max_seq_len, batch, qlen, num_q_heads, pol.block_h, cus, pol.occupancy,
                         pol.min_work, top, pol.balance_chunk);
  return pd_split_rule(max_seq_len, batch, 1, num_kv_heads, pol.block_h, cus, pol.occupancy,
                       pol.min_work, top, pol.balance_chunk);
}

size_t pd_workspace_bytes(int32_t rows, int32_t num_heads, int32_t num_splits, int32_t head_dim_v) {
  if (rows <= 0 || num_heads <= 0 || num_splits <= 1 || head_dim_v <= 0) return 0;
  return (size_t)rows * (size_t)num_heads * (size_t)num_splits * ((size_t)head_dim_v + 1) *
         sizeof(float);
}

namespace {

// New tokens' K and V for the fused append (element strides).
struct AppendSrc {
  const void* k;
  int64_t k_srow, k_sh;
  const void* v;
  int64_t v_srow, v_sh;
};

// GQA decode and verify.  Rows of q / out / lse are (request, verify token)
// pairs, row b * qlen + t; decode is qlen = 1 with no real lengths.
static int gqa_common(const void* q, int64_t q_stride_b, int64_t q_stride_h, const void* kv,
               int32_t kv_dtype, const float* k_scale, const float* v_scale,
               int32_t scale_per_head,
               int64_t kv_stride_page, int64_t kv_stride_head, int32_t num_pages,
               const int32_t* block_table, int64_t bt_stride_b, int32_t max_blocks,
               const int32_t* seq_lens, const int32_t* real_seq_lens, int32_t qlen,
               const float* sinks, int32_t window, float sm_scale,
               int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
               int32_t page_size, int32_t num_kv_splits, float* workspace,
               size_t workspace_bytes, void* out, int64_t o_stride_b, int64_t o_stride_h,
               float* lse, int64_t lse_stride_b, void* stream, bool partials_only,
               const int32_t* cu_seqlens_q = nullptr, int32_t total_rows = -1,
               bool use_scratch = false, const AppendSrc* app = nullptr) {
  if (batch < 0 || qlen < 1 || num_q_heads < 1 || num_kv_heads < 1 || num_kv_splits < 1 ||
      num_pages < 0 || max_blocks < 0 || !std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return PD_ERR_INVALID;
  if (num_q_heads % num_kv_heads != 0) return PD_ERR_INVALID;
  if ((kv_dtype != PD_KV_BF16 && kv_dtype != PD_KV_FP8_E4M3FN) ||
      (scale_per_head != 0 && scale_per_head != 1))
    return PD_ERR_INVALID;
  const bool fp8 = kv_dtype == PD_KV_FP8_E4M3FN;
  const int32_t G = num_q_heads / num_kv_heads;
  if (page_size < 1) return PD_ERR_INVALID;
  // Score columns: at most 64 (verify token, head) pairs per launch.  Fixed
  // verify rows past that run as slices of whole tokens, one launch each
  // (the cache is then read once per slice); variable rows do not.
  if (head_dim != 128 || !page_ok(page_size) || G > 64 ||
      (cu_seqlens_q != nullptr && (int64_t)qlen * G > 64))
    return PD_ERR_UNSUPPORTED;
  if (batch == 0) return PD_OK;
  if (q == nullptr || kv == nullptr || block_table == nullptr || seq_lens == nullptr ||
      (!partials_only && out == nullptr))
    return PD_ERR_INVALID;
  if (q_stride_b < 0 || q_stride_h < 0 || kv_stride_page < 0 || kv_stride_head < 0 ||
      bt_stride_b < 0 || o_stride_b < 0 || o_stride_h < 0 || lse_stride_b < 0)
    return PD_ERR_INVALID;
  const int64_t kv_align = fp8 ? 16 : 8;   // 16-byte rows of the cache
  if (!aligned16(q) || !aligned16(kv) || q_stride_b % 8 || q_stride_h % 8 ||
      kv_stride_page % kv_align || kv_stride_head % kv_align)
    return PD_ERR_ALIGN;
  if (!partials_only && (!aligned16(out) || o_stride_b % 8 || o_stride_h % 8)) return PD_ERR_ALIGN;
  if (app != nullptr) {
    if (app->k == nullptr || app->v == nullptr || app->k_srow < 0 || app->k_sh < 0 ||
        app->v_srow < 0 || app->v_sh < 0)
      return PD_ERR_INVALID;
    // 16-byte chunks of every source row
    if (!aligned16(app->k) || !aligned16(app->v) || app->k_srow % kv_align ||
        app->k_sh % kv_align || app->v_srow % kv_align || app->v_sh % kv_align)
      return PD_ERR_ALIGN;
    // byte offsets row * stride stay inside int64 for any row count
    if (app->k_srow > INT32_MAX || app->k_sh > INT32_MAX || app->v_srow > INT32_MAX ||
        app->v_sh > INT32_MAX)
      return PD_ERR_UNSUPPORTED;
  }
  if (cu_seqlens_q != nullptr && total_rows < 0) return PD_ERR_INVALID;
  const int64_t rows = cu_seqlens_q != nullptr ? (int64_t)total_rows : (int64_t)batch * qlen;
  if (rows > 0x7fffffff) return PD_ERR_UNSUPPORTED;
  const bool needs_ws = num_kv_splits > 1 || partials_only;
  if (needs_ws) {
    const int32_t ws_splits = num_kv_splits > 1 ? num_kv_splits : 2;
    size_t need = pd_workspace_bytes((int32_t)rows, num_q_heads, ws_splits, head_dim);
    if (num_kv_splits == 1) need /= 2;
    if (use_scratch) {
      if (need > kScratchBytes) return PD_ERR_WORKSPACE;
    } else {
      if (workspace == nullptr || workspace_bytes < need) return PD_ERR_WORKSPACE;
      if (!aligned16(workspace)) return PD_ERR_ALIGN;
    }
  }
  if (num_kv_heads > 65535 || batch > 65535 || num_kv_splits > 65535) return PD_ERR_UNSUPPORTED;
  const int64_t kLim = INT32_MAX;
  if (q_stride_b > kLim || q_stride_h > kLim || kv_stride_page > kLim || kv_stride_head > kLim ||
      bt_stride_b > kLim || o_stride_b > kLim || o_stride_h > kLim || lse_stride_b > kLim)
    return PD_ERR_UNSUPPORTED;
  // a unit's query rows are addressed with a 32-bit byte offset from its first row
  if (((int64_t)(qlen - 1) * q_stride_b + (int64_t)(G - 1) * q_stride_h + head_dim) * 2 > kLim)
    return PD_ERR_UNSUPPORTED;
  // the kernel indexes all (request, kv head, 32-token tile) triples with int32
  if ((int64_t)max_blocks * page_size > (int64_t)INT32_MAX / 2 ||
      (int64_t)batch * num_kv_heads * cdiv64((int64_t)max_blocks * page_size, 32) > INT32_MAX / 2)
    return PD_ERR_UNSUPPORTED;

  if (use_scratch && needs_ws) {
    // every argument check has passed: the first HIP call of the entry point
    workspace = scratch_ptr();
    if (workspace == nullptr) return PD_ERR_HIP;
  }

  pd::GqaArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_sb = (int32_t)q_stride_b;
  a.q_sh = (int32_t)q_stride_h;
  a.kv = static_cast<const uint16_t*>(kv);
  a.kv_sp = (int32_t)kv_stride_page;
  a.kv_sh = (int32_t)kv_stride_head;
  a.num_pages = num_pages;
  a.bt = block_table;
  a.bt_sb = (int32_t)bt_stride_b;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.real_lens = real_seq_lens;
  a.qlen = qlen;
  a.q_req_rows = qlen;
  a.t_off = 0;
  a.len_sub = 0;
  a.cu_q = cu_seqlens_q;
  a.total_rows = (int32_t)rows;
  a.kv_fp8 = fp8 ? 1 : 0;
  a.k_scale = fp8 ? k_scale : nullptr;
  a.v_scale = fp8 ? v_scale : nullptr;
  a.scale_stride = scale_per_head;
  a.sinks = sinks;
  a.window = window;
  a.scale_log2 = sm_scale * kLog2eHost;
  a.B = batch;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.G = G;
  a.P = page_size;
  a.p_shift = page_shift(page_size);
  a.S = num_kv_splits;
  a.partials = partials_only ? 1 : 0;
  a.ws = workspace;
  a.out = static_cast<uint16_t*>(out);
  a.o_sb = (int32_t)o_stride_b;
  a.o_sh = (int32_t)o_stride_h;
  a.lse = lse;
  a.lse_sb = (int32_t)lse_stride_b;
  if (app != nullptr) {
    const int64_t eb = fp8 ? 1 : 2;   // bytes per element
    a.kn = static_cast<const char*>(app->k);
    a.vn = static_cast<const char*>(app->v);
    a.kn_srow = app->k_srow * eb;
    a.kn_sh = app->k_sh * eb;
    a.vn_srow = app->v_srow * eb;
    a.vn_sh = app->v_sh * eb;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t per_launch = 64 / G;   // verify tokens of one launch
  if (cu_seqlens_q != nullptr || qlen <= per_launch) {
    if (pd::launch_gqa_decode(a, s) != hipSuccess) return PD_ERR_HIP;
  } else {
    // equal slices (sizes differ by at most one), in token order: with the
    // fused append, a slice's new tokens are in the cache before the next
    // slice attends them
    const int32_t n_sl = (qlen + per_launch - 1) / per_launch;
    int32_t t0 = 0;
    for (int32_t i = 0; i < n_sl; ++i) {
      const int32_t n = qlen / n_sl + (i < qlen % n_sl ? 1 : 0);
      a.qlen = n;
      a.t_off = t0;
      a.len_sub = qlen - t0 - n;
      if (pd::launch_gqa_decode(a, s) != hipSuccess) return PD_ERR_HIP;
      t0 += n;
    }
  }
  if (num_kv_splits > 1 && !partials_only) {
    pd::MergeArgs m{};
    m.ws = workspace;
    m.rows = (int32_t)rows;
    m.H = num_q_heads;
    m.S = num_kv_splits;
    m.Dv = head_dim;
    m.sinks = sinks;
    m.out = static_cast<uint16_t*>(out);
    m.o_srow = o_stride_b;
    m.o_sh = o_stride_h;
    m.lse = lse;
    m.lse_srow = lse_stride_b;
    if (pd::launch_merge(m, s) != hipSuccess) return PD_ERR_HIP;
  }
  return PD_OK;
}

}  // namespace

int paged_decode_gqa(const void* q, int64_t q_stride_b, int64_t q_stride_h, const void* kv,
                     int64_t kv_stride_page, int64_t kv_stride_head, int32_t num_pages,
                     const int32_t* block_table, int64_t bt_stride_b, int32_t max_blocks,
                     const int32_t* seq_lens, const float* sinks, int32_t window, float sm_scale,
                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, int32_t num_kv_splits, float* workspace,
                     size_t workspace_bytes, void* out, int64_t o_stride_b, int64_t o_stride_h,
                     float* lse, int64_t lse_stride_b, void* stream) {
  return gqa_common(q, q_stride_b, q_stride_h, kv, PD_KV_BF16, nullptr, nullptr, 0,
                    kv_stride_page, kv_stride_head, num_pages, block_table, bt_stride_b,
                    max_blocks, seq_lens, nullptr, 1, sinks, window, sm_scale, batch,
                    num_q_heads, num_kv_heads, head_dim, page_size, num_kv_splits, workspace,
                    workspace_bytes, out, o_stride_b, o_stride_h, lse, lse_stride_b, stream,
                    false);
}

int paged_verify_gqa(const void* q, int64_t q_stride_row, int64_t q_stride_h, const void* kv,
                     int32_t kv_dtype, const float* k_scale, const float* v_scale,
                     int32_t scale_per_head,
                     int64_t kv_stride_page, int64_t kv_stride_head, int32_t num_pages,
                     const int32_t* block_table, int64_t bt_stride_b, int32_t max_blocks,
                     const int32_t* seq_lens, const int32_t* real_seq_lens, int32_t qlen,
                     const float* sinks, int32_t window, float sm_scale, int32_t batch,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t page_size, int32_t num_kv_splits, float* workspace,
                     size_t workspace_bytes, void* out, int64_t o_stride_row, int64_t o_stride_h,
                     float* lse, int64_t lse_stride_row, void* stream) {
  return gqa_common(q, q_stride_row, q_stride_h, kv, kv_dtype, k_scale, v_scale,
                    scale_per_head, kv_stride_page, kv_stride_head, num_pages,
                    block_table, bt_stride_b, max_blocks, seq_lens, real_seq_lens, qlen, sinks,
                    window, sm_scale, batch, num_q_heads, num_kv_heads, head_dim, page_size,
                    num_kv_splits, workspace, workspace_bytes, out, o_stride_row, o_stride_h,
                    lse, lse_stride_row, stream, false);
}

int paged_verify_gqa_append(const void* q, int64_t q_stride_row, int64_t q_stride_h, void* kv,
                            int32_t kv_dtype, const float* k_scale, const float* v_scale,
                            int32_t scale_per_head, int64_t kv_stride_page,
                            int64_t kv_stride_head, int32_t num_pages,
                            const int32_t* block_table, int64_t bt_stride_b, int32_t max_blocks,
                            const int32_t* seq_lens, const int32_t* real_seq_lens, int32_t qlen,
                            const void* k_new, int64_t k_new_stride_row, int64_t k_new_stride_h,
                            const void* v_new, int64_t v_new_stride_row, int64_t v_new_stride_h,
                            const float* sinks, int32_t window, float sm_scale, int32_t batch,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t page_size, int32_t num_kv_splits, float* workspace,
                            size_t workspace_bytes, void* out, int64_t o_stride_row,
                            int64_t o_stride_h, float* lse, int64_t lse_stride_row, void* stream) {
  const AppendSrc app{k_new, k_new_stride_row, k_new_stride_h, v_new, v_new_stride_row,
                      v_new_stride_h};
  return gqa_common(q, q_stride_row, q_stride_h, kv, kv_dtype, k_scale, v_scale,
                    scale_per_head, kv_stride_page, kv_stride_head, num_pages,
                    block_table, bt_stride_b, max_blocks, seq_lens, real_seq_lens, qlen, sinks,
                    window, sm_scale, batch, num_q_heads, num_kv_heads, head_dim, page_size,
                    num_kv_splits, workspace, workspace_bytes, out, o_stride_row, o_stride_h,
                    lse, lse_stride_row, stream, false, nullptr, -1, false, &app);
}

int paged_verify_gqa_noalloc(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                             const void* kv, int32_t kv_dtype, const float* k_scale,
                             const float* v_scale, int32_t scale_per_head,
                             int64_t kv_stride_page, int64_t kv_stride_head, int32_t num_pages,
                             const int32_t* block_table, int64_t bt_stride_b, int32_t max_blocks,
                             const int32_t* seq_lens, const int32_t* real_seq_lens, int32_t qlen,
                             const float* sinks, int32_t window, float sm_scale, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t page_size, int32_t num_kv_splits, void* out,
                             int64_t o_stride_row, int64_t o_stride_h, float* lse,
                             int64_t lse_stride_row, void* stream) {
  return gqa_common(q, q_stride_row, q_stride_h, kv, kv_dtype, k_scale, v_scale,
                    scale_per_head, kv_stride_page, kv_stride_head, num_pages,
                    block_table, bt_stride_b, max_blocks, seq_lens, real_seq_lens, qlen, sinks,
                    window, sm_scale, batch, num_q_heads, num_kv_heads, head_dim, page_size,
                    num_kv_splits, nullptr, 0, out, o_stride_row, o_stride_h,
                    lse, lse_stride_row, stream, false, nullptr, -1, true);
}

int paged_verify_gqa_varlen(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                            const void* kv, int32_t kv_dtype, const float* k_scale,
                            const float* v_scale, int32_t scale_per_head,
                            int64_t kv_stride_page, int64_t kv_stride_head, int32_t num_pages,
                            const int32_t* block_table, int64_t bt_stride_b, int32_t max_blocks,
                            const int32_t* seq_lens, const int32_t* real_seq_lens,
                            const int32_t* cu_seqlens_q, int32_t max_qlen, int32_t total_rows,
                            const float* sinks, int32_t window, float sm_scale, int32_t batch,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t page_size, int32_t num_kv_splits, float* workspace,
                            size_t workspace_bytes, void* out, int64_t o_stride_row,
                            int64_t o_stride_h, float* lse, int64_t lse_stride_row, void* stream) {
  if (cu_seqlens_q == nullptr && batch > 0) return PD_ERR_INVALID;
  if (total_rows < 0) return PD_ERR_INVALID;
  if (batch > 0 && total_rows == 0) return PD_OK;   // no query row at all
  return gqa_common(q, q_stride_row, q_stride_h, kv, kv_dtype, k_scale, v_scale,
                    scale_per_head, kv_stride_page, kv_stride_head, num_pages,
                    block_table, bt_stride_b, max_blocks, seq_lens, real_seq_lens, max_qlen,
                    sinks, window, sm_scale, batch, num_q_heads, num_kv_heads, head_dim,
                    page_size, num_kv_splits, workspace, workspace_bytes, out, o_stride_row,
                    o_stride_h, lse, lse_stride_row, stream, false, cu_seqlens_q, total_rows);
}

int paged_decode_gqa_partials(const void* q, int64_t q_stride_b, int64_t q_stride_h,
                              const void* kv, int64_t kv_stride_page, int64_t kv_stride_head,
                              int32_t num_pages, const int32_t* block_table,
                              int64_t bt_stride_b, int32_t max_blocks, const int32_t* seq_lens,
                              int32_t window, float sm_scale, int32_t batch,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t page_size, int32_t num_kv_splits, float* workspace,
                              size_t workspace_bytes, void* stream) {
  return gqa_common(q, q_stride_b, q_stride_h, kv, PD_KV_BF16, nullptr, nullptr, 0,
                    kv_stride_page, kv_stride_head, num_pages,
                    block_table, bt_stride_b, max_blocks, seq_lens, nullptr, 1, nullptr, window,
                    sm_scale, batch, num_q_heads, num_kv_heads, head_dim, page_size,
                    num_kv_splits, workspace, workspace_bytes, nullptr, 0, 0, nullptr, 0, stream,
                    true);
}

int paged_verify_gqa_partials(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                              const void* kv, int32_t kv_dtype, const float* k_scale,
                              const float* v_scale, int32_t scale_per_head,
                              int64_t kv_stride_page, int64_t kv_stride_head, int32_t num_pages,
                              const int32_t* block_table, int64_t bt_stride_b,
                              int32_t max_blocks, const int32_t* seq_lens,
                              const int32_t* real_seq_lens, const int32_t* cu_seqlens_q,
                              int32_t qlen, int32_t total_rows, int32_t window, float sm_scale,
                              int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t num_kv_splits,
                              float* workspace, size_t workspace_bytes, void* stream) {
  if (cu_seqlens_q != nullptr) {
    if (total_rows < 0) return PD_ERR_INVALID;
    if (batch > 0 && total_rows == 0) return PD_OK;   // no query row at all
  }
  return gqa_common(q, q_stride_row, q_stride_h, kv, kv_dtype, k_scale, v_scale,
                    scale_per_head, kv_stride_page, kv_stride_head, num_pages, block_table,
                    bt_stride_b, max_blocks, seq_lens, real_seq_lens, qlen, nullptr, window,
                    sm_scale, batch, num_q_heads, num_kv_heads, head_dim, page_size,
                    num_kv_splits, workspace, workspace_bytes, nullptr, 0, 0, nullptr, 0, stream,
                    true, cu_seqlens_q, cu_seqlens_q != nullptr ? total_rows : -1);
}

int paged_kv_append(const void* src0, int64_t src0_stride_tok, int64_t src0_stride_h,
                    int32_t src0_elems, const void* src1, int64_t src1_stride_tok,
                    int64_t src1_stride_h, int32_t src1_elems, int32_t elem_bytes, void* cache,
                    int64_t cache_stride_page, int64_t cache_stride_head,
                    int64_t cache_stride_tok, int32_t num_pages, const int32_t* block_table,
                    int64_t bt_stride_b, int32_t max_blocks, const int32_t* seq_lens,
                    int32_t qlen, int32_t batch, int32_t num_heads, int32_t page_size,
                    void* stream) {
  if (batch < 0 || qlen < 1 || num_heads < 1 || page_size < 1 || num_pages < 0 ||
      max_blocks < 0 || src0_elems < 1 || src1_elems < 0 || (elem_bytes != 1 && elem_bytes != 2))
    return PD_ERR_INVALID;
  if ((src1 == nullptr) != (src1_elems == 0)) return PD_ERR_INVALID;
  if (batch == 0) return PD_OK;
  if (src0 == nullptr || cache == nullptr || block_table == nullptr || seq_lens == nullptr)
    return PD_ERR_INVALID;
  if (src0_stride_tok < 0 || src0_stride_h < 0 || src1_stride_tok < 0 || src1_stride_h < 0 ||
      cache_stride_page < 0 || cache_stride_head < 0 || cache_stride_tok < 0 || bt_stride_b < 0)
    return PD_ERR_INVALID;
  // a token's row (both sources) must fit its cache row
  if ((int64_t)src0_elems + src1_elems > cache_stride_tok) return PD_ERR_INVALID;
  const int64_t eb = elem_bytes;
  auto a16 = [&](int64_t elems) { return (elems * eb) % 16 == 0; };
  if (!aligned16(src0) || !aligned16(cache) || (src1 != nullptr && !aligned16(src1)) ||
      !a16(src0_elems) || !a16(src1_elems) || !a16(src0_stride_tok) || !a16(src0_stride_h) ||
      !a16(src1_stride_tok) || !a16(src1_stride_h) || !a16(cache_stride_page) ||
      !a16(cache_stride_head) || !a16(cache_stride_tok))
    return PD_ERR_ALIGN;
  if ((int64_t)batch * qlen > 0x7fffffff) return PD_ERR_UNSUPPORTED;
  pd::AppendArgs a{};
  a.src0 = static_cast<const char*>(src0);
  a.s0_tok = src0_stride_tok * eb;
  a.s0_h = src0_stride_h * eb;
  a.src1 = static_cast<const char*>(src1);
  a.s1_tok = src1_stride_tok * eb;
  a.s1_h = src1_stride_h * eb;
  a.c0 = (int32_t)(src0_elems * eb / 16);
  a.c1 = (int32_t)(src1_elems * eb / 16);
  a.cache = static_cast<char*>(cache);
  a.c_sp = cache_stride_page * eb;
  a.c_sh = cache_stride_head * eb;
  a.c_st = cache_stride_tok * eb;
  a.num_pages = num_pages;
  a.bt = block_table;
  a.bt_sb = bt_stride_b;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.qlen = qlen;
  a.B = batch;
  a.H = num_heads;
  a.P = page_size;
  if (pd::launch_kv_append(a, static_cast<hipStream_t>(stream)) != hipSuccess) return PD_ERR_HIP;
  return PD_OK;
}

namespace {

// MLA verify; with partials_only, the split partials without the merge.
int mla_common(const void* q, int64_t q_stride_row, int64_t q_stride_h, const void* kv,
               int32_t kv_dtype, int64_t kv_stride_page, int64_t kv_stride_tok,
               int32_t num_pages, const float* k_scale, const int32_t* block_table,
               int64_t bt_stride_b, int32_t max_blocks, const int32_t* seq_lens,
               const int32_t* real_seq_lens, int32_t qlen, float sm_scale, int32_t batch,
               int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
               int32_t page_size, int32_t num_kv_splits, float* workspace,
               size_t workspace_bytes, void* out, int64_t o_stride_row,
               int64_t o_stride_h, float* lse, int64_t lse_stride_row, void* stream,
               bool partials_only) {
  if (batch < 0 || qlen < 1 || num_heads < 1 || num_kv_splits < 1 || num_pages < 0 ||
      max_blocks < 0 || !std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return PD_ERR_INVALID;
  if (kv_dtype != PD_KV_BF16 && kv_dtype != PD_KV_FP8_E4M3FN) return PD_ERR_INVALID;
  if (page_size < 1) return PD_ERR_INVALID;
  if (head_dim_k != 576 || head_dim_v != 512 || !page_ok(page_size)) return PD_ERR_UNSUPPORTED;
  if (batch == 0) return PD_OK;
  if (q == nullptr || kv == nullptr || block_table == nullptr || seq_lens == nullptr ||
      (!partials_only && out == nullptr))
    return PD_ERR_INVALID;
  if (q_stride_row < 0 || q_stride_h < 0 || kv_stride_page < 0 || kv_stride_tok < 0 ||
      bt_stride_b < 0 || o_stride_row < 0 || o_stride_h < 0 || lse_stride_row < 0)
    return PD_ERR_INVALID;
  const int64_t kv_align = kv_dtype == PD_KV_BF16 ? 8 : 16;
  if (!aligned16(q) || !aligned16(kv) || q_stride_row % 8 || q_stride_h % 8 ||
      kv_stride_page % kv_align || kv_stride_tok % kv_align)
    return PD_ERR_ALIGN;
  {
    // the kernel forms page and token offsets as 32 x 32-bit products
    const int64_t elem = kv_dtype == PD_KV_BF16 ? 2 : 1;
    if (kv_stride_page > (int64_t)UINT32_MAX / elem || kv_stride_tok > (int64_t)UINT32_MAX / elem)
      return PD_ERR_UNSUPPORTED;
  }
  if (!partials_only && (!aligned16(out) || o_stride_row % 8 || o_stride_h % 8))
    return PD_ERR_ALIGN;
  const int64_t rows = (int64_t)batch * qlen;
  if (rows > 0x7fffffff) return PD_ERR_UNSUPPORTED;
  {
    // the kernel's plan counts tiles over all (request, row block) units in int32
    const int64_t rows_req = (int64_t)qlen * num_heads;
    const int64_t keys = (int64_t)max_blocks * page_size;
    if (rows_req > INT32_MAX / 2 || keys > INT32_MAX / 2 ||
        (__int128)batch * cdiv64(rows_req, 128) * cdiv64(keys, 32) > INT32_MAX / 2)
      return PD_ERR_UNSUPPORTED;
  }
  if (num_kv_splits > 1 || partials_only) {
    const int32_t ws_splits = num_kv_splits > 1 ? num_kv_splits : 2;
    size_t need = pd_workspace_bytes((int32_t)rows, num_heads, ws_splits, head_dim_v);
    if (num_kv_splits == 1) need /= 2;
    if (workspace == nullptr || workspace_bytes < need) return PD_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PD_ERR_ALIGN;
  }
  pd::MlaArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_srow = q_stride_row;
  a.q_sh = q_stride_h;
  a.kv = kv;
  a.kv_fp8 = kv_dtype == PD_KV_FP8_E4M3FN;
  a.kv_sp = kv_stride_page;
  a.kv_st = kv_stride_tok;
  a.num_pages = num_pages;
  a.k_scale = k_scale;
  a.bt = block_table;
  a.bt_sb = bt_stride_b;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.real_lens = real_seq_lens;
  a.qlen = qlen;
  a.scale_log2 = sm_scale * kLog2eHost;
  a.B = batch;
  a.H = num_heads;
  a.P = page_size;
  a.p_shift = page_shift(page_size);
  a.S = num_kv_splits;
  a.partials = partials_only ? 1 : 0;
  a.ws = workspace;
  a.out = static_cast<uint16_t*>(out);
  a.o_srow = o_stride_row;
  a.o_sh = o_stride_h;
  a.lse = lse;
  a.lse_srow = lse_stride_row;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pd::launch_mla_verify(a, s) != hipSuccess) return PD_ERR_HIP;
  if (num_kv_splits > 1 && !partials_only) {
    pd::MergeArgs m{};
    m.ws = workspace;
    m.rows = (int32_t)rows;
    m.H = num_heads;
    m.S = num_kv_splits;
    m.Dv = head_dim_v;
    m.sinks = nullptr;
    m.out = static_cast<uint16_t*>(out);
    m.o_srow = o_stride_row;
    m.o_sh = o_stride_h;
    m.lse = lse;
    m.lse_srow = lse_stride_row;
    if (pd::launch_merge(m, s) != hipSuccess) return PD_ERR_HIP;
  }
  return PD_OK;
}

}  // namespace

int paged_verify_mla(const void* q, int64_t q_stride_row, int64_t q_stride_h, const void* kv,
                     int32_t kv_dtype, int64_t kv_stride_page, int64_t kv_stride_tok,
                     int32_t num_pages, const float* k_scale, const int32_t* block_table,
                     int64_t bt_stride_b, int32_t max_blocks, const int32_t* seq_lens,
                     const int32_t* real_seq_lens, int32_t qlen, float sm_scale, int32_t batch,
                     int32_t num_heads, int32_t head_dim_k, int32_t head_dim_v,
                     int32_t page_size, int32_t num_kv_splits, float* workspace,
                     size_t workspace_bytes, void* out, int64_t o_stride_row,
                     int64_t o_stride_h, float* lse, int64_t lse_stride_row, void* stream) {
  return mla_common(q, q_stride_row, q_stride_h, kv, kv_dtype, kv_stride_page, kv_stride_tok,
                    num_pages, k_scale, block_table, bt_stride_b, max_blocks, seq_lens,
                    real_seq_lens, qlen, sm_scale, batch, num_heads, head_dim_k, head_dim_v,
                    page_size, num_kv_splits, workspace, workspace_bytes, out, o_stride_row,
                    o_stride_h, lse, lse_stride_row, stream, false);
}

int paged_verify_mla_partials(const void* q, int64_t q_stride_row, int64_t q_stride_h,
                              const void* kv, int32_t kv_dtype, int64_t kv_stride_page,
                              int64_t kv_stride_tok, int32_t num_pages, const float* k_scale,
                              const int32_t* block_table, int64_t bt_stride_b,
                              int32_t max_blocks, const int32_t* seq_lens,
                              const int32_t* real_seq_lens, int32_t qlen, float sm_scale,
                              int32_t batch, int32_t num_heads, int32_t head_dim_k,
                              int32_t head_dim_v, int32_t page_size, int32_t num_kv_splits,
                              float* workspace, size_t workspace_bytes, void* stream) {
  return mla_common(q, q_stride_row, q_stride_h, kv, kv_dtype, kv_stride_page, kv_stride_tok,
                    num_pages, k_scale, block_table, bt_stride_b, max_blocks, seq_lens,
                    real_seq_lens, qlen, sm_scale, batch, num_heads, head_dim_k, head_dim_v,
                    page_size, num_kv_splits, workspace, workspace_bytes, nullptr, 0, 0, nullptr,
                    0, stream, true);
}

int merge_splits(const float* workspace, int32_t rows, int32_t num_heads, int32_t num_splits,
                 int32_t head_dim_v, const float* sinks, void* out, int64_t o_stride_row,
                 int64_t o_stride_h, float* lse, int64_t lse_stride_row, void* stream) {
  if (rows < 0 || num_heads < 1 || num_splits < 1 || head_dim_v < 1) return PD_ERR_INVALID;
  if (head_dim_v != 128 && head_dim_v != 256 && head_dim_v != 512 && head_dim_v != 1024)
    return PD_ERR_UNSUPPORTED;
  if (rows == 0) return PD_OK;
  if (workspace == nullptr || out == nullptr) return PD_ERR_INVALID;
  if (o_stride_row < 0 || o_stride_h < 0 || lse_stride_row < 0) return PD_ERR_INVALID;
  if (!aligned16(out) || o_stride_row % 8 || o_stride_h % 8 ||
      (reinterpret_cast<uintptr_t>(workspace) & 3u))
    return PD_ERR_ALIGN;
  pd::MergeArgs m{};
  m.ws = workspace;
  m.rows = rows;
  m.H = num_heads;
  m.S = num_splits;
  m.Dv = head_dim_v;
  m.sinks = sinks;
  m.out = static_cast<uint16_t*>(out);
  m.o_srow = o_stride_row;
  m.o_sh = o_stride_h;
  m.lse = lse;
  m.lse_srow = lse_stride_row;
  if (pd::launch_merge(m, static_cast<hipStream_t>(stream)) != hipSuccess) return PD_ERR_HIP;
  return PD_OK;
}

}  // extern "C"
