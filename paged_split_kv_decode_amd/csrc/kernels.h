// Internal launch interface between the C-ABI layer (api.hip) and the
// kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pd {

// Token tile every kernel walks the keys in (one MFMA contraction depth).
constexpr int kTileTokens = 32;
// Fewest 32-token tiles an MLA verify split takes before the request uses
// fewer splits.
constexpr int kMlaMinSplitTiles = 4;

// Strides are in elements and below 2^31 (checked on the host), so the
// kernel keeps them in 32-bit scalar registers.
// GQA decode is the qlen = 1 case of GQA verify: q / out / lse rows are
// (request, verify token) pairs, row b * qlen + t.
struct GqaArgs {
  const uint16_t* q;
  int32_t q_sb, q_sh;   // q_sb: stride between rows
  const uint16_t* kv;
  int32_t kv_sp, kv_sh;
  int32_t num_pages;
  const int32_t* bt;
  int32_t bt_sb;
  int32_t max_blocks;
  const int32_t* seq_lens;
  const int32_t* real_lens;  // nullptr: equal to seq_lens
  int32_t qlen;              // verify tokens per request (the most, with cu_q); qlen * G <= 64
  // Uniform rows (cu_q == nullptr) may be one slice of longer verify rows:
  // the launch's token t of request b is row b * q_req_rows + t_off + t, and
  // len_sub (the request's verify tokens after the slice) comes off every
  // row's causal limit and off the newest-token positions.  A whole call:
  // q_req_rows = qlen, t_off = len_sub = 0.
  int32_t q_req_rows, t_off, len_sub;
  const int32_t* cu_q;       // nullptr: request b has rows b * q_req_rows + t_off + t; else [B + 1]
                             // cumulative query lengths (rows cu_q[b] .. cu_q[b + 1] - 1)
  int32_t total_rows;        // rows of q / out / lse (B * qlen, or cu_q[B])
  int32_t kv_fp8;            // 1: FP8 E4M3FN codes, K scaled by k_scale, V by v_scale
  const float* k_scale;      // nullptr: 1; else k_scale[kvh * scale_stride]
  const float* v_scale;
  int32_t scale_stride;      // 0: one scale for all kv heads, 1: one per kv head
  const float* sinks;
  int32_t window;
  float scale_log2;  // sm_scale * log2(e)
  int32_t B, Hq, Hkv, G, P;
  int32_t p_shift;   // log2(P) when the page size is a power of two, else 0
  int32_t S;         // split cap: no (request, kv head) is cut into more pieces
  int32_t partials;  // 1: always write workspace partials (never O / LSE)
  int32_t pair;      // 1 (set by the launcher; one split, at most 16 columns, few units):
                     // every unit is streamed by two waves of one workgroup, which merge
                     // their halves through LDS
  float* ws;         // [B * qlen, Hq, S, D + 1] when S > 1 or partials
  uint16_t* out;
  int32_t o_sb, o_sh;
  float* lse;
  int32_t lse_sb;
  // Fused append (kn == nullptr: none).  The n newest tokens of request b
  // (positions seq_lens[b] - n .. seq_lens[b] - 1, n its query rows) are
  // rows row0 .. row0 + n - 1 of these sources (byte strides): K of kv head
  // h at kn + row * kn_srow + h * kn_sh, V likewise from vn.  The kernel
  // attends them from the sources and writes them into the cache.
  const char* kn;
  const char* vn;
  int64_t kn_srow, kn_sh, vn_srow, vn_sh;
};

struct MergeArgs {
  const float* ws;   // [rows, H, S, Dv + 1]
  int32_t rows, H, S, Dv;
  const float* sinks;
  uint16_t* out;
  int64_t o_srow, o_sh;
  float* lse;
  int64_t lse_srow;
};

struct MlaArgs {
  const uint16_t* q;
  int64_t q_srow, q_sh;
  const void* kv;
  int32_t kv_fp8;
  int64_t kv_sp, kv_st;
  int32_t num_pages;
  const float* k_scale;
  const int32_t* bt;
  int64_t bt_sb;
  int32_t max_blocks;
  const int32_t* seq_lens;
  const int32_t* real_lens;
  int32_t qlen;
  float scale_log2;
  int32_t B, H, P;
  int32_t p_shift;   // log2(P) when the page size is a power of two, else 0
  int32_t S;
  int32_t partials;  // write split partials even with S == 1 (no merge follows)
  float* ws;
  uint16_t* out;
  int64_t o_srow, o_sh;
  float* lse;
  int64_t lse_srow;
};

// Byte strides; every pointer and stride 16-byte aligned (checked on the host).
struct AppendArgs {
  const char* src0;
  int64_t s0_tok, s0_h;
  const char* src1;            // nullptr when c1 == 0
  int64_t s1_tok, s1_h;
  int32_t c0, c1;              // 16-byte chunks per (token, head) row of each source
  char* cache;
  int64_t c_sp, c_sh, c_st;    // page, head, token strides of the cache
  int32_t num_pages;
  const int32_t* bt;
  int64_t bt_sb;
  int32_t max_blocks;
  const int32_t* seq_lens;
  int32_t qlen, B, H, P;
};

hipError_t launch_gqa_decode(const GqaArgs& a, hipStream_t stream);
// One GQA page class (1, 2, 4, 8, 16, 32 for every power-of-two page of 32
// tokens or more, or 0 for every other page size), with the fused append
// (AP) or not; the classes are instantiated in their own translation units.
template <int PS, bool AP>
hipError_t launch_gqa_class(const GqaArgs& a, bool verify, int n_wg, hipStream_t stream);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
hipError_t launch_mla_verify(const MlaArgs& a, hipStream_t stream);
// One MLA page class (1, 2, 4, 8, 16 for every power-of-two page of 16
// tokens or more, or 0 for every other page size); the classes are
// instantiated in their own translation units.
template <int PC>
hipError_t launch_mla_class(const MlaArgs& a, int n_wg, hipStream_t stream);

}  // namespace pd
