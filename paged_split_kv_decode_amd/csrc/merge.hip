// Split merge for gfx950: fp32 (O_s, lse_s) partials -> bf16 O and fp32 LSE.
//
// Operation: the split combine of "vllm.models.flint.ops.decode_attention"
// (combine_splits: per-head max over splits, per-split weights, weighted sum
// of O and l, sink added to the final denominator), restated for normalised
// partials with natural-log LSEs in the workspace layout of
// "vllm.v1.attention.ops.triton_decode_attention" (attn_logits:
// [rows, H, S, Lv + 1]).
//
// One wave per (row, head).  The slot list is slots 0 .. n - 1, n the first
// slot whose lse is +inf (S if none): the library's own calls end a list
// that way instead of marking every slot past it, and nothing after the end
// is read.  The first 8 slots' lse are read first (most lists end there);
// lane s then holds lse_s (64 slots per pass) to form the wave max M and the
// weights w_s = 2^((lse_s - M) log2 e); the splits with lse_s > -inf are
// gathered in batches of four, every load of a batch issued before any is
// used, each lane accumulating the Lv / 64 contiguous output dims it owns.
// A split with lse_s = -inf is never read or multiplied, so its O_s may hold
// anything.  A NaN lse_s (a partial that saw an invalid block-table entry)
// makes the result NaN.
#include "device_common.h"
#include "kernels.h"

namespace pd {
namespace {

constexpr int kWaves = 4;

template <int E>
__global__ __launch_bounds__(kWaves * 64) void merge_kernel(MergeArgs a) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * kWaves + wave;
  if (pair >= (int64_t)a.rows * a.H) return;
  const int row = (int)(pair / a.H);
  const int h = (int)(pair % a.H);
  const int S = a.S;
  const int stride = a.Dv + 1;
  const float* base = a.ws + pair * (int64_t)S * stride;
  auto lse_at = [&](int s) { return base[(int64_t)s * stride + a.Dv]; };

  // the end of the list: the first 8 slots, then 64 at a time
  int n = S;
  const int c8 = S < 8 ? S : 8;
  const float l8 = lane < c8 ? lse_at(lane) : neg_inf();
  uint64_t end = __ballot(lane < c8 && l8 == end_of_slots());
  if (end != 0ull) {
    n = __builtin_ctzll(end);
  } else {
    for (int s0 = c8; s0 < S; s0 += 64) {
      const bool in = s0 + lane < S;
      const float l = in ? lse_at(s0 + lane) : neg_inf();
      end = __ballot(in && l == end_of_slots());
      if (end != 0ull) {
        n = s0 + __builtin_ctzll(end);
        break;
      }
    }
  }
  // lane s's lse in the pass from s0 (slots >= n read as -inf)
  auto lse_pass = [&](int s0) {
    const int s = s0 + lane;
    return s >= n ? neg_inf() : (s < 8 ? l8 : lse_at(s));
  };

  float M = neg_inf();
  bool nan_seen = false;
  for (int s0 = 0; s0 < n; s0 += 64) {
    const float l = lse_pass(s0);
    nan_seen |= l != l;
    M = fmaxf(M, l);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
  nan_seen = __builtin_amdgcn_readfirstlane(__ballot(nan_seen) != 0ull ? 1 : 0) != 0;

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  const bool empty = M == neg_inf();
  if (!empty && !nan_seen) {
    const float Ml = M * kLog2e;
    for (int s0 = 0; s0 < n; s0 += 64) {
      // this pass's splits: lane s holds w_{s0 + s}; the used ones as a bit mask
      const float l = lse_pass(s0);
      const float w = l == neg_inf() ? 0.f : fast_exp2(l * kLog2e - Ml);
      uint64_t used = __ballot(l != neg_inf());
      while (used != 0ull) {
        // up to four used splits: all loads first, then the sums
        int idx[4];
        int nb = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          idx[j] = used != 0ull ? __builtin_ctzll(used) : -1;
          if (used != 0ull) {
            used &= used - 1;
            ++nb;
          }
        }
        float v[4][E];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float* slot = base + (int64_t)(s0 + (idx[j] < 0 ? idx[0] : idx[j])) * stride + lane * E;
#pragma unroll
          for (int e = 0; e < E; ++e) v[j][e] = slot[e];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < nb) {
            const float wj = readlane(w, idx[j]);
            wsum += wj;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += wj * v[j][e];
          }
        }
      }
    }
  }

  float den = wsum;
  if (a.sinks != nullptr && !empty) den += fast_exp2(a.sinks[h] * kLog2e - M * kLog2e);
  const float inv = empty ? 0.f : 1.f / den;
  uint16_t* orow = a.out + (int64_t)row * a.o_srow + (int64_t)h * a.o_sh + lane * E;
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int e = 0; e < E; e += 2) {
    float x0 = nan_seen ? qnan : acc[e] * inv;
    float x1 = nan_seen ? qnan : acc[e + 1] * inv;
    *(uint32_t*)(orow + e) = pack_bf16x2(x0, x1);
  }
  if (a.lse != nullptr && lane == 0) {
    float v = empty ? neg_inf() : M + fast_log2(wsum) * kLn2;
    a.lse[(int64_t)row * a.lse_srow + h] = nan_seen ? qnan : v;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.rows * a.H;
  if (pairs == 0) return hipSuccess;
  dim3 grid((unsigned)((pairs + kWaves - 1) / kWaves)), block(kWaves * 64);
  switch (a.Dv / 64) {
    case 2: hipLaunchKernelGGL(merge_kernel<2>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(merge_kernel<4>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(merge_kernel<8>, grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL(merge_kernel<16>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pd
