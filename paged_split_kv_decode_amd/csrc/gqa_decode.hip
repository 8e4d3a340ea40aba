// Paged GQA split-KV decode for gfx950 (one query token per request).
//
// Operation: "vllm.models.flint.ops.decode_attention", flint_decode_attention
// and _FlintDecodeAttention.kernel (page range of a request, sliding-window
// start, per-split page interleave, intra-workgroup combine, sink in the final
// denominator); block-table addressing as in "Atención paginada", decode path.
//
// Design on CDNA4
// ---------------
// * One workgroup of 4 waves per (split, kv head, request).  The split's
//   32-token tiles are interleaved over the waves; each wave streams its
//   tiles through a private 2-stage LDS ring and keeps its own online-softmax
//   state, so the hot loop needs no workgroup barrier.
// * Page gather: a tile is 32 token rows of [K | V] (512 B each, 16 KB per
//   tile).  Each wave moves it with 16 `global_load_lds_dwordx4`
//   instructions (1 KB per instruction, HBM -> LDS with no VGPR staging);
//   the physical page of every row comes from the block table with scalar
//   loads.  16-byte chunks are XOR-swizzled per row so the MFMA operand reads
//   below are bank-conflict free.
// * Scores S^T[token, head] = K . Q^T on v_mfma_f32_16x16x32_bf16 with the
//   query heads of the kv head in the N dimension (G <= 16, padded with zero
//   heads).  Each lane then holds 8 scores of one head.
// * Online softmax in fp32 with exp2 and a running max in unscaled logits;
//   the max is reduced over the 4 lanes of a head with two lane exchanges,
//   the row sum is kept per lane and reduced once at the end.
// * P is rounded to bf16 and is already in the B-operand layout of the
//   P.V product O^T[d, head] += V^T . P^T; V^T comes from the LDS tile with
//   `ds_read_b64_tr_b16` (transposing 4x16 bf16 blocks on the fly).
// * Keys outside [lo, hi) get a -inf score and a zero V (select, never a
//   multiply), so stale or NaN cache contents never reach the output.
// * The waves' (m, l, O) are combined through LDS; a single split writes
//   bf16 O and LSE, several splits write fp32 (O/l, lse) partials for the
//   merge kernel.
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "kernels.h"

namespace pd {
namespace {

constexpr int kD = 128;
constexpr int kRowBytes = 2 * kD * 2;                   // K|V row of one token
constexpr int kTileBytes = kTileTokens * kRowBytes;     // 16 KB
constexpr int kLoadsPerTile = kTileBytes / (64 * 16);   // 16 wave loads
constexpr int kCombHeadStride = kD + 4;                 // floats, padded
constexpr int kCombWaveFloats = 16 * kCombHeadStride + 48;

// 16-byte chunk c of token row r is stored at chunk c ^ swz(r).  Rows
// 0..7 get distinct low-3-bit patterns (K reads: 8 consecutive rows, same
// chunk) and rows 4k..4k+3 distinct bits 2:1 (V transpose reads: 4 rows x a
// 32-byte chunk pair).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

__device__ __forceinline__ uint32_t keep_mask(bool lo_ok, bool hi_ok) {
  return (lo_ok ? 0x0000FFFFu : 0u) | (hi_ok ? 0xFFFF0000u : 0u);
}

// kNW waves per workgroup, kNS ring stages (tiles) per wave.
template <int P, int kNW, int kNS>
__global__ __launch_bounds__(kNW * 64) void gqa_decode_kernel(GqaArgs a) {
  constexpr int kLdsBytes = kNW * kNS * kTileBytes;
  static_assert(kLdsBytes >= kNW * kCombWaveFloats * 4, "combine buffer must fit the ring");
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  PD_LDS char* lds = (PD_LDS char*)smem;

  const int tid = threadIdx.x;
  // wave index as an SGPR value: everything derived from it stays scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int G = a.G;
  const int S = a.S;
  const bool direct = S == 1 && !a.partials;   // write O / LSE, no workspace
  const int hq0 = kvh * G;
  const float c = a.scale_log2;

  // ---- key range of this request and the split plan --------------------
  int L = as_const(a.seq_lens)[b];
  L = min(max(L, 0), a.max_blocks * P);
  const int hi = L;
  const int lo = a.window > 0 ? max(hi - a.window, 0) : 0;
  const int t_first = lo >> 5;
  const int n_tiles = hi > lo ? ((hi + 31) >> 5) - t_first : 0;
  int chunk = 1, active = 0;
  if (n_tiles > 0) {
    // (integer division runs on the VALU: pin the results to SGPRs)
    chunk = __builtin_amdgcn_readfirstlane(max((n_tiles + S - 1) / S, kGqaMinSplitTiles));
    active = __builtin_amdgcn_readfirstlane((n_tiles + chunk - 1) / chunk);
  }

  if (split >= active) {
    // Nothing to attend in this slot: zeros / -inf (direct), or an empty
    // partial (lse = -inf) for the merge.
    if (direct) {
      for (int i = tid; i < G * (kD / 8); i += kNW * 64) {
        const int h = i / (kD / 8), d8 = (i % (kD / 8)) * 8;
        *(u32x4*)(a.out + (int64_t)b * a.o_sb + (int64_t)(hq0 + h) * a.o_sh + d8) = u32x4{0, 0, 0, 0};
      }
      if (a.lse != nullptr && tid < G) a.lse[(int64_t)b * a.lse_sb + hq0 + tid] = neg_inf();
    } else if (tid < G) {
      a.ws[((int64_t)(b * a.Hq + hq0 + tid) * S + split) * (kD + 1) + kD] = neg_inf();
    }
    return;
  }

  const int tb = t_first + split * chunk;
  const int te = min(tb + chunk, t_first + n_tiles);
  const int nst = te - tb;
  const int n_w = __builtin_amdgcn_readfirstlane(nst > wave ? (nst - wave + kNW - 1) / kNW : 0);
  const int pg_lo = lo / P;
  const int pg_hi = (hi + P - 1) / P;

  // ---- query fragment: B operand of S^T = K Q^T -------------------------
  bf16x8 qf[4];
  {
    const bool hv = l16 < G;
    const uint16_t* qrow = a.q + (int64_t)b * a.q_sb + (int64_t)(hq0 + (hv ? l16 : 0)) * a.q_sh;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = *(const u32x4*)(qrow + 8 * g4 + 32 * s);
      if (!hv) v = u32x4{0, 0, 0, 0};
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const char* kv_head = (const char*)(a.kv + (int64_t)kvh * a.kv_sh);
  PD_LDS char* ring = lds + wave * kNS * kTileBytes;
  const PD_CONST int32_t* bt_row = as_const(a.bt) + (int64_t)b * a.bt_sb;
  bool bad = false;

  // Issue the 16 HBM->LDS loads of tile T into ring slot `slot`.
  auto issue = [&](int T, int slot) {
    constexpr int PPT = P >= kTileTokens ? 1 : kTileTokens / P;   // pages per tile
    PD_LDS char* dst = ring + slot * kTileBytes;
    const int tok0 = T * kTileTokens;
    int pid[PPT];
    bool pok[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int pidx = tok0 / P + j;
      bool ok = pidx >= pg_lo && pidx < pg_hi;
      int id = ok ? bt_row[pidx] : 0;
      if (ok && (id < 0 || id >= a.num_pages)) {
        bad = true;
        ok = false;
      }
      pid[j] = id;
      pok[j] = ok;
    }
    const int cs = lane & 31;
#pragma unroll
    for (int i = 0; i < kLoadsPerTile; ++i) {
      constexpr int kRowsPerLoad = 2;
      const int j = P >= kTileTokens ? 0 : (kRowsPerLoad * i) / P;
      if (!pok[j]) continue;
      // uniform page base (SGPR pair) + 32-bit per-lane byte offset
      const char* page_base = kv_head + (int64_t)pid[j] * a.kv_sp * 2;
      const int r = kRowsPerLoad * i + (lane >> 5);
      const uint32_t slot_tok = (uint32_t)((tok0 + r) & (P - 1));
      const uint32_t ch = (uint32_t)(cs ^ swz(r));
      global_to_lds_16(page_base, (slot_tok * (2 * kD) + ch * 8) * 2, lds_addr(dst + i * 1024));
    }
  };

  float m_run = neg_inf();
  float l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue
#pragma unroll
  for (int k = 0; k < kNS - 1; ++k)
    if (k < n_w) issue(tb + wave + k * kNW, k);

  for (int k = 0; k < n_w; ++k) {
    const int kn = k + kNS - 1;
    if (kn < n_w) {
      wait_lgkmcnt0();  // this slot's LDS reads of the previous tile are done
      issue(tb + wave + kn * kNW, kn % kNS);
    }
    if (kn >= n_w - 1)
      wait_vmcnt<0>();
    else
      wait_vmcnt<kLoadsPerTile * (kNS - 1)>();

    const int T = tb + wave + k * kNW;
    const int tok0 = T * kTileTokens;
    PD_LDS char* tl = ring + (k % kNS) * kTileBytes;

    // ---- scores ----
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const int sw = swz(l16);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = (g4 + 4 * s) ^ sw;
      bf16x8 k0 = *(PD_LDS bf16x8*)(tl + l16 * kRowBytes + ch * 16);
      bf16x8 k1 = *(PD_LDS bf16x8*)(tl + (16 + l16) * kRowBytes + ch * 16);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[s], s1, 0, 0, 0);
    }

    const bool edge = tok0 < lo || tok0 + kTileTokens > hi;
    bool v0[4], v1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t0 = tok0 + 4 * g4 + i, t1 = t0 + 16;
      v0[i] = !edge || (t0 >= lo && t0 < hi);
      v1[i] = !edge || (t1 >= lo && t1 < hi);
      if (!v0[i]) s0[i] = neg_inf();
      if (!v1[i]) s1[i] = neg_inf();
    }

    // ---- online softmax (fp32, exp2, running max in unscaled logits) ----
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_ref = m_new == neg_inf() ? 0.f : m_new;
    const float mc = m_ref * c;
    const float alpha = fast_exp2(m_run * c - mc);
    float p0[4], p1[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0[i] = fast_exp2(s0[i] * c - mc);
      p1[i] = fast_exp2(s1[i] * c - mc);
      psum += p0[i] + p1[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;

    // P^T as the B operand: k = 8*g4 + j <-> tokens 4*g4 + j (j < 4) and
    // 16 + 4*g4 + (j - 4) (j >= 4), exactly this lane's scores.
    const u32x4 pw = {pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]),
                      pack_bf16x2(p1[0], p1[1]), pack_bf16x2(p1[2], p1[3])};
    const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
    const u32x4 vkeep = {keep_mask(v0[0], v0[1]), keep_mask(v0[2], v0[3]),
                         keep_mask(v1[0], v1[1]), keep_mask(v1[2], v1[3])};

    // ---- O^T += V^T P^T ----
    const int ra = 4 * g4 + (l16 >> 2);
    const int rb = ra + 16;
    const int swa = swz(ra);
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int ch = 16 + 2 * blk + ((l16 & 3) >> 1);
      const int within = (l16 & 1) * 8;
      bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (PD_LDS bf16x4*)(tl + ra * kRowBytes + ((ch ^ swa) << 4) + within));
      bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (PD_LDS bf16x4*)(tl + rb * kRowBytes + ((ch ^ swa) << 4) + within));
      u32x2 ua = __builtin_bit_cast(u32x2, va);
      u32x2 ub = __builtin_bit_cast(u32x2, vb);
      u32x4 vv = {ua[0], ua[1], ub[0], ub[1]};
      if (edge) vv &= vkeep;
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf, o[blk], 0, 0, 0);
    }
  }

  // ---- per-wave row sums, then the workgroup combine through LDS --------
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);

  __syncthreads();  // every wave is done with its ring
  float* comb = (float*)smem;
  {
    float* wb = comb + wave * kCombWaveFloats;
#pragma unroll
    for (int blk = 0; blk < 8; ++blk)
      *(f32x4*)(wb + l16 * kCombHeadStride + 16 * blk + 4 * g4) = o[blk];
    if (g4 == 0) {
      wb[16 * kCombHeadStride + l16] = m_run;
      wb[16 * kCombHeadStride + 16 + l16] = l_run;
    }
    if (lane == 0) wb[16 * kCombHeadStride + 32] = bad ? 1.f : 0.f;
  }
  __syncthreads();

  bool any_bad = false;
#pragma unroll
  for (int w = 0; w < kNW; ++w) any_bad |= comb[w * kCombWaveFloats + 16 * kCombHeadStride + 32] != 0.f;

  for (int idx = tid; idx < G * (kD / 4); idx += kNW * 64) {
    const int h = idx / (kD / 4);
    const int d4 = (idx % (kD / 4)) * 4;
    float mw[kNW];
    float m_all = neg_inf();
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      mw[w] = comb[w * kCombWaveFloats + 16 * kCombHeadStride + h];
      m_all = fmaxf(m_all, mw[w]);
    }
    float l_all = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float corr = mw[w] == neg_inf() ? 0.f : fast_exp2((mw[w] - m_all) * c);
      l_all += corr * comb[w * kCombWaveFloats + 16 * kCombHeadStride + 16 + h];
      const f32x4 ow = *(const f32x4*)(comb + w * kCombWaveFloats + h * kCombHeadStride + d4);
      acc += corr * ow;
    }
    const bool empty = !(l_all > 0.f);
    const float lse_nat = empty ? neg_inf() : (m_all * c + fast_log2(l_all)) * kLn2;
    if (direct) {
      float den = l_all;
      if (a.sinks != nullptr && !empty) den += fast_exp2(a.sinks[hq0 + h] * kLog2e - m_all * c);
      const float inv = empty ? 0.f : 1.f / den;
      f32x4 r = acc * inv;
      if (any_bad) r = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      u32x2 packed = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      *(u32x2*)(a.out + (int64_t)b * a.o_sb + (int64_t)(hq0 + h) * a.o_sh + d4) = packed;
      if (a.lse != nullptr && d4 == 0)
        a.lse[(int64_t)b * a.lse_sb + hq0 + h] = any_bad ? __builtin_nanf("") : lse_nat;
    } else {
      const float inv = empty ? 0.f : 1.f / l_all;
      float* slot = a.ws + ((int64_t)(b * a.Hq + hq0 + h) * S + split) * (kD + 1);
      f32x4 r = acc * inv;
      if (any_bad) r = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
#pragma unroll
      for (int e = 0; e < 4; ++e) slot[d4 + e] = r[e];
      if (d4 == 0) slot[kD] = any_bad ? __builtin_nanf("") : lse_nat;
    }
  }
}

}  // namespace

template <int NW, int NS>
static hipError_t launch_variant(const GqaArgs& a, hipStream_t stream) {
  dim3 grid(a.S, a.Hkv, a.B), block(NW * 64);
  switch (a.P) {
    case 16: hipLaunchKernelGGL((gqa_decode_kernel<16, NW, NS>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((gqa_decode_kernel<32, NW, NS>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tuning override for sweeps (never needed for correctness): PD_GQA_TUNE =
// "<waves>x<stages>" picks another compiled (waves, ring stages) variant.
static int tune_variant() {
  static int v = [] {
    const char* e = getenv("PD_GQA_TUNE");
    if (e == nullptr) return 0;
    if (!strcmp(e, "4x2")) return 0;
    if (!strcmp(e, "2x2")) return 1;
    if (!strcmp(e, "2x4")) return 2;
    if (!strcmp(e, "2x3")) return 3;
    if (!strcmp(e, "1x4")) return 4;
    return 0;
  }();
  return v;
}

hipError_t launch_gqa_decode(const GqaArgs& a, hipStream_t stream) {
  switch (tune_variant()) {
    case 1: return launch_variant<2, 2>(a, stream);
    case 2: return launch_variant<2, 4>(a, stream);
    case 3: return launch_variant<2, 3>(a, stream);
    case 4: return launch_variant<1, 4>(a, stream);
    default: return launch_variant<4, 2>(a, stream);
  }
}

}  // namespace pd
