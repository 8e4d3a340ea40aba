// Paged GQA split-KV decode for gfx950 (one query token per request).
//
// Operation: "vllm.models.flint.ops.decode_attention", flint_decode_attention
// and _FlintDecodeAttention.kernel (key range of a request, sliding-window
// start, per-split partials, sink in the final denominator); block-table
// addressing as in "Atención paginada", section "Ruta de decodificación".
//
// Design on CDNA4: a persistent, length-balanced stream
// -----------------------------------------------------
// * Work unit = (request b, kv head); its keys are cut into 32-token tiles
//   (tile t covers positions [32t, 32t + 32), clipped to the request's key
//   range).  All units' tiles, request-major then kv-head-major, form one
//   flat sequence of U tiles.  The grid is one workgroup per compute unit
//   (4 waves; 8 for FP8 decode), and every wave takes an equal contiguous
//   share of that sequence, so the waves finish together whatever the
//   length mix.
// * A wave streams its share as one pipeline that runs straight across unit
//   boundaries: it has a private ring in LDS (bf16: 2 slots of 16 KB; FP8:
//   2 or 4 slots of 8 KB) and issues the next tiles
//   (`global_load_lds_dwordx4`, 1 KB each, HBM -> LDS with no VGPR staging,
//   non-temporal: the cache is read once) while it computes tile k.  The physical page of
//   each tile row comes from the block table through scalar loads made one
//   tile ahead of their use, so their latency is hidden.  The waves share
//   nothing but the CU (one workgroup barrier exists, in pair mode below).
// * Where a wave's share cuts a unit, each piece is a split: the wave writes
//   its fp32 partial (O / l, lse) to the piece's slot, and the merge kernel
//   combines them.  With the split cap S >= 2 the share size is raised
//   until no unit spans more than S waves; the wave that holds a unit's
//   first tile marks the end of the unit's slot list.  With S == 1 shares
//   are rounded to whole units and the wave writes O and LSE directly.
// * With S == 1 and no more units than waves, each wave takes one unit
//   without scanning the batch (unit mode); with at most two units per
//   compute unit, two waves of a workgroup take half a unit each and merge
//   through LDS (pair mode).
// * Scores S^T[token, head] = K . Q^T on v_mfma_f32_16x16x32_bf16 with the
//   G query heads of the kv head in the N dimension (G <= 16, zero-padded).
//   Online softmax in fp32 with exp2 and a reference max in unscaled logits
//   (moved, with a rescale, only when a score passes it by 2^8),
//   reduced over the 4 lanes of a head with two lane swaps
//   (v_permlane16_swap, v_permlane32_swap).  P (bf16) is already in the
//   B-operand layout of O^T[d, head] += V^T . P^T, and V^T is read from the
//   LDS tile with ds_read_b64_tr_b16 (FP8: ds_read_b64_tr_b8, then an exact
//   in-register conversion to bf16), ahead of the softmax so that the LDS
//   latency overlaps it.
// * Keys outside [lo, hi) get a -inf score and a zero V (select, never a
//   multiply), so stale or NaN cache contents never reach the output.  A
//   block-table entry outside [0, num_pages) is never dereferenced: its
//   rows are loaded from a harmless address and the piece's result is NaN.
#pragma once

#include <algorithm>
#include <utility>

#include "device_common.h"
#include "kernels.h"

namespace pd {
namespace {

constexpr int kD = 128;
// Waves per workgroup: 4 (one per SIMD, a 2-tile bf16 ring each), or 8 for
// the FP8 cache (two per SIMD, so one wave's per-tile conversions and
// products overlap the other's waits; a 2-tile FP8 ring and one query slot
// each keep the 8 waves within the CU's LDS).
__host__ __device__ constexpr int gqa_waves(bool f8, int nc) { return (f8 && nc == 1) ? 8 : 4; }
constexpr int kRowBytes = 2 * kD * 2;                   // K|V row of one token (bf16)
constexpr int kTileBytes = kTileTokens * kRowBytes;     // 16 KB
constexpr int kRowBytes8 = 2 * kD;                      // K|V row of one token (FP8)
constexpr int kTileBytes8 = kTileTokens * kRowBytes8;   // 8 KB
// Ring of a wave: bf16, 2 tiles of 16 KB (one computed, one loading); FP8,
// 4 tiles of 8 KB (one computed, up to three loading) with 4 waves per
// workgroup, 2 tiles with 8.

// LDS bank model (measured with the SQ_LDS_BANK_CONFLICT counter on
// MI355X): 64 banks of 4 bytes; an 8-byte-per-lane read (ds_read_b64, the
// transpose reads) serves 32 lanes per cycle, which must then touch the 16
// distinct 16-byte slots of a 256-byte bank row in both 8-byte halves.
//
// FP8 tile: 16-byte chunk c of token row r (256 bytes, one bank row) is
// stored at chunk c ^ f8(r).  f8 is a permutation of rows 0..15 and of
// 16..31 (K reads: 32 lanes = 16 rows x 2 halves of one chunk) and of the 16
// rows {0..7, 16..23} and {8..15, 24..31} (V^T transpose reads: the first
// and the second 32 lanes read 16 such rows, 2 halves each).
__device__ __forceinline__ int f8(int r) { return (r & 7) | ((((r >> 3) ^ (r >> 4)) & 1) << 3); }
// 1 KB of zeros in device memory: the source of rows of pages that are not
// read in the general page class (any 16-byte chunk of a 512-byte row stays
// inside it).
__device__ __attribute__((aligned(1024))) uint32_t g_zero_rows[256];

// Smallest share a wave takes, in tiles.  Short units (a sliding window of
// 128 keys is 4-5 tiles) are latency-bound, and smaller shares let more
// waves stream at once: 2 measured 6% faster than 4 at the window config
// (11.9 against 12.7 us per call).
constexpr int kMinWaveTiles = 2;
// How far (log2 units of exp2) a score may pass a column's reference max
// before the reference moves: the rescale of O and l (32 multiplies per
// column group) then runs only on the few tiles that raise the max by that
// much, and probabilities stay below 2^8 (with the relative precision they
// have below 1).
constexpr float kRescaleLog2 = 8.f;
// Every wave takes an equal share.  (Shares skewed by a fixed amount
// between even and odd XCDs, which had streamed at different rates, lost
// against equal shares with this kernel: at 2, 3, 4, 6, 8, 10 and 12% on the
// skewed decode batch, at 2 and 8% on the sinks, verify and 8-token-page
// decode workloads; 1.4-2.2% at 8%.)

// bf16 tile: 16-byte chunk c of token row r (512 bytes, two bank rows) is
// stored at chunk c ^ swz(r), inside the row's K or V half.  swz permutes
// rows 0..15 (K reads: 16 rows, one chunk) and its bits 3:1 permute each 8
// consecutive rows (V^T transpose reads: 32 lanes = 8 rows x a chunk pair
// x 2 halves).  The earlier 3-bit swizzle repeated every 8 rows and left
// every transpose read 2-way conflicted.
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ uint32_t keep_mask(bool lo_ok, bool hi_ok) {
  return (lo_ok ? 0x0000FFFFu : 0u) | (hi_ok ? 0xFFFF0000u : 0u);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Key range of one request: positions [lo, hi), tiles lo / 32 ... lo / 32 + nt - 1.
struct Req {
  int lo, hi, nt;
  int n, row0;   // query rows of the request: n tokens from row row0
  int L;         // seq_lens[b] as given, less len_sub (the fused append's tokens end there)
};

// Length bound standing for "no real length given".
constexpr int kNoReal = 1 << 30;

// Key range of verify row t of a request with n query tokens, length L
// (clamped to the block-table row) and real length Lr: [lo_t, hi_t) with
// hi_t = max(min(L - n + 1 + t, Lr), 0) and, with a window,
// lo_t = max(hi_t - window, 0).  A slice of longer verify rows (len_sub
// tokens after it) takes L - len_sub for L after the clamp.
__device__ __forceinline__ int row_hi(const GqaArgs& a, int L, int Lr, int t, int n) {
  L = min(max(L, 0), a.max_blocks * a.P) - a.len_sub;
  return max(min(L - n + 1 + t, Lr), 0);
}
__device__ __forceinline__ int row_lo(const GqaArgs& a, int hi) {
  return a.window > 0 ? max(hi - a.window, 0) : 0;
}

// Keys of a request with n >= 0 query tokens: the union of its rows'
// ranges, [lo_0, hi_{n-1}) (none for n = 0).
__device__ __forceinline__ Req range_of(const GqaArgs& a, int L, int Lr, int n) {
  Req r;
  r.n = n;
  r.row0 = 0;
  r.L = L - a.len_sub;
  r.hi = n > 0 ? row_hi(a, L, Lr, n - 1, n) : 0;
  r.lo = row_lo(a, row_hi(a, L, Lr, 0, n));
  r.nt = r.hi > r.lo ? ((r.hi + 31) >> 5) - (r.lo >> 5) : 0;
  return r;
}

// Query rows of request b: rows row0 .. row0 + n - 1.  Uniform: b *
// q_req_rows + t_off and qlen.  Variable ("cumulative query lengths"): cu_q[b] .. cu_q[b + 1] - 1,
// clamped to [0, total_rows) and to at most qlen rows (the column bound).
struct QRows {
  int row0, n;
};
__device__ __forceinline__ QRows query_rows(const GqaArgs& a, int b) {
  if (a.cu_q == nullptr) return QRows{b * a.q_req_rows + a.t_off, a.qlen};
  const int r0 = min(max((int)as_const(a.cu_q)[b], 0), a.total_rows);
  const int r1 = min(max((int)as_const(a.cu_q)[b + 1], r0), a.total_rows);
  return QRows{r0, min(r1 - r0, a.qlen)};
}

// Variable query length: request b has more query rows than the max_qlen
// bound (its rows are then all NaN, as for an invalid block-table entry).
__device__ __forceinline__ bool rows_over_bound(const GqaArgs& a, int b, const QRows& qr) {
  if (a.cu_q == nullptr) return false;
  const int r1 = min(max((int)as_const(a.cu_q)[b + 1], qr.row0), a.total_rows);
  return r1 - qr.row0 > qr.n;
}

__device__ __forceinline__ int real_len(const GqaArgs& a, int b) {
  return a.real_lens != nullptr ? (int)as_const(a.real_lens)[b] : kNoReal;
}

// V: the verify instantiation (query rows from query_rows); decode: one
// query row per request, row b.
template <bool V>
__device__ __forceinline__ Req request_range(const GqaArgs& a, int b) {
  const QRows qr = V ? query_rows(a, b) : QRows{b, 1};
  Req r = range_of(a, as_const(a.seq_lens)[b], real_len(a, b), qr.n);
  r.row0 = qr.row0;
  return r;
}

// A position in one wave's tile sequence (wave-uniform).  b == B: the share
// is done.
struct Cursor {
  int b, kvh;   // unit
  int p0;       // flat index of the unit's first tile
  int i, i_end; // current tile of the unit, end of this wave's piece of it
  Req r;
};

// The wave's share of the flat tile sequence.
struct Share {
  int g0, g1;   // [g0, g1): raw share (the last used wave also owns every unit past g1)
  int t;        // tiles per share
  bool last;
  bool split;   // S >= 2: pieces may cut units; S == 1: whole units only
  bool range;   // the cursor keeps to [g0, g1) inside units (split, or a pair's half)
  int64_t u_end;   // unit mode: units from this index on are another wave's
  // first tile of the share of wave j, and the share holding tile p
  __device__ int start(int j) const { return j * t; }
  __device__ int of(int p) const { return p / t; }
};

constexpr int kQSlotBytes = 16 * kD * 2;                 // query rows of one piece (16 columns)
constexpr int kCachedChunks = 4;                          // request lengths kept in registers (x64)

// V: verify rows (qlen > 1 or real lengths); the decode instantiation has a
// single column range per unit and none of the per-column limit work.
// PS: the page class.  1, 2, 4, 8 or 16: the page size itself (pages
// smaller than a tile); 32: any power-of-two page of 32 tokens or more (a
// tile then lies inside one page; log2 of the size comes in a.p_shift);
// 0: any other page size of 3 tokens or more (a tile spans at most 12 pages
// and a load's 2 or 4 rows at most 2).
// NC: score column groups of 16 (verify: qlen * G <= 16 NC columns; the
// verify tokens of all groups share each K and V tile as loaded).
// AP: the fused append (the new tokens' rows come from the sources a.kn /
// a.vn and are written into the cache).
template <int PS, bool V, bool F8, int NC, bool AP>
__global__ __launch_bounds__(gqa_waves(F8, NC) * 64) void gqa_decode_kernel(GqaArgs a) {
  static_assert(NC == 1 || (V && (NC == 2 || NC == 4)), "column groups: decode 1, verify 1, 2 or 4");
  constexpr int kSlotBytes = F8 ? kTileBytes8 : kTileBytes;     // one tile as loaded
  constexpr int kLoadsPerTile = kSlotBytes / (64 * 16);         // 16 (bf16) or 8 (FP8) loads
  constexpr int kNW = gqa_waves(F8, NC);
  constexpr int kSlots = F8 ? (kNW == 8 ? 2 : 4) : 2;           // ring slots
  constexpr int kQSlots = kNW == 8 ? 1 : 2;                      // query slots
  constexpr int kRingBytes = kSlots * kSlotBytes;
  constexpr int kWaveLds = kRingBytes + kQSlots * kQSlotBytes;   // 40 KB (4 waves), 20 KB (8)
  static_assert(kNW * kWaveLds <= 160 * 1024, "LDS of one workgroup per CU");
  __shared__ __attribute__((aligned(1024))) char smem[kNW * kWaveLds];

  const int tid = threadIdx.x;
  const int wave_in_wg = uniform(tid >> 6);
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int l16 = lane & 15;
  const int G = a.G;
  // columns in use: (verify token, head) pairs of the current piece (verify:
  // n * G for a request with n query rows; decode: the G heads)
  int R = G;
  const int S = a.S;
  const int Hkv = a.Hkv;
  const bool direct = S == 1 && !a.partials;
  float c = a.scale_log2;   // per piece: times the kv head's k_scale for FP8
  float v_mult = 1.f;        // per piece: the kv head's v_scale for FP8
  const int n_waves = gridDim.x * kNW;
  const int w = uniform(blockIdx.x * kNW + wave_in_wg);
  PD_LDS char* ring = (PD_LDS char*)smem + wave_in_wg * kWaveLds;
  PD_LDS char* qslots = ring + kRingBytes;
  // this lane's score column of group c: verify token t_col[c], head g_col[c]
  // of the kv head (column 16 c + l16)
  int t_col[NC], g_col[NC];
#pragma unroll
  for (int cg = 0; cg < NC; ++cg) {
    t_col[cg] = 0;
    g_col[cg] = 16 * cg + l16;
  }

  // ---- the plan ----------------------------------------------------------
  Share sh;
  int b_s = -1, kvh_s = 0, p0_s = 0;
  Req r_s;
  // Whole units with no more units than waves: one unit per wave, the best
  // whole-unit schedule whatever the lengths, and no wave scans the batch.
  // Unit j goes to wave j / grid of workgroup j % grid, so the busy waves
  // spread over every compute unit (the launch has no more workgroups than
  // units): a window decode of 512 units ran 11% slower on 4 waves of 128
  // workgroups than on 2 waves of 256.
  // Pair mode (a.pair, set by the launcher for at most two units per four
  // waves): unit j goes to waves 2 (j / grid) and 2 (j / grid) + 1 of
  // workgroup j % grid, the first streaming its first ceil(nt / 2) tiles, the
  // second the rest; the second hands its (m, l, O) to the first through
  // LDS at the end, and the first merges and writes the unit's result.  A
  // wave with no unit still meets that workgroup barrier.
  const bool pair_mode = NC == 1 && a.pair != 0;
  const int half = pair_mode ? (wave_in_wg & 1) : 0;
  bool idle = false;
  const bool unit_mode = pair_mode || (S == 1 && (int64_t)a.B * Hkv <= n_waves);
  if (unit_mode) {
    const int j = uniform((pair_mode ? (wave_in_wg >> 1) : wave_in_wg) * (int)gridDim.x + (int)blockIdx.x);
    if (j >= a.B * Hkv) {
      if (!pair_mode) return;
      idle = true;
    }
    sh.split = false;
    sh.range = false;
    sh.t = 1;
    sh.g0 = 0;
    sh.g1 = INT32_MAX;
    sh.last = false;
    sh.u_end = j + 1;
    if (idle) {
      b_s = a.B;   // nothing to stream or to answer for
    } else {
      b_s = uniform(j / Hkv);
      kvh_s = uniform(j - b_s * Hkv);
      r_s = request_range<V>(a, b_s);
      r_s.lo = uniform(r_s.lo);
      r_s.hi = uniform(r_s.hi);
      r_s.nt = uniform(r_s.nt);
      r_s.n = uniform(r_s.n);
      r_s.row0 = uniform(r_s.row0);
      r_s.L = uniform(r_s.L);
      // flat positions are not needed: the cursor stops at unit j + 1 (the
      // unit's first flat tile is 0; a pair's half keeps to its tile range)
      if (pair_mode) {
        // (the first half's range ends past flat tile 0 even for a unit with
        // no tile, so its final pass still answers for that unit)
        const int h = (r_s.nt + 1) >> 1;
        sh.range = true;
        sh.g0 = uniform(half ? h : 0);
        sh.g1 = uniform(half ? r_s.nt : max(h, 1));
      }
    }
  } else {
  // ---- total tiles, longest request, this wave's share ------------------
  // Lane l of chunk c holds the length of request 64c + l (0 past the batch).
  int Lc[kCachedChunks], Lrc[kCachedChunks], Nc[kCachedChunks];
#pragma unroll
  for (int ch = 0; ch < kCachedChunks; ++ch) {
    const int b = 64 * ch + lane;
    Lc[ch] = b < a.B ? as_const(a.seq_lens)[b] : 0;
    Lrc[ch] = b < a.B ? real_len(a, b) : 0;
    Nc[ch] = b < a.B ? (V ? query_rows(a, b).n : 1) : 0;
  }
  int nt_sum = 0, nt_max = 0;
#pragma unroll
  for (int ch = 0; ch < kCachedChunks; ++ch) {
    if (64 * ch >= a.B) break;   // chunks past the batch add nothing
    const int nt = range_of(a, Lc[ch], Lrc[ch], Nc[ch]).nt;
    nt_sum += wave_sum(nt);
    nt_max = max(nt_max, wave_max(nt));
  }
  for (int base = 64 * kCachedChunks; base < a.B; base += 64) {
    const int nt = base + lane < a.B ? request_range<V>(a, base + lane).nt : 0;
    nt_sum += wave_sum(nt);
    nt_max = max(nt_max, wave_max(nt));
  }
  nt_sum = uniform(nt_sum);
  nt_max = uniform(nt_max);
  const int U = nt_sum * Hkv;
  sh.split = S >= 2;
  sh.range = sh.split;
  sh.u_end = INT32_MAX;
  // a unit of n tiles cut every t tiles at an arbitrary offset spans at
  // most floor((n - 1) / t) + 2 shares: keep that <= S
  const int t_min = sh.split ? max((nt_max - 1) / (S - 1) + 1, kMinWaveTiles) : kMinWaveTiles;
  sh.t = uniform(max((U + n_waves - 1) / n_waves, t_min));
  const int w_used = uniform(U > 0 ? sh.of(U - 1) + 1 : 1);
  if (w >= w_used) return;
  sh.g0 = sh.start(w);
  sh.last = w == w_used - 1;
  sh.g1 = sh.last ? U : sh.start(w + 1);

  // ---- first unit of the share ------------------------------------------
  // split: the unit holding tile g0, or an empty unit starting at or after
  // g0; whole units: the first unit starting at or after g0.
  int L_s = 0, Lr_s = 0, N_s = 0, cb_s = 0;
  {
    int C = 0;  // tiles of the requests before this chunk (one kv head)
    auto probe = [&](int base, int L, int Lr, int N) {
      const bool in = base + lane < a.B;
      const int nt = range_of(a, L, Lr, N).nt;
      const int incl = wave_incl_sum(nt);
      const int cb1 = (C + incl) * Hkv;     // flat start of request b + 1
      const int cb = cb1 - nt * Hkv;         // flat start of request b
      const bool pred = in && (sh.split ? (cb1 > sh.g0 || cb >= sh.g0)
                                        : (cb + (Hkv - 1) * nt >= sh.g0));
      const uint64_t m = __ballot(pred);
      if (m != 0) {
        const int l0 = __builtin_ctzll(m);
        b_s = base + l0;
        L_s = __builtin_amdgcn_readlane(L, l0);
        Lr_s = __builtin_amdgcn_readlane(Lr, l0);
        N_s = __builtin_amdgcn_readlane(N, l0);
        cb_s = __builtin_amdgcn_readlane(cb, l0);
        return true;
      }
      C += __builtin_amdgcn_readlane(incl, 63);
      return false;
    };
    bool found = false;
#pragma unroll
    for (int ch = 0; ch < kCachedChunks; ++ch)
      if (!found && 64 * ch < a.B) found = probe(64 * ch, Lc[ch], Lrc[ch], Nc[ch]);
    for (int base = 64 * kCachedChunks; !found && base < a.B; base += 64) {
      const bool in = base + lane < a.B;
      found = probe(base, in ? as_const(a.seq_lens)[base + lane] : 0, in ? real_len(a, base + lane) : 0,
                    in ? (V ? query_rows(a, base + lane).n : 1) : 0);
    }
  }
  if (b_s < 0) return;
  b_s = uniform(b_s);
  r_s = range_of(a, uniform(L_s), uniform(Lr_s), uniform(N_s));
  r_s.row0 = uniform(V ? query_rows(a, b_s).row0 : b_s);
  if (sh.g0 > cb_s)
    kvh_s = sh.split ? (sh.g0 - cb_s) / r_s.nt : (sh.g0 - cb_s + r_s.nt - 1) / r_s.nt;
  kvh_s = uniform(kvh_s);
  p0_s = uniform(cb_s + kvh_s * r_s.nt);
  }
  // the cursor has passed the share's last unit (unit mode)
  auto past_units = [&](const Cursor& cu) { return (int64_t)cu.b * Hkv + cu.kvh >= sh.u_end; };

  // Step to the next unit (no range checks).
  auto next_unit = [&](Cursor& cu) {
    cu.p0 += cu.r.nt;
    if (cu.kvh + 1 < Hkv) {
      ++cu.kvh;
    } else {
      cu.kvh = 0;
      ++cu.b;
      if (cu.b < a.B) cu.r = request_range<V>(a, cu.b);
    }
  };
  // Make the cursor point at a tile, skipping empty units; b = B once the
  // share is done.
  auto settle = [&](Cursor& cu) {
    for (;;) {
      if (cu.b >= a.B || (!sh.last && cu.p0 >= sh.g1) || past_units(cu)) {
        cu.b = a.B;
        return;
      }
      if (cu.r.nt > 0) {
        cu.i = sh.range ? max(sh.g0 - cu.p0, 0) : 0;
        cu.i_end = sh.range ? min(cu.r.nt, sh.g1 - cu.p0) : cu.r.nt;
        if (cu.i < cu.i_end) return;   // (a pair's empty second half: none)
      }
      next_unit(cu);
    }
  };
  // first tile of this wave's piece of the cursor's unit?
  auto piece_start = [&](const Cursor& cu) { return cu.i == (sh.range ? max(sh.g0 - cu.p0, 0) : 0); };
  auto advance = [&](Cursor& cu) {
    if (++cu.i < cu.i_end) return;
    next_unit(cu);
    settle(cu);
  };

  Cursor cc;  // tile being computed
  cc.b = b_s;
  cc.kvh = kvh_s;
  cc.p0 = p0_s;
  cc.r = r_s;
  settle(cc);
  Cursor ci = cc;  // next tile to issue

  // ---- block-table entries of one tile (scalar loads) -------------------
  constexpr bool kGen = PS == 0;
  constexpr bool kBig = PS >= kTileTokens;
  // General pages: a window of 16 consecutive entries from the tile's first
  // page, of which a tile of 32 rows uses at most 12 (pages of 3 tokens or
  // more).
  constexpr int kGenWindow = 16;
  constexpr int kGenPages = 12;
  constexpr int PPT = kGen ? kGenWindow : kBig ? 1 : kTileTokens / (PS > 0 ? PS : 1);   // pages per tile
  // Pages of 1, 2 or 4 tokens (8 or more per tile): each lane computes its
  // own row's source address and checks in vector registers; larger
  // power-of-two pages keep a per-page scalar address and check.  General
  // pages also use per-lane addresses.
  constexpr bool kLaneAddr = !kGen && !kBig && PS <= 4;
  const int p_shift = kBig ? a.p_shift : kGen ? 0 : __builtin_ctz(PS > 0 ? PS : 1);
  auto tile_tok0 = [&](const Cursor& cu) { return ((cu.r.lo >> 5) + cu.i) * kTileTokens; };
  // The entries are only checked when the tile is issued, so the scalar
  // loads stay in flight for a whole iteration.  Only entries of attended
  // pages are read (lane-address classes: clamped to the last attended
  // page), so every read stays inside the request's block-table row.
  struct TilePages {
    int id[PPT];
    bool att[(kLaneAddr || kGen) ? 1 : PPT];   // page attended (scalar classes)
    int first;                                 // general pages: page of the tile's first row
  };
  auto fetch_pages = [&](const Cursor& cu) {
    TilePages tp;
    const PD_CONST int32_t* bt_row = as_const(a.bt) + (int64_t)cu.b * a.bt_sb;
    if constexpr (kGen) {
      // entries of pages first .. first + 15, inside the row: one wide read
      // when the whole window lies in the row, else entry by entry clamped to
      // the last attended page (entries of pages not attended are never used)
      const int first = tile_tok0(cu) / a.P;
      tp.first = first;
      tp.att[0] = false;
      if (first + kGenWindow <= a.max_blocks) {
        typedef int32_t i32x8 __attribute__((ext_vector_type(8), aligned(4)));
        const PD_CONST i32x8* wv = (const PD_CONST i32x8*)(bt_row + first);
#pragma unroll
        for (int q = 0; q < kGenWindow / 8; ++q) {
          const i32x8 v = wv[q];
#pragma unroll
          for (int e = 0; e < 8; ++e) tp.id[8 * q + e] = v[e];
        }
      } else {
        const int last = (cu.r.hi - 1) / a.P;
#pragma unroll
        for (int j = 0; j < kGenWindow; ++j) tp.id[j] = bt_row[min(first + j, last)];
      }
      return tp;
    }
    tp.first = 0;
    const int pidx0 = tile_tok0(cu) >> p_shift;
    if constexpr (kLaneAddr) {
      if (PPT == 32 && pidx0 + PPT <= a.max_blocks) {
        // the tile's window of entries lies inside the row: consecutive
        // loads, merged into a few wide scalar loads (entries of pages
        // that are not attended are read but never used)
        typedef int32_t i32x8 __attribute__((ext_vector_type(8), aligned(4)));
        const PD_CONST i32x8* w = (const PD_CONST i32x8*)(bt_row + pidx0);
#pragma unroll
        for (int q = 0; q < (PPT + 7) / 8; ++q) {
          if constexpr (PPT == 32) {
            const i32x8 v = w[q];
#pragma unroll
            for (int e = 0; e < 8; ++e) tp.id[8 * q + e] = v[e];
          }
        }
      } else {
        const int last = (cu.r.hi - 1) >> p_shift;
#pragma unroll
        for (int j = 0; j < PPT; ++j) tp.id[j] = bt_row[min(pidx0 + j, last)];
      }
    } else {
      const int pg_lo = cu.r.lo >> p_shift, pg_end = ((cu.r.hi - 1) >> p_shift) + 1;
#pragma unroll
      for (int j = 0; j < PPT; ++j) {
        tp.att[j] = pidx0 + j >= pg_lo && pidx0 + j < pg_end;
        tp.id[j] = tp.att[j] ? bt_row[pidx0 + j] : 0;
      }
    }
    return tp;
  };
  TilePages pages_none;
#pragma unroll
  for (int j = 0; j < PPT; ++j) pages_none.id[j] = 0;
  pages_none.first = 0;
  if constexpr (!kLaneAddr && !kGen) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) pages_none.att[j] = false;
  } else {
    pages_none.att[0] = false;
  }

  // ---- HBM -> LDS loads of one tile (and of a new piece's query rows) ----
  // A tile is always exactly kLoadsPerTile loads (rows of a page that is not
  // read come from a harmless 16-byte source), so the vmcnt bookkeeping of
  // the ring is exact.  Query rows go to one of two LDS slots before the
  // tile's loads, so they have landed when the tile has.
  int q_issued = 0, q_used = 0;   // pieces whose query rows were loaded / read
  auto load_q = [&](const Cursor& cu) {
    const uint32_t dst = uniform((int)lds_addr(qslots + (q_issued % kQSlots) * kQSlotBytes));
    const char* qbase =
        (const char*)(a.q + (int64_t)cu.r.row0 * a.q_sb + (int64_t)cu.kvh * G * a.q_sh);
    const int chunk = lane & 15;
    const int Rq = V ? cu.r.n * G : G;   // the piece's columns
    for (int i = 0; i < (Rq + 3) / 4; ++i) {   // 4 columns (1 KB) per load
      const int n = min(4 * i + (lane >> 4), Rq - 1);
      const int t = n / G, g = n - t * G;
      const uint32_t voff = (uint32_t)(t * a.q_sb + g * a.q_sh + chunk * 8) * 2u;
      global_to_lds_16(qbase, voff, dst + i * 1024);
    }
    ++q_issued;
  };
  // Issues the tile's loads; returns whether an attended page has an
  // out-of-range entry (its rows then come from the harmless source).
  auto issue = [&](const Cursor& cu, const TilePages& tp, int slot) {
    // (more than 16 columns: the query fragments come straight from global
    // memory when the piece starts)
    if constexpr (NC == 1) {
      if (piece_start(cu)) load_q(cu);
    }
    const uint32_t dst = uniform((int)lds_addr(ring + slot * kSlotBytes));
    constexpr int kElem = F8 ? 1 : 2;
    constexpr uint32_t kRowB = 2 * kD * kElem;
    // Every kernel argument the loads need is read here, before the first
    // load: each load is an asm statement with a memory clobber, after which
    // the compiler would read the arguments again.
    const char* kv_head = (const char*)a.kv + (int64_t)cu.kvh * a.kv_sh * kElem;
    const int64_t sp_bytes = (int64_t)a.kv_sp * kElem;
    const uint32_t num_pages = (uint32_t)a.num_pages;
    const char* const harmless = (const char*)a.q;
    const int tok0 = tile_tok0(cu);
    // bf16: 2 rows of 32 chunks per load, chunks XOR-swizzled per row;
    // FP8: 4 rows of 16 chunks per load, plain
    constexpr int kRowsPerLoad = F8 ? 4 : 2;
    const int sub = F8 ? (lane >> 4) : (lane >> 5);   // this lane's row within a load
    // bf16: chunk c of row r at position c ^ swz(r); FP8: at c ^ f8(r)
    // (position = lane, so the lane fetches the chunk that lands there)
    auto chunk_of = [&](int r) {
      return F8 ? (uint32_t)((lane & 15) ^ f8(r)) : (uint32_t)((lane & 31) ^ swz(r));
    };
    // Fused append: rows of the request's newest n tokens (positions
    // L - n .. L - 1) are loaded from the new-token sources instead of the
    // cache (written only at the end of the kernel).  Such a tile takes
    // every load in the per-lane address form.
    const int new_lo = cu.r.L - cu.r.n, new_hi = cu.r.L;
    const bool has_new = AP && max(tok0, new_lo) < min(tok0 + kTileTokens, new_hi);
    const char* kn_u = nullptr;
    const char* vn_u = nullptr;
    int64_t kn_srow = 0, vn_srow = 0;
    if (has_new) {
      kn_srow = a.kn_srow;
      vn_srow = a.vn_srow;
      kn_u = a.kn + (int64_t)cu.r.row0 * kn_srow + (int64_t)cu.kvh * a.kn_sh;
      vn_u = a.vn + (int64_t)cu.r.row0 * vn_srow + (int64_t)cu.kvh * a.vn_sh;
    }
    // the source of this lane's chunk of row r of the tile (cache_src if
    // the row is not a new token)
    auto new_src = [&](int r, const char* cache_src) -> const char* {
      constexpr uint32_t kHalf = F8 ? 8u : 16u;   // K chunks of a row
      const int pos = tok0 + r;
      const int t = pos - new_lo;
      const uint32_t c = chunk_of(r);
      const bool kp = c < kHalf;
      const char* s = (kp ? kn_u : vn_u) + (int64_t)t * (kp ? kn_srow : vn_srow) +
                      (kp ? c : c - kHalf) * 16u;
      return pos >= new_lo && pos < new_hi ? s : cache_src;
    };
    // the tile's kLoadsPerTile loads, in the new-row form or not
    auto for_loads = [&](auto one) {
      if (has_new) {
        [&]<int... I>(std::integer_sequence<int, I...>) {
          (one(std::integral_constant<int, I>{}, std::true_type{}), ...);
        }(std::make_integer_sequence<int, kLoadsPerTile>{});
      } else {
        [&]<int... I>(std::integer_sequence<int, I...>) {
          (one(std::integral_constant<int, I>{}, std::false_type{}), ...);
        }(std::make_integer_sequence<int, kLoadsPerTile>{});
      }
    };
    bool bad_page = false;
    if constexpr (kGen) {
      // Every row's source address is computed once per tile, row rho by
      // lanes rho and 32 + rho; each load then fetches its rows' addresses
      // from those lanes with ds_bpermute.  A row of a page that is not read
      // points at a zero block in device memory, so the loads need no mask.
      const int P = a.P;
      // lane j: the entry of page first + j (a tile spans at most 12 pages)
      int win = 0;
#pragma unroll
      for (int j = 0; j < kGenPages; ++j) win = lane == j ? tp.id[j] : win;
      const int pg_lo = cu.r.lo / P, pg_end = (cu.r.hi - 1) / P + 1;   // attended pages
      const int s0 = tok0 - tp.first * P;   // slot of the tile's first row
      const int rho = lane & 31;
      const int e = (s0 + rho) / P;         // page of row rho, from the tile's first page
      const int slot = s0 + rho - e * P;
      const int id = __builtin_amdgcn_ds_bpermute(e << 2, win);
      const int pg = tp.first + e;
      const bool att = pg >= pg_lo && pg < pg_end;
      const bool inr = (uint32_t)id < num_pages;
      bad_page = __ballot(att && !inr) != 0;
      const uint64_t row_src =
          att && inr ? (uint64_t)(uintptr_t)(kv_head + (int64_t)id * sp_bytes + (uint32_t)slot * kRowB)
                     : (uint64_t)(uintptr_t)g_zero_rows;
      const int rs_lo = (int)(uint32_t)row_src, rs_hi = (int)(uint32_t)(row_src >> 32);
      // all the loads' addresses first (one wait for the lane exchanges),
      // then the loads
      uint32_t lo[kLoadsPerTile], hi[kLoadsPerTile];
#pragma unroll
      for (int i = 0; i < kLoadsPerTile; ++i) {
        const int r = kRowsPerLoad * i + sub;
        lo[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(r << 2, rs_lo);
        hi[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(r << 2, rs_hi);
      }
      __builtin_amdgcn_sched_barrier(0);
      auto one = [&](auto ic, auto nw) {
        constexpr int i = decltype(ic)::value;
        const int r = kRowsPerLoad * i + sub;
        const char* src =
            (const char*)(uintptr_t)(((uint64_t)hi[i] << 32) | lo[i]) + chunk_of(r) * 16;
        if constexpr (decltype(nw)::value) src = new_src(r, src);
        global_to_lds_16_stream_v<i * 1024>(src, dst);
      };
      for_loads(one);
    } else if constexpr (kLaneAddr) {
      // bit j: page j of the tile is attended
      const int pidx0 = tok0 >> p_shift;
      const int j_lo = min(max((cu.r.lo >> p_shift) - pidx0, 0), PPT);
      const int j_hi = min(max(((cu.r.hi - 1) >> p_shift) + 1 - pidx0, 0), PPT);
      const uint64_t att_mask = ((1ull << j_hi) - 1) & ~((1ull << j_lo) - 1);
      bool bad_lane = false;
      auto one = [&](auto ic, auto nw) {
        constexpr int i = decltype(ic)::value;
        const int r = kRowsPerLoad * i + sub;
        // the lane's row is in page j = r / PS of the tile: one of the
        // load's kCand pages
        constexpr int kCand = PS >= kRowsPerLoad ? 1 : kRowsPerLoad / PS;
        constexpr int j0 = (kRowsPerLoad * i) / PS;
        // The candidates are read as wave-uniform values first: a select
        // between array elements would otherwise be folded into one load at
        // a per-lane index, which puts the array in scratch memory.
        const int cand = kCand > 1 ? sub / PS : 0;
        int id = kCand > 1 ? uniform(tp.id[j0]) : tp.id[j0];
#pragma unroll
        for (int c = 1; c < kCand; ++c) {
          const int idc = uniform(tp.id[j0 + c]);
          id = cand == c ? idc : id;
        }
        const int j = j0 + cand;
        const bool att = (att_mask >> j) & 1;
        const bool inr = (uint32_t)id < num_pages;
        bad_lane |= att && !inr;
        const uint32_t off = (uint32_t)(r & (PS - 1)) * kRowB + chunk_of(r) * 16;
        const char* src = att && inr ? kv_head + id * sp_bytes + off : harmless;
        if constexpr (decltype(nw)::value) src = new_src(r, src);
        global_to_lds_16_stream_v<i * 1024>(src, dst);
      };
      for_loads(one);
      bad_page = __ballot(bad_lane) != 0;
    } else {
      bool ok[PPT];
      const char* pbase[PPT];
#pragma unroll
      for (int j = 0; j < PPT; ++j) {
        const bool inr = (uint32_t)tp.id[j] < num_pages;
        ok[j] = tp.att[j] && inr;
        bad_page |= tp.att[j] && !inr;
        pbase[j] = ok[j] ? kv_head + tp.id[j] * sp_bytes : harmless;
      }
      // token slot of the tile's first row in its page (a big page holds the
      // whole tile; smaller pages start on tile boundaries)
      const uint32_t slot0 = kBig ? (uint32_t)(tok0 & ((1 << p_shift) - 1)) : 0u;
      auto one = [&](auto ic, auto nw) {
        constexpr int i = decltype(ic)::value;
        const int r = kRowsPerLoad * i + sub;
        constexpr int j = kBig ? 0 : (kRowsPerLoad * i) / PS;   // every row of the load is in page j
        const uint32_t slot_tok = kBig ? slot0 + (uint32_t)r : (uint32_t)(r & (PS - 1));
        const uint32_t voff = ok[j] ? slot_tok * kRowB + chunk_of(r) * 16 : 0u;
        if constexpr (decltype(nw)::value)
          global_to_lds_16_stream_v<i * 1024>(new_src(r, pbase[j] + voff), dst);
        else
          global_to_lds_16_stream<i * 1024>(pbase[j], voff, dst);
      };
      for_loads(one);
    }
    return bad_page;
  };

  // ---- per-piece state ----------------------------------------------------
  bf16x8 qf[NC][4];
  float m_run[NC], l_run[NC];
  f32x4 o[NC][8];
  bool piece_bad = false;
  int bad_slots = 0;   // bit s: the tile in ring slot s read a bad page
  // keys of this lane's column (per group) in the current piece's request,
  // and the range every column attends (tiles inside it need no score mask)
  int col_lo[NC], col_hi[NC], all_lo = 0, all_hi = 0;
#pragma unroll
  for (int cg = 0; cg < NC; ++cg) {
    m_run[cg] = neg_inf();
    l_run[cg] = 0.f;
    col_lo[cg] = col_hi[cg] = 0;
  }
  // (a pair's second half may stream nothing: its accumulator is merged)
#pragma unroll
  for (int cg = 0; cg < NC; ++cg)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[cg][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto finish_piece = [&](const Cursor& cu) {
    // (the lane exchanges run with the whole wave active, before the
    // per-column branch)
    float l_tot[NC];
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) l_tot[cg] = sum_xor32(sum_xor16(l_run[cg]));
#pragma unroll
    for (int cg = 0; cg < NC; ++cg) {
      if (16 * cg + l16 >= R) continue;
      const int hq = cu.kvh * G + g_col[cg];
      const int64_t row = (int64_t)cu.r.row0 + t_col[cg];
      const bool empty = !(l_tot[cg] > 0.f);
      const float lse_nat = empty ? neg_inf() : (m_run[cg] * c + fast_log2(l_tot[cg])) * kLn2;
      const float nan = __builtin_nanf("");
      if (direct) {
        float den = l_tot[cg];
        if (a.sinks != nullptr && !empty) den += fast_exp2(a.sinks[hq] * kLog2e - m_run[cg] * c);
        const float inv = empty ? 0.f : v_mult / den;
        uint16_t* orow = a.out + row * a.o_sb + (int64_t)hq * a.o_sh + 4 * g4;
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
          f32x4 r = o[cg][blk] * inv;
          if (piece_bad) r = f32x4{nan, nan, nan, nan};
          *(u32x2*)(orow + 16 * blk) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
        }
        if (a.lse != nullptr && g4 == 0)
          a.lse[row * a.lse_sb + hq] = piece_bad ? nan : lse_nat;
      } else {
        const int s = sh.split ? w - sh.of(cu.p0) : 0;
        float* slot = a.ws + ((row * a.Hq + hq) * S + s) * (kD + 1);
        const float inv = empty ? 0.f : v_mult / l_tot[cg];
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
          f32x4 r = o[cg][blk] * inv;
          if (piece_bad) r = f32x4{nan, nan, nan, nan};
#pragma unroll
          for (int e = 0; e < 4; ++e) slot[16 * blk + 4 * g4 + e] = r[e];
        }
        if (g4 == 0) slot[kD] = piece_bad ? nan : lse_nat;
      }
    }
  };

  // Fused append: row r of a landed tile (token position pos, a new token of
  // the cursor's unit) to its cache row, skipping a position past the
  // block-table row or behind an entry outside the pool.
  auto store_new_row = [&](const Cursor& cu, PD_LDS const char* tl, int r, int pos) {
    constexpr int kElem = F8 ? 1 : 2;
    constexpr int kRowB = 2 * kD * kElem;
    constexpr int kChunks = kRowB / 16;
    const int pidx = kGen ? pos / a.P : pos >> p_shift;
    if (pidx >= a.max_blocks) return;
    const int page = as_const(a.bt)[(int64_t)cu.b * a.bt_sb + pidx];
    if ((uint32_t)page >= (uint32_t)a.num_pages) return;
    if (lane < kChunks) {
      const u32x4 v = *(PD_LDS const u32x4*)(tl + r * kRowB + lane * 16);
      const int c = F8 ? (lane ^ f8(r)) : (lane ^ swz(r));   // the chunk this position holds
      char* row = const_cast<char*>((const char*)a.kv) + (int64_t)page * a.kv_sp * kElem +
                  (int64_t)cu.kvh * a.kv_sh * kElem + (int64_t)(pos - pidx * a.P) * kRowB;
      *(u32x4*)(row + c * 16) = v;
    }
  };

  if (cc.b < a.B) {
    // ---- prologue -----------------------------------------------------------
    // The block-table entries of the next tile to issue are fetched one
    // iteration ahead of their use.
    TilePages pg_next = fetch_pages(ci);
    bad_slots = issue(ci, pg_next, 0) ? 1 : 0;
    advance(ci);
    pg_next = ci.b < a.B ? fetch_pages(ci) : pages_none;
    int issued = 1;               // tiles issued so far
    int slot_k = 0, slot_i = 1;   // ring slot of the computed tile, of the next issue
    auto issue_next = [&]() {
      wait_lgkmcnt0();  // LDS reads of the slot's old tile and of an old query slot are done
      const bool bad_tile = issue(ci, pg_next, slot_i);
      bad_slots = (bad_slots & ~(1 << slot_i)) | (bad_tile ? 1 << slot_i : 0);
      advance(ci);
      pg_next = ci.b < a.B ? fetch_pages(ci) : pages_none;
      ++issued;
      slot_i = (slot_i + 1) & (kSlots - 1);
    };
    // FP8: up to three tiles in flight.  A tile that starts a piece also
    // needs one of the two query slots; a slot is free again once its
    // piece's first tile has read it into registers.
    auto fill_ring = [&](int k_now) {
      while (ci.b < a.B && issued < k_now + kSlots &&
             (!piece_start(ci) || q_issued - q_used < kQSlots))
        issue_next();
    };
    if constexpr (F8) fill_ring(-1);

    for (int k = 0; cc.b < a.B; ++k) {
      const bool first = piece_start(cc);
      if (first) {
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
          m_run[cg] = neg_inf();
          l_run[cg] = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[cg][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        piece_bad = false;
        if constexpr (F8) {
          const int si = cc.kvh * a.scale_stride;
          c = a.scale_log2 * (a.k_scale != nullptr ? a.k_scale[si] : 1.f);
          v_mult = a.v_scale != nullptr ? a.v_scale[si] : 1.f;
        }
        if constexpr (V) {
          const int n = cc.r.n;   // >= 1: a unit with tiles has query rows
          R = n * G;
          const int L = as_const(a.seq_lens)[cc.b], Lr = real_len(a, cc.b);
#pragma unroll
          for (int cg = 0; cg < NC; ++cg) {
            const int nn = min(16 * cg + l16, R - 1);
            t_col[cg] = nn / G;
            g_col[cg] = nn - t_col[cg] * G;
            col_hi[cg] = row_hi(a, L, Lr, t_col[cg], n);
            col_lo[cg] = row_lo(a, col_hi[cg]);
          }
          all_hi = uniform(row_hi(a, L, Lr, 0, n));                 // first row's limit
          all_lo = uniform(row_lo(a, row_hi(a, L, Lr, n - 1, n)));   // last row's start
          piece_bad |= rows_over_bound(a, cc.b, QRows{cc.r.row0, n});
        }
        if constexpr (NC > 1) {
          // More than 16 columns: the query fragments are loaded here, into
          // registers, and waited for at once (a piece start drains the
          // tiles in flight; the query slots in LDS hold 16 columns only).
          // Column 16 c + l16 past the piece's columns reads the last one:
          // its scores are never written.
#pragma unroll
          for (int cg = 0; cg < NC; ++cg) {
            const bf16x8* qp =
                (const bf16x8*)(a.q + (int64_t)(cc.r.row0 + t_col[cg]) * a.q_sb +
                                (int64_t)(cc.kvh * G + g_col[cg]) * a.q_sh + 8 * g4);
#pragma unroll
            for (int s = 0; s < 4; ++s) qf[cg][s] = qp[4 * s];
          }
          wait_vmcnt<0>();
        }
      }

      if constexpr (F8) {
        // tile k has landed once at most the tiles issued after it are in
        // flight (their query rows were loaded before them, so they count
        // as part of the wait)
        const int after = issued - k - 1;
        if (after >= 2)
          wait_vmcnt<2 * kLoadsPerTile>();
        else if (after == 1)
          wait_vmcnt<kLoadsPerTile>();
        else
          wait_vmcnt<0>();
      } else {
        const bool issuing = ci.b < a.B;
        if (issuing) issue_next();
        if (issuing)
          wait_vmcnt<kLoadsPerTile>();
        else
          wait_vmcnt<0>();
      }

      if (NC == 1 && first) {
        // the piece's query rows (loaded before its first tile): B operand
        // of S^T = K Q^T, zero for padding heads
        PD_LDS const char* qs = qslots + (q_used % kQSlots) * kQSlotBytes + l16 * (kD * 2);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 v = *(PD_LDS const bf16x8*)(qs + (8 * g4 + 32 * s) * 2);
          qf[0][s] = l16 < R ? v : bf16x8{};
        }
        ++q_used;
      }
      // FP8: the next issues go after the query read, so this piece's query
      // slot is free again
      if constexpr (F8) fill_ring(k);

      piece_bad |= (bad_slots >> slot_k) & 1;
      PD_LDS char* tl = ring + slot_k * kSlotBytes;   // tile k as loaded
      if constexpr (AP) {
        // Fused append: the new tokens' rows of this tile came from the
        // sources; copy them from LDS into their cache rows.  (A store does
        // not upset the ring's vmcnt bookkeeping: it can only delay a wait,
        // since loads complete in order.)
        const int t0 = ((cc.r.lo >> 5) + cc.i) * kTileTokens;
        const int p_lo = max(cc.r.L - cc.r.n, t0), p_hi = min(cc.r.L, t0 + kTileTokens);
        for (int pos = p_lo; pos < p_hi; ++pos) store_new_row(cc, tl, pos - t0, pos);
      }
      // bf16: the V half of the tile, row stride 512 bytes, chunk 16 + c at
      // position (16 + c) ^ swz(r)
      PD_LDS char* vt = tl + 256;
      constexpr std::false_type kLo{};
      constexpr std::true_type kHi{};
      // two FP8 codes of a dword (low or high half) -> two packed bf16
      auto cvt8 = [](uint32_t w, auto hi) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, decltype(hi)::value));
      };
      const int lo = cc.r.lo, hi = cc.r.hi;
      const int tok0 = ((lo >> 5) + cc.i) * kTileTokens;

      // ---- scores ----
      // group c is in use while its first column is one of the piece's
      // (wave-uniform); group 0 always is
      bool act[NC];
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) act[cg] = cg == 0 || 16 * cg < R;
      f32x4 s0[NC], s1[NC];
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) s0[cg] = s1[cg] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int sw = swz(l16);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 k0, k1;
        if constexpr (F8) {
          // dims 32 s + 8 g4 .. + 7 of rows l16 and 16 + l16: half g4 % 2 of
          // FP8 chunk 2 s + g4 / 2, converted in registers (exact: every
          // E4M3FN value is a bf16 value)
          const int c8 = 2 * s + (g4 >> 1), h8 = (g4 & 1) * 8;
          const u32x2 w0 = *(PD_LDS const u32x2*)(tl + l16 * kRowBytes8 + ((c8 ^ f8(l16)) << 4) + h8);
          const u32x2 w1 =
              *(PD_LDS const u32x2*)(tl + (16 + l16) * kRowBytes8 + ((c8 ^ f8(16 + l16)) << 4) + h8);
          k0 = __builtin_bit_cast(bf16x8, u32x4{cvt8(w0[0], kLo), cvt8(w0[0], kHi),
                                                cvt8(w0[1], kLo), cvt8(w0[1], kHi)});
          k1 = __builtin_bit_cast(bf16x8, u32x4{cvt8(w1[0], kLo), cvt8(w1[0], kHi),
                                                cvt8(w1[1], kLo), cvt8(w1[1], kHi)});
        } else {
          const int ch = (g4 + 4 * s) ^ sw;
          k0 = *(PD_LDS bf16x8*)(tl + l16 * kRowBytes + ch * 16);
          k1 = *(PD_LDS bf16x8*)(tl + (16 + l16) * kRowBytes + ch * 16);
        }
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
          if (!act[cg]) continue;
          s0[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[cg][s], s0[cg], 0, 0, 0);
          s1[cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[cg][s], s1[cg], 0, 0, 0);
        }
      }

      // V rows outside the request's keys are zeroed; scores outside the
      // lane's column range are -inf (the two differ only for verify rows)
      const bool edge = tok0 < lo || tok0 + kTileTokens > hi;
      bool v0[4], v1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t0 = tok0 + 4 * g4 + i, t1 = t0 + 16;
        v0[i] = !edge || (t0 >= lo && t0 < hi);
        v1[i] = !edge || (t1 >= lo && t1 < hi);
        if constexpr (V) {
          const bool col_edge = tok0 < all_lo || tok0 + kTileTokens > all_hi;
#pragma unroll
          for (int cg = 0; cg < NC; ++cg) {
            if (col_edge && !(t0 >= col_lo[cg] && t0 < col_hi[cg])) s0[cg][i] = neg_inf();
            if (col_edge && !(t1 >= col_lo[cg] && t1 < col_hi[cg])) s1[cg][i] = neg_inf();
          }
        } else {
          if (!v0[i]) s0[0][i] = neg_inf();
          if (!v1[i]) s1[0][i] = neg_inf();
        }
      }

      // ---- V^T fragments of the tile, read before the softmax so their LDS
      // latency overlaps it (they do not depend on the probabilities) ----
      // bf16: two 16-bit transpose reads per block of 16 dims, rows
      // ra = 4 g4 + l16 / 4 and ra + 16 (the k order of P^T).
      // FP8: the 8-bit transpose read gives lane i of a 16-lane group byte
      // i % 8 of the 8 bytes read by lanes 2 e + (i >= 8), e = 0..7; so lane
      // s reads dims 16 blk + 8 (s % 2) .. + 7 of token T(s / 2), with
      // T(e) = 4 g4 + e (e < 4) and 16 + 4 g4 + e - 4 (the same k order);
      // its codes are converted at the product.
      u32x4 vraw[8];
      {
        const int ra = 4 * g4 + (l16 >> 2);
        const int rb = ra + 16;
        const int swa = swz(ra);
        const int tv = (l16 >> 1) < 4 ? 4 * g4 + (l16 >> 1) : 12 + 4 * g4 + (l16 >> 1);
        PD_LDS char* vrow8 = tl + tv * kRowBytes8 + (l16 & 1) * 8;
        const int fv = f8(tv);
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) {
          if constexpr (F8) {
            typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
            const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (PD_LDS i32x2*)(vrow8 + (((8 + blk) ^ fv) << 4)));
            vraw[blk] = u32x4{(uint32_t)w[0], (uint32_t)w[1], 0u, 0u};
          } else {
            const int ch = 2 * blk + ((l16 & 3) >> 1);   // V chunk (16 dims) of this block
            const int within = (l16 & 1) * 8;
            const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (PD_LDS bf16x4*)(vt + ra * kRowBytes + ((ch ^ swa) << 4) + within));
            const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (PD_LDS bf16x4*)(vt + rb * kRowBytes + ((ch ^ swa) << 4) + within));
            const u32x2 ua = __builtin_bit_cast(u32x2, va);
            const u32x2 ub = __builtin_bit_cast(u32x2, vb);
            vraw[blk] = u32x4{ua[0], ua[1], ub[0], ub[1]};
          }
        }
      }
      // keep the reads here (left alone, the scheduler moves them next to
      // their products, behind the softmax)
      __builtin_amdgcn_sched_barrier(0);

      // ---- online softmax (fp32, exp2, reference max in unscaled logits) ----
      // P^T as the B operand: k = 8*g4 + j <-> tokens 4*g4 + j (j < 4) and
      // 16 + 4*g4 + (j - 4) (j >= 4), exactly this lane's scores.
      bf16x8 pf[NC];
#pragma unroll
      for (int cg = 0; cg < NC; ++cg) {
        if (!act[cg]) continue;
        float mx = fmaxf(fmaxf(fmaxf(s0[cg][0], s0[cg][1]), fmaxf(s0[cg][2], s0[cg][3])),
                         fmaxf(fmaxf(s1[cg][0], s1[cg][1]), fmaxf(s1[cg][2], s1[cg][3])));
        mx = max_xor32(max_xor16(mx));
        // The reference m_run moves (and O and l are rescaled) only when a
        // score passes it by more than kRescaleLog2 in the exp2 domain, so
        // p <= 2^kRescaleLog2.  The branch is taken by the whole wave;
        // columns that did not grow keep alpha = 1 (their reference may
        // still be -inf: a verify column whose keys start later).
        const bool grow = (mx - m_run[cg]) * c > kRescaleLog2;   // false while both are -inf
        if (__ballot(grow) != 0ull) {
          const float alpha = grow ? fast_exp2((m_run[cg] - mx) * c) : 1.f;
          l_run[cg] *= alpha;
          m_run[cg] = grow ? mx : m_run[cg];
#pragma unroll
          for (int i = 0; i < 8; ++i) o[cg][i] *= alpha;
        }
        const float mc = (m_run[cg] == neg_inf() ? 0.f : m_run[cg]) * c;
        float p0[4], p1[4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p0[i] = fast_exp2(s0[cg][i] * c - mc);
          p1[i] = fast_exp2(s1[cg][i] * c - mc);
          psum += p0[i] + p1[i];
        }
        l_run[cg] += psum;
        const u32x4 pw = {pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]),
                          pack_bf16x2(p1[0], p1[1]), pack_bf16x2(p1[2], p1[3])};
        pf[cg] = __builtin_bit_cast(bf16x8, pw);
      }
      const u32x4 vkeep = {keep_mask(v0[0], v0[1]), keep_mask(v0[2], v0[3]),
                           keep_mask(v1[0], v1[1]), keep_mask(v1[2], v1[3])};

      // ---- O^T += V^T P^T (one V^T fragment for every column group) ----
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        u32x4 vv = vraw[blk];
        if constexpr (F8)
          vv = u32x4{cvt8(vraw[blk][0], kLo), cvt8(vraw[blk][0], kHi), cvt8(vraw[blk][1], kLo),
                     cvt8(vraw[blk][1], kHi)};
        if (edge) vv &= vkeep;
#pragma unroll
        for (int cg = 0; cg < NC; ++cg) {
          if (!act[cg]) continue;
          o[cg][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pf[cg],
                                                              o[cg][blk], 0, 0, 0);
        }
      }

      if (cc.i + 1 == cc.i_end && !pair_mode) finish_piece(cc);
      advance(cc);
      slot_k = (slot_k + 1) & (kSlots - 1);
    }
  }

  // ---- pair mode: the second half's (m, l, O) to the first, which merges
  // them and writes the unit's result ---------------------------------------
  if (pair_mode) {
    // through the second half's own ring (no tile load is in flight now)
    constexpr int kXO = 8 * 64 * 16;   // O: 8 blocks x 64 lanes x 16 bytes
    if (half == 1) {
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) *(PD_LDS f32x4*)(ring + (blk * 64 + lane) * 16) = o[0][blk];
      ((PD_LDS float*)(ring + kXO))[lane] = m_run[0];
      ((PD_LDS float*)(ring + kXO + 256))[lane] = l_run[0];
      ((PD_LDS int*)(ring + kXO + 512))[lane] = piece_bad ? 1 : 0;
    }
    __syncthreads();
    if (half == 0 && !idle && r_s.nt > 0) {
      PD_LDS const char* pb = ring + kWaveLds;
      const float mb = ((PD_LDS const float*)(pb + kXO))[lane];
      const float lb = ((PD_LDS const float*)(pb + kXO + 256))[lane];
      const bool bb = ((PD_LDS const int*)(pb + kXO + 512))[lane] != 0;
      const float ma = m_run[0];
      const float mm = fmaxf(ma, mb);
      const float wa = ma == neg_inf() ? 0.f : fast_exp2((ma - mm) * c);
      const float wb = mb == neg_inf() ? 0.f : fast_exp2((mb - mm) * c);
      l_run[0] = l_run[0] * wa + lb * wb;
#pragma unroll
      for (int blk = 0; blk < 8; ++blk)
        o[0][blk] = o[0][blk] * wa + *(PD_LDS const f32x4*)(pb + (blk * 64 + lane) * 16) * wb;
      m_run[0] = mm;
      piece_bad = piece_bad || bb;
      Cursor cu;
      cu.b = b_s;
      cu.kvh = kvh_s;
      cu.p0 = 0;
      cu.i = cu.i_end = 0;
      cu.r = r_s;
      finish_piece(cu);
    }
  }

  // ---- units this wave answers for without streaming them ---------------
  // Empty units owned by this share get O = 0 / LSE = -inf; a unit whose
  // first tile is in this share gets its slot list ended after the slots its
  // pieces use.  Partials only: every slot no piece uses gets lse = -inf,
  // as the partials entries promise; a call that merges itself writes just
  // lse = +inf into the first unused slot (the merge reads no further), one
  // store per column instead of one per unused slot.
  // Fused append: the unit's owner writes the new tokens' K and V that no
  // tile of the unit covers (past its attended range) into the cache (a byte
  // copy, skipping positions below 0, past the block-table row or behind an
  // entry outside the pool).  The covered rows are written by the waves that
  // stream their tiles.
  auto append_rows = [&](const Cursor& cu) {
    constexpr int kElem = F8 ? 1 : 2;
    constexpr int kChunks = 2 * kD * kElem / 16;   // 16-byte chunks of a K|V row
    constexpr int kHalf = kChunks / 2;
    constexpr int kPer = 64 / kChunks;             // rows per pass of the wave
    const int n = cu.r.n, L = cu.r.L;
    // tiles of the unit cover positions [c_lo, c_hi); their rows were
    // written by the waves that streamed them
    const int c_lo = (cu.r.lo >> 5) * kTileTokens, c_hi = c_lo + cu.r.nt * kTileTokens;
    const int ch = lane % kChunks;
    const bool kp = ch < kHalf;
    const int64_t srow = kp ? a.kn_srow : a.vn_srow;
    const char* src0 = kp ? a.kn + (int64_t)cu.r.row0 * a.kn_srow + (int64_t)cu.kvh * a.kn_sh + ch * 16
                          : a.vn + (int64_t)cu.r.row0 * a.vn_srow + (int64_t)cu.kvh * a.vn_sh +
                                (ch - kHalf) * 16;
    // the cache is written here only (the argument is const for the reads)
    char* dst0 = const_cast<char*>((const char*)a.kv) + (int64_t)cu.kvh * a.kv_sh * kElem + ch * 16;
    const int64_t sp_bytes = (int64_t)a.kv_sp * kElem;
    const int32_t* bt_row = a.bt + (int64_t)cu.b * a.bt_sb;
    for (int t0 = 0; t0 < n; t0 += kPer) {
      const int t = t0 + lane / kChunks;
      const int pos = L - n + t;
      if (t >= n || pos < 0 || (pos >= c_lo && pos < c_hi)) continue;
      const int pidx = pos / a.P;
      if (pidx >= a.max_blocks) continue;
      const int page = bt_row[pidx];
      if ((uint32_t)page >= (uint32_t)a.num_pages) continue;
      *(u32x4*)(dst0 + (int64_t)page * sp_bytes + (int64_t)(pos - pidx * a.P) * (2 * kD * kElem)) =
          *(const u32x4*)(src0 + (int64_t)t * srow);
    }
  };

  Cursor cw;
  cw.b = b_s;
  cw.kvh = kvh_s;
  cw.p0 = p0_s;
  cw.r = r_s;
  // (pair mode: the first half answers for the unit)
  while (cw.b < a.B && (sh.last || cw.p0 < sh.g1) && !past_units(cw) && half == 0) {
    const int hq0 = cw.kvh * G;
    R = V ? cw.r.n * G : G;   // this unit's columns
    // (row, query head) of column n of this unit
    auto col_row = [&](int n) { return (int64_t)cw.r.row0 + n / G; };
    auto col_head = [&](int n) { return hq0 + n % G; };
    // a request past the max_qlen bound is written NaN below instead
    const bool over = V && rows_over_bound(a, cw.b, QRows{cw.r.row0, cw.r.n});
    if (cw.r.nt == 0 && !over) {
      if (direct) {
        for (int i = lane; i < R * (kD / 8); i += 64) {
          const int n = i / (kD / 8), d8 = (i % (kD / 8)) * 8;
          *(u32x4*)(a.out + col_row(n) * a.o_sb + (int64_t)col_head(n) * a.o_sh + d8) = u32x4{0, 0, 0, 0};
        }
        if (a.lse != nullptr && lane < R) a.lse[col_row(lane) * a.lse_sb + col_head(lane)] = neg_inf();
      } else if (a.partials) {
        for (int i = lane; i < R * S; i += 64) {
          const int n = i / S, s = i % S;
          a.ws[((col_row(n) * a.Hq + col_head(n)) * S + s) * (kD + 1) + kD] = neg_inf();
        }
      } else if (lane < R) {
        a.ws[((col_row(lane) * a.Hq + col_head(lane)) * S) * (kD + 1) + kD] = end_of_slots();
      }
    } else if (sh.split && cw.p0 >= sh.g0) {
      const int nseg = sh.of(cw.p0 + cw.r.nt - 1) - sh.of(cw.p0) + 1;
      if (a.partials) {
        for (int i = lane; i < R * (S - nseg); i += 64) {
          const int n = i / (S - nseg), s = nseg + i % (S - nseg);
          a.ws[((col_row(n) * a.Hq + col_head(n)) * S + s) * (kD + 1) + kD] = neg_inf();
        }
      } else if (nseg < S && lane < R) {
        a.ws[((col_row(lane) * a.Hq + col_head(lane)) * S + nseg) * (kD + 1) + kD] = end_of_slots();
      }
    }
    if constexpr (V) {
      // Variable query length: rows of the request past the max_qlen bound
      // are not computed; the unit's owner writes them NaN (O and LSE, or
      // every split slot), as for an invalid block-table entry.  (The rows
      // it streams are NaN too: the piece is marked bad, or, for a unit
      // with no key, written NaN here.)
      const bool owner = cw.r.nt == 0 || !sh.split || cw.p0 >= sh.g0;
      if (owner && over) {
        const int r1 = min(max((int)as_const(a.cu_q)[cw.b + 1], cw.r.row0), a.total_rows);
        // every row for a unit with no key, else the rows past the first n
        const int first_row = cw.r.nt == 0 ? 0 : cw.r.n;
        const int rows_nan = uniform(r1 - cw.r.row0 - first_row);
        const float nan = __builtin_nanf("");
        for (int i = lane; i < rows_nan * G; i += 64) {
          const int64_t row = (int64_t)cw.r.row0 + first_row + i / G;
          const int hq = hq0 + i % G;
          if (direct) {
            uint16_t* orow = a.out + row * a.o_sb + (int64_t)hq * a.o_sh;
            for (int d = 0; d < kD; d += 8)
              *(u32x4*)(orow + d) = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
            if (a.lse != nullptr) a.lse[row * a.lse_sb + hq] = nan;
          } else {
            for (int sl = 0; sl < S; ++sl) {
              float* slot = a.ws + ((row * a.Hq + hq) * S + sl) * (kD + 1);
              for (int d = 0; d <= kD; ++d) slot[d] = nan;
            }
          }
        }
      }
    }
    // a unit is owned by the share holding its first tile (an empty unit, by
    // the one share that visits it)
    if (AP && (cw.r.nt == 0 || !sh.split || cw.p0 >= sh.g0)) append_rows(cw);
    next_unit(cw);
  }
}

}  // namespace

// Launches page class PS for a decode or verify call with a bf16 or FP8
// cache, with the fused append or not (AP); one workgroup per compute unit.
// With one split (whole units) the grid has no more workgroups than units
// (the kernel's unit mode spreads one unit per wave over them).
// Pair mode (two waves per unit) when every unit fits two waves of the
// 4-wave grid, with at most 16 score columns; the rule does not depend on
// the kernel's waves per workgroup, so the bf16 and FP8 paths take the same
// mode (and round alike).
template <int PS, bool AP>
hipError_t launch_gqa_class(const GqaArgs& args, bool verify, int n_wg, hipStream_t stream) {
  const int64_t units = (int64_t)args.B * args.Hkv;
  GqaArgs a = args;
  a.pair = (a.S == 1 && 2 * units <= 4 * (int64_t)n_wg && (!verify || a.qlen * a.G <= 16)) ? 1 : 0;
  const dim3 grid((unsigned)(a.S == 1 ? std::max<int64_t>(1, std::min<int64_t>(n_wg, units)) : n_wg));
  const dim3 grid8 = grid;
  const dim3 block(gqa_waves(false, 1) * 64), block8(gqa_waves(true, 1) * 64);
  if (verify) {
    // score column groups of 16 for the (verify token, head) pairs
    const int cols = a.qlen * a.G;
    if (a.kv_fp8) {
      if (cols <= 16)
        hipLaunchKernelGGL((gqa_decode_kernel<PS, true, true, 1, AP>), grid8, block8, 0, stream, a);
      else if (cols <= 32)
        hipLaunchKernelGGL((gqa_decode_kernel<PS, true, true, 2, AP>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((gqa_decode_kernel<PS, true, true, 4, AP>), grid, block, 0, stream, a);
    } else {
      if (cols <= 16)
        hipLaunchKernelGGL((gqa_decode_kernel<PS, true, false, 1, AP>), grid, block, 0, stream, a);
      else if (cols <= 32)
        hipLaunchKernelGGL((gqa_decode_kernel<PS, true, false, 2, AP>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((gqa_decode_kernel<PS, true, false, 4, AP>), grid, block, 0, stream, a);
    }
  } else {
    if (a.kv_fp8)
      hipLaunchKernelGGL((gqa_decode_kernel<PS, false, true, 1, AP>), grid8, block8, 0, stream, a);
    else
      hipLaunchKernelGGL((gqa_decode_kernel<PS, false, false, 1, AP>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pd
