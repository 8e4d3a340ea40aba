// Causal MLA verify for gfx950: qlen query tokens per request, all heads,
// over one shared latent cache with V = K[..., :Lv].
//
// Operation: "vllm.v1.attention.ops.triton_decode_attention",
// decode_attention_fwd_verify (row limit max(min(L - qlen + 1 + t, L_real), 0),
// V read from K, natural-log LSE, [rows, H, S, Lv + 1] fp32 partials, scalar
// k_scale for an FP8 cache); the split rule (a request's own length cut into
// max(ceil(L / S), min) chunks) is the one its verify_num_kv_splits describes.
//
// Design on CDNA4
// ---------------
// * The qlen * H (token, head) pairs of a request are the "rows", cut into
//   row blocks of 128.  A workgroup of 4 waves (one per SIMD, 512 registers
//   each) runs one row block over a range of the request's keys.  The grid
//   is persistent (one workgroup per CU); workgroups form groups that take
//   the row blocks of the same requests over the same key range at the same
//   time, on one XCD, so each latent tile is fetched from HBM once per group
//   and served from L2 to the others.  Every group gets the same number of
//   tiles whatever the length mix; a cut request writes one fp32 partial
//   per piece.
// * Latent tiles of 32 tokens (2 pages, 36 KB bf16 / 18 KB fp8) stream from
//   HBM into a 4-slot LDS ring with global_load_lds_dwordx4, each bf16
//   instruction filling 1 KB from 8 whole 128-byte lines.  A tile's loads
//   are spread over the MFMA steps of the tile before (issued at once they
//   fill the request queue and stall the wave).  FP8 fragments are read
//   from the FP8 tile itself (K with 8-byte reads, V^T with
//   ds_read_b64_tr_b8) and converted in registers, exactly
//   (v_cvt_scalef32_pk_bf16_fp8, scale 1); k_scale goes into the
//   softmax scale and the output.
// * Scores: each wave owns 32 rows; S^T[token, row] = K . Q^T with
//   v_mfma_f32_32x32x16_bf16, its query fragment (32 x 576 bf16, 144 VGPRs)
//   held for the whole piece, K fragments read from LDS a few steps ahead,
//   the score accumulator in arch VGPRs (the MFMA's asm form).
// * Product: each wave owns 128 of the 512 output dims for all 128 rows, so
//   every V^T fragment (ds_read_b64_tr_b16 from the same tile) feeds four
//   MFMAs.  The probabilities go through LDS: a wave's packed P of a key
//   step is, lane by lane, the B operand every wave needs for its rows.  The
//   output accumulator (128 dims x 128 rows fp32) takes all 256 AGPRs.
// * Iteration k runs the score MFMAs of tile k and the product of tile k-1:
//   FP8 interleaves the two, bf16 runs the product after the score chain,
//   interleaved with tile k's softmax; one barrier per tile.
// * Online softmax in the exp2 domain (x = score * sm_scale * log2 e) with a
//   fixed per-row reference: a row's reference max is its first non-empty
//   tile's max and is never rescaled, so no vector instruction ever touches
//   the accumulator (which is what keeps it in AGPRs).  The exact row max is
//   tracked alongside; if a later score exceeds the reference by more than
//   2^64 (overflow risk) the workgroup runs the piece a second time with the
//   exact max as reference.  Real attention scores never trigger it.
// * With one split, whole requests are written directly as bf16 O and LSE
//   (unless the caller asked for partials only); with several, every piece
//   writes its fp32 partial (slots no piece uses are marked empty) and the
//   merge pass combines them.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pd {
namespace {

constexpr int kLk = 576;
constexpr int kLv = 512;
constexpr int kWaves = 4;                                          // one per SIMD
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;              // 128
constexpr int kRowBytes = kLk * 2;                                 // bf16 latent row
constexpr int kTileBytes = kTileTokens * kRowBytes;                // 36 KB
constexpr int kPageRegion = 16 * kRowBytes;                        // 18 KB (bf16)
constexpr int kRowBytes8 = kLk;                                    // fp8 latent row
constexpr int kTileBytes8 = kTileTokens * kRowBytes8;              // 18 KB
constexpr int kPageRegion8 = 16 * kRowBytes8;                      // 9 KB (fp8)
constexpr int kKSteps = kLk / 16;                                  // 36
// K fragments read ahead of their score step.  bf16: 5 (the score chain's
// 16-byte reads saturate the LDS, so each queues behind the other waves';
// 3 -> 5 took 2-3% off the kernel, 6, 7 and 9 gained less); FP8: 3 (8-byte
// reads; 4 equal, 5 slower).
constexpr int kKAheadBf16 = 5;
constexpr int kKAheadFp8 = 3;
constexpr int kDimBlocksPerWave = kLv / 32 / kWaves;              // 4 output blocks of 32 dims
constexpr int kPBufBytes = kWaves * 2 * 1024;                      // P^T of one tile: 4 row groups x 2 key steps
// p = 2^(x - m_ref) stays below 2^64 while the row max has not grown more
// than this above the reference (fp32 / bf16 hold 2^127; with up to 2^20
// keys and |V| < 2^40 the accumulator cannot overflow).
constexpr float kRefHeadroomLog2 = 64.f;
// Fixed cost of a piece in tiles' worth of time: its query fragments, the
// refill of the tile ring and the epilogue (statistics through LDS, the
// partial or output write).  Per-workgroup timestamps at the verify config
// put it near 16 us, about 7 tiles: workgroups with three pieces ended 30 us
// after those with one.  The plan counts it as virtual tiles at the start
// of every request, so a share that starts more pieces gets fewer real
// tiles (kernel time -1.4% bf16, -3.7% FP8, -3.9% at page size 1; 4 to 10
// tiles measured, 7 and 10 alike).
constexpr int kPieceTiles = 8;

// LDS layout of a bf16 tile.  A 32-token tile is two 16-row page regions
// of 18 blocks of 1 KB.  Block 2 C + R holds 16-byte chunks 8 C .. 8 C + 7
// (one 128-byte line of the latent row) of rows 8 R .. 8 R + 7, chunk c of
// row r at 16-byte slot 8 (r % 8) + ((c % 8) ^ (r % 8) ^ R).  So
//  * one global_load_lds instruction (64 lanes x 16 bytes) fills one block
//    from 8 whole 128-byte lines; the XOR only permutes lanes inside a line;
//  * a K-operand read (rows 0..15 of a page, one chunk) touches distinct
//    16-byte slots modulo the 256 bytes of the 64 banks.  A transpose read
//    of V serves 32 lanes (4 rows x 4 chunks x 2 halves) per cycle, and rows
//    4k and 4k + 2 share a bank row and chunk group here, so the rocprofv3
//    bank-conflict counter shows it 2-way conflicted.  A layout with bits 1
//    and 2 of the row exchanged in the XOR removes the conflict (measured)
//    but ran 0.6% slower per call on the same box: these reads are not what
//    bounds the kernel, so the layout stays.
__device__ __forceinline__ int tile_off(int c, int r16) {
  return ((c >> 3) * 2 + (r16 >> 3)) * 1024 + (8 * (r16 & 7) + ((c & 7) ^ (r16 & 7) ^ (r16 >> 3))) * 16;
}
// The fp8 ring (before dequantisation) keeps chunk-column-major pages: fp8
// chunk c8 (16 bytes) of row r16 at slot 16 c8 + r16.

// Load j of a wave's share of a tile (global_load_lds_dwordx4: 16 bytes per
// lane): global address base (+ voff) + j kG, LDS address dst + j kL.  The
// instruction's immediate offset (j kG) moves both addresses, so M0 gets
// dst + j (kL - kG), in the same statement.  j is a constant once the
// caller's loop is unrolled, so the switch folds to one statement and a load
// costs no address arithmetic.  kLaneAddr: base is the lane's own 64-bit
// address; otherwise base is wave-uniform and voff the lane's byte offset.
// The s_nop covers the M0-write -> LDS-DMA hazard.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int kG, int kL, bool kLaneAddr>
__device__ __forceinline__ void dma_step(int j, const char* base, uint32_t voff, uint32_t dst) {
  static_assert(kL >= kG, "M0 takes the LDS step less the global step");
  if constexpr (!kLaneAddr) base = (const char*)scalar_ptr(base);
  switch (j) {
#define PD_DMA_CASE(J)                                                                           \
  case J:                                                                                        \
    if constexpr (kLaneAddr)                                                                     \
      asm volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%3"  \
                   :                                                                             \
                   : "s"(dst), "v"(base), "i"((J) * (kL - kG)), "i"((J) * kG)                    \
                   : "memory", "m0", "scc");                                                     \
    else                                                                                         \
      asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%4"   \
                   :                                                                             \
                   : "s"(dst), "v"(voff), "s"(base), "i"((J) * (kL - kG)), "i"((J) * kG)         \
                   : "memory", "m0", "scc");                                                     \
    break;
    PD_DMA_CASE(0) PD_DMA_CASE(1) PD_DMA_CASE(2) PD_DMA_CASE(3) PD_DMA_CASE(4)
    PD_DMA_CASE(5) PD_DMA_CASE(6) PD_DMA_CASE(7) PD_DMA_CASE(8)
#undef PD_DMA_CASE
    default: break;
  }
}
#pragma clang diagnostic pop


// PC: the page class, 1, 2, 4 or 8 (the page size), 16 (every power-of-two
// page of 16 tokens or more; log2 of the size in a.p_shift) or 0 (every
// other page size, 3 tokens or more: an issuing wave's 8 (bf16) or 16 (FP8)
// rows span at most 4 or 6 pages, and each lane divides to find its row's).
template <int NS, bool FP8, int PC>
__global__ __launch_bounds__(kWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_verify_kernel(MlaArgs a) {
  constexpr int kRingTile = FP8 ? kTileBytes8 : kTileBytes;
  constexpr int kLoadsPerTile = kRingTile / 1024;                  // 36 or 18
  constexpr int kLoadsPerPage = kLoadsPerTile / 2;
  // bf16: 4 waves x 9 loads; fp8: waves 0 and 1 load one page (9 loads) each,
  // so every issuing wave has the same count for its vmcnt bookkeeping.
  constexpr int kIssueWaves = FP8 ? 2 : 4;
  static_assert(NS == 4, "ring of 4 tiles: k-1 (product), k (scores), k+1, k+2 (loading)");
  constexpr int kStageOff = NS * kRingTile;
  constexpr int kLoadsPerWave = kLoadsPerTile / kIssueWaves;
  static_assert(kLoadsPerWave * kIssueWaves == kLoadsPerTile, "even load split");
  constexpr int kLoadSpacing = kKSteps / kLoadsPerWave;             // score steps between a wave's loads
  static_assert(kLoadSpacing >= 1 && (kLoadsPerWave - 1) * kLoadSpacing < kKSteps, "loads fit the score steps");
  constexpr int kPOff = kStageOff;                                  // P^T of tiles k-1 and k
  constexpr int kLdsBytes = kPOff + 2 * kPBufBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  PD_LDS char* lds = (PD_LDS char*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g2 = lane >> 5;
  const int S = a.S;
  const bool direct = S == 1 && !a.partials;

  // ---- the plan ----------------------------------------------------------
  // The rows of a request form n_rb row blocks of 128 (token, head) rows;
  // every row block of a request reads the same latent tiles.  Workgroups
  // are grouped gs = min(n_rb, grid) at a time; the members of a group take
  // the row blocks m, m + gs, ... of the same requests over the same tile
  // range at the same time, so a tile fetched from HBM by one member is an
  // L2 hit for the others.  Logical workgroup ids are XCD-remapped (hardware
  // hands consecutive ids to the 8 XCDs round-robin) so a group shares one
  // XCD and its L2.  Request b counts nt_b tiles, those of its last row block
  // (the largest row limit), preceded by kPieceTiles virtual tiles standing
  // for a piece's fixed cost; all requests' tiles in order form one flat
  // sequence of U tiles and group g takes the equal contiguous share
  // [g T, g T + T): every group gets the same time's worth of work whatever
  // the length mix.  Where a share cuts a request, each piece is a split with
  // its own partial slot; T is raised until no request spans more than S
  // shares.  With S == 1 shares are rounded to whole requests and results
  // are written directly (or as the one partial of slot 0).
  const int n_wg = gridDim.x;
  int sid = blockIdx.x;
  const int per_xcd = n_wg / 8;
  if (sid < per_xcd * 8) sid = (sid % 8) * per_xcd + sid / 8;
  sid = __builtin_amdgcn_readfirstlane(sid);
  const int rows_req = a.qlen * a.H;
  const int n_rb = (rows_req + kRowsPerBlock - 1) / kRowsPerBlock;
  const int gs = min(n_rb, n_wg);
  const int n_groups = n_wg / gs;
  const int grp = sid / gs, member = sid % gs;
  if (grp >= n_groups) return;   // the whole workgroup: no barrier was passed
  auto unit_len = [&](int b) { return min(max((int)as_const(a.seq_lens)[b], 0), a.max_blocks * a.P); };
  auto unit_real = [&](int b, int L) { return a.real_lens != nullptr ? (int)as_const(a.real_lens)[b] : L; };
  // largest row limit of row block rb of a request with lengths (L, Lr)
  auto block_hi = [&](int L, int Lr, int rb) {
    const int last_row = min(rb * kRowsPerBlock + kRowsPerBlock, rows_req) - 1;
    return max(min(L - a.qlen + 1 + last_row / a.H, Lr), 0);
  };
  auto block_tiles = [&](int L, int Lr, int rb) { return (block_hi(L, Lr, rb) + kTileTokens - 1) / kTileTokens; };
  auto req_tiles = [&](int b) {
    const int L = unit_len(b);
    return block_tiles(L, unit_real(b, L), n_rb - 1);
  };

  // U counts every request's tiles plus kPieceTiles virtual ones before them
  int nt_sum = 0, nt_max = 0;
  for (int base = 0; base < a.B; base += 64) {
    const bool in = base + lane < a.B;
    const int t = in ? req_tiles(base + lane) : 0;
    nt_sum += wave_sum(in ? t + kPieceTiles : 0);
    nt_max = max(nt_max, wave_max(t));
  }
  const int U = __builtin_amdgcn_readfirstlane(nt_sum);
  nt_max = __builtin_amdgcn_readfirstlane(nt_max);
  const bool split_mode = S >= 2;
  int T = max((U + n_groups - 1) / n_groups, kMlaMinSplitTiles);
  // a request of n tiles cut every T tiles at an arbitrary offset spans at
  // most floor((n - 1) / T) + 2 shares: keep that <= S
  if (split_mode) T = max(T, (nt_max - 1) / (S - 1) + 1);
  T = __builtin_amdgcn_readfirstlane(T);
  const int g_used = __builtin_amdgcn_readfirstlane(max((U + T - 1) / T, 1));
  if (grp >= g_used) return;
  const int g0 = grp * T;
  const bool last = grp == g_used - 1;
  const int g1 = last ? U : g0 + T;

  // first request holding tile g0, or starting at or after it
  int b_s = -1, cb_s = 0;
  {
    int C = 0;
    for (int base = 0; base < a.B; base += 64) {
      const bool in = base + lane < a.B;
      const int req = in ? req_tiles(base + lane) + kPieceTiles : 0;
      const int incl = wave_incl_sum(req);
      const int cb1 = C + incl, cb = cb1 - req;
      const uint64_t m = __ballot(in && (cb1 > g0 || cb >= g0));
      if (m != 0) {
        const int l0 = __builtin_ctzll(m);
        b_s = base + l0;
        cb_s = __builtin_amdgcn_readlane(cb, l0);
        break;
      }
      C += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (b_s < 0) return;
  b_s = __builtin_amdgcn_readfirstlane(b_s);
  cb_s = __builtin_amdgcn_readfirstlane(cb_s);

  // ---- one piece: tiles [tb, tb + n) of unit (b, rb), split slot `split` --
  auto run_piece = [&](const int b, const int rb, const int tb, const int n, const int split) {
    // ---- score rows of this lane (the wave's own 32 rows) and their limits --
    const int L = unit_len(b);
    const int Lr = unit_real(b, L);
    const int my_row = rb * kRowsPerBlock + wave * kRowsPerWave + l32;
    const bool row_ok = my_row < rows_req;
    const int t_row = row_ok ? my_row / a.H : 0;
    const int h_row = row_ok ? my_row % a.H : 0;
    const int hi_row = row_ok ? max(min(L - a.qlen + 1 + t_row, Lr), 0) : 0;
    const int hi_blk = __builtin_amdgcn_readfirstlane(block_hi(L, Lr, rb));
    // the wave's smallest row limit: tiles below it need no causal mask
    const int hi_wmin = __builtin_amdgcn_readfirstlane(-wave_max(-hi_row));

    float kscale = 1.f;
    if constexpr (FP8) {
      if (a.k_scale != nullptr) kscale = a.k_scale[0];
    }
    // log2-domain scale of the scores: x = K . q (FP8: codes . q times
    // k_scale, so both caches give the same x), logit = x * c
    const float c = a.scale_log2;

    // ---- Q fragment: B operand of S^T = K Q^T (32 rows x 576 dims) --------
    // A row past the request's rows reads the request's first row instead:
    // its scores are all masked (hi_row = 0) and its output is never
    // written.  With no select on the loaded values, the 36 loads go
    // straight into the fragment registers and are in flight together, with
    // the block-table reads and the loads of the first two tiles; one wait
    // for all of them precedes the tile loop (left to the compiler, the wait
    // would sit at the fragment's first use inside the tile loop, which does
    // not see the tile loads, and drain the ring on every iteration).
    bf16x8 qf[kKSteps];
    {
      const uint16_t* qp = a.q + ((int64_t)b * a.qlen + t_row) * a.q_srow + (int64_t)h_row * a.q_sh;
      // step kk takes dims 16 kk + 8 g2 .. + 7
  #pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) qf[kk] = *(const bf16x8*)(qp + 16 * kk + 8 * g2);
    }

    const char* kv = (const char*)a.kv;
    const int elem = FP8 ? 1 : 2;
    const int64_t sp_bytes = a.kv_sp * elem;
    const int64_t st_bytes = a.kv_st * elem;
    const uint32_t sp32 = (uint32_t)sp_bytes, st32 = (uint32_t)st_bytes;
    const PD_CONST int32_t* bt_row = as_const(a.bt) + (int64_t)b * a.bt_sb;
    // an attended block-table entry of this wave's rows is out of range
    // (combined over the workgroup at the end of the piece)
    bool bad = false;

    // ---- block-table entries of a tile (scalar loads, one iteration ahead) --
    // The entries are only checked when the tile is issued, so the scalar
    // loads stay in flight for a whole iteration.  Page class PC = 16: every
    // page of 16 tokens or more; a 16-row region of a tile then lies inside
    // one page, and a wave reads the one entry of the region it loads.
    // PC < 16: each issuing wave reads the entries of its own rows' pages
    // only (kCand of them), and each lane picks its row's page.
    constexpr bool kGen = PC == 0;
    constexpr bool kBigP = PC >= 16;
    constexpr int kWaveRows = FP8 ? 16 : 8;                 // rows of a tile one issuing wave loads
    // candidate pages of an issuing wave's rows
    constexpr int kCand = kBigP ? 1 : kGen ? (FP8 ? 6 : 4) : kWaveRows / (PC > 0 ? PC : 1);
    const int p_shift = kBigP ? a.p_shift : kGen ? 0 : __builtin_ctz(PC > 0 ? PC : 1);
    // hi_blk >= 1 whenever a tile is read
    const int last_page = kGen ? (hi_blk - 1) / a.P : (hi_blk - 1) >> p_shift;
    struct TilePages {
      int id[kCand];
      bool att;                      // the wave's region is attended (PC = 16)
      int slot0;                     // token slot of the wave's region's (PC = 16) or the
                                     // wave's (general pages) first row
      int first;                     // page index of entry 0 (PC < 16)
    };
    auto fetch = [&](int T) {
      TilePages tp;
      if constexpr (kBigP) {
        // the entry of region (wave / waves per page) % 2 only, the one this
        // wave loads (the other waves check the other region's entry)
        const int tok = 32 * T + 16 * ((wave / (kIssueWaves / 2)) & 1);
        tp.att = tok < hi_blk;
        tp.slot0 = tok & ((1 << p_shift) - 1);
        tp.id[0] = tp.att ? bt_row[tok >> p_shift] : 0;
      } else {
        // this wave's rows are tile tokens kWaveRows * w .. + kWaveRows - 1
        const int tok = 32 * T + kWaveRows * (wave & (FP8 ? 1 : 3));
        if constexpr (kGen) {
          tp.first = tok / a.P;
          tp.slot0 = tok - tp.first * a.P;
        } else {
          tp.first = tok >> p_shift;
          tp.slot0 = 0;
        }
  #pragma unroll
        for (int c = 0; c < kCand; ++c) tp.id[c] = bt_row[min(tp.first + c, last_page)];
      }
      return tp;
    };

    // Issue this wave's share of the HBM->LDS loads of a tile into a ring
    // slot: issuing wave w loads page w / (waves per page), instructions
    // (w % waves per page) * kLoadsPerWave + j of that page.  An issuing wave
    // always issues exactly kLoadsPerWave loads (a page that is not read comes
    // from a harmless 16-byte source), so its vmcnt bookkeeping is exact.
    constexpr int kWavesPerPage = kIssueWaves / 2;
    const int my_page = wave / kWavesPerPage;
    const int i0 = (wave % kWavesPerPage) * kLoadsPerWave;   // first instruction of this wave
    // fp8: instruction i of a page reads 64 bytes of each of its 16 rows;
    // bf16: wave w reads rows 8 (w % 2) .. + 7 of its page, one 128-byte line
    // of each per instruction (lanes permuted inside the line, see tile_off)
    // fp8: instruction i fills chunks c8 = 4 i + lane / 16 of the region,
    // chunk c8 of row r at slot 16 c8 + (r ^ 4 (c8 % 2)), so the lane loads
    // row (lane % 16) ^ 4 ((lane / 16) % 2)
    const int row8 = (lane & 15) ^ (((lane >> 4) & 1) << 2);
    const uint32_t lane_off =
        FP8 ? (uint32_t)(row8 * st_bytes) + 16u * (uint32_t)(lane >> 4)
            : (uint32_t)((8 * (wave & 1) + (lane >> 3)) * st_bytes) + 16u * (uint32_t)((lane & 7) ^ (lane >> 3) ^ (wave & 1));
    constexpr int kGStep = FP8 ? 64 : 128;     // global bytes per instruction (into every row)
    constexpr int kLStep = FP8 ? 1024 : 2048;  // LDS bytes per instruction
    const int g_first = FP8 ? 64 * i0 : 0;
    const int l_first = FP8 ? i0 * 1024 : (wave & 1) * 1024;
    // A tile's loads for this wave, validated: load j reads base + j kGStep
    // (+ voff, PC = 16) into LDS address dst + j kLStep.  PC < 16: base is
    // the lane's own address.  A page that is not read comes from the first
    // bytes of q (one query row is 1152 bytes, past the last load's end at
    // 8 * 128 + 16 bytes), whose values no product sees.
    static_assert(kLoadsPerWave <= 9 && (kLoadsPerWave - 1) * kGStep + 16 <= kRowBytes, "load steps stay inside one q row");
    struct TileLoads {
      const char* base;
      uint32_t voff;
      uint32_t dst;
    };
    const uint32_t num_pages = (uint32_t)a.num_pages;
    auto prepare = [&](const TilePages& tp, int slot) {
      TileLoads tl;
      tl.dst = lds_addr(lds + slot * kRingTile + my_page * (FP8 ? kPageRegion8 : kPageRegion) + l_first);
      if constexpr (kBigP) {
        const bool inr = (uint32_t)tp.id[0] < num_pages;
        bad |= tp.att && !inr;
        const bool ok = tp.att && inr;
        // 32 x 32-bit products (the host keeps both strides below 4 GiB)
        tl.base = ok ? kv + (uint64_t)(uint32_t)tp.id[0] * sp32 + (uint64_t)(uint32_t)tp.slot0 * st32 + g_first
                     : (const char*)a.q;
        tl.voff = ok ? lane_off : 0u;
      } else {
        // every entry this wave read is of an attended page if at or below
        // the block's last page; general pages: candidates past the page of
        // the wave's last row are read (inside the attended pages) but are
        // not this wave's, so they are neither used nor checked here
        const int n_cand = kGen ? (tp.slot0 + kWaveRows - 1) / a.P + 1 : kCand;
        if (wave < kIssueWaves) {
  #pragma unroll
          for (int c = 0; c < kCand; ++c)
            bad |= c < n_cand && tp.first + c <= last_page && (uint32_t)tp.id[c] >= num_pages;
        }
        // the lane's row (0 .. kWaveRows - 1 of this wave's rows) is in
        // candidate page row / PC (general pages: (slot0 + row) / P); a
        // select tree over wave-uniform values (a select chain over the array
        // would become a per-lane index into scratch memory)
        const int row = FP8 ? row8 : (lane >> 3);
        int cand, slot;
        if constexpr (kGen) {
          const int rr = tp.slot0 + row;
          cand = rr / a.P;
          slot = rr - cand * a.P;
        } else {
          cand = row >> __builtin_ctz(PC > 0 ? PC : 1);
          slot = row & ((PC > 0 ? PC : 1) - 1);
        }
        int v[kCand];
  #pragma unroll
        for (int c = 0; c < kCand; ++c) v[c] = __builtin_amdgcn_readfirstlane(tp.id[c]);
  #pragma unroll
        for (int bit = 1; bit < kCand; bit <<= 1)
  #pragma unroll
          for (int c = 0; c + bit < kCand; c += 2 * bit) v[c] = (cand & bit) ? v[c + bit] : v[c];
        const int id = v[0];
        const bool ok = tp.first + cand <= last_page && (uint32_t)id < num_pages;
        const uint32_t chunk = FP8 ? 16u * (uint32_t)(lane >> 4) + (uint32_t)g_first
                                   : 16u * (uint32_t)((lane & 7) ^ (lane >> 3) ^ (wave & 1));
        tl.base = ok ? kv + (int64_t)id * sp_bytes + slot * st_bytes + chunk : (const char*)a.q;
        tl.voff = 0u;
      }
      return tl;
    };
    auto load_one = [&](const TileLoads& tl, int j) { dma_step<kGStep, kLStep, !kBigP>(j, tl.base, tl.voff, tl.dst); };
    auto issue = [&](const TilePages& tp, int slot) {
      const TileLoads tl = prepare(tp, slot);
      if (wave < kIssueWaves) {
  #pragma unroll
        for (int j = 0; j < kLoadsPerWave; ++j) load_one(tl, j);
      }
    };

    float m_seen = neg_inf();   // exact running max of this lane's score row
    float m_ref = neg_inf();    // fixed reference of the current pass
    float l_run = 0.f;
    // Output accumulator: O^T for the wave's 128 output dims (4 blocks d of
    // 32) x the block's 128 rows (4 groups r of 32), block (d, r) = o[4 d + r],
    // in all 256 AGPRs.  (The score accumulator is in arch VGPRs.)
    f32x16 o[16];

    // lane-constant parts of the transpose-read addresses
    const int q16 = lane >> 4;
    const int L16 = lane & 15;
    const int vrow = 4 * (q16 >> 1) + (L16 >> 2);          // + 16 s (+ 8): rows 0..15 of a page
    const int vcol0 = 16 * (q16 & 1) + 4 * (L16 & 3);      // + 32 blk
    // read a covers row vrow (row octet 0), read b row vrow + 8 (octet 1); chunk
    // 4 blk + vcc0 of dim block blk = 4 wave + d sits in line 2 wave + d / 2 at
    // slot 8 vrow + ((4 (d % 2) + vcc0) ^ vrow ^ octet)
    const int vcc0 = vcol0 >> 3;                           // chunk column within the block
    const int vya = vcc0 ^ vrow, vyb = vcc0 ^ vrow ^ 1;
    const uint32_t vlane_off = (uint32_t)(wave * 4096 + 128 * vrow + (vcol0 & 7) * 2);

    // tile t as loaded: its ring slot (bf16 layout, or fp8 chunk-column-major)
    auto tile_bf16 = [&](int t) -> PD_LDS char* { return lds + (t & (NS - 1)) * kRingTile; };
    // FP8 chunk c8 (16 codes) of row r of a page region: slot 16 c8 + (r ^ 4 (c8 % 2))
    auto slot8 = [](int c8, int r) { return 16 * c8 + (r ^ ((c8 & 1) << 2)); };
    // FP8 V^T (8-bit transpose read): in a 16-lane group, lane j receives
    // byte j % 8 of the 8 bytes addressed by lanes 2 e + (j >= 8), e = 0..7.
    // Lane s of group (m16 = lane / 16 % 2, g = lane / 32) addresses dims
    // 16 m16 + 8 (s % 2) .. + 7 of the block, key 8 (e / 4) + 4 g + e % 4 for
    // e = s / 2: the key order of the P^T operand.
    const int v8e = L16 >> 1;
    const int v8key = 8 * (v8e >> 2) + 4 * g2 + (v8e & 3);
    const int v8m = (lane >> 4) & 1;
    const uint32_t v8lane_off = (uint32_t)(v8m * 256 + ((v8key ^ (v8m << 2)) << 4) + (L16 & 1) * 8);
    // P^T fragment (row group r, key step s) of tile t: 64 lanes x 16 bytes
    PD_LDS char* pbuf = lds + kPOff + lane * 16;
    auto p_slot = [&](int t, int r, int s) { return pbuf + (t & 1) * kPBufBytes + (2 * r + s) * 1024; };

    for (int pass = 0; pass < 2; ++pass) {
    // pass 1 only runs if pass 0 saw a score too far above its reference
    m_ref = pass == 0 ? neg_inf() : m_seen;
    l_run = 0.f;
    bool overflow = false;
  #pragma unroll
    for (int i = 0; i < 16; ++i)
  #pragma unroll
      for (int e = 0; e < 16; ++e) o[i][e] = 0.f;

    // Iteration k computes the scores of tile k and the P.V product of tile
    // k-1 (whose probabilities every wave published in iteration k-1), FP8
    // interleaving the two, bf16 running the product after the score chain
    // with tile k's softmax.  Iteration 0 multiplies the zeroed view of
    // "tile -1" by zeroed probabilities; iteration n computes throw-away
    // scores on stale data to finish tile n-1's product.  Ring: tile t in
    // slot t mod 4; tile k+2 is issued at iteration k into the slot of tile
    // k-2.
    {
      PD_LDS char* z = tile_bf16(-1);
      for (int i = tid; i < kRingTile / 16; i += kWaves * 64) *(PD_LDS u32x4*)(z + i * 16) = u32x4{0, 0, 0, 0};
      PD_LDS char* zp = lds + kPOff + ((-1) & 1) * kPBufBytes;
      for (int i = tid; i < kPBufBytes / 16; i += kWaves * 64) *(PD_LDS u32x4*)(zp + i * 16) = u32x4{0, 0, 0, 0};
    }
    TilePages pg_next;
    if (n > 0) issue(fetch(tb), 0);
    if (n > 1) issue(fetch(tb + 1), 1);
    if (n > 2) pg_next = fetch(tb + 2);
    wait_vmcnt<0>();   // the query fragments (and tiles 0 and 1)

    for (int k = 0; k <= n; ++k) {
      const bool live = k < n;   // iteration n only finishes tile n-1
      if (k + 1 < n)
        wait_vmcnt<kLoadsPerWave>();
      else
        wait_vmcnt<0>();
      // tile k is in LDS, so are the probabilities of tile k-1; every wave is
      // done with iteration k-1
      __syncthreads();
      const int tok0 = (tb + k) * kTileTokens;
      PD_LDS char* tk = tile_bf16(k);       // scores of tile k
      PD_LDS char* tv = tile_bf16(k - 1);   // product of tile k-1
      if (live && tok0 + kTileTokens > hi_blk) {
        // The block's last tile: token rows at or past its largest row limit
        // (stale or never-loaded page slots) become zeros, so no score or V
        // row there can carry a NaN into the products; a barrier orders the
        // zeros before every read of the tile.
        const int r0 = max(hi_blk - tok0, 0);
        constexpr int kChunks = FP8 ? 36 : 72;   // 16-byte chunks per row
        for (int i = tid; i < 2 * kChunks * 16; i += kWaves * 64) {
          const int r16 = i & 15, cc = (i >> 4) % kChunks, pg = i / (kChunks * 16);
          if (16 * pg + r16 >= r0) {
            PD_LDS char* zc = FP8 ? tk + pg * kPageRegion8 + slot8(cc, r16) * 16
                                  : tk + pg * kPageRegion + tile_off(cc, r16);
            *(PD_LDS u32x4*)zc = u32x4{0, 0, 0, 0};
          }
        }
        __syncthreads();
      }
      // Tile k+2 goes into the slot of tile k-2, which every wave finished in
      // iteration k-1.  Its loads are spread over the score steps below: issued
      // all at once they fill the memory request queue and stall the wave.
      const bool load_next = k + 2 < n && wave < kIssueWaves;
      // Where the next tiles' address work and block-table reads go.  A
      // scalar table load still in flight when an LDS wait comes up makes
      // that wait cover it too (the two share the lgkm counter, and scalar
      // loads return out of order), so in the score loop every K fragment
      // wait would stall on it.  FP8 and the classes of pages below 16
      // tokens therefore prepare the loads while the first K reads are in
      // flight and issue the table loads after the score loop, past the
      // iteration's last LDS wait (bf16 at 8-token pages -8.5%, FP8 -1.3%);
      // bf16 at 16-token pages and above measured 0.8% faster with both
      // before the loop (same box, A/B twice).
      constexpr bool kLateFetch = FP8 || !kBigP;
      TileLoads tl_next;
      if (!kLateFetch && k + 2 < n) {
        tl_next = prepare(pg_next, (k + 2) & (NS - 1));
        if (k + 3 < n) pg_next = fetch(tb + k + 3);
      }

      // ---- S^T(k) = K Q^T (36 MFMAs, one chain); FP8: with O^T += V^T P^T of
      // tile k-1 (32 MFMAs) in between ---------------------------------------
      // Fragments are read a few MFMA pairs ahead of their use; scheduling
      // barriers pin that order (left alone, the scheduler moves every read
      // next to its MFMA and the wave stalls on LDS latency at each step).
      // The score accumulator lives in arch VGPRs: the chain is issued in the
      // asm form of the MFMA, with a VGPR destination (compiled MFMAs put
      // every accumulator in AGPRs, where the output blocks take all 256).
      // The hardware forwards a dependent accumulator between back-to-back
      // MFMAs of one shape; the asm carries the wait states the compiler
      // would otherwise insert: 3 before an MFMA reads operands a vector ALU
      // instruction has just written (the FP8 conversions; 2 required), and
      // 24 after the last one before a vector ALU instruction reads the
      // result (11 required after an 8-pass MFMA, 19 after a 16-pass one).
      f32x16 sacc;
      // chunk 2 kk + g2 of row kr = l32 % 16: line kk / 4, slot
      // 8 (kr % 8) + ((2 (kk % 4)) ^ kz) with the lane constant kz
      const int kr = l32 & 15, kz = g2 ^ (kr & 7) ^ (kr >> 3);
      PD_LDS char* kp = tk + (l32 >> 4) * kPageRegion + (kr >> 3) * 1024 + 128 * (kr & 7);
      auto kread = [&](int kk) { return *(PD_LDS bf16x8*)(kp + (kk >> 2) * 2048 + 16 * ((2 * (kk & 3)) ^ kz)); };
      // FP8: 8 codes -> bf16x8, exact (scale 1: every E4M3FN value is a bf16 value)
      auto cvt8x8 = [](uint32_t lo, uint32_t hi) {
        const u32x4 w = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false)),
                         __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true)),
                         __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false)),
                         __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true))};
        return __builtin_bit_cast(bf16x8, w);
      };
      // FP8 K of step kk (dims 16 kk + 8 g2 .. + 7 of row l32): half g2 of
      // chunk kk of row l32 % 16 in region l32 / 16 (the bf16 path's dim
      // order, so the two paths round alike)
      PD_LDS char* kp8 = tk + (l32 >> 4) * kPageRegion8 + g2 * 8;
      const int kr8 = l32 & 15;
      auto kread8 = [&](int kk) { return *(PD_LDS u32x2*)(kp8 + slot8(kk, kr8) * 16); };
      // V^T fragment of key step s (one 16-token page) and this wave's dim
      // block d: read a rows vrow.., read b rows vrow + 8.. (slot + 8)
      PD_LDS char* vbase = tv + vlane_off;
      auto vread = [&](int s, int d) {
        if constexpr (FP8) {
          typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
          const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (PD_LDS i32x2*)(tv + s * kPageRegion8 + (4 * wave + d) * 512 + v8lane_off));
          return cvt8x8((uint32_t)w[0], (uint32_t)w[1]);
        }
        PD_LDS char* pl = vbase + s * kPageRegion + (d >> 1) * 2048;
        PD_LDS char* pa = pl + 16 * ((4 * (d & 1)) ^ vya);
        PD_LDS char* pb = pl + 1024 + 16 * ((4 * (d & 1)) ^ vyb);
        const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PD_LDS bf16x4*)pa);
        const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PD_LDS bf16x4*)pb);
        const u32x2 ua = __builtin_bit_cast(u32x2, va);
        const u32x2 ub = __builtin_bit_cast(u32x2, vb);
        return __builtin_bit_cast(bf16x8, u32x4{ua[0], ua[1], ub[0], ub[1]});
      };
      auto pread = [&](int r, int s) { return *(PD_LDS bf16x8*)p_slot(k - 1, r, s); };
      // product step j (0..29): s = j / 15, block index 4 d + r = j % 15.  V^T
      // fragment v = 4 s + d lives in vf[v & 1]; P^T fragment (r, s) in pf[r].
      {
        constexpr int kKAhead = FP8 ? kKAheadFp8 : kKAheadBf16;
        // kf: bf16 K fragments; vf, pf: the FP8 path's V^T and P^T fragments
        bf16x8 kf[kKAhead], vf[2], pf[4];
        u32x2 kw[kKAhead];   // FP8: raw K codes, a few steps ahead
        if constexpr (FP8) {
  #pragma unroll
          for (int i = 0; i < kKAhead; ++i) kw[i] = kread8(i);
        } else {
  #pragma unroll
          for (int i = 0; i < kKAhead; ++i) kf[i] = kread(i);
        }
        if constexpr (FP8) {
          vf[0] = vread(0, 0);
          vf[1] = vread(0, 1);
  #pragma unroll
          for (int r = 0; r < 4; ++r) pf[r] = pread(r, 0);
        }
        if constexpr (kLateFetch) {
          if (k + 2 < n) tl_next = prepare(pg_next, (k + 2) & (NS - 1));
          __builtin_amdgcn_sched_barrier(0);
        }
        // bf16: the chain in two copies, with and without the next tile's
        // loads, so no step branches on whether this wave loads (FP8, whose
        // chain also carries the products, spills registers that way and
        // branches per load instead).
        // FP8: step kk's K fragment is converted one step ahead, right after
        // step kk-1's score MFMA, into the other of two registers (never the
        // one the MFMA in flight reads)
        bf16x8 kc[2];
        if constexpr (FP8) kc[0] = cvt8x8(kw[0][0], kw[0][1]);
        auto chain = [&](auto with_loads) {
    #pragma unroll
          for (int kk = 0; kk < kKSteps; ++kk) {
            {
              bf16x8 kop;
              if constexpr (FP8)
                kop = kc[kk & 1];
              else
                kop = kf[kk % kKAhead];
              // (FP8: 3 wait states after the conversions: the previous step's
              // product MFMA and K read and one s_nop, or an s_nop 2 where the
              // previous step has neither; last step: 24 before the vector
              // ALU reads the result)
#define PD_MFMA_S(PRE, C, POST)                                                         \
    asm volatile(PRE "v_mfma_f32_32x32x16_bf16 %0, %1, %2, " C POST                      \
                 : "+v"(sacc) : "v"(kop), "v"(qf[kk]))
              // (the first step only writes the accumulator: the previous
              // tile's scores are dead by then, so their registers can hold
              // the softmax's copy without a move)
#define PD_MFMA_S0(PRE)                                                                 \
    asm volatile(PRE "v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"                            \
                 : "=&v"(sacc) : "v"(kop), "v"(qf[kk]))
              if constexpr (FP8) {
                if (kk == 0)
                  PD_MFMA_S0("s_nop 2\n\t");
                else if (kk <= 32)
                  PD_MFMA_S("s_nop 0\n\t", "%0", "");
                else if (kk + 1 < kKSteps)
                  PD_MFMA_S("s_nop 2\n\t", "%0", "");
                else
                  PD_MFMA_S("s_nop 2\n\t", "%0", "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
              } else {
                if (kk == 0)
                  PD_MFMA_S0("");
                else if (kk + 1 < kKSteps)
                  PD_MFMA_S("", "%0", "");
                else
                  PD_MFMA_S("", "%0", "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
              }
#undef PD_MFMA_S
#undef PD_MFMA_S0
            }
            if constexpr (FP8) {
              if (kk + 1 < kKSteps) {
                const u32x2 w = kw[(kk + 1) % kKAhead];
                kc[(kk + 1) & 1] = cvt8x8(w[0], w[1]);
              }
              // (the conversions stay ahead of the product MFMA and the K read)
              __builtin_amdgcn_sched_barrier(0);
            }
            if (FP8 && kk < 32) {
              const int s = kk / 16, idx = kk % 16, d = idx >> 2, r = idx & 3, v = 4 * s + d;
              o[idx] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[v & 1], pf[r], o[idx], 0, 0, 0);
              // V^T fragment v is done after its last row group: fetch v + 2
              if (r == 3 && v + 2 < 8) vf[v & 1] = vread((v + 2) >> 2, (v + 2) & 3);
              // P^T (r, 0) is done after block d = 3: fetch (r, 1)
              if (s == 0 && d == 3) pf[r] = pread(r, 1);
            }
            if constexpr (FP8) {
              if (kk + kKAhead < kKSteps) kw[kk % kKAhead] = kread8(kk + kKAhead);
            } else {
              if (kk + kKAhead < kKSteps) kf[kk % kKAhead] = kread(kk + kKAhead);
              // the product's first V^T and P^T fragments (tile k-1), read
              // in the last score steps, past the chain's last K read, so
              // they have landed when the products start
              if (kk == kKSteps - 5) {
                vf[0] = vread(0, 0);
                vf[1] = vread(0, 1);
              } else if (kk == kKSteps - 4 || kk == kKSteps - 3) {
                const int r0 = 2 * (kk - (kKSteps - 4));
                pf[r0] = pread(r0, 0);
                pf[r0 + 1] = pread(r0 + 1, 0);
              }
            }
            if constexpr (decltype(with_loads)::value) {
              if (kk % kLoadSpacing == 0 && kk / kLoadSpacing < kLoadsPerWave && (!FP8 || load_next))
                load_one(tl_next, kk / kLoadSpacing);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        if (FP8 || load_next)
          chain(std::true_type{});
        else
          chain(std::false_type{});
        if (kLateFetch && k + 3 < n) pg_next = fetch(tb + k + 3);
        // The softmax works on the raw scores x (FP8: code . q, with k_scale
        // in the scale cx = c * k_scale): max(x) * cx is max(x * cx) for
        // cx > 0 (min for cx < 0), and each probability takes one fma,
        // exp2(x * cx - m_ref).  With a power-of-two k_scale both caches give
        // the same products, so they round alike.
        float x[16];
  #pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = sacc[e];
        if constexpr (!FP8) {
          // bf16: tile k-1's 32 products with tile k's softmax
          // interleaved by hand, one product and a slice of the softmax per
          // step, a scheduling barrier closing each step (the products do not
          // depend on the softmax; in the score loop they only padded the
          // score chain, which issues back to back on its own).  The softmax
          // runs on the last pass too (its state only changes for a live
          // tile), so the products and the softmax stay in one block.
          float mt = 0.f, m_a = 0.f, m_ref_n = 0.f, mref = 0.f, lsum = 0.f;
          bool ovf_n = false;
          float p[16];
          u32x4 pw0 = {0, 0, 0, 0}, pw1 = {0, 0, 0, 0};
          // V^T fragment v = 4 s + d in vr[v % 2], P^T (r, s) in pr[r]
          // (the first ones read in the score loop)
          bf16x8 vr[2] = {vf[0], vf[1]}, pr[4] = {pf[0], pf[1], pf[2], pf[3]};
          const bool mask_tile = tok0 + kTileTokens > hi_wmin;   // wave-uniform
  #pragma unroll
          for (int j = 0; j < 32; ++j) {
            const int s = j / 16, idx = j % 16, d = idx >> 2, r = idx & 3, v = 4 * s + d;
            o[idx] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[v & 1], pr[r], o[idx], 0, 0, 0);
            if (r == 3 && v + 2 < 8) vr[v & 1] = vread((v + 2) >> 2, (v + 2) & 3);
            if (s == 0 && d == 3) pr[r] = pread(r, 1);
            if (j < 2) {
              // causal limit of this lane's row: token tok0 + 8 (e / 4) + 4 g2 + e % 4 < hi_row
              if (mask_tile) {
  #pragma unroll
                for (int e = 8 * j; e < 8 * j + 8; ++e) {
                  const int tok = tok0 + 8 * (e >> 2) + 4 * g2 + (e & 3);
                  x[e] = tok >= hi_row ? neg_inf() : x[e];
                }
              }
            } else if (j == 2) {
              // (chains, which the compiler turns into three-input maxima)
              m_a = x[0];
  #pragma unroll
              for (int e = 1; e < 8; ++e) m_a = fmaxf(m_a, x[e]);
            } else if (j == 3) {
              float m_b = x[8];
  #pragma unroll
              for (int e = 9; e < 16; ++e) m_b = fmaxf(m_b, x[e]);
              mt = max_xor32(fmaxf(m_a, m_b)) * c;
            } else if (j == 4) {
              // first non-empty tile of the row: its max becomes the reference
              m_ref_n = m_ref == neg_inf() ? mt : m_ref;
              ovf_n = mt - m_ref_n > kRefHeadroomLog2;   // false while -inf
              mref = m_ref_n == neg_inf() ? 0.f : m_ref_n;
            } else if (j >= 5 && j < 21) {
              // each step adds the previous step's probability (the row sum
              // in the FP8 path's order), so no add waits on the exp just issued
              p[j - 5] = fast_exp2(__builtin_fmaf(x[j - 5], c, -mref));
              if (j > 5) lsum += p[j - 6];
            } else if (j == 21) {
              lsum += p[15];
              pw0 = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7])};
            } else if (j == 22) {
              pw1 = u32x4{pack_bf16x2(p[8], p[9]), pack_bf16x2(p[10], p[11]), pack_bf16x2(p[12], p[13]),
                          pack_bf16x2(p[14], p[15])};
            } else if (j == 23) {
              // publish P^T of this wave's row group (key steps 0 and 1); on
              // the last pass the slot is never read
              *(PD_LDS u32x4*)p_slot(k, wave, 0) = pw0;
              *(PD_LDS u32x4*)p_slot(k, wave, 1) = pw1;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          m_seen = live ? fmaxf(m_seen, mt) : m_seen;
          m_ref = live ? m_ref_n : m_ref;
          overflow = overflow || (live && ovf_n);
          l_run = live ? l_run + lsum : l_run;
          if (!live) break;
        } else {
          if (!live) break;

          // causal limit of this lane's row: token tok0 + 8j + 4 g2 + i < hi_row
          const float cx = c * kscale;
          const bool up = !(cx < 0.f);   // wave-uniform
          // (a masked key's raw score is the one whose probability is 0)
          const float x_masked = up ? neg_inf() : __builtin_inff();
          if (tok0 + kTileTokens > hi_wmin && tok0 + kTileTokens > hi_row) {
  #pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int tok = tok0 + 8 * (e >> 2) + 4 * g2 + (e & 3);
              if (tok >= hi_row) x[e] = x_masked;
            }
          }

          // ---- online softmax against the fixed row reference ----
          float mt = x[0];
          if (up) {
  #pragma unroll
            for (int e = 1; e < 16; ++e) mt = fmaxf(mt, x[e]);
            mt = max_xor32(mt);
          } else {
  #pragma unroll
            for (int e = 1; e < 16; ++e) mt = fminf(mt, x[e]);
            mt = -max_xor32(-mt);
          }
          mt *= cx;
          m_seen = fmaxf(m_seen, mt);
          // first non-empty tile of the row: take its max as the reference (the
          // accumulator and l are still exactly 0, so nothing needs rescaling)
          if (m_ref == neg_inf()) m_ref = mt;
          overflow |= mt - m_ref > kRefHeadroomLog2;           // false while -inf
          const float mref = m_ref == neg_inf() ? 0.f : m_ref;
          float p[16];
          float lsum = 0.f;   // summed as on the bf16 path, so the two round alike
  #pragma unroll
          for (int e = 0; e < 16; ++e) {
            p[e] = fast_exp2(__builtin_fmaf(x[e], cx, -mref));
            lsum += p[e];
          }
          l_run += lsum;
          // Publish P^T (this wave's row group, key step st): the score
          // accumulator's element order (keys 8 (e / 4) + 4 g2 + e % 4) is the
          // key order of the V^T fragments, so each lane's 8 probabilities of a
          // key step are its B-operand fragment as they stand.
  #pragma unroll
          for (int st = 0; st < 2; ++st) {
            const u32x4 w = {pack_bf16x2(p[8 * st + 0], p[8 * st + 1]), pack_bf16x2(p[8 * st + 2], p[8 * st + 3]),
                             pack_bf16x2(p[8 * st + 4], p[8 * st + 5]), pack_bf16x2(p[8 * st + 6], p[8 * st + 7])};
            *(PD_LDS u32x4*)p_slot(k, wave, st) = w;
          }
        }
      }
    }

    // every wave is past its last LDS read of this pass: agree on a rerun and
    // publish the row statistics through the (now idle) ring
    __syncthreads();
    l_run = sum_xor32(l_run);
    PD_LDS int* flags = (PD_LDS int*)lds;
    PD_LDS float* row_l = (PD_LDS float*)(lds + 64);
    PD_LDS float* row_m = row_l + kRowsPerBlock;
    // bit 0: a row overflowed its reference; bit 1: this wave read an
    // out-of-range attended block-table entry
    // (the ballots run with the whole wave active: inside the lane-0 branch
    // they would see lane 0 alone)
    const bool wave_ovf = __ballot(overflow) != 0ull;
    const bool wave_bad = __ballot(bad) != 0ull;
    if (lane == 0) flags[wave] = (wave_ovf ? 1 : 0) | (wave_bad ? 2 : 0);
    if (g2 == 0) {
      row_l[wave * kRowsPerWave + l32] = l_run;
      row_m[wave * kRowsPerWave + l32] = m_ref;
    }
    __syncthreads();
    bool rerun = false;
  #pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      rerun |= (flags[w] & 1) != 0;
      bad |= (flags[w] & 2) != 0;
    }
    float lr[4];
  #pragma unroll
    for (int r = 0; r < 4; ++r) lr[r] = row_l[r * kRowsPerWave + l32];
    __syncthreads();   // the statistics are read before the next pass reuses the ring
    if (!rerun) {
      // ---- epilogue: O for this wave's 128 dims of all 128 rows; the row
      // owner (wave r) also writes the row's LSE ------------------------------
      const float qnan = __builtin_nanf("");
      if (row_ok) {
        const bool empty = !(l_run > 0.f);
        const float lse_nat = empty ? neg_inf() : (m_ref + fast_log2(l_run)) * kLn2;
        const int64_t q_row = (int64_t)b * a.qlen + t_row;
        if (direct) {
          if (a.lse != nullptr && g2 == 0) a.lse[q_row * a.lse_srow + h_row] = bad ? qnan : lse_nat;
        } else {
          if (g2 == 0) a.ws[((q_row * a.H + h_row) * S + split) * (kLv + 1) + kLv] = bad ? qnan : lse_nat;
        }
      }
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rb * kRowsPerBlock + r * kRowsPerWave + l32;
        if (row < rows_req) {
          const int64_t q_row = (int64_t)b * a.qlen + row / a.H;
          const int h = row % a.H;
          const float inv = lr[r] > 0.f ? kscale / lr[r] : 0.f;
          if (direct) {
            uint16_t* orow = a.out + q_row * a.o_srow + (int64_t)h * a.o_sh + 32 * kDimBlocksPerWave * wave;
  #pragma unroll
            for (int d = 0; d < kDimBlocksPerWave; ++d)
  #pragma unroll
              for (int j = 0; j < 4; ++j) {
                const f32x16& ob = o[4 * d + r];
                float x0 = ob[4 * j + 0] * inv, x1 = ob[4 * j + 1] * inv;
                float x2 = ob[4 * j + 2] * inv, x3 = ob[4 * j + 3] * inv;
                if (bad) x0 = x1 = x2 = x3 = qnan;
                *(u32x2*)(orow + 32 * d + 8 * j + 4 * g2) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
              }
          } else {
            float* oslot = a.ws + ((q_row * a.H + h) * S + split) * (kLv + 1) + 32 * kDimBlocksPerWave * wave;
  #pragma unroll
            for (int d = 0; d < kDimBlocksPerWave; ++d)
  #pragma unroll
              for (int j = 0; j < 4; ++j) {
                const f32x16& ob = o[4 * d + r];
  #pragma unroll
                for (int i = 0; i < 4; ++i) oslot[32 * d + 8 * j + 4 * g2 + i] = bad ? qnan : ob[4 * j + i] * inv;
              }
          }
        }
      }
      break;
    }
    }
  };

  // ---- walk the requests of the share --------------------------------------
  int ub = b_s, up0 = cb_s;
  while (ub < a.B && (last || up0 < g1)) {
    const int L = unit_len(ub), Lr = unit_real(ub, L);
    const int ntb = __builtin_amdgcn_readfirstlane(block_tiles(L, Lr, n_rb - 1));
    const bool owner = up0 >= g0;   // the request (its virtual tiles) starts in this share
    const int rs = up0 + kPieceTiles;   // its first real tile
    int i0 = 0, i1 = ntb;
    if (split_mode) {
      i0 = max(g0 - rs, 0);
      i1 = min(ntb, g1 - rs);
    } else if (!owner) {
      i1 = 0;   // whole requests only: it belongs to an earlier share
    }
    // slots count from the share that holds the request's first real tile
    const int slot = split_mode ? __builtin_amdgcn_readfirstlane(grp - rs / T) : 0;
    for (int rb = member; rb < n_rb; rb += gs) {
      const int nt = __builtin_amdgcn_readfirstlane(block_tiles(L, Lr, rb));
      const int j1 = min(i1, nt);
      if (i0 < j1) run_piece(ub, rb, i0, j1 - i0, slot);
      if (owner && (nt == 0 || split_mode)) {
        // Partials only: lse = -inf in the split slots no piece of the unit
        // uses (all of them for a unit with no key); a call that merges
        // itself ends the slot list with lse = +inf in the first unused slot
        // (the merge reads no further); or O = 0 / LSE = -inf written directly
        const int nseg = nt > 0 ? (rs + nt - 1) / T - rs / T + 1 : 0;
        const int my_row = rb * kRowsPerBlock + wave * kRowsPerWave + l32;
        if (my_row < rows_req) {
          const int t_row = my_row / a.H, h_row = my_row % a.H;
          const int64_t q_row = (int64_t)ub * a.qlen + t_row;
          if (direct) {
            uint16_t* orow = a.out + q_row * a.o_srow + (int64_t)h_row * a.o_sh;
            for (int d = g2 * 8; d < kLv; d += 16) *(u32x4*)(orow + d) = u32x4{0, 0, 0, 0};
            if (a.lse != nullptr && g2 == 0) a.lse[q_row * a.lse_srow + h_row] = neg_inf();
          } else if (a.partials) {
            for (int sl = nseg + g2; sl < S; sl += 2)
              a.ws[((q_row * a.H + h_row) * S + sl) * (kLv + 1) + kLv] = neg_inf();
          } else if (nseg < S && g2 == 0) {
            a.ws[((q_row * a.H + h_row) * S + nseg) * (kLv + 1) + kLv] = end_of_slots();
          }
        }
      }
    }
    up0 += ntb + kPieceTiles;
    ++ub;
  }
}

}  // namespace

// Launches page class PC for a bf16 or FP8 cache: one workgroup per compute
// unit (the kernel's LDS fits one workgroup per CU).
template <int PC>
hipError_t launch_mla_class(const MlaArgs& a, int n_wg, hipStream_t stream) {
  const dim3 grid(n_wg), block(kWaves * 64);
  if (a.kv_fp8)
    hipLaunchKernelGGL((mla_verify_kernel<4, true, PC>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((mla_verify_kernel<4, false, PC>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace pd
