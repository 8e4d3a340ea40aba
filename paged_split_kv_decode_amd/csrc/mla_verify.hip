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
// * The qlen * H (token, head) pairs of a request are the "rows".  A
//   workgroup of 4 waves (one per SIMD, 512 registers each) owns 128
//   consecutive rows of one request and one split of its keys; each wave
//   owns 32 rows: its query fragment (32 x 576 bf16, 144 VGPRs) and its
//   output accumulator (512 x 32 fp32, all 256 AGPRs) stay in registers for
//   the whole split.  The 4 row blocks of one (request, split) are placed on
//   the same XCD (workgroup-id remap) so they re-read the latent tiles from
//   that XCD's L2.
// * Latent tiles of 32 tokens (2 pages, 36 KB bf16 / 18 KB fp8) stream from
//   HBM into a 3-stage LDS ring shared by the 4 waves, with
//   global_load_lds_dwordx4 (1 KB per wave instruction); one barrier per tile.
//   The FP8 cache is dequantised exactly (v_cvt_scalef32_pk_bf16_fp8, scale
//   1) into a bf16 staging tile; k_scale is folded into the softmax scale and
//   the output.
// * S^T[token, row] = K . Q^T with v_mfma_f32_32x32x16_bf16 (two independent
//   accumulation chains), K fragments read from LDS in batches ahead of
//   their MFMAs.
// * O^T[d, row] += V^T . P^T: P leaves the score MFMA already in B-operand
//   order; V^T is read from the same LDS tile (first 512 dims) with
//   ds_read_b64_tr_b16, a few blocks ahead of their MFMAs.
// * Online softmax in the exp2 domain (x = score * sm_scale * log2 e) with a
//   fixed per-row reference: a row's reference max is its first non-empty
//   tile's max and is never rescaled, so no vector instruction ever touches
//   the accumulator (which is what keeps it in AGPRs).  The exact row max is
//   tracked alongside; if a later score exceeds the reference by more than
//   2^64 (overflow risk) the workgroup runs the split a second time with the
//   exact max as reference.  Real attention scores never trigger it.
// * Each wave owns its rows, so there is no cross-wave combine: a single
//   split writes bf16 O and LSE, several splits write fp32 partials.
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
constexpr int kKAhead = 3;                                         // K fragments in flight
constexpr int kVAhead = 2;                                         // V^T fragments in flight
constexpr int kRopeSteps = 4;                                      // 64 rope dims = 4 k-steps
constexpr int kRegSteps = kKSteps - kRopeSteps;                    // query k-steps kept in VGPRs
constexpr int kVBlocks = kLv / 32;                                 // 16
// p = 2^(x - m_ref) stays below 2^64 while the row max has not grown more
// than this above the reference (fp32 / bf16 hold 2^127; with up to 2^20
// keys and |V| < 2^40 the accumulator cannot overflow).
constexpr float kRefHeadroomLog2 = 64.f;

// LDS tile layout.  A 32-token tile is two 16-row page regions.  Inside a
// region the 16-byte chunk c (of the latent row) of row r16 is stored at
// 16-byte slot 16 * c + (r16 ^ 4 * (c & 1)): chunk-column-major, so
//  * one global_load_lds instruction (64 slots) fills 4 whole chunk columns
//    of one page, and each lane's global offset is a lane constant plus
//    64 bytes per instruction;
//  * a K-operand read (16 rows, one chunk) touches 16 consecutive slots, and
//    a transpose read of V (4 rows x chunks c, c + 1) touches two groups of 4
//    slots whose bank groups differ by the row XOR: both bank-conflict free.
__device__ __forceinline__ int tile_slot(int c, int r16) { return 16 * c + (r16 ^ (4 * (c & 1))); }


template <int NS, bool FP8>
__global__ __launch_bounds__(kWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_verify_kernel(MlaArgs a) {
  constexpr int kRingTile = FP8 ? kTileBytes8 : kTileBytes;
  constexpr int kLoadsPerTile = kRingTile / 1024;                  // 36 or 18
  constexpr int kLoadsPerPage = kLoadsPerTile / 2;
  // bf16: 4 waves x 9 loads; fp8: waves 0 and 1 load one page (9 loads) each,
  // so every issuing wave has the same count for its vmcnt bookkeeping.
  constexpr int kIssueWaves = FP8 ? 2 : 4;
  static_assert(NS == 4, "ring of 4 tiles: k-1 (product), k (scores), k+1, k+2 (loading)");
  constexpr int kStageOff = NS * kRingTile;                         // 2 fp8 -> bf16 tiles
  constexpr int kLoadsPerWave = kLoadsPerTile / kIssueWaves;
  static_assert(kLoadsPerWave * kIssueWaves == kLoadsPerTile, "even load split");
  constexpr int kRopeOff = kStageOff + (FP8 ? 2 * kTileBytes : 0);  // query rope fragments
  constexpr int kLdsBytes = kRopeOff + kWaves * kRopeSteps * 64 * 16;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];
  PD_LDS char* lds = (PD_LDS char*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g2 = lane >> 5;
  const int S = a.S;
  const bool direct = S == 1;

  // ---- the plan ----------------------------------------------------------
  // Work unit = (request b, row block rb): 128 consecutive (token, head) rows
  // of one request, whose keys are its 32-token tiles up to the block's
  // largest row limit.  All units' tiles, request-major then row-block-major,
  // form one flat sequence of U tiles.  The grid is persistent (one workgroup
  // per CU) and workgroup s takes the equal contiguous share [s T, s T + T):
  // every workgroup streams the same number of tiles whatever the length mix.
  // Where a share cuts a unit, each piece is a split with its own partial
  // slot; T is raised until no unit spans more than S shares.  With S == 1
  // shares are rounded to whole units and results are written directly.
  // Logical share ids are XCD-remapped (hardware hands consecutive workgroup
  // ids to the 8 XCDs round-robin) so consecutive shares, which hold the row
  // blocks of one request at the same tile positions, share an XCD and its L2.
  const int n_wg = gridDim.x;
  int sid = blockIdx.x;
  const int per_xcd = n_wg / 8;
  if (sid < per_xcd * 8) sid = (sid % 8) * per_xcd + sid / 8;
  sid = __builtin_amdgcn_readfirstlane(sid);
  const int rows_req = a.qlen * a.H;
  const int n_rb = (rows_req + kRowsPerBlock - 1) / kRowsPerBlock;
  auto unit_len = [&](int b) { return min(max((int)as_const(a.seq_lens)[b], 0), a.max_blocks * a.P); };
  auto unit_real = [&](int b, int L) { return a.real_lens != nullptr ? (int)as_const(a.real_lens)[b] : L; };
  // largest row limit of row block rb of a request with lengths (L, Lr)
  auto block_hi = [&](int L, int Lr, int rb) {
    const int last_row = min(rb * kRowsPerBlock + kRowsPerBlock, rows_req) - 1;
    return max(min(L - a.qlen + 1 + last_row / a.H, Lr), 0);
  };
  auto block_tiles = [&](int L, int Lr, int rb) { return (block_hi(L, Lr, rb) + kTileTokens - 1) / kTileTokens; };

  int nt_sum = 0, nt_max = 0;
  for (int base = 0; base < a.B; base += 64) {
    int req = 0, mx = 0;
    if (base + lane < a.B) {
      const int L = unit_len(base + lane), Lr = unit_real(base + lane, L);
      for (int rb = 0; rb < n_rb; ++rb) {
        const int t = block_tiles(L, Lr, rb);
        req += t;
        mx = max(mx, t);
      }
    }
    nt_sum += wave_sum(req);
    nt_max = max(nt_max, wave_max(mx));
  }
  const int U = __builtin_amdgcn_readfirstlane(nt_sum);
  nt_max = __builtin_amdgcn_readfirstlane(nt_max);
  const bool split_mode = S >= 2;
  int T = max((U + n_wg - 1) / n_wg, kMlaMinSplitTiles);
  // a unit of n tiles cut every T tiles at an arbitrary offset spans at most
  // floor((n - 1) / T) + 2 shares: keep that <= S
  if (split_mode) T = max(T, (nt_max - 1) / (S - 1) + 1);
  T = __builtin_amdgcn_readfirstlane(T);
  const int w_used = __builtin_amdgcn_readfirstlane(max((U + T - 1) / T, 1));
  if (sid >= w_used) return;   // the whole workgroup: no barrier was passed
  const int g0 = sid * T;
  const bool last = sid == w_used - 1;
  const int g1 = last ? U : g0 + T;

  // first request holding tile g0, or starting at or after it
  int b_s = -1, cb_s = 0;
  {
    int C = 0;
    for (int base = 0; base < a.B; base += 64) {
      const bool in = base + lane < a.B;
      int req = 0;
      if (in) {
        const int L = unit_len(base + lane), Lr = unit_real(base + lane, L);
        for (int rb = 0; rb < n_rb; ++rb) req += block_tiles(L, Lr, rb);
      }
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
    // ---- rows of this lane and their causal limits ------------------------
    const int L = unit_len(b);
    const int Lr = unit_real(b, L);
    const int my_row = rb * kRowsPerBlock + wave * kRowsPerWave + l32;
    const bool row_ok = my_row < rows_req;
    const int t_row = row_ok ? my_row / a.H : 0;
    const int h_row = row_ok ? my_row % a.H : 0;
    const int hi_row = row_ok ? max(min(L - a.qlen + 1 + t_row, Lr), 0) : 0;
    const int last_row = min(rb * kRowsPerBlock + kRowsPerBlock, rows_req) - 1;
    const int hi_blk = __builtin_amdgcn_readfirstlane(max(min(L - a.qlen + 1 + last_row / a.H, Lr), 0));
    const int64_t q_row = (int64_t)b * a.qlen + t_row;

    const int pg_hi = __builtin_amdgcn_readfirstlane((hi_blk + a.P - 1) / a.P);

    float kscale = 1.f;
    if constexpr (FP8) {
      if (a.k_scale != nullptr) kscale = a.k_scale[0];
    }
    const float c = a.scale_log2 * kscale;   // log2-domain scale of raw scores

    // ---- Q fragment: B operand of S^T = K Q^T (32 rows x 576 dims) --------
    // The first kRegSteps fragments stay in VGPRs; the last kRopeSteps (the
    // 64 rope dims) live in this wave's LDS area and are read for the last
    // MFMAs of every tile, which keeps the register file within budget.
    bf16x8 qf[kRegSteps];
    PD_LDS char* qrope = lds + kRopeOff + wave * (kRopeSteps * 64 * 16) + lane * 16;
    {
      const uint16_t* qp = a.q + q_row * a.q_srow + (int64_t)h_row * a.q_sh + 8 * g2;
  #pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        u32x4 v = *(const u32x4*)(qp + 16 * kk);
        if (!row_ok) v = u32x4{0, 0, 0, 0};
        if (kk < kRegSteps)
          qf[kk] = __builtin_bit_cast(bf16x8, v);
        else
          *(PD_LDS u32x4*)(qrope + (kk - kRegSteps) * 1024) = v;   // read after the first tile barrier
      }
    }

    const char* kv = (const char*)a.kv;
    const int elem = FP8 ? 1 : 2;
    const int64_t sp_bytes = a.kv_sp * elem;
    const int64_t st_bytes = a.kv_st * elem;
    const PD_CONST int32_t* bt_row = as_const(a.bt) + (int64_t)b * a.bt_sb;
    bool bad = false;

    // ---- block-table entries of a tile (scalar loads, one iteration ahead) --
    // The entries are only checked when the tile is issued, so the scalar
    // loads stay in flight for a whole iteration.
    struct TilePages {
      int id[2];
      bool att[2];   // page attended
    };
    auto fetch = [&](int T) {
      TilePages tp;
  #pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int pidx = 2 * T + j;
        tp.att[j] = pidx < pg_hi;
        tp.id[j] = tp.att[j] ? bt_row[pidx] : 0;
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
    const uint32_t lane_off = (uint32_t)((FP8 ? (lane & 15) : ((lane & 15) ^ (4 * ((lane >> 4) & 1)))) *
                                         st_bytes) + 16u * (uint32_t)(lane >> 4);
    auto issue = [&](const TilePages& tp, int slot) {
      bool pok[2];
  #pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bool inr = tp.id[j] >= 0 && tp.id[j] < a.num_pages;
        // every wave checks both pages, so the flag is workgroup-uniform
        bad |= tp.att[j] && !inr;
        pok[j] = tp.att[j] && inr;
      }
      if (wave >= kIssueWaves) return;
      const bool ok = (my_page & 1) ? pok[1] : pok[0];
      const int my_pid = (my_page & 1) ? tp.id[1] : tp.id[0];
      // instruction i of a page covers 16-byte slots [64 i, 64 i + 64): chunk
      // columns 4 i .. 4 i + 3, i.e. 64 more bytes into every row
      const char* base = ok ? kv + (int64_t)my_pid * sp_bytes + 64 * i0 : (const char*)a.q;
      const uint32_t voff = ok ? lane_off : 0u;
      PD_LDS char* dst = lds + slot * kRingTile + my_page * (FP8 ? kPageRegion8 : kPageRegion) + i0 * 1024;
  #pragma unroll
      for (int j = 0; j < kLoadsPerWave; ++j)
        global_to_lds_16(base + (ok ? 64 * j : 0), voff, lds_addr(dst + j * 1024));
    };

    float m_seen = neg_inf();   // exact running max of this lane's row
    float m_ref = neg_inf();    // fixed reference of the current pass
    float l_run = 0.f;
    // Output accumulator O^T (512 x 32 fp32).  Blocks 0..14 stay in AGPRs;
    // block 15 is parked in VGPRs between tiles, which leaves 16 AGPRs for
    // the score accumulator (all 256 AGPRs plus 16 = the register budget).
    f32x16 o[kVBlocks - 1];
    f32x16 o_last;

    // lane-constant parts of the transpose-read addresses
    const int q16 = lane >> 4;
    const int L16 = lane & 15;
    const int vrow = 4 * (q16 >> 1) + (L16 >> 2);          // + 16 s (+ 8): rows 0..15 of a page
    const int vcol0 = 16 * (q16 & 1) + 4 * (L16 & 3);      // + 32 blk
    // byte offset of this lane's first transpose read (step 0, block 0, read a)
    const int vcc0 = vcol0 >> 3;                           // chunk column
    const uint32_t vlane_off = (uint32_t)(tile_slot(vcc0, vrow) * 16 + (vcol0 & 7) * 2);

    // the bf16 view of tile t: its ring slot, or its fp8 staging buffer
    auto tile_bf16 = [&](int t) -> PD_LDS char* {
      if constexpr (FP8)
        return lds + kStageOff + (t & 1) * kTileBytes;
      else
        return lds + (t & (NS - 1)) * kRingTile;
    };

    for (int pass = 0; pass < 2; ++pass) {
    // pass 1 only runs if pass 0 saw a score too far above its reference
    m_ref = pass == 0 ? neg_inf() : m_seen;
    l_run = 0.f;
    bool overflow = false;
  #pragma unroll
    for (int i = 0; i < kVBlocks - 1; ++i)
  #pragma unroll
      for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  #pragma unroll
    for (int e = 0; e < 16; ++e) o_last[e] = 0.f;

    // Iteration k computes the scores of tile k interleaved with the P.V
    // product of tile k-1 (whose probabilities pb_prev came out of iteration
    // k-1), so the dependent score chain always has independent MFMAs
    // between its steps.  Iteration 0 multiplies the zeroed view of "tile -1"
    // by zero probabilities; iteration n computes throw-away scores on stale
    // data to finish tile n-1's product.  Ring: tile t in slot t mod 4; tile
    // k+2 is issued at iteration k into the slot of tile k-2.
    {
      // zero the view of tile -1 (read by iteration 0's product)
      PD_LDS char* z = tile_bf16(-1);
      for (int i = tid; i < kTileBytes / 16; i += kWaves * 64) *(PD_LDS u32x4*)(z + i * 16) = u32x4{0, 0, 0, 0};
    }
    bf16x8 pb_prev[2] = {bf16x8{}, bf16x8{}};
    TilePages pg_next;
    if (n > 0) issue(fetch(tb), 0);
    if (n > 1) issue(fetch(tb + 1), 1);
    if (n > 2) pg_next = fetch(tb + 2);

    for (int k = 0; k <= n; ++k) {
      const bool live = k < n;   // iteration n only finishes tile n-1
      if (k + 1 < n)
        wait_vmcnt<kLoadsPerWave>();
      else
        wait_vmcnt<0>();
      __syncthreads();  // tile k is in LDS; every wave is done with iteration k-1
      const int tok0 = (tb + k) * kTileTokens;
      if constexpr (FP8) {
        if (live) {
          // exact fp8 -> bf16 into the staging buffer: item = (page, fp8
          // chunk column c8, row r16) -> bf16 chunk columns 2 c8 and 2 c8 + 1
          PD_LDS char* src = lds + (k & (NS - 1)) * kRingTile;
          PD_LDS char* dst = tile_bf16(k);
          for (int i = tid; i < 2 * 36 * 16; i += kWaves * 64) {
            const int r16 = i & 15;
            const int c8 = (i >> 4) % 36;
            const int pg = i / (36 * 16);
            const u32x4 w = *(PD_LDS u32x4*)(src + pg * kPageRegion8 + (16 * c8 + r16) * 16);
            PD_LDS char* dpg = dst + pg * kPageRegion;
  #pragma unroll
            for (int h = 0; h < 2; ++h) {
              u32x4 cv;
              cv[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * h], 1.f, false));
              cv[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * h], 1.f, true));
              cv[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * h + 1], 1.f, false));
              cv[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * h + 1], 1.f, true));
              *(PD_LDS u32x4*)(dpg + tile_slot(2 * c8 + h, r16) * 16) = cv;
            }
          }
          __syncthreads();
        }
      }
      PD_LDS char* tk = tile_bf16(k);       // scores of tile k
      PD_LDS char* tv = tile_bf16(k - 1);   // product of tile k-1
      if (live && tok0 + kTileTokens > hi_blk) {
        // The block's last tile: token rows at or past its largest row limit
        // (stale or never-loaded page slots) become zeros, so no score or V
        // row there can carry a NaN into the products; a barrier orders the
        // zeros before every read of the tile.
        const int r0 = max(hi_blk - tok0, 0);
        for (int i = tid; i < 2 * 72 * 16; i += kWaves * 64) {
          const int r16 = i & 15, cc = (i >> 4) % 72, pg = i / (72 * 16);
          if (16 * pg + r16 >= r0) *(PD_LDS u32x4*)(tk + pg * kPageRegion + tile_slot(cc, r16) * 16) = u32x4{0, 0, 0, 0};
        }
        __syncthreads();
      }
      if (k + 2 < n) {
        issue(pg_next, (k + 2) & (NS - 1));
        if (k + 3 < n) pg_next = fetch(tb + k + 3);
      }

      // ---- S^T(k) = K Q^T (36 MFMAs, one chain) with O^T += V^T P^T of tile
      // k-1 (30 MFMAs for blocks 0..14) in between -----------------------------
      // Fragments are read a few MFMA pairs ahead of their use; scheduling
      // barriers pin that order (left alone, the scheduler moves every read
      // next to its MFMA and the wave stalls on LDS latency at each step).
      f32x16 sacc;
  #pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
      // chunk g2 + 2 kk of row l32 % 16: slot tile_slot(g2, r16) + 32 kk, i.e.
      // one lane base plus an immediate offset per step
      PD_LDS char* kp = tk + (l32 >> 4) * kPageRegion + tile_slot(g2, l32 & 15) * 16;
      auto kread = [&](int kk) { return *(PD_LDS bf16x8*)(kp + kk * 512); };
      // product step j: st = j / 15 (16-token half), blk = j % 15
      auto vread = [&](int j, int blk_off) {
        // read a: rows vrow.., read b: rows vrow + 8.. (slot + 8); block blk
        // is 4 chunk columns (1 KB) further; step st is the next page
        const int st = j / 15, blk = j % 15 + blk_off;
        PD_LDS char* pa = tv + vlane_off + st * kPageRegion + blk * 1024;
        const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PD_LDS bf16x4*)pa);
        const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((PD_LDS bf16x4*)(pa + 128));
        const u32x2 ua = __builtin_bit_cast(u32x2, va);
        const u32x2 ub = __builtin_bit_cast(u32x2, vb);
        return __builtin_bit_cast(bf16x8, u32x4{ua[0], ua[1], ub[0], ub[1]});
      };
      constexpr int kPv = 2 * (kVBlocks - 1);   // 30 product MFMAs in the interleave
      {
        bf16x8 kf[kKAhead], vf[kVAhead], qr[kRopeSteps];
  #pragma unroll
        for (int i = 0; i < kKAhead; ++i) kf[i] = kread(i);
#pragma unroll
        for (int i = 0; i < kVAhead; ++i) vf[i] = vread(i, 0);
  #pragma unroll
        for (int kk = 0; kk < kKSteps; ++kk) {
          const bf16x8 qv = kk < kRegSteps ? qf[kk < kRegSteps ? kk : 0] : qr[kk < kRegSteps ? 0 : kk - kRegSteps];
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk % kKAhead], qv, sacc, 0, 0, 0);
          if (kk < kPv) {
            const int st = kk / 15, blk = kk % 15;
            o[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kk % kVAhead], pb_prev[st], o[blk], 0, 0, 0);
          }
          if (kk + kKAhead < kKSteps) kf[kk % kKAhead] = kread(kk + kKAhead);
          if (kk + kVAhead < kPv) vf[kk % kVAhead] = vread(kk + kVAhead, 0);
          if (kk + kKAhead == kRegSteps) {
  #pragma unroll
            for (int i = 0; i < kRopeSteps; ++i) qr[i] = *(PD_LDS bf16x8*)(qrope + i * 1024);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float x[16];
  #pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = sacc[e] * c;
      {
        // block 15 of tile k-1's product, after the score accumulator is free
        const bf16x8 va = vread(14, 1), vb = vread(29, 1);   // (st 0, blk 15), (st 1, blk 15)
        f32x16 o15 = o_last;
        o15 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb_prev[0], o15, 0, 0, 0);
        o15 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, pb_prev[1], o15, 0, 0, 0);
        o_last = o15;
        asm volatile("" : "+v"(o_last));
      }
      if (!live) break;

      // causal limit of this lane's row: token tok0 + 8j + 4 g2 + i < hi_row
      if (tok0 + kTileTokens > hi_row) {
  #pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tok = tok0 + 8 * (e >> 2) + 4 * g2 + (e & 3);
          if (tok >= hi_row) x[e] = neg_inf();
        }
      }

      // ---- online softmax against the fixed row reference ----
      float mt = x[0];
  #pragma unroll
      for (int e = 1; e < 16; ++e) mt = fmaxf(mt, x[e]);
      mt = fmaxf(mt, shfl_xor(mt, 32));
      m_seen = fmaxf(m_seen, mt);
      // first non-empty tile of the row: take its max as the reference (the
      // accumulator and l are still exactly 0, so nothing needs rescaling)
      if (m_ref == neg_inf()) m_ref = mt;
      overflow |= mt - m_ref > kRefHeadroomLog2;           // false while -inf
      const float mref = m_ref == neg_inf() ? 0.f : m_ref;
      float p[16];
  #pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = fast_exp2(x[e] - mref);
        l_run += p[e];
      }
  #pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 w = {pack_bf16x2(p[8 * st + 0], p[8 * st + 1]), pack_bf16x2(p[8 * st + 2], p[8 * st + 3]),
                         pack_bf16x2(p[8 * st + 4], p[8 * st + 5]), pack_bf16x2(p[8 * st + 6], p[8 * st + 7])};
        pb_prev[st] = __builtin_bit_cast(bf16x8, w);
      }
    }

    // every wave is past its last LDS read of this pass: agree on a rerun
    // through the (now idle) ring
    __syncthreads();
    PD_LDS int* flags = (PD_LDS int*)lds;
    if (lane == 0) flags[wave] = __ballot(overflow) != 0ull ? 1 : 0;
    __syncthreads();
    bool rerun = false;
  #pragma unroll
    for (int w = 0; w < kWaves; ++w) rerun |= flags[w] != 0;
    __syncthreads();   // the flags are read before the next pass reuses the ring
    if (!rerun) break;
    }

    // ---- epilogue: each wave writes its own 32 rows -------------------------
    l_run += shfl_xor(l_run, 32);
    if (row_ok) {
    const bool empty = !(l_run > 0.f);
    const float qnan = __builtin_nanf("");
    const float lse_nat = empty ? neg_inf() : (m_ref + fast_log2(l_run)) * kLn2;
    if (direct) {
      const float inv = empty ? 0.f : kscale / l_run;
      uint16_t* orow = a.out + q_row * a.o_srow + (int64_t)h_row * a.o_sh;
  #pragma unroll
      for (int blk = 0; blk < kVBlocks; ++blk)
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * blk + 8 * j + 4 * g2;
          const f32x16& ob = blk < kVBlocks - 1 ? o[blk] : o_last;
          float x0 = ob[4 * j + 0] * inv, x1 = ob[4 * j + 1] * inv;
          float x2 = ob[4 * j + 2] * inv, x3 = ob[4 * j + 3] * inv;
          if (bad) x0 = x1 = x2 = x3 = qnan;
          *(u32x2*)(orow + d) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        }
      if (a.lse != nullptr && g2 == 0) a.lse[q_row * a.lse_srow + h_row] = bad ? qnan : lse_nat;
    } else {
      const float inv = empty ? 0.f : kscale / l_run;
      float* slot = a.ws + ((q_row * a.H + h_row) * S + split) * (kLv + 1);
      float* oslot = slot;
  #pragma unroll
      for (int blk = 0; blk < kVBlocks; ++blk)
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * blk + 8 * j + 4 * g2;
          const f32x16& ob = blk < kVBlocks - 1 ? o[blk] : o_last;
  #pragma unroll
          for (int i = 0; i < 4; ++i) oslot[d + i] = bad ? qnan : ob[4 * j + i] * inv;
        }
      if (g2 == 0) slot[kLv] = bad ? qnan : lse_nat;
    }
    }
    };

  // ---- walk the units of the share ----------------------------------------
  int ub = b_s, urb = 0, up0 = cb_s;
  int uL = unit_len(ub), uLr = unit_real(ub, uL);
  while (ub < a.B && (last || up0 < g1)) {
    const int nt = __builtin_amdgcn_readfirstlane(block_tiles(uL, uLr, urb));
    const bool owner = up0 >= g0;   // the unit starts in this share
    if (nt > 0) {
      int i0 = 0, i1 = nt;
      if (split_mode) {
        i0 = max(g0 - up0, 0);
        i1 = min(nt, g1 - up0);
      } else if (!owner) {
        i1 = 0;   // whole units only: it belongs to an earlier share
      }
      if (i0 < i1) {
        const int slot = split_mode ? __builtin_amdgcn_readfirstlane(sid - up0 / T) : 0;
        run_piece(ub, urb, i0, i1 - i0, slot);
      }
    }
    if (owner && (nt == 0 || split_mode)) {
      // lse = -inf in the split slots no piece of the unit uses (all of them
      // for a unit with no key), or O = 0 / LSE = -inf written directly
      const int nseg = nt > 0 ? (up0 + nt - 1) / T - up0 / T + 1 : 0;
      const int my_row = urb * kRowsPerBlock + wave * kRowsPerWave + l32;
      if (my_row < rows_req) {
        const int t_row = my_row / a.H, h_row = my_row % a.H;
        const int64_t q_row = (int64_t)ub * a.qlen + t_row;
        if (direct) {
          uint16_t* orow = a.out + q_row * a.o_srow + (int64_t)h_row * a.o_sh;
          for (int d = g2 * 8; d < kLv; d += 16) *(u32x4*)(orow + d) = u32x4{0, 0, 0, 0};
          if (a.lse != nullptr && g2 == 0) a.lse[q_row * a.lse_srow + h_row] = neg_inf();
        } else {
          for (int sl = nseg + g2; sl < S; sl += 2)
            a.ws[((q_row * a.H + h_row) * S + sl) * (kLv + 1) + kLv] = neg_inf();
        }
      }
    }
    up0 += nt;
    if (++urb == n_rb) {
      urb = 0;
      if (++ub < a.B) {
        uL = unit_len(ub);
        uLr = unit_real(ub, uL);
      }
    }
  }
}

}  // namespace

// Workgroups per launch: one per compute unit (the kernel's LDS fits one
// workgroup per CU).  Queried once per device.
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
  dim3 grid(n), block(kWaves * 64);
  if (a.kv_fp8)
    hipLaunchKernelGGL((mla_verify_kernel<4, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((mla_verify_kernel<4, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace pd
