// Forward attention kernel, bf16 inputs, fp32 accumulation, gfx950.
//
// Tiled forward with an online softmax: each workgroup owns BR query rows of
// one (batch, head) and streams key/value tiles of BC rows through LDS,
// keeping per row a running maximum m and a running sum l and rescaling the
// output accumulator when m grows, so the result equals the one-shot softmax
// (llmis.ru chapter 3.1 "The cost of attention", section 5; the unite.ai page
// "Flash Attention: Revolucionando a Eficiencia dos Modelos Transformer",
// sections "O Algoritmo de Flash Attention" and "A Matematica por tras da
// Flash Attention").  Only O and the per-row log-sum-exp are written; the
// score tile lives in registers.
//
// Data flow per wave (RB blocks of 32 query rows):
//   S^T (keys x rows) = K_tile * Q^T     32x32x16 bf16 MFMA; K from LDS,
//                                        Q^T held in registers all along.
//   each lane owns one query row per row block (lane % 32) and 16 keys per
//   32-key block, so the row max/sum are in-lane reductions plus one
//   lane-pair exchange.
//   O^T (d x rows) += V_tile^T * P^T     P^T comes straight from the S^T
//                                        accumulator registers (converted to
//                                        bf16); V^T is read from LDS with the
//                                        gfx950 transpose read.
// Every K and V^T fragment read from LDS feeds RB matrix products (one per
// row block), so RB = 2 halves the LDS traffic per FLOP at the price of a
// 512-register, one-wave-per-SIMD budget.
// Software pipeline: K tiles are staged one tile ahead of V tiles, so while
// the vector ALU exponentiates tile t the matrix cores already compute S for
// tile t+1; the two instruction streams are interleaved explicitly.
// Scores are handled in the base-2 domain: exp(scale*s) = 2^(scale*log2e*s).
//
// Two instantiations, d = 128 without a mask and d = 256 with a window, are
// compiled in a translation unit of their own (fwd_bf16_ilp.hip includes this
// file with EXATTN_FWD_ILP defined), which the build gives a different
// instruction scheduler; this file's own unit holds the rest and the entry
// points.
#include "device_common.hpp"
#include "launch.hpp"
#include "pattern.hpp"

namespace exattn {
namespace {

// Lazy rescale threshold (log2 units): the running max used for the
// exponentials is only raised when a row's max exceeds it by more than this,
// so probabilities stay <= 2^8 and most tiles skip the O rescale.  The final
// normalisation uses the same max, so the result is unchanged.
constexpr float kRescaleThreshold = 8.0f;

// NW waves per workgroup, RB blocks of 32 query rows per wave, BC keys per
// tile, WPE the waves per SIMD the register budget is sized for.
template <int D>
struct FwdCfg;
template <>
struct FwdCfg<64> {
  static constexpr int NW = 4, RB = 1, BC = 64, WPE = 2;
};
template <>
struct FwdCfg<128> {
  static constexpr int NW = 8, RB = 1, BC = 64, WPE = 2;  // 256 rows: one K/V tile copy per 8 waves
};
template <>
struct FwdCfg<256> {
  static constexpr int NW = 4, RB = 1, BC = 32, WPE = 1;
};

// Waves per workgroup: the full-row pass gathers kFullRows rows; under a
// pattern, 4 waves: a partial tile often keeps only some waves busy, and two
// 4-wave workgroups per CU fill each other's idle SIMDs (8 waves were 14-26%
// slower on the Longformer and BigBird workloads).
template <int D, int MODE>
constexpr int fwd_waves() {
  return MODE == kMaskFull ? kFullRows / 32 : MODE == kMaskPattern ? 4 : FwdCfg<D>::NW;
}

// MODE: kMaskNone, kMaskWindow (contiguous band of key tiles, analytic
// masks), kMaskPattern (the workgroup's tile list from the pattern plan; the
// union mask on partial tiles; full rows are left to the full-row pass), or
// kMaskFull (a pattern's full rows, gathered, against one chunk of key tiles;
// with several chunks the normalised partial O and its log-sum-exp go to the
// partial buffers).
template <int D, int MODE>
__global__ __launch_bounds__((fwd_waves<D, MODE>() * 64), FwdCfg<D>::WPE) void fwd_bf16_kernel(
    const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
    __bf16* __restrict__ Og, float* __restrict__ LSEg, int n, int n_qblocks, int total_blocks,
    float scale_log2, int window, int group, PatternDev pat, FullDev full) {
  constexpr bool WINDOWED = MODE == kMaskWindow;
  constexpr bool PATTERN = MODE == kMaskPattern;
  constexpr bool FULL = MODE == kMaskFull;
  constexpr int NW = fwd_waves<D, MODE>();
  constexpr int RB = FwdCfg<D>::RB;
  constexpr int BC = FwdCfg<D>::BC;
  constexpr int BR = 32 * RB * NW;
  constexpr int NT = NW * 64;
  constexpr int NKB = BC / 32;  // 32-key blocks per tile
  constexpr int NDS = D / 16;   // 16-wide d steps
  constexpr int NDB = D / 32;   // 32-wide d blocks of the output

  __shared__ __attribute__((aligned(16))) __bf16 kbuf[2][BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 vbuf[2][BC * D];
  poison_lds(kbuf, vbuf);

  int head, qb;
  // full rows: this workgroup's chunk and group of rows
  int f_rows = 0, f_groups = 0, f_chunks = 1, f_chunk = 0, f_group = 0;
  if constexpr (FULL) {
    f_rows = full.info[kFullCount];
    f_groups = full.info[kFullGroups];
    f_chunks = full.info[kFullChunks];
    const int per_head = f_groups * f_chunks;
    const int item = blockIdx.x;
    if (item >= (total_blocks / n_qblocks) * per_head) return;  // whole workgroup: no barrier skipped
    head = item / per_head;
    const int r = item - head * per_head;
    f_chunk = r / f_groups;
    f_group = r - f_chunk * f_groups;
    qb = 0;
  } else {
    const int bid = xcd_remap(blockIdx.x, total_blocks);
    head = bid / n_qblocks;
    qb = bid - head * n_qblocks;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Query heads [g*group, (g+1)*group) share key/value head g; consecutive
  // logical blocks of one group land on the same XCD and share its L2.
  const size_t head_off = (size_t)head * n * D;
  const size_t kv_off = (size_t)(head / group) * n * D;
  const __bf16* Q = Qg + head_off;
  const __bf16* K = Kg + kv_off;
  const __bf16* V = Vg + kv_off;

  const int q0 = qb * BR;
  const int w0 = q0 + wave * 32 * RB;  // first row of this wave
  int my_row[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if constexpr (FULL) {  // slot of the full-row list; rows past the list count as past n
      const int slot = f_group * BR + wave * 32 * RB + 32 * rb + l32;
      my_row[rb] = slot < f_rows ? full.idx[slot] : n;
    } else {
      my_row[rb] = w0 + 32 * rb + l32;
    }
  }

  // Q^T operands, kept in registers: lane holds Q[my_row][16*ds + 8*hi .. +8].
  bf16x8 qreg[RB][NDS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const bool ok = my_row[rb] < n;
    const u32x4* src = (const u32x4*)(Q + (size_t)(ok ? my_row[rb] : 0) * D + 8 * hi);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      qreg[rb][ds] = __builtin_bit_cast(bf16x8, ok ? src[2 * ds] : u32x4{0, 0, 0, 0});
  }

  // Key tiles this block visits: a contiguous range (the band of the whole
  // block for a window), or the block's list from the pattern plan.
  int k_lo = 0, k_hi = n;
  if constexpr (WINDOWED) band_keys(q0, q0 + BR, n, window, &k_lo, &k_hi);
  if constexpr (FULL) {
    const int tl = full.info[kFullTilesPerChunk];
    k_lo = f_chunk * tl * BC;
    k_hi = min(n, k_lo + tl * BC);
  }
  const int t_lo = k_lo / BC;
  const int t_hi = (k_hi + BC - 1) / BC;
  // Under a pattern: first the tiles of gathered full keys (every row sees
  // them), then the listed tiles.  Iteration index i < n_gath is gathered
  // tile i; the others are list entry i - n_gath.
  const int* plist = PATTERN ? pat.list + (size_t)qb * pat.stride : nullptr;
  const int n_full_keys = PATTERN ? pat.other_count[0] : 0;
  const int n_gath = (n_full_keys + BC - 1) / BC;
  const int n_listed = PATTERN ? pat.count[qb] : 0;
  const int n_tiles = PATTERN ? (n_listed < 0 ? 0 : n_gath + n_listed) : t_hi - t_lo;
  auto tile_at = [&](int i) { return PATTERN ? plist[i - n_gath] >> kEntryTileShift : t_lo + i; };
  // keys visible to each of this lane's rows through the band
  int key_lo[RB];
  unsigned key_span[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    int lo = 0, hi_k = n;
    if constexpr (WINDOWED) band_keys(my_row[rb], my_row[rb] + 1, n, window, &lo, &hi_k);
    if constexpr (PATTERN) {
      if (pat.window >= 0)
        band_keys(my_row[rb], my_row[rb] + 1, n, pat.window, &lo, &hi_k);
      else
        hi_k = lo;  // no band term
    }
    key_lo[rb] = lo;
    key_span[rb] = (unsigned)max(hi_k - lo, 0);
  }

  using Tile = TileAsync<D, BC, NT>;
  using Dma = TileDma<D, BC, NT>;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t dma_off[Dma::IT];  // this thread's chunk offsets in a full K or V tile
  Dma::init(tid, dma_off);

  // S^T for one K tile in LDS: lanes = query rows, registers = keys.  Each K
  // fragment feeds the RB row blocks.
  // S^T of key block kb of one K tile in LDS.
  auto compute_s_block = [&](const __bf16* Ks, int kb, f32x16 (&s)[RB][NKB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[rb][kb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8 a = lds_row_frag<D>(Ks, kb * 32 + l32, ds, hi);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb][kb] = mfma32(a, qreg[rb][ds], s[rb][kb]);
    }
  };
  auto compute_s = [&](const __bf16* Ks, f32x16 (&s)[RB][NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) compute_s_block(Ks, kb, s);
  };

  f32x16 o[RB][NDB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[rb][i] = f32x16{};
  float m_run[RB], l_part[RB];  // running max (log2 domain) and this lane's share of the sum
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = kNegInf;
    l_part[rb] = 0.0f;
  }

  // Prologue: K and V of the first tile, K of the second.  Key rows past n
  // are clamped copies; their scores are masked to -inf (P = 0).
  // Gathered tiles read the full keys' copies, laid out like the rows of a
  // key/value head (rows past their count: clamped copies, masked below).
  const size_t gath_off = kv_off;
  auto issue_kv = [&](const __bf16* src, const __bf16* gath, int i, __bf16* buf) {
    if constexpr (PATTERN) {
      const bool g = i < n_gath;
      const int r0 = g ? i * BC : tile_at(i) * BC;
      Tile::issue((g ? gath + gath_off : src) + (size_t)r0 * D, (g ? n_full_keys : n) - r0, buf, tid);
    } else {
      const int t = tile_at(i);
      const __bf16* base = src + (size_t)t * BC * D;
      if (t * BC + BC <= n)
        Dma::issue(base, dma_off, buf, wave_s);
      else
        Dma::issue_tail(base, n - t * BC, buf, tid, wave_s);
    }
  };
  auto issue_k = [&](int i, __bf16* buf) { issue_kv(K, pat.gath_a, i, buf); };
  auto issue_v = [&](int i, __bf16* buf) { issue_kv(V, pat.gath_b, i, buf); };
  if (n_tiles > 0) {
    issue_k(0, kbuf[0]);
    issue_v(0, vbuf[0]);
    if (n_tiles > 1) issue_k(1, kbuf[1]);
  }
  wait_all_and_barrier();

  // Under a pattern a wave skips the work of a partial listed tile where
  // none of its rows sees a key (the layout misses the wave and the band
  // misses its rows), and of every tile when its rows are all full rows or
  // past n; the loads and barriers stay shared by the workgroup.
  bool wave_live = true;
  if constexpr (PATTERN) wave_live = w0 < n && pat.own_full[w0 >> 5] != ~0u;
  auto wave_sees = [&](int i) -> bool {
    if constexpr (!PATTERN) {
      return true;
    } else {
      if (!wave_live) return false;
      if (i < n_gath) return true;
      const int entry = plist[i - n_gath];
      if (!(entry & 1)) return true;
      const int c0 = (entry >> kEntryTileShift) * BC;
      const bool a = (entry >> (1 + wave)) & 1;
      return a || (pat.window >= 0 && c0 <= w0 + 31 + pat.window && w0 <= c0 + BC - 1 + pat.window);
    }
  };

  f32x16 s_cur[RB][NKB];
  bool act_cur = !PATTERN || (n_tiles > 0 && wave_sees(0));
  if (act_cur) compute_s(kbuf[0], s_cur);
  // The first iteration copies tile 2's K rows over tile 0's: every wave must
  // have read tile 0's K rows for its scores first.
  wait_all_and_barrier();

  for (int j = 0; j < n_tiles; ++j) {
    // V of tile j+1 into the V buffer read last iteration, K of tile j+2 into
    // the K buffer read last iteration (both released by the last barrier).
    if (j + 1 < n_tiles) issue_v(j + 1, vbuf[(j + 1) & 1]);
    if (j + 2 < n_tiles) issue_k(j + 2, kbuf[j & 1]);
    const bool gathered = PATTERN && j < n_gath;
    const int kbase = gathered ? 0 : tile_at(j) * BC;

    const bool act_next = !PATTERN || (j + 1 < n_tiles && wave_sees(j + 1));
    if (act_cur) {
      // ---- masks: key tail, sliding window, pattern ---------------------------
      bool need_mask = kbase + BC > n;
      if constexpr (WINDOWED) {
        const int r_hi = w0 + 32 * RB - 1;
        need_mask = need_mask || max(r_hi - kbase, kbase + BC - 1 - w0) > window;
      }
      if constexpr (PATTERN) {
        static_assert(RB == 1 && BC % 32 == 0, "pattern masks assume one 32-row block per wave");
        // A gathered tile masks only its slots past the full keys' count (its
        // keys are slots 0.., every row sees them); a listed tile keeps the
        // pairs of its band or layout that are not full keys (those come from
        // the gathered tiles), and a wave the layout covers needs no mask
        // unless the tile crosses the end of the sequence or holds a full key.
        uint32_t lay = 1u;
        int key_end = n_full_keys - j * BC;
        bool mask = key_end < BC;
        if (!gathered) {
          const int entry = plist[j - n_gath];
          lay = (entry >> (1 + wave)) & 1;
          key_end = n;
          mask = (entry & 1) && !(lay && kbase + BC <= n && !(entry & kEntryHasFull));
        }
        if (mask) {
          // visible: key < key_end, (band or layout), and not a full key;
          // bitwise operators into one select per element: no short-circuit
          // branches
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const uint32_t fk = gathered ? 0u : pat.other_full[(kbase >> 5) + kb] >> (4 * hi);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int e = 8 * (r >> 2) + (r & 3);  // acc_row(r, lane) - 4*hi
              const int key = kbase + kb * 32 + e + 4 * hi;
              const uint32_t vis = (uint32_t)(key < key_end) &
                                   ((uint32_t)((unsigned)(key - key_lo[0]) < key_span[0]) | lay) & ~(fk >> e);
              s_cur[0][kb][r] = (vis & 1u) ? s_cur[0][kb][r] : kNegInf;
            }
          }
        }
      } else if (need_mask) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kbase + kb * 32 + acc_row(r, lane);
              s_cur[rb][kb][r] = (unsigned)(key - key_lo[rb]) < key_span[rb] ? s_cur[rb][kb][r] : kNegInf;
            }
      }

      // ---- running max and (rare) rescale -------------------------------------
      float msub[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[rb][kb][r]);
        mx = pair_max(mx);
        const float mx2 = mx * scale_log2;  // -inf stays -inf
        const bool grow = mx2 > m_run[rb] + kRescaleThreshold || (m_run[rb] == kNegInf && mx2 != kNegInf);
        if (__any(grow)) {
          const float m_new = grow ? mx2 : m_run[rb];
          const float alpha = grow ? fast_exp2(m_run[rb] - m_new) : 1.0f;  // m_run=-inf -> 0
          l_part[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][db][r] *= alpha;
          m_run[rb] = m_new;
        }
        msub[rb] = m_run[rb] == kNegInf ? 0.0f : m_run[rb];
      }

      // ---- exponentials (vector ALU) || S of the next tile (matrix cores) -----
      // P of key block kb goes to bf16 (the operand of the P V product); once a
      // block is converted its fp32 registers receive that block of the next
      // tile's S, so the next S needs no registers of its own and the
      // exponentials of block kb+1 run beside the matrix products of block kb.
      // On the last tile the next S reads a stale K buffer; it is unused.  The
      // fp32 row sum is split over independent partial sums.
      bf16x8 pb[RB][BC / 16];
      float lsum[RB][4];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) lsum[rb][i] = 0.0f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s_cur[rb][kb][r] = fast_exp2(__builtin_fmaf(s_cur[rb][kb][r], scale_log2, -msub[rb]));
            lsum[rb][r & 3] += s_cur[rb][kb][r];
          }
          pb[rb][2 * kb] = acc_to_operand(s_cur[rb][kb], 0);
          pb[rb][2 * kb + 1] = acc_to_operand(s_cur[rb][kb], 1);
        }
        if (act_next) compute_s_block(kbuf[(j + 1) & 1], kb, s_cur);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) l_part[rb] += (lsum[rb][0] + lsum[rb][1]) + (lsum[rb][2] + lsum[rb][3]);

      // ---- O^T += V^T P^T -------------------------------------------------------
      // A operand (V^T): lane l needs V[key(t)][db*32 + l%32] with the keys in
      // the k order of pb (the transpose read delivers exactly that).
      const __bf16* Vs = vbuf[j & 1];
#pragma unroll
      for (int st = 0; st < BC / 16; ++st)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 a = lds_col_frag<D>(Vs, 16 * st, 32 * db, lane);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[rb][db] = mfma32(a, pb[rb][st], o[rb][db]);
        }
      {
        constexpr int NP = (BC / 16) * NDB, kLead = 3;
        EXATTN_SCHED(kSchedDSRead, 2 * kLead);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          EXATTN_SCHED(kSchedMFMA, RB);
          if (i + kLead < NP) EXATTN_SCHED(kSchedDSRead, 2);
        }
      }
    } else if (act_next) {
      compute_s(kbuf[(j + 1) & 1], s_cur);
    }
    act_cur = act_next;

    wait_all_and_barrier();
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) -----------------------
  // A row that saw no key (possible only under a pattern without a window)
  // gets O = 0 and LSE = -inf.  Under a pattern the full rows are left to the
  // full-row pass; that pass writes partial results when it has several chunks.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = pair_sum(l_part[rb]);
    bool store = my_row[rb] < n;
    if constexpr (PATTERN) store = store && !bit_of(pat.own_full, my_row[rb]);
    if (FULL && store && f_chunks > 1) {
      const float inv = 1.0f / l_tot;  // every chunk holds at least one key
      const size_t slot = (size_t)(head * f_chunks + f_chunk) * f_groups * BR + f_group * BR + wave * 32 * RB +
                          32 * rb + l32;
      float* prow = full.part + slot * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = db * 32 + 8 * g + 4 * hi;
          *(f32x4*)(prow + dd) = f32x4{o[rb][db][4 * g] * inv, o[rb][db][4 * g + 1] * inv,
                                       o[rb][db][4 * g + 2] * inv, o[rb][db][4 * g + 3] * inv};
        }
      if (hi == 0) full.part_lse[slot] = kLn2 * (m_run[rb] + fast_log2(l_tot));
    } else if (store) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      __bf16* Orow = Og + head_off + (size_t)my_row[rb] * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = db * 32 + 8 * g + 4 * hi;
          u32x2 w;
          w[0] = pack_bf16x2(o[rb][db][4 * g + 0] * inv, o[rb][db][4 * g + 1] * inv);
          w[1] = pack_bf16x2(o[rb][db][4 * g + 2] * inv, o[rb][db][4 * g + 3] * inv);
          *(u32x2*)(Orow + dd) = w;
        }
      if (hi == 0) LSEg[(size_t)head * n + my_row[rb]] = l_tot > 0.0f ? kLn2 * (m_run[rb] + fast_log2(l_tot)) : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// Forward with paired waves (d = 128 and 256, all keys or a window's band).
// ---------------------------------------------------------------------------
// The 8 waves of a workgroup form 4 pairs (wave w and wave w+4 share a SIMD);
// a pair owns 32 query rows.  The S-wave holds the rows' Q in registers,
// forms the scores of each key tile, keeps the running maximum and sum of
// every row and hands P (bf16 MFMA operands) and the rows' rescale factors to
// its partner through LDS; the O-wave holds the output accumulator and adds
// P V.  The O-wave runs one tile behind: in iteration i the S-wave works on
// tile i (matrix products, then exponentials) while the O-wave adds tile i-1
// (matrix products only), so one wave's vector work can run beside the other
// wave's products.  This is the producer / consumer split and the overlap of
// softmax with the matrix products that the unite.ai page "Flash Attention:
// Revolucionando a Eficiencia dos Modelos Transformer" describes in its
// section "FlashAttention-3", applied to the two waves of a SIMD.  Splitting
// the registers this way (Q and the scores in one wave, O in the other) also
// lets d = 256 run two waves per SIMD, where one wave holding Q and O needed
// all 512 registers.
template <int D>
struct PairFwd {
  static constexpr int BC = D == 256 ? 32 : 64;  // keys per tile
  static constexpr int NKB = BC / 32;            // 32-key blocks per tile
  static constexpr int NT = 512, BR = 128;       // threads; query rows per workgroup
  static constexpr int kTile = BC * D * 2;       // bytes of one K or V tile
  // LDS layout (bytes)
  static constexpr int kK = 0;                       // [2] K tiles
  static constexpr int kV = kK + 2 * kTile;          // [2] V tiles
  static constexpr int kPPair = NKB * 2 * 64 * 16;   // one pair's P operands
  static constexpr int kP = kV + 2 * kTile;          // [2][pair]
  static constexpr int kA = kP + 2 * 4 * kPPair;     // [2][pair][32 rows] rescale factors (fp32)
  static constexpr int kBytes = kA + 2 * 4 * 32 * 4;
  static_assert(kBytes <= 160 * 1024, "one workgroup per CU");
};

// Used at d = 256.  (At d = 128 the S-wave's exponentials outweigh its
// partner's products and the kernel that keeps 8 row blocks per workgroup is
// faster.)
template <int D, int MODE>
constexpr bool fwd_pair_dispatch() {
  return D == 256 && (MODE == kMaskNone || MODE == kMaskWindow);
}

template <int D, int MODE>
__global__ __launch_bounds__(512, 2) void fwd_pair_kernel(const __bf16* __restrict__ Qg,
                                                          const __bf16* __restrict__ Kg,
                                                          const __bf16* __restrict__ Vg, __bf16* __restrict__ Og,
                                                          float* __restrict__ LSEg, int n, int n_qblocks,
                                                          int total_blocks, float scale_log2, int window, int group) {
  using C = PairFwd<D>;
  constexpr bool WINDOWED = MODE == kMaskWindow;
  constexpr int BC = C::BC, NKB = C::NKB, NT = C::NT, BR = C::BR;
  constexpr int NDS = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(16))) char lds[C::kBytes];
  poison_lds(lds);

  const int bid = xcd_remap(blockIdx.x, total_blocks);
  const int head = bid / n_qblocks;
  const int qb = bid - head * n_qblocks;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const bool swave = wave < 4;  // S-wave, else O-wave

  // Query heads [g*group, (g+1)*group) share key/value head g.
  const size_t head_off = (size_t)head * n * D;
  const size_t kv_off = (size_t)(head / group) * n * D;
  const __bf16* K = Kg + kv_off;
  const __bf16* V = Vg + kv_off;
  const int q0 = qb * BR;
  const int w0 = q0 + pair * 32;  // first row of the pair
  const int my_row = w0 + l32;    // this lane's row (both waves of the pair)

  // key tiles of the workgroup's band (all keys without a window)
  int k_lo = 0, k_hi = n;
  if constexpr (WINDOWED) band_keys(q0, q0 + BR, n, window, &k_lo, &k_hi);
  const int t_lo = k_lo / BC;
  const int n_tiles = (k_hi + BC - 1) / BC - t_lo;

  // Every thread of the workgroup takes part in every copy.  Key rows past n
  // are clamped copies; their scores are masked (P = 0).
  using Dma = TileDma<D, BC, NT>;
  uint32_t dma_off[Dma::IT];
  Dma::init(tid, dma_off);
  auto issue = [&](const __bf16* src, int i, int buf_off) {
    const int t = t_lo + i;
    const __bf16* base = src + (size_t)t * BC * D;
    __bf16* dst = (__bf16*)(lds + buf_off);
    if (t * BC + BC <= n)
      Dma::issue(base, dma_off, dst, wave);
    else
      Dma::issue_tail(base, n - t * BC, dst, tid, wave);
  };
  // Copies of iteration i: K of tile i+1 (read by the S-wave in iteration
  // i+1) and V of tile i (read by the O-wave in iteration i+1), each into the
  // buffer of its kind read in iteration i-1 (released by that iteration's
  // barrier).
  auto issue_iteration = [&](int i) {
    if (i + 1 < n_tiles) issue(K, i + 1, C::kK + ((i + 1) & 1) * C::kTile);
    if (i < n_tiles) issue(V, i, C::kV + (i & 1) * C::kTile);
  };
  // a pair skips the key tiles its rows' band misses
  auto pair_sees = [&](int i) -> bool {
    if constexpr (WINDOWED) {
      const int c0 = (t_lo + i) * BC;
      return c0 <= w0 + 31 + window && w0 <= c0 + BC - 1 + window;
    } else {
      return true;
    }
  };
  const int p_off = C::kP + pair * C::kPPair + 16 * lane;  // + buffer * 4 * kPPair + operand * 1024
  const int a_off = C::kA + pair * 128 + 4 * l32;          // + buffer * 512

  // The S-wave's Q^T operands (lane: Q[my_row][16*ds + 8*hi .. +8]) are
  // loaded before the first wait, which then covers them: the compiler's own
  // wait for these loads would otherwise sit inside the loop, where it would
  // also wait for the copies just issued.
  bf16x8 qreg[NDS];
  if (swave) {
    const bool ok = my_row < n;
    const u32x4* src = (const u32x4*)(Qg + head_off + (size_t)(ok ? my_row : 0) * D + 8 * hi);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qreg[ds] = __builtin_bit_cast(bf16x8, ok ? src[2 * ds] : u32x4{0, 0, 0, 0});
  }
  if (n_tiles > 0) issue(K, 0, C::kK);
  wait_all_and_barrier();

  if (swave) {
    // keys this lane's row sees: [key_lo, key_lo + key_span)
    int key_lo = 0, key_hi = n;
    if constexpr (WINDOWED) band_keys(my_row, my_row + 1, n, window, &key_lo, &key_hi);
    const unsigned key_span = (unsigned)max(key_hi - key_lo, 0);
    float m_run = kNegInf, l_part = 0.0f;  // running max (log2 domain), this lane's share of the sum

    for (int i = 0; i <= n_tiles; ++i) {
      issue_iteration(i);
      if (i < n_tiles && pair_sees(i)) {
        const __bf16* Ks = (const __bf16*)(lds + C::kK + (i & 1) * C::kTile);
        const int kbase = (t_lo + i) * BC;
        // S^T = K Q^T: lanes = the pair's rows, registers = keys
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          s[kb] = f32x16{};
#pragma unroll
          for (int ds = 0; ds < NDS; ++ds) s[kb] = mfma32(lds_row_frag<D>(Ks, kb * 32 + l32, ds, hi), qreg[ds], s[kb]);
        }
        // masks: the key tail and the band
        bool need_mask = kbase + BC > n;
        if constexpr (WINDOWED) need_mask = need_mask || max(w0 + 31 - kbase, kbase + BC - 1 - w0) > window;
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kbase + kb * 32 + acc_row(r, lane);
              s[kb][r] = (unsigned)(key - key_lo) < key_span ? s[kb][r] : kNegInf;
            }
        }
        // running max with the lazy rescale: the max used for the
        // exponentials is raised only when a row's max exceeds it by more
        // than kRescaleThreshold; alpha (1 otherwise) rescales O and the sum
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        const float mx2 = pair_max(mx) * scale_log2;  // -inf stays -inf
        const bool grow = mx2 > m_run + kRescaleThreshold || (m_run == kNegInf && mx2 != kNegInf);
        const float alpha = grow ? fast_exp2(m_run - mx2) : 1.0f;  // m_run = -inf: 0
        if (grow) m_run = mx2;
        l_part *= alpha;
        const float msub = m_run == kNegInf ? 0.0f : m_run;
        // P = 2^(scale*log2e*s - m), its bf16 operands, and the row sum
        bf16x8 pb[2 * NKB];
        float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -msub));
            lsum[r & 3] += s[kb][r];
          }
          pb[2 * kb] = acc_to_operand(s[kb], 0);
          pb[2 * kb + 1] = acc_to_operand(s[kb], 1);
        }
        l_part += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
        // to the O-wave: lane-private 16-byte slots, consecutive lanes in
        // consecutive slots; the factor once per row
        const int b = i & 1;
#pragma unroll
        for (int c = 0; c < 2 * NKB; ++c)
          *(u32x4*)(lds + p_off + b * (4 * C::kPPair) + c * 1024) = __builtin_bit_cast(u32x4, pb[c]);
        if (hi == 0) *(float*)(lds + a_off + b * 512) = alpha;
      }
      wait_all_and_barrier();
    }
    // 1/l of each row to the O-wave; the log-sum-exp, ln 2 * (m + log2 l)
    // (a row that saw no key: LSE = -inf)
    const float l_tot = pair_sum(l_part);
    if (hi == 0) {
      *(float*)(lds + a_off) = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      if (my_row < n) LSEg[(size_t)head * n + my_row] = l_tot > 0.0f ? kLn2 * (m_run + fast_log2(l_tot)) : kNegInf;
    }
    __syncthreads();
  } else {
    // O^T (d x rows) accumulator: lanes = the pair's rows
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    for (int i = 0; i <= n_tiles; ++i) {
      issue_iteration(i);
      if (i >= 1 && pair_sees(i - 1)) {
        const int b = (i - 1) & 1;
        const float alpha = *(const float*)(lds + a_off + b * 512);
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        }
        bf16x8 pb[2 * NKB];
#pragma unroll
        for (int c = 0; c < 2 * NKB; ++c) pb[c] = *(const bf16x8*)(lds + p_off + b * (4 * C::kPPair) + c * 1024);
        // O^T += V^T P^T: V^T through the transpose read, in the k order of
        // the P operands
        const __bf16* Vs = (const __bf16*)(lds + C::kV + b * C::kTile);
#pragma unroll
        for (int st = 0; st < BC / 16; ++st)
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db] = mfma32(lds_col_frag<D>(Vs, 16 * st, 32 * db, lane), pb[st], o[db]);
      }
      wait_all_and_barrier();
    }
    __syncthreads();  // the S-wave's 1/l
    const float inv = *(const float*)(lds + a_off);
    if (my_row < n) {
      __bf16* Orow = Og + head_off + (size_t)my_row * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = db * 32 + 8 * g + 4 * hi;
          u32x2 w;
          w[0] = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
          w[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
          *(u32x2*)(Orow + dd) = w;
        }
    }
  }
}

// Merge of the full rows' chunks (when there are several): with each
// chunk's normalised O_c and log-sum-exp L_c, L = log sum_c exp(L_c) and
// O = sum_c exp(L_c - L) O_c (the two-block merge of the online softmax,
// applied over all chunks at once).  One thread per four consecutive
// elements of a row, in a grid-stride loop; the chunks are read in order, so
// the result is deterministic.
template <int D>
__global__ __launch_bounds__(256) void fwd_full_merge_kernel(FullDev full, __bf16* __restrict__ Og,
                                                             float* __restrict__ LSEg, int n, int heads) {
  constexpr int Q4 = D / 4;
  const int R = full.info[kFullCount], C = full.info[kFullChunks];
  if (C <= 1) return;
  const size_t GB = (size_t)full.info[kFullGroups] * kFullRows;  // slots per (head, chunk)
  const long items = (long)heads * R * Q4;
  for (long it = (long)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += (long)gridDim.x * blockDim.x) {
    const long hs = it / Q4;
    const int q = (int)(it - hs * Q4);
    const int head = (int)(hs / R), slot = (int)(hs - (long)head * R);
    const size_t s0 = (size_t)head * C * GB + slot;
    float m = kNegInf;
    for (int c = 0; c < C; ++c) m = fmaxf(m, full.part_lse[s0 + c * GB]);
    f32x4 acc = f32x4{};
    float l = 0.0f;
    if (m != kNegInf) {
      for (int c = 0; c < C; ++c) {
        const float w = expf(full.part_lse[s0 + c * GB] - m);
        l += w;
        acc += w * *(const f32x4*)(full.part + (s0 + c * GB) * D + 4 * q);
      }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int row = full.idx[slot];
    u32x2 w;
    w[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    w[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *(u32x2*)(Og + ((size_t)head * n + row) * D + 4 * q) = w;
    if (q == 0) LSEg[(size_t)head * n + row] = l > 0.0f ? m + logf(l) : kNegInf;
  }
}

// The kernels of the modes the paired kernel does not take.
template <int D, int MODE>
hipError_t launch_d_main(const FwdParams& p, hipStream_t stream);

template <int D, int MODE>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  if constexpr (fwd_pair_dispatch<D, MODE>()) {
    constexpr int BR = PairFwd<D>::BR;
    const int nqb = (p.n + BR - 1) / BR;
    const long total = (long)nqb * p.B * p.H;
    if (total > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_pair_kernel<D, MODE>), dim3((unsigned)total), dim3(PairFwd<D>::NT), 0, stream,
                       (const __bf16*)p.q, (const __bf16*)p.k, (const __bf16*)p.v, (__bf16*)p.o, p.lse, p.n, nqb,
                       (int)total, p.scale * kLog2e, p.window, p.group);
    return hipGetLastError();
  } else {
    return launch_d_main<D, MODE>(p, stream);
  }
}

template <int D, int MODE>
hipError_t launch_d_main(const FwdParams& p, hipStream_t stream) {
  constexpr int BR = 32 * FwdCfg<D>::RB * fwd_waves<D, MODE>();
  const int nqb = (p.n + BR - 1) / BR;
  const long total = (long)nqb * p.B * p.H;
  if (total > 0x7fffffffL) return hipErrorInvalidValue;
  const float scale_log2 = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, MODE>), dim3((unsigned)total), dim3(fwd_waves<D, MODE>() * 64), 0, stream,
                     (const __bf16*)p.q, (const __bf16*)p.k, (const __bf16*)p.v, (__bf16*)p.o, p.lse, p.n,
                     nqb, (int)total, scale_log2, p.window, p.group, p.pattern, p.full);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || MODE != kMaskFull) return e;
  hipLaunchKernelGGL((fwd_full_merge_kernel<D>), dim3(1024), dim3(256), 0, stream, p.full, (__bf16*)p.o, p.lse, p.n,
                     p.B * p.H);
  return hipGetLastError();
}

#ifndef EXATTN_FWD_ILP
template <int MODE>
hipError_t launch_mode(const FwdParams& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return launch_d<64, MODE>(p, stream);
    case 128:
      if constexpr (MODE == kMaskNone)
        return launch_fwd_bf16_ilp(p, stream);
      else
        return launch_d<128, MODE>(p, stream);
    case 256:
      if constexpr (MODE == kMaskWindow)
        return launch_fwd_bf16_ilp(p, stream);
      else
        return launch_d<256, MODE>(p, stream);
    default: return hipErrorInvalidValue;
  }
}
#endif

}  // namespace

#ifdef EXATTN_FWD_ILP
hipError_t launch_fwd_bf16_ilp(const FwdParams& p, hipStream_t stream) {
  if (p.d == 128 && p.window < 0) return launch_d<128, kMaskNone>(p, stream);
  if (p.d == 256 && p.window >= 0) return launch_d<256, kMaskWindow>(p, stream);
  return hipErrorInvalidValue;
}
#else

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.pattern.list != nullptr) {
    if (p.pattern.own_full == nullptr || p.pattern.other_full == nullptr || p.pattern.count == nullptr)
      return hipErrorInvalidValue;
    // the full keys' copies, then the pattern pass, then the full rows' pass
    // (its partial results reuse the copies' scratch region)
    hipError_t e = launch_pattern_gather(p.pattern, (const __bf16*)p.k, (const __bf16*)p.v, nullptr, nullptr,
                                         p.B * p.H / p.group, p.n, p.d, stream);
    if (e == hipSuccess) e = launch_mode<kMaskPattern>(p, stream);
    if (e != hipSuccess || p.full.idx == nullptr) return e;
    return launch_mode<kMaskFull>(p, stream);
  }
  return p.window >= 0 ? launch_mode<kMaskWindow>(p, stream) : launch_mode<kMaskNone>(p, stream);
}

void fwd_bf16_geometry(int d, int* rows_per_block, int* keys_per_tile, int* waves) {
  switch (d) {
    case 64: *keys_per_tile = FwdCfg<64>::BC; *waves = fwd_waves<64, kMaskPattern>(); break;
    case 128: *keys_per_tile = FwdCfg<128>::BC; *waves = fwd_waves<128, kMaskPattern>(); break;
    default: *keys_per_tile = FwdCfg<256>::BC; *waves = fwd_waves<256, kMaskPattern>(); break;
  }
  *rows_per_block = 32 * *waves;
}
#endif

}  // namespace exattn
