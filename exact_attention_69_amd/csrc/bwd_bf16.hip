// Backward attention kernels, bf16 inputs, fp32 accumulation, gfx950.
//
// The backward recomputes the probabilities from Q, K and the forward's
// per-row log-sum-exp instead of reading a stored n x n matrix (the unite.ai
// page "Flash Attention: Revolucionando a Eficiencia dos Modelos
// Transformer", section "Entenda a Flash Attention", item 2; llmis.ru
// chapter 3.1, section 5).  The gradient formulas are the chain rule of
// O = softmax(scale Q K^T) V for the loss sum(O * dO):
//   P = exp(scale*S - LSE), dV = P^T dO, dP = dO V^T, D = rowsum(dO * O),
//   dS = P * (dP - D), dK = scale dS^T Q, dQ = scale dS K.
//
// Three launches, all stream ordered and deterministic (no atomics):
//   1. rowdot: D for every query row (fp32 workspace).
//   2. key side (KV-outer): a workgroup owns 32*NW keys, keeps their K rows in
//      registers and V rows in LDS, and accumulates dK, dV over the query tiles in the
//      band; S and dP are computed with lanes indexed by key so that P and dS
//      feed the dV/dK products straight from the accumulator registers.
//   3. query side (Q-outer): a workgroup owns 32*NW query rows and
//      accumulates dQ over the key tiles, recomputing S and dP with lanes
//      indexed by query row.
//
// The d = 128 instantiations without a mask are compiled in a translation
// unit of their own (bwd_bf16_d128.hip includes this file with
// EXATTN_BWD_D128 defined), which the build gives a different instruction
// scheduler; this file's own unit holds the rest and the entry points.
#include "bwd_common.hpp"
#include "device_common.hpp"
#include "launch.hpp"
#include "pattern.hpp"

namespace exattn {
namespace {

// ---------------------------------------------------------------------------
// Key side: dK, dV
// ---------------------------------------------------------------------------
template <int D>
struct KvCfg {
  static constexpr int NW = D == 128 ? 8 : 4;  // waves; each owns 32 keys
  static constexpr int BQ = 32;  // query rows per tile
  static constexpr int WPE = D == 256 ? 1 : 2;  // waves per SIMD
};

// Waves per workgroup: the full-key pass gathers kFullRows keys; 4 under a
// pattern (as in the forward).
template <int D, int MODE>
constexpr int kv_waves() {
  return MODE == kMaskFull ? kFullRows / 32 : MODE == kMaskPattern ? 4 : KvCfg<D>::NW;
}

// This workgroup's item of a full-position launch: (head, chunk, group of
// positions), chunk-major within a head.  False for the spare workgroups of
// the launch, which return at once.
struct FullItem {
  int rows, groups, chunks, chunk, group, head;
};
__device__ __forceinline__ bool full_item(const FullDev& full, int heads, FullItem* f) {
  f->rows = full.info[kFullCount];
  f->groups = full.info[kFullGroups];
  f->chunks = full.info[kFullChunks];
  const int per_head = f->groups * f->chunks;
  const int item = blockIdx.x;
  if (item >= heads * per_head) return false;
  f->head = item / per_head;
  const int r = item - f->head * per_head;
  f->chunk = r / f->groups;
  f->group = r - f->chunk * f->groups;
  return true;
}

// MODE: kMaskNone, kMaskWindow (contiguous band of query tiles),
// kMaskPattern (the workgroup's tile list from the pattern plan; full keys
// are left to the full-key pass) or kMaskFull (a pattern's full keys,
// gathered, against one chunk of query tiles; with several chunks the
// partial dK, dV go to the partial buffer).
template <int D, int MODE>
__global__ __launch_bounds__((kv_waves<D, MODE>() * 64), KvCfg<D>::WPE) void bwd_kv_bf16_kernel(
    const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
    const __bf16* __restrict__ dOg, const float* __restrict__ LSE2g, const float* __restrict__ Dg,
    __bf16* __restrict__ dKg, __bf16* __restrict__ dVg, int n, int n_kblocks, int total_blocks, float scale,
    float scale_log2, int window, int group, PatternDev pat, FullDev full) {
  constexpr bool WINDOWED = MODE == kMaskWindow;
  constexpr bool PATTERN = MODE == kMaskPattern;
  constexpr bool FULL = MODE == kMaskFull;
  constexpr int NW = kv_waves<D, MODE>();
  constexpr int BQ = KvCfg<D>::BQ;
  constexpr int NT = NW * 64;
  constexpr int BKV = 32 * NW;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  static_assert(BQ == 32, "one 32-row query block per tile");

  __shared__ __attribute__((aligned(16))) __bf16 tiles[2][2][BQ * D];  // [buf][Q/dO]
  __shared__ __attribute__((aligned(16))) __bf16 vres[BKV * D];        // this block's V rows
  __shared__ __attribute__((aligned(16))) float rowst[2][2][BQ];       // [buf][LSE*log2(e) / D]
  poison_lds(tiles, vres, rowst);

  int kvh, kblk;  // key/value head (batch-major), key block
  FullItem f{};
  if constexpr (FULL) {
    if (!full_item(full, total_blocks / n_kblocks, &f)) return;  // whole workgroup: no barrier skipped
    kvh = f.head;
    kblk = 0;
  } else {
    const int bid = xcd_remap(blockIdx.x, total_blocks);
    kvh = bid / n_kblocks;
    kblk = bid - kvh * n_kblocks;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;

  // The group's query heads kvh*group .. kvh*group + group - 1 all attend to
  // these keys: their contributions to dK and dV are summed in registers.
  const size_t hoff = (size_t)kvh * n * D;
  const int qh0 = kvh * group;

  const int kb0 = kblk * BKV;
  // full keys: slot of the full-key list; slots past the list count as past n
  const int f_slot = f.group * BKV + wave * 32 + l32;
  const int my_key = FULL ? (f_slot < f.rows ? full.idx[f_slot] : n) : kb0 + wave * 32 + l32;

  // K row of this lane's key as an MFMA B operand (k along d), in registers;
  // the block's V rows (B operand of dP = dO V^T) stay resident in LDS.
  bf16x8 kreg[NDS];
  {
    const bool ok = my_key < n;
    const size_t off = hoff + (size_t)(ok ? my_key : 0) * D + 8 * hi;
    const u32x4* ks = (const u32x4*)(Kg + off);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) kreg[ds] = __builtin_bit_cast(bf16x8, ok ? ks[2 * ds] : u32x4{0, 0, 0, 0});
  }
  // V rows of this block, resident in LDS (visible after the first barrier);
  // key rows past n are clamped copies and only feed unstored dK/dV rows.
  if constexpr (FULL)
    TileAsyncRows<D, BKV, NT>::issue(Vg + hoff, full.idx + f.group * BKV, min(BKV, f.rows - f.group * BKV), vres,
                                     tid);
  else
    TileAsync<D, BKV, NT>::issue(Vg + hoff + (size_t)kb0 * D, n - kb0, vres, tid);

  int q_lo = 0, q_hi = n;
  if constexpr (WINDOWED) band_keys(kb0, kb0 + BKV, n, window, &q_lo, &q_hi);
  if constexpr (FULL) {
    const int tl = full.info[kFullTilesPerChunk];
    q_lo = f.chunk * tl * BQ;
    q_hi = min(n, q_lo + tl * BQ);
  }
  const int t_lo = q_lo / BQ, t_hi = (q_hi + BQ - 1) / BQ;
  // query tiles visited: a contiguous range, or under a pattern the tiles of
  // gathered full rows (they see every key) followed by the plan's list;
  // iteration index i < n_gath is gathered tile i.
  const int* plist = PATTERN ? pat.list + (size_t)kblk * pat.stride : nullptr;
  const int n_full_rows = PATTERN ? pat.other_count[0] : 0;
  const int n_gath = (n_full_rows + BQ - 1) / BQ;
  const int n_listed = PATTERN ? pat.count[kblk] : 0;
  const int n_tiles = PATTERN ? (n_listed < 0 ? 0 : n_gath + n_listed) : t_hi - t_lo;
  auto tile_at = [&](int i) { return PATTERN ? plist[i - n_gath] >> kEntryTileShift : t_lo + i; };
  // query rows that see this lane's key through the band (the window is
  // symmetric), within n
  int row_lo = 0, row_hi = n;
  if constexpr (WINDOWED) band_keys(my_key, my_key + 1, n, window, &row_lo, &row_hi);
  if constexpr (PATTERN) {
    if (pat.window >= 0)
      band_keys(my_key, my_key + 1, n, pat.window, &row_lo, &row_hi);
    else
      row_hi = row_lo;
  }
  const unsigned row_span = (unsigned)max(row_hi - row_lo, 0);
  // Under a pattern a wave skips the work of a partial listed tile where none
  // of its keys is seen (the layout misses the wave and the band misses its
  // keys), and of every tile when its keys are all full keys or past n; loads
  // and barriers stay shared.
  const int kw0 = kb0 + wave * 32;  // first key of this wave
  const bool wave_live = !PATTERN || (kw0 < n && pat.own_full[kw0 >> 5] != ~0u);

  // Q and dO tiles, and the LSE*log2(e) and D values of their rows, go
  // straight from global memory to LDS.  Rows past n (past the count of a
  // gathered tile) are clamped copies of the last row with LSE = +inf, so
  // their probabilities (and dS) are exactly zero without a per-element test.
  using Tile = TileAsync<D, BQ, NT>;
  using Dma = TileDma<D, BQ, NT>;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t dma_off[Dma::IT];  // this thread's chunk offsets in a full Q or dO tile
  Dma::init(tid, dma_off);
  static_assert(BQ == 32, "the row-statistics copy maps 64 lanes to 2 x 32 rows");
  auto load_tile = [&](int i, int qg, int buf) {
    if constexpr (PATTERN) {
      // gathered tiles read the full rows' copies, laid out like the rows of
      // a head; `valid` rows of the tile exist
      const bool g = i < n_gath;
      const int i0 = g ? i * BQ : tile_at(i) * BQ;
      const int valid = (g ? n_full_rows : n) - i0;
      const int qrow = (qh0 + qg) * n + i0;
      Tile::issue((g ? pat.gath_a : Qg) + (size_t)qrow * D, valid, tiles[buf][0], tid);
      Tile::issue((g ? pat.gath_b : dOg) + (size_t)qrow * D, valid, tiles[buf][1], tid);
      if (wave == 0) {  // lanes 0-31: LSE*log2(e) of the tile's rows, lanes 32-63: D
        const int r = qrow + min(l32, valid - 1);
        const float* ls = g ? pat.gath_s0 : LSE2g;
        const float* dd = g ? pat.gath_s1 : Dg;
        const void* src = hi ? (const void*)(dd + r) : l32 < valid ? (const void*)(ls + r) : (const void*)&kPosInf;
        lds_dma4(src, &rowst[buf][0][0]);
      }
    } else {
      const int i0 = tile_at(i) * BQ;
      // first row of the tile in [B*H*n]; B*H*n*D < 2^31 is checked at the ABI
      const int qrow = (qh0 + qg) * n + i0;
      if (i0 + BQ <= n) {
        Dma::issue(Qg + (size_t)qrow * D, dma_off, tiles[buf][0], wave_s);
        Dma::issue(dOg + (size_t)qrow * D, dma_off, tiles[buf][1], wave_s);
      } else {
        Dma::issue_tail(Qg + (size_t)qrow * D, n - i0, tiles[buf][0], tid, wave_s);
        Dma::issue_tail(dOg + (size_t)qrow * D, n - i0, tiles[buf][1], tid, wave_s);
      }
      if (wave == 0) {  // lanes 0-31: LSE*log2(e) of rows i0.., lanes 32-63: D
        const int r = qrow + min(l32, n - 1 - i0);
        const void* src = hi ? (const void*)(Dg + r) : i0 + l32 < n ? (const void*)(LSE2g + r) : (const void*)&kPosInf;
        lds_dma4(src, &rowst[buf][0][0]);
      }
    }
  };

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  // One sweep over the band's query tiles per query head of the group.
  const int steps = n_tiles * group;
  if (steps > 0) load_tile(0, 0, 0);
  wait_all_and_barrier();

  int step = 0;
  for (int qg = 0; qg < group; ++qg)
  for (int it = 0; it < n_tiles; ++it, ++step) {
    const bool gathered = PATTERN && it < n_gath;
    const int t = gathered ? 0 : tile_at(it);
    const int buf = step & 1;
    // prefetch the next tile (the next head's first tile after the last one);
    // its buffer was released by the last barrier
    if (it + 1 < n_tiles)
      load_tile(it + 1, qg, buf ^ 1);
    else if (qg + 1 < group)
      load_tile(0, qg + 1, buf ^ 1);
    const __bf16* Qs = tiles[buf][0];
    const __bf16* dOs = tiles[buf][1];
    const int i0 = t * BQ;

    bool act = true;
    // A wave skips the query tiles its 32 keys' band misses (they add
    // nothing): 5% faster at d=128 with window 512, 3% at d=64; at d=256 (one
    // wave per SIMD) the branch costs 4-10%, so there every tile runs.
    if constexpr (WINDOWED && D != 256) act = i0 <= kw0 + 31 + window && kw0 <= i0 + BQ - 1 + window;
    if constexpr (PATTERN) {
      act = wave_live;
      if (act && !gathered) {
        const int entry = plist[it - n_gath];
        if (entry & 1) {
          const bool lay = (entry >> (1 + wave)) & 1;
          act = lay || (pat.window >= 0 && i0 <= kw0 + 31 + pat.window && kw0 <= i0 + BQ - 1 + pat.window);
        }
      }
    }
    if (act) {
      // S = Q K^T and dP = dO V^T, lanes indexed by key, registers by query
      // row.  The dP accumulator starts at -D of its rows (the workspace holds
      // -D; register r of a lane is row 8*(r/4) + 4*hi + r%4 of the tile), so
      // the product ends as dP - D.
      f32x16 s = f32x16{}, dp;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 nd4 = *(const f32x4*)(&rowst[buf][1][8 * g + 4 * hi]);
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[4 * g + j] = nd4[j];
      }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        s = mfma32(lds_row_frag<D>(Qs, l32, ds, hi), kreg[ds], s);
        dp = mfma32(lds_row_frag<D>(dOs, l32, ds, hi), lds_row_frag<D>(vres, wave * 32 + l32, ds, hi), dp);
      }
      // At d=256 (one wave per SIMD, nothing else to hide the latency) the
      // row reads of Q, dO and V are issued two steps ahead of their
      // products: 7% faster there, slower at d=128.
      if constexpr (D == 256) {
        constexpr int kLead = 2;
        EXATTN_SCHED(kSchedDSRead, 3 * kLead);
#pragma unroll
        for (int i = 0; i < NDS; ++i) {
          EXATTN_SCHED(kSchedMFMA, 2);
          if (i + kLead < NDS) EXATTN_SCHED(kSchedDSRead, 3);
        }
      }

      // The waves of a SIMD reach this vector phase together; the one in it
      // gets priority, so the other's matrix products fill its gaps (1.3%
      // faster at n=8192, d=128; the same in the dQ pass was 2.5% slower).
      __builtin_amdgcn_s_setprio(1);
      // With a window, queries outside this lane's key band get P = 0 (rows
      // past n already have P = 0 through their LSE, and so do the empty
      // slots of a gathered tile).  Under a pattern, a partial listed tile
      // keeps the pairs that the band or the layout make visible, except
      // those of full rows (they come from the gathered tiles).
      bool need_mask = false;
      if constexpr (WINDOWED) {
        const int k_lo_w = kb0 + wave * 32;
        need_mask = max(i0 + BQ - 1 - k_lo_w, k_lo_w + 31 - i0) > window;
      }
      uint32_t lay = 0;  // the layout covers the wave for the tile
      uint32_t fr = 0;   // full-row bits of the tile's rows, shifted to this lane's half
      if constexpr (PATTERN) {
        if (!gathered) {
          const int entry = plist[it - n_gath];
          lay = (entry >> (1 + wave)) & 1;
          need_mask = (entry & 1) && !(lay && !(entry & kEntryHasFull));  // covered by the layout, no full row
          if (need_mask) fr = pat.other_full[t] >> (4 * hi);  // BQ = 32: one bitmap word per tile
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rb = 8 * g + 4 * hi;  // rows rb .. rb+3 of the tile
        const f32x4 l4 = *(const f32x4*)(&rowst[buf][0][rb]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -l4[j]));
          // queries that see this lane's key: [row_lo, row_lo + row_span)
          if (WINDOWED && need_mask) p = (unsigned)(i0 + rb + j - row_lo) < row_span ? p : 0.0f;
          if (PATTERN && need_mask) {  // bitwise: one select, no short-circuit branches
            const uint32_t vis = ((uint32_t)((unsigned)(i0 + rb + j - row_lo) < row_span) | lay) &
                                 ~(fr >> (8 * g + j));
            p = (vis & 1u) ? p : 0.0f;
          }
          s[r] = p;
          dp[r] = p * dp[r];  // dS = P (dP - D) (unscaled)
        }
      }

      __builtin_amdgcn_s_setprio(0);
      // dV^T += dO^T P and dK^T += Q^T dS, k along the tile's query rows.
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 pb = acc_to_operand(s, half);
        const bf16x8 sb = acc_to_operand(dp, half);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dv[db] = mfma32(lds_col_frag<D>(dOs, 16 * half, 32 * db, lane), pb, dv[db]);
          dk[db] = mfma32(lds_col_frag<D>(Qs, 16 * half, 32 * db, lane), sb, dk[db]);
        }
      }

      // Issue each product's two transposed LDS reads kLead products ahead
      // of it; left to itself the compiler waits on every read right before
      // its product.  (1.7% faster at d=128, 15% at d=256; at d=64, where
      // three workgroups share a CU, 3% slower, so not there.)
      if constexpr (D >= 128) {
        constexpr int NP = 2 * 2 * NDB, kLead = 2;
        EXATTN_SCHED(kSchedDSRead, 2 * kLead);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          EXATTN_SCHED(kSchedMFMA, 1);
          if (i + kLead < NP) EXATTN_SCHED(kSchedDSRead, 2);
        }
      }

    }

    wait_all_and_barrier();
  }

  bool store = my_key < n;
  if constexpr (PATTERN) store = store && !bit_of(pat.own_full, my_key);
  if (FULL && store && f.chunks > 1) {
    float* prow = full.part + ((size_t)(kvh * f.chunks + f.chunk) * f.groups * BKV + f_slot) * (2 * D);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hi;
        *(f32x4*)(prow + dd) = f32x4{dk[db][4 * g] * scale, dk[db][4 * g + 1] * scale, dk[db][4 * g + 2] * scale,
                                     dk[db][4 * g + 3] * scale};
        *(f32x4*)(prow + D + dd) = f32x4{dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
      }
  } else if (store) {
    __bf16* dkr = dKg + hoff + (size_t)my_key * D;
    __bf16* dvr = dVg + hoff + (size_t)my_key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hi;
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dk[db][4 * g] * scale, dk[db][4 * g + 1] * scale);
        wk[1] = pack_bf16x2(dk[db][4 * g + 2] * scale, dk[db][4 * g + 3] * scale);
        wv[0] = pack_bf16x2(dv[db][4 * g], dv[db][4 * g + 1]);
        wv[1] = pack_bf16x2(dv[db][4 * g + 2], dv[db][4 * g + 3]);
        *(u32x2*)(dkr + dd) = wk;
        *(u32x2*)(dvr + dd) = wv;
      }
  }
}

// Scheduling of a phase of NF fragment loads, each feeding MPF matrix
// products (one per key block of a pair): the loads (RPF LDS reads per
// fragment) are issued kLead fragments ahead of their products.
template <int NF, int RPF, int kLead = 2, int MPF = 2>
__device__ __forceinline__ void pair_sched_products() {
  EXATTN_SCHED(kSchedDSRead, RPF * kLead);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    EXATTN_SCHED(kSchedMFMA, MPF);
    if (f + kLead < NF) EXATTN_SCHED(kSchedDSRead, RPF);
  }
}

// ---------------------------------------------------------------------------
// Key side without a pattern, d = 128 and 256: paired waves.
// ---------------------------------------------------------------------------
// The 8 waves form 4 pairs (wave w and wave w+4, which share a SIMD); a pair
// owns 32 * NKB keys (NKB = 2 key blocks of 32 at d = 128, one at d = 256).
// The P-wave of a pair keeps their K rows in registers, forms S = Q K^T and
// P = exp(S - LSE) for a query tile, passes P (bf16) to its partner through
// LDS and accumulates dV += P^T dO.  The dS-wave accumulates dK += dS^T Q
// with dS = P (dP - D).  At d = 128 each LDS fragment of Q or dO feeds the
// products of both key blocks.  The two waves of a SIMD are kept in opposite
// phases: in iteration i the P-wave forms S(i) (matrix cores), then P(i)
// (vector ALU), then dV; the dS-wave first forms dS(i-1) from the dP(i-1) it
// carries over in registers and the P(i-1) its partner left in LDS (vector
// ALU), then dK with it and dP(i) for the next iteration (matrix cores), so
// each wave's vector work runs beside the other's products.
// The P-wave keeps the K rows of its keys in registers; the dS-wave keeps the
// V rows of its first key block in registers and, at d = 128, those of the
// second in LDS, which leaves registers for the dP it carries over.  At
// d = 256 this splits the 512 accumulator registers a single wave would need
// for 32 keys (dK and dV, 2 x 256 columns) over the two waves, so two waves
// per SIMD fit where one did.  At d = 256 the dS-wave's instructions win the
// SIMD's issue arbitration throughout: its chain of short phases is the one
// that stalls on LDS reads.  At d = 128 the waves also meet at a second
// barrier once the P-wave has issued S(i), and the priority follows the
// products: the P-wave's while it forms S, the dS-wave's from that barrier
// on.  Left alone, the dS-wave's dK products took the matrix cores while S
// was still waiting for them, and the P-wave's exponentials started late
// (phase timestamps per wave); with the barrier the pass is 1.5% faster there
// (at d = 256 it was 9% slower).  Also at d = 128, the LDS reads run four
// fragments ahead of their products and the P-wave issues its share of the
// next tile's copies after S (see kPairLead and load_tile's call sites).
// Buffers: three Q/dO tiles (tiles i-1 and i are read while i+1 is in
// flight) and two P tiles.  LDS read addresses are per-lane bases (the tile
// buffer's offset added once per iteration) XOR a constant, plus a constant
// offset: four base registers instead of one per fragment, because every
// register is taken.
template <int D>
struct PairKv {
  static constexpr int NKB = D == 128 ? 2 : 1;  // 32-key blocks per pair
  static constexpr int BQ = 32, NBUF = 3, NT = 512;
  static constexpr int BKV = 4 * 32 * NKB;      // keys per workgroup
  static constexpr int RS = 2 * D;              // bytes per tile row
  // LDS layout (bytes)
  static constexpr int kTileBytes = BQ * RS;                       // one Q or dO tile
  static constexpr int kTiles = 0;                                 // [buf][Q, dO]
  static constexpr int kVres = kTiles + NBUF * 2 * kTileBytes;     // [pair]: V rows of key block 1 (d = 128)
  static constexpr int kVresBytes = NKB == 2 ? 4 * 32 * RS : 0;
  static constexpr int kPbufPair = 2 * NKB * 64 * 16;              // one pair's P tile
  static constexpr int kPbuf = kVres + kVresBytes;                 // [buf][pair][block, half][lane] x 16 bytes
  static constexpr int kRowst = kPbuf + 2 * 4 * kPbufPair;         // [buf][LSE*log2(e) / -D][32] floats
  static constexpr int kBytes = kRowst + NBUF * 2 * BQ * 4;
  static_assert(kBytes <= 160 * 1024, "one workgroup per CU");
};

// The key side runs on the paired kernel at d = 256 without a pattern (all
// keys, or a window's band) and at d = 128 over all keys.  (At d = 128 the
// band's per-key row limits do not fit the paired waves' registers: the
// single-wave kernel is faster there.)
template <int D, int MODE>
constexpr bool pair_kv_dispatch() {
  return (D == 256 && (MODE == kMaskNone || MODE == kMaskWindow)) || (D == 128 && MODE == kMaskNone);
}

template <int D, int MODE>
__global__ __launch_bounds__(512, 2) void bwd_kv_pair_kernel(
    const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
    const __bf16* __restrict__ dOg, const float* __restrict__ LSE2g, const float* __restrict__ Dg,
    __bf16* __restrict__ dKg, __bf16* __restrict__ dVg, int n, int n_kblocks, int total_blocks, float scale,
    float scale_log2, int window, int group) {
  using C = PairKv<D>;
  constexpr bool WINDOWED = MODE == kMaskWindow;
  constexpr int NKB = C::NKB, BQ = C::BQ, NBUF = C::NBUF, NT = C::NT, BKV = C::BKV, RS = C::RS;
  constexpr int NDS = D / 16, NDB = D / 32;
  constexpr int kTileBytes = C::kTileBytes, kTiles = C::kTiles, kRowst = C::kRowst;
  __shared__ __attribute__((aligned(16))) char lds[C::kBytes];
  poison_lds(lds);

  const int bid = xcd_remap(blockIdx.x, total_blocks);
  const int kvh = bid / n_kblocks;
  const int kblk = bid - kvh * n_kblocks;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const bool pwave = wave < 4;  // P / dV wave, else dP / dS / dK wave

  const size_t hoff = (size_t)kvh * n * D;
  const int qh0 = kvh * group;
  const int kb0 = kblk * BKV;
  const int kp0 = kb0 + pair * 32 * NKB;  // first key of the pair
  int my_key[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) my_key[kb] = kp0 + 32 * kb + l32;

  int q_lo = 0, q_hi = n;
  if constexpr (WINDOWED) band_keys(kb0, kb0 + BKV, n, window, &q_lo, &q_hi);
  const int t_lo = q_lo / BQ, t_hi = (q_hi + BQ - 1) / BQ;
  const int n_tiles = t_hi - t_lo;
  const int steps = n_tiles * group;

  // Per-lane LDS byte offsets (the tile and buffer parts are constants).
  // Row fragment ds of a swizzled [rows][D] tile, row l32 (k along d):
  //   l32*RS + 16*((2 ds + hi) ^ sw(l32)).
  // Column fragment (k along rows) of query rows 16*half.., columns
  // 32*db..: two 8-byte transpose reads at rows 16 half + 4 hi + q + 8 s
  // (q = (lane%16)/4, s = 0, 1); their offsets are
  //   16 RS half + 8 RS s + (C_s ^ 64 db),
  //   C_s = (4 hi + q)*RS + 64 q + 16*((2 (g&1) + (L/2)%2) ^ hi ^ 2 s) + 8 (L%2)
  // with g = lane/16, L = lane%16 (the swizzle value of those rows is
  // 4 q + (hi ^ 2 s), so the XOR with the chunk index splits by bit fields).
  // Both are a per-lane base XOR a constant: the row base keeps sw(l32)/2 in
  // bits 5-7, which the XOR with 32 ds turns into the swizzled chunk, and
  // C_s keeps q in bits 6-7.  Only the bases stay live across the loop (an
  // XOR per fragment recomputes each offset where it is used).
  const int row_base = l32 * RS + 16 * ((hi ^ swz_chunk<D>(l32, 0)) & 1) + 32 * (swz_chunk<D>(l32, 0) >> 1);
  int col_base[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int g = lane >> 4, L = lane & 15, q = L >> 2;
    col_base[s] = (4 * hi + q) * RS + 64 * q + 16 * (((2 * (g & 1)) + ((L >> 1) & 1)) ^ hi ^ (2 * s)) + 8 * (L & 1);
  }
  auto ld_row = [&](int base, int off) { return *(const bf16x8*)(lds + base + off); };
  auto ld_col = [&](int base, int s0_off, int s1_off) {
    const bf16x4 a = lds_read_tr16((const __bf16*)(lds + base + s0_off));
    const bf16x4 b = lds_read_tr16((const __bf16*)(lds + base + 8 * RS + s1_off));
    return cat8(a, b);
  };

  // step s: query head qh0 + s / n_tiles, tile t_lo + s % n_tiles
  using Dma = TileDma<D, BQ, NT>;
  auto load_tile = [&](int s, int buf) {
    const int qg = s / n_tiles;
    const int i0 = (t_lo + (s - qg * n_tiles)) * BQ;
    // first row of the tile in [B*H*n] (< 2^31, checked at the ABI)
    const int qrow = (qh0 + qg) * n + i0;
    // TileDma's placement; rows past n are clamped copies (their LSE is
    // +inf: P = 0)
    __bf16* qd = (__bf16*)(lds + kTiles + (2 * buf) * kTileBytes);
    __bf16* gd = (__bf16*)(lds + kTiles + (2 * buf + 1) * kTileBytes);
    if (i0 + BQ <= n) {
      // (the chunk offsets are recomputed from a fresh lane index: no
      // register holds them across the loop)
      const int t = wave * 64 + fresh_lane_id();
      uint32_t off[Dma::IT];
#pragma unroll
      for (int it = 0; it < Dma::IT; ++it) off[it] = Dma::chunk_off(it, t, (it * NT + t) / (D / 8));
      Dma::issue(Qg + (size_t)qrow * D, off, qd, wave);
      Dma::issue(dOg + (size_t)qrow * D, off, gd, wave);
    } else {
      Dma::issue_tail(Qg + (size_t)qrow * D, n - i0, qd, tid, wave);
      Dma::issue_tail(dOg + (size_t)qrow * D, n - i0, gd, tid, wave);
    }
    if (wave == 0) {  // lanes 0-31: LSE*log2(e) of rows i0.., lanes 32-63: -D
      const int ln = fresh_lane_id(), r32 = ln & 31;
      const int r = qrow + min(r32, n - 1 - i0);
      const float* lse_src = i0 + r32 < n ? LSE2g + r : &kPosInf;
      lds_dma4(ln >= 32 ? Dg + r : lse_src, lds + kRowst + buf * 2 * BQ * 4);
    }
  };
  auto tile_row0 = [&](int s) { return (t_lo + s % n_tiles) * BQ; };
  // a pair skips the query tiles its keys' band misses
  auto pair_sees = [&](int s) -> bool {
    if constexpr (WINDOWED) {
      const int i0 = tile_row0(s);
      return i0 <= kp0 + 32 * NKB - 1 + window && kp0 <= i0 + BQ - 1 + window;
    } else {
      return true;
    }
  };
  // End of an iteration: the next tile's copies and this wave's LDS writes
  // complete, then the workgroup synchronises.
  auto end_iteration = [&]() { wait_all_and_barrier(); };
  // At d = 128: the barrier after the P-wave's S products (no memory is
  // handed over through it).
  constexpr bool kMidSync = D == 128;
  // LDS reads issued this many fragments ahead of their products (at d = 128
  // 4 rather than 2: 3% faster at n = 8192, 5% at n = 1000; 3, 6 and 8 were
  // slower than 4)
  constexpr int kPairLead = D == 128 ? 4 : 2;
  auto mid_sync = [&]() {
    if constexpr (kMidSync) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16 acc[NKB][NDB];  // dV (P-wave) or dK (dS-wave): [key block][d block], transposed
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[kb][db] = f32x16{};

  // Rows of K or V as MFMA B operands with k along d (lane l: key l % 32 of
  // the block); keys past n read zeros (their rows are not stored)
  auto load_rows = [&](const __bf16* src, int key, bf16x8 (&r)[NDS]) {
    const bool ok = key < n;
    const u32x4* p = (const u32x4*)(src + hoff + (size_t)(ok ? key : 0) * D + 8 * hi);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) r[ds] = __builtin_bit_cast(bf16x8, ok ? p[2 * ds] : u32x4{0, 0, 0, 0});
  };
  // At d = 128 the dS-wave's V rows of the second key block stay in LDS,
  // swizzled like the tiles and read as fragments each tile.
  const int res = C::kVres + pair * 32 * RS;  // wave-uniform
  if constexpr (NKB == 2) {
    if (!pwave) {
#pragma unroll
      for (int it = 0; it < 32 * (D / 8) / 64; ++it) {
        const int slot = it * 64 + lane, row = slot / (D / 8);
        const int key = min(kp0 + 32 + row, n - 1);  // rows past n: clamped copies, not stored
        lds_dma16(Vg + hoff + (size_t)key * D + 8 * swz_chunk<D>(row, slot % (D / 8)), lds + res + 16 * (it * 64));
      }
    }
  }
  const int res_base = row_base + res;  // (res_base ^ 32 ds) = res + (row_base ^ 32 ds)

  if (steps > 0) load_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  if (pwave) {
    bf16x8 kr[NKB][NDS];  // K rows of the pair's key blocks
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) load_rows(Kg, my_key[kb], kr[kb]);
    const int pw_off = C::kPbuf + pair * C::kPbufPair + 16 * lane;  // + buffer and chunk constants
    const int ls_off = kRowst + 16 * hi;                           // + buffer and row-group constants
    // query rows that see each of this lane's keys through the band
    int row_lo[NKB];
    unsigned row_span[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      row_lo[kb] = 0;
      row_span[kb] = 0u;
      if constexpr (WINDOWED) {
        int lo, hi_r;
        band_keys(my_key[kb], my_key[kb] + 1, n, window, &lo, &hi_r);
        row_lo[kb] = lo;
        row_span[kb] = (unsigned)max(hi_r - lo, 0);
      }
    }
    for (int i = 0; i < steps; ++i) {
      const int b = i % NBUF, bn = b == NBUF - 1 ? 0 : b + 1;
      // (at d = 128 the P-wave's share of the next tile's copies waits until
      // S is issued: 1% faster)
      if (!kMidSync && i + 1 < steps) load_tile(i + 1, bn);
      const bool sees = pair_sees(i);
      // tile buffer b: Q rows at qt, dO at qt + kTileBytes (bits 13 and up,
      // clear of the XOR fields)
      const int qt = kTiles + (2 * b) * kTileBytes;
      const int rq = opaque_lane_value(row_base) + qt;
      const int cg0 = opaque_lane_value(col_base[0]) + qt + kTileBytes;
      const int cg1 = opaque_lane_value(col_base[1]) + qt + kTileBytes;
      const int i0 = tile_row0(i);
      // S = Q K^T, lanes indexed by key, registers by query row; each Q
      // fragment feeds every key block
      f32x16 s[NKB];
      if (sees) {
        if constexpr (kMidSync) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const bf16x8 qf = ld_row(0, rq ^ (32 * ds));
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32(qf, kr[kb][ds], s[kb]);
        }
        pair_sched_products<NDS, 1, kPairLead, NKB>();
        __builtin_amdgcn_sched_barrier(0);
      }
      mid_sync();
      if constexpr (kMidSync) __builtin_amdgcn_s_setprio(0);
      if (kMidSync && i + 1 < steps) load_tile(i + 1, bn);
      if (sees) {
        bool need_mask = false;
        if constexpr (WINDOWED) need_mask = max(i0 + BQ - 1 - kp0, kp0 + 32 * NKB - 1 - i0) > window;
        bf16x8 pb[NKB][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            // LSE*log2(e) of rows 8g + 4hi .. +3
            const f32x4 l4 = *(const f32x4*)(lds + ls_off + b * (2 * BQ * 4) + 32 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 4 * g + j;
              float p = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -l4[j]));
              if (WINDOWED && need_mask)
                p = (unsigned)(i0 + 8 * g + 4 * hi + j - row_lo[kb]) < row_span[kb] ? p : 0.0f;
              s[kb][r] = p;
            }
          }
          pb[kb][0] = acc_to_operand(s[kb], 0);
          pb[kb][1] = acc_to_operand(s[kb], 1);
        }
        // P to the partner wave: lane-private 16 bytes per block and half,
        // laid out so that consecutive lanes write consecutive 16-byte slots
#pragma unroll
        for (int c = 0; c < 2 * NKB; ++c)
          *(u32x4*)(lds + pw_off + (i & 1) * (4 * C::kPbufPair) + c * 1024) =
              __builtin_bit_cast(u32x4, pb[c >> 1][c & 1]);
        __builtin_amdgcn_sched_barrier(0);
        // dV^T += dO^T P, k along the tile's query rows; each transposed dO
        // fragment feeds every key block
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 a = ld_col(16 * RS * half, cg0 ^ (64 * db), cg1 ^ (64 * db));
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) acc[kb][db] = mfma32(a, pb[kb][half], acc[kb][db]);
          }
        pair_sched_products<2 * NDB, 2, kPairLead, NKB>();
      }
      end_iteration();
    }
    // the dS-wave's last iteration
    mid_sync();
    end_iteration();
  } else {
    bf16x8 v0[NDS];  // V rows of the first key block
    load_rows(Vg, my_key[0], v0);
    const int pw_off = C::kPbuf + pair * C::kPbufPair + 16 * lane;
    const int ls_off = kRowst + BQ * 4 + 16 * hi;  // the -D row of a buffer
    f32x16 dp[NKB];  // dP - D of the previous iteration's tile
    if constexpr (!kMidSync) __builtin_amdgcn_s_setprio(1);
    for (int i = 0; i <= steps; ++i) {
      if constexpr (kMidSync) __builtin_amdgcn_s_setprio(0);
      const int b = i % NBUF, bn = b == NBUF - 1 ? 0 : b + 1, bp = b == 0 ? NBUF - 1 : b - 1;
      if (i + 1 < steps) load_tile(i + 1, bn);
      // dS(i-1) = P (dP - D), with the partner's P of that tile (bf16), then
      // dK^T += Q^T dS, k along the tile's query rows
      const bool ds_prev = i >= 1 && pair_sees(i - 1);
      const int qt = kTiles + (2 * bp) * kTileBytes;
      const int cq0 = opaque_lane_value(col_base[0]) + qt, cq1 = opaque_lane_value(col_base[1]) + qt;
      bf16x8 sb[NKB][2];
      if (ds_prev) {
#pragma unroll
        for (int c = 0; c < 2 * NKB; ++c) {
          const int kb = c >> 1, half = c & 1;
          const u32x4 pw = *(const u32x4*)(lds + pw_off + ((i - 1) & 1) * (4 * C::kPbufPair) + c * 1024);
          u32x4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float p0 = __builtin_bit_cast(float, pw[t] << 16);
            const float p1 = __builtin_bit_cast(float, pw[t] & 0xffff0000u);
            w[t] = pack_bf16x2(p0 * dp[kb][8 * half + 2 * t], p1 * dp[kb][8 * half + 2 * t + 1]);
          }
          sb[kb][half] = __builtin_bit_cast(bf16x8, w);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      mid_sync();
      if constexpr (kMidSync) __builtin_amdgcn_s_setprio(1);
      if (ds_prev) {
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 a = ld_col(16 * RS * half, cq0 ^ (64 * db), cq1 ^ (64 * db));
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) acc[kb][db] = mfma32(a, sb[kb][half], acc[kb][db]);
          }
        pair_sched_products<2 * NDB, 2, kPairLead, NKB>();
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i < steps && pair_sees(i)) {
        // dP(i) = dO V^T, accumulators starting at -D of their rows
        // (register r of a lane is row 8*(r/4) + 4*hi + r%4 of the tile), so
        // the product ends as dP - D
        const int rg = opaque_lane_value(row_base) + kTiles + (2 * b + 1) * kTileBytes;
        const int vbase = opaque_lane_value(res_base);
        f32x16 nd;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 nd4 = *(const f32x4*)(lds + ls_off + b * (2 * BQ * 4) + 32 * g);
#pragma unroll
          for (int j = 0; j < 4; ++j) nd[4 * g + j] = nd4[j];
        }
        {
          const bf16x8 gf = ld_row(0, rg);
          dp[0] = mfma32(gf, v0[0], nd);
          if constexpr (NKB == 2) dp[1] = mfma32(gf, ld_row(0, vbase), nd);
        }
#pragma unroll
        for (int ds = 1; ds < NDS; ++ds) {
          const bf16x8 gf = ld_row(0, rg ^ (32 * ds));
          dp[0] = mfma32(gf, v0[ds], dp[0]);
          if constexpr (NKB == 2) dp[1] = mfma32(gf, ld_row(0, vbase ^ (32 * ds)), dp[1]);
        }
        pair_sched_products<NDS, NKB, kPairLead, NKB>();
      }
      end_iteration();
    }
  }

  // dV rows (P-wave) or dK rows, scaled (dS-wave), of this lane's keys
  const float f = pwave ? 1.0f : scale;
  __bf16* dst = pwave ? dVg : dKg;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    if (my_key[kb] >= n) continue;
    __bf16* row = dst + hoff + (size_t)my_key[kb] * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hi;
        u32x2 w;
        w[0] = pack_bf16x2(acc[kb][db][4 * g] * f, acc[kb][db][4 * g + 1] * f);
        w[1] = pack_bf16x2(acc[kb][db][4 * g + 2] * f, acc[kb][db][4 * g + 3] * f);
        *(u32x2*)(row + dd) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// Query side: dQ
// ---------------------------------------------------------------------------
template <int D>
struct QCfg;
template <>
struct QCfg<64> {
  static constexpr int NW = 8, BC = 64, WPE = 2;
};
template <>
struct QCfg<128> {
  static constexpr int NW = 8, BC = 32, WPE = 2;
};
template <>
struct QCfg<256> {
  static constexpr int NW = 4, BC = 32, WPE = 1;
};

template <int D, int MODE>
constexpr int q_waves() {
  return MODE == kMaskFull ? kFullRows / 32 : MODE == kMaskPattern ? 4 : QCfg<D>::NW;
}

// MODE as for the key side, with query rows owned: kMaskFull gathers a
// pattern's full rows against one chunk of key tiles.
template <int D, int MODE>
__global__ __launch_bounds__((q_waves<D, MODE>() * 64), QCfg<D>::WPE) void bwd_q_bf16_kernel(
    const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
    const __bf16* __restrict__ dOg, const float* __restrict__ LSE2g, const float* __restrict__ Dg,
    __bf16* __restrict__ dQg, int n, int n_qblocks, int total_blocks, float scale, float scale_log2, int window,
    int group, PatternDev pat, FullDev full) {
  constexpr bool WINDOWED = MODE == kMaskWindow;
  constexpr bool PATTERN = MODE == kMaskPattern;
  constexpr bool FULL = MODE == kMaskFull;
  constexpr int NW = q_waves<D, MODE>();
  constexpr int BC = QCfg<D>::BC;
  constexpr int NT = NW * 64;
  constexpr int BR = 32 * NW;
  constexpr int NKB = BC / 32;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;

  __shared__ __attribute__((aligned(16))) __bf16 tiles[2][2][BC * D];  // [buf][K/V]
  poison_lds(tiles);

  int head, qb;
  FullItem f{};
  if constexpr (FULL) {
    if (!full_item(full, total_blocks / n_qblocks, &f)) return;  // whole workgroup: no barrier skipped
    head = f.head;
    qb = 0;
  } else {
    const int bid = xcd_remap(blockIdx.x, total_blocks);
    head = bid / n_qblocks;
    qb = bid - head * n_qblocks;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;

  const size_t hoff = (size_t)head * n * D;
  const size_t kv_off = (size_t)(head / group) * n * D;  // key/value head of this query head
  const __bf16* K = Kg + kv_off;
  const __bf16* V = Vg + kv_off;
  const int q0 = qb * BR;
  // full rows: slot of the full-row list; slots past the list count as past n
  const int f_slot = f.group * BR + wave * 32 + l32;
  const int my_row = FULL ? (f_slot < f.rows ? full.idx[f_slot] : n) : q0 + wave * 32 + l32;

  bf16x8 qreg[NDS], greg[NDS];
  float lse2, ndl;  // LSE*log2(e) and -D of this lane's row
  {
    const bool ok = my_row < n;
    const size_t off = hoff + (size_t)(ok ? my_row : 0) * D + 8 * hi;
    const u32x4* qs = (const u32x4*)(Qg + off);
    const u32x4* gs = (const u32x4*)(dOg + off);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      qreg[ds] = __builtin_bit_cast(bf16x8, ok ? qs[2 * ds] : u32x4{0, 0, 0, 0});
      greg[ds] = __builtin_bit_cast(bf16x8, ok ? gs[2 * ds] : u32x4{0, 0, 0, 0});
    }
    lse2 = ok ? LSE2g[(size_t)head * n + my_row] : __builtin_huge_valf();
    ndl = ok ? Dg[(size_t)head * n + my_row] : 0.0f;
  }

  int k_lo = 0, k_hi = n;
  if constexpr (WINDOWED) band_keys(q0, q0 + BR, n, window, &k_lo, &k_hi);
  if constexpr (FULL) {
    const int tl = full.info[kFullTilesPerChunk];
    k_lo = f.chunk * tl * BC;
    k_hi = min(n, k_lo + tl * BC);
  }
  const int t_lo = k_lo / BC, t_hi = (k_hi + BC - 1) / BC;
  // key tiles visited: a contiguous range, or under a pattern the tiles of
  // gathered full keys (every row sees them) followed by the plan's list;
  // iteration index i < n_gath is gathered tile i.
  const int* plist = PATTERN ? pat.list + (size_t)qb * pat.stride : nullptr;
  const int n_full_keys = PATTERN ? pat.other_count[0] : 0;
  const int n_gath = (n_full_keys + BC - 1) / BC;
  const int n_listed = PATTERN ? pat.count[qb] : 0;
  const int n_tiles = PATTERN ? (n_listed < 0 ? 0 : n_gath + n_listed) : t_hi - t_lo;
  auto tile_at = [&](int i) { return PATTERN ? plist[i - n_gath] >> kEntryTileShift : t_lo + i; };
  // keys visible to this lane's row through the band
  int key_lo = 0, key_hi = n;
  if constexpr (WINDOWED) band_keys(my_row, my_row + 1, n, window, &key_lo, &key_hi);
  if constexpr (PATTERN) {
    if (pat.window >= 0)
      band_keys(my_row, my_row + 1, n, pat.window, &key_lo, &key_hi);
    else
      key_hi = key_lo;
  }
  const unsigned key_span = (unsigned)max(key_hi - key_lo, 0);
  // Under a pattern a wave skips the work of a partial listed key tile that
  // none of its rows sees, and of every tile when its rows are all full rows
  // or past n.
  const int rw0 = q0 + wave * 32;  // first row of this wave
  const bool wave_live = !PATTERN || (rw0 < n && pat.own_full[rw0 >> 5] != ~0u);

  // K and V tiles go straight from global memory to LDS.  Key rows past n
  // are zeros in the K tile, so whatever their dS, they add exactly nothing
  // to dQ = dS K (their V rows are clamped copies and only feed that dS); the
  // same holds for the slots of a gathered tile past the full keys' count.
  using Tile = TileAsync<D, BC, NT>;
  using TileK = TileAsyncZeroTail<D, BC, NT>;
  using Dma = TileDma<D, BC, NT>;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  uint32_t dma_off[Dma::IT];  // this thread's chunk offsets in a full K or V tile
  Dma::init(tid, dma_off);
  auto load_tile = [&](int i, int buf) {
    if constexpr (PATTERN) {
      // gathered tiles read the full keys' copies, laid out like the rows of
      // a key/value head
      const bool g = i < n_gath;
      const int r0 = g ? i * BC : tile_at(i) * BC;
      const int valid = (g ? n_full_keys : n) - r0;
      TileK::issue((g ? pat.gath_a + kv_off : K) + (size_t)r0 * D, valid, tiles[buf][0], tid);
      Tile::issue((g ? pat.gath_b + kv_off : V) + (size_t)r0 * D, valid, tiles[buf][1], tid);
    } else {
      const int kbase = tile_at(i) * BC;
      if (kbase + BC <= n) {
        Dma::issue(K + (size_t)kbase * D, dma_off, tiles[buf][0], wave_s);
        Dma::issue(V + (size_t)kbase * D, dma_off, tiles[buf][1], wave_s);
      } else {
        TileK::issue(K + (size_t)kbase * D, n - kbase, tiles[buf][0], tid);
        Tile::issue(V + (size_t)kbase * D, n - kbase, tiles[buf][1], tid);
      }
    }
  };

  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};

  if (n_tiles > 0) load_tile(0, 0);
  wait_all_and_barrier();

  for (int it = 0; it < n_tiles; ++it) {
    const bool gathered = PATTERN && it < n_gath;
    const int t = gathered ? 0 : tile_at(it);
    const int buf = it & 1;
    if (it + 1 < n_tiles) load_tile(it + 1, buf ^ 1);  // buffer released by the last barrier
    const __bf16* Ks = tiles[buf][0];
    const __bf16* Vs = tiles[buf][1];
    const int kbase = t * BC;

    bool act = true;
    // As in the key-side pass: a wave skips key tiles its rows' band misses,
    // except at d=256.
    if constexpr (WINDOWED && D != 256) act = kbase <= rw0 + 31 + window && rw0 <= kbase + BC - 1 + window;
    if constexpr (PATTERN) {
      act = wave_live;
      if (act && !gathered) {
        const int entry = plist[it - n_gath];
        if (entry & 1) {
          const bool lay = (entry >> (1 + wave)) & 1;
          act = lay || (pat.window >= 0 && kbase <= rw0 + 31 + pat.window && rw0 <= kbase + BC - 1 + pat.window);
        }
      }
    }
    if (act) {
      // S^T = K Q^T and dP^T = V dO^T: lanes indexed by query row.  The dP
      // accumulator starts at the row's -D, so the product ends as dP - D
      // (the 16 registers holding -D stay live through the loop; at d=64 they
      // would cost a wave per SIMD, so there -D is added afterwards).
      constexpr bool kNegInit = D != 64;
      f32x16 s[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[kb][r] = kNegInit ? ndl : 0.0f;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          s[kb] = mfma32(lds_row_frag<D>(Ks, kb * 32 + l32, ds, hi), qreg[ds], s[kb]);
          dp[kb] = mfma32(lds_row_frag<D>(Vs, kb * 32 + l32, ds, hi), greg[ds], dp[kb]);
        }
      }
      // Row reads of K and V two steps ahead of their products (d=256: 4%
      // faster).
      if constexpr (D == 256) {
        constexpr int NS = NKB * NDS, kLead = 2;
        EXATTN_SCHED(kSchedDSRead, 2 * kLead);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          EXATTN_SCHED(kSchedMFMA, 2);
          if (i + kLead < NS) EXATTN_SCHED(kSchedDSRead, 2);
        }
      }

      // With a window, keys outside this lane's row band get P = 0 (keys past
      // n meet zero K rows).  Under a pattern, a partial listed tile keeps the
      // pairs that the band or the layout make visible, except those of full
      // keys (they come from the gathered tiles).
      bool need_mask = false;
      uint32_t lay = 0;  // the layout covers the wave for the tile
      if constexpr (WINDOWED) {
        const int r_lo = q0 + wave * 32;
        need_mask = max(r_lo + 31 - kbase, kbase + BC - 1 - r_lo) > window;
      }
      if constexpr (PATTERN) {
        if (!gathered) {
          const int entry = plist[it - n_gath];
          lay = (entry >> (1 + wave)) & 1;
          need_mask = (entry & 1) && !(lay && !(entry & kEntryHasFull));  // covered by the layout, no full key
        }
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -lse2));
          if (WINDOWED && need_mask) {
            const int key = kbase + kb * 32 + acc_row(r, lane);
            p = (unsigned)(key - key_lo) < key_span ? p : 0.0f;
          }
          if (PATTERN && need_mask) {  // bitwise: one select, no short-circuit branches
            const int e = 8 * (r >> 2) + (r & 3);  // acc_row(r, lane) - 4*hi
            const int key = kbase + kb * 32 + e + 4 * hi;
            const uint32_t fk = pat.other_full[(kbase >> 5) + kb] >> (4 * hi);
            const uint32_t vis = ((uint32_t)((unsigned)(key - key_lo) < key_span) | lay) & ~(fk >> e);
            p = (vis & 1u) ? p : 0.0f;
          }
          dp[kb][r] = p * (kNegInit ? dp[kb][r] : dp[kb][r] + ndl);  // dS^T = P^T (dP^T - D) (unscaled)
        }

      // dQ^T += K^T dS^T, k along the tile's keys.
#pragma unroll
      for (int st = 0; st < BC / 16; ++st) {
        const bf16x8 sb = acc_to_operand(dp[st >> 1], st & 1);
#pragma unroll
        for (int db = 0; db < NDB; ++db) dq[db] = mfma32(lds_col_frag<D>(Ks, 16 * st, 32 * db, lane), sb, dq[db]);
      }
      // As in the key-side pass: transposed reads two products ahead (1.3%
      // faster at d=128; 12% slower at d=256, so only d=128).
      if constexpr (D == 128) {
        constexpr int NP = (BC / 16) * NDB, kLead = 2;
        EXATTN_SCHED(kSchedDSRead, 2 * kLead);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          EXATTN_SCHED(kSchedMFMA, 1);
          if (i + kLead < NP) EXATTN_SCHED(kSchedDSRead, 2);
        }
      }

    }

    wait_all_and_barrier();
  }

  bool store = my_row < n;
  if constexpr (PATTERN) store = store && !bit_of(pat.own_full, my_row);
  if (FULL && store && f.chunks > 1) {
    float* prow = full.part + ((size_t)(head * f.chunks + f.chunk) * f.groups * BR + f_slot) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hi;
        *(f32x4*)(prow + dd) = f32x4{dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale, dq[db][4 * g + 2] * scale,
                                     dq[db][4 * g + 3] * scale};
      }
  } else if (store) {
    __bf16* dqr = dQg + hoff + (size_t)my_row * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * db + 8 * g + 4 * hi;
        u32x2 w;
        w[0] = pack_bf16x2(dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale);
        w[1] = pack_bf16x2(dq[db][4 * g + 2] * scale, dq[db][4 * g + 3] * scale);
        *(u32x2*)(dqr + dd) = w;
      }
  }
}

// Sum of the full positions' chunks (when there are several), in chunk
// order: each slot holds NOUT vectors of D floats (dK then dV, or dQ), the
// sums go to out[0..NOUT) at the position's row, in bf16.  One thread per
// four consecutive elements, in a grid-stride loop.
template <int D, int NOUT>
__global__ __launch_bounds__(256) void full_sum_kernel(FullDev full, __bf16* __restrict__ out0,
                                                       __bf16* __restrict__ out1, int n, int heads) {
  constexpr int Q4 = NOUT * D / 4;  // groups of four per slot
  const int R = full.info[kFullCount], C = full.info[kFullChunks];
  if (C <= 1) return;
  const size_t GB = (size_t)full.info[kFullGroups] * kFullRows;  // slots per (head, chunk)
  const long items = (long)heads * R * Q4;
  for (long it = (long)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += (long)gridDim.x * blockDim.x) {
    const long hs = it / Q4;
    const int q = (int)(it - hs * Q4);
    const int head = (int)(hs / R), slot = (int)(hs - (long)head * R);
    const float* src = full.part + ((size_t)head * C * GB + slot) * (NOUT * D) + 4 * q;
    const size_t stride = GB * (NOUT * D);
    f32x4 acc = *(const f32x4*)src;
    for (int c = 1; c < C; ++c) acc += *(const f32x4*)(src + c * stride);
    const int k = (4 * q) / D, dd = (4 * q) % D;
    u32x2 w;
    w[0] = pack_bf16x2(acc[0], acc[1]);
    w[1] = pack_bf16x2(acc[2], acc[3]);
    *(u32x2*)((k == 0 ? out0 : out1) + ((size_t)head * n + full.idx[slot]) * D + dd) = w;
  }
}

// ---------------------------------------------------------------------------
// Query side at d = 256 without a pattern: paired waves.
// ---------------------------------------------------------------------------
// The 8 waves form 4 pairs (wave w and wave w+4 share a SIMD); a pair owns 32
// query rows.  The dS-wave holds the rows' Q in registers and their dO rows
// in LDS and, per key tile, forms S = Q K^T and dP = dO V^T, then
// dS = P (dP - D) with P = exp(S - LSE), and hands dS (bf16 MFMA operands)
// to its partner through LDS; the dQ-wave holds the dQ accumulator and adds
// dS K, one tile behind.  One wave holding Q, dO and dQ needed all 512
// registers of a SIMD; split this way the SIMD runs two waves, each one's
// latencies covered by the other's work.  K tiles stay in LDS one iteration
// longer than V tiles (the dQ-wave reads tile i-1 while the dS-wave reads
// tile i): three K buffers, two V buffers; with the dO rows they fill the
// 160 KiB of LDS.
template <int D>
struct PairQ {
  static constexpr int BC = 32, NT = 512, BR = 128;
  static constexpr int kTile = BC * D * 2;       // bytes of one K or V tile
  static constexpr int kK = 0;                   // [3] K tiles
  static constexpr int kV = kK + 3 * kTile;      // [2] V tiles
  static constexpr int kSPair = 2 * 64 * 16;     // one pair's dS operands
  static constexpr int kS = kV + 2 * kTile;      // [2][pair]
  static constexpr int kGPair = 32 * D * 2;      // one pair's dO rows
  static constexpr int kG = kS + 2 * 4 * kSPair; // [pair]
  static constexpr int kBytes = kG + 4 * kGPair;
  static_assert(kBytes <= 160 * 1024, "one workgroup per CU");
};

template <int D, int MODE>
constexpr bool pair_q_dispatch() {
  return D == 256 && (MODE == kMaskNone || MODE == kMaskWindow);
}

template <int D, int MODE>
__global__ __launch_bounds__(512, 2) void bwd_q_pair_kernel(
    const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
    const __bf16* __restrict__ dOg, const float* __restrict__ LSE2g, const float* __restrict__ Dg,
    __bf16* __restrict__ dQg, int n, int n_qblocks, int total_blocks, float scale, float scale_log2, int window,
    int group) {
  using C = PairQ<D>;
  constexpr bool WINDOWED = MODE == kMaskWindow;
  constexpr int BC = C::BC, NT = C::NT, BR = C::BR;
  constexpr int NDS = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(16))) char lds[C::kBytes];
  poison_lds(lds);

  const int bid = xcd_remap(blockIdx.x, total_blocks);
  const int head = bid / n_qblocks;
  const int qb = bid - head * n_qblocks;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const bool swave = wave < 4;  // dS-wave, else dQ-wave

  const size_t hoff = (size_t)head * n * D;
  const size_t kv_off = (size_t)(head / group) * n * D;  // key/value head of this query head
  const __bf16* K = Kg + kv_off;
  const __bf16* V = Vg + kv_off;
  const int q0 = qb * BR;
  const int w0 = q0 + pair * 32;  // first row of the pair
  const int my_row = w0 + l32;

  int k_lo = 0, k_hi = n;
  if constexpr (WINDOWED) band_keys(q0, q0 + BR, n, window, &k_lo, &k_hi);
  const int t_lo = k_lo / BC;
  const int n_tiles = (k_hi + BC - 1) / BC - t_lo;

  // K and V tiles go straight from global memory to LDS.  Key rows past n
  // are zeros in the K tile, so whatever their dS, they add exactly nothing
  // to dQ = dS K (their V rows are clamped copies and only feed that dS).
  using Tile = TileAsync<D, BC, NT>;
  using TileK = TileAsyncZeroTail<D, BC, NT>;
  using Dma = TileDma<D, BC, NT>;
  uint32_t dma_off[Dma::IT];
  Dma::init(tid, dma_off);
  auto load_tile = [&](int i) {
    const int kbase = (t_lo + i) * BC;
    __bf16* kd = (__bf16*)(lds + C::kK + (i % 3) * C::kTile);
    __bf16* vd = (__bf16*)(lds + C::kV + (i & 1) * C::kTile);
    if (kbase + BC <= n) {
      Dma::issue(K + (size_t)kbase * D, dma_off, kd, wave);
      Dma::issue(V + (size_t)kbase * D, dma_off, vd, wave);
    } else {
      TileK::issue(K + (size_t)kbase * D, n - kbase, kd, tid);
      Tile::issue(V + (size_t)kbase * D, n - kbase, vd, tid);
    }
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
  const int s_off = C::kS + pair * C::kSPair + 16 * lane;  // + buffer * 4 * kSPair + operand * 1024

  // The dS-wave's Q^T operands (lane: row my_row, columns 16*ds + 8*hi ..
  // +8), its row's LSE*log2(e) and -D, and its dO rows (to LDS, swizzled like
  // the tiles; rows past n are clamped copies), loaded before the first
  // wait, which then covers them (the compiler's own wait for these loads
  // would otherwise sit inside the loop and also wait for the copies issued
  // there).
  const int g_base = C::kG + pair * C::kGPair;  // wave-uniform
  bf16x8 qreg[NDS];
  float lse2 = 0.0f, ndl = 0.0f;
  if (swave) {
    const bool ok = my_row < n;
    const u32x4* qs = (const u32x4*)(Qg + hoff + (size_t)(ok ? my_row : 0) * D + 8 * hi);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qreg[ds] = __builtin_bit_cast(bf16x8, ok ? qs[2 * ds] : u32x4{0, 0, 0, 0});
    lse2 = ok ? LSE2g[(size_t)head * n + my_row] : __builtin_huge_valf();  // rows past n: P = 0
    ndl = ok ? Dg[(size_t)head * n + my_row] : 0.0f;
#pragma unroll
    for (int it = 0; it < 32 * (D / 8) / 64; ++it) {
      const int slot = it * 64 + lane, row = slot / (D / 8);
      const int r = min(w0 + row, n - 1);
      lds_dma16(dOg + hoff + (size_t)r * D + 8 * swz_chunk<D>(row, slot % (D / 8)), lds + g_base + 16 * (it * 64));
    }
  }
  if (n_tiles > 0) load_tile(0);
  wait_all_and_barrier();

  if (swave) {
    // keys this lane's row sees: [key_lo, key_lo + key_span)
    int key_lo = 0, key_hi = n;
    if constexpr (WINDOWED) band_keys(my_row, my_row + 1, n, window, &key_lo, &key_hi);
    const unsigned key_span = (unsigned)max(key_hi - key_lo, 0);
    for (int i = 0; i <= n_tiles; ++i) {
      if (i + 1 < n_tiles) load_tile(i + 1);
      if (i < n_tiles && pair_sees(i)) {
        const __bf16* Ks = (const __bf16*)(lds + C::kK + (i % 3) * C::kTile);
        const __bf16* Vs = (const __bf16*)(lds + C::kV + (i & 1) * C::kTile);
        const int kbase = (t_lo + i) * BC;
        // S^T = K Q^T and dP^T = V dO^T: lanes = the pair's rows, registers
        // = keys; the dP accumulator starts at the row's -D, so the product
        // ends as dP - D
        f32x16 s = f32x16{}, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = ndl;
        const __bf16* Gs = (const __bf16*)(lds + g_base);
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          s = mfma32(lds_row_frag<D>(Ks, l32, ds, hi), qreg[ds], s);
          dp = mfma32(lds_row_frag<D>(Vs, l32, ds, hi), lds_row_frag<D>(Gs, l32, ds, hi), dp);
        }
        // P = 2^(scale*log2e*s - LSE*log2e) (keys outside the row's band,
        // and past n, get P = 0), dS^T = P^T (dP^T - D) (unscaled)
        bool need_mask = kbase + BC > n;
        if constexpr (WINDOWED) need_mask = need_mask || max(w0 + 31 - kbase, kbase + BC - 1 - w0) > window;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -lse2));
          if (need_mask) {
            const int key = kbase + acc_row(r, lane);
            p = (unsigned)(key - key_lo) < key_span ? p : 0.0f;
          }
          dp[r] *= p;
        }
        // to the dQ-wave: lane-private 16-byte slots, consecutive lanes in
        // consecutive slots
        const int b = i & 1;
#pragma unroll
        for (int c = 0; c < 2; ++c)
          *(u32x4*)(lds + s_off + b * (4 * C::kSPair) + c * 1024) = __builtin_bit_cast(u32x4, acc_to_operand(dp, c));
      }
      wait_all_and_barrier();
    }
  } else {
    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};
    for (int i = 0; i <= n_tiles; ++i) {
      if (i + 1 < n_tiles) load_tile(i + 1);
      if (i >= 1 && pair_sees(i - 1)) {
        const int b = (i - 1) & 1;
        const __bf16* Ks = (const __bf16*)(lds + C::kK + ((i - 1) % 3) * C::kTile);
        // dQ^T += K^T dS^T, k along the tile's keys (K^T through the
        // transpose read)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 sb = *(const bf16x8*)(lds + s_off + b * (4 * C::kSPair) + st * 1024);
#pragma unroll
          for (int db = 0; db < NDB; ++db) dq[db] = mfma32(lds_col_frag<D>(Ks, 16 * st, 32 * db, lane), sb, dq[db]);
        }
      }
      wait_all_and_barrier();
    }
    if (my_row < n) {
      __bf16* dqr = dQg + hoff + (size_t)my_row * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = 32 * db + 8 * g + 4 * hi;
          u32x2 w;
          w[0] = pack_bf16x2(dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale);
          w[1] = pack_bf16x2(dq[db][4 * g + 2] * scale, dq[db][4 * g + 3] * scale);
          *(u32x2*)(dqr + dd) = w;
        }
    }
  }
}

// Key side, then query side, of one mask mode.
template <int D, int W>
hipError_t bwd_passes(const BwdParams& p, unsigned stages, hipStream_t stream) {
  const float scale_log2 = p.scale * kLog2e;
  const long heads = (long)p.B * p.H;
  const long kv_heads = heads / p.group;
  constexpr int BKV = 32 * kv_waves<D, W>();
  const int nkb = (p.n + BKV - 1) / BKV;
  const long tk = (long)nkb * kv_heads;
  constexpr int BR = 32 * q_waves<D, W>();
  const int nqb = (p.n + BR - 1) / BR;
  const long tq = (long)nqb * heads;
  if (tk > 0x7fffffffL || tq > 0x7fffffffL) return hipErrorInvalidValue;
  const PatternDev pkv = W == kMaskFull ? PatternDev{} : p.pattern_kv;
  const PatternDev pq = W == kMaskFull ? PatternDev{} : p.pattern_q;
  if (stages & kStageKV) {
    if constexpr (pair_kv_dispatch<D, W>()) {
      static_assert(BKV == PairKv<D>::BKV, "the paired kernel's key block matches the grid");
      hipLaunchKernelGGL((bwd_kv_pair_kernel<D, W>), dim3((unsigned)tk), dim3(512), 0, stream, (const __bf16*)p.q,
                         (const __bf16*)p.k, (const __bf16*)p.v, (const __bf16*)p.dout, p.lse2, p.delta,
                         (__bf16*)p.dk, (__bf16*)p.dv, p.n, nkb, (int)tk, p.scale, scale_log2, p.window, p.group);
    } else {
      hipLaunchKernelGGL((bwd_kv_bf16_kernel<D, W>), dim3((unsigned)tk), dim3(kv_waves<D, W>() * 64), 0, stream,
                         (const __bf16*)p.q, (const __bf16*)p.k, (const __bf16*)p.v, (const __bf16*)p.dout, p.lse2,
                         p.delta, (__bf16*)p.dk, (__bf16*)p.dv, p.n, nkb, (int)tk, p.scale, scale_log2, p.window,
                         p.group, pkv, p.full_kv);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && W == kMaskFull) {
      hipLaunchKernelGGL((full_sum_kernel<D, 2>), dim3(1024), dim3(256), 0, stream, p.full_kv, (__bf16*)p.dk,
                         (__bf16*)p.dv, p.n, (int)kv_heads);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }
  if (stages & kStageQ) {
    if constexpr (pair_q_dispatch<D, W>()) {
      static_assert(BR == PairQ<D>::BR, "the paired kernel's row block matches the grid");
      hipLaunchKernelGGL((bwd_q_pair_kernel<D, W>), dim3((unsigned)tq), dim3(PairQ<D>::NT), 0, stream,
                         (const __bf16*)p.q, (const __bf16*)p.k, (const __bf16*)p.v, (const __bf16*)p.dout, p.lse2,
                         p.delta, (__bf16*)p.dq, p.n, nqb, (int)tq, p.scale, scale_log2, p.window, p.group);
    } else {
      hipLaunchKernelGGL((bwd_q_bf16_kernel<D, W>), dim3((unsigned)tq), dim3(q_waves<D, W>() * 64), 0, stream,
                         (const __bf16*)p.q, (const __bf16*)p.k, (const __bf16*)p.v, (const __bf16*)p.dout, p.lse2,
                         p.delta, (__bf16*)p.dq, p.n, nqb, (int)tq, p.scale, scale_log2, p.window, p.group, pq,
                         p.full_q);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && W == kMaskFull) {
      hipLaunchKernelGGL((full_sum_kernel<D, 1>), dim3(1024), dim3(256), 0, stream, p.full_q, (__bf16*)p.dq,
                         (__bf16*)nullptr, p.n, (int)heads);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Under a pattern with full positions, each side's pattern pass is followed
// by its full-position pass; the two sides use the partial buffer in turn.
template <int D, int W>
hipError_t bwd_d(const BwdParams& p, unsigned stages, hipStream_t stream) {
  if (stages & kStageRowdot) {
    hipError_t e = launch_rowdot<__bf16>((const __bf16*)p.o, (const __bf16*)p.dout, p.lse, p.delta, p.lse2,
                                         (long)p.B * p.H * p.n, D, stream);
    if (e != hipSuccess) return e;
  }
  const bool with_full = W == kMaskPattern && p.full_kv.idx != nullptr;
  for (unsigned side : {unsigned(kStageKV), unsigned(kStageQ)}) {
    if (!(stages & side)) continue;
    hipError_t e = hipSuccess;
    // under a pattern, first the copies of the other side's full positions
    // (the scratch region they use is free again once the previous side's
    // partial results are summed)
    if (W == kMaskPattern && side == kStageKV)
      e = launch_pattern_gather(p.pattern_kv, (const __bf16*)p.q, (const __bf16*)p.dout, p.lse2, p.delta, p.B * p.H,
                                p.n, D, stream);
    if (W == kMaskPattern && side == kStageQ)
      e = launch_pattern_gather(p.pattern_q, (const __bf16*)p.k, (const __bf16*)p.v, nullptr, nullptr,
                                p.B * p.H / p.group, p.n, D, stream);
    if (e == hipSuccess) e = bwd_passes<D, W>(p, side, stream);
    if (e == hipSuccess && with_full) e = bwd_passes<D, kMaskFull>(p, side, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

#ifndef EXATTN_BWD_D128
template <int MODE>
hipError_t bwd_mode(const BwdParams& p, unsigned stages, hipStream_t stream) {
  switch (p.d) {
    case 64: return bwd_d<64, MODE>(p, stages, stream);
    case 128:
      if constexpr (MODE == kMaskNone)
        return launch_bwd_bf16_d128(p, stages, stream);
      else
        return bwd_d<128, MODE>(p, stages, stream);
    case 256: return bwd_d<256, MODE>(p, stages, stream);
    default: return hipErrorInvalidValue;
  }
}
#endif

}  // namespace

#ifdef EXATTN_BWD_D128
hipError_t launch_bwd_bf16_d128(const BwdParams& p, unsigned stages, hipStream_t stream) {
  return bwd_d<128, kMaskNone>(p, stages, stream);
}
#else

hipError_t launch_bwd_bf16(const BwdParams& p, unsigned stages, hipStream_t stream) {
  if (p.pattern_kv.list != nullptr) {
    for (const PatternDev* q : {&p.pattern_kv, &p.pattern_q})
      if (q->list == nullptr || q->count == nullptr || q->own_full == nullptr || q->other_full == nullptr ||
          q->other_idx == nullptr || q->other_count == nullptr || q->gath_a == nullptr || q->gath_b == nullptr)
        return hipErrorInvalidValue;
    if (p.pattern_kv.gath_s0 == nullptr || p.pattern_kv.gath_s1 == nullptr) return hipErrorInvalidValue;
    return bwd_mode<kMaskPattern>(p, stages, stream);
  }
  return p.window >= 0 ? bwd_mode<kMaskWindow>(p, stages, stream) : bwd_mode<kMaskNone>(p, stages, stream);
}

void bwd_kv_bf16_geometry(int d, int* keys_per_block, int* rows_per_tile, int* waves) {
  *waves = d == 64 ? kv_waves<64, kMaskPattern>() : d == 128 ? kv_waves<128, kMaskPattern>()
                                                             : kv_waves<256, kMaskPattern>();
  *keys_per_block = 32 * *waves;
  *rows_per_tile = KvCfg<128>::BQ;
}

void bwd_q_bf16_geometry(int d, int* rows_per_block, int* keys_per_tile, int* waves) {
  switch (d) {
    case 64: *keys_per_tile = QCfg<64>::BC; *waves = q_waves<64, kMaskPattern>(); break;
    case 128: *keys_per_tile = QCfg<128>::BC; *waves = q_waves<128, kMaskPattern>(); break;
    default: *keys_per_tile = QCfg<256>::BC; *waves = q_waves<256, kMaskPattern>(); break;
  }
  *rows_per_block = 32 * *waves;
}
#endif

}  // namespace exattn
