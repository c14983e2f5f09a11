// Plan kernels for sparse patterns: the global-token bitmap and the full
// positions, then for every workgroup of a kernel the list of tiles that hold
// at least one visible (query, key) pair of a position it stores, each
// classified as fully visible or partial.
#include "device_common.hpp"
#include "pattern.hpp"

namespace exattn {
namespace {

// One workgroup per layout block index r: is layout row r set in every
// block, and is layout column r set in every block?
__global__ __launch_bounds__(256) void pattern_layout_full_kernel(const unsigned char* __restrict__ layout, int nb,
                                                                  int* __restrict__ flags) {
  const int r = blockIdx.x;
  int row_all = 1, col_all = 1;
  for (int c = threadIdx.x; c < nb; c += blockDim.x) {
    row_all &= layout[(size_t)r * nb + c] != 0;
    col_all &= layout[(size_t)c * nb + r] != 0;
  }
  row_all = __syncthreads_and(row_all);
  col_all = __syncthreads_and(col_all);
  if (threadIdx.x == 0) {
    flags[r] = row_all;
    flags[nb + r] = col_all;
  }
}

// Exclusive prefix sum over the workgroup (blockDim.x a multiple of 64, at
// most 1024); `sh` holds 16 ints.  Returns this thread's offset and the total.
__device__ int block_exclusive_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  int x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < nwaves; ++w) {
    const int t = sh[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();  // sh is reused by the next scan
  *total = tot;
  return before + x - v;
}

// Writes the positions of the set bits of words [w0, w1) from `out[pos]` on.
__device__ void write_positions(const uint32_t* bits, int w0, int w1, int* out, int pos) {
  for (int w = w0; w < w1; ++w)
    for (uint32_t m = bits[w]; m != 0u; m &= m - 1u) out[pos++] = 32 * w + __builtin_ctz(m);
}

struct FullSplits {
  FullSplit s[3];
  int count;
};

// One workgroup: the global-token bitmap (padding cleared; positions outside
// [0, n) ignored), the full-row and full-key bitmaps (global tokens, plus the
// layout rows / columns set in every block), their ascending position lists,
// and how each consumer kernel splits them into workgroups and chunks.
__global__ __launch_bounds__(1024) void pattern_bitmap_kernel(PlanInput in, FullSplits sp) {
  __shared__ int sh[16];
  poison_lds(sh);
  const int tid = threadIdx.x, nt = blockDim.x;
  const int n = in.n, nwords = bitmap_words(n), W = (n + 31) / 32;
  for (int w = tid; w < nwords; w += nt) in.gbits[w] = 0u;
  __syncthreads();
  for (int i = tid; i < in.n_global; i += nt) {
    const int p = in.global_idx[i];
    if ((unsigned)p < (unsigned)n) atomicOr(&in.gbits[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  for (int w = tid; w < nwords; w += nt) {
    uint32_t r = in.gbits[w], c = r;
    if (in.layout != nullptr && w < W) {
      const int b = w / (kLayoutBlock / 32);  // the 32 positions of a word lie in one layout block
      if (in.layout_flags[b]) r = ~0u;
      if (in.layout_flags[in.layout_n + b]) c = ~0u;
      if (32 * w + 32 > n) {
        const uint32_t keep = (1u << (n - 32 * w)) - 1u;
        r &= keep;
        c &= keep;
      }
    }
    in.row_full[w] = r;
    in.col_full[w] = c;
  }
  __syncthreads();
  // compaction: each thread takes a contiguous run of words
  const int per = (W + nt - 1) / nt;
  const int w0 = min(W, tid * per), w1 = min(W, w0 + per);
  int nr = 0, nc = 0;
  for (int w = w0; w < w1; ++w) {
    nr += __builtin_popcount(in.row_full[w]);
    nc += __builtin_popcount(in.col_full[w]);
  }
  int rows_total, cols_total;
  const int pr = block_exclusive_scan(nr, sh, &rows_total);
  const int pc = block_exclusive_scan(nc, sh, &cols_total);
  write_positions(in.row_full, w0, w1, in.row_idx, pr);
  write_positions(in.col_full, w0, w1, in.col_idx, pc);
  if (tid == 0) {
    in.counts[0] = rows_total;
    in.counts[1] = cols_total;
    for (int i = 0; i < sp.count; ++i) {
      const FullSplit& f = sp.s[i];
      const int R = f.keys ? cols_total : rows_total;
      const int G = (R + kFullRows - 1) / kFullRows;
      int C = 1;
      if (G > 0) {
        const int cap = full_part_rows(n) / (kFullRows * G);
        const int want = (f.tiles + kFullChunkTiles - 1) / kFullChunkTiles;
        C = max(1, min(cap, want));
      }
      const int tl = (f.tiles + C - 1) / C;
      C = (f.tiles + tl - 1) / tl;  // no empty chunk
      f.info[kFullCount] = R;
      f.info[kFullGroups] = G;
      f.info[kFullChunks] = C;
      f.info[kFullTilesPerChunk] = tl;
    }
  }
}

// Number of set bits of positions [a, b).
__device__ int count_bits(const uint32_t* bits, int a, int b) {
  int c = 0;
  for (int w = a >> 5; w <= (b - 1) >> 5 && a < b; ++w) {
    uint32_t m = bits[w];
    const int lo = w * 32, hi = lo + 32;
    if (a > lo) m &= ~0u << (a - lo);
    if (b < hi) m &= ~0u >> (hi - b);
    c += __builtin_popcount(m);
  }
  return c;
}

// One workgroup (256 threads) per workgroup row of the kernel's grid: each
// thread classifies one tile, and the listed tiles are compacted in tile
// order with wave ballots and a prefix over the four waves.
__global__ __launch_bounds__(256) void pattern_list_kernel(PlanInput in, PlanList pl) {
  __shared__ int wave_count[4];
  poison_lds(wave_count);
  const int blk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = in.n;
  const int r0 = blk * pl.R, r1 = min(n, r0 + pl.R);  // own positions
  const int n_own = r1 - r0;
  // Full own positions are written by the full-position pass: they list no
  // tile, and a block holding only such positions lists none.
  const bool any_part = n_own > count_bits(pl.own_full, r0, r1);
  const int ntile = any_part ? (n + pl.T - 1) / pl.T : 0;
  int* out = pl.list + (size_t)blk * pl.stride;
  int total = 0;  // entries written so far (uniform)
  for (int base = 0; base < ntile; base += 256) {
    const int t = base + tid;
    int entry = -1;
    if (t < ntile) {
      const int c0 = t * pl.T, c1 = min(n, c0 + pl.T);
      // full positions of the other side are gathered apart: a tile made of
      // them only is not listed, and one holding any of them is partial
      const int f_other = count_bits(pl.other_full, c0, c1);
      // queries [q0, q1) against keys [k0, k1)
      const int q0 = pl.transposed ? c0 : r0, q1 = pl.transposed ? c1 : r1;
      const int k0 = pl.transposed ? r0 : c0, k1 = pl.transposed ? r1 : c1;
      bool any_band = false, full_band = false;
      if (in.window >= 0) {
        any_band = k0 <= q1 - 1 + in.window && q0 <= k1 - 1 + in.window;
        full_band = max(q1 - 1 - k0, k1 - 1 - q0) <= in.window;
      }
      // layout bit of each wave's 32 own positions against this tile
      unsigned wbits = 0;
      bool lay_any = false, lay_all = in.layout != nullptr;
      if (in.layout != nullptr) {
        for (int w = 0; w < pl.NW; ++w) {
          const int p = r0 + 32 * w;
          if (p >= n) {  // rows/keys past the end: nothing to compute for them
            wbits |= 1u << w;
            continue;
          }
          const int ob = p / kLayoutBlock, tb = c0 / kLayoutBlock;
          const bool on =
              in.layout[pl.transposed ? (size_t)tb * in.layout_n + ob : (size_t)ob * in.layout_n + tb] != 0;
          if (on) wbits |= 1u << w;
          lay_any = lay_any || (on && pl.own_full[p >> 5] != ~0u);  // a wave of full positions needs no tile
          lay_all = lay_all && on;
        }
      }
      // Global positions are full positions on either side: only the band
      // and the layout list a tile.
      if ((any_band || lay_any) && f_other < c1 - c0) {
        const bool full = (full_band || lay_all) && f_other == 0;
        const bool partial = !full || (pl.tail_partial && c1 - c0 < pl.T);
        entry = (t << kEntryTileShift) | (f_other > 0 ? kEntryHasFull : 0) | (int)(wbits << 1) | (partial ? 1 : 0);
      }
    }
    // compaction: rank among the listed tiles of this chunk, in tile order
    const unsigned long long m = __ballot(entry >= 0);
    if (lane == 0) wave_count[wave] = __popcll(m);
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_count[w];
    const int rank = before + __popcll(m & ((1ull << lane) - 1ull));
    if (entry >= 0) out[total + rank] = entry;
    total += wave_count[0] + wave_count[1] + wave_count[2] + wave_count[3];
    __syncthreads();  // wave_count is rewritten by the next chunk
  }
  if (tid == 0) pl.count[blk] = any_part ? total : -1;  // -1: every own position is full, nothing to do
}

// Gather of the other side's full positions: one thread per 16 bytes of a
// row of a or b (and the row's two values), in a grid-stride loop over
// heads * count rows.
__global__ __launch_bounds__(256) void pattern_gather_kernel(PatternDev pat, const __bf16* __restrict__ a,
                                                             const __bf16* __restrict__ b,
                                                             const float* __restrict__ s0,
                                                             const float* __restrict__ s1, int heads, int n, int d) {
  const int R = pat.other_count[0];
  const int cpr = d / 8;  // 16-byte chunks per row
  const long items = (long)heads * R * cpr;
  __bf16* ga = const_cast<__bf16*>(pat.gath_a);
  __bf16* gb = const_cast<__bf16*>(pat.gath_b);
  for (long it = (long)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += (long)gridDim.x * blockDim.x) {
    const long hs = it / cpr;
    const int c = (int)(it - hs * cpr);
    const int head = (int)(hs / R), slot = (int)(hs - (long)head * R);
    const size_t src = (size_t)head * n + pat.other_idx[slot], dst = (size_t)head * n + slot;
    *(uint4*)(ga + dst * d + 8 * c) = *(const uint4*)(a + src * d + 8 * c);
    *(uint4*)(gb + dst * d + 8 * c) = *(const uint4*)(b + src * d + 8 * c);
    if (s0 != nullptr && c == 0) {
      const_cast<float*>(pat.gath_s0)[dst] = s0[src];
      const_cast<float*>(pat.gath_s1)[dst] = s1[src];
    }
  }
}

}  // namespace

hipError_t launch_pattern_gather(const PatternDev& pat, const __bf16* a, const __bf16* b, const float* s0,
                                 const float* s1, int heads, int n, int d, hipStream_t stream) {
  if (pat.other_idx == nullptr || pat.other_count == nullptr || pat.gath_a == nullptr || pat.gath_b == nullptr ||
      (s0 != nullptr && (s1 == nullptr || pat.gath_s0 == nullptr || pat.gath_s1 == nullptr)))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(pattern_gather_kernel, dim3(1024), dim3(256), 0, stream, pat, a, b, s0, s1, heads, n, d);
  return hipGetLastError();
}

hipError_t launch_pattern_bitmap(const PlanInput& in, const FullSplit* splits, int n_splits, hipStream_t stream) {
  if (n_splits < 0 || n_splits > 3) return hipErrorInvalidValue;
  if (in.layout != nullptr) {
    hipLaunchKernelGGL(pattern_layout_full_kernel, dim3(in.layout_n), dim3(256), 0, stream, in.layout, in.layout_n,
                       in.layout_flags);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  FullSplits sp{};
  for (int i = 0; i < n_splits; ++i) sp.s[i] = splits[i];
  sp.count = n_splits;
  hipLaunchKernelGGL(pattern_bitmap_kernel, dim3(1), dim3(1024), 0, stream, in, sp);
  return hipGetLastError();
}

hipError_t launch_pattern_list(const PlanInput& in, const PlanList& pl, hipStream_t stream) {
  hipLaunchKernelGGL(pattern_list_kernel, dim3(pl.nblocks), dim3(256), 0, stream, in, pl);
  return hipGetLastError();
}

}  // namespace exattn
