// Plan kernels for sparse patterns: the global-token bitmap, then for every
// workgroup of a kernel the list of tiles that hold at least one visible
// (query, key) pair, each classified as fully visible or partial.
#include "pattern.hpp"

namespace exattn {
namespace {

// One workgroup: clear the bitmap (padding included), then set the bit of
// every global position in [0, n); positions outside are ignored.
__global__ __launch_bounds__(1024) void pattern_bitmap_kernel(const int* __restrict__ gidx, int ng, int n,
                                                             uint32_t* __restrict__ bits, int nwords) {
  for (int w = threadIdx.x; w < nwords; w += blockDim.x) bits[w] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < ng; i += blockDim.x) {
    const int p = gidx[i];
    if ((unsigned)p < (unsigned)n) atomicOr(&bits[p >> 5], 1u << (p & 31));
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
  const int blk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = in.n;
  const int r0 = blk * pl.R, r1 = min(n, r0 + pl.R);  // own positions
  const int n_own = r1 - r0;
  const int g_own = count_bits(in.gbits, r0, r1);
  const int ntile = (n + pl.T - 1) / pl.T;
  int* out = pl.list + (size_t)blk * pl.stride;
  int total = 0;  // entries written so far (uniform)
  for (int base = 0; base < ntile; base += 256) {
    const int t = base + tid;
    int entry = -1;
    if (t < ntile) {
      const int c0 = t * pl.T, c1 = min(n, c0 + pl.T);
      const int n_other = c1 - c0;
      const int g_other = count_bits(in.gbits, c0, c1);
      // queries [q0, q1) against keys [k0, k1)
      const int q0 = pl.transposed ? c0 : r0, q1 = pl.transposed ? c1 : r1;
      const int k0 = pl.transposed ? r0 : c0, k1 = pl.transposed ? r1 : c1;
      bool any_band = false, full_band = false;
      if (in.window >= 0) {
        any_band = k0 <= q1 - 1 + in.window && q0 <= k1 - 1 + in.window;
        full_band = max(q1 - 1 - k0, k1 - 1 - q0) <= in.window;
      }
      const int gq = pl.transposed ? g_other : g_own, nq = pl.transposed ? n_other : n_own;
      const int gk = pl.transposed ? g_own : g_other, nk = pl.transposed ? n_own : n_other;
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
          lay_any = lay_any || on;
          lay_all = lay_all && on;
        }
      }
      if (any_band || gq > 0 || gk > 0 || lay_any) {
        const bool full = full_band || gq == nq || gk == nk || lay_all;
        const bool partial = !full || (pl.tail_partial && c1 - c0 < pl.T);
        entry = (t << kEntryTileShift) | (int)(wbits << 1) | (partial ? 1 : 0);
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
  if (tid == 0) pl.count[blk] = total;
}

}  // namespace

hipError_t launch_pattern_bitmap(const PlanInput& in, hipStream_t stream) {
  hipLaunchKernelGGL(pattern_bitmap_kernel, dim3(1), dim3(1024), 0, stream, in.global_idx, in.n_global, in.n,
                     in.gbits, bitmap_words(in.n));
  return hipGetLastError();
}

hipError_t launch_pattern_list(const PlanInput& in, const PlanList& pl, hipStream_t stream) {
  hipLaunchKernelGGL(pattern_list_kernel, dim3(pl.nblocks), dim3(256), 0, stream, in, pl);
  return hipGetLastError();
}

}  // namespace exattn
