// Sparse attention patterns: the union of a sliding window, global tokens
// (whole rows and columns) and a block layout (llmis.ru chapter 3.1, section
// 3: Longformer's window and global tokens, BigBird's local, global and
// random blocks).  Row i sees key j when
//   (window >= 0 and |i - j| <= window) or i is global or j is global
//   or layout[i / 64][j / 64] is set.
//
// A plan step turns the pattern into, for every workgroup of a kernel, the
// list of tiles it must visit.  Each entry is
//   bits 9..31  tile index
//   bits 1..8   per wave: the layout covers this wave's 32 rows (or keys)
//               for the whole tile
//   bit  0      partial: some pair of the tile is not visible (or the tile
//               crosses the end of the sequence), so the kernel applies the
//               element mask; otherwise every pair is visible.
// Tiles with no visible pair are not listed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exattn {

constexpr int kLayoutBlock = 64;
constexpr int kEntryTileShift = 9;
// Extra zero words after the bitmap, so that reads for rows or keys of a
// workgroup that runs past the end of the sequence stay in the allocation.
constexpr int kBitmapPadWords = 16;

__host__ __device__ inline int bitmap_words(int n) { return (n + 31) / 32 + kBitmapPadWords; }

// What a kernel needs at run time.
struct PatternDev {
  int window;              // -1: no band term
  const uint32_t* gbits;   // global-token bitmap (bitmap_words(n) words)
  const int* list;         // entries, `stride` per workgroup row of the grid
  const int* count;        // number of entries per workgroup row
  int stride;
};

// One list to build: workgroups own `R` consecutive positions (queries, or
// keys when `transposed`), tiles span `T` positions of the other side, `NW`
// waves of 32 positions per workgroup.  `tail_partial` marks a tile that
// crosses the end of the sequence as partial.
struct PlanList {
  int R, T, NW;
  bool transposed;
  bool tail_partial;
  int* list;
  int* count;
  int stride;
  int nblocks;
};

struct PlanInput {
  int n;
  int window;
  int n_global;
  const int* global_idx;
  const unsigned char* layout;  // nullptr: no layout
  int layout_n;                 // blocks per layout row
  uint32_t* gbits;              // bitmap to build
};

hipError_t launch_pattern_bitmap(const PlanInput& in, hipStream_t stream);
hipError_t launch_pattern_list(const PlanInput& in, const PlanList& pl, hipStream_t stream);

// Element visibility on a partial tile, given the per-row and per-key terms.
__device__ __forceinline__ bool bit_of(const uint32_t* bits, int pos) { return (bits[pos >> 5] >> (pos & 31)) & 1u; }

}  // namespace exattn
