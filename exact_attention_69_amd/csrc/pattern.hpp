// Sparse attention patterns: the union of a sliding window, global tokens
// (whole rows and columns) and a block layout (llmis.ru chapter 3.1, section
// 3: Longformer's window and global tokens, BigBird's local, global and
// random blocks).  Row i sees key j when
//   (window >= 0 and |i - j| <= window) or i is global or j is global
//   or layout[i / 64][j / 64] is set.
//
// A plan step turns the pattern into, for every workgroup of a kernel, the
// list of tiles it must visit for the positions it stores.  Full positions
// (below) are left out on both sides: the workgroup's own are written by a
// pass of their own, and those of the other side are gathered into tiles that
// every workgroup visits before its list, so a listed tile only serves band
// and layout pairs.  Each entry is
//   bits 10..31 tile index
//   bit  9      the tile holds a full position of the other side (masked
//               out of it)
//   bits 1..8   per wave: the layout covers this wave's 32 rows (or keys)
//               for the whole tile
//   bit  0      partial: some pair of the tile is not visible, or the tile
//               holds a full position of the other side, or it crosses the
//               end of the sequence, so the kernel applies the element mask;
//               otherwise every pair is visible.
// Tiles with no band or layout pair of a stored position are not listed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exattn {

constexpr int kLayoutBlock = 64;
constexpr int kEntryTileShift = 10;
constexpr int kEntryHasFull = 1 << 9;
// Extra zero words after the bitmap, so that reads for rows or keys of a
// workgroup that runs past the end of the sequence stay in the allocation.
constexpr int kBitmapPadWords = 16;

__host__ __device__ inline int bitmap_words(int n) { return (n + 31) / 32 + kBitmapPadWords; }

// What a kernel needs at run time.
struct PatternDev {
  int window;                  // -1: no band term
  const uint32_t* own_full;    // full positions of the side a workgroup owns
                               // (rows, or keys for the key-side pass): not
                               // stored, the full-position pass writes them
  const uint32_t* other_full;  // full positions of the other side: visited
                               // first, gathered into tiles of their own, and
                               // masked out of the listed tiles
  const int* other_idx;        // those positions, ascending
  const int* other_count;      // their number (one int)
  const int* list;             // entries, `stride` per workgroup row of the grid
  const int* count;            // number of entries per workgroup row (-1: the
                               // row's own positions are all full: no work)
  int stride;
  // The other side's full positions copied to slots [head][0, count) (head
  // stride n rows), so that a gathered tile loads like a contiguous one:
  // key-side pass: the full rows' Q, dO (a, b), LSE*log2(e) and D (s0, s1);
  // forward and query-side pass: the full keys' K, V (a, b).
  const __bf16* gath_a;
  const __bf16* gath_b;
  const float* gath_s0;
  const float* gath_s1;
};

// Full positions: a query row that sees every key (a global token, or a row
// whose layout row is set in every block), or a key that every query sees
// (a global token, or a key whose layout column is set in every block).  A
// workgroup holding one would have to visit every tile of the other side, so
// they get a pass of their own: workgroups of kFullRows gathered positions,
// each over one chunk of the other side's tiles, with the chunks' partial
// results merged afterwards (rows: the two-block log-sum-exp merge; keys and
// dQ: a sum in chunk order).
constexpr int kFullRows = 128;
constexpr int kFullChunkTiles = 16;  // target tiles per chunk

// Per consumer kernel, written by the plan: [0] number of full positions R,
// [1] workgroups of positions G = ceil(R / kFullRows), [2] chunks C,
// [3] tiles per chunk.  G * C never exceeds ceil(n / kFullRows), the
// workgroups per head a full-position launch provides (spare ones return).
enum FullInfo : int { kFullCount = 0, kFullGroups = 1, kFullChunks = 2, kFullTilesPerChunk = 3, kFullInfoInts = 4 };

struct FullDev {
  const int* idx;   // full positions, ascending
  const int* info;  // FullInfo
  float* part;      // partial results (used when C > 1)
  float* part_lse;  // forward only: partial log-sum-exp
};

// Partial-result slots per head: at most a quarter of n (rounded up to whole
// workgroups); with more full positions than that, C = 1 and no partials.
__host__ __device__ inline int full_part_rows(int n) {
  const int q = (n + 3) / 4;
  return (q + kFullRows - 1) / kFullRows * kFullRows;
}

// One list to build: workgroups own `R` consecutive positions (queries, or
// keys when `transposed`), tiles span `T` positions of the other side, `NW`
// waves of 32 positions per workgroup.  `tail_partial` marks a tile that
// crosses the end of the sequence as partial.
struct PlanList {
  int R, T, NW;
  bool transposed;
  bool tail_partial;
  const uint32_t* own_full;    // full positions of the owned side: they drive no tile
  const uint32_t* other_full;  // full positions of the other side: gathered, not listed
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
  uint32_t* row_full;           // full query rows (bitmap)
  uint32_t* col_full;           // full keys (bitmap)
  int* layout_flags;            // [layout_n] rows set in every block, [layout_n] columns
  int* row_idx;                 // full rows, ascending (n ints)
  int* col_idx;                 // full keys, ascending (n ints)
  int* counts;                  // [0] full rows, [1] full keys
};

// How one consumer kernel splits its full positions: `tiles` tiles of the
// other side; the chosen G, C and tiles per chunk go to `info`.
struct FullSplit {
  int tiles;
  bool keys;  // over the full keys (else the full rows)
  int* info;
};

hipError_t launch_pattern_bitmap(const PlanInput& in, const FullSplit* splits, int n_splits, hipStream_t stream);
hipError_t launch_pattern_list(const PlanInput& in, const PlanList& pl, hipStream_t stream);
// Copies the other side's full positions of every head into the gather
// slots of `pat`: rows of a and b (bf16, d wide) and, when s0 is not null,
// the values of s0 and s1 (heads of n rows each).
hipError_t launch_pattern_gather(const PatternDev& pat, const __bf16* a, const __bf16* b, const float* s0,
                                 const float* s1, int heads, int n, int d, hipStream_t stream);

// Element visibility on a partial tile, given the per-row and per-key terms.
__device__ __forceinline__ bool bit_of(const uint32_t* bits, int pos) { return (bits[pos >> 5] >> (pos & 31)) & 1u; }

}  // namespace exattn
