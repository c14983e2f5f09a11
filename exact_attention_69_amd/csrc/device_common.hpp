// Device helpers shared by the attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// One 32x32x16 bf16 matrix-core product, fp32 accumulate.
//   a: lane l holds A[l % 32][8*(l/32) .. +8]   (row of A, 8 consecutive k)
//   b: lane l holds B[8*(l/32) .. +8][l % 32]   (column of B, 8 consecutive k)
//   c: lane l holds C[8*(r/4) + 4*(l/32) + r%4][l % 32] in element r.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (r) of the 32x32 accumulator tile that element r of lane l holds.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// A copy of a lane-dependent value that the compiler must treat as new on
// every evaluation (an empty asm that claims to modify it).  LDS addresses
// derived from it inside a loop are then recomputed where they are used
// rather than hoisted and kept live across the loop: a VALU op per address
// instead of a register per address.
__device__ __forceinline__ int opaque_lane_value(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The lane index (0-63), computed afresh (v_mbcnt) at every use, so that no
// register holds it across a loop.
__device__ __forceinline__ int fresh_lane_id() {
  int x;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Exchange a value with the lane 32 positions away (the other half-wave).
__device__ __forceinline__ float swap_half(float x) {
  return __shfl_xor(x, 32, 64);
}

// max / sum of x over the lane pair (l, l^32), with v_permlane32_swap (a
// VALU op; no LDS round trip).  The swap leaves lanes 0-31 of the first
// result and 32-63 of the second holding their own value, the others the
// partner's, so combining both results covers the pair on every lane.
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Instruction-scheduling hints (LLVM sched_group_barrier masks).
enum : int { kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedVMEMRead = 0x020, kSchedDSRead = 0x100,
             kSchedDSWrite = 0x200 };
#define EXATTN_SCHED(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane L receives element L%4 of the 8-byte chunk addressed by lane 4k + L/4,
// in its element k (k = 0..3).
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// LDS tiles of [rows][D] bf16, stored in 16-byte chunks (8 elements) whose
// index is XOR-swizzled per row.  Two read patterns must be conflict-free:
//   * 16-byte row reads, one row per lane (MFMA operand with k along d);
//   * transpose reads, 4 consecutive rows x 4 consecutive chunks per
//     16 lanes (MFMA operand with k along the rows).
// For D >= 128 a row spans the 64 banks; the swizzle value is a bijection of
// row % 16 whose bits 2-3 are row % 4, so 16 consecutive rows hit 16 distinct
// chunk slots and 4 consecutive rows x 4 chunks do too.  For D = 64 two rows
// share the 256-byte bank window and the same idea is applied to row / 2.
template <int D>
__device__ __forceinline__ int swz_chunk(int row, int c) {
  if constexpr (D == 64) return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  else return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int swz_off(int row, int col) {
  return row * D + 8 * swz_chunk<D>(row, col >> 3) + (col & 7);
}

// Global -> registers -> swizzled LDS copy of a ROWS x D bf16 tile by NT
// threads; rows at or beyond `valid` are filled with zeros.
template <int D, int ROWS, int NT>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int IT = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
  u32x4 st[IT];
  __device__ __forceinline__ void load(const __bf16* __restrict__ src, int valid, int tid) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int ch = tid + it * NT;
      const int row = ch / CPR, c = ch % CPR;
      st[it] = row < valid ? *(const u32x4*)(src + (size_t)row * D + 8 * c) : u32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(__bf16* lds, int tid) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int ch = tid + it * NT;
      const int row = ch / CPR, c = ch % CPR;
      *(u32x4*)(lds + row * D + 8 * swz_chunk<D>(row, c)) = st[it];
    }
  }
};

// One direct global -> LDS copy (global_load_lds_dwordx4): lane i's 16 bytes
// at `gsrc` land at LDS address `lds_wave_base` + 16*i (base wave-uniform).
// Issued through inline asm so that the compiler does not treat the copy as
// an LDS store it must wait for before every later LDS read (it cannot tell
// that the reads address other buffers); the callers wait explicitly
// (wait_all_and_barrier) before any wave reads the filled buffer.  Nothing
// else in the loops that use it touches vector memory.
__device__ __forceinline__ void lds_dma16(const void* gsrc, const void* lds_wave_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// As lds_dma16, with a wave-uniform global base address (held in scalar
// registers) and a per-lane 32-bit byte offset from it: a copy then needs no
// 64-bit address arithmetic on the vector ALU.
__device__ __forceinline__ void lds_dma16_sb(const void* gbase, uint32_t voff, const void* lds_wave_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// 4-byte variant (global_load_lds_dword): lane i's 4 bytes land at
// `lds_wave_base` + 4*i.
__device__ __forceinline__ void lds_dma4(const void* gsrc, const void* lds_wave_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// Direct global -> LDS copy of a ROWS x D bf16 tile into the swizzled layout
// (global_load_lds_dwordx4: lane i of a wave writes the 16 bytes at LDS
// base + 16*i, so each lane fetches the logical chunk that belongs in its
// slot; the XOR swizzle is its own inverse).  No registers are staged; the
// data is in LDS once vmcnt drains.  Rows at or beyond `valid` (>= 1) re-read
// row valid-1, so the caller must mask those rows out of every result.
template <int D, int ROWS, int NT>
struct TileAsync {
  static constexpr int CPR = D / 8;
  static constexpr int IT = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
  static __device__ __forceinline__ void issue(const __bf16* __restrict__ src, int valid, __bf16* lds, int tid) {
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int slot0 = it * NT + wave * 64;  // first chunk slot of this wave
      const int p = slot0 + lane;
      const int row = p / CPR;
      const int c = swz_chunk<D>(row, p % CPR);
      const int srow = row < valid ? row : valid - 1;
      lds_dma16(src + (size_t)srow * D + 8 * c, lds + 8 * slot0);
    }
  }
};

// TileAsync with the per-thread chunk offsets computed once (off[], a few
// registers) and a scalar tile base: a full tile costs no vector ALU work per
// copy; the tile that crosses the end of the sequence recomputes its offsets
// with the rows at or beyond `valid` clamped to row valid-1 (the caller masks
// them out of every result).  `wave` must be wave-uniform.
template <int D, int ROWS, int NT>
struct TileDma {
  static constexpr int CPR = D / 8;
  static constexpr int IT = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
  // byte offset of the chunk copy `it` of thread `tid` brings, read from row `src_row`
  static __device__ __forceinline__ uint32_t chunk_off(int it, int tid, int src_row) {
    const int p = it * NT + tid, row = p / CPR;
    return (uint32_t)(src_row * D + 8 * swz_chunk<D>(row, p % CPR)) * 2u;
  }
  static __device__ __forceinline__ void init(int tid, uint32_t (&off)[IT]) {
#pragma unroll
    for (int it = 0; it < IT; ++it) off[it] = chunk_off(it, tid, (it * NT + tid) / CPR);
  }
  static __device__ __forceinline__ void issue(const __bf16* base, const uint32_t (&off)[IT], __bf16* lds, int wave) {
#pragma unroll
    for (int it = 0; it < IT; ++it) lds_dma16_sb(base, off[it], lds + 8 * (it * NT + wave * 64));
  }
  static __device__ __forceinline__ void issue_tail(const __bf16* base, int valid, __bf16* lds, int tid, int wave) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int row = (it * NT + tid) / CPR;
      lds_dma16_sb(base, chunk_off(it, tid, row < valid ? row : valid - 1), lds + 8 * (it * NT + wave * 64));
    }
  }
};

// Constant sources for the direct copies of tile rows past the end of the
// sequence: a row of zeros (any head dim up to 256) and +infinity.
__device__ const __bf16 kZeroRow[256] = {};
__device__ const float kPosInf = __builtin_huge_valf();

// As TileAsync, but rows at or beyond `valid` are copied from kZeroRow, so
// they hold exact zeros in LDS.
template <int D, int ROWS, int NT>
struct TileAsyncZeroTail {
  static_assert(D <= 256, "kZeroRow holds 256 elements");
  static constexpr int CPR = D / 8;
  static constexpr int IT = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
  static __device__ __forceinline__ void issue(const __bf16* __restrict__ src, int valid, __bf16* lds, int tid) {
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int slot0 = it * NT + wave * 64;
      const int p = slot0 + lane;
      const int row = p / CPR;
      const int c = swz_chunk<D>(row, p % CPR);
      lds_dma16(row < valid ? (const void*)(src + (size_t)row * D + 8 * c) : (const void*)(kZeroRow + 8 * c),
                lds + 8 * slot0);
    }
  }
};

// As TileAsync, but tile row r comes from row rows[r] of `src`; rows at or
// beyond `valid` are copied from kZeroRow (no index is read for them).
template <int D, int ROWS, int NT>
struct TileAsyncRows {
  static_assert(D <= 256, "kZeroRow holds 256 elements");
  static constexpr int CPR = D / 8;
  static constexpr int IT = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
  static __device__ __forceinline__ void issue(const __bf16* __restrict__ src, const int* __restrict__ rows, int valid,
                                               __bf16* lds, int tid) {
    const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int slot0 = it * NT + wave * 64;
      const int p = slot0 + lane;
      const int row = p / CPR;
      const int c = swz_chunk<D>(row, p % CPR);
      lds_dma16(row < valid ? (const void*)(src + (size_t)rows[row] * D + 8 * c) : (const void*)(kZeroRow + 8 * c),
                lds + 8 * slot0);
    }
  }
};

// Wait for every outstanding memory operation of this wave (including direct
// global -> LDS copies), then synchronise the workgroup.
__device__ __forceinline__ void wait_all_and_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Debug build with EXATTN_POISON_LDS defined: a kernel first fills its LDS
// arrays with 0xFF bytes (a NaN in bf16, fp32 and fp8 e4m3 alike, -1 in an
// int), then synchronises, so that a read of LDS that no copy or store of the
// kernel wrote before it turns into NaN (or a wrong index) in the results.
// Called at the top of the kernel, where every thread of the workgroup is
// still present.  Without the macro it does nothing.
template <typename T>
__device__ __forceinline__ void poison_one(T& arr) {
  static_assert(sizeof(T) % 4 == 0, "LDS arrays are filled a word at a time");
  uint32_t* p = reinterpret_cast<uint32_t*>(&arr);
  for (int i = (int)threadIdx.x; i < (int)(sizeof(T) / 4); i += (int)blockDim.x) p[i] = 0xffffffffu;
}
template <typename... T>
__device__ __forceinline__ void poison_lds(T&... arrs) {
#ifdef EXATTN_POISON_LDS
  (poison_one(arrs), ...);
  __syncthreads();
#else
  ((void)arrs, ...);
#endif
}

// MFMA operand with k along d: lane reads 8 consecutive columns
// [16*ds + 8*(lane/32), +8) of tile row `row`.
template <int D>
__device__ __forceinline__ bf16x8 lds_row_frag(const __bf16* tile, int row, int ds, int hi) {
  return *(const bf16x8*)(tile + row * D + 8 * swz_chunk<D>(row, 2 * ds + hi));
}

// MFMA operand with k along the tile rows (transposed operand): for output
// columns [col0, col0+32) (one per lane % 32) returns the 8 values at rows
//   r0 + 8*(t/4) + 4*(lane/32) + t%4,  t = 0..7,
// which is the k order of a 32x32 accumulator's rows r0 .. r0+15 when they
// are reused as an operand (see acc_row).
template <int D>
__device__ __forceinline__ bf16x8 lds_col_frag(const __bf16* tile, int r0, int col0, int lane) {
  const int g = lane >> 4, L = lane & 15, hi = lane >> 5;
  const int col = col0 + 16 * (g & 1) + 4 * (L & 3);
  const int row = r0 + 4 * hi + (L >> 2);
  const bf16x4 a = lds_read_tr16(tile + swz_off<D>(row, col));
  const bf16x4 b = lds_read_tr16(tile + swz_off<D>(row + 8, col));
  return cat8(a, b);
}

// Reuse accumulator elements [8*half, 8*half+8) as a bf16 MFMA operand with
// k along the accumulator's rows (rows 16*half .. 16*half+15 in acc_row order).
__device__ __forceinline__ bf16x8 acc_to_operand(const f32x16& c, int half) {
  u32x4 w;
#pragma unroll
  for (int t = 0; t < 4; ++t) w[t] = pack_bf16x2(c[8 * half + 2 * t], c[8 * half + 2 * t + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

// XCD-aware block order: consecutive workgroup ids are dealt out to the 8
// XCDs in turn; remap so that each XCD owns a contiguous range of logical
// tiles, and the tiles of one head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  return (total & 7) == 0 ? (bid & 7) * (total >> 3) + (bid >> 3) : bid;
}

}  // namespace exattn
