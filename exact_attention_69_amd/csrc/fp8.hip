// FP8 (OCP E4M3) attention forward for gfx950, and the quantiser that feeds
// it: FlashAttention-3's FP8 computation and "incoherent processing" (the
// unite.ai page "Flash Attention: Revolucionando a Eficiencia dos Modelos
// Transformer", section "FlashAttention-3", items 2 and 3).
//
// Quantiser (per (batch, head) and tensor):
//   optional rotation x <- (x * signs) H, H the Sylvester Hadamard matrix
//   (a fast Walsh-Hadamard transform of additions and subtractions, stages
//   h = 1, 2, 4, ...), then scale = amax / 448 and code = e4m3(clamp(x *
//   (448 / amax), +-448)).  Rotating Q and K by the same matrix multiplies
//   Q K^T by d, which the forward divides out; it spreads outlier columns
//   so the per-head scale is not set by a few large values.
// Forward: S = scale / d_rot * s_q s_k * Q8 K8^T (32x32x64 FP8 MFMA, fp32
// accumulation), online softmax in fp32 as in the bf16 kernel, P rounded
// to E4M3 (values <= 2^8 by the lazy rescaling), O = s_v * P V8 / l in bf16.
//
// V is stored transposed, [B, H, d, n128] with n128 = n rounded up to 128,
// and within every 64-key group the keys are permuted so that the 32 keys
// a lane holds in its score accumulator (rows 8a + 4h + c, a, c = 0..3, of
// each of two 32-key blocks) form one contiguous 32-byte MFMA operand:
//   key 32*kb + 8*a + 4*h + c  ->  column 32*h + 16*kb + 4*a + c.
// Columns at or beyond n hold zeros.
#include "device_common.hpp"
#include "launch.hpp"

namespace exattn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // cbsz = blgp = 0: both operands E4M3; unit block scales (exponent 127)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four E4M3 codes (ties to even) packed into one dword, a in byte 0.
__device__ __forceinline__ int pack_e4m3x4(float a, float b, float c, float d) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Column of key `k` (within its 64-key group) in the transposed V layout.
__host__ __device__ inline int vt_column(int k) {
  const int g = k >> 6, r = k & 63;
  const int kb = r >> 5, a = (r >> 3) & 3, h = (r >> 2) & 1, c = r & 3;
  return (g << 6) + 32 * h + 16 * kb + 4 * a + c;
}

// ---------------------------------------------------------------------------
// Quantiser
// ---------------------------------------------------------------------------
// Rows in the row-group layout: the G = D/8 consecutive lanes of a group
// hold one row, 8 consecutive elements each (element i = 8*l + j,
// l = lane % G): one 16-byte load per lane.  The rotation's butterfly stages
// run in the order h = 1, 2, 4 (within the lane), then h = 8 .. D/2 (across
// the group's lanes, by shuffles); each stage forms lower + upper and
// lower - upper of its pairs.
// x of the lane whose index differs from this lane's in bit log2(M) (M = 1,
// 2, 4, 8: within a row of 16 lanes), by DPP moves (vector ALU, no LDS):
// XOR 1 and 2 are quad permutations; XOR 4 = XOR 3 (reverse the quad) then
// the mirror of each 8 lanes (XOR 7); XOR 8 = XOR 7 then the mirror of the
// row of 16 (15 - i).
template <int M>
__device__ __forceinline__ float lanes_xor(float x) {
  constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kQuadRev = 0x1B, kHalfMirror = 0x141, kMirror = 0x140;
  int v = __builtin_bit_cast(int, x);
  if constexpr (M == 1) {
    v = __builtin_amdgcn_mov_dpp(v, kQuadXor1, 0xF, 0xF, true);
  } else if constexpr (M == 2) {
    v = __builtin_amdgcn_mov_dpp(v, kQuadXor2, 0xF, 0xF, true);
  } else if constexpr (M == 4) {
    v = __builtin_amdgcn_mov_dpp(v, kQuadRev, 0xF, 0xF, true);
    v = __builtin_amdgcn_mov_dpp(v, kHalfMirror, 0xF, 0xF, true);
  } else {
    static_assert(M == 8, "partners within a row of 16 lanes");
    v = __builtin_amdgcn_mov_dpp(v, kHalfMirror, 0xF, 0xF, true);
    v = __builtin_amdgcn_mov_dpp(v, kMirror, 0xF, 0xF, true);
  }
  return __builtin_bit_cast(float, v);
}

template <int D, int M>
__device__ __forceinline__ void butterfly_across(float (&x)[8], int l) {
  // lower lane: x + b; upper lane: b - x; one fma with a sign, exact
  // before its one rounding, so the same value as the add or subtract
  const float sg = (l & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = __builtin_fmaf(sg, x[j], lanes_xor<M>(x[j]));
  if constexpr (8 * 2 * M < D) butterfly_across<D, 2 * M>(x, l);
}

template <int D>
__device__ __forceinline__ void rotate_row8(const u32x4& w, const float* __restrict__ signs, int l, float (&x)[8]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    x[2 * t] = __builtin_bit_cast(float, w[t] << 16);
    x[2 * t + 1] = __builtin_bit_cast(float, w[t] & 0xffff0000u);
  }
  if (signs == nullptr) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] *= signs[8 * l + j];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & h) == 0) {
        const float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
  butterfly_across<D, 1>(x, l);  // h = 8, 16, .., D/2: partner lane l ^ (h/8)
}

template <int D>
__device__ __forceinline__ void load_rotated_row8(const __bf16* __restrict__ row, const float* __restrict__ signs,
                                                  int l, float (&x)[8]) {
  rotate_row8<D>(*(const u32x4*)(row + 8 * l), signs, l, x);
}

__global__ __launch_bounds__(256) void quant_clear_kernel(uint32_t* __restrict__ amax_bits, int heads) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < heads) amax_bits[i] = 0u;
}

// amax of every head: |x| as uint bits (monotonic for non-negative floats).
// A workgroup reduces kAmaxRows rows of one head in registers, then across
// its waves in LDS, and issues one atomic max: a head's rows meet at one
// address n / kAmaxRows times.  (Atomics on one address are served one after
// another, about half a microsecond each: 64 rows per workgroup took
// 0.075 ms for a 128 MiB tensor, 512 take a fraction of that.)
constexpr int kAmaxRows = 512;

constexpr int kAmaxWaves = 16;  // waves per workgroup: enough of them to cover the rotation's latencies

template <int D>
__global__ __launch_bounds__(kAmaxWaves * 64) void quant_amax_kernel(const __bf16* __restrict__ X,
                                                                     const float* __restrict__ signs,
                                                                     uint32_t* __restrict__ amax_bits, int n,
                                                                     int chunks) {
  constexpr int G = D / 8, RPW = 64 / G, NW = kAmaxWaves;  // lanes per row, rows per wave
  __shared__ float wave_max[NW];
  poison_lds(wave_max);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long head = blockIdx.x / chunks;
  const int r0 = (int)(blockIdx.x - head * chunks) * kAmaxRows;
  const int r1 = min(r0 + kAmaxRows, n);
  float m = 0.0f;
  // Batches of BATCH passes; in pass p a lane takes row
  // r0 + wave*RPW + lane/G + NW*RPW*p.  A batch's rows are all loaded before
  // any is processed (every lane of a row group takes the same rows, so the
  // group's shuffles stay among active lanes; rows past r1 read as zeros,
  // which leave the max alone).
  constexpr int BATCH = kAmaxRows / (NW * RPW) < 8 ? kAmaxRows / (NW * RPW) : 8, PER_BATCH = NW * RPW * BATCH;
  static_assert(kAmaxRows % PER_BATCH == 0, "whole batches per workgroup");
  const int l = lane % G;
  for (int b0 = r0; b0 < r1; b0 += PER_BATCH) {
    u32x4 raw[BATCH];
#pragma unroll
    for (int p = 0; p < BATCH; ++p) {
      const int r = b0 + wave * RPW + lane / G + NW * RPW * p;
      raw[p] = r < r1 ? *(const u32x4*)(X + (head * n + r) * D + 8 * l) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int p = 0; p < BATCH; ++p) {
      float x[8];
      rotate_row8<D>(raw[p], signs, l, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if (lane == 0) wave_max[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float w = wave_max[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) w = fmaxf(w, wave_max[i]);
    atomicMax(&amax_bits[head], __float_as_uint(w));
  }
}

// Codes of the row layout, in the row-group layout: each lane converts and
// stores its 8 codes as one 8-byte word.
template <int D>
__global__ __launch_bounds__(256) void quant_codes_rows_kernel(const __bf16* __restrict__ X,
                                                              const float* __restrict__ signs,
                                                              const uint32_t* __restrict__ amax_bits,
                                                              uint8_t* __restrict__ X8, int n, long rows) {
  constexpr int G = D / 8, RPB = 256 / G;  // lanes per row, rows per workgroup
  const int l = threadIdx.x % G;
  const long prow = (long)blockIdx.x * RPB + threadIdx.x / G;  // row in [heads * n)
  if (prow >= rows) return;  // whole row groups (G divides 64)
  const long head = prow / n;
  float x[8];
  load_rotated_row8<D>(X + prow * D, signs, l, x);
  const float amax = __uint_as_float(amax_bits[head]);
  const float inv = amax > 0.0f ? kE4M3Max / amax : 0.0f;
  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) q[j] = fminf(fmaxf(x[j] * inv, -kE4M3Max), kE4M3Max);
  u32x2 w;
  w[0] = (uint32_t)pack_e4m3x4(q[0], q[1], q[2], q[3]);
  w[1] = (uint32_t)pack_e4m3x4(q[4], q[5], q[6], q[7]);
  *(u32x2*)(X8 + prow * D + 8 * l) = w;
}

// Codes of the transposed V layout: a workgroup takes one 64-key group of a
// head, converts its rows in the row-group layout, transposes the codes
// through LDS (row stride 68 bytes, so that the byte writes of a row
// group's lanes spread over the banks) and writes each of the D output rows'
// 64 columns as four 16-byte words.  Keys at or beyond n give zero columns.
template <int D>
__global__ __launch_bounds__(256) void quant_codes_t_kernel(const __bf16* __restrict__ X,
                                                           const float* __restrict__ signs,
                                                           const uint32_t* __restrict__ amax_bits,
                                                           uint8_t* __restrict__ X8, int n, int n128, int groups) {
  constexpr int G = D / 8, RPP = 256 / G;  // lanes per row, rows per pass
  constexpr int RS = 68;                  // LDS bytes per output row
  __shared__ __attribute__((aligned(16))) uint32_t t[D * RS / 4];
  poison_lds(t);
  const long head = blockIdx.x / groups;
  const int k0 = (int)(blockIdx.x - head * groups) * 64;
  const int tid = threadIdx.x, l = tid % G;
  const float amax = __uint_as_float(amax_bits[head]);
  const float inv = amax > 0.0f ? kE4M3Max / amax : 0.0f;
  uint8_t* tb = (uint8_t*)t;
#pragma unroll
  for (int p = 0; p < 64 / RPP; ++p) {
    const int k = k0 + p * RPP + tid / G;  // key (row of X); groups of G lanes share it
    float x[8];
    if (k < n) {
      load_rotated_row8<D>(X + (head * n + k) * D, signs, l, x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.0f;
    }
    const int c = vt_column(k - k0);  // column within the group
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q = fminf(fmaxf(x[j] * inv, -kE4M3Max), kE4M3Max);
      tb[(8 * l + j) * RS + c] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xff);
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < D * 4 / 256; ++q) {
    const int chunk = tid + 256 * q, i = chunk >> 2, part = chunk & 3;
    const uint32_t* src = t + (i * RS + 16 * part) / 4;
    *(u32x4*)(X8 + ((size_t)head * D + i) * n128 + k0 + 16 * part) = u32x4{src[0], src[1], src[2], src[3]};
  }
}

__global__ __launch_bounds__(256) void quant_scale_kernel(float* __restrict__ scale, int heads) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= heads) return;
  const float amax = scale[i];  // the amax bits left by quant_amax_kernel
  scale[i] = amax > 0.0f ? amax / kE4M3Max : 1.0f;
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
constexpr int kF8NW = 8;    // waves (256 query rows per workgroup)
constexpr int kF8BC = 128;  // keys per tile

// Chunk swizzle of a tile of RB-byte rows (16-byte chunks): 128-byte rows
// use the bf16 kernels' layout for 128-byte rows; 64-byte rows XOR the chunk
// with bits 1-2 of the row, so that eight consecutive rows reading the same
// logical chunk hit eight different 16-byte bank groups.
template <int RB>
__device__ __forceinline__ int swz8(int row, int c) {
  static_assert(RB == 64 || RB == 128, "rows of 64 or 128 bytes");
  if constexpr (RB == 128) return swz_chunk<64>(row, c);
  else return c ^ ((row >> 1) & 3);
}

// Direct global -> LDS copy of ROWS rows of RB bytes (global row stride
// `stride` bytes) into the swizzled layout.  Rows at or beyond `valid`
// re-read row valid-1.
template <int ROWS, int RB, int NT>
__device__ __forceinline__ void tile8_issue(const uint8_t* __restrict__ src, long stride, int valid, uint8_t* lds,
                                            int tid) {
  constexpr int CPR = RB / 16;
  constexpr int IT = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int slot0 = it * NT + wave * 64;
    const int p = slot0 + lane;
    const int row = p / CPR;
    const int c = swz8<RB>(row, p % CPR);
    const int srow = row < valid ? row : valid - 1;
    lds_dma16(src + (long)srow * stride + 16 * c, lds + 16 * slot0);
  }
}

// 32 contiguous bytes [32*j, 32*j + 32) of an RB-byte row of a swizzled tile.
template <int RB>
__device__ __forceinline__ i32x8 lds_frag32(const uint8_t* tile, int row, int j) {
  const u32x4 a = *(const u32x4*)(tile + row * RB + 16 * swz8<RB>(row, 2 * j));
  const u32x4 b = *(const u32x4*)(tile + row * RB + 16 * swz8<RB>(row, 2 * j + 1));
  i32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

template <int D>
__global__ __launch_bounds__(kF8NW * 64, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ V8t,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    __bf16* __restrict__ Og, float* __restrict__ LSEg, int n, int n128, int n_qblocks, int total_blocks,
    float scale_log2_base) {
  static_assert(D == 64 || D == 128, "the FP8 forward is built for d = 64 and 128");
  constexpr int NW = kF8NW, BC = kF8BC, BR = 32 * NW, NT = NW * 64;
  constexpr int NKB = BC / 32;  // 32-key blocks per tile
  constexpr int NDS = D / 64;   // 64-wide d steps of S
  constexpr int NDB = D / 32;   // 32-wide d blocks of O
  constexpr int NPS = BC / 64;  // 64-key steps of P V

  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint8_t vbuf[2][D * BC];
  poison_lds(kbuf, vbuf);

  const int bid = xcd_remap(blockIdx.x, total_blocks);
  const int head = bid / n_qblocks;
  const int qb = bid - head * n_qblocks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hi = lane >> 5;

  const uint8_t* K = K8 + (size_t)head * n * D;
  const uint8_t* Vt = V8t + (size_t)head * D * n128;
  const int my_row = qb * BR + wave * 32 + l32;
  const float scale_log2 = scale_log2_base * q_scale[head] * k_scale[head];

  // Q^T operand in registers: lane holds Q8[my_row][64*ds + 32*hi .. +32]
  i32x8 qreg[NDS];
  {
    const bool ok = my_row < n;
    const i32x8* src = (const i32x8*)(Q8 + ((size_t)head * n + (ok ? my_row : 0)) * D + 32 * hi);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      qreg[ds] = ok ? src[2 * ds] : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // K tile: BC rows of D bytes; V^T tile: D rows of BC bytes
  auto issue_k = [&](int t, uint8_t* buf) { tile8_issue<BC, D, NT>(K + (size_t)t * BC * D, D, n - t * BC, buf, tid); };
  auto issue_v = [&](int t, uint8_t* buf) { tile8_issue<D, BC, NT>(Vt + (size_t)t * BC, n128, D, buf, tid); };
  auto compute_s_block = [&](const uint8_t* Ks, int kb, f32x16 (&s)[NKB]) {
    s[kb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) s[kb] = mfma_f8(lds_frag32<D>(Ks, kb * 32 + l32, 2 * ds + hi), qreg[ds], s[kb]);
  };

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m_run = kNegInf, l_part = 0.0f;

  const int n_tiles = (n + BC - 1) / BC;
  if (n_tiles > 0) {
    issue_k(0, kbuf[0]);
    issue_v(0, vbuf[0]);
    if (n_tiles > 1) issue_k(1, kbuf[1]);
  }
  wait_all_and_barrier();
  f32x16 s_cur[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) compute_s_block(kbuf[0], kb, s_cur);
  // The first iteration copies tile 2's K rows over tile 0's: every wave must
  // have read tile 0's K rows for its scores first.
  wait_all_and_barrier();

  for (int j = 0; j < n_tiles; ++j) {
    if (j + 1 < n_tiles) issue_v(j + 1, vbuf[(j + 1) & 1]);
    if (j + 2 < n_tiles) issue_k(j + 2, kbuf[j & 1]);
    const int kbase = j * BC;
    if (kbase + BC > n) {  // key tail
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + kb * 32 + acc_row(r, lane);
          s_cur[kb][r] = key < n ? s_cur[kb][r] : kNegInf;
        }
    }
    // running max and (rare) rescale, as in the bf16 kernel
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[kb][r]);
    mx = pair_max(mx);
    const float mx2 = mx * scale_log2;
    const bool grow = mx2 > m_run + 8.0f || (m_run == kNegInf && mx2 != kNegInf);
    if (__any(grow)) {
      const float m_new = grow ? mx2 : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_run = m_new;
    }
    const float msub = m_run == kNegInf ? 0.0f : m_run;

    // P in E4M3, packed in the transposed V layout's key order: for P V step
    // ps (keys 64*ps ..), byte 16*kb' + r of the lane's operand is P of
    // accumulator element r of key block 2*ps + kb'.  Each converted block's
    // fp32 registers then receive that block of the next tile's S.
    i32x8 pb[NPS];
    float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s_cur[kb][r] = fast_exp2(__builtin_fmaf(s_cur[kb][r], scale_log2, -msub));
        lsum[r & 3] += s_cur[kb][r];
      }
#pragma unroll
      for (int w = 0; w < 4; ++w)
        pb[kb >> 1][4 * (kb & 1) + w] =
            pack_e4m3x4(s_cur[kb][4 * w], s_cur[kb][4 * w + 1], s_cur[kb][4 * w + 2], s_cur[kb][4 * w + 3]);
      compute_s_block(kbuf[(j + 1) & 1], kb, s_cur);
    }
    l_part += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);

    // O^T += V^T P^T: A = V^T rows (d) with 32 keys per lane, B = P^T.
    const uint8_t* Vs = vbuf[j & 1];
#pragma unroll
    for (int ps = 0; ps < NPS; ++ps)
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] = mfma_f8(lds_frag32<BC>(Vs, db * 32 + l32, 2 * ps + hi), pb[ps], o[db]);
    {  // each product's two LDS reads three products ahead (1.5% faster at
       // d=128, 6% at d=64; the compiler otherwise waits on them in turn)
      constexpr int NP = NPS * NDB, kLead = 3;
      EXATTN_SCHED(kSchedDSRead, 2 * kLead);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        EXATTN_SCHED(kSchedMFMA, 1);
        if (i + kLead < NP) EXATTN_SCHED(kSchedDSRead, 2);
      }
    }

    wait_all_and_barrier();
  }

  const float l_tot = pair_sum(l_part);
  if (my_row < n) {
    const float inv = v_scale[head] / l_tot;
    __bf16* Orow = Og + ((size_t)head * n + my_row) * D;
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
    if (hi == 0) LSEg[(size_t)head * n + my_row] = kLn2 * (m_run + fast_log2(l_tot));
  }
}

}  // namespace

int fp8_padded_n(int n) { return (n + kF8BC - 1) / kF8BC * kF8BC; }

hipError_t launch_quant_fp8(const Fp8QuantParams& p, hipStream_t stream) {
  if (p.d != 64 && p.d != 128) return hipErrorInvalidValue;
  const long heads = (long)p.B * p.H;
  const int chunks = (p.n + kAmaxRows - 1) / kAmaxRows;  // amax workgroups per head
  const int n128 = fp8_padded_n(p.n);
  const long code_rows = heads * (p.transposed ? n128 : p.n);
  // every grid (amax; codes: a 64-key group or 256 / (d/8) rows per
  // workgroup) checked before the first launch
  const long code_blocks = p.transposed ? heads * (n128 / 64) : (code_rows + 256 / (p.d / 8) - 1) / (256 / (p.d / 8));
  if (heads * chunks > 0x7fffffffL || code_blocks > 0x7fffffffL || heads > 0x7fffffffL) return hipErrorInvalidValue;
  uint32_t* amax = (uint32_t*)p.scale;
  hipLaunchKernelGGL(quant_clear_kernel, dim3((unsigned)((heads + 255) / 256)), dim3(256), 0, stream, amax,
                     (int)heads);
  switch (p.d) {
    case 64:
      hipLaunchKernelGGL((quant_amax_kernel<64>), dim3((unsigned)(heads * chunks)), dim3(kAmaxWaves * 64), 0, stream,
                         (const __bf16*)p.x, p.signs, amax, p.n, chunks);
      if (p.transposed)
        hipLaunchKernelGGL((quant_codes_t_kernel<64>), dim3((unsigned)code_blocks), dim3(256), 0, stream,
                           (const __bf16*)p.x, p.signs, amax, (uint8_t*)p.x8, p.n, n128, n128 / 64);
      else
        hipLaunchKernelGGL((quant_codes_rows_kernel<64>), dim3((unsigned)code_blocks), dim3(256), 0,
                           stream, (const __bf16*)p.x, p.signs, amax, (uint8_t*)p.x8, p.n, code_rows);
      break;
    case 128:
      hipLaunchKernelGGL((quant_amax_kernel<128>), dim3((unsigned)(heads * chunks)), dim3(kAmaxWaves * 64), 0, stream,
                         (const __bf16*)p.x, p.signs, amax, p.n, chunks);
      if (p.transposed)
        hipLaunchKernelGGL((quant_codes_t_kernel<128>), dim3((unsigned)code_blocks), dim3(256), 0, stream,
                           (const __bf16*)p.x, p.signs, amax, (uint8_t*)p.x8, p.n, n128, n128 / 64);
      else
        hipLaunchKernelGGL((quant_codes_rows_kernel<128>), dim3((unsigned)code_blocks), dim3(256), 0,
                           stream, (const __bf16*)p.x, p.signs, amax, (uint8_t*)p.x8, p.n, code_rows);
      break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(quant_scale_kernel, dim3((unsigned)((heads + 255) / 256)), dim3(256), 0, stream, p.scale,
                     (int)heads);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream) {
  if (p.d != 64 && p.d != 128) return hipErrorInvalidValue;
  constexpr int BR = 32 * kF8NW;
  const int nqb = (p.n + BR - 1) / BR;
  const long total = (long)nqb * p.B * p.H;
  if (total > 0x7fffffffL) return hipErrorInvalidValue;
  const float scale_log2 = p.scale / (p.rotated ? (float)p.d : 1.0f) * kLog2e;
  auto kernel = p.d == 64 ? fwd_fp8_kernel<64> : fwd_fp8_kernel<128>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)total), dim3(kF8NW * 64), 0, stream, (const uint8_t*)p.q8,
                     (const uint8_t*)p.k8, (const uint8_t*)p.v8t, p.q_scale, p.k_scale, p.v_scale, (__bf16*)p.o,
                     p.lse, p.n, fp8_padded_n(p.n), nqb, (int)total, scale_log2);
  return hipGetLastError();
}

}  // namespace exattn
