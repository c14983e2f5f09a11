// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pattern.hpp"

namespace exattn {

// Masking modes of the kernels.
// kMaskFull: the full positions of a pattern (rows or keys gathered from the
// plan's list), each workgroup over one chunk of the other side's tiles.
enum MaskMode : int { kMaskNone = 0, kMaskWindow = 1, kMaskPattern = 2, kMaskFull = 3 };

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, n, d;
  float scale;
  int window;  // -1: no mask
  int group;   // query heads per key/value head: K, V are [B, H / group, n, d]
  PatternDev pattern;  // list == nullptr: no pattern
  FullDev full;        // with a pattern: its full rows (idx == nullptr: none)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace: [B, H, n] fp32, D = rowsum(dO * O)
  float* lse2;   // workspace: [B, H, n] fp32, LSE * log2(e)
  int B, H, n, d;
  float scale;
  int window;
  int group;  // query heads per key/value head: K, V, dK, dV are [B, H / group, n, d]
  PatternDev pattern_kv;  // lists for the key-side pass (list == nullptr: no pattern)
  PatternDev pattern_q;   // lists for the query-side pass
  FullDev full_kv;        // with a pattern: its full keys
  FullDev full_q;         // with a pattern: its full rows
};

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
// The part of launch_fwd_bf16 for d = 128 without a mask and d = 256 with a
// window, without a pattern (a translation unit of its own).
hipError_t launch_fwd_bf16_ilp(const FwdParams& p, hipStream_t stream);
// Workgroup geometry of the bf16 kernels in pattern mode, for the pattern plan.
void fwd_bf16_geometry(int d, int* rows_per_block, int* keys_per_tile, int* waves);
void bwd_kv_bf16_geometry(int d, int* keys_per_block, int* rows_per_tile, int* waves);
void bwd_q_bf16_geometry(int d, int* rows_per_block, int* keys_per_tile, int* waves);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
// Backward stages: rowdot (D), key side (dK, dV), query side (dQ).
enum BwdStage : unsigned { kStageRowdot = 1, kStageKV = 2, kStageQ = 4, kStageAll = 7 };
hipError_t launch_bwd_bf16(const BwdParams& p, unsigned stages, hipStream_t stream);
// The part of launch_bwd_bf16 for d = 128 without a mask (a translation unit
// of its own).
hipError_t launch_bwd_bf16_d128(const BwdParams& p, unsigned stages, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdParams& p, unsigned stages, hipStream_t stream);

// FP8: per-head quantiser (optional Hadamard rotation) and the forward.
struct Fp8QuantParams {
  int B, H, n, d;
  const void* x;       // bf16 [B, H, n, d]
  const float* signs;  // d signs (+-1) of the rotation, or nullptr
  void* x8;            // E4M3 codes: [B, H, n, d], or the transposed V layout
  float* scale;        // [B, H]
  int transposed;
};
struct Fp8FwdParams {
  int B, H, n, d;
  const void* q8;
  const void* k8;
  const void* v8t;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  float scale;
  int rotated;
  void* o;
  float* lse;
};
int fp8_padded_n(int n);
hipError_t launch_quant_fp8(const Fp8QuantParams& p, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream);

// Band of the sliding window, used to skip tiles (host and device).
// Keys [lo, hi) that any row in [r0, r1) may attend to.
__host__ __device__ inline void band_keys(int r0, int r1, int n, int window, int* lo, int* hi) {
  if (window < 0) {
    *lo = 0;
    *hi = n;
    return;
  }
  long a = (long)r0 - window, b = (long)r1 - 1 + window + 1;
  *lo = a < 0 ? 0 : (int)a;
  *hi = b > n ? n : (int)b;
}

}  // namespace exattn
