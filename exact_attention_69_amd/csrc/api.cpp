// C-ABI entry points: argument validation, workspace sizing and dispatch.
// Every check runs before the first HIP call, so a rejected call touches
// neither the device nor the stream.
#include "../../include/exattn.h"

#include <math.h>
#include <stdint.h>

#include "launch.hpp"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

size_t elem_bytes(int dtype) { return dtype == EXATTN_BF16 ? 2 : 4; }

// Shape/scalar checks common to both passes.
int check_problem(int dtype, int B, int H, int n, int d, float scale, int window) {
  if (B < 1 || H < 1 || n < 1) return EXATTN_EINVAL;
  if (window < -1) return EXATTN_EINVAL;
  if (!isfinite(scale) || !(scale > 0.0f)) return EXATTN_EINVAL;
  if (dtype != EXATTN_F32 && dtype != EXATTN_BF16) return EXATTN_EUNSUPPORTED;
  if (d != 64 && d != 128 && d != 256) return EXATTN_EUNSUPPORTED;
  long long elems = (long long)B * H * n * d;
  if (elems >= (1LL << 31)) return EXATTN_EINVAL;
  return EXATTN_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? EXATTN_OK : EXATTN_EHIP; }

}  // namespace

extern "C" {

const char* exattn_status_string(int status) {
  switch (status) {
    case EXATTN_OK: return "success";
    case EXATTN_EINVAL: return "invalid argument (null/misaligned/overlapping pointer, bad size, window or scale)";
    case EXATTN_EUNSUPPORTED: return "unsupported head dim or dtype (d must be 64, 128 or 256; dtype f32 or bf16)";
    case EXATTN_EWORKSPACE: return "workspace smaller than attn_bwd_workspace_bytes()";
    case EXATTN_EHIP: return "HIP runtime error at kernel launch";
    default: return "unknown status";
  }
}

int attn_fwd(int dtype, int B, int H, int n, int d, const void* Q, const void* K, const void* V,
             float scale, int window, void* O, float* LSE, void* stream) {
  int st = check_problem(dtype, B, H, n, d, scale, window);
  if (st != EXATTN_OK) return st;
  const void* ptrs[] = {Q, K, V, O, LSE};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return EXATTN_EINVAL;
  size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  size_t lb = (size_t)B * H * n * sizeof(float);
  const void* ins[] = {Q, K, V};
  for (const void* in : ins) {
    if (overlaps(O, tb, in, tb) || overlaps(LSE, lb, in, tb)) return EXATTN_EINVAL;
  }
  if (overlaps(O, tb, LSE, lb)) return EXATTN_EINVAL;

  exattn::FwdParams p{Q, K, V, O, LSE, B, H, n, d, scale, window};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == EXATTN_BF16 ? exattn::launch_fwd_bf16(p, s) : exattn::launch_fwd_f32(p, s);
  return from_hip(e);
}

size_t attn_bwd_workspace_bytes(int dtype, int B, int H, int n, int d) {
  if (check_problem(dtype, B, H, n, d, 1.0f, -1) != EXATTN_OK) return 0;
  size_t rows = (size_t)B * H * n;
  return ((rows * sizeof(float) + 255) / 256) * 256;
}

int attn_bwd(int dtype, int B, int H, int n, int d, const void* Q, const void* K, const void* V,
             const void* O, const void* dO, const float* LSE, float scale, int window, void* dQ,
             void* dK, void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(dtype, B, H, n, d, scale, window);
  if (st != EXATTN_OK) return st;
  const void* ptrs[] = {Q, K, V, O, dO, LSE, dQ, dK, dV, workspace};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return EXATTN_EINVAL;
  size_t need = attn_bwd_workspace_bytes(dtype, B, H, n, d);
  if (workspace_bytes < need) return EXATTN_EWORKSPACE;

  size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  size_t lb = (size_t)B * H * n * sizeof(float);
  struct Span { const void* p; size_t n; };
  Span ins[] = {{Q, tb}, {K, tb}, {V, tb}, {O, tb}, {dO, tb}, {LSE, lb}};
  Span outs[] = {{dQ, tb}, {dK, tb}, {dV, tb}, {workspace, need}};
  for (const Span& o : outs) {
    for (const Span& i : ins)
      if (overlaps(o.p, o.n, i.p, i.n)) return EXATTN_EINVAL;
  }
  for (int a = 0; a < 4; ++a)
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n)) return EXATTN_EINVAL;

  exattn::BwdParams p{Q, K, V, O, dO, LSE, dQ, dK, dV, (float*)workspace, B, H, n, d, scale, window};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == EXATTN_BF16 ? exattn::launch_bwd_bf16(p, s) : exattn::launch_bwd_f32(p, s);
  return from_hip(e);
}

}  // extern "C"
