// C-ABI entry points: argument validation, workspace sizing and dispatch.
// Every check runs before the first HIP call, so a rejected call touches
// neither the device nor the stream.
#include "../../include/exattn.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

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
int check_problem(int dtype, int B, int H, int n, int d, float scale, int window, int Hkv) {
  if (B < 1 || H < 1 || n < 1) return EXATTN_EINVAL;
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return EXATTN_EINVAL;
  if (window < -1) return EXATTN_EINVAL;
  if (!isfinite(scale) || !(scale > 0.0f)) return EXATTN_EINVAL;
  if (dtype != EXATTN_F32 && dtype != EXATTN_BF16) return EXATTN_EUNSUPPORTED;
  if (d != 64 && d != 128 && d != 256) return EXATTN_EUNSUPPORTED;
  // Row indices (b, h, i) -> (b*H + h)*n + i are 32-bit in the kernels;
  // element offsets (row * d) are 64-bit, so a tensor may exceed 2^31
  // elements.
  long long rows = (long long)B * H * n;
  if (rows >= (1LL << 31)) return EXATTN_EINVAL;
  return EXATTN_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? EXATTN_OK : EXATTN_EHIP; }

struct Span {
  const void* p;
  size_t n;
};

}  // namespace

extern "C" {

const char* exattn_status_string(int status) {
  switch (status) {
    case EXATTN_OK: return "success";
    case EXATTN_EINVAL: return "invalid argument (null/misaligned/overlapping pointer, bad size, window or scale)";
    case EXATTN_EUNSUPPORTED: return "unsupported head dim or dtype (d must be 64, 128 or 256; dtype f32 or bf16)";
    case EXATTN_EWORKSPACE: return "workspace smaller than attn_bwd_workspace_bytes()";
    case EXATTN_EHIP: return "HIP runtime error at kernel launch";
    case EXATTN_ESCRATCH:
      return "problem needs more scratch than the fixed buffer of attn_bwd_noalloc (EXATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int attn_fwd_gqa(int dtype, int B, int H, int Hkv, int n, int d, const void* Q, const void* K, const void* V,
                 float scale, int window, void* O, float* LSE, void* stream) {
  int st = check_problem(dtype, B, H, n, d, scale, window, Hkv);
  if (st != EXATTN_OK) return st;
  const void* ptrs[] = {Q, K, V, O, LSE};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return EXATTN_EINVAL;
  const size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  const size_t kb = (size_t)B * Hkv * n * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * n * sizeof(float);
  const Span ins[] = {{Q, tb}, {K, kb}, {V, kb}};
  for (const Span& in : ins) {
    if (overlaps(O, tb, in.p, in.n) || overlaps(LSE, lb, in.p, in.n)) return EXATTN_EINVAL;
  }
  if (overlaps(O, tb, LSE, lb)) return EXATTN_EINVAL;

  exattn::FwdParams p{Q, K, V, O, LSE, B, H, n, d, scale, window, H / Hkv};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == EXATTN_BF16 ? exattn::launch_fwd_bf16(p, s) : exattn::launch_fwd_f32(p, s);
  return from_hip(e);
}

int attn_fwd(int dtype, int B, int H, int n, int d, const void* Q, const void* K, const void* V,
             float scale, int window, void* O, float* LSE, void* stream) {
  return attn_fwd_gqa(dtype, B, H, H, n, d, Q, K, V, scale, window, O, LSE, stream);
}

// Workspace layout: [D: B*H*n fp32][LSE*log2(e): B*H*n fp32], each region
// starting on a 256-byte boundary.
static size_t ws_region_bytes(int B, int H, int n) {
  const size_t rows = (size_t)B * H * n;
  return ((rows * sizeof(float) + 255) / 256) * 256;
}

size_t attn_bwd_workspace_bytes(int dtype, int B, int H, int n, int d) {
  if (check_problem(dtype, B, H, n, d, 1.0f, -1, H) != EXATTN_OK) return 0;
  return 2 * ws_region_bytes(B, H, n);
}

}  // extern "C"

namespace {

// Validation shared by the backward entry points: every listed pointer is
// non-null and 16-byte aligned, the workspace is large enough, no output
// overlaps an input or another output.
int check_bwd(int dtype, int B, int H, int Hkv, int n, int d, float scale, int window, const Span* ins, int nin,
              const Span* outs, int nout, size_t workspace_bytes) {
  int st = check_problem(dtype, B, H, n, d, scale, window, Hkv);
  if (st != EXATTN_OK) return st;
  for (int i = 0; i < nin; ++i)
    if (ins[i].p == nullptr || !aligned16(ins[i].p)) return EXATTN_EINVAL;
  for (int i = 0; i < nout; ++i)
    if (outs[i].p == nullptr || !aligned16(outs[i].p)) return EXATTN_EINVAL;
  if (workspace_bytes < attn_bwd_workspace_bytes(dtype, B, H, n, d)) return EXATTN_EWORKSPACE;
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlaps(outs[o].p, outs[o].n, ins[i].p, ins[i].n)) return EXATTN_EINVAL;
    for (int o2 = o + 1; o2 < nout; ++o2)
      if (overlaps(outs[o].p, outs[o].n, outs[o2].p, outs[o2].n)) return EXATTN_EINVAL;
  }
  return EXATTN_OK;
}

exattn::BwdParams bwd_params(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                             const float* LSE, void* dQ, void* dK, void* dV, const void* workspace, int B, int H,
                             int n, int d, float scale, int window, int group) {
  float* ws = (float*)workspace;
  float* lse2 = (float*)((char*)workspace + ws_region_bytes(B, H, n));
  return exattn::BwdParams{Q, K, V, O, dO, LSE, dQ, dK, dV, ws, lse2, B, H, n, d, scale, window, group};
}

// A second stream per device for the key-side pass of a windowed backward.
// With a window each pass has few key tiles per block and leaves part of the
// GPU idle at its tail; once the row statistics exist the two passes are
// independent, so running them side by side fills those gaps (3-9% faster in
// measurement).  Without a window they compete for the same matrix cores and
// the overlap measured slower, so dense and pattern problems stay on one
// stream; so does a call under graph capture.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;  // held from the fork to the join of one call
SideStream g_side[kMaxSideDevices];

// The side stream of the device `s` runs on, created on first use (default
// priority, non-blocking); nullptr when it is unavailable.
SideStream* side_stream_for(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  if (s != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess || sdev != dev) return nullptr;
  }
  SideStream& g = g_side[dev];
  if (g.stream == nullptr) {
    hipStream_t t = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    if (hipStreamCreateWithFlags(&t, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess) {
      if (a != nullptr) (void)hipEventDestroy(a);
      (void)hipStreamDestroy(t);
      return nullptr;
    }
    g.fork = a;
    g.join = b;
    g.stream = t;
  }
  return &g;
}

bool split_backward(int dtype, const exattn::BwdParams& p, unsigned stages, hipStream_t s) {
  if (dtype != EXATTN_BF16 || stages != exattn::kStageAll || p.window < 0 || p.pattern_kv.list != nullptr)
    return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone;
}

// `may_split`: the call may put the key-side pass on the device's side stream
// (the allocation-free entry point passes false: it creates nothing).
int run_bwd(int dtype, const exattn::BwdParams& p, unsigned stages, void* stream, bool may_split = false) {
  hipStream_t s = (hipStream_t)stream;
  if (may_split && split_backward(dtype, p, stages, s)) {
    std::lock_guard<std::mutex> lock(g_side_mu);
    if (SideStream* side = side_stream_for(s)) {
      hipError_t e = exattn::launch_bwd_bf16(p, exattn::kStageRowdot, s);
      if (e != hipSuccess) return from_hip(e);
      e = hipEventRecord(side->fork, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
      if (e != hipSuccess) return from_hip(e);
      // from here the side stream waits on `s`; it is joined back whatever
      // the launches return, so nothing the call started outlives its stream
      hipError_t eq = exattn::launch_bwd_bf16(p, exattn::kStageQ, s);
      hipError_t ekv = eq == hipSuccess ? exattn::launch_bwd_bf16(p, exattn::kStageKV, side->stream) : hipSuccess;
      e = hipEventRecord(side->join, side->stream);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
      return from_hip(eq != hipSuccess ? eq : ekv != hipSuccess ? ekv : e);
    }
  }
  hipError_t e = dtype == EXATTN_BF16 ? exattn::launch_bwd_bf16(p, stages, s) : exattn::launch_bwd_f32(p, stages, s);
  return from_hip(e);
}

}  // namespace

extern "C" {

int attn_bwd_gqa(int dtype, int B, int H, int Hkv, int n, int d, const void* Q, const void* K, const void* V,
                 const void* O, const void* dO, const float* LSE, float scale, int window, void* dQ, void* dK,
                 void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(dtype, B, H, n, d, scale, window, Hkv);
  if (st != EXATTN_OK) return st;
  const size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  const size_t kb = (size_t)B * Hkv * n * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * n * sizeof(float);
  const size_t wb = attn_bwd_workspace_bytes(dtype, B, H, n, d);
  const Span ins[] = {{Q, tb}, {K, kb}, {V, kb}, {O, tb}, {dO, tb}, {LSE, lb}};
  const Span outs[] = {{dQ, tb}, {dK, kb}, {dV, kb}, {workspace, wb}};
  st = check_bwd(dtype, B, H, Hkv, n, d, scale, window, ins, 6, outs, 4, workspace_bytes);
  if (st != EXATTN_OK) return st;
  return run_bwd(dtype, bwd_params(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, B, H, n, d, scale, window, H / Hkv),
                 exattn::kStageAll, stream, true);
}

int attn_bwd(int dtype, int B, int H, int n, int d, const void* Q, const void* K, const void* V,
             const void* O, const void* dO, const float* LSE, float scale, int window, void* dQ,
             void* dK, void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_gqa(dtype, B, H, H, n, d, Q, K, V, O, dO, LSE, scale, window, dQ, dK, dV, workspace,
                      workspace_bytes, stream);
}

int attn_bwd_rowdot(int dtype, int B, int H, int n, int d, const void* O, const void* dO, const float* LSE,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(dtype, B, H, n, d, 1.0f, -1, H);
  if (st != EXATTN_OK) return st;
  const size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * n * sizeof(float);
  const size_t wb = attn_bwd_workspace_bytes(dtype, B, H, n, d);
  const Span ins[] = {{O, tb}, {dO, tb}, {LSE, lb}};
  const Span outs[] = {{workspace, wb}};
  st = check_bwd(dtype, B, H, H, n, d, 1.0f, -1, ins, 3, outs, 1, workspace_bytes);
  if (st != EXATTN_OK) return st;
  return run_bwd(dtype,
                 bwd_params(nullptr, nullptr, nullptr, O, dO, LSE, nullptr, nullptr, nullptr, workspace, B, H, n, d,
                            1.0f, -1, 1),
                 exattn::kStageRowdot, stream);
}

int attn_bwd_dkdv_gqa(int dtype, int B, int H, int Hkv, int n, int d, const void* Q, const void* K,
                      const void* V, const void* dO, const float* LSE, float scale, int window, void* dK, void* dV,
                      const void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(dtype, B, H, n, d, scale, window, Hkv);
  if (st != EXATTN_OK) return st;
  const size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  const size_t kb = (size_t)B * Hkv * n * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * n * sizeof(float);
  const size_t wb = attn_bwd_workspace_bytes(dtype, B, H, n, d);
  const Span ins[] = {{Q, tb}, {K, kb}, {V, kb}, {dO, tb}, {LSE, lb}, {workspace, wb}};
  const Span outs[] = {{dK, kb}, {dV, kb}};
  st = check_bwd(dtype, B, H, Hkv, n, d, scale, window, ins, 6, outs, 2, workspace_bytes);
  if (st != EXATTN_OK) return st;
  return run_bwd(dtype,
                 bwd_params(Q, K, V, nullptr, dO, LSE, nullptr, dK, dV, workspace, B, H, n, d, scale, window,
                            H / Hkv),
                 exattn::kStageKV, stream);
}

int attn_bwd_dkdv(int dtype, int B, int H, int n, int d, const void* Q, const void* K, const void* V,
                  const void* dO, const float* LSE, float scale, int window, void* dK, void* dV,
                  const void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_dkdv_gqa(dtype, B, H, H, n, d, Q, K, V, dO, LSE, scale, window, dK, dV, workspace,
                           workspace_bytes, stream);
}

int attn_bwd_dq_gqa(int dtype, int B, int H, int Hkv, int n, int d, const void* Q, const void* K, const void* V,
                    const void* dO, const float* LSE, float scale, int window, void* dQ, const void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_problem(dtype, B, H, n, d, scale, window, Hkv);
  if (st != EXATTN_OK) return st;
  const size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  const size_t kb = (size_t)B * Hkv * n * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * n * sizeof(float);
  const size_t wb = attn_bwd_workspace_bytes(dtype, B, H, n, d);
  const Span ins[] = {{Q, tb}, {K, kb}, {V, kb}, {dO, tb}, {LSE, lb}, {workspace, wb}};
  const Span outs[] = {{dQ, tb}};
  st = check_bwd(dtype, B, H, Hkv, n, d, scale, window, ins, 6, outs, 1, workspace_bytes);
  if (st != EXATTN_OK) return st;
  return run_bwd(dtype,
                 bwd_params(Q, K, V, nullptr, dO, LSE, dQ, nullptr, nullptr, workspace, B, H, n, d, scale, window,
                            H / Hkv),
                 exattn::kStageQ, stream);
}

int attn_bwd_dq(int dtype, int B, int H, int n, int d, const void* Q, const void* K, const void* V,
                const void* dO, const float* LSE, float scale, int window, void* dQ, const void* workspace,
                size_t workspace_bytes, void* stream) {
  return attn_bwd_dq_gqa(dtype, B, H, H, n, d, Q, K, V, dO, LSE, scale, window, dQ, workspace, workspace_bytes,
                         stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward without allocation: the rowdot stage's -D and LSE*log2(e) rows go
// to a fixed device array instead of a caller workspace.  Each GPU holds its
// own copy of the array (from the library's first use on it until the
// process ends); in host code its name is only a stand-in, so kernels get the
// device address looked up per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[EXATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device (with it current) and kept.
int scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return EXATTN_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return EXATTN_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return EXATTN_OK;
}

}  // namespace

extern "C" {

int attn_bwd_noalloc(int dtype, int B, int H, int n, int d, const void* Q, const void* K, const void* V,
                     const void* O, const void* dO, const float* LSE, float scale, int window, void* dQ, void* dK,
                     void* dV, void* stream) {
  // every check attn_bwd makes on these arguments, before any HIP call
  int st = check_problem(dtype, B, H, n, d, scale, window, H);
  if (st != EXATTN_OK) return st;
  const size_t wb = attn_bwd_workspace_bytes(dtype, B, H, n, d);
  if (wb > (size_t)EXATTN_NOALLOC_SCRATCH_BYTES) return EXATTN_ESCRATCH;
  const size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * n * sizeof(float);
  const Span ins[] = {{Q, tb}, {K, tb}, {V, tb}, {O, tb}, {dO, tb}, {LSE, lb}};
  const Span outs[] = {{dQ, tb}, {dK, tb}, {dV, tb}};
  st = check_bwd(dtype, B, H, H, n, d, scale, window, ins, 6, outs, 3, wb);
  if (st != EXATTN_OK) return st;
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != EXATTN_OK) return st;
  // the rowdot stage overwrites every row of both regions before the
  // gradient kernels read them: nothing needs clearing between calls
  return run_bwd(dtype, bwd_params(Q, K, V, O, dO, LSE, dQ, dK, dV, ws, B, H, n, d, scale, window, 1),
                 exattn::kStageAll, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Sparse patterns (window + global tokens + block layout)
// ---------------------------------------------------------------------------
namespace {

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Workspace layout for a pattern problem: [global bitmap][full-row bitmap]
// [full-key bitmap][layout flags][full-row list][full-key list][split info]
// [forward lists][key-side lists][query-side lists][scratch]
// [D][LSE*log2(e)], each region 256-byte aligned.  Lists hold, per workgroup
// row of the kernel's grid, one entry per tile of the other side (the most a
// workgroup can visit) and a count.  The scratch region serves, in stream
// order, the key-side pass's copies of the full rows (Q and dO [B*H][n][d]
// bf16, then LSE*log2(e) and D [B*H][n] fp32) and the partial results of the
// full positions' passes (full_part_rows(n) slots per head of 2d floats;
// forward: d for O, then one log-sum-exp per slot after all the O slots).
struct PatternLayout {
  size_t bitmap, flags, idx, info, fwd, kv, q, part, rows, total;
  int fwd_R, fwd_T, fwd_NW, kv_R, kv_T, kv_NW, q_R, q_T, q_NW;
  int fwd_blocks, fwd_tiles, kv_blocks, kv_tiles, q_blocks, q_tiles;
  size_t part_floats;   // floats of the partial results
  size_t gather_bytes;  // bytes of the full rows' copies
  // offsets from the start of the workspace
  size_t off_gbits, off_rowfull, off_colfull, off_flags, off_rowidx, off_colidx, off_info, off_fwd, off_kv, off_q,
      off_part, off_rows;
};

PatternLayout pattern_layout(int B, int H, int n, int d) {
  PatternLayout L{};
  exattn::fwd_bf16_geometry(d, &L.fwd_R, &L.fwd_T, &L.fwd_NW);
  exattn::bwd_kv_bf16_geometry(d, &L.kv_R, &L.kv_T, &L.kv_NW);
  exattn::bwd_q_bf16_geometry(d, &L.q_R, &L.q_T, &L.q_NW);
  L.fwd_blocks = (n + L.fwd_R - 1) / L.fwd_R;
  L.fwd_tiles = (n + L.fwd_T - 1) / L.fwd_T;
  L.kv_blocks = (n + L.kv_R - 1) / L.kv_R;
  L.kv_tiles = (n + L.kv_T - 1) / L.kv_T;
  L.q_blocks = (n + L.q_R - 1) / L.q_R;
  L.q_tiles = (n + L.q_T - 1) / L.q_T;
  const size_t nb = (size_t)(n + exattn::kLayoutBlock - 1) / exattn::kLayoutBlock;
  L.bitmap = align256((size_t)exattn::bitmap_words(n) * 4);
  L.flags = align256(2 * nb * 4);
  L.idx = align256((size_t)n * 4);
  L.info = align256((3 * exattn::kFullInfoInts + 2) * 4);  // split info of 3 kernels, then the 2 counts
  L.fwd = align256((size_t)L.fwd_blocks * (L.fwd_tiles + 1) * 4);
  L.kv = align256((size_t)L.kv_blocks * (L.kv_tiles + 1) * 4);
  L.q = align256((size_t)L.q_blocks * (L.q_tiles + 1) * 4);
  L.part_floats = (size_t)B * H * exattn::full_part_rows(n) * 2 * d;
  L.gather_bytes = (size_t)B * H * n * (4 * (size_t)d + 8);
  L.part = align256(L.part_floats * 4 > L.gather_bytes ? L.part_floats * 4 : L.gather_bytes);
  L.rows = 2 * ws_region_bytes(B, H, n);
  L.off_gbits = 0;
  L.off_rowfull = L.off_gbits + L.bitmap;
  L.off_colfull = L.off_rowfull + L.bitmap;
  L.off_flags = L.off_colfull + L.bitmap;
  L.off_rowidx = L.off_flags + L.flags;
  L.off_colidx = L.off_rowidx + L.idx;
  L.off_info = L.off_colidx + L.idx;
  L.off_fwd = L.off_info + L.info;
  L.off_kv = L.off_fwd + L.fwd;
  L.off_q = L.off_kv + L.kv;
  L.off_part = L.off_q + L.q;
  L.off_rows = L.off_part + L.part;
  L.total = L.off_rows + L.rows;
  return L;
}

// Host-side checks of the pattern descriptor (its arrays stay on the device).
int check_pattern(const exattn_pattern* pat, int n) {
  if (pat == nullptr) return EXATTN_EINVAL;
  if (pat->window < -1 || pat->n_global < 0) return EXATTN_EINVAL;
  if (pat->n_global > 0 && (pat->global_idx == nullptr || ((uintptr_t)pat->global_idx & 3u))) return EXATTN_EINVAL;
  if (pat->layout_block != 0 && pat->layout_block != exattn::kLayoutBlock) return EXATTN_EUNSUPPORTED;
  if (pat->layout_block != 0 && pat->layout == nullptr) return EXATTN_EINVAL;
  (void)n;
  return EXATTN_OK;
}

size_t layout_bytes(const exattn_pattern* pat, int n) {
  if (pat->layout_block == 0) return 0;
  const size_t nb = (size_t)(n + exattn::kLayoutBlock - 1) / exattn::kLayoutBlock;
  return nb * nb;
}

exattn::PlanInput plan_input(const exattn_pattern* pat, int n, void* workspace, const PatternLayout& L) {
  char* ws = (char*)workspace;
  exattn::PlanInput in{};
  in.n = n;
  in.window = pat->window;
  in.n_global = pat->n_global;
  in.global_idx = pat->global_idx;
  in.layout = pat->layout_block ? pat->layout : nullptr;
  in.layout_n = (n + exattn::kLayoutBlock - 1) / exattn::kLayoutBlock;
  in.gbits = (uint32_t*)(ws + L.off_gbits);
  in.row_full = (uint32_t*)(ws + L.off_rowfull);
  in.col_full = (uint32_t*)(ws + L.off_colfull);
  in.layout_flags = (int*)(ws + L.off_flags);
  in.row_idx = (int*)(ws + L.off_rowidx);
  in.col_idx = (int*)(ws + L.off_colidx);
  in.counts = (int*)(ws + L.off_info) + 3 * exattn::kFullInfoInts;
  return in;
}

// Split info of consumer kernel `k` (0: forward, 1: key side, 2: query side).
int* full_info(void* workspace, const PatternLayout& L, int k) {
  return (int*)((char*)workspace + L.off_info) + k * exattn::kFullInfoInts;
}

// Builds one list in the region at `base`; returns the run-time descriptor.
hipError_t build_list(const exattn::PlanInput& in, char* base, int R, int T, int NW, int blocks, int tiles,
                      bool transposed, bool tail_partial, exattn::PatternDev* dev, hipStream_t s) {
  exattn::PlanList pl{};
  pl.R = R;
  pl.T = T;
  pl.NW = NW;
  pl.transposed = transposed;
  pl.tail_partial = tail_partial;
  pl.own_full = transposed ? in.col_full : in.row_full;
  pl.other_full = transposed ? in.row_full : in.col_full;
  pl.count = (int*)base;
  pl.list = (int*)base + blocks;
  pl.stride = tiles;
  pl.nblocks = blocks;
  // the other side's full positions: rows for the key-side pass, else keys
  *dev = exattn::PatternDev{in.window,     pl.own_full, pl.other_full, transposed ? in.row_idx : in.col_idx,
                            in.counts + (transposed ? 0 : 1), pl.list, pl.count, tiles};
  return exattn::launch_pattern_list(in, pl, s);
}

}  // namespace

extern "C" {

size_t attn_pattern_workspace_bytes(int dtype, int B, int H, int n, int d) {
  if (check_problem(dtype, B, H, n, d, 1.0f, -1, H) != EXATTN_OK) return 0;
  return pattern_layout(B, H, n, d).total;
}

int attn_fwd_pattern(int dtype, int B, int H, int n, int d, const void* Q, const void* K, const void* V, float scale,
                     const exattn_pattern* pattern, void* O, float* LSE, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = check_problem(dtype, B, H, n, d, scale, -1, H);
  if (st != EXATTN_OK) return st;
  st = check_pattern(pattern, n);
  if (st != EXATTN_OK) return st;
  if (dtype != EXATTN_BF16) return EXATTN_EUNSUPPORTED;
  const void* ptrs[] = {Q, K, V, O, LSE, workspace};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return EXATTN_EINVAL;
  const PatternLayout L = pattern_layout(B, H, n, d);
  if (workspace_bytes < L.total) return EXATTN_EWORKSPACE;
  const size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * n * sizeof(float);
  const Span ins[] = {{Q, tb}, {K, tb}, {V, tb}, {pattern->global_idx, (size_t)pattern->n_global * 4},
                      {pattern->layout, layout_bytes(pattern, n)}};
  const Span outs[] = {{O, tb}, {LSE, lb}, {workspace, L.total}};
  for (int o = 0; o < 3; ++o) {
    for (const Span& in : ins)
      if (in.n && overlaps(outs[o].p, outs[o].n, in.p, in.n)) return EXATTN_EINVAL;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlaps(outs[o].p, outs[o].n, outs[o2].p, outs[o2].n)) return EXATTN_EINVAL;
  }

  hipStream_t s = (hipStream_t)stream;
  const exattn::PlanInput in = plan_input(pattern, n, workspace, L);
  const exattn::FullSplit split{L.fwd_tiles, false, full_info(workspace, L, 0)};
  hipError_t e = exattn::launch_pattern_bitmap(in, &split, 1, s);
  exattn::FwdParams p{Q, K, V, O, LSE, B, H, n, d, scale, -1, 1};
  float* part = (float*)((char*)workspace + L.off_part);
  p.full = exattn::FullDev{in.row_idx, split.info, part, part + (size_t)B * H * exattn::full_part_rows(n) * d};
  if (e == hipSuccess)
    e = build_list(in, (char*)workspace + L.off_fwd, L.fwd_R, L.fwd_T, L.fwd_NW, L.fwd_blocks, L.fwd_tiles, false,
                   true, &p.pattern, s);
  // the full keys' copies (scratch region, before the full rows' partial results)
  p.pattern.gath_a = (const __bf16*)((char*)workspace + L.off_part);
  p.pattern.gath_b = p.pattern.gath_a + (size_t)B * H * n * d;
  if (e == hipSuccess) e = exattn::launch_fwd_bf16(p, s);
  return from_hip(e);
}

int attn_bwd_pattern(int dtype, int B, int H, int n, int d, const void* Q, const void* K, const void* V,
                     const void* O, const void* dO, const float* LSE, float scale, const exattn_pattern* pattern,
                     void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_problem(dtype, B, H, n, d, scale, -1, H);
  if (st != EXATTN_OK) return st;
  st = check_pattern(pattern, n);
  if (st != EXATTN_OK) return st;
  if (dtype != EXATTN_BF16) return EXATTN_EUNSUPPORTED;
  const void* ptrs[] = {Q, K, V, O, dO, LSE, dQ, dK, dV, workspace};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return EXATTN_EINVAL;
  const PatternLayout L = pattern_layout(B, H, n, d);
  if (workspace_bytes < L.total) return EXATTN_EWORKSPACE;
  const size_t tb = (size_t)B * H * n * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * n * sizeof(float);
  const Span ins[] = {{Q, tb},
                      {K, tb},
                      {V, tb},
                      {O, tb},
                      {dO, tb},
                      {LSE, lb},
                      {pattern->global_idx, (size_t)pattern->n_global * 4},
                      {pattern->layout, layout_bytes(pattern, n)}};
  const Span outs[] = {{dQ, tb}, {dK, tb}, {dV, tb}, {workspace, L.total}};
  for (int o = 0; o < 4; ++o) {
    for (const Span& in : ins)
      if (in.n && overlaps(outs[o].p, outs[o].n, in.p, in.n)) return EXATTN_EINVAL;
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlaps(outs[o].p, outs[o].n, outs[o2].p, outs[o2].n)) return EXATTN_EINVAL;
  }

  hipStream_t s = (hipStream_t)stream;
  const exattn::PlanInput in = plan_input(pattern, n, workspace, L);
  char* base = (char*)workspace;
  exattn::BwdParams p = bwd_params(Q, K, V, O, dO, LSE, dQ, dK, dV, base + L.off_rows, B, H, n, d, scale, -1, 1);
  const exattn::FullSplit splits[2] = {{L.kv_tiles, true, full_info(workspace, L, 1)},
                                       {L.q_tiles, false, full_info(workspace, L, 2)}};
  float* part = (float*)(base + L.off_part);
  p.full_kv = exattn::FullDev{in.col_idx, splits[0].info, part, nullptr};
  p.full_q = exattn::FullDev{in.row_idx, splits[1].info, part, nullptr};
  hipError_t e = exattn::launch_pattern_bitmap(in, splits, 2, s);
  if (e == hipSuccess)
    e = build_list(in, base + L.off_kv, L.kv_R, L.kv_T, L.kv_NW, L.kv_blocks, L.kv_tiles, true, false,
                   &p.pattern_kv, s);
  if (e == hipSuccess)
    e = build_list(in, base + L.off_q, L.q_R, L.q_T, L.q_NW, L.q_blocks, L.q_tiles, false, false, &p.pattern_q, s);
  {  // the other side's copies for each pass (scratch region, before its partial
     // results); set after build_list, which writes the whole descriptor
    const size_t rows = (size_t)B * H * n;
    __bf16* g = (__bf16*)(base + L.off_part);
    p.pattern_kv.gath_a = g;
    p.pattern_kv.gath_b = g + rows * d;
    p.pattern_kv.gath_s0 = (const float*)(g + 2 * rows * d);
    p.pattern_kv.gath_s1 = p.pattern_kv.gath_s0 + rows;
    p.pattern_q.gath_a = g;
    p.pattern_q.gath_b = g + rows * d;
  }
  if (e == hipSuccess) e = exattn::launch_bwd_bf16(p, exattn::kStageAll, s);
  return from_hip(e);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// FP8 (E4M3) forward and its quantiser
// ---------------------------------------------------------------------------
extern "C" {

size_t attn_fp8_bytes(int B, int H, int n, int d, int layout) {
  if (check_problem(EXATTN_BF16, B, H, n, d, 1.0f, -1, H) != EXATTN_OK) return 0;
  if (layout != EXATTN_FP8_ROWS && layout != EXATTN_FP8_V_TRANSPOSED) return 0;
  const size_t cols = layout == EXATTN_FP8_ROWS ? (size_t)n : (size_t)exattn::fp8_padded_n(n);
  return (size_t)B * H * cols * d;
}

int attn_quant_fp8(int B, int H, int n, int d, const void* X, const float* signs, int layout, void* X8,
                   float* scale, void* stream) {
  int st = check_problem(EXATTN_BF16, B, H, n, d, 1.0f, -1, H);
  if (st != EXATTN_OK) return st;
  if (d == 256) return EXATTN_EUNSUPPORTED;
  if (layout != EXATTN_FP8_ROWS && layout != EXATTN_FP8_V_TRANSPOSED) return EXATTN_EINVAL;
  const void* ptrs[] = {X, X8, scale};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return EXATTN_EINVAL;
  if (signs != nullptr && ((uintptr_t)signs & 3u)) return EXATTN_EINVAL;
  const size_t xb = (size_t)B * H * n * d * 2, qb = attn_fp8_bytes(B, H, n, d, layout);
  const size_t sb = (size_t)B * H * sizeof(float);
  const Span ins[] = {{X, xb}, {signs, signs ? (size_t)d * 4 : 0}};
  const Span outs[] = {{X8, qb}, {scale, sb}};
  for (const Span& o : outs)
    for (const Span& in : ins)
      if (in.n && overlaps(o.p, o.n, in.p, in.n)) return EXATTN_EINVAL;
  if (overlaps(X8, qb, scale, sb)) return EXATTN_EINVAL;
  exattn::Fp8QuantParams p{B, H, n, d, X, signs, X8, scale, layout == EXATTN_FP8_V_TRANSPOSED};
  return from_hip(exattn::launch_quant_fp8(p, (hipStream_t)stream));
}

int attn_fwd_fp8(int B, int H, int n, int d, const void* Q8, const void* K8, const void* V8t, const float* q_scale,
                 const float* k_scale, const float* v_scale, float scale, int rotated, void* O, float* LSE,
                 void* stream) {
  int st = check_problem(EXATTN_BF16, B, H, n, d, scale, -1, H);
  if (st != EXATTN_OK) return st;
  if (d != 64 && d != 128) return EXATTN_EUNSUPPORTED;
  if (rotated != 0 && rotated != 1) return EXATTN_EINVAL;
  const void* ptrs[] = {Q8, K8, V8t, O, LSE};
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return EXATTN_EINVAL;
  const void* sp[] = {q_scale, k_scale, v_scale};
  for (const void* p : sp)
    if (p == nullptr || ((uintptr_t)p & 3u)) return EXATTN_EINVAL;
  const size_t qb = attn_fp8_bytes(B, H, n, d, EXATTN_FP8_ROWS);
  const size_t vb = attn_fp8_bytes(B, H, n, d, EXATTN_FP8_V_TRANSPOSED);
  const size_t ob = (size_t)B * H * n * d * 2, lb = (size_t)B * H * n * sizeof(float), sb = (size_t)B * H * 4;
  const Span ins[] = {{Q8, qb}, {K8, qb}, {V8t, vb}, {q_scale, sb}, {k_scale, sb}, {v_scale, sb}};
  for (const Span& in : ins)
    if (overlaps(O, ob, in.p, in.n) || overlaps(LSE, lb, in.p, in.n)) return EXATTN_EINVAL;
  if (overlaps(O, ob, LSE, lb)) return EXATTN_EINVAL;
  exattn::Fp8FwdParams p{B, H, n, d, Q8, K8, V8t, q_scale, k_scale, v_scale, scale, rotated, O, LSE};
  return from_hip(exattn::launch_fwd_fp8(p, (hipStream_t)stream));
}

}  // extern "C"

