// fp32 forward and backward kernels (vector ALU, fp32 throughout).
//
// The fp32 element type is the accuracy path: scores, probabilities and
// gradients stay in fp32 with no bf16 rounding.  It follows the same scheme
// as the bf16 path -- key/value tiles staged in LDS, an online softmax with a
// running max and sum in the forward (llmis.ru chapter 3.1, section 5), and
// a backward that recomputes P from the saved log-sum-exp (the unite.ai
// Flash Attention page, "Entenda a Flash Attention", item 2) -- but on the
// vector ALU: a row of d values is split over TPR = 8 lanes, each holding
// d/8 of them, and dot products are finished with xor shuffles.  The four
// waves of a workgroup own the same 8 rows (keys) and take every fourth row
// of each staged tile, so a row's serial chain is a quarter of the other
// side; their partial results are merged through LDS at the end (the
// log-sum-exp merge for the forward, sums for the gradients).
#include <math.h>

#include "bwd_common.hpp"
#include "device_common.hpp"
#include "launch.hpp"

namespace exattn {
namespace {

constexpr int TPR = 8;                  // lanes per row
constexpr int SPLIT = 4;                // waves of a block, each over a quarter of every tile
constexpr int ROWS = 64 / TPR;          // rows (keys) per block, shared by its waves
// rows per staged LDS tile (two tiles of TK x D floats must fit in 64 KiB)
template <int D>
constexpr int tile_rows() { return D == 256 ? 16 : 32; }

__device__ __forceinline__ float row_sum8(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  return x;
}

// Element e of this lane's slice of a row is column TPR*e + sub, so the 8
// lanes of a row read 8 consecutive floats (conflict-free LDS access).

// ----------------------------------------------------------------------------
// Forward: block = 8 query rows; loops over 32-key tiles (16 at d=256).
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Qg, const float* __restrict__ Kg,
                                                      const float* __restrict__ Vg, float* __restrict__ Og,
                                                      float* __restrict__ LSEg, int n, int nqb, float scale,
                                                      int window, int group) {
  constexpr int E = D / TPR;
  constexpr int TK = tile_rows<D>();
  static_assert(2 * TK * D >= SPLIT * ROWS * D, "the merge reuses the tile buffers");
  __shared__ float KVs[2][TK][D];           // the K and V tiles; the merge's partial acc
  __shared__ float stat[SPLIT * ROWS * 2];  // merge: m, l of each wave's share
  poison_lds(KVs, stat);
  float(&Ks)[TK][D] = KVs[0];
  float(&Vs)[TK][D] = KVs[1];
  const int head = blockIdx.x / nqb, qb = blockIdx.x - (blockIdx.x / nqb) * nqb;
  const int tid = threadIdx.x, sub = tid & (TPR - 1), rloc = (tid & 63) / TPR, wave = tid >> 6;
  const int row = qb * ROWS + rloc;
  const size_t hoff = (size_t)head * n * D;
  const size_t kv_off = (size_t)(head / group) * n * D;  // shared key/value head
  const float* K = Kg + kv_off;
  const float* V = Vg + kv_off;

  float q[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = row < n ? Qg[hoff + (size_t)row * D + TPR * e + sub] : 0.0f;
    acc[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;  // this wave's share: keys j = wave (mod SPLIT) of every tile

  int k_lo = 0, k_hi = n;
  if (window >= 0) band_keys(qb * ROWS, qb * ROWS + ROWS, n, window, &k_lo, &k_hi);
  // keys visible to this row: [key_lo, key_lo + key_span)
  int key_lo = 0, key_hi = n;
  band_keys(row, row + 1, n, window, &key_lo, &key_hi);
  const unsigned key_span = (unsigned)max(key_hi - key_lo, 0);
  constexpr int TW = TK / SPLIT;  // keys of a tile per wave
  for (int k0 = (k_lo / TK) * TK; k0 < k_hi; k0 += TK) {
    __syncthreads();
    for (int i = tid; i < TK * D; i += 256) {
      const int r = i / D, c = i - (i / D) * D;
      const bool ok = k0 + r < n;
      Ks[r][c] = ok ? K[(size_t)(k0 + r) * D + c] : 0.0f;
      Vs[r][c] = ok ? V[(size_t)(k0 + r) * D + c] : 0.0f;
    }
    __syncthreads();
    float s[TW];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int j = SPLIT * t + wave;
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) part = fmaf(q[e], Ks[j][TPR * e + sub], part);
      float sj = row_sum8(part) * scale;
      sj = (unsigned)(k0 + j - key_lo) < key_span ? sj : -INFINITY;
      s[t] = sj;
      mx = fmaxf(mx, sj);
    }
    const float m_new = fmaxf(m, mx);
    const float msub = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = expf(m - msub);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= alpha;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int j = SPLIT * t + wave;
      const float p = expf(s[t] - msub);
      l += p;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(p, Vs[j][TPR * e + sub], acc[e]);
    }
    m = m_new;
  }
  // merge of the waves' shares: L = log sum_w exp(L_w) over the partial
  // (m_w, l_w, acc_w) of each wave, O = sum_w exp(m_w - m) acc_w / l
  __syncthreads();
  float* part = &KVs[0][0][0];  // [SPLIT][ROWS][D] partial acc
#pragma unroll
  for (int e = 0; e < E; ++e) part[(wave * ROWS + rloc) * D + TPR * e + sub] = acc[e];
  if (sub == 0) {
    stat[(wave * ROWS + rloc) * 2] = m;
    stat[(wave * ROWS + rloc) * 2 + 1] = l;
  }
  __syncthreads();
  if (wave == 0 && row < n) {
    float mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < SPLIT; ++w) mt = fmaxf(mt, stat[(w * ROWS + rloc) * 2]);
    float f[SPLIT], lt = 0.0f;
#pragma unroll
    for (int w = 0; w < SPLIT; ++w) {
      const float mw = stat[(w * ROWS + rloc) * 2];
      f[w] = mw == -INFINITY ? 0.0f : expf(mw - mt);
      lt += f[w] * stat[(w * ROWS + rloc) * 2 + 1];
    }
    const float inv = 1.0f / lt;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float o = 0.0f;
#pragma unroll
      for (int w = 0; w < SPLIT; ++w) o = fmaf(f[w], part[(w * ROWS + rloc) * D + TPR * e + sub], o);
      Og[hoff + (size_t)row * D + TPR * e + sub] = o * inv;
    }
    if (sub == 0) LSEg[(size_t)head * n + row] = mt + logf(lt);
  }
}

// ----------------------------------------------------------------------------
// Backward, key side: block = 8 keys; accumulates dK and dV over query tiles.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_kv_f32_kernel(const float* __restrict__ Qg, const float* __restrict__ Kg,
                                                         const float* __restrict__ Vg, const float* __restrict__ dOg,
                                                         const float* __restrict__ LSEg, const float* __restrict__ Dg,
                                                         float* __restrict__ dKg, float* __restrict__ dVg, int n,
                                                         int nkb, float scale, int window, int group) {
  constexpr int E = D / TPR;
  constexpr int TK = tile_rows<D>();
  static_assert(2 * TK * D >= SPLIT * ROWS * D, "the merge reuses the tile buffers");
  __shared__ float QdO[2][TK][D];  // the Q and dO tiles; the merge's partial sums
  __shared__ float Ls[TK], Ds[TK];
  poison_lds(QdO, Ls, Ds);
  float(&Qs)[TK][D] = QdO[0];
  float(&dOs)[TK][D] = QdO[1];
  const int kvh = blockIdx.x / nkb, kb = blockIdx.x - (blockIdx.x / nkb) * nkb;  // key/value head, key block
  const int tid = threadIdx.x, sub = tid & (TPR - 1), rloc = (tid & 63) / TPR, wave = tid >> 6;
  const int key = kb * ROWS + rloc;
  const size_t hoff = (size_t)kvh * n * D;

  float k[E], v[E], dk[E], dv[E];  // dk, dv: this wave's share (rows r = wave mod SPLIT of every tile)
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = key < n ? Kg[hoff + (size_t)key * D + TPR * e + sub] : 0.0f;
    v[e] = key < n ? Vg[hoff + (size_t)key * D + TPR * e + sub] : 0.0f;
    dk[e] = 0.0f;
    dv[e] = 0.0f;
  }
  // queries that can see any key of this block
  int q_lo = 0, q_hi = n;
  if (window >= 0) band_keys(kb * ROWS, kb * ROWS + ROWS, n, window, &q_lo, &q_hi);
  // query rows that see this key: [row_lo, row_lo + row_span); none if key >= n
  int row_lo = 0, row_hi = n;
  band_keys(key, key + 1, n, window, &row_lo, &row_hi);
  const unsigned row_span = key < n ? (unsigned)max(row_hi - row_lo, 0) : 0u;
  // dK and dV sum over the group's query heads kvh*group .. kvh*group + group - 1.
  for (int qg = 0; qg < group; ++qg) {
    const size_t qh = (size_t)kvh * group + qg;
    const float* Q = Qg + qh * n * D;
    const float* dO = dOg + qh * n * D;
    const float* lse = LSEg + qh * n;
    const float* dl = Dg + qh * n;
    for (int i0 = (q_lo / TK) * TK; i0 < q_hi; i0 += TK) {
      __syncthreads();
      for (int i = tid; i < TK * D; i += 256) {
        const int r = i / D, c = i - (i / D) * D;
        const bool ok = i0 + r < n;
        Qs[r][c] = ok ? Q[(size_t)(i0 + r) * D + c] : 0.0f;
        dOs[r][c] = ok ? dO[(size_t)(i0 + r) * D + c] : 0.0f;
      }
      if (tid < TK) {
        const bool ok = i0 + tid < n;
        Ls[tid] = ok ? lse[i0 + tid] : 0.0f;
        Ds[tid] = ok ? -dl[i0 + tid] : 0.0f;  // the workspace holds -D
      }
      __syncthreads();
#pragma unroll 2  // full unrolling hoists every row's LDS loads: 400 registers at d=128
      for (int t = 0; t < TK / SPLIT; ++t) {
        const int r = SPLIT * t + wave;
        const int qi = i0 + r;
        float ps = 0.0f, pd = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          ps = fmaf(k[e], Qs[r][TPR * e + sub], ps);
          pd = fmaf(v[e], dOs[r][TPR * e + sub], pd);
        }
        const float sc = row_sum8(ps) * scale;
        const float dp = row_sum8(pd);
        const bool live = (unsigned)(qi - row_lo) < row_span;
        const float p = live ? expf(sc - Ls[r]) : 0.0f;
        const float ds = p * (dp - Ds[r]) * scale;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          dv[e] = fmaf(p, dOs[r][TPR * e + sub], dv[e]);
          dk[e] = fmaf(ds, Qs[r][TPR * e + sub], dk[e]);
        }
      }
    }
  }
  // sums of the waves' shares, in wave order: dK, then dV
  float* part = &QdO[0][0][0];  // [SPLIT][ROWS][D]
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) part[(wave * ROWS + rloc) * D + TPR * e + sub] = pass == 0 ? dk[e] : dv[e];
    __syncthreads();
    if (wave == 0 && key < n) {
      float* dst = (pass == 0 ? dKg : dVg) + hoff + (size_t)key * D;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float acc = part[rloc * D + TPR * e + sub];
#pragma unroll
        for (int w = 1; w < SPLIT; ++w) acc += part[(w * ROWS + rloc) * D + TPR * e + sub];
        dst[TPR * e + sub] = acc;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Backward, query side: block = 8 query rows; accumulates dQ over key tiles.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_q_f32_kernel(const float* __restrict__ Qg, const float* __restrict__ Kg,
                                                        const float* __restrict__ Vg, const float* __restrict__ dOg,
                                                        const float* __restrict__ LSEg, const float* __restrict__ Dg,
                                                        float* __restrict__ dQg, int n, int nqb, float scale,
                                                        int window, int group) {
  constexpr int E = D / TPR;
  constexpr int TK = tile_rows<D>();
  static_assert(2 * TK * D >= SPLIT * ROWS * D, "the merge reuses the tile buffers");
  __shared__ float KVs[2][TK][D];  // the K and V tiles; the merge's partial sums
  poison_lds(KVs);
  float(&Ks)[TK][D] = KVs[0];
  float(&Vs)[TK][D] = KVs[1];
  const int head = blockIdx.x / nqb, qb = blockIdx.x - (blockIdx.x / nqb) * nqb;
  const int tid = threadIdx.x, sub = tid & (TPR - 1), rloc = (tid & 63) / TPR, wave = tid >> 6;
  const int row = qb * ROWS + rloc;
  const size_t hoff = (size_t)head * n * D;
  const size_t kv_off = (size_t)(head / group) * n * D;  // shared key/value head
  const float* K = Kg + kv_off;
  const float* V = Vg + kv_off;

  float q[E], g[E], dq[E];  // dq: this wave's share (keys j = wave mod SPLIT of every tile)
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = row < n ? Qg[hoff + (size_t)row * D + TPR * e + sub] : 0.0f;
    g[e] = row < n ? dOg[hoff + (size_t)row * D + TPR * e + sub] : 0.0f;
    dq[e] = 0.0f;
  }
  const float lse = row < n ? LSEg[(size_t)head * n + row] : 0.0f;
  const float dl = row < n ? -Dg[(size_t)head * n + row] : 0.0f;  // the workspace holds -D

  int k_lo = 0, k_hi = n;
  if (window >= 0) band_keys(qb * ROWS, qb * ROWS + ROWS, n, window, &k_lo, &k_hi);
  // keys visible to this row: [key_lo, key_lo + key_span); none if row >= n
  int key_lo = 0, key_hi = n;
  band_keys(row, row + 1, n, window, &key_lo, &key_hi);
  const unsigned key_span = row < n ? (unsigned)max(key_hi - key_lo, 0) : 0u;
  for (int k0 = (k_lo / TK) * TK; k0 < k_hi; k0 += TK) {
    __syncthreads();
    for (int i = tid; i < TK * D; i += 256) {
      const int r = i / D, c = i - (i / D) * D;
      const bool ok = k0 + r < n;
      Ks[r][c] = ok ? K[(size_t)(k0 + r) * D + c] : 0.0f;
      Vs[r][c] = ok ? V[(size_t)(k0 + r) * D + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TK / SPLIT; ++t) {
      const int j = SPLIT * t + wave;
      const int key = k0 + j;
      float ps = 0.0f, pd = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ps = fmaf(q[e], Ks[j][TPR * e + sub], ps);
        pd = fmaf(g[e], Vs[j][TPR * e + sub], pd);
      }
      const float sc = row_sum8(ps) * scale;
      const float dp = row_sum8(pd);
      const bool live = (unsigned)(key - key_lo) < key_span;
      const float p = live ? expf(sc - lse) : 0.0f;
      const float ds = p * (dp - dl) * scale;
#pragma unroll
      for (int e = 0; e < E; ++e) dq[e] = fmaf(ds, Ks[j][TPR * e + sub], dq[e]);
    }
  }
  // sum of the waves' shares, in wave order
  __syncthreads();
  float* part = &KVs[0][0][0];  // [SPLIT][ROWS][D]
#pragma unroll
  for (int e = 0; e < E; ++e) part[(wave * ROWS + rloc) * D + TPR * e + sub] = dq[e];
  __syncthreads();
  if (wave == 0 && row < n) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float acc = part[rloc * D + TPR * e + sub];
#pragma unroll
      for (int w = 1; w < SPLIT; ++w) acc += part[(w * ROWS + rloc) * D + TPR * e + sub];
      dQg[hoff + (size_t)row * D + TPR * e + sub] = acc;
    }
  }
}

template <int D>
hipError_t fwd_d(const FwdParams& p, hipStream_t stream) {
  const int nqb = (p.n + ROWS - 1) / ROWS;
  const long total = (long)nqb * p.B * p.H;
  if (total > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3((unsigned)total), dim3(256), 0, stream, (const float*)p.q,
                     (const float*)p.k, (const float*)p.v, (float*)p.o, p.lse, p.n, nqb, p.scale, p.window,
                     p.group);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const BwdParams& p, unsigned stages, hipStream_t stream) {
  const int nb = (p.n + ROWS - 1) / ROWS;
  const long total = (long)nb * p.B * p.H;
  const long total_kv = total / p.group;  // key blocks: one set per key/value head
  if (total > 0x7fffffffL) return hipErrorInvalidValue;
  if (stages & kStageRowdot) {
    hipError_t e = launch_rowdot<float>((const float*)p.o, (const float*)p.dout, p.lse, p.delta, p.lse2,
                                        (long)p.B * p.H * p.n, D, stream);
    if (e != hipSuccess) return e;
  }
  if (stages & kStageKV) {
    hipLaunchKernelGGL((bwd_kv_f32_kernel<D>), dim3((unsigned)total_kv), dim3(256), 0, stream, (const float*)p.q,
                       (const float*)p.k, (const float*)p.v, (const float*)p.dout, p.lse, p.delta, (float*)p.dk,
                       (float*)p.dv, p.n, nb, p.scale, p.window, p.group);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kStageQ) {
    hipLaunchKernelGGL((bwd_q_f32_kernel<D>), dim3((unsigned)total), dim3(256), 0, stream, (const float*)p.q,
                       (const float*)p.k, (const float*)p.v, (const float*)p.dout, p.lse, p.delta, (float*)p.dq,
                       p.n, nb, p.scale, p.window, p.group);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  switch (p.d) {
    case 64: return fwd_d<64>(p, stream);
    case 128: return fwd_d<128>(p, stream);
    case 256: return fwd_d<256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_f32(const BwdParams& p, unsigned stages, hipStream_t stream) {
  switch (p.d) {
    case 64: return bwd_d<64>(p, stages, stream);
    case 128: return bwd_d<128>(p, stages, stream);
    case 256: return bwd_d<256>(p, stages, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace exattn
