// Forward attention kernel, bf16 inputs, fp32 accumulation, gfx950.
//
// Tiled forward with an online softmax: each workgroup owns BR = 32*NW query
// rows of one (batch, head) and streams key/value tiles of BC rows through
// LDS, keeping per row a running maximum m and a running sum l and rescaling
// the output accumulator when m grows, so the result equals the one-shot
// softmax (llmis.ru chapter 3.1 "The cost of attention", section 5; the
// unite.ai page "Flash Attention: Revolucionando a Eficiencia dos Modelos
// Transformer", sections "O Algoritmo de Flash Attention" and "A Matematica
// por tras da Flash Attention").  Only O and the per-row log-sum-exp are
// written; the score tile lives in registers.
//
// Data flow per wave (32 query rows):
//   S^T (keys x rows) = K_tile * Q^T     32x32x16 bf16 MFMA; K from LDS,
//                                        Q^T held in registers all along.
//   each lane owns one query row (lane % 32) and 16 keys per 32-key block,
//   so the row max/sum are in-lane reductions plus one swap with lane+32.
//   O^T (d x rows) += V_tile^T * P^T     P^T comes straight from the S^T
//                                        accumulator registers (converted to
//                                        bf16); V^T is read from LDS with the
//                                        gfx950 transpose read.
// Scores are handled in the base-2 domain: exp(scale*s) = 2^(scale*log2e*s).
#include "device_common.hpp"
#include "launch.hpp"

namespace exattn {
namespace {

// Lazy rescale threshold (log2 units): the running max used for the
// exponentials is only raised when a row's max exceeds it by more than this,
// so probabilities stay <= 2^8 and most tiles skip the O rescale.  The final
// normalisation uses the same max, so the result is unchanged.
constexpr float kRescaleThreshold = 8.0f;

// NW waves per workgroup (32 query rows each), BC keys per tile, WPE the
// waves per SIMD the register budget is sized for.
template <int D>
struct FwdCfg;
template <>
struct FwdCfg<64> {
  static constexpr int NW = 4, BC = 64, WPE = 2;
};
template <>
struct FwdCfg<128> {
  static constexpr int NW = 4, BC = 64, WPE = 2;
};
template <>
struct FwdCfg<256> {
  static constexpr int NW = 4, BC = 32, WPE = 1;
};

template <int D, bool WINDOWED>
__global__ __launch_bounds__(FwdCfg<D>::NW * 64, FwdCfg<D>::WPE) void fwd_bf16_kernel(
    const __bf16* __restrict__ Qg, const __bf16* __restrict__ Kg, const __bf16* __restrict__ Vg,
    __bf16* __restrict__ Og, float* __restrict__ LSEg, int n, int n_qblocks, int total_blocks,
    float scale_log2, int window) {
  constexpr int NW = FwdCfg<D>::NW;
  constexpr int BC = FwdCfg<D>::BC;
  constexpr int BR = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int NKB = BC / 32;  // 32-key blocks per tile
  constexpr int NDS = D / 16;   // 16-wide d steps
  constexpr int NDB = D / 32;   // 32-wide d blocks of the output

  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][BC * D];  // [buf][K/V]

  // XCD-aware block order: the hardware deals consecutive workgroups out to
  // the 8 XCDs in turn; remap so that each XCD gets a contiguous range of
  // (head, q-block) tiles and the q-blocks of one head share that XCD's L2.
  const int bid = xcd_remap(blockIdx.x, total_blocks);
  const int head = bid / n_qblocks;
  const int qb = bid - head * n_qblocks;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const size_t head_off = (size_t)head * n * D;
  const __bf16* Q = Qg + head_off;
  const __bf16* K = Kg + head_off;
  const __bf16* V = Vg + head_off;

  const int q0 = qb * BR;
  const int my_row = q0 + wave * 32 + l32;

  // Q^T operand, kept in registers: lane holds Q[my_row][16*ds + 8*hi .. +8].
  bf16x8 qreg[NDS];
  {
    const bool ok = my_row < n;
    const u32x4* src = (const u32x4*)(Q + (size_t)(ok ? my_row : 0) * D + 8 * hi);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      u32x4 v = ok ? src[2 * ds] : u32x4{0, 0, 0, 0};
      qreg[ds] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Key tiles this block visits (band of the whole block for a window).
  int k_lo = 0, k_hi = n;
  if constexpr (WINDOWED) {
    long a = (long)q0 - window, b = (long)q0 + BR - 1 + window + 1;
    k_lo = a < 0 ? 0 : (int)a;
    k_hi = b > n ? n : (int)b;
  }
  const int t_lo = k_lo / BC;
  const int t_hi = (k_hi + BC - 1) / BC;
  // keys visible to this lane's row
  int key_lo = 0, key_hi = n;
  if constexpr (WINDOWED) band_keys(my_row, my_row + 1, n, window, &key_lo, &key_hi);
  const unsigned key_span = (unsigned)max(key_hi - key_lo, 0);

  // Global -> register staging of one K and one V tile (coalesced 16 B loads).
  TileCopy<D, BC, NT> kcp, vcp;
  auto load_tile = [&](int t) {
    const int kbase = t * BC;
    kcp.load(K + (size_t)kbase * D, n - kbase, tid);
    vcp.load(V + (size_t)kbase * D, n - kbase, tid);
  };
  auto store_tile = [&](int buf) {
    kcp.store(smem[buf][0], tid);
    vcp.store(smem[buf][1], tid);
  };

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m_run = kNegInf;  // running max, log2 domain (scale*log2e*s)
  float l_part = 0.0f;    // this lane's share of the running sum

  if (t_lo < t_hi) {
    load_tile(t_lo);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_lo; t < t_hi; ++t) {
    const int buf = (t - t_lo) & 1;
    const bool has_next = t + 1 < t_hi;
    if (has_next) load_tile(t + 1);

    const __bf16* Ks = smem[buf][0];
    const __bf16* Vs = smem[buf][1];
    const int kbase = t * BC;

    // ---- S^T = K Q^T ------------------------------------------------------
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
      const int row = kb * 32 + l32;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        s[kb] = mfma32(lds_row_frag<D>(Ks, row, ds, hi), qreg[ds], s[kb]);
      }
    }

    // ---- masks: key tail and sliding window --------------------------------
    // Branch-free: one unsigned range test per element against this row's
    // visible keys [key_lo, key_hi).
    bool need_mask = kbase + BC > n;
    if constexpr (WINDOWED) {
      const int r_lo = q0 + wave * 32, r_hi = r_lo + 31;
      const int dist = max(r_hi - kbase, kbase + BC - 1 - r_lo);
      need_mask = need_mask || dist > window;
    }
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + kb * 32 + acc_row(r, lane);
          s[kb][r] = (unsigned)(key - key_lo) < key_span ? s[kb][r] : kNegInf;
        }
    }

    // ---- online softmax -----------------------------------------------------
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, swap_half(mx));
    const float mx2 = mx * scale_log2;  // -inf stays -inf
    const bool grow = mx2 > m_run + kRescaleThreshold || (m_run == kNegInf && mx2 != kNegInf);
    if (__any(grow)) {
      const float m_new = grow ? mx2 : m_run;
      const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;  // m_run=-inf -> 0
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_run = m_new;
    }
    const float msub = m_run == kNegInf ? 0.0f : m_run;

    bf16x8 pb[BC / 16];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -msub));
        l_part += s[kb][r];
      }
      pb[2 * kb] = acc_to_operand(s[kb], 0);
      pb[2 * kb + 1] = acc_to_operand(s[kb], 1);
    }

    // ---- O^T += V^T P^T -------------------------------------------------------
    // A operand (V^T): lane l needs V[key(t)][db*32 + l%32] with the keys in
    // the k order of pb (the transpose read delivers exactly that).
#pragma unroll
    for (int st = 0; st < BC / 16; ++st)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        o[db] = mfma32(lds_col_frag<D>(Vs, 16 * st, 32 * db, lane), pb[st], o[db]);

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) -----------------------
  const float l_tot = l_part + swap_half(l_part);
  if (my_row < n) {
    const float inv = 1.0f / l_tot;
    __bf16* Orow = Og + head_off + (size_t)my_row * D;
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

template <int D, bool W>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  constexpr int BR = 32 * FwdCfg<D>::NW;
  const int nqb = (p.n + BR - 1) / BR;
  const long total = (long)nqb * p.B * p.H;
  if (total > 0x7fffffffL) return hipErrorInvalidValue;
  const float scale_log2 = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, W>), dim3((unsigned)total), dim3(FwdCfg<D>::NW * 64), 0, stream,
                     (const __bf16*)p.q, (const __bf16*)p.k, (const __bf16*)p.v, (__bf16*)p.o, p.lse, p.n,
                     nqb, (int)total, scale_log2, p.window);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  const bool w = p.window >= 0;
  switch (p.d) {
    case 64: return w ? launch_d<64, true>(p, stream) : launch_d<64, false>(p, stream);
    case 128: return w ? launch_d<128, true>(p, stream) : launch_d<128, false>(p, stream);
    case 256: return w ? launch_d<256, true>(p, stream) : launch_d<256, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace exattn
