/*
 * exattn.h -- C ABI of the exact scaled dot-product attention library
 * (forward and backward) for AMD Instinct MI355X (gfx950).
 *
 * What is computed
 *   For every (batch b, head h), with Q, K, V, O, dO the (n, d) slices at
 *   (b, h):
 *     S   = scale * Q K^T                     (n x n, never stored)
 *     P   = row-softmax(S) over the keys each row may see
 *     O   = P V
 *     LSE = per-row natural log of sum_j exp(S_ij)
 *   and, for the backward, the gradients of L = sum(O * dO):
 *     dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
 *     dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *   The forward is the scaled dot-product attention of the llmis.ru chapter
 *   3.1 "The cost of attention", section 2; it is evaluated tile by tile with
 *   an online softmax (running row max and row sum, section 5 of the same
 *   chapter), so the n x n matrices S and P are never written to device
 *   memory.  The backward recomputes P from Q, K and the saved LSE instead of
 *   storing it (the unite.ai page "Flash Attention: Revolucionando a
 *   Eficiencia dos Modelos Transformer", section "Entenda a Flash Attention",
 *   item 2); its formulas are the chain rule of the forward definition.
 *
 * Sliding window
 *   window < 0 : every query row sees every key (no mask).
 *   window >= 0: row i sees keys j with |i - j| <= window (the Longformer
 *                local pattern of the llmis.ru chapter's section 3, read as
 *                symmetric and inclusive).  Key tiles that lie wholly outside
 *                a query tile's band are skipped, not computed.
 *
 * Grouped-query and multi-query attention (the *_gqa entry points)
 *   The attention variants the unite.ai page lists under "FlashAttention-2"
 *   (item 3): Hkv key/value heads, each shared by G = H / Hkv consecutive
 *   query heads.  Query head h of batch b attends with key/value head
 *   h / G of batch b; Hkv = 1 is multi-query attention and Hkv = H the plain
 *   multi-head case (the entry points without the suffix are exactly that).
 *   The gradient of a shared key/value head is the sum over its G query heads.
 *
 * Layout and types (all tensors are DEVICE pointers)
 *   Q, K, V, O, dO, dQ, dK, dV : contiguous row-major [B, H, n, d]; element
 *                                type `dtype` (EXATTN_F32 = float,
 *                                EXATTN_BF16 = bfloat16 bit patterns).
 *                                In the *_gqa calls K, V, dK, dV are
 *                                [B, Hkv, n, d].
 *   LSE                        : contiguous [B, H, n], float32, natural log.
 *   workspace                  : device scratch owned by the caller, at least
 *                                attn_bwd_workspace_bytes() bytes.
 *   Arithmetic: bf16 operands with fp32 accumulation and fp32 softmax
 *   statistics; probabilities and dS are rounded to bf16 before the matrix
 *   products that consume them.  The f32 type computes in fp32 throughout.
 *   Supported head dims d: 64, 128, 256.  Any n >= 1 (ragged tails masked).
 *
 * Ownership and execution
 *   The caller allocates and owns every buffer; the library allocates no
 *   device memory besides the fixed buffer of attn_bwd_noalloc, and keeps no
 *   pointer after a call returns.  Inputs are read only; outputs are
 *   completely overwritten (no need to clear them).  Every call only
 *   enqueues work on `stream` (a hipStream_t; NULL = the null stream) and
 *   returns without synchronising; a device fault surfaces at the caller's
 *   next synchronisation.  (The one exception, attn_bwd with a window, also
 *   uses a second stream of the device that it forks from `stream` and
 *   joins back before returning; see attn_bwd.)  Calls are reentrant; two
 *   calls that share an output or workspace buffer must be ordered by the
 *   caller.
 *
 * Errors (no exception crosses the ABI; nothing is launched on error)
 *   EXATTN_EINVAL       null pointer, B/H/n < 1, Hkv < 1 or not dividing H,
 *                       window < -1, non-finite or
 *                       non-positive scale, a pointer not 16-byte aligned,
 *                       an output buffer overlapping an input buffer, or a
 *                       problem of 2^31 rows (B*H*n) or more.
 *   EXATTN_EUNSUPPORTED d not in {64, 128, 256}, or an unknown dtype.
 *   EXATTN_EWORKSPACE   workspace smaller than attn_bwd_workspace_bytes().
 *   EXATTN_EHIP         the HIP runtime reported an error at launch.
 *   EXATTN_ESCRATCH     (attn_bwd_noalloc only) the problem needs more than
 *                       its fixed scratch buffer.
 */
#ifndef EXATTN_H
#define EXATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { EXATTN_F32 = 0, EXATTN_BF16 = 1 } exattn_dtype;

typedef enum {
  EXATTN_OK = 0,
  EXATTN_EINVAL = -1,
  EXATTN_EUNSUPPORTED = -2,
  EXATTN_EWORKSPACE = -3,
  EXATTN_EHIP = -4,
  EXATTN_ESCRATCH = -5
} exattn_status;

/*
 * Forward pass: O = softmax(scale * Q K^T) V and LSE, per (b, h).
 * Defined by: the llmis.ru chapter 3.1 "The cost of attention", section 2
 * (the attention formula); the running max and sum of its section 5 (and of
 * the unite.ai page's section "O Algoritmo de Flash Attention") give LSE as
 * the by-product m + ln(l) that the backward needs.
 *   dtype  : EXATTN_F32 or EXATTN_BF16 (type of Q, K, V and O).
 *   B, H, n, d : batch, heads, sequence length, head dim.
 *   Q, K, V: inputs [B, H, n, d].
 *   scale  : multiplier of Q K^T (normally 1/sqrt(d)); finite, > 0.
 *   window : -1 for full attention, else the half-width w of |i - j| <= w.
 *   O      : output [B, H, n, d], same dtype as the inputs.
 *   LSE    : output [B, H, n] float32, m_i + ln(l_i) per row.
 *   stream : hipStream_t to enqueue on.
 * Returns an exattn_status.
 */
int attn_fwd(int dtype, int B, int H, int n, int d,
             const void *Q, const void *K, const void *V,
             float scale, int window,
             void *O, float *LSE,
             void *stream);

/*
 * Bytes of device workspace that attn_bwd needs for this problem (the row
 * term D of the softmax's chain rule, llmis.ru chapter 3.1 section 2
 * differentiated, and the saved LSE in base 2): two fp32
 * row arrays of [B, H, n] (-D, the negated D = rowsum(dO * O), and
 * LSE * log2(e), the base-2 log-sum-exp the gradient kernels use), each
 * starting on a 256-byte boundary.  Returns 0 for arguments that attn_bwd would reject.
 */
size_t attn_bwd_workspace_bytes(int dtype, int B, int H, int n, int d);

/*
 * Backward pass: gradients of sum(O * dO) with respect to Q, K and V.
 * Defined by: the chain rule of the llmis.ru chapter 3.1 section 2
 * definition (the pages print no backward formulas), evaluated the way the
 * unite.ai page's section "Entenda a Flash Attention", item 2, and the
 * llmis.ru section 5 describe: P is recomputed from Q, K and LSE instead of
 * being read back, so no n x n matrix reaches device memory.
 *   Q, K, V : the forward's inputs; O and LSE: the forward's outputs for
 *             exactly these inputs, scale and window (P is recomputed from
 *             them, so a mismatched O or LSE gives wrong gradients).
 *   dO      : upstream gradient [B, H, n, d], same dtype.
 *   dQ, dK, dV : outputs [B, H, n, d], same dtype; fully overwritten.
 *   workspace, workspace_bytes : caller-owned device scratch, at least
 *             attn_bwd_workspace_bytes(); its contents on entry are ignored
 *             and on return are unspecified.
 *   stream  : hipStream_t to enqueue on.  With a window (bf16, outside
 *             graph capture) the dK/dV stage runs on a second stream of the
 *             same device that the library creates on first use (default
 *             priority); it is forked from `stream` after the rowdot stage
 *             and joined back before the call returns, so all of the call's
 *             work is ordered on `stream` as if it ran there alone.
 * Returns an exattn_status.
 */
int attn_bwd(int dtype, int B, int H, int n, int d,
             const void *Q, const void *K, const void *V,
             const void *O, const void *dO, const float *LSE,
             float scale, int window,
             void *dQ, void *dK, void *dV,
             void *workspace, size_t workspace_bytes,
             void *stream);

/*
 * The backward as three stages, each exactly one kernel launch; attn_bwd is
 * these three (rowdot, then dK/dV and dQ on two streams with a window, else
 * in order on one stream).  Stage 1 must complete before stages
 * 2 and 3 (stream order does it); stages 2 and 3 are independent of each
 * other (they may run on two streams once stage 1 is done) and either may
 * be skipped when its gradients are not wanted.  Arguments mean what they
 * mean for attn_bwd; `workspace` carries D from stage 1 to stages 2 and 3
 * and must not be modified in between.
 *
 * attn_bwd_rowdot: -D_i, the negated D_i = sum_k dO_ik * O_ik, and
 * LSE_i * log2(e) (fp32, into the workspace; LSE is the forward's [B, H, n]
 * output).  D is stored negated because the gradient kernels start the
 * accumulator of their dP = dO V^T product at -D, which leaves dP - D.
 */
int attn_bwd_rowdot(int dtype, int B, int H, int n, int d,
                    const void *O, const void *dO, const float *LSE,
                    void *workspace, size_t workspace_bytes,
                    void *stream);

/* attn_bwd_dkdv: dK and dV (key-side pass: each workgroup owns a block of
 * keys and sweeps the query tiles of its band).  dV = P^T dO and
 * dK = scale dS^T Q of the chain rule described at attn_bwd. */
int attn_bwd_dkdv(int dtype, int B, int H, int n, int d,
                  const void *Q, const void *K, const void *V,
                  const void *dO, const float *LSE,
                  float scale, int window,
                  void *dK, void *dV,
                  const void *workspace, size_t workspace_bytes,
                  void *stream);

/* attn_bwd_dq: dQ (query-side pass: each workgroup owns a block of query
 * rows and sweeps the key tiles of its band, recomputing P and dP).
 * dQ = scale dS K of the chain rule described at attn_bwd. */
int attn_bwd_dq(int dtype, int B, int H, int n, int d,
                const void *Q, const void *K, const void *V,
                const void *dO, const float *LSE,
                float scale, int window,
                void *dQ,
                const void *workspace, size_t workspace_bytes,
                void *stream);

/*
 * attn_bwd_noalloc: attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, meaning, kernels and results (bit for bit) as
 * attn_bwd, minus the workspace: the rowdot stage's two fp32 row arrays go
 * to a fixed device buffer of EXATTN_NOALLOC_SCRATCH_BYTES (16 MiB) that the
 * library holds on each GPU it runs on until the process ends.  The call
 * makes no hipMalloc/hipFree and no allocating library call, and enqueues
 * everything on `stream` (no second stream, with or without a window).  Problems whose
 * attn_bwd_workspace_bytes() exceeds the buffer (B*H*n > 2^21 rows) return
 * EXATTN_ESCRATCH with nothing launched.  All calls on one GPU share its
 * buffer: two calls that may overlap on one GPU (different streams, or
 * different threads without ordering) race and must be ordered by the caller.
 * The buffer keeps the last call's contents; every row a call reads is
 * written by that call first, so nothing needs clearing.
 */
#define EXATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

int attn_bwd_noalloc(int dtype, int B, int H, int n, int d,
                     const void *Q, const void *K, const void *V,
                     const void *O, const void *dO, const float *LSE,
                     float scale, int window,
                     void *dQ, void *dK, void *dV,
                     void *stream);

/*
 * Grouped-query variants (the grouped-query and multi-query attention the
 * unite.ai page lists under "FlashAttention-2", item 3, without formulas;
 * read as below): as attn_fwd, attn_bwd, attn_bwd_dkdv and
 * attn_bwd_dq, with Hkv key/value heads (1 <= Hkv <= H, H % Hkv == 0);
 * K, V, dK and dV are [B, Hkv, n, d], everything else keeps its [B, H, ...]
 * shape.  The workspace is the same as for H heads
 * (attn_bwd_workspace_bytes(dtype, B, H, n, d)), and attn_bwd_rowdot serves
 * as stage 1 unchanged.  attn_bwd_dkdv_gqa writes each dK/dV row once: the
 * workgroup that owns a block of keys sweeps the query tiles of all G query
 * heads of the group, so the group sum needs no atomics.
 */
int attn_fwd_gqa(int dtype, int B, int H, int Hkv, int n, int d,
                 const void *Q, const void *K, const void *V,
                 float scale, int window,
                 void *O, float *LSE,
                 void *stream);

int attn_bwd_gqa(int dtype, int B, int H, int Hkv, int n, int d,
                 const void *Q, const void *K, const void *V,
                 const void *O, const void *dO, const float *LSE,
                 float scale, int window,
                 void *dQ, void *dK, void *dV,
                 void *workspace, size_t workspace_bytes,
                 void *stream);

int attn_bwd_dkdv_gqa(int dtype, int B, int H, int Hkv, int n, int d,
                      const void *Q, const void *K, const void *V,
                      const void *dO, const float *LSE,
                      float scale, int window,
                      void *dK, void *dV,
                      const void *workspace, size_t workspace_bytes,
                      void *stream);

int attn_bwd_dq_gqa(int dtype, int B, int H, int Hkv, int n, int d,
                    const void *Q, const void *K, const void *V,
                    const void *dO, const float *LSE,
                    float scale, int window,
                    void *dQ,
                    const void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * Sparse attention patterns (the Longformer and BigBird patterns of the
 * llmis.ru chapter 3.1 "The cost of attention", section 3).  The pattern is
 * the union of three parts, shared by every (batch, head):
 *   - a sliding window: row i sees key j when |i - j| <= window
 *     (window = -1: no window part);
 *   - global tokens: a global position attends to every key, and every
 *     query attends to it (Longformer's task tokens);
 *   - a block layout: with 64-token blocks, row i sees key j when
 *     layout[(i / 64) * nb + j / 64] != 0, nb = ceil(n / 64) (BigBird's
 *     local, global and random blocks are all entries of the layout; random
 *     blocks are drawn by the caller).
 * Attention over the pattern is the softmax over the visible keys only.  A
 * row that sees no key (possible only without a window) gets O = 0 and
 * LSE = -inf and contributes no gradient.
 *
 * The descriptor is read on the host; its arrays are DEVICE pointers:
 *   global_idx : n_global int32 positions (any order; duplicates allowed;
 *                positions outside [0, n) are ignored), 4-byte aligned.
 *   layout     : nb * nb bytes, row-major (ignored when layout_block = 0).
 */
typedef struct {
  int window;                  /* >= 0: band half-width; -1: no band part */
  int n_global;                /* number of global positions (0: none) */
  const int *global_idx;       /* device: the global positions */
  int layout_block;            /* 0: no layout; 64: block layout present */
  const unsigned char *layout; /* device: nb x nb block layout */
} exattn_pattern;

/*
 * Workspace for attn_fwd_pattern and attn_bwd_pattern (patterns of the
 * llmis.ru chapter 3.1 section 3, see above): the global-token
 * bitmap, the full positions (query rows that see every key: global tokens
 * and rows whose layout row is set in every block; keys that every row sees,
 * likewise) with their index lists, each kernel's per-workgroup tile lists
 * (all built on the device by every call, in stream order, before the
 * attention kernels), a scratch region (about B*H*n*(4d+8) bytes) that holds,
 * in turn, the copies of the other side's full positions each pass reads
 * and the partial results of the full positions' passes, and the backward's
 * row arrays.  Returns 0 for arguments the calls would reject.
 */
size_t attn_pattern_workspace_bytes(int dtype, int B, int H, int n, int d);

/*
 * Forward and backward over a sparse pattern (llmis.ru chapter 3.1 section
 * 3; their block-sparse I/O is the subject of Theorem 4.5 in the
 * gist.science summary of arXiv 2410.09397, section "Contribuicoes
 * Principais e Resultados", item 2); arguments as for attn_fwd and
 * attn_bwd (multi-head layout [B, H, n, d]), with the pattern in place of
 * the window.  Only EXATTN_BF16 is supported (EXATTN_EUNSUPPORTED for f32).
 * The workgroups visit only the tiles that hold a visible pair; tiles the
 * pattern covers completely run unmasked.  Full positions (see above) are
 * computed by a pass of their own, split over chunks of the other side whose
 * partial results are merged in a fixed order, so every call is
 * deterministic.  The backward's O and LSE must
 * come from attn_fwd_pattern with the same pattern.  Besides the errors of
 * attn_fwd / attn_bwd: EXATTN_EINVAL for a NULL descriptor, window < -1,
 * n_global < 0, a NULL or misaligned global_idx with n_global > 0, a NULL
 * layout with layout_block = 64, or an output overlapping global_idx or
 * layout; EXATTN_EUNSUPPORTED for a layout_block other than 0 or 64.
 */
int attn_fwd_pattern(int dtype, int B, int H, int n, int d,
                     const void *Q, const void *K, const void *V,
                     float scale, const exattn_pattern *pattern,
                     void *O, float *LSE,
                     void *workspace, size_t workspace_bytes,
                     void *stream);

int attn_bwd_pattern(int dtype, int B, int H, int n, int d,
                     const void *Q, const void *K, const void *V,
                     const void *O, const void *dO, const float *LSE,
                     float scale, const exattn_pattern *pattern,
                     void *dQ, void *dK, void *dV,
                     void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * FP8 forward (FlashAttention-3's FP8 support and "incoherent processing",
 * the unite.ai page's section "FlashAttention-3", items 2 and 3).  Format:
 * OCP E4M3 (largest finite 448), one scale per (batch, head) and tensor.
 *
 * attn_quant_fp8 quantises a bf16 [B, H, n, d] tensor (d = 64 or 128): with
 * `signs` (a device array of d floats, each +1 or -1) every row is first
 * multiplied by the signs and transformed by the Sylvester Hadamard matrix
 * H of order d (a fast Walsh-Hadamard transform; H H^T = d I); then
 * scale[b, h] = amax / 448 over the head (1 for an all-zero head) and each
 * code is E4M3(clamp(x * 448 / amax, -448, 448)), rounded to nearest even.
 * `layout` EXATTN_FP8_ROWS writes [B, H, n, d] (for Q and K);
 * EXATTN_FP8_V_TRANSPOSED writes V's layout for attn_fwd_fp8: [B, H, d, n128]
 * with n128 = n rounded up to a multiple of 128, and within every 64-key
 * group key 32*kb + 8*a + 4*h + c (kb, h in {0,1}; a, c in {0..3}) stored
 * at column 32*h + 16*kb + 4*a + c (the order in which the forward's score
 * accumulators hold the keys); columns at or beyond n are zero.
 * attn_fp8_bytes returns the byte size of either layout (0 if invalid).
 *
 * attn_fwd_fp8 (d = 64 or 128): O = softmax(S) V with
 *   S = scale / (rotated ? d : 1) * q_scale * k_scale * Q8 K8^T,
 *   V = v_scale * V8,
 * both products on the FP8 matrix cores with fp32 accumulation; the
 * probabilities are rounded to E4M3 before the P V product.  Q and K must
 * have been quantised with the same signs (rotated = 1) or both without
 * (rotated = 0); V without.  O is bf16 [B, H, n, d], LSE fp32 [B, H, n].
 * Errors: EXATTN_EINVAL for null or misaligned pointers (16 bytes; 4 for
 * the scale and sign arrays), a bad layout or rotated flag, or overlapping
 * outputs; EXATTN_EUNSUPPORTED for d other than 64 or 128.
 */
typedef enum { EXATTN_FP8_ROWS = 0, EXATTN_FP8_V_TRANSPOSED = 1 } exattn_fp8_layout;

size_t attn_fp8_bytes(int B, int H, int n, int d, int layout);

int attn_quant_fp8(int B, int H, int n, int d,
                   const void *X, const float *signs, int layout,
                   void *X8, float *scale,
                   void *stream);

int attn_fwd_fp8(int B, int H, int n, int d,
                 const void *Q8, const void *K8, const void *V8t,
                 const float *q_scale, const float *k_scale, const float *v_scale,
                 float scale, int rotated,
                 void *O, float *LSE,
                 void *stream);

/* Static, NUL-terminated description of a status code (never NULL); the
 * codes are this library's own convention (the pages define none). */
const char *exattn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXATTN_H */
