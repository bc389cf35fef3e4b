/*
 * rmm.h -- C ABI of librmm, Reduced Matrix Multiplication (RMM) on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (sources are the public pages about the paper "Reduced Matrix
 * Multiplication: Input-Adaptive Matrix-Product Reduction for LLM
 * Inference"):
 *   For Y = A B with A (n x d) activations and B (d x m), score every
 *   contraction index j by the L2 norm of column j of A over all n rows,
 *   keep the k = ceil(rho d) largest, and multiply over the kept slice only:
 *   Y = A[:, I] B[I, :].
 *   -- "Algorithm Deep-Dive: RMM" (hackcv.com), Core Approach (Formula
 *      Level): Contraction-Dimension TopK Selection and the importance score;
 *      gist.science technical summary, Methodology: Selection Strategy.
 *   The same rule covers linear / MLP projections (contraction over the
 *   hidden dim), Q K^T (per query head, over the head feature dim, K of the
 *   shared kv head gathering the same dims) and P V (over key positions).
 *   -- hackcv.com, Core Approach: Component mapping.
 *
 * Readings fixed by this library where the pages are silent:
 *   - k = ceil(rho d) with rho read as the decimal it was written as: a
 *     product within 1e-9 relative of an integer is that integer (rmm_k).
 *   - Ranking key is the fp32 sum of squares of the stored values (same
 *     order as the norm).  Equal keys: the lower index wins.  The kept set
 *     is written in ascending index order.
 *   - One kept set per call over all rows of A; one per head for QK / PV.
 *   - GQA: query head h reads K/V head h / (hq / hkv).
 *   - Q K^T is the raw product with no 1/sqrt(dh) scale (the softmax
 *     entry point takes the scale); rmm_qk applies no mask, rmm_qk_causal
 *     the causal one.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     allocates nothing and keeps no state between calls; scratch memory is
 *     the caller's workspace (size from the matching *_workspace query).
 *   - Matrices are row-major with unit inner stride; leading dimensions and
 *     head strides are in ELEMENTS.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream); outputs are valid once the stream reaches that point.  The
 *     calls never synchronise the host.
 *   - Every argument is checked before any work is queued: a call that
 *     returns an argument error (anything but RMM_ERR_HIP) has queued
 *     nothing and written nothing.  RMM_ERR_HIP means the runtime refused a
 *     launch; earlier stages of that call may already be queued.
 *     Overlapping calls on different streams must use different workspaces.
 *   - Results are bitwise reproducible for identical inputs and shapes
 *     (fixed reduction order, no floating-point atomics).
 *   - Floating-point inputs are expected finite; results for NaN / Inf
 *     inputs are unspecified (but the call completes).
 *   - Sizes: every dimension in [1, 2^31); per-head operands must stay below
 *     2 GiB (matrix-core loaders use 32-bit byte offsets).
 *   - bf16 products run on the matrix cores (bf16 x bf16, fp32 accumulate);
 *     fp32 products run on the vector ALUs in fp32.
 */
#ifndef RMM_H_
#define RMM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RMM_OK = 0,
  RMM_ERR_NULL = 1,      /* a required pointer is NULL */
  RMM_ERR_RHO = 2,       /* rho not finite or outside (0, 1] */
  RMM_ERR_SHAPE = 3,     /* a dimension < 1, a leading dim too small, hq % hkv != 0, or a size limit */
  RMM_ERR_DTYPE = 4,     /* unsupported dtype or dtype combination */
  RMM_ERR_ALIGN = 5,     /* pointer not aligned to its element size */
  RMM_ERR_WORKSPACE = 6, /* workspace NULL / too small / not 256-byte aligned */
  RMM_ERR_HIP = 7,       /* the HIP runtime refused a launch */
  RMM_ERR_ALIAS = 8      /* an output overlaps an input or another output */
} rmm_status_t;

typedef enum { RMM_FP32 = 0, RMM_BF16 = 1 } rmm_dtype_t;

/* Operations, for the generic workspace query rmm_workspace_bytes. */
typedef enum {
  RMM_OP_SELECT = 0,          /* rmm_select, rmm_select_retained */
  RMM_OP_MATMUL = 1,          /* rmm_matmul (+ _timed) */
  RMM_OP_QK = 2,              /* rmm_qk, rmm_qk_causal (+ _timed) */
  RMM_OP_PV = 3,              /* rmm_pv (+ _timed) */
  RMM_OP_MATMUL_W8 = 4,       /* rmm_matmul_w8 (+ _timed) */
  RMM_OP_MATMUL_IDX = 5,      /* rmm_matmul_idx */
  RMM_OP_SOFTMAX_ENERGY = 6,  /* rmm_softmax_energy */
  RMM_OP_PV_ENERGY = 7,       /* rmm_pv_energy */
  RMM_OP_SOFTMAX_SELECT = 8,  /* rmm_softmax_select */
  RMM_OP_PV_IDX = 9           /* rmm_pv_idx */
} rmm_op_t;

/* Number of kept indices, ceil(rho * d) under the decimal reading above;
 * -1 when rho is not finite, rho <= 0, rho > 1 or d < 1.
 * hackcv.com "Algorithm Deep-Dive: RMM", Core Approach and the
 * retention-ratio section (rho in (0, 1]). */
int64_t rmm_k(double rho, int64_t d);

/* Static, human-readable name of a status code. */
const char* rmm_status_str(int status);

/* Workspace bytes that suffice for every call of operation `op` (an
 * rmm_op_t) of the given sizes, whatever rho in (0, 1], dtypes, strides and
 * pointer alignment the call uses: an upper bound of the matching per-call
 * query (rmm_*_workspace), which gives the exact need of one configuration.
 * The pages define the operator (RMM_rho(A, B) with the retention ratio rho;
 * hackcv.com, Core Approach and the retention-ratio section) and say it
 * wraps the attention and FFN operators (hackcv.com, Engineering Notes);
 * the sizes that bound an operation's scratch are:
 *   RMM_OP_SELECT          n_or_heads = n rows, d = contraction length, m unused
 *   RMM_OP_MATMUL, _W8     n_or_heads = n rows of A, d, m = columns of B
 *   RMM_OP_MATMUL_IDX      n_or_heads = n, d = length of the index list, m
 *   RMM_OP_QK              n_or_heads = hq, d = head dim, m >= max(tq, tk)
 *   RMM_OP_PV, _PV_ENERGY  n_or_heads = h, d = tk (key positions), m >= max(tq, dv)
 *   RMM_OP_SOFTMAX_ENERGY  n_or_heads = h, d = tk, m = tq
 *   RMM_OP_SOFTMAX_SELECT  n_or_heads = h, d = tk, m = tq
 *   RMM_OP_PV_IDX          n_or_heads = h, d = length of each list, m >= max(tq, dv)
 * Returns 0 for an unknown op or a size outside [1, 2^31) (and for
 * softmax rows longer than the softmax pass takes).  Pure host arithmetic:
 * no device call, no allocation. */
size_t rmm_workspace_bytes(int op, int64_t n_or_heads, int64_t d, int64_t m);

/* ---------------------------------------------------------------------
 * rmm_select: the kept index set of A alone.
 *   A       [n x d] (lda >= d), fp32 or bf16.
 *   idx     [k] int32, written ascending, k = rmm_k(rho, d).
 *   scores  optional [d] fp32: s_j = sqrt(fp32 sum of squares of column j);
 *           NULL to skip.
 * Score and TopK: hackcv.com, Core Approach (the importance score and TopK).
 * ------------------------------------------------------------------- */
size_t rmm_select_workspace(int64_t n, int64_t d, int dtype);
rmm_status_t rmm_select(const void* A, int dtype, int64_t n, int64_t d, int64_t lda, double rho,
                        int32_t* idx, float* scores, void* workspace, size_t workspace_bytes, void* stream);

/* rmm_select plus the retained fraction of the activation energy,
 * *retained = (sum over kept j of q_j) / (sum over all j of q_j) in [0, 1]
 * (fp64 sums of the fp32 energies, fixed order; 1 when all are kept).
 * retained: one float in device memory.  Source: hackcv.com, "Attention
 * vs MLP: structural asymmetry" (the supplementary figures quote the
 * retained activation energy of each reduced component); kaelemshawn.blog,
 * the compute-normalized component analysis (same figures).
 * Workspace: rmm_select_workspace(n, d, dtype) bytes. */
rmm_status_t rmm_select_retained(const void* A, int dtype, int64_t n, int64_t d, int64_t lda, double rho,
                                 int32_t* idx, float* scores, float* retained, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * rmm_matmul: Y = A[:, I] B[I, :] with I = rmm_select(A, rho).
 *   A   [n x d] activations (lda >= d), B [d x m] (ldb >= m); both `dtype`.
 *   idx [k] int32 ascending (always written; 0..d-1 when rho = 1).
 *   Y   [n x m] (ldy >= m), y_dtype fp32 or bf16.
 * rho = 1 computes the dense product with no scoring pass.
 * n <= 16 with bf16 takes the decode path (GEMV over the kept rows of B;
 * with rho < 1 and d <= 8192 it ranks A itself, and the first rows of each
 * of its slices of B are requested while it ranks, dropped ones included).
 * Source: hackcv.com, Core Approach: RMM_rho(A, B) = A[:, I] B[I, :];
 * linear / MLP mapping from the Component mapping paragraph.
 * ------------------------------------------------------------------- */
size_t rmm_matmul_workspace(int64_t n, int64_t d, int64_t m, int64_t lda, int dtype, double rho);
rmm_status_t rmm_matmul(const void* A, const void* B, int dtype, int64_t n, int64_t d, int64_t m, int64_t lda,
                        int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype, int64_t ldy,
                        void* workspace, size_t workspace_bytes, void* stream);

/* rmm_matmul for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as rmm_matmul minus the workspace: the call's
 * scratch lives in a fixed array of 32 MiB inside the library, one per GPU
 * (reserved when the library's code is first loaded on that GPU and held
 * until the process ends).  The call allocates nothing and calls no
 * allocating routine.  The first call on a device looks up that device's
 * array (the calling thread's current device must be the device of `stream`
 * and of the operands).  A call whose rmm_matmul_workspace need exceeds 32
 * MiB is refused with RMM_ERR_WORKSPACE before anything is queued (e.g. the
 * packed prefill path needs about 2 n ceil(rho d) bytes; the decode path,
 * n <= 16, needs under 4 MiB for d, m <= 16384).  Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (different streams, or
 * host threads) race and must be serialised by the caller. */
rmm_status_t rmm_matmul_noalloc(const void* A, const void* B, int dtype, int64_t n, int64_t d, int64_t m,
                                int64_t lda, int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype,
                                int64_t ldy, void* stream);

/* Instrumented rmm_matmul: the same computation, and in addition records
 * five caller-created HIP events (hipEvent_t, timing enabled) on `stream`
 * at the stage boundaries: [0] before scoring, [1] before TopK, [2] before
 * the gather-pack, [3] before the product kernel, [4] after it.  A stage a
 * path does not run leaves its two events back to back; where one launch
 * ranks and gathers (prefill with bf16 rows of whole 16-byte pieces and
 * d <= 15360), [1] to [2] brackets it and [2], [3] are back to back.  For
 * per-kernel timing by benchmarks; stage_events and its five entries must be
 * non-NULL. */
rmm_status_t rmm_matmul_timed(const void* A, const void* B, int dtype, int64_t n, int64_t d, int64_t m, int64_t lda,
                              int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype, int64_t ldy,
                              void* workspace, size_t workspace_bytes, void* stream, void* const* stage_events);

/* ---------------------------------------------------------------------
 * rmm_matmul_w8: the reduced product with int8 weights,
 *   Y[i][c] = scale[c] * sum over t < k of A[i][I_t] Bq[I_t][c],
 * i.e. A[:, I] (Bq[I, :] diag(scale)) with I selected from A exactly as in
 * rmm_matmul.  The weights are symmetric per-output-channel int8 (one fp32
 * scale per column of B): hackcv.com, "Compatibility & generalization"
 * (RMM combines with INT8 weights), and gist.science, Experimental Results
 * (the compatibility item on INT8 weight quantisation); neither page gives the
 * quantisation scheme, so this per-channel form is the one fixed here.
 *   A      bf16 (a_dtype must be RMM_BF16), row-major, lda >= d.
 *   Bq     int8 [d][ldb] row-major, ldb >= m, Bq 8-byte aligned, and m and
 *          ldb multiples of 8.  Values in [-128, 127], widened to bf16
 *          exactly on the device.
 *   scale  fp32 [m], device.
 *   idx, Y, y_dtype, ldy, rho as in rmm_matmul (n <= 16 runs the GEMV over
 *   the kept rows of Bq: half the bytes of bf16 weights).
 *   Workspace: rmm_matmul_w8_workspace(n, d, m, lda, rho) bytes, 256-byte
 *   aligned (0 means none needed).
 * Errors as rmm_matmul; RMM_ERR_DTYPE for an A that is not bf16,
 * RMM_ERR_SHAPE for m or ldb not a multiple of 8, RMM_ERR_ALIGN for a
 * misaligned Bq, scale, idx or Y.
 * ------------------------------------------------------------------- */
size_t rmm_matmul_w8_workspace(int64_t n, int64_t d, int64_t m, int64_t lda, double rho);
rmm_status_t rmm_matmul_w8(const void* A, int a_dtype, const int8_t* Bq, const float* scale, int64_t n, int64_t d,
                           int64_t m, int64_t lda, int64_t ldb, double rho, int32_t* idx, void* Y, int y_dtype,
                           int64_t ldy, void* workspace, size_t workspace_bytes, void* stream);
/* rmm_matmul_w8 with the five stage events of rmm_matmul_timed. */
rmm_status_t rmm_matmul_w8_timed(const void* A, int a_dtype, const int8_t* Bq, const float* scale, int64_t n,
                                 int64_t d, int64_t m, int64_t lda, int64_t ldb, double rho, int32_t* idx, void* Y,
                                 int y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* stage_events);

/* ---------------------------------------------------------------------
 * rmm_matmul_idx: Y = sum over t < k of A[:, idx[t]] B[idx[t], :], the
 * reduced product over an index set the caller supplies (for instance one
 * rmm_select on X reused for the Q, K and V projections, or a random set
 * of the same size as an ablation of the norm-based choice).
 *   A, B, Y as in rmm_matmul; idx: k int32 device values in any order.
 *   An entry outside [0, d) contributes nothing; a repeated entry
 *   contributes once per occurrence.
 *   Workspace: rmm_matmul_idx_workspace(n, k, m, dtype) bytes, 256-byte
 *   aligned (always needed: the padded copy of idx lives there).
 * Source: hackcv.com, Core Approach (Formula Level): RMM_rho(A, B) =
 * A[:, I] B[I, :] for the kept set I; gist.science, Selection Strategy (the
 * random-selection comparison uses a set of the same size).
 * ------------------------------------------------------------------- */
size_t rmm_matmul_idx_workspace(int64_t n, int64_t k, int64_t m, int dtype);
rmm_status_t rmm_matmul_idx(const void* A, const void* B, int dtype, int64_t n, int64_t d, int64_t m, int64_t lda,
                            int64_t ldb, const int32_t* idx, int64_t k, void* Y, int y_dtype, int64_t ldy,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * rmm_qk: per query head h, S[h] = Q[h][:, I_h] K[g(h)][:, I_h]^T with
 * I_h the ceil(rho dh) head-feature dims of largest column norm of Q[h]
 * over its tq rows, g(h) = h / (hq / hkv).
 *   Q   element (h, t, f) at Q[h*q_hs + t*q_ts + f]; K likewise with k_hs,
 *       k_ts.  Q and K share `dtype` (fp32 or bf16).
 *   idx [hq][k] int32, each row ascending, k = rmm_k(rho, dh).
 *   S   [hq][tq][tk] contiguous, s_dtype fp32 or bf16.
 * With bf16 Q and K, at most 8 query rows per kv head ((hq / hkv) * tq),
 * dh a multiple of 8 up to 256 and 16-byte aligned K rows (decode), the
 * selection and the product run in one streaming pass over K; otherwise
 * the column energies, TopK, packs of Q and K and a batched matrix-core
 * product (with bf16 heads of at most 256 features and 16-byte aligned rows,
 * TopK and both packs are one launch).
 * Source: hackcv.com, Component mapping (QK^T over the head feature dim,
 * selection on Q, K gathers the matching dims under GQA).
 * ------------------------------------------------------------------- */
size_t rmm_qk_workspace(int64_t hq, int64_t tq, int64_t tk, int64_t dh, int dtype, double rho);
rmm_status_t rmm_qk(const void* Q, const void* K, int dtype, int64_t hq, int64_t hkv, int64_t tq, int64_t tk,
                    int64_t dh, int64_t q_hs, int64_t q_ts, int64_t k_hs, int64_t k_ts, double rho,
                    int32_t* idx, void* S, int s_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* rmm_qk with the five stage events of rmm_matmul_timed recorded on `stream`
 * ([0] start, [1] after the column energies, [2] after TopK, [3] after the
 * packs of Q and K, [4] after the batched product; when TopK and the packs
 * are one launch, [2] follows it and [3] follows [2]).  Same arguments,
 * results and errors as rmm_qk; stage_events and its entries non-NULL. */
rmm_status_t rmm_qk_timed(const void* Q, const void* K, int dtype, int64_t hq, int64_t hkv, int64_t tq, int64_t tk,
                          int64_t dh, int64_t q_hs, int64_t q_ts, int64_t k_hs, int64_t k_ts, double rho,
                          int32_t* idx, void* S, int s_dtype, void* workspace, size_t workspace_bytes, void* stream,
                          void* const* stage_events);

/* Causal rmm_qk, for prefill over a key cache: the tq queries are the last
 * tq of the tk key positions (tq <= tk), so query row r sees keys
 * t <= r + tk - tq and S[h][r][t] = -inf (fp32 or bf16) for every later t.
 * "Algorithm Deep-Dive: RMM" (hackcv.com), Component mapping: the kept
 * features I_h still come from the column norms of Q[h] over all tq rows;
 * the mask acts on the scores only.  Tiles of S that lie wholly above the
 * shifted diagonal store -inf (small launches skip their product; large
 * ones, bound by the store of S, multiply every tile alike).  Arguments, idx,
 * workspace (rmm_qk_workspace) and errors as rmm_qk, and RMM_ERR_SHAPE when
 * tq > tk.  The scores go straight to rmm_softmax_energy. */
rmm_status_t rmm_qk_causal(const void* Q, const void* K, int dtype, int64_t hq, int64_t hkv, int64_t tq, int64_t tk,
                           int64_t dh, int64_t q_hs, int64_t q_ts, int64_t k_hs, int64_t k_ts, double rho,
                           int32_t* idx, void* S, int s_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * rmm_pv: per head h, O[h] = P[h][:, I_h] V[g(h)][I_h, :] with I_h the
 * ceil(rho tk) key positions of largest column norm of P[h] over its tq
 * query rows, g(h) = h / (h_count / hkv).
 *   P   element (h, q, t) at P[h*p_hs + q*p_ts + t], p_dtype fp32 or bf16.
 *   V   element (g, t, c) at V[g*v_hs + t*v_ts + c], v_dtype bf16 or fp32.
 *       bf16 V uses the matrix cores and rounds P to bf16 (nearest even);
 *       fp32 V requires fp32 P and runs in fp32.  With bf16 V, P 16-byte
 *       aligned, tk a multiple of 64 and at least one key in eight kept,
 *       the product reads P in place over all tk positions with the
 *       dropped rows of V read as zeros (the same sum over I_h; P is
 *       bandwidth-bound either way); otherwise the kept columns of P are
 *       packed first.  tq <= 16 with bf16 V (decode) runs a GEMV per head
 *       that reads only the kept rows of V.
 *   idx [h][k] int32, each row ascending, k = rmm_k(rho, tk).
 *   O   [h][tq][dv] contiguous, o_dtype fp32 or bf16.
 * Source: hackcv.com, Component mapping (PV optionally over token
 * positions); kaelemshawn.blog, section on where RMM cuts inside the
 * Transformer (column norm of P over the history positions).
 * ------------------------------------------------------------------- */
size_t rmm_pv_workspace(int64_t h, int64_t tq, int64_t tk, int64_t dv, int p_dtype, int v_dtype, double rho);
rmm_status_t rmm_pv(const void* P, int p_dtype, const void* V, int v_dtype, int64_t h, int64_t hkv, int64_t tq,
                    int64_t tk, int64_t dv, int64_t p_hs, int64_t p_ts, int64_t v_hs, int64_t v_ts, double rho,
                    int32_t* idx, void* O, int o_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Producer-side scoring for PV: the pass that writes P also emits the
 * column energies that PV selects on, so PV never reads P twice.
 * Source: kaelemshawn.blog, section on where RMM cuts inside the
 * Transformer (PV keys scored by the column norm of P over the history
 * positions); hackcv.com, Core Approach (scores are column L2 norms).
 *
 * rmm_softmax_energy: for every head h and query row i,
 *   P[h][i][:] = softmax(scale * L[h][i][:]) (max subtracted; fp32; scale
 *   finite and > 0, e.g. 1/sqrt(head dim) for raw QK^T scores), and
 *   energy[h][j] = sum over i of P[h][i][j]^2 (fixed order).
 *   L, P: fp32, element (h, i, j) at [h*hs + i*ts + j]; tk <= 16384;
 *   energy: [h][tk] fp32 contiguous.  Logits must be finite.  L and P may
 *   not overlap.  Workspace: rmm_softmax_energy_workspace(h, tq, tk) bytes.
 *
 * rmm_pv_energy: rmm_pv with the energies supplied (energy[h][tk], e.g. from
 *   rmm_softmax_energy over the same P) instead of computed from P: I_h is
 *   the ceil(rho tk) positions of largest energy[h][:], ties to the lowest
 *   index.  Same arguments, results and errors as rmm_pv otherwise;
 *   workspace: rmm_pv_energy_workspace(...).
 * ------------------------------------------------------------------- */
size_t rmm_softmax_energy_workspace(int64_t h, int64_t tq, int64_t tk);
rmm_status_t rmm_softmax_energy(const float* L, float scale, int64_t h, int64_t tq, int64_t tk, int64_t l_hs,
                                int64_t l_ts, float* P, int64_t p_hs, int64_t p_ts, float* energy, void* workspace,
                                size_t workspace_bytes, void* stream);
size_t rmm_pv_energy_workspace(int64_t h, int64_t tq, int64_t tk, int64_t dv, int p_dtype, int v_dtype, double rho);
rmm_status_t rmm_pv_energy(const void* P, int p_dtype, const void* V, int v_dtype, const float* energy, int64_t h,
                           int64_t hkv, int64_t tq, int64_t tk, int64_t dv, int64_t p_hs, int64_t p_ts, int64_t v_hs,
                           int64_t v_ts, double rho, int32_t* idx, void* O, int o_dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * rmm_softmax_select: rmm_softmax_energy, and in addition the kept key
 * positions of every head, idx[h][0..k) ascending with k = rmm_k(rho, tk):
 * the k largest energy[h][:], ties to the lowest index (the PV selection of
 * rmm_pv_energy at the same rho).  kaelemshawn.blog, section on where RMM
 * cuts inside the Transformer (PV contracts over key positions, scored by
 * the column norms of P); hackcv.com, Core Approach (TopK of the scores).
 * When one workgroup takes every query row of a head (decode-shaped calls,
 * tk <= 8192) the ranking runs inside the softmax pass and needs no
 * workspace; otherwise the softmax pass is followed by a TopK launch.
 *   idx  [h][k] int32, written.  Other arguments and errors as
 *        rmm_softmax_energy (RMM_ERR_RHO for rho outside (0, 1]).
 *   Workspace: rmm_softmax_select_workspace(h, tq, tk) bytes (0: none).
 *
 * rmm_pv_idx: PV over given key lists, for every head h
 *   O_h = sum over t < k of P_h[:, idx[h][t]] V_g(h)[idx[h][t], :],
 * g(h) = h / (h / hkv); entries outside [0, tk) contribute nothing, repeats
 * count once per occurrence (hackcv.com, Core Approach: the product over a
 * kept index set; kaelemshawn.blog, the PV mapping).  For lists made once
 * and used by the product that follows (rmm_softmax_select's).
 *   idx  [h][k] int32 (row stride k), k >= 1, any order.
 *   Other arguments, layouts and errors as rmm_pv (no rho).  tq <= 16
 *   with bf16 V reads only the listed rows of V (a GEMV per head).
 *   Workspace: rmm_pv_idx_workspace(h, tq, k, dv, v_dtype) bytes.
 * ------------------------------------------------------------------- */
size_t rmm_softmax_select_workspace(int64_t h, int64_t tq, int64_t tk);
rmm_status_t rmm_softmax_select(const float* L, float scale, int64_t h, int64_t tq, int64_t tk, int64_t l_hs,
                                int64_t l_ts, float* P, int64_t p_hs, int64_t p_ts, float* energy, double rho,
                                int32_t* idx, void* workspace, size_t workspace_bytes, void* stream);
size_t rmm_pv_idx_workspace(int64_t h, int64_t tq, int64_t k, int64_t dv, int v_dtype);
rmm_status_t rmm_pv_idx(const void* P, int p_dtype, const void* V, int v_dtype, const int32_t* idx, int64_t k,
                        int64_t h, int64_t hkv, int64_t tq, int64_t tk, int64_t dv, int64_t p_hs, int64_t p_ts,
                        int64_t v_hs, int64_t v_ts, void* O, int o_dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/* rmm_pv with the five stage events of rmm_matmul_timed recorded on `stream`
 * ([0] start, [1] after the column energies of P, [2] after TopK, [3] after
 * the pack of P when the path packs it, [4] after the batched product).
 * Same arguments, results and errors as rmm_pv; stage_events and its
 * entries non-NULL. */
rmm_status_t rmm_pv_timed(const void* P, int p_dtype, const void* V, int v_dtype, int64_t h, int64_t hkv, int64_t tq,
                          int64_t tk, int64_t dv, int64_t p_hs, int64_t p_ts, int64_t v_hs, int64_t v_ts, double rho,
                          int32_t* idx, void* O, int o_dtype, void* workspace, size_t workspace_bytes, void* stream,
                          void* const* stage_events);

#ifdef __cplusplus
}
#endif

#endif /* RMM_H_ */
