// Host-side launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmm {

// Column energy sweep: partial[h][s][j] = sum of A[h][r][j]^2 over the rows r
// of split s.  elt_bf16 selects bf16 (else fp32) input.
hipError_t launch_colnorm(const void* A, bool elt_bf16, int64_t head_stride, int64_t lda,
                          int heads, int n, int d, int splits, float* partial, hipStream_t s);

// Picks the number of row splits for the sweep (deterministic in the shape).
int colnorm_splits(int heads, int n, int d, bool elt_bf16);

// TopK over the summed partials of each head: writes idx[h][0..k) ascending,
// optionally the same list padded with -1 to k_pad entries (pad[h][...]),
// optional scores[h][j] = sqrt(energy), and optionally the keep mask
// mask[h][j] = j if column j is kept else -1 (all d entries), and optionally
// retained[h] = (sum of kept energies) / (sum of all energies).  gkeys:
// [heads][d] uint32 scratch, used only when d exceeds the LDS key capacity
// (may be null otherwise).
hipError_t launch_topk(const float* partial, int heads, int splits, int d, int k,
                       int32_t* idx, int64_t idx_hs, int32_t* pad, int64_t pad_hs, int k_pad,
                       float* scores, int64_t scores_hs, uint32_t* gkeys, hipStream_t s,
                       int32_t* mask = nullptr, int64_t mask_hs = 0, float* retained = nullptr);
int topk_lds_capacity();

// Selection and gather in one launch for a single bf16 matrix A (n x d, row
// stride lda): from the summed partials it writes the ascending kept list
// idx[0..k), the same list padded with -1 to k_pad entries (pad), and the
// panel out[r][t] = A[r][idx[t]] for t < k, 0 for k <= t < k_pad (out
// 16-byte aligned, k_pad a multiple of 8).  select_pack_fits tells whether
// the shape and alignment allow it (d within the LDS key capacity, rows
// whole 16-byte pieces).
bool select_pack_fits(const void* A, int64_t lda, int64_t d);
hipError_t launch_select_pack(const float* partial, int splits, const uint16_t* A, int64_t lda, int n, int d, int k,
                              int k_pad, int32_t* idx, int32_t* pad, uint16_t* out, hipStream_t s);

// The same gather by a caller's list: given[0..k) in any order (entries
// outside [0, d) read as zeros), out[r][t] = A[r][given[t]] for t < k and 0
// up to k_pad, pad[t] = given[t] if in range else -1 (k_pad entries).
// gather_pack_fits adds k_pad <= the LDS list capacity to select_pack_fits.
bool gather_pack_fits(const void* A, int64_t lda, int64_t d, int64_t k_pad);
hipError_t launch_gather_pack(const int32_t* given, int k, const uint16_t* A, int64_t lda, int n, int d, int k_pad,
                              int32_t* pad, uint16_t* out, hipStream_t s);

// Writes idx[h][t] = t for t < d (the rho = 1 selection), and optionally
// the padded copy pad[h][t] (t < k_pad, -1 past d).
hipError_t launch_iota(int32_t* idx, int64_t idx_hs, int heads, int d, int32_t* pad, int64_t pad_hs, int k_pad,
                       hipStream_t s);

// pad[b][t] = idx[b][t] for t < k when 0 <= idx[b][t] < d, else -1 (t < k_pad),
// for each of `heads` lists (strides idx_hs, pad_hs).
hipError_t launch_pad_index(const int32_t* idx, int k, int d, int32_t* pad, int k_pad, hipStream_t s,
                            int heads = 1, int64_t idx_hs = 0, int64_t pad_hs = 0);

// QK^T selection and gather in one launch (heads of dh <= 256 features,
// 16-byte aligned rows): from the summed partials of each query head it
// writes the ascending kept list idx[h][0..k), and the panels
// qp[h][r][t] = Q[h][r][idx[h][t]], kp[h][r][t] = K[h / group][r][idx[h][t]]
// for t < k, 0 up to k_pad.
bool qk_select_pack_fits(const void* Q, const void* K, int64_t q_hs, int64_t q_ts, int64_t k_hs, int64_t k_ts,
                         int64_t dh);
hipError_t launch_qk_select_pack(const float* partial, int splits, const uint16_t* Q, int64_t q_hs, int64_t q_ts,
                                 const uint16_t* K, int64_t k_hs, int64_t k_ts, int hq, int group, int tq, int tk,
                                 int dh, int k, int k_pad, int32_t* idx, uint16_t* qp, uint16_t* kp, hipStream_t s);

// Gather-pack: out[b][r][t] = t < k && idx[b][t] >= 0 ? bf16(src[b / src_group][r][idx[b][t]]) : 0
// for t < k_pad, rows r < rows.  src_bf16 selects bf16 (else fp32) input.
// k_pad must be a multiple of 8 and out 16-byte aligned (16-byte stores).
hipError_t launch_pack(const void* src, bool src_bf16, int64_t src_hs, int64_t src_rs, int src_group,
                       const int32_t* idx, int64_t idx_hs, int k, int k_pad,
                       int batch, int rows, uint16_t* out, int64_t out_hs, hipStream_t s);

// Softmax with the kept key lists (decode: every query row of a head in one
// workgroup, tk <= softmax_select_max_keys()): writes P and the energies as
// launch_softmax_energy does, and idx[h][0..k) ascending, the k largest
// energies of head h (ties to the lower index).
int softmax_select_max_keys();
hipError_t launch_softmax_select(const float* L, int64_t l_hs, int64_t l_ts, float* P, int64_t p_hs, int64_t p_ts,
                                 int heads, int tq, int tk, float scale, float* energy, int k, int32_t* idx,
                                 hipStream_t s);

// bf16 MFMA GEMM with fp32 accumulation.
struct GemmArgs {
  const uint16_t* A;    // [M][K] row-major, K contiguous (bf16 bits)
  int64_t a_bs, lda;
  const uint16_t* B;    // b_kmajor: [K][N] rows gathered by idx; else [N][K] K contiguous
  int64_t b_bs, ldb;
  int b_group;          // batch b reads B head b / b_group
  const int32_t* idx;   // row gather for b_kmajor, padded to K with -1 (null: row t is row t)
  int64_t idx_bs;
  void* C;              // [M][N] fp32 or bf16
  int64_t c_bs, ldc;
  bool c_bf16;
  int M, N, K, batch;   // K: multiple of 64 (A zero padded / B rows -1 padded)
  bool b_kmajor;
  uint32_t a_bytes, b_bytes;  // per-batch extents (bytes) for the buffer descriptors
  bool b_i8;                  // K-major B holds int8 weights (widened to bf16 exactly)
  const float* col_scale;     // int8 B only (required there): C[i][j] *= col_scale[j]
  bool causal;          // C[i][j] = -inf where j > i + causal_off (the non-persistent kernel skips the
                        // product of tiles wholly above)
  int64_t causal_off;
  // split K: k_split contraction ranges of K / k_split (a multiple of 64)
  // multiplied by separate workgroups into partial[k_split][batch][M][N]
  // (fp32), then added in range order into C; 1 = no split
  int k_split = 1;
  float* partial = nullptr;
  // optional identity index lists, written by the first workgroup (the
  // dense products' idx output, so that no separate launch writes it):
  // iota_out[h * iota_hs + t] = t for h < iota_heads, t < iota_n
  int32_t* iota_out = nullptr;
  int iota_heads = 0, iota_n = 0;
  int64_t iota_hs = 0;
};
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s);
// Same product with A given as fp32 (rounded to bf16 while staged); a gather
// list (idx) is honoured for K-major B only.
hipError_t launch_gemm_bf16_af32(const GemmArgs& g, hipStream_t s);
// Same product with int8 K-major B (b_i8, rows 8-byte aligned) and the
// per-column scale col_scale; a gather list (idx) is honoured.
hipError_t launch_gemm_w8(const GemmArgs& g, hipStream_t s);

// Generic FMA GEMM over strided, optionally gathered operands (fp32 or bf16
// inputs, any alignment):
//   C[b][i][j] = sum_{t<k} A(b,i,col(t)) * B(b/group, row(t), j)
struct SimtArgs {
  const void* A; bool a_bf16; int64_t a_bs, a_rs, a_cs;
  const void* B; bool b_bf16; int64_t b_bs, b_ts, b_js; int b_group;
  const int32_t* idx; int64_t idx_bs;   // null: identity
  void* C; bool c_bf16; int64_t c_bs, ldc;
  int M, N, k, batch;
  bool causal; int64_t causal_off;      // C[i][j] = -inf where j > i + causal_off
};
hipError_t launch_gemm_simt(const SimtArgs& g, hipStream_t s);

// Decode path (n <= 16): one workgroup computes the column energies over the
// n rows and selects the k kept columns into idx (ascending).
hipError_t launch_decode_select(const void* A, bool a_bf16, int64_t lda, int n, int d, int k, int32_t* idx,
                                float* scores, uint32_t* gkeys, hipStream_t s);

// GEMV over the kept rows of B (bf16, or int8) on the matrix cores (n <= 16
// rows of A, read in place and rounded to bf16: exact for bf16 A), split into `splits`
// slices of kept rows (gemv_splits) whose partial sums
// partial[splits][n][m] are added in slice order by a second kernel
// (splits == 1 writes Y directly).  idx == nullptr means the identity
// (dense).  m must be a multiple of 8, B rows 16-byte aligned.  Batched (per
// attention head b < batch): A + b*a_bs, B + (b / b_group)*b_bs,
// idx + b*idx_bs, Y + b*y_bs (element strides; batch 1 needs none).
// b_i8: B holds int8 weights (rows 8-byte aligned), widened to bf16 exactly;
// col_scale (if not null) multiplies output column c by col_scale[c] once
// the sum over the kept rows is complete.
// select: the kernel ranks the d columns of A itself (batch 1, d <=
// gemv_select_max_d(), idx must be null) and keeps the k largest column
// energies; idx_out (optional, [batch][k], stride idx_bs) receives the
// ascending kept lists (the identity lists when idx is null and select is
// false).
struct GemvArgs {
  const void* A; bool a_bf16; int64_t lda;
  const void* B; int64_t ldb;
  const int32_t* idx;
  int k, n, m;
  float* partial; int splits;
  void* Y; bool y_bf16; int64_t ldy;
  int batch = 1; int64_t a_bs = 0, b_bs = 0, idx_bs = 0, y_bs = 0; int b_group = 1;
  bool b_i8 = false; const float* col_scale = nullptr;
  // select: rank the d columns of A in every workgroup (idx unused);
  // otherwise d > 0 makes entries of idx outside [0, d) zero rows
  bool select = false; int d = 0; int32_t* idx_out = nullptr;
};
int gemv_select_max_d();
// slices for a list of k rows (with select: k = d, the source rows of B)
int gemv_splits(int k, int m, int batch = 1);
int gemv_splits_bound(int kmax, int m, int batch = 1);   // >= gemv_splits(k, m, batch) for all k <= kmax
hipError_t launch_gemv(const GemvArgs& g, hipStream_t s);

// Decode-shaped QK^T (tq <= 16, group * tq <= 8, dh <= 256 and a multiple
// of 8, bf16 Q (q_bf16 must be set; the launch rejects fp32 queries), bf16 K
// with 16-byte aligned rows): S[h][r][t] = sum over the k
// features idx[h][0..k) (all dh when idx is null) of Q[h][r][f] K[g(h)][t][f].
// The kernel also selects: idx_out[h][0..k) receives the kept features of
// head h (ascending; all dh of them when select is false).
struct QkDecodeArgs {
  const void* Q; bool q_bf16; int64_t q_hs, q_ts;
  const uint16_t* K; int64_t k_hs, k_ts;
  int32_t* idx_out; int k; bool select;
  int hq, hkv, tq, tk, dh;
  void* S; bool s_bf16;
  bool causal;          // S[h][r][t] = -inf where t > r + tk - tq
  int tok_per_block;
};
bool qk_decode_fits(int group, int tq, int dh);
hipError_t launch_qk_decode(QkDecodeArgs a, hipStream_t s);

// Row softmax of scale * L[h][q][:] (fp32, tk <= softmax_max_keys()) into P,
// with the column energies q[h][j] = sum over rows of P^2 (row blocks summed
// in order through partial[h][blocks][tk]).  blocks = softmax_row_blocks().
int softmax_max_keys();
int softmax_row_blocks(int heads, int tq);
hipError_t launch_softmax_energy(const float* L, int64_t l_hs, int64_t l_ts, float* P, int64_t p_hs, int64_t p_ts,
                                 int heads, int tq, int tk, int blocks, float scale, float* partial, float* q,
                                 hipStream_t s);

}  // namespace rmm
