// Host-side launchers of the libckl kernels (internal; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckl {

hipError_t launch_fill_i32(int* p, int n, int v, hipStream_t st);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st);
hipError_t launch_count_mask(const uint8_t* mask, int T, int* N, hipStream_t st);
// packed = 1: rows are the N kept rows first (mask NULL): s_t = 0 for t >= N.
hipError_t launch_row_scale(const uint8_t* mask, const float* grad_loss, const int* N, int T, int Tp, int packed,
                            float* s, hipStream_t st);
// Packed rows of a mask: perm[i] = i-th kept row, rank[t] = its position (-1
// masked), *N = kept rows.  One workgroup.
hipError_t launch_compact_rows(const uint8_t* mask, int T, int* perm, int* rank, int* N, hipStream_t st);
// dst row i = src row perm[i] for i < *N, zeros up to `rows` (row_bytes % 16 == 0).
hipError_t launch_gather_rows(const void* src, int rows, int64_t row_bytes, const int* perm, const int* N, void* dst,
                              hipStream_t st);
// dst[i] = src[perm[i]] for i < *N, 0 up to `rows`.
hipError_t launch_gather_f32(const float* src, const int* perm, const int* N, int rows, float* dst, hipStream_t st);
// dst[t] = src[rank[t]] (0 for masked rows), t < T.
hipError_t launch_scatter_f32(const float* src, const int* rank, int T, float* dst, hipStream_t st);
// dst rows (fp32 or bf16, d elements) = packed fp32 rows src[rank[t]], zero rows for masked t.
hipError_t launch_scatter_rows(const float* src, const int* rank, int T, int d, void* dst, int dst_bf16,
                               hipStream_t st);
// Zero the rows t of dst with rank[t] < 0.
hipError_t launch_zero_masked_rows(const int* rank, int T, int64_t row_bytes, void* dst, hipStream_t st);
// dst[i] = scale * src[i] rounded once to dst's type (scale NULL = 1), n % 4 == 0.
hipError_t launch_scale_cast(const float* src, void* dst, int64_t n, int dst_bf16, const float* scale,
                             hipStream_t st);
// logprob = 0: tlogit holds logits (softmax over the K entries); 1: it holds
// log-probabilities, used as given.  Indices are checked against [0, V) and
// stored sorted, minus voff (the first vocabulary row of this shard's W).
// rowmap not NULL: row t takes teacher row rowmap[t] for t < *nrows, an empty
// teacher past it.
hipError_t launch_teacher_prep(const int* idx, const float* tlogit, int T, int K, int V, int voff, int* idx_s,
                               float* p_s, float* Erow, float* Mrow, float* zg_s, int* bad, int logprob,
                               const int* rowmap, const int* nrows, hipStream_t st);
// Vocabulary shards: per-row partial LSE and cross term of one shard; and the
// merge of S shards' partials ([S][T] each) into LSE, row loss and the mean.
hipError_t launch_fwd_shard_rows(const void* part, int S, int T, int K, const float* p_s, const float* zg_s,
                                 float* lse_part, float* cross_part, hipStream_t st);
hipError_t launch_shard_combine(const float* lse_parts, const float* cross_parts, int S, int T, const float* Erow,
                                const float* Mrow, const uint8_t* mask, float* lse, float* row_loss, double* row_ld,
                                const int* N, float* loss, hipStream_t st);
// G == nullptr: log-sum-exp partials only.  Otherwise also the exponentials
// u (G, row stride ldG) and the per-tile maxima (mtab, row stride ldm) of the
// fused forward + backward.  nrows not NULL: only rows below *nrows - row0
// are kept rows; token blocks past them are skipped.
hipError_t launch_fwd_lse(int in_bf16, const void* H, const void* W, int T, int d, int V, int K, const int* idx_s,
                          float* zg_s, void* part, int n_splits, int tiles_per_split, void* G, int64_t ldG,
                          float* mtab, int64_t ldm, const int* nrows, int row0, hipStream_t st);
// Per-row LSE and loss of rows [0, T) of `part` (S split states per row),
// and each row's loss term in fp64 at row_ld[t] (0 for masked rows).
hipError_t launch_fwd_rows(const void* part, int S, int T, int K, const float* p_s, const float* zg_s,
                           const float* Erow, const float* Mrow, const uint8_t* mask, float* lse, float* row_loss,
                           double* row_ld, const int* nrows, int row0, hipStream_t st);
// loss = sum of row_ld[0 .. T) (fp64, fixed order) / *N
hipError_t launch_loss_reduce(const double* row_ld, int T, const int* N, float* loss, hipStream_t st);
// Fused path, fp32, after the rows' LSE is known: G[t][v] (holding u) becomes
// g = s_t M_t u 2^(m - lse_t log2e) in place, zero for t >= rows, v >= V or
// s_t = 0, and G^T[v][t] = g, over t < rows_p and v < Vp (tile multiples).
hipError_t launch_gpass(int in_bf16, void* G, int64_t ldG, void* Gt, int64_t ldGt, const float* mtab, int64_t ldm,
                        const float* srow, const float* Mrow, const float* lse, int rows, int rows_p, int V, int Vp,
                        hipStream_t st);
// Teacher columns of rows < rows: g = s_t (M_t exp(zg - lse_t) - p), from the
// fp32 logits kept by the forward, into G and G^T (indices outside [0, V) are
// skipped).
// bf16 fused path: G and G^T of a row chunk from u in the forward's tile order
// (n_tblocks x n_vtiles tiles of 256 x 256).
hipError_t launch_gpass_tiles(const void* U, int n_vtiles, int n_tblocks, void* G, int64_t ldG, void* Gt,
                              int64_t ldGt, const float* mtab, int64_t ldm, const float* srow, const float* Mrow,
                              const float* lse, int rows, int V, const int* nrows, int row0, hipStream_t st);
hipError_t launch_gfix(int in_bf16, int rows, int K, int V, const int* idx_s, const float* p_s, const float* zg_s,
                       const float* srow, const float* Mrow, const float* lse, void* G, int64_t ldG, void* Gt,
                       int64_t ldGt, hipStream_t st);
// out[i] = sum_{s < S} part[s * pstride + i] for i < n (fixed order), as fp32
// or bf16.  rowmap not NULL: rows of d elements, row r written to row
// rowmap[r] of out, only for r < *nrows - row0.
hipError_t launch_splitk_sum(const float* part, int64_t pstride, int S, int64_t n, void* out, int out_bf16,
                             const int* rowmap, const int* nrows, int row0, int d, hipStream_t st);
hipError_t launch_transpose_pad(int in_bf16, const void* src, int R, int C, int Rp, void* dst, int64_t ldd,
                                hipStream_t st);
hipError_t launch_cast_f32_bf16(const float* src, void* dst, int64_t n, hipStream_t st);
hipError_t launch_bwd_grad(int in_bf16, const void* H, const void* W, int T, int d, int V, int K, const int* idx_s,
                           const float* p_s, const float* Mrow, const float* lse, const float* srow, int tb0,
                           int t_rows, int vb0, int v_rows, int n_splits, int tiles_per_split, void* G, int64_t ldG,
                           void* Gt, int64_t ldGt, const int* nrows, hipStream_t st);
// out[m, n] (+)= sum_k X[m, k] Y[n, k]; row-major operands contiguous in k.
// batches > 1: that many products xb / yb / ob elements apart, the last with
// k extent kdim_last.
struct GemmArgs {
  const void* X;
  int64_t ldx;
  const void* Y;
  int64_t ldy;
  float* out;
  int64_t ldo;
  int M, N, kdim, beta;
  int batches = 1, kdim_last = 0;
  int64_t xb = 0, yb = 0, ob = 0;
  // X stored k-major: element (m, k) at X[k ldx + m] (bf16 only; the
  // buffer must hold whole 256-column tiles along m)
  int xt = 0;
  // packed rows: lim_kind 1 bounds M by *lim - lim_base (tiles past it are
  // skipped), 2 bounds kdim by it rounded up to lim_round (a multiple of 8)
  const int* lim = nullptr;
  int lim_base = 0, lim_kind = 0, lim_round = 1;
};
// Two independent products in one launch (problem 0's tiles are scheduled first).
hipError_t launch_gemm_pair(int in_bf16, const GemmArgs& a0, const GemmArgs& a1, hipStream_t st);

// Tile extents of the contraction kernels: G blocks are whole tiles.
int tile_rows_m(int in_bf16);  // vocabulary rows per logit tile (BM)
int tile_rows_n(int in_bf16);  // token rows per logit tile (BN)
int gemm_tile_m(int in_bf16);  // output tile rows of the plain contraction
int gemm_tile_n(int in_bf16);  // and columns
// running-maximum groups per logit tile kept by the fused forward
int lse_groups_per_tile(int in_bf16);

}  // namespace ckl
