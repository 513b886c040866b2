// Host-side launchers of the libckl kernels (internal; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckl {

hipError_t launch_fill_i32(int* p, int n, int v, hipStream_t st);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st);
hipError_t launch_count_mask(const uint8_t* mask, int T, int* N, hipStream_t st);
hipError_t launch_row_scale(const uint8_t* mask, const float* grad_loss, const int* N, int T, int Tp, float* s,
                            hipStream_t st);
hipError_t launch_teacher_prep(const int* idx, const float* tlogit, int T, int K, int V, int* idx_s, float* p_s,
                               float* Erow, float* Mrow, float* zg_s, int* bad, hipStream_t st);
hipError_t launch_fwd_lse(int in_bf16, const void* H, const void* W, int T, int d, int V, int K, const int* idx_s,
                          float* zg_s, void* part, int n_splits, int tiles_per_split, hipStream_t st);
hipError_t launch_fwd_finalize(const void* part, int S, int T, int K, const float* p_s, const float* zg_s,
                               const float* Erow, const float* Mrow, const uint8_t* mask, float* lse,
                               float* row_loss, double* blk_sum, const int* N, float* loss, hipStream_t st);
hipError_t launch_transpose_pad(int in_bf16, const void* src, int R, int C, int Rp, void* dst, int64_t ldd,
                                hipStream_t st);
hipError_t launch_cast_f32_bf16(const float* src, void* dst, int64_t n, hipStream_t st);
hipError_t launch_bwd_grad(int in_bf16, const void* H, const void* W, int T, int d, int V, int K, const int* idx_s,
                           const float* p_s, const float* Mrow, const float* lse, const float* srow, int tb0,
                           int t_rows, int vb0, int v_rows, int n_splits, int tiles_per_split, void* G, int64_t ldG,
                           void* Gt, int64_t ldGt, hipStream_t st);
// out[m, n] (+)= sum_k X[m, k] Y[n, k]; row-major operands contiguous in k.
struct GemmArgs {
  const void* X;
  int64_t ldx;
  const void* Y;
  int64_t ldy;
  float* out;
  int64_t ldo;
  int M, N, kdim, beta;
};
// Two independent products in one launch (problem 0's tiles are scheduled first).
hipError_t launch_gemm_pair(int in_bf16, const GemmArgs& a0, const GemmArgs& a1, hipStream_t st);

// Tile extents of the contraction kernels: G blocks are whole tiles.
int tile_rows_m(int in_bf16);  // vocabulary rows per logit tile (BM)
int tile_rows_n(int in_bf16);  // token rows per logit tile (BN)

}  // namespace ckl
