// LDS-tiled MFMA main loop shared by every contraction of the loss.
//
// Every product on the path is computed as C[m, n] = sum_k X[m, k] * Y[n, k]
// with both operands row-major and contiguous along k ("NT"):
//   logits      z^T[v, t] = sum_j W[v, j]  H[t, j]      (X = W,   Y = H)
//   dH          dH[t, j]  = sum_v G[t, v]  W^T[j, v]    (X = G,   Y = W^T)
//   dW          dW[v, j]  = sum_t G^T[v, t] H^T[j, t]   (X = G^T, Y = H^T)
// so one main loop serves all of them and only the epilogues differ.
//
// A workgroup owns a BM x BN output tile split over a WAVES_M x WAVES_N grid
// of 64-wide wavefronts; each wave owns WM x WN = (MB x NB) blocks of the
// 32x32 MFMA.  K is walked in BK slices staged through two LDS buffers; the
// next slice is fetched into registers while the current one is multiplied.
#pragma once

#include "ckl_common.hpp"

namespace ckl {

template <typename TIn>
struct MfmaTraits;

// v_mfma_f32_32x32x16_bf16: lane l supplies X[l % 32][8 (l / 32) + e] and
// Y[l % 32][8 (l / 32) + e], e = 0..7.
template <>
struct MfmaTraits<bf16_t> {
  static constexpr int KSTEP = 16;  // k per MFMA
  static constexpr int BK = 64;     // k per LDS slice
  static constexpr int VEC = 8;     // elements per 16-byte load
};

// v_mfma_f32_32x32x2_f32: lane l supplies one element per operand; the k
// order inside a slice is permuted identically for both operands (lane half
// h = l / 32 owns k = 16 h + s at step s), which leaves the sum unchanged.
template <>
struct MfmaTraits<float> {
  static constexpr int KSTEP = 2;
  static constexpr int BK = 32;
  static constexpr int VEC = 4;
};

template <typename TIn_, int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  using TIn = TIn_;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NTHREADS = 64 * NWAVES;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int BK = MfmaTraits<TIn>::BK;
  static constexpr int VEC = MfmaTraits<TIn>::VEC;
  static constexpr int LDK = BK + VEC;  // LDS row stride in elements (16 B pad)
  static constexpr int CHUNKS_PER_ROW = BK / VEC;
  static constexpr int X_LOADS = BM * CHUNKS_PER_ROW / NTHREADS;
  static constexpr int Y_LOADS = BN * CHUNKS_PER_ROW / NTHREADS;
  static constexpr int STAGE_ELEMS = (BM + BN) * LDK;
  static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * (int)sizeof(TIn);
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
  static_assert(BM * CHUNKS_PER_ROW % NTHREADS == 0 && BN * CHUNKS_PER_ROW % NTHREADS == 0, "loads");
};

// Accumulator coordinates: register r of block (mb, nb) in lane l holds
//   row m = wave_m*WM + mb*32 + 8*(r/4) + 4*(l/32) + r%4,
//   col n = wave_n*WN + nb*32 + l%32.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <class C>
struct Tile {
  using TIn = typename C::TIn;
  f32x16 acc[C::MB][C::NB];
};

// Computes the tile C[m0 .. m0+BM) x [n0 .. n0+BN) over k in [0, kdim).
//   X points at row m0 of the X operand (row stride ldx, xrows valid rows);
//   Y points at row n0 of the Y operand (row stride ldy, yrows valid rows).
// Rows past xrows / yrows and k past kdim read as zero.  kdim must be a
// multiple of VEC.  Ends with a barrier, so the LDS may be reused at once.
template <class C>
__device__ __forceinline__ void tile_mma(Tile<C>& tile, const typename C::TIn* __restrict__ X, int64_t ldx,
                                         int xrows, const typename C::TIn* __restrict__ Y, int64_t ldy,
                                         int yrows, int kdim, typename C::TIn* smem) {
  using TIn = typename C::TIn;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave / C::WAVES_N;
  const int wave_n = wave % C::WAVES_N;

#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tile.acc[mb][nb][r] = 0.f;

  u32x4 xr[C::X_LOADS], yr[C::Y_LOADS];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::X_LOADS; ++i) {
      const int lin = tid + i * C::NTHREADS;
      const int row = lin / C::CHUNKS_PER_ROW;
      const int kc = (lin % C::CHUNKS_PER_ROW) * C::VEC + k0;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < xrows && kc < kdim) v = *reinterpret_cast<const u32x4*>(X + (int64_t)row * ldx + kc);
      xr[i] = v;
    }
#pragma unroll
    for (int i = 0; i < C::Y_LOADS; ++i) {
      const int lin = tid + i * C::NTHREADS;
      const int row = lin / C::CHUNKS_PER_ROW;
      const int kc = (lin % C::CHUNKS_PER_ROW) * C::VEC + k0;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < yrows && kc < kdim) v = *reinterpret_cast<const u32x4*>(Y + (int64_t)row * ldy + kc);
      yr[i] = v;
    }
  };
  auto sstore = [&](int buf) {
    TIn* xs = smem + buf * C::STAGE_ELEMS;
    TIn* ys = xs + C::BM * C::LDK;
#pragma unroll
    for (int i = 0; i < C::X_LOADS; ++i) {
      const int lin = tid + i * C::NTHREADS;
      const int row = lin / C::CHUNKS_PER_ROW;
      const int kc = (lin % C::CHUNKS_PER_ROW) * C::VEC;
      *reinterpret_cast<u32x4*>(xs + row * C::LDK + kc) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < C::Y_LOADS; ++i) {
      const int lin = tid + i * C::NTHREADS;
      const int row = lin / C::CHUNKS_PER_ROW;
      const int kc = (lin % C::CHUNKS_PER_ROW) * C::VEC;
      *reinterpret_cast<u32x4*>(ys + row * C::LDK + kc) = yr[i];
    }
  };
  auto compute = [&](int buf) {
    const TIn* xs = smem + buf * C::STAGE_ELEMS + (wave_m * C::WM) * C::LDK;
    const TIn* ys = smem + buf * C::STAGE_ELEMS + C::BM * C::LDK + (wave_n * C::WN) * C::LDK;
    const int lrow = lane & 31;
    const int half = lane >> 5;
    if constexpr (sizeof(TIn) == 2) {
#pragma unroll
      for (int s = 0; s < C::BK / 16; ++s) {
        bf16x8 a[C::MB], b[C::NB];
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
          a[mb] = *reinterpret_cast<const bf16x8*>(xs + (mb * 32 + lrow) * C::LDK + s * 16 + half * 8);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
          b[nb] = *reinterpret_cast<const bf16x8*>(ys + (nb * 32 + lrow) * C::LDK + s * 16 + half * 8);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
            tile.acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], b[nb], tile.acc[mb][nb], 0, 0, 0);
      }
    } else {
      // fp32: lane half h covers k = 16 h .. 16 h + 15 of the slice.
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 a[C::MB], b[C::NB];
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
          a[mb] = *reinterpret_cast<const f32x4*>(xs + (mb * 32 + lrow) * C::LDK + half * 16 + q * 4);
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
          b[nb] = *reinterpret_cast<const f32x4*>(ys + (nb * 32 + lrow) * C::LDK + half * 16 + q * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
              tile.acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[mb][e], b[nb][e], tile.acc[mb][nb], 0, 0, 0);
      }
    }
  };

  const int nk = (kdim + C::BK - 1) / C::BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload((kt + 1) * C::BK);
    compute(kt & 1);
    if (more) sstore((kt + 1) & 1);
    __syncthreads();
  }
}

}  // namespace ckl
