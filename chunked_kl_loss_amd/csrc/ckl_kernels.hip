// gfx950 kernels of libckl: the fused chunked forward-KL loss.
//
// Forward (objective section of the README page "Chunked KL loss, running
// Knowledge Distillation locally in less <6GB VRAM"):
//   teacher_prep   p = softmax of the K cached logits per row, sorted by
//                  vocabulary index, with E = sum p log p and M = sum p
//   fwd_lse        logit tiles z^T = W H^T on MFMA, never stored; per row an
//                  online base-2 log-sum-exp over the vocabulary tiles of one
//                  split, and the logits at the teacher indices picked out of
//                  the accumulators
//   fwd_finalize   merge the splits into LSE, l_t = E - sum p z_idx + M LSE,
//                  deterministic masked sum
// Backward (Full Chunked KL paragraph of the same page: recompute each chunk,
// apply the closed-form gradient):
//   bwd_grad       recompute the logit tiles of one G block and turn them into
//                  G = s (M 2^{z log2 e - LSE log2 e} - p~), rounded once to
//                  the input dtype, stored as G (fp32: also as G^T)
//   gemm_store     dH (+)= G W and dW (+)= G^T H on the same MFMA main loop
//                  (bf16 reads G itself k-major for dW)
// One call without recompute (forward and backward together, per row chunk):
//   fwd_lse<STORE> as fwd_lse, keeping u = 2^{z log2 e - m} of every tile
//   gpass_tiles    once the chunk's LSE is known, u -> G (gpass_kernel: fp32)
//   gfix           the teacher columns of G, from the gathered logits
//   gemm_store     dH of the chunk as split-k parts, dW once per group of chunks
//   splitk_sum     the parts summed in a fixed order
#include "ckl_kernels.hpp"

#include <type_traits>

#include "ckl_tile.hpp"

namespace ckl {

// ----------------------------------------------------------- configurations --
// bf16: 256 x 256 tiles on 64-wide k slices, 8 waves (2 per SIMD, so one
// wave's loads, barriers and epilogue overlap the other's MFMAs), fragment
// reads pipelined per k16 substep; the logit kernels (forward and the
// recomputing backward) take 128 x 64 per wave, the dH / dW contraction
// 256 x 320 tiles of 64 x 160.  fp32 (small problems): 128 x 128 tiles,
// register-staged loads.
using CfgBF16 = Dma64Cfg<256, 256, 128, 64>;
using CfgBF16Bwd = CfgBF16;
using CfgBF16Gemm = Dma64Cfg<256, 320, 64, 160>;
using CfgF32 = TileCfg<float, 128, 128, 64, 64>;

// ---------------------------------------------------------------- helpers --
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  u32x2 v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<u32x2*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}
template <typename T>
__device__ __forceinline__ void store2(T* p, float a, float b);
template <>
__device__ __forceinline__ void store2<bf16_t>(bf16_t* p, float a, float b) {
  *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}
template <>
__device__ __forceinline__ void store2<float>(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

// First position k in the ascending row idx_s[0..K) with idx_s[k] >= v.
__device__ __forceinline__ int lower_bound_row(const int* __restrict__ row, int K, int v) {
  int lo = 0, hi = K;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// ----------------------------------------------------------- small kernels --
__global__ void fill_i32_kernel(int* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// N = number of kept rows (mask NULL: all T).  One workgroup, fixed order.
__global__ __launch_bounds__(1024) void count_mask_kernel(const uint8_t* __restrict__ mask, int T, int* N) {
  __shared__ int red[1024];
  int c = 0;
  if (mask == nullptr) {
    c = (threadIdx.x == 0) ? T : 0;
  } else {
    for (int t = threadIdx.x; t < T; t += 1024) c += mask[t] != 0;
  }
  red[threadIdx.x] = c;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *N = red[0];
}

// s[t] = grad_loss * keep_t / N for t < T, 0 for T <= t < Tp.  Packed rows
// (mask NULL, N kept rows first): keep_t = t < N.
__global__ void row_scale_kernel(const uint8_t* __restrict__ mask, const float* __restrict__ grad_loss,
                                 const int* __restrict__ N, int T, int Tp, int packed, float* __restrict__ s) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= Tp) return;
  const int n = *N;
  const float g = grad_loss ? *grad_loss : 1.f;
  float v = 0.f;
  if (t < T && n > 0 && (mask == nullptr || mask[t] != 0) && (!packed || t < n)) v = g / (float)n;
  s[t] = v;
}

// ------------------------------------------------------- packed rows --
// The kept rows of a mask, in ascending order: perm[i] (i < N) is the i-th
// kept row, rank[t] its position among them (-1 for a masked row), *N their
// number.  One workgroup; thread j scans rows [j seg, (j + 1) seg), the
// counts of the segments are scanned in LDS.
__global__ __launch_bounds__(1024) void compact_rows_kernel(const uint8_t* __restrict__ mask, int T,
                                                            int* __restrict__ perm, int* __restrict__ rank,
                                                            int* __restrict__ N) {
  __shared__ int cnt[1024];
  const int seg = (T + 1023) / 1024;
  const int a = min(T, (int)threadIdx.x * seg), b = min(T, a + seg);
  int c = 0;
  for (int t = a; t < b; ++t) c += mask[t] != 0;
  cnt[threadIdx.x] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan
    const int v = threadIdx.x >= (unsigned)o ? cnt[threadIdx.x - o] : 0;
    __syncthreads();
    cnt[threadIdx.x] += v;
    __syncthreads();
  }
  int pos = cnt[threadIdx.x] - c;
  for (int t = a; t < b; ++t) {
    if (mask[t] != 0) {
      perm[pos] = t;
      rank[t] = pos++;
    } else {
      rank[t] = -1;
    }
  }
  if (threadIdx.x == 1023) *N = cnt[1023];
}

// dst row i = src row perm[i] for i < *N, zeros for *N <= i < rows; rows of
// `chunks` 16-byte pieces.
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4* __restrict__ src, int64_t chunks,
                                                          const int* __restrict__ perm, const int* __restrict__ N,
                                                          int rows, u32x4* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * chunks) return;
  const int r = (int)(i / chunks);
  const int64_t c = i - (int64_t)r * chunks;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < *N) v = src[(int64_t)perm[r] * chunks + c];
  dst[i] = v;
}

// dst[i] = src[perm[i]] for i < *N, 0 for *N <= i < rows.
__global__ __launch_bounds__(256) void gather_f32_kernel(const float* __restrict__ src, const int* __restrict__ perm,
                                                         const int* __restrict__ N, int rows, float* __restrict__ dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  dst[i] = i < *N ? src[perm[i]] : 0.f;
}

// dst[t] = src[rank[t]] for kept rows, 0 for masked rows (rank -1).
__global__ __launch_bounds__(256) void scatter_f32_kernel(const float* __restrict__ src, const int* __restrict__ rank,
                                                          int T, float* __restrict__ dst) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int r = rank[t];
  dst[t] = r >= 0 ? src[r] : 0.f;
}

// dst row t (d elements, fp32 or bf16) = packed fp32 row rank[t], or zeros
// for a masked row; four elements per thread.
__global__ __launch_bounds__(256) void scatter_rows_kernel(const float* __restrict__ src, const int* __restrict__ rank,
                                                           int T, int d, void* __restrict__ dst, int dst_bf16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = d / 4;
  if (i >= (int64_t)T * q) return;
  const int t = (int)(i / q);
  const int c = (int)(i - (int64_t)t * q);
  const int r = rank[t];
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  if (r >= 0) a = reinterpret_cast<const f32x4*>(src + (int64_t)r * d)[c];
  if (dst_bf16)
    *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(dst) + (int64_t)t * d + 4 * c) =
        u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
  else
    reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dst) + (int64_t)t * d)[c] = a;
}

// Rows t of dst (`chunks` 16-byte pieces each) with rank[t] < 0 set to zero.
__global__ __launch_bounds__(256) void zero_masked_rows_kernel(const int* __restrict__ rank, int T, int64_t chunks,
                                                               u32x4* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * chunks) return;
  const int t = (int)(i / chunks);
  if (rank[t] < 0) dst[i] = u32x4{0u, 0u, 0u, 0u};
}

// dst[i] = scale * src[i], rounded once to dst's type; four per thread.
// (src and dst may be the same fp32 array: each element is read before the
// same thread overwrites it)
__global__ __launch_bounds__(256) void scale_cast_kernel(const float* src, void* dst, int64_t n4, int dst_bf16,
                                                         const float* __restrict__ scale) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float g = scale ? *scale : 1.f;
  const f32x4 a = reinterpret_cast<const f32x4*>(src)[i] * g;
  if (dst_bf16)
    reinterpret_cast<u32x2*>(dst)[i] = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
  else
    reinterpret_cast<f32x4*>(dst)[i] = a;
}

// One wavefront per row.  Softmax of the K cached logits (fp32), then a
// bitonic sort of (idx, p) by idx in LDS.  Optional outputs: E (sum p log p),
// zero-filled zg.  `bad` collects out-of-range / repeated indices.  Packed
// rows (rowmap not NULL): row t takes the teacher of row rowmap[t] for
// t < *nrows; rows past *nrows get an empty teacher (no index, p = E = M = 0).
__global__ __launch_bounds__(64) void teacher_prep_kernel(const int* __restrict__ idx, const float* __restrict__ tlogit,
                                                          int T, int K, int Kp, int V, int voff, int* __restrict__ idx_s,
                                                          float* __restrict__ p_s, float* __restrict__ Erow,
                                                          float* __restrict__ Mrow, float* __restrict__ zg_s,
                                                          int* __restrict__ bad, int logprob,
                                                          const int* __restrict__ rowmap,
                                                          const int* __restrict__ nrows) {
  extern __shared__ int sm_dyn[];
  int* key = sm_dyn;
  float* val = reinterpret_cast<float*>(sm_dyn + Kp);
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  int src = t;
  if (rowmap != nullptr) {
    if (t >= *nrows) {
      for (int k = lane; k < K; k += 64) {
        idx_s[(int64_t)t * K + k] = kIdxEnd;
        p_s[(int64_t)t * K + k] = 0.f;
        if (zg_s) zg_s[(int64_t)t * K + k] = 0.f;
      }
      if (lane == 0) {
        if (Erow) Erow[t] = 0.f;
        Mrow[t] = 0.f;
      }
      return;
    }
    src = rowmap[t];
  }
  const int* irow = idx + (int64_t)src * K;
  const float* lrow = tlogit + (int64_t)src * K;

  // logits: p = softmax over the K entries (shifted by the row maximum);
  // log-probabilities: p = exp(entry) as given (mass M may be below one)
  float mx = 0.f, inv = 1.f, logse = 0.f;
  if (!logprob) {
    mx = -INFINITY;
    for (int k = lane; k < K; k += 64) mx = fmaxf(mx, lrow[k]);
    mx = wave_max(mx);
    float se = 0.f;
    for (int k = lane; k < K; k += 64) se += expf(lrow[k] - mx);
    se = wave_sum(se);
    inv = 1.f / se;
    logse = logf(se);
  }
  float ent = 0.f, mass = 0.f;
  for (int k = lane; k < Kp; k += 64) {
    if (k < K) {
      const float a = lrow[k] - mx;
      const float p = expf(a) * inv;
      if (p > 0.f) ent += p * (a - logse);  // p log p, with 0 log 0 = 0
      mass += p;
      key[k] = irow[k];
      val[k] = p;
    } else {
      key[k] = kIdxEnd;
      val[k] = 0.f;
    }
  }
  ent = wave_sum(ent);
  mass = wave_sum(mass);
  __syncthreads();
  for (int size = 2; size <= Kp; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = lane; i < (Kp >> 1); i += 64) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const int a = key[lo], b = key[hi];
        if ((a > b) == asc) {
          key[lo] = b; key[hi] = a;
          const float va = val[lo];
          val[lo] = val[hi]; val[hi] = va;
        }
      }
      __syncthreads();
    }
  }
  int badl = 0;
  for (int k = lane; k < K; k += 64) {
    const int v = key[k];
    idx_s[(int64_t)t * K + k] = v - voff;  // vocabulary row of this shard's W (out of range: another shard's)
    p_s[(int64_t)t * K + k] = val[k];
    if (zg_s) zg_s[(int64_t)t * K + k] = 0.f;
    if (v < 0 || v >= V || (k + 1 < K && key[k + 1] == v)) badl = 1;
  }
  if (bad && badl) atomicOr(bad, 1);
  if (lane == 0) {
    if (Erow) Erow[t] = ent;
    Mrow[t] = mass;
  }
}

// ------------------------------------------------------------ forward LSE --
// One workgroup per (token block of BN rows, vocabulary split of
// tiles_per_split tiles of BM rows), n_tblocks x n_splits in all, laid out
// XCD-aware (kGroupT token blocks per group).  Output part[split * T + t] =
// (m, s): the base-2 log-sum-exp state of row t over the split.
//
// STORE (the fused forward + backward): the exponentials the running sum is
// built from are also kept.  The lanes holding one token's column of a wave's
// WM vocabulary rows keep a common running maximum m over them (base 2); they
// store u = 2^(z log2e - m) <= 1 (zero for v >= V) and m itself at
// mtab[(vt WAVES_M + wave_m) ldm + t], so that exp(z - LSE) = u 2^(m - LSE
// log2e) can be formed once the LSE is known, without recomputing z.  No
// overflow: u <= 1 and m <= LSE log2e.  fp32 stores u at G[t][v]; bf16 in
// tile order (see the store below), which gpass_tiles_kernel reads.
constexpr int kGroupT = 8;

template <class C, bool STORE>
__global__ __launch_bounds__(C::NTHREADS) void fwd_lse_kernel(
    const typename C::TIn* __restrict__ H, const typename C::TIn* __restrict__ W, int T, int d, int V, int K,
    const int* __restrict__ idx_s, float* __restrict__ zg_s, float2* __restrict__ part, int n_vtiles,
    int tiles_per_split, int n_tblocks, int n_splits, typename C::TIn* __restrict__ G, int64_t ldG,
    float* __restrict__ mtab, int64_t ldm, const int* __restrict__ nrows, int row0) {
  using TIn = typename C::TIn;
  using TileT = typename C::TileT;
  using L = typename TileT::L;
  constexpr int MBK = TileT::MBK, NBK = TileT::NBK, BLK = L::BLK, RPB = L::RPB;
  constexpr int GLANES = 64 / L::GROUPS;  // lanes l, l + GLANES, ... hold the rows of one column
  // Lane group g owns column block nb = g: it keeps that token's running LSE
  // state and its place in the sorted teacher list, the other groups only
  // contribute partial maxima, sums and gathered logits for the tile.
  static_assert(NBK == L::GROUPS && GLANES == BLK, "one column block per lane group");
  // bf16 keeps u in tile order (whole 1 KiB stores; gpass_tiles_kernel lays
  // it out as G), fp32 at G[t][v] directly
  constexpr bool kTileU = sizeof(TIn) == 2;
  static_assert(!kTileU || (RPB == 16 && C::BM == 256 && C::BN == 256), "tile order of the bf16 configuration");
  // Between tiles the entry after the owner's next teacher index waits in
  // LDS after the k-loop stages, fetched by a global->LDS load: a later
  // epilogue reads it there, so no epilogue waits for a global load of its own
  // (which would also wait for the next tile's slices and this tile's stores).
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES + C::NTHREADS * 4];
  int* s_nxt2 = reinterpret_cast<int*>(smem + C::LDS_BYTES);
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wave_m = wave / C::WAVES_N;
  const int wave_n = wave % C::WAVES_N;
  int tblock, split;
  grouped_mn(xcd_remap(blockIdx.x, n_tblocks * n_splits), n_tblocks, n_splits, kGroupT, tblock, split);
  const int t0 = tblock * C::BN;
  // packed rows: only the first *nrows - row0 rows of this call hold kept
  // rows (the rest are zero rows); whole token blocks past them are skipped
  // (their split states, u and maxima are never read)
  if (nrows != nullptr && t0 >= *nrows - row0) return;
  const int vt0 = split * tiles_per_split;
  const int vt1 = min(n_vtiles, vt0 + tiles_per_split);
  const int own_nb = lane / GLANES;
  const int own_tok = t0 + wave_n * C::WN + own_nb * BLK + (lane & (BLK - 1));

  // the owner's state: running maximum and sum (base 2), position cur of the
  // next teacher index nxt at or after this split's first row
  float rm = -INFINITY, rs = 0.f;
  int cur = K, nxt = kIdxEnd;
  {
    int nxt2 = kIdxEnd;
    if (own_tok < T) {
      const int* row = idx_s + (int64_t)own_tok * K;
      cur = lower_bound_row(row, K, vt0 * C::BM);
      nxt = cur < K ? row[cur] : kIdxEnd;
      nxt2 = cur + 1 < K ? row[cur + 1] : kIdxEnd;
    }
    s_nxt2[threadIdx.x] = nxt2;
  }

  TileT tile;
  // With the substep loop, the next tile's first two slices are issued at the
  // end of a tile's epilogue (registers and global memory only; the LDS
  // stages are untouched), after its stores: the next k loop starts by
  // waiting for both, and the stores, issued first, are then mostly done.
  constexpr bool kAhead = PrefetchOK<C>::value;
  const TIn* Ht0 = H + (int64_t)t0 * d;
  if constexpr (kAhead)
    if (vt0 < vt1) tile_k64_prologue<C>(W + (int64_t)vt0 * C::BM * d, d, V - vt0 * C::BM, Ht0, d, T - t0, d, smem);
  for (int vt = vt0; vt < vt1; ++vt) {
    const int v0 = vt * C::BM;
    if constexpr (kAhead) {
      run_mma<C, true>(tile, W + (int64_t)v0 * d, d, V - v0, Ht0, d, T - t0, d, smem);
    } else {
      run_mma(tile, W + (int64_t)v0 * d, d, V - v0, Ht0, d, T - t0, d, smem);
    }
    // (without the prefetch, the k loop need not have waited for every
    // load: the teacher-list entries loaded into LDS must have landed)
    if constexpr (!kAhead) wait_vmcnt<0>();
    const int vbase = v0 + wave_m * C::WM;
    const int vend = min(v0 + C::BM, V);
    const bool full = vbase + C::WM <= V;  // every row of the wave's slice is a vocabulary row
#pragma unroll
    for (int nb = 0; nb < NBK; ++nb) {
      const int src = (lane & (GLANES - 1)) + nb * GLANES;  // the owner of column nb
      const bool own = own_nb == nb;
      const int tok = opaque(t0 + wave_n * C::WN + nb * BLK + (lane & (BLK - 1)));
      // (max before the scaling by log2e > 0: the same value, one multiply)
      float mx = -INFINITY;
      if (full) {
#pragma unroll
        for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
          for (int r = 0; r < RPB; ++r) mx = fmaxf(mx, tile.acc[mb][nb][r]);
      } else {
#pragma unroll
        for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
          for (int r = 0; r < RPB; ++r) {
            const int v = vbase + mb * BLK + L::row_in(r, lane);
            if (v < V) mx = fmaxf(mx, tile.acc[mb][nb][r]);
          }
      }
#pragma unroll
      for (int o = GLANES; o < 64; o *= 2) mx = fmaxf(mx, __shfl_xor(mx, o));
      mx *= kLog2e;
      const float crm = __shfl(rm, src);
      const float mn = fmaxf(crm, mx);
      // logits at the teacher indices of this token that fall in this tile;
      // the lanes of the column walk the list together
      int ccur = __shfl(cur, src), cnxt = __shfl(nxt, src);
      if (cnxt < vend) {
        auto gather = [&]() {  // teacher entry ccur (index cnxt) lies in this tile
          const int vl = cnxt - vbase;
          if (vl >= 0 && vl < C::WM) {
            const int rr = vl % BLK;
            if (L::group_of(rr) == own_nb) {
              const int sel = (vl / BLK) * RPB + L::reg_of(rr);
              float val = 0.f;
#pragma unroll
              for (int q = 0; q < MBK * RPB; ++q) val = (q == sel) ? tile.acc[q / RPB][nb][q % RPB] : val;
              zg_s[(int64_t)tok * K + ccur] = val;
            }
          }
          ++ccur;
        };
        gather();
        // the entry after it waits in LDS; a second hit in one tile (rare)
        // reads the list directly
        cnxt = s_nxt2[wave * 64 + src];
        while (cnxt < vend) {
          gather();
          cnxt = ccur < K ? idx_s[(int64_t)tok * K + ccur] : kIdxEnd;
        }
        if (own) {
          cur = ccur;
          nxt = cnxt;
          if (ccur + 1 < K)
            lds_dma4(idx_s + (int64_t)tok * K + ccur + 1, s_nxt2 + wave * 64);
          else
            s_nxt2[threadIdx.x] = kIdxEnd;
        }
      }
      float ssum = 0.f;
      if (mn != -INFINITY) {
        if (full) {
#pragma unroll
          for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
            for (int r = 0; r < RPB; ++r) {
              const float u = fast_exp2(tile.acc[mb][nb][r] * kLog2e - mn);
              ssum += u;
              if constexpr (STORE) tile.acc[mb][nb][r] = u;
            }
        } else {
#pragma unroll
          for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
            for (int r = 0; r < RPB; ++r) {
              const int v = vbase + mb * BLK + L::row_in(r, lane);
              const float u = v < V ? fast_exp2(tile.acc[mb][nb][r] * kLog2e - mn) : 0.f;
              ssum += u;
              if constexpr (STORE) tile.acc[mb][nb][r] = u;
            }
        }
#pragma unroll
        for (int o = GLANES; o < 64; o *= 2) ssum += __shfl_xor(ssum, o);
        if (own) {
          rs = rs * fast_exp2(rm - mn) + ssum;
          rm = mn;
        }
      } else if constexpr (STORE) {
#pragma unroll
        for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
          for (int r = 0; r < RPB; ++r) tile.acc[mb][nb][r] = 0.f;
      }
      if constexpr (STORE) {
        const int64_t trow = tok;
        if constexpr (kTileU) {
          // u in tile order: the tile's (tblock, vt) block of BM x BN entries,
          // within it 1 KiB per (wave, mb, nb, h), lane l at 16 l: registers
          // 8h .. 8h + 7 of the lane's block (mb, nb)
          TIn* ut = G + ((int64_t)tblock * n_vtiles + vt) * (C::BM * C::BN);
#pragma unroll
          for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              u32x4 y;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                y[e] = pack_bf16x2(tile.acc[mb][nb][8 * h + 2 * e], tile.acc[mb][nb][8 * h + 2 * e + 1]);
              *reinterpret_cast<u32x4*>(ut + ((((wave * MBK + mb) * NBK + nb) * 2 + h) * 64 + lane) * 8) = y;
            }
        } else {
          // registers 4i .. 4i + 3 of a block hold four consecutive rows
#pragma unroll
          for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
            for (int i = 0; i < RPB / 4; ++i) {
              const int vcol = vbase + mb * BLK + L::row_in(4 * i, lane);
              store4<TIn>(G + trow * ldG + vcol, tile.acc[mb][nb][4 * i], tile.acc[mb][nb][4 * i + 1],
                          tile.acc[mb][nb][4 * i + 2], tile.acc[mb][nb][4 * i + 3]);
            }
        }
        if (own) mtab[((int64_t)vt * C::WAVES_M + wave_m) * ldm + trow] = mn;
      }
    }
    if constexpr (kAhead)
      if (vt + 1 < vt1)
        tile_k64_prologue<C>(W + (int64_t)(v0 + C::BM) * d, d, V - v0 - C::BM, Ht0, d, T - t0, d, smem);
  }

  // merge across the WAVES_M waves sharing the same tokens (each lane owns
  // the column wave_n WN + lane); no load into LDS outlives the workgroup
  wait_vmcnt<0>();
  float2* red = reinterpret_cast<float2*>(smem);  // [WAVES_M][BN]
  red[wave_m * C::BN + wave_n * C::WN + lane] = make_float2(rm, rs);
  __syncthreads();
  for (int i = threadIdx.x; i < C::BN; i += C::NTHREADS) {
    float m = -INFINITY, s = 0.f;
#pragma unroll
    for (int w = 0; w < C::WAVES_M; ++w) {
      const float2 x = red[w * C::BN + i];
      lse2_merge(m, s, x.x, x.y);
    }
    if (t0 + i < T) part[(int64_t)split * T + t0 + i] = make_float2(m, s);
  }
}

// Sixteen lanes per row: LSE from the split states, l_t = E_t - sum_k p z +
// M_t LSE, and l_t in fp64 at row_ld[t] for the deterministic mean (0 for
// masked rows).  Lane j of a row takes splits j, j + 16, .. and teacher
// entries j, j + 16, ..; the partials merge by shuffles in a fixed order.
// Packed rows (nrows not NULL): rows t >= *nrows - row0 are padding, treated
// as masked.
__global__ __launch_bounds__(256) void fwd_finalize_kernel(const float2* __restrict__ part, int S, int T, int K,
                                                           const float* __restrict__ p_s,
                                                           const float* __restrict__ zg_s,
                                                           const float* __restrict__ Erow,
                                                           const float* __restrict__ Mrow,
                                                           const uint8_t* __restrict__ mask,
                                                           float* __restrict__ lse_out,
                                                           float* __restrict__ row_loss,
                                                           double* __restrict__ row_ld,
                                                           const int* __restrict__ nrows, int row0) {
  const int sub = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool valid = t < T;
  const bool keep =
      valid && (mask == nullptr || mask[t] != 0) && (nrows == nullptr || t < *nrows - row0);
  float m = -INFINITY, s = 0.f;
  double x = 0.0;
  if (keep) {
    for (int sp = sub; sp < S; sp += 16) {
      const float2 v = part[(int64_t)sp * T + t];
      lse2_merge(m, s, v.x, v.y);
    }
    const float* pr = p_s + (int64_t)t * K;
    const float* zr = zg_s + (int64_t)t * K;
    for (int k = sub; k < K; k += 16) x += (double)pr[k] * (double)zr[k];
  }
#pragma unroll
  for (int o = 1; o < 16; o *= 2) {
    const float om = __shfl_xor(m, o), os = __shfl_xor(s, o);
    lse2_merge(m, s, om, os);
    x += __shfl_xor(x, o);
  }
  if (sub == 0 && valid) {
    float lse = 0.f, l = 0.f;
    double ld = 0.0;
    if (keep) {
      lse = (m + fast_log2(s)) * kLn2;
      ld = (double)Erow[t] - x + (double)Mrow[t] * (double)lse;
      l = (float)ld;
    }
    lse_out[t] = lse;
    if (row_loss) row_loss[t] = l;
    row_ld[t] = ld;
  }
}

// loss = sum_t row_ld[t] / N, summed in a fixed order (one block).
__global__ __launch_bounds__(1024) void loss_reduce_kernel(const double* __restrict__ row_ld, int T,
                                                           const int* __restrict__ N, float* __restrict__ loss) {
  __shared__ double red[1024];
  double a = 0.0;
  for (int i = threadIdx.x; i < T; i += 1024) a += row_ld[i];
  red[threadIdx.x] = a;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = *N;
    *loss = n > 0 ? (float)(red[0] / (double)n) : 0.f;
  }
}

// ------------------------------------------------ vocabulary shards --
// One thread per row: the shard's natural-log LSE over its vocabulary rows
// (split states merged) and its share of the cross term, sum over the
// teacher entries that fall in the shard of p * z (fp64 sum).
__global__ __launch_bounds__(256) void fwd_shard_rows_kernel(const float2* __restrict__ part, int S, int T, int K,
                                                             const float* __restrict__ p_s,
                                                             const float* __restrict__ zg_s,
                                                             float* __restrict__ lse_part,
                                                             float* __restrict__ cross_part) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  float m = -INFINITY, s = 0.f;
  for (int sp = 0; sp < S; ++sp) {
    const float2 x = part[(int64_t)sp * T + t];
    lse2_merge(m, s, x.x, x.y);
  }
  lse_part[t] = (m + fast_log2(s)) * kLn2;
  double x = 0.0;
  const float* pr = p_s + (int64_t)t * K;
  const float* zr = zg_s + (int64_t)t * K;
  for (int k = 0; k < K; ++k) x += (double)pr[k] * (double)zr[k];
  cross_part[t] = (float)x;
}

// One thread per row: merge the shards' partial LSE (fp64 log-sum-exp of the
// natural-log partials) and cross terms into LSE and l_t = E - sum cross +
// M LSE; masked rows give 0; l_t in fp64 at row_ld[t] as in fwd_finalize.
__global__ __launch_bounds__(256) void shard_combine_kernel(const float* __restrict__ lse_parts,
                                                            const float* __restrict__ cross_parts, int S, int T,
                                                            const float* __restrict__ Erow,
                                                            const float* __restrict__ Mrow,
                                                            const uint8_t* __restrict__ mask,
                                                            float* __restrict__ lse_out, float* __restrict__ row_loss,
                                                            double* __restrict__ row_ld) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  double contrib = 0.0;
  if (t < T) {
    const bool keep = mask == nullptr || mask[t] != 0;
    float lse = 0.f, l = 0.f;
    if (keep) {
      double m = -INFINITY;
      for (int sh = 0; sh < S; ++sh) m = fmax(m, (double)lse_parts[(int64_t)sh * T + t]);
      double sum = 0.0, cross = 0.0;
      for (int sh = 0; sh < S; ++sh) {
        sum += exp((double)lse_parts[(int64_t)sh * T + t] - m);
        cross += (double)cross_parts[(int64_t)sh * T + t];
      }
      const double L = m + log(sum);
      const double ld = (double)Erow[t] - cross + (double)Mrow[t] * L;
      lse = (float)L;
      l = (float)ld;
      contrib = ld;
    }
    lse_out[t] = lse;
    if (row_loss) row_loss[t] = l;
    row_ld[t] = contrib;
  }
}

// ----------------------------------------------------- transposes / casts --
// dst[c * ldd + r] = src[r * C + c] for r < R; 0 for R <= r < Rp.
template <typename T>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const T* __restrict__ src, int R, int C, int Rp,
                                                            T* __restrict__ dst, int64_t ldd) {
  __shared__ T tileS[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    T v = T(0.f);
    if (r < R && c < C) v = src[(int64_t)r * C + c];
    tileS[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) dst[(int64_t)c * ldd + r] = tileS[tx][i];
  }
}

// bf16, 128 x 128 tiles: 16-byte loads of the rows into LDS (the 16-byte
// chunk c of row r at c ^ (r / 8 mod 16)), then each thread transposes one
// 8 x 8 block in registers and writes eight 16-byte pieces of dst rows;
// requires C % 8 == 0 and Rp % 128 == 0.  Four waves per SIMD (five blocks
// per CU by LDS): left to itself the compiler spends ~250 registers here and
// runs two, which made the transposes 1.6x slower.
__global__ __launch_bounds__(256, 4) void transpose_bf16_kernel(const bf16_t* __restrict__ src, int R, int C, int Rp,
                                                                bf16_t* __restrict__ dst, int64_t ldd) {
  __shared__ __attribute__((aligned(16))) uint16_t tr[128 * 128];
  const int r0 = blockIdx.x * 128, c0 = blockIdx.y * 128;
  const int tid = threadIdx.x;
  u32x4 x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = j * 256 + tid, rl = q >> 4, cc = q & 15;
    const int r = r0 + rl, c = c0 + cc * 8;
    x[j] = u32x4{0u, 0u, 0u, 0u};
    if (r < R && c < C) x[j] = *reinterpret_cast<const u32x4*>(src + (int64_t)r * C + c);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = j * 256 + tid, rl = q >> 4, cc = q & 15;
    reinterpret_cast<u32x4*>(tr + rl * 128)[cc ^ ((rl >> 3) & 15)] = x[j];
  }
  __syncthreads();
  const int rb = tid & 15, cb = tid >> 4;
  u32x4 a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = reinterpret_cast<const u32x4*>(tr + (rb * 8 + i) * 128)[cb ^ rb];
  if (r0 + rb * 8 >= Rp) return;
#pragma unroll
  for (int w = 0; w < 4; ++w) {  // dst rows 2w (low halves) and 2w + 1 (high halves) of the block
    u32x4 lo, hi;
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      lo[i2] = __builtin_amdgcn_perm(a[2 * i2 + 1][w], a[2 * i2][w], 0x05040100u);
      hi[i2] = __builtin_amdgcn_perm(a[2 * i2 + 1][w], a[2 * i2][w], 0x07060302u);
    }
    const int c = c0 + cb * 8 + 2 * w;
    if (c < C) *reinterpret_cast<u32x4*>(dst + (int64_t)c * ldd + r0 + rb * 8) = lo;
    if (c + 1 < C) *reinterpret_cast<u32x4*>(dst + (int64_t)(c + 1) * ldd + r0 + rb * 8) = hi;
  }
}

__global__ void cast_f32_bf16_kernel(const float* __restrict__ src, bf16_t* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const uint32_t b = f32_to_bf16_bits(src[i]);
    reinterpret_cast<uint16_t*>(dst)[i] = (uint16_t)b;
  }
}

// ------------------------------------------------------------ backward G --
// Recomputes the logit tiles of the G block rows [tb0, tb0 + BN n_tblocks),
// vocabulary [vb0, vb0 + BM n_vtiles) (same workgroup layout as the forward)
// and writes
//   G [t - tb0][v - vb0]  (row stride ldG)  and  Gt[v - vb0][t - tb0] (ldGt)
// with G = s_t (M_t q_t[v] - p~_t[v]); rows t >= T and columns v >= V get 0.
// bf16 writes G alone (Gt must be null: its contractions read G k-major).
template <class C>
__global__ __launch_bounds__(C::NTHREADS) void bwd_grad_kernel(
    const typename C::TIn* __restrict__ H, const typename C::TIn* __restrict__ W, int T, int d, int V, int K,
    const int* __restrict__ idx_s, const float* __restrict__ p_s, const float* __restrict__ Mrow,
    const float* __restrict__ lse, const float* __restrict__ srow, int tb0, int vb0, int n_vtiles,
    int tiles_per_split, int n_tblocks, int n_splits, typename C::TIn* __restrict__ G, int64_t ldG,
    typename C::TIn* __restrict__ Gt, int64_t ldGt, const int* __restrict__ nrows) {
  using TIn = typename C::TIn;
  // bf16 256 x 256 tiles leave the kernel through the LDS (the whole tile,
  // 128 KiB, once the main loop is done with it) as 16-byte stores that
  // form 512-byte runs of G rows; otherwise straight from registers.
  // Staging also frees the registers the substep pipeline of the main loop
  // needs.
  constexpr bool kStage = std::is_same<TIn, bf16_t>::value && C::BM == 256 && C::BN == 256 && C::WM == 128 &&
                          C::LDS_BYTES >= 256 * 256 * 2 && PrefetchOK<C>::value;
  // after the stages: the row constants and the teacher walk's slots (below)
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES + C::BN * 16 + C::NB * C::NTHREADS * 8];
  uint16_t* stg = reinterpret_cast<uint16_t*>(smem);
  // 16-byte chunk c of token row t sits at c ^ (t / 8): the column reads of
  // eight consecutive rows spread over the banks
  auto stage_chunk = [](int t, int c) { return c ^ ((t >> 3) & 31); };
  (void)stg;
  (void)stage_chunk;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wave_m = wave / C::WAVES_N;
  const int wave_n = wave % C::WAVES_N;
  int tblock, split;
  grouped_mn(xcd_remap(blockIdx.x, n_tblocks * n_splits), n_tblocks, n_splits, kGroupT, tblock, split);
  const int t0 = tb0 + tblock * C::BN;
  // packed rows: token blocks wholly past the kept rows are skipped (the
  // contractions read no G row of them)
  if (nrows != nullptr && t0 >= *nrows) return;
  const int vt0 = split * tiles_per_split;
  const int vt1 = min(n_vtiles, vt0 + tiles_per_split);

  // Row constants of the block's BN token rows, read by every tile's
  // epilogue from LDS (after the main loop's stages): (s M, LSE log2e, s).
  // Rows past T and rows of zero scale get (0, +inf, 0), which makes their g
  // exactly zero (their logits are finite: operand rows past T load as zeros).
  float4* s_row = reinterpret_cast<float4*>(smem + C::LDS_BYTES);
  // Teacher walk, one cursor per lane and column block: position cur of the
  // next teacher entry nxt at or after the tile's first row (registers), and
  // that entry's p and the index after it in LDS, refilled by global->LDS
  // loads after the tile that moved the cursor, so that an epilogue with at
  // most one hit per token waits for no global load.
  int* s_nx = reinterpret_cast<int*>(smem + C::LDS_BYTES + C::BN * sizeof(float4));  // [NB][NTHREADS]
  float* s_pc = reinterpret_cast<float*>(s_nx + C::NB * C::NTHREADS);                 // [NB][NTHREADS]
  for (int i = threadIdx.x; i < C::BN; i += C::NTHREADS) {
    const int tok = t0 + i;
    float4 rc = make_float4(0.f, INFINITY, 0.f, 0.f);
    if (tok < T) {
      const float sc = srow[tok];
      if (sc != 0.f) rc = make_float4(sc * Mrow[tok], lse[tok] * kLog2e, sc, 0.f);
    }
    s_row[i] = rc;
  }
  int cur[C::NB], nxt[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    const int tok = t0 + wave_n * C::WN + nb * 32 + (lane & 31);
    cur[nb] = K;
    nxt[nb] = kIdxEnd;
    int nx = kIdxEnd;
    float pc = 0.f;
    if (tok < T) {
      const int* row = idx_s + (int64_t)tok * K;
      cur[nb] = lower_bound_row(row, K, vb0 + vt0 * C::BM);
      if (cur[nb] < K) {
        nxt[nb] = row[cur[nb]];
        pc = p_s[(int64_t)tok * K + cur[nb]];
      }
      if (cur[nb] + 1 < K) nx = row[cur[nb] + 1];
    }
    s_nx[nb * C::NTHREADS + threadIdx.x] = nx;
    s_pc[nb * C::NTHREADS + threadIdx.x] = pc;
  }
  __syncthreads();

  // The slots of the lanes whose cursor moved in a tile are refilled after
  // that tile's LDS work (p of entry cur, index of entry cur + 1; a slot
  // past the list is never read: the walk stops at K), by global->LDS loads
  // that the next tile's main loop waits for.
  auto refill = [&](int moved) {
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
      if (moved & (1 << nb)) {
        const int64_t e = (int64_t)(t0 + wave_n * C::WN + nb * 32 + (lane & 31)) * K + cur[nb];
        if (cur[nb] < K) lds_dma4(p_s + e, s_pc + nb * C::NTHREADS + wave * 64);
        if (cur[nb] + 1 < K) lds_dma4(idx_s + e + 1, s_nx + nb * C::NTHREADS + wave * 64);
      }
  };
  typename C::TileT tile;
  if constexpr (kStage)
    if (vt0 < vt1)
      tile_k64_prologue<C>(W + (int64_t)(vb0 + vt0 * C::BM) * d, d, V - vb0 - vt0 * C::BM, H + (int64_t)t0 * d, d,
                           T - t0, d, smem);
  for (int vt = vt0; vt < vt1; ++vt) {
    const int v0 = vb0 + vt * C::BM;
    if constexpr (kStage) {
      run_mma<C, true>(tile, W + (int64_t)v0 * d, d, V - v0, H + (int64_t)t0 * d, d, T - t0, d, smem);
    } else {
      run_mma(tile, W + (int64_t)v0 * d, d, V - v0, H + (int64_t)t0 * d, d, T - t0, d, smem);
    }
    if constexpr (!kStage) wait_vmcnt<0>();  // the slots refilled after the previous tile
    const int vbase = v0 + wave_m * C::WM;
    const int vend = min(v0 + C::BM, V);
    const bool full = vbase + C::WM <= V;  // every row of the wave's slice is a vocabulary row
    int moved = 0;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      // (opaque: the addresses derived from it are formed here, not held in
      // registers across the main loop)
      const int tl = opaque(wave_n * C::WN + nb * 32 + (lane & 31));
      const int tok = t0 + tl;
      const float4 rc = s_row[tl];
      const float coef = rc.x, lse2 = rc.y;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tile.acc[mb][nb][r] = coef * fast_exp2(tile.acc[mb][nb][r] * kLog2e - lse2);
      if (!full) {  // the last tile: columns v >= V (zero operand rows) get 0
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vbase + mb * 32 + acc_row(r, lane) >= V) tile.acc[mb][nb][r] = 0.f;
      }
      int ccur = cur[nb], cnxt = nxt[nb];
      if (cnxt < vend) {
        const int slot = nb * C::NTHREADS + threadIdx.x;
        float pc = s_pc[slot];  // p of entry ccur
        int nx = s_nx[slot];    // index of entry ccur + 1
        do {
          // entry ccur (index cnxt) lies in this tile: subtract s p at its
          // register (in the lane of the right half of the 32-row block)
          const int vl = cnxt - vbase;
          const int rr = vl & 31;
          if (vl >= 0 && vl < C::WM && ((rr >> 2) & 1) == (lane >> 5)) {
            const int sel = (vl >> 5) * 16 + (rr >> 3) * 4 + (rr & 3);
            const float sp = rc.z * pc;
#pragma unroll
            for (int q = 0; q < C::MB * 16; ++q)
              if (q == sel) tile.acc[q / 16][nb][q % 16] -= sp;
          }
          ++ccur;
          cnxt = ccur < K ? nx : kIdxEnd;
          if (cnxt < vend) {  // another entry in this tile (rare): read the list directly
            pc = p_s[(int64_t)tok * K + ccur];
            nx = ccur + 1 < K ? idx_s[(int64_t)tok * K + ccur + 1] : kIdxEnd;
          }
        } while (cnxt < vend);
        cur[nb] = ccur;
        nxt[nb] = cnxt;
        moved |= 1 << nb;
      }
      if constexpr (kStage) {
        // g of this lane's token column into the LDS tile [t][v]: registers
        // 4i .. 4i + 3 hold vocabulary rows 8i + 4 (lane / 32) .. + 3, one
        // 8-byte half of the 16-byte chunk (wave_m 16 + mb 4 + i)
        uint2* row = reinterpret_cast<uint2*>(stg + tl * 256);
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            row[stage_chunk(tl, wave_m * 16 + mb * 4 + i) * 2 + (lane >> 5)] =
                make_uint2(pack_bf16x2(tile.acc[mb][nb][4 * i], tile.acc[mb][nb][4 * i + 1]),
                           pack_bf16x2(tile.acc[mb][nb][4 * i + 2], tile.acc[mb][nb][4 * i + 3]));
      } else {
        // G rows: four consecutive vocabulary entries per register group
        const int64_t trow = tok - tb0;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int vcol = vbase - vb0 + mb * 32 + 8 * i + 4 * (lane >> 5);
            store4<TIn>(G + trow * ldG + vcol, tile.acc[mb][nb][4 * i], tile.acc[mb][nb][4 * i + 1],
                        tile.acc[mb][nb][4 * i + 2], tile.acc[mb][nb][4 * i + 3]);
          }
        // G^T rows: neighbouring lanes hold neighbouring tokens; swap one value
        // so that each lane writes a pair of tokens for one vocabulary entry.
        const bool odd = lane & 1;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float a0 = tile.acc[mb][nb][r], a1 = tile.acc[mb][nb][r + 1];
            const float recv = __shfl_xor(odd ? a0 : a1, 1);
            const int vrow = vbase - vb0 + mb * 32 + acc_row(r, lane);
            if (!odd) store2<TIn>(Gt + (int64_t)vrow * ldGt + trow, a0, recv);
            else store2<TIn>(Gt + (int64_t)(vrow + 1) * ldGt + trow - 1, recv, a1);
          }
      }
    }
    if constexpr (kStage) {
      // G rows: 32 threads per token row of 256 entries (512 bytes).  The
      // tile is read out of the LDS into registers first, so that the next
      // tile's first two slices go into the stages before the stores are
      // issued: their latencies overlap, and the next loop waits for both.
      __syncthreads();
      const int tid = opaque(threadIdx.x);  // (addresses formed here, not held across the loop)
      constexpr int kPasses = 256 / (C::NTHREADS / 32);
      u32x4 out[kPasses];
#pragma unroll
      for (int pass = 0; pass < kPasses; ++pass) {
        const int tl = pass * (C::NTHREADS / 32) + (tid >> 5), q = tid & 31;
        out[pass] = reinterpret_cast<const u32x4*>(stg + tl * 256)[stage_chunk(tl, q)];
      }
      __syncthreads();
      if (vt + 1 < vt1)
        tile_k64_prologue<C>(W + (int64_t)(v0 + C::BM) * d, d, V - v0 - C::BM, H + (int64_t)t0 * d, d, T - t0, d,
                             smem);
      refill(moved);
      bf16_t* Gtile = G + (int64_t)(t0 - tb0) * ldG + (v0 - vb0);
      // non-temporal: the G block (hundreds of MB) is read back by the
      // contractions from memory anyway, so its lines need not stay in the
      // caches that hold this kernel's operand panels (measured -1.5% on
      // this kernel)
#pragma unroll
      for (int pass = 0; pass < kPasses; ++pass) {
        const int tl = pass * (C::NTHREADS / 32) + (tid >> 5), q = tid & 31;
        __builtin_nontemporal_store(out[pass], reinterpret_cast<u32x4*>(Gtile + (int64_t)tl * ldG + q * 8));
      }
    } else {
      refill(moved);
    }
  }
}

// ------------------------------------------------ fused G formation (gpass) --
// fp32: the fused forward + backward keeps u = 2^(z log2e - m) of every logit
// of a row chunk in G (see fwd_lse_kernel).  Once the chunk's LSE is known, one
// 128 x 128 (token x vocabulary) tile per block turns u into
//   g = s_t M_t u 2^(m - LSE_t log2e)  ( = s_t M_t exp(z - LSE_t) )
// in place and writes the transpose G^T through LDS; HBM traffic 3 elements
// per entry.  The teacher columns are corrected afterwards (gfix_kernel).
template <typename TIn>
__global__ __launch_bounds__(256) void gpass_kernel(TIn* __restrict__ G, int64_t ldG, TIn* __restrict__ Gt,
                                                    int64_t ldGt, const float* __restrict__ mtab, int64_t ldm,
                                                    const float* __restrict__ srow, const float* __restrict__ Mrow,
                                                    const float* __restrict__ lse, int rows, int V, int tile_m,
                                                    int wave_rows) {
  constexpr bool kBF16 = sizeof(TIn) == 2;
  constexpr int E = 16 / (int)sizeof(TIn);  // entries per 16-byte chunk
  constexpr int CPR = 128 / E;              // chunks per 128-entry row
  constexpr int RPP = 256 / CPR;            // rows per pass of the block
  constexpr int LDT = kBF16 ? 130 : 129;    // LDS row stride (elements)
  using TS = typename std::conditional<kBF16, uint16_t, float>::type;
  __shared__ TS tr[128 * LDT];  // tr[v_local][t_local]
  const int t0 = blockIdx.y * 128, v0 = blockIdx.x * 128;
  const int c = threadIdx.x % CPR, rr = threadIdx.x / CPR;
  const int vc = v0 + c * E;  // first vocabulary entry of this thread's chunks
  // all E entries of a chunk share the tile and the wave row block, whose
  // maximum m the forward kept in mtab
  const int64_t grp = (int64_t)(vc / tile_m) * (tile_m / wave_rows) + (vc % tile_m) / wave_rows;
  constexpr int NR = 128 / RPP;  // rows per thread
  // all loads first (the in-place stores would otherwise order each row's
  // load after the previous row's store, leaving one load in flight)
  using VT = typename std::conditional<kBF16, u32x4, f32x4>::type;
  VT x[NR];
  float f0[NR];
  bool ok[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int t = t0 + rr + j * RPP;
    x[j] = *reinterpret_cast<const VT*>(G + (int64_t)t * ldG + vc);
    f0[j] = 0.f;
    ok[j] = false;
    if (t < rows) {
      const float sc = srow[t];
      if (sc != 0.f) {
        ok[j] = true;
        const float coef = sc * Mrow[t];
        const float l2 = lse[t] * kLog2e;
        f0[j] = coef * fast_exp2(mtab[grp * ldm + t] - l2);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int i = rr + j * RPP;
    const int t = t0 + i;
    // rows past `rows` and masked rows may hold stale u: select, never
    // multiply, so that they come out as exact zeros
    TIn* gp = G + (int64_t)t * ldG + vc;
    if constexpr (kBF16) {
      u32x4 y;
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        const float u0 = bf16_bits_to_f32(x[j][e >> 1] & 0xffffu);
        const float u1 = bf16_bits_to_f32(x[j][e >> 1] >> 16);
        const float g0 = (ok[j] && vc + e < V) ? u0 * f0[j] : 0.f;
        const float g1 = (ok[j] && vc + e + 1 < V) ? u1 * f0[j] : 0.f;
        y[e >> 1] = pack_bf16x2(g0, g1);
      }
      *reinterpret_cast<u32x4*>(gp) = y;
#pragma unroll
      for (int e = 0; e < E; ++e) tr[(c * E + e) * LDT + i] = (uint16_t)((y[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    } else {
      f32x4 y;
#pragma unroll
      for (int e = 0; e < E; ++e) y[e] = (ok[j] && vc + e < V) ? x[j][e] * f0[j] : 0.f;
      *reinterpret_cast<f32x4*>(gp) = y;
#pragma unroll
      for (int e = 0; e < E; ++e) tr[(c * E + e) * LDT + i] = y[e];
    }
  }
  __syncthreads();
  for (int i = rr; i < 128; i += RPP) {  // vocabulary row v0 + i, tokens t0 + c E ..
    TIn* dst = Gt + (int64_t)(v0 + i) * ldGt + t0 + c * E;
    const TS* src = tr + i * LDT + c * E;
    if constexpr (kBF16) {
      u32x4 y;
#pragma unroll
      for (int e = 0; e < E; e += 2) y[e >> 1] = (uint32_t)src[e] | ((uint32_t)src[e + 1] << 16);
      *reinterpret_cast<u32x4*>(dst) = y;
    } else {
      f32x4 y;
#pragma unroll
      for (int e = 0; e < E; ++e) y[e] = src[e];
      *reinterpret_cast<f32x4*>(dst) = y;
    }
  }
}

// bf16: u arrives in the forward's tile order (one 256 x 256 token x
// vocabulary tile = 128 KiB, whole 1 KiB runs per wave store).  One block per
// half tile (128 tokens: the forward waves with wave_n in {2 th, 2 th + 1},
// four runs of 16 KiB) reads it in 16-byte chunks, forms g as above and
// stages it in LDS as [t][v] (rows of 512 bytes; the 16-byte chunk c of row t
// sits at c ^ (t / 8), so that eight-row column reads spread over the banks),
// then writes G rows and, through 8 x 8 register transposes, G^T rows, in
// 512- and 256-byte runs (G^T only when Gt is not null: the dW contraction
// can read G itself k-major).  64 KiB of LDS: two blocks per CU, one reading
// while the other writes.  HBM traffic 3 elements per entry (2 without G^T),
// in whole cache lines.
template <int TH>
__global__ __launch_bounds__(256 * TH) void gpass_tiles_kernel(const bf16_t* __restrict__ U, int n_vtiles,
                                                               bf16_t* __restrict__ G, int64_t ldG,
                                                               bf16_t* __restrict__ Gt, int64_t ldGt,
                                                               const float* __restrict__ mtab, int64_t ldm,
                                                               const float* __restrict__ srow,
                                                               const float* __restrict__ Mrow,
                                                               const float* __restrict__ lse, int rows, int V,
                                                               const int* __restrict__ nrows, int row0) {
  using C = CfgBF16;
  static_assert(C::BM == 256 && C::BN == 256 && C::WM == 128 && C::WN == 64 && C::MB == 4 && C::NB == 2 &&
                    C::WAVES_M == 2 && C::WAVES_N == 4,
                "tile order written by fwd_lse_kernel");
  static_assert(TH == 1 || TH == 2, "64 or 128 tokens per block");
  constexpr int NT = 256 * TH;    // threads
  constexpr int TR = 64 * TH;     // token rows of the slab
  constexpr int NCH = TR * 32;    // 16-byte chunks of the slab (and per thread: NCH / NT = 8)
  __shared__ __attribute__((aligned(16))) uint16_t tr[TR * 256];
  __shared__ float fs[2][TR];  // g / u per (wave_m, token): s_t M_t 2^(m - LSE_t log2e), 0 for no gradient
  const int vt = blockIdx.x, tb = blockIdx.y / (4 / TH), th = blockIdx.y % (4 / TH);
  const int t0 = tb * 256 + th * TR, v0 = vt * 256;
  // packed rows: whole 256-row tiles past the kept rows are skipped (the
  // forward kept no u for them; the contractions read none of their rows)
  if (nrows != nullptr && tb * 256 >= *nrows - row0) return;
  const int tid = threadIdx.x;
  const u32x4* ut = reinterpret_cast<const u32x4*>(U + ((int64_t)tb * n_vtiles + vt) * (256 * 256));
  auto phys = [](int t, int c) { return c ^ ((t >> 3) & 31); };
  // wave w of the forward wrote its 16 KiB (1024 chunks) at chunk 1024 w; this
  // slab holds the waves with wave_n in [TH th, TH th + TH), for wave_m 0 and 1
  auto src_chunk = [&](int c) {
    const int p = c >> 10;  // TH pieces per wave_m
    return (((p % TH) + TH * th + 4 * (p / TH)) << 10) + (c & 1023);
  };
  // u is read once: non-temporal loads (measured ~6% faster on this kernel)
  u32x4 x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = __builtin_nontemporal_load(&ut[src_chunk(j * NT + tid)]);
  if (tid < 2 * TR) {
    const int wm = tid / TR, tl = tid % TR, t = t0 + tl;
    float f = 0.f;
    if (t < rows) {
      const float sc = srow[t];
      if (sc != 0.f) f = sc * Mrow[t] * fast_exp2(mtab[((int64_t)vt * C::WAVES_M + wm) * ldm + t] - lse[t] * kLog2e);
    }
    fs[wm][tl] = f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = j * NT + tid;
    const int p = c >> 10, cw = c & 1023;
    const int lane = cw & 63, h = (cw >> 6) & 1, nb = (cw >> 7) & 1, mb = (cw >> 8) & 3, wm = p / TH;
    const int tl = (p % TH) * 64 + nb * 32 + (lane & 31);
    const int vl = wm * 128 + mb * 32 + 16 * h + 4 * (lane >> 5);  // elements 0-3: vl.., 4-7: vl + 8..
    const float f = fs[wm][tl];
    // rows past `rows` and masked rows (f = 0) may hold stale u: select,
    // never multiply, so that they come out as exact zeros
    uint32_t y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int va = v0 + vl + (e < 2 ? 2 * e : 8 + 2 * (e - 2));
      const float u0 = bf16_bits_to_f32(x[j][e] & 0xffffu), u1 = bf16_bits_to_f32(x[j][e] >> 16);
      const float g0 = (f != 0.f && va < V) ? u0 * f : 0.f;
      const float g1 = (f != 0.f && va + 1 < V) ? u1 * f : 0.f;
      y[e] = pack_bf16x2(g0, g1);
    }
    uint2* row = reinterpret_cast<uint2*>(tr + tl * 256);
    // 8-byte halves: v = vl .. vl + 3 (chunk vl / 8, half (vl / 4) % 2) and v + 8 (next chunk)
    row[phys(tl, vl >> 3) * 2 + ((vl >> 2) & 1)] = make_uint2(y[0], y[1]);
    row[phys(tl, (vl >> 3) + 1) * 2 + ((vl >> 2) & 1)] = make_uint2(y[2], y[3]);
  }
  __syncthreads();
  // G rows: 32 threads per row of 256 entries
#pragma unroll
  for (int pass = 0; pass < 8; ++pass) {
    const int tl = pass * (NT / 32) + (tid >> 5), q = tid & 31;
    const u32x4 v = reinterpret_cast<const u32x4*>(tr + tl * 256)[phys(tl, q)];
    *reinterpret_cast<u32x4*>(G + (int64_t)(t0 + tl) * ldG + v0 + q * 8) = v;
  }
  // G^T rows (when asked for): thread (tq, vb) transposes the 8 x 8 block of
  // tokens 8 tq .., vocabulary rows 8 vb ..; TR / 8 threads write one row run
  // of 2 TR bytes
  if (Gt != nullptr) {
    constexpr int NTQ = TR / 8;
    const int tq = tid % NTQ, vb = tid / NTQ;
    u32x4 a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = reinterpret_cast<const u32x4*>(tr + (tq * 8 + i) * 256)[vb ^ tq];
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // vocabulary rows 2w (low halves) and 2w + 1 (high halves)
      u32x4 lo, hi;
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        lo[i2] = __builtin_amdgcn_perm(a[2 * i2 + 1][w], a[2 * i2][w], 0x05040100u);
        hi[i2] = __builtin_amdgcn_perm(a[2 * i2 + 1][w], a[2 * i2][w], 0x07060302u);
      }
      *reinterpret_cast<u32x4*>(Gt + (int64_t)(v0 + vb * 8 + 2 * w) * ldGt + t0 + tq * 8) = lo;
      *reinterpret_cast<u32x4*>(Gt + (int64_t)(v0 + vb * 8 + 2 * w + 1) * ldGt + t0 + tq * 8) = hi;
    }
  }
}

// Teacher columns: g = s_t (M_t 2^(zg log2e - LSE_t log2e) - p), the same
// fp32 expression the recomputing backward evaluates, rounded once (into G,
// and into G^T when Gt is not null).
template <typename TIn>
__global__ __launch_bounds__(256) void gfix_kernel(int rows, int K, int V, const int* __restrict__ idx_s,
                                                   const float* __restrict__ p_s, const float* __restrict__ zg_s,
                                                   const float* __restrict__ srow, const float* __restrict__ Mrow,
                                                   const float* __restrict__ lse, TIn* __restrict__ G, int64_t ldG,
                                                   TIn* __restrict__ Gt, int64_t ldGt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * K) return;
  const int t = (int)(i / K);
  const float sc = srow[t];
  if (sc == 0.f) return;  // the row is already zero
  const int v = idx_s[i];
  if (v < 0 || v >= V) return;  // unchecked bad index: matches no column
  const float coef = sc * Mrow[t];
  const float g = coef * fast_exp2(zg_s[i] * kLog2e - lse[t] * kLog2e) - sc * p_s[i];
  if constexpr (sizeof(TIn) == 2) {
    const uint16_t b = (uint16_t)f32_to_bf16_bits(g);
    reinterpret_cast<uint16_t*>(G)[(int64_t)t * ldG + v] = b;
    if (Gt != nullptr) reinterpret_cast<uint16_t*>(Gt)[(int64_t)v * ldGt + t] = b;
  } else {
    G[(int64_t)t * ldG + v] = g;
    if (Gt != nullptr) Gt[(int64_t)v * ldGt + t] = g;
  }
}

// out[i] = part[i] + part[pstride + i] + ... (S terms, this order), 4 per thread.
// Packed rows (rowmap not NULL, rows of d elements): row r of the sum goes to
// row rowmap[r] of out, for r < *nrows - row0 only.
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* __restrict__ part, int64_t pstride, int S,
                                                         int64_t n4, void* __restrict__ out, int out_bf16,
                                                         const int* __restrict__ rowmap, const int* __restrict__ nrows,
                                                         int row0, int d) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  int64_t o = i;
  if (rowmap != nullptr) {
    const int q = d / 4;
    const int r = (int)(i / q);
    if (r >= *nrows - row0) return;
    o = (int64_t)rowmap[r] * q + (i - (int64_t)r * q);
  }
  f32x4 a = reinterpret_cast<const f32x4*>(part)[i];
  for (int s = 1; s < S; ++s) a += reinterpret_cast<const f32x4*>(part + s * pstride)[i];
  if (out_bf16)
    store4<bf16_t>(reinterpret_cast<bf16_t*>(out) + 4 * o, a[0], a[1], a[2], a[3]);
  else
    reinterpret_cast<f32x4*>(out)[o] = a;
}

// ------------------------------------------------------ plain contraction --
// out[m, n] (+)= sum_k X[m, k] Y[n, k] for m < M, n < N (fp32 out).  Two
// independent problems share one launch (the dH and dW products of a G
// block): workgroups [0, p0.tiles) take problem 0, the rest problem 1 (each
// spread over the XCDs separately), so the tail of one fills the machine with
// tiles of the other.
//
// A problem may be a batch of `batches` products of the same shape whose
// operands and outputs sit xb, yb and ob elements apart, the last one with
// k extent kdim_last (split-k over a long contraction: each split writes its
// own partial output, summed later in a fixed order).
template <typename TIn>
struct GemmProblem {
  const TIn* X;
  int64_t ldx;
  const TIn* Y;
  int64_t ldy;
  float* out;
  int64_t ldo;
  int M, N, kdim, beta;
  int batches, kdim_last;
  int64_t xb, yb, ob;
  int xt;              // X k-major (Dma64 configurations with the substep pipeline)
  int tiles_m, tiles;  // tiles_m = ceil(M / BM); tiles = tiles_m * ceil(N / BN) * batches
  // packed rows: lim_kind 1 bounds M, 2 bounds kdim, by *lim - lim_base
  // (kdim rounded up to lim_round, the rows of whole G tiles)
  const int* lim;
  int lim_base, lim_kind, lim_round;
};

constexpr int kGroupM = 2;

// Configurations whose main loop can take X k-major.
template <class C>
constexpr bool kXtOK = false;
template <int BM, int BN, int WM, int WN>
constexpr bool kXtOK<Dma64Cfg<BM, BN, WM, WN>> = BM % 128 == 0;

template <class C>
__global__ __launch_bounds__(C::NTHREADS) void gemm_store_kernel(GemmProblem<typename C::TIn> p0,
                                                                 GemmProblem<typename C::TIn> p1) {
  // bf16 configurations stage the fp32 output through LDS one wave row block
  // at a time and bring the old values of the read-modify-write in beside it
  // by global->LDS loads: two blocks of WM x BN fp32, up to 160 KiB.
  constexpr int kOldDma = std::is_same<typename C::TIn, bf16_t>::value && 2 * C::WM * C::BN * 4 <= 160 * 1024 ? 1 : 0;
  constexpr int kSmem = kOldDma && 2 * C::WM * C::BN * 4 > C::LDS_BYTES ? 2 * C::WM * C::BN * 4 : C::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wave_m = wave / C::WAVES_N;
  const int wave_n = wave % C::WAVES_N;
  // Each problem is spread over all XCDs on its own (problem 1 starts at a
  // multiple of 8 workgroups, so w % 8 still names the XCD): remapping the
  // two together would put the first problem's tiles, often the long ones,
  // on the first XCDs only.
  const int n0p = (p0.tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  int bid = blockIdx.x;
  const bool second = bid >= n0p;  // workgroup-uniform
  if (!second) {
    bid = xcd_remap(bid, n0p);
    if (bid >= p0.tiles) return;  // padding workgroup
  } else {
    bid = xcd_remap(bid - n0p, p1.tiles);
  }
  // field-wise selection keeps the by-value kernel arguments in registers
  const typename C::TIn* X = second ? p1.X : p0.X;
  const typename C::TIn* Y = second ? p1.Y : p0.Y;
  float* out = second ? p1.out : p0.out;
  const int64_t ldx = second ? p1.ldx : p0.ldx, ldy = second ? p1.ldy : p0.ldy, ldo = second ? p1.ldo : p0.ldo;
  const int M = second ? p1.M : p0.M, N = second ? p1.N : p0.N, kdim_all = second ? p1.kdim : p0.kdim;
  const int beta = second ? p1.beta : p0.beta;
  const int tiles_m = second ? p1.tiles_m : p0.tiles_m, tiles = second ? p1.tiles : p0.tiles;
  const int batches = second ? p1.batches : p0.batches;
  const int per_batch = tiles / batches;
  const int bt = bid / per_batch;
  bid -= bt * per_batch;
  if (bt > 0) {
    X += bt * (second ? p1.xb : p0.xb);
    Y += bt * (second ? p1.yb : p0.yb);
    out += bt * (second ? p1.ob : p0.ob);
  }
  int kdim = bt == batches - 1 ? (second ? p1.kdim_last : p0.kdim_last) : kdim_all;
  int tm, tn;
  grouped_mn(bid, tiles_m, per_batch / tiles_m, kGroupM, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  // packed rows: tiles past the kept rows are skipped, contractions over
  // token rows stop after them (a skipped k range adds nothing: with beta the
  // tile is left as it is, without it the zero tile is still written)
  int M_eff = M;
  {
    const int* lim = second ? p1.lim : p0.lim;
    if (lim != nullptr) {
      const int kind = second ? p1.lim_kind : p0.lim_kind;
      const int n_lim = *lim - (second ? p1.lim_base : p0.lim_base);
      if (kind == 1) {
        M_eff = max(0, min(M, n_lim));
        if (m0 >= M_eff) return;
      } else if (kind == 2) {
        const int rnd = second ? p1.lim_round : p0.lim_round;
        const int kl = n_lim <= 0 ? 0 : (n_lim + rnd - 1) / rnd * rnd;
        kdim = min(kdim, kl);
        if (kdim <= 0 && beta) return;
      }
    }
  }
  using TileT = typename C::TileT;
  using L = typename TileT::L;
  TileT tile;
  if constexpr (kXtOK<C>) {
    if (second ? p1.xt : p0.xt)
      run_mma<C, false, true>(tile, X + m0, ldx, M_eff - m0, Y + (int64_t)n0 * ldy, ldy, N - n0, kdim, smem);
    else
      run_mma(tile, X + (int64_t)m0 * ldx, ldx, M_eff - m0, Y + (int64_t)n0 * ldy, ldy, N - n0, kdim, smem);
  } else {
    run_mma(tile, X + (int64_t)m0 * ldx, ldx, M_eff - m0, Y + (int64_t)n0 * ldy, ldy, N - n0, kdim, smem);
  }
  if constexpr (C::WM * C::BN * 4 <= C::LDS_BYTES) {
    // The fp32 tile goes out through LDS, the WM rows of one wave_m at a
    // time, so that each thread reads / writes 16 contiguous bytes of an
    // output row: in the MFMA layout a lane holds one column, and the
    // read-modify-write would take 4-byte accesses to 32 rows per
    // instruction (measured ~1.6x slower for the fp32 dW update).
    float* st = reinterpret_cast<float*>(smem);
    constexpr int PART = C::WM;
    // the lane groups of a column write rows 4 apart: their columns are
    // offset by BLK per group so that one store touches distinct banks
    // (16-byte runs stay contiguous for the reads below)
    auto stage_swz = [](int ml) { return ((ml >> 2) & (L::GROUPS - 1)) * L::BLK; };
    static_assert(C::BN % (L::GROUPS * L::BLK) == 0, "the swizzle stays inside a row");
    const bool vec_ok = (ldo % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & 15) == 0);
    if constexpr (kOldDma) {
      if (vec_ok) {
        // Old values (dW update): the part's rows go global->LDS into the
        // second block (chunk q = row * BN / 4 + column / 4 at 16 q bytes,
        // 64 chunks per wave load), issued before the staging so that their
        // latency overlaps it; one wait and barrier per part.
        float* oldb = st + PART * C::BN;
        constexpr int CPR = C::BN / 4;                 // 16-byte chunks per row
        constexpr int NLD = PART * CPR / 64 / C::NWAVES;  // wave loads per part
        static_assert(PART * CPR % (64 * C::NWAVES) == 0, "whole wave loads");
#pragma unroll 1
        for (int part = 0; part < C::WAVES_M; ++part) {
          const int r0 = m0 + part * PART;
          if (beta && r0 < M_eff) {
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(out + (int64_t)r0 * ldo, (uint32_t)(min(M_eff - r0, PART) * ldo * 4));
#pragma unroll
            for (int k = 0; k < NLD; ++k) {
              const int q = (k * C::NWAVES + wave) * 64 + lane;
              const int row = q / CPR, c4 = (q % CPR) * 4;
              const bool in = n0 + c4 + 4 <= N;
              lds_dma_buf(ro, in ? (uint32_t)((row * ldo + n0 + c4) * 4) : kOutOfRange, 0u,
                          oldb + (k * C::NWAVES + wave) * 256);
            }
          }
          if (wave_m == part) {
#pragma unroll
            for (int mb = 0; mb < TileT::MBK; ++mb)
#pragma unroll
              for (int nb = 0; nb < TileT::NBK; ++nb) {
                const int nl = wave_n * C::WN + nb * L::BLK + (lane & (L::BLK - 1));
#pragma unroll
                for (int r = 0; r < L::RPB; ++r) {
                  const int ml = mb * L::BLK + L::row_in(r, lane);
                  st[ml * C::BN + (nl ^ stage_swz(ml))] = tile.acc[mb][nb][r];
                }
              }
          }
          wait_vmcnt<0>();
          __syncthreads();
          for (int i = threadIdx.x; i < PART * CPR; i += C::NTHREADS) {
            const int ml = i / CPR, c4 = (i % CPR) * 4;
            const int m = r0 + ml, n = n0 + c4;
            if (m >= M_eff || n >= N) continue;
            const f32x4 a = *reinterpret_cast<const f32x4*>(st + ml * C::BN + (c4 ^ stage_swz(ml)));
            float* o = out + (int64_t)m * ldo + n;
            if (n + 4 <= N) {
              *reinterpret_cast<f32x4*>(o) = beta ? a + *reinterpret_cast<const f32x4*>(oldb + i * 4) : a;
            } else {
              for (int e = 0; e < 4 && n + e < N; ++e) o[e] = beta ? o[e] + a[e] : a[e];
            }
          }
          __syncthreads();
        }
        return;
      }
    }
#pragma unroll
    for (int part = 0; part < C::WAVES_M; ++part) {
      if (wave_m == part) {
#pragma unroll
        for (int mb = 0; mb < TileT::MBK; ++mb)
#pragma unroll
          for (int nb = 0; nb < TileT::NBK; ++nb) {
            const int nl = wave_n * C::WN + nb * L::BLK + (lane & (L::BLK - 1));
#pragma unroll
            for (int r = 0; r < L::RPB; ++r) {
              const int ml = mb * L::BLK + L::row_in(r, lane);
              st[ml * C::BN + (nl ^ stage_swz(ml))] = tile.acc[mb][nb][r];
            }
          }
      }
      __syncthreads();
      // Every thread's old values are loaded before any of its stores: loads
      // and stores of one output array would otherwise stay in program order,
      // one round trip per 16 bytes.
      constexpr int PER = PART * (C::BN / 4) / C::NTHREADS;
      // float4 loads in flight (registers: the other parts' accumulators are live)
      constexpr int BATCH = PER % 8 == 0 ? 8 : PER % 5 == 0 ? 5 : PER % 4 == 0 ? 4 : PER < 8 ? PER : 1;
      static_assert(PART * (C::BN / 4) % C::NTHREADS == 0 && PER % BATCH == 0, "whole float4 batches");
#pragma unroll
      for (int j0 = 0; j0 < PER; j0 += BATCH) {
      f32x4 old[BATCH];
#pragma unroll
      for (int jj = 0; jj < BATCH; ++jj) {
        const int i = threadIdx.x + (j0 + jj) * C::NTHREADS;
        const int ml = i / (C::BN / 4), c4 = (i % (C::BN / 4)) * 4;
        const int m = m0 + part * PART + ml, n = n0 + c4;
        old[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (beta && vec_ok && m < M_eff && n + 4 <= N)
          old[jj] = *reinterpret_cast<const f32x4*>(out + (int64_t)m * ldo + n);
      }
#pragma unroll
      for (int jj = 0; jj < BATCH; ++jj) {
        const int j = jj;
        const int i = threadIdx.x + (j0 + jj) * C::NTHREADS;
        const int ml = i / (C::BN / 4), c4 = (i % (C::BN / 4)) * 4;
        const int m = m0 + part * PART + ml, n = n0 + c4;
        if (m >= M_eff || n >= N) continue;
        const float* sv = st + ml * C::BN + (c4 ^ stage_swz(ml));
        float* o = out + (int64_t)m * ldo + n;
        if (vec_ok && n + 4 <= N) {
          *reinterpret_cast<f32x4*>(o) = *reinterpret_cast<const f32x4*>(sv) + old[j];
        } else {
          for (int e = 0; e < 4 && n + e < N; ++e) o[e] = beta ? o[e] + sv[e] : sv[e];
        }
      }
      }
      __syncthreads();
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < TileT::MBK; ++mb)
#pragma unroll
      for (int nb = 0; nb < TileT::NBK; ++nb) {
        const int n = n0 + wave_n * C::WN + nb * L::BLK + (lane & (L::BLK - 1));
#pragma unroll
        for (int r = 0; r < L::RPB; ++r) {
          const int m = m0 + wave_m * C::WM + mb * L::BLK + L::row_in(r, lane);
          if (m < M_eff && n < N) {
            float* o = out + (int64_t)m * ldo + n;
            const float a = tile.acc[mb][nb][r];
            *o = beta ? *o + a : a;
          }
        }
      }
  }
}

// ---------------------------------------------------------------- launchers --

template <typename TIn>
struct CfgOf;
template <>
struct CfgOf<bf16_t> { using type = CfgBF16; using bwd = CfgBF16Bwd; using gemm = CfgBF16Gemm; };
template <>
struct CfgOf<float> { using type = CfgF32; using bwd = CfgF32; using gemm = CfgF32; };
static_assert(CfgBF16::BM == CfgBF16Gemm::BM && CfgBF16::BM == CfgBF16Bwd::BM && CfgBF16::BN == CfgBF16Bwd::BN,
              "row blocks of one size per dtype");

#define CKL_LAUNCH_CHECK() \
  do { hipError_t e_ = hipGetLastError(); if (e_ != hipSuccess) return e_; } while (0)

hipError_t launch_fill_i32(int* p, int n, int v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_count_mask(const uint8_t* mask, int T, int* N, hipStream_t st) {
  hipLaunchKernelGGL(count_mask_kernel, dim3(1), dim3(1024), 0, st, mask, T, N);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_row_scale(const uint8_t* mask, const float* grad_loss, const int* N, int T, int Tp, int packed,
                            float* s, hipStream_t st) {
  hipLaunchKernelGGL(row_scale_kernel, dim3((Tp + 255) / 256), dim3(256), 0, st, mask, grad_loss, N, T, Tp, packed, s);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_compact_rows(const uint8_t* mask, int T, int* perm, int* rank, int* N, hipStream_t st) {
  hipLaunchKernelGGL(compact_rows_kernel, dim3(1), dim3(1024), 0, st, mask, T, perm, rank, N);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_gather_rows(const void* src, int rows, int64_t row_bytes, const int* perm, const int* N, void* dst,
                              hipStream_t st) {
  if (row_bytes % 16) return hipErrorInvalidValue;
  const int64_t chunks = row_bytes / 16, n = (int64_t)rows * chunks;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const u32x4*)src,
                     chunks, perm, N, rows, (u32x4*)dst);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_gather_f32(const float* src, const int* perm, const int* N, int rows, float* dst, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_f32_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, src, perm, N, rows, dst);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_scatter_f32(const float* src, const int* rank, int T, float* dst, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_f32_kernel, dim3((T + 255) / 256), dim3(256), 0, st, src, rank, T, dst);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_scatter_rows(const float* src, const int* rank, int T, int d, void* dst, int dst_bf16,
                               hipStream_t st) {
  if (d % 4) return hipErrorInvalidValue;
  const int64_t n = (int64_t)T * (d / 4);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, rank, T, d, dst,
                     dst_bf16);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_zero_masked_rows(const int* rank, int T, int64_t row_bytes, void* dst, hipStream_t st) {
  if (row_bytes % 16) return hipErrorInvalidValue;
  const int64_t chunks = row_bytes / 16, n = (int64_t)T * chunks;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_masked_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, rank, T, chunks,
                     (u32x4*)dst);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_scale_cast(const float* src, void* dst, int64_t n, int dst_bf16, const float* scale,
                             hipStream_t st) {
  if (n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  hipLaunchKernelGGL(scale_cast_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, src, dst, n4, dst_bf16,
                     scale);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_teacher_prep(const int* idx, const float* tlogit, int T, int K, int V, int voff, int* idx_s,
                               float* p_s, float* Erow, float* Mrow, float* zg_s, int* bad, int logprob,
                               const int* rowmap, const int* nrows, hipStream_t st) {
  int Kp = 64;
  while (Kp < K) Kp <<= 1;
  const size_t lds = (size_t)Kp * 8;
  hipLaunchKernelGGL(teacher_prep_kernel, dim3(T), dim3(64), lds, st, idx, tlogit, T, K, Kp, V, voff, idx_s, p_s,
                     Erow, Mrow, zg_s, bad, logprob, rowmap, nrows);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

template <typename TIn>
static hipError_t fwd_lse_t(const void* H, const void* W, int T, int d, int V, int K, const int* idx_s, float* zg_s,
                            void* part, int n_splits, int tiles_per_split, void* G, int64_t ldG, float* mtab,
                            int64_t ldm, const int* nrows, int row0, hipStream_t st) {
  using C = typename CfgOf<TIn>::type;
  const int n_vtiles = (V + C::BM - 1) / C::BM;
  const int n_tblocks = (T + C::BN - 1) / C::BN;
  if (G)
    hipLaunchKernelGGL((fwd_lse_kernel<C, true>), dim3(n_tblocks * n_splits), dim3(C::NTHREADS), 0, st,
                       (const TIn*)H, (const TIn*)W, T, d, V, K, idx_s, zg_s, (float2*)part, n_vtiles,
                       tiles_per_split, n_tblocks, n_splits, (TIn*)G, ldG, mtab, ldm, nrows, row0);
  else
    hipLaunchKernelGGL((fwd_lse_kernel<C, false>), dim3(n_tblocks * n_splits), dim3(C::NTHREADS), 0, st,
                       (const TIn*)H, (const TIn*)W, T, d, V, K, idx_s, zg_s, (float2*)part, n_vtiles,
                       tiles_per_split, n_tblocks, n_splits, (TIn*)nullptr, (int64_t)0, (float*)nullptr,
                       (int64_t)0, nrows, row0);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_fwd_lse(int in_bf16, const void* H, const void* W, int T, int d, int V, int K, const int* idx_s,
                          float* zg_s, void* part, int n_splits, int tiles_per_split, void* G, int64_t ldG,
                          float* mtab, int64_t ldm, const int* nrows, int row0, hipStream_t st) {
  return in_bf16 ? fwd_lse_t<bf16_t>(H, W, T, d, V, K, idx_s, zg_s, part, n_splits, tiles_per_split, G, ldG, mtab,
                                     ldm, nrows, row0, st)
                 : fwd_lse_t<float>(H, W, T, d, V, K, idx_s, zg_s, part, n_splits, tiles_per_split, G, ldG, mtab,
                                    ldm, nrows, row0, st);
}

hipError_t launch_fwd_rows(const void* part, int S, int T, int K, const float* p_s, const float* zg_s,
                           const float* Erow, const float* Mrow, const uint8_t* mask, float* lse, float* row_loss,
                           double* row_ld, const int* nrows, int row0, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_finalize_kernel, dim3((T + 15) / 16), dim3(256), 0, st, (const float2*)part, S, T, K, p_s,
                     zg_s, Erow, Mrow, mask, lse, row_loss, row_ld, nrows, row0);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_loss_reduce(const double* row_ld, int T, const int* N, float* loss, hipStream_t st) {
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(1024), 0, st, row_ld, T, N, loss);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_fwd_shard_rows(const void* part, int S, int T, int K, const float* p_s, const float* zg_s,
                                 float* lse_part, float* cross_part, hipStream_t st) {
  hipLaunchKernelGGL(fwd_shard_rows_kernel, dim3((T + 255) / 256), dim3(256), 0, st, (const float2*)part, S, T, K, p_s,
                     zg_s, lse_part, cross_part);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_shard_combine(const float* lse_parts, const float* cross_parts, int S, int T, const float* Erow,
                                const float* Mrow, const uint8_t* mask, float* lse, float* row_loss, double* row_ld,
                                const int* N, float* loss, hipStream_t st) {
  const int nblk = (T + 255) / 256;
  hipLaunchKernelGGL(shard_combine_kernel, dim3(nblk), dim3(256), 0, st, lse_parts, cross_parts, S, T, Erow, Mrow,
                     mask, lse, row_loss, row_ld);
  CKL_LAUNCH_CHECK();
  return launch_loss_reduce(row_ld, T, N, loss, st);
}

hipError_t launch_transpose_pad(int in_bf16, const void* src, int R, int C, int Rp, void* dst, int64_t ldd,
                                hipStream_t st) {
  if (in_bf16 && C % 8 == 0 && Rp % 128 == 0 && ldd % 8 == 0) {
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3(Rp / 128, (C + 127) / 128), dim3(256), 0, st, (const bf16_t*)src, R,
                       C, Rp, (bf16_t*)dst, ldd);
    CKL_LAUNCH_CHECK();
    return hipSuccess;
  }
  dim3 grid((Rp + 63) / 64, (C + 63) / 64);
  if (in_bf16)
    hipLaunchKernelGGL(transpose_pad_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)src, R, C, Rp,
                       (bf16_t*)dst, ldd);
  else
    hipLaunchKernelGGL(transpose_pad_kernel<float>, grid, dim3(256), 0, st, (const float*)src, R, C, Rp, (float*)dst,
                       ldd);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_cast_f32_bf16(const float* src, void* dst, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(cast_f32_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, (bf16_t*)dst, n);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

template <typename TIn>
static hipError_t bwd_grad_t(const void* H, const void* W, int T, int d, int V, int K, const int* idx_s,
                             const float* p_s, const float* Mrow, const float* lse, const float* srow, int tb0,
                             int t_rows, int vb0, int v_rows, int n_splits, int tiles_per_split, void* G,
                             int64_t ldG, void* Gt, int64_t ldGt, const int* nrows, hipStream_t st) {
  using C = typename CfgOf<TIn>::bwd;
  if (sizeof(TIn) == 2 && Gt != nullptr) return hipErrorInvalidValue;  // bf16 forms G only
  const int n_vtiles = v_rows / C::BM;
  const int n_tblocks = t_rows / C::BN;
  hipLaunchKernelGGL(bwd_grad_kernel<C>, dim3(n_tblocks * n_splits), dim3(C::NTHREADS), 0, st, (const TIn*)H,
                     (const TIn*)W, T, d, V, K, idx_s, p_s, Mrow, lse, srow, tb0, vb0, n_vtiles, tiles_per_split,
                     n_tblocks, n_splits, (TIn*)G, ldG, (TIn*)Gt, ldGt, nrows);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_bwd_grad(int in_bf16, const void* H, const void* W, int T, int d, int V, int K, const int* idx_s,
                           const float* p_s, const float* Mrow, const float* lse, const float* srow, int tb0,
                           int t_rows, int vb0, int v_rows, int n_splits, int tiles_per_split, void* G, int64_t ldG,
                           void* Gt, int64_t ldGt, const int* nrows, hipStream_t st) {
  return in_bf16 ? bwd_grad_t<bf16_t>(H, W, T, d, V, K, idx_s, p_s, Mrow, lse, srow, tb0, t_rows, vb0, v_rows,
                                      n_splits, tiles_per_split, G, ldG, Gt, ldGt, nrows, st)
                 : bwd_grad_t<float>(H, W, T, d, V, K, idx_s, p_s, Mrow, lse, srow, tb0, t_rows, vb0, v_rows,
                                     n_splits, tiles_per_split, G, ldG, Gt, ldGt, nrows, st);
}

template <typename TIn>
static hipError_t gemm_pair_t(const GemmArgs& a0, const GemmArgs& a1, hipStream_t st) {
  using C = typename CfgOf<TIn>::gemm;
  GemmProblem<TIn> p[2];
  const GemmArgs* a[2] = {&a0, &a1};
  for (int i = 0; i < 2; ++i) {
    p[i].X = (const TIn*)a[i]->X;
    p[i].ldx = a[i]->ldx;
    p[i].Y = (const TIn*)a[i]->Y;
    p[i].ldy = a[i]->ldy;
    p[i].out = a[i]->out;
    p[i].ldo = a[i]->ldo;
    p[i].M = a[i]->M;
    p[i].N = a[i]->N;
    p[i].kdim = a[i]->kdim;
    p[i].beta = a[i]->beta;
    p[i].batches = a[i]->batches > 0 ? a[i]->batches : 1;
    p[i].kdim_last = a[i]->batches > 1 ? a[i]->kdim_last : a[i]->kdim;
    p[i].xb = a[i]->xb;
    p[i].yb = a[i]->yb;
    p[i].ob = a[i]->ob;
    p[i].xt = a[i]->xt;
    p[i].lim = a[i]->lim;
    p[i].lim_base = a[i]->lim_base;
    p[i].lim_kind = a[i]->lim ? a[i]->lim_kind : 0;
    p[i].lim_round = a[i]->lim_round > 0 ? a[i]->lim_round : 1;
    if (a[i]->lim && (a[i]->lim_kind < 1 || a[i]->lim_kind > 2 || (a[i]->lim_kind == 2 && a[i]->lim_round % 8)))
      return hipErrorInvalidValue;
    // k-major X: every tile reads BM whole columns of each k row
    if (a[i]->xt && (!kXtOK<C> || a[i]->batches > 1 || (int64_t)(a[i]->M + C::BM - 1) / C::BM * C::BM > a[i]->ldx))
      return hipErrorInvalidValue;
    p[i].tiles_m = a[i]->M > 0 ? (a[i]->M + C::BM - 1) / C::BM : 0;
    p[i].tiles = a[i]->M > 0 && a[i]->N > 0 ? p[i].tiles_m * ((a[i]->N + C::BN - 1) / C::BN) * p[i].batches : 0;
  }
  if (p[0].tiles + p[1].tiles == 0) return hipSuccess;
  const int n = (p[0].tiles + kNumXcd - 1) / kNumXcd * kNumXcd + p[1].tiles;
  hipLaunchKernelGGL(gemm_store_kernel<C>, dim3(n), dim3(C::NTHREADS), 0, st, p[0], p[1]);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_gemm_pair(int in_bf16, const GemmArgs& a0, const GemmArgs& a1, hipStream_t st) {
  return in_bf16 ? gemm_pair_t<bf16_t>(a0, a1, st) : gemm_pair_t<float>(a0, a1, st);
}

hipError_t launch_gpass(int in_bf16, void* G, int64_t ldG, void* Gt, int64_t ldGt, const float* mtab, int64_t ldm,
                        const float* srow, const float* Mrow, const float* lse, int rows, int rows_p, int V, int Vp,
                        hipStream_t st) {
  // (bf16 takes launch_gpass_tiles: the forward keeps its u in tile order)
  if (in_bf16 || rows_p % 128 || Vp % 128) return hipErrorInvalidValue;
  const dim3 grid(Vp / 128, rows_p / 128);
  hipLaunchKernelGGL(gpass_kernel<float>, grid, dim3(256), 0, st, (float*)G, ldG, (float*)Gt, ldGt, mtab, ldm, srow,
                     Mrow, lse, rows, V, CfgF32::BM, CfgF32::WM);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

constexpr int kGpassTH = 2;  // forward wave columns (64 tokens each) per G-formation block

hipError_t launch_gpass_tiles(const void* U, int n_vtiles, int n_tblocks, void* G, int64_t ldG, void* Gt,
                              int64_t ldGt, const float* mtab, int64_t ldm, const float* srow, const float* Mrow,
                              const float* lse, int rows, int V, const int* nrows, int row0, hipStream_t st) {
  if (n_vtiles < 1 || n_tblocks < 1) return hipSuccess;
  hipLaunchKernelGGL(gpass_tiles_kernel<kGpassTH>, dim3(n_vtiles, (4 / kGpassTH) * n_tblocks), dim3(256 * kGpassTH), 0,
                     st, (const bf16_t*)U, n_vtiles, (bf16_t*)G, ldG, (bf16_t*)Gt, ldGt, mtab, ldm, srow, Mrow, lse,
                     rows, V, nrows, row0);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_gfix(int in_bf16, int rows, int K, int V, const int* idx_s, const float* p_s, const float* zg_s,
                       const float* srow, const float* Mrow, const float* lse, void* G, int64_t ldG, void* Gt,
                       int64_t ldGt, hipStream_t st) {
  const int64_t n = (int64_t)rows * K;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (in_bf16)
    hipLaunchKernelGGL(gfix_kernel<bf16_t>, grid, dim3(256), 0, st, rows, K, V, idx_s, p_s, zg_s, srow, Mrow, lse,
                       (bf16_t*)G, ldG, (bf16_t*)Gt, ldGt);
  else
    hipLaunchKernelGGL(gfix_kernel<float>, grid, dim3(256), 0, st, rows, K, V, idx_s, p_s, zg_s, srow, Mrow, lse,
                       (float*)G, ldG, (float*)Gt, ldGt);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

hipError_t launch_splitk_sum(const float* part, int64_t pstride, int S, int64_t n, void* out, int out_bf16,
                             const int* rowmap, const int* nrows, int row0, int d, hipStream_t st) {
  if (n % 4 || pstride % 4 || (rowmap && (d % 4 || n % d))) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, pstride, S, n4,
                     out, out_bf16, rowmap, nrows, row0, d);
  CKL_LAUNCH_CHECK();
  return hipSuccess;
}

int tile_rows_m(int in_bf16) { return in_bf16 ? CfgBF16::BM : CfgF32::BM; }
int tile_rows_n(int in_bf16) { return in_bf16 ? CfgBF16::BN : CfgF32::BN; }
int gemm_tile_m(int in_bf16) { return in_bf16 ? CfgBF16Gemm::BM : CfgF32::BM; }
int gemm_tile_n(int in_bf16) { return in_bf16 ? CfgBF16Gemm::BN : CfgF32::BN; }
int lse_groups_per_tile(int in_bf16) { return in_bf16 ? CfgBF16::WAVES_M : CfgF32::WAVES_M; }

}  // namespace ckl
