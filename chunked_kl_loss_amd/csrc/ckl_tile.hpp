// LDS-tiled MFMA main loop shared by every contraction of the loss.
//
// Every product on the path is computed as C[m, n] = sum_k X[m, k] * Y[n, k]
// with both operands row-major and contiguous along k ("NT"):
//   logits      z^T[v, t] = sum_j W[v, j]  H[t, j]      (X = W,   Y = H)
//   dH          dH[t, j]  = sum_v G[t, v]  W^T[j, v]    (X = G,   Y = W^T)
//   dW          dW[v, j]  = sum_t G^T[v, t] H^T[j, t]   (X = G^T, Y = H^T)
// so one main loop serves all of them and only the epilogues differ; the bf16
// loop also takes X k-major (dW reads G itself, no G^T is formed).
//
// A workgroup owns a BM x BN output tile split over a WAVES_M x WAVES_N grid
// of 64-wide wavefronts; each wave owns WM x WN = (MB x NB) blocks of the
// 32x32 MFMA.  K is walked in BK slices staged through two LDS buffers: the
// bf16 loop loads them global->LDS directly (buffer_load ... lds), the fp32
// loop fetches the next slice into registers while the current one is
// multiplied.
#pragma once

#include <type_traits>

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

template <class C>
struct Tile;

template <typename TIn_, int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  using TIn = TIn_;
  using TileT = Tile<TileCfg>;
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

// The wave's index in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Accumulator layout of the 32 x 32 blocks, as the epilogues see it: BLK x
// BLK blocks, RPB registers per block and lane; GROUPS lanes (l, l ^ 32) hold
// the rows of one column; register r of lane l sits in block row row_in(r, l);
// block row rr lives in lane group group_of(rr), register reg_of(rr).
struct AccLayout32 {
  static constexpr int BLK = 32, RPB = 16, GROUPS = 2;
  static __device__ __forceinline__ int row_in(int r, int lane) { return acc_row(r, lane); }
  static __device__ __forceinline__ int group_of(int rr) { return (rr >> 2) & 1; }
  static __device__ __forceinline__ int reg_of(int rr) { return (rr >> 3) * 4 + (rr & 3); }
};

template <class C>
struct Tile {
  using TIn = typename C::TIn;
  using L = AccLayout32;
  static constexpr int MBK = C::MB, NBK = C::NB;
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
  const int wave = wave_id();
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

// ---------------------------------------------------------------------------
// Direct global->LDS load helpers of the bf16 main loop.
// ---------------------------------------------------------------------------
// global_load_lds_dword: 4 bytes per lane into LDS at `lds` + 4 * lane
// (`lds` wave-uniform).
__device__ __forceinline__ void lds_dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// Raw buffer resource (stride 0) over `bytes` bytes from `base`: loads at
// offsets past `bytes` return zeros.  Word 3 is the gfx9-family default for
// raw dword access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// An offset past any record the library builds (buffers stay below 2^31 bytes).
constexpr uint32_t kOutOfRange = 0x80000000u;
// buffer_load_dwordx4 ... lds: 16 bytes per lane at voffset + soffset into LDS
// at `lds` + 16 * lane.
__device__ __forceinline__ void lds_dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t voffset, uint32_t soffset, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset, 0, 0);
}

// vmcnt(n) for n < 64 (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Accumulators of one wave's MB x NB blocks of 32 x 32 outputs.
template <class C>
struct DmaTile {
  using L = AccLayout32;
  static constexpr int MBK = C::MB, NBK = C::NB;
  f32x16 acc[C::MB][C::NB];
};

// Workgroup barrier the compiler may not move work across.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// MFMA operand fragments of one k16 substep, read from LDS.
template <class C>
struct SubFrags {
  bf16x8 a[C::MB], b[C::NB];
};

// ---------------------------------------------------------------------------
// bf16 main loop on 64-wide k slices in two LDS stages.
//
// A stage row holds 64 k values = 128 bytes = eight 16-byte chunks, so one
// global_load_lds instruction of a wave moves 8 rows x 128 bytes, i.e. whole
// cache lines: half the texture-address and L1 requests per byte of a
// 32-wide layout, whose instructions touch sixteen half lines.  Chunk c of
// row r sits in slot c ^ ((r >> 1) & 7): with 64 four-byte banks the sixteen
// lanes of a ds_read_b128 quarter-wave (sixteen consecutive rows, one chunk)
// then fall in sixteen distinct 16-byte bank groups.
//
// The pipeline runs per k16 substep: the MFMAs of substep q use fragments
// read under the MFMAs of substep q - 1 (two fragment sets of one substep
// each).  At the last substep of stage kt every wave has finished reading it:
// after the wait for slice kt + 1 and a barrier, stage kt is refilled with
// slice kt + 2, its loads spread over that substep's MFMAs.  Operands go
// global->LDS with buffer_load ... lds (see K64Loader).
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_>
struct Dma64Cfg {
  using TIn = bf16_t;
  using TileT = DmaTile<Dma64Cfg>;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NSTAGE = 2;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NTHREADS = 64 * NWAVES;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int BK = 64;
  static constexpr int ROW_BYTES = 128;
  static constexpr int X_BYTES = BM * ROW_BYTES, Y_BYTES = BN * ROW_BYTES;
  static constexpr int STAGE_BYTES = X_BYTES + Y_BYTES;
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;
  // one wave-instruction fills 8 rows; loads per thread per stage
  static constexpr int X_LOADS = BM / 8 / NWAVES, Y_LOADS = BN / 8 / NWAVES;
  static constexpr int LOADS_PER_STAGE = X_LOADS + Y_LOADS;
  static_assert(BM % (8 * NWAVES) == 0 && BN % (8 * NWAVES) == 0, "row groups per wave");
  static_assert(NWAVES % 2 == 0, "the row groups of a wave share one swizzle phase");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Operand loader of the 64-wide loop: buffer_load ... lds through one buffer
// resource per operand, based at the tile's first row and bounded by its
// valid rows, so rows past xrows / yrows read as zero without a clamp;
// per-lane byte offsets stay fixed and the k slice advances in the scalar
// offset.  Lane -> (row within its 8-row group, slot); the rows of load i are
// (wave + i NWAVES) 8 + lrow, whose (r >> 1) & 7 is the same for every i since
// NWAVES is even.
//
// XT: X is stored k-major, element (m, k) at X[k ldx + m] (X
// points at the tile's first column).  A stage's X part then holds 64 k rows
// of BM columns; slot s = (i NWAVES + wave) 64 + lane of load i takes k row
// s / (BM / 8), 16-byte chunk (s % (BM / 8)) ^ 4 (k % 4), so that the
// transposing fragment reads below touch distinct banks.  Each slice gets a
// buffer resource of its own, based at its first k row and bounded by the
// rows below kdim (so operands larger than 4 GiB work).
template <class C, bool XT = false>
struct K64Loader {
  static_assert(!XT || C::BM % 128 == 0, "k-major X: at least 16 chunks per k row");
  const bf16_t* X;
  const bf16_t* Y;
  __amdgpu_buffer_rsrc_t rx, ry;
  int64_t ldx_;
  uint32_t xoff[XT ? C::X_LOADS : 1];
  // byte offsets of this lane's first X and Y loads; load i adds i steps (the
  // steps are workgroup-uniform)
  uint32_t off[2];
  uint32_t xstep, ystep;
  int wave, lchunk, kdim;
  __device__ __forceinline__ K64Loader(const bf16_t* X_, int64_t ldx, int xrows, const bf16_t* Y_, int64_t ldy,
                                       int yrows, int kdim_)
      : X(X_),
        Y(Y_),
        rx(make_rsrc(X_, (uint32_t)(min(xrows, C::BM) * ldx * 2))),
        ry(make_rsrc(Y_, (uint32_t)(min(yrows, C::BN) * ldy * 2))),
        ldx_(ldx),
        xstep((uint32_t)(C::NWAVES * 8 * ldx * 2)),
        ystep((uint32_t)(C::NWAVES * 8 * ldy * 2)),
        kdim(kdim_) {
    const int lane = threadIdx.x & 63;
    wave = wave_id();
    const int lrow = lane >> 3;
    lchunk = (lane & 7) ^ ((((wave & 1) << 2) | (lrow >> 1)) & 7);
    if constexpr (XT) {
      constexpr int XCH = C::BM / 8;
#pragma unroll
      for (int i = 0; i < C::X_LOADS; ++i) {
        const int sl = (i * C::NWAVES + wave) * 64 + lane, k = sl / XCH, pc = sl % XCH;
        xoff[i] = (uint32_t)(k * ldx * 2 + ((pc ^ (4 * (k & 3))) * 16));
      }
    }
    off[0] = (uint32_t)((wave * 8 + lrow) * ldx * 2 + lchunk * 16);
    off[1] = (uint32_t)((wave * 8 + lrow) * ldy * 2 + lchunk * 16);
  }
  __device__ __forceinline__ char* lds_at(char* smem, int kt, int i) const {
    char* st = smem + (kt & 1) * C::STAGE_BYTES;
    return i < C::X_LOADS ? st + (wave + i * C::NWAVES) * 1024
                          : st + C::X_BYTES + (wave + (i - C::X_LOADS) * C::NWAVES) * 1024;
  }
  // load i of slice kt; `whole`: the slice lies inside [0, kdim).  Chunks past
  // kdim load zeros: an offset past every record.
  __device__ __forceinline__ void dma(char* smem, int kt, int i, bool whole) const {
    if constexpr (XT) {
      if (i < C::X_LOADS) {
        const int rows = min(C::BK, kdim - kt * C::BK);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(X + (int64_t)kt * C::BK * ldx_, (uint32_t)(rows * ldx_ * 2));
        lds_dma_buf(r, xoff[i], 0u, lds_at(smem, kt, i));
        return;
      }
    }
    const bool in = whole || kt * C::BK + lchunk * 8 < kdim;
    // the offset is formed here rather than kept per load in registers
    const uint32_t o = i < C::X_LOADS ? off[0] + (uint32_t)i * xstep : off[1] + (uint32_t)(i - C::X_LOADS) * ystep;
    lds_dma_buf(i < C::X_LOADS ? rx : ry, in ? o : kOutOfRange, (uint32_t)(kt * C::BK * 2), lds_at(smem, kt, i));
  }
  // the first two slices (the loop's prologue)
  __device__ __forceinline__ void prologue(char* smem) const {
    const int nk = (kdim + C::BK - 1) / C::BK, n_full = kdim / C::BK;
    if (nk > 0) {
#pragma unroll
      for (int i = 0; i < C::LOADS_PER_STAGE; ++i) dma(smem, 0, i, n_full > 0);
    }
    if (nk > 1) {
#pragma unroll
      for (int i = 0; i < C::LOADS_PER_STAGE; ++i) dma(smem, 1, i, n_full > 1);
    }
  }
};

// Issue the first two slices of a tile whose loop runs later with PRE = true
// (the caller may do other work meanwhile, without touching the LDS stages).
template <class C>
__device__ __forceinline__ void tile_k64_prologue(const bf16_t* __restrict__ X, int64_t ldx, int xrows,
                                                  const bf16_t* __restrict__ Y, int64_t ldy, int yrows, int kdim,
                                                  char* smem) {
  K64Loader<C>(X, ldx, xrows, Y, ldy, yrows, kdim).prologue(smem);
}

// Computes the BM x BN tile over k in [0, kdim) (kdim a multiple of 8).  k
// past kdim reads as zero; rows past xrows / yrows give outputs that callers
// must discard (select, never multiply).  Byte offsets BM * ldx * 2 and
// BN * ldy * 2 must stay below 2^31.  Ends with a barrier after which the LDS
// may be reused.  PRE: the prologue was issued by
// tile_k64_prologue with the same arguments; the loop starts by waiting for
// every outstanding vector memory operation (stores count on this GPU).
//
// XT: X stored k-major (see K64Loader); its fragments are read with
// ds_read_b64_tr_b16, which hands each lane of a 16-lane group one column of
// the 4 x 16 block whose rows the group's lanes address (lane 4 r + c gives
// row r, columns 4 c .. 4 c + 3): two such reads (k rows 0-3, 4-7 of the
// lane's half) make the lane's eight k values of its m row.
template <class C, bool PRE = false, bool XT = false>
__device__ __forceinline__ void tile_mma_k64(DmaTile<C>& tile, const bf16_t* __restrict__ X, int64_t ldx, int xrows,
                                             const bf16_t* __restrict__ Y, int64_t ldy, int yrows, int kdim,
                                             char* smem) {
  static_assert(C::BK == 64 && C::NSTAGE == 2, "two 64-wide stages");
  static_assert(!XT || !PRE, "k-major X: the prologue is issued here");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int wave_m = wave / C::WAVES_N;
  const int wave_n = wave % C::WAVES_N;

#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tile.acc[mb][nb][r] = 0.f;

  const K64Loader<C, XT> ld(X, ldx, xrows, Y, ldy, yrows, kdim);
  auto dma = [&](int kt, int i, bool whole) { ld.dma(smem, kt, i, whole); };

  // Reader: lane reads row (lane & 31) + 32 block of its wave's rows, chunk
  // 2 sub + (lane >> 5) for k16 substep sub of the stage.
  const int rrow = lane & 31;
  const int rsw = (rrow >> 1) & 7;
  int roff[4];
#pragma unroll
  for (int sub = 0; sub < 4; ++sub) roff[sub] = rrow * C::ROW_BYTES + (((2 * sub + (lane >> 5)) ^ rsw) * 16);
  const int xwave = wave_m * C::WM * C::ROW_BYTES;
  const int ywave = C::X_BYTES + wave_n * C::WN * C::ROW_BYTES;
  constexpr int kDma = C::LOADS_PER_STAGE;

  const int nk = (kdim + C::BK - 1) / C::BK;
  const int n_full = kdim / C::BK;
  {
    // the fragments of k16 substep q + 1 are read under the MFMAs of substep
    // q; at the last substep of stage kt every wave has finished reading it:
    // after the wait for slice kt + 1 and the barrier, stage kt is refilled
    // with slice kt + 2
    using SF = SubFrags<C>;
    // XT: this lane's byte offsets of its first transposing read per m block
    // (group g = lane / 16 reads k rows 8 (g / 2) + 4 h + r, columns
    // 16 (g % 2) + 4 c .. of its 32-block, chunk-swizzled as stored)
    constexpr int XROW = C::BM * 2;
    int xr[XT ? C::MB : 1];
    if constexpr (XT) {
      const int g = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) {
        const int mc = wave_m * (C::WM / 8) + mb * 4 + (g & 1) * 2 + (c >> 1);
        xr[mb] = ((g >> 1) * 8 + r) * XROW + ((mc ^ (4 * r)) * 16) + (c & 1) * 8;
      }
    }
    auto sread = [&](int kt, int sub, SF& f, int w) {
      const char* st = smem + (kt & 1) * C::STAGE_BYTES;
      if (w < C::MB) {
        if constexpr (XT) {
          typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
          const char* p = st + sub * 16 * XROW + xr[w];
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(__attribute__((address_space(3))) char*)(p));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(__attribute__((address_space(3))) char*)(p + 4 * XROW));
          f.a[w] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
          f.a[w] = *reinterpret_cast<const bf16x8*>(st + xwave + w * 32 * C::ROW_BYTES + roff[sub]);
        }
      } else
        f.b[w - C::MB] =
            *reinterpret_cast<const bf16x8*>(st + ywave + (w - C::MB) * 32 * C::ROW_BYTES + roff[sub]);
    };
    constexpr int kM = C::MB * C::NB, kR = C::MB + C::NB;
    // one substep: MFMAs with `cur`; reads of (rkt, rsub) into `nxt`, and at
    // the last substep the refill of slice kt + 2 first
    auto substep = [&](int kt, const SF& cur, SF& nxt, int rkt, int rsub, bool rd, bool last, bool refill,
                       bool whole) {
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkm0();
      if (last && rd) {
        wait_vmcnt<0>();
        phase_barrier();
      }
      constexpr int kOps = kR + kDma;
#pragma unroll
      for (int j = 0; j < kM; ++j) {
        tile.acc[j / C::NB][j % C::NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            cur.a[j / C::NB], cur.b[j % C::NB], tile.acc[j / C::NB][j % C::NB], 0, 0, 0);
        if (last) {
#pragma unroll
          for (int q = j * kOps / kM; q < (j + 1) * kOps / kM; ++q) {
            if (q < kDma) {
              if (refill) dma(kt + 2, q, whole);
            } else if (rd) {
              sread(rkt, rsub, nxt, q - kDma);
            }
          }
        } else {
#pragma unroll
          for (int q = j * kR / kM; q < (j + 1) * kR / kM; ++q) sread(rkt, rsub, nxt, q);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (nk > 0) {
      if constexpr (PRE) {
        wait_vmcnt<0>();
      } else {
#pragma unroll
        for (int i = 0; i < kDma; ++i) dma(0, i, n_full > 0);
        if (nk > 1) {
#pragma unroll
          for (int i = 0; i < kDma; ++i) dma(1, i, n_full > 1);
          wait_vmcnt<kDma>();
        } else {
          wait_vmcnt<0>();
        }
      }
      phase_barrier();
      SF fa, fb;
#pragma unroll
      for (int w = 0; w < kR; ++w) sread(0, 0, fa, w);
      int kt = 0;
      for (; kt + 2 < n_full; ++kt) {  // steady state: the refilled slice is whole
        substep(kt, fa, fb, kt, 1, true, false, false, true);
        substep(kt, fb, fa, kt, 2, true, false, false, true);
        substep(kt, fa, fb, kt, 3, true, false, false, true);
        substep(kt, fb, fa, kt + 1, 0, true, true, true, true);
      }
      for (; kt < nk; ++kt) {
        const bool next = kt + 1 < nk;
        substep(kt, fa, fb, kt, 1, true, false, false, true);
        substep(kt, fb, fa, kt, 2, true, false, false, true);
        substep(kt, fa, fb, kt, 3, true, false, false, true);
        substep(kt, fb, fa, kt + 1, 0, next, true, kt + 2 < nk, kt + 2 < n_full);
      }
    }
  }
  __syncthreads();
}

// ------------------------------------------------------ tile scheduling --
// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2.  xcd_remap(w, total) is a bijection of [0, total) that
// hands XCD x (= w % 8) a contiguous range of logical tile ids, so the ~32
// workgroups an XCD runs at once take neighbouring tiles and share operand
// panels in that XCD's L2.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int xcd = w % kNumXcd, j = w / kNumXcd;
  const int base = total / kNumXcd, rem = total % kNumXcd;
  return xcd < rem ? xcd * (base + 1) + j : rem * (base + 1) + (xcd - rem) * base + j;
}

// Grouped order of a tiles_m x tiles_n grid: logical ids walk gm tiles down m,
// then step along n, group after group, so any run of gm * k consecutive ids
// touches gm m-panels and k n-panels.
__device__ __forceinline__ void grouped_mn(int L, int tiles_m, int tiles_n, int gm, int& m, int& n) {
  const int per_group = gm * tiles_n;
  const int g = L / per_group;
  const int first = g * gm;
  const int rows = min(gm, tiles_m - first);
  const int r = L - g * per_group;
  m = first + r % rows;
  n = r / rows;
}

// Configurations whose loop can take a prologue issued ahead (tile_k64_prologue).
template <class C>
struct PrefetchOK : std::false_type {};
template <int BM, int BN, int WM, int WN>
struct PrefetchOK<Dma64Cfg<BM, BN, WM, WN>> : std::true_type {};

// One entry point for both main loops.
template <class C>
__device__ __forceinline__ void run_mma(Tile<C>& t, const typename C::TIn* X, int64_t ldx, int xrows,
                                        const typename C::TIn* Y, int64_t ldy, int yrows, int kdim, char* smem) {
  tile_mma<C>(t, X, ldx, xrows, Y, ldy, yrows, kdim, reinterpret_cast<typename C::TIn*>(smem));
}
template <class C, bool PRE = false, bool XT = false>
__device__ __forceinline__ void run_mma(DmaTile<C>& t, const bf16_t* X, int64_t ldx, int xrows, const bf16_t* Y,
                                        int64_t ldy, int yrows, int kdim, char* smem) {
  tile_mma_k64<C, PRE, XT>(t, X, ldx, xrows, Y, ldy, yrows, kdim, smem);
}

}  // namespace ckl
