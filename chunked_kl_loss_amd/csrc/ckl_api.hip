// Host side of libckl: argument checks, workspace planning and the launch
// sequence behind the C ABI declared in include/ckl.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ckl.h"
#include "ckl_kernels.hpp"

namespace {

thread_local std::string g_last_error;

ckl_status fail(ckl_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ckl_status fail(ckl_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

ckl_status hip_fail(hipError_t e, const char* what) {
  return fail(CKL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                         \
  do {                                              \
    hipError_t e__ = (expr);                        \
    if (e__ != hipSuccess) return hip_fail(e__, what); \
  } while (0)

constexpr int64_t kMaxK = 4096;
// Rows of H and W: the contraction loads address a 256-row tile of H^T, W^T,
// G or G^T with 32-bit byte offsets (256 * (rows + padding) * 2 < 2^31).
constexpr int64_t kMaxRows = 4000000;
// Compute units of an MI355X; the logit and contraction kernels fit one
// workgroup per CU (128 KiB of LDS each), so kCUs workgroups make one wave.
constexpr int64_t kCUs = 256;
// dH split-k parts of the fused call: at most this many, and the fp32 store
// of one part's tile costs about as long as this many k columns of its
// main loop (a 256 x 256 fp32 tile at one CU's share of HBM bandwidth).
constexpr int64_t kMaxSplit = 64;
constexpr int64_t kEpilogueK = 512;
// Fused call: G (bf16; G^T for fp32) of consecutive row chunks is kept for
// a group of chunks, so the dW update (an fp32 read-modify-write of all of
// dW) runs once per group with k = group rows instead of once per chunk.
// Default group: at most kDwRows rows and at most kDwChunks chunks, so that a
// smaller chunk also holds less (ckl_problem.dw_group_rows overrides it).
constexpr int64_t kDwRows = 16384;
constexpr int64_t kDwChunks = 8;
// Row padding (elements) of G^T in the fused call (fp32; bf16 keeps no G^T).
// Its rows are written in short runs for consecutive rows; some strides put
// those runs on few memory channels (with eight 2048-row chunks of bf16, a
// stride of 32 KiB + 256 bytes made the G formation ~1.2x slower than
// 32 KiB + 640 bytes).
constexpr int64_t kGtPad = 320;
// The backward keeps one G block (fp32: and its transpose) within chunk * V
// elements.  (Double-buffering it to overlap the recompute of block i+1 with
// the contraction of block i on a second stream measured no faster: both
// kernels are throughput-bound, so concurrency only splits the CUs.)
constexpr int kGBuffers = 1;
// Row padding (elements) of every matrix whose leading dimension the library
// picks (H^T, W^T, G, G^T): 256 bytes keeps the stride away from large powers
// of two, so the 16 rows one global->LDS load touches spread over memory
// channels instead of all hitting one.
constexpr int64_t kLdPad = 128;

// ------------------------------------------------------------------ timing --
struct TimingState {
  std::mutex mu;
  bool on = false;
  struct Rec { int cls; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  double total_ms[CKL_KERNEL_CLASSES] = {};
  int64_t launches[CKL_KERNEL_CLASSES] = {};
};
TimingState g_timing;

// Launch `fn` (returning hipError_t), bracketed by timing events when enabled.
// Set while ckl_forward_noalloc runs: its launches record no timing events
// (creating events would allocate).
thread_local bool g_no_events = false;

template <class Fn>
hipError_t timed(int cls, hipStream_t st, Fn&& fn) {
  if (!g_timing.on || g_no_events) return fn();
  std::pair<hipEvent_t, hipEvent_t> ev{};
  {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!g_timing.pool.empty()) { ev = g_timing.pool.back(); g_timing.pool.pop_back(); }
  }
  hipError_t e;
  if (!ev.first) {
    if ((e = hipEventCreate(&ev.first)) != hipSuccess) return e;
    if ((e = hipEventCreate(&ev.second)) != hipSuccess) return e;
  }
  if ((e = hipEventRecord(ev.first, st)) != hipSuccess) return e;
  if ((e = fn()) != hipSuccess) return e;
  if ((e = hipEventRecord(ev.second, st)) != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.pending.push_back({cls, ev.first, ev.second});
  return hipSuccess;
}

hipError_t timing_drain() {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto& r : g_timing.pending) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return e;
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return e;
    g_timing.total_ms[r.cls] += ms;
    g_timing.launches[r.cls] += 1;
    g_timing.pool.push_back({r.a, r.b});
  }
  g_timing.pending.clear();
  return hipSuccess;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  int64_t T, d, V, K;
  int in_bf16;
  int64_t esz;
  int64_t BM, BN;  // logit tile: vocabulary rows x token rows
  int64_t Tp, Vp;
  // backward G blocks
  int64_t Tc, Vc, nT, nV;
  // row chunks of Cs rows, nS of them (both forwards; the fused backward),
  // vocabulary splits per chunk; dH split-k into Sh parts of Vs vocabulary
  // columns (fused)
  int64_t Cs, nS, Gc, c_splits, c_tps, Sh, Vs, groups;
};

// Vocabulary splits of the logit kernels: each workgroup sweeps a run of
// tiles_per_split vocabulary tiles for one block of rows (the teacher cursors
// advance monotonically along a split).  Picks the split count with the
// shortest makespan in tile-times, ceil(workgroups / kCUs) x tiles_per_split,
// and among equals the fewest splits.
void pick_splits(int64_t row_blocks, int64_t vtiles, int64_t* splits, int64_t* tps) {
  int64_t best = -1;
  for (int64_t s = 1; s <= vtiles; ++s) {
    const int64_t t = ceil_div(vtiles, s);
    const int64_t sp = ceil_div(vtiles, t);
    if (sp != s) continue;  // the same split as a smaller count
    const int64_t cost = ceil_div(row_blocks * sp, kCUs) * t;
    if (best < 0 || cost < best) {
      best = cost;
      *splits = sp;
      *tps = t;
    }
  }
}

// Full vocabulary size (v_total = 0: W holds all of it).
int64_t vtotal(const ckl_problem* p) { return p->v_total ? p->v_total : p->V; }
bool sharded(const ckl_problem* p) { return p->v_offset != 0 || vtotal(p) != p->V; }

ckl_status check_problem(const ckl_problem* p) {
  if (!p) return fail(CKL_ERR_INVALID_ARG, "problem is NULL");
  if (p->T < 1) return fail(CKL_ERR_INVALID_ARG, "T=%lld must be >= 1", (long long)p->T);
  if (p->V < 1) return fail(CKL_ERR_INVALID_ARG, "V=%lld must be >= 1", (long long)p->V);
  if (p->T > kMaxRows || p->V > kMaxRows)
    return fail(CKL_ERR_UNSUPPORTED, "T=%lld, V=%lld: at most %lld rows each", (long long)p->T, (long long)p->V,
                (long long)kMaxRows);
  if (p->d < 8 || p->d % 8 != 0) return fail(CKL_ERR_INVALID_ARG, "d=%lld must be a positive multiple of 8", (long long)p->d);
  if (p->d > 65536) return fail(CKL_ERR_UNSUPPORTED, "d=%lld exceeds 65536", (long long)p->d);
  if (p->v_offset < 0 || p->v_total < 0) return fail(CKL_ERR_INVALID_ARG, "v_offset and v_total must be >= 0");
  if (vtotal(p) < p->v_offset + p->V)
    return fail(CKL_ERR_INVALID_ARG, "v_offset + V = %lld exceeds v_total = %lld", (long long)(p->v_offset + p->V),
                (long long)vtotal(p));
  if (vtotal(p) >= ((int64_t)1 << 31)) return fail(CKL_ERR_UNSUPPORTED, "v_total must stay below 2^31 (int32 idx)");
  if (p->K < 1 || p->K > vtotal(p))
    return fail(CKL_ERR_INVALID_ARG, "K=%lld must satisfy 1 <= K <= v_total", (long long)p->K);
  if (p->K > kMaxK) return fail(CKL_ERR_UNSUPPORTED, "K=%lld exceeds %lld", (long long)p->K, (long long)kMaxK);
  if (p->T * p->K >= ((int64_t)1 << 31)) return fail(CKL_ERR_UNSUPPORTED, "T*K must stay below 2^31");
  if (p->chunk < 1) return fail(CKL_ERR_INVALID_ARG, "chunk=%lld must be >= 1", (long long)p->chunk);
  auto dt_ok = [](int32_t t) { return t == CKL_F32 || t == CKL_BF16; };
  if (!dt_ok(p->in_dtype) || !dt_ok(p->dh_dtype) || !dt_ok(p->dw_dtype))
    return fail(CKL_ERR_INVALID_ARG, "dtype codes must be CKL_F32 (0) or CKL_BF16 (1)");
  if (p->validate != 0 && p->validate != 1) return fail(CKL_ERR_INVALID_ARG, "validate must be 0 or 1");
  if (p->teacher_form != CKL_TEACHER_LOGITS && p->teacher_form != CKL_TEACHER_LOGPROBS)
    return fail(CKL_ERR_INVALID_ARG, "teacher_form must be CKL_TEACHER_LOGITS (0) or CKL_TEACHER_LOGPROBS (1)");
  if (p->dw_group_rows < 0) return fail(CKL_ERR_INVALID_ARG, "dw_group_rows must be >= 0");
  if (p->compact_mask != 0 && p->compact_mask != 1) return fail(CKL_ERR_INVALID_ARG, "compact_mask must be 0 or 1");
  if (p->reserved_ != 0) return fail(CKL_ERR_INVALID_ARG, "reserved_ must be 0");
  return CKL_OK;
}

Plan make_plan(const ckl_problem* p) {
  Plan q{};
  q.T = p->T; q.d = p->d; q.V = p->V; q.K = p->K;
  q.in_bf16 = p->in_dtype == CKL_BF16;
  q.esz = q.in_bf16 ? 2 : 4;
  q.BM = ckl::tile_rows_m(q.in_bf16);
  q.BN = ckl::tile_rows_n(q.in_bf16);
  q.Tp = round_up(q.T, q.BN);
  q.Vp = round_up(q.V, q.BM);

  // G blocks of Tc token rows x Vc vocabulary columns, within chunk * V
  // elements for G and G^T together (bf16 keeps G alone and still takes half
  // the budget: a G block of the whole budget measured slower at 32K rows,
  // faster at 131K).  Among the admissible shapes pick
  // the one with the least fp32 read-modify-write of dH (once per extra
  // vocabulary block) and dW (once per extra token block).
  const int64_t per_layout = std::max<int64_t>(p->chunk * p->V / (2 * kGBuffers), q.BM * q.BN);
  double best = -1.0;
  for (int64_t nT = 1; nT <= q.Tp / q.BN; ++nT) {
    const int64_t Tc = round_up(ceil_div(q.Tp, nT), q.BN);
    if (nT > 1 && Tc == round_up(ceil_div(q.Tp, nT - 1), q.BN)) continue;
    const int64_t nTr = ceil_div(q.Tp, Tc);
    int64_t vmax = (per_layout / Tc) / q.BM * q.BM;
    if (vmax < q.BM) vmax = q.BM;
    if (Tc * vmax > per_layout && Tc > q.BN) continue;  // only the smallest block may exceed the budget
    const int64_t nV = ceil_div(q.Vp, vmax);
    const int64_t Vc = round_up(ceil_div(q.Vp, nV), q.BM);
    const double cost = (double)(nTr - 1) * q.V * q.d * 8.0 + (double)(nV - 1) * q.T * q.d * 8.0 +
                        (double)(nTr * nV) * 3.0 * 4.0e6;  // ~launch overhead in byte-equivalents
    if (best < 0 || cost < best) {
      best = cost;
      q.Tc = Tc; q.Vc = Vc; q.nT = nTr; q.nV = ceil_div(q.Vp, Vc);
    }
  }

  // Fused call: chunks of `chunk` rows in whole 256-row blocks (the loss
  // block sums are per 256 rows), at most the padded row count.
  q.Cs = std::min(round_up(p->chunk, 256), round_up(q.Tp, 256));
  q.nS = ceil_div(q.Tp, q.Cs);
  {
    const int64_t group_rows = p->dw_group_rows > 0 ? p->dw_group_rows : std::min(kDwRows, kDwChunks * q.Cs);
    q.Gc = std::max<int64_t>(1, std::min(group_rows / q.Cs, q.nS));  // chunks per dW group
  }
  pick_splits(q.Cs / q.BN, q.Vp / q.BM, &q.c_splits, &q.c_tps);
  // dH split-k parts: the count whose tiles finish in the fewest k-steps when
  // dealt to kCUs workgroups in rounds (whole rounds: a launch that holds only
  // dH tiles ends with its slowest round), each part also paying its epilogue.
  const int64_t dh_tiles = ceil_div(q.Cs, (int64_t)ckl::gemm_tile_m(q.in_bf16)) *
                           ceil_div(q.d, (int64_t)ckl::gemm_tile_n(q.in_bf16));
  const int64_t sh_max = std::max<int64_t>(1, std::min<int64_t>(kMaxSplit, q.Vp / 256));
  int64_t best_cost = -1;
  for (int64_t sh = 1; sh <= sh_max; ++sh) {
    // (at most Vp: fp32 pads the vocabulary to 128 columns, and a part may
    // not reach into the row padding of G and W^T past it)
    const int64_t vs = std::min(round_up(ceil_div(q.Vp, sh), 256), q.Vp);
    const int64_t parts = ceil_div(q.Vp, vs);
    if (parts != sh) continue;  // the same split as a smaller count
    const int64_t cost = ceil_div(dh_tiles * parts, kCUs) * (vs + kEpilogueK);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      q.Vs = vs;
      q.Sh = parts;
    }
  }
  q.groups = (q.Vp / q.BM) * ckl::lse_groups_per_tile(q.in_bf16);
  return q;
}

// Packed rows (compact_mask with a mask): the kept rows' positions, each
// row's rank, their number, a packed copy of their H rows and packed per-row
// results, laid out after a call's own workspace.
struct PackWs {
  size_t perm, rank, N, Hc, lse, rl, total;
};
PackWs pack_layout(const Plan& q, size_t o) {
  PackWs w{};
  auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes); return at; };
  w.perm = take(q.T * 4);
  w.rank = take(q.T * 4);
  w.N = take(4);
  w.Hc = take((size_t)q.T * q.d * q.esz);
  w.lse = take(q.T * 4);
  w.rl = take(q.T * 4);
  w.total = o;
  return w;
}

struct FwdWs {
  size_t idx_s, p_s, zg_s, E, M, part, blk, N, bad, total;
  PackWs pk;
};
FwdWs fwd_layout(const Plan& q, const ckl_problem* p) {
  FwdWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes); return at; };
  w.idx_s = take(q.T * q.K * 4);
  w.p_s = take(q.T * q.K * 4);
  w.zg_s = take(q.T * q.K * 4);
  w.E = take(q.T * 4);
  w.M = take(q.T * 4);
  w.part = take(q.c_splits * q.Cs * 8);  // split LSE states of one chunk
  w.blk = take(q.T * 8);  // per-row fp64 loss terms
  w.N = take(4);
  w.bad = take(4);
  w.total = o;
  if (p->compact_mask) {
    w.pk = pack_layout(q, o);
    w.total = w.pk.total;
  }
  return w;
}

struct BwdWs {
  size_t idx_s, p_s, M, s, N, bad, Ht, Wt, G[kGBuffers], Gt[kGBuffers], dH, dW, total;
  PackWs pk;
};
BwdWs bwd_layout(const Plan& q, const ckl_problem* p) {
  BwdWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes); return at; };
  w.idx_s = take(q.T * q.K * 4);
  w.p_s = take(q.T * q.K * 4);
  w.M = take(q.T * 4);
  w.s = take(q.Tp * 4);
  w.N = take(4);
  w.bad = take(4);
  w.Ht = take((size_t)q.d * (q.Tp + kLdPad) * q.esz);
  // W^T of one vocabulary block at a time (the blocks are the outer loop)
  w.Wt = take((size_t)q.d * (q.Vc + kLdPad) * q.esz);
  // bf16 keeps G only (the dW contraction reads it k-major); fp32 also G^T
  for (int i = 0; i < kGBuffers; ++i) {
    w.G[i] = take((size_t)q.Tc * (q.Vc + kLdPad) * q.esz);
    w.Gt[i] = q.in_bf16 ? 0 : take((size_t)q.Vc * (q.Tc + kLdPad) * q.esz);
  }
  // fp32 accumulator of dH when dH is bf16, or when packed rows are
  // scattered back at the end
  w.dH = (p->dh_dtype == CKL_BF16 || p->compact_mask) ? take((size_t)q.T * q.d * 4) : 0;
  w.dW = p->dw_dtype == CKL_BF16 ? take((size_t)q.V * q.d * 4) : 0;
  w.total = o;
  if (p->compact_mask) {
    w.pk = pack_layout(q, o);
    w.total = w.pk.total;
  }
  return w;
}

struct FusedWs {
  size_t idx_s, p_s, zg_s, E, M, part, blk, N, bad, s, Ht, Wt, U, G, Gt, mtab, dHp, dW, total;
  PackWs pk;
};
FusedWs fused_layout(const Plan& q, const ckl_problem* p) {
  FusedWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes); return at; };
  w.idx_s = take(q.T * q.K * 4);
  w.p_s = take(q.T * q.K * 4);
  w.zg_s = take(q.T * q.K * 4);
  w.E = take(q.T * 4);
  w.M = take(q.T * 4);
  w.part = take(q.c_splits * q.Cs * 8);
  w.blk = take(q.T * 8);  // per-row fp64 loss terms
  w.N = take(4);
  w.bad = take(4);
  w.s = take(q.Tp * 4);
  // H^T of one dW group's rows at a time (its update reads no other rows)
  w.Ht = take((size_t)q.d * (q.Gc * q.Cs + kLdPad) * q.esz);
  w.Wt = take((size_t)q.d * (q.Vp + kLdPad) * q.esz);
  // bf16: u of a chunk in the forward's tile order, laid out as G by
  // gpass_tiles (fp32 keeps u in G itself)
  w.U = q.in_bf16 ? take((size_t)q.Cs * q.Vp * q.esz) : 0;
  // bf16: G of the group's chunks, read k-major by the dW update (no G^T);
  // fp32: G of one chunk and G^T of the group's chunks
  w.G = take((size_t)(q.in_bf16 ? q.Gc : 1) * q.Cs * (q.Vp + kLdPad) * q.esz);
  w.Gt = q.in_bf16 ? 0 : take((size_t)q.Vp * (q.Gc * q.Cs + kGtPad) * q.esz);
  w.mtab = take((size_t)q.groups * q.Cs * 4);
  w.dHp = take((size_t)q.Sh * q.Cs * q.d * 4);
  w.dW = p->dw_dtype == CKL_BF16 ? take((size_t)q.V * q.d * 4) : 0;
  w.total = o;
  if (p->compact_mask) {
    w.pk = pack_layout(q, o);
    w.total = w.pk.total;
  }
  return w;
}

struct CombineWs {
  size_t idx_s, p_s, E, M, blk, N, bad, total;
};
CombineWs combine_layout(const Plan& q) {
  CombineWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += align256(bytes); return at; };
  w.idx_s = take(q.T * q.K * 4);
  w.p_s = take(q.T * q.K * 4);
  w.E = take(q.T * 4);
  w.M = take(q.T * 4);
  w.blk = take(q.T * 8);  // per-row fp64 loss terms
  w.N = take(4);
  w.bad = take(4);
  w.total = o;
  return w;
}

// Device pointers of the packed-row area of a workspace (all NULL when the
// call does not pack).
struct Packed {
  int* perm = nullptr;
  int* rank = nullptr;
  int* N = nullptr;
  void* Hc = nullptr;
  float* lse = nullptr;
  float* rl = nullptr;
  bool on() const { return perm != nullptr; }
};
Packed packed_at(char* b, const PackWs& w) {
  Packed k;
  k.perm = (int*)(b + w.perm);
  k.rank = (int*)(b + w.rank);
  k.N = (int*)(b + w.N);
  k.Hc = b + w.Hc;
  k.lse = (float*)(b + w.lse);
  k.rl = (float*)(b + w.rl);
  return k;
}

// The kept rows of `mask`, packed: their positions and ranks, their number
// (the N of the mean) and the packed copy of their H rows (zero rows after
// them, up to T).
hipError_t pack_rows(const Plan& q, const Packed& k, const uint8_t* mask, const void* H, hipStream_t st) {
  hipError_t e = timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_compact_rows(mask, (int)q.T, k.perm, k.rank, k.N, st); });
  if (e != hipSuccess) return e;
  return timed(CKL_KERNEL_OTHER, st,
               [&] { return ckl::launch_gather_rows(H, (int)q.T, q.d * q.esz, k.perm, k.N, k.Hc, st); });
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// A buffer of an entry point: where it starts, its bytes, its name.
struct Span {
  const void* p;
  size_t n;
  const char* name;
};
bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || !a.n || !b.n) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}
// Every buffer the call writes (outputs, the used part of the workspace) must
// be disjoint from every other buffer of the call: an output that aliases an
// input or the workspace would be read after the library overwrote it.
ckl_status check_disjoint(std::initializer_list<Span> written, std::initializer_list<Span> read) {
  for (auto w = written.begin(); w != written.end(); ++w) {
    for (auto o = w + 1; o != written.end(); ++o)
      if (overlap(*w, *o)) return fail(CKL_ERR_INVALID_ARG, "%s and %s overlap", w->name, o->name);
    for (const Span& r : read)
      if (overlap(*w, r)) return fail(CKL_ERR_INVALID_ARG, "%s overlaps %s", w->name, r.name);
  }
  return CKL_OK;
}

// ------------------------------------------------ allocation-free forward --
// ckl_forward_noalloc takes its workspace from this file-scope device array
// instead of a caller's buffer.  Every device the library runs on holds its
// own copy until the process ends; host code must never pass the array's
// name to a kernel (in host code it is only a stand-in): it uses the device
// address looked up once per device, with that device current, on the entry
// point's first call there.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

ckl_status scratch_on_current_device(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CKL_ERR_UNSUPPORTED, "device ordinal %d above %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "looking up the device scratch array");
    if (ptr == nullptr) return fail(CKL_ERR_HIP, "the device scratch array has no address");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return CKL_OK;
}

ckl_status check_validate_flag(int* bad_dev, hipStream_t st) {
  int h = 0;
  HIP_TRY(hipMemcpyAsync(&h, bad_dev, sizeof(int), hipMemcpyDeviceToHost, st), "reading index check flag");
  HIP_TRY(hipStreamSynchronize(st), "synchronising for the index check");
  if (h) return fail(CKL_ERR_BAD_INDEX, "teacher indices out of [0, V) or repeated within a row");
  return CKL_OK;
}

}  // namespace

extern "C" {

ckl_status ckl_workspace_size(const ckl_problem* p, int which, size_t* bytes) {
  ckl_status s = check_problem(p);
  if (s != CKL_OK) return s;
  if (!bytes) return fail(CKL_ERR_INVALID_ARG, "bytes is NULL");
  if (which < 0 || which > 3)
    return fail(CKL_ERR_INVALID_ARG,
                "which must be 0 (forward, shard forward), 1 (backward), 2 (forward + backward) or 3 (shard combine)");
  const Plan q = make_plan(p);
  *bytes = which == 0   ? fwd_layout(q, p).total
           : which == 1 ? bwd_layout(q, p).total
           : which == 2 ? fused_layout(q, p).total
                        : combine_layout(q).total;
  return CKL_OK;
}

ckl_status ckl_forward(const ckl_problem* p, const void* H, const void* W, const int32_t* idx, const float* tlogit,
                       const uint8_t* mask, float* loss, float* lse, float* row_loss, void* ws, size_t ws_bytes,
                       void* stream) {
  ckl_status s = check_problem(p);
  if (s != CKL_OK) return s;
  if (sharded(p))
    return fail(CKL_ERR_UNSUPPORTED, "W is a vocabulary shard: use ckl_shard_forward and ckl_shard_combine");
  if (!H || !W || !idx || !tlogit || !loss || !lse) return fail(CKL_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(H) || !aligned16(W) || !aligned16(idx) || !aligned16(tlogit) || !aligned16(ws))
    return fail(CKL_ERR_INVALID_ARG, "H, W, idx, tlogit and ws must be 16-byte aligned");
  if (((uintptr_t)loss & 3u) || ((uintptr_t)lse & 3u) || ((uintptr_t)row_loss & 3u))
    return fail(CKL_ERR_INVALID_ARG, "loss, lse and row_loss must be 4-byte aligned");
  const Plan q = make_plan(p);
  const FwdWs w = fwd_layout(q, p);
  if (!ws || ws_bytes < w.total)
    return fail(CKL_ERR_WORKSPACE, "forward workspace needs %zu bytes, got %zu", w.total, ws ? ws_bytes : (size_t)0);
  {
    const size_t T = q.T, K = q.K;
    s = check_disjoint({{loss, 4, "loss"}, {lse, T * 4, "lse"}, {row_loss, T * 4, "row_loss"}, {ws, w.total, "ws"}},
                       {{H, T * q.d * q.esz, "H"}, {W, (size_t)q.V * q.d * q.esz, "W"}, {idx, T * K * 4, "idx"},
                        {tlogit, T * K * 4, "tlogit"}, {mask, T, "mask"}});
    if (s != CKL_OK) return s;
  }
  hipStream_t st = (hipStream_t)stream;
  char* b = (char*)ws;
  int* idx_s = (int*)(b + w.idx_s);
  float* p_s = (float*)(b + w.p_s);
  float* zg_s = (float*)(b + w.zg_s);
  float* E = (float*)(b + w.E);
  float* M = (float*)(b + w.M);
  int* N = (int*)(b + w.N);
  int* bad = (int*)(b + w.bad);
  const int T = (int)q.T, d = (int)q.d, V = (int)q.V, K = (int)q.K;
  // packed rows: the kept rows first, everything below runs over them only
  const Packed pk = (p->compact_mask && mask) ? packed_at(b, w.pk) : Packed{};
  const void* Hs = H;
  const uint8_t* mk = mask;
  float* lse_o = lse;
  float* rl_o = row_loss;
  if (pk.on()) {
    HIP_TRY(pack_rows(q, pk, mask, H, st), "packing kept rows");
    N = pk.N;
    Hs = pk.Hc;
    mk = nullptr;
    lse_o = pk.lse;
    rl_o = row_loss ? pk.rl : nullptr;
  } else {
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_count_mask(mask, T, N, st); }), "count_mask");
  }
  if (p->validate) HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_fill_i32(bad, 1, 0, st); }), "fill");
  HIP_TRY(timed(CKL_KERNEL_TEACHER_PREP, st,
                [&] {
                  return ckl::launch_teacher_prep(idx, tlogit, T, K, (int)vtotal(p), (int)p->v_offset, idx_s, p_s, E, M, zg_s,
                                                  p->validate ? bad : nullptr, p->teacher_form, pk.perm, pk.N, st);
                }),
          "teacher_prep");
  if (p->validate) {
    s = check_validate_flag(bad, st);
    if (s != CKL_OK) return s;
  }
  // chunk by chunk ([README] Full Chunked KL): a chunk's logit tiles give its
  // rows' split LSE states and teacher logits, then its rows' LSE and loss
  // terms; the vocabulary sweep of one chunk shares each W tile between the
  // chunk's row blocks while it is in the L2
  double* blk = (double*)(b + w.blk);
  for (int64_t c = 0; c < q.nS; ++c) {
    const int64_t tb0 = c * q.Cs;
    const int rows = (int)std::min(q.Cs, q.T - tb0);
    if (rows <= 0) break;
    const char* Hc = (const char*)Hs + tb0 * q.d * q.esz;
    HIP_TRY(timed(CKL_KERNEL_FWD_LSE, st,
                  [&] {
                    return ckl::launch_fwd_lse(q.in_bf16, Hc, W, rows, d, V, K, idx_s + tb0 * K, zg_s + tb0 * K,
                                               b + w.part, (int)q.c_splits, (int)q.c_tps, nullptr, 0, nullptr, 0,
                                               pk.N, (int)tb0, st);
                  }),
            "fwd_lse");
    HIP_TRY(timed(CKL_KERNEL_FWD_FINALIZE, st,
                  [&] {
                    return ckl::launch_fwd_rows(b + w.part, (int)q.c_splits, rows, K, p_s + tb0 * K, zg_s + tb0 * K,
                                                E + tb0, M + tb0, mk ? mk + tb0 : nullptr, lse_o + tb0,
                                                rl_o ? rl_o + tb0 : nullptr, blk + tb0, pk.N, (int)tb0, st);
                  }),
            "fwd_rows");
  }
  HIP_TRY(timed(CKL_KERNEL_FWD_FINALIZE, st, [&] { return ckl::launch_loss_reduce(blk, T, N, loss, st); }),
          "loss_reduce");
  if (pk.on()) {
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_scatter_f32(pk.lse, pk.rank, T, lse, st); }),
            "scatter lse");
    if (row_loss)
      HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_scatter_f32(pk.rl, pk.rank, T, row_loss, st); }),
              "scatter row loss");
  }
  return CKL_OK;
}

ckl_status ckl_forward_noalloc(const ckl_problem* p, const void* H, const void* W, const int32_t* idx,
                               const float* tlogit, const uint8_t* mask, float* loss, float* lse, float* row_loss,
                               void* stream) {
  ckl_status s = check_problem(p);
  if (s != CKL_OK) return s;
  if (p->validate)
    return fail(CKL_ERR_UNSUPPORTED, "ckl_forward_noalloc does not validate indices (that reads a flag back "
                                     "and synchronises): use ckl_forward");
  const Plan q = make_plan(p);
  const size_t need = fwd_layout(q, p).total;
  if (need > kScratchBytes)
    return fail(CKL_ERR_UNSUPPORTED,
                "forward workspace of %zu bytes exceeds the %zu-byte device scratch array of ckl_forward_noalloc "
                "(use ckl_forward with a workspace)",
                need, kScratchBytes);
  hipStream_t st = (hipStream_t)stream;
  if (st != nullptr) {
    int cur = -1, sdev = -1;
    HIP_TRY(hipGetDevice(&cur), "hipGetDevice");
    HIP_TRY(hipStreamGetDevice(st, &sdev), "hipStreamGetDevice");
    if (cur != sdev)
      return fail(CKL_ERR_INVALID_ARG, "the stream belongs to device %d but device %d is current", sdev, cur);
  }
  void* ws = nullptr;
  s = scratch_on_current_device(&ws);
  if (s != CKL_OK) return s;
  g_no_events = true;
  s = ckl_forward(p, H, W, idx, tlogit, mask, loss, lse, row_loss, ws, kScratchBytes, stream);
  g_no_events = false;
  return s;
}

ckl_status ckl_backward(const ckl_problem* p, const void* H, const void* W, const int32_t* idx, const float* tlogit,
                        const uint8_t* mask, const float* lse, const float* grad_loss, void* dH, void* dW, void* ws,
                        size_t ws_bytes, void* stream) {
  ckl_status s = check_problem(p);
  if (s != CKL_OK) return s;
  if (!H || !W || !idx || !tlogit || !lse || !dH || !dW) return fail(CKL_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(H) || !aligned16(W) || !aligned16(idx) || !aligned16(tlogit) || !aligned16(dH) || !aligned16(dW) ||
      !aligned16(ws))
    return fail(CKL_ERR_INVALID_ARG, "H, W, idx, tlogit, dH, dW and ws must be 16-byte aligned");
  if (((uintptr_t)lse & 3u) || ((uintptr_t)grad_loss & 3u))
    return fail(CKL_ERR_INVALID_ARG, "lse and grad_loss must be 4-byte aligned");
  const Plan q = make_plan(p);
  const BwdWs w = bwd_layout(q, p);
  if (!ws || ws_bytes < w.total)
    return fail(CKL_ERR_WORKSPACE, "backward workspace needs %zu bytes, got %zu", w.total, ws ? ws_bytes : (size_t)0);
  {
    const size_t T = q.T, K = q.K, d = q.d;
    s = check_disjoint({{dH, T * d * (p->dh_dtype == CKL_BF16 ? 2 : 4), "dH"},
                        {dW, (size_t)q.V * d * (p->dw_dtype == CKL_BF16 ? 2 : 4), "dW"}, {ws, w.total, "ws"}},
                       {{H, T * d * q.esz, "H"}, {W, (size_t)q.V * d * q.esz, "W"}, {idx, T * K * 4, "idx"},
                        {tlogit, T * K * 4, "tlogit"}, {mask, T, "mask"}, {lse, T * 4, "lse"},
                        {grad_loss, 4, "grad_loss"}});
    if (s != CKL_OK) return s;
  }
  hipStream_t st = (hipStream_t)stream;
  char* b = (char*)ws;
  int* idx_s = (int*)(b + w.idx_s);
  float* p_s = (float*)(b + w.p_s);
  float* M = (float*)(b + w.M);
  float* srow = (float*)(b + w.s);
  int* N = (int*)(b + w.N);
  int* bad = (int*)(b + w.bad);
  void* Ht = b + w.Ht;
  void* Wt = b + w.Wt;
  void* Gbuf[kGBuffers];
  void* Gtbuf[kGBuffers];
  for (int i = 0; i < kGBuffers; ++i) {
    Gbuf[i] = b + w.G[i];
    Gtbuf[i] = q.in_bf16 ? nullptr : b + w.Gt[i];
  }
  const int T = (int)q.T, d = (int)q.d, V = (int)q.V, K = (int)q.K;
  const Packed pk = (p->compact_mask && mask) ? packed_at(b, w.pk) : Packed{};
  // dH accumulates in fp32: in dH itself, or in the workspace when dH is
  // bf16 or its rows are packed (scattered back at the end)
  float* dHacc = (p->dh_dtype == CKL_BF16 || pk.on()) ? (float*)(b + w.dH) : (float*)dH;
  float* dWacc = p->dw_dtype == CKL_BF16 ? (float*)(b + w.dW) : (float*)dW;
  const void* Hs = H;
  const uint8_t* mk = mask;
  const float* lse_s = lse;
  if (pk.on()) {
    HIP_TRY(pack_rows(q, pk, mask, H, st), "packing kept rows");
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_gather_f32(lse, pk.perm, pk.N, T, pk.lse, st); }),
            "gather lse");
    N = pk.N;
    Hs = pk.Hc;
    mk = nullptr;
    lse_s = pk.lse;
  } else {
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_count_mask(mask, T, N, st); }), "count_mask");
  }
  if (p->validate) HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_fill_i32(bad, 1, 0, st); }), "fill");
  HIP_TRY(timed(CKL_KERNEL_TEACHER_PREP, st,
                [&] {
                  return ckl::launch_teacher_prep(idx, tlogit, T, K, (int)vtotal(p), (int)p->v_offset, idx_s, p_s, nullptr, M, nullptr,
                                                  p->validate ? bad : nullptr, p->teacher_form, pk.perm, pk.N, st);
                }),
          "teacher_prep");
  if (p->validate) {
    s = check_validate_flag(bad, st);
    if (s != CKL_OK) return s;
  }
  HIP_TRY(timed(CKL_KERNEL_OTHER, st,
                [&] { return ckl::launch_row_scale(mk, grad_loss, N, T, (int)q.Tp, pk.on(), srow, st); }),
          "row_scale");
  HIP_TRY(timed(CKL_KERNEL_TRANSPOSE, st,
                [&] { return ckl::launch_transpose_pad(q.in_bf16, Hs, T, d, (int)q.Tp, Ht, q.Tp + kLdPad, st); }),
          "transpose H");

  const char* Htb = (const char*)Ht;
  const int64_t ldWt = q.Vc + kLdPad;
  for (int64_t vb = 0; vb < q.nV; ++vb) {
    const int64_t vb0 = vb * q.Vc;
    const int64_t vrows = std::min(q.Vc, q.Vp - vb0);
    // W^T of this vocabulary block (zero columns past V)
    HIP_TRY(timed(CKL_KERNEL_TRANSPOSE, st,
                  [&] {
                    return ckl::launch_transpose_pad(q.in_bf16, (const char*)W + vb0 * q.d * q.esz,
                                                     (int)std::min(q.Vc, q.V - vb0), d, (int)vrows, Wt, ldWt, st);
                  }),
            "transpose W block");
    for (int64_t tb = 0; tb < q.nT; ++tb) {
      const int64_t tb0 = tb * q.Tc;
      const int64_t trows = std::min(q.Tc, q.Tp - tb0);
      void* G = Gbuf[0];
      void* Gt = Gtbuf[0];
      int64_t splits, tps;
      pick_splits(trows / q.BN, vrows / q.BM, &splits, &tps);
      HIP_TRY(timed(CKL_KERNEL_BWD_GRAD, st,
                    [&] {
                      return ckl::launch_bwd_grad(q.in_bf16, Hs, W, T, d, V, K, idx_s, p_s, M, lse_s, srow, (int)tb0,
                                                  (int)trows, (int)vb0, (int)vrows, (int)splits, (int)tps, G,
                                                  vrows + kLdPad, Gt, trows + kLdPad, pk.N, st);
                    }),
              "bwd_grad");
      // dW[vb0 .. vb0 + vrows) (+)= G^T H[tb0 .. tb0 + trows)  (longer k: scheduled first)
      // dH[tb0 .. tb0 + trows) (+)= G W[vb0 .. vb0 + vrows)
      // (bf16: G itself, k-major: element (v, t) at G[t ldG + v]; fp32: G^T)
      ckl::GemmArgs gdw{q.in_bf16 ? G : Gt, q.in_bf16 ? vrows + kLdPad : trows + kLdPad, Htb + tb0 * q.esz,
                        q.Tp + kLdPad, dWacc + vb0 * q.d, q.d, (int)std::min(vrows, q.V - vb0), d, (int)trows, tb > 0};
      gdw.xt = q.in_bf16;
      ckl::GemmArgs gdh{G, vrows + kLdPad, Wt, ldWt, dHacc + tb0 * q.d, q.d,
                        (int)std::min(trows, q.T - tb0), d, (int)vrows, vb > 0};
      if (pk.on()) {
        // packed rows: the token rows of this block past the kept rows are
        // skipped (their G rows were not formed)
        gdw.lim = pk.N; gdw.lim_base = (int)tb0; gdw.lim_kind = 2; gdw.lim_round = (int)q.BN;
        gdh.lim = pk.N; gdh.lim_base = (int)tb0; gdh.lim_kind = 1;
      }
      HIP_TRY(timed(CKL_KERNEL_GEMM_DHDW, st, [&] { return ckl::launch_gemm_pair(q.in_bf16, gdw, gdh, st); }),
              "gemm dW + dH");
    }
  }
  if (pk.on()) {
    HIP_TRY(timed(CKL_KERNEL_OTHER, st,
                  [&] { return ckl::launch_scatter_rows(dHacc, pk.rank, T, d, dH, p->dh_dtype == CKL_BF16, st); }),
            "scatter dH");
  } else if (p->dh_dtype == CKL_BF16) {
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_cast_f32_bf16(dHacc, dH, q.T * q.d, st); }),
            "cast dH");
  }
  if (p->dw_dtype == CKL_BF16)
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_cast_f32_bf16(dWacc, dW, q.V * q.d, st); }),
            "cast dW");
  return CKL_OK;
}

ckl_status ckl_forward_backward(const ckl_problem* p, const void* H, const void* W, const int32_t* idx,
                                const float* tlogit, const uint8_t* mask, const float* grad_loss, float* loss,
                                float* lse, float* row_loss, void* dH, void* dW, void* ws, size_t ws_bytes,
                                void* stream) {
  ckl_status s = check_problem(p);
  if (s != CKL_OK) return s;
  if (sharded(p))
    return fail(CKL_ERR_UNSUPPORTED, "W is a vocabulary shard: the one-call path needs the whole vocabulary");
  if (!H || !W || !idx || !tlogit || !loss || !lse || !dH || !dW)
    return fail(CKL_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(H) || !aligned16(W) || !aligned16(idx) || !aligned16(tlogit) || !aligned16(dH) || !aligned16(dW) ||
      !aligned16(ws))
    return fail(CKL_ERR_INVALID_ARG, "H, W, idx, tlogit, dH, dW and ws must be 16-byte aligned");
  if (((uintptr_t)loss & 3u) || ((uintptr_t)lse & 3u) || ((uintptr_t)row_loss & 3u) || ((uintptr_t)grad_loss & 3u))
    return fail(CKL_ERR_INVALID_ARG, "loss, lse, row_loss and grad_loss must be 4-byte aligned");
  const Plan q = make_plan(p);
  const FusedWs w = fused_layout(q, p);
  if (!ws || ws_bytes < w.total)
    return fail(CKL_ERR_WORKSPACE, "forward + backward workspace needs %zu bytes, got %zu", w.total,
                ws ? ws_bytes : (size_t)0);
  {
    const size_t T = q.T, K = q.K, d = q.d;
    s = check_disjoint({{loss, 4, "loss"}, {lse, T * 4, "lse"}, {row_loss, T * 4, "row_loss"},
                        {dH, T * d * (p->dh_dtype == CKL_BF16 ? 2 : 4), "dH"},
                        {dW, (size_t)q.V * d * (p->dw_dtype == CKL_BF16 ? 2 : 4), "dW"}, {ws, w.total, "ws"}},
                       {{H, T * d * q.esz, "H"}, {W, (size_t)q.V * d * q.esz, "W"}, {idx, T * K * 4, "idx"},
                        {tlogit, T * K * 4, "tlogit"}, {mask, T, "mask"}, {grad_loss, 4, "grad_loss"}});
    if (s != CKL_OK) return s;
  }
  hipStream_t st = (hipStream_t)stream;
  char* b = (char*)ws;
  int* idx_s = (int*)(b + w.idx_s);
  float* p_s = (float*)(b + w.p_s);
  float* zg_s = (float*)(b + w.zg_s);
  float* E = (float*)(b + w.E);
  float* M = (float*)(b + w.M);
  double* blk = (double*)(b + w.blk);
  int* N = (int*)(b + w.N);
  int* bad = (int*)(b + w.bad);
  float* srow = (float*)(b + w.s);
  char* Ht = b + w.Ht;
  char* Wt = b + w.Wt;
  char* U = b + w.U;
  char* G = b + w.G;
  char* Gt = q.in_bf16 ? nullptr : b + w.Gt;
  float* mtab = (float*)(b + w.mtab);
  float* dHp = (float*)(b + w.dHp);
  float* dWacc = p->dw_dtype == CKL_BF16 ? (float*)(b + w.dW) : (float*)dW;
  const int T = (int)q.T, d = (int)q.d, V = (int)q.V, K = (int)q.K;
  const int64_t ldG = q.Vp + kLdPad, ldGt = q.Gc * q.Cs + kGtPad, ldW = q.Vp + kLdPad, ldH = q.Gc * q.Cs + kLdPad;
  const int64_t dh_esz = p->dh_dtype == CKL_BF16 ? 2 : 4;
  const Packed pk = (p->compact_mask && mask) ? packed_at(b, w.pk) : Packed{};
  const void* Hs = H;
  const uint8_t* mk = mask;
  float* lse_o = lse;
  float* rl_o = row_loss;
  if (pk.on()) {
    HIP_TRY(pack_rows(q, pk, mask, H, st), "packing kept rows");
    N = pk.N;
    Hs = pk.Hc;
    mk = nullptr;
    lse_o = pk.lse;
    rl_o = row_loss ? pk.rl : nullptr;
  } else {
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_count_mask(mask, T, N, st); }), "count_mask");
  }
  if (p->validate) HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_fill_i32(bad, 1, 0, st); }), "fill");
  HIP_TRY(timed(CKL_KERNEL_TEACHER_PREP, st,
                [&] {
                  return ckl::launch_teacher_prep(idx, tlogit, T, K, (int)vtotal(p), (int)p->v_offset, idx_s, p_s, E, M, zg_s,
                                                  p->validate ? bad : nullptr, p->teacher_form, pk.perm, pk.N, st);
                }),
          "teacher_prep");
  if (p->validate) {
    s = check_validate_flag(bad, st);
    if (s != CKL_OK) return s;
  }
  HIP_TRY(timed(CKL_KERNEL_OTHER, st,
                [&] { return ckl::launch_row_scale(mk, grad_loss, N, T, (int)q.Tp, pk.on(), srow, st); }),
          "row_scale");
  HIP_TRY(timed(CKL_KERNEL_TRANSPOSE, st,
                [&] { return ckl::launch_transpose_pad(q.in_bf16, W, V, d, (int)q.Vp, Wt, ldW, st); }),
          "transpose W");

  for (int64_t c = 0; c < q.nS; ++c) {
    const int64_t tb0 = c * q.Cs;
    const int rows = (int)std::min(q.Cs, q.T - tb0);           // real rows of the chunk
    const int rows_p = (int)std::min(q.Cs, q.Tp - tb0);        // whole logit tiles
    const int64_t slot = c % q.Gc;                               // this chunk's columns of G^T
    // this chunk's rows of G (bf16) or columns of G^T (fp32)
    char* Gc = q.in_bf16 ? G + slot * q.Cs * ldG * q.esz : G;
    char* Gtc = q.in_bf16 ? nullptr : Gt + slot * q.Cs * q.esz;
    const bool dw_now = slot == q.Gc - 1 || c == q.nS - 1;       // the group's last chunk
    const char* Hc = (const char*)Hs + tb0 * q.d * q.esz;
    if (slot == 0) {
      // H^T of this dW group's rows (zero columns past T); the previous
      // group's update, which read the buffer, is ahead on the stream
      const int64_t grows = std::min(q.Gc * q.Cs, q.T - tb0), grows_p = std::min(q.Gc * q.Cs, q.Tp - tb0);
      HIP_TRY(timed(CKL_KERNEL_TRANSPOSE, st,
                    [&] { return ckl::launch_transpose_pad(q.in_bf16, Hc, (int)grows, d, (int)grows_p, Ht, ldH, st); }),
              "transpose H group");
    }
    HIP_TRY(timed(CKL_KERNEL_FWD_LSE, st,
                  [&] {
                    return ckl::launch_fwd_lse(q.in_bf16, Hc, W, rows, d, V, K, idx_s + tb0 * K, zg_s + tb0 * K,
                                               b + w.part, (int)q.c_splits, (int)q.c_tps, q.in_bf16 ? U : G, ldG,
                                               mtab, q.Cs, pk.N, (int)tb0, st);
                  }),
            "fwd_lse (store)");
    HIP_TRY(timed(CKL_KERNEL_FWD_FINALIZE, st,
                  [&] {
                    return ckl::launch_fwd_rows(b + w.part, (int)q.c_splits, rows, K, p_s + tb0 * K, zg_s + tb0 * K,
                                                E + tb0, M + tb0, mk ? mk + tb0 : nullptr, lse_o + tb0,
                                                rl_o ? rl_o + tb0 : nullptr, blk + tb0, pk.N, (int)tb0, st);
                  }),
            "fwd_rows");
    HIP_TRY(timed(CKL_KERNEL_G_PASS, st,
                  [&] {
                    if (q.in_bf16)
                      return ckl::launch_gpass_tiles(U, (int)(q.Vp / q.BM), rows_p / (int)q.BN, Gc, ldG, Gtc, ldGt,
                                                     mtab, q.Cs, srow + tb0, M + tb0, lse_o + tb0, rows, V, pk.N,
                                                     (int)tb0, st);
                    return ckl::launch_gpass(q.in_bf16, G, ldG, Gtc, ldGt, mtab, q.Cs, srow + tb0, M + tb0,
                                             lse_o + tb0, rows, rows_p, V, (int)q.Vp, st);
                  }),
            "gpass");
    HIP_TRY(timed(CKL_KERNEL_OTHER, st,
                  [&] {
                    return ckl::launch_gfix(q.in_bf16, rows, K, V, idx_s + tb0 * K, p_s + tb0 * K, zg_s + tb0 * K,
                                            srow + tb0, M + tb0, lse_o + tb0, Gc, ldG, Gtc, ldGt, st);
                  }),
            "gfix");
    // dH rows of the chunk as Sh split-k partials (long k: scheduled first);
    // at the group's last chunk also dW (+)= G^T H over the group's rows
    ckl::GemmArgs gdh{Gc, ldG, Wt, ldW, dHp, q.d, rows, d, (int)q.Vs, 0};
    gdh.batches = (int)q.Sh;
    gdh.kdim_last = (int)(q.Vp - (q.Sh - 1) * q.Vs);
    gdh.xb = q.Vs;
    gdh.yb = q.Vs;
    gdh.ob = q.Cs * q.d;
    const int64_t g0 = c - slot;  // first chunk of the group
    // dW (+)= G^T H over the group's rows: bf16 reads G itself k-major
    // (element (v, t) at G[t ldG + v]), fp32 reads G^T
    ckl::GemmArgs gdw{q.in_bf16 ? (void*)G : (void*)Gt, q.in_bf16 ? ldG : ldGt, Ht, ldH,
                      dWacc, q.d, dw_now ? V : 0, d, (int)(slot * q.Cs + rows_p), g0 > 0};
    gdw.xt = q.in_bf16;
    if (pk.on()) {
      // packed rows: rows past the kept rows are skipped (no G formed for
      // their tiles)
      gdh.lim = pk.N; gdh.lim_base = (int)tb0; gdh.lim_kind = 1;
      gdw.lim = pk.N; gdw.lim_base = (int)(g0 * q.Cs); gdw.lim_kind = 2; gdw.lim_round = (int)q.BN;
    }
    HIP_TRY(timed(CKL_KERNEL_GEMM_DHDW, st, [&] { return ckl::launch_gemm_pair(q.in_bf16, gdh, gdw, st); }),
            "gemm dH parts + dW");
    HIP_TRY(timed(CKL_KERNEL_OTHER, st,
                  [&] {
                    if (pk.on())
                      return ckl::launch_splitk_sum(dHp, q.Cs * q.d, (int)q.Sh, (int64_t)rows * q.d, dH,
                                                    p->dh_dtype == CKL_BF16, pk.perm + tb0, pk.N, (int)tb0, d, st);
                    return ckl::launch_splitk_sum(dHp, q.Cs * q.d, (int)q.Sh, (int64_t)rows * q.d,
                                                  (char*)dH + tb0 * q.d * dh_esz, p->dh_dtype == CKL_BF16, nullptr,
                                                  nullptr, 0, d, st);
                  }),
            "dH sum");
  }
  HIP_TRY(timed(CKL_KERNEL_FWD_FINALIZE, st,
                [&] { return ckl::launch_loss_reduce(blk, (int)q.T, N, loss, st); }),
          "loss_reduce");
  if (pk.on()) {
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_zero_masked_rows(pk.rank, T, q.d * dh_esz, dH, st); }),
            "zero masked dH rows");
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_scatter_f32(pk.lse, pk.rank, T, lse, st); }),
            "scatter lse");
    if (row_loss)
      HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_scatter_f32(pk.rl, pk.rank, T, row_loss, st); }),
              "scatter row loss");
  }
  if (p->dw_dtype == CKL_BF16)
    HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_cast_f32_bf16(dWacc, dW, q.V * q.d, st); }),
            "cast dW");
  return CKL_OK;
}

ckl_status ckl_shard_forward(const ckl_problem* p, const void* H, const void* W, const int32_t* idx,
                             const float* tlogit, float* lse_part, float* cross_part, void* ws, size_t ws_bytes,
                             void* stream) {
  ckl_status s = check_problem(p);
  if (s != CKL_OK) return s;
  if (!H || !W || !idx || !tlogit || !lse_part || !cross_part)
    return fail(CKL_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(H) || !aligned16(W) || !aligned16(idx) || !aligned16(tlogit) || !aligned16(ws))
    return fail(CKL_ERR_INVALID_ARG, "H, W, idx, tlogit and ws must be 16-byte aligned");
  if (((uintptr_t)lse_part & 3u) || ((uintptr_t)cross_part & 3u))
    return fail(CKL_ERR_INVALID_ARG, "lse_part and cross_part must be 4-byte aligned");
  const Plan q = make_plan(p);
  const FwdWs w = fwd_layout(q, p);
  if (!ws || ws_bytes < w.total)
    return fail(CKL_ERR_WORKSPACE, "shard forward workspace needs %zu bytes, got %zu", w.total,
                ws ? ws_bytes : (size_t)0);
  {
    const size_t T = q.T, K = q.K;
    s = check_disjoint({{lse_part, T * 4, "lse_part"}, {cross_part, T * 4, "cross_part"}, {ws, w.total, "ws"}},
                       {{H, T * q.d * q.esz, "H"}, {W, (size_t)q.V * q.d * q.esz, "W"}, {idx, T * K * 4, "idx"},
                        {tlogit, T * K * 4, "tlogit"}});
    if (s != CKL_OK) return s;
  }
  hipStream_t st = (hipStream_t)stream;
  char* b = (char*)ws;
  int* idx_s = (int*)(b + w.idx_s);
  float* p_s = (float*)(b + w.p_s);
  float* zg_s = (float*)(b + w.zg_s);
  int* bad = (int*)(b + w.bad);
  const int T = (int)q.T, d = (int)q.d, V = (int)q.V, K = (int)q.K;
  if (p->validate) HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_fill_i32(bad, 1, 0, st); }), "fill");
  HIP_TRY(timed(CKL_KERNEL_TEACHER_PREP, st,
                [&] {
                  return ckl::launch_teacher_prep(idx, tlogit, T, K, (int)vtotal(p), (int)p->v_offset, idx_s, p_s,
                                                  (float*)(b + w.E), (float*)(b + w.M), zg_s,
                                                  p->validate ? bad : nullptr, p->teacher_form, nullptr, nullptr, st);
                }),
          "teacher_prep");
  if (p->validate) {
    s = check_validate_flag(bad, st);
    if (s != CKL_OK) return s;
  }
  // chunk by chunk, as ckl_forward
  for (int64_t c = 0; c < q.nS; ++c) {
    const int64_t tb0 = c * q.Cs;
    const int rows = (int)std::min(q.Cs, q.T - tb0);
    if (rows <= 0) break;
    const char* Hc = (const char*)H + tb0 * q.d * q.esz;
    HIP_TRY(timed(CKL_KERNEL_FWD_LSE, st,
                  [&] {
                    return ckl::launch_fwd_lse(q.in_bf16, Hc, W, rows, d, V, K, idx_s + tb0 * K, zg_s + tb0 * K,
                                               b + w.part, (int)q.c_splits, (int)q.c_tps, nullptr, 0, nullptr, 0,
                                               nullptr, 0, st);
                  }),
            "fwd_lse");
    HIP_TRY(timed(CKL_KERNEL_FWD_FINALIZE, st,
                  [&] {
                    return ckl::launch_fwd_shard_rows(b + w.part, (int)q.c_splits, rows, K, p_s + tb0 * K,
                                                      zg_s + tb0 * K, lse_part + tb0, cross_part + tb0, st);
                  }),
            "fwd_shard_rows");
  }
  return CKL_OK;
}

ckl_status ckl_shard_combine(const ckl_problem* p, int32_t n_shards, const float* lse_parts,
                             const float* cross_parts, const int32_t* idx, const float* tlogit, const uint8_t* mask,
                             float* loss, float* lse, float* row_loss, void* ws, size_t ws_bytes, void* stream) {
  ckl_status s = check_problem(p);
  if (s != CKL_OK) return s;
  if (n_shards < 1) return fail(CKL_ERR_INVALID_ARG, "n_shards=%d must be >= 1", (int)n_shards);
  if (!lse_parts || !cross_parts || !idx || !tlogit || !loss || !lse)
    return fail(CKL_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(idx) || !aligned16(tlogit) || !aligned16(ws))
    return fail(CKL_ERR_INVALID_ARG, "idx, tlogit and ws must be 16-byte aligned");
  if (((uintptr_t)lse_parts & 3u) || ((uintptr_t)cross_parts & 3u) || ((uintptr_t)loss & 3u) ||
      ((uintptr_t)lse & 3u) || ((uintptr_t)row_loss & 3u))
    return fail(CKL_ERR_INVALID_ARG, "float arrays must be 4-byte aligned");
  const Plan q = make_plan(p);
  const CombineWs w = combine_layout(q);
  if (!ws || ws_bytes < w.total)
    return fail(CKL_ERR_WORKSPACE, "shard combine workspace needs %zu bytes, got %zu", w.total,
                ws ? ws_bytes : (size_t)0);
  {
    const size_t T = q.T, K = q.K, parts = (size_t)n_shards * T * 4;
    s = check_disjoint({{loss, 4, "loss"}, {lse, T * 4, "lse"}, {row_loss, T * 4, "row_loss"}, {ws, w.total, "ws"}},
                       {{lse_parts, parts, "lse_parts"}, {cross_parts, parts, "cross_parts"}, {idx, T * K * 4, "idx"},
                        {tlogit, T * K * 4, "tlogit"}, {mask, T, "mask"}});
    if (s != CKL_OK) return s;
  }
  hipStream_t st = (hipStream_t)stream;
  char* b = (char*)ws;
  int* N = (int*)(b + w.N);
  const int T = (int)q.T, K = (int)q.K;
  HIP_TRY(timed(CKL_KERNEL_OTHER, st, [&] { return ckl::launch_count_mask(mask, T, N, st); }), "count_mask");
  HIP_TRY(timed(CKL_KERNEL_TEACHER_PREP, st,
                [&] {
                  return ckl::launch_teacher_prep(idx, tlogit, T, K, (int)vtotal(p), 0, (int*)(b + w.idx_s),
                                                  (float*)(b + w.p_s), (float*)(b + w.E), (float*)(b + w.M), nullptr,
                                                  nullptr, p->teacher_form, nullptr, nullptr, st);
                }),
          "teacher_prep");
  HIP_TRY(timed(CKL_KERNEL_FWD_FINALIZE, st,
                [&] {
                  return ckl::launch_shard_combine(lse_parts, cross_parts, (int)n_shards, T, (float*)(b + w.E),
                                                   (float*)(b + w.M), mask, lse, row_loss, (double*)(b + w.blk), N,
                                                   loss, st);
                }),
          "shard_combine");
  return CKL_OK;
}

ckl_status ckl_fused_plan(const ckl_problem* p, int64_t out[5]) {
  ckl_status s = check_problem(p);
  if (s != CKL_OK) return s;
  if (!out) return fail(CKL_ERR_INVALID_ARG, "out is NULL");
  const Plan q = make_plan(p);
  out[0] = q.Cs;
  out[1] = q.nS;
  out[2] = q.Sh;
  out[3] = q.Vs;
  out[4] = q.Gc;
  return CKL_OK;
}

ckl_status ckl_scale_cast(const float* src, void* dst, int64_t n, int32_t dst_dtype, const float* scale,
                          void* stream) {
  if (!src || !dst) return fail(CKL_ERR_INVALID_ARG, "src and dst must not be NULL");
  if (n < 0 || n % 4) return fail(CKL_ERR_INVALID_ARG, "n=%lld must be a non-negative multiple of 4", (long long)n);
  if (dst_dtype != CKL_F32 && dst_dtype != CKL_BF16)
    return fail(CKL_ERR_INVALID_ARG, "dst_dtype must be CKL_F32 (0) or CKL_BF16 (1)");
  if (!aligned16(src) || !aligned16(dst)) return fail(CKL_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  if ((uintptr_t)scale & 3u) return fail(CKL_ERR_INVALID_ARG, "scale must be 4-byte aligned");
  if (dst_dtype == CKL_BF16 && (const char*)dst < (const char*)(src + n) && (const char*)src < (const char*)dst + n * 2)
    return fail(CKL_ERR_INVALID_ARG, "a bf16 dst must not overlap src");
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(timed(CKL_KERNEL_OTHER, st,
                [&] { return ckl::launch_scale_cast(src, dst, n, dst_dtype == CKL_BF16, scale, st); }),
          "scale_cast");
  return CKL_OK;
}

ckl_status ckl_backward_plan(const ckl_problem* p, int64_t out[5]) {
  ckl_status s = check_problem(p);
  if (s != CKL_OK) return s;
  if (!out) return fail(CKL_ERR_INVALID_ARG, "out is NULL");
  const Plan q = make_plan(p);
  out[0] = q.Tc;
  out[1] = q.Vc;
  out[2] = q.nT;
  out[3] = q.nV;
  out[4] = kGBuffers;
  return CKL_OK;
}

ckl_status ckl_timing_enable(int on) {
  if (on != 0 && on != 1) return fail(CKL_ERR_INVALID_ARG, "on must be 0 or 1");
  if (on) {
    hipError_t e = timing_drain();
    if (e != hipSuccess) return hip_fail(e, "draining timing events");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    for (int i = 0; i < CKL_KERNEL_CLASSES; ++i) { g_timing.total_ms[i] = 0.0; g_timing.launches[i] = 0; }
  }
  g_timing.on = on != 0;
  return CKL_OK;
}

ckl_status ckl_timing_read(int kernel_class, double* total_ms, int64_t* launches) {
  if (kernel_class < 0 || kernel_class >= CKL_KERNEL_CLASSES) return fail(CKL_ERR_INVALID_ARG, "bad kernel class");
  if (!total_ms || !launches) return fail(CKL_ERR_INVALID_ARG, "output pointer is NULL");
  hipError_t e = timing_drain();
  if (e != hipSuccess) return hip_fail(e, "reading timing events");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  *total_ms = g_timing.total_ms[kernel_class];
  *launches = g_timing.launches[kernel_class];
  return CKL_OK;
}

const char* ckl_status_string(ckl_status s) {
  switch (s) {
    case CKL_OK: return "ok";
    case CKL_ERR_INVALID_ARG: return "invalid argument";
    case CKL_ERR_UNSUPPORTED: return "unsupported problem";
    case CKL_ERR_WORKSPACE: return "workspace missing or too small";
    case CKL_ERR_BAD_INDEX: return "teacher index out of range or repeated";
    case CKL_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* ckl_last_error(void) { return g_last_error.c_str(); }

int32_t ckl_version(void) { return (2 << 16) | 0; }

}  // extern "C"
