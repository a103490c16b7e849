// libflce: C ABI, argument validation, chunk planner and the per-chunk launch
// sequence of the chunked fused linear cross-entropy (see include/flce.h).
//
// Per chunk of c <= C consecutive tokens (the overview page of Liger Kernel,
// "Computação em Chunk", splits memory-heavy work into chunks to cut peak
// memory), all on the caller's stream:
//   1. forward tile GEMM  Z_c^T = W X_c^T, per (token, vocab tile) max and
//      sum-exp partials, target logit, Z_c stored to scratch (bf16 or fp32);
//   2. combine partials -> lse, per-token loss;
//   3. rewrite Z_c in place into G_c = (softmax - onehot) / N_valid (the
//      page's "Operações In-Place");
//   4. dW  (+)= G_c^T X_c (the first chunk stores);
//   5. dX_c = G_c W.
// Before the chunks a label pass counts N_valid and checks label ranges; after
// them one kernel forms the mean loss, which returns to the host with the
// label flag in the call's single stream synchronisation.
//
// The other entry points reuse the chunk forward and backward below: the
// reductions and per-token outputs change only the weights of step 3;
// cross-entropy on given logits runs its own row kernel; the preference
// losses insert a per-pair (or per-sequence) step between steps 2 and 3 that
// turns the chunk's log-probabilities into loss terms and per-token weights.
#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/flce.h"
#include "flce_internal.h"

#define FLCE_API extern "C" __attribute__((visibility("default")))

namespace flce {
namespace {

thread_local std::string g_last_error;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Shape limits.  N_valid is counted in 32 bits; a chunk's tokens are indexed
// with 32-bit integers; V and H keep every offset inside a tile, a slice or a
// packed block within 32 bits.  On top of these, every launch of a plan must
// stay below 2^32 work-items (grid_fits).
constexpr int64_t kMaxV = 8000000;
constexpr int64_t kMaxH = 1 << 20;
constexpr int64_t kMaxN = ((int64_t)1 << 31) - 1;
constexpr int64_t kMaxChunk = (int64_t)1 << 23;
constexpr int64_t kMaxGridItems = ((int64_t)1 << 32) - 1;
// Rows of cross-entropy on given logits: one workgroup of 1024 work-items per row.
constexpr int64_t kMaxCeRows = kMaxGridItems / 1024;

int check_sizes(int64_t N, int64_t H, int64_t V, int dtype) {
  if (dtype != FLCE_F32 && dtype != FLCE_BF16) return FLCE_EINVAL;
  if (N < 0 || H <= 0 || V <= 0) return FLCE_EINVAL;
  if (V > kMaxV || H > kMaxH || N > kMaxN) return FLCE_EUNSUPPORTED;
  if (dtype == FLCE_BF16 && (H % 8) != 0) return FLCE_EUNSUPPORTED;
  return FLCE_OK;
}

// Largest work-item count of any launch of a call with plan p (chunks of at
// most p.C tokens).
int64_t max_grid_items(const Plan &p) {
  const int64_t C = std::max<int64_t>(p.C, 1), H = p.H, V = p.V;
  int64_t m = C * 256;                                            // lse_combine
  if (p.dtype == FLCE_BF16) {
    const int64_t ct = cdiv(C, 256), vt = cdiv(V, 256);
    m = std::max(m, (ct * (p.nks_h / 2) + cdiv(H, 256) * (p.nks_c / 2)) * 256);  // pack X_c and X_c^T
    m = std::max(m, vt * ct * 256);                               // forward tiles
    m = std::max(m, ct * p.nks_z * 256);                          // dlogits
    m = std::max(m, (int64_t)p.splitk * ct * cdiv(H, 256) * 256); // dX
    m = std::max(m, vt * cdiv(H, 128) * 256);                     // dW
  } else {
    const int64_t T = kTileVF32;
    m = std::max(m, cdiv(V, T) * cdiv(C, T) * 256);               // forward tiles
    m = std::max(m, cdiv(C, T) * cdiv(H, T) * 256);               // dX
    m = std::max(m, cdiv(V, T) * cdiv(H, T) * 256);               // dW
  }
  return m;
}

bool grid_fits(const Plan &p) { return max_grid_items(p) <= kMaxGridItems; }

// Bytes of one row of W in the input dtype.
inline size_t elem_bytes(int dtype) { return dtype == FLCE_BF16 ? 2 : 4; }

// The budget used when the caller gives none: W's own size, at least
// FLCE_DEFAULT_SCRATCH_FLOOR.
size_t default_budget(int64_t H, int64_t V, int dtype) {
  const size_t w = (size_t)H * (size_t)V * elem_bytes(dtype);
  return std::max<size_t>(w, FLCE_DEFAULT_SCRATCH_FLOOR);
}

// Largest power-of-two multiple of 256 tokens (capped at N) whose whole
// workspace fits the budget and whose launches fit their grids; -1 if even the
// smallest does not.
int64_t auto_chunk(int64_t N, int64_t H, int64_t V, int dtype, size_t budget) {
  if (N <= 0) return 0;
  int64_t best = -1;
  for (int64_t C = 256; C <= kMaxChunk; C *= 2) {
    const int64_t Cc = std::min(C, N);
    Plan p;
    make_plan(N, H, V, dtype, Cc, &p);
    if (p.total > budget || !grid_fits(p)) break;
    best = Cc;
    if (C >= N) break;
  }
  return best;
}

// The chunk of a call: the requested one (clamped to N and kMaxChunk) or, for
// req <= 0, the largest that fits the budget (0: the default budget).  *fits
// says whether the workspace of the returned chunk fits the budget; when
// nothing fits, the smallest chunk is returned.
int64_t resolve_chunk(int64_t N, int64_t H, int64_t V, int dtype, int64_t req, size_t budget,
                      bool *fits) {
  *fits = true;
  if (N <= 0) return 0;
  if (req > 0) return std::min(std::min(req, N), kMaxChunk);
  const int64_t c = auto_chunk(N, H, V, dtype, budget ? budget : default_budget(H, V, dtype));
  if (c > 0) return c;
  *fits = false;
  return std::min<int64_t>(256, N);
}

int hip_fail(hipError_t e, const char *what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return FLCE_EHIP;
}

#define CK(x)                                           \
  do {                                                  \
    hipError_t e_ = (x);                                \
    if (e_ != hipSuccess) return hip_fail(e_, #x);      \
  } while (0)

bool misaligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) != 0; }

// ---------------------------------------------------------------- kernel timing
struct Profiler {
  std::atomic<bool> on{false};
  std::atomic<uint32_t> mask{0xffffffffu};   // kernel classes timed while on
  std::mutex mu;
  struct Rec {
    int cls;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;

  hipError_t take(hipEvent_t *e) {
    if (!pool.empty()) {
      *e = pool.back();
      pool.pop_back();
      return hipSuccess;
    }
    return hipEventCreate(e);
  }
};

Profiler &prof() {
  static Profiler p;
  return p;
}

// Run one launcher; while timing is on, bracket it with events on stream s.
template <class F>
hipError_t timed(int cls, hipStream_t s, F &&launch) {
  Profiler &P = prof();
  if (!P.on.load(std::memory_order_relaxed) || !((P.mask.load(std::memory_order_relaxed) >> cls) & 1u))
    return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> g(P.mu);
    hipError_t e = P.take(&a);
    if (e != hipSuccess) return e;
    e = P.take(&b);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(P.mu);
  P.recs.push_back({cls, a, b});
  return hipSuccess;
}

#define LAUNCH(cls, call) CK(timed(cls, s, [&]() { return (call); }))

// How the per-token losses are reduced and what else a call returns.
struct Options {
  int reduction = kReduceMean;
  const float *grad_rows = nullptr;   // per-token upstream gradient (reduction none)
  bool accumulate_dw = false;         // dW += instead of dW =
  float *logprob = nullptr;           // per-token z_y - lse
};

// One chunk's rows, contiguous in memory, and where its per-row outputs go.
struct ChunkIO {
  const void *Xc = nullptr;        // [c, H] rows of X (dtype of the plan)
  const int64_t *lab = nullptr;    // [c] labels
  int c = 0;
  float *rl = nullptr;             // [c] per-token loss (required)
  float *rs = nullptr;             // [c] log-sum-exp or null
  float *lp = nullptr;             // [c] log-probability of the target or null
  const float *wr = nullptr;       // [c] per-token loss weights, or null for sc->scale
  bool acc_dw = false;             // dW += (else dW =)
  void *dXc = nullptr;             // [c, H] rows of dX (backward)
};

// Forward of one chunk: pack X_c (bf16), logits tile GEMM with the LSE
// epilogue (Z_c kept when the backward follows), per-token lse and loss.
int chunk_forward(const Plan &p, char *ws, const void *W, int64_t ii, bool keep_z,
                  const ChunkIO &io, hipStream_t s) {
  const int Hi = (int)p.H, Vi = (int)p.V;
  float *pm = (float *)(ws + p.off_pm);
  float *ps = (float *)(ws + p.off_ps);
  float *pmt = (float *)(ws + p.off_pmt);
  float *zy = (float *)(ws + p.off_zy);
  float *lse = (float *)(ws + p.off_lse);
  if (p.dtype == FLCE_BF16) {
    uint16_t *Zp = (uint16_t *)(ws + p.off_z);
    uint16_t *Xp = (uint16_t *)(ws + p.off_xp);
    // with the backward to follow, X_c transposed for dW too (same launch)
    uint16_t *XpT = keep_z ? (uint16_t *)(ws + p.off_xpt) : nullptr;
    LAUNCH(FLCE_K_PACK, launch_pack_bf16((const uint16_t *)io.Xc, io.c, Hi, Xp, p.nks_h, XpT, p.nks_c, s));
    LAUNCH(FLCE_K_FWD_TILE, launch_fwd_tile_bf16((const uint16_t *)W, Xp, io.lab, ii, io.c, Hi, Vi,
                                                 Zp, p.nks_z, pm, ps, pmt, zy, p.nvt, keep_z, s));
  } else {
    float *z = (float *)(ws + p.off_z);
    LAUNCH(FLCE_K_FWD_TILE, launch_fwd_tile_f32((const float *)W, (const float *)io.Xc, io.lab,
                                                ii, io.c, Hi, Vi, z, p.ldz, pm, ps, zy, p.nvt,
                                                keep_z, s));
  }
  LAUNCH(FLCE_K_LSE_COMBINE, launch_lse_combine(pm, ps, zy, io.lab, ii, io.c, p.nvt, lse, io.rl,
                                                io.rs, io.lp, s));
  return FLCE_OK;
}

// Backward of one chunk after chunk_forward: G_c in place, dX_c, dW.
int chunk_backward(const Plan &p, char *ws, const void *W, int64_t ii, const ChunkIO &io,
                   float *dW, const Scalars *sc, hipStream_t s) {
  const int Hi = (int)p.H, Vi = (int)p.V;
  const float *lse = (const float *)(ws + p.off_lse);
  if (p.dtype == FLCE_BF16) {
    uint16_t *Zp = (uint16_t *)(ws + p.off_z);
    const uint16_t *XpT = (const uint16_t *)(ws + p.off_xpt);
    float *dxp = (float *)(ws + p.off_dxp);
    LAUNCH(FLCE_K_DLOGITS, launch_dlogits_bf16(Zp, p.nks_z, io.c, Vi,
                                               (const float *)(ws + p.off_pmt), lse, io.lab, ii,
                                               io.wr, sc, s));
    // dW first: it reads G while dlogits' writes of it are still in the
    // caches (3% faster per chunk than after dX, whose W stream evicts G)
    LAUNCH(FLCE_K_DW_GEMM, launch_dw_bf16(Zp, p.nks_z, XpT, p.nks_c, io.c, Hi, Vi, dW, io.acc_dw, s));
    LAUNCH(FLCE_K_DX_GEMM, launch_dx_bf16(Zp, p.nks_z, (const uint16_t *)W, io.c, Hi, Vi,
                                          p.splitk, p.ksplit, dxp, s));
    LAUNCH(FLCE_K_DX_REDUCE, launch_dx_reduce_bf16(dxp, p.splitk, io.c, Hi, (uint16_t *)io.dXc, s));
  } else {
    const float *Wf = (const float *)W;
    float *z = (float *)(ws + p.off_z);
    LAUNCH(FLCE_K_DLOGITS, launch_dlogits_f32(z, p.ldz, io.c, Vi, lse, io.lab, ii, io.wr, sc, s));
    LAUNCH(FLCE_K_DW_GEMM, launch_dw_f32(z, p.ldz, (const float *)io.Xc, io.c, Hi, Vi, dW,
                                         io.acc_dw, s));
    LAUNCH(FLCE_K_DX_GEMM, launch_dx_f32(z, p.ldz, Wf, io.c, Hi, Vi, (float *)io.dXc, s));
  }
  return FLCE_OK;
}

int run(bool bwd, const void *X, const void *W, const int64_t *labels, int64_t N, int64_t H,
        int64_t V, int dtype, int64_t ii, int64_t chunk_tokens, float *loss, void *dX, float *dW,
        float *row_loss, float *row_lse, const Options &o, void *workspace,
        size_t workspace_bytes, void *stream) {
  int st = check_sizes(N, H, V, dtype);
  if (st != FLCE_OK) return st;
  if (!loss || !W || !workspace) return FLCE_EINVAL;
  if (o.reduction != kReduceMean && o.reduction != kReduceSum && o.reduction != kReduceNone)
    return FLCE_EINVAL;
  if (o.grad_rows && (o.reduction != kReduceNone || !bwd)) return FLCE_EINVAL;
  if (o.reduction == kReduceNone && N > 0 && !row_loss) return FLCE_EINVAL;
  if (misaligned(o.grad_rows, 4) || misaligned(o.logprob, 4) || misaligned(row_loss, 4) ||
      misaligned(row_lse, 4))
    return FLCE_EINVAL;
  if (N > 0 && (!X || !labels)) return FLCE_EINVAL;
  if (bwd && (!dW || (N > 0 && !dX))) return FLCE_EINVAL;
  if (misaligned(workspace, 256)) return FLCE_EINVAL;
  if (dtype == FLCE_BF16 && (misaligned(X, 16) || misaligned(W, 16) || (bwd && misaligned(dX, 16))))
    return FLCE_EUNSUPPORTED;
  if (dtype == FLCE_F32 && (misaligned(X, 4) || misaligned(W, 4) || (bwd && misaligned(dX, 4))))
    return FLCE_EINVAL;
  if (misaligned(labels, 8) || (bwd && misaligned(dW, 4))) return FLCE_EINVAL;

  bool fits;
  const int64_t C = resolve_chunk(N, H, V, dtype, chunk_tokens, 0, &fits);
  Plan p;
  make_plan(N, H, V, dtype, C, &p);
  if (!grid_fits(p)) return FLCE_EUNSUPPORTED;
  if (workspace_bytes < p.total) return FLCE_EWORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  Scalars *sc = (Scalars *)(ws + p.off_scal);
  float *rowloss = row_loss ? row_loss : (float *)(ws + p.off_rowloss);

  LAUNCH(FLCE_K_LABELS, launch_label_check(labels, N, V, ii, o.reduction, sc, s));
  if (bwd && N == 0 && !o.accumulate_dw) LAUNCH(FLCE_K_FINAL, launch_fill_f32(dW, V * H, 0.f, s));

  for (int64_t c0 = 0; c0 < N; c0 += C) {
    ChunkIO io;
    io.c = (int)std::min(C, N - c0);
    io.Xc = (const char *)X + c0 * H * (dtype == FLCE_BF16 ? 2 : 4);
    io.lab = labels + c0;
    io.rl = rowloss + c0;
    io.rs = row_lse ? row_lse + c0 : nullptr;
    io.lp = o.logprob ? o.logprob + c0 : nullptr;
    io.wr = o.grad_rows ? o.grad_rows + c0 : nullptr;
    io.acc_dw = c0 > 0 || o.accumulate_dw;
    io.dXc = bwd ? (char *)dX + c0 * H * (dtype == FLCE_BF16 ? 2 : 4) : nullptr;
    st = chunk_forward(p, ws, W, ii, bwd, io, s);
    if (st != FLCE_OK) return st;
    if (bwd) {
      st = chunk_backward(p, ws, W, ii, io, dW, sc, s);
      if (st != FLCE_OK) return st;
    }
  }
  LAUNCH(FLCE_K_FINAL, launch_final_loss(rowloss, N, o.reduction, sc, s));
  float host[2];
  CK(hipMemcpyAsync(host, sc, sizeof(host), hipMemcpyDeviceToHost, s));
  CK(hipStreamSynchronize(s));
  int flag;
  std::memcpy(&flag, &host[1], sizeof(flag));
  if (flag) return FLCE_ELABEL;
  *loss = host[0];
  return FLCE_OK;
}

}  // namespace

int choose_splitk(int64_t C, int64_t H, int64_t V) {
  // Spread the dX GEMM's few output tiles over the 256 CUs by splitting the
  // vocabulary (its k) S ways, every split at least 1024 rows deep.  Time
  // model: the main loop takes ceil(units / 256) waves of units = tiles S
  // workgroups, each wave the time of 256 units' share of the GEMM; the S
  // fp32 partial sums are written and read back once.  On the Llama-3-8B head
  // at chunk 1024 it picks one full wave (S = 4); measured, one wave beats two
  // (dX 0.797 against 0.802 ms, the reduction 0.014 against 0.024 ms).
  const double tiles = (double)(cdiv(C, 256) * cdiv(H, 256));
  const double gemm = 2.0 * (double)C * (double)H * (double)V / 1.3e15;   // s at one full wave
  const double part = 8.0 * (double)C * (double)H / 6.0e12;              // s per split
  double best = 1e300;
  int bestS = 1;
  for (int S = 1; S <= kMaxSplitK; ++S) {
    if (S > 1 && V / S < 1024) break;
    const double units = tiles * S;
    const double waves = std::ceil(units / 256.0);
    const double t = gemm * waves * 256.0 / units + (S > 1 ? part * S : 0.0);
    if (t < best * (1.0 - 1e-9)) {
      best = t;
      bestS = S;
    }
  }
  return bestS;
}

void make_plan(int64_t N, int64_t H, int64_t V, int dtype, int64_t C, Plan *p) {
  const bool bf = dtype == FLCE_BF16;
  const int64_t esz = bf ? 2 : 4;
  p->dtype = dtype;
  p->N = N;
  p->H = H;
  p->V = V;
  p->C = C;
  p->ldz = bf ? round_up(V, 8) : round_up(V, 4);
  p->nvt = bf ? 2 * cdiv(V, kTileVBf16) : cdiv(V, kTileVF32);
  if (bf && C > 0) {
    int S = choose_splitk(C, H, V);
    p->ksplit = round_up(cdiv(V, S), 64);
    p->splitk = (int)cdiv(V, p->ksplit);
  } else {
    p->splitk = 0;
    p->ksplit = 0;
  }
  size_t o = 0;
  p->off_scal = o;
  o += 256;
  if (bf) {
    // packed layouts: rows and columns padded to 256 (see flce_internal.h)
    p->nks_z = cdiv(V, 256) * 8;
    p->nks_h = cdiv(H, 256) * 8;
    const size_t cpad = (size_t)round_up(C, 256);
    p->off_z = o;                        // logits, then G, of the chunk (rows = tokens)
    o += align256(cpad * p->nks_z * 64);
    p->off_xp = o;                       // the chunk's X (rows = tokens)
    o += align256(cpad * p->nks_h * 64);
    p->nks_c = cdiv(C, 256) * 8;
    p->off_xpt = o;                      // the chunk's X transposed (rows = hidden), for dW
    o += align256((size_t)round_up(H, 256) * p->nks_c * 64);
  } else {
    p->off_z = o;
    o += align256((size_t)C * p->ldz * esz);
  }
  p->off_pm = o;
  o += align256((size_t)C * p->nvt * 4);
  p->off_ps = o;
  o += align256((size_t)C * p->nvt * 4);
  if (bf) {
    p->off_pmt = o;
    o += align256((size_t)C * p->nvt * 4);
  }
  p->off_zy = o;
  o += align256((size_t)C * 4);
  p->off_lse = o;
  o += align256((size_t)C * 4);
  p->off_rowloss = o;
  o += align256((size_t)N * 4);
  p->off_dxp = o;
  o += align256((size_t)p->splitk * C * H * 4);
  p->total = o;
}

}  // namespace flce

using namespace flce;

FLCE_API size_t flce_workspace_bytes(int64_t N, int64_t H, int64_t V, int dtype,
                                     int64_t chunk_tokens) {
  if (check_sizes(N, H, V, dtype) != FLCE_OK) return 0;
  bool fits;
  const int64_t C = resolve_chunk(N, H, V, dtype, chunk_tokens, 0, &fits);
  Plan p;
  make_plan(N, H, V, dtype, C, &p);
  return p.total;
}

FLCE_API int flce_plan(int64_t N, int64_t H, int64_t V, int dtype, int64_t *chunk_tokens,
                       size_t scratch_budget_bytes, size_t *peak_scratch_bytes) {
  const int st = check_sizes(N, H, V, dtype);
  if (st != FLCE_OK) return st;
  if (!chunk_tokens) return FLCE_EINVAL;
  bool fits;
  const int64_t C = resolve_chunk(N, H, V, dtype, *chunk_tokens, scratch_budget_bytes, &fits);
  Plan p;
  make_plan(N, H, V, dtype, C, &p);
  *chunk_tokens = C;
  if (peak_scratch_bytes) *peak_scratch_bytes = p.total;
  if (!grid_fits(p)) return FLCE_EUNSUPPORTED;
  // an explicit chunk is checked against an explicit budget too
  if (scratch_budget_bytes && p.total > scratch_budget_bytes) fits = false;
  return fits ? FLCE_OK : FLCE_EWORKSPACE;
}

FLCE_API int flce_fwd_bwd(const void *X, const void *W, const int64_t *labels, int64_t N,
                          int64_t H, int64_t V, int dtype, int64_t ignore_index,
                          int64_t chunk_tokens, float *loss, void *dX, float *dW, float *row_loss,
                          float *row_lse, void *workspace, size_t workspace_bytes, void *stream) {
  return run(true, X, W, labels, N, H, V, dtype, ignore_index, chunk_tokens, loss, dX, dW,
             row_loss, row_lse, Options{}, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- no device allocation
// flce_fwd_bwd for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops): its workspace is a file-scope
// device array of fixed size instead of a caller buffer.  In host code the
// array's name is only a stand-in; its device address, one per GPU, comes
// from hipGetSymbolAddress with that GPU current and is what the kernels
// get.  Nothing in the workspace has to start at zero (every call writes its
// scratch before reading it), so the array is never cleared.  Calls that
// overlap in time on one GPU share the array and race.

namespace flce {
namespace {

constexpr size_t kStaticScratchBytes = FLCE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device, looked up once per device.
int static_scratch(void **out) {
  int dev = -1;
  CK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "flce_fwd_bwd_noalloc: device ordinal beyond the supported range";
    return FLCE_EUNSUPPORTED;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    CK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) {
      g_last_error = "flce_fwd_bwd_noalloc: no device address for the scratch array";
      return FLCE_EHIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FLCE_OK;
}

}  // namespace
}  // namespace flce

FLCE_API size_t flce_noalloc_scratch_bytes(void) { return flce::kStaticScratchBytes; }

FLCE_API int flce_fwd_bwd_noalloc(const void *X, const void *W, const int64_t *labels, int64_t N,
                                  int64_t H, int64_t V, int dtype, int64_t ignore_index,
                                  int64_t chunk_tokens, float *loss, void *dX, float *dW,
                                  float *row_loss, float *row_lse, void *stream) {
  // sizes first, on the host: a call that cannot fit the array touches no device
  int st = check_sizes(N, H, V, dtype);
  if (st != FLCE_OK) return st;
  bool fits;
  const int64_t C = resolve_chunk(N, H, V, dtype, chunk_tokens, kStaticScratchBytes, &fits);
  Plan p;
  make_plan(N, H, V, dtype, C, &p);
  if (!fits || p.total > kStaticScratchBytes) {
    g_last_error = "flce_fwd_bwd_noalloc: the workspace of this call (" + std::to_string(p.total) +
                   " bytes) exceeds the static scratch of " + std::to_string(kStaticScratchBytes) +
                   " bytes";
    return FLCE_EWORKSPACE;
  }
  void *ws = nullptr;
  st = static_scratch(&ws);
  if (st != FLCE_OK) return st;
  return run(true, X, W, labels, N, H, V, dtype, ignore_index, C, loss, dX, dW, row_loss,
             row_lse, Options{}, ws, kStaticScratchBytes, stream);
}

FLCE_API int flce_fwd(const void *X, const void *W, const int64_t *labels, int64_t N, int64_t H,
                      int64_t V, int dtype, int64_t ignore_index, int64_t chunk_tokens,
                      float *loss, float *row_loss, float *row_lse, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return run(false, X, W, labels, N, H, V, dtype, ignore_index, chunk_tokens, loss, nullptr,
             nullptr, row_loss, row_lse, Options{}, workspace, workspace_bytes, stream);
}

FLCE_API int flce_fwd_bwd_ex(const void *X, const void *W, const int64_t *labels, int64_t N,
                             int64_t H, int64_t V, int dtype, int64_t ignore_index,
                             int64_t chunk_tokens, int reduction, const float *grad_rows,
                             int accumulate_dw, float *loss, void *dX, float *dW,
                             float *row_loss, float *row_lse, float *logprob, void *workspace,
                             size_t workspace_bytes, void *stream) {
  Options o;
  o.reduction = reduction;
  o.grad_rows = grad_rows;
  o.accumulate_dw = accumulate_dw != 0;
  o.logprob = logprob;
  return run(true, X, W, labels, N, H, V, dtype, ignore_index, chunk_tokens, loss, dX, dW,
             row_loss, row_lse, o, workspace, workspace_bytes, stream);
}

FLCE_API int flce_fwd_ex(const void *X, const void *W, const int64_t *labels, int64_t N,
                         int64_t H, int64_t V, int dtype, int64_t ignore_index,
                         int64_t chunk_tokens, int reduction, float *loss, float *row_loss,
                         float *row_lse, float *logprob, void *workspace,
                         size_t workspace_bytes, void *stream) {
  Options o;
  o.reduction = reduction;
  o.logprob = logprob;
  return run(false, X, W, labels, N, H, V, dtype, ignore_index, chunk_tokens, loss, nullptr,
             nullptr, row_loss, row_lse, o, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- cross-entropy on given logits

namespace flce {
namespace {

constexpr size_t kCeRowLossOffset = 256;

int run_ce(bool grad, void *logits, const int64_t *labels, int64_t N, int64_t V, int dtype,
           int64_t ii, int reduction, const float *grad_rows, float *loss, float *row_loss,
           float *row_lse, float *logprob, void *workspace, size_t workspace_bytes,
           void *stream) {
  if (dtype != FLCE_F32 && dtype != FLCE_BF16) return FLCE_EINVAL;
  if (N < 0 || V <= 0 || !loss || !workspace) return FLCE_EINVAL;
  if (N > kMaxCeRows || V > ((int64_t)1 << 31)) return FLCE_EUNSUPPORTED;
  if (N > 0 && (!logits || !labels)) return FLCE_EINVAL;
  if (reduction != kReduceMean && reduction != kReduceSum && reduction != kReduceNone)
    return FLCE_EINVAL;
  if (grad_rows && (reduction != kReduceNone || !grad)) return FLCE_EINVAL;
  if (reduction == kReduceNone && N > 0 && !row_loss) return FLCE_EINVAL;
  if (misaligned(workspace, 256) || misaligned(labels, 8) ||
      misaligned(logits, dtype == FLCE_F32 ? 4 : 2) || misaligned(grad_rows, 4) ||
      misaligned(row_loss, 4) || misaligned(row_lse, 4) || misaligned(logprob, 4))
    return FLCE_EINVAL;
  if (workspace_bytes < flce_ce_workspace_bytes(N)) return FLCE_EWORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  Scalars *sc = (Scalars *)ws;
  float *rl = row_loss ? row_loss : (float *)(ws + kCeRowLossOffset);
  LAUNCH(FLCE_K_LABELS, launch_label_check(labels, N, V, ii, reduction, sc, s));
  LAUNCH(FLCE_K_CE_ROWS, launch_ce_rows(logits, N, V, dtype, labels, ii, grad, grad_rows, sc, rl,
                                        row_lse, logprob, s));
  LAUNCH(FLCE_K_FINAL, launch_final_loss(rl, N, reduction, sc, s));
  float host[2];
  CK(hipMemcpyAsync(host, sc, sizeof(host), hipMemcpyDeviceToHost, s));
  CK(hipStreamSynchronize(s));
  int flag;
  std::memcpy(&flag, &host[1], sizeof(flag));
  if (flag) return FLCE_ELABEL;
  *loss = host[0];
  return FLCE_OK;
}

}  // namespace
}  // namespace flce

FLCE_API size_t flce_ce_workspace_bytes(int64_t N) {
  if (N < 0) return 0;
  return flce::kCeRowLossOffset + flce::align256((size_t)N * 4);
}

FLCE_API int flce_ce_fwd_bwd(void *logits, const int64_t *labels, int64_t N, int64_t V, int dtype,
                             int64_t ignore_index, int reduction, const float *grad_rows,
                             float *loss, float *row_loss, float *row_lse, float *logprob,
                             void *workspace, size_t workspace_bytes, void *stream) {
  return flce::run_ce(true, logits, labels, N, V, dtype, ignore_index, reduction, grad_rows, loss,
                      row_loss, row_lse, logprob, workspace, workspace_bytes, stream);
}

FLCE_API int flce_ce_fwd(const void *logits, const int64_t *labels, int64_t N, int64_t V,
                         int dtype, int64_t ignore_index, int reduction, float *loss,
                         float *row_loss, float *row_lse, float *logprob, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return flce::run_ce(false, const_cast<void *>(logits), labels, N, V, dtype, ignore_index,
                      reduction, nullptr, loss, row_loss, row_lse, logprob, workspace,
                      workspace_bytes, stream);
}

// ---------------------------------------------------------------- pairwise preference losses
// A chunk holds k whole pairs: their chosen rows, then their rejected rows,
// gathered from the two halves of X into one contiguous chunk, so the fused
// pipeline runs on it unchanged.  Between its forward and its backward the
// per-pair step turns the chunk's per-token log-probabilities into the loss
// terms and the per-token weights of the backward (pair_kernels.hip).

namespace flce {
namespace {

constexpr int64_t kPrefAutoRows = 4096;

struct PairLayout {
  Plan p;                 // the fused pipeline for chunks of C = 2 k T rows
  int64_t k = 0;          // pairs per chunk
  size_t off_x = 0, off_lab = 0, off_lp = 0, off_w = 0, off_dx = 0, off_nll = 0, off_or = 0,
         off_clp = 0, off_rlp = 0, off_lor = 0, total = 0;
};

int pair_check(int64_t B, int64_t T, int64_t H, int64_t V, int dtype) {
  if (B <= 0 || T <= 0) return FLCE_EINVAL;
  if (T > ((int64_t)1 << 29) || B > kMaxN / (2 * T)) return FLCE_EUNSUPPORTED;
  return check_sizes(2 * B * T, H, V, dtype);
}

void pair_layout(int64_t B, int64_t T, int64_t H, int64_t V, int dtype, int64_t chunk_pairs,
                 PairLayout *L) {
  int64_t k = chunk_pairs > 0 ? chunk_pairs : kPrefAutoRows / (2 * T);
  k = std::max<int64_t>(1, std::min({k, B, kMaxChunk / (2 * T)}));
  const int64_t C = 2 * k * T;
  const size_t esz = dtype == FLCE_BF16 ? 2 : 4;
  make_plan(C, H, V, dtype, C, &L->p);       // its per-token loss array holds one chunk
  L->k = k;
  size_t o = L->p.total;
  L->off_x = o;
  o += align256((size_t)C * H * esz);
  L->off_lab = o;
  o += align256((size_t)C * 8);
  L->off_lp = o;
  o += align256((size_t)C * 4);
  L->off_w = o;
  o += align256((size_t)C * 4);
  L->off_dx = o;
  o += align256((size_t)C * H * esz);
  size_t *pair_arrays[5] = {&L->off_nll, &L->off_or, &L->off_clp, &L->off_rlp, &L->off_lor};
  for (size_t *q : pair_arrays) {
    *q = o;
    o += align256((size_t)B * 4);
  }
  L->total = o;
}

int run_pairs(bool bwd, int kind, const void *X, const void *W, const int64_t *labels, int64_t B,
              int64_t T, int64_t H, int64_t V, int dtype, int64_t ii, const PairParams &pp,
              int64_t chunk_pairs, float *loss, float *nll, void *dX, float *dW,
              float *chosen_logp, float *rejected_logp, float *log_odds_ratio, void *workspace,
              size_t workspace_bytes, void *stream) {
  int st = pair_check(B, T, H, V, dtype);
  if (st != FLCE_OK) return st;
  if (kind != kPairOrpo && kind != kPairSimpo && kind != kPairCpo && kind != kPairDpo)
    return FLCE_EINVAL;
  if (kind == kPairDpo && (!pp.ref_c || !pp.ref_r)) return FLCE_EINVAL;
  if (misaligned(pp.ref_c, 4) || misaligned(pp.ref_r, 4)) return FLCE_EINVAL;
  if (!loss || !X || !W || !labels || !workspace) return FLCE_EINVAL;
  if (bwd && (!dX || !dW)) return FLCE_EINVAL;
  if (misaligned(workspace, 256) || misaligned(labels, 8) || misaligned(chosen_logp, 4) ||
      misaligned(rejected_logp, 4) || misaligned(log_odds_ratio, 4))
    return FLCE_EINVAL;
  if (dtype == FLCE_BF16 && (misaligned(X, 16) || misaligned(W, 16) || (bwd && misaligned(dX, 16))))
    return FLCE_EUNSUPPORTED;
  if (dtype == FLCE_F32 && (misaligned(X, 4) || misaligned(W, 4) || (bwd && misaligned(dX, 4))))
    return FLCE_EINVAL;
  if (bwd && misaligned(dW, 4)) return FLCE_EINVAL;
  PairLayout L;
  pair_layout(B, T, H, V, dtype, chunk_pairs, &L);
  if (!grid_fits(L.p)) return FLCE_EUNSUPPORTED;
  if (workspace_bytes < L.total) return FLCE_EWORKSPACE;

  const Plan &p = L.p;
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  Scalars *sc = (Scalars *)(ws + p.off_scal);
  const int64_t esz = dtype == FLCE_BF16 ? 2 : 4;
  const int64_t half = B * T;                        // rows of each half of X
  char *xbuf = ws + L.off_x, *dxbuf = ws + L.off_dx;
  int64_t *lab = (int64_t *)(ws + L.off_lab);
  float *rl = (float *)(ws + p.off_rowloss), *lp = (float *)(ws + L.off_lp);
  float *wrow = (float *)(ws + L.off_w);
  float *nll_sum = (float *)(ws + L.off_nll), *or_term = (float *)(ws + L.off_or);
  float *clp = chosen_logp ? chosen_logp : (float *)(ws + L.off_clp);
  float *rlp = rejected_logp ? rejected_logp : (float *)(ws + L.off_rlp);
  float *lor = log_odds_ratio ? log_odds_ratio : (float *)(ws + L.off_lor);

  LAUNCH(FLCE_K_PAIRS, launch_pairs_labels(labels, 2 * half, half, V, ii, sc, s));
  for (int64_t p0 = 0; p0 < B; p0 += L.k) {
    const int64_t kk = std::min(L.k, B - p0);
    const int64_t rows = kk * T;                     // rows of each half in this chunk
    const int64_t rb = rows * H * esz;
    const char *xc = (const char *)X + p0 * T * H * esz;
    const char *xr = (const char *)X + (half + p0 * T) * H * esz;
    const CopySeg gather[4] = {{xbuf, xc, rb},
                               {xbuf + rb, xr, rb},
                               {lab, labels + p0 * T, rows * 8},
                               {lab + rows, labels + half + p0 * T, rows * 8}};
    LAUNCH(FLCE_K_PAIR_ROWS, launch_copy_segments(gather, 4, s));
    ChunkIO io;
    io.Xc = xbuf;
    io.lab = lab;
    io.c = (int)(2 * rows);
    io.rl = rl;
    io.lp = lp;
    io.wr = bwd ? wrow : nullptr;
    io.acc_dw = p0 > 0;
    io.dXc = dxbuf;
    st = chunk_forward(p, ws, W, ii, bwd, io, s);
    if (st != FLCE_OK) return st;
    LAUNCH(FLCE_K_PAIRS, launch_pairs(kind, lp, rl, lab, ii, T, (int)kk, p0, B, pp, sc,
                                      bwd ? wrow : nullptr, nll_sum, or_term, clp, rlp, lor, s));
    if (bwd) {
      st = chunk_backward(p, ws, W, ii, io, dW, sc, s);
      if (st != FLCE_OK) return st;
      const CopySeg scatter[2] = {{(char *)dX + p0 * T * H * esz, dxbuf, rb},
                                  {(char *)dX + (half + p0 * T) * H * esz, dxbuf + rb, rb}};
      LAUNCH(FLCE_K_PAIR_ROWS, launch_copy_segments(scatter, 2, s));
    }
  }
  LAUNCH(FLCE_K_PAIRS, launch_pairs_final(nll_sum, or_term, B, pp.alpha, pp.lambda, sc, s));
  Scalars host;
  CK(hipMemcpyAsync(&host, sc, sizeof(host), hipMemcpyDeviceToHost, s));
  CK(hipStreamSynchronize(s));
  if (host.flag) return FLCE_ELABEL;
  *loss = host.loss;
  if (nll) *nll = host.aux;
  return FLCE_OK;
}

}  // namespace
}  // namespace flce

namespace flce {
namespace {

PairParams orpo_params(float beta) {
  PairParams pp{};
  pp.beta = beta;
  pp.alpha = 1.f;
  pp.lambda = beta;
  return pp;
}

PairParams pair_params(int kind, float beta, float gamma, float alpha, const float *ref_c,
                       const float *ref_r) {
  PairParams pp{};
  pp.beta = beta;
  pp.gamma = gamma;
  pp.alpha = alpha;
  pp.lambda = kind == kPairOrpo ? beta : 1.f;
  pp.ref_c = ref_c;
  pp.ref_r = ref_r;
  return pp;
}

}  // namespace
}  // namespace flce

FLCE_API size_t flce_pair_workspace_bytes(int64_t n_pairs, int64_t T, int64_t H, int64_t V,
                                          int dtype, int64_t chunk_pairs) {
  if (flce::pair_check(n_pairs, T, H, V, dtype) != FLCE_OK) return 0;
  flce::PairLayout L;
  flce::pair_layout(n_pairs, T, H, V, dtype, chunk_pairs, &L);
  return L.total;
}

FLCE_API size_t flce_orpo_workspace_bytes(int64_t n_pairs, int64_t T, int64_t H, int64_t V,
                                          int dtype, int64_t chunk_pairs) {
  return flce_pair_workspace_bytes(n_pairs, T, H, V, dtype, chunk_pairs);
}

FLCE_API int flce_pair_fwd_bwd(int kind, const void *X, const void *W, const int64_t *labels,
                               int64_t n_pairs, int64_t T, int64_t H, int64_t V, int dtype,
                               int64_t ignore_index, float beta, float gamma, float alpha,
                               const float *ref_chosen_logp, const float *ref_rejected_logp,
                               int64_t chunk_pairs, float *loss, float *nll, void *dX, float *dW,
                               float *chosen_logp, float *rejected_logp, float *pair_logit,
                               void *workspace, size_t workspace_bytes, void *stream) {
  return flce::run_pairs(true, kind, X, W, labels, n_pairs, T, H, V, dtype, ignore_index,
                         flce::pair_params(kind, beta, gamma, alpha, ref_chosen_logp,
                                           ref_rejected_logp),
                         chunk_pairs, loss, nll, dX, dW, chosen_logp, rejected_logp, pair_logit,
                         workspace, workspace_bytes, stream);
}

FLCE_API int flce_pair_fwd(int kind, const void *X, const void *W, const int64_t *labels,
                           int64_t n_pairs, int64_t T, int64_t H, int64_t V, int dtype,
                           int64_t ignore_index, float beta, float gamma, float alpha,
                           const float *ref_chosen_logp, const float *ref_rejected_logp,
                           int64_t chunk_pairs, float *loss, float *nll, float *chosen_logp,
                           float *rejected_logp, float *pair_logit, void *workspace,
                           size_t workspace_bytes, void *stream) {
  return flce::run_pairs(false, kind, X, W, labels, n_pairs, T, H, V, dtype, ignore_index,
                         flce::pair_params(kind, beta, gamma, alpha, ref_chosen_logp,
                                           ref_rejected_logp),
                         chunk_pairs, loss, nll, nullptr, nullptr, chosen_logp, rejected_logp,
                         pair_logit, workspace, workspace_bytes, stream);
}

FLCE_API int flce_orpo_fwd_bwd(const void *X, const void *W, const int64_t *labels,
                               int64_t n_pairs, int64_t T, int64_t H, int64_t V, int dtype,
                               int64_t ignore_index, float beta, int64_t chunk_pairs, float *loss,
                               float *nll, void *dX, float *dW, float *chosen_logp,
                               float *rejected_logp, float *log_odds_ratio, void *workspace,
                               size_t workspace_bytes, void *stream) {
  return flce::run_pairs(true, flce::kPairOrpo, X, W, labels, n_pairs, T, H, V, dtype,
                         ignore_index, flce::orpo_params(beta), chunk_pairs, loss, nll, dX, dW,
                         chosen_logp, rejected_logp, log_odds_ratio, workspace, workspace_bytes,
                         stream);
}

FLCE_API int flce_orpo_fwd(const void *X, const void *W, const int64_t *labels, int64_t n_pairs,
                           int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                           float beta, int64_t chunk_pairs, float *loss, float *nll,
                           float *chosen_logp, float *rejected_logp, float *log_odds_ratio,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return flce::run_pairs(false, flce::kPairOrpo, X, W, labels, n_pairs, T, H, V, dtype,
                         ignore_index, flce::orpo_params(beta), chunk_pairs, loss, nll, nullptr,
                         nullptr, chosen_logp, rejected_logp, log_odds_ratio, workspace,
                         workspace_bytes, stream);
}

// ---------------------------------------------------------------- unpaired preference loss (KTO)
// A chunk holds k whole consecutive sequences, already contiguous in X; the
// per-sequence step runs between the chunk's forward and backward.

namespace flce {
namespace {

struct KtoLayout {
  Plan p;
  int64_t k = 0;          // sequences per chunk
  size_t off_lp = 0, off_w = 0, off_term = 0, off_logp = 0, off_rew = 0, total = 0;
};

int kto_check(int64_t S, int64_t T, int64_t H, int64_t V, int dtype) {
  if (S <= 0 || T <= 0) return FLCE_EINVAL;
  if (T > ((int64_t)1 << 30) || S > kMaxN / T) return FLCE_EUNSUPPORTED;
  return check_sizes(S * T, H, V, dtype);
}

void kto_layout(int64_t S, int64_t T, int64_t H, int64_t V, int dtype, int64_t chunk_seqs,
                KtoLayout *L) {
  int64_t k = chunk_seqs > 0 ? chunk_seqs : kPrefAutoRows / T;
  k = std::max<int64_t>(1, std::min({k, S, kMaxChunk / T}));
  const int64_t C = k * T;
  make_plan(C, H, V, dtype, C, &L->p);
  L->k = k;
  size_t o = L->p.total;
  L->off_lp = o;
  o += align256((size_t)C * 4);
  L->off_w = o;
  o += align256((size_t)C * 4);
  size_t *seq_arrays[3] = {&L->off_term, &L->off_logp, &L->off_rew};
  for (size_t *q : seq_arrays) {
    *q = o;
    o += align256((size_t)S * 4);
  }
  L->total = o;
}

// refpoint: forward only, and the call's scalar result is the reference point
// z0 = max(0, mean of r) instead of the loss (the flags do not enter r).
int run_kto(bool bwd, const void *X, const void *W, const int64_t *labels, int64_t S, int64_t T,
            int64_t H, int64_t V, int dtype, int64_t ii, const KtoParams &kp, int64_t chunk_seqs,
            float *loss, void *dX, float *dW, float *logp, float *reward, void *workspace,
            size_t workspace_bytes, void *stream, bool refpoint = false) {
  int st = kto_check(S, T, H, V, dtype);
  if (st != FLCE_OK) return st;
  if (!loss || !X || !W || !labels || !workspace || !kp.ref) return FLCE_EINVAL;
  if (!kp.desirable && !refpoint) return FLCE_EINVAL;
  if (bwd && (!dX || !dW)) return FLCE_EINVAL;
  if (misaligned(workspace, 256) || misaligned(labels, 8) || misaligned(kp.desirable, 4) ||
      misaligned(kp.ref, 4) || misaligned(logp, 4) || misaligned(reward, 4))
    return FLCE_EINVAL;
  if (dtype == FLCE_BF16 && (misaligned(X, 16) || misaligned(W, 16) || (bwd && misaligned(dX, 16))))
    return FLCE_EUNSUPPORTED;
  if (dtype == FLCE_F32 && (misaligned(X, 4) || misaligned(W, 4) || (bwd && misaligned(dX, 4))))
    return FLCE_EINVAL;
  if (bwd && misaligned(dW, 4)) return FLCE_EINVAL;
  KtoLayout L;
  kto_layout(S, T, H, V, dtype, chunk_seqs, &L);
  if (!grid_fits(L.p)) return FLCE_EUNSUPPORTED;
  if (workspace_bytes < L.total) return FLCE_EWORKSPACE;

  const Plan &p = L.p;
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  Scalars *sc = (Scalars *)(ws + p.off_scal);
  const int64_t esz = dtype == FLCE_BF16 ? 2 : 4;
  float *rl = (float *)(ws + p.off_rowloss), *lp = (float *)(ws + L.off_lp);
  float *wrow = (float *)(ws + L.off_w), *term = (float *)(ws + L.off_term);
  float *lpo = logp ? logp : (float *)(ws + L.off_logp);
  float *rwo = reward ? reward : (float *)(ws + L.off_rew);

  LAUNCH(FLCE_K_PAIRS, launch_pairs_labels(labels, S * T, 0, V, ii, sc, s));
  for (int64_t s0 = 0; s0 < S; s0 += L.k) {
    const int64_t kk = std::min(L.k, S - s0);
    ChunkIO io;
    io.Xc = (const char *)X + s0 * T * H * esz;
    io.lab = labels + s0 * T;
    io.c = (int)(kk * T);
    io.rl = rl;
    io.lp = lp;
    io.wr = bwd ? wrow : nullptr;
    io.acc_dw = s0 > 0;
    io.dXc = bwd ? (char *)dX + s0 * T * H * esz : nullptr;
    st = chunk_forward(p, ws, W, ii, bwd, io, s);
    if (st != FLCE_OK) return st;
    LAUNCH(FLCE_K_PAIRS, launch_kto_seqs(lp, io.lab, ii, T, (int)kk, s0, S, kp,
                                         bwd ? wrow : nullptr, term, lpo, rwo, s));
    if (bwd) {
      st = chunk_backward(p, ws, W, ii, io, dW, sc, s);
      if (st != FLCE_OK) return st;
    }
  }
  if (refpoint)     // z0 = max(0, mean over sequences of r = S - R)
    LAUNCH(FLCE_K_PAIRS, launch_kto_refpoint(rwo, S, sc, s));
  else              // loss = mean of the terms (no NLL term)
    LAUNCH(FLCE_K_PAIRS, launch_pairs_final(term, term, S, 0.f, 1.f, sc, s));
  Scalars host;
  CK(hipMemcpyAsync(&host, sc, sizeof(host), hipMemcpyDeviceToHost, s));
  CK(hipStreamSynchronize(s));
  if (host.flag) return FLCE_ELABEL;
  *loss = host.loss;
  return FLCE_OK;
}

KtoParams kto_params(const int32_t *desirable, const float *ref, float beta, float z0,
                     float lambda_d, float lambda_u) {
  KtoParams kp{};
  kp.beta = beta;
  kp.z0 = z0;
  kp.lambda_d = lambda_d;
  kp.lambda_u = lambda_u;
  kp.desirable = desirable;
  kp.ref = ref;
  return kp;
}

}  // namespace
}  // namespace flce

FLCE_API size_t flce_kto_workspace_bytes(int64_t n_seq, int64_t T, int64_t H, int64_t V,
                                         int dtype, int64_t chunk_seqs) {
  if (flce::kto_check(n_seq, T, H, V, dtype) != FLCE_OK) return 0;
  flce::KtoLayout L;
  flce::kto_layout(n_seq, T, H, V, dtype, chunk_seqs, &L);
  return L.total;
}

FLCE_API int flce_kto_fwd_bwd(const void *X, const void *W, const int64_t *labels, int64_t n_seq,
                              int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                              const int32_t *desirable, const float *ref_logp, float beta,
                              float z0, float lambda_d, float lambda_u, int64_t chunk_seqs,
                              float *loss, void *dX, float *dW, float *logp, float *reward,
                              void *workspace, size_t workspace_bytes, void *stream) {
  return flce::run_kto(true, X, W, labels, n_seq, T, H, V, dtype, ignore_index,
                       flce::kto_params(desirable, ref_logp, beta, z0, lambda_d, lambda_u),
                       chunk_seqs, loss, dX, dW, logp, reward, workspace, workspace_bytes, stream);
}

FLCE_API int flce_kto_fwd(const void *X, const void *W, const int64_t *labels, int64_t n_seq,
                          int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                          const int32_t *desirable, const float *ref_logp, float beta, float z0,
                          float lambda_d, float lambda_u, int64_t chunk_seqs, float *loss,
                          float *logp, float *reward, void *workspace, size_t workspace_bytes,
                          void *stream) {
  return flce::run_kto(false, X, W, labels, n_seq, T, H, V, dtype, ignore_index,
                       flce::kto_params(desirable, ref_logp, beta, z0, lambda_d, lambda_u),
                       chunk_seqs, loss, nullptr, nullptr, logp, reward, workspace,
                       workspace_bytes, stream);
}

FLCE_API int flce_kto_reference_point(const void *X, const void *W, const int64_t *labels,
                                      int64_t n_seq, int64_t T, int64_t H, int64_t V, int dtype,
                                      int64_t ignore_index, const float *ref_logp,
                                      int64_t chunk_seqs, float *z0, float *logp, float *reward,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  return flce::run_kto(false, X, W, labels, n_seq, T, H, V, dtype, ignore_index,
                       flce::kto_params(nullptr, ref_logp, 0.f, 0.f, 1.f, 1.f), chunk_seqs, z0,
                       nullptr, nullptr, logp, reward, workspace, workspace_bytes, stream, true);
}

FLCE_API int flce_scale_inplace(void *buf, int64_t n, int dtype, const float *scale,
                                void *stream) {
  if (dtype != FLCE_F32 && dtype != FLCE_BF16) return FLCE_EINVAL;
  if (n < 0 || !scale || (n > 0 && !buf)) return FLCE_EINVAL;
  CK(launch_scale(buf, n, dtype, scale, (hipStream_t)stream));
  return FLCE_OK;
}

FLCE_API int flce_profile_enable(int enable) {
  prof().on.store(enable != 0);
  return FLCE_OK;
}

FLCE_API int flce_profile_select(uint32_t class_mask) {
  prof().mask.store(class_mask);
  return FLCE_OK;
}

FLCE_API int flce_profile_read(double *ms, int64_t *launches, int n) {
  Profiler &P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  for (int k = 0; k < n; ++k) {
    if (ms) ms[k] = 0.0;
    if (launches) launches[k] = 0;
  }
  int st = FLCE_OK;
  for (auto &r : P.recs) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess && st == FLCE_OK) st = hip_fail(e, "flce_profile_read");
    if (r.cls >= 0 && r.cls < n) {
      if (ms) ms[r.cls] += t;
      if (launches) launches[r.cls] += 1;
    }
    P.pool.push_back(r.a);
    P.pool.push_back(r.b);
  }
  P.recs.clear();
  return st;
}

FLCE_API const char *flce_kernel_name(int k) {
  static const char *names[FLCE_K_COUNT] = {"label_check", "fwd_tile", "lse_combine", "dlogits",
                                            "dx_gemm", "dx_reduce", "dw_gemm", "final",
                                            "pack_x", "ce_rows", "pairs",
                                            "pair_rows"};
  return (k >= 0 && k < FLCE_K_COUNT) ? names[k] : "";
}

FLCE_API const char *flce_status_string(int status) {
  switch (status) {
    case FLCE_OK: return "ok";
    case FLCE_EINVAL: return "invalid argument";
    case FLCE_ELABEL: return "label outside [0, V) that is not ignore_index";
    case FLCE_EWORKSPACE: return "workspace too small";
    case FLCE_EHIP: return "HIP runtime error";
    case FLCE_EUNSUPPORTED: return "unsupported shape or alignment";
    default: return "unknown status";
  }
}

FLCE_API const char *flce_last_error(void) { return g_last_error.c_str(); }
