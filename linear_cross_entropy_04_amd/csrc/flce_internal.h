// Internal declarations of libflce: the chunk plan and the kernel launchers.
// Not part of the ABI (see include/flce.h for that).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace flce {

// Vocabulary width of one log-sum-exp partial: 128 on the bf16 MFMA path (one
// wave's half of a 256-row workgroup tile; 2 per tile), 64 on the fp32 path.
constexpr int kTileVBf16 = 256;
constexpr int kTileVF32 = 64;
constexpr int kMaxSplitK = 32;

// Device-side scalars kept in the workspace.  loss and flag sit first so a
// single 8-byte copy returns both to the host.
struct Scalars {
  float loss;        // final loss (mean, or sum of the per-token losses)
  int flag;          // 1 if a label was neither ignore_index nor in [0, V)
  int nvalid;        // number of non-ignored labels
  float inv_nvalid;  // 1 / max(nvalid, 1)
  float scale;       // weight of a valid token's loss: 1 / max(nvalid, 1) for the mean, else 1
  float aux;         // a second result of the call (the preference loss: its NLL term)
};

// Reductions of the per-token losses (values of flce_reduction).
constexpr int kReduceMean = 0, kReduceSum = 1, kReduceNone = 2;

// Sizes and workspace layout of one call.
struct Plan {
  int dtype = 0;
  int64_t N = 0, H = 0, V = 0;
  int64_t C = 0;        // tokens per chunk (last chunk may be shorter)
  int64_t ldz = 0;      // fp32 path: leading dimension (elements) of the chunk logits scratch
  int64_t nks_z = 0, nks_h = 0;   // bf16 path: 32-column slices of V and H, padded to 256
  int64_t nks_c = 0;    // bf16 path: 32-column slices of the chunk's tokens, padded to 256
  int64_t nvt = 0;      // vocabulary tiles = log-sum-exp partials per token
  int splitk = 0;       // K-splits of the dX GEMM (0: the fp32 path writes dX directly)
  int64_t ksplit = 0;   // vocabulary rows per split (multiple of 64)
  size_t off_z = 0, off_xp = 0, off_pm = 0, off_ps = 0, off_zy = 0, off_lse = 0,
         off_rowloss = 0, off_dxp = 0, off_scal = 0, total = 0;
  size_t off_pmt = 0;   // bf16 path: the partial maxima again, [partial][token]
  size_t off_xpt = 0;   // bf16 path: the chunk's X transposed and packed (rows = hidden) for dW
};

// Fill *p for the given sizes and chunk (C >= 1, C <= N or N == 0).
void make_plan(int64_t N, int64_t H, int64_t V, int dtype, int64_t C, Plan *p);
// Number of dX K-splits chosen for a chunk of C tokens.
int choose_splitk(int64_t C, int64_t H, int64_t V);

// ---------------------------------------------------------------- common kernels
hipError_t launch_label_check(const int64_t *labels, int64_t N, int64_t V, int64_t ii,
                              int reduction, Scalars *sc, hipStream_t s);
hipError_t launch_lse_combine(const float *pm, const float *ps, const float *zy,
                              const int64_t *labels_c, int64_t ii, int c, int64_t nvt,
                              float *lse_c, float *rowloss_c, float *rowlse_c,
                              float *logprob_c, hipStream_t s);
hipError_t launch_final_loss(const float *rowloss, int64_t N, int reduction, Scalars *sc,
                             hipStream_t s);
hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t s);
hipError_t launch_scale(void *buf, int64_t n, int dtype, const float *scale, hipStream_t s);

// ---------------------------------------------------------------- bf16 path (MFMA)
// Packed matrices (Xp, Zp) are 16 KB blocks of 256 rows x 32 columns; a
// matrix with nks column slices (nks a multiple of 8) stores row tile rt,
// slice ks at element (rt * nks + ks) * 8192.  Each GEMM reads them either
// along their rows or transposed, so no transposed copy is ever made.  W is
// read where it lies, row-major [V][H], along its rows by the forward and
// transposed by dX.
// Pack a row-major [R][K] matrix into P (rows R padded to 256, nks_p slices)
// and, if PT is not null, its transpose into PT (K rows padded to 256, nks_t
// slices of the R columns), in one launch.
hipError_t launch_pack_bf16(const uint16_t *src, int R, int K, uint16_t *P, int64_t nks_p,
                            uint16_t *PT, int64_t nks_t, hipStream_t s);
// Logits tile GEMM with the log-sum-exp epilogue.  pm, ps: [token][partial]
// maximum and sum of exp per 128 vocabulary ids; with store_z, Zp receives
// bf16((z - m) log2 e) for the partial's maximum m, and pmt[partial * c +
// token] the m that was subtracted.
hipError_t launch_fwd_tile_bf16(const uint16_t *W, const uint16_t *Xp,
                                const int64_t *labels_c, int64_t ii, int c, int H, int V,
                                uint16_t *Zp, int64_t nks_z, float *pm, float *ps, float *pmt,
                                float *zy, int64_t nvt, bool store_z, hipStream_t s);
// G in place over the stored bf16((z - m) log2 e), with m from pmt.
// wrow_c (may be null): per-token weight of the loss (the upstream gradient
// of a per-token loss vector); null: sc->scale for every valid token.
hipError_t launch_dlogits_bf16(uint16_t *Zp, int64_t nks_z, int c, int V, const float *pmt,
                               const float *lse_c, const int64_t *labels_c, int64_t ii,
                               const float *wrow_c, const Scalars *sc, hipStream_t s);
// dX partials from G (Zp) and W (row-major [V][H]) read transposed.
hipError_t launch_dx_bf16(const uint16_t *Gp, int64_t nks_z, const uint16_t *W,
                          int c, int H, int V, int splitk, int64_t ksplit, float *dxp,
                          hipStream_t s);
hipError_t launch_dx_reduce_bf16(const float *dxp, int splitk, int c, int H, uint16_t *dXc,
                                 hipStream_t s);
// dW (+)= G^T X_c with G from Zp (read transposed) and X_c^T packed (XpT,
// rows = hidden, nks_c slices of the tokens).
hipError_t launch_dw_bf16(const uint16_t *Gp, int64_t nks_z, const uint16_t *XpT, int64_t nks_c,
                          int c, int H, int V, float *dW, bool accumulate, hipStream_t s);

// ---------------------------------------------------------------- cross-entropy on given logits
// One workgroup per row of logits [N][V] (dtype 0 = fp32, 1 = bf16): lse,
// per-token loss / log-sum-exp / log-probability (each may be null), and with
// grad the gradient written over the row (wrow: per-token weights or null).
hipError_t launch_ce_rows(void *logits, int64_t N, int64_t V, int dtype, const int64_t *labels,
                          int64_t ii, bool grad, const float *wrow, const Scalars *sc,
                          float *row_loss, float *row_lse, float *logprob, hipStream_t s);

// ---------------------------------------------------------------- pairwise preference losses
// Kinds (values of flce_pair_loss).
constexpr int kPairOrpo = 0, kPairSimpo = 1, kPairCpo = 2, kPairDpo = 3;
struct PairParams {
  float beta, gamma, alpha, lambda;   // lambda: weight of the pair term (beta for ORPO, else 1)
  const float *ref_c, *ref_r;         // DPO: the reference model's sequence log-probabilities
};
// Label pass: N_c = scored tokens among rows < n_chosen_rows, label flag.
hipError_t launch_pairs_labels(const int64_t *labels, int64_t N, int64_t n_chosen_rows, int64_t V,
                               int64_t ii, Scalars *sc, hipStream_t s);
// Up to 4 device copies of whole numbers of 4-byte words, in one launch.
struct CopySeg {
  void *dst;
  const void *src;
  int64_t bytes;
};
hipError_t launch_copy_segments(const CopySeg *segs, int nseg, hipStream_t s);
// Per pair of a chunk of k pairs (chosen rows first, then rejected, T rows
// each): the sequence log-probabilities the loss uses, the pair logit z, the
// pair's NLL sum and pair term at pair p0 + j, and (wrow not null) the
// per-row weights w = -dL/dlogp of the backward.
hipError_t launch_pairs(int kind, const float *lp, const float *rl, const int64_t *labels_c,
                        int64_t ii, int64_t T, int k, int64_t p0, int64_t n_pairs,
                        const PairParams &pp, const Scalars *sc, float *wrow, float *nll_sum,
                        float *pair_term, float *chosen_logp, float *rejected_logp,
                        float *pair_logit, hipStream_t s);
// KTO: per sequence of a chunk of k sequences (T rows each): S, r = S - R, the
// loss term at s0 + j and (wrow not null) the per-row backward weights.
struct KtoParams {
  float beta, z0, lambda_d, lambda_u;
  const int32_t *desirable;   // [n_seq], nonzero: desirable (null: all desirable)
  const float *ref;           // [n_seq] the reference model's S
};
hipError_t launch_kto_seqs(const float *lp, const int64_t *labels_c, int64_t ii, int64_t T,
                          int k, int64_t s0, int64_t n_seq, const KtoParams &kp, float *wrow,
                          float *term, float *logp, float *reward, hipStream_t s);
// sc->loss = max(0, mean of the n_seq rewards): KTO's reference point.
hipError_t launch_kto_refpoint(const float *reward, int64_t n_seq, Scalars *sc, hipStream_t s);
// sc->loss = alpha NLL + lambda mean pair term, sc->aux = NLL.
hipError_t launch_pairs_final(const float *nll_sum, const float *pair_term, int64_t n_pairs,
                              float alpha, float lambda, Scalars *sc, hipStream_t s);

// ---------------------------------------------------------------- fp32 path (SIMT)
hipError_t launch_fwd_tile_f32(const float *W, const float *Xc, const int64_t *labels_c,
                               int64_t ii, int c, int H, int V, float *zbuf, int64_t ldz,
                               float *pm, float *ps, float *zy, int64_t nvt, bool store_z,
                               hipStream_t s);
hipError_t launch_dlogits_f32(float *zbuf, int64_t ldz, int c, int V, const float *lse_c,
                              const int64_t *labels_c, int64_t ii, const float *wrow_c,
                              const Scalars *sc, hipStream_t s);
hipError_t launch_dx_f32(const float *G, int64_t ldz, const float *W, int c, int H, int V,
                         float *dXc, hipStream_t s);
hipError_t launch_dw_f32(const float *G, int64_t ldz, const float *Xc, int c, int H, int V,
                         float *dW, bool accumulate, hipStream_t s);

}  // namespace flce
