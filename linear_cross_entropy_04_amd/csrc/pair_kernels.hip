// Pairwise preference losses on the fused projection: the per-pair step
// between a chunk's forward and its backward.  The project overview page
// lists fused-linear post-training losses ("Kernels de Pós-Treinamento":
// DPO, ORPO, CPO, SimPO, KTO) and calls the ORPO one as
// orpo_loss(lm_head.weight, x, target) ("Exemplo de Uso de Perda de
// Pós-Treinamento"); the pages give no formula, so each follows its published
// pairwise form.  With S = sum and a = S / n = mean of log p(y_t) over a
// sequence's n scored tokens (c: chosen, r: rejected):
//   ORPO  (Hong, Lee and Thorne, 2024)  z = log odds(a_c) - log odds(a_r),
//                                         log odds(a) = a - log(1 - e^a)
//   SimPO (Meng, Xia and Chen, 2024)    z = beta (a_c - a_r) - gamma
//   CPO   (Xu et al., 2024)             z = beta (S_c - S_r)
//   DPO   (Rafailov et al., 2023)       z = beta ((S_c - R_c) - (S_r - R_r)),
//                                         R the reference model's S (input)
//   L = alpha NLL + lambda mean over pairs of -log sigmoid(z)
// with NLL the mean of -log p over the chosen half's scored tokens, lambda =
// beta for ORPO (its weight of the odds-ratio term) and 1 otherwise.  The
// gradient reaches the logits through the per-token log-probabilities only,
// so the backward is the fused one with the per-token weight
//   w_t = -dL / d log p(y_t)
// and every GEMM of the chunk pipeline is reused unchanged.
#include "flce_internal.h"

namespace flce {
namespace {

constexpr int kPairThreads = 256;
constexpr int kMaxSegs = 4;

// One workgroup: N_c = scored tokens of the chosen half (rows < n_chosen_rows)
// and the flag for a label that is neither ignore_index nor in [0, V).
__global__ __launch_bounds__(1024) void pairs_labels_kernel(const int64_t *__restrict__ labels,
                                                           int64_t N, int64_t n_chosen_rows,
                                                           int64_t V, int64_t ii,
                                                           Scalars *__restrict__ sc) {
  __shared__ int s_cnt[16], s_bad[16];
  int cnt = 0, bad = 0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) {
    const int64_t y = labels[i];
    if (y != ii) {
      cnt += i < n_chosen_rows ? 1 : 0;
      bad |= (y < 0 || y >= V) ? 1 : 0;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    cnt += __shfl_xor(cnt, o);
    bad |= __shfl_xor(bad, o);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_cnt[w] = cnt;
    s_bad[w] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0, b = 0;
    for (int q = 0; q < 16; ++q) {
      c += s_cnt[q];
      b |= s_bad[q];
    }
    sc->nvalid = c;
    sc->inv_nvalid = 1.0f / (float)(c > 0 ? c : 1);
    sc->scale = sc->inv_nvalid;
    sc->flag = b;
    sc->loss = 0.f;
    sc->aux = 0.f;
  }
}

// Up to kMaxSegs independent copies in one launch: blockIdx.y picks the
// segment; dst[i] = src[i] for its n 4-byte words, 16 bytes per thread where
// both ends are 16-byte aligned.
struct CopySegs {
  uint32_t *dst[kMaxSegs];
  const uint32_t *src[kMaxSegs];
  int64_t n[kMaxSegs];
  int vec[kMaxSegs];
};

__global__ __launch_bounds__(256) void copy_segments_kernel(CopySegs segs) {
  const int q = blockIdx.y;
  uint32_t *__restrict__ dst = segs.dst[q];
  const uint32_t *__restrict__ src = segs.src[q];
  const int64_t n = segs.n[q];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (segs.vec[q]) {
    const int64_t n4 = n >> 2;
    for (int64_t j = i; j < n4; j += stride) ((uint4 *)dst)[j] = ((const uint4 *)src)[j];
    for (int64_t j = (n4 << 2) + i; j < n; j += stride) dst[j] = src[j];
  } else {
    for (int64_t j = i; j < n; j += stride) dst[j] = src[j];
  }
}

// Sum over a workgroup of kPairThreads; every thread gets the total.
__device__ __forceinline__ float block_sum(float v, float *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int q = 0; q < kPairThreads / 64; ++q) t += red[q];
  return t;
}

// One workgroup per pair j of a chunk of k pairs: the chosen sequence is
// chunk rows j T .. j T + T - 1, the rejected one rows k T + j T ...; lp and
// rl are the rows' log-probabilities and losses (0 on unscored rows).
__global__ __launch_bounds__(kPairThreads) void pairs_kernel(
    int kind, const float *__restrict__ lp, const float *__restrict__ rl,
    const int64_t *__restrict__ labels_c, int64_t ii, int64_t T, int k, int64_t p0,
    int64_t n_pairs, PairParams pp, const Scalars *__restrict__ sc, float *__restrict__ wrow,
    float *__restrict__ nll_sum, float *__restrict__ pair_term, float *__restrict__ chosen_logp,
    float *__restrict__ rejected_logp, float *__restrict__ pair_logit) {
  __shared__ float red[kPairThreads / 64];
  const int j = blockIdx.x;
  const int64_t rc = (int64_t)j * T, rr = (int64_t)k * T + rc;
  float sc_lp = 0.f, sc_n = 0.f, sc_rl = 0.f, sr_lp = 0.f, sr_n = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += kPairThreads) {
    if (labels_c[rc + t] != ii) {
      sc_lp += lp[rc + t];
      sc_rl += rl[rc + t];
      sc_n += 1.f;
    }
    if (labels_c[rr + t] != ii) {
      sr_lp += lp[rr + t];
      sr_n += 1.f;
    }
  }
  sc_lp = block_sum(sc_lp, red);
  sc_rl = block_sum(sc_rl, red);
  sc_n = block_sum(sc_n, red);
  sr_lp = block_sum(sr_lp, red);
  sr_n = block_sum(sr_n, red);

  const bool live = sc_n > 0.f && sr_n > 0.f;
  const float ac = sc_n > 0.f ? sc_lp / sc_n : 0.f;
  const float ar = sr_n > 0.f ? sr_lp / sr_n : 0.f;
  const bool mean_based = kind == kPairOrpo || kind == kPairSimpo;
  float z = 0.f, term = 0.f, dzc = 0.f, dzr = 0.f;
  if (live) {
    if (kind == kPairOrpo) {
      const float omc = -expm1f(ac), omr = -expm1f(ar);         // 1 - p
      z = (ac - logf(omc)) - (ar - logf(omr));
      dzc = 1.f / omc / sc_n;
      dzr = -1.f / omr / sr_n;
    } else if (kind == kPairSimpo) {
      z = pp.beta * (ac - ar) - pp.gamma;
      dzc = pp.beta / sc_n;
      dzr = -pp.beta / sr_n;
    } else {
      const float rc_ref = kind == kPairDpo ? pp.ref_c[p0 + j] : 0.f;
      const float rr_ref = kind == kPairDpo ? pp.ref_r[p0 + j] : 0.f;
      z = pp.beta * ((sc_lp - rc_ref) - (sr_lp - rr_ref));
      dzc = pp.beta;
      dzr = -pp.beta;
    }
    term = fmaxf(-z, 0.f) + log1pf(expf(-fabsf(z)));             // -log sigmoid(z)
  }
  // dL/dz = -lambda sigmoid(-z) / n_pairs
  const float g = live ? -pp.lambda / (float)n_pairs / (1.f + expf(z)) : 0.f;
  if (threadIdx.x == 0) {
    nll_sum[p0 + j] = sc_rl;
    pair_term[p0 + j] = term;
    if (chosen_logp) chosen_logp[p0 + j] = mean_based ? ac : sc_lp;
    if (rejected_logp) rejected_logp[p0 + j] = mean_based ? ar : sr_lp;
    if (pair_logit) pair_logit[p0 + j] = z;
  }
  if (wrow) {
    const float wc = pp.alpha * sc->inv_nvalid - g * dzc, wr = -g * dzr;   // w = -dL/d lp
    for (int64_t t = threadIdx.x; t < T; t += kPairThreads) {
      wrow[rc + t] = labels_c[rc + t] != ii ? wc : 0.f;
      wrow[rr + t] = labels_c[rr + t] != ii ? wr : 0.f;
    }
  }
}

// KTO (Ethayarajh et al., 2024), the unpaired loss of the same list: one
// workgroup per sequence j of a chunk (rows j T .. j T + T - 1) forms S = the
// sum of its tokens' log-probabilities, the reward r = S - R (R the
// reference model's, an input) and its loss term against the reference
// point z0 (an input taking no gradient),
//   desirable:    lambda_d (1 - sigmoid(beta (r - z0)))
//   undesirable:  lambda_u (1 - sigmoid(beta (z0 - r)))
// and every scored row's weight w = -(dl/dr) / n_seq for the backward.
__global__ __launch_bounds__(kPairThreads) void kto_seq_kernel(
    const float *__restrict__ lp, const int64_t *__restrict__ labels_c, int64_t ii, int64_t T,
    int64_t s0, int64_t n_seq, KtoParams kp, float *__restrict__ wrow, float *__restrict__ term,
    float *__restrict__ logp, float *__restrict__ reward) {
  __shared__ float red[kPairThreads / 64];
  const int j = blockIdx.x;
  const int64_t r0 = (int64_t)j * T;
  float sum = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += kPairThreads)
    if (labels_c[r0 + t] != ii) sum += lp[r0 + t];
  const float S = block_sum(sum, red);
  const float r = S - kp.ref[s0 + j];
  const bool des = kp.desirable ? kp.desirable[s0 + j] != 0 : true;
  const float u = des ? kp.beta * (r - kp.z0) : kp.beta * (kp.z0 - r);
  // sigmoid(u) and 1 - sigmoid(u) = sigmoid(-u), each from its own exp so
  // that neither loses its digits when the other rounds to 1
  const float sg = 1.f / (1.f + expf(-u)), sgn = 1.f / (1.f + expf(u));
  const float lam = des ? kp.lambda_d : kp.lambda_u;
  const float dl_dr = -lam * sg * sgn * (des ? kp.beta : -kp.beta);
  if (threadIdx.x == 0) {
    term[s0 + j] = lam * sgn;
    if (logp) logp[s0 + j] = S;
    if (reward) reward[s0 + j] = r;
  }
  if (wrow) {
    const float w = -dl_dr / (float)n_seq;
    for (int64_t t = threadIdx.x; t < T; t += kPairThreads)
      wrow[r0 + t] = labels_c[r0 + t] != ii ? w : 0.f;
  }
}

// loss = alpha (sum of the chosen tokens' losses) / N_c + lambda mean_i of
// the pair terms; aux = the NLL.  One workgroup; fixed summation order.
__global__ __launch_bounds__(256) void pairs_final_kernel(const float *__restrict__ nll_sum,
                                                          const float *__restrict__ or_term,
                                                          int64_t n_pairs, float alpha,
                                                          float lambda,
                                                          Scalars *__restrict__ sc) {
  __shared__ float red[4];
  float a = 0.f, b = 0.f;
  for (int64_t i = threadIdx.x; i < n_pairs; i += 256) {
    a += nll_sum[i];
    b += or_term[i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
  __shared__ float red2[4];
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = a;
    red2[threadIdx.x >> 6] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float nll = (red[0] + red[1] + red[2] + red[3]) * sc->inv_nvalid;
    const float orl = (red2[0] + red2[1] + red2[2] + red2[3]) / (float)n_pairs;
    sc->aux = nll;
    sc->loss = alpha * nll + lambda * orl;
  }
}

// KTO's reference point from the per-sequence rewards r = S - R of a batch of
// mismatched completions: z0 = max(0, mean r), summed in fp64 in a fixed
// order; the result goes to sc->loss, the call's scalar output.
__global__ __launch_bounds__(256) void kto_refpoint_kernel(const float *__restrict__ r,
                                                           int64_t n, Scalars *__restrict__ sc) {
  __shared__ double part[256];
  double a = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) a += (double)r[i];
  part[threadIdx.x] = a;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double m = part[0] / (double)(n > 0 ? n : 1);
    sc->loss = (float)(m > 0.0 ? m : 0.0);
  }
}

}  // namespace

hipError_t launch_pairs_labels(const int64_t *labels, int64_t N, int64_t n_chosen_rows, int64_t V,
                              int64_t ii, Scalars *sc, hipStream_t s) {
  hipLaunchKernelGGL(pairs_labels_kernel, dim3(1), dim3(1024), 0, s, labels, N, n_chosen_rows, V,
                     ii, sc);
  return hipGetLastError();
}

hipError_t launch_copy_segments(const CopySeg *segs, int nseg, hipStream_t s) {
  if (nseg <= 0 || nseg > kMaxSegs) return hipErrorInvalidValue;
  CopySegs a = {};
  int64_t most = 0;
  for (int q = 0; q < nseg; ++q) {
    a.dst[q] = (uint32_t *)segs[q].dst;
    a.src[q] = (const uint32_t *)segs[q].src;
    a.n[q] = segs[q].bytes / 4;                  // every caller copies whole 4-byte words
    a.vec[q] = ((uintptr_t)segs[q].dst % 16 == 0 && (uintptr_t)segs[q].src % 16 == 0) ? 1 : 0;
    const int64_t work = a.vec[q] ? (a.n[q] + 3) / 4 : a.n[q];
    most = work > most ? work : most;
  }
  if (most == 0) return hipSuccess;
  int64_t g = (most + 255) / 256;
  if (g > 2048) g = 2048;
  hipLaunchKernelGGL(copy_segments_kernel, dim3((unsigned)g, (unsigned)nseg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pairs(int kind, const float *lp, const float *rl, const int64_t *labels_c,
                        int64_t ii, int64_t T, int k, int64_t p0, int64_t n_pairs,
                        const PairParams &pp, const Scalars *sc, float *wrow, float *nll_sum,
                        float *pair_term, float *chosen_logp, float *rejected_logp,
                        float *pair_logit, hipStream_t s) {
  if (k <= 0) return hipSuccess;
  hipLaunchKernelGGL(pairs_kernel, dim3((unsigned)k), dim3(kPairThreads), 0, s, kind, lp, rl,
                     labels_c, ii, T, k, p0, n_pairs, pp, sc, wrow, nll_sum, pair_term,
                     chosen_logp, rejected_logp, pair_logit);
  return hipGetLastError();
}

hipError_t launch_kto_seqs(const float *lp, const int64_t *labels_c, int64_t ii, int64_t T,
                          int k, int64_t s0, int64_t n_seq, const KtoParams &kp, float *wrow,
                          float *term, float *logp, float *reward, hipStream_t s) {
  if (k <= 0) return hipSuccess;
  hipLaunchKernelGGL(kto_seq_kernel, dim3((unsigned)k), dim3(kPairThreads), 0, s, lp, labels_c,
                     ii, T, s0, n_seq, kp, wrow, term, logp, reward);
  return hipGetLastError();
}

hipError_t launch_pairs_final(const float *nll_sum, const float *pair_term, int64_t n_pairs,
                              float alpha, float lambda, Scalars *sc, hipStream_t s) {
  hipLaunchKernelGGL(pairs_final_kernel, dim3(1), dim3(256), 0, s, nll_sum, pair_term, n_pairs,
                     alpha, lambda, sc);
  return hipGetLastError();
}

hipError_t launch_kto_refpoint(const float *reward, int64_t n_seq, Scalars *sc, hipStream_t s) {
  hipLaunchKernelGGL(kto_refpoint_kernel, dim3(1), dim3(256), 0, s, reward, n_seq, sc);
  return hipGetLastError();
}

}  // namespace flce
