// Small kernels shared by both precisions: the label pre-pass, the
// log-sum-exp combine over vocabulary tiles, the final loss, fills, scaling.
// All reductions use a fixed order, so results are bitwise reproducible.
#include "flce_internal.h"

namespace flce {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// N_valid = #{i : y_i != ii}; flag if a valid label lies outside [0, V).
// One workgroup of 1024 threads.
// scale = the weight of each valid token's loss: 1 / max(N_valid, 1) for the
// mean, 1 for the sum (and for per-token losses without upstream weights).
__global__ __launch_bounds__(1024) void label_check_kernel(const int64_t *__restrict__ labels,
                                                           int64_t N, int64_t V, int64_t ii,
                                                           int reduction,
                                                           Scalars *__restrict__ sc) {
  __shared__ int s_cnt[16], s_bad[16];
  int cnt = 0, bad = 0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) {
    const int64_t y = labels[i];
    if (y != ii) {
      ++cnt;
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
    sc->scale = reduction == kReduceMean ? sc->inv_nvalid : 1.0f;
    sc->flag = b;
    sc->loss = 0.f;
  }
}

// Merge two (max, sum) pairs; a side whose max is -inf holds a sum of 0 and
// must not contribute exp(nan).
__device__ __forceinline__ void lse_merge(float &M, float &S, float Mo, float So) {
  const float Mn = fmaxf(M, Mo);
  const float a = M > -INFINITY ? __builtin_amdgcn_exp2f((M - Mn) * kLog2e) : 0.f;
  const float b = Mo > -INFINITY ? __builtin_amdgcn_exp2f((Mo - Mn) * kLog2e) : 0.f;
  S = S * a + So * b;
  M = Mn;
}

// One workgroup of 256 threads per token: lse = M + ln sum_t s_t exp(m_t - M)
// over the token's vocabulary-tile partials (m_t = tile max, s_t = sum of
// exp(z - m_t)); the token's loss lse - z_y and, if asked, its
// log-probability z_y - lse (both 0 on ignored tokens).  One pass: each
// thread keeps a running (max, sum) over its partials, rescaling the sum when
// the max grows; threads then merge within the wave, and the four waves
// through LDS.  A partial with m = -inf (vocabulary ids past V) has s = 0 and
// adds nothing; a NaN partial still reaches the sum.
constexpr int kLseThreads = 256;

__global__ __launch_bounds__(kLseThreads) void lse_combine_kernel(
    const float *__restrict__ pm, const float *__restrict__ ps, const float *__restrict__ zy,
    const int64_t *__restrict__ labels_c, int64_t ii, int c, int64_t nvt, float *__restrict__ lse_c,
    float *__restrict__ rowloss_c, float *__restrict__ rowlse_c, float *__restrict__ logprob_c) {
  __shared__ float wm[kLseThreads / 64], wsum[kLseThreads / 64];
  const int tok = blockIdx.x;
  const float *m = pm + (int64_t)tok * nvt;
  const float *s = ps + (int64_t)tok * nvt;
  float M = -INFINITY, S = 0.f;
#pragma unroll 4
  for (int64_t t = threadIdx.x; t < nvt; t += kLseThreads) {
    const float mt = m[t], st = s[t];
    if (mt > M) {
      S = S * __builtin_amdgcn_exp2f((M - mt) * kLog2e) + st;
      M = mt;
    } else if (!(mt == -INFINITY)) {
      S += st * __builtin_amdgcn_exp2f((mt - M) * kLog2e);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lse_merge(M, S, __shfl_xor(M, o), __shfl_xor(S, o));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    wm[w] = M;
    wsum[w] = S;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 1; k < kLseThreads / 64; ++k) lse_merge(M, S, wm[k], wsum[k]);
    const float lse = M + __builtin_amdgcn_logf(S) * kLn2;
    const int64_t y = labels_c[tok];
    lse_c[tok] = lse;
    rowloss_c[tok] = (y != ii) ? lse - zy[tok] : 0.f;
    if (rowlse_c) rowlse_c[tok] = lse;
    if (logprob_c) logprob_c[tok] = (y != ii) ? zy[tok] - lse : 0.f;
  }
}

// loss = sum_i rowloss_i, divided by max(N_valid, 1) for the mean; summed in
// fp64 in a fixed tree.
__global__ __launch_bounds__(1024) void final_loss_kernel(const float *__restrict__ rowloss,
                                                          int64_t N, int reduction,
                                                          Scalars *__restrict__ sc) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < N; i += 1024) acc += (double)rowloss[i];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int nv = sc->nvalid;
    sc->loss = reduction == kReduceMean ? (float)(part[0] / (double)(nv > 0 ? nv : 1))
                                        : (float)part[0];
  }
}

__global__ void fill_f32_kernel(float *__restrict__ p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void scale_f32_kernel(float *__restrict__ p, int64_t n, const float *__restrict__ sc) {
  const float a = *sc;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] *= a;
}

__global__ void scale_bf16_kernel(uint16_t *__restrict__ p, int64_t n, const float *__restrict__ sc) {
  const float a = *sc;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float x = __builtin_bit_cast(float, (uint32_t)p[i] << 16) * a;
    p[i] = __builtin_bit_cast(uint16_t, (__bf16)x);
  }
}

inline int grid_for(int64_t n, int block, int cap) {
  int64_t g = (n + block - 1) / block;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace

hipError_t launch_label_check(const int64_t *labels, int64_t N, int64_t V, int64_t ii,
                              int reduction, Scalars *sc, hipStream_t s) {
  hipLaunchKernelGGL(label_check_kernel, dim3(1), dim3(1024), 0, s, labels, N, V, ii, reduction,
                     sc);
  return hipGetLastError();
}

hipError_t launch_lse_combine(const float *pm, const float *ps, const float *zy,
                              const int64_t *labels_c, int64_t ii, int c, int64_t nvt,
                              float *lse_c, float *rowloss_c, float *rowlse_c,
                              float *logprob_c, hipStream_t s) {
  if (c <= 0) return hipSuccess;
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)c), dim3(kLseThreads), 0, s, pm, ps, zy,
                     labels_c, ii, c, nvt, lse_c, rowloss_c, rowlse_c, logprob_c);
  return hipGetLastError();
}

hipError_t launch_final_loss(const float *rowloss, int64_t N, int reduction, Scalars *sc,
                             hipStream_t s) {
  hipLaunchKernelGGL(final_loss_kernel, dim3(1), dim3(1024), 0, s, rowloss, N, reduction, sc);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n, 256, 256 * 64)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_scale(void *buf, int64_t n, int dtype, const float *scale, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int g = grid_for(n, 256, 256 * 64);
  if (dtype == 0)
    hipLaunchKernelGGL(scale_f32_kernel, dim3(g), dim3(256), 0, s, (float *)buf, n, scale);
  else
    hipLaunchKernelGGL(scale_bf16_kernel, dim3(g), dim3(256), 0, s, (uint16_t *)buf, n, scale);
  return hipGetLastError();
}

}  // namespace flce
