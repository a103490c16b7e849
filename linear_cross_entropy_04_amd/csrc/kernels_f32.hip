// fp32 path of the chunked fused linear cross-entropy: the same five steps as
// the bf16 path (forward tile with log-sum-exp partials, combine, in-place
// dlogits, dX, dW) with fp32 operands, fp32 scratch and FMA arithmetic.  It
// serves fp32 callers and small shapes; every value stays fp32 end to end.
//
// GEMM tiles are 64 x 64 per 256-thread workgroup (4 x 4 outputs per thread),
// K staged through LDS 16 deep.  Operand element (r, k) is base[r*sr + k*sk].
#include "flce_internal.h"

namespace flce {
namespace {

constexpr int T = 64, TK = 16;
constexpr float kLog2e = 1.4426950408889634f;

struct OpF {
  const float *base;
  int64_t sr, sk;
  int rows;
};

__device__ __forceinline__ void simt_tile(const OpF a, const OpF b, int m0, int n0, int64_t kb,
                                          int64_t ke, float (&acc)[4][4],
                                          float (*sA)[T], float (*sB)[T]) {
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int64_t k0 = kb; k0 < ke; k0 += TK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = t + 256 * q, r = e & 63, kk = e >> 6;
      const int64_t gk = k0 + kk;
      const int ra = m0 + r, rb = n0 + r;
      sA[kk][r] = (ra < a.rows && gk < ke) ? a.base[(int64_t)ra * a.sr + gk * a.sk] : 0.f;
      sB[kk][r] = (rb < b.rows && gk < ke) ? b.base[(int64_t)rb * b.sr + gk * b.sk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
}

// Z^T tile: rows = 64 vocabulary ids from m0, columns = 64 tokens from n0.
__global__ __launch_bounds__(256) void fwd_tile_f32_kernel(
    const float *__restrict__ W, const float *__restrict__ Xc, const int64_t *__restrict__ labels_c,
    int64_t ii, int c, int H, int V, float *__restrict__ zbuf, int64_t ldz, float *__restrict__ pm,
    float *__restrict__ ps, float *__restrict__ zy, int64_t nvt, int nct, int store_z) {
  __shared__ float sA[TK][T], sB[TK][T];
  __shared__ float red[16][T];
  const int vt = blockIdx.x / nct, ct = blockIdx.x - vt * nct;
  const int m0 = vt * T, n0 = ct * T;
  float acc[4][4];
  simt_tile(OpF{W, H, 1, V}, OpF{Xc, H, 1, c}, m0, n0, 0, H, acc, sA, sB);

  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  // column max over the tile's 64 vocabulary rows
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (m0 + ty * 4 + i < V) mx = fmaxf(mx, acc[i][j]);
    red[ty][tx * 4 + j] = mx;
  }
  __syncthreads();
  float cm[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float mx = -INFINITY;
    for (int q = 0; q < 16; ++q) mx = fmaxf(mx, red[q][tx * 4 + j]);
    cm[j] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = n0 + tx * 4 + j;
    const int64_t y = tok < c ? labels_c[tok] : ii;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = m0 + ty * 4 + i;
      if (v < V) {
        s += __builtin_amdgcn_exp2f((acc[i][j] - cm[j]) * kLog2e);
        if ((int64_t)v == y && tok < c) zy[tok] = acc[i][j];
        if (store_z && tok < c) zbuf[(int64_t)tok * ldz + v] = acc[i][j];
      }
    }
    red[ty][tx * 4 + j] = s;
  }
  __syncthreads();
  if (t < T) {
    const int tok = n0 + t;
    if (tok < c) {
      float s = 0.f;
      for (int q = 0; q < 16; ++q) s += red[q][t];
      ps[(int64_t)tok * nvt + vt] = s;
    }
  }
  if (ty == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = n0 + tx * 4 + j;
      if (tok < c) pm[(int64_t)tok * nvt + vt] = cm[j];
    }
  }
}

// dXc[tok][h] = sum_v G[tok][v] W[v][h], written directly (fp32).
__global__ __launch_bounds__(256) void dx_f32_kernel(const float *__restrict__ G, int64_t ldz,
                                                     const float *__restrict__ W, int c, int H,
                                                     int V, int nht, float *__restrict__ dXc) {
  __shared__ float sA[TK][T], sB[TK][T];
  const int mt = blockIdx.x / nht, ht = blockIdx.x - mt * nht;
  const int m0 = mt * T, n0 = ht * T;
  float acc[4][4];
  simt_tile(OpF{G, ldz, 1, c}, OpF{W, 1, H, H}, m0, n0, 0, V, acc, sA, sB);
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = m0 + ty * 4 + i, h = n0 + tx * 4 + j;
      if (tok < c && h < H) dXc[(int64_t)tok * H + h] = acc[i][j];
    }
}

// dW[v][h] (+)= sum_tok G[tok][v] X[tok][h].
__global__ __launch_bounds__(256) void dw_f32_kernel(const float *__restrict__ G, int64_t ldz,
                                                     const float *__restrict__ Xc, int c, int H,
                                                     int V, int nht, float *__restrict__ dW,
                                                     int accumulate) {
  __shared__ float sA[TK][T], sB[TK][T];
  const int vt = blockIdx.x / nht, ht = blockIdx.x - vt * nht;
  const int m0 = vt * T, n0 = ht * T;
  float acc[4][4];
  simt_tile(OpF{G, 1, ldz, V}, OpF{Xc, 1, H, H}, m0, n0, 0, c, acc, sA, sB);
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = m0 + ty * 4 + i, h = n0 + tx * 4 + j;
      if (v < V && h < H) {
        float *p = dW + (int64_t)v * H + h;
        *p = accumulate ? *p + acc[i][j] : acc[i][j];
      }
    }
}

// G = w_r (exp(Z - lse) - onehot(y)) in place, w_r = wrow_c[r] if given, else
// sc->scale; 0 on ignored rows and padding.
__global__ void dlogits_f32_kernel(float *__restrict__ z, int64_t ldz, int c, int V,
                                   const float *__restrict__ lse_c,
                                   const int64_t *__restrict__ labels_c, int64_t ii,
                                   const float *__restrict__ wrow_c,
                                   const Scalars *__restrict__ sc) {
  const int64_t n = (int64_t)c * ldz;
  const float scale = sc->scale;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / ldz;
    const int v = (int)(i - r * ldz);
    const int64_t y = labels_c[r];
    float g = 0.f;
    if (y != ii && v < V)
      g = (__builtin_amdgcn_exp2f((z[i] - lse_c[r]) * kLog2e) - ((int64_t)v == y ? 1.f : 0.f)) *
          (wrow_c ? wrow_c[r] : scale);
    z[i] = g;
  }
}

}  // namespace

hipError_t launch_fwd_tile_f32(const float *W, const float *Xc, const int64_t *labels_c,
                               int64_t ii, int c, int H, int V, float *zbuf, int64_t ldz,
                               float *pm, float *ps, float *zy, int64_t nvt, bool store_z,
                               hipStream_t s) {
  const int nct = (c + T - 1) / T;
  hipLaunchKernelGGL(fwd_tile_f32_kernel, dim3((int)nvt * nct), dim3(256), 0, s, W, Xc, labels_c,
                     ii, c, H, V, zbuf, ldz, pm, ps, zy, nvt, nct, store_z ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_dlogits_f32(float *zbuf, int64_t ldz, int c, int V, const float *lse_c,
                              const int64_t *labels_c, int64_t ii, const float *wrow_c,
                              const Scalars *sc, hipStream_t s) {
  const int64_t n = (int64_t)c * ldz;
  int64_t g = (n + 255) / 256;
  if (g > 256 * 64) g = 256 * 64;
  hipLaunchKernelGGL(dlogits_f32_kernel, dim3((int)g), dim3(256), 0, s, zbuf, ldz, c, V, lse_c,
                     labels_c, ii, wrow_c, sc);
  return hipGetLastError();
}

hipError_t launch_dx_f32(const float *G, int64_t ldz, const float *W, int c, int H, int V,
                         float *dXc, hipStream_t s) {
  const int nmt = (c + T - 1) / T, nht = (H + T - 1) / T;
  hipLaunchKernelGGL(dx_f32_kernel, dim3(nmt * nht), dim3(256), 0, s, G, ldz, W, c, H, V, nht, dXc);
  return hipGetLastError();
}

hipError_t launch_dw_f32(const float *G, int64_t ldz, const float *Xc, int c, int H, int V,
                         float *dW, bool accumulate, hipStream_t s) {
  const int nvt = (V + T - 1) / T, nht = (H + T - 1) / T;
  hipLaunchKernelGGL(dw_f32_kernel, dim3(nvt * nht), dim3(256), 0, s, G, ldz, Xc, c, H, V, nht, dW,
                     accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace flce
