// Cross-entropy on given logits (no projection): the loss the Liger Kernel
// pages list beside the fused one (project overview page, "Modelos e
// Operações": the plain cross-entropy loss), with its gradient written over
// the logits in place (overview page, "Princípios Técnicos", in-place
// operations).
//
// One workgroup of 1024 threads per logits row.  Pass 1 reads the row once
// with 16-byte loads and keeps, per thread, an online maximum and sum of
// exp(z - max) (rescaled when the maximum grows); the workgroup combines the
// 1024 pairs into lse = M + ln S and takes the target logit.  Pass 2 (with
// gradients) reads the row again and writes w_r (exp(z - lse) - onehot(y))
// in place, w_r the token's weight (1/N_valid for the mean, 1 for the sum,
// the upstream gradient for per-token losses) and 0 on ignored rows.
#include "flce_internal.h"

namespace flce {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = 1024;          // a row finishes sooner, so its second read hits in cache

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __builtin_bit_cast(float, (uint32_t)u << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Elements of a row as floats: E = elements per 16-byte vector.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ float get(const float *p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void put(float *p, int64_t i, float v) { p[i] = v; }
  static __device__ __forceinline__ void load(const float *p, float (&v)[4]) {
    const f32x4 x = *(const f32x4 *)p;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x[e];
  }
  static __device__ __forceinline__ void store(float *p, const float (&v)[4]) {
    *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int E = 8;
  static __device__ __forceinline__ float get(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ void put(uint16_t *p, int64_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
  static __device__ __forceinline__ void load(const uint16_t *p, float (&v)[8]) {
    const u32x4 x = *(const u32x4 *)p;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v[2 * d] = __builtin_bit_cast(float, x[d] << 16);
      v[2 * d + 1] = __builtin_bit_cast(float, x[d] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t *p, const float (&v)[8]) {
    u32x4 x;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      x[d] = (uint32_t)f32_to_bf16(v[2 * d]) | ((uint32_t)f32_to_bf16(v[2 * d + 1]) << 16);
    *(u32x4 *)p = x;
  }
};

// (m, s) <- (m, s) merged with (m2, s2): one online-softmax pair.
__device__ __forceinline__ void merge(float &m, float &s, float m2, float s2) {
  const float mx = fmaxf(m, m2);
  if (mx == -INFINITY) return;                      // both empty
  s = s * __builtin_amdgcn_exp2f((m - mx) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mx) * kLog2e);
  m = mx;
}

// VEC: the buffer is 16-byte aligned and the row length a multiple of the
// vector width, so every row starts 16-byte aligned; otherwise one element
// at a time.
template <typename T, bool VEC, bool GRAD>
__global__ __launch_bounds__(kThreads) void ce_row_kernel(
    T *__restrict__ logits, int64_t V, const int64_t *__restrict__ labels, int64_t ii,
    const float *__restrict__ wrow, const Scalars *__restrict__ sc, float *__restrict__ row_loss,
    float *__restrict__ row_lse, float *__restrict__ logprob) {
  using El = Elem<T>;
  constexpr int E = El::E;
  __shared__ float s_m[kThreads / 64], s_s[kThreads / 64], s_lse;
  const int64_t r = blockIdx.x;
  T *row = logits + r * V;
  const int t = threadIdx.x;

  // pass 1: online maximum and sum of exp per thread
  float m = -INFINITY, s = 0.f;
  if constexpr (VEC) {
    for (int64_t i = (int64_t)t * E; i < V; i += (int64_t)kThreads * E) {
      float v[E];
      El::load(row + i, v);
      float mx = v[0];
#pragma unroll
      for (int e = 1; e < E; ++e) mx = fmaxf(mx, v[e]);
      const float mn = fmaxf(m, mx);
      if (mn == -INFINITY) continue;               // masked (-inf) logits so far
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc += __builtin_amdgcn_exp2f((v[e] - mn) * kLog2e);
      s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - mn) * kLog2e)) + acc;
      m = mn;
    }
  } else {
    for (int64_t i = t; i < V; i += kThreads) merge(m, s, El::get(row, i), 1.f);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    merge(m, s, m2, s2);
  }
  if ((t & 63) == 0) {
    s_m[t >> 6] = m;
    s_s[t >> 6] = s;
  }
  __syncthreads();
  const int64_t y = labels[r];
  const bool valid = y != ii;
  if (t == 0) {
    float M = s_m[0], S = s_s[0];
    for (int q = 1; q < kThreads / 64; ++q) merge(M, S, s_m[q], s_s[q]);
    const float lse = M + __builtin_amdgcn_logf(S) * kLn2;
    s_lse = lse;
    // a valid label outside [0, V) is reported by the label pass; read nothing then
    const float zy = (valid && y >= 0 && y < V) ? El::get(row, y) : 0.f;
    if (row_loss) row_loss[r] = valid ? lse - zy : 0.f;
    if (row_lse) row_lse[r] = lse;
    if (logprob) logprob[r] = valid ? zy - lse : 0.f;
  }
  if constexpr (GRAD) {
    __syncthreads();                               // every thread has read the row; lse is known
    const float l2 = s_lse * kLog2e;
    const float w = valid ? (wrow ? wrow[r] : sc->scale) : 0.f;
    if constexpr (VEC) {
      for (int64_t i = (int64_t)t * E; i < V; i += (int64_t)kThreads * E) {
        float v[E];
        El::load(row + i, v);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float g = __builtin_amdgcn_exp2f(v[e] * kLog2e - l2) - (i + e == y ? 1.f : 0.f);
          v[e] = valid ? g * w : 0.f;
        }
        El::store(row + i, v);
      }
    } else {
      for (int64_t i = t; i < V; i += kThreads) {
        const float g = __builtin_amdgcn_exp2f(El::get(row, i) * kLog2e - l2) - (i == y ? 1.f : 0.f);
        El::put(row, i, valid ? g * w : 0.f);
      }
    }
  }
}

template <typename T, bool GRAD>
hipError_t launch_ce_t(T *logits, int64_t N, int64_t V, const int64_t *labels, int64_t ii,
                       const float *wrow, const Scalars *sc, float *row_loss, float *row_lse,
                       float *logprob, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (V % Elem<T>::E == 0 && (uintptr_t)logits % 16 == 0)
    hipLaunchKernelGGL((ce_row_kernel<T, true, GRAD>), dim3((unsigned)N), dim3(kThreads), 0, s,
                       logits, V, labels, ii, wrow, sc, row_loss, row_lse, logprob);
  else
    hipLaunchKernelGGL((ce_row_kernel<T, false, GRAD>), dim3((unsigned)N), dim3(kThreads), 0, s,
                       logits, V, labels, ii, wrow, sc, row_loss, row_lse, logprob);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ce_rows(void *logits, int64_t N, int64_t V, int dtype, const int64_t *labels,
                          int64_t ii, bool grad, const float *wrow, const Scalars *sc,
                          float *row_loss, float *row_lse, float *logprob, hipStream_t s) {
  if (dtype == 0) {
    float *p = (float *)logits;
    return grad ? launch_ce_t<float, true>(p, N, V, labels, ii, wrow, sc, row_loss, row_lse,
                                           logprob, s)
                : launch_ce_t<float, false>(p, N, V, labels, ii, wrow, sc, row_loss, row_lse,
                                            logprob, s);
  }
  uint16_t *p = (uint16_t *)logits;
  return grad ? launch_ce_t<uint16_t, true>(p, N, V, labels, ii, wrow, sc, row_loss, row_lse,
                                            logprob, s)
              : launch_ce_t<uint16_t, false>(p, N, V, labels, ii, wrow, sc, row_loss, row_lse,
                                             logprob, s);
}

}  // namespace flce
