// bf16 MFMA GEMMs of the chunked fused linear cross-entropy (gfx950).
//
// Three contractions per chunk of c tokens (the chain rule through the
// LM-head projection Z = X W^T that the Liger Kernel pages fuse with the
// cross-entropy loss):
//   forward   Z_c^T = W X_c^T      M = V (vocab), N = c (tokens), K = H
//             + epilogue: per (token, 256-vocab tile) max and sum of exp,
//               the target logit, and the bf16 logits tile into scratch;
//   dX        dX_c  = G_c W        M = c, N = H, K = V (split-K, fp32 partials)
//   dW        dW   (+)= G_c^T X_c  M = V, N = H, K = c (fp32, first chunk stores)
//
// One workgroup = 4 waves of 64 lanes computes a 256 x 256 fp32 tile with
// v_mfma_f32_32x32x16_bf16; each wave owns a 128 x 128 quarter as 4 x 4 MFMA
// blocks.  Operands are staged through LDS in 64-deep K slices, double
// buffered (2 x (32 KB + 32 KB) = 128 KB of the 160 KB LDS), each LDS row
// holding 64 k-values of one m (or n) index as eight 16-byte chunks whose
// position is XOR-swizzled by the row so 16-byte fragment reads and writes
// avoid bank conflicts.
//
// Operands whose K index is the contiguous one (W and X in the forward GEMM,
// G in the dX GEMM) are copied 16 bytes at a time.  Operands whose M/N index
// is contiguous (W in the dX GEMM, G and X in the dW GEMM) are read as 8 x 8
// blocks (eight 16-byte rows) and transposed in registers with byte permutes
// before the LDS write, so every MFMA fragment is one 16-byte LDS read.
#include "flce_internal.h"

namespace flce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NTHREADS = 256;
constexpr int ROW_BYTES = BK * 2;               // one LDS row: 64 bf16
constexpr int TILE_BYTES = 256 * ROW_BYTES;     // 32 KB per operand per stage
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }
__device__ __forceinline__ int lds_off(int row, int q) { return row * ROW_BYTES + ((q ^ swz(row)) << 4); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Map the hardware's round-robin placement of workgroups over the 8 XCDs to
// a logical tile order in which consecutive logical tiles share an XCD (and
// its L2).  Bijective for any grid size.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  int xcd = b & 7, idx = b >> 3;
  int per = nb >> 3, rem = nb & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// ---------------------------------------------------------------- loaders
// Element (r, k) of a K-major operand is p[r * ld + k]; r in [r0, r0+256).
// Thread t copies chunk q = t % 8 (k = 8q..8q+7) of rows t/8 + 32 j.
struct LoadK {
  const uint16_t *p;   // element (r0, k of the current slice)
  int64_t ld;
  int off[8];          // per-thread offsets (elements) of its 8 rows
  bool rok[8];
  int kq;              // k offset of the thread's chunk within a slice

  __device__ void init(const uint16_t *base, int64_t ld_, int rows, int r0, int kb) {
    ld = ld_;
    p = base + (int64_t)r0 * ld_ + kb;
    kq = (threadIdx.x & 7) * 8;
    int rl = threadIdx.x >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int r = rl + 32 * j;
      rok[j] = (r0 + r) < rows;
      off[j] = r * (int)ld_ + kq;
    }
  }
  // Load the slice starting kofs elements after kb; k valid while < klim.
  __device__ __forceinline__ void load(int kofs, int klim, u32x4 (&reg)[8]) const {
    bool kok = (kofs + kq) < klim;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      reg[j] = (rok[j] && kok) ? *(const u32x4 *)(p + off[j] + kofs) : zero4();
  }
  __device__ __forceinline__ static void store(char *s, const u32x4 (&reg)[8]) {
    int q = threadIdx.x & 7, rl = threadIdx.x >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) *(u32x4 *)(s + lds_off(rl + 32 * j, q)) = reg[j];
  }
};

// Element (r, k) of an MN-major operand is p[k * ld + r]; r in [r0, r0+256).
// Thread t reads the 8 x 8 block k = 8 (t/32) + i, r = 8 (t%32) + 0..7.
struct LoadMN {
  const uint16_t *p;   // element (r0, kb)
  int64_t ld;
  int off;             // per-thread offset of its block's first row
  bool cok;
  int kr;              // first k row of the thread's block within a slice

  __device__ void init(const uint16_t *base, int64_t ld_, int rows, int r0, int kb) {
    ld = ld_;
    p = base + (int64_t)kb * ld_ + r0;
    int rc = 8 * (threadIdx.x & 31);
    kr = 8 * (threadIdx.x >> 5);
    cok = (r0 + rc) < rows;
    off = kr * (int)ld_ + rc;
  }
  __device__ __forceinline__ void load(int kofs, int klim, u32x4 (&reg)[8]) const {
    const uint16_t *q = p + (int64_t)kofs * ld + off;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      reg[i] = (cok && (kofs + kr + i) < klim) ? *(const u32x4 *)(q + i * ld) : zero4();
  }
  // Transpose the 8 x 8 block of 16-bit values: output vector j holds
  // k = 0..7 of column r = 8 (t%32) + j, two k per dword, low half first.
  __device__ __forceinline__ static void store(char *s, const u32x4 (&reg)[8]) {
    int rc = 8 * (threadIdx.x & 31), q = threadIdx.x >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 v;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        uint32_t lo = reg[2 * pp][j >> 1], hi = reg[2 * pp + 1][j >> 1];
        v[pp] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      *(u32x4 *)(s + lds_off(rc + j, q)) = v;
    }
  }
};

// ---------------------------------------------------------------- main loop
// acc[i][j] is the 32 x 32 block (i, j) of the wave's 128 x 128 quarter.
// Lane l of block (i, j), register e, holds row 32 i + 8 (e/4) + 4 (l/32) + e%4,
// column 32 j + l%32 of the quarter.
template <class LA, class LB>
__device__ __forceinline__ void mainloop(const LA &la, const LB &lb, int klen, char *smem,
                                         f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  int nk = (klen + BK - 1) / BK;
  if (nk <= 0) return;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int frow = lane & 31, fq = lane >> 5;

  u32x4 ra[8], rb[8];
  la.load(0, klen, ra);
  lb.load(0, klen, rb);
  LA::store(smem, ra);
  LB::store(smem + TILE_BYTES, rb);
  __syncthreads();

  for (int t = 0; t < nk; ++t) {
    char *sA = smem + (t & 1) * 2 * TILE_BYTES;
    char *sB = sA + TILE_BYTES;
    const bool more = t + 1 < nk;
    if (more) {
      la.load((t + 1) * BK, klen, ra);
      lb.load((t + 1) * BK, klen, rb);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *(const bf16x8 *)(sA + lds_off(wm * 128 + i * 32 + frow, kk * 2 + fq));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *(const bf16x8 *)(sB + lds_off(wn * 128 + j * 32 + frow, kk * 2 + fq));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      char *nA = smem + ((t + 1) & 1) * 2 * TILE_BYTES;
      LA::store(nA, ra);
      LB::store(nA + TILE_BYTES, rb);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// ---------------------------------------------------------------- forward tile
// Z^T tile: rows = 256 vocabulary ids from m0, columns = 256 tokens from n0.
__global__ __launch_bounds__(NTHREADS, 1) void fwd_tile_kernel(
    const uint16_t *__restrict__ W, const uint16_t *__restrict__ Xc,
    const int64_t *__restrict__ labels_c, int64_t ii, int c, int H, int V,
    uint16_t *__restrict__ zbuf, int64_t ldz, float *__restrict__ pm, float *__restrict__ ps,
    float *__restrict__ zy, int64_t nvt, int nct, int store_z) {
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int vt = tile / nct, ct = tile - vt * nct;
  const int m0 = vt * BM, n0 = ct * BN;

  LoadK la, lb;
  la.init(W, H, V, m0, 0);
  lb.init(Xc, H, c, n0, 0);
  f32x16 acc[4][4];
  mainloop(la, lb, H, smem, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int vrow0 = m0 + wm * 128 + 4 * (lane >> 5);   // + 32 i + 8 (e/4) + e%4
  float *red = (float *)smem;                          // [2][256] max, [2][256] sum

  float cmax[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int v = vrow0 + 32 * i + 8 * (e >> 2) + (e & 3);
        if (v < V) mx = fmaxf(mx, acc[i][j][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    cmax[j] = mx;
  }
  if (lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wm * 256 + wn * 128 + j * 32 + lane] = cmax[j];
  }
  __syncthreads();
  float csum[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = wn * 128 + j * 32 + (lane & 31);
    const int tok = n0 + col;
    const float m = fmaxf(red[col], red[256 + col]);
    cmax[j] = m;
    const int64_t y = tok < c ? labels_c[tok] : ii;
    const float ml = m * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int v = vrow0 + 32 * i + 8 * (e >> 2) + (e & 3);
        float z = acc[i][j][e];
        if (v < V) s += __builtin_amdgcn_exp2f(z * kLog2e - ml);
        if ((int64_t)v == y && v < V && tok < c) zy[tok] = z;   // single writer per token
      }
    s += __shfl_xor(s, 32);
    csum[j] = s;
  }
  if (lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[512 + wm * 256 + wn * 128 + j * 32 + lane] = csum[j];
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 128 + j * 32 + lane;
      const int tok = n0 + col;
      if (tok < c) {
        pm[(int64_t)tok * nvt + vt] = cmax[j];
        ps[(int64_t)tok * nvt + vt] = red[512 + col] + red[768 + col];
      }
    }
  }
  if (store_z) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = n0 + wn * 128 + j * 32 + (lane & 31);
      if (tok >= c) continue;
      uint16_t *zrow = zbuf + (int64_t)tok * ldz;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int v0 = vrow0 + 32 * i + 8 * g;
          if (v0 < V) {   // v0 % 4 == 0 and ldz % 8 == 0: v0 + 3 < ldz
            uint2 pk;
            pk.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
            pk.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
            *(uint2 *)(zrow + v0) = pk;
          }
        }
    }
  }
}

// ---------------------------------------------------------------- dX (split-K)
// Unit (s, mt, nt): dxp[s][tok][h] = sum over vocab in split s of G[tok][v] W[v][h].
__global__ __launch_bounds__(NTHREADS, 1) void dx_kernel(
    const uint16_t *__restrict__ G, int64_t ldz, const uint16_t *__restrict__ W, int c, int H,
    int V, int64_t ksplit, int nmt, int nnt, float *__restrict__ dxp) {
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int per = nmt * nnt;
  const int s = unit / per, rem = unit - s * per;
  const int mt = rem / nnt, nt = rem - mt * nnt;
  const int m0 = mt * BM, n0 = nt * BN;
  const int64_t kb = (int64_t)s * ksplit;
  const int64_t ke = kb + ksplit < V ? kb + ksplit : V;

  LoadK la;     // G[tok][v]: rows = tokens, k = vocab
  LoadMN lb;    // W[v][h]:   rows (N) = hidden, k = vocab
  la.init(G, ldz, c, m0, (int)kb);
  lb.init(W, H, H, n0, (int)kb);
  f32x16 acc[4][4];
  mainloop(la, lb, (int)(ke - kb), smem, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  float *out = dxp + (int64_t)s * c * H;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tok = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (tok < c && h < H) out[(int64_t)tok * H + h] = acc[i][j][e];
      }
    }
}

// dXc[tok][h] = bf16(sum_s dxp[s][tok][h]), 4 columns per thread (H % 8 == 0).
__global__ void dx_reduce_kernel(const float *__restrict__ dxp, int splitk, int c, int H,
                                 uint16_t *__restrict__ dXc) {
  const int64_t n4 = (int64_t)c * H / 4;
  const int64_t stride = (int64_t)c * H;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    float4 a = ((const float4 *)dxp)[i];
    for (int s = 1; s < splitk; ++s) {
      float4 b = ((const float4 *)(dxp + s * stride))[i];
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    uint2 pk;
    pk.x = pack_bf16x2(a.x, a.y);
    pk.y = pack_bf16x2(a.z, a.w);
    ((uint2 *)dXc)[i] = pk;
  }
}

// ---------------------------------------------------------------- dW
// dW[v][h] (+)= sum over the chunk's tokens of G[tok][v] X[tok][h].
__global__ __launch_bounds__(NTHREADS, 1) void dw_kernel(
    const uint16_t *__restrict__ G, int64_t ldz, const uint16_t *__restrict__ Xc, int c, int H,
    int V, int nht, float *__restrict__ dW, int accumulate) {
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int vt = tile / nht, ht = tile - vt * nht;
  const int m0 = vt * BM, n0 = ht * BN;

  LoadMN la;    // G[tok][v]: rows (M) = vocab, k = tokens
  LoadMN lb;    // X[tok][h]: rows (N) = hidden, k = tokens
  la.init(G, ldz, V, m0, 0);
  lb.init(Xc, H, H, n0, 0);
  f32x16 acc[4][4];
  mainloop(la, lb, c, smem, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int v = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (v < V && h < H) {
          float *p = dW + (int64_t)v * H + h;
          *p = accumulate ? *p + acc[i][j][e] : acc[i][j][e];
        }
      }
    }
}

// ---------------------------------------------------------------- dlogits in place
// G = (exp(Z - lse) - onehot(y)) / N_valid on valid rows, 0 on ignored rows and
// on the padding columns [V, ldz); 8 bf16 per thread.
__global__ void dlogits_kernel(uint16_t *__restrict__ z, int64_t ldz, int c, int V,
                               const float *__restrict__ lse_c, const int64_t *__restrict__ labels_c,
                               int64_t ii, const Scalars *__restrict__ sc) {
  const int64_t g8 = ldz / 8;
  const int64_t n = (int64_t)c * g8;
  const float inv = sc->inv_nvalid;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / g8;
    const int v0 = (int)(i - r * g8) * 8;
    const int64_t y = labels_c[r];
    const bool valid = y != ii;
    const float l2 = lse_c[r] * kLog2e;
    u32x4 *p = (u32x4 *)(z + r * ldz + v0);
    u32x4 in = *p, out;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float f[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int v = v0 + 2 * d + h;
        const float zz = __builtin_bit_cast(float, (h ? (in[d] & 0xFFFF0000u) : (in[d] << 16)));
        float g = __builtin_amdgcn_exp2f(zz * kLog2e - l2) - ((int64_t)v == y ? 1.f : 0.f);
        f[h] = (valid && v < V) ? g * inv : 0.f;
      }
      out[d] = pack_bf16x2(f[0], f[1]);
    }
    *p = out;
  }
}

inline int grid_for(int64_t n, int block, int cap) {
  int64_t g = (n + block - 1) / block;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace

hipError_t launch_fwd_tile_bf16(const uint16_t *W, const uint16_t *Xc, const int64_t *labels_c,
                                int64_t ii, int c, int H, int V, uint16_t *zbuf, int64_t ldz,
                                float *pm, float *ps, float *zy, int64_t nvt, bool store_z,
                                hipStream_t s) {
  const int nct = (c + BN - 1) / BN;
  const int grid = (int)nvt * nct;
  hipLaunchKernelGGL(fwd_tile_kernel, dim3(grid), dim3(NTHREADS), 0, s, W, Xc, labels_c, ii, c,
                     H, V, zbuf, ldz, pm, ps, zy, nvt, nct, store_z ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_dlogits_bf16(uint16_t *zbuf, int64_t ldz, int c, int V, const float *lse_c,
                               const int64_t *labels_c, int64_t ii, const Scalars *sc,
                               hipStream_t s) {
  const int64_t n = (int64_t)c * (ldz / 8);
  hipLaunchKernelGGL(dlogits_kernel, dim3(grid_for(n, 256, 256 * 64)), dim3(256), 0, s, zbuf, ldz,
                     c, V, lse_c, labels_c, ii, sc);
  return hipGetLastError();
}

hipError_t launch_dx_bf16(const uint16_t *G, int64_t ldz, const uint16_t *W, int c, int H, int V,
                          int splitk, int64_t ksplit, float *dxp, hipStream_t s) {
  const int nmt = (c + BM - 1) / BM, nnt = (H + BN - 1) / BN;
  hipLaunchKernelGGL(dx_kernel, dim3(splitk * nmt * nnt), dim3(NTHREADS), 0, s, G, ldz, W, c, H,
                     V, ksplit, nmt, nnt, dxp);
  return hipGetLastError();
}

hipError_t launch_dx_reduce_bf16(const float *dxp, int splitk, int c, int H, uint16_t *dXc,
                                 hipStream_t s) {
  const int64_t n4 = (int64_t)c * H / 4;
  hipLaunchKernelGGL(dx_reduce_kernel, dim3(grid_for(n4, 256, 256 * 32)), dim3(256), 0, s, dxp,
                     splitk, c, H, dXc);
  return hipGetLastError();
}

hipError_t launch_dw_bf16(const uint16_t *G, int64_t ldz, const uint16_t *Xc, int c, int H, int V,
                          float *dW, bool accumulate, hipStream_t s) {
  const int nvt = (V + BM - 1) / BM, nht = (H + BN - 1) / BN;
  hipLaunchKernelGGL(dw_kernel, dim3(nvt * nht), dim3(NTHREADS), 0, s, G, ldz, Xc, c, H, V, nht,
                     dW, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace flce
