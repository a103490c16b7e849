// bf16 MFMA GEMMs of the chunked fused linear cross-entropy (gfx950).
//
// Three contractions per chunk of c tokens (the chain rule through the
// LM-head projection Z = X W^T that the Liger Kernel pages fuse with the
// cross-entropy loss):
//   forward   Z_c^T = W X_c^T      M = V (vocab), N = c (tokens), K = H
//             + epilogue: per (token, 256-vocab tile) max and sum of exp,
//               the target logit, and the bf16 logits tile into scratch;
//   dX        dX_c  = G_c W        M = c, N = H, K = V (split-K, fp32 partials)
//   dW        dW   (+)= G_c^T X_c  M = V, N = H, K = c (fp32; the accumulator
//             starts from the previous chunks' dW, the first chunk from 0)
//
// A workgroup of 4 waves (64 lanes each, 2 x 2) computes a BM x BN fp32 tile
// with v_mfma_f32_32x32x16_bf16; each wave owns a (BM/2) x (BN/2) quarter as
// 32 x 32 MFMA blocks.  Operands flow global -> LDS through direct-to-LDS
// copies (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at LDS
// base + 16 l) in k-slices of 32, with STAGES slices in flight; each slice's
// arrival is awaited with an explicit vmcnt wait and one s_barrier, so no
// register staging and no full drain of the copy pipeline at the barrier.
//
// LDS layouts (both XOR-swizzled at 16-byte granularity so that reads and
// writes are free of bank conflicts on 128-byte and 256-byte bank lines):
//   K-major operand (K contiguous in memory: W and X in the forward GEMM, G
//   in the dX GEMM): one 64-byte row per m (or n) index; MFMA fragments are
//   single 16-byte reads.
//   MN-major operand (M/N contiguous: W in the dX GEMM, G and X in the dW
//   GEMM): one row per k holding the tile's M/N extent; fragments are read
//   with ds_read_b64_tr_b16, which transposes 16-bit data across each group
//   of 16 lanes (lane j names a 4-element row R_j; lane i receives element
//   i%4 of R_{i/4}, R_{4+i/4}, R_{8+i/4}, R_{12+i/4}), two reads per fragment.
//
// Tiles that reach past an operand's extent copy 16 zero bytes for the lanes
// outside it, so every thread issues the same number of copies per slice and
// the vmcnt arithmetic holds; full tiles skip the checks.
#include "flce_internal.h"

namespace flce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BK = 32;             // k per pipeline slice
constexpr int NTHREADS = 256;
constexpr float kLog2e = 1.4426950408889634f;

// The source of the copies of out-of-range lanes.
__device__ const uint4 g_zero16 = {0u, 0u, 0u, 0u};

// K-major slice: 64-byte rows; chunk q (8 k values) of row r sits at slot q ^ fk(r).
__device__ __forceinline__ int fk(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
// MN-major slice: one row per k; 16-byte slot s of row k sits at s ^ fmn(k).
__device__ __forceinline__ int fmn(int k) { return (k & 3) << 1; }

// Map the hardware's round-robin placement of workgroups over the 8 XCDs to
// a logical tile order in which consecutive logical tiles share an XCD (and
// its L2).  Bijective for any grid size.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  int xcd = b & 7, idx = b >> 3;
  int per = nb >> 3, rem = nb & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

template <int BM_, int BN_, int STAGES_, bool AK_, bool BK_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, STAGES = STAGES_;
  static constexpr bool AKM = AK_, BKM = BK_;      // operand is K-major
  static constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int NA = A_BYTES / 4096, NB = B_BYTES / 4096;
  static constexpr int NPER = NA + NB;             // copies per thread per slice
  static constexpr int LDS = STAGES * STAGE_BYTES;
};

// One operand of a tile.  K-major: element (r, k) at p[r * ld + k];
// MN-major: element (r, k) at p[k * ld + r].  r counts from the tile's first
// row, k from the start of the reduction range; rows / klen bound them.
struct Op {
  const uint16_t *p;
  int64_t ld;
  int rows;
  int klen;
};

// Copy k-slice [k0, k0 + 32) of an operand tile of ROWS rows into LDS.
template <bool KMAJ, int ROWS, bool CHECK>
__device__ __forceinline__ void issue_tile(const Op &op, int k0, char *tile) {
  constexpr int N = ROWS * BK * 2 / 4096;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int blk = i * 4 + w;                   // 1 KB block written by this wave
    const uint16_t *src;
    bool ok = true;
    if constexpr (KMAJ) {
      const int r = blk * 16 + (l >> 2);
      const int q = (l & 3) ^ fk(r);
      src = op.p + (int64_t)r * op.ld + (k0 + q * 8);
      if (CHECK) ok = (r < op.rows) && (k0 + q * 8 < op.klen);
    } else {
      constexpr int KPB = 1024 / (ROWS * 2);     // k rows per block
      constexpr int LPR = 64 / KPB;              // lanes per k row
      const int kr = blk * KPB + l / LPR;
      const int sl = (l % LPR) ^ fmn(kr);
      src = op.p + (int64_t)(k0 + kr) * op.ld + sl * 8;
      if (CHECK) ok = (k0 + kr < op.klen) && (sl * 8 < op.rows);
    }
    if (CHECK && !ok) src = (const uint16_t *)&g_zero16;
    __builtin_amdgcn_global_load_lds(src, tile + blk * 1024, 16, 0, 0);
  }
}

// MFMA fragment of rows r0..r0+31, k = 16 kk .. 16 kk + 15 of an LDS slice:
// lane l holds row r0 + l%32, k = 16 kk + 8 (l/32) + 0..7.
template <bool KMAJ, int ROWS>
__device__ __forceinline__ bf16x8 frag(const char *tile, int r0, int kk) {
  const int l = threadIdx.x & 63;
  if constexpr (KMAJ) {
    const int r = r0 + (l & 31);
    const int q = kk * 2 + (l >> 5);
    return *(const bf16x8 *)(tile + r * (BK * 2) + ((q ^ fk(r)) << 4));
  } else {
    const int g = l >> 4, j = l & 15;
    const int m = r0 + ((g & 1) << 4) + ((j & 3) << 2);
    const int k = kk * 16 + ((g >> 1) << 3) + (j >> 2);
    const char *base = tile + (((m >> 3) ^ fmn(k)) << 4) + ((m & 7) << 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + k * (ROWS * 2)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + (k + 4) * (ROWS * 2)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
}

// s_waitcnt vmcnt(N) leaving the other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// drain every copy in flight); the empty asm keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// acc[i][j] is the 32 x 32 block (i, j) of the wave's quarter.  Lane l of
// block (i, j), register e, holds row 32 i + 8 (e/4) + 4 (l/32) + e%4 and
// column 32 j + l%32 of the quarter.  acc enters initialised by the caller.
template <class T, bool CHECK>
__device__ __forceinline__ void mainloop(const Op &a, const Op &b, int klen, char *smem,
                                         f32x16 (&acc)[T::MI][T::NI]) {
  const int nk = (klen + BK - 1) / BK;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int s = 0; s < T::STAGES - 1; ++s) {
    if (s < nk) {
      char *st = smem + s * T::STAGE_BYTES;
      issue_tile<T::AKM, T::BM, CHECK>(a, s * BK, st);
      issue_tile<T::BKM, T::BN, CHECK>(b, s * BK, st + T::A_BYTES);
    }
  }
  for (int t = 0; t < nk; ++t) {
    // slices issued after t that may stay in flight
    const int ahead = min(nk - 1 - t, T::STAGES - 2);
    if (ahead >= 2) wait_vm<2 * T::NPER>();
    else if (ahead == 1) wait_vm<T::NPER>();
    else wait_vm<0>();
    bar();
    if (t + T::STAGES - 1 < nk) {
      char *st = smem + ((t + T::STAGES - 1) % T::STAGES) * T::STAGE_BYTES;
      issue_tile<T::AKM, T::BM, CHECK>(a, (t + T::STAGES - 1) * BK, st);
      issue_tile<T::BKM, T::BN, CHECK>(b, (t + T::STAGES - 1) * BK, st + T::A_BYTES);
    }
    const char *sA = smem + (t % T::STAGES) * T::STAGE_BYTES;
    const char *sB = sA + T::A_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[T::MI], bfr[T::NI];
#pragma unroll
      for (int i = 0; i < T::MI; ++i) af[i] = frag<T::AKM, T::BM>(sA, wm * T::WM + 32 * i, kk);
#pragma unroll
      for (int j = 0; j < T::NI; ++j) bfr[j] = frag<T::BKM, T::BN>(sB, wn * T::WN + 32 * j, kk);
#pragma unroll
      for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int j = 0; j < T::NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  bar();    // every wave is done with the LDS slices; the caller may reuse LDS
}

template <class T>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[T::MI][T::NI]) {
#pragma unroll
  for (int i = 0; i < T::MI; ++i)
#pragma unroll
    for (int j = 0; j < T::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

using FwdTile = Tile<256, 256, 4, true, true>;
using DxTile = Tile<256, 256, 4, true, false>;
using DwTile = Tile<256, 128, 3, false, false>;

// ---------------------------------------------------------------- forward tile
// Z^T tile: rows = 256 vocabulary ids from m0, columns = 256 tokens from n0.
// VTAIL instantiates the tile that reaches past V (its rows >= V are masked).
//
// Epilogue, wave by wave: each wave reduces its own 128 vocabulary rows, so a
// token gets one (max, sum of exp) partial per 128 vocabulary ids, at index
// 2 vt + wm.  The target logit is taken from the fp32 accumulators by the
// lane that holds it.  The bf16 logits tile then goes through LDS
// ([token][vocab], 16-byte slots XOR-swizzled by the token) so that it
// leaves as contiguous 512-byte token rows.
__device__ __forceinline__ int zlds_off(int row, int vl) {
  return row * 512 + (((vl >> 3) ^ (row & 31)) << 4) + ((vl & 7) << 1);
}

template <bool VTAIL>
__global__ __launch_bounds__(NTHREADS, 1) void fwd_tile_kernel(
    const uint16_t *__restrict__ W, const uint16_t *__restrict__ Xc,
    const int64_t *__restrict__ labels_c, int64_t ii, int c, int H, int V,
    uint16_t *__restrict__ zbuf, int64_t ldz, float *__restrict__ pm, float *__restrict__ ps,
    float *__restrict__ zy, int64_t nvt, int vt0, int nct, int store_z) {
  using T = FwdTile;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int vt = vt0 + tile / nct, ct = tile % nct;
  const int m0 = vt * T::BM, n0 = ct * T::BN;

  const Op a{W + (int64_t)m0 * H, H, V - m0, H};
  const Op b{Xc + (int64_t)n0 * H, H, c - n0, H};
  f32x16 acc[4][4];
  zero_acc<T>(acc);
  if (!VTAIL && n0 + T::BN <= c && H % BK == 0)
    mainloop<T, false>(a, b, H, smem, acc);
  else
    mainloop<T, true>(a, b, H, smem, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int vrow0 = m0 + wm * 128 + 4 * (lane >> 5);   // row r = 32 i + 8 (e/4) + e%4
  const int vlim = V - vrow0;                          // rows r < vlim exist
  const int64_t part = 2 * (int64_t)vt + wm;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = n0 + wn * 128 + j * 32 + (lane & 31);
    const bool tok_ok = tok < c;
    const int64_t y = tok_ok ? labels_c[tok] : ii;
    const int yr = (y != ii && y >= 0 && y < V) ? (int)y - vrow0 : -1;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + (e & 3);
        const float z = (VTAIL && r >= vlim) ? -INFINITY : acc[i][j][e];
        mx = fmaxf(mx, z);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // a wave whose rows all lie past V has mx = -inf: its sum must be 0, not NaN
    const float ml = (VTAIL && mx == -INFINITY) ? 0.f : mx * kLog2e;
    float sum = 0.f, zsel = 0.f;
    bool found = false;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + (e & 3);
        const float z = (VTAIL && r >= vlim) ? -INFINITY : acc[i][j][e];
        sum += __builtin_amdgcn_exp2f(z * kLog2e - ml);
        zsel = (r == yr) ? acc[i][j][e] : zsel;
        found = found || (r == yr);
      }
    sum += __shfl_xor(sum, 32);
    if (found && tok_ok) zy[tok] = zsel;             // one lane holds the target
    if (lane < 32 && tok_ok) {
      pm[(int64_t)tok * nvt + part] = mx;
      ps[(int64_t)tok * nvt + part] = sum;
    }
  }

  if (store_z) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int vl = wm * 128 + 32 * i + 8 * g + 4 * (lane >> 5);
          uint2 pk;
          pk.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
          pk.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *(uint2 *)(smem + zlds_off(row, vl)) = pk;
        }
    }
    __syncthreads();
    // 256 token rows x 32 slots of 16 bytes; thread t takes slot t % 32 of
    // rows t / 32 + 8 q.
    const int sl = threadIdx.x & 31;
    const int vl = sl * 8;
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int row = (threadIdx.x >> 5) + 8 * q;
      const int tok = n0 + row;
      if (tok < c && (!VTAIL || m0 + vl < V)) {   // ldz % 8 == 0: a started slot fits
        const u32x4 v = *(const u32x4 *)(smem + zlds_off(row, vl));
        *(u32x4 *)(zbuf + (int64_t)tok * ldz + m0 + vl) = v;
      }
    }
  }
}

// ---------------------------------------------------------------- dX (split-K)
// Unit (s, mt, nt): dxp[s][tok][h] = sum over vocab in split s of G[tok][v] W[v][h].
__global__ __launch_bounds__(NTHREADS, 1) void dx_kernel(
    const uint16_t *__restrict__ G, int64_t ldz, const uint16_t *__restrict__ W, int c, int H,
    int V, int64_t ksplit, int nmt, int nnt, float *__restrict__ dxp) {
  using T = DxTile;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int per = nmt * nnt;
  const int s = unit / per, rem = unit - s * per;
  const int mt = rem / nnt, nt = rem - mt * nnt;
  const int m0 = mt * T::BM, n0 = nt * T::BN;
  const int64_t kb = (int64_t)s * ksplit;
  const int64_t ke = kb + ksplit < V ? kb + ksplit : V;
  const int klen = (int)(ke - kb);

  const Op a{G + (int64_t)m0 * ldz + kb, ldz, c - m0, klen};   // G[tok][v]: K-major
  const Op b{W + kb * H + n0, H, H - n0, klen};                 // W[v][h]: MN-major
  f32x16 acc[4][4];
  zero_acc<T>(acc);
  if (m0 + T::BM <= c && n0 + T::BN <= H && klen % BK == 0)
    mainloop<T, false>(a, b, klen, smem, acc);
  else
    mainloop<T, true>(a, b, klen, smem, acc);

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
// dW[v][h] (+)= sum over the chunk's tokens of G[tok][v] X[tok][h], in
// 256 x 128 tiles, two workgroups per CU so that one's dW traffic overlaps the
// other's MFMA work.  With accumulate, the accumulators start from the
// current dW (loaded before the slices), so the epilogue only stores.
__global__ __launch_bounds__(NTHREADS, 2) void dw_kernel(
    const uint16_t *__restrict__ G, int64_t ldz, const uint16_t *__restrict__ Xc, int c, int H,
    int V, int nht, float *__restrict__ dW, int accumulate) {
  using T = DwTile;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int vt = tile / nht, ht = tile - vt * nht;
  const int m0 = vt * T::BM, n0 = ht * T::BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const bool full = m0 + T::BM <= V && n0 + T::BN <= H;

  f32x16 acc[T::MI][T::NI];
  zero_acc<T>(acc);

  const Op a{G + m0, ldz, V - m0, c};          // G[tok][v]: MN-major, rows = vocab
  const Op b{Xc + n0, H, H - n0, c};           // X[tok][h]: MN-major, rows = hidden
  if (full && c % BK == 0)
    mainloop<T, false>(a, b, c, smem, acc);
  else
    mainloop<T, true>(a, b, c, smem, acc);

  // Read-modify-write of dW, one 32 x 32 block at a time; each access
  // instruction covers two full 128-byte row segments.
  float *tb = dW + (int64_t)(m0 + wm * T::WM + 4 * (lane >> 5)) * H + (n0 + wn * T::WN + (lane & 31));
#pragma unroll
  for (int i = 0; i < T::MI; ++i)
#pragma unroll
    for (int j = 0; j < T::NI; ++j) {
      float old[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + (e & 3);
        const bool ok = full || (m0 + wm * T::WM + 4 * (lane >> 5) + r < V &&
                                 n0 + wn * T::WN + j * 32 + (lane & 31) < H);
        old[e] = (accumulate && ok) ? tb[(int64_t)r * H + j * 32] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + (e & 3);
        const bool ok = full || (m0 + wm * T::WM + 4 * (lane >> 5) + r < V &&
                                 n0 + wn * T::WN + j * 32 + (lane & 31) < H);
        if (ok) tb[(int64_t)r * H + j * 32] = old[e] + acc[i][j][e];
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
  const int nct = (c + FwdTile::BN - 1) / FwdTile::BN;
  const int nfull = V / FwdTile::BM;                 // vocabulary tiles inside V
  if (nfull > 0) {
    hipLaunchKernelGGL(fwd_tile_kernel<false>, dim3(nfull * nct), dim3(NTHREADS), 0, s, W, Xc,
                       labels_c, ii, c, H, V, zbuf, ldz, pm, ps, zy, nvt, 0, nct, store_z ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (V % FwdTile::BM != 0) {
    hipLaunchKernelGGL(fwd_tile_kernel<true>, dim3(nct), dim3(NTHREADS), 0, s, W, Xc, labels_c,
                       ii, c, H, V, zbuf, ldz, pm, ps, zy, nvt, nfull, nct, store_z ? 1 : 0);
  }
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
  const int nmt = (c + DxTile::BM - 1) / DxTile::BM, nnt = (H + DxTile::BN - 1) / DxTile::BN;
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
  const int nvt = (V + DwTile::BM - 1) / DwTile::BM, nht = (H + DwTile::BN - 1) / DwTile::BN;
  hipLaunchKernelGGL(dw_kernel, dim3(nvt * nht), dim3(NTHREADS), 0, s, G, ldz, Xc, c, H, V, nht,
                     dW, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace flce
