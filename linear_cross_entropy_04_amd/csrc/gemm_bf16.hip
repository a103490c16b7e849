// bf16 MFMA GEMMs of the chunked fused linear cross-entropy (gfx950), and
// the data movement that feeds them.
//
// Per chunk of c tokens (the chain rule through the LM-head projection
// Z = X W^T that the Liger Kernel pages fuse with the cross-entropy loss):
//   pack      X_c -> Xp (rows = tokens, k = hidden) and XTp (rows = hidden,
//             k = tokens), both in the packed layout below;
//   forward   Z_c^T = W X_c^T      M = V (vocab), N = c (tokens), K = H
//             + epilogue: per (token, 128-vocab half tile) max and sum of exp,
//               the target logit, and the bf16 logits into Zp (packed, rows =
//               tokens, k = vocab);
//   dlogits   Zp rewritten in place into G = (softmax - onehot) / N_valid, and
//             G^T written to GTp (packed, rows = vocab, k = tokens);
//   dX        dX_c  = G_c W        M = c, N = H, K = V (split-K, fp32 partials)
//   dW        dW   (+)= G_c^T X_c  M = V, N = H, K = c (fp32)
//
// GEMM tiles: a workgroup of 4 waves (2 x 2) computes a BM x BN fp32 tile with
// v_mfma_f32_32x32x16_bf16, each wave a (BM/2) x (BN/2) quarter of 32 x 32
// blocks.  Operands flow global -> LDS through direct-to-LDS copies
// (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at LDS base +
// 16 l) in k-slices of 32, STAGES slices in flight, each admitted by an
// explicit vmcnt wait and one s_barrier.
//
// Operand kinds:
//   PACKED  (Xp, XTp, Zp/G, GTp): the matrix is stored as 16 KB blocks of 256
//           rows x 32 k; a block is 16 fragments of 1 KB, fragment (r/32, k/16)
//           holding in lane order what lane l of an MFMA operand read needs
//           (row r0 + l%32, k = 8 (l/32) + 0..7).  A slice copy is contiguous
//           on both sides and every fragment read is 1 KB contiguous, which
//           measured at full copy and LDS rates.  Padding rows and k are zero.
//   KMAJOR  (W in the forward GEMM): rows of K-contiguous data; 64-byte row
//           pieces XOR-swizzled by row bits 2..3 in LDS.
//   MNMAJOR (W in the dX GEMM): k rows of M/N-contiguous data; fragments read
//           with ds_read_b64_tr_b16, which transposes 16-bit data across each
//           group of 16 lanes (lane j names a 4-element row R_j; lane i gets
//           element i%4 of R_{i/4}, R_{4+i/4}, R_{8+i/4}, R_{12+i/4}).
// Plain-layout tiles that reach past an operand's extent copy 16 zero bytes
// for the lanes outside it, so every thread issues the same number of copies
// per slice and the vmcnt arithmetic holds.
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

enum Kind { KMAJOR = 0, MNMAJOR = 1, PACKED = 2 };

// The source of the copies of out-of-range lanes.
__device__ const uint4 g_zero16 = {0u, 0u, 0u, 0u};

// ---------------------------------------------------------------- packed layout
// Element offset of (r, k) in a packed matrix with nks slices of 32 k per row tile.
__device__ __forceinline__ int64_t pk_off(int64_t r, int64_t k, int64_t nks) {
  const int64_t blk = (r >> 8) * nks + (k >> 5);
  const int rr = (int)(r & 255), kk = (int)(k & 31);
  const int in = ((((rr >> 5) * 2 + (kk >> 4)) * 64 + ((kk >> 3) & 1) * 32 + (rr & 31)) << 3) + (kk & 7);
  return (blk << 13) + in;
}

// K-major slice: 64-byte rows; chunk q (8 k values) of row r sits at slot q ^ fk(r).
// Rows r..r+3 already span one 256-byte bank line; rows 4 apart share it, so
// the swizzle takes row bits 2 and 3 (measured conflict-free; swizzles using
// row bit 0 or 1 leave a two-way conflict).
__device__ __forceinline__ int fk(int r) { return (r >> 2) & 3; }
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

template <int BM_, int BN_, int STAGES_, int KA_, int KB_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, STAGES = STAGES_;
  static constexpr int KA = KA_, KB = KB_;
  static constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int NPER = (A_BYTES + B_BYTES) / 4096;   // copies per thread per slice
  static constexpr int LDS = STAGES * STAGE_BYTES;
};

// One operand of a tile.  KMAJOR: element (r, k) at p[r * ld + k]; MNMAJOR:
// at p[k * ld + r]; PACKED: p is the tile's first block, slice s at p + s * ld
// (ld = 8192 elements).  r counts from the tile's first row, k from the start
// of the reduction range; rows / klen bound the plain layouts.
struct Op {
  const uint16_t *p;
  int64_t ld;
  int rows;
  int klen;
};

// Copy k-slice [k0, k0 + 32) of an operand tile of ROWS rows into LDS.
template <int KIND, int ROWS, bool CHECK>
__device__ __forceinline__ void issue_tile(const Op &op, int k0, char *tile) {
  constexpr int N = ROWS * BK * 2 / 4096;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int blk = i * 4 + w;                   // 1 KB block written by this wave
    const uint16_t *src;
    bool ok = true;
    if constexpr (KIND == PACKED) {
      src = op.p + (int64_t)(k0 >> 5) * op.ld + blk * 512 + l * 8;
    } else if constexpr (KIND == KMAJOR) {
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
    if (KIND != PACKED && CHECK && !ok) src = (const uint16_t *)&g_zero16;
    __builtin_amdgcn_global_load_lds(src, tile + blk * 1024, 16, 0, 0);
  }
}

// MFMA fragment of rows r0..r0+31, k = 16 kk .. 16 kk + 15 of an LDS slice:
// lane l holds row r0 + l%32, k = 16 kk + 8 (l/32) + 0..7.
template <int KIND, int ROWS>
__device__ __forceinline__ bf16x8 frag(const char *tile, int r0, int kk) {
  const int l = threadIdx.x & 63;
  if constexpr (KIND == PACKED) {
    return *(const bf16x8 *)(tile + ((((r0 >> 5) << 1) + kk) << 10) + (l << 4));
  } else if constexpr (KIND == KMAJOR) {
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

// s_waitcnt vmcnt(groups * PER) for a runtime number of groups in 0..2.
template <int PER>
__device__ __forceinline__ void wait_groups(int groups) {
  if (groups >= 2) wait_vm<2 * PER>();
  else if (groups == 1) wait_vm<PER>();
  else wait_vm<0>();
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// drain every copy in flight); the empty asm keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <class T>
__device__ __forceinline__ void load_frags(const char *st, int kk, bf16x8 (&fa)[T::MI],
                                           bf16x8 (&fb)[T::NI]) {
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int i = 0; i < T::MI; ++i) fa[i] = frag<T::KA, T::BM>(st, wm * T::WM + 32 * i, kk);
#pragma unroll
  for (int j = 0; j < T::NI; ++j)
    fb[j] = frag<T::KB, T::BN>(st + T::A_BYTES, wn * T::WN + 32 * j, kk);
}

template <class T>
__device__ __forceinline__ void mfma_block(const bf16x8 (&fa)[T::MI], const bf16x8 (&fb)[T::NI],
                                           f32x16 (&acc)[T::MI][T::NI]) {
#pragma unroll
  for (int i = 0; i < T::MI; ++i)
#pragma unroll
    for (int j = 0; j < T::NI; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

template <class T, bool CHECK>
__device__ __forceinline__ void issue_stage(const Op &a, const Op &b, int step, char *smem) {
  char *st = smem + (step % T::STAGES) * T::STAGE_BYTES;
  issue_tile<T::KA, T::BM, CHECK>(a, step * BK, st);
  issue_tile<T::KB, T::BN, CHECK>(b, step * BK, st + T::A_BYTES);
}

// acc[i][j] is the 32 x 32 block (i, j) of the wave's quarter.  Lane l of
// block (i, j), register e, holds row 32 i + 8 (e/4) + 4 (l/32) + e%4 and
// column 32 j + l%32 of the quarter.  acc enters initialised by the caller.
//
// Each 32-deep slice is two MFMA half-steps (k 0..15, 16..31).  The wait and
// barrier that admit slice t+1 sit between the two half-steps of slice t, so
// the fragments of slice t+1's first half-step are read from LDS while the
// MFMAs of slice t's second half-step run, and the barrier itself waits with
// MFMAs in flight.  Slice t+STAGES-1 is copied into the buffer of slice t-1,
// whose reads every wave finished before that barrier.
// acc[i][j] is the 32 x 32 block (i, j) of the wave's quarter.  Lane l of
// block (i, j), register e, holds row 32 i + 8 (e/4) + 4 (l/32) + e%4 and
// column 32 j + l%32 of the quarter.  acc enters initialised by the caller.
//
// Each 32-deep slice is two MFMA half-steps (k 0..15, 16..31).  The wait and
// barrier that admit slice t+1 sit between the two half-steps of slice t, so
// the fragments of slice t+1's first half-step are read from LDS while the
// MFMAs of slice t's second half-step run, and the barrier itself waits with
// MFMAs in flight.  Slice t+STAGES-1 is copied into the buffer of slice t-1,
// whose reads every wave finished before that barrier.
template <class T, bool CHECK>
__device__ __forceinline__ void mainloop(const Op &a, const Op &b, int klen, char *smem,
                                         f32x16 (&acc)[T::MI][T::NI]) {
  const int nk = (klen + BK - 1) / BK;
  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < T::STAGES - 1; ++s)
      if (s < nk) issue_stage<T, CHECK>(a, b, s, smem);
    wait_groups<T::NPER>(min(T::STAGES - 2, nk - 1));
    bar();
    bf16x8 fa0[T::MI], fb0[T::NI], fa1[T::MI], fb1[T::NI];
    load_frags<T>(smem, 0, fa0, fb0);
    for (int t = 0; t < nk; ++t) {
      const char *st = smem + (t % T::STAGES) * T::STAGE_BYTES;
      load_frags<T>(st, 1, fa1, fb1);
      mfma_block<T>(fa0, fb0, acc);
      if (t + 1 < nk) {
        // slice t+1 must have landed; slices up to t+STAGES-2 may stay in flight
        wait_groups<T::NPER>(min(t + T::STAGES - 2, nk - 1) - (t + 1));
        bar();
        if (t + T::STAGES - 1 < nk) issue_stage<T, CHECK>(a, b, t + T::STAGES - 1, smem);
        load_frags<T>(smem + ((t + 1) % T::STAGES) * T::STAGE_BYTES, 0, fa0, fb0);
      }
      mfma_block<T>(fa1, fb1, acc);
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

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// Transpose an 8 x 8 block of 16-bit values held as 8 rows of 16 bytes:
// out[j] holds element j of rows 0..7, two per dword, low half first.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const uint32_t lo = in[2 * pp][j >> 1], hi = in[2 * pp + 1][j >> 1];
      out[j][pp] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
}

using FwdTile = Tile<256, 256, 4, PACKED, PACKED>;
using DxTile = Tile<256, 256, 4, PACKED, MNMAJOR>;
using DwTile = Tile<256, 128, 3, PACKED, PACKED>;

// ---------------------------------------------------------------- packing
// One thread per 8 x 8 block (rows t0..t0+7, columns h0..h0+7) of a row-major
// bf16 matrix [R][K] padded to 256 x 256: P gets the 8 rows (k = columns) in
// the packed layout, and, when PT is given, PT gets the 8 columns as rows (k =
// rows of the source).  Values outside [0, R) x [0, K) are zero.  The 32
// threads sharing t0 read 8 rows x 512 contiguous bytes.
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t *__restrict__ src, int R, int K,
                                                  int kb8, int64_t nblk,
                                                  uint16_t *__restrict__ P, int64_t nks_p,
                                                  uint16_t *__restrict__ PT, int64_t nks_pt) {
  const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (gid >= nblk) return;
  const int h0 = (int)(gid % kb8) * 8;
  const int64_t t0 = (gid / kb8) * 8;
  u32x4 rows[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    rows[i] = (t0 + i < R && h0 < K) ? *(const u32x4 *)(src + (t0 + i) * K + h0)
                                     : u32x4{0u, 0u, 0u, 0u};
  if (h0 < nks_p * 32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4 *)(P + pk_off(t0 + i, h0, nks_p)) = rows[i];
  }
  if (PT != nullptr && t0 < nks_pt * 32) {
    u32x4 cols[8];
    transpose8x8(rows, cols);
#pragma unroll
    for (int j = 0; j < 8; ++j) *(u32x4 *)(PT + pk_off(h0 + j, t0, nks_pt)) = cols[j];
  }
}

// ---------------------------------------------------------------- forward tile
// Z^T tile: rows = 256 vocabulary ids from m0, columns = 256 tokens from n0;
// both operands packed (Wp rows = vocabulary, Xp rows = tokens, k = hidden).
// VTAIL instantiates the tile that reaches past V (its rows >= V are masked).
//
// Epilogue, wave by wave: each wave reduces its own 128 vocabulary rows, so a
// token gets one (max, sum of exp) partial per 128 vocabulary ids, at index
// 2 vt + wm.  The target logit is taken from the fp32 accumulators by the
// lane that holds it.  The bf16 logits tile is laid out in LDS in Zp's packed
// order (it is 8 consecutive blocks of Zp) and leaves as one 128 KB copy.
__device__ __forceinline__ int zst_off(int r, int v) {     // bytes, tile-local
  const int kk = v & 31;
  return ((v >> 5) << 14) +
         (((((r >> 5) * 2 + (kk >> 4)) * 64 + ((kk >> 3) & 1) * 32 + (r & 31)) << 4)) +
         ((kk & 7) << 1);
}

template <bool VTAIL>
__global__ __launch_bounds__(NTHREADS, 1) void fwd_tile_kernel(
    const uint16_t *__restrict__ Wp, const uint16_t *__restrict__ Xp, int64_t nks_h,
    const int64_t *__restrict__ labels_c, int64_t ii, int c, int H, int V,
    uint16_t *__restrict__ Zp, int64_t nks_z, float *__restrict__ pm, float *__restrict__ ps,
    float *__restrict__ zy, int64_t nvt, int vt0, int nct, int store_z) {
  using T = FwdTile;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int vt = vt0 + tile / nct, ct = tile % nct;
  const int m0 = vt * T::BM, n0 = ct * T::BN;

  const Op a{Wp + (int64_t)vt * nks_h * 8192, 8192, 256, H};
  const Op b{Xp + (int64_t)ct * nks_h * 8192, 8192, 256, H};
  f32x16 acc[4][4];
  zero_acc<T>(acc);
  mainloop<T, false>(a, b, H, smem, acc);      // packed operands carry their zero padding

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
    // rows past V hold -inf here; the dlogits pass zeroes them
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int v = wm * 128 + 32 * i + 8 * g + 4 * (lane >> 5);
          uint2 pk;
          pk.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
          pk.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *(uint2 *)(smem + zst_off(r, v)) = pk;
        }
    }
    __syncthreads();
    // blocks (ct, 8 vt + s) of Zp, s < 8, that exist (the tail tile may have fewer)
    const int nslices = (int)min((int64_t)8, nks_z - 8 * (int64_t)vt);
    uint16_t *dst = Zp + ((int64_t)ct * nks_z + 8 * (int64_t)vt) * 8192;
    const int n16 = nslices * 1024;                     // 16-byte units to copy
    for (int q = threadIdx.x; q < n16; q += NTHREADS)
      *(u32x4 *)(dst + q * 8) = *(const u32x4 *)(smem + q * 16);
  }
}

// ---------------------------------------------------------------- dlogits
// One thread per 128-byte unit of Zp, in Zp's memory order: the unit holds
// tokens r0..r0+7 x vocabulary v0..v0+7 (8 lanes of one fragment half).
// G = (exp(Z - lse) - onehot(y)) / N_valid on valid tokens, 0 on ignored
// tokens and outside [0, c) x [0, V); rewritten in place in Zp and written
// transposed to GTp.  Units of vocabulary tiles past Zp's slices (they only
// exist in GTp's 256-row padding) are zero.
__global__ __launch_bounds__(256) void dlogits_kernel(
    uint16_t *__restrict__ Zp, int64_t nks_z, uint16_t *__restrict__ GTp, int64_t nks_c,
    int c, int V, int64_t nks_zt, int64_t nunit, const float *__restrict__ lse_c,
    const int64_t *__restrict__ labels_c, int64_t ii, const Scalars *__restrict__ sc) {
  const int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (u >= nunit) return;
  // u = ((rt * nks_zt + ks) * 16 + f) * 8 + hk * 4 + rg
  const int rg = (int)(u & 3), hk = (int)((u >> 2) & 1), f = (int)((u >> 3) & 15);
  const int64_t blk = u >> 7;
  const int64_t rt = blk / nks_zt, ks = blk - rt * nks_zt;
  const int r0 = (int)(rt * 256) + (f >> 1) * 32 + rg * 8;
  const int v0 = (int)(ks * 32) + (f & 1) * 16 + hk * 8;
  const float inv = sc->inv_nvalid;
  const bool inz = ks < nks_z;                       // the unit lies inside Zp
  uint16_t *zu = Zp + ((rt * nks_z + ks) << 13) + (((f * 64 + hk * 32 + rg * 8)) << 3);
  u32x4 g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + i;
    int64_t y = ii;
    float l2 = 0.f;
    if (r < c) {
      y = labels_c[r];
      l2 = lse_c[r] * kLog2e;
    }
    const bool valid = r < c && y != ii;
    u32x4 z = inz ? *(const u32x4 *)(zu + i * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float fv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int v = v0 + 2 * d + h;
        const float zz = h ? bf16_hi(z[d]) : bf16_lo(z[d]);
        const float e = __builtin_amdgcn_exp2f(zz * kLog2e - l2) - ((int64_t)v == y ? 1.f : 0.f);
        fv[h] = (valid && v < V) ? e * inv : 0.f;
      }
      g[i][d] = pack_bf16x2(fv[0], fv[1]);
    }
    if (inz) *(u32x4 *)(zu + i * 8) = g[i];
  }
  if (r0 < nks_c * 32) {
    u32x4 gt[8];
    transpose8x8(g, gt);
#pragma unroll
    for (int j = 0; j < 8; ++j) *(u32x4 *)(GTp + pk_off(v0 + j, r0, nks_c)) = gt[j];
  }
}

// ---------------------------------------------------------------- dX (split-K)
// Unit (s, mt, nt): dxp[s][tok][h] = sum over vocabulary in split s of
// G[tok][v] W[v][h].  G comes packed (rows = tokens), W as stored (MN-major).
__global__ __launch_bounds__(NTHREADS, 1) void dx_kernel(
    const uint16_t *__restrict__ Gp, int64_t nks_z, const uint16_t *__restrict__ W, int c, int H,
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

  const Op a{Gp + ((int64_t)mt * nks_z + (kb >> 5)) * 8192, 8192, 256, klen};
  const Op b{W + kb * H + n0, H, H - n0, klen};
  f32x16 acc[4][4];
  zero_acc<T>(acc);
  if (n0 + T::BN <= H && klen % BK == 0)
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
// other's MFMA work.  Both operands come packed (GTp rows = vocabulary, XTp
// rows = hidden, k = tokens).
//
// The epilogue goes through LDS in two halves of 128 rows (64 KB of fp32 each)
// so that dW is read and written in row-contiguous 16-byte pieces: the waves
// holding a half write their accumulators, then every thread moves 16 such
// pieces, with all 16 loads of the current dW in flight before the adds.
// LDS rows are 512 bytes; 128-byte column blocks are XOR-swizzled by row
// bit 2 so the two row groups a write instruction covers use both bank halves.
__device__ __forceinline__ int dwst_off(int r, int col) {   // bytes
  return r * 512 + ((((col >> 5) ^ ((r >> 2) & 1))) << 7) + ((col & 31) << 2);
}

__global__ __launch_bounds__(NTHREADS, 2) void dw_kernel(
    const uint16_t *__restrict__ GTp, const uint16_t *__restrict__ XTp, int64_t nks_c, int c,
    int H, int V, int nht, float *__restrict__ dW, int accumulate) {
  using T = DwTile;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int vt = tile / nht, ht = tile - vt * nht;
  const int m0 = vt * T::BM, n0 = ht * T::BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;

  f32x16 acc[T::MI][T::NI];
  zero_acc<T>(acc);
  const Op a{GTp + (int64_t)vt * nks_c * 8192, 8192, 256, c};
  const Op b{XTp + (int64_t)(ht >> 1) * nks_c * 8192 + (ht & 1) * 4096, 8192, 128, c};
  mainloop<T, false>(a, b, c, smem, acc);

  static_assert(T::LDS >= 128 * 512, "epilogue half tile must fit in LDS");
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int j = 0; j < T::NI; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int col = wn * T::WN + 32 * j + (lane & 31);
            *(float *)(smem + dwst_off(r, col)) = acc[i][j][e];
          }
    }
    __syncthreads();
    // 128 rows x 32 pieces of 16 bytes; thread t takes piece t % 32 of rows t/32 + 8 q
    const int pc = threadIdx.x & 31, col = pc * 4;
    const int h = n0 + col;
    float4 old[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int v = m0 + half * 128 + (threadIdx.x >> 5) + 8 * q;
      const bool ok = v < V && h < H;            // H % 8 == 0: a started piece fits
      old[q] = (accumulate && ok) ? *(const float4 *)(dW + (int64_t)v * H + h)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = (threadIdx.x >> 5) + 8 * q;
      const int v = m0 + half * 128 + r;
      if (v < V && h < H) {
        const float4 add = *(const float4 *)(smem + dwst_off(r, col));
        float4 o = old[q];
        o.x += add.x; o.y += add.y; o.z += add.z; o.w += add.w;
        *(float4 *)(dW + (int64_t)v * H + h) = o;
      }
    }
    __syncthreads();
  }
}

inline int grid_for(int64_t n, int block, int cap) {
  int64_t g = (n + block - 1) / block;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace

hipError_t launch_pack_bf16(const uint16_t *src, int R, int K, uint16_t *P, int64_t nks_p,
                            uint16_t *PT, int64_t nks_pt, hipStream_t s) {
  const int kb8 = (K + 255) / 256 * 32;              // 8-wide column blocks over K rounded to 256
  const int64_t rb8 = (int64_t)(R + 255) / 256 * 32;  // 8-tall row blocks over R rounded to 256
  const int64_t nblk = rb8 * kb8;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, src, R, K,
                     kb8, nblk, P, nks_p, PT, nks_pt);
  return hipGetLastError();
}

hipError_t launch_fwd_tile_bf16(const uint16_t *Wp, const uint16_t *Xp, int64_t nks_h,
                                const int64_t *labels_c, int64_t ii, int c, int H, int V,
                                uint16_t *Zp, int64_t nks_z, float *pm, float *ps, float *zy,
                                int64_t nvt, bool store_z, hipStream_t s) {
  const int nct = (c + FwdTile::BN - 1) / FwdTile::BN;
  const int nfull = V / FwdTile::BM;                 // vocabulary tiles inside V
  if (nfull > 0) {
    hipLaunchKernelGGL(fwd_tile_kernel<false>, dim3(nfull * nct), dim3(NTHREADS), 0, s, Wp, Xp,
                       nks_h, labels_c, ii, c, H, V, Zp, nks_z, pm, ps, zy, nvt, 0, nct,
                       store_z ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (V % FwdTile::BM != 0) {
    hipLaunchKernelGGL(fwd_tile_kernel<true>, dim3(nct), dim3(NTHREADS), 0, s, Wp, Xp, nks_h,
                       labels_c, ii, c, H, V, Zp, nks_z, pm, ps, zy, nvt, nfull, nct,
                       store_z ? 1 : 0);
  }
  return hipGetLastError();
}

hipError_t launch_dlogits_bf16(uint16_t *Zp, int64_t nks_z, uint16_t *GTp, int64_t nks_c, int c,
                               int V, const float *lse_c, const int64_t *labels_c, int64_t ii,
                               const Scalars *sc, hipStream_t s) {
  // units over tokens [0, c rounded to 256) x vocabulary [0, V rounded to 256)
  const int64_t nks_zt = (V + 255) / 256 * 8;        // Zp slices padded to whole 256 tiles
  const int64_t nunit = (int64_t)((c + 255) / 256) * nks_zt * 128;
  hipLaunchKernelGGL(dlogits_kernel, dim3((unsigned)((nunit + 255) / 256)), dim3(256), 0, s, Zp,
                     nks_z, GTp, nks_c, c, V, nks_zt, nunit, lse_c, labels_c, ii, sc);
  return hipGetLastError();
}

hipError_t launch_dx_bf16(const uint16_t *Gp, int64_t nks_z, const uint16_t *W, int c, int H,
                          int V, int splitk, int64_t ksplit, float *dxp, hipStream_t s) {
  const int nmt = (c + DxTile::BM - 1) / DxTile::BM, nnt = (H + DxTile::BN - 1) / DxTile::BN;
  hipLaunchKernelGGL(dx_kernel, dim3(splitk * nmt * nnt), dim3(NTHREADS), 0, s, Gp, nks_z, W, c,
                     H, V, ksplit, nmt, nnt, dxp);
  return hipGetLastError();
}

hipError_t launch_dx_reduce_bf16(const float *dxp, int splitk, int c, int H, uint16_t *dXc,
                                 hipStream_t s) {
  const int64_t n4 = (int64_t)c * H / 4;
  hipLaunchKernelGGL(dx_reduce_kernel, dim3(grid_for(n4, 256, 256 * 32)), dim3(256), 0, s, dxp,
                     splitk, c, H, dXc);
  return hipGetLastError();
}

hipError_t launch_dw_bf16(const uint16_t *GTp, const uint16_t *XTp, int64_t nks_c, int c, int H,
                          int V, float *dW, bool accumulate, hipStream_t s) {
  const int nvt = (V + DwTile::BM - 1) / DwTile::BM, nht = (H + DwTile::BN - 1) / DwTile::BN;
  hipLaunchKernelGGL(dw_kernel, dim3(nvt * nht), dim3(NTHREADS), 0, s, GTp, XTp, nks_c, c, H, V,
                     nht, dW, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace flce
