// bf16 MFMA GEMMs of the chunked fused linear cross-entropy (gfx950), and
// the data movement that feeds them.
//
// Per call, W is packed once into Wp (rows = vocabulary, k = hidden).  Per
// chunk of c tokens (the chain rule through the LM-head projection
// Z = X W^T that the Liger Kernel pages fuse with the cross-entropy loss):
//   pack      X_c -> Xp (rows = tokens, k = hidden);
//   forward   Z_c^T = W X_c^T      M = V (vocab), N = c (tokens), K = H
//             + epilogue: per (token, 128-vocab half tile) max m and sum of
//               exp, the target logit, and bf16(z - m) into Zp (rows =
//               tokens, k = vocabulary);
//   dlogits   Zp rewritten in place into G = (softmax - onehot) / N_valid;
//   dX        dX_c  = G_c W        M = c, N = H, K = V (split-K, fp32 partials),
//             W from WTp, a second packed copy of W made once per call (rows =
//             hidden, k = vocabulary);
//   dW        dW   (+)= G_c^T X_c  M = V, N = H, K = c (fp32)
//
// GEMM tiles: a workgroup of 4 waves (2 x 2) computes a BM x BN fp32 tile with
// v_mfma_f32_32x32x16_bf16, each wave a (BM/2) x (BN/2) quarter of 32 x 32
// blocks.  Operands flow global -> LDS through direct-to-LDS copies
// (global_load_lds_dwordx4: lane l of a wave writes 16 bytes at LDS base +
// 16 l) in k-slices of 32, STAGES slices in flight, each admitted by an
// explicit vmcnt wait and one s_barrier.
//
// The packed layout (Wp, Xp, Zp): a matrix of R rows and K columns is stored
// as 16 KB blocks of 256 rows x 32 columns; block (rt, ks) at element
// (rt * nks + ks) * 8192, nks = 8 ceil(K / 256) (columns padded to 256 so a
// 256-wide tile of columns always exists).  A block is 16 fragments of 1 KB;
// fragment (r/32, k/16) holds 32 rows x 16 columns as 64 slots of 16 bytes (8
// consecutive columns of one row): row r%32 of column half h = (k/8)%2 sits
// at slot 32 h + (r%32 ^ 4 h ^ 8 f), f = (k/16)%2.  Padding rows and columns
// are zero.  Each GEMM reads a packed matrix in one of two directions:
//   PACKED   rows of the matrix are rows of the GEMM operand (k runs along
//            the matrix's columns): a slice is 1 KB pieces of one 16 KB block
//            and an MFMA fragment is one 16-byte read per lane;
//   PACKED_T columns of the matrix are rows of the GEMM operand (k runs along
//            the matrix's rows): a slice is 2 KB pieces (two fragments) of
//            consecutive blocks, and a fragment comes from two
//            ds_read_b64_tr_b16, which transpose 16-bit data across each group
//            of 16 lanes (lane j names a 4-element row R_j; lane i gets element
//            i%4 of R_{i/4}, R_{4+i/4}, R_{8+i/4}, R_{12+i/4}).
// The two XOR terms of the slot index make both read kinds free of LDS bank
// conflicts: an aligned group of 16 lanes of a 16-byte read covers 256
// distinct bytes, and each half-wave of a transposing read covers 32 distinct
// 8-byte bank pairs.
#include "flce_internal.h"

namespace flce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BK = 32;             // k per pipeline slice
constexpr int NTHREADS = 256;
constexpr float kLog2e = 1.4426950408889634f;

enum Kind { PACKED = 0, PACKED_T = 1 };

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a pointer into __shared__ memory, made wave-uniform so
// that the copies' destinations are computed in scalar registers.
__device__ __forceinline__ uint32_t lds_addr(const char *p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p);
}

// ---------------------------------------------------------------- packed layout
// 16-byte slot of row r32 = r % 32, column half h = (k / 8) % 2 and fragment
// half f = (k / 16) % 2 inside a 1 KB fragment.
__device__ __forceinline__ int pk_slot(int r32, int h, int f) {
  return (h << 5) + (r32 ^ (h << 2) ^ (f << 3));
}

// Element offset of (r, k) in a packed matrix with nks 32-column slices.
__device__ __forceinline__ int64_t pk_off(int64_t r, int64_t k, int64_t nks) {
  const int64_t blk = (r >> 8) * nks + (k >> 5);
  const int rr = (int)(r & 255), kk = (int)(k & 31);
  const int frag = ((rr >> 5) << 1) + (kk >> 4);
  return (blk << 13) + (frag << 9) + (pk_slot(rr & 31, (kk >> 3) & 1, kk >> 4) << 3) + (kk & 7);
}

// Map the hardware's round-robin placement of workgroups over the 8 XCDs to
// a logical tile order in which consecutive logical tiles share an XCD (and
// its L2).  Bijective for any grid size.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  int xcd = b & 7, idx = b >> 3;
  int per = nb >> 3, rem = nb & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// Grouped order of an nrow x ncol tile grid: logical tiles run down a group
// of G rows, then on to the next column, so that the tiles resident on one
// XCD at a time form a G x (slots / G) block whose row and column operand
// strips both stay in its L2.  Bijective.
template <int G>
__device__ __forceinline__ void grouped(int t, int nrow, int ncol, int &row, int &col) {
  const int g = t / (G * ncol);
  const int r0 = g * G;
  const int gs = min(G, nrow - r0);
  const int l = t - g * G * ncol;
  row = r0 + l % gs;
  col = l / gs;
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

// One GEMM operand tile in a packed matrix P.
//   PACKED:   p = the block of the tile's first row and of the range's first
//             k; slice s at p + s * 8192.
//   PACKED_T: p = the block of row tile 0 and of the column slice of the
//             tile's first operand row; ld = nks_P * 8192 (one row tile of P);
//             kb = the range's first k, a row of P (a multiple of 32).
struct Op {
  const uint16_t *p;
  int64_t ld;
  int64_t kb;
};

// Copy k-slice [k0, k0 + 32) (relative to the range) of an operand tile of
// ROWS rows into LDS: ROWS / 16 pieces of 1 KB, piece b at LDS byte address
// tile + 1 KB b.  PACKED_T pieces 2q, 2q+1 are the two fragments of operand
// rows 32q..32q+31.  Only the source's lane offset is per lane.
template <int KIND, int ROWS>
__device__ __forceinline__ void issue_tile(const Op &op, int k0, uint32_t tile) {
  constexpr int N = ROWS * BK * 2 / 4096;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const uint16_t *base;
  if constexpr (KIND == PACKED) {
    base = op.p + (int64_t)(k0 >> 5) * 8192;
  } else {
    const int64_t kr = op.kb + k0;                 // row of P
    base = op.p + (kr >> 8) * op.ld + (((kr & 255) >> 5) << 10);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int blk = i * 4 + w;                   // 1 KB piece written by this wave
    const uint16_t *src;
    if constexpr (KIND == PACKED)
      src = base + blk * 512 + l * 8;
    else
      src = base + (blk >> 1) * 8192 + (blk & 1) * 512 + l * 8;
    __builtin_amdgcn_global_load_lds(src, (lds_void *)(uintptr_t)(tile + blk * 1024), 16, 0, 0);
  }
}

// MFMA fragment of operand rows r0..r0+31 (r0 % 32 == 0), k = 16 kk .. 16 kk
// + 15 of an LDS slice: lane l holds row r0 + l%32, k = 16 kk + 8 (l/32) + 0..7.
template <int KIND>
__device__ __forceinline__ bf16x8 frag(const char *tile, int r0, int kk) {
  const int l = threadIdx.x & 63;
  if constexpr (KIND == PACKED) {
    const char *f = tile + ((((r0 >> 5) << 1) + kk) << 10);
    return *(const bf16x8 *)(f + (pk_slot(l & 31, l >> 5, kk) << 4));
  } else {
    // operand row r is column r of the slice's P rows, operand k its row;
    // lane j of a 16-lane group names the 4 operand rows r..r+3 at one k
    const int g = l >> 4, j = l & 15;
    const int r = r0 + ((g & 1) << 4) + ((j & 3) << 2);
    const int k = kk * 16 + ((g >> 1) << 3) + (j >> 2);
    const int h = (r >> 3) & 1, f = (r >> 4) & 1;
    const char *p = tile + ((((r >> 5) << 1) + f) << 10) + ((r & 7) << 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + (pk_slot(k, h, f) << 4)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + (pk_slot(k + 4, h, f) << 4)));
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

// s_waitcnt vmcnt(groups * PER) for a runtime number of groups in 0..3.
template <int PER>
__device__ __forceinline__ void wait_groups(int groups) {
  if (groups >= 3) wait_vm<3 * PER>();
  else if (groups == 2) wait_vm<2 * PER>();
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
  for (int i = 0; i < T::MI; ++i) fa[i] = frag<T::KA>(st, wm * T::WM + 32 * i, kk);
#pragma unroll
  for (int j = 0; j < T::NI; ++j) fb[j] = frag<T::KB>(st + T::A_BYTES, wn * T::WN + 32 * j, kk);
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

// Copies of slice `step` into the ring slot at LDS byte address lds0 +
// (step % STAGES) slots; past the last slice (step >= nk) they copy the last
// slice again (still in cache) into a slot that is not read again.
template <class T>
__device__ __forceinline__ void issue_stage(const Op &a, const Op &b, int step, int nk,
                                            uint32_t lds0) {
  const uint32_t st = lds0 + (uint32_t)((step % T::STAGES) * T::STAGE_BYTES);
  const int k0 = (step < nk ? step : nk - 1) * BK;
  issue_tile<T::KA, T::BM>(a, k0, st);
  issue_tile<T::KB, T::BN>(b, k0, st + T::A_BYTES);
}

// Instruction-group order for the scheduler (sched_group_barrier masks:
// 0x008 MFMA, 0x010 VMEM, 0x100 DS read).  Before the barrier: each of the
// half-step's MFMAs is followed by one fragment read of the next half-step.
// After it: each MFMA is followed by one fragment read, then by one slice
// copy, so the reads start first and the MFMA pipe never waits on issue.
template <class T>
__device__ __forceinline__ void order_first_half() {
  constexpr int M = T::MI * T::NI, R = T::MI + T::NI;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

template <class T>
__device__ __forceinline__ void order_second_half() {
  constexpr int M = T::MI * T::NI, R = T::MI + T::NI, G = T::NPER;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    else if (i < R + G) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  }
  if (R + G > M) __builtin_amdgcn_sched_group_barrier(0x010, R + G - M, 0);
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
// whose reads every wave finished before that barrier.  Every iteration
// issues one slice of copies (the last slice again past the end), so the wait is always for
// all but the newest STAGES-3 slices, and the last slice is peeled: the loop
// body is one straight path.  Packed operands carry zero padding up to whole
// slices, so no copy needs a bounds check.
template <class T>
__device__ __forceinline__ void mainloop(const Op &a, const Op &b, int klen, char *smem,
                                         f32x16 (&acc)[T::MI][T::NI]) {
  const int nk = (klen + BK - 1) / BK;
  if (nk > 0) {
    const uint32_t lds0 = lds_addr(smem);
#pragma unroll
    for (int s = 0; s < T::STAGES - 1; ++s) issue_stage<T>(a, b, s, nk, lds0);
    wait_vm<(T::STAGES - 2) * T::NPER>();
    bar();
    bf16x8 fa0[T::MI], fb0[T::NI], fa1[T::MI], fb1[T::NI];
    load_frags<T>(smem, 0, fa0, fb0);
    for (int t = 0; t < nk - 1; ++t) {
      const char *st = smem + (t % T::STAGES) * T::STAGE_BYTES;
      load_frags<T>(st, 1, fa1, fb1);
      mfma_block<T>(fa0, fb0, acc);
      order_first_half<T>();
      // slice t+1 must have landed; slices t+2 .. t+STAGES-2 may stay in flight
      wait_vm<(T::STAGES - 3) * T::NPER>();
      bar();
      load_frags<T>(smem + ((t + 1) % T::STAGES) * T::STAGE_BYTES, 0, fa0, fb0);
      issue_stage<T>(a, b, t + T::STAGES - 1, nk, lds0);
      mfma_block<T>(fa1, fb1, acc);
      order_second_half<T>();
    }
    load_frags<T>(smem + ((nk - 1) % T::STAGES) * T::STAGE_BYTES, 1, fa1, fb1);
    mfma_block<T>(fa0, fb0, acc);
    mfma_block<T>(fa1, fb1, acc);
  }
  // every wave is done with the LDS slices and no copy is still writing them;
  // the caller may reuse LDS
  wait_vm<0>();
  bar();
}

// ---------------------------------------------------------------- transposed main loop
// Main loop of a tile whose operands are both read transposed (dW).  The
// compiler guards every ds_read_b64_tr_b16 it emits with a wait for all
// direct-to-LDS copies in flight, which would drain the copy pipeline once
// per slice; so here the transposing reads are issued as inline asm, their
// completion is awaited explicitly (s_waitcnt lgkmcnt(0), tied to the
// fragment registers so no MFMA can move above it), and the source order of
// reads, copies and MFMAs is the issue order (volatile asm statements keep
// their order).  Same pipeline as mainloop: the wait and barrier admitting
// slice t+1 sit between the half-steps of slice t.
struct TrFrag {
  i16x4 lo, hi;
};

// Compile-time loop: f(ic<B>{}), ..., f(ic<E - 1>{}), so that loop indices
// can select immediates.
template <int V>
struct ic {
  static constexpr int value = V;
};
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(ic<B>{});
    static_for<B + 1, E>(f);
  }
}

// ds_read_b64_tr_b16 from LDS byte address a + IMM.
template <int IMM>
__device__ __forceinline__ void tr_read(i16x4 &dst, uint32_t a) {
  static_assert(IMM >= 0 && IMM < 65536, "LDS instruction offset range");
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(dst) : "v"(a), "i"(IMM));
}

// Byte offsets, within a slice, of this lane's two transposing reads for the
// fragment of operand rows r0..r0+31, half-step kk (see frag<PACKED_T>).
// For the fragments r0 + 32 i of one wave and the two half-steps they differ
// from those of (r0, 0) by exactly 2048 i + 256 kk in every lane (fragment
// r/32 moves by two 1 KB pieces; k + 16 flips bit 4 of the slot, which no XOR
// term touches), so a wave keeps one address per read half and operand and
// reaches every read through the instruction's immediate offset.
__device__ __forceinline__ void tr_offsets(int r0, int kk, uint32_t &lo, uint32_t &hi) {
  const int l = threadIdx.x & 63;
  const int g = l >> 4, j = l & 15;
  const int r = r0 + ((g & 1) << 4) + ((j & 3) << 2);
  const int k = kk * 16 + ((g >> 1) << 3) + (j >> 2);
  const int h = (r >> 3) & 1, f = (r >> 4) & 1;
  const int p = ((((r >> 5) << 1) + f) << 10) + ((r & 7) << 1);
  lo = (uint32_t)(p + (pk_slot(k, h, f) << 4));
  hi = (uint32_t)(p + (pk_slot(k + 4, h, f) << 4));
}

// LDS addresses of this lane's reads of fragment 0, half-step 0, in one stage.
struct TrBase {
  uint32_t alo, ahi, blo, bhi;
};

// Read Q (0 .. 2 (MI + NI) - 1) of half-step KK: fragment Q/2 (A fragments
// first), low or high half.
template <class T, int KK, int Q>
__device__ __forceinline__ void tr_issue(const TrBase &b, TrFrag (&fa)[T::MI],
                                         TrFrag (&fb)[T::NI]) {
  constexpr int fi = Q >> 1;
  if constexpr (fi < T::MI) {
    constexpr int imm = 2048 * fi + 256 * KK;
    if constexpr (Q & 1) tr_read<imm>(fa[fi].hi, b.ahi);
    else tr_read<imm>(fa[fi].lo, b.alo);
  } else {
    constexpr int imm = 2048 * (fi - T::MI) + 256 * KK;
    if constexpr (Q & 1) tr_read<imm>(fb[fi - T::MI].hi, b.bhi);
    else tr_read<imm>(fb[fi - T::MI].lo, b.blo);
  }
}

// Wait for every LDS read of this wave and tie the fragments to the wait.
template <class T>
__device__ __forceinline__ void tr_wait(TrFrag (&fa)[T::MI], TrFrag (&fb)[T::NI]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < T::MI; ++i) asm volatile("" : "+v"(fa[i].lo), "+v"(fa[i].hi));
#pragma unroll
  for (int j = 0; j < T::NI; ++j) asm volatile("" : "+v"(fb[j].lo), "+v"(fb[j].hi));
}

__device__ __forceinline__ bf16x8 tr_join(const TrFrag &f) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(f.lo, f.hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One MFMA of a half-step, fenced so that the scheduler keeps the source
// order of MFMAs, reads and copies.
template <class T>
__device__ __forceinline__ void tr_mfma(int i, const TrFrag (&fa)[T::MI], const TrFrag (&fb)[T::NI],
                                        f32x16 (&acc)[T::MI][T::NI]) {
  const int a = i / T::NI, b = i % T::NI;
  __builtin_amdgcn_sched_barrier(0);
  acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_join(fa[a]), tr_join(fb[b]), acc[a][b], 0,
                                                      0, 0);
  __builtin_amdgcn_sched_barrier(0);
}

template <class T>
__device__ __forceinline__ void mainloop_tt(const Op &a, const Op &b, int klen, char *smem,
                                            f32x16 (&acc)[T::MI][T::NI]) {
  static_assert(T::KA == PACKED_T && T::KB == PACKED_T, "transposed operands only");
  constexpr int M = T::MI * T::NI;             // MFMAs per half-step
  constexpr int R = 2 * (T::MI + T::NI);       // transposing reads per half-step
  const int nk = (klen + BK - 1) / BK;
  if (nk > 0) {
    const int w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
    const uint32_t lds0 = lds_addr(smem);
    TrBase b0;
    tr_offsets(wm * T::WM, 0, b0.alo, b0.ahi);
    tr_offsets(wn * T::WN, 0, b0.blo, b0.bhi);
    b0.alo += lds0;
    b0.ahi += lds0;
    b0.blo += lds0 + T::A_BYTES;
    b0.bhi += lds0 + T::A_BYTES;
    auto stage_base = [&](int stage) {
      const uint32_t o = (uint32_t)(stage * T::STAGE_BYTES);
      return TrBase{b0.alo + o, b0.ahi + o, b0.blo + o, b0.bhi + o};
    };
#pragma unroll
    for (int s = 0; s < T::STAGES - 1; ++s) issue_stage<T>(a, b, s, nk, lds0);
    wait_vm<(T::STAGES - 2) * T::NPER>();
    bar();
    TrFrag fa0[T::MI], fb0[T::NI], fa1[T::MI], fb1[T::NI];
    TrBase cur = b0;                             // the stage of slice t
    int st = 0;
    static_for<0, R>([&](auto q) { tr_issue<T, 0, decltype(q)::value>(cur, fa0, fb0); });
    // the last slice is peeled so that the loop body is one straight path
    for (int t = 0; t < nk - 1; ++t) {
      const int sn = st + 1 == T::STAGES ? 0 : st + 1;
      const TrBase nxt = stage_base(sn);
      tr_wait<T>(fa0, fb0);
      // first half-step; the reads of the second go out between its MFMAs
      static_for<0, M>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        tr_mfma<T>(i, fa0, fb0, acc);
        static_for<i * R / M, (i + 1) * R / M>(
            [&](auto q) { tr_issue<T, 1, decltype(q)::value>(cur, fa1, fb1); });
      });
      // slice t+1 must have landed; slices t+2 .. t+STAGES-2 may stay in flight
      wait_vm<(T::STAGES - 3) * T::NPER>();
      bar();
      tr_wait<T>(fa1, fb1);
      // second half-step: the next copies after its first MFMA, then the
      // next slice's first reads between the rest
      tr_mfma<T>(0, fa1, fb1, acc);
      issue_stage<T>(a, b, t + T::STAGES - 1, nk, lds0);
      static_for<1, M>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        tr_mfma<T>(i, fa1, fb1, acc);
        static_for<(i - 1) * R / (M - 1), i * R / (M - 1)>(
            [&](auto q) { tr_issue<T, 0, decltype(q)::value>(nxt, fa0, fb0); });
      });
      cur = nxt;
      st = sn;
    }
    tr_wait<T>(fa0, fb0);
    static_for<0, M>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      tr_mfma<T>(i, fa0, fb0, acc);
      static_for<i * R / M, (i + 1) * R / M>(
          [&](auto q) { tr_issue<T, 1, decltype(q)::value>(cur, fa1, fb1); });
    });
    tr_wait<T>(fa1, fb1);
    static_for<0, M>([&](auto ii) { tr_mfma<T>(decltype(ii)::value, fa1, fb1, acc); });
  }
  // every wave is done with the LDS slices and no copy is still writing them;
  // the caller may reuse LDS
  wait_vm<0>();
  bar();
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

using FwdTile = Tile<256, 256, 4, PACKED, PACKED>;     // A = Wp, B = Xp
using DxTile = Tile<256, 256, 4, PACKED, PACKED>;      // A = G (Zp), B = WTp
using DwTile = Tile<256, 128, 3, PACKED_T, PACKED_T>;  // A = G (Zp), B = Xp, both transposed
constexpr int kDwOcc = 2;                              // dW workgroups per CU

// ---------------------------------------------------------------- packing
// One workgroup per 256 rows x 64 columns (two packed blocks, 32 KB) of a
// row-major bf16 matrix [R][K]: it reads the rows' 128-byte pieces (8 full
// rows per wave instruction), places them in LDS in packed order, and writes
// the two blocks as one contiguous 32 KB copy.  Zero outside [0, R) x [0, K).
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t *__restrict__ src, int R, int K,
                                                  uint16_t *__restrict__ P, int64_t nks_p) {
  __shared__ __attribute__((aligned(1024))) char lds[32768];
  const int npair = (int)(nks_p >> 1);
  const int64_t rt = blockIdx.x / npair;
  const int kp = blockIdx.x - (int)(rt * npair);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int piece = i * 256 + threadIdx.x;          // 16-byte piece: row piece/8, columns 8 (piece%8)
    const int row = piece >> 3, cp = piece & 7;
    const int64_t gr = rt * 256 + row;
    const int col = kp * 64 + cp * 8;
    const u32x4 v = (gr < R && col < K) ? *(const u32x4 *)(src + gr * K + col)
                                        : u32x4{0u, 0u, 0u, 0u};
    const int kk = (cp * 8) & 31;
    const int off = ((cp >> 2) << 14) + (((((row >> 5) << 1) + (kk >> 4))) << 10) +
                    (pk_slot(row & 31, (kk >> 3) & 1, kk >> 4) << 4);
    *(u32x4 *)(lds + off) = v;
  }
  __syncthreads();
  uint16_t *dst = P + ((rt * nks_p + 2 * kp) << 13);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = i * 256 + threadIdx.x;
    *(u32x4 *)(dst + q * 8) = *(const u32x4 *)(lds + q * 16);
  }
}

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

// Transposed packing: the packed matrix PT has the columns of a row-major
// bf16 [R][K] source as rows (rows = K, columns = R, nks_t column slices).
// One workgroup per 256 rows x 64 columns of PT (two blocks, 32 KB): thread t
// loads the 8 x 8 source block at source rows 64 p + 8 (t / 32) and columns
// 256 rt + 8 (t % 32) (a wave reads 2 source rows x 512 contiguous bytes per
// instruction), transposes it in registers, places its 8 row pieces in LDS in
// packed order and the workgroup writes both blocks as one 32 KB copy.
// With PLAIN the same loads also fill the untransposed packed matrix P (rows
// R, nks_p column slices): the 64 source rows x 256 columns are the same two
// 32-row groups of 8 consecutive P blocks, i.e. 8 pieces of 4 KB, so the
// source is read once for both.  The two outputs take turns in one 32 KB LDS
// buffer, which keeps several workgroups (and their loads) per CU.
template <bool PLAIN>
__global__ __launch_bounds__(256) void pack_t_kernel(const uint16_t *__restrict__ src, int R,
                                                    int K, uint16_t *__restrict__ PT,
                                                    int64_t nks_t, uint16_t *__restrict__ P,
                                                    int64_t nks_p) {
  __shared__ __attribute__((aligned(1024))) char lds[32768];
  const int npair = (int)(nks_t >> 1);
  const int rt = blockIdx.x / npair;                  // row tile of PT = 256 source columns
  const int kp = blockIdx.x - rt * npair;             // pair of PT column slices = 64 source rows
  const int t = threadIdx.x;
  const int r0 = kp * 64 + (t >> 5) * 8;              // source rows r0..r0+7 = PT columns
  const int c0 = rt * 256 + (t & 31) * 8;             // source columns c0..c0+7 = PT rows
  u32x4 in[8], out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    in[i] = (r0 + i < R && c0 < K) ? *(const u32x4 *)(src + (int64_t)(r0 + i) * K + c0)
                                   : u32x4{0u, 0u, 0u, 0u};
  transpose8x8(in, out);
  const int k = (t >> 5) * 8;                         // PT column within the pair, 0..56
  const int kk = k & 31;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (t & 31) * 8 + j;                   // PT row within the tile
    const int off = ((k >> 5) << 14) + ((((r >> 5) << 1) + (kk >> 4)) << 10) +
                    (pk_slot(r & 31, (kk >> 3) & 1, kk >> 4) << 4);
    *(u32x4 *)(lds + off) = out[j];
  }
  __syncthreads();
  uint16_t *dst = PT + (((int64_t)rt * nks_t + 2 * kp) << 13);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = i * 256 + t;
    *(u32x4 *)(dst + q * 8) = *(const u32x4 *)(lds + q * 16);
  }
  if constexpr (PLAIN) {
    __syncthreads();                                  // every wave has copied PT out of LDS
    // P piece (t % 32) / 4 (column slice), fragment (row group, column half)
    const int kk = (c0 & 31);
    char *lp = lds + (((t & 31) >> 2) << 12);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (t >> 5) * 8 + i;                 // source row within the 64
      const int off = ((((r >> 5) << 1) + (kk >> 4)) << 10) +
                      (pk_slot(r & 31, (kk >> 3) & 1, kk >> 4) << 4);
      *(u32x4 *)(lp + off) = in[i];
    }
    __syncthreads();
    // 64 source rows = row groups 2 (kp % 4), +1 of P's row tile kp / 4
    const int64_t rtp = kp >> 2;
    uint16_t *dp = P + ((rtp * nks_p + 8 * (int64_t)rt) << 13) + ((kp & 3) << 11);
#pragma unroll
    for (int i = 0; i < 8; ++i)       // piece i: P block (rtp, 8 rt + i), 4 KB
      *(u32x4 *)(dp + ((int64_t)i << 13) + t * 8) = *(const u32x4 *)(lds + (i << 12) + t * 16);
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
// lane that holds it.  The logits tile (8 consecutive blocks of Zp) is
// stored straight from the accumulators in 512-byte half-fragments, as
// bf16(z - m) with m the token's maximum over the wave's 128 vocabulary ids
// (written to pmt for dlogits).  Rounding then costs a relative 2^-9 of
// m - z, not of z: exp(z - lse) keeps its accuracy however large the
// logits or a common shift of a token's logits, and the entries that carry
// the probability (z near m) are stored almost exactly.
template <bool VTAIL>
__global__ __launch_bounds__(NTHREADS, 1) void fwd_tile_kernel(
    const uint16_t *__restrict__ Wp, const uint16_t *__restrict__ Xp, int64_t nks_h,
    const int64_t *__restrict__ labels_c, int64_t ii, int c, int H, int V,
    uint16_t *__restrict__ Zp, int64_t nks_z, float *__restrict__ pm, float *__restrict__ ps,
    float *__restrict__ pmt, float *__restrict__ zy, int64_t nvt, int vt0, int nct, int store_z) {
  using T = FwdTile;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int vt = vt0 + tile / nct, ct = tile % nct;
  const int m0 = vt * T::BM, n0 = ct * T::BN;

  const Op a{Wp + (int64_t)vt * nks_h * 8192, 0, 0};
  const Op b{Xp + (int64_t)ct * nks_h * 8192, 0, 0};
  f32x16 acc[4][4];
  zero_acc<T>(acc);
  mainloop<T>(a, b, H, smem, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int vrow0 = m0 + wm * 128 + 4 * (lane >> 5);   // row r = 32 i + 8 (e/4) + e%4
  const int vlim = V - vrow0;                          // rows r < vlim exist
  const int64_t part = 2 * (int64_t)vt + wm;
  float msub[4];                                       // the maximum each token's stored logits are taken from
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
    const float ms = (VTAIL && mx == -INFINITY) ? 0.f : mx;
    const float ml = ms * kLog2e;
    msub[j] = ms;
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
      if (store_z) pmt[part * c + tok] = ms;
    }
  }

  if (store_z) {
    // Straight from the accumulators: for one (i, j, g) the lanes hold 32
    // consecutive tokens x 4 consecutive vocabulary ids each (lanes 32..63
    // the next 4), i.e. the 32 slots of one half of a Zp fragment, so each
    // store instruction writes 512 contiguous bytes.  Rows past V hold
    // products with Wp's zero padding; dlogits zeroes them.
    uint16_t *zt = Zp + ((int64_t)ct * nks_z + 8 * (int64_t)vt) * 8192 + 4 * (lane >> 5);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int h = g & 1, f = g >> 1;
      uint16_t *zg = zt + (f << 9) + (pk_slot(lane & 31, h, f) << 3);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // vocabulary slice wm 4 + i of the tile, token row group wn 4 + j
          uint2 pk;
          pk.x = pack_bf16x2(acc[i][j][4 * g] - msub[j], acc[i][j][4 * g + 1] - msub[j]);
          pk.y = pack_bf16x2(acc[i][j][4 * g + 2] - msub[j], acc[i][j][4 * g + 3] - msub[j]);
          *(uint2 *)(zg + ((wm * 4 + i) << 13) + ((wn * 4 + j) << 10)) = pk;
        }
    }
  }
}

// ---------------------------------------------------------------- dlogits
// One workgroup per 16 KB block of Zp (256 tokens x 32 vocabulary columns),
// four 16-byte slots per thread (one token, 8 consecutive vocabulary columns
// each), in memory order: pass k of a wave covers 1 KB contiguous, and all
// four loads are in flight before any arithmetic.  In place, from the stored
// Z - m (m the token's maximum over the block's 128-wide partial, from pmt):
// G = w_r (exp(Z - lse) - onehot(y)) on valid tokens, 0 on ignored tokens and
// outside [0, c) x [0, V); w_r = wrow_c[r] if given, else sc->scale
// (1 / N_valid for the mean loss).
constexpr int kDlSlots = 4;

__global__ __launch_bounds__(256) void dlogits_kernel(
    uint16_t *__restrict__ Zp, int64_t nks_z, int c, int V, const float *__restrict__ pmt,
    const float *__restrict__ lse_c, const int64_t *__restrict__ labels_c, int64_t ii,
    const float *__restrict__ wrow_c, const Scalars *__restrict__ sc) {
  // slot u = (blk * 16 + f) * 64 + sl of block blk = (rt, ks); thread t of the
  // block takes f = t / 64 + 4 k, sl = t % 64: slot sl = 32 h + (r % 32 ^ 4 h ^ 8 (f % 2))
  const int64_t blk = blockIdx.x;
  const int64_t rt = blk / nks_z, ks = blk - rt * nks_z;
  const int w = threadIdx.x >> 6, sl = threadIdx.x & 63, h = sl >> 5;
  const int v0 = (int)(ks * 32) + (w & 1) * 16 + h * 8;
  const int rr = ((sl & 31) ^ (h << 2) ^ ((w & 1) << 3));
  uint16_t *zb = Zp + (blk << 13) + ((int64_t)threadIdx.x << 3);
  // the block's 32 vocabulary columns lie in one 128-wide partial
  const float *mrow = pmt + (ks >> 2) * c;
  u32x4 z[kDlSlots];
#pragma unroll
  for (int k = 0; k < kDlSlots; ++k) z[k] = *(const u32x4 *)(zb + (k << 11));
#pragma unroll
  for (int k = 0; k < kDlSlots; ++k) {
    const int r = (int)(rt * 256) + ((w >> 1) + 2 * k) * 32 + rr;
    int64_t y = ii;
    float l2 = 0.f, inv = 0.f;
    if (r < c) {
      y = labels_c[r];
      l2 = (lse_c[r] - mrow[r]) * kLog2e;     // stored values are z - m
      inv = wrow_c ? wrow_c[r] : sc->scale;
    }
    const bool valid = r < c && y != ii;
    u32x4 g;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      float fv[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int v = v0 + 2 * d + hh;
        const float zz = hh ? bf16_hi(z[k][d]) : bf16_lo(z[k][d]);
        const float e = __builtin_amdgcn_exp2f(zz * kLog2e - l2) - ((int64_t)v == y ? 1.f : 0.f);
        fv[hh] = (valid && v < V) ? e * inv : 0.f;
      }
      g[d] = pack_bf16x2(fv[0], fv[1]);
    }
    *(u32x4 *)(zb + (k << 11)) = g;
  }
}

// ---------------------------------------------------------------- dX (split-K)
// Unit (s, mt, nt): dxp[s][tok][h] = sum over vocabulary in split s of
// G[tok][v] W[v][h].  G from Zp (rows = tokens), W from WTp (rows = hidden),
// both with the vocabulary along k.
__global__ __launch_bounds__(NTHREADS, 1) void dx_kernel(
    const uint16_t *__restrict__ Gp, int64_t nks_z, const uint16_t *__restrict__ WTp,
    int c, int H, int V, int64_t ksplit, int nmt, int nnt, float *__restrict__ dxp) {
  using T = DxTile;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int per = nmt * nnt;
  // token tile fastest: the few token tiles of a split share each W block
  const int s = unit / per, rem = unit - s * per;
  const int nt = rem / nmt, mt = rem - nt * nmt;
  const int m0 = mt * T::BM, n0 = nt * T::BN;
  const int64_t kb = (int64_t)s * ksplit;
  const int64_t ke = kb + ksplit < V ? kb + ksplit : V;
  const int klen = (int)(ke - kb);

  const Op a{Gp + ((int64_t)mt * nks_z + (kb >> 5)) * 8192, 0, 0};
  const Op b{WTp + ((int64_t)nt * nks_z + (kb >> 5)) * 8192, 0, 0};
  f32x16 acc[4][4];
  zero_acc<T>(acc);
  mainloop<T>(a, b, klen, smem, acc);

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
// BM x BN = 256 x 128 tiles, two workgroups per CU so that one's dW traffic
// overlaps the other's MFMA work; G from Zp and X from Xp, both read
// transposed.
//
// The epilogue goes through LDS in two halves of 128 rows (BN fp32 per row)
// so that dW is read and written in row-contiguous 16-byte pieces: the waves
// holding a half write their accumulators, then every thread moves its
// pieces.  A thread's loads of the current dW for a half are issued before
// the accumulators of that half reach LDS (for the second half, right after
// the first half's stores), so their latency overlaps the staging; the
// barriers wait for LDS only, not for these loads.
// 128-byte column blocks of an LDS row are XOR-swizzled by row bit 2 so the
// two rows a write instruction covers use both halves of the banks.
template <int BN>
__device__ __forceinline__ int dwst_off(int r, int col) {   // bytes
  return r * (BN * 4) + (((col >> 5) ^ ((r >> 2) & 1)) << 7) + ((col & 31) << 2);
}

template <class T, int OCC>
__global__ __launch_bounds__(NTHREADS, OCC) void dw_kernel(
    const uint16_t *__restrict__ Gp, int64_t nks_z, const uint16_t *__restrict__ Xp,
    int64_t nks_h, int c, int H, int V, int nvt, int nht, float *__restrict__ dW, int accumulate) {
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  int vt, ht;
  grouped<8>(xcd_remap(blockIdx.x, gridDim.x), nvt, nht, vt, ht);
  const int m0 = vt * T::BM, n0 = ht * T::BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;

  f32x16 acc[T::MI][T::NI];
  zero_acc<T>(acc);
  const Op a{Gp + (int64_t)(m0 >> 5) * 8192, nks_z * 8192, 0};
  const Op b{Xp + (int64_t)(n0 >> 5) * 8192, nks_h * 8192, 0};
  mainloop_tt<T>(a, b, c, smem, acc);

  constexpr int TPR = T::BN / 4;            // threads per row: one 16-byte piece each
  constexpr int RPP = NTHREADS / TPR;       // rows per pass of the workgroup
  constexpr int NQ = 128 / RPP;             // pieces per thread per half
  static_assert(T::BM == 256 && T::LDS >= 128 * T::BN * 4, "epilogue half tile must fit in LDS");
  // thread t takes piece t % TPR of rows t / TPR + RPP q of each half
  const int col = (threadIdx.x % TPR) * 4;
  const int h = n0 + col;
  const int rb = threadIdx.x / TPR;
  // dW is touched once per chunk: non-temporal accesses keep it from
  // evicting the G and X strips that the next tiles reuse from L2
  f32x4 old[NQ];
  auto load_old = [&](int half) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int v = m0 + half * 128 + rb + RPP * q;
      const bool ok = v < V && h < H;            // H % 8 == 0: a started piece fits
      old[q] = (accumulate && ok) ? __builtin_nontemporal_load((const f32x4 *)(dW + (int64_t)v * H + h))
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_old(0);
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
            const int cc = wn * T::WN + 32 * j + (lane & 31);
            *(float *)(smem + dwst_off<T::BN>(r, cc)) = acc[i][j][e];
          }
    }
    // the half is in LDS (a fence-free barrier: the loads stay in flight)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    bar();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int r = rb + RPP * q;
      const int v = m0 + half * 128 + r;
      if (v < V && h < H) {
        const f32x4 add = *(const f32x4 *)(smem + dwst_off<T::BN>(r, col));
        __builtin_nontemporal_store(old[q] + add, (f32x4 *)(dW + (int64_t)v * H + h));
      }
    }
    if (half == 0) load_old(1);
    // every thread has read its pieces before the next half overwrites LDS
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    bar();
  }
}

inline int grid_for(int64_t n, int block, int cap) {
  int64_t g = (n + block - 1) / block;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace

hipError_t launch_pack_bf16(const uint16_t *src, int R, int K, uint16_t *P, int64_t nks_p,
                            hipStream_t s) {
  // nks_p is a multiple of 8, so column pairs of slices tile it exactly
  const int64_t nwg = (int64_t)(R + 255) / 256 * (nks_p / 2);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)nwg), dim3(256), 0, s, src, R, K, P, nks_p);
  return hipGetLastError();
}

hipError_t launch_fwd_tile_bf16(const uint16_t *Wp, const uint16_t *Xp, int64_t nks_h,
                                const int64_t *labels_c, int64_t ii, int c, int H, int V,
                                uint16_t *Zp, int64_t nks_z, float *pm, float *ps, float *pmt,
                                float *zy, int64_t nvt, bool store_z, hipStream_t s) {
  const int nct = (c + FwdTile::BN - 1) / FwdTile::BN;
  const int nfull = V / FwdTile::BM;                 // vocabulary tiles inside V
  if (nfull > 0) {
    hipLaunchKernelGGL(fwd_tile_kernel<false>, dim3(nfull * nct), dim3(NTHREADS), 0, s, Wp, Xp,
                       nks_h, labels_c, ii, c, H, V, Zp, nks_z, pm, ps, pmt, zy, nvt, 0, nct,
                       store_z ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (V % FwdTile::BM != 0) {
    hipLaunchKernelGGL(fwd_tile_kernel<true>, dim3(nct), dim3(NTHREADS), 0, s, Wp, Xp, nks_h,
                       labels_c, ii, c, H, V, Zp, nks_z, pm, ps, pmt, zy, nvt, nfull, nct,
                       store_z ? 1 : 0);
  }
  return hipGetLastError();
}

hipError_t launch_dlogits_bf16(uint16_t *Zp, int64_t nks_z, int c, int V, const float *pmt,
                               const float *lse_c, const int64_t *labels_c, int64_t ii,
                               const float *wrow_c, const Scalars *sc, hipStream_t s) {
  // one workgroup per 16 KB block of the row tiles that cover [0, c), every slice of Zp
  const int64_t nblk = (int64_t)((c + 255) / 256) * nks_z;
  static_assert(kDlSlots * 256 * 16 == 16384, "a workgroup covers one block");
  hipLaunchKernelGGL(dlogits_kernel, dim3((unsigned)nblk), dim3(256), 0, s, Zp, nks_z, c, V, pmt,
                     lse_c, labels_c, ii, wrow_c, sc);
  return hipGetLastError();
}

hipError_t launch_pack_t_bf16(const uint16_t *src, int R, int K, uint16_t *PT, int64_t nks_t,
                              uint16_t *P, int64_t nks_p, hipStream_t s) {
  // nks_t is a multiple of 8, so column pairs of slices tile it exactly
  const int64_t nwg = (int64_t)(K + 255) / 256 * (nks_t / 2);
  if (P)
    hipLaunchKernelGGL(pack_t_kernel<true>, dim3((unsigned)nwg), dim3(256), 0, s, src, R, K, PT,
                       nks_t, P, nks_p);
  else
    hipLaunchKernelGGL(pack_t_kernel<false>, dim3((unsigned)nwg), dim3(256), 0, s, src, R, K, PT,
                       nks_t, P, nks_p);
  return hipGetLastError();
}

hipError_t launch_dx_bf16(const uint16_t *Gp, int64_t nks_z, const uint16_t *WTp, int c, int H,
                          int V, int splitk, int64_t ksplit, float *dxp, hipStream_t s) {
  const int nmt = (c + DxTile::BM - 1) / DxTile::BM, nnt = (H + DxTile::BN - 1) / DxTile::BN;
  hipLaunchKernelGGL(dx_kernel, dim3(splitk * nmt * nnt), dim3(NTHREADS), 0, s, Gp, nks_z, WTp,
                     c, H, V, ksplit, nmt, nnt, dxp);
  return hipGetLastError();
}

hipError_t launch_dx_reduce_bf16(const float *dxp, int splitk, int c, int H, uint16_t *dXc,
                                 hipStream_t s) {
  const int64_t n4 = (int64_t)c * H / 4;
  hipLaunchKernelGGL(dx_reduce_kernel, dim3(grid_for(n4, 256, 256 * 32)), dim3(256), 0, s, dxp,
                     splitk, c, H, dXc);
  return hipGetLastError();
}

hipError_t launch_dw_bf16(const uint16_t *Gp, int64_t nks_z, const uint16_t *Xp, int64_t nks_h,
                          int c, int H, int V, float *dW, bool accumulate, hipStream_t s) {
  const int nvt = (V + DwTile::BM - 1) / DwTile::BM, nht = (H + DwTile::BN - 1) / DwTile::BN;
  hipLaunchKernelGGL((dw_kernel<DwTile, kDwOcc>), dim3(nvt * nht), dim3(NTHREADS), 0, s, Gp, nks_z, Xp, nks_h, c, H,
                     V, nvt, nht, dW, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace flce
