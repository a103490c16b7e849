// bf16 MFMA GEMMs of the chunked fused linear cross-entropy (gfx950), and
// the data movement that feeds them.
//
// W is read where it lies (row-major [V][H], never copied).  Per chunk of c
// tokens (the chain rule through the LM-head projection
// Z = X W^T that the Liger Kernel pages fuse with the cross-entropy loss):
//   pack      X_c -> Xp (rows = tokens, k = hidden);
//   forward   Z_c^T = W X_c^T      M = V (vocab), N = c (tokens), K = H
//             + epilogue: per (token, 128-vocab half tile) max m and sum of
//               exp, the target logit, and bf16((z - m) log2 e) into Zp (rows =
//               tokens, k = vocabulary);
//   dlogits   Zp rewritten in place into G = (softmax - onehot) / N_valid;
//   dX        dX_c  = G_c W        M = c, N = H, K = V (split-K, fp32 partials),
//             W read transposed;
//   dW        dW   (+)= G_c^T X_c  M = V, N = H, K = c (fp32)
//
// GEMM tiles: a workgroup of 4 waves (2 x 2) computes a BM x BN fp32 tile with
// v_mfma_f32_32x32x16_bf16, each wave a (BM/2) x (BN/2) quarter of 32 x 32
// blocks.  Operands flow global -> LDS through direct-to-LDS buffer loads
// (buffer_load_dwordx4 ... lds: lane l of a wave writes 16 bytes at the LDS
// address in M0 + 16 l; the source is a buffer descriptor for the slice, a
// scalar offset for the 1 KB piece and the lane's constant 16-byte offset,
// or for W read in place the lane's offset into the rows) in k-slices of 32,
// STAGES slices in flight, each admitted by an explicit vmcnt wait and one
// s_barrier.
//
// The packed layout (Xp, Zp): a matrix of R rows and K columns is stored
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

#include <atomic>
#include <type_traits>

namespace flce {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 32;             // k per pipeline slice
constexpr int NTHREADS = 256;
constexpr float kLog2e = 1.4426950408889634f;

enum Kind { PACKED = 0, PACKED_T = 1, ROW = 2, ROWT = 3 };

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
  static constexpr int NA = A_BYTES / 4096, NB = B_BYTES / 4096;   // copies per thread per slice
  static constexpr int NPER = NA + NB;
  static constexpr int LDS = STAGES * STAGE_BYTES;
};

// One GEMM operand tile in a packed matrix (byte addresses).
//   PACKED:   base = the block of the tile's first row and of the range's
//             first k; slice s at base + 16 KB s.
//   PACKED_T: base = the block of row tile 0 and of the column slice of the
//             tile's first operand row; ld = bytes of one row tile of the
//             matrix; kb = the range's first k, a row of the matrix (a
//             multiple of 32).
//   ROW:      base = the tile's first row; ld = bytes per matrix row; kb =
//             the range's first k (a column of the matrix, a multiple of 32);
//             end = the end of the matrix (rows past it read as zero).
//   ROWT:     base = the matrix's first row at the tile's first column; ld =
//             bytes per matrix row; kb = the range's first k (a row of the
//             matrix, a multiple of 32); end as for ROW.
struct Op {
  const char *base;
  int64_t ld;
  int64_t kb;
  const char *end;
};

// Buffer descriptor of a slice: raw (stride 0) 32-bit words, no range check
// that a packed slice could reach.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const char *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, 0x7fffffff, 0x00020000);
}

// The copies of one operand tile: this wave's pieces of a k-slice, at
// scalar offsets fixed for the whole loop, and the slice's address, advanced
// once per slice (no per-copy address arithmetic in the loop).  Piece i of
// the wave is 1 KB piece blk = 4 i + wave of the slice, written at LDS byte
// address stage + 1 KB blk.  PACKED_T pieces 2q, 2q+1 are the two fragments
// of operand rows 32q..32q+31.  Only the lane's 16-byte offset is per lane.
//   ROW:      piece blk = 16 matrix rows x 64 bytes (rows 16 blk ..); lane l
//             copies row 16 blk + l/4, 16-byte chunk (l%4) ^ (l/16 % 4), so
//             that its LDS position holds the swizzled layout;
//   ROWT:     piece blk = matrix rows 2 blk, 2 blk + 1 of the slice, 512
//             bytes each; lane l copies row 2 blk + l/32, chunk
//             (l%32) ^ 4 ((2 blk + l/32) % 4).
// Row-major pieces take their offsets in the lane's offset, where the
// descriptor's range check applies: rows past the matrix's end read as
// zero.
template <int KIND, int NP>
struct OpStream {
  static constexpr bool RM = KIND == ROW || KIND == ROWT;
  const char *ptr;         // the slice copied next
  const char *end;         // row-major: the end of the matrix
  int64_t ld;              // PACKED_T: bytes of one row tile; row-major: bytes per row
  int kr;                  // PACKED_T: the matrix row of ptr's slice
  int soff[NP];            // packed: piece offsets within a slice (bytes)
  int voff[RM ? NP : 1];   // row-major: the lane's offsets of the pieces
  uint32_t loff[NP];       // piece offsets within the operand's stage area

  __device__ __forceinline__ void init(const Op &op) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    ld = op.ld;
    kr = (int)op.kb;
    end = op.end;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int blk = i * 4 + w;
      soff[i] = KIND == PACKED ? blk * 1024 : (blk >> 1) * 16384 + (blk & 1) * 1024;
      loff[i] = (uint32_t)(blk * 1024);
      if constexpr (KIND == ROW)
        voff[i] = (int)((16 * blk + (l >> 2)) * ld) + 16 * ((l & 3) ^ ((l >> 4) & 3));
      else if constexpr (KIND == ROWT)
        voff[i] = (int)((2 * blk + (l >> 5)) * ld) + 16 * ((l & 31) ^ (4 * ((2 * blk + (l >> 5)) & 3)));
    }
    if constexpr (KIND == PACKED) ptr = op.base;
    else if constexpr (KIND == PACKED_T) ptr = op.base + (int64_t)(kr >> 8) * ld + (((kr & 255) >> 5) << 11);
    else if constexpr (KIND == ROW) ptr = op.base + 2 * op.kb;
    else ptr = op.base + op.kb * ld;
  }
  // on to the next k-slice if go (selects, not a branch, inside the loop)
  __device__ __forceinline__ void advance(bool go = true) {
    if constexpr (KIND == PACKED) {
      ptr += go ? 16384 : 0;
    } else if constexpr (KIND == PACKED_T) {
      const int64_t inc = (kr & 255) == 224 ? ld - 7 * 2048 : 2048;
      ptr += go ? inc : 0;
      kr += go ? 32 : 0;
    } else if constexpr (KIND == ROW) {
      ptr += go ? 64 : 0;
    } else {
      ptr += go ? 32 * ld : 0;
    }
  }
  // on to slice CK of a range that starts at a multiple of 256 rows (the
  // wrap into the next row tile known at compile time)
  template <int CK>
  __device__ __forceinline__ void advance_to() {
    if constexpr (KIND == PACKED_T) {
      ptr += (CK - 1) % 8 == 7 ? ld - 7 * 2048 : 2048;
      kr += 32;
    } else {
      advance();
    }
  }
  __device__ __forceinline__ void copy(int i, uint32_t stage) const {
    if constexpr (RM) {
      // bytes from ptr to the matrix's end (ptr never passes it: every slice
      // starts inside the matrix), clamped to the descriptor's range; 32-bit
      // scalar arithmetic only
      const uint64_t left = (uint64_t)(end - ptr);
      uint32_t lo = (uint32_t)left, hi = (uint32_t)(left >> 32);
      asm("" : "+s"(hi));               // keeps the test a 32-bit scalar compare
      const int nrec = hi ? 0x7fffffff : (int)min(lo, 0x7fffffffu);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(ptr), (short)0, nrec, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(uintptr_t)(stage + loff[i]), 16, voff[i], 0, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(slice_rsrc(ptr), (lds_void *)(uintptr_t)(stage + loff[i]), 16,
                                               (threadIdx.x & 63) * 16, soff[i], 0, 0);
    }
  }
};

template <class T>
struct Streams {
  OpStream<T::KA, T::NA> a;
  OpStream<T::KB, T::NB> b;
  // copy g (0 .. NPER - 1) of a stage: the A operand's pieces, then B's
  __device__ __forceinline__ void copy(int g, uint32_t st) const {
    if (g < T::NA) a.copy(g, st);
    else b.copy(g - T::NA, st + T::A_BYTES);
  }
  __device__ __forceinline__ void advance(bool go = true) {
    a.advance(go);
    b.advance(go);
  }
  template <int CK>
  __device__ __forceinline__ void advance_to() {
    a.template advance_to<CK>();
    b.template advance_to<CK>();
  }
};

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

// Compile-time loop: f(ic<B>{}), ..., f(ic<E - 1>{}), so that loop indices
// can select immediates.
template <int V>
struct ic {
  static constexpr int value = V;
};
template <bool V>
struct bc {
  static constexpr bool value = V;
};
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(ic<B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------- fragment reads
// The fragment reads are issued as inline asm and awaited explicitly
// (s_waitcnt lgkmcnt(0), tied to the fragment registers so that no MFMA
// moves above it): the compiler would otherwise guard each LDS read with a
// wait for every direct-to-LDS copy in flight, draining the copy pipeline
// once per slice.  Volatile asm statements keep their source order, which is
// the issue order.
//
// Two more layouts read an operand straight from a row-major bf16 matrix
// (the weight W), without a packed copy:
//   ROW   rows of the matrix are rows of the GEMM operand (k runs along a
//         row): a stage holds the tile's rows as 64-byte pieces (32 k), one
//         after another, with the four 16-byte chunks of row r XOR-swizzled
//         by (r/4) % 4; a fragment is one 16-byte read per lane;
//   ROWT  columns of the matrix are rows of the GEMM operand (k runs down
//         the matrix's rows): a stage holds 32 matrix rows of 512 bytes (the
//         tile's 256 columns), the 16-byte chunks of matrix row k
//         XOR-swizzled by 4 (k % 4); a fragment is two transposing reads.
// Both swizzles keep every read conflict-free (an aligned group of 16 lanes
// of a 16-byte read covers 256 distinct bytes; each half-wave of a
// transposing read, 32 distinct 8-byte bank pairs).
constexpr bool kind_tr(int kind) { return kind == PACKED_T || kind == ROWT; }

template <int KIND>
struct Frag {                // one 16-byte read
  bf16x8 v;
};
template <>
struct Frag<PACKED_T> {      // two transposing 8-byte reads
  i16x4 lo, hi;
};
template <>
struct Frag<ROWT> {
  i16x4 lo, hi;
};
template <int KIND>
constexpr int reads_per_frag() { return kind_tr(KIND) ? 2 : 1; }

template <int IMM>
__device__ __forceinline__ void rd_b128(bf16x8 &dst, uint32_t a) {
  static_assert(IMM >= 0 && IMM < 65536, "LDS instruction offset range");
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(a), "i"(IMM));
}
template <int IMM>
__device__ __forceinline__ void rd_tr(i16x4 &dst, uint32_t a) {
  static_assert(IMM >= 0 && IMM < 65536, "LDS instruction offset range");
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(dst) : "v"(a), "i"(IMM));
}

// A lane's read addresses (bytes, within a stage) for an operand block of NF
// fragments, rows r0 ... (r0 a multiple of 32):
//   PACKED, ROW  v[kk]: fragment 0's read of half-step kk;
//   PACKED_T     v[0], v[1]: fragment 0's low and high reads of half-step 0;
//   ROWT         v[i]: fragment i's low read of half-step 0.
// Every other read is a fixed offset away, reached through the
// instruction's immediate: fragment i of PACKED, ROW and PACKED_T at
// 2048 i; PACKED_T's half-step kk at 256 kk more (k + 16 flips bit 4 of
// the slot, which no XOR term touches; this was checked for every lane);
// ROWT's high read at 2048 (k + 4, same swizzle) and half-step kk at
// 8192 kk (k + 16).
template <int KIND, int NF>
struct OpBases {
  uint32_t v[KIND == ROWT ? NF : 2];
};

template <int KIND, int NF>
__device__ __forceinline__ void rd_bases(int r0, OpBases<KIND, NF> &b) {
  const int l = threadIdx.x & 63;
  if constexpr (KIND == PACKED) {
    b.v[0] = (uint32_t)((((r0 >> 5) << 1) << 10) + (pk_slot(l & 31, l >> 5, 0) << 4));
    b.v[1] = (uint32_t)(((((r0 >> 5) << 1) + 1) << 10) + (pk_slot(l & 31, l >> 5, 1) << 4));
  } else if constexpr (KIND == ROW) {
    // lane l: row r0 + l%32, k-half l/32 of a 16-k half-step
    const int r = l & 31, h = l >> 5, sw = (r >> 2) & 3;
    b.v[0] = (uint32_t)((r0 + r) * 64 + 16 * ((0 + h) ^ sw));
    b.v[1] = (uint32_t)((r0 + r) * 64 + 16 * ((2 + h) ^ sw));
  } else {
    // lane j of a 16-lane group names the 4 operand rows n..n+3 at one k
    const int g = l >> 4, j = l & 15;
    const int n = r0 + ((g & 1) << 4) + ((j & 3) << 2);
    const int k = ((g >> 1) << 3) + (j >> 2);
    if constexpr (KIND == PACKED_T) {
      const int h = (n >> 3) & 1, f = (n >> 4) & 1;
      const int p = ((((n >> 5) << 1) + f) << 10) + ((n & 7) << 1);
      b.v[0] = (uint32_t)(p + (pk_slot(k, h, f) << 4));
      b.v[1] = (uint32_t)(p + (pk_slot(k + 4, h, f) << 4));
    } else {
#pragma unroll
      for (int i = 0; i < NF; ++i)
        b.v[i] = (uint32_t)(k * 512 + 16 * (((n >> 3) + 4 * i) ^ (4 * (k & 3))) + 2 * (n & 7));
    }
  }
}

// Read Q of half-step KK of an operand with NF fragments.
template <int KIND, int KK, int Q, int NF>
__device__ __forceinline__ void rd_issue(const OpBases<KIND, NF> &b, Frag<KIND> (&f)[NF]) {
  if constexpr (KIND == PACKED || KIND == ROW) {
    rd_b128<2048 * Q>(f[Q].v, b.v[KK]);
  } else if constexpr (KIND == PACKED_T) {
    constexpr int fi = Q >> 1;
    constexpr int imm = 2048 * fi + 256 * KK;
    if constexpr (Q & 1) rd_tr<imm>(f[fi].hi, b.v[1]);
    else rd_tr<imm>(f[fi].lo, b.v[0]);
  } else {
    constexpr int fi = Q >> 1;
    constexpr int imm = 8192 * KK + 2048 * (Q & 1);
    if constexpr (Q & 1) rd_tr<imm>(f[fi].hi, b.v[fi]);
    else rd_tr<imm>(f[fi].lo, b.v[fi]);
  }
}

template <int KIND, int NF>
__device__ __forceinline__ void frag_tie(Frag<KIND> (&f)[NF]) {
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    if constexpr (!kind_tr(KIND)) asm volatile("" : "+v"(f[i].v));
    else asm volatile("" : "+v"(f[i].lo), "+v"(f[i].hi));
  }
}

template <int KIND>
__device__ __forceinline__ bf16x8 frag_val(const Frag<KIND> &f) {
  if constexpr (!kind_tr(KIND)) return f.v;
  else return __builtin_bit_cast(bf16x8, __builtin_shufflevector(f.lo, f.hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A wave's fragments of one half-step.
template <class T>
struct Frags {
  Frag<T::KA> a[T::MI];
  Frag<T::KB> b[T::NI];
};

// Wait for every LDS read of this wave and tie the fragments to the wait.
template <class T>
__device__ __forceinline__ void frags_wait(Frags<T> &f) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  frag_tie<T::KA>(f.a);
  frag_tie<T::KB>(f.b);
}

// Read addresses of one stage, A's then B's.
template <class T>
struct Bases {
  OpBases<T::KA, T::MI> a;
  OpBases<T::KB, T::NI> b;
  __device__ __forceinline__ Bases plus(uint32_t o) const {
    Bases r = *this;
#pragma unroll
    for (auto &x : r.a.v) x += o;
#pragma unroll
    for (auto &x : r.b.v) x += o;
    return r;
  }
};

// Read Q of half-step KK (A's reads first, then B's).
template <class T, int KK, int Q>
__device__ __forceinline__ void frag_read(const Bases<T> &s, Frags<T> &f) {
  constexpr int RA = T::MI * reads_per_frag<T::KA>();
  if constexpr (Q < RA) rd_issue<T::KA, KK, Q>(s.a, f.a);
  else rd_issue<T::KB, KK, Q - RA>(s.b, f.b);
}

// MFMA i of a half-step (block row i / NI, block column i % NI), fenced so
// that the scheduler keeps the source order of MFMAs, reads and copies.
template <class T>
__device__ __forceinline__ void mfma_at(int i, const Frags<T> &f, f32x16 (&acc)[T::MI][T::NI]) {
  const int a = i / T::NI, b = i % T::NI;
  __builtin_amdgcn_sched_barrier(0);
  acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_val<T::KA>(f.a[a]), frag_val<T::KB>(f.b[b]),
                                                      acc[a][b], 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// A main-loop hook issues vector-memory loads of its own during the first NU
// iterations (compile-time indices, so that the values can go to fixed
// registers) and works on the accumulators during those iterations and after
// the loop.  Its loads are issued in the first half-step of an iteration:
// LP of them in the prologue, after the prologue's copies, and loads(u) in
// iteration u.  NoHook issues none.
struct NoHook {
  static constexpr int NU = 0, LP = 0;
  static constexpr int loads(int) { return 0; }
  template <int U, int I>
  __device__ __forceinline__ void load() {}
  template <int U, int I, class A>
  __device__ __forceinline__ void add(A &) {}
  __device__ __forceinline__ void prologue() {}
  template <class A>
  __device__ __forceinline__ void drain(A &) {}
};

// vmcnt of the wait in iteration t (slice t+1 must have landed): the number
// of vector-memory operations issued after slice t+1's last copy, for the
// issue order prologue = copies of slices 0 .. S-2 (G each) then LP loads;
// iteration u = loads(u) loads, then the G copies of slice u + S - 1.  t = -1
// is the prologue's own wait (slice 0).  Vector-memory operations complete
// in issue order, so waiting for this count admits slice t+1 and everything
// issued before it.
template <class H>
constexpr int hook_loads_upto(int t) {
  int n = 0;
  for (int u = 0; u <= t; ++u) n += H::loads(u);
  return n;
}
template <class H, int S, int G>
constexpr int wait_count(int t) {
  if (t < 0) return (S - 2) * G + H::LP;
  if (t + 1 <= S - 2) return (S - 3) * G + H::LP + hook_loads_upto<H>(t);
  return (S - 3) * G + hook_loads_upto<H>(t) - hook_loads_upto<H>(t - S + 2);
}
template <class H, int S, int G>
constexpr int max_wait_count() {
  int m = 0;
  for (int t = -1; t <= H::NU + S; ++t) m = wait_count<H, S, G>(t) > m ? wait_count<H, S, G>(t) : m;
  return m;
}

// Tiles worked one after another by a resident workgroup: the main loop's
// last iterations copy the next tile's first STAGES - 1 slices into the ring
// instead of the last slice again, so that they arrive while the caller
// stores the tile.  The next tile's loop then starts warm: it issues its
// hook's prologue, and one full wait (which also covers the stores still in
// flight, whose completion order against loads is not guaranteed) admits
// them.  The caller guarantees
// nk >= Hook::NU + STAGES slices (the unrolled iterations never reach the
// tile's end) and ranges that start at row 0.  NoChain is the single-tile
// loop.
struct NoChain {
  static constexpr bool on = false;
};
struct Chain {
  static constexpr bool on = true;
  bool warm;               // this tile's first slices were copied by the previous tile's loop
  int rb;                  // ring slot of this tile's slice 0
  bool has_next;           // a next tile follows
  Op na, nb;               // its operands
};

// acc[i][j] is the 32 x 32 block (i, j) of the wave's quarter.  Lane l of
// block (i, j), register e, holds row 32 i + 8 (e/4) + 4 (l/32) + e%4 and
// column 32 j + l%32 of the quarter.  acc enters initialised by the caller.
//
// Each 32-deep slice is two MFMA half-steps (k 0..15, 16..31).  The wait and
// barrier that admit slice t+1 sit between the two half-steps of slice t, so
// the barrier waits with MFMAs in flight.  The reads of a half-step's
// fragments go out during the previous half-step, RPM after each MFMA from
// its first one, so they have most of a half-step to land.  Slice
// t+STAGES-1 is copied into the buffer of slice t-1, whose reads every wave
// finished before that barrier; its copies go out one after every CSP-th
// MFMA of the second half-step rather than in one burst, which would hold up
// the MFMA issue.  Every iteration issues one slice of copies (past the end,
// the last slice again into a slot that is not read again, or the next
// tile's first slices), so the wait is always for all but the newest
// STAGES-3 slices (plus the hook's loads), and every slice, the last one
// included, runs the same loop body (its reads of the half-step after the
// last fetch a slice that nothing uses; a peeled last slice made the
// compiler move the accumulators to other registers after the loop).  Packed
// operands carry zero padding up to whole slices, so their copies need no
// bounds check; row-major ones (W) end their descriptors at the matrix's
// end.  The first Hook::NU iterations are unrolled; the caller guarantees
// that the loop has at least that many (nk >= NU).
template <class T, int RPM, int CSP, class Hook = NoHook, class Ch = NoChain>
__device__ __forceinline__ void mainloop(const Op &a, const Op &b, int klen, char *smem,
                                         f32x16 (&acc)[T::MI][T::NI], Hook &&hook = Hook{},
                                         const Ch &ch = Ch{}) {
  using HK = std::remove_reference_t<Hook>;
  constexpr int M = T::MI * T::NI;                 // MFMAs per half-step
  constexpr int R = T::MI * reads_per_frag<T::KA>() + T::NI * reads_per_frag<T::KB>();
  constexpr int G = T::NPER;
  constexpr int S = T::STAGES;
  static_assert(S >= 3, "the wait below admits one slice of STAGES - 1 in flight");
  static_assert(RPM * M >= R, "every fragment read of a half-step must be issued during the previous one");
  static_assert(max_wait_count<HK, S, G>() < 64, "vmcnt range");
  const int nk = (klen + BK - 1) / BK;
  if (Ch::on || nk > 0) {                          // chained tiles have nk >= NU + S
    const int w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
    const uint32_t lds0 = lds_addr(smem);
    Bases<T> z;
    rd_bases<T::KA>(wm * T::WM, z.a);
    rd_bases<T::KB>(wn * T::WN, z.b);
#pragma unroll
    for (auto &x : z.a.v) x += lds0;
#pragma unroll
    for (auto &x : z.b.v) x += lds0 + T::A_BYTES;
    auto stage_bases = [&](int s) { return z.plus((uint32_t)(s * T::STAGE_BYTES)); };
    int rb = 0;                                    // ring slot of slice 0
    if constexpr (Ch::on) rb = ch.rb;
    auto slot = [&](int s) { return (rb + s) % S; };
    // the prologue's slices 0 .. S-2 (the last slice again past the end)
    Streams<T> cs;
    cs.a.init(a);
    cs.b.init(b);
    bool warm = false;
    if constexpr (Ch::on) warm = ch.warm;
    if constexpr (Ch::on) {
      // ranges start at row 0 and have nk >= NU + S slices
      if (warm) {
        // slices 0 .. S-2 were copied by the previous tile's loop
        static_for<1, S - 1>([&](auto ss) { cs.template advance_to<decltype(ss)::value>(); });
        hook.prologue();
        wait_vm<0>();
      } else {
        static_for<0, S - 1>([&](auto ss) {
          constexpr int sl = decltype(ss)::value;
          if constexpr (sl > 0) cs.template advance_to<sl>();
#pragma unroll
          for (int g = 0; g < G; ++g) cs.copy(g, lds0 + (uint32_t)(slot(sl) * T::STAGE_BYTES));
        });
        hook.prologue();
        wait_vm<wait_count<HK, S, G>(-1)>();
      }
    } else {
#pragma unroll
      for (int s = 0; s < S - 1; ++s) {
        if (s > 0 && s < nk) cs.advance();
#pragma unroll
        for (int g = 0; g < G; ++g) cs.copy(g, lds0 + (uint32_t)(slot(s) * T::STAGE_BYTES));
      }
      hook.prologue();
      wait_vm<wait_count<HK, S, G>(-1)>();
    }
    bar();
    Frags<T> f0, f1;
    Bases<T> cur = stage_bases(rb);                // the stage of slice t
    int st = rb;
    static_for<0, R>([&](auto q) { frag_read<T, 0, decltype(q)::value>(cur, f0); });
    // one iteration; U >= 0 is an unrolled iteration of the hook, U < 0 a
    // runtime one
    auto body = [&](int t, auto uu) {
      constexpr int U = decltype(uu)::value;
      const int sn = st + 1 == S ? 0 : st + 1;
      const Bases<T> nxt = stage_bases(sn);
      const int ck = t + S - 1;                    // slice copied in this iteration
      const uint32_t cst = lds0 + (uint32_t)(slot(ck) * T::STAGE_BYTES);
      frags_wait<T>(f0);
      // first half-step; the reads of the second go out between its MFMAs
      static_for<0, M>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        mfma_at<T>(i, f0, acc);
        constexpr int q0 = i * RPM < R ? i * RPM : R, q1 = (i + 1) * RPM < R ? (i + 1) * RPM : R;
        static_for<q0, q1>([&](auto q) { frag_read<T, 1, decltype(q)::value>(cur, f1); });
        if constexpr (U >= 0) hook.template load<U, i>();
      });
      // slice t+1 must have landed; slices t+2 .. t+STAGES-2 may stay in flight
      if constexpr (U >= 0) wait_vm<wait_count<HK, S, G>(U)>();
      else wait_vm<(S - 3) * G>();                 // at most the exact count: safe
      bar();
      if constexpr (Ch::on && U >= 0) {
        cs.template advance_to<U + S - 1>();       // ck < nk: the caller has nk >= NU + S
      } else if constexpr (Ch::on && U == -1) {
        cs.advance();                              // ck < nk
      } else if constexpr (Ch::on) {
        // past the end (ck = nk + j): the next tile's slices, or the last
        // slice again
        constexpr int j = -2 - U;
        if constexpr (j == 0) {
          if (ch.has_next) {
            cs.a.init(ch.na);
            cs.b.init(ch.nb);
          }
        } else {
          cs.advance(ch.has_next);
        }
      } else {
        cs.advance(ck < nk);                       // else the last slice again
      }
      frags_wait<T>(f1);
      // second half-step: the next slice's copies and first reads between its MFMAs
      static_for<0, M>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        if constexpr (U >= 0) hook.template add<U, i>(acc);
        mfma_at<T>(i, f1, acc);
        if constexpr (i % CSP == 0 && i / CSP < G) cs.copy(i / CSP, cst);
        constexpr int q0 = i * RPM < R ? i * RPM : R, q1 = (i + 1) * RPM < R ? (i + 1) * RPM : R;
        static_for<q0, q1>([&](auto q) { frag_read<T, 0, decltype(q)::value>(nxt, f0); });
      });
      if constexpr (G > (M + CSP - 1) / CSP)
        static_for<(M + CSP - 1) / CSP, G>([&](auto g) { cs.copy(decltype(g)::value, cst); });
      cur = nxt;
      st = sn;
    };
    static_for<0, HK::NU>([&](auto uu) { body(decltype(uu)::value, uu); });
    if constexpr (Ch::on) {
      // the slices of this tile, then S - 1 iterations that copy past its end
      for (int t = HK::NU; t < nk - S + 1; ++t) body(t, ic<-1>{});
      static_for<0, S - 1>([&](auto jj) { body(nk - S + 1 + decltype(jj)::value, ic<-2 - decltype(jj)::value>{}); });
    } else {
      for (int t = HK::NU; t < nk; ++t) body(t, ic<-1>{});
    }
    // (the last iteration's reads of the next half-step fetch a slice past
    // the end that nothing uses: one loop shape for every slice keeps the
    // accumulators in the loop's registers)
  }
  if constexpr (Ch::on) {
    // the next tile's first slices stay in flight while the caller stores
    if (!ch.has_next) wait_vm<0>();
    bar();
    hook.drain(acc);
  } else {
    // every wave is done with the LDS slices and no copy or load is still in
    // flight; the caller may reuse LDS
    wait_vm<0>();
    bar();
    if (nk > 0) hook.drain(acc);
  }
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// a in the low half, b in the high half, each rounded to nearest even (one
// packed conversion)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

using FwdTile = Tile<256, 256, 4, ROW, PACKED>;        // A = W (row-major), B = Xp
using DxTile = Tile<256, 256, 4, PACKED, ROWT>;        // A = G (Zp), B = W read transposed
using DwTile = Tile<256, 256, 4, PACKED_T, PACKED>;    // A = G (Zp) transposed, B = XpT
constexpr int kDwGroup = 4;                            // vocabulary strips per group of dW tiles
constexpr int kDwOcc = 1;                              // dW workgroups per CU
// Main-loop schedules (reads per MFMA, MFMAs per copy), the fastest of those
// measured per kernel on the Llama-3-8B head at chunk 1024.
constexpr int kFwdRpm = 2, kFwdCsp = 2;
constexpr int kDxRpm = 2, kDxCsp = 2;
constexpr int kDwRpm = 1, kDwCsp = 2;

// ---------------------------------------------------------------- packing
// Workgroups [0, ndirect): one per 256 rows x 64 columns (two packed blocks,
// 32 KB) of a row-major bf16 matrix [R][K] (the chunk's X: rows = tokens,
// k = hidden): it reads the rows' 128-byte pieces (8 full rows per wave
// instruction), places them in LDS in packed order, and writes the two blocks
// as one contiguous 32 KB copy.  Zero outside [0, R) x [0, K).
// Workgroups from ndirect on: the transpose, a packed matrix of K rows and R
// columns (rows = hidden, k = tokens), for dW's operand: one per 256 of its
// rows x 64 of its columns.  Lane t loads an 8 x 8 group (8 consecutive
// source rows, 16 bytes = 8 consecutive columns each; one wave instruction
// reads two whole 512-byte row pieces), transposes it in registers, and
// writes eight 16-byte slots (one transposed row, 8 consecutive k) to their
// packed place in LDS; the two blocks then go out as one 32 KB copy.
__device__ __forceinline__ void pack_transposed(const uint16_t *__restrict__ src, int R, int K,
                                                uint16_t *__restrict__ PT, int64_t nks_t, int b,
                                                char *lds) {
  const int npair = (int)(nks_t >> 1);
  const int rt = b / npair, kp = b - rt * npair;      // output rows 256 rt .., columns 64 kp ..
  const int t = threadIdx.x, hg = t & 31, tg = t >> 5;
  const int h0 = rt * 256 + 8 * hg, r0 = kp * 64 + 8 * tg;  // source columns h0 .., rows r0 ..
  u32x4 in[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    in[j] = (r0 + j < R && h0 < K) ? *(const u32x4 *)(src + (int64_t)(r0 + j) * K + h0)
                                    : u32x4{0u, 0u, 0u, 0u};
  // out[q] = column h0 + q of source rows r0 .. r0 + 7: word w holds rows
  // 2w (low half) and 2w + 1 (high half)
  const int f = (tg >> 1) & 1, hh = tg & 1, blk = tg >> 2;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      o[w] = __builtin_amdgcn_perm(in[2 * w + 1][q >> 1], in[2 * w][q >> 1], (q & 1) ? 0x07060302u : 0x05040100u);
    const int hr = 8 * hg + q;                          // row of the output block
    const int off = (blk << 14) + ((((hr >> 5) << 1) + f) << 10) + (pk_slot(hr & 31, hh, f) << 4);
    *(u32x4 *)(lds + off) = o;
  }
  __syncthreads();
  uint16_t *dst = PT + (((int64_t)rt * nks_t + 2 * kp) << 13);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = i * 256 + t;
    *(u32x4 *)(dst + q * 8) = *(const u32x4 *)(lds + q * 16);
  }
}

__global__ __launch_bounds__(256) void pack_kernel(const uint16_t *__restrict__ src, int R, int K,
                                                  uint16_t *__restrict__ P, int64_t nks_p, int ndirect,
                                                  uint16_t *__restrict__ PT, int64_t nks_t) {
  __shared__ __attribute__((aligned(1024))) char lds[32768];
  if ((int)blockIdx.x >= ndirect) {
    pack_transposed(src, R, K, PT, nks_t, (int)blockIdx.x - ndirect, lds);
    return;
  }
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

// ---------------------------------------------------------------- forward tile
// Z^T tile: rows = 256 vocabulary ids from m0, columns = 256 tokens from n0;
// A = W along its rows (vocabulary), B = Xp (rows = tokens), k = hidden.
// VTAIL instantiates the tile that reaches past V (its rows >= V are masked).
//
// Epilogue, wave by wave: each wave reduces its own 128 vocabulary rows, so a
// token gets one (max, sum of exp) partial per 128 vocabulary ids, at index
// 2 vt + wm.  The target logit is taken from the fp32 accumulators by the
// lane that holds it.  The logits tile (8 consecutive blocks of Zp) is
// stored straight from the accumulators in 512-byte half-fragments, as
// bf16((z - m) log2 e) with m the token's maximum over the wave's 128
// vocabulary ids (written to pmt for dlogits): the argument of the
// exponential the sum needs anyway, so one fma serves both.  Rounding then
// costs a relative 2^-9 of m - z, not of z: exp(z - lse) keeps its accuracy
// however large the logits or a common shift of a token's logits, and the
// entries that carry the probability (z near m) are stored almost exactly.
// Rows past V (VTAIL) are stored as -inf; dlogits zeroes them.
// The forward tile's epilogue (see fwd_tile_kernel): per-token partials, the
// target logit and, with STORE, the logits tile from the accumulators of
// tile (vt, ct).
template <bool VTAIL, bool STORE, class T>
__device__ __forceinline__ void fwd_epilogue(
    f32x16 (&acc)[4][4], int vt, int ct, const int *lab_s, int c, int V,
    uint16_t *__restrict__ Zp, int64_t nks_z, float *__restrict__ pm, float *__restrict__ ps,
    float *__restrict__ pmt, float *__restrict__ zy, int64_t nvt) {
  const int m0 = vt * T::BM, n0 = ct * T::BN;

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int vrow0 = m0 + wm * 128 + 4 * (lane >> 5);   // row r = 32 i + 8 (e/4) + e%4
  const int vlim = V - vrow0;                          // rows r < vlim exist
  const int64_t part = 2 * (int64_t)vt + wm;
  // The tile's logits are the 8 blocks of vocabulary slices 8 vt .. 8 vt + 7
  // in token row tile ct of Zp, 128 KB from zbase.  For one (i, j, g) the
  // lanes hold 32 consecutive tokens x 4 consecutive vocabulary ids each
  // (lanes 32..63 the next 4), i.e. the 32 slots of one half of a Zp
  // fragment, so each store instruction writes 512 contiguous bytes: the
  // lane's part of the address depends on g only, the wave's on (i, j).
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      Zp + ((int64_t)ct * nks_z + 8 * (int64_t)vt) * 8192, (short)0, 131072, 0x00020000);
  int zvoff[4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    zvoff[g] = 2 * (4 * (lane >> 5) + ((g >> 1) << 9) + (pk_slot(lane & 31, g & 1, g >> 1) << 3));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tl = wn * 128 + j * 32 + (lane & 31), tok = n0 + tl;
    const bool tok_ok = tok < c;
    const int y = lab_s[tl];
    const int yr = y >= 0 ? y - vrow0 : -1;
    // this token group's accumulators, read here (volatile asm keeps the
    // compiler from reading every group's at the start and spilling them)
    float av[4][16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(av[i][e]) : "a"(acc[i][j][e]));
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 32 * i + 8 * (e >> 2) + (e & 3);
        const float z = (VTAIL && r >= vlim) ? -INFINITY : av[i][e];
        mx = fmaxf(mx, z);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // a wave whose rows all lie past V has mx = -inf: its sum must be 0, not NaN
    const float ms = (VTAIL && mx == -INFINITY) ? 0.f : mx;
    const float ml = ms * kLog2e;
    // The lane's rows r = 32 i + 8 (e/4) + e%4 have bit 2 clear (4 (lane/32)
    // is in vrow0), so it holds the target exactly when yr is such a row,
    // namely value 16 i + e with i = yr/32, e = 4 ((yr/8) % 4) + yr % 4.  A
    // tree of selects on the six bits of that index picks it: its first two
    // levels (e % 4) inside the loop below, the other four after it.
    const bool found = (unsigned)yr < 128u && (yr & 4) == 0;
    const int ti = ((yr >> 5) << 4) | (((yr >> 3) & 3) << 2) | (yr & 3);
    const bool b0 = ti & 1, b1 = ti & 2;
    float zt[16];
    // four independent partial sums, so that the exponentials do not wait
    // on one another; each group of four values goes out as it is formed
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float t[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 4 * g + q, r = 32 * i + 8 * g + q;
          const float z = (VTAIL && r >= vlim) ? -INFINITY : av[i][e];
          t[q] = __builtin_fmaf(z, kLog2e, -ml);
          s4[q] += __builtin_amdgcn_exp2f(t[q]);
        }
        const float z01 = b0 ? av[i][4 * g + 1] : av[i][4 * g];
        const float z23 = b0 ? av[i][4 * g + 3] : av[i][4 * g + 2];
        zt[4 * i + g] = b1 ? z23 : z01;
        if constexpr (STORE) {
          // vocabulary slice wm 4 + i of the tile, token row group wn 4 + j
          const u32x2 pk = {pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
          __builtin_amdgcn_raw_buffer_store_b64(pk, zrs, zvoff[g],
                                                2 * (((wm * 4 + i) << 13) + ((wn * 4 + j) << 10)), 0);
        }
      }
    float sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    sum += __shfl_xor(sum, 32);
#pragma unroll
    for (int bit = 2; bit < 6; ++bit) {
      const bool hi = (ti >> bit) & 1;
#pragma unroll
      for (int x = 0; x < (32 >> bit); ++x) zt[x] = hi ? zt[2 * x + 1] : zt[2 * x];
    }
    const float zsel = zt[0];
    if (found && tok_ok) zy[tok] = zsel;             // one lane holds the target
    if (lane < 32 && tok_ok) {
      pm[(int64_t)tok * nvt + part] = mx;
      ps[(int64_t)tok * nvt + part] = sum;
      if constexpr (STORE) pmt[part * c + tok] = ms;
    }
  }
}

// The forward's main-loop hook: the tile's labels, loaded from global memory
// before the prologue's copies, are written to LDS once those copies are
// issued, so that their latency overlaps the pipeline fill instead of the
// epilogue.  y is the label if it is a vocabulary id, else -1 (ignored, out
// of range, or a token past the chunk).
struct FwdLabels : NoHook {
  int *lab_s;
  int y;
  __device__ __forceinline__ void prologue() { lab_s[threadIdx.x] = y; }
};

template <bool VTAIL, bool STORE, class T = FwdTile, int RPM = kFwdRpm, int CSP = kFwdCsp>
__global__ __launch_bounds__(NTHREADS, 1) void fwd_tile_kernel(
    const uint16_t *__restrict__ W, const uint16_t *__restrict__ Xp,
    const int64_t *__restrict__ labels_c, int64_t ii, int c, int H, int V,
    uint16_t *__restrict__ Zp, int64_t nks_z, float *__restrict__ pm, float *__restrict__ ps,
    float *__restrict__ pmt, float *__restrict__ zy, int64_t nvt, int vt0, int nct) {
  static_assert(T::BM == 256 && T::BN == 256 && NTHREADS == T::BN, "the epilogue reduces a 256 x 256 tile");
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  __shared__ int lab_s[T::BN];
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int vt = vt0 + tile / nct, ct = tile % nct;
  FwdLabels hook;
  hook.lab_s = lab_s;
  {
    const int tok = ct * T::BN + (int)threadIdx.x;
    const int64_t y = tok < c ? labels_c[tok] : ii;
    hook.y = (y != ii && y >= 0 && y < V) ? (int)y : -1;
  }

  const int64_t nks_h = (int64_t)((H + 255) >> 8) << 3;
  const Op a{(const char *)(W + (int64_t)vt * T::BM * H), 2 * (int64_t)H, 0, (const char *)(W + (int64_t)V * H)};
  const Op b{(const char *)(Xp + (int64_t)ct * nks_h * 8192), 0, 0, nullptr};
  f32x16 acc[4][4];
  zero_acc<T>(acc);
  mainloop<T, RPM, CSP>(a, b, H, smem, acc, hook);
  fwd_epilogue<VTAIL, STORE, T>(acc, vt, ct, lab_s, c, V, Zp, nks_z, pm, ps, pmt, zy, nvt);
}

// ---------------------------------------------------------------- dlogits
// One workgroup per 16 KB block of Zp (256 tokens x 32 vocabulary columns),
// four 16-byte slots per thread (one token, 8 consecutive vocabulary columns
// each), in memory order: pass k of a wave covers 1 KB contiguous, and all
// four loads are in flight before any arithmetic.  In place, from the stored
// (Z - m) log2 e (m the token's maximum over the block's 128-wide partial, from pmt):
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
  // blocks in reverse order: dW, which reads G next, measured 2% faster per
  // chunk after this order than after the forward one
  const int64_t blk = (int64_t)gridDim.x - 1 - blockIdx.x;
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
      l2 = (lse_c[r] - mrow[r]) * kLog2e;     // stored values are (z - m) log2 e
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
        const float e = __builtin_amdgcn_exp2f(zz - l2) - ((int64_t)v == y ? 1.f : 0.f);
        fv[hh] = (valid && v < V) ? e * inv : 0.f;
      }
      g[d] = pack_bf16x2(fv[0], fv[1]);
    }
    *(u32x4 *)(zb + (k << 11)) = g;
  }
}

// ---------------------------------------------------------------- dW
// dW[v][h] (+)= sum over the chunk's tokens of G[tok][v] X[tok][h], in
// 256 x 256 tiles, one workgroup per CU; G from Zp and X from Xp, both read
// transposed.  Lane l of wave (wm, wn) holds, in acc[i][j][e], dW row
// v0 + 128 wm + 32 i + 8 (e/4) + 4 (l/32) + e%4 and column
// h0 + 128 wn + 32 j + l%32, so one dword access per (i, j, e) moves two
// whole 128-byte row pieces per wave.
//
// Accumulating into dW (every chunk after the first) needs the tile's old
// values.  Loaded in one burst after the main loop, they compete with the
// operand copies of the workgroups still in their main loops for each CU's
// vector-memory path; instead, the old values reach the accumulators during
// the main loop (DwOld): the first 15 iterations (one fewer than a wave's
// 16 accumulator blocks) are unrolled, and iteration u loads block u + 1's
// 16 values per lane (block 0 in the prologue), one after each MFMA of its
// first half-step.  Two iterations later, once the
// loop's own wait has admitted a copy issued after them, the block is added
// into its accumulators as a whole, right before the second half-step's MFMA
// on it.  (Adding single registers of a block makes the compiler copy the
// whole block out of and back into the accumulator registers around every
// MFMA.)  After the loop only stores remain.  Tiles that reach past V or H,
// chunks of fewer than 16 slices and the first chunk (nothing to add) take
// the plain path: the main loop alone, then a predicated read-add-store (or
// store) pass.
constexpr int kDwAux = 2;          // non-temporal: dW is touched once per chunk

// Scalar byte offset of row `row` of a dW quarter, computed where it is used:
// the empty asm keeps the compiler from hoisting the row offsets of a whole
// tile (up to 256 distinct values) into scalar registers.
__device__ __forceinline__ int row_off(int row, int ldb) {
  asm volatile("" : "+s"(ldb));
  return row * ldb;
}

template <class T>
struct DwOld {
  static constexpr int S = T::STAGES, NI = T::NI;
  static constexpr int NB = T::MI * T::NI;         // blocks = MFMAs per half-step
  static constexpr int NU = NB - 1;                // iteration u loads block u + 1
  static constexpr int LP = 16;                    // the prologue loads block 0
  static_assert(16 % NB == 0 || NB % 16 == 0, "a block's loads spread evenly over a half-step");
  static constexpr int loads(int u) { return u < NU ? 16 : 0; }
  // the first iteration whose wait admits a copy issued after block b's loads
  static constexpr int add_iter(int b) { return b == 0 ? S - 2 : b + S - 3; }

  __amdgpu_buffer_rsrc_t rs;       // this wave's 128 x 128 quarter of dW
  int voff;                        // the lane's byte offset in it
  int ldb;                         // bytes per dW row
  float v[NB][16];

  template <int b, int e>
  __device__ __forceinline__ void load_one() {
    constexpr int i = b / NI, j = b % NI, row = 32 * i + 8 * (e / 4) + e % 4;
    v[b][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 128 * j,
                                                                              row_off(row, ldb), kDwAux));
  }
  template <int b, class A>
  __device__ __forceinline__ void add_block(A &acc) {
    f32x16 o;
    static_for<0, 16>([&](auto e) { o[decltype(e)::value] = v[b][decltype(e)::value]; });
    acc[b / NI][b % NI] += o;
  }
  __device__ __forceinline__ void prologue() {
    static_for<0, 16>([&](auto e) { load_one<0, decltype(e)::value>(); });
  }
  // iteration U: block U + 1's 16 values spread over the first half-step's
  // NB MFMAs, 16 / NB after each
  template <int U, int I>
  __device__ __forceinline__ void load() {
    if constexpr (U + 1 < NB) {
      constexpr int per = 16 / NB > 0 ? 16 / NB : 1, first = I * per;
      if constexpr (first < 16) static_for<first, first + per>([&](auto e) { load_one<U + 1, decltype(e)::value>(); });
    }
  }
  // iteration U, before the second half-step's MFMA on block I
  template <int U, int I, class A>
  __device__ __forceinline__ void add(A &acc) {
    if constexpr (add_iter(I) == U) add_block<I>(acc);
  }
  template <class A>
  __device__ __forceinline__ void drain(A &acc) {
    static_for<0, NB>([&](auto bb) {
      constexpr int b = decltype(bb)::value;
      if constexpr (add_iter(b) >= NU) add_block<b>(acc);
    });
  }
};

// Write a wave's 128 x 128 quarter of an fp32 tile with row stride ldb
// bytes (rs: the quarter's first element; voff: the lane's byte offset,
// column and row half): out = acc, or out + acc with OLD.  CHECK masks rows
// >= vlim and columns >= hlim (relative to the quarter).  AUX: the accesses'
// cache policy.
template <class T, bool OLD, bool CHECK, int AUX = kDwAux, class A>
__device__ __forceinline__ void dw_store(const A &acc, __amdgpu_buffer_rsrc_t rs, int voff, int ldb,
                                         int vlim, int hlim) {
  const int lane = threadIdx.x & 63;
  static_for<0, T::MI * T::NI>([&](auto bb) {
    constexpr int b = decltype(bb)::value, i = b / T::NI, j = b % T::NI;
    const bool col_ok = !CHECK || 32 * j + (lane & 31) < hlim;
    float old[16];
    static_for<0, 16>([&](auto ee) {
      constexpr int e = decltype(ee)::value, row = 32 * i + 8 * (e / 4) + e % 4;
      old[e] = 0.f;
      if constexpr (OLD) {
        if (col_ok && (!CHECK || row + 4 * (lane >> 5) < vlim))
          old[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff + 128 * j,
                                                                                  row_off(row, ldb), AUX));
      }
    });
    static_for<0, 16>([&](auto ee) {
      constexpr int e = decltype(ee)::value, row = 32 * i + 8 * (e / 4) + e % 4;
      // read the accumulator here, not all of them after the main loop
      float x;
      asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(acc[i][j][e]));
      if constexpr (OLD) x += old[e];
      if (col_ok && (!CHECK || row + 4 * (lane >> 5) < vlim))
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rs, voff + 128 * j,
                                              row_off(row, ldb), AUX);
    });
    // one block's old values at a time in registers
    asm volatile("" ::: "memory");
  });
}

// Tile (vt, ht) of launch index t.  SPREAD launches cover the nvt x nht
// tiles inside V and H; the others cover all nvt x nht tiles (tails = 0), or
// only those that reach past V or H (tails = 1): first the last vocabulary
// row of tiles when V has a tail (vtail), then the last hidden column when H
// has one (htail), without the corner twice.
template <int GROUP>
__device__ __forceinline__ void dw_tile(int t, int nvt, int nht, int tails, int vtail, int htail, int &vt,
                                        int &ht) {
  if (!tails) {
    grouped<GROUP>(xcd_remap(t, nvt * nht), nvt, nht, vt, ht);
  } else if (vtail && t < nht) {
    vt = nvt - 1;
    ht = t;
  } else {
    vt = t - (vtail ? nht : 0);
    ht = nht - 1;
  }
}

template <bool SPREAD, class T = DwTile, int RPM = kDwRpm, int CSP = kDwCsp, int GROUP = kDwGroup,
          int OCC = kDwOcc>
__global__ __launch_bounds__(NTHREADS, OCC) void dw_kernel(
    const uint16_t *__restrict__ Gp, int64_t nks_z, const uint16_t *__restrict__ XpT,
    int64_t nks_c, int c, int H, int V, int nvt, int nht, int tails, int vtail, int htail,
    float *__restrict__ dW, int accumulate) {
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  int vt, ht;
  dw_tile<GROUP>(blockIdx.x, nvt, nht, tails, vtail, htail, vt, ht);
  const int m0 = vt * T::BM, n0 = ht * T::BN;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;

  f32x16 acc[T::MI][T::NI];
  zero_acc<T>(acc);
  const Op a{(const char *)(Gp + (int64_t)(m0 >> 5) * 8192), nks_z * 16384, 0};
  const Op b{(const char *)(XpT + (int64_t)ht * nks_c * 8192), 0, 0, nullptr};
  // the wave's quarter of dW; offsets stay below 2^31 for H <= 2^20
  const int vq = m0 + wm * T::WM, hq = n0 + wn * T::WN;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      dW + (int64_t)vq * H + hq, (short)0, 0x7fffffff, 0x00020000);
  const int voff = ((lane >> 5) * 4 * H + (lane & 31)) * 4, ldb = H * 4;
  if constexpr (SPREAD) {
    // the launch guarantees: accumulate, tile inside V and H, c >= 16 slices
    DwOld<T> hk{rs, voff, ldb};
    mainloop<T, RPM, CSP>(a, b, c, smem, acc, hk);
    dw_store<T, false, false>(acc, rs, voff, ldb, 0, 0);
  } else {
    mainloop<T, RPM, CSP>(a, b, c, smem, acc);
    const int vlim = V - vq, hlim = H - hq;
    if (accumulate) dw_store<T, true, true>(acc, rs, voff, ldb, vlim, hlim);
    else dw_store<T, false, true>(acc, rs, voff, ldb, vlim, hlim);
  }
}

// dW of the tiles inside V and H, one resident workgroup per CU working
// through tiles t = blockIdx.x, + gridDim.x, ... (the order of the
// one-tile-per-workgroup launch, since gridDim.x is a multiple of the 8
// XCDs), each tile's loop fetching the next tile's first slices while the
// tile's stores go out (Chain).  OLD: accumulate, with the old values added
// in the main loop (DwOld; needs c >= NU + STAGES = 19 slices); else store
// (c >= STAGES slices).
template <bool OLD, class T = DwTile, int RPM = kDwRpm, int CSP = kDwCsp, int GROUP = kDwGroup>
__global__ __launch_bounds__(NTHREADS, 1) void dw_chain_kernel(
    const uint16_t *__restrict__ Gp, int64_t nks_z, const uint16_t *__restrict__ XpT,
    int64_t nks_c, int c, int H, int V, int nvt, int nht, float *__restrict__ dW) {
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  const int ntiles = nvt * nht;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int voff = ((lane >> 5) * 4 * H + (lane & 31)) * 4, ldb = H * 4;
  const int nk = (c + BK - 1) / BK;
  // operands and this wave's quarter of dW for tile t
  auto tile_ops = [&](int t, Op &a, Op &b, __amdgpu_buffer_rsrc_t &rs) {
    int vt, ht;
    dw_tile<GROUP>(t, nvt, nht, 0, 0, 0, vt, ht);
    const int m0 = vt * T::BM, n0 = ht * T::BN;
    a = Op{(const char *)(Gp + (int64_t)(m0 >> 5) * 8192), nks_z * 16384, 0};
    b = Op{(const char *)(XpT + (int64_t)ht * nks_c * 8192), 0, 0, nullptr};
    rs = __builtin_amdgcn_make_buffer_rsrc(dW + (int64_t)(m0 + wm * T::WM) * H + n0 + wn * T::WN, (short)0,
                                           0x7fffffff, 0x00020000);
  };
  int t = blockIdx.x;
  Op a, b;
  __amdgpu_buffer_rsrc_t rs;
  tile_ops(t, a, b, rs);
  bool warm = false;
  int rb = 0;
  while (true) {
    const int tn = t + (int)gridDim.x;
    Chain ch;
    ch.warm = warm;
    ch.rb = rb;
    ch.has_next = tn < ntiles;
    __amdgpu_buffer_rsrc_t rsn = rs;
    if (ch.has_next) tile_ops(tn, ch.na, ch.nb, rsn);
    f32x16 acc[T::MI][T::NI];
    zero_acc<T>(acc);
    if constexpr (OLD) mainloop<T, RPM, CSP>(a, b, c, smem, acc, DwOld<T>{rs, voff, ldb}, ch);
    else mainloop<T, RPM, CSP>(a, b, c, smem, acc, NoHook{}, ch);
    dw_store<T, false, false>(acc, rs, voff, ldb, 0, 0);
    if (!ch.has_next) break;
    t = tn;
    a = ch.na;
    b = ch.nb;
    rs = rsn;
    warm = true;
    rb = (rb + nk) % T::STAGES;
  }
}

// ---------------------------------------------------------------- dX (split-K)
// Unit (s, mt, nt): dxp[s][tok][h] = sum over vocabulary in split s of
// G[tok][v] W[v][h].  G from Zp (rows = tokens, k = vocabulary), W read
// transposed in place (its columns, the hidden ids, are the operand rows;
// its rows, the vocabulary, are k), so no copy of W is made.
template <class T = DxTile, int RPM = kDxRpm, int CSP = kDxCsp>
__global__ __launch_bounds__(NTHREADS, 1) void dx_kernel(
    const uint16_t *__restrict__ Gp, int64_t nks_z, const uint16_t *__restrict__ W,
    int c, int H, int V, int64_t ksplit, int nmt, int nnt, float *__restrict__ dxp) {
  static_assert(T::BM == 256 && T::BN == 256, "256 x 256 output tiles");
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

  const Op a{(const char *)(Gp + ((int64_t)mt * nks_z + (kb >> 5)) * 8192), 0, 0, nullptr};
  const Op b{(const char *)(W + n0), 2 * (int64_t)H, kb, (const char *)(W + (int64_t)V * H)};
  f32x16 acc[4][4];
  zero_acc<T>(acc);
  mainloop<T, RPM, CSP>(a, b, klen, smem, acc);

  // the partials straight from the accumulators, as dW stores its tiles
  // (plain stores: dx_reduce reads them right after); only tiles that reach
  // past c tokens or H columns check their rows and columns
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int r0 = m0 + wm * T::WM, c0 = n0 + wn * T::WN;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      dxp + (int64_t)s * c * H + (int64_t)r0 * H + c0, (short)0, 0x7fffffff, 0x00020000);
  const int voff = ((lane >> 5) * 4 * H + (lane & 31)) * 4, ldb = H * 4;
  if (m0 + T::BM <= c && n0 + T::BN <= H) dw_store<T, false, false, 0>(acc, rs, voff, ldb, 0, 0);
  else dw_store<T, false, true, 0>(acc, rs, voff, ldb, c - r0, H - c0);
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

inline int grid_for(int64_t n, int block, int cap) {
  int64_t g = (n + block - 1) / block;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace

// Compute units of the current device (looked up once per device).
static int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_pack_bf16(const uint16_t *src, int R, int K, uint16_t *P, int64_t nks_p,
                            uint16_t *PT, int64_t nks_t, hipStream_t s) {
  // nks_p and nks_t are multiples of 8, so column pairs of slices tile them exactly
  const int64_t ndirect = (int64_t)(R + 255) / 256 * (nks_p / 2);
  const int64_t ntrans = PT ? (int64_t)(K + 255) / 256 * (nks_t / 2) : 0;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)(ndirect + ntrans)), dim3(256), 0, s, src, R, K, P, nks_p,
                     (int)ndirect, PT, nks_t);
  return hipGetLastError();
}

hipError_t launch_fwd_tile_bf16(const uint16_t *W, const uint16_t *Xp,
                                const int64_t *labels_c, int64_t ii, int c, int H, int V,
                                uint16_t *Zp, int64_t nks_z, float *pm, float *ps, float *pmt,
                                float *zy, int64_t nvt, bool store_z, hipStream_t s) {
  const int nct = (c + FwdTile::BN - 1) / FwdTile::BN;
  const int nfull = V / FwdTile::BM;                 // vocabulary tiles inside V
  auto launch = [&](auto vtail, auto store, int ntiles, int vt0) {
    hipLaunchKernelGGL((fwd_tile_kernel<decltype(vtail)::value, decltype(store)::value>), dim3(ntiles),
                       dim3(NTHREADS), 0, s, W, Xp, labels_c, ii, c, H, V, Zp, nks_z, pm, ps, pmt, zy,
                       nvt, vt0, nct);
    return hipGetLastError();
  };
  hipError_t e = hipSuccess;
  if (nfull > 0)
    e = store_z ? launch(bc<false>{}, bc<true>{}, nfull * nct, 0) : launch(bc<false>{}, bc<false>{}, nfull * nct, 0);
  if (e == hipSuccess && V % FwdTile::BM != 0)
    e = store_z ? launch(bc<true>{}, bc<true>{}, nct, nfull) : launch(bc<true>{}, bc<false>{}, nct, nfull);
  return e;
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

hipError_t launch_dx_bf16(const uint16_t *Gp, int64_t nks_z, const uint16_t *W,
                          int c, int H, int V, int splitk, int64_t ksplit, float *dxp,
                          hipStream_t s) {
  const int nmt = (c + DxTile::BM - 1) / DxTile::BM, nnt = (H + DxTile::BN - 1) / DxTile::BN;
  hipLaunchKernelGGL((dx_kernel<>), dim3(splitk * nmt * nnt), dim3(NTHREADS), 0, s, Gp, nks_z, W,
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

hipError_t launch_dw_bf16(const uint16_t *Gp, int64_t nks_z, const uint16_t *XpT, int64_t nks_c,
                          int c, int H, int V, float *dW, bool accumulate, hipStream_t s) {
  const int nvt = (V + DwTile::BM - 1) / DwTile::BM, nht = (H + DwTile::BN - 1) / DwTile::BN;
  const int nvi = V / DwTile::BM, nhi = H / DwTile::BN;        // tiles inside V, H
  const int vtail = nvi < nvt, htail = nhi < nht;
  const int nk = (c + BK - 1) / BK;
  const dim3 block(NTHREADS);
  constexpr int S = DwTile::STAGES, NB = DwOld<DwTile>::NB, NU = DwOld<DwTile>::NU;
  // the tiles inside V and H: chained through resident workgroups, or one
  // workgroup per tile; the tail tiles then take the plain kernel
  const bool chain = nk >= (accumulate ? NU + S : S);
  const bool spread = accumulate && nk >= NB;
  if (nvi > 0 && nhi > 0 && (chain || spread)) {
    const int ntiles = nvi * nhi;
    if (chain) {
      // one resident workgroup per CU (a multiple of the 8 XCDs)
      const int ncu = cu_count();
      if (ncu <= 0) return hipErrorInvalidDevice;
      const int nres = ncu >= 8 ? ncu / 8 * 8 : ncu;
      const dim3 grid(ntiles < nres ? ntiles : nres);
      if (accumulate)
        hipLaunchKernelGGL((dw_chain_kernel<true>), grid, block, 0, s, Gp, nks_z, XpT, nks_c, c, H, V, nvi, nhi, dW);
      else
        hipLaunchKernelGGL((dw_chain_kernel<false>), grid, block, 0, s, Gp, nks_z, XpT, nks_c, c, H, V, nvi, nhi,
                           dW);
    } else {
      hipLaunchKernelGGL((dw_kernel<true>), dim3(ntiles), block, 0, s, Gp, nks_z, XpT, nks_c, c, H, V, nvi, nhi, 0,
                         0, 0, dW, 1);
    }
    const int ntail = (vtail ? nht : 0) + (htail ? nvt - vtail : 0);
    if (ntail > 0)
      hipLaunchKernelGGL((dw_kernel<false>), dim3(ntail), block, 0, s, Gp, nks_z, XpT, nks_c, c, H, V, nvt, nht, 1,
                         vtail, htail, dW, accumulate ? 1 : 0);
  } else {
    hipLaunchKernelGGL((dw_kernel<false>), dim3(nvt * nht), block, 0, s, Gp, nks_z, XpT, nks_c, c, H, V, nvt, nht,
                       0, 0, 0, dW, accumulate ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace flce
