// rz_gemm.h -- the one MFMA tile engine behind every contraction of the path.
//
// C[m, n] = sum_k A[m, k] * B[n, k] with both operands K-contiguous ("NT"),
// computed by one fixed 256 x 256 output tile per workgroup, K consumed in
// fixed 128-byte stages (64 bf16 or 32 fp32 values) from k = 0 upwards, no
// split-K.  The instruction sequence that produces C[m, n] is the same for
// every m and n, and does not depend on M: the basis of the batch-invariant
// logprobs (the trainer-inference invariance of the REINFORCE Zero project
// page, section 02 "Remove kernel mismatch").
//
// Layout of the work (gfx950, CDNA4):
//  * gemm_mainloop: 512 threads = 8 wave64s, two per SIMD, wave w owning
//    rows 64 (w % 4) .. + 63 of column half w / 4 = 2 x 4 blocks of
//    v_mfma_f32_32x32x16_bf16 (fp32 inputs use v_mfma_f32_32x32x2_f32, four
//    per 16-byte fragment); the 64-row tiles for small row counts
//    (gemm_mainloop_rows64) take the same blocks, fragments and K steps on
//    four waves;
//  * A and B stages go straight from global memory into LDS
//    (global_load_lds_dwordx4, no register round trip), double-buffered
//    (2 x 64 KB), with a 16-byte-chunk XOR swizzle (see swz) so the fragment
//    reads are bank-conflict free;
//  * stage kt + 1 is in flight while stage kt feeds the MFMAs, and the
//    fragments of the next 16-byte K step are read while the current
//    step's MFMAs run;
//  * workgroups are numbered XCD-aware: the dispatcher places workgroup i on
//    XCD i % 8, so logical tiles are renumbered to give each XCD a
//    contiguous range, and within it tiles are walked in groups of tile-rows
//    so the co-resident workgroups of one XCD share A and B stages in its L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace rz {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256;          // tile rows (M)
constexpr int kBN = 256;          // tile columns (N)
constexpr int kRowBytes = 128;    // K bytes per stage row
constexpr int kThreads = 256;     // the 64-row tiles; the 256 x 256 tile 2 kThreads
constexpr int kTM = 4;            // 32 x 32 blocks per wave along M (rz_calib's four-wave layout)
constexpr int kTN = 4;            // ... along N (every layout)
constexpr int kOperandBytes = kBM * kRowBytes;      // 32 KB
constexpr int kStageBytes = 2 * kOperandBytes;      // A + B
constexpr int kLdsBytes = 2 * kStageBytes;          // double buffer, 128 KB
constexpr int kGroupM = 8;        // tile-rows walked together per XCD
// the 64-row tile (gemm_mainloop_rows64)
constexpr int kBM64 = 64;
constexpr int kOperandBytesA64 = kBM64 * kRowBytes;              // 8 KB
constexpr int kStageBytes64 = kOperandBytesA64 + kOperandBytes;  // 40 KB
constexpr int kLdsBytes64 = 2 * kStageBytes64;                   // 80 KB

template <typename T>
struct Stage {
  static constexpr int kK = kRowBytes / (int)sizeof(T);  // K values per stage
};

// Cache-policy operand of a load: the non-temporal hint ("nt" on gfx950),
// for data each workgroup streams once and no other reads again.
constexpr int kPolicyNT = 2;

constexpr float kLog2e = 1.4426950408889634f;  // log2(e), for exp via exp2

__device__ __forceinline__ float exp_approx(float x) {
  // e^x = 2^(x log2 e); v_exp_f32 evaluates 2^y
  return __builtin_amdgcn_exp2f(x * kLog2e);
}

// One 16-byte fragment step of the MFMA pipe: 32x32x16 for bf16 ...
__device__ __forceinline__ void mfma_step(f32x16& acc, u32x4 a, u32x4 b,
                                          const bf16*) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0,
      0);
}
// ... or four 32x32x2 steps for fp32 (lane half h holds k = 4h .. 4h+3 of the
// 8-value slice; both operands use the same mapping, so the K sum is exact).
// The whole 16-byte vector is reinterpreted first: bit-casting single vector
// elements is miscompiled by this toolchain (every element reads lane 0).
__device__ __forceinline__ void mfma_step(f32x16& acc, u32x4 a, u32x4 b,
                                          const float*) {
  const f32x4 af = __builtin_bit_cast(f32x4, a);
  const f32x4 bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[j], bf[j], acc, 0, 0, 0);
}

// Rows of a launch whose count may live on the device (valid-row count).
struct RowCount {
  const int* count;  // device count of rows in the whole list (nullable)
  int64_t base;      // first list position covered by this launch
  int cap;           // rows of this launch when count is null; upper bound
  __device__ __forceinline__ int get() const {
    if (!count) return cap;
    const int64_t r = (int64_t)(*count) - base;
    return r <= 0 ? 0 : (r < cap ? (int)r : cap);
  }
};

struct TileCoord {
  int tm, tn;
};

// XCD-aware, grouped tile order.  Bijective on [0, mt * nt).
__device__ __forceinline__ TileCoord map_tile(int bid, int nblk, int mt,
                                              int nt) {
  const int per = nblk >> 3, rem = nblk & 7;
  const int x = bid & 7, local = bid >> 3;
  const int logical = x * per + (x < rem ? x : rem) + local;
  const int width = kGroupM * nt;
  const int g = logical / width;
  const int first = g * kGroupM;
  const int gm = (mt - first) < kGroupM ? (mt - first) : kGroupM;
  const int in = logical - g * width;
  return {first + in % gm, in / gm};
}

// Position of accumulator register r of block (mi, ni) inside the 256 x 256
// tile, for v_mfma_*_32x32 output (operands not swapped) of a wave whose
// blocks start at tile row wrow and column wcol (gemm_mainloop: wrow =
// 64 (w % 4), wcol = 128 (w / 4)): lane l holds column l % 32 and rows
// 8 * (r / 4) + 4 * (l / 32) + (r % 4) of its 32 x 32 block.
__device__ __forceinline__ int acc_row(int wrow, int mi, int r, int lane) {
  return wrow + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wcol, int ni, int lane) {
  return wcol + ni * 32 + (lane & 31);
}

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct GemmOperands {
  const char* A;        // A[m, :] row base is A + row(m) * lda
  int64_t lda;          // bytes
  const int* a_rows;    // optional gather: row(m) = a_rows[a_base + m]
  int64_t a_base;       // else row(m) = a_base + m
  const char* B;        // B[n, :] row base is B + n * ldb
  int64_t ldb;          // bytes
  int N;                // rows of B (columns of C)
};

// Accumulate acc over K stages [0, nk) for the 256 x 256 tile at (m0, n0),
// on eight waves (512 threads), two per SIMD: wave w owns rows
// 64 (w % 4) .. + 63 (two 32-row blocks) of column half w / 4 (four
// 32-column blocks); while one wave of a SIMD waits on its LDS reads, loads
// or a barrier, the other can issue.  Rows of A at or past M (and rows of B
// at or past N) are read from row M-1 (N-1) so every load stays in bounds;
// their results are discarded by the epilogue.  Each 32 x 32 block sees the
// same MFMA on the same fragments in K order k = 0, 1, 2, ..., whichever
// wave or tile form computes it.  Leaves the LDS free (all waves past the
// last barrier) on return.
//
// kTransA = true (16-bit values only) takes A stored K-major instead:
// A[m, k] at A + k * lda + 2 m, i.e. rows of the memory matrix are K and
// M is contiguous.  A stage is then 64 K-rows x 512 bytes in LDS, and the
// MFMA fragments come out of gfx950's transposing LDS read
// (ds_read_b64_tr_b16, see lread), so no transposed copy of A is needed.
//
// kSwap = true issues each MFMA with the operands exchanged, which computes
// the same products but leaves the transposed block in the accumulators:
// lane l then holds row l % 32 of its 32 x 32 block (an A row) and registers
// r hold columns 8 (r / 4) + 4 (l / 32) + (r % 4), i.e. every lane owns
// four runs of four consecutive B rows of one A row.
template <typename T, bool kSwap = true, bool kTransA = false>
__device__ __forceinline__ void gemm_mainloop(const GemmOperands& op, int M,
                                              int m0, int n0, int nk,
                                              f32x16 (&acc)[2][kTN],
                                              char* lds) {
  static_assert(!kTransA || sizeof(T) == 2, "K-major A needs 16-bit values");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wrow = (wid & 3) * 64, wcol = (wid >> 2) * 128;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  if (nk <= 0) return;

  int a_off[2], b_off[kTN];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
    a_off[mi] = (wrow + mi * 32 + (lane & 31)) * kRowBytes;
#pragma unroll
  for (int ni = 0; ni < kTN; ++ni)
    b_off[ni] = (wcol + ni * 32 + (lane & 31)) * kRowBytes;
  // fragment read offsets: row (block base + lane % 32), chunk 2 s + lane / 32.
  // 16-byte chunk c of LDS row r lives at chunk c ^ swz(r), swz(r) =
  // (r & 7) ^ ((r >> 3) & 1): any 8 consecutive rows (a 128-byte bank line)
  // and the same-parity rows of any 16 (a 256-byte line) get distinct
  // chunks, so the fragment reads are bank-conflict free.
  int c_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c_off[s] = ((2 * s + (lane >> 5)) ^ swz(lane & 31)) << 4;

  // Global -> LDS without a register round trip: global_load_lds_dwordx4
  // writes lane l's 16 bytes at (LDS base + 16 l).  Wave w fills rows
  // [32 w, 32 w + 32) of each operand, 8 rows per instruction; lane l lands
  // in row l / 8 at physical chunk l % 8, so it fetches the logical chunk
  // (l % 8) ^ swz(row) that the swizzle places there.
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  const int wu = __builtin_amdgcn_readfirstlane(wid);
  const char* ga[4];
  const char* gb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wu * 32 + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    if constexpr (kTransA) {
      // K-major A: instruction i of wave wu fills K-rows 2 (4 wu + i) and
      // 2 (4 wu + i) + 1 of the stage (512 bytes each, lane / 32 picks the
      // row); lane % 32 is the physical 16-byte chunk, which holds logical
      // chunk (lane % 32) ^ 4 (row % 4), i.e. columns m0 + 8 chunk .. + 7.
      // Columns past M - 8 read the last 8 (discarded by the epilogue).
      const int kr = 2 * (wu * 4 + i) + (lane >> 5);
      const int lc = (lane & 31) ^ (4 * (kr & 3));
      int mm = m0 + 8 * lc;
      mm = mm <= M - 8 ? mm : M - 8;
      ga[i] = op.A + (int64_t)kr * op.lda + (int64_t)mm * 2;
    } else {
      int m = m0 + r;
      m = m < M ? m : M - 1;
      const int64_t prow = op.a_rows ? (int64_t)op.a_rows[op.a_base + m]
                                     : op.a_base + m;
      ga[i] = op.A + prow * op.lda + c * 16;
    }
    int n = n0 + r;
    n = n < op.N ? n : op.N - 1;
    gb[i] = op.B + (int64_t)n * op.ldb + c * 16;
  }
  // load j of a stage: j < 4 fills A rows 32 wu + 8 j .. + 7 (K-major:
  // K-rows 8 wu + 2 j, + 1), j >= 4 the same rows of B
  auto dma1 = [&](int kt, int stage, int j) {
    const int64_t k = (int64_t)kt * kRowBytes;
    const int64_t ka = kTransA ? (int64_t)kt * 64 * op.lda : k;
    char* st = lds + stage * kStageBytes + (wu * 32 + (j & 3) * 8) * kRowBytes;
    if (j < 4)
      __builtin_amdgcn_global_load_lds(ga[j] + ka, (lds_ptr_t)st, 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(gb[j - 4] + k,
                                       (lds_ptr_t)(st + kOperandBytes), 16, 0, 0);
  };
  // K-major A: ds_read_b64_tr_b16 works on groups of 16 lanes; lane q of
  // a group names 8 bytes (4 values) at K-row q / 4 of a 4-row slab and
  // columns 4 (q % 4) .. + 3, and lane 4 a + b of the group receives column
  // 4 a + b of all four rows -- four consecutive K values of one M row, the
  // MFMA A-operand layout.  Group g of the wave covers the 16 columns
  // 16 (g % 2) .. of the 32-row block and K-rows 8 (g / 2) + 4 r .. of the
  // step; two reads (r = 0, 1) make the 8 values of one fragment.  The
  // XOR of the chunk with 4 (row % 4) puts the 8 rows one read touches in
  // four different 64-byte bank groups (two rows each, the minimum for
  // 512 bytes).
  int a_tr[2][2];
  if constexpr (kTransA) {
    const int g = lane >> 4, q = lane & 15;
    const int X = 4 * (q >> 2);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int kq = 8 * (g >> 1) + 4 * r + (q >> 2);
        const int mloc = wrow + mi * 32 + 16 * (g & 1) + 4 * (q & 3);
        a_tr[mi][r] = kq * 512 + (((mloc >> 3) ^ X) << 4) + (mloc & 7) * 2;
      }
  }
  typedef __attribute__((address_space(3))) const char* lds_cptr_t;
  u32x4 fa[2][2], fb[2][kTN];
  auto lread = [&](int buf, int stage, int s) {
    const char* sa = lds + stage * kStageBytes;
    const char* sb = sa + kOperandBytes;
    if constexpr (kTransA) {
      // Issued by hand: the compiler waits for every outstanding LDS-DMA
      // load (vmcnt(0)) before its own form of this read.  The B reads
      // below are issued after these ("memory" keeps them there) and LDS
      // reads retire in order, so the lgkmcnt wait the compiler places
      // before the first MFMA that uses B also covers these.
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const uint32_t p0 = (uint32_t)(uintptr_t)(lds_cptr_t)(sa + a_tr[mi][0]);
        const uint32_t p1 = (uint32_t)(uintptr_t)(lds_cptr_t)(sa + a_tr[mi][1]);
        u32x2 lo, hi;
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                     : "=v"(lo) : "v"(p0), "i"(s * 8192) : "memory");
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                     : "=v"(hi) : "v"(p1), "i"(s * 8192) : "memory");
        fa[buf][mi] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    } else {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        fa[buf][mi] = *reinterpret_cast<const u32x4*>(sa + a_off[mi] + c_off[s]);
    }
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni)
      fb[buf][ni] = *reinterpret_cast<const u32x4*>(sb + b_off[ni] + c_off[s]);
  };
  // block q = 4 mi + ni of one K step
  auto mm1 = [&](int buf, int q) {
    if constexpr (kSwap)
      mfma_step(acc[q / kTN][q % kTN], fb[buf][q % kTN], fa[buf][q / kTN],
                (const T*)nullptr);
    else
      mfma_step(acc[q / kTN][q % kTN], fa[buf][q / kTN], fb[buf][q % kTN],
                (const T*)nullptr);
  };
  auto mmr = [&](int buf, int lo, int hi) {
#pragma unroll
    for (int q = lo; q < hi; ++q) mm1(buf, q);
  };
  // Schedule: stage kt lives in LDS buffer kt & 1 and is consumed as four
  // 16-byte K steps s, each a phase of 8 MFMAs per wave on fragments read
  // during the previous phase.  A phase starts with one MFMA, which needs
  // the previous phase's reads, and only then issues the next step's reads,
  // so the LDS wait before it never covers reads that were just issued.
  // Each wave's eight loads of stage kt + 1 go out one per MFMA: four right
  // after the barrier that frees its buffer (among the last four MFMAs of
  // stage kt - 1) and four in the first phase of stage kt; a burst of loads
  // stalls the in-order wave.  Before the barrier that ends stage kt, each
  // wave waits for its own loads (vmcnt(0)), so the barrier makes stage
  // kt + 1 complete in LDS and buffer kt & 1 free.  sched_barrier(0) pins
  // this order against the scheduler.
#define RZ_SB() __builtin_amdgcn_sched_barrier(0)
  // Plain operands: a wave's 32-column blocks wholly at or past column N
  // (uniform per wave; the narrow last column tile of the LoRA-widened
  // dHidden, the adapter's own 64 columns) issue no MFMA: their
  // accumulators stay 0 and no epilogue stores them.  The swapped form
  // keeps every MFMA: the forward's row maxima read every accumulator.
  int nlive = kTN;
  if constexpr (!kSwap) {
    const int left = op.N - n0 - wcol;
    nlive = left <= 0 ? 0 : (left >= 32 * kTN ? kTN : (left + 31) / 32);
  }
  // (the forward below writes the schedule out itself)
  auto sched = [&](auto part_c) {
    constexpr bool kPart = decltype(part_c)::value;
    auto mmx = [&](int buf, int q) {
      if constexpr (kPart) {
        if (q % kTN >= nlive) return;
      }
      mm1(buf, q);
    };
    auto mmrx = [&](int buf, int lo, int hi) {
#pragma unroll
      for (int q = lo; q < hi; ++q) mmx(buf, q);
    };
#pragma unroll
    for (int j = 0; j < 8; ++j) dma1(0, 0, j);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (nk > 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma1(1, 1, j);
    }
    lread(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool nx = kt + 1 < nk, nx2 = kt + 2 < nk;
      RZ_SB(); mmx(0, 0); RZ_SB(); lread(1, cur, 1); RZ_SB();
#pragma unroll
      for (int q = 1; q < 8; ++q) {
        mmx(0, q);
        RZ_SB();
        if (q <= 4 && nx) dma1(kt + 1, cur ^ 1, 3 + q);
        RZ_SB();
      }
      mmx(1, 0); RZ_SB(); lread(0, cur, 2); RZ_SB(); mmrx(1, 1, 8); RZ_SB();
      mmx(0, 0); RZ_SB(); lread(1, cur, 3); RZ_SB(); mmrx(0, 1, 8); RZ_SB();
      mmrx(1, 0, 4);
      RZ_SB();
      if (nx) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      RZ_SB();
      if (nx) lread(0, cur ^ 1, 0);
      RZ_SB();
#pragma unroll
      for (int q = 4; q < 8; ++q) {
        mmx(1, q);
        RZ_SB();
        if (nx2) dma1(kt + 2, cur, q - 4);
        RZ_SB();
      }
    }
  };
  if constexpr (kSwap) {
    // the same schedule written out with every MFMA (the forward)
#pragma unroll
    for (int j = 0; j < 8; ++j) dma1(0, 0, j);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (nk > 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dma1(1, 1, j);
    }
    lread(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool nx = kt + 1 < nk, nx2 = kt + 2 < nk;
      RZ_SB(); mm1(0, 0); RZ_SB(); lread(1, cur, 1); RZ_SB();
#pragma unroll
      for (int q = 1; q < 8; ++q) {
        mm1(0, q);
        RZ_SB();
        if (q <= 4 && nx) dma1(kt + 1, cur ^ 1, 3 + q);
        RZ_SB();
      }
      mm1(1, 0); RZ_SB(); lread(0, cur, 2); RZ_SB(); mmr(1, 1, 8); RZ_SB();
      mm1(0, 0); RZ_SB(); lread(1, cur, 3); RZ_SB(); mmr(0, 1, 8); RZ_SB();
      mmr(1, 0, 4);
      RZ_SB();
      if (nx) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      RZ_SB();
      if (nx) lread(0, cur ^ 1, 0);
      RZ_SB();
#pragma unroll
      for (int q = 4; q < 8; ++q) {
        mm1(1, q);
        RZ_SB();
        if (nx2) dma1(kt + 2, cur, q - 4);
        RZ_SB();
      }
    }
  } else if (nlive == kTN) {
    sched(std::integral_constant<bool, false>{});
  } else {
    sched(std::integral_constant<bool, true>{});
  }
#undef RZ_SB
}

// The 64-row tile for small row counts (the rollout at decode size): each
// wave owns one 32-row block (wm) and the four 32-column blocks of its column
// half (wn), and issues each MFMA with swapped operands on fragments taken
// from the same swizzled LDS layout and K steps as gemm_mainloop<T, true>,
// so every 32 x 32 block's accumulators are bit-identical to that tile's.
// A stage is 64 A rows and 256 B rows (40 KB); stage kt + 1 streams in
// (global_load_lds_dwordx4: two loads for A and eight for B per wave) while
// stage kt feeds the MFMAs; each stage ends with every wave's loads complete
// and a barrier.  At these row counts the B stream (the head W, read once
// per column tile) bounds the kernel, not the MFMAs.  Rows of A at or past M
// (B rows past N) read row M - 1 (N - 1), as in gemm_mainloop.  Leaves the
// LDS free on return.
//
// kStages = 1 keeps a single 40 KB stage instead (load, wait, compute, in
// turn): three workgroups then share a CU, so the 675 workgroups of a
// 151936-word head (512 of 256 columns and 163 of 128) run in one round,
// and a workgroup's wait or epilogue overlaps the other two's streams.  Same stages, reads and MFMAs.  This
// form runs for one row block only, where every byte of the head is read
// once per call, so its head loads carry the non-temporal hint (the hidden
// rows, which every workgroup reads, keep the default policy).
//
// one_half = true computes the first 128 columns only (a 64 x 128 tile): the
// waves of column half 1 load no B rows and issue no MFMAs (their
// accumulators stay 0), but still take part in the A loads and barriers.
template <typename T, int kStages = 2>
__device__ __forceinline__ void gemm_mainloop_rows64(const GemmOperands& op, int M,
                                                     int m0, int n0, int nk,
                                                     f32x16 (&acc)[1][kTN],
                                                     char* lds,
                                                     bool one_half = false) {
  static_assert(kStages == 1 || kStages == 2, "one or two stages");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
#pragma unroll
  for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][ni][r] = 0.f;
  if (nk <= 0) return;

  const int a_off = (wm * 32 + (lane & 31)) * kRowBytes;
  int b_off[kTN];
#pragma unroll
  for (int ni = 0; ni < kTN; ++ni)
    b_off[ni] = (wn * 128 + ni * 32 + (lane & 31)) * kRowBytes;
  int c_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c_off[s] = ((2 * s + (lane >> 5)) ^ swz(lane & 31)) << 4;

  // load i of wave wu fills 8 rows (lane / 8 picks the row, lane % 8 the
  // physical chunk, which holds logical chunk (lane % 8) ^ swz(row)):
  // A rows 16 wu + 8 i (i < 2), B rows 64 wu + 8 i (i < 8)
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  const int wu = __builtin_amdgcn_readfirstlane(wid);
  const bool mma = !(one_half && (wu & 1));       // column half wn = wu & 1
  const bool loads_b = !(one_half && wu >= 2);    // B rows 64 wu .. + 63
  const char* ga[2];
  const char* gb[8];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wu * 16 + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    int m = m0 + r;
    m = m < M ? m : M - 1;
    const int64_t prow = op.a_rows ? (int64_t)op.a_rows[op.a_base + m] : op.a_base + m;
    ga[i] = op.A + prow * op.lda + c * 16;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = wu * 64 + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    int n = n0 + r;
    n = n < op.N ? n : op.N - 1;
    gb[i] = op.B + (int64_t)n * op.ldb + c * 16;
  }
  auto dma = [&](int kt, int stage) {
    const int64_t k = (int64_t)kt * kRowBytes;
    char* sa = lds + stage * kStageBytes64;
    char* sb = sa + kOperandBytesA64;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(ga[i] + k,
                                       (lds_ptr_t)(sa + (wu * 16 + 8 * i) * kRowBytes),
                                       16, 0, 0);
    if (loads_b) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_global_load_lds(gb[i] + k,
                                         (lds_ptr_t)(sb + (wu * 64 + 8 * i) * kRowBytes),
                                         16, 0, kStages == 1 ? kPolicyNT : 0);
    }
  };

  if constexpr (kStages == 2) {
    dma(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kStages == 2 ? kt & 1 : 0;
    if constexpr (kStages == 2) {
      // buffer cur ^ 1 was drained by the barrier that ended stage kt - 1
      if (kt + 1 < nk) dma(kt + 1, cur ^ 1);
    } else {
      // the one buffer was drained by the barrier that ended stage kt - 1
      dma(kt, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    const char* sa = lds + cur * kStageBytes64;
    const char* sb = sa + kOperandBytesA64;
    if (mma) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 fa = *reinterpret_cast<const u32x4*>(sa + a_off + c_off[s]);
        u32x4 fb[kTN];
#pragma unroll
        for (int ni = 0; ni < kTN; ++ni)
          fb[ni] = *reinterpret_cast<const u32x4*>(sb + b_off[ni] + c_off[s]);
#pragma unroll
        for (int ni = 0; ni < kTN; ++ni)
          mfma_step(acc[0][ni], fb[ni], fa, (const T*)nullptr);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

// ---- MX-format B operand (the release-precision head) ----
// gfx950's scaled conversions
// (v_cvt_scalef32_pk_bf16_fp4 / _fp8: two codes times a float scale to two
// bf16 values, low nibble / low byte first), which an exhaustive check over
// every code at every E8M0 scale found exact wherever the result is a bf16
// number -- the whole valid range, subnormal results included.  The scale
// 2^s is the float with exponent field s + 127 (2^-127: the subnormal
// 0x00400000).
__device__ __forceinline__ float e8m0_scale(int code) {
  return __builtin_bit_cast(float, code == 0 ? 0x00400000u : (uint32_t)code << 23);
}

// 8 E2M1 codes (4 bytes, low nibble first) -> 8 bf16 values
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t c, float sc) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 0)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 1)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 2)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, sc, 3))};
}
// 8 E4M3 codes (8 bytes, low byte first) -> 8 bf16 values
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 c, float sc) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, true))};
}

__device__ __forceinline__ bool mx_scale_ok(int fmt, int code) {
  const int s = code - 127;
  return code != 255 && (fmt == 0 ? s <= 125 : (s >= -124 && s <= 119));
}

// The 64-row tile with the head W read from MX storage (codes and E8M0
// block scales) instead of bf16.  Each fragment of W is made in registers by
// the scaled conversions above -- exact on every valid block -- so the MFMA
// operands, and with them every accumulator, equal those of
// gemm_mainloop_rows64 on the expanded bf16 head.  A stage is 64 A rows
// (bf16, swizzled as in gemm_mainloop), the stage's 64 K values of the 256 W
// rows as codes, and one dword of scales per W row (4 blocks: this stage and
// its even/odd partner); all arrive by LDS DMA in a ring of kRing stages, so
// kRing - 1 stages stream while one feeds the MFMAs, one barrier per stage.
// Code rows are 32 (E2M1) or 64 (E4M3) bytes whose 16-byte chunks are XOR
// swizzled by row bits 3 (E2M1) or 2..3 (E4M3), which keeps the fragment
// reads bank-conflict free.  Needs H % 128 == 0 (whole scale dwords).
// A block with an invalid scale gives NaN fragments and sets `bad`.
template <int kFmt>
struct MxStage {
  static constexpr int kCodeRow = kFmt == 0 ? 32 : 64;
  static constexpr int kCodes = 256 * kCodeRow;
  static constexpr int kScales = 256 * 4;
  static constexpr int kBytes = kOperandBytesA64 + kCodes + kScales;
  // stages in the ring: three (E2M1: 51 KB, three workgroups share a CU, so
  // the Qwen3-4B head's 594 tiles of 256 columns run in one round; E4M3:
  // 75 KB, two)
  static constexpr int kRing = 3;
  static constexpr int kLds = kRing * kBytes;
  static constexpr int kCodeLoads = kCodes / 4096;      // per wave per stage
  static constexpr int kLoads = 2 + kCodeLoads + 1;     // A, codes, scales
};

template <int kFmt>
__device__ __forceinline__ void gemm_mainloop_rows64_mx(
    const GemmOperands& op, const uint8_t* wcodes, const uint8_t* wscales,
    int H, int M, int m0, int n0, int nk, f32x16 (&acc)[1][kTN], char* lds,
    bool& bad) {
  using S = MxStage<kFmt>;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1, half = lane >> 5;
#pragma unroll
  for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[0][ni][r] = 0.f;
  if (nk <= 0) return;

  const int a_off = (wm * 32 + (lane & 31)) * kRowBytes;
  int c_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c_off[s] = ((2 * s + (lane >> 5)) ^ swz(lane & 31)) << 4;
  int brow[kTN];
#pragma unroll
  for (int ni = 0; ni < kTN; ++ni) brow[ni] = wn * 128 + ni * 32 + (lane & 31);

  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  const int wu = __builtin_amdgcn_readfirstlane(wid);
  const int64_t code_ld = kFmt == 0 ? H / 2 : H, scale_ld = H / 32;
  const char* ga[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wu * 16 + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    int m = m0 + r;
    m = m < M ? m : M - 1;
    const int64_t prow = op.a_rows ? (int64_t)op.a_rows[op.a_base + m] : op.a_base + m;
    ga[i] = op.A + prow * op.lda + c * 16;
  }
  // code loads: lane l of load i lands at LDS offset 16 l of its 1 KB span,
  // i.e. physical chunk l % (kCodeRow / 16) of row l / (kCodeRow / 16); it
  // fetches the logical chunk the swizzle places there
  // sized 4, the larger count (the host pass rejects capturing an array
  // whose size depends on the local alias)
  const char* gc[4] = {nullptr, nullptr, nullptr, nullptr};
#pragma unroll
  for (int i = 0; i < S::kCodeLoads; ++i) {
    constexpr int kChunks = S::kCodeRow / 16;
    const int r = wu * 64 + i * (64 / S::kCodeLoads) + lane / kChunks;
    const int phys = lane % kChunks;
    const int logical = kFmt == 0 ? phys ^ ((r >> 3) & 1) : phys ^ ((r >> 2) & 3);
    int n = n0 + r;
    n = n < op.N ? n : op.N - 1;
    gc[i] = (const char*)wcodes + (int64_t)n * code_ld + logical * 16;
  }
  int ns = n0 + wu * 64 + lane;
  ns = ns < op.N ? ns : op.N - 1;
  const char* gs = (const char*)wscales + (int64_t)ns * scale_ld;

  constexpr int kStB = MxStage<kFmt>::kBytes, kCL = MxStage<kFmt>::kCodeLoads;
  constexpr int kCR = MxStage<kFmt>::kCodeRow, kCB = MxStage<kFmt>::kCodes;
  auto dma = [&](int kt, int buf) {
    char* st = lds + buf * kStB;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_global_load_lds(ga[i] + (int64_t)kt * kRowBytes,
                                       (lds_ptr_t)(st + (wu * 16 + 8 * i) * kRowBytes),
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < kCL; ++i)
      __builtin_amdgcn_global_load_lds(
          gc[i] + (int64_t)kt * kCR,
          (lds_ptr_t)(st + kOperandBytesA64 + (wu * 64 + i * (64 / kCL)) * kCR),
          16, 0, 0);
    __builtin_amdgcn_global_load_lds(gs + (kt >> 1) * 4,
                                     (lds_ptr_t)(st + kOperandBytesA64 + kCB + wu * 256),
                                     4, 0, 0);
  };

#pragma unroll
  for (int p = 0; p < S::kRing - 1; ++p)
    if (p < nk) dma(p, p);
  bool anybad = false;
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt are done when at most those of the
    // stages after it (up to kRing - 2 of them) are outstanding; the barrier
    // then makes every wave's visible and retires the reads of stage kt - 1,
    // whose buffer takes stage kt + kRing - 1
    const int later = (nk - 1 - kt) < (S::kRing - 2) ? (nk - 1 - kt) : (S::kRing - 2);
    if constexpr (S::kLoads == 5) {
      if (later >= 2) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
      else if (later == 1) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      if (later >= 2) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
      else if (later == 1) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (kt + S::kRing - 1 < nk) dma(kt + S::kRing - 1, (kt + S::kRing - 1) % S::kRing);
    const char* st = lds + (kt % S::kRing) * S::kBytes;
    const char* sc = st + kOperandBytesA64;
    const char* ss = sc + S::kCodes;
    // everything the stage needs from LDS first (one wait), then all 16
    // fragments of W, then the 16 MFMAs: per accumulator still k = 0, 1, ...
    uint32_t sw[kTN];
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni)
      sw[ni] = *reinterpret_cast<const uint32_t*>(ss + brow[ni] * 4);
    u32x4 fa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      fa[s] = *reinterpret_cast<const u32x4*>(st + a_off + c_off[s]);
    constexpr int kCh = S::kCodeRow / 16;  // 16-byte chunks per code row
    u32x4 cw[kTN][kCh];
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
      for (int c = 0; c < kCh; ++c) {
        const int sw_bits = kFmt == 0 ? ((brow[ni] >> 3) & 1) : ((brow[ni] >> 2) & 3);
        cw[ni][c] = *reinterpret_cast<const u32x4*>(sc + brow[ni] * S::kCodeRow +
                                                    ((c ^ sw_bits) << 4));
      }
    const int sbyte = 2 * (kt & 1);
    u32x4 fb[4][kTN];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ni = 0; ni < kTN; ++ni) {
        const int code = (sw[ni] >> (8 * (sbyte + (s >> 1)))) & 0xFF;
        const bool ok = mx_scale_ok(kFmt, code);
        anybad |= !ok;
        u32x4 v;
        if constexpr (kFmt == 0) {
          // K values 16 s + 8 half .. + 7: chunk s / 2, word 2 (s % 2) + half
          const u32x4 ch = cw[ni][s >> 1];
          const uint32_t c4 = (s & 1) ? (half ? ch[3] : ch[2]) : (half ? ch[1] : ch[0]);
          v = fp4x8_to_bf16(c4, e8m0_scale(code));
        } else {
          // chunk s, words 2 half and 2 half + 1
          const u32x4 ch = cw[ni][s];
          const u32x2 c8 = half ? u32x2{ch[2], ch[3]} : u32x2{ch[0], ch[1]};
          v = fp8x8_to_bf16(c8, e8m0_scale(code));
        }
        fb[s][ni] = ok ? v : u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
      }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ni = 0; ni < kTN; ++ni)
        mfma_step(acc[0][ni], fb[s][ni], fa[s], (const bf16*)nullptr);
  }
  __syncthreads();  // the caller may reuse the ring's LDS
  bad = anybad;
}

}  // namespace rz
