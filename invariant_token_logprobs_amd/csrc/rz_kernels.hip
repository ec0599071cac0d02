// rz_kernels.hip -- the HIP kernels of the REINFORCE Zero learner hot path.
//
// Sources (page title and section): the REINFORCE Zero project page
// ("hujian.website"), section 02 "A minimal REINFORCE objective" (loss,
// T_i, gradient through the numerator); the vLLM blog "Zero mismatch, simple
// async RL" (zh translation), sections 2-4 (w = pi / mu unclipped, group-mean
// advantage, D3, rollout-to-learner KL) and section 5 ("diff 0": bitwise
// identical logprobs between rollout and trainer).
#include <math.h>

#include "rz_gemm.h"
#include "rz_internal.h"

// the 256 x 256 tile on eight waves (gemm_mainloop), two per SIMD
#define RZ_GEMM_ATTR \
  __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))

namespace rz {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kIntMin = -2147483647 - 1;

// Row counts up to which the forward runs on the 64-row tile, measured at
// the Qwen3-4B head against the eight-wave 256-row tile: the logits forward
// gains up to 128 rows, the draw, whose epilogue spreads over four times the
// workgroups, up to 192 (per call at 96 / 128 / 192 / 256 rows: 0.249 /
// 0.262 / 0.310 / 0.385 ms against 0.302 / 0.310 / 0.317 / 0.331 ms).  The
// MX head keeps the 64-row tile up to 256 rows for the draw: past it the
// head is expanded on every call.  Up to 64 rows (one row block) the
// single-stage form runs, three workgroups per CU.
constexpr int kRows64MaxLogits = 128;
constexpr int kRows64MaxSample = 192;
constexpr int kRows64MaxMxSample = 256;

// Logits of vocabulary columns >= V inside the last statistics tile: finite, so
// the row maximum stays finite and no (-inf) - (-inf) can appear.
constexpr float kMaskedLogit = -1.0e30f;

__device__ __forceinline__ RowCount to_rc(const DevRows& r) {
  return RowCount{r.count, r.base, r.cap};
}

template <typename T>
__device__ __forceinline__ float load_f(const T* p) {
  return (float)(*p);
}

template <typename T>
__device__ __forceinline__ T from_f(float x) {
  return (T)x;
}

}  // namespace

// ===================================================================
// bi_lmhead_gemm (forward): z = h W^T on one 256 x 256 tile, with the
// log-softmax partials and the sampled-token gather fused in the epilogue.
// Per (row, statistics tile of 128 columns) it writes m = max_v z and
// s = sum_v exp(z - m) over the tile's columns (pad columns >= V excluded),
// and z[a_t] when the row's token falls in the tile.  Nothing of the logits
// leaves the chip.
// ===================================================================
struct FwdArgs {
  GemmOperands op;
  DevRows rows;
  int V, Vpad, nk, mt, nt;
  float2* partials;       // (tile j, list position p) at j * ldp + p * ldr
  int64_t ldp, ldr;
  void* e;                // learner call only: e (see EStore) [rows][lde]
  int64_t lde;
  const uint64_t* row_ids;  // sampling call only: the rows' identities
  uint64_t seed;
  float2* cand;           // sampling call only, as partials: (best z + g, index)
  float* candz;           // sampling call only, as partials: the best column's z
  const int* row_tokens;  // logits calls: a_t by list position (nullable)
  float* ztgt;            // logits calls: z[t, a_t] by list position
  const uint8_t* wcodes;  // MX head only: codes and E8M0 scales of W
  const uint8_t* wscales;
  int H;                  // MX head only: hidden size
  int* err;               // MX head only: RZ_DEVERR_MX_SCALE
  int nfull;              // single-stage 64-row form: 256-column workgroups
};

// What the learner's forward stores for the backward.
//
// fp32 inputs: e = exp(z - m_j) in (0, 1], m_j the maximum of the statistics
// tile j holding the column, which the dz rescale turns into
// dz = c_t exp(m_j - lse_t) e (and dz^T) once lse is known.
//
// bf16 inputs: e = exp(z - r ln 2) rounded to bf16, the backward GEMMs' A
// operand as it stands.  r is an integer fixed by the tile maximum alone
// (e_ref2): 0 while m_j log2 e lies in [-kERefLo2, kERefHi2], else the
// nearest integer that brings the tile maximum's e back to that window, so
// e never overflows and a tile's largest terms stay normal.  With r the same
// over a row's tiles, dz = c_t exp(r ln 2 - lse_t) e: one factor per row,
// which the dHidden epilogue applies in fp32 and the dW GEMM takes through
// its other operand (h^T scaled per row).  A row whose tiles straddle the
// window (a tile maximum past 2^80 or below 2^-32 in e units; no realistic
// logits do this) has its tiles rebased to the row's own r by exact powers of
// two (k_erebase).  The row's own token column and the rows past the chunk's
// count up to the next multiple of 64 (the dW GEMM's last K stage) are 0.
template <typename T> struct EStore { typedef float type; };
template <> struct EStore<bf16> { typedef bf16 type; };
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
constexpr float kERefHi2 = 80.f;  // e <= 2^80: V e |W| stays far inside fp32
constexpr float kERefLo2 = 32.f;  // a tile maximum's e >= 2^-32
__device__ __forceinline__ float e_ref2(float m) {
  const float mu = m * kLog2e;
  return mu > kERefHi2 ? ceilf(mu - kERefHi2)
                       : (mu < -kERefLo2 ? floorf(mu + kERefLo2) : 0.f);
}
// two bf16 values in one word, each times f and rounded to bf16 (nearest
// even)
__device__ __forceinline__ uint32_t scale_bf16x2(uint32_t w, float f) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {__builtin_bit_cast(float, w << 16) * f,
                   __builtin_bit_cast(float, w & 0xffff0000u) * f};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
template <bool B> struct BoolC { static constexpr bool value = B; };
template <int I> struct IntC { static constexpr int value = I; };
// f(IntC<I>{}) for I = B .. E - 1: indices stay compile-time constants
// whatever the unroller decides about a loop this large
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

// LDS staging of a 256 x 256 fp16 e tile, 512 bytes per row, for coalesced
// 16-byte stores.  The 16-byte chunk k of row R sits at chunk k ^ (R % 32):
// the 8-byte writes of one instruction (32 rows, one chunk) then hit every
// bank exactly twice, and a row read back by 32 lanes is a permutation of
// its own 512 bytes.
__device__ __forceinline__ int e_stage_off(int R, int k) {
  return R * 512 + ((k ^ (R & 31)) << 4);
}

// ---- the rollout-side draw ----
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3", SC 2011): ten rounds of two 32 x 32 -> 64-bit
// products on counter words 0 and 2, the halves and the key XORed into the
// next counter; the key grows by fixed Weyl increments between rounds.
// Four blocks at once (counters c[0..3], one key), the four independent
// chains interleaved in each round, so each wave has four products in
// flight instead of waiting on each round's product in turn.  The round
// loop is unrolled by two only: the counters then alternate between two
// register sets with no copies at the loop's end, while a fully unrolled
// loop at the draw's call sites stops the enclosing loops from unrolling
// (the accumulators they index would move to scratch memory).  One 64-bit
// product gives both halves (v_mad_u64_u32).
__device__ __forceinline__ void philox4x32_10_x4(u32x4 (&c)[4], uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll 2
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t p0 = (uint64_t)c[i][0] * 0xD2511F53u;
      const uint64_t p1 = (uint64_t)c[i][2] * 0xCD9E8D57u;
      // a ^ b ^ c in one v_bitop3_b32 (truth table 0x96)
      c[i] = u32x4{(uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[i][1], k0, 0x96),
                   (uint32_t)p1,
                   (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[i][3], k1, 0x96),
                   (uint32_t)p0};
    }
  }
}

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kTwoM32 = 2.3283064365386963e-10f;  // 2^-32
constexpr float kTwoM33 = 1.1641532182693481e-10f;  // 2^-33

// The draw's score of logit z with Gumbel noise g = -ln(-ln u), u =
// (x + 1/2) 2^-32, up to one constant: z + g + ln(ln 2) = z - ln(E2) with
// E2 = -log2 u, so a single log2 forms E2 and the constant ln(ln 2), the
// same for every column, never changes a comparison.  The largest g come
// from u near 1, where E2 ~ w / ln 2, w = 1 - u.  There, for
// x >= 2^32 - 2^26 (w < 2^-6), E2 is a three-term series in w, which is
// exact from the integer (w = (~x + 1/2) 2^-32) and truncated at w^4 / 4
// (<= 2^-20 relative); elsewhere E2 = -log2 of u rounded to fp32, whose
// rounding (at most 2^-25 near 1) moves E2 by at most 2^-25 / w <= 2^-19
// relative.  Either way the score moves by at most 2^-19.  Every lane
// evaluates both forms and selects (no divergent branches).
__device__ __forceinline__ float draw_score(float z, uint32_t x) {
  // (x + 1/2) 2^-32 as one fma: the scaling by a power of two is exact, so
  // this rounds once, as (float(x) + 1/2) then * 2^-32 does
  const float u = __builtin_fmaf((float)x, kTwoM32, kTwoM33);
  const float w = __builtin_fmaf((float)(~x), kTwoM32, kTwoM33);  // 1 - u
  const float L = -__builtin_amdgcn_logf(u);
  // -log2(1 - w) = (w / ln 2) (1 + w / 2 + w^2 / 3 + ...)
  const float series = w * (kLog2e + w * (0.5f * kLog2e + w * (kLog2e / 3.f)));
  const float E2 = x < 0xFC000000u ? L : series;
  return __builtin_fmaf(__builtin_amdgcn_logf(E2), -kLn2, z);
}

// (score, index) order of the draw: larger score first, then smaller index
__device__ __forceinline__ bool draw_better(float s, int v, float bs, int bv) {
  return s > bs || (s == bs && v < bv);
}

// bi_lmhead_gemm + the log-softmax statistics of a logits tile: per row t
// and statistics tile j (128 vocabulary columns, one wave's column half),
// m_j = max_v z[t, v] and s_j = sum_v exp(z[t, v] - m_j), written to
// partials[j ldp + t ldr]; on the learner call also e for the backward (see
// EStore).
//
// The MFMAs run with swapped operands (see gemm_mainloop), so each lane
// holds one row t and, per 32 x 32 block, four runs of four consecutive
// vocabulary columns.  A wave owns whole statistics tiles, so row statistics
// are in-lane folds over the wave's 128 columns and one exchange with lane
// l ^ 32, in a fixed order that depends only on the column, never on the
// row's position or the batch: the per-row result is the same in every
// launch (batch invariance).  The maximum is exact in any order, so it is
// taken first over the statistics tile; one exp per element then serves
// both s_j and e.
//
// TM = 32-row blocks per wave: 2 for the 256-row tile on eight waves
// (gemm_mainloop; wave w owns rows 64 (w % 4) .. + 63 of column half
// w / 4), 1 for the 64-row tiles for small row counts (four waves, wave w
// owning rows 32 (w / 2) .. + 31 of column half w % 2).  The single-stage
// 64-row form (kStages64 = 1, one row block) takes 256 columns in workgroups
// [0, nfull) and 128 columns (one statistics tile; the column-half-1 waves
// idle) in the rest, so that the head's columns spread evenly over the CUs
// (see split_columns).  Every form runs the same MFMA per 32 x 32 block
// in the same K order and the same per-wave folds below, so a row's
// statistics and draw are bit-identical whichever tile computes them.
// kWFmt: -1 for a bf16 / fp32 head, 0 / 1 for an MXFP4 / MXFP8 head read
// by the 64-row tile (the accumulators are those of the expanded head).
// kTokOff: byte offset in lds of the tile's row tokens for the gather
// (-1: none; the gather then reads them from global memory).
template <typename T, bool kStoreE, bool kSample, int TM, int kWFmt = -1,
          int kStages64 = 2, int kTokOff = -1>
__device__ __forceinline__ void fwd_logits_body(const FwdArgs& a, char* lds) {
  static_assert(TM == 2 || (TM == 1 && !kStoreE), "64-row tiles: no e output");
  constexpr bool kW8 = TM == 2;  // the 256-row tile on eight waves
  constexpr int NT = kW8 ? 2 * kThreads : kThreads;  // threads per workgroup
  constexpr bool kMixed = TM == 1 && kStages64 == 1 && kWFmt < 0;
  constexpr int BM = kW8 ? kBM : 64 * TM;  // tile rows
  constexpr int RW = 32 * TM;       // rows per wave
  const RowCount rc = to_rc(a.rows);
  const int M = rc.get();
  int m0, n0;
  bool one_half = false;  // a 128-column workgroup of the single-stage form
  if constexpr (kMixed) {
    // one row block (the host launches this form for at most 64 rows);
    // a.nt counts the workgroups
    if (M <= 0 || (int)blockIdx.x >= a.nt) return;
    const int b = blockIdx.x;
    one_half = b >= a.nfull;
    m0 = 0;
    n0 = one_half ? a.nfull * kBN + (b - a.nfull) * (kBN / 2) : b * kBN;
  } else {
    // Only the tiles of the M rows present are numbered (M may be a device
    // count below the launch bound), so the active tiles spread over all
    // XCDs.
    const int mt = (M + BM - 1) / BM;
    if ((int)blockIdx.x >= mt * a.nt) return;
    const TileCoord tc = map_tile(blockIdx.x, mt * a.nt, mt, a.nt);
    m0 = tc.tm * BM;
    n0 = tc.tn * kBN;
  }

  // The 256-row tile's row tokens for the gather, brought into LDS (stok,
  // outside the stage buffers) by one 4-byte DMA load per lane of waves
  // 0 .. 3 before the main loop: the main loop's stage waits and barriers
  // complete it, so the epilogue reads them without waiting on global
  // memory.  (The 64-row forms have no LDS to spare at their occupancy and
  // read them in the epilogue.)
  if constexpr (kTokOff >= 0) {
    if (a.row_tokens && threadIdx.x < kBM) {
      typedef __attribute__((address_space(3))) void* lds_ptr_t;
      const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      // an opaque copy of the thread index: the row computed here must not
      // be merged with the epilogue's (it would live, spilled, through the
      // whole main loop)
      int t = (int)threadIdx.x;
      asm volatile("" : "+v"(t));
      const int m = min(m0 + t, M - 1);  // in bounds; rows >= M unused
      __builtin_amdgcn_global_load_lds(a.row_tokens + rc.base + m,
                                       (lds_ptr_t)(lds + kTokOff + 256 * w), 4, 0, 0);
    }
  }

  f32x16 acc[TM][kTN];
  if constexpr (kW8) {
    gemm_mainloop<T>(a.op, M, m0, n0, a.nk, acc, lds);
  } else if constexpr (kWFmt < 0) {
    gemm_mainloop_rows64<T, kStages64>(a.op, M, m0, n0, a.nk, acc, lds, one_half);
  } else {
    bool bad = false;
    gemm_mainloop_rows64_mx<kWFmt>(a.op, a.wcodes, a.wscales, a.H, M, m0, n0,
                                   a.nk, acc, lds, bad);
    if (bad && a.err) atomicOr(a.err, 8);
  }

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // rows wm RW .. + RW - 1 and columns wn 128 .. + 127 of the tile
  const int wm = kW8 ? (wid & 3) : wid >> 1, wn = kW8 ? (wid >> 2) : (wid & 1);
  // the idle waves of a 128-column workgroup are done (no barrier follows
  // in this form's epilogue)
  if (one_half && wn) return;
  const int half = lane >> 5, l32 = lane & 31;
  // the wave's statistics tile: columns js * 128 .. + 127; none of them
  // below V only in the last tile column of a V that is not a multiple of
  // 256 (uniform across the wave)
  const int js = (n0 + wn * 128) / 128;
  const bool wvalid = js * 128 < a.V;
  // column of register r in block ni: cbase + 32 ni + 8 (r / 4) + (r % 4)
  const int cbase = n0 + wn * 128 + 4 * half;

  // The gather: z[t, a_t] straight from the accumulator that holds it, in the
  // one tile whose columns contain a_t (one lane of the workgroup), so
  // log pi = z[a_t] - lse subtracts two results of one accumulation.  The
  // branch is taken by about one row in six hundred per tile.
  if (a.row_tokens) {
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      const int R = wm * RW + mi * 32 + l32;
      const int m = m0 + R;
      int tok = -1;
      if constexpr (kTokOff >= 0) {
        if (m < M) tok = reinterpret_cast<const int*>(lds + kTokOff)[R];
      } else {
        if (m < M) tok = a.row_tokens[rc.base + m];
      }
      const int off = tok - cbase;  // this lane's columns: 32 ni + 8 q + j
      if (tok >= 0 && tok < a.V && off >= 0 && off < 128 && (off & 4) == 0) {
        const int want = ((off >> 5) << 4) | (((off >> 3) & 3) << 2) | (off & 3);
        float z = 0.f;
#pragma unroll
        for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
          for (int r = 0; r < 16; ++r) z = want == ni * 16 + r ? acc[mi][ni][r] : z;
        a.ztgt[rc.base + m] = z;
      }
    }
  }

  // Statistics-tile row maxima.  Columns >= V (last statistics tile only)
  // hold a copy of column V - 1 (the main loop reads B rows >= N from row
  // N - 1), which cannot change a maximum, so no mask is needed here.
  float rm[TM];
#pragma unroll
  for (int mi = 0; mi < TM; ++mi) {
    float mx = acc[mi][0][0];
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[mi][ni][r]);
    rm[mi] = fmaxf(mx, __shfl_xor(mx, 32, 64));
  }

  // exp(z - m) once per element, 0 for columns >= V; row sums in a fixed
  // order; the wave's partials straight to global memory
  typedef typename EStore<T>::type E;
  E* e = reinterpret_cast<E*>(a.e);
  auto pass2 = [&](auto full_c) {
    constexpr bool kFull = decltype(full_c)::value;
#pragma unroll
    for (int mi = 0; mi < TM; ++mi) {
      // a 32-row block wholly past the row count: nothing to compute
      // (uniform across the wave; its rows are never read back)
      if (m0 + wm * RW + mi * 32 >= M) continue;
      const int R = wm * RW + mi * 32 + l32;
      const bool rvalid = m0 + R < M;
      // exp(z - m) = 2^((z - m) log2 e).  z - m is formed first, so the
      // maximum's own term is 2^0 = 1 exactly: s >= 1, lse >= m, and
      // log pi = z[a_t] - lse <= 0 with lse = m exactly on a row whose other
      // tokens carry less than an ulp of mass.
      const float mrow = rm[mi];
      // bf16 store: exp(z - r ln 2) = exp(z - m) 2^(m log2 e - r)
      float esc = 0.f;
      if constexpr (kStoreE && sizeof(T) == 2)
        esc = __builtin_amdgcn_exp2f(mrow * kLog2e - e_ref2(mrow));
      float s = 0.f;
#pragma unroll
      for (int ni = 0; ni < kTN; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c0 = cbase + ni * 32 + 8 * q;  // multiple of 4
          float ev[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ev[j] = __builtin_amdgcn_exp2f((acc[mi][ni][4 * q + j] - mrow) * kLog2e);
            if constexpr (!kFull) ev[j] = c0 + j < a.V ? ev[j] : 0.f;
            s += ev[j];
          }
          if constexpr (kStoreE) {
            if constexpr (sizeof(T) == 2) {
              const bf16x4 hv = {(bf16)(ev[0] * esc), (bf16)(ev[1] * esc),
                                 (bf16)(ev[2] * esc), (bf16)(ev[3] * esc)};
              *reinterpret_cast<u32x2*>(
                  lds + e_stage_off(R, wn * 16 + ni * 4 + q) + half * 8) =
                  __builtin_bit_cast(u32x2, hv);
            } else {
              if (rvalid && c0 < a.Vpad)
                *reinterpret_cast<f32x4*>(e + (int64_t)(m0 + R) * a.lde + c0) =
                    f32x4{ev[0], ev[1], ev[2], ev[3]};
            }
          }
        }
      // the wave's 128 columns: lower lane half first
      const float so = __shfl_xor(s, 32, 64);
      if (half == 0 && rvalid && wvalid)
        a.partials[(int64_t)js * a.ldp + (rc.base + m0 + R) * a.ldr] =
            make_float2(mrow, s + so);
    }
  };
  if (n0 + wn * 128 + 128 <= a.V) pass2(BoolC<true>{});
  else pass2(BoolC<false>{});
  if constexpr (kStoreE && sizeof(T) == 2 && kTokOff >= 0) {
    // the row's own token column stays 0 in e (its dL/dz is applied exactly
    // in fp32 elsewhere): the lane that holds it clears its staged value
    if (a.row_tokens) {
#pragma unroll
      for (int mi = 0; mi < TM; ++mi) {
        const int R = wm * RW + mi * 32 + l32;
        if (m0 + R >= M) continue;
        const int tok = reinterpret_cast<const int*>(lds + kTokOff)[R];
        const int off = tok - cbase;
        if (tok >= 0 && tok < a.V && off >= 0 && off < 128 && (off & 4) == 0)
          *reinterpret_cast<uint16_t*>(
              lds + e_stage_off(R, wn * 16 + (off >> 5) * 4 + ((off >> 3) & 3)) +
              half * 8 + 2 * (off & 3)) = 0;
      }
    }
  }
  if constexpr (kSample) {
    // The draw: per row, the best z + g over the statistics tile's columns
    // < V (see draw_score; counter (v / 4, id_lo, id_hi, 0), key = the seed,
    // word v % 4), under draw_better's total order, so the order in which
    // lanes meet does not matter; one candidate per statistics tile.
    const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
    static_for<0, TM>([&](auto mi_c) {
      constexpr int mi = decltype(mi_c)::value;
      if (m0 + wm * RW + mi * 32 >= M) return;  // block past the row count
      const int R = wm * RW + mi * 32 + l32;
      const uint64_t id = m0 + R < M ? a.row_ids[rc.base + m0 + R] : 0;
      float bs = -__builtin_inff();
      int bo = -1;     // the best column's offset from cbase (-1: none)
      float bz = 0.f;  // the best column's logit: the record's z[a_t]
      // block ni of the lane: its four runs q = 0..3 of four columns, the
      // four Philox blocks computed together.  A lane meets its columns in
      // increasing order, so a strict > keeps the smallest index among equal
      // scores (draw_better's order); the winner's column is kept as its
      // offset from cbase, a constant per register.  Columns >= V (offset >=
      // lim, in the last statistics tile only) never win; the other tiles
      // take a copy of the loop without that test.
      const int lim = a.V - cbase;
      auto scan = [&](auto all_c) {
        constexpr bool kAll = decltype(all_c)::value;  // every column < V
        static_for<0, kTN>([&](auto ni_c) {
          constexpr int ni = decltype(ni_c)::value;
          u32x4 x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            x[q] = u32x4{(uint32_t)(cbase + ni * 32 + 8 * q) >> 2, (uint32_t)id,
                         (uint32_t)(id >> 32), 0u};
          philox4x32_10_x4(x, k0, k1);
          static_for<0, 16>([&](auto qj_c) {
            constexpr int q = decltype(qj_c)::value / 4, j = decltype(qj_c)::value % 4;
            constexpr int off = ni * 32 + 8 * q + j;
            const float z = acc[mi][ni][4 * q + j];
            const float sc = draw_score(z, x[q][j]);
            const bool take = kAll ? sc > bs : (sc > bs && off < lim);
            bs = take ? sc : bs;
            bo = take ? off : bo;
            bz = take ? z : bz;
          });
        });
      };
      if (n0 + wn * 128 + 128 <= a.V) scan(BoolC<true>{});
      else scan(BoolC<false>{});
      int bv = bo < 0 ? 0x7fffffff : cbase + bo;
      const float os = __shfl_xor(bs, 32, 64);
      const int ov = __shfl_xor(bv, 32, 64);
      const float oz = __shfl_xor(bz, 32, 64);
      if (draw_better(os, ov, bs, bv)) {
        bs = os;
        bv = ov;
        bz = oz;
      }
      if (half == 0 && m0 + R < M && wvalid) {
        const int64_t o = (int64_t)js * a.ldp + (rc.base + m0 + R) * a.ldr;
        a.cand[o] = make_float2(bs, __builtin_bit_cast(float, bv));
        a.candz[o] = bz;
      }
    });
  }
  if constexpr (kStoreE && sizeof(T) == 2) {
    __syncthreads();  // every wave's staged e
    // 16-byte row chunks: 32 lanes cover one 512-byte tile row.  Columns
    // >= V hold 0; rows from M up to the next multiple of 64 (read by the
    // dW GEMM's last K stage) are stored as 0, rows past that and columns
    // >= Vpad not at all.  The e stream (2 bytes per logit) is read back by
    // the backward GEMMs, long after: non-temporal stores keep it from
    // evicting the operand panels that the co-resident tiles share in L2.
    const int Mz = (M + 63) & ~63;
#pragma unroll 4
    for (int it = 0; it < 8192 / NT; ++it) {
      const int idx = it * NT + tid;
      const int R = idx >> 5, k = idx & 31;
      const int col = n0 + k * 8;
      if (m0 + R < Mz && col < a.Vpad)
        __builtin_nontemporal_store(
            m0 + R < M ? *reinterpret_cast<const u32x4*>(lds + e_stage_off(R, k))
                       : u32x4{0u, 0u, 0u, 0u},
            reinterpret_cast<u32x4*>(e + (int64_t)(m0 + R) * a.lde + col));
    }
  }
}

// The 256-row tile: eight waves (2 kThreads threads), two per SIMD.
template <typename T, bool kStoreE, bool kSample = false>
__global__ RZ_GEMM_ATTR void k_fwd_logits(FwdArgs a) {
  // [0, 128 KB): main-loop stages, then (learner call, bf16) the e tile;
  // then the row tokens (the draw gathers nothing: its tokens are drawn
  // later)
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes + (kSample ? 0 : 4 * kBM)];
  fwd_logits_body<T, kStoreE, kSample, 2, -1, 2, kSample ? -1 : kLdsBytes>(a, lds);
}

// The 64-row tile: 80 KB of LDS and a quarter of the accumulators, so two
// workgroups share a CU; for row counts where the 256-row tile would mostly
// compute rows that are not there.
template <typename T, bool kSample>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_fwd_logits64(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes64];
  fwd_logits_body<T, false, kSample, 1>(a, lds);
}

// The single-stage 64-row tile for at most 64 rows (one row block): 40 KB of
// LDS and at most 168 VGPRs, three workgroups per CU (see
// gemm_mainloop_rows64); same per-row results.  Workgroups [0, nfull) take
// 256 columns, the rest 128 (see split_columns).
template <typename T, bool kSample>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void k_fwd_logits64_1s(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kStageBytes64];
  fwd_logits_body<T, false, kSample, 1, -1, 1>(a, lds);
}

// The 64-row tile on an MX-format head (bf16 hidden states); E2M1 is sized
// for three workgroups per CU (LDS and at most 168 VGPRs), E4M3 for two.
template <int kFmt, bool kSample>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(kFmt == 0 ? 3 : 2, kFmt == 0 ? 3 : 2)))
void k_fwd_logits64_mx(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[MxStage<kFmt>::kLds];
  fwd_logits_body<bf16, false, kSample, 1, kFmt>(a, lds);
}

// ===================================================================
// bi_logsoftmax_gather merge: one wave per row.  Lane q folds the
// statistics-tile partials q, q + 64, q + 128, ... in ascending order with
// (m, s) <- (m', s e^(m - m') + s_j e^(m_j - m')), m' = max(m, m_j); the
// 64 lane results then meet in a fixed xor tree (offsets 32, 16, ..., 1),
// and lane 0's result is used.  lse = m + log s and log pi = z[a_t] - lse.
// The tree's shape and the tiles each lane folds depend only on V, never on
// the number of rows or the row's position.
// ===================================================================
constexpr int kMergeBatch = 20;  // tile partials loaded ahead per lane (1280 per wave)

__device__ __forceinline__ void ms_fold(float& m, float& s, float mj,
                                        float sj) {
  const float mn = fmaxf(m, mj);
  s = s * exp_approx(m - mn) + sj * exp_approx(mj - mn);
  m = mn;
}

// fold of two pairs where either may be empty (-inf, 0)
__device__ __forceinline__ void ms_merge(float& m, float& s, float mj, float sj) {
  if (mj == kNegInf) return;
  if (m == kNegInf) {
    m = mj;
    s = sj;
    return;
  }
  ms_fold(m, s, mj, sj);
}

// One row's log-sum-exp over its statistics tiles, by one wave: lane q
// folds tiles q, q + 64, ... in ascending order (loads kMergeBatch ahead),
// then the lanes meet in a fixed butterfly (offsets 32, 16, ..., 1).  The
// order depends on nt only, never on the row or the batch.  mlo: the
// smallest tile maximum (learner call only).
__device__ __forceinline__ float row_lse(const float2* __restrict__ partials,
                                         int64_t ldp, int64_t ldr, int nt,
                                         int64_t pos,
                                         bool want_mlo, float* m_out,
                                         float* mlo_out) {
  const int q = threadIdx.x & 63;
  float m = kNegInf, s = 0.f, mlo = __builtin_inff();
  for (int t0 = q; t0 < nt; t0 += 64 * kMergeBatch) {
    float2 ms[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int t = t0 + 64 * j;
      if (t < nt) ms[j] = partials[(int64_t)t * ldp + pos * ldr];
    }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      if (t0 + 64 * j < nt) {
        ms_merge(m, s, ms[j].x, ms[j].y);
        mlo = fminf(mlo, ms[j].x);
      }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mj = __shfl_xor(m, o, 64);
    const float sj = __shfl_xor(s, o, 64);
    ms_merge(m, s, mj, sj);
    if (want_mlo) mlo = fminf(mlo, __shfl_xor(mlo, o, 64));
  }
  *m_out = m;
  *mlo_out = mlo;
  return m + logf(s);
}

// log pi = z[a_t] - lse for a token in range, else NaN (and err bit 1).
// z[a_t] is an element of the tile statistics' own accumulators, so
// z[a_t] <= m <= lse (the tile holding the maximum adds exp2(0) = 1 to s)
// and log pi <= 0 already; the clamp keeps that promise for any input (NaN
// stays NaN).
__device__ __forceinline__ float logpi_of(int tok, int V, float z, float lse,
                                          int* err) {
  if (tok >= 0 && tok < V) {
    const float lp = z - lse;
    return lp > 0.f ? 0.f : lp;
  }
  if (err) atomicOr(err, 1);
  return __builtin_nanf("");
}

// Learner call (eref non-null): also the row's e reference r* = e_ref2 of
// the row maximum, and whether any of its tiles was stored against another
// (e_ref2 is monotone, so that is exactly when the smallest tile maximum
// maps elsewhere); k_erebase fixes those rows.
__global__ __launch_bounds__(256) void k_lse_merge(
    const float2* __restrict__ partials, int64_t ldp, int64_t ldr, int nt,
    DevRows rows,
    const float* __restrict__ ztgt, const int* __restrict__ row_tokens, int V,
    float* lse_out, float* logpi_out, const int* scatter_idx,
    float* logprobs_rows, int* err, float* eref, int* eflag) {
  const RowCount rc = to_rc(rows);
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= rc.get()) return;  // uniform per wave
  const int64_t pos = rc.base + p;
  float m, mlo;
  const float lse = row_lse(partials, ldp, ldr, nt, pos, eref != nullptr, &m, &mlo);
  if ((threadIdx.x & 63) != 0) return;
  const int tok = row_tokens[pos];
  const float lp = logpi_of(tok, V, tok >= 0 && tok < V ? ztgt[pos] : 0.f, lse, err);
  if (lse_out) lse_out[pos] = lse;
  if (logpi_out) logpi_out[pos] = lp;
  if (scatter_idx) logprobs_rows[scatter_idx[pos]] = lp;
  if (eref) {
    const float r = e_ref2(m);
    eref[pos] = r;
    eflag[pos] = e_ref2(mlo) != r;
  }
}

// The draw's merge and record, per row (one wave): the best (score, index)
// over the statistics tiles' candidates under draw_better's total order (so
// any meeting order of lanes and tiles gives the same winner), whose logit
// comes along as the record's z[a_t]; then the row's lse by row_lse, the
// fold k_lse_merge takes, and log mu = z[a_t] - lse.
__global__ __launch_bounds__(256) void k_draw_merge(
    const float2* __restrict__ cand, const float* __restrict__ candz,
    const float2* __restrict__ partials, int64_t ldp, int64_t ldr, int nt,
    int64_t n, int V,
    int* __restrict__ tokens, float* __restrict__ logmu, float* __restrict__ lse_out) {
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int q = threadIdx.x & 63;
  if (p >= n) return;  // uniform per wave
  float bs = -__builtin_inff();
  int bv = 0x7fffffff;
  float bz = 0.f;
  for (int t0 = q; t0 < nt; t0 += 64 * kMergeBatch) {
    float2 c[kMergeBatch];
    float cz[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int t = t0 + 64 * j;
      if (t < nt) {
        c[j] = cand[(int64_t)t * ldp + p * ldr];
        cz[j] = candz[(int64_t)t * ldp + p * ldr];
      }
    }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int v = __builtin_bit_cast(int, c[j].y);
      if (t0 + 64 * j < nt && draw_better(c[j].x, v, bs, bv)) {
        bs = c[j].x;
        bv = v;
        bz = cz[j];
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float os = __shfl_xor(bs, o, 64);
    const int ov = __shfl_xor(bv, o, 64);
    const float oz = __shfl_xor(bz, o, 64);
    if (draw_better(os, ov, bs, bv)) {
      bs = os;
      bv = ov;
      bz = oz;
    }
  }
  float m, mlo;
  const float lse = row_lse(partials, ldp, ldr, nt, p, false, &m, &mlo);
  if (q == 0) {
    tokens[p] = bv;
    logmu[p] = logpi_of(bv, V, bz, lse, nullptr);
    if (lse_out) lse_out[p] = lse;
  }
}

// ===================================================================
// Valid-row compaction (T_i counts valid action tokens): stable ascending
// list of rows with mask = 1, their tokens and their responses.
// ===================================================================
constexpr int kCompactRows = 1024;

__device__ __forceinline__ int block_excl_scan256(int x, int* sh, int* total) {
  // Hillis-Steele over 256 threads (exact integer arithmetic)
  const int tid = threadIdx.x;
  sh[tid] = x;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int y = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += y;
    __syncthreads();
  }
  const int incl = sh[tid];
  if (total) *total = sh[255];
  __syncthreads();
  return incl - x;
}

__global__ __launch_bounds__(256) void k_mask_count(const uint8_t* mask,
                                                    int64_t n, int* blk) {
  __shared__ int sh[256];
  const int64_t base = (int64_t)blockIdx.x * kCompactRows + threadIdx.x * 4;
  int c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (base + i < n) c += mask[base + i] != 0;
  int total;
  block_excl_scan256(c, sh, &total);
  if (threadIdx.x == 0) blk[blockIdx.x] = total;
}

__global__ __launch_bounds__(1024) void k_mask_scan(int* blk, int nblk,
                                                    const int* cu, int B,
                                                    int64_t n, int* nvalid,
                                                    int* bad_cu, int* err) {
  __shared__ int sh[1024];
  const int tid = threadIdx.x;
  const int per = (nblk + 1023) / 1024;
  const int lo = tid * per, hi = min(nblk, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += blk[i];
  sh[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int y = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += y;
    __syncthreads();
  }
  int run = sh[tid] - sum;
  for (int i = lo; i < hi; ++i) {
    const int c = blk[i];
    blk[i] = run;
    run += c;
  }
  if (tid == 1023) *nvalid = sh[1023];
  // cu_rows must run 0 = cu[0] <= cu[1] <= ... <= cu[B] = n
  __shared__ int bad;
  if (tid == 0) bad = (cu[0] != 0) || ((int64_t)cu[B] != n);
  __syncthreads();
  for (int i = tid; i < B; i += 1024)
    if (cu[i] > cu[i + 1]) bad = 1;
  __syncthreads();
  if (tid == 0) {
    *bad_cu = bad;
    if (bad && err) atomicOr(err, 4);
  }
}

__device__ __forceinline__ int response_of(const int* cu, int B, int64_t row) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void k_mask_scatter(
    const uint8_t* mask, int64_t n, const int* blk_off, const int* tokens,
    const int* cu, int B, int* idx, int* tokv, int* respv) {
  __shared__ int sh[256];
  const int64_t base = (int64_t)blockIdx.x * kCompactRows + threadIdx.x * 4;
  uint8_t mk[4];
  int c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mk[i] = (base + i < n) ? (mask[base + i] != 0) : 0;
    c += mk[i];
  }
  int pos = blk_off[blockIdx.x] + block_excl_scan256(c, sh, nullptr);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (mk[i]) {
      const int64_t row = base + i;
      idx[pos] = (int)row;
      tokv[pos] = tokens[row];
      respv[pos] = response_of(cu, B, row);
      ++pos;
    }
}

// Masked rows: log pi reported as 0 and a zero gradient row.
__global__ __launch_bounds__(256) void k_rows_finalize(const uint8_t* mask,
                                                       int64_t n, int H,
                                                       float* logprobs,
                                                       float* d_hidden) {
  const int64_t row = blockIdx.x;
  if (row >= n || mask[row] != 0) return;
  if (threadIdx.x == 0) logprobs[row] = 0.f;
  float4* d = reinterpret_cast<float4*>(d_hidden + row * (int64_t)H);
  for (int i = threadIdx.x; i < H / 4; i += 256) d[i] = make_float4(0, 0, 0, 0);
}

// ===================================================================
// rz_loss.  Per response i (one workgroup): T_i = sum of mask, S_i = sum of
// w_t = exp(log pi_t - log mu_t) over valid rows (no clipping), summed in
// fp64 in a fixed order (per-thread strided partials, then a fixed tree).
// ===================================================================
__device__ __forceinline__ double block_sum_d(double x, double* sh) {
  const int tid = threadIdx.x;
  sh[tid] = x;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) sh[tid] += sh[tid + off];
    __syncthreads();
  }
  const double r = sh[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_sum_i(int x, int* sh) {
  const int tid = threadIdx.x;
  sh[tid] = x;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) sh[tid] += sh[tid + off];
    __syncthreads();
  }
  const int r = sh[0];
  __syncthreads();
  return r;
}

// T_i: valid rows of response i (cu_rows clamped to [0, n] so that a bad
// cu_rows cannot send the reads out of bounds; it is flagged separately).
__global__ __launch_bounds__(256) void k_resp_counts(const uint8_t* mask,
                                                     int64_t n, const int* cu,
                                                     int* T) {
  __shared__ int shi[256];
  const int i = blockIdx.x;
  int64_t lo = cu[i], hi = cu[i + 1];
  lo = lo < 0 ? 0 : (lo > n ? n : lo);
  hi = hi < lo ? lo : (hi > n ? n : hi);
  int c = 0;
  for (int64_t t = lo + threadIdx.x; t < hi; t += 256) c += mask[t] != 0;
  c = block_sum_i(c, shi);
  if (threadIdx.x == 0) T[i] = c;
}

// Group sums over the responses ordered by group id (stable, so ascending
// i within a group): the first response of each group's run sums the
// group's rewards in that order (fp64) and counts them.  Invalid ids sort
// last (as B), so the last entry tells whether there was one.
__global__ __launch_bounds__(256) void k_group_sums(int B, const int* skey,
                                                    const int* sval,
                                                    const float* rewards,
                                                    int* gcnt, double* gsum,
                                                    int* bad_gid) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= B) return;
  const int g = skey[q];
  if (q == B - 1) *bad_gid = g >= B;
  if (g >= B || (q > 0 && skey[q - 1] == g)) return;
  int c = 0;
  double r = 0.0;
  for (int j = q; j < B && skey[j] == g; ++j) {
    ++c;
    r += (double)rewards[sval[j]];
  }
  gcnt[g] = c;
  gsum[g] = r;
}

// Advantages: A_i = r_i - mean of r over the group of i, and the
// per-response factor A_i / (B T_i) of c_t (NaN when a group id or cu_rows
// is invalid).
__global__ __launch_bounds__(256) void k_advantages(
    const float* rewards, const int* gid, int B, const int* T,
    const int* bad_cu, const int* bad_gid, const int* gcnt, const double* gsum,
    double* Ad, double* fcoef, float* adv, int* err) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= B) return;
  const bool bad = *bad_cu || *bad_gid;
  double A = __builtin_nan(""), f = __builtin_nan("");
  if (!bad) {
    const int g = gid[i];
    A = (double)rewards[i] - gsum[g] / (double)gcnt[g];
    f = T[i] > 0 ? A / ((double)B * (double)T[i]) : 0.0;
  }
  Ad[i] = A;
  fcoef[i] = f;
  if (adv) adv[i] = (float)A;
  if (i == 0 && err && *bad_gid) atomicOr(err, 2);
}

// S_i = sum of w_t = exp(log pi_t - log mu_t) over the valid rows of
// response i (no clipping), fp64, per-thread strided partials then a fixed
// tree: the order depends only on the response's rows.  Score centering
// (sc = 1) sums log pi_t instead: its surrogate has w = 1 and the gradient
// of log pi.
__global__ __launch_bounds__(256) void k_resp_sums(const uint8_t* mask,
                                                   const float* logprobs,
                                                   const float* logmu,
                                                   int64_t n, const int* cu,
                                                   int sc, double* S) {
  __shared__ double shd[256];
  const int i = blockIdx.x;
  int64_t lo = cu[i], hi = cu[i + 1];
  lo = lo < 0 ? 0 : (lo > n ? n : lo);
  hi = hi < lo ? lo : (hi > n ? n : hi);
  double s = 0.0;
  for (int64_t t = lo + threadIdx.x; t < hi; t += 256)
    if (mask[t])
      s += sc ? (double)logprobs[t] : (double)expf(logprobs[t] - logmu[t]);
  s = block_sum_d(s, shd);
  if (threadIdx.x == 0) S[i] = s;
}

// L = -(1/B) sum_i [T_i > 0] A_i S_i / T_i, a fixed tree over responses.
__global__ __launch_bounds__(256) void k_loss_value(const double* Ad,
                                                    const int* T,
                                                    const double* S, int B,
                                                    float* loss) {
  __shared__ double shd[256];
  double part = 0.0;
  for (int i = threadIdx.x; i < B; i += 256)
    part += T[i] > 0 ? Ad[i] * S[i] / (double)T[i] : 0.0;
  part = block_sum_d(part, shd);
  if (threadIdx.x == 0) *loss = (float)(-part / (double)B);
}

// c_t = A_i w_t / (B T_i): minus the derivative of L by log pi_t (the
// gradient flows through the numerator pi_theta only).  Score centering
// (sc = 1): c_t = A_i / (B T_i), the weight replaced by 1.  Also the whole
// dL/dz of the row's own token, c_t (p[a_t] - 1) = -c_t expm1(log pi_t),
// kept in fp32 (coef1 holds its negative): the bf16 dlogits leave that
// column out, because on a row whose token takes nearly all the mass
// c_t p[a_t] and c_t cancel to far less than bf16's rounding of either.
//
// bf16 learner (eref non-null): also g_t = exp(r*_t ln 2 - lse_t), the
// factor that turns the stored e into the softmax, and per workgroup the
// largest binary exponent of a finite nonzero c_t g_t (fexp_part); the
// chunk's scale 2^sigma (k_chunk_scale) brings the largest to [1/2, 1).
__global__ __launch_bounds__(256) void k_coef(DevRows rows,
                                              const float* logpi_v,
                                              const float* logmu,
                                              const int* idx,
                                              const int* respv,
                                              const double* fcoef, int sc,
                                              float* coef, float* coef1,
                                              const float* lse_v,
                                              const float* eref, float* gsc,
                                              int* fexp_part) {
  const RowCount rc = to_rc(rows);
  const int q = blockIdx.x * 256 + threadIdx.x;
  int ex = kIntMin;
  if (q < rc.get()) {
    const int64_t p = rc.base + q;
    const float lp = logpi_v[p];
    const double c = sc ? fcoef[respv[p]]
                        : fcoef[respv[p]] * (double)expf(lp - logmu[idx[p]]);
    coef[p] = (float)c;
    coef1[p] = (float)(-c * expm1((double)lp));
    if (eref) {
      const float g = (float)exp2((double)eref[p] - (double)lse_v[p] * 1.4426950408889634);
      gsc[p] = g;
      const double f = (double)(float)c * (double)g;
      if (f != 0.0 && isfinite(f)) ex = ilogb(f);
    }
  }
  if (!eref) return;
  // the workgroup's largest exponent: a fixed tree over exact integers
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ex = max(ex, __shfl_xor(ex, o, 64));
  __shared__ int wex[4];
  if ((threadIdx.x & 63) == 0) wex[threadIdx.x >> 6] = ex;
  __syncthreads();
  if (threadIdx.x == 0)
    fexp_part[blockIdx.x] = max(max(wex[0], wex[1]), max(wex[2], wex[3]));
}

// sigma = -(1 + the largest exponent of the chunk's c_t g_t), or 0 if none
// is finite and nonzero: the dW operand h^T carries c_t g_t 2^sigma <= 1 in
// magnitude and the dW store takes 2^-sigma back (both exact powers of two).
__global__ __launch_bounds__(256) void k_chunk_scale(const int* fexp_part,
                                                     int nblk, int* sigma) {
  int ex = kIntMin;
  for (int i = threadIdx.x; i < nblk; i += 256) ex = max(ex, fexp_part[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ex = max(ex, __shfl_xor(ex, o, 64));
  __shared__ int wex[4];
  if ((threadIdx.x & 63) == 0) wex[threadIdx.x >> 6] = ex;
  __syncthreads();
  if (threadIdx.x == 0) {
    ex = max(max(wex[0], wex[1]), max(wex[2], wex[3]));
    *sigma = ex == kIntMin ? 0 : -(ex + 1);
  }
}

// ===================================================================
// rz_diagnostics: D3 = mean(expm1(d) - d), KL = mean(-d), d = log pi - log mu
// over valid entries.  Fixed 2048-entry chunks, each reduced by one fixed
// tree, then one fixed tree over the chunks: the order depends only on n.
// ===================================================================
constexpr int kDiagChunk = 2048;
struct DiagPartial {
  double d3, kl;
  long long cnt;
};

__global__ __launch_bounds__(256) void k_diag_partial(const float* logpi,
                                                      const float* logmu,
                                                      const uint8_t* mask,
                                                      int64_t n,
                                                      DiagPartial* out) {
  __shared__ double shd[256];
  __shared__ int shi[256];
  const int64_t base = (int64_t)blockIdx.x * kDiagChunk;
  double d3 = 0.0, kl = 0.0;
  int c = 0;
#pragma unroll
  for (int i = 0; i < kDiagChunk / 256; ++i) {
    const int64_t t = base + threadIdx.x + 256 * i;
    if (t < n && (!mask || mask[t])) {
      const double d = (double)logpi[t] - (double)logmu[t];
      d3 += expm1(d) - d;
      kl += -d;
      ++c;
    }
  }
  d3 = block_sum_d(d3, shd);
  kl = block_sum_d(kl, shd);
  c = block_sum_i(c, shi);
  if (threadIdx.x == 0) out[blockIdx.x] = DiagPartial{d3, kl, c};
}

__global__ __launch_bounds__(256) void k_diag_final(const DiagPartial* in,
                                                    int nchunk, float* diag) {
  __shared__ double shd[256];
  __shared__ long long shl[256];
  double d3 = 0.0, kl = 0.0;
  long long c = 0;
  for (int i = threadIdx.x; i < nchunk; i += 256) {
    d3 += in[i].d3;
    kl += in[i].kl;
    c += in[i].cnt;
  }
  d3 = block_sum_d(d3, shd);
  kl = block_sum_d(kl, shd);
  shl[threadIdx.x] = c;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) shl[threadIdx.x] += shl[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const long long cnt = shl[0];
    const float qnan = __builtin_nanf("");
    diag[0] = cnt ? (float)(d3 / (double)cnt) : qnan;
    diag[1] = cnt ? (float)(kl / (double)cnt) : qnan;
  }
}

// ===================================================================
// Run-level diagnostics ([P2] section 4 "What happens without alignment":
// the largest gradient norm; [P2] section 3, Figure 1: D3 per update).
// ===================================================================
// Sum over a 1024-thread block in a fixed order: an xor tree inside each
// wave (every lane ends with the same bits), then the 16 wave sums in
// ascending wave order.  sh holds 16 doubles.
template <typename T>
__device__ __forceinline__ T block1024_sum(T x, T* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  T r = sh[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) r += sh[w];
  __syncthreads();
  return r;
}

// Gradient norms: sums of squares in float64 over fixed chunks of
// kNormChunk values (thread t takes 16-byte groups t, t + 256, ... of its
// chunk in order, then a 256-wide fixed tree), then one fixed tree over the
// chunks.
constexpr int kNormChunk = 65536;
constexpr int kNormBatch = 8;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(256) void k_sumsq_partial(const float* __restrict__ x,
                                                       int64_t n, double* out) {
  __shared__ double shd[256];
  const int64_t base = (int64_t)blockIdx.x * kNormChunk;
  double acc = 0.0;
  if (base + kNormChunk <= n) {  // whole chunk (x is 16-byte aligned)
    const f32x4* p = reinterpret_cast<const f32x4*>(x + base) + threadIdx.x;
    for (int i = 0; i < kNormChunk / 1024; i += kNormBatch) {
      f32x4 v[kNormBatch];
#pragma unroll
      for (int j = 0; j < kNormBatch; ++j) v[j] = __builtin_nontemporal_load(p + (i + j) * 256);
#pragma unroll
      for (int j = 0; j < kNormBatch; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc += (double)v[j][k] * (double)v[j][k];
    }
  } else {  // the tail chunk: same order, element-guarded
    for (int i = 0; i < kNormChunk / 1024; ++i) {
      const int64_t t = base + 4 * ((int64_t)i * 256 + threadIdx.x);
      for (int k = 0; k < 4; ++k)
        if (t + k < n) acc += (double)x[t + k] * (double)x[t + k];
    }
  }
  acc = block_sum_d(acc, shd);
  if (threadIdx.x == 0) out[blockIdx.x] = acc;
}

__global__ __launch_bounds__(1024) void k_sumsq_final(const double* in, int nchunk,
                                                      float* norm) {
  __shared__ double shd[16];
  double acc = 0.0;
  for (int i = threadIdx.x; i < nchunk; i += 1024) acc += in[i];
  acc = block1024_sum(acc, shd);
  if (threadIdx.x == 0) *norm = (float)sqrt(acc);
}

// Per-response D3 and KL: one 1024-thread workgroup per response; thread t
// takes rows r0 + t, r0 + t + 1024, ... in order (float64; rows are loaded
// kRespBatch at a time), then block1024_sum.  The order is fixed relative to
// the response's first row, so a response's values do not depend on where it
// sits in the batch.  NaN for a response without valid rows or with a bad
// cu_rows range.
constexpr int kRespBatch = 8;

__global__ __launch_bounds__(1024) void k_resp_diag(
    const float* __restrict__ logpi, const float* __restrict__ logmu,
    const uint8_t* __restrict__ mask, const int* __restrict__ cu, int B,
    int64_t n, float* d3_out, float* kl_out, int* err) {
  __shared__ double shd[16];
  __shared__ int shc[16];
  const int i = blockIdx.x;
  const int64_t r0 = cu[i], r1 = cu[i + 1];
  const bool bad = r0 < 0 || r1 < r0 || r1 > n || (i == 0 && r0 != 0) ||
                   (i == B - 1 && r1 != n);
  double d3 = 0.0, kl = 0.0;
  int c = 0;
  if (!bad) {
    for (int64_t t0 = r0 + threadIdx.x; t0 < r1; t0 += 1024 * kRespBatch) {
      float a[kRespBatch], m[kRespBatch];
      bool v[kRespBatch];
#pragma unroll
      for (int j = 0; j < kRespBatch; ++j) {
        const int64_t t = t0 + (int64_t)j * 1024;
        v[j] = t < r1;
        a[j] = v[j] ? logpi[t] : 0.f;
        m[j] = v[j] ? logmu[t] : 0.f;
        if (v[j] && mask) v[j] = mask[t] != 0;
      }
#pragma unroll
      for (int j = 0; j < kRespBatch; ++j)
        if (v[j]) {
          const double d = (double)a[j] - (double)m[j];
          d3 += expm1(d) - d;
          kl += -d;
          ++c;
        }
    }
  }
  d3 = block1024_sum(d3, shd);
  kl = block1024_sum(kl, shd);
  c = block1024_sum(c, shc);
  if (threadIdx.x == 0) {
    const float qnan = __builtin_nanf("");
    d3_out[i] = (!bad && c) ? (float)(d3 / c) : qnan;
    kl_out[i] = (!bad && c) ? (float)(kl / c) : qnan;
    if (bad && err) atomicOr(err, 4);
  }
}

// ===================================================================
// MX-format head -> bfloat16 ("Zero mismatch, simple async RL", vLLM blog:
// the aligned path keeps release precision, FP8 and MXFP4 weights included).
// Encodings of the OCP Microscaling Formats v1.0: E2M1 and E4M3 elements,
// one E8M0 scale 2^(code - 127) per 32 consecutive values along H.  The
// scale range checked per block makes every value of a valid block exactly a
// bf16 number (normal or subnormal), so nothing is rounded.
// ===================================================================
// Valid blocks go through the scaled conversions of rz_gemm.h
// (fp4x8_to_bf16 / fp8x8_to_bf16).

// A wave expands 64 consecutive blocks (4 KB of bf16) with every load and
// store instruction covering one contiguous span: in step j = 0..3, lane l
// takes the 8 values 8 (l % 4) .. + 7 of block 16 j + l / 4, reading their
// 4 (E2M1) or 8 (E4M3) code bytes and writing 16 bytes at 1 KB j + 16 l.
template <int kFmt>  // 0: E2M1 (two codes per byte), 1: E4M3
__global__ __launch_bounds__(256) void k_mx_dequant(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales,
                                                    int64_t nblk, uint32_t* __restrict__ out,
                                                    int* err) {
  const int lane = threadIdx.x & 63;
  const int64_t wbase = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t b = wbase + 16 * j + (lane >> 2);
    if (b >= nblk) break;
    const int part = lane & 3;  // values 8 part .. 8 part + 7 of block b
    const int sc = scales[b];
    const bool ok = mx_scale_ok(kFmt, sc);
    uint32_t w[4];  // 8 bf16 values, value 2i in the low half of w[i]
    u32x4 v;
    if constexpr (kFmt == 0)
      v = fp4x8_to_bf16(*reinterpret_cast<const uint32_t*>(codes + b * 16 + 4 * part),
                        e8m0_scale(sc));
    else
      v = fp8x8_to_bf16(*reinterpret_cast<const u32x2*>(codes + b * 32 + 8 * part),
                        e8m0_scale(sc));
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = v[i];
    if (!ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = 0x7FC07FC0u;
      bad = true;
    }
    *reinterpret_cast<u32x4*>(out + b * 16 + 4 * part) = u32x4{w[0], w[1], w[2], w[3]};
  }
  if (bad && err) atomicOr(err, 8);
}

// ===================================================================
// LoRA adapter on the head ("Zero mismatch, simple async RL", vLLM blog,
// Kimi K3.1 section: zero mismatch with LoRA adapters on every module).
// z = h W^T + u B^T with u = s h A^T rounded to the head's precision, i.e.
// the plain head over [h | u] and [W | B]: the adapter runs on the path's
// own kernels, so the rollout and the learner agree bit for bit.  The
// augmented width is H + kLoraPad; columns of u past the rank r hold 0.
// ===================================================================
constexpr int kLoraPad = 64;     // the largest rank, and the u block width
static_assert(kLoraPad == kLoraCols, "one LoRA width for kernels and ABI");
constexpr int kLoraChunk = 4096; // rows per dL/dA partial sum

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);  // finite x
}
__device__ __forceinline__ void store_val(bf16* p, float x) {
  *reinterpret_cast<uint16_t*>(p) = bf16_rne(x);
}
__device__ __forceinline__ void store_val(float* p, float x) { *p = x; }

struct LoraUArgs {
  GemmOperands op;  // A = hidden rows, B = lora_A rows (N = r)
  int n, nk, H, r;
  int64_t ld_aug;   // row stride of the augmented hidden (values)
  float scale;
  void* out;        // augmented hidden [n, H + kLoraPad]
};

// u = s (h A^T) for one 256-row tile on the tile engine (fixed K order: a
// row's u does not depend on the batch), written as columns H .. H + 63.
template <typename T>
__global__ RZ_GEMM_ATTR void k_lora_u(LoraUArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int m0 = blockIdx.x * kBM;
  f32x16 acc[2][kTN];
  gemm_mainloop<T, false>(a.op, a.n, m0, 0, a.nk, acc, lds);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wrow = (wid & 3) * 64, wcol = (wid >> 2) * 128;
  T* out = reinterpret_cast<T*>(a.out);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni) {
      const int j = acc_col(wcol, ni, lane);
      if (j >= kLoraPad) continue;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = m0 + acc_row(wrow, mi, rr, lane);
        if (row < a.n)
          store_val(out + (int64_t)row * a.ld_aug + a.H + j,
                    j < a.r ? a.scale * acc[mi][ni][rr] : 0.f);
      }
    }
}

// dst[row, col0 + j] = j < nsrc ? src[row, j] : 0 for j < kLoraPad
template <typename T>
__global__ __launch_bounds__(64) void k_lora_cols(T* __restrict__ dst, int64_t ld,
                                                  int col0, const T* __restrict__ src,
                                                  int64_t ld_src, int nsrc) {
  const int64_t row = blockIdx.x;
  const int j = threadIdx.x;
  dst[row * ld + col0 + j] = j < nsrc ? src[row * ld_src + j] : T(0.f);
}

// Marks the values as used, in one empty asm: every load that produces them
// must be complete before it, and none can be moved under a later select's
// condition.  A fill's loads all go before it, so they are in flight
// together instead of one round trip each.
__device__ __forceinline__ void pin8(float* v) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]),
               "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}
__device__ __forceinline__ void pin16(float* v) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]),
               "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]),
               "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]),
               "+v"(v[12]), "+v"(v[13]), "+v"(v[14]), "+v"(v[15]));
}

// Eight consecutive values of a row of T as floats (16-byte loads; p is
// 16-byte aligned).
__device__ __forceinline__ void load8_f(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[k] = a[k];
    v[4 + k] = b[k];
  }
}
__device__ __forceinline__ void load8_f(const bf16* p, float (&v)[8]) {
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = (float)a[k];
}

// dL/dh = dL/dh_aug[:, :H] + s (dL/du) A with dL/du = dL/dh_aug[:, H:]:
// 64 rows per workgroup, A staged 256 columns at a time; each thread holds
// an 8 x 8 block of outputs (rows 8 (tid / 32) .., columns 8 (tid % 32) ..)
// in registers, fed per rank index by two 16-byte LDS reads of dL/du and
// two of A.  Every output's sum over the rank runs in ascending order.
template <typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_lora_dh(const float* __restrict__ dh_aug, int64_t ld_aug, int H,
               const T* __restrict__ A, int r, float scale, int64_t n,
               float* __restrict__ d_hidden) {
  // 80 KB of LDS and at most 256 VGPRs: two workgroups per CU
  __shared__ __attribute__((aligned(16))) float duT[kLoraPad][64];     // [j][row]
  __shared__ __attribute__((aligned(16))) float ab[kLoraPad][256];     // [j][column]
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
  // All loads of a fill first, from clamped (in-bounds) addresses; then
  // pin16 (else the compiler moves each load under its select's condition,
  // a round trip of its own); then the selects.
  {
    constexpr int kN = 64 * kLoraPad / 256;
    float v[kN];
#pragma unroll
    for (int k = 0; k < kN; ++k) {
      const int i = tid + 256 * k;
      const int t = i / kLoraPad, j = i % kLoraPad;
      const int64_t row = r0 + t < n ? r0 + t : n - 1;
      v[k] = dh_aug[row * ld_aug + H + j];
    }
    static_assert(kN == 16, "one pin");
    pin16(v);
#pragma unroll
    for (int k = 0; k < kN; ++k) {
      const int i = tid + 256 * k;
      const int t = i / kLoraPad, j = i % kLoraPad;
      duT[j][t] = (r0 + t < n && j < r) ? v[k] : 0.f;
    }
  }
  const int rg = tid >> 5, cg = tid & 31;
  for (int hb = 0; hb < H; hb += 256) {
    __syncthreads();
    {
      // A[j, hb + 8 c8 .. + 7] for j = tid / 32 + 8 k, c8 = tid % 32: eight
      // 16-byte-aligned runs of eight values per thread, as the fill above
      const int c8 = tid & 31, col = hb + 8 * c8;
      const int cc = col < H ? col : H - 8;  // H % 64 == 0
      float v[8][8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = (tid >> 5) + 8 * k;
        load8_f(A + (int64_t)(j < r ? j : r - 1) * H + cc, v[k]);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) pin8(v[k]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = (tid >> 5) + 8 * k;
        const bool ok = j < r && col < H;
        *reinterpret_cast<f32x4*>(&ab[j][8 * c8]) =
            ok ? f32x4{v[k][0], v[k][1], v[k][2], v[k][3]} : f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(&ab[j][8 * c8 + 4]) =
            ok ? f32x4{v[k][4], v[k][5], v[k][6], v[k][7]} : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    __syncthreads();
    const int h = hb + cg * 8;
    if (h >= H) continue;  // H % 64 == 0: eight columns are all in or all out
    float acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[a][c] = 0.f;
    for (int j = 0; j < kLoraPad; ++j) {
      float d[8], w[8];
      load8_f(&duT[j][rg * 8], d);
      load8_f(&ab[j][cg * 8], w);
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[a][c] = fmaf(d[a], w[c], acc[a][c]);
    }
    float x[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int64_t row = r0 + rg * 8 + a < n ? r0 + rg * 8 + a : n - 1;
      load8_f(dh_aug + row * ld_aug + h, x[a]);
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int64_t row = r0 + rg * 8 + a;
      if (row >= n) continue;
      float* o = d_hidden + row * H + h;
      *reinterpret_cast<f32x4*>(o) =
          f32x4{x[a][0] + scale * acc[a][0], x[a][1] + scale * acc[a][1],
                x[a][2] + scale * acc[a][2], x[a][3] + scale * acc[a][3]};
      *reinterpret_cast<f32x4*>(o + 4) =
          f32x4{x[a][4] + scale * acc[a][4], x[a][5] + scale * acc[a][5],
                x[a][6] + scale * acc[a][6], x[a][7] + scale * acc[a][7]};
    }
  }
}

// dL/dA partials: part[c][j][h] = sum over the rows of chunk c (ascending)
// of (dL/du)[t, j] h[t, h].  A workgroup takes one chunk and 256 columns;
// 64 rows of dL/du and of h are staged in LDS at a time (h as floats, by
// 16-byte loads) and each thread holds an 8 x 8 block of (j, h) sums.
template <typename T>
__global__ __launch_bounds__(256) void k_lora_da_partial(
    const float* __restrict__ dh_aug, int64_t ld_aug, int H,
    const T* __restrict__ hidden, int64_t n, int r, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float du[64][kLoraPad];  // [row][j]
  __shared__ __attribute__((aligned(16))) float hs[64][256];       // [row][column]
  constexpr int kV = 8;                                            // values per load
  const int c = blockIdx.x;
  const int hb = blockIdx.y * 256;
  const int tid = threadIdx.x;
  const int jg = tid >> 5, cg = tid & 31;
  const int64_t t_begin = (int64_t)c * kLoraChunk;
  const int64_t t_end = t_begin + kLoraChunk < n ? t_begin + kLoraChunk : n;
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.f;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 64) {
    __syncthreads();
    // all loads first, from clamped addresses, then the selects (see the
    // fills of k_lora_dh)
    constexpr int kND = 64 * kLoraPad / 256, kNH = 64 * (256 / kV) / 256;
    float vd[kND], vh[kNH][8];
#pragma unroll
    for (int k = 0; k < kND; ++k) {
      const int i = tid + 256 * k;
      const int t = i / kLoraPad, j = i % kLoraPad;
      const int64_t row = t0 + t < t_end ? t0 + t : t_end - 1;
      vd[k] = dh_aug[row * ld_aug + H + j];
    }
#pragma unroll
    for (int k = 0; k < kNH; ++k) {
      const int i = tid + 256 * k;
      const int t = i / (256 / kV), col = (i % (256 / kV)) * kV;
      const int64_t row = t0 + t < t_end ? t0 + t : t_end - 1;
      const int cc = hb + col < H ? hb + col : H - kV;
      load8_f(hidden + row * H + cc, vh[k]);
    }
    static_assert(kND == 16 && kNH == 8, "the pins below");
    pin16(vd);
#pragma unroll
    for (int k = 0; k < kNH; ++k) pin8(vh[k]);
#pragma unroll
    for (int k = 0; k < kND; ++k) {
      const int i = tid + 256 * k;
      const int t = i / kLoraPad, j = i % kLoraPad;
      du[t][j] = (t0 + t < t_end && j < r) ? vd[k] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kNH; ++k) {
      const int i = tid + 256 * k;
      const int t = i / (256 / kV), col = (i % (256 / kV)) * kV;
      // H % 64 == 0: eight columns are all in or all out
      const bool ok = t0 + t < t_end && hb + col < H;
      const float* v = vh[k];
      *reinterpret_cast<f32x4*>(&hs[t][col]) =
          ok ? f32x4{v[0], v[1], v[2], v[3]} : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(&hs[t][col + 4]) =
          ok ? f32x4{v[4], v[5], v[6], v[7]} : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    const int nt = t_end - t0 < 64 ? (int)(t_end - t0) : 64;
    for (int t = 0; t < nt; ++t) {
      float d[8], w[8];
      load8_f(&du[t][jg * 8], d);
      load8_f(&hs[t][cg * 8], w);
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = fmaf(d[a], w[b], acc[a][b]);
    }
  }
  const int h = hb + cg * 8;
  if (h < H)
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int j = jg * 8 + a;
      if (j >= r) continue;
      float* o = part + ((int64_t)c * r + j) * H + h;
      *reinterpret_cast<f32x4*>(o) = f32x4{acc[a][0], acc[a][1], acc[a][2], acc[a][3]};
      *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[a][4], acc[a][5], acc[a][6], acc[a][7]};
    }
}

// dL/dA = s * sum of the partials in ascending chunk order
__global__ __launch_bounds__(256) void k_lora_da_final(const float* __restrict__ part,
                                                       int nchunk, int r, int H,
                                                       float scale, float* __restrict__ dA) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)r * H) return;
  float acc = 0.f;
  for (int c = 0; c < nchunk; ++c) acc += part[(int64_t)c * r * H + i];
  dA[i] = scale * acc;
}

// ===================================================================
// Transposes feeding the backward GEMMs their K-contiguous operands:
// out[c, r] = in[row(r), c] for r < rows, and 0 for rows <= r < the row
// count rounded up to 64 (the last K stage a GEMM reads; never past
// rows_pad).
// ===================================================================
// Each lane moves a kVec x kVec block (kVec = values per 16 bytes): kVec
// 16-byte row pieces in, a transpose in registers, kVec 16-byte column
// pieces out.  Eight lanes (bf16) cover one 128-byte line on either side.
// rows_pad and cols are multiples of 64.
//
// Row scale (bf16 only, rs_c non-null): row r is multiplied by
// c_r g_r 2^sigma (k_coef, k_chunk_scale) and rounded to bf16 once: the dW
// GEMM's B operand then carries the row's whole softmax factor.
template <typename T, bool kScale = false>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ in,
                                                   int64_t ld_in,
                                                   const int* rowmap,
                                                   DevRows rows, int rows_pad,
                                                   int cols, T* __restrict__ out,
                                                   int64_t ld_out,
                                                   const float* rs_c,
                                                   const float* rs_g,
                                                   const int* rs_sigma) {
  constexpr int kVec = 16 / (int)sizeof(T);       // 8 (bf16) or 4 (fp32)
  constexpr int kG = 64 / kVec;                   // row blocks per wave
  constexpr int kWaveCols = (64 / kG) * kVec;     // 64 (bf16) or 16 (fp32)
  const RowCount rc = to_rc(rows);
  const int R = rc.get();
  const int r0 = blockIdx.x * 64;
  if (r0 >= rows_pad || r0 >= ((R + 63) & ~63)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int cw = blockIdx.y * (4 * kWaveCols) + wid * kWaveCols;
  if (cw >= cols) return;
  const int tr = (lane % kG) * kVec;          // first row of the block
  const int col = cw + (lane / kG) * kVec;    // first column
  u32x4 x[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const int r = r0 + tr + i;
    x[i] = u32x4{0u, 0u, 0u, 0u};
    if (r < R) {
      const int64_t pr = rowmap ? (int64_t)rowmap[rc.base + r] : rc.base + r;
      x[i] = *reinterpret_cast<const u32x4*>(in + pr * ld_in + col);
    }
  }
  if constexpr (kScale) {
    // rows past R hold 0 and stay 0 (their scale is read from row R - 1)
    const int sg = *rs_sigma;
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      const int64_t p = rc.base + min(r0 + tr + i, R - 1);
      const float f = (float)ldexp((double)rs_c[p] * (double)rs_g[p], sg);
#pragma unroll
      for (int w = 0; w < 4; ++w) x[i][w] = scale_bf16x2(x[i][w], f);
    }
  }
  if constexpr (sizeof(T) == 2) {
    // column q: the q-th 16-bit value of the 8 row pieces
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int sh = (q & 1) * 16;
      uint32_t o[4];
#pragma unroll
      for (int w = 0; w < 4; ++w)
        o[w] = ((x[2 * w][q >> 1] >> sh) & 0xffffu) |
               (((x[2 * w + 1][q >> 1] >> sh) & 0xffffu) << 16);
      *reinterpret_cast<u32x4*>(out + (int64_t)(col + q) * ld_out + r0 + tr) =
          u32x4{o[0], o[1], o[2], o[3]};
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(out + (int64_t)(col + q) * ld_out + r0 + tr) =
          u32x4{x[0][q], x[1][q], x[2][q], x[3][q]};
  }
}

// ===================================================================
// Backward, part 1: dlogits.
//
// fp32 inputs: the forward stored e[t, v] = exp(z[t, v] - m_j) in the dz
// buffer, m_j the maximum of the statistics tile j holding v; with lse_t
// known, dz[t, v] = c_t exp(m_j - lse_t) e[t, v] is dL/dz for v != a_t; the
// token's own column is left at 0 and its whole dL/dz, c_t (p[a_t] - 1), is
// applied exactly in fp32 by the dHidden epilogue and the dW fix-up.
// k_dz_scale rescales e in place into the token-major dz [C, Vpad], the A
// operand of dHidden, and also writes the vocab-major dz^T [Vpad, C] for
// dW (fp32 has no transposing LDS read).  Rows from the chunk's count up to
// the next multiple of 64 (the last K stage of dW) become zero columns of
// dz^T.  Each lane owns a 4 x 4 block: four 16-byte row pieces in and back
// rescaled, a transpose in registers, four 16-byte column pieces of dz^T out.
//
// bf16 inputs need no pass here: the stored e is already the A operand
// (see EStore), and the factor c_t exp(r*_t ln 2 - lse_t) rides on the other
// side of each GEMM.  Only the rows whose tiles straddle the e window are
// rebased (k_erebase).
// ===================================================================
__global__ __launch_bounds__(256) void k_dz_scale(
    float* __restrict__ dz, int64_t ldz, float* __restrict__ dzT, int64_t ldzt,
    DevRows rows, const float2* __restrict__ partials, int64_t ldp,
    const float* __restrict__ lse, const float* __restrict__ coef,
    const int* __restrict__ tokv, int Vpad) {
  __shared__ float sc[64];
  __shared__ int stok[64];  // the rows' tokens: their column is left at 0
  const RowCount rc = to_rc(rows);
  const int R = rc.get();
  const int r0 = blockIdx.y * 64;
  if (r0 >= ((R + 63) & ~63)) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int tr = (lane % 16) * 4;  // first row of the block
  // one scale per row: c_t exp(m_j - lse_t), j the statistics tile (128
  // columns) holding the workgroup's 64 columns
  if (tid < 64) {
    const int t = r0 + tid;
    const int j = (blockIdx.x * 64) / 128;
    float v = 0.f;
    if (t < R) {
      const int64_t pos = rc.base + t;
      v = coef[pos] * exp_approx(partials[(int64_t)j * ldp + pos].x - lse[pos]);
    }
    sc[tid] = v;
    stok[tid] = t < R ? tokv[rc.base + t] : -1;
  }
  __syncthreads();
  const int cw = blockIdx.x * 64 + wid * 16;
  if (cw >= Vpad) return;
  const int col = cw + (lane / 16) * 4;
  f32x4 y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = r0 + tr + i;
    if (t < R) {
      float* p = dz + (int64_t)t * ldz + col;
      y[i] = sc[tr + i] * *reinterpret_cast<const f32x4*>(p);
      const uint32_t own = (uint32_t)(stok[tr + i] - col);  // stays 0
#pragma unroll
      for (int w = 0; w < 4; ++w) y[i][w] = own == (uint32_t)w ? 0.f : y[i][w];
      *reinterpret_cast<f32x4*>(p) = y[i];
    } else {
      y[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<f32x4*>(dzT + (int64_t)(col + q) * ldzt + r0 + tr) =
        f32x4{y[0][q], y[1][q], y[2][q], y[3][q]};
}

// bf16 rows whose statistics tiles were stored against different e references
// (k_lse_merge's flag): each tile j with r_j != r*_t is multiplied by
// 2^(r_j - r*_t) <= 1, an exact power of two, so those tiles share the row's
// reference without a second rounding.  One wave per row; the other rows
// return at once.
__global__ __launch_bounds__(256) void k_erebase(
    bf16* __restrict__ e, int64_t lde, DevRows rows,
    const float2* __restrict__ partials, int64_t ldp, int nt,
    const float* __restrict__ eref, const int* __restrict__ eflag, int Vpad) {
  const RowCount rc = to_rc(rows);
  const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= rc.get()) return;
  const int64_t pos = rc.base + p;
  if (!eflag[pos]) return;  // uniform per wave
  const float rs = eref[pos];
  const int lane = threadIdx.x & 63;
  bf16* row = e + (int64_t)p * lde;
  for (int j = 0; j < nt; ++j) {  // statistics tiles of 128 columns
    const float d = e_ref2(partials[(int64_t)j * ldp + pos].x) - rs;
    if (d == 0.f) continue;  // uniform per wave
    const int c = j * 128 + lane * 2;
    if (c >= Vpad) continue;
    // d <= 0 (e_ref2 is monotone and r* is the row maximum's); far below,
    // the products flush to 0 (their terms are below 2^-1000 of the row's)
    const int k = d < -1000.f || d != d ? -1000 : (int)d;
    uint32_t* q = reinterpret_cast<uint32_t*>(row + c);
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = __builtin_bit_cast(bf16x2, *q);
#pragma unroll
    for (int i = 0; i < 2; ++i) v[i] = (bf16)ldexpf((float)v[i], k);
    *q = __builtin_bit_cast(uint32_t, v);
  }
}

// ===================================================================
// The last round of a GEMM's tiles split along K.  One workgroup per CU per
// round: when the tiles of the last round leave most CUs idle, each of them
// runs as up to kSplitMax pieces over consecutive K ranges, parked as raw
// accumulators and summed in piece order by a second kernel (a fixed order,
// so the result is the same in every run).  The split depends on the tile
// count and the CU count only.
// ===================================================================
constexpr int kPartTileFloats = kBM * kBN;  // one parked 256 x 256 fp32 tile
constexpr int kSplitMax = 4;                // pieces per tile of the last round
constexpr int kSplitWGs = 256;              // parked tiles at most

struct RoundSplit {
  int tail, split;  // tail: tiles T - tail .. T - 1 run as split pieces each
};
__host__ __device__ inline RoundSplit round_split(int T, int ncu) {
  RoundSplit r{0, 1};
  if (T <= 0 || ncu < 1) return r;
  const int tail = T - ((T + ncu - 1) / ncu - 1) * ncu;
  int split = ncu / tail;
  if (split > kSplitMax) split = kSplitMax;
  if (tail * split > kSplitWGs) split = kSplitWGs / tail;
  if (split >= 2) r = RoundSplit{tail, split};
  return r;
}

// Parked tile q (the eight-wave tile, 512 threads): 16-byte chunk c of
// thread t at part + q kPartTileFloats + 4 (512 c + t), chunk c holding
// registers 4 (c % 4) .. + 3 of block (c / 16, (c / 4) % 4).
__device__ __forceinline__ f32x4* part_chunk(float* part, int q, int c) {
  return reinterpret_cast<f32x4*>(part + (int64_t)q * kPartTileFloats) +
         c * (2 * kThreads) + threadIdx.x;
}

__device__ __forceinline__ void park_tile(float* part, int q,
                                          const f32x16 (&acc)[2][kTN]) {
#pragma unroll
  for (int c = 0; c < 4 * 2 * kTN; ++c) {
    const f32x16& blk = acc[c / 16][(c / 4) % 4];
    const int r = 4 * (c % 4);
    *part_chunk(part, q, c) = f32x4{blk[r], blk[r + 1], blk[r + 2], blk[r + 3]};
  }
}

// the pieces q0 .. q0 + n - 1 summed in order (only the accumulators of
// block row mi_only when it is >= 0)
__device__ __forceinline__ void sum_parked(float* part, int q0, int n,
                                           f32x16 (&acc)[2][kTN],
                                           int mi_only = -1) {
#pragma unroll
  for (int c = 0; c < 4 * 2 * kTN; ++c) {
    if (mi_only >= 0 && c / 16 != mi_only) continue;
    f32x4 v = *part_chunk(part, q0, c);
    for (int p = 1; p < n; ++p) v += *part_chunk(part, q0 + p, c);
    f32x16& blk = acc[c / 16][(c / 4) % 4];
    const int r = 4 * (c % 4);
    blk[r] = v[0];
    blk[r + 1] = v[1];
    blk[r + 2] = v[2];
    blk[r + 3] = v[3];
  }
}

// ===================================================================
// Backward, part 2: dHidden = dz W (K = Vpad in fixed order) plus the token
// column's exact term c_t (p[a_t] - 1) W[a_t, :] (coef holds its
// negative), scattered to the rows' positions.  bf16: the A operand is the
// stored e, and the row's factor is applied here in fp32 as
// c_t (g_t acc) (two products, so that neither factor's range limits the
// other's).
// ===================================================================
template <typename T>
struct DhArgs {
  GemmOperands op;
  DevRows rows;
  const int* idx;
  const int* tokv;
  const float* coef;   // the token column's term (negated)
  const float* rc;     // bf16: c_t; fp32: nullptr (dz is already scaled)
  const float* rg;     // bf16: g_t
  const T* W;
  int H, V, nk, mt, nt;
  int ncu;      // compute units: the last round's split (round_split)
  float* part;  // parked pieces of the last round (null: no split)
  float* dh;
};

// The epilogue of one dHidden tile (eight waves, see gemm_mainloop): the
// rows' factors (bf16), the token column's exact term, the scatter to the
// rows' positions.
template <typename T>
__device__ __forceinline__ void dh_epilogue(const DhArgs<T>& a, const RowCount& rc,
                                            int M, int m0, int n0,
                                            f32x16 (&acc)[2][kTN], char* lds,
                                            int mi_only = -1) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wrow = (wid & 3) * 64, wcol = (wid >> 2) * 128;
  int* sidx = reinterpret_cast<int*>(lds);
  int* stok = sidx + 256;
  float* scoef = reinterpret_cast<float*>(stok + 256);
  float* src = scoef + 256;
  float* srg = src + 256;
  constexpr bool kScaled = sizeof(T) == 2;  // bf16: A was the stored e
  if (tid < kBM) {  // one tile row per thread of waves 0 .. 3
    const int m = m0 + tid;
    const int64_t p = rc.base + m;
    sidx[tid] = m < M ? a.idx[p] : 0;
    int tk = m < M ? a.tokv[p] : 0;
    stok[tid] = (tk >= 0 && tk < a.V) ? tk : 0;
    scoef[tid] = m < M ? a.coef[p] : 0.f;
    if constexpr (kScaled) {
      src[tid] = m < M ? a.rc[p] : 0.f;
      srg[tid] = m < M ? a.rg[p] : 0.f;
    }
  }
  __syncthreads();
  if constexpr (kScaled) {
    // the rows' factors in place, one row's pair of scales at a time
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (mi_only >= 0 && mi != mi_only) continue;
        const int row = acc_row(wrow, mi, r, lane);
        const float c = src[row], g = srg[row];
#pragma unroll
        for (int ni = 0; ni < kTN; ++ni) acc[mi][ni][r] = c * (g * acc[mi][ni][r]);
        __builtin_amdgcn_sched_barrier(0);
      }
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni) {
      if (mi_only >= 0 && mi != mi_only) continue;
      const int h = n0 + acc_col(wcol, ni, lane);
      if (h >= a.H) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(wrow, mi, r, lane);
        if (m0 + row < M) {
          const float w = load_f(a.W + (int64_t)stok[row] * a.H + h);
          a.dh[(int64_t)sidx[row] * a.H + h] = acc[mi][ni][r] - scoef[row] * w;
        }
      }
    }
}

// kPiece = false: the tiles of the M rows present (M may be a device count
// below the launch bound; only those tiles are numbered, so they spread over
// all XCDs), except the last round's when it is split (round_split of that
// tile count); kPiece = true: those tiles' K pieces, parked for k_dh_tail.
// Workgroups past their share return at once.  The split's whole rounds
// come first, so running the pieces as a second launch costs one launch.
template <typename T, bool kPiece>
__global__ RZ_GEMM_ATTR void k_bwd_dh(DhArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const RowCount rc = to_rc(a.rows);
  const int M = rc.get();
  const int mt = (M + kBM - 1) / kBM;
  const int ntile = mt * a.nt;
  const RoundSplit sp = a.part ? round_split(ntile, a.ncu) : RoundSplit{0, 1};
  const int full = ntile - sp.tail;
  int tb = blockIdx.x, piece = 0, pieces = 1;
  if constexpr (kPiece) {
    if (tb >= sp.tail * sp.split) return;
    piece = tb % sp.split;
    tb = full + tb / sp.split;
    pieces = sp.split;
  } else {
    if (tb >= full) return;
  }
  const TileCoord tc = map_tile(tb, ntile, mt, a.nt);
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
  // the piece's K stages [k0, k1); both operands are K-contiguous
  const int k0 = (int)((int64_t)a.nk * piece / pieces);
  const int k1 = (int)((int64_t)a.nk * (piece + 1) / pieces);
  GemmOperands op = a.op;
  const int64_t kb = (int64_t)k0 * Stage<T>::kK * (int64_t)sizeof(T);
  op.A += kb;
  op.B += kb;

  f32x16 acc[2][kTN];
  gemm_mainloop<T, false>(op, M, m0, n0, k1 - k0, acc, lds);
  // piece q = (tile - full) split + piece is parked at q, the launch index
  if constexpr (kPiece) park_tile(a.part, blockIdx.x, acc);
  else dh_epilogue(a, rc, M, m0, n0, acc, lds);
}

// The last round's tiles: their pieces summed in piece order, then the same
// epilogue.  Two workgroups of 512 threads per tail tile (kSplitWGs tiles at
// most), one per block row mi of every wave.
template <typename T>
__global__ __launch_bounds__(512) void k_dh_tail(DhArgs<T> a) {
  __shared__ __attribute__((aligned(16))) char lds[5 * 256 * 4];
  const RowCount rc = to_rc(a.rows);
  const int M = rc.get();
  const int mt = (M + kBM - 1) / kBM;
  const int ntile = mt * a.nt;
  const RoundSplit sp = round_split(ntile, a.ncu);
  const int i = blockIdx.x / 2, mi = blockIdx.x % 2;
  if (i >= sp.tail) return;
  const TileCoord tc = map_tile(ntile - sp.tail + i, ntile, mt, a.nt);
  f32x16 acc[2][kTN];
  sum_parked(a.part, i * sp.split, sp.split, acc, mi);
  dh_epilogue(a, rc, M, tc.tm * kBM, tc.tn * kBN, acc, lds, mi);
}

// ===================================================================
// Backward, part 3: dW (+)= dz^T h over this chunk's tokens (K in fixed
// order); chunks are accumulated in order, the first one overwrites.  bf16:
// A is the stored e (read K-major) and B is h^T with row t scaled by
// c_t g_t 2^sigma, so the tile holds 2^sigma dW; the store takes 2^-sigma
// back exactly.
// ===================================================================
struct DwArgs {
  GemmOperands op;  // bf16: A = e [K rows][Vpad], K-major; fp32: A = dz^T
  DevRows krows;
  const int* sigma;  // bf16: the chunk's power of two; fp32: nullptr
  int V, H, amax, kstage, mt, nt, first;  // amax: A columns (bf16) / rows
  // The last round of tiles splits K: T = mt nt tiles, of which the tail
  // (those map_tile numbers T - tail .. T - 1) run as split pieces each,
  // parked in part and summed in order by k_dw_tail.  tail = 0: no split.
  int T, tail, split;
  float* part;
  float* dw;
};


// dW (+)= acc for one tile (eight waves, see gemm_mainloop): rows v
// (vocabulary), columns h (hidden); the first chunk overwrites.
__device__ __forceinline__ void dw_store(const DwArgs& a, int m0, int n0,
                                         f32x16 (&acc)[2][kTN],
                                         int mi_only = -1) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wrow = (wid & 3) * 64, wcol = (wid >> 2) * 128;
  const int unscale = a.sigma ? -*a.sigma : 0;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < kTN; ++ni) {
      if (mi_only >= 0 && mi != mi_only) continue;
      // one 32 x 32 block at a time keeps the in-flight loads bounded
      __builtin_amdgcn_sched_barrier(0);
      const int h = n0 + acc_col(wcol, ni, lane);
      if (h >= a.H) continue;
      float prev[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = m0 + acc_row(wrow, mi, r, lane);
        prev[r] = (!a.first && v < a.V) ? a.dw[(int64_t)v * a.H + h] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = m0 + acc_row(wrow, mi, r, lane);
        if (v < a.V)
          a.dw[(int64_t)v * a.H + h] = prev[r] + ldexpf(acc[mi][ni][r], unscale);
      }
    }
}


template <typename T>
__global__ RZ_GEMM_ATTR void k_bwd_dw(DwArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int K = to_rc(a.krows).get();
  const int nk = (K + a.kstage - 1) / a.kstage;
  if (nk == 0 && !a.first) return;
  // workgroups past the first T - tail take piece `piece` of a last-round tile
  const int full = a.T - a.tail;
  int tb = blockIdx.x, piece = 0, pieces = 1;
  if (tb >= full) {
    piece = (tb - full) % a.split;
    tb = full + (tb - full) / a.split;
    pieces = a.split;
  }
  const TileCoord tc = map_tile(tb, a.T, a.mt, a.nt);
  const int m0 = tc.tm * kBM, n0 = tc.tn * kBN;
  // the piece's K stages [k0, k1); the operands start at stage k0
  const int k0 = (int)((int64_t)nk * piece / pieces);
  const int k1 = (int)((int64_t)nk * (piece + 1) / pieces);
  GemmOperands op = a.op;
  const int64_t kr = (int64_t)k0 * a.kstage;  // K rows (tokens) before the piece
  op.A += sizeof(T) == 2 ? kr * op.lda : kr * (int64_t)sizeof(T);
  op.B += kr * (int64_t)sizeof(T);

  f32x16 acc[2][kTN];
  // bf16 reads dz itself through transposing LDS reads; fp32 has no such
  // read and takes the transposed copy dz^T
  gemm_mainloop<T, false, sizeof(T) == 2>(op, a.amax, m0, n0, k1 - k0, acc, lds);
  if (pieces > 1) {
    park_tile(a.part, (tb - full) * pieces + piece, acc);
    return;
  }
  dw_store(a, m0, n0, acc);
}

// The last round's tiles: the pieces summed in piece order (a fixed order,
// so dW stays run-to-run deterministic), then stored like any other tile.
// Two workgroups of 512 threads per last-round tile, one per block row mi
// of every wave: the same sums and stores, spread over twice the CUs.
__global__ __launch_bounds__(512) void k_dw_tail(DwArgs a) {
  const int K = to_rc(a.krows).get();
  const int nk = (K + a.kstage - 1) / a.kstage;
  if (nk == 0 && !a.first) return;
  const int i = blockIdx.x / 2, mi = blockIdx.x % 2;
  const TileCoord tc = map_tile(a.T - a.tail + i, a.T, a.mt, a.nt);
  f32x16 acc[2][kTN];
  sum_parked(a.part, i * a.split, a.split, acc, mi);
  dw_store(a, tc.tm * kBM, tc.tn * kBN, acc, mi);
}

// ===================================================================
// Stable ordering by an integer key (the dW fix-up's tokens, the group ids
// of the advantages): an LSD radix sort over 8-bit digits.  Each pass is a
// per-tile digit histogram, one exclusive scan over (digit, tile) in that
// order, and a scatter in which each tile places its elements in index
// order: ranks among equal digits come from wave ballots, then from the
// waves before, then from the tile's earlier rounds.  Equal keys therefore
// keep their input order (stability), every pass moves each element once,
// and the work does not depend on how the keys are distributed (one key on
// every element costs what distinct keys cost).  All counts are exact
// integers, so the result is the same in every run.
// ===================================================================
constexpr int kSortTile = 2048;  // elements per workgroup per pass (8 rounds)

__device__ __forceinline__ int sort_key_in(const int* keys, int i, int kmax,
                                           bool clamp) {
  const int k = keys[i];
  // keys outside [0, kmax) (bad tokens or group ids) sort last, as kmax
  return clamp ? ((unsigned)k < (unsigned)kmax ? k : kmax) : k;
}

__global__ __launch_bounds__(256) void k_sort_hist(DevRows rows,
                                                   const int* __restrict__ keys,
                                                   int kmax, int clamp,
                                                   int shift, int ntiles,
                                                   int* __restrict__ ghist) {
  __shared__ int hist[256];
  const int tid = threadIdx.x;
  const int n = to_rc(rows).get();
  hist[tid] = 0;
  __syncthreads();
  const int base = blockIdx.x * kSortTile;
#pragma unroll
  for (int r = 0; r < kSortTile / 256; ++r) {
    const int i = base + r * 256 + tid;
    if (i < n) atomicAdd(&hist[(sort_key_in(keys, i, kmax, clamp) >> shift) & 255], 1);
  }
  __syncthreads();
  ghist[(int64_t)tid * ntiles + blockIdx.x] = hist[tid];
}

// Exclusive prefix sum of n counts by one 1024-thread workgroup: each
// thread sums a contiguous slice, a Hillis-Steele scan over the slice sums,
// then each thread writes its slice's offsets; offsets[n] = the total.
__global__ __launch_bounds__(1024) void k_scan_excl(const int* counts, int n,
                                                    int* offsets) {
  __shared__ int sh[1024];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += counts[i];
  sh[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int y = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += y;
    __syncthreads();
  }
  int run = sh[tid] - sum;
  for (int i = lo; i < hi; ++i) {
    offsets[i] = run;
    run += counts[i];
  }
  if (tid == 1023) offsets[n] = sh[1023];
}

__global__ __launch_bounds__(256) void k_sort_scatter(
    DevRows rows, const int* __restrict__ keys_in, const int* __restrict__ vals_in,
    int kmax, int clamp, int shift, int ntiles, const int* __restrict__ goff,
    int* __restrict__ keys_out, int* __restrict__ vals_out) {
  __shared__ int run[256];      // next free slot of each digit in this tile
  __shared__ int wcnt[4][256];  // this round's count per wave and digit
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = to_rc(rows).get();
  run[tid] = goff[(int64_t)tid * ntiles + blockIdx.x];
  const uint64_t below = (1ull << lane) - 1ull;  // lanes before this one
  for (int r = 0; r < kSortTile / 256; ++r) {
    const int i = blockIdx.x * kSortTile + r * 256 + tid;
    const bool ok = i < n;
    int key = 0, val = 0;
    if (ok) {
      key = sort_key_in(keys_in, i, kmax, clamp);
      val = vals_in ? vals_in[i] : i;
    }
    const int d = (key >> shift) & 255;
    // lanes of this wave holding the same digit: eight ballots
    uint64_t peers = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) wcnt[w][tid] = 0;
    __syncthreads();
    if (ok && (peers & below) == 0) wcnt[wid][d] = __popcll(peers);
    __syncthreads();
    if (ok) {
      int pos = run[d] + __popcll(peers & below);
      for (int w = 0; w < wid; ++w) pos += wcnt[w][d];
      keys_out[pos] = key;
      vals_out[pos] = val;
    }
    __syncthreads();
    run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

// ===================================================================
// dW token-column fix-up: dW[v, :] -= sum over valid t with a_t = v of
// c_t (1 - p[a_t]) h_t (the exact fp32 term of each row's own token).
// The valid-row positions, ordered by token (stable, so ascending within a
// token), are cut into fixed pieces of kFixPiece entries.  A workgroup sums
// each run of equal tokens in its piece in list order; a run that lies
// wholly inside the piece updates dW at once, a run continuing from the
// previous piece is parked (cont_first), and a run that starts in the piece
// but continues past it is parked too (cont_last).  k_dw_fix_span then adds,
// for each run that crosses pieces, its parked sums in piece order.  Every
// token's row of dW is written by one workgroup, each sum has a fixed order
// that depends only on the sorted list, and no workgroup handles more than
// a piece of rows (plus, for a run crossing pieces, one parked sum per
// piece), however often a token occurs.
// ===================================================================
constexpr int kFixPiece = 256;  // sorted entries per fix-up workgroup
constexpr int kFixBatch = 8;    // row chunks loaded ahead per thread

template <typename T>
__global__ __launch_bounds__(256) void k_dw_fix(
    DevRows rows, const int* __restrict__ skey, const int* __restrict__ sval,
    const int* __restrict__ idx, const float* __restrict__ coef,
    const T* __restrict__ hidden, int64_t ld, int H, int V,
    float* __restrict__ cont_first, float* __restrict__ cont_last,
    float* __restrict__ dw) {
  constexpr int kVec = 16 / (int)sizeof(T);  // values per 16-byte chunk
  __shared__ int sk[kFixPiece];
  __shared__ int srow[kFixPiece];
  __shared__ float sc[kFixPiece];
  const int n = to_rc(rows).get();
  const int k = blockIdx.x;
  const int q0 = k * kFixPiece;
  if (q0 >= n) return;
  const int cnt = min(n - q0, kFixPiece);
  const int tid = threadIdx.x;
  if (tid < cnt) {
    const int p = sval[q0 + tid];
    sk[tid] = skey[q0 + tid];
    srow[tid] = idx[p];
    sc[tid] = coef[p];
  }
  const int prev_key = q0 > 0 ? skey[q0 - 1] : -1;
  const int next_key = q0 + cnt < n ? skey[q0 + cnt] : -1;
  __syncthreads();
  const int nch = H / kVec;
  for (int c = tid; c < nch; c += 256) {
    const int col = c * kVec;
    float acc[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) acc[j] = 0.f;
    int start = 0;
    for (int j0 = 0; j0 < cnt; j0 += kFixBatch) {
      // loads of kFixBatch rows first, with each row's token row of dW (a
      // token's run ends in this piece at most once, and nothing else here
      // writes that row before its run ends), then the ordered accumulation
      u32x4 x[kFixBatch];
      f32x4 y[kFixBatch][kVec / 4];
#pragma unroll
      for (int b = 0; b < kFixBatch; ++b)
        if (j0 + b < cnt) {
          x[b] = *reinterpret_cast<const u32x4*>(hidden + (int64_t)srow[j0 + b] * ld + col);
          const int v = sk[j0 + b];
          const float* o = dw + (int64_t)(v < V ? v : 0) * H + col;
#pragma unroll
          for (int w = 0; w < kVec / 4; ++w) y[b][w] = *reinterpret_cast<const f32x4*>(o + 4 * w);
        }
#pragma unroll
      for (int b = 0; b < kFixBatch; ++b) {
        const int j = j0 + b;
        if (j >= cnt) break;
        const float cf = sc[j];
        if constexpr (sizeof(T) == 2) {
          const u32x4 hi_mask = {0xffff0000u, 0xffff0000u, 0xffff0000u, 0xffff0000u};
          const f32x4 lo = __builtin_bit_cast(f32x4, x[b] << 16);
          const f32x4 hi = __builtin_bit_cast(f32x4, x[b] & hi_mask);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc[2 * w] = fmaf(cf, lo[w], acc[2 * w]);
            acc[2 * w + 1] = fmaf(cf, hi[w], acc[2 * w + 1]);
          }
        } else {
          const f32x4 f = __builtin_bit_cast(f32x4, x[b]);
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[w] = fmaf(cf, f[w], acc[w]);
        }
        const int v = sk[j];
        if (j + 1 < cnt && sk[j + 1] == v) continue;  // the run goes on
        // the run [start, j] of token v ends here (uniform across the block)
        const bool from_prev = start == 0 && prev_key == v;
        const bool into_next = j == cnt - 1 && next_key == v;
        if (v < V) {
          float* dst;
          if (from_prev) dst = cont_first + (int64_t)k * H + col;
          else if (into_next) dst = cont_last + (int64_t)k * H + col;
          else dst = nullptr;
          if (dst) {
#pragma unroll
            for (int w = 0; w < kVec; w += 4)
              *reinterpret_cast<f32x4*>(dst + w) =
                  f32x4{acc[w], acc[w + 1], acc[w + 2], acc[w + 3]};
          } else {
            float* o = dw + (int64_t)v * H + col;
#pragma unroll
            for (int w = 0; w < kVec; w += 4)
              *reinterpret_cast<f32x4*>(o + w) =
                  y[b][w / 4] - f32x4{acc[w], acc[w + 1], acc[w + 2], acc[w + 3]};
          }
        }
#pragma unroll
        for (int w = 0; w < kVec; ++w) acc[w] = 0.f;
        start = j + 1;
      }
    }
  }
}

// Runs crossing pieces: the piece where such a run starts adds its parked
// sums in piece order (its own cont_last, then each following piece's
// cont_first) and subtracts the total from the token's row of dW.
__global__ __launch_bounds__(256) void k_dw_fix_span(
    DevRows rows, const int* __restrict__ skey, int H, int V,
    const float* __restrict__ cont_first, const float* __restrict__ cont_last,
    float* __restrict__ dw) {
  const int n = to_rc(rows).get();
  const int k = blockIdx.x;
  const int q0 = k * kFixPiece;
  if (q0 >= n) return;
  const int q1 = min(n, q0 + kFixPiece);
  const int v = skey[q1 - 1];
  if (v >= V || q1 >= n || skey[q1] != v) return;  // last run ends here
  // the run began in an earlier piece: that piece owns it
  if (q0 > 0 && skey[q0] == v && skey[q0 - 1] == v) return;
  int last = k + 1;  // the last piece the run reaches
  while ((last + 1) * (int64_t)kFixPiece < n && skey[(last + 1) * kFixPiece] == v) ++last;
  for (int c = threadIdx.x; c < H / 4; c += 256) {
    f32x4 s = *reinterpret_cast<const f32x4*>(cont_last + (int64_t)k * H + 4 * c);
    for (int j = k + 1; j <= last; ++j)
      s += *reinterpret_cast<const f32x4*>(cont_first + (int64_t)j * H + 4 * c);
    f32x4* o = reinterpret_cast<f32x4*>(dw + (int64_t)v * H + 4 * c);
    *o = *o - s;
  }
}

// ===================================================================
// launchers
// ===================================================================
namespace {

template <typename F>
hipError_t timed(int kid, hipStream_t s, F&& launch) {
  Timer::before(kid, s);
  launch();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return Timer::after(kid, s);
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// compute units of the current device (256 if the runtime cannot say)
inline int cu_count() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      ncu < 1)
    ncu = 256;
  return ncu;
}

// The workgroups of the single-stage 64-row form (one row block, where each
// CU streams its share of the head): whole rounds of 256-column workgroups
// over the CUs, then the statistics tiles left (128 columns each) as
// 128-column workgroups when there are at most as many as CUs, else as
// 256-column workgroups: at most one more workgroup per CU either way.  For
// a 151936-word head on 256 CUs that is 512 workgroups of 256 columns and
// 163 of 128, so no CU streams more than 640 of the head's columns (594
// tiles of 256 put 768 on some).
struct ColSplit {
  int nfull, nblk;  // 256-column workgroups first, then 128-column ones
};
inline ColSplit split_columns(int V) {
  const int units = cdiv(V, kBN / 2), ncu = cu_count();
  const int nfull = units / (2 * ncu) * ncu;
  const int rest = units - 2 * nfull;
  if (rest > ncu) return {nfull + cdiv(rest, 2), nfull + cdiv(rest, 2)};
  return {nfull, nfull + rest};
}

}  // namespace

const char* kernel_name(int k) {
  static const char* names[K_NUM_KERNELS] = {
      "mask_count",  "mask_scan",   "mask_scatter", "resp_counts",
      "advantages",  "fwd_logits_gemm", "lse_merge", "rows_finalize",
      "coef",        "dz_scale",    "erebase",      "chunk_scale",
      "resp_sums",   "loss_value",
      "diag_partial", "diag_final", "transpose_w",  "transpose_h",
      "bwd_dh_gemm", "bwd_dw_gemm", "sort_hist",    "sort_scan",
      "sort_scatter", "dw_fix",     "dw_fix_span",
      "fwd_sample_gemm", "draw_merge", "grad_norm",
      "grad_norm_final", "resp_diag", "mx_dequant", "lora_u", "lora_cols",
      "lora_dh", "lora_da"};
  return (k >= 0 && k < K_NUM_KERNELS) ? names[k] : "?";
}

hipError_t launch_fwd_sample(int dt, const void* hidden, int64_t n,
                             const void* lm_head, int H, int V,
                             const uint64_t* row_ids, uint64_t seed,
                             float2* partials, float2* cand, float* candz,
                             int64_t ldp, int64_t ldr, hipStream_t s) {
  FwdArgs a{};
  a.op = GemmOperands{(const char*)hidden, (int64_t)H * (dt ? 2 : 4), nullptr,
                      0, (const char*)lm_head, (int64_t)H * (dt ? 2 : 4), V};
  a.rows = DevRows{nullptr, 0, (int)n};
  a.V = V;
  a.Vpad = V;
  a.nk = H / (dt ? Stage<bf16>::kK : Stage<float>::kK);
  const bool small = n <= kRows64MaxSample;
  const bool one = small && n <= kBM64;  // the single-stage 64-row tile
  a.mt = cdiv(n, small ? kBM64 : kBM);
  a.nt = cdiv(V, kBN);
  if (one) {
    const ColSplit cs = split_columns(V);
    a.nfull = cs.nfull;
    a.nt = cs.nblk;
  }
  a.partials = partials;
  a.ldp = ldp;
  a.ldr = ldr;
  a.row_ids = row_ids;
  a.seed = seed;
  a.cand = cand;
  a.candz = candz;
  const int nblk = a.mt * a.nt;
  return timed(K_FWD_SAMPLE, s, [&] {
    if (one) {
      if (dt) k_fwd_logits64_1s<bf16, true><<<nblk, kThreads, 0, s>>>(a);
      else k_fwd_logits64_1s<float, true><<<nblk, kThreads, 0, s>>>(a);
    } else if (small) {
      if (dt) k_fwd_logits64<bf16, true><<<nblk, kThreads, 0, s>>>(a);
      else k_fwd_logits64<float, true><<<nblk, kThreads, 0, s>>>(a);
    } else {
      if (dt) k_fwd_logits<bf16, false, true><<<nblk, 2 * kThreads, 0, s>>>(a);
      else k_fwd_logits<float, false, true><<<nblk, 2 * kThreads, 0, s>>>(a);
    }
  });
}

// The forward of rz_token_logprobs_mx / rz_sample_tokens_mx on the 64-row
// tile (host-known rows, n <= mx_rows64_max(sample), H % 128 == 0): the
// logits GEMM with its statistics and the gather (or the draw).
int mx_rows64_max(int sample) { return sample ? kRows64MaxMxSample : kRows64MaxLogits; }

hipError_t launch_fwd_mx(int fmt, const void* hidden, int64_t n,
                         const uint8_t* codes, const uint8_t* scales, int H,
                         int V, const int* row_tokens, float2* partials,
                         int64_t ldp, int64_t ldr, float* ztgt, const uint64_t* row_ids,
                         uint64_t seed, float2* cand, float* candz, int* err,
                         hipStream_t s) {
  FwdArgs a{};
  a.op = GemmOperands{(const char*)hidden, (int64_t)H * 2, nullptr, 0, nullptr, 0, V};
  a.rows = DevRows{nullptr, 0, (int)n};
  a.V = V;
  a.Vpad = V;
  a.nk = H / Stage<bf16>::kK;
  a.mt = cdiv(n, kBM64);
  a.nt = cdiv(V, kBN);
  a.partials = partials;
  a.ldp = ldp;
  a.ldr = ldr;
  a.row_ids = row_ids;
  a.seed = seed;
  a.cand = cand;
  a.candz = candz;
  a.row_tokens = cand ? nullptr : row_tokens;
  a.ztgt = ztgt;
  a.wcodes = codes;
  a.wscales = scales;
  a.H = H;
  a.err = err;
  const int nblk = a.mt * a.nt;
  return timed(cand ? K_FWD_SAMPLE : K_FWD_LOGITS, s, [&] {
    if (cand) {
      if (fmt == 0) k_fwd_logits64_mx<0, true><<<nblk, kThreads, 0, s>>>(a);
      else k_fwd_logits64_mx<1, true><<<nblk, kThreads, 0, s>>>(a);
    } else {
      if (fmt == 0) k_fwd_logits64_mx<0, false><<<nblk, kThreads, 0, s>>>(a);
      else k_fwd_logits64_mx<1, false><<<nblk, kThreads, 0, s>>>(a);
    }
  });
}

hipError_t launch_draw_merge(const float2* cand, const float* candz,
                             const float2* partials, int64_t ldp, int64_t ldr,
                             int nt, int64_t n, int V, int* tokens, float* logmu,
                             float* lse, hipStream_t s) {
  return timed(K_DRAW_MERGE, s, [&] {
    k_draw_merge<<<cdiv(n, 4), 256, 0, s>>>(cand, candz, partials, ldp, ldr, nt, n, V,
                                            tokens, logmu, lse);
  });
}

hipError_t launch_fwd_logits(int dt, const void* hidden, int64_t lda_bytes,
                             const int* a_rows, DevRows rows,
                             const void* lm_head, int H, int V,
                             const int* row_tokens, float2* partials,
                             int64_t ldp, int64_t ldr, float* ztgt, void* e,
                             int64_t lde, int Vpad, hipStream_t s) {
  FwdArgs a{};
  a.op = GemmOperands{(const char*)hidden, lda_bytes, a_rows, rows.base,
                      (const char*)lm_head, (int64_t)H * (dt ? 2 : 4), V};
  a.rows = rows;
  a.V = V;
  a.Vpad = Vpad;
  a.nk = H / (dt ? Stage<bf16>::kK : Stage<float>::kK);
  // host-known small row counts without the e output take the 64-row tile
  // (same per-row results, a quarter of the MFMA work per W byte)
  const bool small = !rows.count && !e && rows.cap <= kRows64MaxLogits;
  const bool one = small && rows.cap <= kBM64;  // the single-stage 64-row tile
  a.mt = cdiv(rows.cap, small ? kBM64 : kBM);
  a.nt = cdiv(V, kBN);
  if (one) {
    const ColSplit cs = split_columns(V);
    a.nfull = cs.nfull;
    a.nt = cs.nblk;
  }
  a.partials = partials;
  a.ldp = ldp;
  a.ldr = ldr;
  a.e = e;
  a.lde = lde;
  a.row_tokens = row_tokens;
  a.ztgt = ztgt;
  const int nblk = a.mt * a.nt;
  if (small)
    return timed(K_FWD_LOGITS, s, [&] {
      if (one) {
        if (dt) k_fwd_logits64_1s<bf16, false><<<nblk, kThreads, 0, s>>>(a);
        else k_fwd_logits64_1s<float, false><<<nblk, kThreads, 0, s>>>(a);
      } else {
        if (dt) k_fwd_logits64<bf16, false><<<nblk, kThreads, 0, s>>>(a);
        else k_fwd_logits64<float, false><<<nblk, kThreads, 0, s>>>(a);
      }
    });
  return timed(K_FWD_LOGITS, s, [&] {
    if (dt) {
      if (e) k_fwd_logits<bf16, true><<<nblk, 2 * kThreads, 0, s>>>(a);
      else k_fwd_logits<bf16, false><<<nblk, 2 * kThreads, 0, s>>>(a);
    } else {
      if (e) k_fwd_logits<float, true><<<nblk, 2 * kThreads, 0, s>>>(a);
      else k_fwd_logits<float, false><<<nblk, 2 * kThreads, 0, s>>>(a);
    }
  });
}

hipError_t launch_lse_merge(const float2* partials, int64_t ldp, int64_t ldr, int nt,
                            DevRows rows, const float* ztgt,
                            const int* row_tokens, int V, float* lse_out,
                            float* logpi_out, const int* scatter_idx,
                            float* logprobs_rows, int* err, float* eref,
                            int* eflag, hipStream_t s) {
  return timed(K_LSE_MERGE, s, [&] {
    k_lse_merge<<<cdiv(rows.cap, 4), 256, 0, s>>>(
        partials, ldp, ldr, nt, rows, ztgt, row_tokens, V, lse_out, logpi_out,
        scatter_idx, logprobs_rows, err, eref, eflag);
  });
}

hipError_t launch_erebase(void* e, int64_t lde, DevRows rows,
                          const float2* partials, int64_t ldp, int nt,
                          const float* eref, const int* eflag, int Vpad,
                          hipStream_t s) {
  return timed(K_EREBASE, s, [&] {
    k_erebase<<<cdiv(rows.cap, 4), 256, 0, s>>>((bf16*)e, lde, rows, partials,
                                                 ldp, nt, eref, eflag, Vpad);
  });
}

hipError_t launch_mask_compact(const uint8_t* mask, int64_t n,
                               const int* tokens, const int* cu, int B,
                               int* blk, int* nvalid, int* bad_cu, int* idx,
                               int* tokv, int* respv, int* err,
                               hipStream_t s) {
  const int nblk = cdiv(n, kCompactRows);
  hipError_t e = hipSuccess;
  if (nblk > 0) {
    e = timed(K_MASK_COUNT, s, [&] {
      k_mask_count<<<nblk, 256, 0, s>>>(mask, n, blk);
    });
    if (e != hipSuccess) return e;
  }
  e = timed(K_MASK_SCAN, s, [&] {
    k_mask_scan<<<1, 1024, 0, s>>>(blk, nblk, cu, B, n, nvalid, bad_cu, err);
  });
  if (e != hipSuccess || nblk == 0) return e;
  return timed(K_MASK_SCATTER, s, [&] {
    k_mask_scatter<<<nblk, 256, 0, s>>>(mask, n, blk, tokens, cu, B, idx,
                                        tokv, respv);
  });
}

hipError_t launch_rows_finalize(const uint8_t* mask, int64_t n, int H,
                                float* logprobs, float* d_hidden,
                                hipStream_t s) {
  return timed(K_ROWS_FINALIZE, s, [&] {
    k_rows_finalize<<<(unsigned)n, 256, 0, s>>>(mask, n, H, logprobs,
                                                 d_hidden);
  });
}

size_t sort_ws_ints(int64_t cap) {
  const int64_t nt = cap > 0 ? cdiv(cap, kSortTile) : 0;
  return (size_t)(2 * (256 * nt + 1) + 4 * cap);
}

// Stable LSD radix sort of the positions 0 .. n-1 (n = rows' count, at most
// cap) by keys[position] clamped to [0, kmax] (out-of-range keys as kmax):
// *skey / *sval receive the sorted keys and positions.  ws holds
// sort_ws_ints(cap) ints.
hipError_t launch_stable_sort(DevRows rows, int64_t cap, const int* keys,
                              int kmax, int* ws, const int** skey,
                              const int** sval, hipStream_t s) {
  const int ntiles = cap > 0 ? cdiv(cap, kSortTile) : 0;
  int* ghist = ws;
  int* goff = ghist + 256 * (int64_t)ntiles + 1;
  int* buf[4] = {goff + 256 * (int64_t)ntiles + 1, nullptr, nullptr, nullptr};
  for (int i = 1; i < 4; ++i) buf[i] = buf[i - 1] + cap;
  int bits = 0;
  while (bits < 31 && (kmax >> bits) != 0) ++bits;
  const int passes = bits > 8 ? (bits + 7) / 8 : 1;
  const int* kin = keys;
  const int* vin = nullptr;
  for (int p = 0; p < passes; ++p) {
    int* kout = buf[(p & 1) * 2];
    int* vout = buf[(p & 1) * 2 + 1];
    const int clamp = p == 0;
    if (ntiles > 0) {
      hipError_t e = timed(K_SORT_HIST, s, [&] {
        k_sort_hist<<<ntiles, 256, 0, s>>>(rows, kin, kmax, clamp, 8 * p, ntiles, ghist);
      });
      if (e != hipSuccess) return e;
      e = timed(K_SORT_SCAN, s, [&] {
        k_scan_excl<<<1, 1024, 0, s>>>(ghist, 256 * ntiles, goff);
      });
      if (e != hipSuccess) return e;
      e = timed(K_SORT_SCATTER, s, [&] {
        k_sort_scatter<<<ntiles, 256, 0, s>>>(rows, kin, vin, kmax, clamp, 8 * p,
                                              ntiles, goff, kout, vout);
      });
      if (e != hipSuccess) return e;
    }
    kin = kout;
    vin = vout;
  }
  *skey = kin;
  *sval = vin;
  return hipSuccess;
}

hipError_t launch_advantages(const uint8_t* mask, int64_t n, const int* cu,
                             const float* rewards, const int* gid, int B,
                             const int* bad_cu, int* T, int* gcnt, double* gsum,
                             double* Ad, double* fcoef, float* adv, int* bad_gid,
                             int* sort_ws, int* err, hipStream_t s) {
  hipError_t e = timed(K_RESP_COUNTS, s, [&] {
    k_resp_counts<<<B, 256, 0, s>>>(mask, n, cu, T);
  });
  if (e != hipSuccess) return e;
  const int* skey = nullptr;
  const int* sval = nullptr;
  e = launch_stable_sort(DevRows{nullptr, 0, B}, B, gid, B, sort_ws, &skey, &sval, s);
  if (e != hipSuccess) return e;
  e = timed(K_ADVANTAGES, s, [&] {
    k_group_sums<<<cdiv(B, 256), 256, 0, s>>>(B, skey, sval, rewards, gcnt, gsum,
                                              bad_gid);
  });
  if (e != hipSuccess) return e;
  return timed(K_ADVANTAGES, s, [&] {
    k_advantages<<<cdiv(B, 256), 256, 0, s>>>(rewards, gid, B, T, bad_cu, bad_gid,
                                              gcnt, gsum, Ad, fcoef, adv, err);
  });
}

hipError_t launch_loss_value(const uint8_t* mask, const float* logprobs,
                             const float* logmu, int64_t n, const int* cu,
                             int B, int sc, const int* T, const double* Ad,
                             double* S, float* loss, hipStream_t s) {
  hipError_t e = timed(K_RESP_SUMS, s, [&] {
    k_resp_sums<<<B, 256, 0, s>>>(mask, logprobs, logmu, n, cu, sc, S);
  });
  if (e != hipSuccess) return e;
  return timed(K_LOSS_VALUE, s, [&] {
    k_loss_value<<<1, 256, 0, s>>>(Ad, T, S, B, loss);
  });
}

int coef_blocks(int cap) { return cdiv(cap, 256); }

hipError_t launch_coef(DevRows rows, const float* logpi_v, const float* logmu,
                       const int* idx, const int* respv, const double* fcoef,
                       int sc, float* coef, float* coef1, const float* lse_v,
                       const float* eref, float* gsc, int* fexp_part,
                       int* sigma, hipStream_t s) {
  const int nblk = coef_blocks(rows.cap);
  hipError_t e = timed(K_COEF, s, [&] {
    k_coef<<<nblk, 256, 0, s>>>(rows, logpi_v, logmu, idx, respv, fcoef, sc,
                                coef, coef1, lse_v, eref, gsc, fexp_part);
  });
  if (e != hipSuccess || !eref) return e;
  return timed(K_CHUNK_SCALE, s, [&] {
    k_chunk_scale<<<1, 256, 0, s>>>(fexp_part, nblk, sigma);
  });
}

size_t diag_partials_bytes(int64_t n) {
  return (size_t)(n > 0 ? cdiv(n, kDiagChunk) : 1) * sizeof(DiagPartial);
}

hipError_t launch_diagnostics(const float* logpi, const float* logmu,
                              const uint8_t* mask, int64_t n, void* partials,
                              float* diag, hipStream_t s) {
  const int nchunk = cdiv(n, kDiagChunk);
  DiagPartial* p = reinterpret_cast<DiagPartial*>(partials);
  hipError_t e = hipSuccess;
  if (nchunk > 0) {
    e = timed(K_DIAG_PARTIAL, s, [&] {
      k_diag_partial<<<nchunk, 256, 0, s>>>(logpi, logmu, mask, n, p);
    });
    if (e != hipSuccess) return e;
  }
  return timed(K_DIAG_FINAL, s, [&] {
    k_diag_final<<<1, 256, 0, s>>>(p, nchunk, diag);
  });
}

hipError_t launch_mx_dequant(int fmt, const uint8_t* codes, const uint8_t* scales,
                             int64_t nblk, void* out, int* err, hipStream_t s) {
  if (nblk == 0) return hipSuccess;
  const int64_t grid = cdiv(nblk, 256);  // 4 waves x 64 blocks per workgroup
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  return timed(K_MX_DEQUANT, s, [&] {
    if (fmt == 0)
      k_mx_dequant<0><<<grid, 256, 0, s>>>(codes, scales, nblk, o, err);
    else
      k_mx_dequant<1><<<grid, 256, 0, s>>>(codes, scales, nblk, o, err);
  });
}

hipError_t launch_lora_u(int dt, const void* hidden, const void* lora_A,
                         float scale, int64_t n, int H, int r, void* hidden_aug,
                         hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int es = dt ? 2 : 4;
  const int64_t ld_aug = (int64_t)H + kLoraPad;
  // h into the first H columns
  hipError_t e = hipMemcpy2DAsync(hidden_aug, (size_t)ld_aug * es, hidden, (size_t)H * es,
                                  (size_t)H * es, (size_t)n, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return e;
  LoraUArgs a{};
  a.op = GemmOperands{(const char*)hidden, (int64_t)H * es, nullptr, 0,
                      (const char*)lora_A, (int64_t)H * es, r};
  a.n = (int)n;
  a.nk = H / (dt ? Stage<bf16>::kK : Stage<float>::kK);
  a.H = H;
  a.r = r;
  a.ld_aug = ld_aug;
  a.scale = scale;
  a.out = hidden_aug;
  return timed(K_LORA_U, s, [&] {
    if (dt) k_lora_u<bf16><<<cdiv(n, kBM), 2 * kThreads, 0, s>>>(a);
    else k_lora_u<float><<<cdiv(n, kBM), 2 * kThreads, 0, s>>>(a);
  });
}

hipError_t launch_lora_head(int dt, const void* lm_head, const void* lora_B,
                            int V, int H, int r, void* head_aug, hipStream_t s) {
  const int es = dt ? 2 : 4;
  const int64_t ld_aug = (int64_t)H + kLoraPad;
  hipError_t e = hipMemcpy2DAsync(head_aug, (size_t)ld_aug * es, lm_head, (size_t)H * es,
                                  (size_t)H * es, (size_t)V, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return e;
  return timed(K_LORA_COLS, s, [&] {
    if (dt)
      k_lora_cols<bf16><<<V, kLoraPad, 0, s>>>((bf16*)head_aug, ld_aug, H,
                                               (const bf16*)lora_B, r, r);
    else
      k_lora_cols<float><<<V, kLoraPad, 0, s>>>((float*)head_aug, ld_aug, H,
                                                (const float*)lora_B, r, r);
  });
}

size_t lora_da_partials(int64_t n, int r, int H) {
  return (size_t)cdiv(n > 0 ? n : 1, kLoraChunk) * (size_t)r * (size_t)H;
}

hipError_t launch_lora_grads(int dt, const float* dh_aug, int64_t n, int H,
                             const void* hidden, const void* lora_A, int r,
                             float scale, float* part, float* d_hidden,
                             float* d_lora_A, hipStream_t s) {
  const int64_t ld_aug = (int64_t)H + kLoraPad;
  hipError_t e = hipSuccess;
  if (n > 0) {
    e = timed(K_LORA_DH, s, [&] {
      if (dt)
        k_lora_dh<bf16><<<cdiv(n, 64), 256, 0, s>>>(dh_aug, ld_aug, H, (const bf16*)lora_A,
                                                    r, scale, n, d_hidden);
      else
        k_lora_dh<float><<<cdiv(n, 64), 256, 0, s>>>(dh_aug, ld_aug, H, (const float*)lora_A,
                                                     r, scale, n, d_hidden);
    });
    if (e != hipSuccess) return e;
  }
  const int nchunk = (int)cdiv(n > 0 ? n : 1, kLoraChunk);
  if (n > 0) {
    dim3 grid(nchunk, cdiv(H, 256));
    e = timed(K_LORA_DA, s, [&] {
      if (dt)
        k_lora_da_partial<bf16><<<grid, 256, 0, s>>>(dh_aug, ld_aug, H, (const bf16*)hidden,
                                                     n, r, part);
      else
        k_lora_da_partial<float><<<grid, 256, 0, s>>>(dh_aug, ld_aug, H, (const float*)hidden,
                                                      n, r, part);
    });
    if (e != hipSuccess) return e;
  }
  return timed(K_LORA_DA, s, [&] {
    k_lora_da_final<<<cdiv((int64_t)r * H, 256), 256, 0, s>>>(part, n > 0 ? nchunk : 0,
                                                             r, H, scale, d_lora_A);
  });
}

size_t norm_partials(int64_t n) { return (size_t)cdiv(n, kNormChunk); }

hipError_t launch_grad_norm(const float* x, int64_t n, double* partials,
                            float* norm, hipStream_t s) {
  const int nchunk = (int)norm_partials(n);
  hipError_t e = hipSuccess;
  if (nchunk > 0) {
    e = timed(K_GRAD_NORM, s, [&] {
      k_sumsq_partial<<<nchunk, 256, 0, s>>>(x, n, partials);
    });
    if (e != hipSuccess) return e;
  }
  return timed(K_GRAD_NORM_FINAL, s, [&] {
    k_sumsq_final<<<1, 1024, 0, s>>>(partials, nchunk, norm);
  });
}

hipError_t launch_resp_diag(const float* logpi, const float* logmu,
                            const uint8_t* mask, const int* cu, int B,
                            int64_t n, float* d3, float* kl, int* err,
                            hipStream_t s) {
  return timed(K_RESP_DIAG, s, [&] {
    k_resp_diag<<<B, 1024, 0, s>>>(logpi, logmu, mask, cu, B, n, d3, kl, err);
  });
}

hipError_t launch_transpose(int dt, int kid, const void* in, int64_t ld_in,
                            const int* rowmap, DevRows rows, int rows_pad,
                            int cols, void* out, int64_t ld_out,
                            const float* rs_c, const float* rs_g,
                            const int* rs_sigma, hipStream_t s) {
  // 64 rows x (4 waves x 64 bf16 or 16 fp32 columns) per workgroup
  dim3 grid(cdiv(rows_pad, 64), cdiv(cols, dt ? 256 : 64));
  return timed(kid, s, [&] {
    if (dt && rs_c)
      k_transpose<bf16, true><<<grid, 256, 0, s>>>((const bf16*)in, ld_in,
                                                   rowmap, rows, rows_pad, cols,
                                                   (bf16*)out, ld_out, rs_c,
                                                   rs_g, rs_sigma);
    else if (dt)
      k_transpose<bf16><<<grid, 256, 0, s>>>((const bf16*)in, ld_in, rowmap,
                                             rows, rows_pad, cols, (bf16*)out,
                                             ld_out, nullptr, nullptr, nullptr);
    else
      k_transpose<float><<<grid, 256, 0, s>>>((const float*)in, ld_in,
                                              rowmap, rows, rows_pad, cols,
                                              (float*)out, ld_out, nullptr,
                                              nullptr, nullptr);
  });
}

hipError_t launch_dz_scale(float* dz, int64_t ldz, float* dzT, int64_t ldzt,
                           DevRows rows, const float2* partials, int64_t ldp,
                           const float* lse, const float* coef,
                           const int* tokv, int Vpad, hipStream_t s) {
  // 64 rows x (4 waves x 16 columns) per workgroup
  dim3 grid(cdiv(Vpad, 64), cdiv(rows.cap, 64));
  return timed(K_DZ_SCALE, s, [&] {
    k_dz_scale<<<grid, 256, 0, s>>>(dz, ldz, dzT, ldzt, rows, partials, ldp,
                                    lse, coef, tokv, Vpad);
  });
}

template <typename T>
static hipError_t launch_bwd_dh_t(const void* dz, int64_t ldz, DevRows rows,
                                  const void* WT, int64_t ldwt, int H, int V,
                                  int Vpad, const int* idx, const int* tokv,
                                  const float* coef, const float* rcoef,
                                  const float* rg, const void* lm_head,
                                  float* d_hidden, float* part, hipStream_t s) {
  DhArgs<T> a;
  a.op = GemmOperands{(const char*)dz, ldz * (int64_t)sizeof(T), nullptr,
                      rows.base * 0, (const char*)WT,
                      ldwt * (int64_t)sizeof(T), H};
  a.rows = rows;
  a.idx = idx;
  a.tokv = tokv;
  a.coef = coef;
  a.rc = rcoef;
  a.rg = rg;
  a.W = (const T*)lm_head;
  a.H = H;
  a.V = V;
  a.nk = Vpad / Stage<T>::kK;
  a.mt = cdiv(rows.cap, kBM);
  a.nt = cdiv(H, kBN);
  a.ncu = cu_count();
  a.part = part;
  a.dh = d_hidden;
  return timed(K_BWD_DH, s, [&] {
    // launch bounds: every tile of rows.cap rows; the pieces and their sums
    // of at most kSplitWGs parked tiles
    k_bwd_dh<T, false><<<a.mt * a.nt, 2 * kThreads, 0, s>>>(a);
    if (part) {
      k_bwd_dh<T, true><<<kSplitWGs, 2 * kThreads, 0, s>>>(a);
      k_dh_tail<T><<<kSplitWGs * 2, 2 * kThreads, 0, s>>>(a);
    }
  });
}

hipError_t launch_bwd_dh(int dt, const void* dz, int64_t ldz, DevRows rows,
                         const void* WT, int64_t ldwt, int H, int V, int Vpad,
                         const int* idx, const int* tokv, const float* coef,
                         const float* rcoef, const float* rg,
                         const void* lm_head, float* d_hidden, float* part,
                         hipStream_t s) {
  return dt ? launch_bwd_dh_t<bf16>(dz, ldz, rows, WT, ldwt, H, V, Vpad, idx,
                                    tokv, coef, rcoef, rg, lm_head, d_hidden,
                                    part, s)
            : launch_bwd_dh_t<float>(dz, ldz, rows, WT, ldwt, H, V, Vpad, idx,
                                     tokv, coef, nullptr, nullptr, lm_head,
                                     d_hidden, part, s);
}

int64_t dw_part_floats(int V, int H) {
  const int64_t T = (int64_t)cdiv(V, kBM) * cdiv(H, kBN);
  const int64_t tiles = T * kSplitMax < kSplitWGs ? T * kSplitMax : kSplitWGs;
  return tiles * kPartTileFloats;
}

int64_t dh_part_floats(int64_t rows, int H) {
  const int64_t T = (int64_t)cdiv(rows, kBM) * cdiv(H, kBN);
  const int64_t tiles = T * kSplitMax < kSplitWGs ? T * kSplitMax : kSplitWGs;
  return tiles * kPartTileFloats;
}

hipError_t launch_bwd_dw(int dt, const void* dz, int64_t ld, DevRows krows,
                         const void* hT, int64_t ldht, int H, int V, int Vpad,
                         float* d_lm_head, int first, float* part,
                         const int* sigma, hipStream_t s) {
  const int esz = dt ? 2 : 4;
  DwArgs a;
  a.op = GemmOperands{(const char*)dz, ld * esz, nullptr, 0,
                      (const char*)hT, ldht * esz, H};
  a.krows = krows;
  a.sigma = dt ? sigma : nullptr;
  a.V = V;
  a.H = H;
  a.amax = dt ? Vpad : V;
  a.kstage = dt ? Stage<bf16>::kK : Stage<float>::kK;
  a.mt = cdiv(V, kBM);
  a.nt = cdiv(H, kBN);
  a.first = first;
  a.dw = d_lm_head;
  // One workgroup per CU per round: the last round's tiles (tail) would
  // leave most CUs idle, so each is split into up to kSplitMax pieces
  // along K (fixed by V, H and the CU count, never by the row count).
  a.T = a.mt * a.nt;
  const RoundSplit rs = part ? round_split(a.T, cu_count()) : RoundSplit{0, 1};
  a.tail = rs.tail;
  a.split = rs.split;
  a.part = part;
  return timed(K_BWD_DW, s, [&] {
    const int grid = a.T - a.tail + a.tail * a.split;
    if (dt) k_bwd_dw<bf16><<<grid, 2 * kThreads, 0, s>>>(a);
    else k_bwd_dw<float><<<grid, 2 * kThreads, 0, s>>>(a);
    if (a.tail) k_dw_tail<<<a.tail * 2, 2 * kThreads, 0, s>>>(a);
  });
}

int64_t dw_fix_cont_floats(int64_t cap, int H) {
  return 2 * (int64_t)(cap > 0 ? cdiv(cap, kFixPiece) : 0) * H;
}

hipError_t launch_dw_fix(int dt, const int* nvalid, int64_t cap,
                         const int* tokv, const int* idx, const float* coef,
                         const void* hidden, int64_t ld, int H, int V,
                         int* sort_ws, float* cont, float* d_lm_head,
                         hipStream_t s) {
  if (cap == 0) return hipSuccess;
  DevRows rows{nvalid, 0, (int)cap};
  const int* skey = nullptr;
  const int* sval = nullptr;
  hipError_t e = launch_stable_sort(rows, cap, tokv, V, sort_ws, &skey, &sval, s);
  if (e != hipSuccess) return e;
  const int npieces = cdiv(cap, kFixPiece);
  float* cont_first = cont;
  float* cont_last = cont + (int64_t)npieces * H;
  e = timed(K_DW_FIX, s, [&] {
    if (dt)
      k_dw_fix<bf16><<<npieces, 256, 0, s>>>(rows, skey, sval, idx, coef,
                                             (const bf16*)hidden, ld, H, V,
                                             cont_first, cont_last, d_lm_head);
    else
      k_dw_fix<float><<<npieces, 256, 0, s>>>(rows, skey, sval, idx, coef,
                                              (const float*)hidden, ld, H, V,
                                              cont_first, cont_last, d_lm_head);
  });
  if (e != hipSuccess) return e;
  return timed(K_DW_FIX_SPAN, s, [&] {
    k_dw_fix_span<<<npieces, 256, 0, s>>>(rows, skey, H, V, cont_first, cont_last,
                                          d_lm_head);
  });
}

}  // namespace rz
