// rz_internal.h -- launchers shared by the kernel and API translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rz {

// Kernel classes, in the order the timer reports them.
enum KernelId {
  K_MASK_COUNT = 0,
  K_MASK_SCAN,
  K_MASK_SCATTER,
  K_RESP_COUNTS,     // rz_loss: T_i
  K_ADVANTAGES,      // rz_loss: groups, A_i, per-response factors
  K_FWD_LOGITS,      // bi_lmhead_gemm with the fused log-softmax epilogue
  K_LSE_MERGE,       // bi_logsoftmax_gather merge
  K_ROWS_FINALIZE,
  K_COEF,
  K_DZ_SCALE,        // fp32 dlogits from the forward's stored exp(z - m_j)
  K_EREBASE,         // bf16 e: rows whose tiles straddle the e window
  K_CHUNK_SCALE,     // bf16 dW: the chunk's power of two
  K_RESP_SUMS,       // rz_loss: S_i
  K_LOSS_VALUE,      // rz_loss: L
  K_DIAG_PARTIAL,    // rz_diagnostics
  K_DIAG_FINAL,
  K_TRANSPOSE_W,
  K_TRANSPOSE_H,
  K_BWD_DH,          // dHidden GEMM
  K_BWD_DW,          // dW GEMM
  K_SORT_HIST,       // stable radix sort by key: digit histograms
  K_SORT_SCAN,       //   their exclusive scan
  K_SORT_SCATTER,    //   the stable scatter
  K_DW_FIX,          // dW one-hot fix-up over pieces of the sorted list
  K_DW_FIX_SPAN,     //   runs crossing pieces
  K_FWD_SAMPLE,      // rollout-side logits GEMM with the draw in the epilogue
  K_DRAW_MERGE,      // per-row best draw over the statistics tiles + the record
  K_GRAD_NORM,       // run-level: float64 sums of squares per chunk
  K_GRAD_NORM_FINAL, // run-level: fixed tree over the chunks, sqrt
  K_RESP_DIAG,       // run-level: per-response D3 and KL
  K_MX_DEQUANT,      // MX-format head -> bf16
  K_LORA_U,          // LoRA: u = s h A^T into the augmented hidden
  K_LORA_COLS,       // LoRA: B into the augmented head
  K_LORA_DH,         // LoRA: dL/dh through both paths
  K_LORA_DA,         // LoRA: dL/dA partials and their ordered sum
  K_NUM_KERNELS
};

const char* kernel_name(int k);

// Brackets launches with events when the timer is on.
struct Timer {
  static bool on();
  static void before(int k, hipStream_t s);
  static hipError_t after(int k, hipStream_t s);
};

// Device counts live in the workspace; a null pointer means "use cap".
struct DevRows {
  const int* count;
  int64_t base;
  int cap;
};

// ---- launchers (return the launch status) ----
hipError_t launch_fwd_logits(int dt, const void* hidden, int64_t lda_bytes,
                             const int* a_rows, DevRows rows,
                             const void* lm_head, int H, int V,
                             const int* row_tokens, float2* partials,
                             int64_t ldp, int64_t ldr, float* ztgt, void* e,
                             int64_t lde, int Vpad, hipStream_t s);
// The logits GEMM with the draw in its epilogue: per (statistics tile, row)
// the best (z + g, index) in cand and that column's z in candz.
hipError_t launch_fwd_sample(int dt, const void* hidden, int64_t n,
                             const void* lm_head, int H, int V,
                             const uint64_t* row_ids, uint64_t seed,
                             float2* partials, float2* cand, float* candz,
                             int64_t ldp, int64_t ldr, hipStream_t s);
// The draw's winner per row (tokens) and the record: log mu = z[a_t] - lse
// (and lse, nullable), lse by k_lse_merge's fold.
hipError_t launch_draw_merge(const float2* cand, const float* candz,
                             const float2* partials, int64_t ldp, int64_t ldr,
                             int nt, int64_t n, int V, int* tokens, float* logmu,
                             float* lse, hipStream_t s);
hipError_t launch_mx_dequant(int fmt, const uint8_t* codes, const uint8_t* scales,
                             int64_t nblk, void* out, int* err, hipStream_t s);
constexpr int kLoraCols = 64;  // LoRA: largest rank and u block width
hipError_t launch_lora_u(int dt, const void* hidden, const void* lora_A,
                         float scale, int64_t n, int H, int r, void* hidden_aug,
                         hipStream_t s);
hipError_t launch_lora_head(int dt, const void* lm_head, const void* lora_B,
                            int V, int H, int r, void* head_aug, hipStream_t s);
size_t lora_da_partials(int64_t n, int r, int H);
hipError_t launch_lora_grads(int dt, const float* dh_aug, int64_t n, int H,
                             const void* hidden, const void* lora_A, int r,
                             float scale, float* part, float* d_hidden,
                             float* d_lora_A, hipStream_t s);
int mx_rows64_max(int sample);
hipError_t launch_fwd_mx(int fmt, const void* hidden, int64_t n,
                         const uint8_t* codes, const uint8_t* scales, int H,
                         int V, const int* row_tokens, float2* partials,
                         int64_t ldp, int64_t ldr, float* ztgt, const uint64_t* row_ids,
                         uint64_t seed, float2* cand, float* candz, int* err,
                         hipStream_t s);
size_t norm_partials(int64_t n);
hipError_t launch_grad_norm(const float* x, int64_t n, double* partials,
                            float* norm, hipStream_t s);
hipError_t launch_resp_diag(const float* logpi, const float* logmu,
                            const uint8_t* mask, const int* cu, int B,
                            int64_t n, float* d3, float* kl, int* err,
                            hipStream_t s);
// eref / eflag (bf16 learner call, else null): the row's e reference and
// whether its tiles need k_erebase
hipError_t launch_lse_merge(const float2* partials, int64_t ldp, int64_t ldr, int nt,
                            DevRows rows, const float* ztgt,
                            const int* row_tokens, int V, float* lse_out,
                            float* logpi_out, const int* scatter_idx,
                            float* logprobs_rows, int* err, float* eref,
                            int* eflag, hipStream_t s);
// bf16 e [rows][lde]: the flagged rows' tiles rebased to the row reference
hipError_t launch_erebase(void* e, int64_t lde, DevRows rows,
                          const float2* partials, int64_t ldp, int nt,
                          const float* eref, const int* eflag, int Vpad,
                          hipStream_t s);
hipError_t launch_mask_compact(const uint8_t* mask, int64_t n,
                               const int* tokens, const int* cu, int B,
                               int* blk, int* nvalid, int* bad_cu, int* idx,
                               int* tokv, int* respv, int* err, hipStream_t s);
hipError_t launch_rows_finalize(const uint8_t* mask, int64_t n, int H,
                                float* logprobs, float* d_hidden,
                                hipStream_t s);
// ints of workspace launch_stable_sort needs for at most cap elements
size_t sort_ws_ints(int64_t cap);
hipError_t launch_stable_sort(DevRows rows, int64_t cap, const int* keys,
                              int kmax, int* ws, const int** skey,
                              const int** sval, hipStream_t s);
hipError_t launch_advantages(const uint8_t* mask, int64_t n, const int* cu,
                             const float* rewards, const int* gid, int B,
                             const int* bad_cu, int* T, int* gcnt, double* gsum,
                             double* Ad, double* fcoef, float* adv, int* bad_gid,
                             int* sort_ws, int* err, hipStream_t s);
// sc = 1: score centering (S_i sums log pi; c_t = A_i / (B T_i))
hipError_t launch_loss_value(const uint8_t* mask, const float* logprobs,
                             const float* logmu, int64_t n, const int* cu,
                             int B, int sc, const int* T, const double* Ad,
                             double* S, float* loss, hipStream_t s);
// coef = c_t; coef1 = c_t (1 - p[a_t]), the token column's exact term.
// bf16 learner (eref non-null): also gsc = g_t = exp(r*_t ln 2 - lse_t),
// fexp_part [coef_blocks(rows.cap)] and the chunk's sigma
int coef_blocks(int cap);
hipError_t launch_coef(DevRows rows, const float* logpi_v, const float* logmu,
                       const int* idx, const int* respv, const double* fcoef,
                       int sc, float* coef, float* coef1, const float* lse_v,
                       const float* eref, float* gsc, int* fexp_part,
                       int* sigma, hipStream_t s);
size_t diag_partials_bytes(int64_t n);
hipError_t launch_diagnostics(const float* logpi, const float* logmu,
                              const uint8_t* mask, int64_t n, void* partials,
                              float* diag, hipStream_t s);
// rs_c / rs_g / rs_sigma (bf16 only, else null): row r scaled by
// c_r g_r 2^sigma before the transpose
hipError_t launch_transpose(int dt, int kid, const void* in, int64_t ld_in,
                            const int* rowmap, DevRows rows, int rows_pad,
                            int cols, void* out, int64_t ld_out,
                            const float* rs_c, const float* rs_g,
                            const int* rs_sigma, hipStream_t s);
// fp32 learner only
hipError_t launch_dz_scale(float* dz, int64_t ldz, float* dzT, int64_t ldzt,
                           DevRows rows, const float2* partials, int64_t ldp,
                           const float* lse, const float* coef,
                           const int* tokv, int Vpad, hipStream_t s);
// bf16: dz = the stored e, scaled by rcoef (c_t) and rg (g_t) in the
// epilogue; fp32: dz, rcoef = rg = null
// part: room for the last round's K pieces, dh_part_floats(rows.cap, H)
// floats (null: no split)
int64_t dh_part_floats(int64_t rows, int H);
hipError_t launch_bwd_dh(int dt, const void* dz, int64_t ldz, DevRows rows,
                         const void* WT, int64_t ldwt, int H, int V, int Vpad,
                         const int* idx, const int* tokv, const float* coef,
                         const float* rcoef, const float* rg,
                         const void* lm_head, float* d_hidden, float* part,
                         hipStream_t s);
// bf16: dz = e [C][Vpad] (ld = Vpad), read K-major, hT scaled per row and
// sigma the chunk's power of two; fp32: dz = dz^T [Vpad][C] (ld = C)
// Floats of the dW split workspace (launch_bwd_dw's part) for a head of
// V rows and H gradient columns.
int64_t dw_part_floats(int V, int H);
hipError_t launch_bwd_dw(int dt, const void* dz, int64_t ld, DevRows krows,
                         const void* hT, int64_t ldht, int H, int V, int Vpad,
                         float* d_lm_head, int first, float* part,
                         const int* sigma, hipStream_t s);
// floats of the parked run sums of launch_dw_fix for at most cap rows
int64_t dw_fix_cont_floats(int64_t cap, int H);
hipError_t launch_dw_fix(int dt, const int* nvalid, int64_t cap,
                         const int* tokv, const int* idx, const float* coef,
                         const void* hidden, int64_t ld, int H, int V,
                         int* sort_ws, float* cont, float* d_lm_head,
                         hipStream_t s);

}  // namespace rz
