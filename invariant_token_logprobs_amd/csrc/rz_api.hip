// rz_api.hip -- the C ABI of librz (declared in include/rz.h): host-side
// argument checks, workspace layout and the launch sequence of each entry
// point on the caller's stream.  No allocation, no host synchronisation.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/rz.h"
#include "rz_internal.h"

// Scratch of rz_sample_tokens_noalloc: RZ_NOALLOC_SCRATCH_BYTES per GPU.
static __device__ __align__(256) char scratch[RZ_NOALLOC_SCRATCH_BYTES];

namespace rz {
namespace {

constexpr size_t kAlign = 256;
constexpr int kChunkRows = 32768;  // backward token chunk (a multiple of 256)
// vocabulary columns per statistics tile: one (m, s) partial, and one draw
// candidate, per row and tile
constexpr int kVocabTile = 128;

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Layout of the statistics-tile partials and draw candidates: (tile j, row
// p) at j * lt + p * lr.  Host-known row counts up to 256 keep one row's
// tiles contiguous (the merge's loads of a row coalesce; the forward stores
// few of them); larger ones keep one tile's rows contiguous (the forward's
// stores coalesce).
struct PartLayout {
  int64_t lt, lr;
};
inline PartLayout part_layout(int64_t n, int nt) {
  return n <= 256 ? PartLayout{1, nt} : PartLayout{n, 1};
}
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline size_t esize(rz_dtype dt) { return dt == RZ_DTYPE_BF16 ? 2 : 4; }

// Bump allocator over the caller's workspace; with base == nullptr it only
// measures.
struct Carver {
  char* base;
  size_t off = 0;
  template <typename P>
  P* take(size_t bytes) {
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += align_up(bytes);
    return p;
  }
};

bool dims_ok(int32_t H, int32_t V, rz_dtype dt) {
  return (dt == RZ_DTYPE_F32 || dt == RZ_DTYPE_BF16) && H > 0 &&
         H <= RZ_MAX_HIDDEN && (H % 64) == 0 && V > 0 && V <= RZ_MAX_VOCAB;
}

int chunk_rows(int64_t n) {
  const int64_t c = round_up(n > 0 ? n : 1, 256);
  return (int)(c < kChunkRows ? c : kChunkRows);
}

// ---- token_logprobs layout ----
struct TlpWs {
  float2* partials;
  float* ztgt;
};
size_t carve_tlp(Carver& c, int64_t n, int32_t V, TlpWs* w) {
  const int nt = (int)((V + kVocabTile - 1) / kVocabTile);
  TlpWs t;
  t.partials = c.take<float2>(sizeof(float2) * (size_t)nt * (size_t)n);
  t.ztgt = c.take<float>(sizeof(float) * (size_t)n);
  if (w) *w = t;
  return c.off;
}

// ---- sample layout ----
struct SmpWs {
  float2* partials;
  float2* cand;
  float* candz;
};
size_t carve_smp(Carver& c, int64_t n, int32_t V, SmpWs* w) {
  const int nt = (int)((V + kVocabTile - 1) / kVocabTile);
  SmpWs t;
  t.partials = c.take<float2>(sizeof(float2) * (size_t)nt * (size_t)n);
  t.cand = c.take<float2>(sizeof(float2) * (size_t)nt * (size_t)n);
  t.candz = c.take<float>(sizeof(float) * (size_t)nt * (size_t)n);
  if (w) *w = t;
  return c.off;
}

// ---- grad_norms layout: float64 chunk sums of each gradient ----
constexpr int64_t kMaxNormElems = (int64_t)1 << 36;  // 256 GiB of fp32
struct GnWs {
  double* ph;
  double* pw;
};
size_t carve_gn(Carver& c, int64_t n, int32_t H, int32_t V, GnWs* w) {
  GnWs t;
  t.ph = c.take<double>(sizeof(double) * (norm_partials(n * H) + 1));
  t.pw = c.take<double>(sizeof(double) * (norm_partials((int64_t)V * H) + 1));
  if (w) *w = t;
  return c.off;
}

// ---- MX-format head: the 64-row tile reads the codes itself; otherwise the
// head is expanded to bf16 at the end of the workspace first ----
bool mx_fused(int64_t n, int32_t H, bool sample) {
  return n <= mx_rows64_max(sample ? 1 : 0) && H % 128 == 0;
}

// ---- fwd_bwd layout ----
struct FbWs {
  int* nvalid;
  int* bad_cu;
  int* blk;
  int* idx;
  int* tokv;
  int* respv;
  float2* partials;
  float* ztgt;
  float* lse_v;
  float* logpi_v;
  float* coef;
  float* coef1;
  float* eref;    // bf16: the row's e reference r*_t
  int* eflag;     // bf16: the row's tiles need rebasing
  float* gsc;     // bf16: g_t = exp(r*_t ln 2 - lse_t)
  int* fexp_part; // bf16: per-workgroup largest exponent of c_t g_t
  int* sigma;     // bf16: the chunk's power of two for dW
  int* T;
  double* S;
  int* gcnt;
  double* gsum;
  double* fcoef;
  double* Ad;
  float* diag_tmp;
  void* diag_part;
  void* WT;
  void* hT;
  void* dz;
  void* dzT;
  int* bad_gid;
  int* sort_ws;
  float* fix_cont;
  float* dwpart;
};
// H: the GEMM width (hidden and head row length); dw_cols: the columns of
// the head that get a gradient (all H, or a LoRA adapter's window)
size_t carve_fb(Carver& c, int64_t n, int32_t B, int32_t H, int32_t V,
                rz_dtype dt, FbWs* w, int32_t dw_cols) {
  if (dw_cols < 0) dw_cols = H;
  const int nt = (int)((V + kVocabTile - 1) / kVocabTile);
  const int64_t Vpad = round_up(V, 64);
  const int C = chunk_rows(n);
  const size_t es = esize(dt);
  FbWs t;
  t.nvalid = c.take<int>(sizeof(int));
  t.bad_cu = c.take<int>(sizeof(int));
  t.blk = c.take<int>(sizeof(int) * (size_t)((n + 1023) / 1024 + 1));
  t.idx = c.take<int>(sizeof(int) * (size_t)n);
  t.tokv = c.take<int>(sizeof(int) * (size_t)n);
  t.respv = c.take<int>(sizeof(int) * (size_t)n);
  t.partials = c.take<float2>(sizeof(float2) * (size_t)nt * (size_t)n);
  t.ztgt = c.take<float>(sizeof(float) * (size_t)n);
  t.lse_v = c.take<float>(sizeof(float) * (size_t)n);
  t.logpi_v = c.take<float>(sizeof(float) * (size_t)n);
  t.coef = c.take<float>(sizeof(float) * (size_t)n);
  t.coef1 = c.take<float>(sizeof(float) * (size_t)n);
  t.eref = c.take<float>(sizeof(float) * (size_t)n);
  t.eflag = c.take<int>(sizeof(int) * (size_t)n);
  t.gsc = c.take<float>(sizeof(float) * (size_t)n);
  t.fexp_part = c.take<int>(sizeof(int) * (size_t)coef_blocks(C));
  t.sigma = c.take<int>(sizeof(int));
  t.T = c.take<int>(sizeof(int) * (size_t)B);
  t.S = c.take<double>(sizeof(double) * (size_t)B);
  t.gcnt = c.take<int>(sizeof(int) * (size_t)B);
  t.gsum = c.take<double>(sizeof(double) * (size_t)B);
  t.fcoef = c.take<double>(sizeof(double) * (size_t)B);
  t.Ad = c.take<double>(sizeof(double) * (size_t)B);
  t.diag_tmp = c.take<float>(2 * sizeof(float));
  t.diag_part = c.take<char>(diag_partials_bytes(n));
  t.WT = c.take<char>(es * (size_t)H * (size_t)Vpad);
  t.hT = c.take<char>(es * (size_t)dw_cols * (size_t)C);
  // bf16: the stored e, the backward GEMMs' A operand; fp32: e, then dz
  t.dz = c.take<char>(es * (size_t)C * (size_t)Vpad);
  // dz^T only for fp32 (bf16 dW reads e through transposing LDS reads)
  t.dzT = dt == RZ_DTYPE_F32 ? c.take<char>(es * (size_t)Vpad * (size_t)C)
                             : nullptr;
  t.bad_gid = c.take<int>(sizeof(int));
  // one sort buffer serves the group ids (B keys) and then the tokens (n)
  t.sort_ws = c.take<int>(sizeof(int) * sort_ws_ints(std::max<int64_t>(n, B)));
  t.fix_cont = c.take<float>(sizeof(float) * (size_t)dw_fix_cont_floats(n, dw_cols));
  // parked K pieces of the last round: the dHidden GEMM's, then (after it)
  // the dW GEMM's
  t.dwpart = c.take<float>(sizeof(float) *
                           (size_t)std::max(dw_part_floats(V, dw_cols),
                                            dh_part_floats(C, H)));
  if (w) *w = t;
  return c.off;
}

// ---- LoRA learner layout: augmented operands, dL/dh_aug, dB, dA partials,
// then the core's own workspace for the augmented width ----
struct LoraWs {
  void* h_aug;
  void* head_aug;
  float* dh_aug;
  float* dB;
  float* part;
  char* core;
};
size_t carve_lora(Carver& c, int64_t n, int32_t B, int32_t H, int32_t V,
                  rz_dtype dt, LoraWs* w) {
  const size_t es = esize(dt);
  const int64_t Ha = (int64_t)H + kLoraCols;
  LoraWs t;
  t.h_aug = c.take<char>(es * (size_t)n * (size_t)Ha);
  t.head_aug = c.take<char>(es * (size_t)V * (size_t)Ha);
  t.dh_aug = c.take<float>(sizeof(float) * (size_t)n * (size_t)Ha);
  t.dB = c.take<float>(sizeof(float) * (size_t)V * kLoraCols);
  t.part = c.take<float>(sizeof(float) * lora_da_partials(n, kLoraCols, H));
  t.core = c.base ? c.base + c.off : nullptr;
  Carver cc{t.core};
  c.off += carve_fb(cc, n, B, (int32_t)Ha, V, dt, nullptr, kLoraCols);
  if (w) *w = t;
  return c.off;
}


// Arrays the kernels move in 16-byte pieces must start 16-byte aligned.
bool misaligned(const void* a, const void* b = nullptr, const void* c = nullptr,
                const void* d = nullptr) {
  return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
           reinterpret_cast<uintptr_t>(c) | reinterpret_cast<uintptr_t>(d)) & 15) != 0;
}

rz_status ws_check(void* ws, size_t have, size_t need) {
  if (need == 0) return RZ_OK;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0 || have < need)
    return RZ_ERR_WORKSPACE;
  return RZ_OK;
}

#define RZ_TRY(expr)                                  \
  do {                                                \
    hipError_t e_ = (expr);                           \
    if (e_ != hipSuccess) return RZ_ERR_HIP;          \
  } while (0)

// ---- kernel timer ----
struct TimerState {
  bool on = false;
  struct Pending {
    int k;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double total[K_NUM_KERNELS] = {};
  int64_t count[K_NUM_KERNELS] = {};
  hipEvent_t cur_a = nullptr;
};
thread_local TimerState g_timer;

hipEvent_t take_event() {
  if (!g_timer.pool.empty()) {
    hipEvent_t e = g_timer.pool.back();
    g_timer.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// ---- the allocation-free draw's scratch (rz_sample_tokens_noalloc) ----
// `scratch` (file scope, above) is one static device array per GPU, held
// until the process ends.  In host code its name is a host-side stand-in,
// never a device address, so the device address is looked up once per
// device (with that device current) and kept, and only that address is
// ever handed to kernels.
constexpr size_t kScratchBytes = (size_t)RZ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

rz_status scratch_on_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return RZ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RZ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return RZ_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return RZ_OK;
}

}  // namespace

bool Timer::on() { return g_timer.on; }

void Timer::before(int, hipStream_t s) {
  if (!g_timer.on) return;
  g_timer.cur_a = take_event();
  if (g_timer.cur_a) (void)hipEventRecord(g_timer.cur_a, s);
}

hipError_t Timer::after(int k, hipStream_t s) {
  if (!g_timer.on || !g_timer.cur_a) return hipSuccess;
  hipEvent_t b = take_event();
  if (!b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(b, s);
  g_timer.pending.push_back({k, g_timer.cur_a, b});
  g_timer.cur_a = nullptr;
  return e;
}

}  // namespace rz

using namespace rz;

extern "C" {

const char* rz_status_string(rz_status s) {
  switch (s) {
    case RZ_OK: return "ok";
    case RZ_ERR_INVALID_ARG: return "invalid argument";
    case RZ_ERR_UNSUPPORTED: return "unsupported dtype or size";
    case RZ_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case RZ_ERR_HIP: return "HIP launch or event failure";
    case RZ_ERR_SCRATCH: return "sizes exceed the static scratch of the allocation-free call";
  }
  return "unknown status";
}

size_t rz_workspace_bytes_op(rz_op op, int64_t n_rows, int32_t n_resp,
                             int32_t H, int32_t V, rz_dtype dt) {
  if (n_rows < 0 || n_rows > RZ_MAX_ROWS) return 0;
  Carver c{nullptr};
  switch (op) {
    case RZ_OP_TOKEN_LOGPROBS:
      if (!dims_ok(H, V, dt)) return 0;
      return n_rows == 0 ? 0 : carve_tlp(c, n_rows, V, nullptr);
    case RZ_OP_FWD_BWD:
    case RZ_OP_SCORE_CENTERING:
      if (!dims_ok(H, V, dt) || n_resp < 1 || n_resp > RZ_MAX_RESPONSES) return 0;
      return carve_fb(c, n_rows, n_resp, H, V, dt, nullptr, -1);
    case RZ_OP_DIAGNOSTICS:
      return align_up(diag_partials_bytes(n_rows));
    case RZ_OP_SAMPLE:
      if (!dims_ok(H, V, dt)) return 0;
      return n_rows == 0 ? 0 : carve_smp(c, n_rows, V, nullptr);
    case RZ_OP_TOKEN_LOGPROBS_MX:
    case RZ_OP_SAMPLE_MX: {
      if (!dims_ok(H, V, RZ_DTYPE_BF16) || n_rows == 0) return 0;
      const bool smp = op == RZ_OP_SAMPLE_MX;
      return (smp ? carve_smp(c, n_rows, V, nullptr) : carve_tlp(c, n_rows, V, nullptr)) +
             (mx_fused(n_rows, H, smp) ? 0 : align_up(2 * (size_t)V * (size_t)H));
    }
    case RZ_OP_FWD_BWD_LORA:
      if (!dims_ok(H, V, dt) || n_resp < 1 || n_resp > RZ_MAX_RESPONSES ||
          H + kLoraCols > RZ_MAX_HIDDEN)
        return 0;
      return carve_lora(c, n_rows, n_resp, H, V, dt, nullptr);
    case RZ_OP_GRAD_NORMS:
      if (H <= 0 || H > RZ_MAX_HIDDEN || V <= 0 || V > RZ_MAX_VOCAB) return 0;
      return carve_gn(c, n_rows, H, V, nullptr);
  }
  return 0;
}

size_t rz_workspace_bytes(int64_t n_rows, int32_t n_resp, int32_t H, int32_t V,
                          rz_dtype dt) {
  const size_t a = rz_workspace_bytes_op(RZ_OP_TOKEN_LOGPROBS, n_rows, 1, H, V, dt);
  const size_t b = rz_workspace_bytes_op(RZ_OP_FWD_BWD, n_rows, n_resp, H, V, dt);
  const size_t d = rz_workspace_bytes_op(RZ_OP_DIAGNOSTICS, n_rows, 1, H, V, dt);
  return std::max(a, std::max(b, d));
}

rz_status rz_grad_norms(const float* d_hidden, int64_t n_rows, int32_t H,
                        const float* d_lm_head, int32_t V, float* norms,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (n_rows < 0 || n_rows > RZ_MAX_ROWS) return RZ_ERR_INVALID_ARG;
  if (H <= 0 || H > RZ_MAX_HIDDEN || V <= 0 || V > RZ_MAX_VOCAB)
    return RZ_ERR_INVALID_ARG;
  if (!norms || !d_lm_head || (n_rows > 0 && !d_hidden))
    return RZ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(d_hidden) |
       reinterpret_cast<uintptr_t>(d_lm_head)) & 15)
    return RZ_ERR_INVALID_ARG;
  if (n_rows * H > kMaxNormElems || (int64_t)V * H > kMaxNormElems)
    return RZ_ERR_INVALID_ARG;
  Carver meas{nullptr};
  const size_t need = carve_gn(meas, n_rows, H, V, nullptr);
  rz_status st = ws_check(workspace, workspace_bytes, need);
  if (st != RZ_OK) return st;
  Carver c{reinterpret_cast<char*>(workspace)};
  GnWs w;
  carve_gn(c, n_rows, H, V, &w);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  RZ_TRY(launch_grad_norm(d_hidden, n_rows * H, w.ph, norms, s));
  RZ_TRY(launch_grad_norm(d_lm_head, (int64_t)V * H, w.pw, norms + 1, s));
  return RZ_OK;
}

rz_status rz_dequantize_head(const uint8_t* codes, const uint8_t* scales,
                             int32_t V, int32_t H, rz_mx_format fmt,
                             void* lm_head, int32_t* err_flag, hipStream_t stream) {
  if (fmt != RZ_MX_FP4 && fmt != RZ_MX_FP8) return RZ_ERR_UNSUPPORTED;
  if (V <= 0 || V > RZ_MAX_VOCAB || H <= 0 || H > RZ_MAX_HIDDEN || H % 32)
    return RZ_ERR_INVALID_ARG;
  if (!codes || !scales || !lm_head) return RZ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(lm_head)) & 15)
    return RZ_ERR_INVALID_ARG;
  RZ_TRY(launch_mx_dequant(fmt == RZ_MX_FP4 ? 0 : 1, codes, scales,
                           (int64_t)V * (H / 32), lm_head, err_flag,
                           reinterpret_cast<hipStream_t>(stream)));
  return RZ_OK;
}

rz_status rz_response_diagnostics(const float* logpi, const float* logmu,
                                  const uint8_t* mask, const int32_t* cu_rows,
                                  int64_t n_rows, int32_t n_resp, float* d3,
                                  float* kl, int32_t* err_flag, hipStream_t stream) {
  if (n_rows < 0 || n_rows > RZ_MAX_ROWS) return RZ_ERR_INVALID_ARG;
  if (n_resp < 0 || n_resp > RZ_MAX_RESPONSES) return RZ_ERR_INVALID_ARG;
  if (n_resp == 0) return RZ_OK;
  if (!cu_rows || !d3 || !kl || (n_rows > 0 && (!logpi || !logmu)))
    return RZ_ERR_INVALID_ARG;
  RZ_TRY(launch_resp_diag(logpi, logmu, mask, cu_rows, n_resp, n_rows, d3, kl,
                          err_flag, reinterpret_cast<hipStream_t>(stream)));
  return RZ_OK;
}

// Host-side checks of the draw (n_rows = 0 is checked by the caller).
static rz_status sample_args_ok(const void* hidden, const void* lm_head,
                                const uint64_t* row_ids, int64_t n_rows,
                                int32_t H, int32_t V, rz_dtype dt,
                                const int32_t* tokens, const float* logmu) {
  if (n_rows < 0 || n_rows > RZ_MAX_ROWS) return RZ_ERR_INVALID_ARG;
  if (dt != RZ_DTYPE_F32 && dt != RZ_DTYPE_BF16) return RZ_ERR_UNSUPPORTED;
  if (H <= 0 || V <= 0) return RZ_ERR_INVALID_ARG;
  if (!dims_ok(H, V, dt)) return RZ_ERR_UNSUPPORTED;
  if (n_rows == 0) return RZ_OK;
  if (!hidden || !lm_head || !row_ids || !tokens || !logmu)
    return RZ_ERR_INVALID_ARG;
  if (misaligned(hidden, lm_head)) return RZ_ERR_INVALID_ARG;
  return RZ_OK;
}

// The draw's launch sequence over scratch carved by carve_smp from ws.
static rz_status sample_core(const void* hidden, const void* lm_head,
                             const uint64_t* row_ids, int64_t n_rows, int32_t H,
                             int32_t V, rz_dtype dt, uint64_t seed,
                             int32_t* tokens, float* logmu, float* lse,
                             char* ws, hipStream_t s) {
  Carver c{ws};
  SmpWs w;
  carve_smp(c, n_rows, V, &w);
  const int nt = (V + kVocabTile - 1) / kVocabTile;
  // the logits GEMM with the draw in its epilogue (the winning column's
  // logit comes along), then the draw's merge
  const PartLayout pl = part_layout(n_rows, nt);
  RZ_TRY(launch_fwd_sample(dt, hidden, n_rows, lm_head, H, V, row_ids, seed,
                           w.partials, w.cand, w.candz, pl.lt, pl.lr, s));
  // the draw's merge and the record (rz_token_logprobs' own lse fold)
  RZ_TRY(launch_draw_merge(w.cand, w.candz, w.partials, pl.lt, pl.lr, nt,
                           n_rows, V, tokens, logmu, lse, s));
  return RZ_OK;
}

rz_status rz_sample_tokens(const void* hidden, const void* lm_head,
                           const uint64_t* row_ids, int64_t n_rows, int32_t H,
                           int32_t V, rz_dtype dt, uint64_t seed,
                           int32_t* tokens, float* logmu, float* lse,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  rz_status st = sample_args_ok(hidden, lm_head, row_ids, n_rows, H, V, dt,
                                tokens, logmu);
  if (st != RZ_OK || n_rows == 0) return st;
  Carver meas{nullptr};
  const size_t need = carve_smp(meas, n_rows, V, nullptr);
  st = ws_check(workspace, workspace_bytes, need);
  if (st != RZ_OK) return st;
  return sample_core(hidden, lm_head, row_ids, n_rows, H, V, dt, seed, tokens,
                     logmu, lse, reinterpret_cast<char*>(workspace), stream);
}

rz_status rz_sample_tokens_noalloc(const void* hidden, const void* lm_head,
                                   const uint64_t* row_ids, int64_t n_rows,
                                   int32_t H, int32_t V, rz_dtype dt,
                                   uint64_t seed, int32_t* tokens, float* logmu,
                                   float* lse, hipStream_t stream) {
  rz_status st = sample_args_ok(hidden, lm_head, row_ids, n_rows, H, V, dt,
                                tokens, logmu);
  if (st != RZ_OK || n_rows == 0) return st;
  Carver meas{nullptr};
  if (carve_smp(meas, n_rows, V, nullptr) > kScratchBytes) return RZ_ERR_SCRATCH;
  char* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != RZ_OK) return st;
  return sample_core(hidden, lm_head, row_ids, n_rows, H, V, dt, seed, tokens,
                     logmu, lse, ws, stream);
}

rz_status rz_token_logprobs(const void* hidden, const void* lm_head,
                            const int32_t* tokens, int64_t n_rows, int32_t H,
                            int32_t V, rz_dtype dt, float* logprobs,
                            float* lse, int32_t* err_flag, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (n_rows < 0 || n_rows > RZ_MAX_ROWS) return RZ_ERR_INVALID_ARG;
  if (dt != RZ_DTYPE_F32 && dt != RZ_DTYPE_BF16) return RZ_ERR_UNSUPPORTED;
  if (H <= 0 || V <= 0) return RZ_ERR_INVALID_ARG;
  if (!dims_ok(H, V, dt)) return RZ_ERR_UNSUPPORTED;
  if (n_rows == 0) return RZ_OK;
  if (!hidden || !lm_head || !tokens || !logprobs) return RZ_ERR_INVALID_ARG;
  if (misaligned(hidden, lm_head)) return RZ_ERR_INVALID_ARG;
  Carver meas{nullptr};
  const size_t need = carve_tlp(meas, n_rows, V, nullptr);
  rz_status st = ws_check(workspace, workspace_bytes, need);
  if (st != RZ_OK) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Carver c{reinterpret_cast<char*>(workspace)};
  TlpWs w;
  carve_tlp(c, n_rows, V, &w);
  const int nt = (V + kVocabTile - 1) / kVocabTile;
  DevRows rows{nullptr, 0, (int)n_rows};
  const PartLayout pl = part_layout(n_rows, nt);
  RZ_TRY(launch_fwd_logits(dt, hidden, (int64_t)H * esize(dt), nullptr, rows,
                           lm_head, H, V, tokens, w.partials, pl.lt, pl.lr,
                           w.ztgt, nullptr, 0, 0, s));
  RZ_TRY(launch_lse_merge(w.partials, pl.lt, pl.lr, nt, rows, w.ztgt, tokens, V,
                          lse, logprobs, nullptr, nullptr, err_flag, nullptr,
                          nullptr, s));
  return RZ_OK;
}

rz_status rz_diagnostics(const float* logpi, const float* logmu,
                         const uint8_t* mask, int64_t n, float* diag,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (n < 0 || n > RZ_MAX_ROWS) return RZ_ERR_INVALID_ARG;
  if (!diag) return RZ_ERR_INVALID_ARG;
  if (n > 0 && (!logpi || !logmu)) return RZ_ERR_INVALID_ARG;
  const size_t need = align_up(diag_partials_bytes(n));
  rz_status st = ws_check(workspace, workspace_bytes, need);
  if (st != RZ_OK) return st;
  RZ_TRY(launch_diagnostics(logpi, logmu, mask, n, workspace, diag,
                            reinterpret_cast<hipStream_t>(stream)));
  return RZ_OK;
}

// The learner step over hidden [n_rows, H] and head [V, H] (H is the GEMM
// width and the row stride of both; d_hidden is [n_rows, H]); the head's
// gradient is taken for columns [dw_col0, dw_col0 + dw_cols) only and
// written as [V, dw_cols].  The workspace is carve_fb(..., dw_cols) and has
// been checked by the caller.
static rz_status fwd_bwd_core(
    const void* hidden, const void* lm_head, const int32_t* tokens,
    const float* logmu, const uint8_t* mask, const int32_t* cu_rows,
    const float* rewards, const int32_t* group_ids, int64_t n_rows,
    int32_t n_resp, int32_t H, int32_t V, rz_dtype dt, int32_t dw_col0,
    int32_t dw_cols, int sc, float* logprobs, float* loss, float* d_hidden,
    float* d_lm_head, float* diag, float* adv, int32_t* err_flag,
    void* workspace, hipStream_t stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Carver c{reinterpret_cast<char*>(workspace)};
  FbWs w;
  carve_fb(c, n_rows, n_resp, H, V, dt, &w, dw_cols);
  const int64_t N = n_rows;
  const int nt = (V + kVocabTile - 1) / kVocabTile;
  const int Vpad = (int)round_up(V, 64);
  const int C = chunk_rows(N);
  const size_t es = esize(dt);
  const int64_t lda = (int64_t)H * es;

  // a0: valid-row list (device count), cu_rows validation
  RZ_TRY(launch_mask_compact(mask, N, tokens, cu_rows, n_resp, w.blk,
                             w.nvalid, w.bad_cu, w.idx, w.tokv, w.respv,
                             err_flag, s));
  // a5 (inputs only): T_i, group means, A_i and the factors A_i / (B T_i)
  RZ_TRY(launch_advantages(mask, N, cu_rows, rewards, group_ids, n_resp,
                           w.bad_cu, w.T, w.gcnt, w.gsum, w.Ad, w.fcoef, adv,
                           w.bad_gid, w.sort_ws, err_flag, s));
  RZ_TRY(launch_transpose(dt, K_TRANSPOSE_W, lm_head, H, nullptr,
                          DevRows{nullptr, 0, V}, Vpad, H, w.WT, Vpad, nullptr,
                          nullptr, nullptr, s));
  // a1-a4, a7-a9 in chunks of C valid rows (the count lives on the device;
  // chunks past it do no work):
  //   logits GEMM + log-softmax epilogue, also storing e (bf16:
  //   exp(z - r ln 2), the backward's A operand; fp32: exp(z - m_j));
  //   ordered merge -> lse, log pi; c_t;
  //   bf16: g_t and the chunk's scale, flagged rows rebased, h^T scaled by
  //   c_t g_t 2^sigma; fp32: dz = c_t e^(m_j - lse) e and dz^T;
  //   dHidden GEMM; dW GEMM accumulated over chunks in order.
  const bool b16 = dt == RZ_DTYPE_BF16;
  const int64_t nchunks = N > 0 ? (N + C - 1) / C : 1;
  for (int64_t k = 0; k < nchunks; ++k) {
    DevRows crow{w.nvalid, k * C, C};
    if (N > 0) {
      RZ_TRY(launch_fwd_logits(dt, hidden, lda, w.idx, crow, lm_head, H, V,
                               w.tokv, w.partials, N, 1, w.ztgt, w.dz, Vpad,
                               Vpad, s));
      RZ_TRY(launch_lse_merge(w.partials, N, 1, nt, crow, w.ztgt, w.tokv, V,
                              w.lse_v, w.logpi_v, w.idx, logprobs, err_flag,
                              b16 ? w.eref : nullptr, w.eflag, s));
      RZ_TRY(launch_coef(crow, w.logpi_v, logmu, w.idx, w.respv, w.fcoef, sc,
                         w.coef, w.coef1, w.lse_v, b16 ? w.eref : nullptr,
                         w.gsc, w.fexp_part, w.sigma, s));
      if (b16) {
        RZ_TRY(launch_erebase(w.dz, Vpad, crow, w.partials, N, nt, w.eref,
                              w.eflag, Vpad, s));
      } else {
        RZ_TRY(launch_dz_scale((float*)w.dz, Vpad, (float*)w.dzT, C, crow,
                               w.partials, N, w.lse_v, w.coef, w.tokv, Vpad, s));
      }
      RZ_TRY(launch_transpose(dt, K_TRANSPOSE_H,
                              (const char*)hidden + (size_t)dw_col0 * es, H,
                              w.idx, crow, C, dw_cols, w.hT, C,
                              b16 ? w.coef : nullptr, w.gsc, w.sigma, s));
      RZ_TRY(launch_bwd_dh(dt, w.dz, Vpad, crow, w.WT, Vpad, H, V, Vpad,
                           w.idx, w.tokv, w.coef1, b16 ? w.coef : nullptr,
                           w.gsc, lm_head, d_hidden, w.dwpart, s));
    }
    RZ_TRY(launch_bwd_dw(dt, b16 ? w.dz : w.dzT, b16 ? Vpad : C,
                         N > 0 ? crow : DevRows{nullptr, 0, 0}, w.hT, C,
                         dw_cols, V, Vpad, d_lm_head, k == 0, w.dwpart,
                         N > 0 ? w.sigma : nullptr, s));
  }
  if (N > 0) RZ_TRY(launch_rows_finalize(mask, N, H, logprobs, d_hidden, s));
  // a5: S_i from this call's logprobs, then L
  RZ_TRY(launch_loss_value(mask, logprobs, logmu, N, cu_rows, n_resp, sc, w.T,
                           w.Ad, w.S, loss, s));
  // a6: diagnostics over this call's outputs (same kernels as rz_diagnostics;
  // score centering without recorded log mu has none)
  if (logmu || N == 0)
    RZ_TRY(launch_diagnostics(logprobs, logmu, mask, N, w.diag_part,
                              diag ? diag : w.diag_tmp, s));
  // a9: exact one-hot part of dW
  RZ_TRY(launch_dw_fix(dt, w.nvalid, N, w.tokv, w.idx, w.coef1,
                       (const char*)hidden + (size_t)dw_col0 * es, H, dw_cols,
                       V, w.sort_ws, w.fix_cont, d_lm_head, s));
  return RZ_OK;
}

// Host-side checks shared by the learner entry points (logmu required
// unless need_logmu is false).
static rz_status fb_args_ok(const void* hidden, const void* lm_head,
                            const int32_t* tokens, const float* logmu,
                            bool need_logmu, const uint8_t* mask,
                            const int32_t* cu_rows, const float* rewards,
                            const int32_t* group_ids, int64_t n_rows,
                            int32_t n_resp, int32_t H, int32_t V, rz_dtype dt,
                            const float* logprobs, const float* loss,
                            const float* d_hidden, const float* d_lm_head) {
  if (n_rows < 0 || n_rows > RZ_MAX_ROWS) return RZ_ERR_INVALID_ARG;
  if (n_resp < 1 || n_resp > RZ_MAX_RESPONSES) return RZ_ERR_INVALID_ARG;
  if (dt != RZ_DTYPE_F32 && dt != RZ_DTYPE_BF16) return RZ_ERR_UNSUPPORTED;
  if (H <= 0 || V <= 0) return RZ_ERR_INVALID_ARG;
  if (!dims_ok(H, V, dt)) return RZ_ERR_UNSUPPORTED;
  if (!lm_head || !cu_rows || !rewards || !group_ids || !loss || !d_lm_head)
    return RZ_ERR_INVALID_ARG;
  if (n_rows > 0 && (!hidden || !tokens || (need_logmu && !logmu) || !mask ||
                     !logprobs || !d_hidden))
    return RZ_ERR_INVALID_ARG;
  if (misaligned(hidden, lm_head, d_hidden, d_lm_head)) return RZ_ERR_INVALID_ARG;
  return RZ_OK;
}

rz_status rz_reinforce_zero_fwd_bwd(
    const void* hidden, const void* lm_head, const int32_t* tokens,
    const float* logmu, const uint8_t* mask, const int32_t* cu_rows,
    const float* rewards, const int32_t* group_ids, int64_t n_rows,
    int32_t n_resp, int32_t H, int32_t V, rz_dtype dt, float* logprobs,
    float* loss, float* d_hidden, float* d_lm_head, float* diag, float* adv,
    int32_t* err_flag, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  rz_status st = fb_args_ok(hidden, lm_head, tokens, logmu, true, mask, cu_rows,
                            rewards, group_ids, n_rows, n_resp, H, V, dt,
                            logprobs, loss, d_hidden, d_lm_head);
  if (st != RZ_OK) return st;
  Carver meas{nullptr};
  const size_t need = carve_fb(meas, n_rows, n_resp, H, V, dt, nullptr, -1);
  st = ws_check(workspace, workspace_bytes, need);
  if (st != RZ_OK) return st;

  return fwd_bwd_core(hidden, lm_head, tokens, logmu, mask, cu_rows, rewards,
                      group_ids, n_rows, n_resp, H, V, dt, 0, H, 0, logprobs,
                      loss, d_hidden, d_lm_head, diag, adv, err_flag,
                      workspace, stream);
}

rz_status rz_score_centering_fwd_bwd(
    const void* hidden, const void* lm_head, const int32_t* tokens,
    const float* logmu, const uint8_t* mask, const int32_t* cu_rows,
    const float* rewards, const int32_t* group_ids, int64_t n_rows,
    int32_t n_resp, int32_t H, int32_t V, rz_dtype dt, float* logprobs,
    float* loss, float* d_hidden, float* d_lm_head, float* diag, float* adv,
    int32_t* err_flag, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  rz_status st = fb_args_ok(hidden, lm_head, tokens, logmu, false, mask,
                            cu_rows, rewards, group_ids, n_rows, n_resp, H, V,
                            dt, logprobs, loss, d_hidden, d_lm_head);
  if (st != RZ_OK) return st;
  if (diag && !logmu && n_rows > 0) return RZ_ERR_INVALID_ARG;
  Carver meas{nullptr};
  const size_t need = carve_fb(meas, n_rows, n_resp, H, V, dt, nullptr, -1);
  st = ws_check(workspace, workspace_bytes, need);
  if (st != RZ_OK) return st;
  return fwd_bwd_core(hidden, lm_head, tokens, logmu, mask, cu_rows, rewards,
                      group_ids, n_rows, n_resp, H, V, dt, 0, H, 1, logprobs,
                      loss, d_hidden, d_lm_head, diag, adv, err_flag,
                      workspace, stream);
}


rz_status rz_run_summary(const float* d3, const float* kl,
                         const float* grad_norm, int64_t n_steps,
                         int32_t window, double* out) {
  if (!out || n_steps < 0 || window < 1) return RZ_ERR_INVALID_ARG;
  const double qnan = NAN;
  // median of x[lo, hi), the mean of the two middle values for an even count;
  // NaN when the range is empty or holds a NaN
  auto median = [&](const float* x, int64_t lo, int64_t hi) {
    if (!x || hi <= lo) return qnan;
    std::vector<double> v(x + lo, x + hi);
    for (double e : v)
      if (e != e) return qnan;
    const size_t m = v.size() / 2;
    std::nth_element(v.begin(), v.begin() + m, v.end());
    const double upper = v[m];
    if (v.size() % 2) return upper;
    const double lower = *std::max_element(v.begin(), v.begin() + m);
    return 0.5 * (lower + upper);
  };
  auto maximum = [&](const float* x) {
    if (!x || n_steps == 0) return qnan;
    double m = -INFINITY;
    for (int64_t i = 0; i < n_steps; ++i) {
      if (x[i] != x[i]) return qnan;
      m = std::max(m, (double)x[i]);
    }
    return m;
  };
  const int64_t w = std::min<int64_t>(window, n_steps);
  out[0] = maximum(d3);
  out[1] = median(d3, 0, n_steps);
  out[2] = out[0] / out[1];
  out[3] = median(kl, 0, w);
  out[4] = median(kl, n_steps - w, n_steps);
  out[5] = out[4] / out[3];
  out[6] = maximum(grad_norm);
  return RZ_OK;
}

static rz_status mx_args_ok(const void* hidden, const uint8_t* codes,
                            const uint8_t* scales, rz_mx_format fmt,
                            int64_t n_rows, int32_t H, int32_t V) {
  if (fmt != RZ_MX_FP4 && fmt != RZ_MX_FP8) return RZ_ERR_UNSUPPORTED;
  if (n_rows < 0 || n_rows > RZ_MAX_ROWS) return RZ_ERR_INVALID_ARG;
  if (H <= 0 || V <= 0) return RZ_ERR_INVALID_ARG;
  if (!dims_ok(H, V, RZ_DTYPE_BF16)) return RZ_ERR_UNSUPPORTED;
  if (n_rows > 0 && (!hidden || !codes || !scales)) return RZ_ERR_INVALID_ARG;
  if (misaligned(codes, scales, hidden)) return RZ_ERR_INVALID_ARG;
  return RZ_OK;
}

rz_status rz_token_logprobs_mx(const void* hidden, const uint8_t* codes,
                               const uint8_t* scales, rz_mx_format fmt,
                               const int32_t* tokens, int64_t n_rows, int32_t H,
                               int32_t V, float* logprobs, float* lse,
                               int32_t* err_flag, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  rz_status st = mx_args_ok(hidden, codes, scales, fmt, n_rows, H, V);
  if (st != RZ_OK) return st;
  if (n_rows == 0) return RZ_OK;
  if (!tokens || !logprobs) return RZ_ERR_INVALID_ARG;
  const bool fused = mx_fused(n_rows, H, false);
  Carver meas{nullptr};
  const size_t need = carve_tlp(meas, n_rows, V, nullptr) +
                      (fused ? 0 : align_up(2 * (size_t)V * (size_t)H));
  st = ws_check(workspace, workspace_bytes, need);
  if (st != RZ_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Carver c{reinterpret_cast<char*>(workspace)};
  TlpWs w;
  carve_tlp(c, n_rows, V, &w);
  const int nt = (V + kVocabTile - 1) / kVocabTile;
  DevRows rows{nullptr, 0, (int)n_rows};
  const PartLayout pl = part_layout(n_rows, nt);
  if (fused) {
    RZ_TRY(launch_fwd_mx(fmt, hidden, n_rows, codes, scales, H, V, tokens,
                         w.partials, pl.lt, pl.lr, w.ztgt, nullptr, 0, nullptr,
                         nullptr, err_flag, s));
  } else {
    void* Wb = c.take<char>(2 * (size_t)V * (size_t)H);
    RZ_TRY(launch_mx_dequant(fmt, codes, scales, (int64_t)V * (H / 32), Wb,
                             err_flag, s));
    RZ_TRY(launch_fwd_logits(RZ_DTYPE_BF16, hidden, (int64_t)H * 2, nullptr,
                             rows, Wb, H, V, tokens, w.partials, pl.lt, pl.lr,
                             w.ztgt, nullptr, 0, 0, s));
  }
  RZ_TRY(launch_lse_merge(w.partials, pl.lt, pl.lr, nt, rows, w.ztgt, tokens, V,
                          lse, logprobs, nullptr, nullptr, err_flag, nullptr,
                          nullptr, s));
  return RZ_OK;
}

rz_status rz_sample_tokens_mx(const void* hidden, const uint8_t* codes,
                              const uint8_t* scales, rz_mx_format fmt,
                              const uint64_t* row_ids, int64_t n_rows,
                              int32_t H, int32_t V, uint64_t seed,
                              int32_t* tokens, float* logmu, float* lse,
                              int32_t* err_flag, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  rz_status st = mx_args_ok(hidden, codes, scales, fmt, n_rows, H, V);
  if (st != RZ_OK) return st;
  if (n_rows == 0) return RZ_OK;
  if (!row_ids || !tokens || !logmu) return RZ_ERR_INVALID_ARG;
  const bool fused = mx_fused(n_rows, H, true);
  Carver meas{nullptr};
  const size_t need = carve_smp(meas, n_rows, V, nullptr) +
                      (fused ? 0 : align_up(2 * (size_t)V * (size_t)H));
  st = ws_check(workspace, workspace_bytes, need);
  if (st != RZ_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  Carver c{reinterpret_cast<char*>(workspace)};
  SmpWs w;
  carve_smp(c, n_rows, V, &w);
  const int nt = (V + kVocabTile - 1) / kVocabTile;
  const PartLayout pl = part_layout(n_rows, nt);
  if (fused) {
    RZ_TRY(launch_fwd_mx(fmt, hidden, n_rows, codes, scales, H, V, nullptr,
                         w.partials, pl.lt, pl.lr, nullptr, row_ids, seed, w.cand,
                         w.candz, err_flag, s));
  } else {
    void* Wb = c.take<char>(2 * (size_t)V * (size_t)H);
    RZ_TRY(launch_mx_dequant(fmt, codes, scales, (int64_t)V * (H / 32), Wb,
                             err_flag, s));
    RZ_TRY(launch_fwd_sample(RZ_DTYPE_BF16, hidden, n_rows, Wb, H, V, row_ids,
                             seed, w.partials, w.cand, w.candz, pl.lt, pl.lr, s));
  }
  RZ_TRY(launch_draw_merge(w.cand, w.candz, w.partials, pl.lt, pl.lr, nt,
                           n_rows, V, tokens, logmu, lse, s));
  return RZ_OK;
}

rz_status rz_lora_augment(const void* hidden, const void* lora_A, float scale,
                          int64_t n_rows, int32_t H, int32_t r, rz_dtype dt,
                          void* hidden_aug, hipStream_t stream) {
  if (dt != RZ_DTYPE_F32 && dt != RZ_DTYPE_BF16) return RZ_ERR_UNSUPPORTED;
  if (n_rows < 0 || n_rows > RZ_MAX_ROWS) return RZ_ERR_INVALID_ARG;
  if (r < 1 || r > kLoraCols) return RZ_ERR_INVALID_ARG;
  if (!dims_ok(H, 1, dt) || H + kLoraCols > RZ_MAX_HIDDEN) return RZ_ERR_UNSUPPORTED;
  if (n_rows == 0) return RZ_OK;
  if (!hidden || !lora_A || !hidden_aug) return RZ_ERR_INVALID_ARG;
  if (misaligned(hidden, lora_A)) return RZ_ERR_INVALID_ARG;
  RZ_TRY(launch_lora_u(dt, hidden, lora_A, scale, n_rows, H, r, hidden_aug,
                       reinterpret_cast<hipStream_t>(stream)));
  return RZ_OK;
}

rz_status rz_lora_merge_head(const void* lm_head, const void* lora_B, int32_t V,
                             int32_t H, int32_t r, rz_dtype dt, void* head_aug,
                             hipStream_t stream) {
  if (dt != RZ_DTYPE_F32 && dt != RZ_DTYPE_BF16) return RZ_ERR_UNSUPPORTED;
  if (r < 1 || r > kLoraCols) return RZ_ERR_INVALID_ARG;
  if (!dims_ok(H, V, dt) || H + kLoraCols > RZ_MAX_HIDDEN) return RZ_ERR_UNSUPPORTED;
  if (!lm_head || !lora_B || !head_aug) return RZ_ERR_INVALID_ARG;
  RZ_TRY(launch_lora_head(dt, lm_head, lora_B, V, H, r, head_aug,
                          reinterpret_cast<hipStream_t>(stream)));
  return RZ_OK;
}

rz_status rz_reinforce_zero_fwd_bwd_lora(
    const void* hidden, const void* lm_head, const void* lora_A,
    const void* lora_B, float scale, int32_t r, const int32_t* tokens,
    const float* logmu, const uint8_t* mask, const int32_t* cu_rows,
    const float* rewards, const int32_t* group_ids, int64_t n_rows,
    int32_t n_resp, int32_t H, int32_t V, rz_dtype dt, float* logprobs,
    float* loss, float* d_hidden, float* d_lora_A, float* d_lora_B,
    float* diag, float* adv, int32_t* err_flag, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (n_rows < 0 || n_rows > RZ_MAX_ROWS) return RZ_ERR_INVALID_ARG;
  if (n_resp < 1 || n_resp > RZ_MAX_RESPONSES) return RZ_ERR_INVALID_ARG;
  if (dt != RZ_DTYPE_F32 && dt != RZ_DTYPE_BF16) return RZ_ERR_UNSUPPORTED;
  if (H <= 0 || V <= 0 || r < 1 || r > kLoraCols) return RZ_ERR_INVALID_ARG;
  if (!dims_ok(H, V, dt) || H + kLoraCols > RZ_MAX_HIDDEN) return RZ_ERR_UNSUPPORTED;
  if (!lm_head || !lora_A || !lora_B || !cu_rows || !rewards || !group_ids ||
      !loss || !d_lora_A || !d_lora_B)
    return RZ_ERR_INVALID_ARG;
  if (n_rows > 0 && (!hidden || !tokens || !logmu || !mask || !logprobs ||
                     !d_hidden))
    return RZ_ERR_INVALID_ARG;
  if (misaligned(hidden, lm_head, lora_A, d_hidden)) return RZ_ERR_INVALID_ARG;
  Carver meas{nullptr};
  const size_t need = carve_lora(meas, n_rows, n_resp, H, V, dt, nullptr);
  rz_status st = ws_check(workspace, workspace_bytes, need);
  if (st != RZ_OK) return st;
  Carver c{reinterpret_cast<char*>(workspace)};
  LoraWs w;
  carve_lora(c, n_rows, n_resp, H, V, dt, &w);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int32_t Ha = H + kLoraCols;
  // [h | u] and [W | B]: the learner then runs on the same kernels as the
  // rollout's rz_token_logprobs / rz_sample_tokens over these operands
  if (n_rows > 0)
    RZ_TRY(launch_lora_u(dt, hidden, lora_A, scale, n_rows, H, r, w.h_aug, s));
  RZ_TRY(launch_lora_head(dt, lm_head, lora_B, V, H, r, w.head_aug, s));
  // the step over the augmented operands; the head's gradient only for the
  // adapter's columns (W is frozen): dL/dB
  rz_status core = fwd_bwd_core(w.h_aug, w.head_aug, tokens, logmu, mask,
                                cu_rows, rewards, group_ids, n_rows, n_resp,
                                Ha, V, dt, H, kLoraCols, 0, logprobs, loss,
                                w.dh_aug, w.dB, diag, adv, err_flag, w.core,
                                stream);
  if (core != RZ_OK) return core;
  // chain rule through u: dL/dh and dL/dA; dL/dB without the padding
  RZ_TRY(launch_lora_grads(dt, w.dh_aug, n_rows, H, hidden, lora_A, r, scale,
                           w.part, d_hidden, d_lora_A, s));
  RZ_TRY(hipMemcpy2DAsync(d_lora_B, (size_t)r * sizeof(float), w.dB,
                          kLoraCols * sizeof(float), (size_t)r * sizeof(float),
                          (size_t)V, hipMemcpyDeviceToDevice, s));
  return RZ_OK;
}

rz_status rz_timing_enable(int on) {
  if (on) {
    g_timer.on = true;
    return RZ_OK;
  }
  g_timer.on = false;
  for (auto& p : g_timer.pending) {
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
  }
  g_timer.pending.clear();
  for (auto e : g_timer.pool) (void)hipEventDestroy(e);
  g_timer.pool.clear();
  return RZ_OK;
}

int rz_timing_num_kernels(void) { return K_NUM_KERNELS; }

const char* rz_timing_kernel_name(int k) { return kernel_name(k); }

rz_status rz_timing_read(double* total_ms, int64_t* launches, int reset) {
  for (auto& p : g_timer.pending) {
    if (hipEventSynchronize(p.b) != hipSuccess) return RZ_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) return RZ_ERR_HIP;
    g_timer.total[p.k] += ms;
    g_timer.count[p.k] += 1;
    g_timer.pool.push_back(p.a);
    g_timer.pool.push_back(p.b);
  }
  g_timer.pending.clear();
  for (int k = 0; k < K_NUM_KERNELS; ++k) {
    if (total_ms) total_ms[k] = g_timer.total[k];
    if (launches) launches[k] = g_timer.count[k];
    if (reset) {
      g_timer.total[k] = 0.0;
      g_timer.count[k] = 0;
    }
  }
  return RZ_OK;
}

}  // extern "C"
