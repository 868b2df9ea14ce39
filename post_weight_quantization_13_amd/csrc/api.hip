// extern "C" entry points of libgptq: argument checks, workspace sizing and
// the launch sequence of each call.  Declarations and contracts: include/gptq.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/gptq.h"

namespace gptq {
hipError_t launch_hessian(double* H, int64_t n, const void* X, int dt, int64_t tokens, int64_t ldx, double alpha,
                          double beta, void* ws, hipStream_t s);
size_t hessian_workspace(int64_t n, int64_t tokens, int dt);
int64_t hessian_chain_tokens();
size_t prepare_workspace(int64_t n);
hipError_t launch_prepare(const double* H, int64_t n, double damp, int desc_act, float* U, int32_t* perm,
                          uint8_t* dead, void* ws, hipStream_t s, int* info_host, int32_t* info_dev);
size_t quantize_workspace(int64_t rows, int64_t n);
hipError_t launch_quantize(const float* U, const int32_t* perm, const uint8_t* dead, int64_t n, int bits, int sym,
                           int group_size, const void* W, int wdt, int64_t rows, int64_t ldw, int32_t* qweight,
                           uint16_t* scales, uint16_t* zeros, int32_t* g_idx, double* loss_host,
                           double* loss_dev, void* ws, hipStream_t s);
hipError_t zero_loss(double* loss, hipStream_t s);
size_t loss_workspace(int64_t rows, int64_t n);
hipError_t launch_layer_loss(const double* H, int64_t n, const void* W, int wdt, int64_t rows, int64_t ldw,
                             const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                             const int32_t* g_idx, int bits, double* rel_host, void* ws, hipStream_t s);
size_t matmul_packed_bytes(int64_t rows, int64_t n, int bits, int group_size);
bool matmul_fits(int64_t n, int group_size);
hipError_t launch_matmul_pack(const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                              const int32_t* g_idx, int64_t rows, int64_t n, int bits, int group_size,
                              void* packed, int32_t* col_order, uint32_t* flags_host, hipStream_t s);
size_t matmul_workspace_bytes(int64_t M, int64_t n);
hipError_t launch_matmul(const void* A, int64_t M, int64_t lda, const void* packed, const int32_t* col_order,
                         int64_t rows, int64_t n, int bits, int group_size, void* Y, int ydt, int64_t ldy,
                         void* ws, hipStream_t s);
size_t matmul_static_scratch_bytes();
hipError_t matmul_static_scratch(void** ptr);
int attention_head_dim();
hipError_t launch_rmsnorm(const void* X, int dt, int64_t ldx, const float* R, int64_t T, int64_t d, double eps,
                          float* hout, uint16_t* Y, hipStream_t s);
hipError_t launch_rope(float* Q, float* K, int64_t T, int64_t d, int64_t hd, int64_t L, double base, hipStream_t s);
hipError_t launch_attention(const float* Q, const float* K, const float* V, int64_t T, int64_t d, int64_t L,
                            uint16_t* O, hipStream_t s);
hipError_t launch_silu_mul(const float* G, const float* U, int64_t count, uint16_t* Y, hipStream_t s);
}  // namespace gptq

namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxDim = 65535 * 32;  // keeps every grid dimension in range

gptq_status fail(gptq_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gptq_status fail(gptq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gptq_status ok() {
  g_last_error.clear();
  return GPTQ_OK;
}

gptq_status hip_fail(const char* where, hipError_t e) {
  return fail(GPTQ_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool valid_dtype(int dt) { return dt == GPTQ_BF16 || dt == GPTQ_FP16 || dt == GPTQ_FP32; }

gptq_status check_config(const gptq_config* cfg, bool for_quantize) {
  if (!cfg) return fail(GPTQ_ERR_INVALID_ARG, "cfg is NULL");
  if (!(cfg->damp_percent >= 0.0f) || !std::isfinite(cfg->damp_percent))
    return fail(GPTQ_ERR_INVALID_ARG, "damp_percent must be finite and >= 0 (got %g)", cfg->damp_percent);
  if (cfg->desc_act != 0 && cfg->desc_act != 1) return fail(GPTQ_ERR_INVALID_ARG, "desc_act must be 0 or 1");
  if (!for_quantize) return GPTQ_OK;
  if (cfg->sym < 0 || cfg->sym > 2) return fail(GPTQ_ERR_INVALID_ARG, "sym must be 0, 1 or 2");
  if (cfg->bits != 2 && cfg->bits != 3 && cfg->bits != 4 && cfg->bits != 8)
    return fail(GPTQ_ERR_UNSUPPORTED, "bits=%d (supported: 2, 3, 4, 8)", cfg->bits);
  if (cfg->group_size != 32 && cfg->group_size != 64 && cfg->group_size != 128 && cfg->group_size != -1)
    return fail(GPTQ_ERR_UNSUPPORTED, "group_size=%d (supported: 32, 64, 128, -1)", cfg->group_size);
  if (cfg->block_size != 128)
    return fail(GPTQ_ERR_UNSUPPORTED, "block_size=%d (supported: 128)", cfg->block_size);
  return GPTQ_OK;
}

// Shape and format checks shared by the matmul pack and the matmul.
gptq_status check_matmul_format(int64_t rows, int64_t n, int32_t bits, int32_t group_size) {
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_ERR_UNSUPPORTED, "bits=%d (supported: 2, 3, 4, 8)", bits);
  if (group_size != 32 && group_size != 64 && group_size != 128 && group_size != -1)
    return fail(GPTQ_ERR_UNSUPPORTED, "group_size=%d (supported: 32, 64, 128, -1)", group_size);
  if (n < 128 || n > kMaxDim || n % 128 != 0)
    return fail(GPTQ_ERR_UNSUPPORTED, "n=%lld must be a positive multiple of 128 up to %lld", (long long)n,
                (long long)kMaxDim);
  if (rows < 1 || rows > (int64_t)1 << 30) return fail(GPTQ_ERR_INVALID_ARG, "rows=%lld out of range", (long long)rows);
  if (!gptq::matmul_fits(n, group_size))
    return fail(GPTQ_ERR_UNSUPPORTED, "n=%lld has too many groups of %d for the matmul (at most 1528)", (long long)n,
                group_size);
  return GPTQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Checks shared by gptq_matmul and gptq_matmul_static (everything but the workspace).
gptq_status check_matmul_call(const void* A, gptq_dtype adt, int64_t M, int64_t lda, const void* packed,
                              const int32_t* col_order, int64_t rows, int64_t n, int32_t bits, int32_t group_size,
                              const void* Y, gptq_dtype ydt, int64_t ldy) {
  gptq_status st = check_matmul_format(rows, n, bits, group_size);
  if (st != GPTQ_OK) return st;
  if (adt != GPTQ_FP16) return fail(GPTQ_ERR_UNSUPPORTED, "activations must be fp16 (got dtype %d)", (int)adt);
  if (ydt != GPTQ_FP16 && ydt != GPTQ_FP32)
    return fail(GPTQ_ERR_UNSUPPORTED, "output must be fp16 or fp32 (got dtype %d)", (int)ydt);
  if (M < 0 || M > (int64_t)65535 * 16) return fail(GPTQ_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
  if (M == 0) return GPTQ_OK;
  if (!A || !packed || !Y) return fail(GPTQ_ERR_INVALID_ARG, "NULL pointer argument");
  if (lda < n || ldy < rows)
    return fail(GPTQ_ERR_INVALID_ARG, "lda=%lld < n or ldy=%lld < rows", (long long)lda, (long long)ldy);
  if (!aligned16(packed)) return fail(GPTQ_ERR_INVALID_ARG, "packed must be 16-byte aligned");
  if (!col_order && (!aligned16(A) || lda % 8 != 0))
    return fail(GPTQ_ERR_INVALID_ARG, "A must be 16-byte aligned with lda a multiple of 8");
  return GPTQ_OK;
}

}  // namespace

extern "C" {

const char* gptq_last_error(void) { return g_last_error.c_str(); }

const char* gptq_version(void) { return "gptq-gfx950 0.1.0"; }

// ----------------------------------------------------------------------------- Hessian
size_t gptq_hessian_workspace_bytes(int64_t n, int64_t tokens, gptq_dtype xdt) {
  if (n < 1 || n > kMaxDim || tokens < 1 || !valid_dtype(xdt)) return 0;
  return gptq::hessian_workspace(n, tokens, static_cast<int>(xdt));
}

int64_t gptq_hessian_chain_tokens(void) { return gptq::hessian_chain_tokens(); }

gptq_status gptq_hessian_accumulate(double* H, int64_t n, int64_t* n_tokens, const void* X, gptq_dtype xdt,
                                    int64_t tokens, int64_t ldx, void* workspace, size_t ws_bytes,
                                    void* stream) {
  if (!H) return fail(GPTQ_ERR_INVALID_ARG, "H is NULL");
  if (!n_tokens) return fail(GPTQ_ERR_INVALID_ARG, "n_tokens is NULL");
  if (n < 1 || n > kMaxDim) return fail(GPTQ_ERR_INVALID_ARG, "n=%lld out of range", (long long)n);
  if (*n_tokens < 0) return fail(GPTQ_ERR_INVALID_ARG, "*n_tokens=%lld < 0", (long long)*n_tokens);
  if (tokens < 0) return fail(GPTQ_ERR_INVALID_ARG, "tokens=%lld < 0", (long long)tokens);
  if (!valid_dtype(xdt)) return fail(GPTQ_ERR_INVALID_ARG, "unknown dtype %d", (int)xdt);
  if (tokens == 0) return ok();
  if (!X) return fail(GPTQ_ERR_INVALID_ARG, "X is NULL");
  if (ldx < n) return fail(GPTQ_ERR_INVALID_ARG, "ldx=%lld < n=%lld", (long long)ldx, (long long)n);
  const size_t need = gptq::hessian_workspace(n, tokens, static_cast<int>(xdt));
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace ? ws_bytes : 0, need);
  const int64_t n_old = *n_tokens;
  const int64_t n_new = n_old + tokens;
  const double alpha = 2.0 / static_cast<double>(n_new);
  const double beta = static_cast<double>(n_old) / static_cast<double>(n_new);
  hipError_t e = gptq::launch_hessian(H, n, X, static_cast<int>(xdt), tokens, ldx, alpha, beta, workspace,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gptq_hessian_accumulate", e);
  *n_tokens = n_new;
  return ok();
}

// ----------------------------------------------------------------------------- prepare
size_t gptq_prepare_workspace_bytes(int64_t n, const gptq_config* cfg) {
  (void)cfg;
  if (n < 1 || n > 65535) return 0;  // the sizes gptq_prepare_hinv accepts
  return gptq::prepare_workspace(n);
}

static gptq_status check_prepare(const double* H, int64_t n, const gptq_config* cfg, const float* U,
                                 const int32_t* perm, const uint8_t* dead, const void* workspace, size_t ws_bytes) {
  gptq_status st = check_config(cfg, false);
  if (st != GPTQ_OK) return st;
  if (!H || !U || !perm || !dead) return fail(GPTQ_ERR_INVALID_ARG, "NULL H, U, perm or dead");
  if (n < 1 || n > 65535) return fail(GPTQ_ERR_INVALID_ARG, "n=%lld out of range [1, 65535]", (long long)n);
  const size_t need = gptq::prepare_workspace(n);
  if (!workspace || ws_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace ? ws_bytes : 0, need);
  return GPTQ_OK;
}

gptq_status gptq_prepare_hinv(const double* H, int64_t n, const gptq_config* cfg, float* U, int32_t* perm,
                              uint8_t* dead, void* workspace, size_t ws_bytes, void* stream) {
  gptq_status st = check_prepare(H, n, cfg, U, perm, dead, workspace, ws_bytes);
  if (st != GPTQ_OK) return st;
  int info = 0;
  hipError_t e = gptq::launch_prepare(H, n, static_cast<double>(cfg->damp_percent), cfg->desc_act, U, perm, dead,
                                      workspace, static_cast<hipStream_t>(stream), &info, nullptr);
  if (e != hipSuccess) return hip_fail("gptq_prepare_hinv", e);
  if (info != 0) return fail(GPTQ_ERR_NOT_PD, "damped Hessian is not positive definite");
  return ok();
}

gptq_status gptq_prepare_hinv_async(const double* H, int64_t n, const gptq_config* cfg, float* U, int32_t* perm,
                                    uint8_t* dead, int32_t* info, void* workspace, size_t ws_bytes, void* stream) {
  gptq_status st = check_prepare(H, n, cfg, U, perm, dead, workspace, ws_bytes);
  if (st != GPTQ_OK) return st;
  if (!info) return fail(GPTQ_ERR_INVALID_ARG, "NULL info");
  hipError_t e = gptq::launch_prepare(H, n, static_cast<double>(cfg->damp_percent), cfg->desc_act, U, perm, dead,
                                      workspace, static_cast<hipStream_t>(stream), nullptr, info);
  if (e != hipSuccess) return hip_fail("gptq_prepare_hinv_async", e);
  return ok();
}

// ----------------------------------------------------------------------------- quantize
size_t gptq_quantize_workspace_bytes(int64_t rows, int64_t n, const gptq_config* cfg) {
  (void)cfg;
  if (rows < 1 || rows > (int64_t)1 << 30 || n < 1 || n > kMaxDim) return 0;  // as gptq_quantize_layer
  return gptq::quantize_workspace(rows, n);
}

// Shared by both forms: loss_host (sync form) or loss_dev (stream-ordered form).
static gptq_status quantize_layer(const char* who, const float* U, const int32_t* perm, const uint8_t* dead,
                                  int64_t n, const gptq_config* cfg, const void* W, gptq_dtype wdt, int64_t rows,
                                  int64_t ldw, int32_t* qweight, uint16_t* scales, uint16_t* zeros, int32_t* g_idx,
                                  double* loss_out, double* loss_dev, void* workspace, size_t ws_bytes,
                                  void* stream) {
  gptq_status st = check_config(cfg, true);
  if (st != GPTQ_OK) return st;
  if (n < 1 || n > kMaxDim) return fail(GPTQ_ERR_INVALID_ARG, "n=%lld out of range", (long long)n);
  if (n % cfg->block_size != 0)
    return fail(GPTQ_ERR_UNSUPPORTED, "n=%lld is not a multiple of block_size=%d", (long long)n, cfg->block_size);
  if (rows < 0 || rows > (int64_t)1 << 30) return fail(GPTQ_ERR_INVALID_ARG, "rows=%lld out of range", (long long)rows);
  if (!valid_dtype(wdt)) return fail(GPTQ_ERR_INVALID_ARG, "unknown dtype %d", (int)wdt);
  if (rows == 0) {
    if (loss_out) *loss_out = 0.0;
    if (loss_dev) {
      hipError_t e = gptq::zero_loss(loss_dev, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail(who, e);
    }
    return ok();
  }
  if (!U || !perm || !dead || !W || !qweight || !scales || !zeros || !g_idx)
    return fail(GPTQ_ERR_INVALID_ARG, "NULL input or output pointer");
  if (ldw < n) return fail(GPTQ_ERR_INVALID_ARG, "ldw=%lld < n=%lld", (long long)ldw, (long long)n);
  const size_t need = gptq::quantize_workspace(rows, n);
  if (!workspace || ws_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace ? ws_bytes : 0, need);
  hipError_t e = gptq::launch_quantize(U, perm, dead, n, cfg->bits, cfg->sym, cfg->group_size, W,
                                       static_cast<int>(wdt), rows, ldw, qweight, scales, zeros, g_idx, loss_out,
                                       loss_dev, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(who, e);
  return ok();
}

gptq_status gptq_quantize_layer(const float* U, const int32_t* perm, const uint8_t* dead, int64_t n,
                                const gptq_config* cfg, const void* W, gptq_dtype wdt, int64_t rows, int64_t ldw,
                                int32_t* qweight, uint16_t* scales, uint16_t* zeros, int32_t* g_idx,
                                double* loss_out, void* workspace, size_t ws_bytes, void* stream) {
  return quantize_layer("gptq_quantize_layer", U, perm, dead, n, cfg, W, wdt, rows, ldw, qweight, scales, zeros,
                        g_idx, loss_out, nullptr, workspace, ws_bytes, stream);
}

gptq_status gptq_quantize_layer_async(const float* U, const int32_t* perm, const uint8_t* dead, int64_t n,
                                      const gptq_config* cfg, const void* W, gptq_dtype wdt, int64_t rows,
                                      int64_t ldw, int32_t* qweight, uint16_t* scales, uint16_t* zeros,
                                      int32_t* g_idx, double* loss, void* workspace, size_t ws_bytes,
                                      void* stream) {
  return quantize_layer("gptq_quantize_layer_async", U, perm, dead, n, cfg, W, wdt, rows, ldw, qweight, scales,
                        zeros, g_idx, nullptr, loss, workspace, ws_bytes, stream);
}

// ----------------------------------------------------------------------------- loss
size_t gptq_layer_loss_workspace_bytes(int64_t rows, int64_t n) {
  if (rows < 1 || rows > (int64_t)1 << 30 || n < 1 || n > kMaxDim) return 0;  // as gptq_layer_loss
  return gptq::loss_workspace(rows, n);
}

gptq_status gptq_layer_loss(const double* H, int64_t n, const void* W, gptq_dtype wdt, int64_t rows, int64_t ldw,
                            const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                            const int32_t* g_idx, const gptq_config* cfg, double* rel_loss, void* workspace,
                            size_t ws_bytes, void* stream) {
  gptq_status st = check_config(cfg, true);
  if (st != GPTQ_OK) return st;
  if (!H || !W || !qweight || !scales || !zeros || !g_idx || !rel_loss)
    return fail(GPTQ_ERR_INVALID_ARG, "NULL pointer argument");
  if (n < 1 || n > kMaxDim || (cfg->group_size > 0 && n % cfg->group_size != 0))
    return fail(GPTQ_ERR_INVALID_ARG, "n=%lld invalid", (long long)n);
  if (rows < 1 || rows > (int64_t)1 << 30) return fail(GPTQ_ERR_INVALID_ARG, "rows=%lld invalid", (long long)rows);
  if (!valid_dtype(wdt)) return fail(GPTQ_ERR_INVALID_ARG, "unknown dtype %d", (int)wdt);
  if (ldw < n) return fail(GPTQ_ERR_INVALID_ARG, "ldw=%lld < n=%lld", (long long)ldw, (long long)n);
  const size_t need = gptq::loss_workspace(rows, n);
  if (!workspace || ws_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace ? ws_bytes : 0, need);
  hipError_t e = gptq::launch_layer_loss(H, n, W, static_cast<int>(wdt), rows, ldw, qweight, scales, zeros, g_idx,
                                         cfg->bits, rel_loss, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gptq_layer_loss", e);
  return ok();
}

// ----------------------------------------------------------------------------- dequantizing matmul
size_t gptq_matmul_packed_bytes(int64_t rows, int64_t n, int32_t bits, int32_t group_size) {
  if (check_matmul_format(rows, n, bits, group_size) != GPTQ_OK) return 0;
  return gptq::matmul_packed_bytes(rows, n, bits, group_size);
}

gptq_status gptq_matmul_pack(const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                             const int32_t* g_idx, int64_t rows, int64_t n, int32_t bits, int32_t group_size,
                             void* packed, size_t packed_bytes, int32_t* col_order, int32_t* identity,
                             void* stream) {
  gptq_status st = check_matmul_format(rows, n, bits, group_size);
  if (st != GPTQ_OK) return st;
  if (!qweight || !scales || !zeros || !g_idx || !packed || !col_order)
    return fail(GPTQ_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned16(packed) || !aligned16(col_order))
    return fail(GPTQ_ERR_INVALID_ARG, "packed and col_order must be 16-byte aligned");
  const size_t need = gptq::matmul_packed_bytes(rows, n, bits, group_size);
  if (packed_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE, "packed buffer %zu bytes < required %zu", packed_bytes, need);
  uint32_t flags = 0;
  hipError_t e = gptq::launch_matmul_pack(qweight, scales, zeros, g_idx, rows, n, bits, group_size, packed,
                                          col_order, &flags, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gptq_matmul_pack", e);
  if (flags & 1u)
    return fail(GPTQ_ERR_INVALID_ARG, "g_idx does not split the %lld columns into groups of %d", (long long)n,
                group_size > 0 ? group_size : (int)n);
  if (identity) *identity = (flags & 2u) ? 0 : 1;
  return ok();
}

size_t gptq_matmul_workspace_bytes(int64_t M, int64_t n, int32_t has_col_order) {
  if (M < 1 || M > (int64_t)65535 * 16 || n < 1 || n > kMaxDim || !has_col_order) return 0;  // as gptq_matmul
  return gptq::matmul_workspace_bytes(M, n);
}

size_t gptq_matmul_static_scratch_bytes(void) { return gptq::matmul_static_scratch_bytes(); }

gptq_status gptq_matmul_static(const void* A, gptq_dtype adt, int64_t M, int64_t lda, const void* packed,
                               const int32_t* col_order, int64_t rows, int64_t n, int32_t bits, int32_t group_size,
                               void* Y, gptq_dtype ydt, int64_t ldy, void* stream) {
  gptq_status st = check_matmul_call(A, adt, M, lda, packed, col_order, rows, n, bits, group_size, Y, ydt, ldy);
  if (st != GPTQ_OK) return st;
  if (M == 0) return ok();
  void* ws = nullptr;
  if (col_order) {
    const size_t need = gptq::matmul_workspace_bytes(M, n);
    if (need > gptq::matmul_static_scratch_bytes())
      return fail(GPTQ_ERR_WORKSPACE, "M=%lld x n=%lld activations need %zu bytes of gather scratch, more than the "
                  "%zu the library holds", (long long)M, (long long)n, need, gptq::matmul_static_scratch_bytes());
    hipError_t e = gptq::matmul_static_scratch(&ws);
    if (e != hipSuccess) return hip_fail("gptq_matmul_static (scratch address)", e);
  }
  hipError_t e = gptq::launch_matmul(A, M, lda, packed, col_order, rows, n, bits, group_size, Y,
                                     static_cast<int>(ydt), ldy, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gptq_matmul_static", e);
  return ok();
}

gptq_status gptq_matmul(const void* A, gptq_dtype adt, int64_t M, int64_t lda, const void* packed,
                        const int32_t* col_order, int64_t rows, int64_t n, int32_t bits, int32_t group_size,
                        void* Y, gptq_dtype ydt, int64_t ldy, void* workspace, size_t ws_bytes, void* stream) {
  gptq_status st = check_matmul_format(rows, n, bits, group_size);
  if (st != GPTQ_OK) return st;
  if (adt != GPTQ_FP16) return fail(GPTQ_ERR_UNSUPPORTED, "activations must be fp16 (got dtype %d)", (int)adt);
  if (ydt != GPTQ_FP16 && ydt != GPTQ_FP32)
    return fail(GPTQ_ERR_UNSUPPORTED, "output must be fp16 or fp32 (got dtype %d)", (int)ydt);
  if (M < 0 || M > (int64_t)65535 * 16) return fail(GPTQ_ERR_INVALID_ARG, "M=%lld out of range", (long long)M);
  if (M == 0) return ok();
  if (!A || !packed || !Y) return fail(GPTQ_ERR_INVALID_ARG, "NULL pointer argument");
  if (lda < n || ldy < rows)
    return fail(GPTQ_ERR_INVALID_ARG, "lda=%lld < n or ldy=%lld < rows", (long long)lda, (long long)ldy);
  if (!aligned16(packed)) return fail(GPTQ_ERR_INVALID_ARG, "packed must be 16-byte aligned");
  if (col_order) {
    const size_t need = gptq::matmul_workspace_bytes(M, n);
    if (!workspace || ws_bytes < need || !aligned16(workspace))
      return fail(GPTQ_ERR_WORKSPACE, "workspace %zu bytes < required %zu (or not 16-byte aligned)",
                  workspace ? ws_bytes : 0, need);
  } else if (!aligned16(A) || lda % 8 != 0) {
    return fail(GPTQ_ERR_INVALID_ARG, "A must be 16-byte aligned with lda a multiple of 8");
  }
  hipError_t e = gptq::launch_matmul(A, M, lda, packed, col_order, rows, n, bits, group_size, Y,
                                     static_cast<int>(ydt), ldy, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gptq_matmul", e);
  return ok();
}

// ----------------------------------------------------------------------------- block forward
gptq_status gptq_rmsnorm(const void* X, gptq_dtype xdt, int64_t ldx, const float* R, int64_t T, int64_t d,
                         double eps, float* H_out, uint16_t* Y, void* stream) {
  if (T < 0 || T > ((int64_t)1 << 31) - 4) return fail(GPTQ_ERR_INVALID_ARG, "T=%lld out of range", (long long)T);
  if (d < 1 || d > kMaxDim) return fail(GPTQ_ERR_INVALID_ARG, "d=%lld out of range", (long long)d);
  if (!valid_dtype(xdt)) return fail(GPTQ_ERR_INVALID_ARG, "unknown dtype %d", (int)xdt);
  if (!(eps >= 0.0) || !std::isfinite(eps)) return fail(GPTQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (T == 0) return ok();
  if (!X || !Y) return fail(GPTQ_ERR_INVALID_ARG, "NULL X or Y");
  if (ldx < d) return fail(GPTQ_ERR_INVALID_ARG, "ldx=%lld < d=%lld", (long long)ldx, (long long)d);
  hipError_t e = gptq::launch_rmsnorm(X, static_cast<int>(xdt), ldx, R, T, d, eps, H_out, Y,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gptq_rmsnorm", e);
  return ok();
}

gptq_status gptq_rope(float* Q, float* K, int64_t T, int64_t d, int64_t head_dim, int64_t seq_len, double base,
                      void* stream) {
  if (head_dim < 2 || head_dim % 2 || head_dim > 1024)
    return fail(GPTQ_ERR_INVALID_ARG, "head_dim=%lld must be even, 2..1024", (long long)head_dim);
  if (d < head_dim || d % head_dim || d > kMaxDim)
    return fail(GPTQ_ERR_INVALID_ARG, "d=%lld must be a multiple of head_dim=%lld", (long long)d, (long long)head_dim);
  if (seq_len < 1 || T < 0 || T % seq_len)
    return fail(GPTQ_ERR_INVALID_ARG, "T=%lld must be a multiple of seq_len=%lld >= 1", (long long)T,
                (long long)seq_len);
  if (T > ((int64_t)1 << 40) / (head_dim / 2)) return fail(GPTQ_ERR_INVALID_ARG, "T too large");
  if (!(base > 0.0) || !std::isfinite(base)) return fail(GPTQ_ERR_INVALID_ARG, "base must be finite and > 0");
  if (T == 0) return ok();
  if (!Q || !K) return fail(GPTQ_ERR_INVALID_ARG, "NULL Q or K");
  hipError_t e = gptq::launch_rope(Q, K, T, d, head_dim, seq_len, base, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gptq_rope", e);
  return ok();
}

gptq_status gptq_causal_attention(const float* Q, const float* K, const float* V, int64_t T, int64_t d,
                                  int64_t head_dim, int64_t seq_len, uint16_t* O, void* stream) {
  if (head_dim != gptq::attention_head_dim())
    return fail(GPTQ_ERR_UNSUPPORTED, "head_dim=%lld (supported: %d)", (long long)head_dim,
                gptq::attention_head_dim());
  if (d < head_dim || d % head_dim || d / head_dim > 65535)
    return fail(GPTQ_ERR_INVALID_ARG, "d=%lld must be a multiple of head_dim=%lld", (long long)d, (long long)head_dim);
  if (seq_len < 1 || seq_len > ((int64_t)1 << 24) || T < 0 || T % seq_len || T / seq_len > 65535)
    return fail(GPTQ_ERR_INVALID_ARG, "T=%lld must be a multiple of seq_len=%lld (at most 65535 sequences)",
                (long long)T, (long long)seq_len);
  if (T == 0) return ok();
  if (!Q || !K || !V || !O) return fail(GPTQ_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V))
    return fail(GPTQ_ERR_INVALID_ARG, "Q, K and V must be 16-byte aligned");
  hipError_t e = gptq::launch_attention(Q, K, V, T, d, seq_len, O, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gptq_causal_attention", e);
  return ok();
}

gptq_status gptq_silu_mul(const float* G, const float* U, int64_t count, uint16_t* Y, void* stream) {
  if (count < 0) return fail(GPTQ_ERR_INVALID_ARG, "count=%lld < 0", (long long)count);
  if (count == 0) return ok();
  if (!G || !U || !Y) return fail(GPTQ_ERR_INVALID_ARG, "NULL pointer argument");
  hipError_t e = gptq::launch_silu_mul(G, U, count, Y, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gptq_silu_mul", e);
  return ok();
}

}  // extern "C"
