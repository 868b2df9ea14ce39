// Drives every validation path of the C ABI (include/gptq.h) with arguments
// that must be rejected before any device work, and the size queries with
// sizes outside their range.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the library and of this
// driver (tests/test_abi_sanitize.py), so an out-of-bounds access, an
// overflowing signed product or a bad format string in that layer stops the
// run.  Needs no GPU: no call below reaches a HIP call.  Pointer arguments
// that pass the null checks point at small host buffers; none is
// dereferenced by a rejected call.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "gptq.h"

static int failures = 0;
static int checks = 0;

#define EXPECT(call, want)                                                                               \
  do {                                                                                                   \
    const int got_ = static_cast<int>(call);                                                             \
    ++checks;                                                                                            \
    const char* msg_ = gptq_last_error();                                                                \
    const bool msg_ok_ = (want == GPTQ_OK) ? msg_[0] == '\0' : (msg_[0] != '\0' && strlen(msg_) < 512); \
    if (got_ != static_cast<int>(want) || !msg_ok_) {                                                    \
      ++failures;                                                                                        \
      fprintf(stderr, "line %d: %s -> %d (want %d), message '%s'\n", __LINE__, #call, got_,              \
              static_cast<int>(want), msg_);                                                             \
    }                                                                                                    \
  } while (0)

#define EXPECT_SIZE(expr, cond)                                       \
  do {                                                                \
    const size_t v_ = (expr);                                         \
    ++checks;                                                         \
    if (!(cond)) {                                                    \
      ++failures;                                                     \
      fprintf(stderr, "line %d: %s = %zu\n", __LINE__, #expr, v_);    \
    }                                                                 \
  } while (0)

int main() {
  alignas(256) static unsigned char buf[4096];
  void* p = buf;              // a non-null, 16-byte aligned stand-in
  void* mis = buf + 1;        // not 16-byte aligned
  double d0 = 0.0;
  int64_t cnt = 0;
  const int64_t BIG = std::numeric_limits<int64_t>::max();
  const gptq_dtype BAD = static_cast<gptq_dtype>(7);

  if (strncmp(gptq_version(), "gptq-gfx950", 11) != 0) ++failures;

  // ---------------------------------------------------------------- size queries
  EXPECT_SIZE(gptq_hessian_workspace_bytes(4096, 65536, GPTQ_BF16), v_ > 0);
  EXPECT_SIZE(gptq_hessian_workspace_bytes(4096, 65536, GPTQ_FP32), v_ == 0);
  EXPECT_SIZE(gptq_hessian_workspace_bytes(0, 65536, GPTQ_BF16), v_ == 0);
  EXPECT_SIZE(gptq_hessian_workspace_bytes(BIG, BIG, GPTQ_BF16), v_ == 0);
  EXPECT_SIZE(gptq_hessian_workspace_bytes(4096, 65536, BAD), v_ == 0);
  gptq_config cfg{4, 128, 0, 0, 0.01f, 128};
  EXPECT_SIZE(gptq_prepare_workspace_bytes(4096, &cfg), v_ >= size_t(2) * 4096 * 4096 * 8);
  EXPECT_SIZE(gptq_prepare_workspace_bytes(0, &cfg), v_ == 0);
  EXPECT_SIZE(gptq_prepare_workspace_bytes(BIG, &cfg), v_ == 0);
  EXPECT_SIZE(gptq_quantize_workspace_bytes(4096, 4096, &cfg), v_ > 0);
  EXPECT_SIZE(gptq_quantize_workspace_bytes(BIG, BIG, &cfg), v_ == 0);
  EXPECT_SIZE(gptq_quantize_workspace_bytes(-1, 4096, &cfg), v_ == 0);
  EXPECT_SIZE(gptq_layer_loss_workspace_bytes(4096, 4096), v_ > 0);
  EXPECT_SIZE(gptq_layer_loss_workspace_bytes(BIG, BIG), v_ == 0);
  EXPECT_SIZE(gptq_matmul_packed_bytes(4096, 4096, 4, 128), v_ > 0);
  EXPECT_SIZE(gptq_matmul_packed_bytes(BIG, BIG, 4, 128), v_ == 0);
  EXPECT_SIZE(gptq_matmul_packed_bytes(4096, 4096, 5, 128), v_ == 0);
  EXPECT_SIZE(gptq_matmul_workspace_bytes(16, 4096, 1), v_ >= size_t(16) * 4096 * 2);
  EXPECT_SIZE(gptq_matmul_workspace_bytes(16, 4096, 0), v_ == 0);
  EXPECT_SIZE(gptq_matmul_workspace_bytes(BIG, BIG, 1), v_ == 0);
  EXPECT_SIZE(gptq_matmul_static_scratch_bytes(), v_ > 0);
  if (gptq_hessian_chain_tokens() <= 0) ++failures;

  // ---------------------------------------------------------------- Hessian
  double* H = static_cast<double*>(p);
  EXPECT(gptq_hessian_accumulate(nullptr, 64, &cnt, p, GPTQ_BF16, 8, 64, p, 4096, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(H, 64, nullptr, p, GPTQ_BF16, 8, 64, p, 4096, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(H, 0, &cnt, p, GPTQ_BF16, 8, 64, p, 4096, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(H, BIG, &cnt, p, GPTQ_BF16, 8, BIG, p, 4096, nullptr), GPTQ_ERR_INVALID_ARG);
  cnt = -1;
  EXPECT(gptq_hessian_accumulate(H, 64, &cnt, p, GPTQ_BF16, 8, 64, p, 4096, nullptr), GPTQ_ERR_INVALID_ARG);
  cnt = 0;
  EXPECT(gptq_hessian_accumulate(H, 64, &cnt, p, GPTQ_BF16, -1, 64, p, 4096, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(H, 64, &cnt, p, BAD, 8, 64, p, 4096, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(H, 64, &cnt, p, GPTQ_BF16, 0, 64, nullptr, 0, nullptr), GPTQ_OK);
  EXPECT(gptq_hessian_accumulate(H, 64, &cnt, nullptr, GPTQ_BF16, 8, 64, p, 4096, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(H, 64, &cnt, p, GPTQ_BF16, 8, 63, p, 4096, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(H, 4096, &cnt, p, GPTQ_BF16, 65536, 4096, nullptr, 0, nullptr), GPTQ_ERR_WORKSPACE);
  EXPECT(gptq_hessian_accumulate(H, 4096, &cnt, p, GPTQ_BF16, 65536, 4096, p, 16, nullptr), GPTQ_ERR_WORKSPACE);
  if (cnt != 0) ++failures;  // no rejected call may touch the running count

  // ---------------------------------------------------------------- prepare
  float* U = static_cast<float*>(p);
  int32_t* perm = static_cast<int32_t*>(p);
  uint8_t* dead = static_cast<uint8_t*>(p);
  gptq_config c = cfg;
  EXPECT(gptq_prepare_hinv(H, 64, nullptr, U, perm, dead, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  c.damp_percent = NAN;
  EXPECT(gptq_prepare_hinv(H, 64, &c, U, perm, dead, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  c.damp_percent = -0.5f;
  EXPECT(gptq_prepare_hinv(H, 64, &c, U, perm, dead, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  c = cfg;
  c.desc_act = 2;
  EXPECT(gptq_prepare_hinv(H, 64, &c, U, perm, dead, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv(nullptr, 64, &cfg, U, perm, dead, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv(H, 0, &cfg, U, perm, dead, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv(H, BIG, &cfg, U, perm, dead, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv(H, 64, &cfg, U, perm, dead, nullptr, 0, nullptr), GPTQ_ERR_WORKSPACE);
  EXPECT(gptq_prepare_hinv(H, 64, &cfg, U, perm, dead, p, 8, nullptr), GPTQ_ERR_WORKSPACE);
  // the stream-ordered form: the same checks, and its device flag
  int32_t* info = static_cast<int32_t*>(p);
  EXPECT(gptq_prepare_hinv_async(H, 64, nullptr, U, perm, dead, info, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv_async(nullptr, 64, &cfg, U, perm, dead, info, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv_async(H, 64, &cfg, U, perm, dead, nullptr, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv_async(H, BIG, &cfg, U, perm, dead, info, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv_async(H, 64, &cfg, U, perm, dead, info, p, 8, nullptr), GPTQ_ERR_WORKSPACE);

  // ---------------------------------------------------------------- quantize
  int32_t* qw = static_cast<int32_t*>(p);
  uint16_t* sc = static_cast<uint16_t*>(p);
  int32_t* gi = static_cast<int32_t*>(p);
  const int32_t bad_bits[] = {0, 1, 5, 16, -4};
  for (int32_t b : bad_bits) {
    c = cfg;
    c.bits = b;
    EXPECT(gptq_quantize_layer(U, perm, dead, 256, &c, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
           GPTQ_ERR_UNSUPPORTED);
  }
  const int32_t bad_groups[] = {0, 16, 100, 256, -2};
  for (int32_t g : bad_groups) {
    c = cfg;
    c.group_size = g;
    EXPECT(gptq_quantize_layer(U, perm, dead, 256, &c, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
           GPTQ_ERR_UNSUPPORTED);
  }
  c = cfg;
  c.block_size = 64;
  EXPECT(gptq_quantize_layer(U, perm, dead, 256, &c, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_UNSUPPORTED);
  c = cfg;
  c.sym = 3;
  EXPECT(gptq_quantize_layer(U, perm, dead, 256, &c, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer(U, perm, dead, 0, &cfg, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer(U, perm, dead, BIG, &cfg, p, GPTQ_FP32, 8, BIG, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer(U, perm, dead, 200, &cfg, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_quantize_layer(U, perm, dead, 256, &cfg, p, GPTQ_FP32, -1, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer(U, perm, dead, 256, &cfg, p, GPTQ_FP32, BIG, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer(U, perm, dead, 256, &cfg, p, BAD, 8, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  d0 = 1.0;
  EXPECT(gptq_quantize_layer(nullptr, nullptr, nullptr, 256, &cfg, nullptr, GPTQ_FP32, 0, 256, nullptr, nullptr, nullptr,
                             nullptr, &d0, nullptr, 0, nullptr),
         GPTQ_OK);
  if (d0 != 0.0) ++failures;  // an empty layer reports zero loss
  EXPECT(gptq_quantize_layer(nullptr, perm, dead, 256, &cfg, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer(U, perm, dead, 256, &cfg, p, GPTQ_FP32, 8, 255, qw, sc, sc, gi, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer(U, perm, dead, 256, &cfg, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &d0, nullptr, 0, nullptr),
         GPTQ_ERR_WORKSPACE);
  EXPECT(gptq_quantize_layer(U, perm, dead, 256, &cfg, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &d0, p, 64, nullptr),
         GPTQ_ERR_WORKSPACE);
  // the stream-ordered form (its loss pointer is device memory: never touched on these paths)
  double* dloss = static_cast<double*>(p);
  c = cfg;
  c.bits = 5;
  EXPECT(gptq_quantize_layer_async(U, perm, dead, 256, &c, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, dloss, p, 1 << 20,
                                   nullptr),
         GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_quantize_layer_async(nullptr, perm, dead, 256, &cfg, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, dloss, p,
                                   1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer_async(U, perm, dead, 256, &cfg, p, GPTQ_FP32, 8, 255, qw, sc, sc, gi, dloss, p, 1 << 20,
                                   nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer_async(U, perm, dead, 256, &cfg, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, dloss, p, 64,
                                   nullptr),
         GPTQ_ERR_WORKSPACE);

  // ---------------------------------------------------------------- layer loss
  EXPECT(gptq_layer_loss(H, 256, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, nullptr, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_layer_loss(H, 256, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &cfg, nullptr, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_layer_loss(H, 200, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &cfg, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_layer_loss(H, BIG, p, GPTQ_FP32, 8, BIG, qw, sc, sc, gi, &cfg, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_layer_loss(H, 256, p, GPTQ_FP32, 0, 256, qw, sc, sc, gi, &cfg, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_layer_loss(H, 256, p, BAD, 8, 256, qw, sc, sc, gi, &cfg, &d0, p, 1 << 20, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_layer_loss(H, 256, p, GPTQ_FP32, 8, 100, qw, sc, sc, gi, &cfg, &d0, p, 1 << 20, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_layer_loss(H, 256, p, GPTQ_FP32, 8, 256, qw, sc, sc, gi, &cfg, &d0, p, 8, nullptr), GPTQ_ERR_WORKSPACE);

  // ---------------------------------------------------------------- matmul pack
  int32_t* order = static_cast<int32_t*>(p);
  int32_t ident = 7;
  EXPECT(gptq_matmul_pack(qw, sc, sc, gi, 64, 256, 5, 128, p, 1 << 20, order, &ident, nullptr), GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_matmul_pack(qw, sc, sc, gi, 64, 256, 4, 100, p, 1 << 20, order, &ident, nullptr), GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_matmul_pack(qw, sc, sc, gi, 64, 200, 4, 128, p, 1 << 20, order, &ident, nullptr), GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_matmul_pack(qw, sc, sc, gi, 64, BIG, 4, 128, p, 1 << 20, order, &ident, nullptr), GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_matmul_pack(qw, sc, sc, gi, 0, 256, 4, 128, p, 1 << 20, order, &ident, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul_pack(qw, sc, sc, gi, BIG, 256, 4, 128, p, 1 << 20, order, &ident, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul_pack(qw, sc, sc, gi, 64, 65536 * 32, 4, 32, p, 1 << 20, order, &ident, nullptr),
         GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_matmul_pack(nullptr, sc, sc, gi, 64, 256, 4, 128, p, 1 << 20, order, &ident, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul_pack(qw, sc, sc, gi, 64, 256, 4, 128, mis, 1 << 20, order, &ident, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul_pack(qw, sc, sc, gi, 64, 256, 4, 128, p, 16, order, &ident, nullptr), GPTQ_ERR_WORKSPACE);
  if (ident != 7) ++failures;  // rejected calls leave the flag alone

  // ---------------------------------------------------------------- matmul
  EXPECT(gptq_matmul(p, GPTQ_BF16, 1, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_matmul(p, GPTQ_FP16, 1, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_BF16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_matmul(p, GPTQ_FP16, -1, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul(p, GPTQ_FP16, BIG, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul(nullptr, GPTQ_FP16, 0, 256, nullptr, nullptr, 64, 256, 4, 128, nullptr, GPTQ_FP16, 64, nullptr, 0,
                     nullptr),
         GPTQ_OK);
  EXPECT(gptq_matmul(nullptr, GPTQ_FP16, 1, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul(p, GPTQ_FP16, 1, 255, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul(p, GPTQ_FP16, 1, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 63, nullptr, 0, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul(p, GPTQ_FP16, 1, 256, mis, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul(mis, GPTQ_FP16, 1, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul(p, GPTQ_FP16, 1, 260, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul(p, GPTQ_FP16, 4, 256, p, order, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr, 0, nullptr),
         GPTQ_ERR_WORKSPACE);
  EXPECT(gptq_matmul(p, GPTQ_FP16, 4, 256, p, order, 64, 256, 4, 128, p, GPTQ_FP16, 64, p, 8, nullptr),
         GPTQ_ERR_WORKSPACE);
  EXPECT(gptq_matmul(p, GPTQ_FP16, 4, 256, p, order, 64, 256, 4, 128, p, GPTQ_FP16, 64, mis, 1 << 20, nullptr),
         GPTQ_ERR_WORKSPACE);

  // ---------------------------------------------------------------- matmul without a workspace
  EXPECT(gptq_matmul_static(p, GPTQ_BF16, 1, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr),
         GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_matmul_static(p, GPTQ_FP16, -1, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul_static(nullptr, GPTQ_FP16, 0, 256, nullptr, nullptr, 64, 256, 4, 128, nullptr, GPTQ_FP16, 64,
                            nullptr),
         GPTQ_OK);
  EXPECT(gptq_matmul_static(p, GPTQ_FP16, 1, 256, nullptr, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr),
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_matmul_static(mis, GPTQ_FP16, 1, 256, p, nullptr, 64, 256, 4, 128, p, GPTQ_FP16, 64, nullptr),
         GPTQ_ERR_INVALID_ARG);
  // act-order activations whose gathered copy would exceed the library's scratch
  EXPECT(gptq_matmul_static(p, GPTQ_FP16, 65535 * 16, 65536, p, order, 64, 65536, 4, 128, p, GPTQ_FP16, 64, nullptr),
         GPTQ_ERR_WORKSPACE);

  // ---------------------------------------------------------------- block forward
  uint16_t* Y16 = static_cast<uint16_t*>(p);
  float* F = static_cast<float*>(p);
  EXPECT(gptq_rmsnorm(p, GPTQ_FP32, 64, nullptr, -1, 64, 1e-5, F, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rmsnorm(p, GPTQ_FP32, 64, nullptr, BIG, 64, 1e-5, F, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rmsnorm(p, GPTQ_FP32, 64, nullptr, 8, 0, 1e-5, F, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rmsnorm(p, GPTQ_FP32, BIG, nullptr, 8, BIG, 1e-5, F, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rmsnorm(p, BAD, 64, nullptr, 8, 64, 1e-5, F, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rmsnorm(p, GPTQ_FP32, 64, nullptr, 8, 64, NAN, F, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rmsnorm(p, GPTQ_FP32, 64, nullptr, 8, 64, -1.0, F, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rmsnorm(nullptr, GPTQ_FP32, 64, nullptr, 0, 64, 1e-5, nullptr, nullptr, nullptr), GPTQ_OK);
  EXPECT(gptq_rmsnorm(nullptr, GPTQ_FP32, 64, nullptr, 8, 64, 1e-5, F, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rmsnorm(p, GPTQ_FP32, 63, nullptr, 8, 64, 1e-5, F, Y16, nullptr), GPTQ_ERR_INVALID_ARG);

  EXPECT(gptq_rope(F, F, 16, 256, 3, 16, 1e4, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rope(F, F, 16, 256, 2048, 16, 1e4, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rope(F, F, 16, 200, 128, 16, 1e4, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rope(F, F, 16, 256, 128, 0, 1e4, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rope(F, F, 17, 256, 128, 16, 1e4, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rope(F, F, BIG - BIG % 16, 256, 128, 16, 1e4, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rope(F, F, 16, 256, 128, 16, 0.0, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rope(F, F, 16, 256, 128, 16, INFINITY, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_rope(nullptr, nullptr, 0, 256, 128, 16, 1e4, nullptr), GPTQ_OK);
  EXPECT(gptq_rope(nullptr, F, 16, 256, 128, 16, 1e4, nullptr), GPTQ_ERR_INVALID_ARG);

  EXPECT(gptq_causal_attention(F, F, F, 16, 256, 64, 16, Y16, nullptr), GPTQ_ERR_UNSUPPORTED);
  EXPECT(gptq_causal_attention(F, F, F, 16, 200, 128, 16, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_causal_attention(F, F, F, 16, BIG - BIG % 128, 128, 16, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_causal_attention(F, F, F, 17, 256, 128, 16, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_causal_attention(F, F, F, BIG - BIG % 16, 256, 128, 16, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_causal_attention(F, F, F, 16, 256, 128, 0, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_causal_attention(nullptr, nullptr, nullptr, 0, 256, 128, 16, nullptr, nullptr), GPTQ_OK);
  EXPECT(gptq_causal_attention(F, F, nullptr, 16, 256, 128, 16, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_causal_attention(static_cast<const float*>(mis), F, F, 16, 256, 128, 16, Y16, nullptr),
         GPTQ_ERR_INVALID_ARG);

  EXPECT(gptq_silu_mul(F, F, -1, Y16, nullptr), GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_silu_mul(nullptr, nullptr, 0, nullptr, nullptr), GPTQ_OK);
  EXPECT(gptq_silu_mul(F, nullptr, 8, Y16, nullptr), GPTQ_ERR_INVALID_ARG);

  printf("%d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
