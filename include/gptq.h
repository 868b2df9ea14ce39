/*
 * gptq.h -- C ABI of the GPTQ layer-wise quantization solver for AMD Instinct
 * MI355X (gfx950).
 *
 * Method (web pages about GPTQ, cited by title and section):
 *   polydesk.ai glossary "GPTQ (Generative Pre-trained Transformer Quantization)":
 *     "Comment fonctionne l'algorithme GPTQ"  -- per-layer objective ||W X - W_hat X||^2
 *     "Étape 1 : Ordre arbitraire"             -- one fixed column order for all rows
 *     "Étape 2 : Compensation d'erreur via la Hessienne" -- H = 2 X X^T, errors pushed
 *                                                 onto later columns through the
 *                                                 Cholesky factor of H^-1
 *     "Étape 3 : Mises à jour par blocs"       -- lazy updates in blocks of 128 columns
 *     "Paramètres clés de GPTQ"                -- bits, group_size, desc_act, sym
 *   skillmd.com "Gptq" skill page, "Quantização group-wise" and
 *     "Configurações de quantização"           -- groups of 128 with own scale/zero,
 *                                                 damp_percent
 *   ayinedjimi-consultants "Quantization : GPTQ, GGUF, AWQ", "Calibration et dataset"
 *                                              -- fp16 scale/zero, packed low-bit weights
 *
 * Conventions shared by every call
 *   - All array pointers are DEVICE pointers (memory of the current HIP device)
 *     unless a comment says "host".  The caller owns every buffer; the library
 *     never allocates or frees device memory.  Scratch space is passed in as a
 *     workspace whose size is given by the matching *_workspace_bytes() query;
 *     a query returns 0 for sizes its call rejects.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it in order; calls return once the work is enqueued, except
 *     where a comment says the call synchronizes the stream.
 *   - Matrices are row-major.  W is [rows, n] (out features x in features);
 *     X is [tokens, n] (one calibration token per row); H and U are [n, n].
 *   - Errors are returned as gptq_status; arguments are checked before any
 *     device work is enqueued, so an error other than GPTQ_ERR_HIP /
 *     GPTQ_ERR_NOT_PD leaves every output untouched.  gptq_last_error() gives a
 *     message for the last failing call on the calling thread.
 *   - Calls that share a workspace or outputs must not overlap on different
 *     streams.
 */
#ifndef GPTQ_H
#define GPTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad leading dimension   */
  GPTQ_ERR_UNSUPPORTED = -2,  /* valid but not supported: bits, group size, dtype ... */
  GPTQ_ERR_NOT_PD = -3,       /* damped Hessian not positive definite                 */
  GPTQ_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed           */
  GPTQ_ERR_WORKSPACE = -5     /* workspace null or smaller than the query returned    */
} gptq_status;

/* In C++ the element type's underlying type is fixed to int32_t, so every
 * int32 a caller passes is a value of the type and an unknown code can be
 * rejected (without a fixed type C++ leaves such a value undefined); the
 * layout is the same 32-bit integer as the C declaration's. */
#ifdef __cplusplus
typedef enum : int32_t { GPTQ_BF16 = 0, GPTQ_FP16 = 1, GPTQ_FP32 = 2 } gptq_dtype;
#else
typedef enum { GPTQ_BF16 = 0, GPTQ_FP16 = 1, GPTQ_FP32 = 2 } gptq_dtype;
#endif

/* The quantize config of the pages ("Configurações de quantização", "Paramètres clés"). */
typedef struct {
  int32_t bits;          /* code width: 2, 3, 4 or 8 ("Paramètres clés", bits)             */
  int32_t group_size;    /* weights per scale/zero group along a row: 128, 64, 32, or -1 for  */
                         /* one group per row ("Paramètres clés", group_size)                */
  int32_t sym;           /* 0: asymmetric grid (zero point in [0, 2^bits-1]);               */
                         /* 1: symmetric grid, levels -(2^(b-1)-1)..2^(b-1)-1, zero exact    */
                         /*    (the grid "Paramètres clés" describes);                       */
                         /* 2: symmetric range [-a, a] over all 2^bits codes, zero point     */
                         /*    2^(b-1) (a variant outside the pages' text)                   */
  int32_t desc_act;      /* 1: act-order, columns visited by decreasing diag(H)              */
  float damp_percent;    /* lambda = damp_percent * mean(diag H) is added to the diagonal    */
  int32_t block_size;    /* lazy-batch width in columns: 128                                 */
} gptq_config;

/* ------------------------------------------------------------------------- *
 * Calibration Hessian ("Étape 2": H = 2 X X^T).
 *
 * Maintains the running mean H = (2 / N) * sum_t x_t x_t^T over all tokens fed
 * so far, N = *n_tokens.  One call adds `tokens` rows of X:
 *     H <- (N_old / N_new) * H + (2 / N_new) * X^T X,   N_new = N_old + tokens.
 * If *n_tokens == 0 on entry the previous contents of H are ignored (no need to
 * clear it).  tokens == 0 is a no-op returning GPTQ_OK.
 *   H        device fp64 [n, n]; the full symmetric matrix is written (both
 *            triangles, bit-identical mirror).  1 <= n <= 2097120.
 *   n_tokens HOST int64 in/out: running token count, updated on success.
 *   X        device [tokens, ldx] of dtype xdt (bf16, fp16 or fp32), ldx >= n;
 *            only columns 0..n-1 are read.  Not modified.
 *   workspace, ws_bytes: device scratch of at least
 *            gptq_hessian_workspace_bytes(n, tokens, xdt) bytes (token pieces of
 *            the tiles that do not fill the last round of the current device's
 *            compute units); NULL is accepted when that size is 0.
 * bf16/fp16 products are summed by MFMA with fp32 accumulation in chains of at
 * most gptq_hessian_chain_tokens() tokens; chains are combined in fp64, which
 * is also the storage precision of H (GPTQ's codes react to Hessian error far
 * below fp32 chain-summation error).  fp32 inputs accumulate in fp64.
 * Deterministic: same inputs, same bits.
 * ------------------------------------------------------------------------- */
size_t gptq_hessian_workspace_bytes(int64_t n, int64_t tokens, gptq_dtype xdt);
int64_t gptq_hessian_chain_tokens(void);
gptq_status gptq_hessian_accumulate(double* H, int64_t n, int64_t* n_tokens,
                                    const void* X, gptq_dtype xdt, int64_t tokens,
                                    int64_t ldx, void* workspace, size_t ws_bytes,
                                    void* stream);

/* ------------------------------------------------------------------------- *
 * Prepare ("Étape 2": Cholesky factor of the inverse Hessian; damp_percent;
 * desc_act).  Reads H, writes
 *   perm  device int32 [n]: sweep position j visits original column perm[j]
 *         (identity unless cfg->desc_act; else stable sort of diag(H), largest
 *         first, ties by lower index),
 *   dead  device uint8 [n]: 1 where H_ii == 0 (original column order); such a
 *         diagonal is taken as 1 and the weight column is zeroed by the quantizer,
 *   U     device fp32 [n, n]: the upper triangular factor with positive diagonal
 *         and U^T U = (H_p + lambda I)^-1, H_p = H permuted to sweep order,
 *         lambda = damp_percent * mean(diag H_p).  Entries below the diagonal
 *         are written as 0.
 * H is device fp64 [n, n] as written by gptq_hessian_accumulate (symmetric;
 * entries of both triangles are read) and is not modified.
 * The factorization runs in fp64 on the device (the result is rounded to fp32).
 * Synchronizes `stream` once, to read back the positive-definiteness flag:
 * returns GPTQ_ERR_NOT_PD (U then undefined) if a pivot is not > 0 or not
 * finite, or a diagonal entry of H is negative or not finite.
 * 1 <= n <= 65535.
 * ------------------------------------------------------------------------- */
size_t gptq_prepare_workspace_bytes(int64_t n, const gptq_config* cfg);
gptq_status gptq_prepare_hinv(const double* H, int64_t n, const gptq_config* cfg,
                              float* U, int32_t* perm, uint8_t* dead,
                              void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * Quantize one layer ("Étape 1/2/3", "Quantização group-wise").
 *   U, perm, dead  as written by gptq_prepare_hinv for this n and cfg (several
 *                  layers that share a Hessian may reuse them).
 *   W        device [rows, ldw] of dtype wdt, ldw >= n.  Not modified.
 * Outputs (caller-allocated device buffers):
 *   qweight  int32 [n*bits/32, rows]: row r's codes in ORIGINAL column order form
 *            a little-endian bit stream, column i at bits [bits*i, bits*i+bits);
 *            qweight[k, r] is word k of that stream (2-bit: 16 codes per word;
 *            3-bit: 32 codes per 3 words; 4-bit: 8; 8-bit: 4).
 *   scales   fp16 bits [G, rows], G = n/group_size (1 for group_size -1):
 *            group g = sweep columns [g*gs, (g+1)*gs).  A group's grid is
 *            taken at its first column from the current (compensated) weights
 *            of its columns; for group_size -1 from the whole row before the
 *            sweep.
 *   zeros    fp16 bits [G, rows]: integer-valued zero points.
 *   g_idx    int32 [n]: g_idx[perm[j]] = j / group_size (0 for group_size -1).
 *   loss_out HOST double, may be NULL: sum over rows and columns of e^2 / 2 with
 *            e = (w - w_hat) / U[j, j] (equals tr(D H_d D^T) / 2, D = W - W_hat).
 * Dequantization: W_hat[r, i] = scales[g_idx[i], r] * (code[r, i] - zeros[g_idx[i], r]).
 * Supported: bits in {2, 3, 4, 8}; group_size in {32, 64, 128, -1}; block_size == 128;
 * n % 128 == 0 (GPTQ_ERR_UNSUPPORTED otherwise).
 * rows == 0 is a no-op.  Synchronizes `stream` once when loss_out != NULL.
 * ------------------------------------------------------------------------- */
size_t gptq_quantize_workspace_bytes(int64_t rows, int64_t n, const gptq_config* cfg);
gptq_status gptq_quantize_layer(const float* U, const int32_t* perm, const uint8_t* dead,
                                int64_t n, const gptq_config* cfg,
                                const void* W, gptq_dtype wdt, int64_t rows, int64_t ldw,
                                int32_t* qweight, uint16_t* scales, uint16_t* zeros,
                                int32_t* g_idx, double* loss_out,
                                void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * Stream-ordered forms of prepare and quantize ("Étape 2", "Étape 1/2/3": the
 * same computation).  A model is quantized layer after layer; these forms let
 * a caller queue the Hessian, prepare and quantize calls of many layers
 * without a host round trip between them, and read every status afterwards.
 *
 * gptq_prepare_hinv_async: as gptq_prepare_hinv (same arguments, checks,
 * workspace and outputs, bit-identical U, perm and dead), except that the
 * positive-definiteness result is written in stream order to
 *   info  device int32 [1]: 0 if the damped Hessian is positive definite,
 *         1 if not (U then undefined),
 * and the call does not synchronize `stream`.  A nonzero status is returned
 * only for argument errors and failed launches.
 *
 * gptq_quantize_layer_async: as gptq_quantize_layer (same arguments, checks,
 * workspace and outputs, bit-identical codes, scales, zeros, g_idx), except
 * that the loss goes to
 *   loss  device double [1], may be NULL: the same sum as loss_out, written
 *         in stream order (rows == 0 writes 0),
 * and the call never synchronizes `stream`.
 * ------------------------------------------------------------------------- */
gptq_status gptq_prepare_hinv_async(const double* H, int64_t n, const gptq_config* cfg,
                                    float* U, int32_t* perm, uint8_t* dead, int32_t* info,
                                    void* workspace, size_t ws_bytes, void* stream);
gptq_status gptq_quantize_layer_async(const float* U, const int32_t* perm, const uint8_t* dead,
                                      int64_t n, const gptq_config* cfg,
                                      const void* W, gptq_dtype wdt, int64_t rows, int64_t ldw,
                                      int32_t* qweight, uint16_t* scales, uint16_t* zeros,
                                      int32_t* g_idx, double* loss,
                                      void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * Relative layer loss ("Comment fonctionne l'algorithme GPTQ": the objective is
 * the squared output error).  Dequantizes the packed outputs and returns
 *   *rel_loss (HOST) = tr(D H D^T) / tr(W H W^T),  D = W - W_hat,
 * which equals ||W X - W_hat X||^2 / ||W X||^2 for H = (2/N) X^T X.
 * H is the undamped fp64 Hessian in original column order.  Synchronizes `stream`.
 * A measurement helper: not part of the quantization itself.
 * ------------------------------------------------------------------------- */
size_t gptq_layer_loss_workspace_bytes(int64_t rows, int64_t n);
gptq_status gptq_layer_loss(const double* H, int64_t n, const void* W, gptq_dtype wdt,
                            int64_t rows, int64_t ldw, const int32_t* qweight,
                            const uint16_t* scales, const uint16_t* zeros, const int32_t* g_idx,
                            const gptq_config* cfg, double* rel_loss,
                            void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * Dequantizing matmul for inference with a quantized layer (ayinedjimi-
 * consultants "Quantization : GPTQ, GGUF, AWQ", "Calibration et dataset" and
 * "Kernels d'inférence": the serving kernels unpack and dequantize the packed
 * low-bit weights on the fly and multiply them with fp16 activations).
 *
 * gptq_matmul_pack: once per layer, converts the outputs of
 * gptq_quantize_layer into the tiled layout gptq_matmul reads.
 *   qweight, scales, zeros, g_idx  as gptq_quantize_layer writes them for
 *            (rows, n, bits, group_size); not modified.
 *   packed   device buffer of at least gptq_matmul_packed_bytes(rows, n, bits,
 *            group_size) bytes (packed_bytes gives its size), 16-byte aligned.
 *   col_order device int32 [n], 16-byte aligned: the input columns listed group
 *            by group (ascending column index inside a group).  It is the
 *            identity unless act-order scattered the groups.
 *   identity HOST int32 out, may be NULL: 1 if col_order is the identity.
 * Synchronizes `stream` (to read the validation flag).  Returns
 * GPTQ_ERR_INVALID_ARG if g_idx does not split the n columns into n/group_size
 * groups (one for group_size -1) of group_size columns each; the codes are not
 * retiled then, and packed and col_order hold no usable layout.
 *
 * gptq_matmul: Y[m, o] = sum_i A[m, i] * W_hat[o, i] for m < M, o < rows, with
 * W_hat[o, i] = scales[g_idx[i], o] * (code[o, i] - zeros[g_idx[i], o]).
 *   A        device fp16 [M, lda], lda >= n (adt must be GPTQ_FP16).  With
 *            col_order NULL, A must be 16-byte aligned and lda a multiple of 8.
 *   packed   as written by gptq_matmul_pack for the same rows, n, bits, group_size.
 *   col_order NULL when the pack reported identity (the activations are then
 *            read in place), else the col_order the pack wrote: the
 *            activations are first copied in that order into the workspace.
 *   workspace, ws_bytes: device scratch of gptq_matmul_workspace_bytes(M, n,
 *            col_order != NULL) bytes, 16-byte aligned (0 bytes, NULL accepted,
 *            without col_order).
 *   Y        device [M, ldy] of ydt (GPTQ_FP16 or GPTQ_FP32), ldy >= rows; only
 *            columns 0..rows-1 of rows 0..M-1 are written.
 * Products of the fp16 activations with the exact integers code - zero are
 * summed in fp32, each group's sum is scaled by its fp16 scale in fp32, and the
 * result is rounded once to ydt.  Up to 255 tokens they are processed 16 at a
 * time, the weights read once per 16 (the decoding path); from 256 tokens a
 * tiled kernel reads each weight tile once per 128 tokens.  Both round alike.
 * Does not synchronize, allocate or clear memory, so it can be captured in a
 * graph; calls that share a workspace must not overlap.  M == 0 is a no-op.  Deterministic.
 * Supported: bits 2, 3, 4, 8; group_size 32, 64, 128, -1; n a multiple of 128
 * with at most 1528 groups per row (n <= 48896 at group_size 32, 195584 at 128).
 * ------------------------------------------------------------------------- */
size_t gptq_matmul_packed_bytes(int64_t rows, int64_t n, int32_t bits, int32_t group_size);
gptq_status gptq_matmul_pack(const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                             const int32_t* g_idx, int64_t rows, int64_t n, int32_t bits, int32_t group_size,
                             void* packed, size_t packed_bytes, int32_t* col_order, int32_t* identity,
                             void* stream);
size_t gptq_matmul_workspace_bytes(int64_t M, int64_t n, int32_t has_col_order);
gptq_status gptq_matmul(const void* A, gptq_dtype adt, int64_t M, int64_t lda, const void* packed,
                        const int32_t* col_order, int64_t rows, int64_t n, int32_t bits, int32_t group_size,
                        void* Y, gptq_dtype ydt, int64_t ldy, void* workspace, size_t ws_bytes,
                        void* stream);

/* ------------------------------------------------------------------------- *
 * gptq_matmul without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc.  Same arguments, result and rules as gptq_matmul, minus
 * workspace/ws_bytes.  It calls no hipMalloc, hipFree or allocating routine.
 * Act-order layers (col_order != NULL) gather their activations into a
 * library-owned device array of gptq_matmul_static_scratch_bytes() bytes
 * (4 MiB): one copy per device, reserved when the library is loaded on that
 * device and held until the process ends.  Returns GPTQ_ERR_WORKSPACE if the
 * gathered activations, M * n * 2 bytes rounded up to 256, do not fit it
 * (nothing is launched then).  Layers without col_order use no scratch.
 * All calls on one device share that array, and each call overwrites what it
 * uses before reading it (nothing needs clearing); calls that overlap on one
 * device (on different streams or host threads) race on it.  The first call
 * on a device looks up the array's device address (hipGetSymbolAddress, with
 * that device current).
 * ------------------------------------------------------------------------- */
size_t gptq_matmul_static_scratch_bytes(void);
gptq_status gptq_matmul_static(const void* A, gptq_dtype adt, int64_t M, int64_t lda, const void* packed,
                               const int32_t* col_order, int64_t rows, int64_t n, int32_t bits, int32_t group_size,
                               void* Y, gptq_dtype ydt, int64_t ldy, void* stream);

/* ------------------------------------------------------------------------- *
 * Forward of one decoder block, for block-sequential calibration (wikiprompt.org
 * "GPTQ", "Approche technique": the layers are treated one after another;
 * polydesk.ai "GPTQ", "Comment fonctionne l'algorithme GPTQ": each linear is
 * solved on the activations that reach it).  Together with gptq_matmul (fp32
 * output) they produce the inputs of o_proj, gate/up and down_proj of a
 * Llama-2-shaped block from the already-quantized q/k/v and gate/up weights.
 * All pointers are device pointers; arrays are row-major; T tokens are whole
 * sequences of seq_len tokens, one after another.  Every call only enqueues
 * work on `stream`, allocates nothing and returns GPTQ_ERR_INVALID_ARG /
 * GPTQ_ERR_UNSUPPORTED before any launch on bad arguments; T == 0 is a no-op.
 *
 * gptq_rmsnorm: h = X (+ R when R != NULL), per token
 *     Y = fp16(h / sqrt(mean(h^2) + eps))        (unit norm weight)
 *   X   [T, ldx] of xdt, ldx >= d; R fp32 [T, d] or NULL;
 *   H_out fp32 [T, d] or NULL: receives h;  Y fp16 bits [T, d].
 *   The mean and the scaling are computed in fp64, Y rounded once (to nearest
 *   even).
 * gptq_rope: rotary position embedding, in place on Q and K (fp32 [T, d],
 *   heads of head_dim): inside each head, features i and i + head_dim/2 are
 *   rotated by the angle p * base^(-2i/head_dim), p = token index mod seq_len.
 *   Angles, sines and cosines in fp64; the rotation in fp32.
 * gptq_causal_attention: O = fp16(softmax(q k^T / sqrt(head_dim)) v) per head
 *   and sequence, each token attending to itself and the tokens before it in
 *   its sequence.  Q, K, V fp32 [T, d] (16-byte aligned), O fp16 bits [T, d].
 *   fp32 arithmetic (online softmax over key steps of 32), one rounding to
 *   fp16.  head_dim must be 128 (GPTQ_ERR_UNSUPPORTED otherwise).
 * gptq_silu_mul: Y[i] = fp16(silu(G[i]) * U[i]), silu(x) = x / (1 + e^-x),
 *   in fp64 with one rounding; G, U fp32 [count], Y fp16 bits [count].
 * ------------------------------------------------------------------------- */
gptq_status gptq_rmsnorm(const void* X, gptq_dtype xdt, int64_t ldx, const float* R, int64_t T, int64_t d,
                         double eps, float* H_out, uint16_t* Y, void* stream);
gptq_status gptq_rope(float* Q, float* K, int64_t T, int64_t d, int64_t head_dim, int64_t seq_len, double base,
                      void* stream);
gptq_status gptq_causal_attention(const float* Q, const float* K, const float* V, int64_t T, int64_t d,
                                  int64_t head_dim, int64_t seq_len, uint16_t* O, void* stream);
gptq_status gptq_silu_mul(const float* G, const float* U, int64_t count, uint16_t* Y, void* stream);

/* Message for the last failing call on this thread (empty string if none). */
const char* gptq_last_error(void);
/* Library version string. */
const char* gptq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_H */
