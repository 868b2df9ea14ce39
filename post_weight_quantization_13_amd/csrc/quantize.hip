// Per-layer GPTQ sweep on gfx950: group-wise grid, fixed-order column sweep
// with error compensation, lazy block updates, packing.
//
// polydesk.ai "GPTQ" glossary:
//   "Étape 1 : Ordre arbitraire"  -- all rows visit the columns in one fixed order
//                                     (act-order permutation or identity),
//   "Étape 2 : Compensation d'erreur via la Hessienne" -- quantize a column,
//                                     e = (w - w_hat) / U[j, j], and push e onto the
//                                     later columns: W[:, k] -= e U[j, k],
//   "Étape 3 : Mises à jour par blocs" -- updates beyond the current block of 128
//                                     columns are delayed and applied as one product
//                                     W[:, i2:] -= E U[i1:i2, i2:],
//   "Paramètres clés" (sym)        -- symmetric grid with levels -(2^(b-1)-1)..2^(b-1)-1.
// skillmd.com "Gptq", "Quantização group-wise": one scale and zero point per
// group of 128 weights of a row.
//
// Kernels, per layer:
//   gather_w      W (bf16/fp16/fp32, original order) -> Wk fp32 [rows, n] in sweep
//                 order, dead columns zeroed.
//   sweep_block   one block of 128 columns for 64 rows per workgroup (lane = row):
//                 group scale/zero, the sequential quantize/compensate chain, codes,
//                 E for the block, fp16 scale/zero, per-row loss.
//   trailing      Wk[:, i2:] -= E U[i1:i2, i2:] with fp32 MFMA (v_mfma_f32_32x32x2f32).
//   pack          codes back to the original column order, little-endian bit stream
//                 per row, int32 words.
#include "common.hpp"

namespace gptq {

constexpr int kBlk = 128;     // lazy-batch block = group size
constexpr int kSub = 16;      // sub-block kept in registers inside the sweep
constexpr int kRowsSweep = 64;

// ---------------------------------------------------------------- gather
template <int DT>
__global__ void gather_w_kernel(const void* __restrict__ W, int64_t ldw, const int32_t* __restrict__ perm,
                                const uint8_t* __restrict__ dead, int rows, int n, float* __restrict__ Wk) {
  for (int r = blockIdx.y; r < rows; r += gridDim.y) {
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x) {
      const int src = perm[j];
      float v = dead[src] ? 0.0f : load_as_float<DT>(W, static_cast<int64_t>(r) * ldw + src);
      Wk[static_cast<int64_t>(r) * n + j] = v;
    }
  }
}

// g_idx[perm[j]] = j / gs;  invperm[perm[j]] = j.
__global__ void gidx_kernel(const int32_t* __restrict__ perm, int n, int gs, int32_t* __restrict__ g_idx,
                            int32_t* __restrict__ invperm) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int p = perm[j];
  g_idx[p] = j / gs;
  invperm[p] = j;
}

// ---------------------------------------------------------------- sweep
// Grid: ceil(rows / 64) workgroups of 64 threads (one wave).  LDS: the block
// of U transposed (UT[k][j] = U[i1+j][i1+k], 64 KB) and the 64 x 128 block of
// Wk column-major over lanes (32 KB).
template <int BITS, bool SYM>
__global__ void __launch_bounds__(64) sweep_block_kernel(
    float* __restrict__ Wk, const float* __restrict__ U, int n, int rows, int i1,
    uint8_t* __restrict__ codes, float* __restrict__ E, uint16_t* __restrict__ scales,
    uint16_t* __restrict__ zeros, double* __restrict__ rowloss) {
  __shared__ float UT[kBlk][kBlk];
  __shared__ float Ws[kBlk][kRowsSweep];
  const int lane = threadIdx.x;
  const int r = blockIdx.x * kRowsSweep + lane;
  const bool valid = r < rows;

  for (int e = lane; e < kBlk * kBlk; e += 64) {
    const int j = e / kBlk, k = e % kBlk;  // U row j, column k (coalesced read)
    UT[k][j] = U[static_cast<int64_t>(i1 + j) * n + i1 + k];
  }
  if (valid) {
    const float* wrow = Wk + static_cast<int64_t>(r) * n + i1;
    for (int k = 0; k < kBlk; k += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(wrow + k);
      Ws[k][lane] = v[0];
      Ws[k + 1][lane] = v[1];
      Ws[k + 2][lane] = v[2];
      Ws[k + 3][lane] = v[3];
    }
  } else {
    for (int k = 0; k < kBlk; ++k) Ws[k][lane] = 0.0f;
  }
  __syncthreads();

  // Group parameters from the block-entry values (group = block).
  constexpr float maxq = static_cast<float>((1 << BITS) - 1);
  float xmin = 0.0f, xmax = 0.0f;
  for (int k = 0; k < kBlk; ++k) {
    const float v = Ws[k][lane];
    xmin = fminf(xmin, v);
    xmax = fmaxf(xmax, v);
  }
  if (xmin == 0.0f && xmax == 0.0f) {
    xmin = -1.0f;
    xmax = 1.0f;
  }
  float s, z;
  if constexpr (SYM) {
    const float a = fmaxf(-xmin, xmax);
    s = a / static_cast<float>((1 << (BITS - 1)) - 1);
    z = static_cast<float>(1 << (BITS - 1));
  } else {
    s = (xmax - xmin) / maxq;
    z = rintf(-xmin / s);
  }
  const float lo = SYM ? 1.0f : 0.0f;

  double loss = 0.0;
  float* erow = E + static_cast<int64_t>(valid ? r : 0) * kBlk;
  uint8_t* crow = codes + static_cast<int64_t>(valid ? r : 0) * n + i1;
  for (int sb = 0; sb < kBlk / kSub; ++sb) {
    const int j0 = sb * kSub;
    float w[kSub], e[kSub];
#pragma unroll
    for (int t = 0; t < kSub; ++t) w[t] = Ws[j0 + t][lane];
#pragma unroll
    for (int t = 0; t < kSub; ++t) {
      const int j = j0 + t;
      const float c = fminf(fmaxf(rintf(w[t] / s) + z, lo), maxq);
      const float q = s * (c - z);
      const float et = (w[t] - q) / UT[j][j];
      e[t] = et;
      loss += static_cast<double>(et) * static_cast<double>(et);
      if (valid) crow[j] = static_cast<uint8_t>(c);
#pragma unroll
      for (int u = t + 1; u < kSub; ++u) w[u] = fmaf(-et, UT[j0 + u][j], w[u]);
    }
    if (valid) {
#pragma unroll
      for (int t = 0; t < kSub; t += 4) {
        *reinterpret_cast<f32x4*>(erow + j0 + t) = f32x4{e[t], e[t + 1], e[t + 2], e[t + 3]};
      }
    }
    // Apply this sub-block's errors to the rest of the block.
    for (int k = j0 + kSub; k < kBlk; ++k) {
      float acc = Ws[k][lane];
      const f32x4* ucol = reinterpret_cast<const f32x4*>(&UT[k][j0]);
#pragma unroll
      for (int t4 = 0; t4 < kSub / 4; ++t4) {
        const f32x4 u = ucol[t4];
        acc = fmaf(-e[4 * t4 + 0], u[0], acc);
        acc = fmaf(-e[4 * t4 + 1], u[1], acc);
        acc = fmaf(-e[4 * t4 + 2], u[2], acc);
        acc = fmaf(-e[4 * t4 + 3], u[3], acc);
      }
      Ws[k][lane] = acc;
    }
  }
  if (valid) {
    const int g = i1 / kBlk;
    scales[static_cast<int64_t>(g) * rows + r] = float_to_half_bits(s);
    zeros[static_cast<int64_t>(g) * rows + r] = float_to_half_bits(z);
    rowloss[r] += 0.5 * loss;
  }
}

// ---------------------------------------------------------------- trailing update
// Wk[r0:r0+128, c0:c0+128] -= E[r0:r0+128, 0:128] U[i1:i1+128, c0:c0+128],
// c0 = i2 + 128*blockIdx.x, r0 = 128*blockIdx.y.  256 threads; wave (wm, wn)
// owns a 64x64 quarter = 2x2 tiles of v_mfma_f32_32x32x2f32 (lane l supplies
// A[l%32][l/32] and B[l/32][l%32]; accumulator r is D[8(r/4)+4(l/32)+r%4][l%32]).
__global__ void __launch_bounds__(256) trailing_kernel(float* __restrict__ Wk, const float* __restrict__ E,
                                                       const float* __restrict__ U, int n, int rows, int i1,
                                                       int i2) {
  __shared__ float sE[128][33];
  __shared__ float sU[32][129];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r0 = blockIdx.y * 128;
  const int c0 = i2 + blockIdx.x * 128;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  for (int kc = 0; kc < kBlk; kc += 32) {
    __syncthreads();
    for (int e = tid; e < 128 * 32; e += 256) {
      const int m = e >> 5, kk = e & 31;
      const int rr = r0 + m;
      sE[m][kk] = (rr < rows) ? E[static_cast<int64_t>(rr) * kBlk + kc + kk] : 0.0f;
    }
    for (int e = tid; e < 32 * 128; e += 256) {
      const int kk = e >> 7, c = e & 127;
      const int cc = c0 + c;
      sU[kk][c] = (cc < n) ? U[static_cast<int64_t>(i1 + kc + kk) * n + cc] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int ks = 0; ks < 16; ++ks) {
      const int kk = ks * 2 + (lane >> 5);
      float fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = sE[wm * 64 + i * 32 + (lane & 31)][kk];
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = sU[kk][wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rr = r0 + wm * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const int cc = c0 + wn * 64 + j * 32 + (lane & 31);
        if (rr < rows && cc < n) Wk[static_cast<int64_t>(rr) * n + cc] -= acc[i][j][q];
      }
}

// ---------------------------------------------------------------- pack
// Thread per (row r, chunk c of 32 original columns): the 32 codes form a
// 32*BITS-bit little-endian stream written as BITS words qweight[c*BITS + t, r].
template <int BITS>
__global__ void pack_kernel(const uint8_t* __restrict__ codes, const int32_t* __restrict__ invperm, int n,
                            int rows, int32_t* __restrict__ qweight) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  const int c = blockIdx.y;
  if (r >= rows) return;
  const uint8_t* crow = codes + static_cast<int64_t>(r) * n;
  uint32_t words[BITS];
#pragma unroll
  for (int t = 0; t < BITS; ++t) words[t] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t v = crow[invperm[c * 32 + i]];
    const int bit = BITS * i;
    const int wi = bit >> 5, off = bit & 31;
    words[wi] |= v << off;
    if (off + BITS > 32) words[wi + 1] |= v >> (32 - off);
  }
#pragma unroll
  for (int t = 0; t < BITS; ++t) qweight[static_cast<int64_t>(c * BITS + t) * rows + r] = static_cast<int32_t>(words[t]);
}

// Fixed-order sum of the per-row losses.
__global__ void __launch_bounds__(256) loss_reduce_kernel(const double* __restrict__ rowloss, int rows,
                                                          double* __restrict__ out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < rows; i += 256) s += rowloss[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

// ---------------------------------------------------------------- host launcher
static inline size_t al256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t quantize_workspace(int64_t rows, int64_t n) {
  return al256(static_cast<size_t>(rows) * n * 4)      // Wk
         + al256(static_cast<size_t>(rows) * kBlk * 4) // E block
         + al256(static_cast<size_t>(rows) * n)        // codes
         + al256(static_cast<size_t>(rows) * 8)        // rowloss
         + al256(static_cast<size_t>(n) * 4)           // invperm
         + 256;                                        // loss scalar
}

template <int BITS, bool SYM>
static void launch_sweep(dim3 g, hipStream_t s, float* Wk, const float* U, int n, int rows, int i1, uint8_t* codes,
                         float* E, uint16_t* scales, uint16_t* zeros, double* rowloss) {
  hipLaunchKernelGGL((sweep_block_kernel<BITS, SYM>), g, dim3(64), 0, s, Wk, U, n, rows, i1, codes, E, scales,
                     zeros, rowloss);
}

hipError_t launch_quantize(const float* U, const int32_t* perm, const uint8_t* dead, int64_t n64, int bits,
                           int sym, const void* W, int wdt, int64_t rows64, int64_t ldw, int32_t* qweight,
                           uint16_t* scales, uint16_t* zeros, int32_t* g_idx, double* loss_host, void* ws,
                           hipStream_t s) {
  const int n = static_cast<int>(n64), rows = static_cast<int>(rows64);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* Wk = reinterpret_cast<float*>(p);
  p += al256(static_cast<size_t>(rows) * n * 4);
  float* E = reinterpret_cast<float*>(p);
  p += al256(static_cast<size_t>(rows) * kBlk * 4);
  uint8_t* codes = p;
  p += al256(static_cast<size_t>(rows) * n);
  double* rowloss = reinterpret_cast<double*>(p);
  p += al256(static_cast<size_t>(rows) * 8);
  int32_t* invperm = reinterpret_cast<int32_t*>(p);
  p += al256(static_cast<size_t>(n) * 4);
  double* loss_dev = reinterpret_cast<double*>(p);

  hipError_t e;
#define GPTQ_CHECK_LAUNCH()        \
  do {                             \
    e = hipGetLastError();         \
    if (e != hipSuccess) return e; \
  } while (0)
  e = hipMemsetAsync(rowloss, 0, static_cast<size_t>(rows) * 8, s);
  if (e != hipSuccess) return e;
  dim3 gg((n + 255) / 256, rows < 65535 ? rows : 65535);
  if (wdt == DT_BF16) hipLaunchKernelGGL(gather_w_kernel<DT_BF16>, gg, dim3(256), 0, s, W, ldw, perm, dead, rows, n, Wk);
  else if (wdt == DT_FP16) hipLaunchKernelGGL(gather_w_kernel<DT_FP16>, gg, dim3(256), 0, s, W, ldw, perm, dead, rows, n, Wk);
  else hipLaunchKernelGGL(gather_w_kernel<DT_FP32>, gg, dim3(256), 0, s, W, ldw, perm, dead, rows, n, Wk);
  GPTQ_CHECK_LAUNCH();
  hipLaunchKernelGGL(gidx_kernel, dim3((n + 255) / 256), dim3(256), 0, s, perm, n, kBlk, g_idx, invperm);
  GPTQ_CHECK_LAUNCH();

  const dim3 gs((rows + kRowsSweep - 1) / kRowsSweep);
  for (int i1 = 0; i1 < n; i1 += kBlk) {
    const int i2 = i1 + kBlk;
    if (bits == 4 && !sym) launch_sweep<4, false>(gs, s, Wk, U, n, rows, i1, codes, E, scales, zeros, rowloss);
    else if (bits == 4 && sym) launch_sweep<4, true>(gs, s, Wk, U, n, rows, i1, codes, E, scales, zeros, rowloss);
    else if (bits == 3 && !sym) launch_sweep<3, false>(gs, s, Wk, U, n, rows, i1, codes, E, scales, zeros, rowloss);
    else launch_sweep<3, true>(gs, s, Wk, U, n, rows, i1, codes, E, scales, zeros, rowloss);
    GPTQ_CHECK_LAUNCH();
    if (i2 < n) {
      dim3 gt((n - i2 + 127) / 128, (rows + 127) / 128);
      hipLaunchKernelGGL(trailing_kernel, gt, dim3(256), 0, s, Wk, E, U, n, rows, i1, i2);
      GPTQ_CHECK_LAUNCH();
    }
  }
  dim3 gp((rows + 255) / 256, n / 32);  // n <= 65535 * 32 is checked by the caller
  if (bits == 4) hipLaunchKernelGGL(pack_kernel<4>, gp, dim3(256), 0, s, codes, invperm, n, rows, qweight);
  else hipLaunchKernelGGL(pack_kernel<3>, gp, dim3(256), 0, s, codes, invperm, n, rows, qweight);
  GPTQ_CHECK_LAUNCH();
  if (loss_host) {
    hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(256), 0, s, rowloss, rows, loss_dev);
    GPTQ_CHECK_LAUNCH();
    e = hipMemcpyAsync(loss_host, loss_dev, sizeof(double), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return e;
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
  }
#undef GPTQ_CHECK_LAUNCH
  return hipSuccess;
}

}  // namespace gptq
