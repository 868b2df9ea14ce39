// Relative layer loss tr(D H D^T) / tr(W H W^T), D = W - W_hat.
//
// polydesk.ai "GPTQ" glossary, "Comment fonctionne l'algorithme GPTQ": the
// per-layer objective is the squared output error ||W X - W_hat X||^2; with
// H = (2/N) X X^T the ratio of the two traces equals the ratio of output errors.
// A measurement helper: dequantizes the packed outputs (exercising the storage
// format) and evaluates both quadratic forms with fp32 MFMA products.
#include "common.hpp"

namespace gptq {

// D[r][i] = W[r][i] - scale * (code - zero), Wf[r][i] = W[r][i], from the packed outputs.
template <int DT, int BITS>
__global__ void dequant_diff_kernel(const void* __restrict__ W, int64_t ldw, int rows, int n,
                                    const int32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
                                    const uint16_t* __restrict__ zeros, const int32_t* __restrict__ g_idx,
                                    float* __restrict__ D, float* __restrict__ Wf) {
  for (int r = blockIdx.y; r < rows; r += gridDim.y) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
      const int bit = BITS * i;
      const int wi = bit >> 5, off = bit & 31;
      uint32_t v = static_cast<uint32_t>(qweight[static_cast<int64_t>(wi) * rows + r]) >> off;
      if (off + BITS > 32) v |= static_cast<uint32_t>(qweight[static_cast<int64_t>(wi + 1) * rows + r]) << (32 - off);
      const float code = static_cast<float>(v & ((1u << BITS) - 1u));
      const int g = g_idx[i];
      const float sc = half_bits_to_float(scales[static_cast<int64_t>(g) * rows + r]);
      const float zp = half_bits_to_float(zeros[static_cast<int64_t>(g) * rows + r]);
      const float w = load_as_float<DT>(W, static_cast<int64_t>(r) * ldw + i);
      D[static_cast<int64_t>(r) * n + i] = w - sc * (code - zp);
      Wf[static_cast<int64_t>(r) * n + i] = w;
    }
  }
}

__global__ void h_to_f32_kernel(const double* __restrict__ H, int64_t count, float* __restrict__ Hf) {
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < count;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x)
    Hf[e] = static_cast<float>(H[e]);
}

// partial[tile] = sum over the 128x128 tile of A[r][c] * (A Hf)[r][c].
// Same MFMA tiling as the trailing update (v_mfma_f32_32x32x2f32, 2x2 per wave).
__global__ void __launch_bounds__(256) quad_form_kernel(const float* __restrict__ A, const float* __restrict__ Hf,
                                                        int rows, int n, double* __restrict__ partial) {
  __shared__ float sA[128][33];
  __shared__ float sH[32][129];
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r0 = blockIdx.y * 128, c0 = blockIdx.x * 128;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  for (int kc = 0; kc < n; kc += 32) {
    __syncthreads();
    for (int e = tid; e < 128 * 32; e += 256) {
      const int m = e >> 5, kk = e & 31;
      const int rr = r0 + m, k = kc + kk;
      sA[m][kk] = (rr < rows && k < n) ? A[static_cast<int64_t>(rr) * n + k] : 0.0f;
    }
    for (int e = tid; e < 32 * 128; e += 256) {
      const int kk = e >> 7, c = e & 127;
      const int k = kc + kk, cc = c0 + c;
      sH[kk][c] = (k < n && cc < n) ? Hf[static_cast<int64_t>(k) * n + cc] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int ks = 0; ks < 16; ++ks) {
      const int kk = ks * 2 + (lane >> 5);
      float fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = sA[wm * 64 + i * 32 + (lane & 31)][kk];
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = sH[kk][wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rr = r0 + wm * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const int cc = c0 + wn * 64 + j * 32 + (lane & 31);
        if (rr < rows && cc < n)
          s += static_cast<double>(acc[i][j][q]) * static_cast<double>(A[static_cast<int64_t>(rr) * n + cc]);
      }
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) partial[blockIdx.y * gridDim.x + blockIdx.x] = red[0];
}

__global__ void __launch_bounds__(256) ratio_kernel(const double* __restrict__ pn, const double* __restrict__ pd,
                                                    int count, double* __restrict__ out) {
  __shared__ double a[256], b[256];
  double sn = 0.0, sd = 0.0;
  for (int i = threadIdx.x; i < count; i += 256) {
    sn += pn[i];
    sd += pd[i];
  }
  a[threadIdx.x] = sn;
  b[threadIdx.x] = sd;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      a[threadIdx.x] += a[threadIdx.x + w];
      b[threadIdx.x] += b[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = a[0] / b[0];
}

static inline size_t al256l(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t loss_workspace(int64_t rows, int64_t n) {
  const size_t tiles = static_cast<size_t>((rows + 127) / 128) * ((n + 127) / 128);
  return 2 * al256l(static_cast<size_t>(rows) * n * 4) + al256l(static_cast<size_t>(n) * n * 4) +
         2 * al256l(tiles * 8) + 256;
}

hipError_t launch_layer_loss(const double* H, int64_t n64, const void* W, int wdt, int64_t rows64, int64_t ldw,
                             const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                             const int32_t* g_idx, int bits, double* rel_host, void* ws, hipStream_t s) {
  const int n = static_cast<int>(n64), rows = static_cast<int>(rows64);
  const int tr = (rows + 127) / 128, tc = (n + 127) / 128;
  const size_t tiles = static_cast<size_t>(tr) * tc;
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* D = reinterpret_cast<float*>(p);
  p += al256l(static_cast<size_t>(rows) * n * 4);
  float* Wf = reinterpret_cast<float*>(p);
  p += al256l(static_cast<size_t>(rows) * n * 4);
  float* Hf = reinterpret_cast<float*>(p);
  p += al256l(static_cast<size_t>(n) * n * 4);
  double* pn = reinterpret_cast<double*>(p);
  p += al256l(tiles * 8);
  double* pd = reinterpret_cast<double*>(p);
  p += al256l(tiles * 8);
  double* out = reinterpret_cast<double*>(p);

  dim3 g((n + 255) / 256, rows < 65535 ? rows : 65535);
#define GPTQ_DQ(DTV, B)                                                                                       \
  hipLaunchKernelGGL((dequant_diff_kernel<DTV, B>), g, dim3(256), 0, s, W, ldw, rows, n, qweight, scales, zeros, \
                     g_idx, D, Wf)
#define GPTQ_DQ_BITS(B)                         \
  do {                                          \
    if (wdt == DT_BF16) GPTQ_DQ(DT_BF16, B);    \
    else if (wdt == DT_FP16) GPTQ_DQ(DT_FP16, B); \
    else GPTQ_DQ(DT_FP32, B);                   \
  } while (0)
  if (bits == 2) GPTQ_DQ_BITS(2);
  else if (bits == 3) GPTQ_DQ_BITS(3);
  else if (bits == 4) GPTQ_DQ_BITS(4);
  else GPTQ_DQ_BITS(8);
#undef GPTQ_DQ_BITS
#undef GPTQ_DQ
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(h_to_f32_kernel, dim3(4096), dim3(256), 0, s, H, static_cast<int64_t>(n) * n, Hf);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(quad_form_kernel, dim3(tc, tr), dim3(256), 0, s, D, Hf, rows, n, pn);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(quad_form_kernel, dim3(tc, tr), dim3(256), 0, s, Wf, Hf, rows, n, pd);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(ratio_kernel, dim3(1), dim3(256), 0, s, pn, pd, static_cast<int>(tiles), out);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = hipMemcpyAsync(rel_host, out, sizeof(double), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace gptq
