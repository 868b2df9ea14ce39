// Forward of one decoder block on gfx950, for block-sequential calibration.
//
// wikiprompt.org "GPTQ", "Approche technique": the layers are treated one after
// another; polydesk.ai "GPTQ", "Comment fonctionne l'algorithme GPTQ": each
// linear is solved on the input activations that calibration data produce.
// Inside a Llama-2-shaped block the inputs of o_proj and down_proj are
// therefore produced by the already-quantized q/k/v and gate/up projections
// (gptq_matmul, fp32 outputs) through the pieces below:
//   rmsnorm_kernel      y = fp16(h / sqrt(mean(h^2) + eps)), h = x (+ residual)
//   rope_kernel         rotary embedding of q and k, in place (fp32)
//   attention_kernel    causal softmax(q k^T / sqrt(128)) v per head -> fp16
//   silu_mul_kernel     y = fp16(silu(g) * u)
// Every linear's input is held in fp16 (rounded to nearest even), the form the
// dequantizing matmul reads.  The row statistics of the norm, the rotation
// angles and the gating are computed in fp64 so that the only rounding that
// matters is the final one to fp16; the attention runs in fp32.
#include "common.hpp"

#include <cmath>

namespace gptq {
namespace {

// ---------------------------------------------------------------- fp64 -> fp16
__device__ __forceinline__ double half_value(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return static_cast<double>(h);
}

// Next fp16 bit pattern toward +inf / -inf (finite inputs).
__device__ __forceinline__ uint16_t half_up(uint16_t b) {
  if (b & 0x8000u) return b == 0x8000u ? uint16_t(1) : uint16_t(b - 1);
  return uint16_t(b + 1);
}
__device__ __forceinline__ uint16_t half_down(uint16_t b) {
  if (b & 0x8000u) return uint16_t(b + 1);
  return b == 0 ? uint16_t(0x8001u) : uint16_t(b - 1);
}

// fp64 -> fp16 bit pattern, round to nearest even, in one rounding: the
// conversion through fp32 can round twice when the fp32 value falls exactly
// on an fp16 midpoint; the neighbour on v's side is then the nearer one.
__device__ __forceinline__ uint16_t double_to_half_bits(double v) {
  uint16_t b = float_to_half_bits(static_cast<float>(v));
  const double hv = half_value(b);
  if (hv != v && fabs(hv) < 65504.0) {
    const uint16_t nb = v > hv ? half_up(b) : half_down(b);
    if (fabs(v - half_value(nb)) < fabs(v - hv)) b = nb;
  }
  return b;
}

// ---------------------------------------------------------------- RMSNorm
// One wave per row: h = x + r (r optional, fp32), s = sum h^2 in fp64,
// y = fp16(h / sqrt(s / d + eps)); h is also written as fp32 when hout != null.
template <int DT>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ X, int64_t ldx,
                                                      const float* __restrict__ R, int64_t T, int d, double eps,
                                                      float* __restrict__ hout, uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  const int64_t xo = row * ldx, ro = row * static_cast<int64_t>(d);
  double ss = 0.0;
  for (int c = lane; c < d; c += 64) {
    double h = load_as_float<DT>(X, xo + c);
    if (R) h += R[ro + c];
    ss = fma(h, h, ss);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  const double inv = 1.0 / sqrt(ss / d + eps);
  for (int c = lane; c < d; c += 64) {
    double h = load_as_float<DT>(X, xo + c);
    if (R) h += R[ro + c];
    if (hout) hout[ro + c] = static_cast<float>(h);
    Y[ro + c] = double_to_half_bits(h * inv);
  }
}

// ---------------------------------------------------------------- RoPE
// Thread (t, i): position p = t mod L, frequency base^(-2i/hd); rotates the
// pair (i, i + hd/2) of every head of q and k at token t.  Angle and its sine
// and cosine in fp64, the rotation in fp32.
__global__ __launch_bounds__(256) void rope_kernel(float* __restrict__ Q, float* __restrict__ K, int64_t T, int d,
                                                   int hd, int L, double base) {
  const int half = hd / 2;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= T * half) return;
  const int64_t t = id / half;
  const int i = static_cast<int>(id % half);
  const double ang = static_cast<double>(t % L) * pow(base, -2.0 * i / hd);
  double sd, cd;
  sincos(ang, &sd, &cd);
  const float s = static_cast<float>(sd), c = static_cast<float>(cd);
  float* q = Q + t * d;
  float* k = K + t * d;
  for (int h = 0; h < d / hd; ++h) {
    const int a = h * hd + i, b = a + half;
    const float qa = q[a], qb = q[b], ka = k[a], kb = k[b];
    q[a] = qa * c - qb * s;
    q[b] = qb * c + qa * s;
    k[a] = ka * c - kb * s;
    k[b] = kb * c + ka * s;
  }
}

// ---------------------------------------------------------------- attention
// Work-group: 64 queries of one head of one sequence, wave w owning queries
// 16w .. 16w+15; keys in steps of 64 with an online softmax (running max and
// sum per query).  Both products run on the fp32 MFMA 16x16x4, transposed so
// that a lane's query never changes:
//   scores  S^T = K Q^T: A = a key row from LDS, B = the lane's own query
//           (128 dims held in registers), 32 steps over the head dimension;
//           lane (i, g) = (lane % 16, lane / 16) gets keys 16t + 4g + r of
//           query i for r = 0..3;
//   output  O^T += V^T P^T: B = those same probabilities, straight from the
//           lane's registers (the MFMA's k index r is the key 16t + 4g + r),
//           A = V[16t + 4g + r][16u + i] read from LDS one float at a time;
//           lane (i, g) holds dims 16u + 4g + r of query i.
// The dimension order of a dot product is free as long as K and Q agree: lane
// group g takes the 32 dims 32 s(g) .. 32 s(g) + 31, s = (0, 2, 1, 3), so a K
// fragment is a 16-byte LDS read.  K and V are staged as loaded, rows padded
// to 132 floats.  A 16-byte LDS read on this chip serves each half-wave in two
// cycles, lanes split by the parity of lane bits 2-4, and is conflict-free
// when each such set of 16 lanes touches 16 distinct 16-byte bank groups
// (measured with a probe): with 132-float rows the order s meets that, the
// plain order g conflicts 2-way.  A V read puts lane (i, g) on bank 16g + i
// (+ a constant).  (V staged transposed, for 16-byte reads, took 4-byte
// writes that met eight to a bank.)  fp32 products and sums; the
// output is divided by the softmax sum and rounded to fp16 once.  Query
// blocks are dealt longest first (the causal key range grows with them).
constexpr int kHD = 128;
constexpr int kQB = 64;
constexpr int kKB = 64;
constexpr int kKRow = kHD + 4;
struct AttnSmem {
  float k[kKB][kKRow];
  float v[kKB][kKRow];
};

__global__ __launch_bounds__(256, 2) void attention_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                           const float* __restrict__ V, int d, int L,
                                                           uint16_t* __restrict__ O) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnSmem& sm = *reinterpret_cast<AttnSmem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int q0 = (gridDim.x - 1 - blockIdx.x) * kQB;
  const int64_t base = static_cast<int64_t>(blockIdx.z) * L;
  const int col = blockIdx.y * kHD;
  const int qi = q0 + 16 * wave + i16;   // this lane's query; past L it reads row L - 1, output dropped
  const float scale = 0.08838834764831845f;   // 1 / sqrt(128)

  const int gs32 = 32 * (2 * (g & 1) + (g >> 1));   // this lane group's 32 dims
  float qf[32];
  {
    const float* qp = Q + (base + min(qi, L - 1)) * d + col + gs32;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(qp + 4 * v);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * v + e] = t[e];
    }
  }
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;   // lsum: this lane's share of the query's sum

  // K and V of a key step, 8 pieces of 16 bytes each per thread; rows past
  // L re-read row L - 1 (their scores are masked, their probabilities 0)
  f32x4 kreg[8], vreg[8];
  auto load = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int e = tid + 256 * r, row = min(k0 + (e >> 5), L - 1), c4 = (e & 31) * 4;
      kreg[r] = *reinterpret_cast<const f32x4*>(K + (base + row) * d + col + c4);
      vreg[r] = *reinterpret_cast<const f32x4*>(V + (base + row) * d + col + c4);
    }
  };
  const int kend = min(q0 + kQB, L);
  const int klast = (kend - 1) / kKB * kKB;
  load(0);
  for (int k0 = 0; k0 < kend; k0 += kKB) {
    __syncthreads();   // every wave is done with the previous step's tiles
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int e = tid + 256 * r, row = e >> 5, c4 = (e & 31) * 4;
      *reinterpret_cast<f32x4*>(&sm.k[row][c4]) = kreg[r];
      *reinterpret_cast<f32x4*>(&sm.v[row][c4]) = vreg[r];
    }
    __syncthreads();
    // the next step's tiles load while this one is computed (the last step
    // re-reads its own: no branch around the loads)
    load(min(k0 + kKB, klast));
    __builtin_amdgcn_sched_barrier(0);
    f32x4 st[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x4 kf = *reinterpret_cast<const f32x4*>(&sm.k[16 * t + i16][gs32 + 4 * c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) st[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[e], qf[4 * c + e], st[t], 0, 0, 0);
      }
    }
    float bm = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kj = k0 + 16 * t + 4 * g + r;
        st[t][r] = (kj <= qi && kj < L) ? st[t][r] * scale : -INFINITY;
        bm = fmaxf(bm, st[t][r]);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float mn = fmaxf(m, bm);   // key k0 <= q0 <= qi and k0 < L: finite
    const float alpha = expf(m - mn);
    float bs = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st[t][r] = expf(st[t][r] - mn);
        bs += st[t][r];
      }
    lsum = lsum * alpha + bs;
    m = mn;
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[u][r] *= alpha;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.v[16 * t + 4 * g + r][16 * u + i16], st[t][r], acc[u], 0, 0, 0);
      }
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (qi < L) {
    const float inv = 1.0f / lsum;
    uint16_t* o = O + (base + qi) * d + col + 4 * g;
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[16 * u + r] = float_to_half_bits(acc[u][r] * inv);
  }
}

// ---------------------------------------------------------------- SiLU gate
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ G, const float* __restrict__ U,
                                                       int64_t count, uint16_t* __restrict__ Y) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const double gv = G[i];
    Y[i] = double_to_half_bits(gv / (1.0 + exp(-gv)) * static_cast<double>(U[i]));
  }
}

}  // namespace

int attention_head_dim() { return kHD; }

hipError_t launch_rmsnorm(const void* X, int dt, int64_t ldx, const float* R, int64_t T, int64_t d, double eps,
                          float* hout, uint16_t* Y, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>((T + 3) / 4);
  const int dd = static_cast<int>(d);
  switch (dt) {
    case DT_BF16: hipLaunchKernelGGL(rmsnorm_kernel<DT_BF16>, dim3(blocks), dim3(256), 0, s, X, ldx, R, T, dd, eps, hout, Y); break;
    case DT_FP16: hipLaunchKernelGGL(rmsnorm_kernel<DT_FP16>, dim3(blocks), dim3(256), 0, s, X, ldx, R, T, dd, eps, hout, Y); break;
    case DT_FP32: hipLaunchKernelGGL(rmsnorm_kernel<DT_FP32>, dim3(blocks), dim3(256), 0, s, X, ldx, R, T, dd, eps, hout, Y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rope(float* Q, float* K, int64_t T, int64_t d, int64_t hd, int64_t L, double base, hipStream_t s) {
  const int64_t threads = T * (hd / 2);
  hipLaunchKernelGGL(rope_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s, Q, K, T,
                     static_cast<int>(d), static_cast<int>(hd), static_cast<int>(L), base);
  return hipGetLastError();
}

hipError_t launch_attention(const float* Q, const float* K, const float* V, int64_t T, int64_t d, int64_t L,
                            uint16_t* O, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(attention_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sizeof(AttnSmem)));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(static_cast<unsigned>((L + kQB - 1) / kQB), static_cast<unsigned>(d / kHD), static_cast<unsigned>(T / L));
  hipLaunchKernelGGL(attention_kernel, grid, dim3(256), sizeof(AttnSmem), s, Q, K, V, static_cast<int>(d),
                     static_cast<int>(L), O);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* G, const float* U, int64_t count, uint16_t* Y, hipStream_t s) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(silu_mul_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, G, U, count, Y);
  return hipGetLastError();
}

}  // namespace gptq
