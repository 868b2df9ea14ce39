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
//   sweep_block   one block of 128 columns for 64 rows per workgroup (lane = row;
//                 one wave runs the sequential chain, three apply its errors):
//                 group scale/zero, quantize/compensate, codes, E for the block,
//                 fp16 scale/zero, per-row loss.
//   trailing      Wk[:, i2:] -= E U[i1:i2, i2:] as a split-bf16 product on the bf16
//                 MFMA (three products per operand pair, fp32 accumulation).
//   pack          codes back to the original column order, little-endian bit stream
//                 per row, int32 words.
#include <type_traits>

#include "common.hpp"

namespace gptq {

constexpr int kBlk = 128;     // lazy-batch block = group size
constexpr int kSuper = 512;   // columns per outer lazy batch (a multiple of kBlk)
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
// One workgroup (4 waves) per strip of 64 rows and one block of 128 columns;
// lane = row in every wave.  LDS: UT[k][j] = U[i1+j][i1+k] (the block of U,
// transposed), the 64x128 block of Wk column-major over rows, and the errors
// of the last two 16-column sub-blocks.
// Sub-block s (16 columns), two barriers:
//   wave 0   : the sequential chain -- quantize column j, e_j = (w - q) / U_jj,
//              rank-1 update of the remaining columns of the sub-block (the
//              16x16 block of U is read into registers first);
//   waves 1-3: meanwhile apply the errors of sub-block s-1 to the columns past
//              sub-block s+1 ("far" update);
//   barrier; all waves apply the errors of sub-block s to the columns of
//   sub-block s+1 ("near" update, which the next chain step needs); barrier.
// Codes: c = clamp(rint(w / s) + z).  Each sub-block's chain first runs with
// the quotient formed as w * (1/s).  If any quotient lay within 2^-18 of a
// rounding midpoint (that form errs by at most ~2 ulp = 2^-18 for |w/s| < 16,
// the only range where rint decides a code), the sub-block is replayed from
// its saved inputs with IEEE division, so the codes equal those of a
// correctly rounded w / s.  The fast path has no branch inside the chain.
constexpr int kSubs = kBlk / kSub;  // 8

template <int BITS, bool SYM>
__global__ void __launch_bounds__(256) sweep_block_kernel(
    float* __restrict__ Wk, const float* __restrict__ U, int n, int rows, int i1,
    uint8_t* __restrict__ codes, float* __restrict__ E, int ldE, uint16_t* __restrict__ scales,
    uint16_t* __restrict__ zeros, double* __restrict__ rowloss) {
  __shared__ __attribute__((aligned(16))) float UT[kBlk][kBlk + 4];
  __shared__ float Ws[kBlk][kRowsSweep];
  __shared__ float Es[2][kSub][kRowsSweep];
  __shared__ float rdiag[kBlk];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = blockIdx.x * kRowsSweep + lane;
  const bool valid = r < rows;

  // Staging: every global load of the block is issued before the LDS stores.
  {
    f32x4 ut[16];  // U rows: unit i -> row j = e4 / 32, columns 4*(e4 % 32) ..
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e4 = tid + 256 * i;
      ut[i] = *reinterpret_cast<const f32x4*>(U + static_cast<int64_t>(i1 + (e4 >> 5)) * n + i1 + 4 * (e4 & 31));
    }
    // Ws[k][row]: thread -> (row rr, quarter q of 32 columns)
    const int rr = tid >> 2, q = tid & 3;
    const int gr = blockIdx.x * kRowsSweep + rr;
    f32x4 wv[8];
#pragma unroll
    for (int k4 = 0; k4 < 8; ++k4)
      wv[k4] = (gr < rows) ? *reinterpret_cast<const f32x4*>(Wk + static_cast<int64_t>(gr) * n + i1 + q * 32 + 4 * k4)
                           : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float dg = (tid < kBlk) ? U[static_cast<int64_t>(i1 + tid) * n + i1 + tid] : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e4 = tid + 256 * i;
      const int j = e4 >> 5, k = 4 * (e4 & 31);
      UT[k][j] = ut[i][0];
      UT[k + 1][j] = ut[i][1];
      UT[k + 2][j] = ut[i][2];
      UT[k + 3][j] = ut[i][3];
    }
#pragma unroll
    for (int k4 = 0; k4 < 8; ++k4) {
      Ws[q * 32 + 4 * k4 + 0][rr] = wv[k4][0];
      Ws[q * 32 + 4 * k4 + 1][rr] = wv[k4][1];
      Ws[q * 32 + 4 * k4 + 2][rr] = wv[k4][2];
      Ws[q * 32 + 4 * k4 + 3][rr] = wv[k4][3];
    }
    if (tid < kBlk) rdiag[tid] = 1.0f / dg;
  }
  __syncthreads();

  constexpr float maxq = static_cast<float>((1 << BITS) - 1);
  const float lo = SYM ? 1.0f : 0.0f;
  float sv = 1.0f, zv = 0.0f, rs = 1.0f;
  double loss = 0.0;
  if (wave == 0) {
    // group parameters from the block-entry values (group = block)
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
    if constexpr (SYM) {
      const float a = fmaxf(-xmin, xmax);
      sv = a / static_cast<float>((1 << (BITS - 1)) - 1);
      zv = static_cast<float>(1 << (BITS - 1));
    } else {
      sv = (xmax - xmin) / maxq;
      zv = rintf(-xmin / sv);
    }
    rs = 1.0f / sv;
  }

  float* erow = E + static_cast<int64_t>(valid ? r : 0) * ldE;
  uint8_t* crow = codes + static_cast<int64_t>(valid ? r : 0) * n + i1;
  for (int sb = 0; sb < kSubs; ++sb) {
    const int j0 = sb * kSub;
    if (wave == 0) {
      float w0[kSub];
#pragma unroll
      for (int t = 0; t < kSub; ++t) w0[t] = Ws[j0 + t][lane];
      // The 16x16 diagonal sub-block of U in registers (uniform values), read
      // as LDS broadcasts: ub[t][u] = U[j0+t][j0+u] = UT[j0+u][j0+t].
      float ub[kSub][kSub];
#pragma unroll
      for (int u = 1; u < kSub; ++u) {
#pragma unroll
        for (int t4 = 0; t4 < kSub / 4; ++t4) {
          if (4 * t4 >= u) continue;
          const f32x4 v = *reinterpret_cast<const f32x4*>(&UT[j0 + u][j0 + 4 * t4]);
          ub[4 * t4][u] = v[0];
          ub[4 * t4 + 1][u] = v[1];
          ub[4 * t4 + 2][u] = v[2];
          ub[4 * t4 + 3][u] = v[3];
        }
      }
      // The chain of one sub-block.  EXACT = false forms w / s as w * (1/s)
      // and reports whether any quotient came within 2^-18 of a rounding
      // midpoint; EXACT = true uses IEEE division throughout.
      auto chain = [&](auto exact_tag, uint32_t (&cw)[kSub / 4], float& lsum) -> bool {
        constexpr bool EXACT = decltype(exact_tag)::value;
        float w[kSub];
#pragma unroll
        for (int t = 0; t < kSub; ++t) w[t] = w0[t];
        bool near = false;
#pragma unroll
        for (int t = 0; t < kSub; ++t) {
          float qt;
          if constexpr (EXACT) {
            qt = w[t] / sv;
          } else {
            qt = w[t] * rs;
            near |= fabsf(fabsf(qt - rintf(qt)) - 0.5f) < 3.814697265625e-06f;
          }
          const float c = fminf(fmaxf(rintf(qt) + zv, lo), maxq);
          const float q = sv * (c - zv);
          const float et = (w[t] - q) * rdiag[j0 + t];
          Es[sb & 1][t][lane] = et;
          lsum = fmaf(et, et, lsum);
          cw[t >> 2] |= static_cast<uint32_t>(c) << (8 * (t & 3));
#pragma unroll
          for (int u = t + 1; u < kSub; ++u) w[u] = fmaf(-et, ub[t][u], w[u]);
        }
        return near;
      };
      uint32_t cw[kSub / 4] = {0u, 0u, 0u, 0u};
      float lsum = 0.0f;
      const bool near = chain(std::false_type{}, cw, lsum);
      if (__builtin_expect(__any(near), 0)) {  // rare: replay with IEEE division
#pragma unroll
        for (int t4 = 0; t4 < kSub / 4; ++t4) cw[t4] = 0u;
        lsum = 0.0f;
        chain(std::true_type{}, cw, lsum);
      }
      loss += static_cast<double>(lsum);
      if (valid) {
#pragma unroll
        for (int t4 = 0; t4 < kSub / 4; ++t4) {
          *reinterpret_cast<uint32_t*>(crow + j0 + 4 * t4) = cw[t4];
          *reinterpret_cast<f32x4*>(erow + j0 + 4 * t4) =
              f32x4{Es[sb & 1][4 * t4][lane], Es[sb & 1][4 * t4 + 1][lane], Es[sb & 1][4 * t4 + 2][lane],
                    Es[sb & 1][4 * t4 + 3][lane]};
        }
      }
    } else if (sb >= 1) {
      // far update: errors of sub-block sb-1 onto columns >= j0 + 16
      const int jp = j0 - kSub;
      float ep[kSub];
#pragma unroll
      for (int t = 0; t < kSub; ++t) ep[t] = Es[(sb - 1) & 1][t][lane];
      // columns k = j0 + 16 + (wave-1) + 3m, four per pass with the loads first
      for (int k = j0 + kSub + (wave - 1); k < kBlk; k += 12) {
        float acc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = (k + 3 * q < kBlk) ? Ws[k + 3 * q][lane] : 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kq = (k + 3 * q < kBlk) ? k + 3 * q : k;
          const f32x4* uc = reinterpret_cast<const f32x4*>(&UT[kq][jp]);
#pragma unroll
          for (int t4 = 0; t4 < kSub / 4; ++t4) {
            const f32x4 u = uc[t4];
            acc[q] = fmaf(-ep[4 * t4 + 0], u[0], acc[q]);
            acc[q] = fmaf(-ep[4 * t4 + 1], u[1], acc[q]);
            acc[q] = fmaf(-ep[4 * t4 + 2], u[2], acc[q]);
            acc[q] = fmaf(-ep[4 * t4 + 3], u[3], acc[q]);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (k + 3 * q < kBlk) Ws[k + 3 * q][lane] = acc[q];
      }
    }
    __syncthreads();
    if (sb + 1 < kSubs) {
      // near update: errors of sub-block sb onto the 16 columns of sub-block sb+1
      float ec[kSub];
#pragma unroll
      for (int t = 0; t < kSub; ++t) ec[t] = Es[sb & 1][t][lane];
      const int kn = j0 + kSub + wave * (kSub / 4);
      float acc[kSub / 4];
#pragma unroll
      for (int kk = 0; kk < kSub / 4; ++kk) acc[kk] = Ws[kn + kk][lane];
#pragma unroll
      for (int kk = 0; kk < kSub / 4; ++kk) {
        const f32x4* uc = reinterpret_cast<const f32x4*>(&UT[kn + kk][j0]);
#pragma unroll
        for (int t4 = 0; t4 < kSub / 4; ++t4) {
          const f32x4 u = uc[t4];
          acc[kk] = fmaf(-ec[4 * t4 + 0], u[0], acc[kk]);
          acc[kk] = fmaf(-ec[4 * t4 + 1], u[1], acc[kk]);
          acc[kk] = fmaf(-ec[4 * t4 + 2], u[2], acc[kk]);
          acc[kk] = fmaf(-ec[4 * t4 + 3], u[3], acc[kk]);
        }
      }
#pragma unroll
      for (int kk = 0; kk < kSub / 4; ++kk) Ws[kn + kk][lane] = acc[kk];
      __syncthreads();
    }
  }
  if (wave == 0 && valid) {
    const int g = i1 / kBlk;
    scales[static_cast<int64_t>(g) * rows + r] = float_to_half_bits(sv);
    zeros[static_cast<int64_t>(g) * rows + r] = float_to_half_bits(zv);
    rowloss[r] += 0.5 * loss;
  }
}

// ---------------------------------------------------------------- trailing update
// Wk[r0:r0+128, c0:c0+128] -= E[r0:r0+128, 0:K] U[i1:i1+K, c0:c0+128] for
// columns c < ce, c0 = cb + 128*blockIdx.x, r0 = 128*blockIdx.y; E has row
// stride ldE.
// Split-bf16 product on the bf16 MFMA: each fp32 operand x = hi + lo with
// hi = bf16(x), lo = bf16(x - hi) (round to nearest even), and
//   E U ~ Ehi Uhi + Ehi Ulo + Elo Uhi   (fp32 accumulation),
// which leaves a relative error near 2^-16 per product (the dropped Elo Ulo
// term and the rounding of lo), against 2^-24 for an fp32 product.
// K runs in chunks of 64 staged in LDS as bf16 hi/lo planes: E as [row][k], U
// transposed as [col][k], so each MFMA operand fragment (8 consecutive k) is
// one 16-byte read; the next chunk's global loads are in flight during the
// current chunk's MFMAs.  The 16-byte chunk c of a 128-byte row r sits at slot
// c ^ (r & 7), which keeps the fragment reads conflict-free.
// 256 threads; wave (wm, wn) owns a 64x64 quarter = 2x2 v_mfma_f32_32x32x16_bf16
// tiles (accumulator q of lane l is row 8(q/4) + 4(l/32) + q%4, column l%32).
constexpr int kTK = 64;

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// 8 fp32 values -> hi and lo bf16 planes (16 bytes each).
__device__ __forceinline__ void split8(const float (&v)[8], u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t h0 = bf16_rne_bits(v[2 * d]), h1 = bf16_rne_bits(v[2 * d + 1]);
    const uint32_t l0 = bf16_rne_bits(v[2 * d] - __uint_as_float(h0 << 16));
    const uint32_t l1 = bf16_rne_bits(v[2 * d + 1] - __uint_as_float(h1 << 16));
    hi[d] = h0 | (h1 << 16);
    lo[d] = l0 | (l1 << 16);
  }
}

__device__ __forceinline__ int tk_offset(int row, int c) { return row * (kTK * 2) + ((c ^ (row & 7)) << 4); }

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, f32x16 c) {
  bf16x8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

__global__ void __launch_bounds__(256, 2) trailing_kernel(float* __restrict__ Wk, const float* __restrict__ E,
                                                       int ldE, const float* __restrict__ U, int n, int rows,
                                                       int i1, int K, int cb, int ce) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4][128 * kTK * 2];  // Ehi, Elo, Uhi, Ulo: 64 KB
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r0 = blockIdx.y * 128;
  const int c0 = cb + blockIdx.x * 128;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  float ev[4][8], uv[4][8];
  auto gload = [&](int kc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // E: unit -> (row, k-octet); 8 consecutive k of one row
      const int u = tid + 256 * q;
      const int row = u >> 3, ko = u & 7;
      if (r0 + row < rows) {
        const float* src = E + static_cast<int64_t>(r0 + row) * ldE + kc + 8 * ko;
        const f32x4 a = *reinterpret_cast<const f32x4*>(src);
        const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
        ev[q][0] = a[0]; ev[q][1] = a[1]; ev[q][2] = a[2]; ev[q][3] = a[3];
        ev[q][4] = b[0]; ev[q][5] = b[1]; ev[q][6] = b[2]; ev[q][7] = b[3];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ev[q][e] = 0.0f;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // U: unit -> (col, k-octet); 8 rows of U at one column, transposed into LDS
      const int u = tid + 256 * q;
      const int col = u & 127, ko = u >> 7;
      const bool ok = c0 + col < ce;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        uv[q][e] = ok ? U[static_cast<int64_t>(i1 + kc + 8 * ko + e) * n + c0 + col] : 0.0f;
    }
  };
  gload(0);
  for (int kc = 0; kc < K; kc += kTK) {
    if (kc) __syncthreads();  // the previous chunk's fragments have been read
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + 256 * q;
      const int row = u >> 3, ko = u & 7;
      u32x4 hi, lo;
      split8(ev[q], hi, lo);
      *reinterpret_cast<u32x4*>(lds[0] + tk_offset(row, ko)) = hi;
      *reinterpret_cast<u32x4*>(lds[1] + tk_offset(row, ko)) = lo;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + 256 * q;
      const int col = u & 127, ko = u >> 7;
      u32x4 hi, lo;
      split8(uv[q], hi, lo);
      *reinterpret_cast<u32x4*>(lds[2] + tk_offset(col, ko)) = hi;
      *reinterpret_cast<u32x4*>(lds[3] + tk_offset(col, ko)) = lo;
    }
    __syncthreads();
    if (kc + kTK < K) gload(kc + kTK);
#pragma unroll
    for (int kk = 0; kk < kTK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      u32x4 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = wm * 64 + i * 32 + (lane & 31);
        ah[i] = *reinterpret_cast<const u32x4*>(lds[0] + tk_offset(m, c));
        al[i] = *reinterpret_cast<const u32x4*>(lds[1] + tk_offset(m, c));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cc = wn * 64 + j * 32 + (lane & 31);
        bh[j] = *reinterpret_cast<const u32x4*>(lds[2] + tk_offset(cc, c));
        bl[j] = *reinterpret_cast<const u32x4*>(lds[3] + tk_offset(cc, c));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mfma_bf16(al[i], bh[j], acc[i][j]);
          acc[i][j] = mfma_bf16(ah[i], bl[j], acc[i][j]);
          acc[i][j] = mfma_bf16(ah[i], bh[j], acc[i][j]);
        }
    }
  }
  // Epilogue: all 64 loads of this lane's W values are issued before any store
  // (a load after a store to the same array would otherwise wait for it).
  float old[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rr = r0 + wm * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const int cc = c0 + wn * 64 + j * 32 + (lane & 31);
        old[i][j][q] = (rr < rows && cc < ce) ? Wk[static_cast<int64_t>(rr) * n + cc] : 0.0f;
      }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rr = r0 + wm * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const int cc = c0 + wn * 64 + j * 32 + (lane & 31);
        if (rr < rows && cc < ce) Wk[static_cast<int64_t>(rr) * n + cc] = old[i][j][q] - acc[i][j][q];
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
         + al256(static_cast<size_t>(rows) * kSuper * 4) // E of a super-block
         + al256(static_cast<size_t>(rows) * n)        // codes
         + al256(static_cast<size_t>(rows) * 8)        // rowloss
         + al256(static_cast<size_t>(n) * 4)           // invperm
         + 256;                                        // loss scalar
}

template <int BITS, bool SYM>
static void launch_sweep(dim3 g, hipStream_t s, float* Wk, const float* U, int n, int rows, int i1, uint8_t* codes,
                         float* E, int ldE, uint16_t* scales, uint16_t* zeros, double* rowloss) {
  hipLaunchKernelGGL((sweep_block_kernel<BITS, SYM>), g, dim3(256), 0, s, Wk, U, n, rows, i1, codes, E, ldE, scales,
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
  p += al256(static_cast<size_t>(rows) * kSuper * 4);
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
  e = zero_words(rowloss, static_cast<size_t>(rows), s);
  if (e != hipSuccess) return e;
  dim3 gg((n + 255) / 256, rows < 65535 ? rows : 65535);
  if (wdt == DT_BF16) hipLaunchKernelGGL(gather_w_kernel<DT_BF16>, gg, dim3(256), 0, s, W, ldw, perm, dead, rows, n, Wk);
  else if (wdt == DT_FP16) hipLaunchKernelGGL(gather_w_kernel<DT_FP16>, gg, dim3(256), 0, s, W, ldw, perm, dead, rows, n, Wk);
  else hipLaunchKernelGGL(gather_w_kernel<DT_FP32>, gg, dim3(256), 0, s, W, ldw, perm, dead, rows, n, Wk);
  GPTQ_CHECK_LAUNCH();
  hipLaunchKernelGGL(gidx_kernel, dim3((n + 255) / 256), dim3(256), 0, s, perm, n, kBlk, g_idx, invperm);
  GPTQ_CHECK_LAUNCH();

  // Two-level lazy batching: inside a super-block of kSuper columns each
  // 128-column block updates only the rest of its super-block; the columns
  // beyond it receive the whole super-block's errors in one K = kSuper update,
  // so the working weights are read and written once per super-block rather
  // than once per block.  E holds the super-block's scaled errors [rows, kSuper].
  const dim3 gs((rows + kRowsSweep - 1) / kRowsSweep);
  const int rt = (rows + 127) / 128;
  for (int s1 = 0; s1 < n; s1 += kSuper) {
    const int s2 = (s1 + kSuper < n) ? s1 + kSuper : n;
    for (int i1 = s1; i1 < s2; i1 += kBlk) {
      const int i2 = i1 + kBlk;
      float* Eb = E + (i1 - s1);
      if (bits == 4 && !sym) launch_sweep<4, false>(gs, s, Wk, U, n, rows, i1, codes, Eb, kSuper, scales, zeros, rowloss);
      else if (bits == 4 && sym) launch_sweep<4, true>(gs, s, Wk, U, n, rows, i1, codes, Eb, kSuper, scales, zeros, rowloss);
      else if (bits == 3 && !sym) launch_sweep<3, false>(gs, s, Wk, U, n, rows, i1, codes, Eb, kSuper, scales, zeros, rowloss);
      else launch_sweep<3, true>(gs, s, Wk, U, n, rows, i1, codes, Eb, kSuper, scales, zeros, rowloss);
      GPTQ_CHECK_LAUNCH();
      if (i2 < s2) {
        hipLaunchKernelGGL(trailing_kernel, dim3((s2 - i2 + 127) / 128, rt), dim3(256), 0, s, Wk, Eb, kSuper, U, n,
                           rows, i1, kBlk, i2, s2);
        GPTQ_CHECK_LAUNCH();
      }
    }
    if (s2 < n) {
      hipLaunchKernelGGL(trailing_kernel, dim3((n - s2 + 127) / 128, rt), dim3(256), 0, s, Wk, E, kSuper, U, n, rows,
                         s1, s2 - s1, s2, n);
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
