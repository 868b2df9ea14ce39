// Prepare: dead columns, act-order, damping and U = chol(H_d^-1) on gfx950.
//
// polydesk.ai "GPTQ" glossary, "Étape 2 : Compensation d'erreur via la
// Hessienne": errors are propagated through the inverse Hessian by way of a
// Cholesky decomposition, for numerical stability.  "Paramètres clés"
// (desc_act): columns in decreasing activation magnitude.  skillmd.com "Gptq",
// "Configurações de quantização": damp_percent.
//
// Route.  With J the index reversal, P = J H_d J = L L^T (lower Cholesky) gives
// H_d = (J L J)(J L J)^T with J L J upper triangular, hence
//     U = (J L J)^-1 = J L^-1 J,   U^T U = H_d^-1,
// one Cholesky plus one triangular inverse (2n^3/3 flops).  Both run in fp64:
// an fp32 factorization of these Hessians (condition numbers ~1e5) changes
// enough codes to matter; U is rounded to fp32 at the end.
//
// Blocked right-looking Cholesky with 64x64 blocks, per block column k:
//   chol_diag  one wave factors A_kk (rows in registers),
//   diag_inv   one wave inverts L_kk into the diagonal block of Linv,
//   chol_trsm  L_ik = A_ik inv(L_kk)^T for every block row i > k  (fp64 MFMA),
//   chol_syrk  A_ij -= L_ik L_jk^T for k < j <= i                   (fp64 MFMA).
// Triangular inverse by recursive doubling: with the diagonal blocks already
// inverted, each level joins pairs of inverted blocks of size s,
//   inv([L11 0; L21 L22]) = [X11 0; -X22 L21 X11  X22],
// as two GEMMs per pair; all pairs of a level run in one launch.  The
// temporary T = L21 X11 is kept, transposed, in the strict upper triangle of A,
// which the factorization never uses; the upper triangle of Linv stays zero so
// the triangular operands X11, X22 can be read as full blocks.
#include "common.hpp"

namespace gptq {

constexpr int kB = 64;  // block edge of the factorization

// ---------------------------------------------------------------- small kernels
// dd[i] = H_ii, or 1 for a dead column (H_ii == 0); dead flag; a NaN/inf or
// negative diagonal marks the matrix as not positive definite and is replaced
// by 1 in dd so that the act-order sort stays a permutation.
__global__ void prep_diag_kernel(const double* __restrict__ H, int n, double* __restrict__ dd,
                                 uint8_t* __restrict__ dead, int* __restrict__ info) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double d = H[static_cast<int64_t>(i) * n + i];
  const bool isdead = (d == 0.0);
  dead[i] = isdead ? 1 : 0;
  double v = isdead ? 1.0 : d;
  if (!(v > 0.0) || !(v < INFINITY)) {  // NaN, inf or negative
    atomicOr(info, 1);
    v = 1.0;
  }
  dd[i] = v;
}

// Stable descending sort by rank counting: rank(i) = #{j: d_j > d_i} + #{j < i: d_j == d_i}.
__global__ void __launch_bounds__(256) prep_rank_kernel(const double* __restrict__ dd, int n,
                                                        int desc_act, int32_t* __restrict__ perm) {
  __shared__ double chunk[1024];
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const double di = (i < n) ? dd[i] : 0.0;
  int rank = 0;
  if (!desc_act) {
    if (i < n) perm[i] = i;
    return;
  }
  for (int base = 0; base < n; base += 1024) {
    __syncthreads();
    for (int e = threadIdx.x; e < 1024; e += blockDim.x) chunk[e] = (base + e < n) ? dd[base + e] : 0.0;
    __syncthreads();
    const int lim = (n - base < 1024) ? n - base : 1024;
    for (int e = 0; e < lim; ++e) {
      const double dj = chunk[e];
      const int j = base + e;
      rank += (dj > di) || (dj == di && j < i);
    }
  }
  if (i < n) perm[rank] = i;
}

// lambda = damp * mean(dd); one workgroup, fixed-order tree reduction in fp64.
__global__ void __launch_bounds__(256) prep_lambda_kernel(const double* __restrict__ dd, int n,
                                                          double damp, double* __restrict__ lam) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) s += dd[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *lam = damp * (red[0] / n);
}

// A[a][b] (lower part, b <= a) = H_p[n-1-a][n-1-b] + lambda*delta, with
// H_p[x][y] = H[perm[x]][perm[y]] and dead diagonals taken as 1.
__global__ void prep_gather_kernel(const double* __restrict__ H, const int32_t* __restrict__ perm,
                                   const double* __restrict__ dd, const double* __restrict__ lam,
                                   int n, double* __restrict__ A) {
  for (int a = blockIdx.y; a < n; a += gridDim.y) {
    const int x = n - 1 - a;
    const int px = perm[x];
    const double* hrow = H + static_cast<int64_t>(px) * n;
    for (int b = blockIdx.x * blockDim.x + threadIdx.x; b <= a; b += gridDim.x * blockDim.x) {
      const int y = n - 1 - b;
      double v = (a == b) ? dd[px] + *lam : hrow[perm[y]];
      A[static_cast<int64_t>(a) * n + b] = v;
    }
  }
}

// ---------------------------------------------------------------- diagonal block
// Factor the 64x64 diagonal block k (rows/cols beyond n are identity) and
// write L_kk back to A; a second kernel writes inv(L_kk) to the diagonal block
// of Linv.  One wave each.
// Factorization, right-looking, lane i keeps row i in registers: for column j
// the pivot comes from lane j (readlane), each lane scales its entry, the
// column goes through LDS and every lane applies the rank-1 update to its row.
// Inverse, lane c keeps column c of inv(L) in registers:
//   x_r = (delta_rc - sum_{q<r} l_rq x_q) / l_rr, rows of L read as LDS broadcasts.
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(b), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(b >> 32), lane);
  return __longlong_as_double((static_cast<uint64_t>(hi) << 32) | lo);
}

__global__ void __launch_bounds__(64) chol_diag_kernel(double* __restrict__ A, int n, int k,
                                                       int* __restrict__ info) {
  __shared__ __attribute__((aligned(16))) double col[2][kB];
  const int i = threadIdx.x;
  const int r0 = k * kB;
  const int m = (n - r0 < kB) ? n - r0 : kB;
  const double* arow = A + static_cast<int64_t>(r0 + i) * n + r0;
  double a[kB];
#pragma unroll
  for (int c = 0; c < kB; ++c) {
    double v = (i == c) ? 1.0 : 0.0;
    if (i < m && c < m && c <= i) v = arow[c];
    a[c] = v;
  }
  int bad = 0;
#pragma unroll
  for (int j = 0; j < kB; ++j) {
    double piv = readlane_f64(a[j], j);
    if (!(piv > 0.0) || !(piv < INFINITY)) {  // uniform across the wave
      bad = 1;
      piv = 1.0;
    }
    const double rs = 1.0 / sqrt(piv);
    const double l = a[j] * rs;
    a[j] = l;
    col[j & 1][i] = l;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the column is in LDS
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = j + 1; c < kB; ++c) a[c] = fma(-l, col[j & 1][c], a[c]);
  }
  if (bad && i == 0) atomicOr(info, 1);
  double* wrow = A + static_cast<int64_t>(r0 + i) * n + r0;
#pragma unroll
  for (int c = 0; c < kB; ++c)
    if (i < m && c < m && c <= i) wrow[c] = a[c];
}

// inv(L_kk) into the diagonal block of Linv; lane c keeps column c in registers.
__global__ void __launch_bounds__(64) diag_inv_kernel(const double* __restrict__ A, double* __restrict__ Linv,
                                                      int n, int k) {
  __shared__ __attribute__((aligned(16))) double Ls[kB][kB];
  __shared__ double rinv[kB];
  const int i = threadIdx.x;
  const int r0 = k * kB;
  const int m = (n - r0 < kB) ? n - r0 : kB;
  for (int c = 0; c < kB; ++c) {
    double v = (i == c) ? 1.0 : 0.0;
    if (i < m && c < m && c <= i) v = A[static_cast<int64_t>(r0 + i) * n + r0 + c];
    Ls[i][c] = v;
  }
  rinv[i] = 1.0 / Ls[i][i];
  __syncthreads();
  const int cc = i;
  double x[kB];
#pragma unroll
  for (int r = 0; r < kB; ++r) {
    double acc0 = (r == cc) ? 1.0 : 0.0, acc1 = 0.0;
#pragma unroll
    for (int q = 0; q < r; q += 2) {
      acc0 = fma(-Ls[r][q], x[q], acc0);
      if (q + 1 < r) acc1 = fma(-Ls[r][q + 1], x[q + 1], acc1);
    }
    x[r] = (r >= cc) ? (acc0 + acc1) * rinv[r] : 0.0;
  }
  __syncthreads();  // L no longer needed: the block goes out through LDS
#pragma unroll
  for (int r = 0; r < kB; ++r) Ls[r][cc] = x[r];
  __syncthreads();
  for (int r = 0; r < m; ++r)
    if (cc < m) Linv[static_cast<int64_t>(r0 + r) * n + r0 + cc] = Ls[r][cc];
}

// ---------------------------------------------------------------- fp64 MFMA tile
// acc += A[0:64, k0:k1] * B[k0:k1, 0:64] for a 64x64 output tile, 256 threads.
// A is addressed A[m*lda + k]; B as B[k*ldb + n] (BT = false) or B[n*ldb + k]
// (BT = true).  Rows >= mv, columns >= nv and k >= k1 read as 0.
// v_mfma_f64_16x16x4: lane l supplies A[l%16][l/16] and B[l/16][l%16];
// accumulator r of lane l is D[l/16 + 4*r][l%16] (rows interleaved across the
// four accumulators; measured on gfx950).  Wave (wm, wn) owns the
// 32x32 quarter (wm*32.., wn*32..): 2x2 MFMA tiles.
struct TileSmem {
  double a[kB][17];
  double b[16][kB + 1];
};

template <bool BT>
__device__ __forceinline__ void tile_gemm_f64(const double* __restrict__ A, int64_t lda,
                                              const double* __restrict__ B, int64_t ldb, int mv, int nv,
                                              int k0, int k1, f64x4 (&acc)[2][2], TileSmem& sm) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  for (int kc = k0; kc < k1; kc += 16) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      const int r = e >> 4, kk = e & 15;
      const int kg = kc + kk;
      sm.a[r][kk] = (r < mv && kg < k1) ? A[static_cast<int64_t>(r) * lda + kg] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;
      if (!BT) {
        const int kk = e >> 6, c = e & 63;
        const int kg = kc + kk;
        sm.b[kk][c] = (c < nv && kg < k1) ? B[static_cast<int64_t>(kg) * ldb + c] : 0.0;
      } else {
        const int c = e >> 4, kk = e & 15;
        const int kg = kc + kk;
        sm.b[kk][c] = (c < nv && kg < k1) ? B[static_cast<int64_t>(c) * ldb + kg] : 0.0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = ks * 4 + (lane >> 4);
      double fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = sm.a[wm * 32 + i * 16 + (lane & 15)][kk];
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = sm.b[kk][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }
}

// Visit the 64x64 output elements held by this thread: f(row, col, value).
template <typename F>
__device__ __forceinline__ void tile_foreach(const f64x4 (&acc)[2][2], F f) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        f(wm * 32 + i * 16 + (lane >> 4) + 4 * r, wn * 32 + j * 16 + (lane & 15), acc[i][j][r]);
}

// The same element map with a second accumulator-shaped array.
template <typename F>
__device__ __forceinline__ void tile_foreach2(const f64x4 (&acc)[2][2], const f64x4 (&o)[2][2], F f) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        f(wm * 32 + i * 16 + (lane >> 4) + 4 * r, wn * 32 + j * 16 + (lane & 15), acc[i][j][r], o[i][j][r]);
}

// Loads the 64x64 tile at p (row stride ld) in accumulator layout, all loads
// issued before anything else touches memory; rows >= mv or columns >= nv read 0.
__device__ __forceinline__ void tile_load(f64x4 (&o)[2][2], const double* p, int64_t ld, int mv, int nv) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = wm * 32 + i * 16 + (lane >> 4) + 4 * r, cc = wn * 32 + j * 16 + (lane & 15);
        o[i][j][r] = (rr < mv && cc < nv) ? p[static_cast<int64_t>(rr) * ld + cc] : 0.0;
      }
}

__device__ __forceinline__ void zero_acc(f64x4 (&acc)[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
}

// L_ik = A_ik * inv(L_kk)^T for block rows i = k+1+blockIdx.x.
__global__ void __launch_bounds__(256) chol_trsm_kernel(double* __restrict__ A, const double* __restrict__ Linv,
                                                        int n, int k) {
  __shared__ TileSmem sm;
  const int i = k + 1 + blockIdx.x;
  const int r0 = i * kB, c0 = k * kB;
  const int mv = (n - r0 < kB) ? n - r0 : kB;
  const int kv = (n - c0 < kB) ? n - c0 : kB;
  f64x4 acc[2][2];
  zero_acc(acc);
  // B(q, c) = inv(L_kk)[c][q]: transposed access of the diagonal block; inv is lower
  // triangular so only q <= c contributes, but the zero entries are stored.
  tile_gemm_f64<true>(A + static_cast<int64_t>(r0) * n + c0, n, Linv + static_cast<int64_t>(c0) * n + c0, n,
                      mv, kv, 0, kv, acc, sm);
  __syncthreads();
  tile_foreach(acc, [&](int r, int c, double v) {
    if (r < mv && c < kv) A[static_cast<int64_t>(r0 + r) * n + c0 + c] = v;
  });
}

// A_ij -= L_ik L_jk^T for all lower tiles k < j <= i; blockIdx.x enumerates them.
__global__ void __launch_bounds__(256) chol_syrk_kernel(double* __restrict__ A, int n, int k, int nblk) {
  __shared__ TileSmem sm;
  // lower tiles of the trailing (nblk-k-1)^2 block, row by row
  int t = blockIdx.x;
  int ii = 0;
  while (t > ii) {
    t -= ii + 1;
    ++ii;
  }
  const int i = k + 1 + ii, j = k + 1 + t;
  const int r0 = i * kB, cc0 = j * kB, k0 = k * kB;
  const int mv = (n - r0 < kB) ? n - r0 : kB;
  const int nv = (n - cc0 < kB) ? n - cc0 : kB;
  const int kv = (n - k0 < kB) ? n - k0 : kB;
  f64x4 acc[2][2];
  zero_acc(acc);
  tile_gemm_f64<true>(A + static_cast<int64_t>(r0) * n + k0, n, A + static_cast<int64_t>(cc0) * n + k0, n,
                      mv, nv, 0, kv, acc, sm);
  __syncthreads();
  // all loads of the tile issued before any store (see tile_load)
  f64x4 old[2][2];
  tile_load(old, A + static_cast<int64_t>(r0) * n + cc0, n, mv, nv);
  tile_foreach2(acc, old, [&](int r, int c, double v, double o) {
    if (r < mv && c < nv && (i != j || c <= r)) A[static_cast<int64_t>(r0 + r) * n + cc0 + c] = o - v;
  });
}

// One level of the recursive-doubling inverse.  Pair p joins blocks
// [b1, b1+s) and [b2, b2+s2), b1 = 2ps, b2 = b1+s.  phase 0: T = L21 X11,
// stored transposed at A[b1.., b2..] (strict upper triangle of A); phase 1:
// X21 = -X22 T.  grid.x = pairs, grid.y = output tiles of the pair (s/64 x s/64).
__global__ void __launch_bounds__(256) trtri_level_kernel(double* __restrict__ L, double* __restrict__ Linv,
                                                          int n, int s, int phase) {
  __shared__ TileSmem sm;
  const int b1 = blockIdx.x * 2 * s;
  const int b2 = b1 + s;
  if (b2 >= n) return;
  const int s2 = (n - b2 < s) ? n - b2 : s;
  const int tcols = s / kB;
  const int tr = blockIdx.y / tcols, tc = blockIdx.y % tcols;
  const int rows0 = tr * kB, cols0 = tc * kB;  // within the s2 x s output
  if (rows0 >= s2) return;
  const int mv = (s2 - rows0 < kB) ? s2 - rows0 : kB;
  const int nv = kB;
  f64x4 acc[2][2];
  zero_acc(acc);
  if (phase == 0) {
    // T[r][c] = sum_q L21[r][q] X11[q][c], X11 lower: q >= c.
    const int kbeg = cols0;
    tile_gemm_f64<false>(L + static_cast<int64_t>(b2 + rows0) * n + b1, n,
                         Linv + static_cast<int64_t>(b1) * n + b1 + cols0, n, mv, nv, kbeg, s, acc, sm);
    __syncthreads();
    tile_foreach(acc, [&](int r, int c, double v) {
      if (r < mv) L[static_cast<int64_t>(b1 + cols0 + c) * n + b2 + rows0 + r] = v;  // T^T, upper part of A
    });
  } else {
    // X21[r][c] = -sum_q X22[r][q] T[q][c], X22 lower: q <= r.  T is stored
    // transposed: T[q][c] = A[b1 + c][b2 + q]  ->  BT access with ldb = n.
    const int kend = (rows0 + kB < s2) ? rows0 + kB : s2;
    tile_gemm_f64<true>(Linv + static_cast<int64_t>(b2 + rows0) * n + b2, n,
                        L + static_cast<int64_t>(b1 + cols0) * n + b2, n, mv, nv, 0, kend, acc, sm);
    __syncthreads();
    tile_foreach(acc, [&](int r, int c, double v) {
      if (r < mv) Linv[static_cast<int64_t>(b2 + rows0 + r) * n + b1 + cols0 + c] = -v;
    });
  }
}

// U[i][j] = Linv[n-1-i][n-1-j] for j >= i, 0 below the diagonal; fp32.
__global__ void write_u_kernel(const double* __restrict__ Linv, int n, float* __restrict__ U) {
  for (int i = blockIdx.y; i < n; i += gridDim.y) {
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x) {
      float v = 0.0f;
      if (j >= i) v = static_cast<float>(Linv[static_cast<int64_t>(n - 1 - i) * n + (n - 1 - j)]);
      U[static_cast<int64_t>(i) * n + j] = v;
    }
  }
}

// ---------------------------------------------------------------- host launcher
size_t prepare_workspace(int64_t n) {
  // A (n*n fp64) + Linv (n*n fp64) + dd (n) + lambda + info, 256-byte aligned pieces
  auto al = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  return al(static_cast<size_t>(n) * n * 8) * 2 + al(static_cast<size_t>(n) * 8) + 256 + 256;
}

hipError_t launch_prepare(const double* H, int64_t n64, double damp, int desc_act, float* U, int32_t* perm,
                          uint8_t* dead, void* ws, hipStream_t s, int* info_host) {
  const int n = static_cast<int>(n64);
  auto al = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  uint8_t* p = static_cast<uint8_t*>(ws);
  double* A = reinterpret_cast<double*>(p);
  p += al(static_cast<size_t>(n) * n * 8);
  double* Linv = reinterpret_cast<double*>(p);
  p += al(static_cast<size_t>(n) * n * 8);
  double* dd = reinterpret_cast<double*>(p);
  p += al(static_cast<size_t>(n) * 8);
  double* lam = reinterpret_cast<double*>(p);
  p += 256;
  int* info = reinterpret_cast<int*>(p);

  hipError_t e;
#define GPTQ_CHECK_LAUNCH()          \
  do {                               \
    e = hipGetLastError();           \
    if (e != hipSuccess) return e;   \
  } while (0)
  e = hipMemsetAsync(info, 0, sizeof(int), s);
  if (e != hipSuccess) return e;
  e = hipMemsetAsync(Linv, 0, static_cast<size_t>(n) * n * 8, s);
  if (e != hipSuccess) return e;
  const int nb = (n + 255) / 256;
  hipLaunchKernelGGL(prep_diag_kernel, dim3(nb), dim3(256), 0, s, H, n, dd, dead, info);
  GPTQ_CHECK_LAUNCH();
  hipLaunchKernelGGL(prep_rank_kernel, dim3(nb), dim3(256), 0, s, dd, n, desc_act, perm);
  GPTQ_CHECK_LAUNCH();
  hipLaunchKernelGGL(prep_lambda_kernel, dim3(1), dim3(256), 0, s, dd, n, damp, lam);
  GPTQ_CHECK_LAUNCH();
  const unsigned gy = n < 65535 ? n : 65535;
  hipLaunchKernelGGL(prep_gather_kernel, dim3((n + 255) / 256, gy), dim3(256), 0, s, H, perm, dd, lam, n, A);
  GPTQ_CHECK_LAUNCH();

  const int nblk = (n + kB - 1) / kB;
  for (int k = 0; k < nblk; ++k) {
    hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(64), 0, s, A, n, k, info);
    GPTQ_CHECK_LAUNCH();
    hipLaunchKernelGGL(diag_inv_kernel, dim3(1), dim3(64), 0, s, A, Linv, n, k);
    GPTQ_CHECK_LAUNCH();
    const int rest = nblk - k - 1;
    if (rest > 0) {
      hipLaunchKernelGGL(chol_trsm_kernel, dim3(rest), dim3(256), 0, s, A, Linv, n, k);
      GPTQ_CHECK_LAUNCH();
      hipLaunchKernelGGL(chol_syrk_kernel, dim3(rest * (rest + 1) / 2), dim3(256), 0, s, A, n, k, nblk);
      GPTQ_CHECK_LAUNCH();
    }
  }
  for (int sz = kB; sz < n; sz *= 2) {
    const int pairs = (n + 2 * sz - 1) / (2 * sz);
    const int tiles = (sz / kB) * (sz / kB);
    hipLaunchKernelGGL(trtri_level_kernel, dim3(pairs, tiles), dim3(256), 0, s, A, Linv, n, sz, 0);
    GPTQ_CHECK_LAUNCH();
    hipLaunchKernelGGL(trtri_level_kernel, dim3(pairs, tiles), dim3(256), 0, s, A, Linv, n, sz, 1);
    GPTQ_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(write_u_kernel, dim3((n + 255) / 256, gy), dim3(256), 0, s, Linv, n, U);
  GPTQ_CHECK_LAUNCH();
#undef GPTQ_CHECK_LAUNCH
  e = hipMemcpyAsync(info_host, info, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace gptq
