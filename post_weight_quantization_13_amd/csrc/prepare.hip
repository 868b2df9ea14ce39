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
// Blocked Cholesky with 64x64 blocks, panels taken in groups of kGroup.
// Inside a group (left-looking), one launch per block column k:
//   chol_step      every work-group factors and inverts A_kk with one wave
//                  (rows in registers) while its other waves apply the
//                  group's earlier panels to its block A_ik,
//                  A_ik -= sum_{k0 <= q < k} L_iq L_kq^T   (fp64 MFMA),
//                  then forms L_ik = A_ik inv(L_kk)^T; work-group 0 writes
//                  inv(L_kk) into the diagonal block of Linv;
// after the group (right-looking), one chol_update pass applies all of the
// group's panels to the trailing matrix with K = 64 kGroup, so the trailing
// matrix is read and written once per group instead of once per panel.
// Triangular inverse by recursive doubling: with the diagonal blocks already
// inverted, each level joins pairs of inverted blocks of size s,
//   inv([L11 0; L21 L22]) = [X11 0; -X22 L21 X11  X22],
// as two GEMMs per pair; all pairs of a level run in one launch.  The
// temporary T = L21 X11 is kept, transposed, in the strict upper triangle of A,
// which the factorization never uses; the upper triangle of Linv stays zero so
// the triangular operands X11, X22 can be read as full blocks.
#include "common.hpp"

namespace gptq {

constexpr int kB = 64;     // block edge of the factorization
constexpr int kGroup = 4;  // panels whose trailing update is applied in one pass

// ---------------------------------------------------------------- small kernels
// dd[i] = H_ii, or 1 for a dead column (H_ii == 0); dead flag; a NaN/inf or
// negative diagonal marks the matrix as not positive definite and is replaced
// by 1 in dd so that the act-order sort stays a permutation.
// Without act-order the sweep order is the original one: perm is written here
// and the rank kernel is not launched.
__global__ void prep_diag_kernel(const double* __restrict__ H, int n, double* __restrict__ dd,
                                 uint8_t* __restrict__ dead, int* __restrict__ info, int desc_act,
                                 int32_t* __restrict__ perm) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (!desc_act) perm[i] = i;
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

// lambda = damp * mean(dd); one workgroup of 1024, fixed-order reduction in
// fp64: each thread sums its strided entries in four independent chains (so
// their loads are in flight together), then a tree over the threads.
__global__ void __launch_bounds__(1024) prep_lambda_kernel(const double* __restrict__ dd, int n,
                                                           double damp, double* __restrict__ lam) {
  __shared__ double red[1024];
  const int t = threadIdx.x;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  int i = t;
  for (; i + 3 * 1024 < n; i += 4 * 1024) {
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] += dd[i + q * 1024];
  }
  for (int q = 0; i < n; i += 1024, ++q) s[q] += dd[i];
  red[t] = (s[0] + s[1]) + (s[2] + s[3]);
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) *lam = damp * (red[0] / n);
}

// A[a][b] (lower part, b <= a) = H_p[n-1-a][n-1-b] + lambda*delta, with
// H_p[x][y] = H[perm[x]][perm[y]] and dead diagonals taken as 1.  One
// work-group per pair of rows a and n-1-a (a + 1 and n - a entries: n + 1 in
// all, so every work-group moves the same amount); without act-order the
// source row is read directly (H_p = H).
__global__ void __launch_bounds__(256) prep_gather_kernel(const double* __restrict__ H,
                                                          const int32_t* __restrict__ perm,
                                                          const double* __restrict__ dd,
                                                          const double* __restrict__ lam, int n, int desc_act,
                                                          double* __restrict__ A) {
  const double l = *lam;
  for (int p = blockIdx.x; 2 * p < n; p += gridDim.x) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int a = h ? n - 1 - p : p;
      if (h && a == p) break;  // the middle row of an odd n
      const int x = n - 1 - a;
      const int px = desc_act ? perm[x] : x;
      const double* hrow = H + static_cast<int64_t>(px) * n;
      double* arow = A + static_cast<int64_t>(a) * n;
      for (int b = threadIdx.x; b <= a; b += blockDim.x) {
        const int y = n - 1 - b;
        arow[b] = (a == b) ? dd[px] + l : hrow[desc_act ? perm[y] : y];
      }
    }
  }
}

// ---------------------------------------------------------------- diagonal block
// A 64x64 diagonal block is factored by the four waves of a work-group and
// inverted by one.  1/sqrt(pivot) is the hardware estimate refined by two
// Newton steps.
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(b), lane);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(b >> 32), lane);
  return __longlong_as_double((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ double rsqrt_refined(double x) {
  double r = __builtin_amdgcn_rsq(x);
  const double h = 0.5 * x;
  r = r * fma(-(h * r), r, 1.5);
  r = r * fma(-(h * r), r, 1.5);
  return r;
}

struct DiagSmem {
  double L[kB][kB + 1];                      // the block, then its factor, row-major, padded
  alignas(16) double pan[4][kB][4];          // panel columns, [row][column]
  double rinv[kB];                           // 1 / l_ii
  double X[kB][kB + 1];                      // inv(L)
};

// All four waves: factors the block held in d.L and writes L back (zeros
// above the diagonal).  Columns go in 16 panels of four, panel p owned by
// wave p % 4; lane i keeps row i of its wave's 16 columns in registers.  The
// owner finishes panel p (pivots; the panel's own updates take pivot-row
// entries by readlane) and publishes it in LDS; after a barrier every wave
// applies the rank-4 update to its columns beyond the panel.  The owner of
// panel p + 1 first updates that panel, factors and publishes it, and only
// after the next barrier applies panel p to its other columns, so the chain
// of pivots never waits for that work.  Panels rotate through four LDS
// buffers: panel p is read until barrier p + 2 and rewritten after barrier
// p + 3.  Returns nonzero when a pivot is not a positive finite number (it
// is then taken as 1).
__device__ __forceinline__ int factor_block4(DiagSmem& d) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double a[4][4];  // slot s: panel 4 s + wave, columns 4 (4 s + wave) .. +3
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 4; ++t) a[s][t] = d.L[lane][4 * (4 * s + wave) + t];
  int bad = 0;
  auto pivots = [&](int s) {
    const int j0 = 4 * (4 * s + wave);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + q;
#pragma unroll
      for (int pp = 0; pp < q; ++pp) a[s][q] = fma(-a[s][pp], readlane_f64(a[s][pp], j), a[s][q]);
      double piv = readlane_f64(a[s][q], j);
      if (!(piv > 0.0) || !(piv < INFINITY)) {  // uniform across the wave
        bad = 1;
        piv = 1.0;
      }
      const double rs = rsqrt_refined(piv);
      a[s][q] = (lane >= j) ? a[s][q] * rs : 0.0;
    }
  };
  auto publish = [&](int s, int p) {
    double* pp = &d.pan[p & 3][lane][0];
    *reinterpret_cast<double2*>(pp) = double2{a[s][0], a[s][1]};
    *reinterpret_cast<double2*>(pp + 2) = double2{a[s][2], a[s][3]};
  };
  // a[s] -= (row of panel p) (columns of slot s in panel p)^T
  auto apply = [&](int p, int s, const double2 (&mine)[2]) {
    const int c0 = 4 * (4 * s + wave);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const double* col = &d.pan[p & 3][c0 + t][0];
      const double2 u = *reinterpret_cast<const double2*>(col);
      const double2 v = *reinterpret_cast<const double2*>(col + 2);
      double x = fma(-mine[0].x, u.x, a[s][t]);
      x = fma(-mine[0].y, u.y, x);
      x = fma(-mine[1].x, v.x, x);
      a[s][t] = fma(-mine[1].y, v.y, x);
    }
  };
  auto row_of = [&](int p, double2 (&mine)[2]) {
    const double* r = &d.pan[p & 3][lane][0];
    mine[0] = *reinterpret_cast<const double2*>(r);
    mine[1] = *reinterpret_cast<const double2*>(r + 2);
  };
  if (wave == 0) {
    pivots(0);
    publish(0, 0);
  }
  int deferred = -1;  // a panel still to be applied to this wave's later slots
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    lds_barrier();
    double2 mine[2];
    if (deferred >= 0) {
      row_of(deferred, mine);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (4 * s + wave > p) apply(deferred, s, mine);
      deferred = -1;
    }
    row_of(p, mine);
    if (p + 1 < 16 && ((p + 1) & 3) == wave) {
      const int sn = (p + 1) >> 2;
      apply(p, sn, mine);
      pivots(sn);
      publish(sn, p + 1);
      deferred = p;
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (4 * s + wave > p) apply(p, s, mine);
    }
  }
  // deferred is -1 here: panel 15's owner has no next panel
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 4; ++t) d.L[lane][4 * (4 * s + wave) + t] = a[s][t];
  lds_barrier();
  return bad;
}

// Wave 0: d.X = inv(L) for the factor in d.L.  The strictly upper 16x16
// blocks of d.X are left unwritten.
__device__ __forceinline__ void invert_block(DiagSmem& d) {
  const int i = threadIdx.x & 63;
  // Inverse by 16x16 blocks, X = inv(L):
  //   X_bb = inv(L_bb)          forward substitution, lane = (b, column),
  //   X_ij = -X_ii sum_{k=j}^{i-1} L_ik X_kj   for i > j, by block distance,
  // the products on v_mfma_f64_16x16x4 (lane l supplies A[l%16][l/16] and
  // B[l/16][l%16]; accumulator r of lane l is D[l/16 + 4r][l%16], which is
  // also the B-operand layout, so L_ik X_kj feeds the product with X_ii
  // straight from the accumulators).
  {
    const int b = i >> 4, c = i & 15, o = 16 * b;
    double x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      double s0 = 0.0, s1 = 0.0;
#pragma unroll
      for (int q = 0; q < r; q += 2) {
        s0 = fma(d.L[o + r][o + q], x[q], s0);
        if (q + 1 < r) s1 = fma(d.L[o + r][o + q + 1], x[q + 1], s1);
      }
      const double t = ((r == c) ? 1.0 : 0.0) - (s0 + s1);
      x[r] = (r >= c) ? t * d.rinv[o + r] : 0.0;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) d.X[o + r][o + c] = x[r];
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  {
    const int lr = i & 15, lk = i >> 4;
#pragma unroll
    for (int dist = 1; dist < 4; ++dist) {
#pragma unroll
      for (int bi = dist; bi < 4; ++bi) {
        const int bj = bi - dist;
        f64x4 t = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int bk = bj; bk < bi; ++bk)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            t = __builtin_amdgcn_mfma_f64_16x16x4f64(d.L[16 * bi + lr][16 * bk + 4 * ks + lk],
                                                     d.X[16 * bk + 4 * ks + lk][16 * bj + lr], t, 0, 0, 0);
        f64x4 u = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          u = __builtin_amdgcn_mfma_f64_16x16x4f64(d.X[16 * bi + lr][16 * bi + 4 * ks + lk], t[ks], u, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) d.X[16 * bi + lk + 4 * r][16 * bj + lr] = -u[r];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ---------------------------------------------------------------- fp64 MFMA tile
// acc += A[0:64, k0:k1] * B[k0:k1, 0:64] for a 64x64 output tile, 256 threads.
// A is addressed A[m*lda + k]; B as B[k*ldb + n] (BT = false) or B[n*ldb + k]
// (BT = true).  Rows >= mv, columns >= nv and k >= k1 read as 0.
// v_mfma_f64_16x16x4: lane l supplies A[l%16][l/16] and B[l/16][l%16];
// accumulator r of lane l is D[l/16 + 4*r][l%16] (rows interleaved across the
// four accumulators; measured on gfx950).  Wave (wm, wn) owns the
// 32x32 quarter (wm*32.., wn*32..): 2x2 MFMA tiles.
// K runs in chunks of 64: each chunk is loaded into registers (coalesced rows
// of 64 consecutive k), stored to LDS, and the next chunk's loads are issued
// before the current chunk's 64 MFMAs per wave.  LDS rows are padded to 65
// doubles.
constexpr int kKC = 64;
struct TileSmem {
  double a[kB][kKC + 1];  // a[m][k]
  double b[kKC][kB + 1];  // b[k][n]
};

template <bool BT>
__device__ __forceinline__ void tile_gemm_f64(const double* __restrict__ A, int64_t lda,
                                              const double* __restrict__ B, int64_t ldb, int mv, int nv,
                                              int k0, int k1, f64x4 (&acc)[2][2], TileSmem& sm) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  double ra[16], rb[16];
  auto gload = [&](int kc) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q;
      const int r = e >> 6, kk = e & 63;  // A: row r, k = kc + kk
      const int kg = kc + kk;
      ra[q] = (r < mv && kg < k1) ? A[static_cast<int64_t>(r) * lda + kg] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q;
      if (!BT) {
        const int kk = e >> 6, c = e & 63;  // B[k][c]
        const int kg = kc + kk;
        rb[q] = (c < nv && kg < k1) ? B[static_cast<int64_t>(kg) * ldb + c] : 0.0;
      } else {
        const int c = e >> 6, kk = e & 63;  // B[c][k]
        const int kg = kc + kk;
        rb[q] = (c < nv && kg < k1) ? B[static_cast<int64_t>(c) * ldb + kg] : 0.0;
      }
    }
  };
  if (k0 >= k1) return;
  gload(k0);
  for (int kc = k0; kc < k1; kc += kKC) {
    __syncthreads();  // the previous chunk's operands have been read
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = tid + 256 * q;
      sm.a[e >> 6][e & 63] = ra[q];
      if (!BT) sm.b[e >> 6][e & 63] = rb[q];
      else sm.b[e & 63][e >> 6] = rb[q];
    }
    __syncthreads();
    if (kc + kKC < k1) gload(kc + kKC);
#pragma unroll
    for (int ks = 0; ks < kKC / 4; ++ks) {
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

// ---------------------------------------------------------------- panel step
// One launch per block column k of a panel group [k0, ke); work-group t
// handles block row i = k + t.  Every work-group factors the diagonal block
// A_kk itself (all four waves) and inverts it (wave 0), so the panel solve
// needs no second launch; work-group 0 writes inv(L_kk) into the diagonal
// block of Linv.  For t > 0, while wave 0 inverts, waves 1-3 apply the
// group's earlier panels to A_ik (left-looking),
//   C = A_ik - sum_{k0 <= q < k} L_iq L_kq^T,
// keeping C in registers until the inverse is done; then the four waves form
// L_ik = C inv(L_kk)^T and store it, and a block row inside the group also
// takes its own diagonal block's share A_ii -= L_ik L_ik^T, so that A_kk is
// complete when step k starts.  L_kk itself is not written back: the rest of
// the factorization and the triangular inverse read only the blocks below the
// diagonal and the inverted diagonal blocks.
__global__ void __launch_bounds__(256) chol_step_kernel(double* __restrict__ A, double* __restrict__ Linv, int n,
                                                        int k, int k0, int ke, int* __restrict__ info) {
  __shared__ DiagSmem d;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lk = lane >> 4;
  const int t = blockIdx.x;
  const int bi = k + t;
  const int c0 = k * kB, r0 = bi * kB;
  const int m = (n - c0 < kB) ? n - c0 : kB;   // valid size of the diagonal block
  const int mv = (n - r0 < kB) ? n - r0 : kB;  // valid rows of this block row
  // All four waves bring in A_kk (16 coalesced rows each, loads in flight
  // together); identity padding beyond n.
  {
    double v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = wave * 16 + q;
      v[q] = (r < m && lane < m) ? A[static_cast<int64_t>(c0 + r) * n + c0 + lane] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = wave * 16 + q;
      d.L[r][lane] = (r >= m || lane >= m) ? ((r == lane) ? 1.0 : 0.0) : ((lane <= r) ? v[q] : 0.0);
    }
  }
  __syncthreads();
  // Column update, waves 1-3 of work-groups t > 0: minus C in accumulator
  // layout, waves 1-2 on block rows 2(w-1), 2(w-1)+1 by block columns 0..2,
  // wave 3 on block rows 0..3 by block column 3; five fragment rows each
  // (wave 1-2: two of A_i., three of A_k.; wave 3: four of A_i., one of A_k.).
  // Operands come straight from memory: per chunk of 16 k a lane loads 4
  // consecutive k of its fragment row, and MFMA sub-step u takes the u-th of
  // them on both operands, so each product pairs equal k.  Loads run three
  // chunks ahead in a ring of four; the first three and the tile's previous
  // values are issued before the factorization, which hides them.
  const bool cu = (t > 0) && (wave > 0);
  const bool wide = wave < 3;
  const int nk = 4 * (k - k0);  // chunks of 16 in K = 64 (k - k0), a multiple of 4
  const double* fp[5];
#pragma unroll
  for (int e = 0; e < 5; ++e) {
    const bool isa = wide ? (e < 2) : (e < 4);
    const int row = wide ? (isa ? 16 * (2 * (wave - 1) + e) + lr : 16 * (e - 2) + lr) : (isa ? 16 * e + lr : 48 + lr);
    fp[e] = A + static_cast<int64_t>(isa ? r0 + (row < mv ? row : 0) : c0 + row) * n + k0 * kB + 4 * lk;
  }
  double fr[4][5][4];
  // A row of the block row beyond the matrix (row >= mv) reads row 0 of the
  // block row instead: it only feeds the same row of C, L_ik and A_ii, none
  // of which is stored.  The loads are unconditional, so nothing waits for
  // them before the factorization.
  auto load = [&](int sl, int q) {
#pragma unroll
    for (int e = 0; e < 5; ++e)
#pragma unroll
      for (int u = 0; u < 4; ++u) fr[sl][e][u] = fp[e][16 * q + u];
  };
  auto mma = [&](int sl, f64x4 (&cc)[6]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (wide) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 3; ++j)
            cc[3 * i + j] = __builtin_amdgcn_mfma_f64_16x16x4f64(fr[sl][i][u], fr[sl][2 + j][u], cc[3 * i + j], 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          cc[i] = __builtin_amdgcn_mfma_f64_16x16x4f64(fr[sl][i][u], fr[sl][4][u], cc[i], 0, 0, 0);
      }
    }
  };
  // tile x of this wave's share -> (block row, block column)
  auto tile_rc = [&](int x, int& rb, int& cb) {
    rb = wide ? 2 * (wave - 1) + x / 3 : x;
    cb = wide ? x % 3 : 3;
  };
  f64x4 cc[6];
  // the quarter of A_ii that waves 1-3 update last: (0,0), (1,0), (1,1)
  const int qm = (wave >= 2) ? 1 : 0, qn = (wave == 3) ? 1 : 0;
  double old[2][2][4];  // raw; only entries inside the block are used
  // previous values of the tile (loads in flight through the factorization;
  // negated into cc only after it)
  double craw[6][4];
  if (cu) {
#pragma unroll
    for (int x = 0; x < 6; ++x) {
      int rb, cb;
      tile_rc(x, rb, cb);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rb + lk + 4 * r, col = 16 * cb + lr;
        craw[x][r] = (x < (wide ? 6 : 4)) ? A[static_cast<int64_t>(r0 + (row < mv ? row : 0)) * n + c0 + col] : 0.0;
      }
    }
    if (bi < ke) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = qm * 32 + 16 * i + lk + 4 * r, col = qn * 32 + 16 * j + lr;
            const bool on = row < mv && col < mv;
            old[i][j][r] = A[static_cast<int64_t>(r0 + (on ? row : 0)) * n + r0 + (on ? col : 0)];
          }
    }
    if (nk > 0) {
      load(0, 0);
      load(1, 1);
      load(2, 2);
    }
  }
  const int bad = factor_block4(d);
  if (bad && t == 0 && lane == 0) atomicOr(info, 1);
  if (wave == 0) {
    d.rinv[lane] = 1.0 / d.L[lane][lane];
    invert_block(d);
  } else if (cu) {
#pragma unroll
    for (int x = 0; x < 6; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) cc[x][r] = -craw[x][r];
    for (int q = 0; q < nk; q += 4) {
      load(3, q + 3);
      mma(0, cc);
      if (q + 4 < nk) load(0, q + 4);
      mma(1, cc);
      if (q + 5 < nk) load(1, q + 5);
      mma(2, cc);
      if (q + 6 < nk) load(2, q + 6);
      mma(3, cc);
    }
  }
  __syncthreads();
  if (t == 0) {
    double v[16];  // all LDS reads first, then the guarded stores
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = wave * 16 + q;
      v[q] = ((r >> 4) >= (lane >> 4)) ? d.X[r][lane] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = wave * 16 + q;
      if (r < m && lane < m) Linv[static_cast<int64_t>(c0 + r) * n + c0 + lane] = v[q];
    }
    return;
  }
  // C into d.L, which the inverse no longer needs
  if (wave > 0) {
#pragma unroll
    for (int x = 0; x < 6; ++x) {
      if (x < (wide ? 6 : 4)) {
        int rb, cb;
        tile_rc(x, rb, cb);
#pragma unroll
        for (int r = 0; r < 4; ++r) d.L[16 * rb + lk + 4 * r][16 * cb + lr] = -cc[x][r];
      }
    }
  }
  __syncthreads();
  // L_ik = C inv(L_kk)^T.  inv(L_kk) is lower triangular, so result column
  // block cb needs k blocks <= cb only (4 cb + 4 k-steps; the unwritten upper
  // blocks of d.X are never read).  Wave (wm, wn) owns row blocks 2 wm, 2 wm + 1
  // and column blocks {0, 3} (wn = 0) or {1, 2} (wn = 1): 40 products each.
  const int wm = wave >> 1, wn = wave & 1;
  f64x4 acc[2][2];
  zero_acc(acc);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    if (ks < 16 - 4 * wn) {
      const int kk = 4 * ks + lk;
      double fa[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = d.L[wm * 32 + 16 * i + lr][kk];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cb = (j == 0) ? wn : 3 - wn;
        if (ks < 4 * cb + 4) {
          const double fb = d.X[16 * cb + lr][kk];
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[i], fb, acc[i][j], 0, 0, 0);
        }
      }
    }
  }
  auto visit = [&](auto f) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          f(wm * 32 + 16 * i + lk + 4 * r, 16 * ((j == 0) ? wn : 3 - wn) + lr, acc[i][j][r]);
  };
  visit([&](int r, int c, double v) {
    if (r < mv) A[static_cast<int64_t>(r0 + r) * n + c0 + c] = v;
  });
  if (bi >= ke) return;
  // A_ii -= L_ik L_ik^T on the lower triangle, L_ik through LDS; waves 1-3
  // take the quarters (0,0), (1,0), (1,1) with the old values they loaded
  // while wave 0 factored.
  __syncthreads();
  visit([&](int r, int c, double v) { d.L[r][c] = v; });
  __syncthreads();
  if (wave == 0) return;
  f64x4 sy[2][2];
  zero_acc(sy);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const int kk = 4 * ks + lk;
    double fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = d.L[qm * 32 + 16 * i + lr][kk];
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = d.L[qn * 32 + 16 * j + lr][kk];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) sy[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[i], fb[j], sy[i][j], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = qm * 32 + 16 * i + lk + 4 * r, col = qn * 32 + 16 * j + lr;
        if (row < mv && col <= row) A[static_cast<int64_t>(r0 + row) * n + r0 + col] = old[i][j][r] - sy[i][j][r];
      }
}

// A_ij -= sum_{q0 <= q < q1} L_iq L_jq^T (K = 64 (q1 - q0)) over the tiles
// of one launch: mode 0, the lower triangle j0 <= j <= i < nblk, row by row;
// mode 2, the block columns j0 <= j < j0 + w, rows j <= i < nblk, column by
// column.
__global__ void __launch_bounds__(256) chol_update_kernel(double* __restrict__ A, int n, int q0, int q1, int j0,
                                                          int mode, int nblk, int w) {
  __shared__ TileSmem sm;
  int i, j;
  if (mode == 0) {
    int t = blockIdx.x;
    int ii = 0;
    while (t > ii) {
      t -= ii + 1;
      ++ii;
    }
    i = j0 + ii;
    j = j0 + t;
  } else {
    int t = blockIdx.x;
    j = j0;
    for (int c = 0; c + 1 < w && t >= nblk - j; ++c) {
      t -= nblk - j;
      ++j;
    }
    i = j + t;
  }
  const int r0 = i * kB, cc0 = j * kB, k0 = q0 * kB;
  const int mv = (n - r0 < kB) ? n - r0 : kB;
  const int nv = (n - cc0 < kB) ? n - cc0 : kB;
  const int kv = (q1 - q0) * kB;
  // the tile's previous values are loaded first, in flight during the GEMM
  f64x4 old[2][2];
  tile_load(old, A + static_cast<int64_t>(r0) * n + cc0, n, mv, nv);
  f64x4 acc[2][2];
  zero_acc(acc);
  tile_gemm_f64<true>(A + static_cast<int64_t>(r0) * n + k0, n, A + static_cast<int64_t>(cc0) * n + k0, n,
                      mv, nv, 0, kv, acc, sm);
  tile_foreach2(acc, old, [&](int r, int c, double v, double o) {
    if (r < mv && c < nv && (i != j || c <= r)) A[static_cast<int64_t>(r0 + r) * n + cc0 + c] = o - v;
  });
}

// ---------------------------------------------------------------- fp64 MFMA, 128x128 tiles
// acc += A[0:128, k0:k1] * B[k0:k1, 0:128], 256 threads, wave (wm, wn) owns
// the 64x64 quarter (wm*64.., wn*64..) as 4x4 v_mfma_f64_16x16x4 tiles.
// A is addressed A[m*lda + k]; B as B[k*ldb + n] (BT = false) or B[n*ldb + k]
// (BT = true).  Rows >= mv, columns >= nv and k >= k1 read as 0.  K runs in
// chunks of KC staged as [row][k] planes (odd row stride KC + 1: the fragment
// reads and the stores are free of LDS bank conflicts), LDS double buffered,
// the next chunk's global loads in flight in registers during the current
// chunk's 4 KC MFMAs per wave.
constexpr int kT2 = 128;
// 128x128 tiles pay off only with enough of them to keep every compute unit
// busy with two; below that the 64x64 kernels run more tiles in parallel.
constexpr int kBigTiles = 512;
// The factorization's trailing passes switch to 128x128 tiles from this many
// when n <= kSmallN (measured, prepare alone at n = 4096: 2.716-2.719 against
// 2.753-2.755 ms with kBigTiles; at n = 11008 the smaller threshold was 0.3 %
// slower, so larger n keep kBigTiles).
constexpr int kTrailBigTilesSmallN = 128;
constexpr int kSmallN = 4096;
// LDS requested per work-group of the overlapped top level of the inverse
constexpr int kTopLds = 96 * 1024;
// largest top-level split h whose first product runs on part of the chip
constexpr int kTopSplitMax = 2048;
static_assert(kTopLds >= static_cast<int>(sizeof(TileSmem)) && kTopLds + static_cast<int>(sizeof(TileSmem)) > 160 * 1024,
              "top-level LDS");
template <int KC>
struct BigSmemT {
  double a[2][kT2][KC + 1];
  double b[2][kT2][KC + 1];
};
using BigSmem = BigSmemT<16>;

template <bool BT, int KC>
__device__ __forceinline__ void gemm128(const double* __restrict__ A, int64_t lda, const double* __restrict__ B,
                                        int64_t ldb, int mv, int nv, int k0, int k1, f64x4 (&acc)[4][4],
                                        BigSmemT<KC>& sm) {
  constexpr int E = KC / 2;  // elements of each operand per thread and chunk
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  double ra[E], rb[E];
  // A (and B^T): thread -> row tid/2, k = E*(tid%2) .. +E-1 (contiguous)
  // B: thread -> column tid%128, k = E*(tid/128) .. +E-1 (rows of B, coalesced)
  auto gload = [&](int kc) {
    const int m = tid >> 1, kb = kc + E * (tid & 1);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int kg = kb + e;
      ra[e] = (m < mv && kg < k1) ? A[static_cast<int64_t>(m) * lda + kg] : 0.0;
    }
    if (BT) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int kg = kb + e;
        rb[e] = (m < nv && kg < k1) ? B[static_cast<int64_t>(m) * ldb + kg] : 0.0;
      }
    } else {
      const int c = tid & 127, kb2 = kc + E * (tid >> 7);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int kg = kb2 + e;
        rb[e] = (c < nv && kg < k1) ? B[static_cast<int64_t>(kg) * ldb + c] : 0.0;
      }
    }
  };
  auto lstore = [&](int buf) {
    const int m = tid >> 1, kh = E * (tid & 1);
#pragma unroll
    for (int e = 0; e < E; ++e) sm.a[buf][m][kh + e] = ra[e];
    if (BT) {
#pragma unroll
      for (int e = 0; e < E; ++e) sm.b[buf][m][kh + e] = rb[e];
    } else {
      const int c = tid & 127, kh2 = E * (tid >> 7);
#pragma unroll
      for (int e = 0; e < E; ++e) sm.b[buf][c][kh2 + e] = rb[e];
    }
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < KC / 4; ++ks) {
      const int kk = ks * 4 + (lane >> 4);
      double fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = sm.a[buf][wm * 64 + i * 16 + (lane & 15)][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = sm.b[buf][wn * 64 + j * 16 + (lane & 15)][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  if (k0 >= k1) return;
  const int nch = (k1 - k0 + KC - 1) / KC;
  gload(k0);
  lstore(0);
  if (nch > 1) gload(k0 + KC);
  __syncthreads();
  int buf = 0;
  for (int c = 0; c < nch; ++c) {
    compute(buf);
    if (c + 1 >= nch) break;
    lstore(buf ^ 1);
    if (c + 2 < nch) gload(k0 + (c + 2) * KC);
    __syncthreads();
    buf ^= 1;
  }
  __syncthreads();  // LDS free for the caller
}

__device__ __forceinline__ void zero_acc4(f64x4 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
}

// Visit this thread's elements of the 128x128 tile: f(i, j, r, row, col).
template <typename F>
__device__ __forceinline__ void big_foreach(F f) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) f(i, j, r, wm * 64 + i * 16 + (lane >> 4) + 4 * r, wn * 64 + j * 16 + (lane & 15));
}

// Trailing pass on 128x128 tiles: A_IJ -= sum_{q0 <= q < q1} L_Iq L_Jq^T over
// the lower triangle of tiles of the square [s0, n) x [s0, n).
__global__ void __launch_bounds__(256, 2) chol_trail_kernel(double* __restrict__ A, int n, int q0, int q1, int s0) {
  __shared__ BigSmem sm;
  {
    int t = blockIdx.x;
    int I = 0;
    while (t > I) {
      t -= I + 1;
      ++I;
    }
    const int J = t;
    const int r0 = s0 + I * kT2, c0 = s0 + J * kT2, k0 = q0 * kB;
    const int mv = (n - r0 < kT2) ? n - r0 : kT2;
    const int nv = (n - c0 < kT2) ? n - c0 : kT2;
    f64x4 acc[4][4];
    zero_acc4(acc);
    gemm128<true, 16>(A + static_cast<int64_t>(r0) * n + k0, n, A + static_cast<int64_t>(c0) * n + k0, n, mv, nv, 0,
                  (q1 - q0) * kB, acc, sm);
    // read-modify-write one 16x16 column strip at a time: its 16 loads first
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double old[4][4];
      big_foreach([&](int ii, int j, int r, int row, int col) {
        if (ii == i) old[j][r] = (row < mv && col < nv) ? A[static_cast<int64_t>(r0 + row) * n + c0 + col] : 0.0;
      });
      big_foreach([&](int ii, int j, int r, int row, int col) {
        if (ii == i && row < mv && col < nv && (I != J || col <= row))
          A[static_cast<int64_t>(r0 + row) * n + c0 + col] = old[j][r] - acc[ii][j][r];
      });
    }
  }
}

// One recursive-doubling level (see trtri_level_kernel) on 128x128 tiles, s >= 128.
__global__ void __launch_bounds__(256, 2) trtri_big_kernel(double* __restrict__ L, double* __restrict__ Linv, int n,
                                                        int s, int phase, int pair0) {
  __shared__ BigSmem sm;
  const int b1 = (pair0 + blockIdx.x) * 2 * s;
  const int b2 = b1 + s;
  if (b2 >= n) return;
  const int s2 = (n - b2 < s) ? n - b2 : s;
  // longest K first (see trtri_level_kernel)
  const int tcols = s / kT2;
  const int yq = blockIdx.y / tcols, yr = blockIdx.y % tcols;
  const int tr = (phase == 0) ? yr : tcols - 1 - yq;
  const int tc = (phase == 0) ? yq : yr;
  const int rows0 = tr * kT2, cols0 = tc * kT2;
  if (rows0 >= s2) return;
  const int mv = (s2 - rows0 < kT2) ? s2 - rows0 : kT2;
  f64x4 acc[4][4];
  zero_acc4(acc);
  if (phase == 0) {
    // T = L21 X11 over q >= cols0, written transposed (T^T) into the strict
    // upper triangle of A through LDS, 64 columns at a time, so rows coalesce.
    gemm128<false, 16>(L + static_cast<int64_t>(b2 + rows0) * n + b1, n, Linv + static_cast<int64_t>(b1) * n + b1 + cols0,
                   n, mv, kT2, cols0, s, acc, sm);
    double* st = &sm.a[0][0][0];  // [64 columns][128 rows + 1]
    constexpr int kSt = kT2 + 1;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      big_foreach([&](int i, int j, int r, int row, int col) {
        if ((col >> 6) == half) st[(col & 63) * kSt + row] = acc[i][j][r];
      });
      __syncthreads();
      for (int e = threadIdx.x; e < 64 * kT2; e += 256) {
        const int c = e >> 7, r = e & 127;
        if (r < mv) L[static_cast<int64_t>(b1 + cols0 + 64 * half + c) * n + b2 + rows0 + r] = st[c * kSt + r];
      }
      __syncthreads();
    }
  } else {
    // X21 = -X22 T over q < rows0 + 128, T read back from its transposed copy.
    const int kend = (rows0 + kT2 < s2) ? rows0 + kT2 : s2;
    gemm128<true, 16>(Linv + static_cast<int64_t>(b2 + rows0) * n + b2, n, L + static_cast<int64_t>(b1 + cols0) * n + b2,
                  n, mv, kT2, 0, kend, acc, sm);
    big_foreach([&](int i, int j, int r, int row, int col) {
      if (row < mv) Linv[static_cast<int64_t>(b2 + rows0 + row) * n + b1 + cols0 + col] = -acc[i][j][r];
    });
  }
}

// One level of the recursive-doubling inverse.  Pair p = pair0 + blockIdx.x
// joins blocks [b1, b1+s) and [b2, b2+s2), b1 = 2ps, b2 = b1+s.  phase 0: T = L21 X11,
// stored transposed at A[b1.., b2..] (strict upper triangle of A); phase 1:
// X21 = -X22 T.  grid.x = pairs, grid.y = output tiles of the pair (s/64 x s/64).
__global__ void __launch_bounds__(256) trtri_level_kernel(double* __restrict__ L, double* __restrict__ Linv,
                                                          int n, int s, int phase, int pair0) {
  __shared__ TileSmem sm;
  const int b1 = (pair0 + blockIdx.x) * 2 * s;
  const int b2 = b1 + s;
  if (b2 >= n) return;
  const int s2 = (n - b2 < s) ? n - b2 : s;
  // Tiles are dispatched longest K first: phase 0 sums over q >= cols0
  // (longest for the first tile column), phase 1 over q < rows0 + 64 (longest
  // for the last tile row).  Work-group y takes tiles y, y + gridDim.y, ...
  const int tcols = s / kB;
  for (int y = blockIdx.y; y < tcols * tcols; y += gridDim.y) {
    const int yq = y / tcols, yr = y % tcols;
    const int tr = (phase == 0) ? yr : tcols - 1 - yq;
    const int tc = (phase == 0) ? yq : yr;
    const int rows0 = tr * kB, cols0 = tc * kB;  // within the s2 x s output
    if (rows0 >= s2) continue;
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

// info_dev == nullptr: the flag lives in the workspace and is read back into
// *info_host (one synchronization); else it is written to info_dev in stream
// order and the call does not synchronize.
hipError_t launch_prepare(const double* H, int64_t n64, double damp, int desc_act, float* U, int32_t* perm,
                          uint8_t* dead, void* ws, hipStream_t s, int* info_host, int32_t* info_dev) {
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
  int* info = info_dev ? info_dev : reinterpret_cast<int*>(p);

  hipError_t e;
#define GPTQ_CHECK_LAUNCH()          \
  do {                               \
    e = hipGetLastError();           \
    if (e != hipSuccess) return e;   \
  } while (0)
  e = zero_i32(info, s);
  if (e != hipSuccess) return e;
  const int nblk = (n + kB - 1) / kB;
  // Look-ahead: after a group, only the next group's block columns are
  // updated on the caller's stream (the strip); the rest of the trailing
  // matrix is updated on a second stream while the next group's
  // latency-bound panel steps run.
  // The strip of group g+1 waits for the side pass of group g, which covers
  // its columns; nothing else the chain touches overlaps the side pass.
  hipStream_t side = nullptr;
  EventPair ev;
  if (nblk > 2 * kGroup) {
    e = side_stream(&side);
    if (e == hipSuccess) e = ev.create();
    if (e != hipSuccess) return e;
  }
  hipEvent_t ev_fork = ev.fork, ev_join = ev.join;
  // Linv is cleared on the side stream beside the prologue kernels below,
  // none of which touch it; the first panel step, its first writer, waits.
  if (side) {
    e = hipEventRecord(ev_fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, ev_fork, 0);
    if (e == hipSuccess) e = zero_words(Linv, static_cast<size_t>(n) * n, side);
    if (e == hipSuccess) e = hipEventRecord(ev_join, side);
  } else {
    e = zero_words(Linv, static_cast<size_t>(n) * n, s);
  }
  if (e != hipSuccess) return e;
  const int nb = (n + 255) / 256;
  hipLaunchKernelGGL(prep_diag_kernel, dim3(nb), dim3(256), 0, s, H, n, dd, dead, info, desc_act, perm);
  GPTQ_CHECK_LAUNCH();
  if (desc_act) {
    hipLaunchKernelGGL(prep_rank_kernel, dim3(nb), dim3(256), 0, s, dd, n, desc_act, perm);
    GPTQ_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(prep_lambda_kernel, dim3(1), dim3(1024), 0, s, dd, n, damp, lam);
  GPTQ_CHECK_LAUNCH();
  const unsigned gy = n < 65535 ? n : 65535;
  hipLaunchKernelGGL(prep_gather_kernel, dim3((n + 1) / 2), dim3(256), 0, s, H, perm, dd, lam, n, desc_act, A);
  GPTQ_CHECK_LAUNCH();
  if (side) {
    e = hipStreamWaitEvent(s, ev_join, 0);   // Linv cleared
    if (e != hipSuccess) return e;
  }
  // Triangular inverse by recursive doubling over levels sz = 64, 128, ...,
  // h, where h (the largest such size below n) is the top level: one pair,
  // [0, h) and [h, n).  The levels inside [0, h) and the top level's first
  // product T = L21 X11 need only block columns < h of L, so they run on a
  // second side stream as soon as the step for block column h/64 - 1 is done,
  // beside the rest of the factorization, which writes nothing they read.
  // For h <= 2048 the first product runs on 3/8 of the compute units, each
  // held whole, so the strips and steps keep the rest; for larger h on the
  // whole chip.  The levels inside [h, n) and the top level's second product
  // follow the factorization on the caller's stream.
  auto level = [&](int sz, int phase, int pair0, int npairs, hipStream_t st) -> hipError_t {
    if (npairs <= 0) return hipSuccess;
    if (sz < kT2 || npairs * (sz / kT2) * (sz / kT2) < kBigTiles) {
      hipLaunchKernelGGL(trtri_level_kernel, dim3(npairs, (sz / kB) * (sz / kB)), dim3(256), 0, st, A, Linv, n, sz,
                         phase, pair0);
    } else {
      hipLaunchKernelGGL(trtri_big_kernel, dim3(npairs, (sz / kT2) * (sz / kT2)), dim3(256), 0, st, A, Linv, n, sz,
                         phase, pair0);
    }
    return hipGetLastError();
  };
  int h = 0;
  for (int sz = kB; sz < n; sz *= 2) h = sz;
  hipStream_t side2 = nullptr;
  EventPair ev2;
  int top_wgs = 0;
  if (side && h >= 4 * kB) {
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = side_stream(&side2, 1);
    if (e == hipSuccess) e = ev2.create();
    if (e != hipSuccess) return e;
    top_wgs = (cus * 3 / 8 > 1) ? cus * 3 / 8 : 1;
  }
  bool pending = false;  // a side pass is in flight
  for (int k0 = 0; k0 < nblk; k0 += kGroup) {
    const int ke = (k0 + kGroup < nblk) ? k0 + kGroup : nblk;
    for (int k = k0; k < ke; ++k) {
      // Events that other streams wait for are recorded by the launch of the
      // kernel they follow (hipExtLaunchKernelGGL's stop event) rather than by
      // a separate record, which costs the stream a further 1-2 us.
      const bool top_fork = side2 && k == h / kB - 1;  // block columns < h are final
      hipExtLaunchKernelGGL(chol_step_kernel, dim3(nblk - k), dim3(256), 0, s, nullptr, top_fork ? ev2.fork : nullptr,
                            0, A, Linv, n, k, k0, ke, info);
      GPTQ_CHECK_LAUNCH();
      if (top_fork) {
        e = hipStreamWaitEvent(side2, ev2.fork, 0);
        for (int sz = kB; e == hipSuccess && sz < h; sz *= 2) {
          e = level(sz, 0, 0, h / (2 * sz), side2);
          if (e == hipSuccess) e = level(sz, 1, 0, h / (2 * sz), side2);
        }
        // the top level's first product, long before the factorization ends:
        // up to h = 2048, on a few compute units held whole (enough LDS per
        // work-group that no step, strip or trailing-pass work-group fits
        // beside one), since the panel steps left after block column h are a
        // long latency-bound chain beside a small product; beyond that on the
        // whole chip, since the product (about h^3/2 flop) then outweighs the
        // rest of the factorization, which finishes early and would wait for
        // it (measured: 502 -> 354 ms at n = 28672, 13.4 -> 12.3 ms at 8192,
        // but 2.95 -> 3.7 ms at 4096)
        if (e == hipSuccess && h > kTopSplitMax) {
          e = level(h, 0, 0, 1, side2);
        } else if (e == hipSuccess) {
          const int tiles = (h / kB) * (h / kB);
          const int wgs = (top_wgs < tiles) ? top_wgs : tiles;
          hipExtLaunchKernelGGL(trtri_level_kernel, dim3(1, wgs), dim3(256), kTopLds - sizeof(TileSmem), side2, nullptr,
                                ev2.join, 0, A, Linv, n, h, 0, 0);
          e = hipGetLastError();
        }
        if (e == hipSuccess && h > kTopSplitMax) e = hipEventRecord(ev2.join, side2);
        if (e != hipSuccess) return e;
      }
    }
    if (ke >= nblk) break;
    const int ne = (ke + kGroup < nblk) ? ke + kGroup : nblk;
    // the strip (block columns ke .. ne-1), after the previous side pass
    if (pending) {
      e = hipStreamWaitEvent(s, ev_join, 0);
      if (e != hipSuccess) return e;
      pending = false;
    }
    int strip = 0;
    for (int j = ke; j < ne; ++j) strip += nblk - j;
    const bool fork = side && ne < nblk;  // a side pass follows: its fork is recorded by the strip's launch
    hipExtLaunchKernelGGL(chol_update_kernel, dim3(strip), dim3(256), 0, s, nullptr, fork ? ev_fork : nullptr, 0, A, n,
                          k0, ke, ke, 2, nblk, ne - ke);
    GPTQ_CHECK_LAUNCH();
    // the rest (block columns >= ne), K = 64 * group width; forked after the
    // strip so that the strip, which the next panel step waits for, is not
    // queued behind the larger pass for compute units
    if (ne < nblk) {
      hipStream_t st = side ? side : s;
      if (side) {
        e = hipStreamWaitEvent(side, ev_fork, 0);
        if (e != hipSuccess) return e;
      }
      hipEvent_t done = side ? ev_join : nullptr;
      const int nt = (n - ne * kB + kT2 - 1) / kT2;
      if (nt * (nt + 1) / 2 >= (n <= kSmallN ? kTrailBigTilesSmallN : kBigTiles)) {
        hipExtLaunchKernelGGL(chol_trail_kernel, dim3(nt * (nt + 1) / 2), dim3(256), 0, st, nullptr, done, 0, A, n, k0,
                              ke, ne * kB);
      } else {
        const int rest = nblk - ne;
        hipExtLaunchKernelGGL(chol_update_kernel, dim3(rest * (rest + 1) / 2), dim3(256), 0, st, nullptr, done, 0, A, n,
                              k0, ke, ne, 0, nblk, 1);
      }
      GPTQ_CHECK_LAUNCH();
      if (side) pending = true;
    }
  }
  if (pending) {
    e = hipStreamWaitEvent(s, ev_join, 0);
    if (e != hipSuccess) return e;
  }
  if (side2) {
    for (int sz = kB; sz < h; sz *= 2) {
      const int p0 = h / (2 * sz), np = (n - h + 2 * sz - 1) / (2 * sz);
      e = level(sz, 0, p0, np, s);
      if (e == hipSuccess) e = level(sz, 1, p0, np, s);
      if (e != hipSuccess) return e;
    }
    e = hipStreamWaitEvent(s, ev2.join, 0);
    if (e == hipSuccess) e = level(h, 1, 0, 1, s);
    if (e != hipSuccess) return e;
  } else {
    for (int sz = kB; sz < n; sz *= 2) {
      const int pairs = (n + 2 * sz - 1) / (2 * sz);
      e = level(sz, 0, 0, pairs, s);
      if (e == hipSuccess) e = level(sz, 1, 0, pairs, s);
      if (e != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(write_u_kernel, dim3((n + 255) / 256, gy), dim3(256), 0, s, Linv, n, U);
  GPTQ_CHECK_LAUNCH();
#undef GPTQ_CHECK_LAUNCH
  if (info_dev) return hipSuccess;
  e = hipMemcpyAsync(info_host, info, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace gptq
