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
// Row stride of the sweep's staged block of W (Ws[column][row]): one float of
// padding, so that 32 lanes reading 32 different columns at one row offset
// (the MFMA accumulator layout of the far and pending updates) hit 32
// different banks, while the chain's reads (one column, lane = row) stay
// conflict-free.
constexpr int kWs = kRowsSweep + 1;
// The errors of a sub-block, Es[t][row ^ es_swz(t)]: the far update's MFMA
// operand has lanes 0-31 on column t and lanes 32-63 on t + 1 at the same
// rows; flipping bit 5 of the row on odd t puts the two halves on disjoint
// banks.
__device__ __forceinline__ int es_swz(int t) { return (t & 1) << 5; }

// ---------------------------------------------------------------- gather
// Wk[r][j] = W[r][perm[j]] as fp32 (0 for dead columns).  Four consecutive
// output columns per thread, written as one 16-byte store when n % 4 == 0
// and Wk is 16-byte aligned (every row start then is), else one by one.
template <int DT>
__global__ void gather_w_kernel(const void* __restrict__ W, int64_t ldw, const int32_t* __restrict__ perm,
                                const uint8_t* __restrict__ dead, int rows, int n, float* __restrict__ Wk,
                                bool aligned) {
  const int nq = (n + 3) / 4;
  const bool vec = (n % 4) == 0 && (reinterpret_cast<uintptr_t>(Wk) & 15) == 0;
  for (int r = blockIdx.y; r < rows; r += gridDim.y) {
    for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += gridDim.x * blockDim.x) {
      const int j0 = 4 * q;
      float v[4];
      // Without act-order perm is the identity: with W, perm and dead aligned
      // (checked by the caller) the four weights, their indexes and their
      // dead flags then come in one load each instead of through perm.
      bool ident = false;
      if (aligned && vec) {
        const int4 pj = *reinterpret_cast<const int4*>(perm + j0);
        ident = pj.x == j0 && pj.y == j0 + 1 && pj.z == j0 + 2 && pj.w == j0 + 3;
      }
      if (ident) {
        const int64_t o = static_cast<int64_t>(r) * ldw + j0;
        const uint32_t dflags = *reinterpret_cast<const uint32_t*>(dead + j0);
        float w[4];
        if constexpr (DT == DT_FP32) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(W) + o);
          w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
        } else {
          const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(W) + o);
          const uint16_t h[4] = {static_cast<uint16_t>(x.x), static_cast<uint16_t>(x.x >> 16),
                                 static_cast<uint16_t>(x.y), static_cast<uint16_t>(x.y >> 16)};
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (DT == DT_BF16) ? bf16_bits_to_float(h[e]) : half_bits_to_float(h[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ((dflags >> (8 * e)) & 0xFFu) ? 0.0f : w[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = j0 + e;
          v[e] = 0.0f;
          if (j < n) {
            const int src = perm[j];
            if (!dead[src]) v[e] = load_as_float<DT>(W, static_cast<int64_t>(r) * ldw + src);
          }
        }
      }
      float* dst = Wk + static_cast<int64_t>(r) * n + j0;
      if (vec) {
        *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + e < n) dst[e] = v[e];
      }
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

// ---------------------------------------------------------------- split-bf16 helpers
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

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, f32x16 c) {
  bf16x8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
}

// ---------------------------------------------------------------- pre-split operands
// The block updates multiply fp32 errors E by rows of U on the bf16 MFMA as
// E U ~ Ehi Uhi + Ehi Ulo + Elo Uhi (see the trailing update).  Both operands
// are split once, not per tile: U is transposed and split at the start of a
// layer (UTh/UTl [n][n], UT[c][k] = U[k][c], so a column's k values are
// contiguous), and the sweep writes its errors already split (Eh/El).  The
// update kernels then stage 16-byte copies into LDS, no arithmetic.
__global__ void __launch_bounds__(256) split_ut_kernel(const float* __restrict__ U, int n, uint16_t* __restrict__ UTh,
                                                       uint16_t* __restrict__ UTl) {
  __shared__ float t[64][65];
  const int k0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 16; ++q) t[ty + 4 * q][tx] = U[static_cast<int64_t>(k0 + ty + 4 * q) * n + c0 + tx];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int c = ty + 4 * q;
    const float v = t[tx][c];
    const uint32_t h = bf16_rne_bits(v);
    const uint32_t l = bf16_rne_bits(v - __uint_as_float(h << 16));
    UTh[static_cast<int64_t>(c0 + c) * n + k0 + tx] = static_cast<uint16_t>(h);
    UTl[static_cast<int64_t>(c0 + c) * n + k0 + tx] = static_cast<uint16_t>(l);
  }
}

// Staged operand planes: rows of 64 bf16 values (128 bytes = eight 16-byte
// units of 8 k); unit u of row r sits at slot u ^ ((r >> 1) & 7).  LDS has
// 64 banks of 4 bytes and serves 16 lanes of a 16-byte access per cycle: the
// fragment reads (16 lanes on 16 consecutive rows, one unit) then touch 16
// distinct 16-byte bank groups (even and odd rows fall in different halves
// of 256 bytes, and the 8 rows of one parity on 8 slots), as do the stores
// (16 lanes on two rows, all eight units of each).  Keyed on r & 7 instead,
// rows r and r + 8 shared a slot and every read took two cycles.
constexpr int kTK = 64;
// 128-wide trailing tiles from this many tiles on (one per compute unit);
// fewer tiles run 64 wide, twice as many work-groups
constexpr int kTrailWideTiles = 256;
__device__ __forceinline__ int tk_offset(int row, int c) {
  return row * (kTK * 2) + ((c ^ ((row >> 1) & 7)) << 4);
}

// ---------------------------------------------------------------- pending block update
// Before its chain, a sweep workgroup applies to its own 64 rows x 128
// columns of the working weights (held in LDS) the updates of earlier blocks
// that have not been written to memory: Ws -= Ea Ua + Eb Ub, split-bf16 MFMA
// with fp32 accumulation.  Each segment is split errors (Eh/El [rows, K], row
// stride ldE) and the K matching rows of U at this block's columns (from
// UTh/UTl).  K runs in chunks of 64 staged in LDS, the next two chunks' copies
// in flight in registers during the current chunk's MFMAs.  Wave w owns columns
// 32w..32w+31 as two v_mfma_f32_32x32x16_bf16 tiles (rows 0-31 and 32-63);
// accumulator q of lane l is row 8(q/4) + 4(l/32) + q%4, column l%32.
struct PendSmem {
  uint8_t eh[kRowsSweep * kTK * 2], el[kRowsSweep * kTK * 2];
  uint8_t uh[kBlk * kTK * 2], ul[kBlk * kTK * 2];
};
struct PendSeg {
  const uint16_t* Eh;  // split errors, columns 0 .. K-1
  const uint16_t* El;
  int K;               // a multiple of kTK
  int urow;            // first row of U matching column 0 of E
};

__device__ __forceinline__ void pending_update(float (*Ws)[kWs], const uint16_t* __restrict__ UTh,
                                               const uint16_t* __restrict__ UTl, int n, int rows, int rbase, int i1,
                                               int ldE, const PendSeg& sa, const PendSeg& sb, PendSmem& sm) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nca = sa.K / kTK, nc = nca + sb.K / kTK;
  if (nc == 0) return;
  // two register sets: while one chunk is in LDS, the next two are in flight
  u32x4 re[2][2][2], ru[2][2][4];  // [set][plane][unit]
  auto gload = [&](int c, int set) {
    const bool first = c < nca;
    const uint16_t* Eh = first ? sa.Eh : sb.Eh;
    const uint16_t* El = first ? sa.El : sb.El;
    const int kc = (first ? c : c - nca) * kTK;
    const int ur = (first ? sa.urow : sb.urow) + kc;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int u = tid + 256 * q, row = u >> 3, unit = u & 7;
      const int r = rbase + row;
      const int64_t off = static_cast<int64_t>(r) * ldE + kc + 8 * unit;
      const u32x4 z = {0u, 0u, 0u, 0u};
      re[set][0][q] = (r < rows) ? *reinterpret_cast<const u32x4*>(Eh + off) : z;
      re[set][1][q] = (r < rows) ? *reinterpret_cast<const u32x4*>(El + off) : z;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + 256 * q, col = u >> 3, unit = u & 7;
      const int64_t off = static_cast<int64_t>(i1 + col) * n + ur + 8 * unit;
      ru[set][0][q] = *reinterpret_cast<const u32x4*>(UTh + off);
      ru[set][1][q] = *reinterpret_cast<const u32x4*>(UTl + off);
    }
  };
  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[i][q] = 0.0f;
  auto step = [&](int c, int set) {
    if (c) __syncthreads();  // the previous chunk's fragments have been read
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int u = tid + 256 * q;
      *reinterpret_cast<u32x4*>(sm.eh + tk_offset(u >> 3, u & 7)) = re[set][0][q];
      *reinterpret_cast<u32x4*>(sm.el + tk_offset(u >> 3, u & 7)) = re[set][1][q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + 256 * q;
      *reinterpret_cast<u32x4*>(sm.uh + tk_offset(u >> 3, u & 7)) = ru[set][0][q];
      *reinterpret_cast<u32x4*>(sm.ul + tk_offset(u >> 3, u & 7)) = ru[set][1][q];
    }
    __syncthreads();
    if (c + 2 < nc) gload(c + 2, set);
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
      const int unit = 2 * ks + (lane >> 5);
      u32x4 ah[2], al[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 32 * i + (lane & 31);
        ah[i] = *reinterpret_cast<const u32x4*>(sm.eh + tk_offset(row, unit));
        al[i] = *reinterpret_cast<const u32x4*>(sm.el + tk_offset(row, unit));
      }
      const int col = 32 * wave + (lane & 31);
      const u32x4 bh = *reinterpret_cast<const u32x4*>(sm.uh + tk_offset(col, unit));
      const u32x4 bl = *reinterpret_cast<const u32x4*>(sm.ul + tk_offset(col, unit));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        acc[i] = mfma_bf16(al[i], bh, acc[i]);
        acc[i] = mfma_bf16(ah[i], bl, acc[i]);
        acc[i] = mfma_bf16(ah[i], bh, acc[i]);
      }
    }
  };
  gload(0, 0);
  if (nc > 1) gload(1, 1);
  for (int c = 0; c < nc; c += 2) {
    step(c, 0);
    if (c + 1 < nc) step(c + 1, 1);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q)
      Ws[32 * wave + (lane & 31)][32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)] -= acc[i][q];
}

// ---------------------------------------------------------------- quantization grid
// Scale and zero point of a group whose values span [xmin, xmax] with
// xmin <= 0 <= xmax (the range always includes 0); a range of {0} takes
// [-1, 1].  polydesk.ai "GPTQ" glossary, "Paramètres clés" (sym): the
// asymmetric grid has a non-zero zero point; the symmetric grid spans
// -(2^(b-1)-1) .. 2^(b-1)-1 steps with zero exact (SYM = 1).  SYM = 2 spreads
// the symmetric range [-a, a] over all 2^b codes (zero still exact, the zero
// point being the integer 2^(b-1)).
//   SYM 0: s = (xmax - xmin) / maxq,           z = rint(-xmin / s)
//   SYM 1: s = max(-xmin, xmax) / (2^(b-1)-1), z = 2^(b-1)
//   SYM 2: s = (a - (-a)) / maxq,              z = 2^(b-1),  a = max(-xmin, xmax)
template <int BITS, int SYM>
__device__ __forceinline__ void grid_from_range(float xmin, float xmax, float& s, float& z) {
  constexpr float maxq = static_cast<float>((1 << BITS) - 1);
  if (xmin == 0.0f && xmax == 0.0f) {
    xmin = -1.0f;
    xmax = 1.0f;
  }
  if constexpr (SYM == 1) {
    const float a = fmaxf(-xmin, xmax);
    s = a / static_cast<float>((1 << (BITS - 1)) - 1);
    z = static_cast<float>(1 << (BITS - 1));
  } else if constexpr (SYM == 2) {
    const float a = fmaxf(-xmin, xmax);
    s = (a - (-a)) / maxq;
    z = static_cast<float>(1 << (BITS - 1));
  } else {
    s = (xmax - xmin) / maxq;
    z = rintf(-xmin / s);
  }
}

// One group per row (group_size -1): the grid of each row from all n of its
// columns as gathered, before any of them is updated.  grid.x = rows.
template <int BITS, int SYM>
__global__ void __launch_bounds__(256) row_params_kernel(const float* __restrict__ Wk, int n, int rows,
                                                          float* __restrict__ rowsz) {
  __shared__ float smin[256], smax[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  float xmin = 0.0f, xmax = 0.0f;
  for (int k = tid; k < n; k += 256) {
    const float v = Wk[static_cast<int64_t>(r) * n + k];
    xmin = fminf(xmin, v);
    xmax = fmaxf(xmax, v);
  }
  smin[tid] = xmin;
  smax[tid] = xmax;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      smin[tid] = fminf(smin[tid], smin[tid + w]);
      smax[tid] = fmaxf(smax[tid], smax[tid + w]);
    }
    __syncthreads();
  }
  if (tid == 0) {
    float sv, zv;
    grid_from_range<BITS, SYM>(smin[0], smax[0], sv, zv);
    rowsz[2 * r] = sv;
    rowsz[2 * r + 1] = zv;
  }
}

// ---------------------------------------------------------------- sweep
// One workgroup (4 waves) per strip of 64 rows and one block of 128 columns;
// lane = row in every wave.  LDS: UT[k][j] = U[i1+j][i1+k] (the block of U,
// transposed), the 64x128 block of Wk column-major over rows, and the errors
// of the last two 16-column sub-blocks.  The block first receives its pending
// updates (pending_update above), then the chain runs.
// Sub-block s (16 columns), two barriers:
//   wave 0   : the sequential chain -- quantize column j, e_j = (w - q) / U_jj,
//              rank-1 update of the remaining columns of the sub-block (the
//              16x16 block of U is read into registers first);
//   waves 1-3: meanwhile write the split errors of sub-block s-1 and apply
//              them to the columns from sub-block s+1 on ("far" update, fp32
//              MFMA);
//   barrier; all waves apply the errors of sub-block s to the columns of
//   sub-block s+1 ("near" update, which the next chain step needs); barrier.
// Codes: c = clamp(rint(w / s) + z).  Each sub-block's chain first runs with
// the quotient formed as w * (1/s).  rint decides a code only while
// |w / s| <= maxq + 1/2 < 2^b (beyond that the clamp does); there w * (1/s)
// errs by at most ~2 ulp, under 2^(b-22) (2^-18 for b <= 4).  If any quotient
// lay within that distance of a rounding midpoint, the sub-block is replayed
// from its saved inputs with IEEE division, so the codes equal those of a
// correctly rounded w / s.  The fast path has no branch inside the chain.
constexpr int kSubs = kBlk / kSub;  // 8
template <int BITS>
constexpr float near_midpoint() {
  return (BITS <= 4) ? 3.814697265625e-06f : 3.814697265625e-06f * static_cast<float>(1 << (BITS - 4));
}

// One launch sweeps the nb blocks of a super-block from column s1: a
// work-group's pending updates need only its own rows' errors of the earlier
// blocks (written to Ejh/Ejl, read back after a work-group barrier), so the
// blocks follow one another inside the work-group without a launch between.
template <int BITS, int SYM>
__global__ void __launch_bounds__(256) sweep_block_kernel(
    const float* __restrict__ Wk, const float* __restrict__ U, const uint16_t* __restrict__ UTh,
    const uint16_t* __restrict__ UTl, int n, int rows, int s1, int nb, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ Ejh, uint16_t* __restrict__ Ejl, int ldE, PendSeg sa,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, double* __restrict__ rowloss, int gs,
    const float* __restrict__ rowsz) {
  __shared__ __attribute__((aligned(16))) float UT[kBlk][kBlk + 4];
  __shared__ float Ws[kBlk][kWs];
  __shared__ __attribute__((aligned(16))) PendSmem psm;
  __shared__ float Es[2][kSub][kRowsSweep];
  __shared__ float rdiag[kBlk];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = blockIdx.x * kRowsSweep + lane;
  const bool valid = r < rows;
  double loss = 0.0;
  for (int blk = 0; blk < nb; ++blk) {
  const int i1 = s1 + blk * kBlk;
  uint16_t* const Eh = Ejh + blk * kBlk;  // this block's columns of the split errors
  uint16_t* const El = Ejl + blk * kBlk;
  const PendSeg sb{Ejh, Ejl, blk * kBlk, s1};  // the earlier blocks of the super-block
  if (blk > 0) {
    // the previous block's split errors (global) are visible to every wave,
    // and its LDS contents are no longer read
    __threadfence_block();
    __syncthreads();
  }

  // Staging: every global load of the block is issued before the LDS stores.
  // LDS banks on this chip: 4-byte stores see word % 32 per half-wave, 16-byte
  // stores unit % 8 per 8 consecutive lanes.  UT[k][j] = U[i1+j][i1+k] is
  // staged with the lanes on consecutive columns k (coalesced loads), four
  // rows j .. j+3 per 16-byte store, which lands 8 consecutive lanes on 8
  // distinct units (rows of 33 units); a lane per row j with 4-byte stores
  // met 16 to a bank.  Ws[k][row] takes a row per lane and a quarter of the
  // 32-column range per wave: a half-wave's stores hit 32 distinct banks
  // (with four lanes per row they met 4 to a bank).
  {
    float ut[16][4];  // unit i: column k = e & 127, rows 4 (e >> 7) .. + 3, e = tid + 256 i
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = tid + 256 * i, k = e & 127, j = 4 * (e >> 7);
#pragma unroll
      for (int r = 0; r < 4; ++r) ut[i][r] = U[static_cast<int64_t>(i1 + j + r) * n + i1 + k];
    }
    const int rr = tid & 63, q = tid >> 6;
    const int gr = blockIdx.x * kRowsSweep + rr;
    f32x4 wv[8];
#pragma unroll
    for (int k4 = 0; k4 < 8; ++k4)
      wv[k4] = (gr < rows) ? *reinterpret_cast<const f32x4*>(Wk + static_cast<int64_t>(gr) * n + i1 + q * 32 + 4 * k4)
                           : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const float dg = (tid < kBlk) ? U[static_cast<int64_t>(i1 + tid) * n + i1 + tid] : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = tid + 256 * i, k = e & 127, j = 4 * (e >> 7);
      *reinterpret_cast<f32x4*>(&UT[k][j]) = f32x4{ut[i][0], ut[i][1], ut[i][2], ut[i][3]};
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
  pending_update(Ws, UTh, UTl, n, rows, blockIdx.x * kRowsSweep, i1, ldE, sa, sb, psm);
  __syncthreads();

  constexpr float maxq = static_cast<float>((1 << BITS) - 1);
  const float lo = (SYM == 1) ? 1.0f : 0.0f;
  float sv = 1.0f, zv = 0.0f, rs = 1.0f;
  // Wave 0: scale and zero point of the group of columns c0 .. c0 + cnt - 1
  // of the block, from their current (compensated) values, written out as
  // group (i1 + c0) / gs.  The range includes 0; a group whose range is {0}
  // takes [-1, 1].
  auto group_params = [&](int c0, int cnt) {
    float xmin = 0.0f, xmax = 0.0f;
    for (int k = c0; k < c0 + cnt; ++k) {
      const float v = Ws[k][lane];
      xmin = fminf(xmin, v);
      xmax = fmaxf(xmax, v);
    }
    grid_from_range<BITS, SYM>(xmin, xmax, sv, zv);
    rs = 1.0f / sv;
    if (valid) {
      const int g = (i1 + c0) / gs;
      scales[static_cast<int64_t>(g) * rows + r] = float_to_half_bits(sv);
      zeros[static_cast<int64_t>(g) * rows + r] = float_to_half_bits(zv);
    }
  };
  if (wave == 0) {
    if (gs > 0) {
      group_params(0, gs < kBlk ? gs : kBlk);
    } else {  // one group per row, its parameters taken before the sweep
      sv = valid ? rowsz[2 * r] : 1.0f;
      zv = valid ? rowsz[2 * r + 1] : 0.0f;
      rs = 1.0f / sv;
      if (valid && i1 == 0) {
        scales[r] = float_to_half_bits(sv);
        zeros[r] = float_to_half_bits(zv);
      }
    }
  }
  // groups narrower than a block start at sub-blocks sb % (gs / 16) == 0
  const int gsub = (gs > 0 && gs < kBlk) ? gs / kSub : kSubs;

  uint16_t* ehrow = Eh + static_cast<int64_t>(valid ? r : 0) * ldE;
  uint16_t* elrow = El + static_cast<int64_t>(valid ? r : 0) * ldE;
  uint8_t* crow = codes + static_cast<int64_t>(valid ? r : 0) * n + i1;
  // Waves 1-3: errors of sub-block sb-1 onto the columns from sub-block sb+1 on.
  auto far_update = [&](int sb) {
    const int j0 = sb * kSub;
    // fp32 MFMA: Ws[c][r] -= sum_t E[r][t] U[jp + t][c] over 32x32 tiles
    // (v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][l/32] and
    // B[l/32][l%32]; accumulator q of lane l is row 8(q/4) + 4(l/32) + q%4,
    // column l%32).  Column tiles are aligned to 32; columns of the first
    // tile below j0 + 16 (the chain's own sub-block) read U as 0 and are not
    // written.  Tiles (row tile, column tile) are dealt to waves 1-3.
    const int jp = j0 - kSub;
    const int cfirst = j0 + kSub, ct0 = cfirst >> 5;
    const int ntl = 2 * (kBlk / 32 - ct0);
    const float(*Ep)[kRowsSweep] = Es[(sb - 1) & 1];
    for (int x = wave - 1; x < ntl; x += 3) {
      const int rt = x & 1, ct = ct0 + (x >> 1);
      const int col = 32 * ct + (lane & 31);
      const bool on = col >= cfirst;
      // every LDS read of the tile first (operands and the old weights),
      // then the MFMAs, then the writes
      float a[kSub / 2], b[kSub / 2], w[16];
#pragma unroll
      for (int ks = 0; ks < kSub / 2; ++ks) {
        const int t = 2 * ks + (lane >> 5);
        a[ks] = Ep[t][(32 * rt + (lane & 31)) ^ es_swz(t)];
        b[ks] = on ? UT[col][jp + t] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) w[q] = Ws[col][32 * rt + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)];
      f32x16 acc;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kSub / 2; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[ks], b[ks], acc, 0, 0, 0);
      if (on) {
#pragma unroll
        for (int q = 0; q < 16; ++q) Ws[col][32 * rt + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)] = w[q] - acc[q];
      }
    }
  };
  // Waves 1-3: the errors of sub-block sp as split bf16 planes (hi, lo) into
  // Eh/El for the later lazy updates, off the chain wave.  Wave 1 writes
  // columns 0-7 of the sub-block, wave 2 columns 8-15 (four per 8-byte store).
  auto store_split = [&](int sp) {
    if (!valid || wave == 3) return;
    const int jp = sp * kSub + 8 * (wave - 1);
#pragma unroll
    for (int h4 = 0; h4 < 2; ++h4) {
      uint32_t h[4], l[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int t = 8 * (wave - 1) + 4 * h4 + d;
        const float v = Es[sp & 1][t][lane ^ es_swz(t)];
        h[d] = bf16_rne_bits(v);
        l[d] = bf16_rne_bits(v - __uint_as_float(h[d] << 16));
      }
      *reinterpret_cast<uint2*>(ehrow + jp + 4 * h4) = uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *reinterpret_cast<uint2*>(elrow + jp + 4 * h4) = uint2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
    }
  };
  for (int sb = 0; sb < kSubs; ++sb) {
    const int j0 = sb * kSub;
    // A group starting inside the block: the errors of sub-block sb-1 reach
    // all of its columns first, then its parameters are taken.
    const bool gstart = sb > 0 && sb % gsub == 0;
    if (gstart) {
      if (wave > 0) {
        store_split(sb - 1);
        far_update(sb);
      }
      __syncthreads();
      if (wave == 0) group_params(j0, gs);
    }
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
      // and reports whether any quotient came within near_midpoint<BITS>() of
      // a rounding midpoint; EXACT = true uses IEEE division throughout.
      float rd[kSub];  // 1 / U_jj of the sub-block, read once, off the chain
#pragma unroll
      for (int t = 0; t < kSub; ++t) rd[t] = rdiag[j0 + t];
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
            near |= fabsf(fabsf(qt - rintf(qt)) - 0.5f) < near_midpoint<BITS>();
          }
          const float c = fminf(fmaxf(rintf(qt) + zv, lo), maxq);
          const float q = sv * (c - zv);
          const float et = (w[t] - q) * rd[t];
          Es[sb & 1][t][lane ^ es_swz(t)] = et;
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
        for (int t4 = 0; t4 < kSub / 4; ++t4) *reinterpret_cast<uint32_t*>(crow + j0 + 4 * t4) = cw[t4];
      }
    } else if (sb >= 1 && !gstart) {
      store_split(sb - 1);
      far_update(sb);
    }
    __syncthreads();
    if (sb + 1 < kSubs) {
      // near update: errors of sub-block sb onto the 16 columns of sub-block
      // sb+1, four columns per wave
      float ec[kSub];
#pragma unroll
      for (int t = 0; t < kSub; ++t) ec[t] = Es[sb & 1][t][lane ^ es_swz(t)];
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
  if (wave > 0) store_split(kSubs - 1);   // Es of the last sub-block is final after the last barrier
  }
  if (wave == 0 && valid) rowloss[r] += 0.5 * loss;
}

// ---------------------------------------------------------------- trailing update
// Wk[r0:r0+128, c0:c0+TN] -= E[r0:r0+128, 0:K] U[i1:i1+K, c0:c0+TN] for
// columns c < ce; E given split (Eh/El, row stride ldE), U as its split
// transpose (UTh/UTl).
// Split-bf16 product on the bf16 MFMA: each fp32 operand x = hi + lo with
// hi = bf16(x), lo = bf16(x - hi) (round to nearest even), and
//   E U ~ Ehi Uhi + Ehi Ulo + Elo Uhi   (fp32 accumulation),
// which leaves a relative error near 2^-16 per product (the dropped Elo Ulo
// term and the rounding of lo), against 2^-24 for an fp32 product.
// K runs in chunks of 64 staged in LDS as bf16 hi/lo planes: E as [row][k], U
// transposed as [col][k], so each MFMA operand fragment (8 consecutive k) is
// one 16-byte read; the next chunk's copies are in flight during the current
// chunk's MFMAs.
// 256 threads; wave (wm, wn) owns a 64 x TN/2 block = 2 x TN/64
// v_mfma_f32_32x32x16_bf16 tiles (accumulator q of lane l is row
// 8(q/4) + 4(l/32) + q%4, column l%32).  TN = 128, or 64 for launches with
// too few 128-wide tiles to occupy every compute unit.
// Tiles are numbered row-major (tiles_x per 128-row band) and dealt so that
// the work-groups of one XCD (block index mod 8) take one contiguous range of
// that order: they share E rows and U columns in that XCD's L2.  The grid is
// a multiple of 8; XCD k's gridDim.x / 8 work-groups walk its range with
// that stride (one tile each when the grid is 8 * ceil(tiles / 8)).
template <int TN>
__global__ void __launch_bounds__(256, 2) trailing_kernel(float* __restrict__ Wk, const uint16_t* __restrict__ Eh,
                                                       const uint16_t* __restrict__ El, int ldE,
                                                       const uint16_t* __restrict__ UTh,
                                                       const uint16_t* __restrict__ UTl, int n, int rows, int i1,
                                                       int K, int cb, int ce, int tiles_x, int tiles) {
  constexpr int NJ = TN / 64;   // MFMA tiles per wave along the columns
  constexpr int QU = TN / 32;   // 16-byte U units per thread and chunk
  __shared__ __attribute__((aligned(16))) uint8_t lds_e[2][128 * kTK * 2];  // Ehi, Elo
  __shared__ __attribute__((aligned(16))) uint8_t lds_u[2][TN * kTK * 2];   // Uhi, Ulo
  const int per = (tiles + 7) / 8;
  const int xcd = static_cast<int>(blockIdx.x % 8);
  const int t_end = ((xcd + 1) * per < tiles) ? (xcd + 1) * per : tiles;
  const int stride = static_cast<int>(gridDim.x / 8);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  for (int t = xcd * per + static_cast<int>(blockIdx.x / 8); t < t_end; t += stride) {
  const int r0 = (t / tiles_x) * 128;
  const int c0 = cb + (t % tiles_x) * TN;
  f32x16 acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  u32x4 re[2][4], ru[2][QU];  // [plane][unit]: unit u = tid + 256q -> (row or column u/8, k-octet u%8)
  auto gload = [&](int kc) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + 256 * q, row = u >> 3, unit = u & 7;
      const bool ok = r0 + row < rows;
      const int64_t off = static_cast<int64_t>(r0 + row) * ldE + kc + 8 * unit;
      re[0][q] = ok ? *reinterpret_cast<const u32x4*>(Eh + off) : z;
      re[1][q] = ok ? *reinterpret_cast<const u32x4*>(El + off) : z;
    }
#pragma unroll
    for (int q = 0; q < QU; ++q) {
      const int u = tid + 256 * q, col = u >> 3, unit = u & 7;
      const bool ok = c0 + col < ce;
      const int64_t off = static_cast<int64_t>(c0 + col) * n + i1 + kc + 8 * unit;
      ru[0][q] = ok ? *reinterpret_cast<const u32x4*>(UTh + off) : z;
      ru[1][q] = ok ? *reinterpret_cast<const u32x4*>(UTl + off) : z;
    }
  };
  gload(0);
  for (int kc = 0; kc < K; kc += kTK) {
    if (kc) __syncthreads();  // the previous chunk's fragments have been read
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = tid + 256 * q;
      *reinterpret_cast<u32x4*>(lds_e[0] + tk_offset(u >> 3, u & 7)) = re[0][q];
      *reinterpret_cast<u32x4*>(lds_e[1] + tk_offset(u >> 3, u & 7)) = re[1][q];
    }
#pragma unroll
    for (int q = 0; q < QU; ++q) {
      const int u = tid + 256 * q;
      *reinterpret_cast<u32x4*>(lds_u[0] + tk_offset(u >> 3, u & 7)) = ru[0][q];
      *reinterpret_cast<u32x4*>(lds_u[1] + tk_offset(u >> 3, u & 7)) = ru[1][q];
    }
    __syncthreads();
    if (kc + kTK < K) gload(kc + kTK);
#pragma unroll
    for (int kk = 0; kk < kTK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      u32x4 ah[2], al[2], bh[NJ], bl[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int m = wm * 64 + i * 32 + (lane & 31);
        ah[i] = *reinterpret_cast<const u32x4*>(lds_e[0] + tk_offset(m, c));
        al[i] = *reinterpret_cast<const u32x4*>(lds_e[1] + tk_offset(m, c));
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int cc = wn * (TN / 2) + j * 32 + (lane & 31);
        bh[j] = *reinterpret_cast<const u32x4*>(lds_u[0] + tk_offset(cc, c));
        bl[j] = *reinterpret_cast<const u32x4*>(lds_u[1] + tk_offset(cc, c));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          acc[i][j] = mfma_bf16(al[i], bh[j], acc[i][j]);
          acc[i][j] = mfma_bf16(ah[i], bl[j], acc[i][j]);
          acc[i][j] = mfma_bf16(ah[i], bh[j], acc[i][j]);
        }
    }
  }
  // Epilogue: all loads of this lane's W values are issued before any store
  // (a load after a store to the same array would otherwise wait for it).
  float old[2][NJ][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rr = r0 + wm * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const int cc = c0 + wn * (TN / 2) + j * 32 + (lane & 31);
        old[i][j][q] = (rr < rows && cc < ce) ? Wk[static_cast<int64_t>(rr) * n + cc] : 0.0f;
      }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rr = r0 + wm * 64 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        const int cc = c0 + wn * (TN / 2) + j * 32 + (lane & 31);
        if (rr < rows && cc < ce) Wk[static_cast<int64_t>(rr) * n + cc] = old[i][j][q] - acc[i][j][q];
      }
  __syncthreads();  // the next tile's first staging overwrites this tile's LDS
  }
}

// Launches the trailing update of columns [cb, ce) by K rows of U from i1, on
// at most max_wgs work-groups (a multiple of 8).  A non-null `done` is
// recorded by the launch itself when the kernel completes (no separate marker
// on the stream: a marker between two kernels of a stream delays the second
// by about 7 us).
static hipError_t launch_trailing(hipStream_t st, float* Wk, const uint16_t* Eh, const uint16_t* El, int ldE,
                                  const uint16_t* UTh, const uint16_t* UTl, int n, int rows, int i1, int K, int cb,
                                  int ce, int max_wgs, hipEvent_t done = nullptr) {
  const int64_t bands = (rows + 127) / 128;
  if (bands * ((ce - cb + 63) / 64) > (int64_t{1} << 30)) return hipErrorInvalidValue;  // grid size
  const int wide_tiles = static_cast<int>(bands * ((ce - cb + 127) / 128));
  if (wide_tiles >= kTrailWideTiles) {
    const int tx = (ce - cb + 127) / 128, tiles = static_cast<int>(bands) * tx;
    const int grid = (tiles < max_wgs) ? 8 * ((tiles + 7) / 8) : max_wgs;
    hipExtLaunchKernelGGL(trailing_kernel<128>, dim3(grid), dim3(256), 0, st, nullptr, done, 0, Wk, Eh, El, ldE, UTh,
                          UTl, n, rows, i1, K, cb, ce, tx, tiles);
  } else {
    const int tx = (ce - cb + 63) / 64, tiles = static_cast<int>(bands) * tx;
    hipExtLaunchKernelGGL(trailing_kernel<64>, dim3(8 * ((tiles + 7) / 8)), dim3(256), 0, st, nullptr, done, 0, Wk, Eh,
                          El, ldE, UTh, UTl, n, rows, i1, K, cb, ce, tx, tiles);
  }
  return hipGetLastError();
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
  // Without act-order the 32 codes are consecutive in the row: two 16-byte
  // loads instead of 32 byte loads (the check is uniform: c is the block's).
  bool ident = (n % 16) == 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) ident = ident && invperm[c * 32 + i] == c * 32 + i;
  uint8_t cv[32];
  if (ident) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(crow + c * 32);
    const u32x4 b = *reinterpret_cast<const u32x4*>(crow + c * 32 + 16);
    __builtin_memcpy(cv, &a, 16);
    __builtin_memcpy(cv + 16, &b, 16);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) cv[i] = crow[invperm[c * 32 + i]];
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t v = cv[i];
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
  return al256(static_cast<size_t>(rows) * n * 4)           // Wk
         + 4 * al256(static_cast<size_t>(rows) * kSuper * 2) // Eh, El of two super-blocks
         + 2 * al256(static_cast<size_t>(n) * n * 2)         // UTh, UTl
         + al256(static_cast<size_t>(rows) * n)             // codes
         + al256(static_cast<size_t>(rows) * 8)             // rowloss
         + al256(static_cast<size_t>(n) * 4)                // invperm
         + al256(static_cast<size_t>(rows) * 8)             // per-row scale, zero (group_size -1)
         + 256;                                             // loss scalar
}

template <int BITS, int SYM>
static void launch_sweep(dim3 g, hipStream_t s, const float* Wk, const float* U, const uint16_t* UTh,
                         const uint16_t* UTl, int n, int rows, int s1, int nb, uint8_t* codes, uint16_t* Ejh,
                         uint16_t* Ejl, const PendSeg& sa, uint16_t* scales, uint16_t* zeros, double* rowloss,
                         int gs, const float* rowsz) {
  hipLaunchKernelGGL((sweep_block_kernel<BITS, SYM>), g, dim3(256), 0, s, Wk, U, UTh, UTl, n, rows, s1, nb, codes, Ejh,
                     Ejl, kSuper, sa, scales, zeros, rowloss, gs, rowsz);
}

template <int BITS, int SYM>
static void launch_row_params(hipStream_t s, const float* Wk, int n, int rows, float* rowsz) {
  hipLaunchKernelGGL((row_params_kernel<BITS, SYM>), dim3(rows), dim3(256), 0, s, Wk, n, rows, rowsz);
}

// Calls M(bits, sym) with compile-time constants for the runtime bits (2, 3,
// 4, 8) and sym (0, 1, 2).
#define GPTQ_BY_SYM(M, B) \
  do {                    \
    if (sym == 0) M(B, 0); \
    else if (sym == 1) M(B, 1); \
    else M(B, 2);         \
  } while (0)
#define GPTQ_BY_BITS_SYM(M)                 \
  do {                                      \
    if (bits == 2) GPTQ_BY_SYM(M, 2);       \
    else if (bits == 3) GPTQ_BY_SYM(M, 3);  \
    else if (bits == 4) GPTQ_BY_SYM(M, 4);  \
    else GPTQ_BY_SYM(M, 8);                 \
  } while (0)

hipError_t zero_loss(double* loss, hipStream_t s) { return zero_words(loss, 1, s); }

hipError_t launch_quantize(const float* U, const int32_t* perm, const uint8_t* dead, int64_t n64, int bits,
                           int sym, int group_size, const void* W, int wdt, int64_t rows64, int64_t ldw,
                           int32_t* qweight, uint16_t* scales, uint16_t* zeros, int32_t* g_idx, double* loss_host,
                           double* loss_out_dev, void* ws, hipStream_t s) {
  const int n = static_cast<int>(n64), rows = static_cast<int>(rows64);
  uint8_t* p = static_cast<uint8_t*>(ws);
  float* Wk = reinterpret_cast<float*>(p);
  p += al256(static_cast<size_t>(rows) * n * 4);
  uint16_t* Ebuf[4];  // Eh, El of super-block parity 0, then parity 1
  for (int q = 0; q < 4; ++q) {
    Ebuf[q] = reinterpret_cast<uint16_t*>(p);
    p += al256(static_cast<size_t>(rows) * kSuper * 2);
  }
  uint16_t* UTh = reinterpret_cast<uint16_t*>(p);
  p += al256(static_cast<size_t>(n) * n * 2);
  uint16_t* UTl = reinterpret_cast<uint16_t*>(p);
  p += al256(static_cast<size_t>(n) * n * 2);
  uint8_t* codes = p;
  p += al256(static_cast<size_t>(rows) * n);
  double* rowloss = reinterpret_cast<double*>(p);
  p += al256(static_cast<size_t>(rows) * 8);
  int32_t* invperm = reinterpret_cast<int32_t*>(p);
  p += al256(static_cast<size_t>(n) * 4);
  float* rowsz = reinterpret_cast<float*>(p);
  p += al256(static_cast<size_t>(rows) * 8);
  double* loss_dev = reinterpret_cast<double*>(p);
  // group width in the sweep: 32, 64 or 128 columns; 0 = one group per row
  const int gs = (group_size > 0) ? group_size : 0;

  hipError_t e;
#define GPTQ_CHECK_LAUNCH()        \
  do {                             \
    e = hipGetLastError();         \
    if (e != hipSuccess) return e; \
  } while (0)
  e = zero_words(rowloss, static_cast<size_t>(rows), s);
  if (e != hipSuccess) return e;
  dim3 gg(((n + 3) / 4 + 255) / 256, rows < 65535 ? rows : 65535);
  // one vector load per four weights needs W rows, perm and dead aligned to them
  const size_t wsz = (wdt == DT_FP32) ? 4 : 2;
  const bool waligned = (reinterpret_cast<uintptr_t>(W) % (4 * wsz)) == 0 && (ldw % 4) == 0 &&
                        (reinterpret_cast<uintptr_t>(perm) % 16) == 0 && (reinterpret_cast<uintptr_t>(dead) % 4) == 0;
  if (wdt == DT_BF16)
    hipLaunchKernelGGL(gather_w_kernel<DT_BF16>, gg, dim3(256), 0, s, W, ldw, perm, dead, rows, n, Wk, waligned);
  else if (wdt == DT_FP16)
    hipLaunchKernelGGL(gather_w_kernel<DT_FP16>, gg, dim3(256), 0, s, W, ldw, perm, dead, rows, n, Wk, waligned);
  else
    hipLaunchKernelGGL(gather_w_kernel<DT_FP32>, gg, dim3(256), 0, s, W, ldw, perm, dead, rows, n, Wk, waligned);
  GPTQ_CHECK_LAUNCH();
  hipLaunchKernelGGL(gidx_kernel, dim3((n + 255) / 256), dim3(256), 0, s, perm, n, gs > 0 ? gs : n, g_idx, invperm);
  GPTQ_CHECK_LAUNCH();
  if (gs == 0) {
#define GPTQ_ROWP(B, S) launch_row_params<B, S>(s, Wk, n, rows, rowsz)
    GPTQ_BY_BITS_SYM(GPTQ_ROWP);
#undef GPTQ_ROWP
    GPTQ_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(split_ut_kernel, dim3(n / 64, n / 64), dim3(256), 0, s, U, n, UTh, UTl);
  GPTQ_CHECK_LAUNCH();

  // Lazy updates in super-blocks of kSuper columns.  A block's sweep applies
  // to its own rows and columns the errors of the earlier blocks of its
  // super-block (pending_update).  The errors of super-block j reach the next
  // super-block's columns in one update over the whole chip on the caller's
  // stream right after its sweeps (K = kSuper; a sweep work-group would apply
  // the same product to its 64 x 128 block through a latency-bound chunk
  // pipeline, several times slower), and the columns from super-block j+2
  // on in one wide update on a second stream, overlapping the sweeps of
  // super-block j+1.  The caller's stream joins that wide update before the
  // update of super-block j+2's columns from super-block j+1, the next write
  // of those columns there.
  // E holds the errors of two super-blocks (alternating), [rows, kSuper] each.
  const dim3 grid((rows + kRowsSweep - 1) / kRowsSweep);
  const int nsb = (n + kSuper - 1) / kSuper;
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join[2] = {nullptr, nullptr};
  struct Events {
    hipEvent_t* e[3];
    ~Events() {
      for (hipEvent_t* p : e)
        if (*p) (void)hipEventDestroy(*p);
    }
  } events{{&ev_fork, &ev_join[0], &ev_join[1]}};
  if (nsb > 2) {
    e = side_stream(&side);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_join[0], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_join[1], hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  bool joined[2] = {true, true};  // no wide update of that parity in flight
  // The wide update runs on 1.5 work-groups per compute unit (each looping
  // over its XCD's tiles): with one per tile its 768 work-groups (4096 x 4096)
  // took every slot, and the sweep block beside it waited for slots (42-58 us
  // against 24 us).  Measured inside the 4096 x 4096 layer step: quantize
  // 1.13-1.16 -> 1.04-1.07 ms.
  int wide_wgs = 384;
  if (side) {
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    wide_wgs = (3 * cus / 2) & ~7;
    if (wide_wgs < 8) wide_wgs = 8;
  }
  for (int j = 0; j < nsb; ++j) {
    const int s1 = j * kSuper;
    const int s2 = (s1 + kSuper < n) ? s1 + kSuper : n;
    uint16_t* Ejh = Ebuf[2 * (j & 1)];
    uint16_t* Ejl = Ebuf[2 * (j & 1) + 1];
    const uint16_t* Eph = Ebuf[2 * ((j + 1) & 1)];
    const uint16_t* Epl = Ebuf[2 * ((j + 1) & 1) + 1];
    if (!joined[j & 1]) {  // the wide update of super-block j-2 (columns >= s1; reads E[j & 1])
      e = hipStreamWaitEvent(s, ev_join[j & 1], 0);
      if (e != hipSuccess) return e;
      joined[j & 1] = true;
    }
    const PendSeg sa{Eph, Epl, 0, s1 - kSuper};  // the previous super-block: already applied
    {
      const int nbk = (s2 - s1) / kBlk;  // blocks of this super-block, one launch
#define GPTQ_SWEEP(B, S) \
  launch_sweep<B, S>(grid, s, Wk, U, UTh, UTl, n, rows, s1, nbk, codes, Ejh, Ejl, sa, scales, zeros, rowloss, gs, rowsz)
      GPTQ_BY_BITS_SYM(GPTQ_SWEEP);
#undef GPTQ_SWEEP
      GPTQ_CHECK_LAUNCH();
    }
    if (s2 < n) {  // the next super-block's columns, before its sweeps
      // The wide update of super-block j-1 writes these columns too (it
      // covers every column from super-block j+1 on): join it first, or the
      // two read-modify-writes of the same columns race.
      if (!joined[(j + 1) & 1]) {
        e = hipStreamWaitEvent(s, ev_join[(j + 1) & 1], 0);
        if (e != hipSuccess) return e;
        joined[(j + 1) & 1] = true;
      }
      const int ne = (s2 + kSuper < n) ? s2 + kSuper : n;
      // when a wide update follows (it waits for this kernel), the fork event
      // is recorded by this launch
      const bool fork = side && s2 + kSuper < n;
      e = launch_trailing(s, Wk, Ejh, Ejl, kSuper, UTh, UTl, n, rows, s1, s2 - s1, s2, ne, 1 << 30,
                          fork ? ev_fork : nullptr);
      if (e != hipSuccess) return e;
    }
    const int wide = s2 + kSuper;  // first column of super-block j+2
    if (wide < n) {
      hipStream_t st = side ? side : s;
      if (side) {  // ev_fork was recorded by the next super-block's update above
        e = hipStreamWaitEvent(side, ev_fork, 0);
        if (e != hipSuccess) return e;
      }
      e = launch_trailing(st, Wk, Ejh, Ejl, kSuper, UTh, UTl, n, rows, s1, s2 - s1, wide, n, wide_wgs,
                          side ? ev_join[j & 1] : nullptr);
      if (e != hipSuccess) return e;
      if (side) joined[j & 1] = false;
    }
  }
  for (int par = 0; par < 2; ++par) {
    if (!joined[par]) {
      e = hipStreamWaitEvent(s, ev_join[par], 0);
      if (e != hipSuccess) return e;
    }
  }
  dim3 gp((rows + 255) / 256, n / 32);  // n <= 65535 * 32 is checked by the caller
  if (bits == 2) hipLaunchKernelGGL(pack_kernel<2>, gp, dim3(256), 0, s, codes, invperm, n, rows, qweight);
  else if (bits == 3) hipLaunchKernelGGL(pack_kernel<3>, gp, dim3(256), 0, s, codes, invperm, n, rows, qweight);
  else if (bits == 4) hipLaunchKernelGGL(pack_kernel<4>, gp, dim3(256), 0, s, codes, invperm, n, rows, qweight);
  else hipLaunchKernelGGL(pack_kernel<8>, gp, dim3(256), 0, s, codes, invperm, n, rows, qweight);
  GPTQ_CHECK_LAUNCH();
  if (loss_out_dev) {  // stream order, no synchronization
    hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(256), 0, s, rowloss, rows, loss_out_dev);
    GPTQ_CHECK_LAUNCH();
  } else if (loss_host) {
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
