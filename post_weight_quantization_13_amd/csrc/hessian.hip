// Calibration Hessian H = (2/N) X^T X on gfx950.
//
// polydesk.ai "GPTQ" glossary, "Étape 2 : Compensation d'erreur via la
// Hessienne": the Hessian is twice X X^T over the calibration activations
// (kept here as a running mean over tokens).
//
// Design
//   * A workgroup of 8 waves (two per SIMD, so one wave's MFMAs overlap the
//     other's LDS and memory work) computes 128x128 tiles (I, J), I <= J, of
//     the upper triangle over the whole token range.  Each wave computes a
//     64x32 block with bf16/fp16 MFMA (v_mfma_f32_32x32x16, 2x1 MFMA tiles).
//     The launch is balanced over the compute units (see syrk_mfma_kernel).
//   * Precision: the fp32 MFMA accumulators are flushed into an fp64 master
//     copy (in registers) every kFlushSteps stages of 128 tokens, so no fp32
//     accumulation chain is longer than 256 tokens.  The codes GPTQ
//     produces are very sensitive to Hessian error (one flipped code changes
//     the rest of its row), and long fp32 chains measurably lower agreement
//     with an exact Hessian; short chains summed in fp64 do not.  H is stored
//     in fp64 for the same reason.
//   * Operand staging: per stage of 128 tokens every thread loads 8 tokens x 8
//     features (eight 16-byte loads), transposes the 8x8 block of 16-bit
//     values in registers and stores 8 feature rows of 8 consecutive tokens
//     into LDS, so each MFMA operand fragment (8 consecutive tokens of one
//     feature) is a single 16-byte LDS read.  LDS is double buffered and one
//     further stage is in flight into registers ahead of the MFMAs; the
//     per-stage barrier waits for LDS traffic only, so that stage's global
//     loads overlap the current stage's MFMAs.
//   * Epilogue: H <- beta*H + alpha*master; each element is written once and
//     mirrored through LDS so H is exactly symmetric and both writes coalesce.
//   * fp32 inputs use a VALU kernel accumulating in fp64.
#include "common.hpp"

namespace gptq {

constexpr int kTile = 128;       // output tile edge (features)
constexpr int kKStep = 128;      // tokens per LDS stage
constexpr int kFlushSteps = 2;   // stages per fp32 chain: 2 x 128 = 256 tokens (16 MFMAs)
constexpr int kThreads = 512;    // 8 waves

// LDS panel: kTile features x kKStep tokens of 16-bit values = 32 KB; a feature
// row is 256 bytes = sixteen 16-byte chunks of 8 tokens.  Chunk c of feature f
// sits at 16-byte unit f*16 + (c ^ s(f)), s(f) = (f ^ (f >> 4)) & 15: fragment
// reads (16 lanes on 16 consecutive features, one chunk) and the transposed
// stores (16 lanes on features 8l + q, one chunk) each touch 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int panel_offset_bytes(int f, int c) {
  return ((f << 4) | (c ^ ((f ^ (f >> 4)) & 15))) << 4;
}

// Upper-triangle tile enumeration: t -> (ti, tj), ti <= tj, row by row.
__device__ __forceinline__ void upper_tile(int t, int nt, int& ti, int& tj) {
  int i = 0;
  int rem = t;
  while (rem >= nt - i) {
    rem -= nt - i;
    ++i;
  }
  ti = i;
  tj = i + rem;
}

template <int DT>
__device__ __forceinline__ f32x16 mfma_32x32x16(const u32x4& a, const u32x4& b, f32x16 c) {
  if constexpr (DT == DT_BF16) {
    bf16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
  } else {
    f16x8 av, bv;
    __builtin_memcpy(&av, &a, 16);
    __builtin_memcpy(&bv, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
  }
}

// 8x8 transpose of 16-bit values: in[t] holds features 0..7 of token t (two per
// dword, lower feature in the low half); out[f] holds tokens 0..7 of feature f.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int f = 0; f < 8; ++f) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = in[2 * d][f >> 1];      // token 2d
      const uint32_t hi = in[2 * d + 1][f >> 1];  // token 2d+1
      // one v_perm_b32: bytes {lo.0, lo.1, hi.0, hi.1} for even f, {lo.2, lo.3, hi.2, hi.3} for odd f
      out[f][d] = __builtin_amdgcn_perm(hi, lo, (f & 1) ? 0x07060302u : 0x05040100u);
    }
  }
}

// Schedule order of the upper-triangle tiles: super-blocks of sbr tile-rows x
// 8 tile-columns, row-major over the super-blocks that meet the triangle,
// tiles row-major inside each.  The work-groups that one XCD receives in a
// round take consecutive indices, so they need few panels of X between them
// and the XCD's L2 serves most operand loads: 32 work-groups (one per
// compute unit) on a 4 x 8 super-block need about 12 panels instead of 33;
// 64 (two per compute unit) on an 8 x 8 one, 16 instead of 24 on two 4 x 8.
// index -> (ti, tj): whole super-block rows skipped by their tile counts in
// closed form, then super-blocks of that row, then tile rows.
__device__ void sched_tile(int idx, int nt, int sbr, int& ti, int& tj) {
  constexpr int sbc = 8;
  const int nsr = (nt + sbr - 1) / sbr, nsc = (nt + sbc - 1) / sbc;
  int rem = idx;
  ti = 0;
  tj = 0;
  // super-block row: its rows a0 .. a1-1 hold sum (nt - a) tiles
  int SR = 0, a0 = 0, a1 = 0;
  for (; SR < nsr; ++SR) {
    a0 = sbr * SR;
    a1 = (a0 + sbr < nt) ? a0 + sbr : nt;
    const int cnt = (a1 - a0) * nt - (a0 + a1 - 1) * (a1 - a0) / 2;
    if (rem < cnt) break;
    rem -= cnt;
  }
  if (SR >= nsr) return;
  for (int SC = a0 / sbc; SC < nsc; ++SC) {
    const int c_lo = sbc * SC, c_hi = (c_lo + sbc < nt) ? c_lo + sbc : nt;
    int cnt = 0;
    for (int a = a0; a < a1; ++a) {
      const int lo = (a > c_lo) ? a : c_lo;
      cnt += (c_hi > lo) ? c_hi - lo : 0;
    }
    if (rem >= cnt) {
      rem -= cnt;
      continue;
    }
    for (int a = a0; a < a1; ++a) {
      const int lo = (a > c_lo) ? a : c_lo;
      const int c = (c_hi > lo) ? c_hi - lo : 0;
      if (rem < c) {
        ti = a;
        tj = lo + rem;
        return;
      }
      rem -= c;
    }
  }
}

struct TileCtx {
  const uint16_t* X;
  int64_t ldx;
  int n;
  int vec_ok;
  uint8_t* lds;  // 2 buffers x 2 panels x 32 KB
};

// Wave w of the workgroup owns rows 64*(w & 1) .. +63 and columns
// 32*(w >> 1) .. +31 of the 128x128 tile.  MFMA 32x32 output layout:
// accumulator r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ int acc_row(int i, int r, int lane) {
  return i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}

// master (this wave's 64x32 block, fp64) += X[t0:t1, I]^T X[t0:t1, J] for
// tile (ti, tj).  Pipeline: stage s computes from LDS buffer s%2 while stage
// s+1 waits in LDS and stage s+2 is in flight into registers; fp32 chains are
// flushed every 256 tokens.
template <int DT>
__device__ __forceinline__ void tile_accumulate(const TileCtx& cx, int ti, int tj, int64_t t0, int64_t t1,
                                                double (&master)[2][16]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const bool diag = (ti == tj);
  const int n = cx.n;
  const int fo = tid & 15;          // 8-feature chunk this thread loads
  const int to = (tid >> 4) & 15;   // 8-token group this thread loads
  const int ld_p = tid >> 8;        // panel: 0 = rows (I), 1 = columns (J)
  const int ld_feat = (ld_p ? tj : ti) * kTile + 8 * fo;
  const bool ld_on = !(diag && ld_p == 1);
  const bool ld_vec = ld_on && cx.vec_ok && (ld_feat + 8 <= n);
  auto panel = [&](int buf, int p) { return cx.lds + (buf * 2 + p) * (kTile * kKStep * 2); };

  auto global_load = [&](u32x4 (&regs)[8], int64_t ts) {
    const int64_t tb = ts + to * 8;
    if (ld_vec && tb + 8 <= t1) {
      const uint16_t* p = cx.X + tb * cx.ldx + ld_feat;
#pragma unroll
      for (int e = 0; e < 8; ++e) regs[e] = *reinterpret_cast<const u32x4*>(p + e * cx.ldx);
      return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t t = tb + e;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ld_on && t < t1) {
        const uint16_t* p = cx.X + t * cx.ldx + ld_feat;
        if (ld_vec) {
          v = *reinterpret_cast<const u32x4*>(p);
        } else {
          uint16_t tmp[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) tmp[q] = (ld_feat + q < n) ? p[q] : 0;
          __builtin_memcpy(&v, tmp, 16);
        }
      }
      regs[e] = v;
    }
  };
  auto lds_store = [&](const u32x4 (&regs)[8], int buf) {
    if (!ld_on) return;
    u32x4 out[8];
    transpose8x8(regs, out);
    uint8_t* base = panel(buf, ld_p);
#pragma unroll
    for (int f = 0; f < 8; ++f) *reinterpret_cast<u32x4*>(base + panel_offset_bytes(8 * fo + f, to)) = out[f];
  };

  const int wm = wave & 1;
  const int wn = wave >> 1;
  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  const int b_panel = diag ? 0 : 1;
  // The stage's 8 slices of 16 tokens; the next slice's fragments are read
  // from LDS while the current slice's two MFMAs run.
  auto compute = [&](int buf) {
    const uint8_t* pa = panel(buf, 0);
    const uint8_t* pb = panel(buf, b_panel);
    u32x4 fa[2][2], fb[2];
    auto frag = [&](int kk, int slot) {
      const int c = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[slot][i] = *reinterpret_cast<const u32x4*>(pa + panel_offset_bytes(wm * 64 + i * 32 + (lane & 31), c));
      fb[slot] = *reinterpret_cast<const u32x4*>(pb + panel_offset_bytes(wn * 32 + (lane & 31), c));
    };
    frag(0, 0);
#pragma unroll
    for (int kk = 0; kk < kKStep / 16; ++kk) {
      if (kk + 1 < kKStep / 16) frag(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i] = mfma_32x32x16<DT>(fa[kk & 1][i], fb[kk & 1], acc[i]);
    }
  };
  int step = 0;
  auto flush = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        master[i][r] += static_cast<double>(acc[i][r]);
        acc[i][r] = 0.0f;
      }
  };

  const int64_t nstages = (t1 - t0 + kKStep - 1) / kKStep;
  if (nstages <= 0) return;
  u32x4 ra[8];
  global_load(ra, t0);
  lds_store(ra, 0);
  global_load(ra, t0 + kKStep);
  __syncthreads();
  int buf = 0;
  for (int64_t s = 0; s < nstages; ++s) {
    compute(buf);
    if (++step == kFlushSteps) {
      flush();
      step = 0;
    }
    if (s + 1 >= nstages) break;
    lds_store(ra, buf ^ 1);
    global_load(ra, t0 + (s + 2) * kKStep);
    // LDS-only barrier: the loads of stage s + 2 stay in flight across it and
    // land while stage s + 1 computes (a full barrier would wait for them).
    lds_barrier();
    buf ^= 1;
  }
  flush();
  __syncthreads();  // staging buffers free for the next user
}

// H <- beta*H + alpha*master for tile (ti, tj): each element written once, the
// mirror staged through LDS (the whole 128x128 fp64 tile, transposed, 128 KB)
// so both writes coalesce.
__device__ __forceinline__ void tile_epilogue(const double (&master)[2][16], int ti, int tj, int n, double alpha,
                                              double beta, double* __restrict__ H, uint8_t* lds) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const bool diag = (ti == tj);
  const int rw = (wave & 1) * 64, cw = (wave >> 1) * 32;
  double* stage = reinterpret_cast<double*>(lds);  // [column][row ^ column], 128 KB
  const int lc = cw + (lane & 31);
  const int gj = tj * kTile + lc;
  double old[2][16];  // previous H, all loads issued before any store
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gi = ti * kTile + rw + acc_row(i, r, lane);
      const bool own = gi < n && gj < n && !(diag && gi > gj);
      old[i][r] = (beta != 0.0 && own) ? H[static_cast<int64_t>(gi) * n + gj] : 0.0;
    }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = rw + acc_row(i, r, lane);
      const int gi = ti * kTile + lr;
      double v = alpha * master[i][r];
      const bool own = gi < n && gj < n && !(diag && gi > gj);
      if (own) {
        if (beta != 0.0) v += beta * old[i][r];
        H[static_cast<int64_t>(gi) * n + gj] = v;
      }
      stage[lc * kTile + (lr ^ lc)] = v;
    }
  __syncthreads();
  for (int e = tid; e < kTile * kTile; e += kThreads) {
    const int c = e >> 7, r = e & 127;
    const int gi = ti * kTile + r, gjj = tj * kTile + c;
    if (gi < n && gjj < n && gi < gjj) H[static_cast<int64_t>(gjj) * n + gi] = stage[c * kTile + (r ^ c)];
  }
}

// Raw fp64 partial tile (row-major 128x128) for a token piece of a leftover tile.
__device__ __forceinline__ void tile_store_partial(const double (&master)[2][16], double* __restrict__ dst) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int rw = (wave & 1) * 64, cw = (wave >> 1) * 32;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[(rw + acc_row(i, r, lane)) * kTile + cw + (lane & 31)] = master[i][r];
}

// Balanced launch over T = nt(nt+1)/2 tiles with P = min(T, #CUs): a first
// launch of R*P workgroups (R = T / P) runs whole tiles, one per workgroup, in
// R rounds; the workgroups of round r take schedule indices r*P + slot, the
// slot chosen so that the 32 workgroups one XCD receives share a compact
// group of tiles.  The L = T % P leftover tiles are cut into S = P / L token
// pieces, one per workgroup of a second launch, whose fp64 partials
// syrk_reduce_kernel sums in a fixed order (S == 1: the pieces are whole tiles).
struct HessSched {
  int nt, T, P, R, L, S;
  int sbr;        // super-block rows of the schedule order
  int64_t chunk;  // tokens per piece
};

template <int DT>
__global__ void __launch_bounds__(kThreads) syrk_mfma_kernel(const uint16_t* __restrict__ X, int64_t ldx, int n,
                                                             int64_t tokens, HessSched sc, int pieces, int vec_ok,
                                                             double alpha, double beta, double* __restrict__ H,
                                                             double* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 2 * kTile * kKStep * 2];  // 128 KB
  const TileCtx cx{X, ldx, n, vec_ok, lds};
  const int b = blockIdx.x;
  int idx;
  int64_t p0 = 0, p1 = tokens;
  bool partial_out = false;
  if (!pieces) {
    const int r = b / sc.P, s = b % sc.P;
    idx = r * sc.P + ((sc.P % 8 == 0) ? (s % 8) * (sc.P / 8) + s / 8 : s);
  } else {
    idx = sc.R * sc.P + b / sc.S;
    if (sc.S > 1) {
      partial_out = true;
      p0 = (b % sc.S) * sc.chunk;
      p1 = (p0 + sc.chunk < tokens) ? p0 + sc.chunk : tokens;
    }
  }
  int ti, tj;
  sched_tile(idx, sc.nt, sc.sbr, ti, tj);
  double master[2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) master[i][e] = 0.0;
  tile_accumulate<DT>(cx, ti, tj, p0, p1, master);
  if (partial_out) tile_store_partial(master, partial + static_cast<int64_t>(b) * kTile * kTile);
  else tile_epilogue(master, ti, tj, n, alpha, beta, H, lds);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS path (16-byte aligned rows, n a multiple of 8).
//
// Four waves per work-group, each a 64x64 block of the 128x128 tile (2x2 MFMA
// 32x32x16 tiles), so one LDS fragment feeds two MFMAs instead of 1.5, and
// two work-groups share a compute unit (64 KB of LDS each, at most 256
// registers per wave): their barriers are independent, so one work-group's
// MFMAs run while the other waits.
//   * Staging: buffer loads write X straight into LDS in its natural
//     [token][feature] order, 32 tokens per stage, four stages resident (one
//     computed, three in flight).  No staging registers and no transposes: a
//     lane's MFMA operand (8 consecutive tokens of one feature) comes from
//     two ds_read_b64_tr_b16, each handing a 16-lane group 4 tokens x 16
//     features.  The buffer's range check returns zeros past the last token
//     and for features >= n, so ragged tails need no branches.
//   * LDS panel: 32 token rows of 256 bytes (16 chunks of 8 features); chunk
//     c of row r sits at 16-byte slot c ^ 4 (r & 3), so the 32 lanes of a
//     transposing read (4 rows x 64 bytes) touch 64 distinct banks and a
//     load instruction still writes 1 KB contiguously.
//   * Precision as above: fp32 chains of 256 tokens (8 stages) summed into an
//     fp64 master in registers.
constexpr int kDKS = 32;                       // tokens per stage
constexpr int kDBufs = 4;                      // resident stages
constexpr int kDThreads = 256;                 // 4 waves
constexpr int kDPanel = kDKS * kTile * 2;      // 8 KB
constexpr int kDStage = 2 * kDPanel;           // both panels
constexpr int kDLds = kDBufs * kDStage;        // 64 KB
constexpr int kDChain = 256 / kDKS;            // stages per fp32 chain
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;  // a byte offset past any range
static_assert(kDChain * kDKS == kFlushSteps * kKStep, "both paths keep 256-token fp32 chains");
static_assert(kDKS % 16 == 0 && kDBufs >= 2 && kDLds <= 80 * 1024, "whole k-steps; two work-groups per compute unit");
static_assert(kDLds >= 64 * kTile * 8, "the epilogue stages 64 columns of the fp64 tile in LDS");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// One 16-byte-per-lane buffer load into LDS: lane L's 16 bytes land at
// lds_addr + 16 L.  Written out rather than through the compiler's builtin,
// whose wait-count tracking would make every later LDS read wait for all
// loads in flight, including those of stages not yet needed; the waits on
// these loads are explicit (vm_wait_barrier).  M0 is saved and restored
// around the load, and one wait state separates its write from the load.
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory");
}

// Loads per wave and stage: DIAG tiles stage one panel, others two; each
// load fills 4 token rows.
template <bool DIAG>
constexpr int dma_loads_per_wave() { return DIAG ? kDKS / 16 : kDKS / 8; }

// Per-tile constants of this lane's stage loads.  Wave w fills rows of panel
// p as whole 1 KB blocks of 4 rows; lane L of a block fills slot L % 16 of row
// L / 16, which holds chunk (L % 16) ^ 4 (L / 16) of that row.  off[q] is the
// byte offset of that chunk from the stage's first token (out of range for
// features >= n); lds is the wave's first row in a stage buffer.
template <bool DIAG>
struct DmaLane {
  uint32_t off[dma_loads_per_wave<DIAG>()];
  uint32_t lds;
};

template <bool DIAG>
__device__ __forceinline__ DmaLane<DIAG> dma_lane(int64_t ldx, int n, int fI, int fJ) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int c = (lane & 15) ^ ((lane >> 4) << 2);
  const int p = DIAG ? 0 : (wave >> 1);
  const int f = (p ? fJ : fI) + 8 * c;
  const int rw = DIAG ? (kDKS / 4) * wave : (kDKS / 2) * (wave & 1);
  DmaLane<DIAG> d;
#pragma unroll
  for (int q = 0; q < dma_loads_per_wave<DIAG>(); ++q) {
    const int r = rw + 4 * q + (lane >> 4);
    d.off[q] = (f < n) ? static_cast<uint32_t>((r * ldx + f) * 2) : kOutOfRange;
  }
  d.lds = static_cast<uint32_t>(p * kDPanel + rw * 256);
  return d;
}

// Issue one stage's loads into the stage buffer at LDS address stage_lds.  The
// buffer's range ends at token t1 (nothing at all past the end), so later rows
// read as zeros.
template <bool DIAG>
__device__ __forceinline__ void dma_stage(const uint16_t* X, int64_t ldx, int64_t tstage, int64_t t1,
                                          const DmaLane<DIAG>& d, uint32_t stage_lds) {
  int64_t rows = t1 - tstage;
  rows = rows < 0 ? 0 : (rows > kDKS ? kDKS : rows);
  const uint64_t base = reinterpret_cast<uint64_t>(X + (rows > 0 ? tstage * ldx : 0));
  u32x4 rs;
  rs[0] = static_cast<uint32_t>(base);
  rs[1] = static_cast<uint32_t>(base >> 32);  // stride 0
  rs[2] = static_cast<uint32_t>(rows * ldx * 2);
  rs[3] = kRsrcWord3;
#pragma unroll
  for (int q = 0; q < dma_loads_per_wave<DIAG>(); ++q) lds_dma16(rs, stage_lds + d.lds + q * 1024, d.off[q]);
}

// This lane's MFMA operand for features fb .. fb+31 and tokens 16 kk ..
// 16 kk + 15 of a staged panel: two transposing reads of 4 tokens each.
__device__ __forceinline__ u32x4 dma_frag(const uint8_t* panel, int fb, int kk, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int rl = 8 * (g >> 1) + (j >> 2);                    // row within the k-step (h = 0)
  const int slot = ((fb >> 3) ^ ((j >> 2) << 2)) + 2 * (g & 1) + ((j & 3) >> 1);
  const uint8_t* p = panel + (16 * kk + rl) * 256 + 16 * slot + 8 * (j & 1);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p + 4 * 256));
  u32x4 v;
  __builtin_memcpy(&v, &lo, 8);
  __builtin_memcpy(reinterpret_cast<uint8_t*>(&v) + 8, &hi, 8);
  return v;
}

template <int N>
__device__ __forceinline__ void vm_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// master (this wave's 64x64 block, fp64) += X[t0:t1, I]^T X[t0:t1, J].
template <int DT, bool DIAG>
__device__ __forceinline__ void tile_accumulate_dma(const uint16_t* X, int64_t ldx, int n, int ti, int tj,
                                                    int64_t t0, int64_t t1, uint8_t* lds, double (&master)[2][2][16]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int fI = ti * kTile, fJ = tj * kTile;
  // the strictly lower block of a diagonal tile is never stored
  const bool idle = DIAG && wm == 1 && wn == 0;
  constexpr int NL = dma_loads_per_wave<DIAG>();
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto flush = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          master[i][j][r] += static_cast<double>(acc[i][j][r]);
          acc[i][j][r] = 0.0f;
        }
  };
  const int64_t nst = (t1 - t0 + kDKS - 1) / kDKS;
  if (nst <= 0) return;
  // three stages in flight before the first is computed; stages past the end
  // load zeros without touching memory, which keeps the wait counts fixed
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds));
  const DmaLane<DIAG> dl = dma_lane<DIAG>(ldx, n, fI, fJ);
#pragma unroll
  for (int s = 0; s < kDBufs - 1; ++s) dma_stage<DIAG>(X, ldx, t0 + s * kDKS, t1, dl, lds_addr + s * kDStage);
  int chain = 0;
  for (int64_t s = 0; s < nst; ++s) {
    // this wave's loads of stage s have landed (those of the later stages in
    // flight may not); after the barrier every wave's have, and every wave is
    // done with stage s-1, whose buffer the next loads reuse
    vm_wait_barrier<(kDBufs - 2) * NL>();
    const int64_t sn = s + kDBufs - 1;
    dma_stage<DIAG>(X, ldx, t0 + sn * kDKS, t1, dl, lds_addr + static_cast<uint32_t>(sn % kDBufs) * kDStage);
    const uint8_t* pa = lds + (s % kDBufs) * kDStage;
    const uint8_t* pb = DIAG ? pa : pa + kDPanel;
    if (!idle) {
#pragma unroll
      for (int kk = 0; kk < kDKS / 16; ++kk) {
        u32x4 fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = dma_frag(pa, wm * 64 + 32 * i, kk, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = dma_frag(pb, wn * 64 + 32 * j, kk, lane);
        // raised wave priority while MFMAs issue: the other work-group's wave
        // on this SIMD, busy with loads and LDS reads, yields to them
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            __builtin_amdgcn_s_setprio(1);
            acc[i][j] = mfma_32x32x16<DT>(fa[i], fb[j], acc[i][j]);
          }
        __builtin_amdgcn_s_setprio(0);
      }
    }
    if (++chain == kDChain) {
      flush();
      chain = 0;
    }
  }
  flush();
  vm_wait_barrier<0>();  // the trailing zero loads have landed; LDS free for the epilogue
}

// Element (i, j, r) of a wave's 64x64 block -> row / column inside the tile.
__device__ __forceinline__ int dma_row(int wm, int i, int r, int lane) { return wm * 64 + acc_row(i, r, lane); }
__device__ __forceinline__ int dma_col(int wn, int j, int lane) { return wn * 64 + j * 32 + (lane & 31); }

// H <- beta*H + alpha*master, each element written once; the mirror goes
// through LDS in two halves of 64 columns (64 KB each), so both writes
// coalesce.
__device__ __forceinline__ void tile_epilogue_dma(const double (&master)[2][2][16], int ti, int tj, int n,
                                                  double alpha, double beta, double* __restrict__ H, uint8_t* lds) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const bool diag = (ti == tj);
  double* stage = reinterpret_cast<double*>(lds);  // [64 columns][128 rows], rows XOR-swizzled
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wn == half) {
      // one 32x32 MFMA block at a time, so the previous values of H take
      // 32 registers beside the master copy instead of 128
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          double old[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int gi = ti * kTile + dma_row(wm, i, r, lane), gj = tj * kTile + dma_col(wn, j, lane);
            const bool own = gi < n && gj < n && !(diag && gi > gj);
            old[r] = (beta != 0.0 && own) ? H[static_cast<int64_t>(gi) * n + gj] : 0.0;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = dma_row(wm, i, r, lane), lc = j * 32 + (lane & 31);
            const int gi = ti * kTile + lr, gj = tj * kTile + half * 64 + lc;
            double v = alpha * master[i][j][r];
            const bool own = gi < n && gj < n && !(diag && gi > gj);
            if (own) {
              if (beta != 0.0) v += beta * old[r];
              H[static_cast<int64_t>(gi) * n + gj] = v;
            }
            stage[lc * kTile + (lr ^ lc)] = v;
          }
        }
    }
    __syncthreads();
    for (int e = tid; e < 64 * kTile; e += kDThreads) {
      const int c = e >> 7, r = e & 127;
      const int gi = ti * kTile + r, gjj = tj * kTile + half * 64 + c;
      if (gi < n && gjj < n && gi < gjj) H[static_cast<int64_t>(gjj) * n + gi] = stage[c * kTile + (r ^ c)];
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void tile_store_partial_dma(const double (&master)[2][2][16], double* __restrict__ dst) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[dma_row(wm, i, r, lane) * kTile + dma_col(wn, j, lane)] = master[i][j][r];
}

template <int DT>
__global__ void __launch_bounds__(kDThreads) __attribute__((amdgpu_waves_per_eu(2)))
syrk_dma_kernel(const uint16_t* __restrict__ X, int64_t ldx, int n, int64_t tokens, HessSched sc, int pieces,
                double alpha, double beta, double* __restrict__ H, double* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDLds];
  const int b = blockIdx.x;
  int idx;
  int64_t p0 = 0, p1 = tokens;
  bool partial_out = false;
  if (!pieces) {
    const int r = b / sc.P, s = b % sc.P;
    idx = r * sc.P + ((sc.P % 8 == 0) ? (s % 8) * (sc.P / 8) + s / 8 : s);
  } else {
    idx = sc.R * sc.P + b / sc.S;
    if (sc.S > 1) {
      partial_out = true;
      p0 = (b % sc.S) * sc.chunk;
      p1 = (p0 + sc.chunk < tokens) ? p0 + sc.chunk : tokens;
    }
  }
  int ti, tj;
  sched_tile(idx, sc.nt, sc.sbr, ti, tj);
  double master[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) master[i][j][e] = 0.0;
  if (ti == tj) tile_accumulate_dma<DT, true>(X, ldx, n, ti, tj, p0, p1, lds, master);
  else tile_accumulate_dma<DT, false>(X, ldx, n, ti, tj, p0, p1, lds, master);
  if (partial_out) tile_store_partial_dma(master, partial + static_cast<int64_t>(b) * kTile * kTile);
  else tile_epilogue_dma(master, ti, tj, n, alpha, beta, H, lds);
}

// Leftover tiles split into S pieces: sum the pieces in piece order (fp64),
// apply H <- beta*H + alpha*sum, write tile and mirror.  grid = (L, 64): one
// 16x16 block of a tile per work-group, one element per thread, so the S
// loads of every element are in flight together across the whole chip.
__global__ void __launch_bounds__(256) syrk_reduce_kernel(const double* __restrict__ partial, HessSched sc, int n,
                                                          double alpha, double beta, double* __restrict__ H) {
  __shared__ double stage[16 * 17];  // [column][row], padded
  const int q = blockIdx.x;
  const int w = blockIdx.y;
  int ti, tj;
  sched_tile(sc.R * sc.P + q, sc.nt, sc.sbr, ti, tj);
  const bool diag = (ti == tj);
  const int rb = (w >> 3) * 16, cb = (w & 7) * 16;
  const int tid = threadIdx.x;
  const int lr = tid >> 4, lc = tid & 15;
  const int gi = ti * kTile + rb + lr, gj = tj * kTile + cb + lc;
  const double* src = partial + static_cast<int64_t>(q) * sc.S * kTile * kTile + (rb + lr) * kTile + cb + lc;
  double s = 0.0;
  for (int p = 0; p < sc.S; ++p) s += src[static_cast<int64_t>(p) * kTile * kTile];
  double v = alpha * s;
  if (gi < n && gj < n && !(diag && gi > gj)) {
    if (beta != 0.0) v += beta * H[static_cast<int64_t>(gi) * n + gj];
    H[static_cast<int64_t>(gi) * n + gj] = v;
  }
  stage[lc * 17 + lr] = v;
  __syncthreads();
  // mirror: thread (c, r) = (tid / 16, tid % 16) writes H[col][row], rows consecutive
  const int c = tid >> 4, r = tid & 15;
  const int mi = ti * kTile + rb + r, mj = tj * kTile + cb + c;
  if (mi < n && mj < n && mi < mj) H[static_cast<int64_t>(mj) * n + mi] = stage[c * 17 + r];
}

// fp32 inputs: 64x64 tiles of the upper triangle, fp64 accumulation on the VALU.
__global__ void __launch_bounds__(256) syrk_f32_kernel(
    const float* __restrict__ X, int64_t ldx, int n, int64_t tokens, int nt64,
    double alpha, double beta, double* __restrict__ H) {
  __shared__ float sa[32][65];
  __shared__ float sb[32][65];
  int ti, tj;
  upper_tile(blockIdx.x, nt64, ti, tj);
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;  // 16x16 threads, 4x4 outputs each
  double acc[4][4] = {};
  for (int64_t t0 = 0; t0 < tokens; t0 += 32) {
    for (int e = tid; e < 32 * 64; e += 256) {
      const int k = e / 64, f = e % 64;
      const int64_t t = t0 + k;
      const int fa = ti * 64 + f, fb = tj * 64 + f;
      sa[k][f] = (t < tokens && fa < n) ? X[t * ldx + fa] : 0.0f;
      sb[k][f] = (t < tokens && fb < n) ? X[t * ldx + fb] : 0.0f;
    }
    __syncthreads();
    for (int k = 0; k < 32; ++k) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sa[k][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sb[k][tc * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const bool diag = (ti == tj);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gi = ti * 64 + tr * 4 + i, gj = tj * 64 + tc * 4 + j;
      if (gi >= n || gj >= n || (diag && gi > gj)) continue;
      double v = alpha * acc[i][j];
      if (beta != 0.0) v += beta * H[static_cast<int64_t>(gi) * n + gj];
      H[static_cast<int64_t>(gi) * n + gj] = v;
      if (gi != gj) H[static_cast<int64_t>(gj) * n + gi] = v;
    }
}

// ----------------------------------------------------------------------------
// Host-side launcher (called from api.hip).
// ----------------------------------------------------------------------------
static inline int64_t upper_tiles(int64_t nt) { return nt * (nt + 1) / 2; }

int64_t hessian_chain_tokens() { return static_cast<int64_t>(kFlushSteps) * kKStep; }

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

// per_cu: work-groups resident on one compute unit (1 for syrk_mfma_kernel,
// 2 for syrk_dma_kernel).
static HessSched make_sched(int64_t n, int64_t tokens, int per_cu) {
  HessSched sc{};
  sc.nt = static_cast<int>((n + kTile - 1) / kTile);
  sc.T = static_cast<int>(upper_tiles(sc.nt));
  const int slots = device_cus() * per_cu;
  sc.P = sc.T < slots ? sc.T : slots;
  sc.sbr = 4 * per_cu;
  sc.R = sc.T / sc.P;
  sc.L = sc.T % sc.P;
  sc.S = sc.L > 0 ? sc.P / sc.L : 0;
  if (sc.S > 1) {
    const int64_t per = (tokens + sc.S - 1) / sc.S;
    const int64_t chain = hessian_chain_tokens();
    sc.chunk = (per + chain - 1) / chain * chain;
  } else {
    sc.chunk = tokens;
  }
  return sc;
}

static size_t sched_workspace(const HessSched& sc) {
  return sc.S <= 1 ? 0 : static_cast<size_t>(sc.L) * sc.S * kTile * kTile * sizeof(double);
}

// Enough for either path: which one runs depends on X's alignment.
size_t hessian_workspace(int64_t n, int64_t tokens, int dt) {
  if (dt == DT_FP32 || n <= 0 || tokens <= 0) return 0;
  const size_t a = sched_workspace(make_sched(n, tokens, 1)), b = sched_workspace(make_sched(n, tokens, 2));
  return a > b ? a : b;
}

hipError_t launch_hessian(double* H, int64_t n, const void* X, int dt, int64_t tokens, int64_t ldx, double alpha,
                          double beta, void* ws, hipStream_t s) {
  if (dt == DT_FP32) {
    const int nt64 = static_cast<int>((n + 63) / 64);
    hipLaunchKernelGGL(syrk_f32_kernel, dim3(static_cast<unsigned>(upper_tiles(nt64))), dim3(256), 0, s,
                       static_cast<const float*>(X), ldx, static_cast<int>(n), tokens, nt64, alpha, beta, H);
    return hipGetLastError();
  }
  const int vec_ok = (ldx % 8 == 0) && (reinterpret_cast<uintptr_t>(X) % 16 == 0);
  double* partial = static_cast<double*>(ws);
  const uint16_t* Xp = static_cast<const uint16_t*>(X);
  // the direct-to-LDS path: whole 8-feature chunks, 32-bit byte offsets
  // within a stage
  if (vec_ok && n % 8 == 0 && ldx <= (int64_t{1} << 24)) {
    // Token chunks of about 256 MB of X each (16384 to 65536 tokens), one
    // pass over all tiles per chunk, the first applying beta and the rest
    // adding on: a work-group then walks at most one chunk of tokens, so the
    // work-groups sharing an XCD stay close enough in token position to find
    // each other's operand panels in its L2.  Over long token ranges they
    // drift apart, and the operand traffic (measured: twice the fetched bytes
    // at 11008 features x 65536 tokens) outweighs the chunk's extra read and
    // write of H.
    int64_t chunk = ((int64_t{1} << 28) / n) / 256 * 256;
    chunk = chunk < 16384 ? 16384 : (chunk > 65536 ? 65536 : chunk);
    auto kd = (dt == DT_BF16) ? syrk_dma_kernel<DT_BF16> : syrk_dma_kernel<DT_FP16>;
    for (int64_t c0 = 0; c0 < tokens; c0 += chunk) {
      const int64_t tc = (tokens - c0 < chunk) ? tokens - c0 : chunk;
      const double bc = (c0 == 0) ? beta : 1.0;
      const uint16_t* Xc = Xp + c0 * ldx;
      const HessSched sc = make_sched(n, tc, 2);
      hipLaunchKernelGGL(kd, dim3(sc.R * sc.P), dim3(kDThreads), 0, s, Xc, ldx, static_cast<int>(n), tc, sc, 0, alpha,
                         bc, H, partial);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (sc.L == 0) continue;
      hipLaunchKernelGGL(kd, dim3(sc.L * sc.S), dim3(kDThreads), 0, s, Xc, ldx, static_cast<int>(n), tc, sc, 1, alpha,
                         bc, H, partial);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (sc.S <= 1) continue;
      hipLaunchKernelGGL(syrk_reduce_kernel, dim3(sc.L, 64), dim3(256), 0, s, partial, sc, static_cast<int>(n), alpha,
                         bc, H);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const HessSched sc = make_sched(n, tokens, 1);
  auto kern = (dt == DT_BF16) ? syrk_mfma_kernel<DT_BF16> : syrk_mfma_kernel<DT_FP16>;
  hipLaunchKernelGGL(kern, dim3(sc.R * sc.P), dim3(kThreads), 0, s, Xp, ldx, static_cast<int>(n), tokens, sc, 0, vec_ok,
                     alpha, beta, H, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sc.L == 0) return e;
  hipLaunchKernelGGL(kern, dim3(sc.L * sc.S), dim3(kThreads), 0, s, Xp, ldx, static_cast<int>(n), tokens, sc, 1, vec_ok,
                     alpha, beta, H, partial);
  e = hipGetLastError();
  if (e != hipSuccess || sc.S <= 1) return e;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3(sc.L, 64), dim3(256), 0, s, partial, sc, static_cast<int>(n), alpha,
                     beta, H);
  return hipGetLastError();
}

}  // namespace gptq
