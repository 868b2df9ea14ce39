// Dequantizing matmul for inference with the packed layer: Y = A W_hat^T with
// fp16 activations A [M, n] and W_hat[o, i] = s[g(i), o] * (code[o, i] - z[g(i), o]).
//
// ayinedjimi-consultants "Quantization : GPTQ, GGUF, AWQ", "Calibration et
// dataset" and "Kernels d'inférence": a GPTQ layer is served by a kernel that
// unpacks and dequantizes the low-bit weights on the fly and multiplies them
// with fp16 activations; such kernels are judged by the fraction of memory
// bandwidth they reach.  This is a gfx950 design of that role, not of the
// NVIDIA kernels the page names.
//
// Two calls:
//   pack (once per layer): orders the columns group by group (identity unless
//     act-order scattered the groups), retiles the codes so that one lane's
//     16-byte load is exactly its B operand of four 16x16x32 f16 MFMAs, and
//     interleaves scale and zero per 16-output tile.
//   matmul (per token batch): one workgroup of 8 waves per 16 outputs; wave w
//     takes 128-column chunks w, w+8, ...; its chunk loads run 4 chunks ahead
//     in registers.  The activations of each 1024-column window are staged in
//     LDS (double buffered).  Codes are turned into the exact integers c - z
//     in fp16 with the 0x6400 exponent trick (0x6400 | c is 1024 + c), so the
//     MFMA products are exact and only fp32 accumulation rounds; each group's
//     partial sum is scaled by its fp32 scale when the group ends.
//
// Packed layout (bytes):
//   [0, 256)           header: flags word written by pack (bit 0: g_idx is not a
//                      grouping into groups of group_size; bit 1: order not identity)
//   Q   at 256         [T][C][64 lanes][bits words]: T = ceil(rows/16) output
//                      tiles, C = n/128 chunks.  Lane l = 16q + j holds, for
//                      the four 32-column steps t of the chunk, the eight codes
//                      of output 16T + j at grouped columns 128c + 32t + 8q + s,
//                      s = 0..7, as an 8*bits-bit field per step (step t at bit
//                      8*bits*t of the lane's stream); inside a field the code
//                      of slot s sits at field position field_pos(bits, s), so the
//                      unpacking below yields the slots in order.
//   SZ  after Q        [T][Cs][16][spc] u32: low half the fp16 scale, high half
//                      the fp16 zero (0 for padding outputs).  spc = 128/gs
//                      words per chunk (groups c*spc .. c*spc+spc-1) and
//                      Cs = C; for one group per row Cs = spc = 1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace gptq {
namespace {

constexpr int kWinWaves = 8;         // waves per workgroup of the windowed variant
constexpr int kChunk = 128;          // columns per chunk (four 32-column MFMA steps)
constexpr int kWin = kWinWaves * kChunk;  // columns per LDS window (one chunk per wave)
constexpr int kWinStride = kWin + 8;     // halves per staged row (16-byte pad against bank conflicts)
constexpr int kMTile = 16;           // tokens per MFMA tile
constexpr int kAhead = 4;            // chunks of codes each wave keeps in flight (even)
constexpr size_t kFullLds = 80 * 1024;  // largest slice of activations staged whole
constexpr int kFullPieces = 8;          // ... in at most this many 16-byte pieces per thread
constexpr size_t kWinLds = 160 * 1024;  // windowed variant: two windows of 16 tokens and the scale/zero words
constexpr size_t kHeader = 256;
// s_waitcnt immediate for vmcnt(0) with the other counters left alone (gfx9
// layout: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kVmcntZero = 0x0F70;
constexpr int kWaveSlots = 256 * 32;   // waves the chip holds at once (256 CUs x 32)

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Position of slot s inside a step's field, per code width: the unpacking
// makes half-pairs of fields (0,4), (1,5), (2,6), (3,7) (2-, 3-, 4-bit) or
// (0,2), (1,3), (4,6), (5,7) (8-bit), and the MFMA operand wants slots
// (0,1), (2,3), (4,5), (6,7) in that order.
__host__ __device__ constexpr int field_pos(int bits, int s) {
  return bits == 8 ? ((s >> 2) << 2) + ((s & 1) << 1) + ((s >> 1) & 1)
                   : ((s & 1) << 2) + (s >> 1);
}

// ------------------------------------------------------------------ pack side
// Column order: workgroup g lists the columns with g_idx == g in ascending
// order into col_order[g*gs ...].  Flags bit 0 when a group does not hold
// exactly gs columns (which also catches g_idx values outside [0, G)), bit 1
// when some column moves.
__global__ __launch_bounds__(256) void group_order_kernel(const int32_t* __restrict__ g_idx, int n, int gs,
                                                         int32_t* __restrict__ col_order,
                                                         uint32_t* __restrict__ flags) {
  __shared__ int wave_cnt[4];
  const int g = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = g * gs;
  int count = 0;
  uint32_t moved = 0, bad = 0;
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + tid;
    const bool mine = i < n && g_idx[i] == g;
    const uint64_t mask = __ballot(mine);
    const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
    if (lane == 0) wave_cnt[wave] = __popcll(mask);
    __syncthreads();
    int before = 0, total = 0;
    for (int v = 0; v < 4; ++v) {
      before += v < wave ? wave_cnt[v] : 0;
      total += wave_cnt[v];
    }
    if (mine) {
      const int pos = count + before + rank;
      if (pos < gs) {
        col_order[base + pos] = i;
        moved |= (base + pos != i) ? 2u : 0u;
      } else {
        bad = 1u;
      }
    }
    count += total;
    __syncthreads();
  }
  if (tid == 0 && count != gs) bad = 1u;
  const uint32_t f = bad | moved;
  if (f) atomicOr(flags, f);
}

// Codes: thread per (tile, chunk, lane) writes the lane's bits words.
template <int BITS>
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint32_t* __restrict__ qweight,
                                                        const int32_t* __restrict__ col_order, int rows, int n,
                                                        int T, uint32_t* __restrict__ Q) {
  const int C = n / kChunk;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= static_cast<int64_t>(T) * C * 64) return;
  const int lane = static_cast<int>(id & 63);
  const int64_t tc = id >> 6;
  const int c = static_cast<int>(tc % C);
  const int tile = static_cast<int>(tc / C);
  const int q = lane >> 4, j = lane & 15;
  const int o = tile * 16 + j;
  uint32_t out[BITS];
  for (int v = 0; v < BITS; ++v) out[v] = 0;
  if (o < rows) {
    for (int t = 0; t < 4; ++t) {
      for (int s = 0; s < 8; ++s) {
        const int kp = c * kChunk + 32 * t + 8 * q + s;
        // col_order holds a permutation by the time this runs (the host
        // checks it first); the clamp keeps any other value inside qweight
        const int col = col_order ? min(max(col_order[kp], 0), n - 1) : kp;
        const int64_t bit = static_cast<int64_t>(BITS) * col;
        const int64_t wi = bit >> 5;
        const int off = static_cast<int>(bit & 31);
        uint64_t v = qweight[wi * rows + o];
        if (off + BITS > 32) v |= static_cast<uint64_t>(qweight[(wi + 1) * rows + o]) << 32;
        const uint32_t code = static_cast<uint32_t>(v >> off) & ((1u << BITS) - 1u);
        const int dst = 8 * BITS * t + BITS * field_pos(BITS, s);
        out[dst >> 5] |= code << (dst & 31);
        if ((dst & 31) + BITS > 32) out[(dst >> 5) + 1] |= code >> (32 - (dst & 31));
      }
    }
  }
  uint32_t* dst = Q + id * BITS;
  for (int v = 0; v < BITS; ++v) dst[v] = out[v];
}

// Scale/zero words in [T][Cs][16][spc] order: spc = 128/gs words (one per
// group a 128-column chunk touches) for each chunk, or a single word per
// output (Cs = spc = 1) for one group per row.
__global__ __launch_bounds__(256) void pack_sz_kernel(const uint16_t* __restrict__ scales,
                                                     const uint16_t* __restrict__ zeros, int rows, int G, int gs,
                                                     int T, int Cs, uint32_t* __restrict__ SZ) {
  const int spc = gs > 0 ? kChunk / gs : 1;
  const int64_t id = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (id >= static_cast<int64_t>(T) * Cs * 16 * spc) return;
  const int i = static_cast<int>(id % spc);
  const int j = static_cast<int>((id / spc) & 15);
  const int64_t tc = id / (16 * spc);
  const int c = static_cast<int>(tc % Cs);
  const int tile = static_cast<int>(tc / Cs);
  const int g = gs > 0 ? c * spc + i : 0;
  const int o = tile * 16 + j;
  uint32_t v = 0;
  if (o < rows && g < G) {
    const int64_t src = static_cast<int64_t>(g) * rows + o;
    v = static_cast<uint32_t>(scales[src]) | (static_cast<uint32_t>(zeros[src]) << 16);
  }
  SZ[id] = v;
}

// Activations in the packed column order (act-order layers): At[m, k] =
// A[m, col_order[k]], row stride n.  A work-group takes whole rows: the row
// is staged in LDS (16-byte loads when A is 16-byte aligned with lda a
// multiple of 8, else 2-byte loads, both coalesced), then each thread
// gathers 8 consecutive outputs from LDS and writes them as one 16-byte
// store.  Rows up to kGatherLdsMax columns; longer ones use the plain kernel
// below.
constexpr int kGatherLdsMax = 32768;
template <bool VEC>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                          const int32_t* __restrict__ col_order, int M, int n,
                                                          uint16_t* __restrict__ At) {
  extern __shared__ __align__(16) uint16_t row_lds[];
  const int tid = threadIdx.x, pieces = n / 8;
  for (int m = blockIdx.x; m < M; m += gridDim.x) {
    const uint16_t* row = A + static_cast<int64_t>(m) * lda;
    if constexpr (VEC) {
      for (int p = tid; p < pieces; p += 256)
        *reinterpret_cast<u32x4*>(&row_lds[8 * p]) = *reinterpret_cast<const u32x4*>(row + 8 * p);
    } else {
      for (int k = tid; k < n; k += 256) row_lds[k] = row[k];
    }
    __syncthreads();
    uint16_t* out = At + static_cast<int64_t>(m) * n;
    for (int p = tid; p < pieces; p += 256) {
      const int32_t* ix = col_order + 8 * p;   // 4-byte aligned only: plain loads
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = row_lds[ix[2 * e]] | (static_cast<uint32_t>(row_lds[ix[2 * e + 1]]) << 16);
      *reinterpret_cast<u32x4*>(out + 8 * p) = v;
    }
    __syncthreads();  // the row buffer is reloaded next
  }
}

__global__ __launch_bounds__(256) void gather_cols_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                         const int32_t* __restrict__ col_order, int M, int n,
                                                         uint16_t* __restrict__ At) {
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const uint16_t* row = A + static_cast<int64_t>(m) * lda;
    uint16_t* out = At + static_cast<int64_t>(m) * n;
    for (int k = blockIdx.x * 256 + threadIdx.x; k < n; k += gridDim.x * 256) out[k] = row[col_order[k]];
  }
}

// ------------------------------------------------------------------ matmul side
__device__ __forceinline__ h2 as_h2(uint32_t x) { return __builtin_bit_cast(h2, x); }

// (x & mask) | 0x64006400 in one v_and_or_b32.  The compiler splits it into
// two instructions, since gfx9 three-operand encodings take no literal: here
// the mask is passed in a vector register and the exponent pattern in a
// scalar one.  ALU only.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(mask), "s"(0x64006400u));
  return r;
}

__device__ __forceinline__ h2 pk_fma(uint32_t x, h2 m, h2 c) { return __builtin_elementwise_fma(as_h2(x), m, c); }

// The 8-bit-per-field step values of one lane: the lane's codes for step t as
// the MFMA B operand, each half the exact integer code - z.  `zc[v]` holds
// -(base_v + z) for the exponent bias base_v of half-pair v.
template <int BITS>
struct Unpack;

template <>
struct Unpack<4> {
  static constexpr int kWords = 4;   // per lane per chunk
  // pairs (0,4), (1,5) from bits 0..7 of each half; (2,6), (3,7) after >> 8
  static constexpr float kBase[4] = {1024.f, 64.f, 1024.f, 64.f};
  __device__ static __forceinline__ h8 step(const uint32_t* w, int t, const h2* zc) {
    const uint32_t x = w[t];
    const uint32_t y = x >> 8;
    const h2 m1 = {(_Float16)1.0f, (_Float16)1.0f};
    const h2 m16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 p0 = pk_fma(and_or(x, 0x000F000Fu), m1, zc[0]);
    const h2 p1 = pk_fma(and_or(x, 0x00F000F0u), m16, zc[1]);
    const h2 p2 = pk_fma(and_or(y, 0x000F000Fu), m1, zc[2]);
    const h2 p3 = pk_fma(and_or(y, 0x00F000F0u), m16, zc[3]);
    return h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
};

template <>
struct Unpack<8> {
  static constexpr int kWords = 8;
  static constexpr float kBase[4] = {1024.f, 1024.f, 1024.f, 1024.f};
  __device__ static __forceinline__ h8 step(const uint32_t* w, int t, const h2* zc) {
    const uint32_t x0 = w[2 * t], x1 = w[2 * t + 1];
    const h2 m1 = {(_Float16)1.0f, (_Float16)1.0f};
    const h2 p0 = pk_fma(and_or(x0, 0x00FF00FFu), m1, zc[0]);
    const h2 p1 = pk_fma(and_or((x0 >> 8), 0x00FF00FFu), m1, zc[0]);
    const h2 p2 = pk_fma(and_or(x1, 0x00FF00FFu), m1, zc[0]);
    const h2 p3 = pk_fma(and_or((x1 >> 8), 0x00FF00FFu), m1, zc[0]);
    return h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
};

template <>
struct Unpack<2> {
  static constexpr int kWords = 2;
  static constexpr float kBase[4] = {1024.f, 256.f, 64.f, 16.f};
  __device__ static __forceinline__ h8 step(const uint32_t* w, int t, const h2* zc) {
    // field t = half (t & 1) of word t >> 1; bytes 0/1 of that half go to
    // bytes 0 and 2 of x, so each half of x holds four codes
    const uint32_t word = w[t >> 1];
    const uint32_t sel = (t & 1) ? 0x0C030C02u : 0x0C010C00u;
    const uint32_t x = __builtin_amdgcn_perm(0u, word, sel);
    const h2 m1 = {(_Float16)1.0f, (_Float16)1.0f};
    const h2 m4 = {(_Float16)0.25f, (_Float16)0.25f};
    const h2 m16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 m64 = {(_Float16)0.015625f, (_Float16)0.015625f};
    const h2 p0 = pk_fma(and_or(x, 0x00030003u), m1, zc[0]);
    const h2 p1 = pk_fma(and_or(x, 0x000C000Cu), m4, zc[1]);
    const h2 p2 = pk_fma(and_or(x, 0x00300030u), m16, zc[2]);
    const h2 p3 = pk_fma(and_or(x, 0x00C000C0u), m64, zc[3]);
    return h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
};

template <>
struct Unpack<3> {
  static constexpr int kWords = 3;
  static constexpr float kBase[4] = {1024.f, 128.f, 16.f, 1024.f};
  __device__ static __forceinline__ h8 step(const uint32_t* w, int t, const h2* zc) {
    // the 24-bit field of step t starts at bit 24t of the lane's 96-bit stream
    uint32_t v;
    if (t == 0) v = w[0];
    else if (t == 1) v = __builtin_amdgcn_alignbit(w[1], w[0], 24);
    else if (t == 2) v = __builtin_amdgcn_alignbit(w[2], w[1], 16);
    else v = w[2] >> 8;
    // fields 0..3 stay in bits 0..11, fields 4..7 move to bits 16..27
    const uint32_t x = __builtin_amdgcn_ubfe(v, 0, 12) | ((v << 4) & 0x0FFF0000u);
    const uint32_t y = x >> 9;
    const h2 m1 = {(_Float16)1.0f, (_Float16)1.0f};
    const h2 m8 = {(_Float16)0.125f, (_Float16)0.125f};
    const h2 m64 = {(_Float16)0.015625f, (_Float16)0.015625f};
    const h2 p0 = pk_fma(and_or(x, 0x00070007u), m1, zc[0]);
    const h2 p1 = pk_fma(and_or(x, 0x00380038u), m8, zc[1]);
    const h2 p2 = pk_fma(and_or(x, 0x01C001C0u), m64, zc[2]);
    const h2 p3 = pk_fma(and_or(y, 0x00070007u), m1, zc[3]);
    return h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  }
};

// The codes are read once: non-temporal loads keep them from displacing the
// activations and scale/zero words in the caches.
template <int BITS>
__device__ __forceinline__ void load_chunk(const uint32_t* __restrict__ p, uint32_t* w) {
  if constexpr (BITS == 4) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (BITS == 8) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  } else if constexpr (BITS == 2) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    w[0] = v[0]; w[1] = v[1];
  } else {
    w[0] = __builtin_nontemporal_load(p);
    w[1] = __builtin_nontemporal_load(p + 1);
    w[2] = __builtin_nontemporal_load(p + 2);
  }
}

// The same through a buffer resource: lane offset voff, uniform offset soff
// (bytes).  Word 3 of a raw buffer resource: 32-bit data format.
constexpr int kBufWord3 = 0x00020000;
template <int BITS>
__device__ __forceinline__ void load_chunk_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t* w) {
  if constexpr (BITS == 4) {
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  } else if constexpr (BITS == 8) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, 0));
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  } else if constexpr (BITS == 2) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    w[0] = v[0]; w[1] = v[1];
  } else {
    typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
    const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0));
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  }
}

// Accumulator layout of the 16x16 f32 MFMA tiles: lane l, register r holds
// row 4*(l/16) + r (token), column l%16 (output).
__device__ __forceinline__ int acc_row(int lane, int r) { return 4 * (lane >> 4) + r; }

// SPC: scale/zero words per chunk (128 / group size; 1 also for one group per
// row, gs == 0).  A holds the activations in the packed (grouped) column order.
// FULL: the slice's activations are staged in LDS once, before the loop
// (decode sizes); else 1024-column windows are staged round by round (NW = 8).
// NW: waves per workgroup, all on the same 16 outputs, splitting the chunks.
// PIECES: 16-byte pieces of activations and scale/zero words each thread
// stages (FULL).
template <int BITS, int SPC, bool FULL, int NW, int PIECES>
__global__ __launch_bounds__(NW * 64) void dequant_matmul_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int M, const uint32_t* __restrict__ Q,
    const uint32_t* __restrict__ SZ, int rows, int n, int gs, void* __restrict__ Y, int ydt, int64_t ldy) {
  using U = Unpack<BITS>;
  extern __shared__ __align__(16) unsigned char mm_smem[];
  _Float16* abuf = reinterpret_cast<_Float16*>(mm_smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x;
  const int m0 = blockIdx.y * kMTile;
  const int ms = min(kMTile, M - m0);           // tokens of this slice
  const int C = n / kChunk;
  static_assert(FULL || NW == kWinWaves, "windowed staging assumes one window chunk per wave");
  constexpr int kThreads = NW * 64;
  const int R = (C + NW - 1) / NW;  // rounds: one chunk per wave each
  const int j = lane & 15, q = lane >> 4;
  const int arow = min(j, ms - 1);              // rows >= ms repeat the last one; their outputs are dropped
  const uint32_t* qbase = Q + (static_cast<int64_t>(tile) * C * 64 + lane) * U::kWords;
  // The tile's scale/zero words ([Cs][16][SPC], G * 16 in all) are staged in
  // LDS after the activations.
  const int Cs = gs > 0 ? C : 1;
  const int szw = Cs * 16 * SPC;
  const uint32_t* sztile = SZ + static_cast<int64_t>(tile) * szw;
  const int astride = FULL ? n + 8 : kWinStride;   // halves per staged row (16-byte pad)
  uint32_t* szs = reinterpret_cast<uint32_t*>(abuf + (FULL ? ms * astride : 2 * ms * kWinStride));

  // ---- codes: kAhead chunks in flight per wave.  Chunk indexes past the
  // last are clamped (loaded, never used), so the loop issues exactly one
  // unconditional load per round and the compiler can count those in flight.
  uint32_t breg[kAhead][U::kWords];
  auto b_load = [&](int c, int d) {
    load_chunk<BITS>(qbase + static_cast<int64_t>(min(c, C - 1)) * 64 * U::kWords, breg[d]);
  };
  // ---- windowed staging: window r (columns 1024 r ...) in pieces of 8 halves;
  // piece p = tid + 512 v is token p / 128, columns 8 (p % 128).  Whether a
  // piece exists is uniform per wave (pieces is a multiple of 64); columns
  // past n are clamped (those LDS columns belong to chunks no wave visits).
  // Two register sets, so a window's loads never wait for the previous one.
  const int pieces = ms * (kWin / 8);
  uint32_t areg[2][4][4];
  auto a_load = [&](int r, int set) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (wave * 64 + v * kThreads < pieces) {
        const int p = tid + v * kThreads;
        const int m = p / (kWin / 8), kp = p % (kWin / 8);
        const int k = min(r * kWin + 8 * kp, n - 8);
        const u32x4 x = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(m0 + m) * lda + k);
        areg[set][v][0] = x[0]; areg[set][v][1] = x[1]; areg[set][v][2] = x[2]; areg[set][v][3] = x[3];
      }
    }
  };
  auto a_store = [&](int buf, int set) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (wave * 64 + v * kThreads < pieces) {
        const int p = tid + v * kThreads;
        const int m = p / (kWin / 8), kp = p % (kWin / 8);
        u32x4 x = {areg[set][v][0], areg[set][v][1], areg[set][v][2], areg[set][v][3]};
        *reinterpret_cast<u32x4*>(abuf + (buf * ms + m) * kWinStride + 8 * kp) = x;
      }
    }
  };

  if constexpr (FULL) {
    // The slice's activations and the tile's scale/zero words, at most
    // PIECES pieces of 16 bytes per thread, are loaded before the code
    // prefetch is issued, so the stores below wait only for them and the first
    // chunk is consumed as soon as it lands.  Loads are clamped, not skipped.
    const int per_row = n / 8;
    const int total_a = ms * per_row;
    const int total = total_a + szw / 4;
    u32x4 x[PIECES];
#pragma unroll
    for (int v = 0; v < PIECES; ++v) {
      const int p = min(tid + v * kThreads, total - 1);
      const int m = p / per_row, kp = p % per_row;
      const u32x4* src = p < total_a
          ? reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(m0 + m) * lda + 8 * kp)
          : reinterpret_cast<const u32x4*>(sztile) + (p - total_a);
      x[v] = *src;
    }
#pragma unroll
    for (int d = 0; d < kAhead; ++d) b_load(wave + NW * d, d);
#pragma unroll
    for (int v = 0; v < PIECES; ++v) {
      const int p = tid + v * kThreads;
      if (p < total_a) {
        const int m = p / per_row, kp = p % per_row;
        *reinterpret_cast<u32x4*>(abuf + m * astride + 8 * kp) = x[v];
      } else if (p < total) {
        reinterpret_cast<u32x4*>(szs)[p - total_a] = x[v];
      }
    }
  } else {
    for (int p = tid; p < szw / 4; p += kThreads)
      reinterpret_cast<u32x4*>(szs)[p] = reinterpret_cast<const u32x4*>(sztile)[p];
#pragma unroll
    for (int d = 0; d < kAhead; ++d) b_load(wave + NW * d, d);
    a_load(0, 0);
    a_store(0, 0);
    // Everything issued so far has landed (the staging stores needed their
    // loads, which were issued after the code prefetches).  Saying so tells
    // the compiler that no load is in flight at the top of the loop, so inside
    // it it waits only for the chunk it is about to use.
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
  }
  lds_barrier();

  f4 yacc = {0.f, 0.f, 0.f, 0.f};
  f4 gacc = {0.f, 0.f, 0.f, 0.f};
  // A group covers 4 / SPC steps of a chunk (one group per row: the chunk's
  // four steps, all with the row's one scale and zero).
  constexpr int kGroupSteps = 4 / SPC;

  // One chunk: four MFMA steps over the prefetched codes of slot d.  Waves
  // past the last chunk run on the clamped chunk with their result dropped
  // (live false), so that every round is the same straight-line code.
  auto chunk = [&](int d, int cc, bool live, const _Float16* ap) {
    const uint32_t* szc = szs + ((gs > 0 ? cc : 0) * 16 + j) * SPC;
    h2 zc[4];
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t % kGroupSteps == 0) {
        const uint32_t sz = szc[t / kGroupSteps];
        s = live ? half_bits_to_float(static_cast<uint16_t>(sz & 0xFFFFu)) : 0.f;
        const _Float16 z = __builtin_bit_cast(_Float16, static_cast<uint16_t>(sz >> 16));
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const _Float16 c0 = -(static_cast<_Float16>(U::kBase[v]) + z);
          zc[v] = h2{c0, c0};
        }
      }
      const h8 b = U::step(breg[d], t, zc);
      const h8 a = *reinterpret_cast<const h8*>(ap + 32 * t);
      gacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, gacc, 0, 0, 0);
      // the group ends here (or, one group per row, continues in another
      // chunk): scale this wave's partial sum of it now (exact scaling, one
      // fp32 rounding)
      if (t % kGroupSteps == kGroupSteps - 1) {
        yacc += s * gacc;
        gacc = f4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  // Whole groups of kAhead rounds: a round past the end runs like the rest
  // on the clamped chunk with its result dropped.  (Skipping it instead makes
  // the compiler lose count of the loads in flight and wait for all of them
  // in every round.)
  const int Rp = (R + kAhead - 1) / kAhead * kAhead;
  for (int r0 = 0; r0 < Rp; r0 += kAhead) {
#pragma unroll
    for (int d = 0; d < kAhead; ++d) {
      const int r = r0 + d;
      const int c = wave + NW * r;
      const bool live = c < C;
      const int cc = live ? c : C - 1;
      if constexpr (FULL) {
        chunk(d, cc, live, abuf + arow * astride + cc * kChunk + 8 * q);
        b_load(c + NW * kAhead, d);
      } else {
        // window r + 1 goes to buffer and register set (r + 1) & 1 = (d + 1) & 1
        if (r + 1 < R) a_load(r + 1, (d + 1) & 1);
        const int rc = cc / NW;   // window holding chunk cc (r when live)
        chunk(d, cc, live, abuf + ((rc & 1) * ms + arow) * kWinStride + (cc - NW * rc) * kChunk + 8 * q);
        b_load(c + NW * kAhead, d);
        if (r + 1 < R) a_store((d + 1) & 1, (d + 1) & 1);
        lds_barrier();
      }
    }
  }

  // ---- sum the 8 waves' partial tiles and store
  float* red = reinterpret_cast<float*>(mm_smem);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(wave * 64 + lane) * 4 + r] = yacc[r];
  __syncthreads();
  if (tid < kMTile * 16) {
    const int mm = tid >> 4, o_in = tid & 15;
    const int l = 16 * (mm >> 2) + o_in, r = mm & 3;   // inverse of acc_row
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) sum += red[(v * 64 + l) * 4 + r];
    const int o = tile * 16 + o_in;
    if (mm < ms && o < rows) {
      const int64_t idx = static_cast<int64_t>(m0 + mm) * ldy + o;
      if (ydt == DT_FP32) static_cast<float*>(Y)[idx] = sum;
      else static_cast<uint16_t*>(Y)[idx] = float_to_half_bits(sum);
    }
  }
}

// ------------------------------------------------------------------ persistent decode
// One slice of up to 16 tokens whose activations fit LDS whole beside two
// tiles' scale/zero words (10-16 tokens at n = 4096), where the decode kernel
// above would stage the activations window by window for every 16-output
// tile (four times the tile's weight bytes at 16 tokens): one work-group of
// 8 waves per compute unit stages the activations once and walks the output
// tiles b, b + G, b + 2G, ... (G work-groups).  The waves split each tile's
// chunks as in the decode kernel, and their rounds run as one sequence across
// the tiles, so the code prefetch (kAhead chunks per wave) runs on into the
// next tile while the current one is summed.  A tile's scale/zero words are
// loaded when the tile two before it starts (before that tile's code loads,
// so no wait for them ever waits for codes) and staged after that tile's
// closing barrier, into the LDS buffer it has just finished reading.  The
// per-chunk arithmetic is the decode kernel's, so the two round alike.
constexpr int kPersistWaves = 8;
constexpr size_t kPersistLds = 160 * 1024;
constexpr int kPersistSzPieces = 2;   // 16-byte pieces of scale/zero words per thread

inline size_t persist_lds_bytes(int ms, int n, int szw) {
  return static_cast<size_t>(ms) * (n + 8) * 2 + static_cast<size_t>(2) * szw * 4 +
         static_cast<size_t>(2) * kPersistWaves * 64 * 4 * sizeof(float);
}

template <int BITS, int SPC>
__global__ __launch_bounds__(kPersistWaves * 64) void decode_persist_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int ms, const uint32_t* __restrict__ Q,
    const uint32_t* __restrict__ SZ, int rows, int n, int gs, void* __restrict__ Y, int ydt, int64_t ldy, int T) {
  using U = Unpack<BITS>;
  constexpr int NW = kPersistWaves, kThreads = NW * 64;
  extern __shared__ __align__(16) unsigned char mm_smem[];
  _Float16* abuf = reinterpret_cast<_Float16*>(mm_smem);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int C = n / kChunk;
  const int Rp = ((C + NW - 1) / NW + kAhead - 1) / kAhead * kAhead;   // rounds per tile, whole groups of kAhead
  const int j = lane & 15, q = lane >> 4;
  const int arow = min(j, ms - 1);               // rows >= ms repeat the last one; their outputs are dropped
  const int Cs = gs > 0 ? C : 1;
  const int szw = Cs * 16 * SPC;                 // scale/zero words of a tile
  const int szp = szw / 4;                       // ... in 16-byte pieces (<= kPersistSzPieces * kThreads)
  const int astride = n + 8;
  uint32_t* szs = reinterpret_cast<uint32_t*>(abuf + ms * astride);   // [2][szw]
  float* red = reinterpret_cast<float*>(szs + 2 * szw);               // [2][NW * 64 * 4]
  const int G = gridDim.x;
  const int ntiles = (T - 1 - static_cast<int>(blockIdx.x)) / G + 1;  // blockIdx.x < T
  const int nrounds = ntiles * Rp;
  auto tile_of = [&](int k) { return static_cast<int>(blockIdx.x) + min(k, ntiles - 1) * G; };

  // codes of flat round rho = k * Rp + r (tile k, chunk wave + NW r), clamped
  // past the last round and the last chunk: loaded, never used
  uint32_t breg[kAhead][U::kWords];
  auto b_load = [&](int rho, int d) {
    const int rr = min(rho, nrounds - 1);
    const int k = rr / Rp;
    const int c = min(wave + NW * (rr - k * Rp), C - 1);
    load_chunk<BITS>(Q + ((static_cast<int64_t>(tile_of(k)) * C + c) * 64 + lane) * U::kWords, breg[d]);
  };
  u32x4 szr[kPersistSzPieces];
  auto sz_load = [&](int k) {
    const u32x4* src = reinterpret_cast<const u32x4*>(SZ + static_cast<int64_t>(tile_of(k)) * szw);
#pragma unroll
    for (int v = 0; v < kPersistSzPieces; ++v) szr[v] = src[min(tid + v * kThreads, szp - 1)];
  };
  auto sz_store = [&](int buf) {
#pragma unroll
    for (int v = 0; v < kPersistSzPieces; ++v) {
      const int p = tid + v * kThreads;
      if (p < szp) reinterpret_cast<u32x4*>(szs + buf * szw)[p] = szr[v];
    }
  };

  // The code prefetch first, so that the codes are on their way while the
  // activations are staged (once, 16 pieces of 16 bytes per thread in flight
  // at a time: 16 tokens at n = 4096 in one batch), then the first two
  // tiles' scale/zero words.
#pragma unroll
  for (int d = 0; d < kAhead; ++d) b_load(d, d);
  {
    constexpr int kBatch = 16;
    const int per_row = n / 8, total_a = ms * per_row;
    for (int p0 = 0; p0 < total_a; p0 += kBatch * kThreads) {
      u32x4 x[kBatch];
#pragma unroll
      for (int v = 0; v < kBatch; ++v) {
        const int p = min(p0 + tid + v * kThreads, total_a - 1);
        const int m = p / per_row, kp = p - m * per_row;
        x[v] = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(m) * lda + 8 * kp);
      }
#pragma unroll
      for (int v = 0; v < kBatch; ++v) {
        const int p = p0 + tid + v * kThreads;
        if (p < total_a) {
          const int m = p / per_row, kp = p - m * per_row;
          *reinterpret_cast<u32x4*>(abuf + m * astride + 8 * kp) = x[v];
        }
      }
    }
  }
  sz_load(0);
  sz_store(0);
  sz_load(1);
  sz_store(1);
  lds_barrier();

  f4 yacc = {0.f, 0.f, 0.f, 0.f};
  f4 gacc = {0.f, 0.f, 0.f, 0.f};
  constexpr int kGroupSteps = 4 / SPC;
  auto chunk = [&](int d, int cc, bool live, const uint32_t* szb, const _Float16* ap) {
    const uint32_t* szc = szb + ((gs > 0 ? cc : 0) * 16 + j) * SPC;
    h2 zc[4];
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t % kGroupSteps == 0) {
        const uint32_t sz = szc[t / kGroupSteps];
        s = live ? half_bits_to_float(static_cast<uint16_t>(sz & 0xFFFFu)) : 0.f;
        const _Float16 z = __builtin_bit_cast(_Float16, static_cast<uint16_t>(sz >> 16));
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const _Float16 c0 = -(static_cast<_Float16>(U::kBase[v]) + z);
          zc[v] = h2{c0, c0};
        }
      }
      const h8 b = U::step(breg[d], t, zc);
      const h8 a = *reinterpret_cast<const h8*>(ap + 32 * t);
      gacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, gacc, 0, 0, 0);
      if (t % kGroupSteps == kGroupSteps - 1) {
        yacc += s * gacc;
        gacc = f4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  for (int k = 0; k < ntiles; ++k) {
    sz_load(k + 2);   // staged at the end of this tile, into the buffer this tile reads
    const uint32_t* szb = szs + (k & 1) * szw;
    for (int r0 = 0; r0 < Rp; r0 += kAhead) {
#pragma unroll
      for (int d = 0; d < kAhead; ++d) {
        const int r = r0 + d;
        const int c = wave + NW * r;
        const bool live = c < C;
        const int cc = live ? c : C - 1;
        chunk(d, cc, live, szb, abuf + arow * astride + cc * kChunk + 8 * q);
        b_load(k * Rp + r + kAhead, d);
      }
    }
    // the 8 waves' partial tiles: summed and stored; then the scale/zero
    // words of tile k + 2 replace this tile's
    float* rk = red + (k & 1) * (NW * 64 * 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) rk[(wave * 64 + lane) * 4 + rr] = yacc[rr];
    __syncthreads();
    if (tid < kMTile * 16) {
      const int mm = tid >> 4, o_in = tid & 15;
      const int l = 16 * (mm >> 2) + o_in, rr = mm & 3;   // inverse of acc_row
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) sum += rk[(v * 64 + l) * 4 + rr];
      const int o = tile_of(k) * 16 + o_in;
      if (mm < ms && o < rows) {
        const int64_t idx = static_cast<int64_t>(mm) * ldy + o;
        if (ydt == DT_FP32) static_cast<float*>(Y)[idx] = sum;
        else static_cast<uint16_t*>(Y)[idx] = float_to_half_bits(sum);
      }
    }
    sz_store(k & 1);
    yacc = f4{0.f, 0.f, 0.f, 0.f};
  }
}

// ------------------------------------------------------------------ prefill
// Many tokens (M >= kPrefillMin): one workgroup of 4 waves per tile of 128
// tokens x 64 outputs, wave (wm, wn) owning 64 x 32 as 4 x 2 MFMA tiles of
// 16 x 16 (at 64 x 64 a wave needs every register, one wave per SIMD, and
// cannot hide its own loads: 315 TFLOP/s on a 262144-token projection).  For
// each 128-column chunk the tile's activations (128 x 128 halves) are staged
// in LDS, double buffered, rows padded to 144 halves.  On this chip a 16-byte
// LDS read serves each half-wave in two cycles, lanes split by the parity of
// lane bits 2-4, and is conflict-free when each such set of 16 lanes touches
// 16 distinct 16-byte bank groups (measured with a probe); a fragment read
// (lane j of 16 on token j, 16 bytes at column 32t + 8q) meets that with
// 18-unit rows, not with 17.  A 16-byte write serves 8 consecutive lanes per
// cycle, which the staging stores (consecutive columns) always meet.  The activations
// and codes of the two chunks after it are in flight in registers meanwhile.
// Each wave loads its output tiles' codes straight from the
// packed layer (a lane's bytes of a chunk are its B operand for the chunk's
// four steps), turns them into the exact fp16 integers code - zero and scales
// each group's fp32 partial sum by the group's scale when the group ends, as
// the decode kernel does, so the two kernels round alike.  The hardware
// deals work-group b to XCD b % 8; the tiles are ordered so that all output
// tiles of a token tile go to one XCD, which then fetches those 128 token
// rows from memory once and serves the rest from its L2.
constexpr int kPM = 128;                 // tokens per tile
constexpr int kPNT = 2;                  // 16-output tiles per wave
constexpr int kPN = 2 * 16 * kPNT;       // outputs per tile (two waves across)
constexpr int kPStride = kChunk + 16;    // halves per staged token row (18 units of 16 bytes: the
                                         // fragment reads are conflict-free, 17 units conflict 2-way)
constexpr int kPrefillMin = 256;         // tokens from which the prefill kernel runs: from here on it
                                         // is no slower than the decode kernel's 16-token slices
                                         // (4096 x 4096 layer, 256 tokens: 52.7 against 51.4 us;
                                         // 512 tokens: 55 against 119 us)
// activations two chunks ahead where that fits in registers without spilling
// (not with two groups per chunk), else one
template <int BITS, int SPC>
constexpr int kPrefillDepth = 2;

template <int BITS, int SPC, int DEPTH>
__global__ __launch_bounds__(256, 2) void prefill_matmul_kernel(const uint16_t* __restrict__ A, int64_t lda, int M,
                                                             const uint32_t* __restrict__ Q,
                                                             const uint32_t* __restrict__ SZ, int rows, int n, int gs,
                                                             void* __restrict__ Y, int ydt, int64_t ldy, int tm_count,
                                                             int tn_count) {
  using U = Unpack<BITS>;
  __shared__ __align__(16) _Float16 abuf[2][kPM][kPStride];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
  const int tmt = 8 * (local / tn_count) + xcd, tnt = local % tn_count;
  if (tmt >= tm_count) return;  // the grid is rounded up to whole groups of 8 token tiles
  const int m0 = tmt * kPM, o0 = tnt * kPN;
  const int C = n / kChunk;
  const int Cs = gs > 0 ? C : 1;
  const int j = lane & 15, q = lane >> 4;
  const int Tcount = (rows + 15) / 16;
  // this wave's packed output tiles (clamped past the last: loaded, dropped)
  // Every load is a buffer load: a resource over the region the loop reads
  // (uniform across the wave), a lane offset fixed for the whole loop and a
  // scalar offset per chunk, so the loads need no per-chunk vector address
  // arithmetic.  Every offset stays inside its resource's range (tokens past
  // M are clamped to M - 1, output tiles past the last to the last).
  __amdgpu_buffer_rsrc_t qr[kPNT], szr_rs[kPNT];   // this wave's output tiles' codes, scale/zero words
#pragma unroll
  for (int nt = 0; nt < kPNT; ++nt) {
    const int T = min(o0 / 16 + kPNT * wn + nt, Tcount - 1);
    qr[nt] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(Q + static_cast<int64_t>(T) * C * 64 * U::kWords),
                                               0, C * 64 * U::kWords * 4, kBufWord3);
    szr_rs[nt] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(SZ + static_cast<int64_t>(T) * Cs * 16 * SPC),
                                                   0, Cs * 16 * SPC * 4, kBufWord3);
  }
  const int qoff = lane * U::kWords * 4;   // bytes
  const int szoff = j * SPC * 4;
  // activations: piece p = tid + 256 v is token p / 16, halves 8 (p % 16) ..
  // of the chunk; tokens past M read token M - 1 (their outputs are dropped)
  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A + static_cast<int64_t>(m0) * lda), 0,
      static_cast<int>((static_cast<int64_t>(min(M - m0, kPM) - 1) * lda + n) * 2), kBufWord3);
  int aoff[8];   // bytes from the tile's first token
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int p = tid + 256 * v;
    const int tm = min(m0 + (p >> 4), M - 1);
    aoff[v] = ((tm - m0) * lda + 8 * (p & 15)) * 2;
  }
  u32x4 areg[DEPTH][8];  // DEPTH register sets of activations on their way to LDS
  auto a_load = [&](int c, int set) {
#pragma unroll
    for (int v = 0; v < 8; ++v)
      areg[set][v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[v], c * kChunk * 2, 0));
  };
  auto a_store = [&](int buf, int set) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int p = tid + 256 * v;
      *reinterpret_cast<u32x4*>(&abuf[buf][p >> 4][8 * (p & 15)]) = areg[set][v];
    }
  };
  // codes and scale/zero words of a chunk, two slots
  uint32_t breg[2][kPNT][U::kWords];
  uint32_t szr[2][kPNT][SPC];
  auto b_load = [&](int c, int d) {
#pragma unroll
    for (int nt = 0; nt < kPNT; ++nt) {
      load_chunk_buf<BITS>(qr[nt], qoff, c * 64 * U::kWords * 4, breg[d][nt]);
#pragma unroll
      for (int g = 0; g < SPC; ++g)
        szr[d][nt][g] = __builtin_amdgcn_raw_buffer_load_b32(szr_rs[nt], szoff + 4 * g, (gs > 0 ? c : 0) * 16 * SPC * 4, 0);
    }
  };
  f4 yacc[4][kPNT], gacc[4][kPNT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < kPNT; ++nt) {
      yacc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
      gacc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
    }
  constexpr int kGroupSteps = 4 / SPC;

  // one chunk from LDS buffer `buf` and code slot `d`
  auto chunk = [&](int buf, int d) {
    h2 zc[kPNT][4];
    float sc[kPNT];
    // activation fragments one k-step ahead of the products that use them
    h8 an[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) an[mt] = *reinterpret_cast<const h8*>(&abuf[buf][64 * wm + 16 * mt + j][8 * q]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t % kGroupSteps == 0) {
#pragma unroll
        for (int nt = 0; nt < kPNT; ++nt) {
          const uint32_t sz = szr[d][nt][t / kGroupSteps];
          sc[nt] = half_bits_to_float(static_cast<uint16_t>(sz & 0xFFFFu));
          const _Float16 z = __builtin_bit_cast(_Float16, static_cast<uint16_t>(sz >> 16));
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const _Float16 c0 = -(static_cast<_Float16>(U::kBase[v]) + z);
            zc[nt][v] = h2{c0, c0};
          }
        }
      }
      h8 bb[kPNT], aa[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) aa[mt] = an[mt];
      if (t < 3) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          an[mt] = *reinterpret_cast<const h8*>(&abuf[buf][64 * wm + 16 * mt + j][32 * (t + 1) + 8 * q]);
      }
#pragma unroll
      for (int nt = 0; nt < kPNT; ++nt) bb[nt] = U::step(breg[d][nt], t, zc[nt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < kPNT; ++nt)
          gacc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aa[mt], bb[nt], gacc[mt][nt], 0, 0, 0);
      if (t % kGroupSteps == kGroupSteps - 1) {  // the group ends: scale its partial sums
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < kPNT; ++nt) {
            yacc[mt][nt] += sc[nt] * gacc[mt][nt];
            gacc[mt][nt] = f4{0.f, 0.f, 0.f, 0.f};
          }
        if constexpr (SPC == 2) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Chunk c is computed from LDS buffer c & 1 and code slot c & 1; the chunk
  // after it is staged into the other buffer (last read in chunk c - 1,
  // before the previous barrier).  DEPTH 2: chunk c + 2's activations are
  // loaded before chunk c is computed, its codes after; DEPTH 1: chunk c + 1's
  // codes before, chunk c + 2's activations after.  Loads past the last chunk
  // re-read it, so every step issues the same loads with no branch (a branch
  // around a load makes the compiler wait for all loads in flight where the
  // paths join); the loop is unrolled by two so that the register slots are
  // compile-time constants (indexed at run time they would live in scratch).
  const int last = C - 1;
  a_load(0, 0);
  b_load(0, 0);
  if constexpr (DEPTH == 2) {
    a_load(min(1, last), 1);
    b_load(min(1, last), 1);
    a_store(0, 0);
  } else {
    a_store(0, 0);
    a_load(min(1, last), 0);
  }
  __syncthreads();
  auto step = [&](auto par, int c) {
    constexpr int P = decltype(par)::value;
    if constexpr (DEPTH == 2) {
      a_load(min(c + 2, last), P);
      __builtin_amdgcn_sched_barrier(0);  // issued before the chunk, not sunk below it
      chunk(P, P);
      b_load(min(c + 2, last), P);
      a_store(P ^ 1, P ^ 1);
    } else {
      b_load(min(c + 1, last), P ^ 1);
      chunk(P, P);
      a_store(P ^ 1, 0);
      a_load(min(c + 2, last), 0);
    }
    __syncthreads();
  };
  int c = 0;
  for (; c + 1 < C; c += 2) {
    step(std::integral_constant<int, 0>{}, c);
    step(std::integral_constant<int, 1>{}, c + 1);
  }
  if (c < C) step(std::integral_constant<int, 0>{}, c);

#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < kPNT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = m0 + 64 * wm + 16 * mt + acc_row(lane, r);
        const int o = o0 + 16 * kPNT * wn + 16 * nt + j;
        if (tok < M && o < rows) {
          const int64_t idx = static_cast<int64_t>(tok) * ldy + o;
          if (ydt == DT_FP32) static_cast<float*>(Y)[idx] = yacc[mt][nt][r];
          else static_cast<uint16_t*>(Y)[idx] = float_to_half_bits(yacc[mt][nt][r]);
        }
      }
}

template <int BITS, int SPC>
hipError_t launch_prefill(const uint16_t* A, int64_t lda, int M, const uint32_t* Q, const uint32_t* SZ, int rows,
                          int n, int gs, void* Y, int ydt, int64_t ldy, hipStream_t s) {
  const int tm = (M + kPM - 1) / kPM, tn = (rows + kPN - 1) / kPN;
  const int64_t blocks = static_cast<int64_t>((tm + 7) / 8) * 8 * tn;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_matmul_kernel<BITS, SPC, kPrefillDepth<BITS, SPC>>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, A, lda,
                     M, Q, SZ, rows, n, gs, Y, ydt, ldy, tm, tn);
  return hipGetLastError();
}

// Compute units of the current device (looked up once per device).
inline hipError_t device_cus(int* cus) {
  static int cached[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!cached[dev]) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[dev] = v;
  }
  *cus = cached[dev];
  return hipSuccess;
}

template <int BITS, int SPC>
hipError_t launch_persist(const uint16_t* A, int64_t lda, int M, const uint32_t* Q, const uint32_t* SZ, int rows,
                          int n, int gs, void* Y, int ydt, int64_t ldy, size_t lds, hipStream_t s) {
  auto kern = decode_persist_kernel<BITS, SPC>;
  static bool attr_set = false;   // per instantiation; idempotent if raced
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kPersistLds));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  int cus = 0;
  hipError_t e = device_cus(&cus);
  if (e != hipSuccess) return e;
  const int T = (rows + 15) / 16;
  const int G = T < cus ? T : cus;   // one work-group per compute unit (its LDS holds one)
  hipLaunchKernelGGL(kern, dim3(G), dim3(kPersistWaves * 64), lds, s, A, lda, M, Q, SZ, rows, n, gs, Y, ydt, ldy, T);
  return hipGetLastError();
}

template <int BITS, int SPC, bool FULL, int NW, int PIECES = 1>
hipError_t launch_mm_v(const uint16_t* A, int64_t lda, int M, const uint32_t* Q, const uint32_t* SZ, int rows,
                       int n, int gs, void* Y, int ydt, int64_t ldy, size_t lds, hipStream_t s) {
  auto kern = dequant_matmul_kernel<BITS, SPC, FULL, NW, PIECES>;
  static bool attr_set = false;   // per instantiation; idempotent if raced
  if (!attr_set) {
    const size_t most = FULL ? kFullLds : kWinLds;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(most));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int T = (rows + 15) / 16;
  dim3 grid(T, (M + kMTile - 1) / kMTile);
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, A, lda, M, Q, SZ, rows, n, gs, Y, ydt, ldy);
  return hipGetLastError();
}

template <int BITS, int SPC>
hipError_t launch_mm(const uint16_t* A, int64_t lda, int M, const uint32_t* Q, const uint32_t* SZ, int rows, int n,
                     int gs, void* Y, int ydt, int64_t ldy, hipStream_t s) {
  if (M >= kPrefillMin) return launch_prefill<BITS, SPC>(A, lda, M, Q, SZ, rows, n, gs, Y, ydt, ldy, s);
  const int ms = M < kMTile ? M : kMTile;
  const int T = (rows + 15) / 16;
  const int64_t tiles = static_cast<int64_t>(T) * ((M + kMTile - 1) / kMTile);
  const int G = gs > 0 ? n / gs : 1;
  const size_t sz_bytes = static_cast<size_t>(G) * 16 * 4;          // the tile's scale/zero words
  auto red = [](int nw) { return static_cast<size_t>(nw) * 64 * 4 * sizeof(float); };   // final sum of the waves
  const size_t full = static_cast<size_t>(ms) * (n + 8) * sizeof(_Float16) + sz_bytes;
  const int64_t pieces = static_cast<int64_t>(ms) * (n / 8) + G * 4;
  if (full <= kFullLds) {
    // 8 waves per tile, or 4 when 8 would not put every tile on the chip at
    // once; the fewest staging pieces per thread that cover the slice
#define GPTQ_MM_FULL(NW)                                                                                   \
    if (pieces <= 2 * NW * 64)                                                                             \
      return launch_mm_v<BITS, SPC, true, NW, 2>(A, lda, M, Q, SZ, rows, n, gs, Y, ydt, ldy,               \
                                                 std::max(full, red(NW)), s);                              \
    if (pieces <= 4 * NW * 64)                                                                             \
      return launch_mm_v<BITS, SPC, true, NW, 4>(A, lda, M, Q, SZ, rows, n, gs, Y, ydt, ldy,               \
                                                 std::max(full, red(NW)), s);                              \
    if (pieces <= kFullPieces * NW * 64)                                                                   \
      return launch_mm_v<BITS, SPC, true, NW, kFullPieces>(A, lda, M, Q, SZ, rows, n, gs, Y, ydt, ldy,     \
                                                           std::max(full, red(NW)), s);
    if (tiles * 8 <= kWaveSlots) {
      GPTQ_MM_FULL(8)
    }
    GPTQ_MM_FULL(4)
#undef GPTQ_MM_FULL
  }
  // one slice whose activations fit LDS whole beside two tiles' scale/zero
  // words: staged once per compute unit instead of once per tile
  if (M <= kMTile) {
    const int szw = (gs > 0 ? n / kChunk : 1) * 16 * SPC;
    const size_t plds = persist_lds_bytes(ms, n, szw);
    if (plds <= kPersistLds && szw / 4 <= kPersistSzPieces * kPersistWaves * 64)
      return launch_persist<BITS, SPC>(A, lda, M, Q, SZ, rows, n, gs, Y, ydt, ldy, plds, s);
  }
  const size_t win = static_cast<size_t>(2) * ms * kWinStride * sizeof(_Float16) + sz_bytes;
  if (win > kWinLds) return hipErrorInvalidValue;   // the entry point bounds n so this cannot happen
  return launch_mm_v<BITS, SPC, false, kWinWaves>(A, lda, M, Q, SZ, rows, n, gs, Y, ydt, ldy,
                                                  std::max(win, red(kWinWaves)), s);
}

}  // namespace

// The windowed variant keeps a tile's scale/zero words in LDS beside two
// windows of 16 tokens: n / group_size groups must fit.
bool matmul_fits(int64_t n, int group_size) {
  const int64_t G = group_size > 0 ? n / group_size : 1;
  return static_cast<size_t>(2) * kMTile * kWinStride * sizeof(_Float16) + static_cast<size_t>(G) * 64 <= kWinLds;
}

size_t matmul_packed_bytes(int64_t rows, int64_t n, int bits, int group_size) {
  const int64_t T = (rows + 15) / 16;
  const int64_t C = n / kChunk;
  const int64_t G = group_size > 0 ? n / group_size : 1;
  return kHeader + align256(static_cast<size_t>(T * C * 64 * bits) * 4) + static_cast<size_t>(T * G * 16) * 4;
}

hipError_t launch_matmul_pack(const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                              const int32_t* g_idx, int64_t rows, int64_t n, int bits, int group_size,
                              void* packed, int32_t* col_order, uint32_t* flags_host, hipStream_t s) {
  const int gs = group_size > 0 ? group_size : static_cast<int>(n);
  const int G = static_cast<int>(n / gs);
  const int T = static_cast<int>((rows + 15) / 16);
  const int C = static_cast<int>(n / kChunk);
  unsigned char* base = static_cast<unsigned char*>(packed);
  uint32_t* flags = reinterpret_cast<uint32_t*>(base);
  uint32_t* Q = reinterpret_cast<uint32_t*>(base + kHeader);
  uint32_t* SZ = reinterpret_cast<uint32_t*>(base + kHeader + align256(static_cast<size_t>(T) * C * 64 * bits * 4));
  hipError_t e = zero_words(flags, 1, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(group_order_kernel, dim3(G), dim3(256), 0, s, g_idx, static_cast<int>(n), gs, col_order, flags);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the order must be a valid grouping before the codes are gathered through it
  if ((e = hipMemcpyAsync(flags_host, flags, sizeof(uint32_t), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  if (*flags_host & 1u) return hipSuccess;
  const int64_t qthreads = static_cast<int64_t>(T) * C * 64;
  const unsigned qblocks = static_cast<unsigned>((qthreads + 255) / 256);
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(qweight);
  const int r32 = static_cast<int>(rows), n32 = static_cast<int>(n);
  switch (bits) {
    case 2: hipLaunchKernelGGL(pack_codes_kernel<2>, dim3(qblocks), dim3(256), 0, s, qw, col_order, r32, n32, T, Q); break;
    case 3: hipLaunchKernelGGL(pack_codes_kernel<3>, dim3(qblocks), dim3(256), 0, s, qw, col_order, r32, n32, T, Q); break;
    case 4: hipLaunchKernelGGL(pack_codes_kernel<4>, dim3(qblocks), dim3(256), 0, s, qw, col_order, r32, n32, T, Q); break;
    case 8: hipLaunchKernelGGL(pack_codes_kernel<8>, dim3(qblocks), dim3(256), 0, s, qw, col_order, r32, n32, T, Q); break;
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int gsk = group_size > 0 ? group_size : 0;
  const int Cs = group_size > 0 ? C : 1;
  const int64_t zthreads = static_cast<int64_t>(T) * G * 16;   // = T * Cs * 16 * spc
  hipLaunchKernelGGL(pack_sz_kernel, dim3(static_cast<unsigned>((zthreads + 255) / 256)), dim3(256), 0, s, scales,
                     zeros, r32, G, gsk, T, Cs, SZ);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

size_t matmul_workspace_bytes(int64_t M, int64_t n) { return align256(static_cast<size_t>(M * n) * 2); }

// Library-owned scratch of the allocation-free matmul entry point: the
// gathered activations of act-order layers.  One copy per device, at its own
// address on each, held until the process ends.
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

size_t matmul_static_scratch_bytes() { return kStaticScratchBytes; }

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.  In host
// code the array's name is only a stand-in for the device symbol: it is never
// passed to a kernel or a copy; the looked-up address is.
hipError_t matmul_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices] = {};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_matmul(const void* A, int64_t M, int64_t lda, const void* packed, const int32_t* col_order,
                         int64_t rows, int64_t n, int bits, int group_size, void* Y, int ydt, int64_t ldy,
                         void* ws, hipStream_t s) {
  const int gs = group_size > 0 ? group_size : 0;
  const int T = static_cast<int>((rows + 15) / 16);
  const int C = static_cast<int>(n / kChunk);
  const unsigned char* base = static_cast<const unsigned char*>(packed);
  const uint32_t* Q = reinterpret_cast<const uint32_t*>(base + kHeader);
  const uint32_t* SZ =
      reinterpret_cast<const uint32_t*>(base + kHeader + align256(static_cast<size_t>(T) * C * 64 * bits * 4));
  const uint16_t* a = static_cast<const uint16_t*>(A);
  if (col_order) {
    uint16_t* at = static_cast<uint16_t*>(ws);
    if (n <= kGatherLdsMax) {
      const bool vec = (reinterpret_cast<uintptr_t>(a) & 15) == 0 && lda % 8 == 0;
      const unsigned blocks = static_cast<unsigned>(M < 2048 ? M : 2048);
      const size_t lds = static_cast<size_t>(n) * 2;
      if (vec)
        hipLaunchKernelGGL(gather_rows_kernel<true>, dim3(blocks), dim3(256), lds, s, a, lda, col_order,
                           static_cast<int>(M), static_cast<int>(n), at);
      else
        hipLaunchKernelGGL(gather_rows_kernel<false>, dim3(blocks), dim3(256), lds, s, a, lda, col_order,
                           static_cast<int>(M), static_cast<int>(n), at);
    } else {
      unsigned gx = static_cast<unsigned>((n + 255) / 256);
      if (gx > 64) gx = 64;
      const unsigned gy = static_cast<unsigned>(M < 1024 ? M : 1024);
      hipLaunchKernelGGL(gather_cols_kernel, dim3(gx, gy), dim3(256), 0, s, a, lda, col_order, static_cast<int>(M),
                         static_cast<int>(n), at);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a = at;
    lda = n;
  }
  const int m = static_cast<int>(M), r = static_cast<int>(rows), nn = static_cast<int>(n);
#define GPTQ_MM(B)                                                                                    \
  if (bits == B) {                                                                                    \
    if (gs == 32) return launch_mm<B, 4>(a, lda, m, Q, SZ, r, nn, gs, Y, ydt, ldy, s);     \
    if (gs == 64) return launch_mm<B, 2>(a, lda, m, Q, SZ, r, nn, gs, Y, ydt, ldy, s);     \
    return launch_mm<B, 1>(a, lda, m, Q, SZ, r, nn, gs, Y, ydt, ldy, s);                   \
  }
  GPTQ_MM(2)
  GPTQ_MM(3)
  GPTQ_MM(4)
  GPTQ_MM(8)
#undef GPTQ_MM
  return hipErrorInvalidValue;
}

}  // namespace gptq
