// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4 only).
//
// Matrix products run on the 32x32 MFMA shapes: v_mfma_f32_32x32x16_bf16 for bf16 operands and
// v_mfma_f32_32x32x2_f32 for fp32 operands, always accumulating in fp32.  Lane layouts (wave64):
//   A operand (32 x K):  lane l holds A[l % 32][KPL * (l / 32) + s], s < KPL
//   B operand (K x 32):  lane l holds B[KPL * (l / 32) + s][l % 32]
//   accumulator (32x32): lane l, element e holds C[8 * (e / 4) + 4 * (l / 32) + e % 4][l % 32]
// with KPL = 8 (bf16, K = 16) or 1 (fp32, K = 2).
//
// An accumulator can be fed back as the B operand of a product that reduces over its rows:
// each lane already owns one column.  Its rows arrive in a fixed order (see acc_row below), so
// the operand on the other side, read from LDS, must walk the reduction dimension in that same
// order; frag_trans does that.  For bf16 it uses ds_read_b64_tr_b16: inside each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte chunks read by lanes 4e + i / 4, e < 4,
// i.e. a 4 x 16 block of a row-major tile comes back as 16 lanes x 4 rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "block_order.h"
#include "lds_layout.h"

namespace attn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) char lds_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Masked scores are pushed to this value (log2 domain) before exp2, so their weight underflows
// to exactly 0 and a row can never produce inf - inf.
constexpr float kMaskedScore = -1.0e30f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Row (within a 32-row block) held by accumulator element e of lane l.
__device__ __forceinline__ int acc_row(int e, int half) { return 8 * (e >> 2) + 4 * half + (e & 3); }

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  static constexpr int KPL = 8;     // reduction elements per lane per instruction
  static constexpr int KSTEP = 16;  // reduction depth of one instruction
  static constexpr int CALLS32 = 2; // instructions to reduce over a 32-row accumulator block
  using frag = bf16x8;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // 32 x KSTEP operand whose rows are tile rows and whose reduction runs along tile columns.
  // Tile is row-major with a row stride of `ld` elements; `off` is the element offset of
  // (row0, col0).  One 16-byte LDS read per lane.
  __device__ __forceinline__ static frag frag_direct(const lds_t* tile, int ld, int off) {
    const int l = lane_id();
    const int e = off + lds::direct_row(l) * ld + lds::direct_byte(l, 0) / 2;
    return frag_at(tile + 2 * e);
  }
  // 32-column operand whose reduction runs down tile rows in accumulator row order, for the
  // c-th instruction of a 32-row block: slot s of lane l takes tile row
  // 16c + 8(s/4) + 4(l/32) + s%4 and column l % 32 (relative to `off`).
  __device__ __forceinline__ static frag frag_trans(const lds_t* tile, int ld, int off, int c) {
    const int l = lane_id();
    const lds_t* p0 = tile + 2 * (off + lds::trans_row(l, c, 0) * ld + lds::trans_byte(l, 0) / 2);
    return frag_tr_at(p0, p0 + 2 * 8 * ld);
  }
  // The 16 bytes at p as an operand fragment.
  __device__ __forceinline__ static frag frag_at(const lds_t* p) {
    return *reinterpret_cast<const __attribute__((address_space(3))) frag*>(p);
  }
  // The transposing reads at p0 (slots 0-3) and p1 (slots 4-7) as an operand fragment.
  __device__ __forceinline__ static frag frag_tr_at(const lds_t* p0, const lds_t* p1) {
    i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
    i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
    frag f;
    __builtin_memcpy(reinterpret_cast<char*>(&f), &r0, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&f) + 8, &r1, 8);
    return f;
  }
  // Accumulator elements 8c..8c+7, rounded to bf16 (round to nearest even).
  __device__ __forceinline__ static frag acc_frag(const f32x16& a, int c) {
    frag f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = (__bf16)a[8 * c + s];
    return f;
  }
  // acc + the sum of the 8 elements, two per v_dot2 against (1, 1) with fp32 accumulation.
  __device__ __forceinline__ static float frag_sum(const frag& f, float acc) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x2 pr = {f[2 * t], f[2 * t + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
    }
    return acc;
  }
  // Operand straight from global memory (row r of a row-major matrix, columns col0..col0+7).
  __device__ __forceinline__ static frag load_global(const __bf16* rowp, int col0, bool valid) {
    frag f = {};
    if (valid) f = *reinterpret_cast<const frag*>(rowp + col0 + KPL * (lane_id() >> 5));
    return f;
  }

  // 16-wide products for output blocks of 16 rows (the last 16 of a head dim that is 16 modulo 32),
  // v_mfma_f32_16x16x32_bf16: A (16 x 32): lane l holds A[l % 16][8 (l / 16) + s]; B (32 x 16): lane
  // l holds B[8 (l / 16) + s][l % 16]; accumulator (16 x 16): lane l, element e holds
  // C[4 (l / 16) + e][l % 16].
  __device__ __forceinline__ static f32x4 mma16(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // The two B operands of a 32-row accumulator block's weights (p0, p1: acc_frag c = 0, 1) for the
  // 16-wide products over its 32 rows: `lo` for accumulator columns 0-15, `hi` for 16-31.  Lane
  // group g = l / 16 of either holds the rows that acc_frag g % 2 holds in lane half g / 2, which
  // one v_permlane16_swap per register moves into place (rows of 16 lanes: the odd rows of p0 trade
  // places with the even rows of p1).
  __device__ __forceinline__ static void tail_weights(const frag& p0, const frag& p1, frag& lo, frag& hi) {
    const u32x4 a = __builtin_bit_cast(u32x4, p0), b = __builtin_bit_cast(u32x4, p1);
    u32x4 x, y;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto r = __builtin_amdgcn_permlane16_swap(a[k], b[k], false, false);
      x[k] = r[0];
      y[k] = r[1];
    }
    lo = __builtin_bit_cast(frag, x);
    hi = __builtin_bit_cast(frag, y);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  static constexpr int CALLS32 = 16;
  using frag = float;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag frag_direct(const lds_t* tile, int ld, int off) {
    const int l = lane_id();
    const int e = off + (l & 31) * ld + (l >> 5);
    return *reinterpret_cast<const __attribute__((address_space(3))) float*>(tile + 4 * e);
  }
  // Instruction c reduces over accumulator element c: tile row 8(c/4) + 4(l/32) + c%4.
  __device__ __forceinline__ static frag frag_trans(const lds_t* tile, int ld, int off, int c) {
    const int l = lane_id();
    const int row = acc_row(c, l >> 5);
    return *reinterpret_cast<const __attribute__((address_space(3))) float*>(tile + 4 * (off + row * ld + (l & 31)));
  }
  __device__ __forceinline__ static frag acc_frag(const f32x16& a, int c) { return a[c]; }
  __device__ __forceinline__ static float frag_sum(frag f, float acc) { return acc + f; }
  __device__ __forceinline__ static frag load_global(const float* rowp, int col0, bool valid) {
    return valid ? rowp[col0 + (lane_id() >> 5)] : 0.0f;
  }
};

// LDS row pitch (in elements) of a padded tile whose rows hold DP elements of T and are read both
// as 32-row operands and transposed (lds::padded_pitch).
template <typename T, int DP>
constexpr int lds_pitch() {
  return lds::padded_pitch(DP * (int)sizeof(T)) / (int)sizeof(T);
}

// LDS row pitch (in elements) of a tile that is only read with transposing reads (frag_trans):
// lds::padded_pitch_tr for bfloat16; float32 tiles are read with plain 4-byte reads and keep
// lds_pitch.
template <typename T, int DP>
constexpr int lds_pitch_tr() {
  if constexpr (sizeof(T) != 2) {
    return lds_pitch<T, DP>();
  } else {
    return lds::padded_pitch_tr(DP * (int)sizeof(T)) / (int)sizeof(T);
  }
}

// A staged tile of rows of D values of T that is read both as 32-row operands and transposed (the
// Q and dO tiles of the dK/dV kernel, the K and V tiles of the dQ kernel): the layout lds::kind_for
// picks (skewed rows for bfloat16 at d = 64 and 128, where both read forms are conflict-free;
// padded rows, lds_pitch, otherwise).
template <typename T, int D>
struct StageTile {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int KIND = lds::stage_kind((int)sizeof(T), D);
  static constexpr int RB = lds::stage_row_bytes((int)sizeof(T), D);
  static constexpr int LD = RB / (int)sizeof(T);  // row pitch in elements (padded layout)
  static constexpr int bytes(int rows) { return lds::tile_bytes(KIND, RB, rows); }
  __device__ __forceinline__ static int offset(int row, int byte) { return lds::offset(KIND, RB, row, byte); }
  __device__ __forceinline__ static int block(int row0) { return lds::block(KIND, RB, row0); }
};

// A staged tile that is only read transposed (the forward's V tiles): bfloat16 at d = 64 in the
// lds::kSkewTr layout (conflict-free, no larger than padded rows), at d = 80 in lds::kShift16 rows
// of lds_pitch_tr (the 32- and 16-column reads conflict-free), padded at lds_pitch_tr above d = 64
// (conflict-free), and at lds_pitch below.
template <typename T, int D>
struct TransTile {
  static constexpr int DP = (D + 31) / 32 * 32;
  static constexpr int KIND = lds::trans_kind((int)sizeof(T), D);
  static constexpr int RB = lds::trans_row_bytes((int)sizeof(T), D);
  static constexpr int LD = RB / (int)sizeof(T);
  static constexpr int bytes(int rows) { return lds::tile_bytes(KIND, RB, rows); }
  __device__ __forceinline__ static int offset(int row, int byte) { return lds::offset(KIND, RB, row, byte); }
  __device__ __forceinline__ static int block(int row0) { return lds::block(KIND, RB, row0); }
};

// Operand reads from StageTile / TransTile tiles (S).  In the skewed layouts each lane's offsets
// within a 16-row-aligned block depend only on the lane, so they are computed once (one register
// per read form) and every read is a register plus an immediate; padded tiles use the plain reads.
template <typename T, class S>
struct TileReader {
  using M = Mfma<T>;
  static constexpr bool SKEW = S::KIND != lds::kPadded;
  // The second transposing read of a fragment is 8 rows below the first, at a lane-independent
  // distance (rows 0-7 and 8-15 of a group differ by the same shift).
  static constexpr int TR1 = lds::offset(S::KIND, S::RB, 8, 0) - lds::offset(S::KIND, S::RB, 0, 0);
  int dir = 0, tr0 = 0, t16 = 0;
  __device__ __forceinline__ TileReader(bool with16 = false) {
    const int l = lane_id();
    if constexpr (SKEW) {
      if constexpr (S::KIND == lds::kSkewed) dir = S::offset(lds::direct_row(l), lds::direct_byte(l, 0));
      tr0 = S::offset(lds::trans_row(l, 0, 0), lds::trans_byte(l, 0));
    }
    if (with16) t16 = S::offset(lds::trans16_row(l, 0), lds::trans16_byte(l, 0));
  }
  // 32 x KSTEP operand of tile rows row0 .. row0 + 31 (row0 a multiple of 16), reduction step ks.
  __device__ __forceinline__ typename M::frag direct(const lds_t* tile, int row0, int ks) const {
    static_assert(S::KIND != lds::kSkewTr && S::KIND != lds::kShift16, "transposing reads only");
    if constexpr (SKEW) return M::frag_at(tile + S::block(row0) + dir + 2 * ks * M::KSTEP);
    else return M::frag_direct(tile, S::LD, row0 * S::LD + ks * M::KSTEP);
  }
  // Transposed operand of the 32-row block at row0 (a multiple of 16), columns 32 db .., instruction c.
  __device__ __forceinline__ typename M::frag trans(const lds_t* tile, int row0, int db, int c) const {
    if constexpr (SKEW) {
      const lds_t* b = tile + S::block(row0 + 16 * c) + 64 * db + tr0;
      return M::frag_tr_at(b, b + TR1);
    } else {
      return M::frag_trans(tile, S::LD, row0 * S::LD + db * 32, c);
    }
  }
  // A operand of Mfma<__bf16>::mma16 over the 32-row block at row0 (a multiple of 32) and tile
  // columns col0 .. col0 + 15, rows in the order of Mfma<__bf16>::tail_weights (the reader must be
  // constructed with with16).
  __device__ __forceinline__ typename M::frag trans16(const lds_t* tile, int row0, int col0) const {
    const lds_t* b = tile + S::block(row0) + t16 + 2 * col0;
    return M::frag_tr_at(b, b + TR1);
  }
};
template <typename T, int D>
using StageReader = TileReader<T, StageTile<T, D>>;

// Exchange a value with the lane 32 positions away (lanes l and l ^ 32 hold the two halves of
// an accumulator column).
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((lane_id() < 32) ? r[1] : r[0]);
}

// From a per-lane value of query (column) l % 32, the values of columns l % 16 (lo) and 16 + l % 16
// (hi): the per-column factors of 16-wide accumulators.
__device__ __forceinline__ void split16(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Raw buffer resource over `bytes` bytes at `base`: loads at offsets >= bytes return zero, which
// is how rows past the end of a sequence (or past the key length) come in as zeros without a
// branch.  Word 3 is the gfx9-family default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Cooperative copy of a ROWS x COLS tile (row-major, global row stride = COLS elements) into LDS
// with row stride LD, 16 bytes per thread per step, through registers so the global latency can
// hide behind compute.  Rows outside the resource read as zero.
template <typename T, int ROWS, int COLS, int LD, int NTHREADS>
struct TileCopy {
  static constexpr int CPR = COLS * (int)sizeof(T) / 16;  // 16-byte chunks per row
  static constexpr int CHUNKS = ROWS * CPR;
  static constexpr int PER_THREAD = (CHUNKS + NTHREADS - 1) / NTHREADS;
  static_assert(COLS * sizeof(T) % 16 == 0, "tile rows must be a multiple of 16 bytes");
  u32x4 r[PER_THREAD];

  // Load the tile whose first row is `row0` of the matrix behind `rs`.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int row0) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      const int row = c / CPR, cc = c % CPR;
      if (CHUNKS % NTHREADS == 0 || c < CHUNKS)
        r[i] = buffer_load16(rs, (uint32_t)((row0 + row) * COLS * (int)sizeof(T) + cc * 16));
    }
  }
  __device__ __forceinline__ void store(lds_t* tile) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (CHUNKS % NTHREADS == 0 || c < CHUNKS) {
        const int row = lds::store_row(c, CPR);
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(tile + (row * LD) * (int)sizeof(T) +
                                                                    lds::store_byte(c, CPR)) = r[i];
      }
    }
  }
  // Store into a tile laid out as S (a StageTile).
  template <class S>
  __device__ __forceinline__ void store_to(lds_t* tile) const {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = threadIdx.x + i * NTHREADS;
      if (CHUNKS % NTHREADS == 0 || c < CHUNKS)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
            tile + S::offset(lds::store_row(c, CPR), lds::store_byte(c, CPR))) = r[i];
    }
  }
};

// MFMA operand of `Mfma<T>` read straight from global memory through a buffer resource: row `row`
// of a row-major matrix with `cols` columns, reduction columns col0.. (zero if out of range).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_global(__amdgpu_buffer_rsrc_t rs, int row, int cols, int col0) {
  const uint32_t off = (uint32_t)((row * cols + col0 + Mfma<T>::KPL * (lane_id() >> 5)) * (int)sizeof(T));
  if constexpr (sizeof(T) == 2) {
    u32x4 v = buffer_load16(rs, off);
    typename Mfma<T>::frag f;
    __builtin_memcpy(&f, &v, 16);
    return f;
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0));
  }
}

// Sum of elementwise products of two MFMA operand fragments, in fp32 with one fused multiply-add
// per element in fragment order.  The D pre-pass and the dQ kernel both reduce a row of O o dO with
// it, fragment by fragment in the same order, so their D values agree bitwise.
__device__ __forceinline__ float frag_dot(const bf16x8& a, const bf16x8& b, float acc) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = __builtin_fmaf((float)a[t], (float)b[t], acc);
  return acc;
}
__device__ __forceinline__ float frag_dot(float a, float b, float acc) { return __builtin_fmaf(a, b, acc); }

// Zero the columns [COLS, LDZ) of every row of a tile (padding read by 32-wide operand blocks
// when the head dim is not a multiple of 32).
template <typename T, int ROWS, int COLS, int LD, int LDZ, int NTHREADS>
__device__ __forceinline__ void zero_pad_cols(lds_t* tile) {
  if constexpr (LDZ > COLS) {
    constexpr int W = LDZ - COLS;
    for (int i = threadIdx.x; i < ROWS * W; i += NTHREADS) {
      const int row = i / W, col = COLS + i % W;
      *reinterpret_cast<__attribute__((address_space(3))) T*>(tile + (row * LD + col) * (int)sizeof(T)) = T(0);
    }
  }
}

// zero_pad_cols for a tile laid out as S (a StageTile): columns [D, DP) of ROWS rows.
template <class S, typename T, int ROWS, int D, int NTHREADS>
__device__ __forceinline__ void zero_pad_stage(lds_t* tile) {
  if constexpr (S::DP > D) {
    constexpr int W = S::DP - D;
    for (int i = threadIdx.x; i < ROWS * W; i += NTHREADS) {
      const int row = i / W, col = D + i % W;
      *reinterpret_cast<__attribute__((address_space(3))) T*>(tile + S::offset(row, col * (int)sizeof(T))) = T(0);
    }
  }
}

// Wait, outside any loop, until registers filled by global loads have arrived.  Without it the
// compiler may place the vector-memory wait for them inside the following loop, where in-order
// counting makes it also wait for every tile prefetch issued since -- exposing a full memory
// latency per iteration.
template <typename F>
__device__ __forceinline__ void settle(const F& f) { asm volatile("" ::"v"(f)); }

// ------------------------------------------------------------------------------------------
// Block-sparse masks.  A mask is uint8 [TB][TB], TB = ceil(N / kMaskBlock), row-major, shared by
// every (batch, head): entry (r, c) non-zero lets queries [64r, 64r + 64) attend keys
// [64c, 64c + 64).  Every kernel tile lies inside one mask block along each dimension (tiles of
// 32 or 64 rows, 64-aligned workgroup ranges), so each wave can skip a whole tile.
constexpr int kMaskBlock = 64;
constexpr int kMaxMaskBlocks = 1024;  // block-sparse calls need N <= 64 * kMaxMaskBlocks

// A workgroup's view of the mask, one byte per mask block along the dimension it loops over:
// bit j says whether the j-th mask block along its own dimension (j < 8) may meet that block.
// `owned0` is the workgroup's first mask block along its own dimension, `nowned` how many it
// spans; `by_row` selects whether the loop runs over mask columns (forward, dQ: the workgroup owns
// query rows) or over mask rows (dK/dV: it owns key columns).
__device__ __forceinline__ void build_tile_map(lds_t* map, const uint8_t* __restrict__ bmask, int tb, int owned0,
                                               int nowned, bool by_row, int nthreads) {
  for (int t = threadIdx.x; t < tb; t += nthreads) {
    unsigned bits = 0;
    for (int j = 0; j < nowned; ++j) {
      const int o = owned0 + j;
      if (o < tb) {
        const uint8_t v = by_row ? bmask[(size_t)t * tb + o] : bmask[(size_t)o * tb + t];
        bits |= (v != 0 ? 1u : 0u) << j;
      }
    }
    reinterpret_cast<__attribute__((address_space(3))) uint8_t*>(map)[t] = (uint8_t)bits;
  }
}

// Bits of the map entry for loop tile t (tiles of 64 >> shift rows along the loop dimension).
__device__ __forceinline__ unsigned tile_bits(const lds_t* map, int t, int shift) {
  return reinterpret_cast<const __attribute__((address_space(3))) uint8_t*>(map)[t >> shift];
}

// Smallest loop tile index t in [from, end) whose map entry is non-zero, or end.  Each wave scans
// 64 candidates per step with a ballot, so the answer is the same in every wave.
__device__ __forceinline__ int next_live_tile(const lds_t* map, int from, int end, int shift) {
  for (int base = from; base < end; base += 64) {
    const int t = base + lane_id();
    const bool live = t < end && tile_bits(map, t, shift) != 0;
    const unsigned long long m = __ballot(live);
    if (m) return base + __builtin_ctzll(m);
  }
  return end;
}

}  // namespace attn
