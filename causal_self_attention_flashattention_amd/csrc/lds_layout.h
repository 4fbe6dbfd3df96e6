// LDS tile layouts and the lane -> address maps of the fragment reads (gfx950), as plain constexpr
// integer arithmetic so that the same functions serve the kernels and a host-side check of their
// bank behaviour.
//
// Bank model (gfx950, measured with SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE on single-pattern
// probes): 64 banks of 4 bytes.  A 16-byte-per-lane read is served 16 lanes at a time (lanes
// 16p .. 16p + 15) and is conflict-free when those lanes' 16-byte chunks fall in distinct 16-byte
// slots modulo 256 bytes.  A transposing 8-byte read (ds_read_b64_tr_b16) is served 32 lanes at a
// time and is conflict-free when those lanes' 8-byte words fall in distinct 8-byte slots modulo
// 256 bytes.  A 16-byte store is served 8 lanes at a time, with 16-byte chunks modulo 128 bytes.
// A conflict of degree k costs k - 1 extra cycles per pass.
//
// Tiles hold rows of bfloat16 (or float32) values.  Three layouts:
//  * padded: row r at r * P bytes, P = the row's data bytes plus padding (lds_pitch,
//    lds_pitch_tr);
//  * skewed: rows of RB = 128 or 256 bytes in groups of 16, row r of a group shifted by a function
//    of r mod 16.  Rows stay contiguous, so each lane's reads are one register plus an
//    immediate offset;
//  * skewed for transposing reads only: 128-byte rows, row r shifted by 64 (r / 4 + (r / 2) mod 2)
//    bytes (144 bytes per row on average, as the padded pitch of such rows);
//  * shifted by 16: padded rows whose rows 16-31 of every 32 are shifted by 32 bytes, for the
//    16-column transposing reads (trans16_row), which pair rows 16 apart in one pass.
// A tile read both as 32-row operands (16 bytes per lane) and transposed can be conflict-free for
// both only in the skewed layout: no padded pitch is (a pitch that is an odd number of 16-byte
// chunks suits the first, one that is 64 bytes modulo 128 the second).  Row-contiguous stores are
// conflict-free in every layout whose rows are a multiple of 128 data bytes.
#pragma once

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__
#else
#define ATTN_HD
#endif

namespace attn {
namespace lds {

// Row pitch in bytes of a padded tile whose rows hold `row_bytes` bytes of data (a multiple of 16)
// and are read both ways: an odd number of 16-byte chunks, and not within 16 bytes of a multiple of
// 256 (those pitches were measured slower for the transposing reads than the others).
ATTN_HD constexpr int padded_pitch(int row_bytes) {
  int bytes = row_bytes + 16;
  const int m = bytes % 256;
  if (m == 0 || m == 16 || m == 240) bytes += 32;
  return bytes;
}

// Row pitch in bytes of a padded bfloat16 tile that is only read transposed: 64 modulo 128, where
// every transposing read is conflict-free.
ATTN_HD constexpr int padded_pitch_tr(int row_bytes) {
  int bytes = row_bytes;
  while (bytes % 128 != 64) bytes += 16;
  return bytes;
}

// Layout of a bfloat16 tile read both ways: skewed rows at head dims 64 (128-byte rows) and 128
// (256-byte rows); padded otherwise.  (Skewed 192-byte rows for d = 80 are defined below too; the
// d = 80 backward kernels measured slower with them than with padded rows.)
enum Kind { kPadded = 0, kSkewed = 1, kSkewTr = 2, kShift16 = 3 };
ATTN_HD constexpr int kind_for(int elem_bytes, int d) {
  return elem_bytes == 2 && (d == 64 || d == 128) ? kSkewed : kPadded;
}
ATTN_HD constexpr int row_bytes_for(int d) { return d <= 64 ? 128 : d <= 96 ? 192 : 256; }

// Shift in bytes of row r (a = bits 2-3 of r) in a skewed tile, and the bytes of a group of 16
// rows.  With it, over 16 consecutive rows from a multiple of 16: (a) a given 16-byte chunk of each
// row lands in 16 different 16-byte slots modulo 256 bytes (32-row operand reads), and (b) 4
// consecutive rows from a multiple of 4 place the 4 chunks 4u .. 4u + 3 of each row in 16
// different slots (transposing reads).  Rows do not overlap.
//  * 256-byte rows: 64 (r mod 4) + 208 a.  Row r = 4a + i sits in slot 4i + 13a (mod 16): 4i
//    spreads 4 consecutive rows over disjoint groups of 4 slots (b), and 13a takes the 4 values of a
//    to 4 different residues modulo 4 (a).  The 208-byte step clears the previous 4 rows' shifts.
//  * 192-byte rows: 16 a.  Rows start at 0, 192, 128, 64 modulo 256 bytes with period 4, which
//    gives (b) and a different group of 4 slots to each of 4 consecutive rows; the shift separates
//    the 4 rows that share a group (a).
//  * 128-byte rows (two rows per 256 bytes): 64 (bit 1 of r) + 80 a.  Rows 4a .. 4a + 3 start at
//    slots 0, 8, 4, 12 plus 5a: (b), and 5a has 4 different residues modulo 4: (a).
ATTN_HD constexpr int skew(int rb, int r) {
  return rb == 256 ? 64 * (r & 3) + 208 * ((r >> 2) & 3)
         : rb == 192 ? 16 * ((r >> 2) & 3)
                     : 64 * ((r >> 1) & 1) + 80 * ((r >> 2) & 3);
}
ATTN_HD constexpr int skew_group_bytes(int rb) { return rb == 256 ? 4928 : rb == 192 ? 3136 : 2368; }

// The kernels' tiles, by element size and head dim d (dp = d rounded up to 32 columns):
//  * stage tiles, read both ways (dK/dV's Q and dO, dQ's K and V): skewed where kind_for says so,
//    else padded at padded_pitch;
//  * forward K tiles (32-row operand reads only): padded at padded_pitch;
//  * forward V tiles (transposing reads only): kSkewTr for bfloat16 at d = 64; for bfloat16 at
//    d = 80, whose last 16 columns take the 16-column reads, kShift16 with rows at padded_pitch_tr
//    (192 bytes: 160 of data, room for the shift); padded at padded_pitch_tr above d = 64 and at
//    padded_pitch below.
ATTN_HD constexpr int dp_for(int d) { return (d + 31) / 32 * 32; }
ATTN_HD constexpr int stage_kind(int elem_bytes, int d) { return kind_for(elem_bytes, d); }
ATTN_HD constexpr int stage_row_bytes(int elem_bytes, int d) {
  return kind_for(elem_bytes, d) != kPadded ? row_bytes_for(d) : padded_pitch(dp_for(d) * elem_bytes);
}
ATTN_HD constexpr int trans_kind(int elem_bytes, int d) {
  return elem_bytes == 2 && d == 64 ? kSkewTr : elem_bytes == 2 && d == 80 ? kShift16 : kPadded;
}
ATTN_HD constexpr int trans_row_bytes(int elem_bytes, int d) {
  return trans_kind(elem_bytes, d) == kSkewTr ? 128
         : dp_for(d) > 64 && elem_bytes == 2 ? padded_pitch_tr(dp_for(d) * elem_bytes)
                                             : padded_pitch(dp_for(d) * elem_bytes);
}

// Transposing reads only, 128-byte rows: rows 4a .. 4a + 3 start at 16-byte slots 0, 8, 4, 12 plus
// 4a modulo 16, so the 4 chunks 4u .. 4u + 3 of the 4 rows fill 16 different slots: (b).
ATTN_HD constexpr int skew_tr(int r) { return 64 * ((r >> 2) + ((r >> 1) & 1)); }

// Byte offset of byte b of row r of a tile of the given layout with rows of rb bytes.  (kShift16:
// a row's data plus the shift fit its rb bytes, so rows do not overlap.)
ATTN_HD constexpr int offset(int kind, int rb, int r, int b) {
  return kind == kSkewed  ? (r >> 4) * skew_group_bytes(rb) + (r & 15) * rb + skew(rb, r) + b
         : kind == kSkewTr ? r * rb + skew_tr(r) + b
         : kind == kShift16 ? r * rb + 32 * ((r >> 4) & 1) + b
                            : r * rb + b;
}
// Byte offset of row r0 (a multiple of 16; of 32 for kShift16 reads that span rows r0 + 16 ..):
// row r0 + r, r < 16, lies at block(r0) + offset(r, b).
ATTN_HD constexpr int block(int kind, int rb, int r0) {
  return kind == kSkewed    ? (r0 >> 4) * skew_group_bytes(rb)
         : kind == kSkewTr  ? r0 * rb + 16 * r0
         : kind == kShift16 ? r0 * rb + 32 * ((r0 >> 4) & 1)
                            : r0 * rb;
}
// Bytes of a tile of `rows` rows (a multiple of 16 for the skewed layouts).
ATTN_HD constexpr int tile_bytes(int kind, int rb, int rows) {
  return kind == kSkewed ? (rows + 15) / 16 * skew_group_bytes(rb) : kind == kSkewTr ? rows * (rb + 16) : rows * rb;
}

// Lane maps of the bfloat16 operand reads (lane layouts of v_mfma_f32_32x32x16_bf16).
// 32 x 16 operand whose rows are tile rows, reduction along a row from column col0: lane l reads
// the 16 bytes at row (l % 32), column col0 + 8 (l / 32).
ATTN_HD constexpr int direct_row(int lane) { return lane & 31; }
ATTN_HD constexpr int direct_byte(int lane, int col0) { return 2 * (col0 + 8 * (lane >> 5)); }
// 32-column operand whose reduction runs down tile rows in accumulator row order, instruction c of a
// 32-row block: two transposing reads h = 0, 1; in each, lane l (group g = l / 16, j = l % 16) reads
// the 8 bytes at row 16c + 8h + 4(g / 2) + j / 4, column col0 + 16(g % 2) + 4(j % 4).
ATTN_HD constexpr int trans_row(int lane, int c, int h) {
  return 16 * c + 8 * h + 4 * ((lane >> 4) >> 1) + ((lane & 15) >> 2);
}
ATTN_HD constexpr int trans_byte(int lane, int col0) { return 2 * (col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)); }
// 16-column operand of v_mfma_f32_16x16x32_bf16 (16 tile columns, reduction over the 32 rows of a
// block): two transposing reads h = 0, 1; lane l (group g = l / 16, j = l % 16) reads the 8 bytes at
// row 16(g % 2) + 8h + 4(g / 2) + j / 4, column col0 + 4(j % 4).  Lane group g thus walks the rows
// that instruction c = g % 2 of the 32-column form gives to lane half g / 2.
ATTN_HD constexpr int trans16_row(int lane, int h) { return trans_row(lane, (lane >> 4) & 1, h); }
ATTN_HD constexpr int trans16_byte(int lane, int col0) { return 2 * (col0 + 4 * (lane & 3)); }
// Cooperative 16-byte stores of a tile (TileCopy): chunk c = thread + i * threads goes to row
// c / (chunks per row), byte 16 (c % chunks per row).
ATTN_HD constexpr int store_row(int c, int chunks_per_row) { return c / chunks_per_row; }
ATTN_HD constexpr int store_byte(int c, int chunks_per_row) { return 16 * (c % chunks_per_row); }

}  // namespace lds
}  // namespace attn
