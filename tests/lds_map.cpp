// Lane -> LDS address maps of the attention kernels' tile accesses, printed for the host-side bank
// check in test_lds_layout.py.  Every address comes from the kernels' own layout header
// (csrc/lds_layout.h); this program only enumerates instructions and lanes.
//
// Output lines (whitespace separated):
//   T name kind row_bytes rows data_bytes tile_bytes   start of a tile
//   C row byte offset                                   every 16-byte chunk of every row
//   D row0 ks a0 .. a63                                  16-byte operand read (lanes 0..63)
//   R row0 c db h a0 .. a63                              8-byte transposing read
//   Q row0 h a0 .. a63                                   8-byte transposing read, 16-column form
//   S threads step wave a0 .. a63                        16-byte tile store
// With arguments `probe FORM KIND ROW_BYTES DATA_BYTES` it prints instead the instructions of one
// pattern of the LDS microbenchmark (P line, then D / R / S lines); with `rows`, the tile row each
// lane reads in the transposing forms (W16 lane h row byte, W32 lane c h row).
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include <string>

#include "lds_layout.h"

using namespace attn::lds;

namespace {

constexpr int kRows = 64;

// tail16: the last 16 columns (d = 16 modulo 32) are read with the 16-column form instead of
// 32-column reads that reach zero columns up to dp.
void tile(const char* name, int kind, int rb, int d, bool direct, bool trans, bool tail16 = false) {
  const int dp = dp_for(d);
  const int data = 2 * d;  // bytes of data per row (bfloat16)
  std::printf("T %s %d %d %d %d %d\n", name, kind, rb, kRows, data, tile_bytes(kind, rb, kRows));
  const int cols = trans && !tail16 ? 2 * dp : data;  // 32-column reads reach the zero columns up to dp
  for (int r = 0; r < kRows; ++r)
    for (int b = 0; b < cols; b += 16) std::printf("C %d %d %d\n", r, b, offset(kind, rb, r, b));
  if (direct)
    for (int row0 = 0; row0 < kRows; row0 += 32)
      for (int ks = 0; ks < d / 16; ++ks) {
        std::printf("D %d %d", row0, ks);
        for (int l = 0; l < 64; ++l) std::printf(" %d", offset(kind, rb, row0 + direct_row(l), direct_byte(l, 16 * ks)));
        std::printf("\n");
      }
  if (trans)
    for (int row0 = 0; row0 < kRows; row0 += 32)
      for (int c = 0; c < 2; ++c)
        for (int db = 0; db < (tail16 ? d / 32 : dp / 32); ++db)
          for (int h = 0; h < 2; ++h) {
            std::printf("R %d %d %d %d", row0, c, db, h);
            for (int l = 0; l < 64; ++l)
              std::printf(" %d", offset(kind, rb, row0 + trans_row(l, c, h), trans_byte(l, 32 * db)));
            std::printf("\n");
          }
  if (trans && tail16)
    for (int row0 = 0; row0 < kRows; row0 += 32)
      for (int h = 0; h < 2; ++h) {
        std::printf("Q %d %d", row0, h);
        for (int l = 0; l < 64; ++l)
          std::printf(" %d", offset(kind, rb, row0 + trans16_row(l, h), trans16_byte(l, 32 * (d / 32))));
        std::printf("\n");
      }
  const int cpr = data / 16;
  for (int nt : {256, 512})
    for (int step = 0; step * nt < kRows * cpr; ++step)
      for (int w = 0; w < nt / 64; ++w) {
        std::printf("S %d %d %d", nt, step, w);
        for (int l = 0; l < 64; ++l) {
          const int c = w * 64 + l + step * nt;
          std::printf(" %d", c < kRows * cpr ? offset(kind, rb, store_row(c, cpr), store_byte(c, cpr)) : -1);
        }
        std::printf("\n");
      }
}

// The instructions the LDS microbenchmark (microbench/lds_banks.hip) issues for one pattern, in
// its lane formulas: 8 per loop iteration for a wave; stores for all 8 waves of its workgroup.
void probe(int form, int kind, int rb, int db) {
  const int ks_n = db / 32, ndb = (db + 63) / 64, cpr = db / 16;
  std::printf("P %d %d %d %d\n", form, kind, rb, db);
  for (int r = 0; r < 8; ++r) {
    if (form == 0) {
      std::printf("D 0 %d", r);
      for (int l = 0; l < 64; ++l)
        std::printf(" %d", block(kind, rb, 32 * ((r / ks_n) & 1)) + offset(kind, rb, direct_row(l), direct_byte(l, 0)) +
                               32 * (r % ks_n));
      std::printf("\n");
    } else if (form == 1) {
      const int c = r & 1, dbl = (r >> 1) % ndb, blk = ((r >> 1) / ndb) & 1;
      const int tr1 = offset(kind, rb, 8, 0) - offset(kind, rb, 0, 0);
      for (int h = 0; h < 2; ++h) {
        std::printf("R 0 %d %d %d", c, dbl, h);
        for (int l = 0; l < 64; ++l)
          std::printf(" %d", block(kind, rb, 32 * blk + 16 * c) + 64 * dbl +
                                 offset(kind, rb, trans_row(l, 0, 0), trans_byte(l, 0)) + h * tr1);
        std::printf("\n");
      }
    } else if (form == 3) {
      const int tr1 = offset(kind, rb, 8, 0) - offset(kind, rb, 0, 0);
      for (int h = 0; h < 2; ++h) {
        std::printf("Q 0 %d", h);
        for (int l = 0; l < 64; ++l)
          std::printf(" %d", block(kind, rb, 32 * (r & 1)) + offset(kind, rb, trans16_row(l, 0), trans16_byte(l, db / 2 - 16)) +
                                 h * tr1);
        std::printf("\n");
      }
    } else {
      for (int w = 0; w < 8; ++w) {
        std::printf("S 512 %d %d", r, w);
        for (int l = 0; l < 64; ++l) {
          const int c = w * 64 + l + r * 512;
          std::printf(" %d", offset(kind, rb, store_row(c, cpr) % kRows, store_byte(c, cpr)));
        }
        std::printf("\n");
      }
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc == 2 && std::string(argv[1]) == "rows") {  // the row maps of the transposing reads
    for (int l = 0; l < 64; ++l)
      for (int h = 0; h < 2; ++h) {
        std::printf("W16 %d %d %d %d\n", l, h, trans16_row(l, h), trans16_byte(l, 0));
        for (int c = 0; c < 2; ++c) std::printf("W32 %d %d %d %d\n", l, c, h, trans_row(l, c, h));
      }
    return 0;
  }
  if (argc == 6) {  // probe FORM KIND ROW_BYTES DATA_BYTES
    probe(std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]));
    return 0;
  }
  char name[64];
  for (int d : {16, 32, 64, 80, 128}) {
    std::snprintf(name, sizeof name, "stage_d%d", d);
    tile(name, stage_kind(2, d), stage_row_bytes(2, d), d, true, true, d % 32 == 16);
    std::snprintf(name, sizeof name, "fwdK_d%d", d);
    tile(name, kPadded, padded_pitch(2 * dp_for(d)), d, true, false);
    std::snprintf(name, sizeof name, "fwdV_d%d", d);
    tile(name, trans_kind(2, d), trans_row_bytes(2, d), d, false, true, d % 32 == 16);
  }
  return 0;
}
