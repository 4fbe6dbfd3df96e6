// LDS access rates of the attention kernels' tile layouts on gfx950, one access pattern per launch.
//
// Each pattern is one instruction form (16-byte operand read, transposing 8-byte read pair in the
// 32- or the 16-column form, 16-byte tile store) applied to one tile layout from lds_layout.h, with
// the lane addresses the kernels use.  Every launch runs 256 workgroups of 8 waves; each wave issues 8 x 2048 instructions of the
// pattern against a tile of 64 rows, with all addresses computed before the timed loop.  Run it
// under `rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS GRBM_GUI_ACTIVE` to
// see the bank-conflict cycles of each pattern (one dispatch per pattern, named by its template
// arguments: instruction form, layout kind, row bytes, chunks per stored row).
//
// Output: one line per pattern with its time and bytes moved per clock per CU (at the clock given
// with --ghz, default 2.0).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../csrc/lds_layout.h"

namespace {

typedef __attribute__((address_space(3))) char lds_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

constexpr int kIters = 2048;
constexpr int kTileRows = 64;
constexpr int kLdsBytes = 65536;

enum Form { kDirect = 0, kTrans = 1, kStore = 2, kTrans16 = 3 };

// Byte size of a 64-row tile of the layout (kept below a third of the array: waves use 3 tiles).
constexpr int tile_bytes(int kind, int rb) { return attn::lds::tile_bytes(kind, rb, kTileRows); }

// FORM on a 64-row tile of layout (KIND, RB) whose rows hold DB data bytes (CPR = DB / 16 chunks).
template <int FORM, int KIND, int RB, int DB>
__global__ __launch_bounds__(512) void pattern(float* out) {
  namespace L = attn::lds;
  static_assert(3 * tile_bytes(KIND, RB) <= kLdsBytes, "three tiles fit in the array");
  constexpr int CPR = DB / 16;      // 16-byte chunks per row
  constexpr int KS = DB / 32;       // operand reads per 32-row block (16 columns each)
  constexpr int NDB = (DB + 63) / 64;  // 32-column blocks per row
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  for (int i = threadIdx.x; i < kLdsBytes / 16; i += 512)
    reinterpret_cast<__attribute__((address_space(3))) u32x4*>((lds_t*)smem)[i] = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  lds_t* tile = (lds_t*)smem + (w % 3) * tile_bytes(KIND, RB);
  unsigned x = 0;
  if constexpr (FORM == kDirect) {
    const int base = L::offset(KIND, RB, L::direct_row(l), L::direct_byte(l, 0));
    for (int it = 0; it < kIters; ++it) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const lds_t* p = tile + L::block(KIND, RB, 32 * ((r / KS) & 1)) + base + 32 * (r % KS);
        const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
        x ^= v[0] ^ v[3];
      }
    }
  } else if constexpr (FORM == kTrans) {
    constexpr int TR1 = L::offset(KIND, RB, 8, 0) - L::offset(KIND, RB, 0, 0);
    const int base = L::offset(KIND, RB, L::trans_row(l, 0, 0), L::trans_byte(l, 0));
    for (int it = 0; it < kIters; ++it) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int c = r & 1, db = (r >> 1) % NDB, blk = ((r >> 1) / NDB) & 1;
        const lds_t* p0 = tile + L::block(KIND, RB, 32 * blk + 16 * c) + 64 * db + base;
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0 + TR1));
        x ^= (unsigned)(r0[0] ^ r1[3]);
      }
    }
  } else if constexpr (FORM == kTrans16) {
    // The 16-column form on the last 16 columns of the row's data (bytes DB - 32 .. DB - 1), both
    // 32-row blocks in turn.
    constexpr int TR1 = L::offset(KIND, RB, 8, 0) - L::offset(KIND, RB, 0, 0);
    const int base = L::offset(KIND, RB, L::trans16_row(l, 0), L::trans16_byte(l, DB / 2 - 16));
    for (int it = 0; it < kIters; ++it) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        // only two addresses: kept opaque so that every read is issued
        int b = base;
        asm volatile("" : "+v"(b));
        const lds_t* p0 = tile + L::block(KIND, RB, 32 * (r & 1)) + b;
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0 + TR1));
        x ^= (unsigned)(r0[0] ^ r1[3]);
      }
    }
  } else {
    // A tile store as the kernels' TileCopy issues it: chunk c of the 512 threads' i-th step goes to
    // row c / CPR, byte 16 (c % CPR); the 8 steps per iteration cover 8 x 512 chunks, folded into
    // the tile's 64 rows.
    int a[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int c = (int)threadIdx.x + r * 512;
      a[r] = L::offset(KIND, RB, L::store_row(c, CPR) % kTileRows, L::store_byte(c, CPR));
    }
    const u32x4 v = {(unsigned)l, (unsigned)w, 7u, 9u};
    for (int it = 0; it < kIters; ++it) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 8; ++r)  // volatile: steps that fold onto the same row are all issued
        *reinterpret_cast<volatile __attribute__((address_space(3))) u32x4*>(tile + a[r]) = v;
    }
    __syncthreads();
    x = *reinterpret_cast<const __attribute__((address_space(3))) unsigned*>(tile + 4 * l);
  }
  out[blockIdx.x * 512 + threadIdx.x] = (float)x;
}

double g_ghz = 2.0;

template <int FORM, int KIND, int RB, int DB>
void run(const char* tile, float* out) {
  hipEvent_t e0, e1;
  hipEventCreate(&e0);
  hipEventCreate(&e1);
  hipLaunchKernelGGL((pattern<FORM, KIND, RB, DB>), dim3(256), dim3(512), 0, 0, out);  // warm-up
  hipEventRecord(e0);
  hipLaunchKernelGGL((pattern<FORM, KIND, RB, DB>), dim3(256), dim3(512), 0, 0, out);
  hipEventRecord(e1);
  hipEventSynchronize(e1);
  float ms = 0.f;
  hipEventElapsedTime(&ms, e0, e1);
  // bytes per instruction per wave: 1 KB (16-byte forms), 2 x 512 B (transposing pair)
  const double bytes = 8.0 * kIters * 256 * 8 * 1024;
  const double tbs = bytes / (ms * 1e-3) / 1e12;
  static const char* forms[] = {"direct16", "trans8x2", "store16", "trans16x2"};
  static const char* kinds[] = {"padded", "skewed", "skew_tr", "shift16"};
  static_assert(FORM >= 0 && FORM < 4 && KIND >= 0 && KIND < 4, "named form and layout");
  printf("%-34s %-9s %-8s row_bytes=%3d data_bytes=%3d  %7.3f ms  %6.1f B/clk/CU\n", tile, forms[FORM], kinds[KIND], RB,
         DB, ms, tbs * 1e12 / 256 / (g_ghz * 1e9));
  hipEventDestroy(e0);
  hipEventDestroy(e1);
}

}  // namespace

int main(int argc, char** argv) {
  using namespace attn::lds;
  for (int i = 1; i + 1 < argc; ++i)
    if (!strcmp(argv[i], "--ghz")) g_ghz = atof(argv[i + 1]);
  float* out = nullptr;
  if (hipMalloc(&out, 256 * 512 * sizeof(float)) != hipSuccess) return 1;
  // Stage tiles (read both ways), as the kernels lay them out now.
  constexpr int S128 = stage_row_bytes(2, 128), S64 = stage_row_bytes(2, 64), S80 = stage_row_bytes(2, 80);
  run<kDirect, stage_kind(2, 128), S128, 256>("stage tile d=128", out);
  run<kTrans, stage_kind(2, 128), S128, 256>("stage tile d=128", out);
  run<kStore, stage_kind(2, 128), S128, 256>("stage tile d=128", out);
  run<kDirect, stage_kind(2, 64), S64, 128>("stage tile d=64", out);
  run<kTrans, stage_kind(2, 64), S64, 128>("stage tile d=64", out);
  run<kStore, stage_kind(2, 64), S64, 128>("stage tile d=64", out);
  run<kDirect, stage_kind(2, 80), S80, 160>("stage tile d=80", out);
  run<kTrans, stage_kind(2, 80), S80, 128>("stage tile d=80", out);
  run<kTrans16, stage_kind(2, 80), S80, 160>("stage tile d=80", out);
  run<kStore, stage_kind(2, 80), S80, 160>("stage tile d=80", out);
  // The same tiles at the padded pitch they had before (both read forms).
  run<kDirect, kPadded, padded_pitch(256), 256>("padded stage tile d=128", out);
  run<kTrans, kPadded, padded_pitch(256), 256>("padded stage tile d=128", out);
  run<kDirect, kPadded, padded_pitch(128), 128>("padded stage tile d=64", out);
  run<kTrans, kPadded, padded_pitch(128), 128>("padded stage tile d=64", out);
  // Forward K tiles (operand reads only) and V tiles (transposing reads only).
  run<kDirect, kPadded, padded_pitch(256), 256>("forward K tile d=128", out);
  run<kDirect, kPadded, padded_pitch(128), 128>("forward K tile d=64", out);
  run<kDirect, kPadded, padded_pitch(192), 160>("forward K tile d=80", out);
  run<kTrans, trans_kind(2, 128), trans_row_bytes(2, 128), 256>("forward V tile d=128", out);
  run<kTrans, trans_kind(2, 80), trans_row_bytes(2, 80), 128>("forward V tile d=80", out);
  run<kTrans16, trans_kind(2, 80), trans_row_bytes(2, 80), 160>("forward V tile d=80", out);
  run<kTrans, trans_kind(2, 64), trans_row_bytes(2, 64), 128>("forward V tile d=64", out);
  run<kStore, trans_kind(2, 64), trans_row_bytes(2, 64), 128>("forward V tile d=64", out);
  run<kStore, trans_kind(2, 80), trans_row_bytes(2, 80), 160>("forward V tile d=80", out);
  // Pitches that break one read form or the other (model checks).
  run<kDirect, kPadded, 320, 256>("pitch 320", out);
  run<kTrans, kPadded, 272, 256>("pitch 272", out);
  run<kDirect, kPadded, 192, 128>("pitch 192", out);
  run<kTrans16, kPadded, 192, 160>("pitch 192", out);
  hipFree(out);
  printf("done\n");
  return 0;
}
