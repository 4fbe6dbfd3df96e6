// Attention backward with recomputation (gfx950): three kernels on one stream.
//
// The math is eqs. (13)-(19) of the CS336 Assignment 2 (systems) handout, §4.2.2 ("backward
// pass with recomputation"): S = scale Q K^T, P_ij = exp(S_ij - L_i), dV = P^T dO,
// dP = dO V^T, dS_ij = P_ij (dP_ij - D_i), dQ = scale dS K, dK = scale dS^T Q, with
// D = rowsum(O o dO) computed first.  Following the key idea of the handout's tiled backward
// (§4.2.3), P is recomputed twice -- once in a kernel that owns key tiles and accumulates dK
// and dV, once in a kernel that owns query tiles and accumulates dQ -- so no workgroup ever
// writes another's output and no atomics are needed (results are bitwise reproducible).
//
//  rowdot_kernel  D_i = sum_c O_ic dO_ic (fp32), one pass over O and dO, bandwidth bound.
//  dkdv_kernel    per (head, 32*NW keys): S and dP with queries on MFMA rows and keys on
//                 columns, so P and dS come out of the accumulators already shaped as the B
//                 operand of dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by LDS transpose reads).
//  dq_kernel      per (head, 32*NW queries): S^T and dP^T with keys on rows, so dS^T feeds
//                 dQ^T += K^T dS^T directly.
// The causal / key-padding mask is regenerated from indices; whole blocks above the diagonal or
// past the key length are skipped.
#include "attn_device.h"
#include "launch.h"

namespace attn {

#ifndef ATTN_BWD_STORE_EARLY
#define ATTN_BWD_STORE_EARLY 1
#endif
constexpr bool kBwdStoreEarly = ATTN_BWD_STORE_EARLY;
#ifndef ATTN_XCD_MAP
#define ATTN_XCD_MAP 1
#endif
constexpr bool kXcdMap = ATTN_XCD_MAP;

// ------------------------------------------------------------------------------------------
// D = rowsum(O o dO)

// Rows of O and dO staged per workgroup: read with contiguous 16-byte loads (consecutive lanes,
// consecutive chunks of a row), so every HBM line is fetched once, then reduced from LDS.
constexpr int kRowdotRows = 128;

template <typename T, int D>
constexpr int rowdot_pitch() { return D + 16 / (int)sizeof(T); }  // one 16-byte chunk of padding per row

template <typename T, int D>
__global__ __launch_bounds__(256) void rowdot_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                     float* __restrict__ Dv, int rows) {
  // Thread pair (2i, 2i+1) owns row i of the workgroup's block; thread `half` of the pair reduces
  // the columns an MFMA operand fragment of that half holds (fragments ks = 0.. in order), then the
  // two halves are added -- the order the dQ kernel uses for the same rows, so D agrees bitwise.
  using M = Mfma<T>;
  constexpr int KS = D / M::KSTEP;
  constexpr int R = kRowdotRows;
  constexpr int LDP = rowdot_pitch<T, D>();
  constexpr int TILE = R * LDP * (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[2 * TILE];
  lds_t* lds = (lds_t*)smem;
  const int r0 = blockIdx.x * R;
  const int nr = min(R, rows - r0);
  const uint32_t bytes = (uint32_t)(nr * D * (int)sizeof(T));  // rows past the end read as zero
  const auto ro = make_rsrc(O + (size_t)r0 * D, bytes);
  const auto rg = make_rsrc(dO + (size_t)r0 * D, bytes);
  TileCopy<T, R, D, LDP, 256> oc, gc;
  oc.load(ro, 0);
  gc.load(rg, 0);
  oc.store(lds);
  gc.store(lds + TILE);
  __syncthreads();
  const int half = threadIdx.x & 1, row = threadIdx.x >> 1;
  typedef const __attribute__((address_space(3))) typename M::frag lfrag;
  const lds_t* orow = lds + (row * LDP + M::KPL * half) * (int)sizeof(T);
  const lds_t* grow = orow + TILE;
  float part = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const typename M::frag a = *reinterpret_cast<lfrag*>(orow + ks * M::KSTEP * (int)sizeof(T));
    const typename M::frag g = *reinterpret_cast<lfrag*>(grow + ks * M::KSTEP * (int)sizeof(T));
    part = frag_dot(a, g, part);
  }
  const float other = __shfl_xor(part, 1, 2);
  if (half == 0 && row < nr) Dv[r0 + row] = part + other;
}

// ------------------------------------------------------------------------------------------
// dK, dV: one workgroup per (head, 32*KB*NW keys); each wave owns KB blocks of 32 keys and loops
// over query tiles of BQ rows, double buffered in LDS together with the tile's L*log2(e) and D
// values.  With KB = 2 every Q / dO operand read from LDS feeds the products of two key blocks,
// which halves the LDS read traffic per MFMA.

// LDS bytes of the dK/dV body: two stages of (Q tile, dO tile, L row, D row), then either (DSELF)
// one float of D per query row for rows up to kDselfMaxN, or (VLDS) the workgroup's V rows.
constexpr int kDselfMaxN = 4096;
#ifndef ATTN_DQ_FULL
#define ATTN_DQ_FULL 1
#endif
constexpr bool kDqFull = ATTN_DQ_FULL;
#ifndef ATTN_DKDV_FULL
#define ATTN_DKDV_FULL 1
#endif
constexpr bool kDkdvFull = ATTN_DKDV_FULL;
#ifndef ATTN_DQ_DSTEP
#define ATTN_DQ_DSTEP 1
#endif
constexpr bool kDqDstep = ATTN_DQ_DSTEP;
template <typename T, int D, int NW, int BQ, bool DSELF, bool VLDS, int KB = 1, bool BSP = false, int G = 1>
constexpr int dkdv_lds_bytes() {
  constexpr int DP = (D + 31) / 32 * 32;
  constexpr int TILE = StageTile<T, D>::bytes(G * BQ);
  return 2 * (2 * TILE + 2 * G * BQ * (int)sizeof(float)) + (DSELF ? kDselfMaxN * (int)sizeof(float) : 0) +
         (VLDS ? 32 * KB * NW * lds_pitch<T, DP>() * (int)sizeof(T) : 0) + (BSP ? kMaxMaskBlocks : 0);
}

// One dK/dV work item (logical block `block` of the grid described by BH, N).  With DSELF the body
// does not read D: it first computes D = rowsum(O o dO) for every query row it will visit, in the
// same fragment order as the D pre-pass, into LDS (requires N <= kDselfMaxN).  With VLDS the
// workgroup's V rows are kept in LDS and read per block instead of being held in registers (frees
// 32 VGPRs per key block at d = 128, where the register file is otherwise too small).  With G = 2
// the workgroup has two groups of NW waves over the same keys and stages of 2 BQ query rows: group
// g takes rows [g BQ, (g + 1) BQ) of every stage, so each wave's chain of stages is half as long
// (for grids too small to fill the chip); group 1's dK, dV are added to group 0's through LDS at
// the end.  With BSP
// the query tiles whose mask row meets none of the workgroup's key blocks are skipped, and each
// wave skips the tiles its own mask block excludes.  With SPLIT the query tiles of every key tile
// are cut into `nsplit` chunks, one workgroup each, which write unscaled float32 partial dK and dV
// rows to `part` ([nsplit][BH*N][D] for dK, then the same for dV) for bwd_sum_kernel to add up.
template <typename T, int D, int NW, int BQ, bool DSELF, bool VLDS, int KB = 1, bool BSP = false, bool SPLIT = false,
          int G = 1, bool XCD = false>
__device__ __forceinline__ void dkdv_body(
    char* smem, int block, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const T* __restrict__ Oin, const float* __restrict__ Lse,
    const float* __restrict__ Dv, T* __restrict__ dK, T* __restrict__ dV, int BH, int H, int N, int causal,
    float scale, float scale_log2, const int32_t* __restrict__ kv_len, const uint8_t* __restrict__ bmask,
    int nsplit = 1, float* __restrict__ part = nullptr) {
  using M = Mfma<T>;
  constexpr int NT = G * NW * 64;  // threads of the workgroup
  constexpr int KW = 32 * KB;  // keys per wave
  constexpr int KT = KW * NW;  // keys per workgroup
  constexpr int DP = (D + 31) / 32 * 32;
  constexpr int NDB = DP / 32;
  // bf16 head dims of 16 modulo 32 (16, 80): the last 16 columns of dK and dV run on 16-wide
  // products (two 16 x 16 accumulators per key block, for its keys 0-15 and 16-31); NDA full
  // 32-row blocks precede them.
  constexpr bool T16 = sizeof(T) == 2 && DP - D == 16;
  constexpr int NDA = T16 ? D / 32 : NDB;
  constexpr int KS = D / M::KSTEP;
  constexpr int NQB = BQ / 32;   // query blocks per wave and stage
  constexpr int BQS = G * BQ;    // query rows per stage
  constexpr int LD = lds_pitch<T, DP>();  // V rows (VLDS)
  using ST = StageTile<T, D>;              // Q and dO tiles (read directly and transposed)
  constexpr int TILE = ST::bytes(BQS);
  constexpr int STAGE = 2 * TILE + 2 * BQS * (int)sizeof(float);  // Q tile, dO tile, L row, D row
  constexpr int SHIFT = BQ == 64 ? 0 : 1;                         // query tiles per mask block = 1 << SHIFT
  static_assert(2 * BQS <= NT, "one thread per staged L / D value");
  // K and V rows staged through the second stage (see kst below): the D-computing bodies of two-group
  // workgroups, whose stage tiles hold exactly the workgroup's KT keys.
  constexpr bool STK = DSELF && G == 2 && KB == 1 && !VLDS && !BSP && BQS == 32 * NW && sizeof(T) == 2;
  static_assert(G == 1 || (G == 2 && !BSP && !SPLIT), "two query groups: dense and unsplit only");
  static_assert(!BSP || ((BQ == 32 || BQ == 64) && KT % kMaskBlock == 0 && KT / kMaskBlock <= 8),
                "block-sparse tiles must nest in the 64 x 64 mask blocks");

  lds_t* lds = (lds_t*)smem;
  lds_t* map = lds + dkdv_lds_bytes<T, D, NW, BQ, DSELF, VLDS, KB, false, G>();

  const int TK = (N + KT - 1) / KT;
  const int nsp = SPLIT ? nsplit : 1;
  const int logical = XCD ? xcd_block(BH, TK * nsp, block) : rank_major_block(BH, TK * nsp, block);
  if (logical < 0) return;
  const int split = logical % nsp;
  const int bh = logical / nsp / TK;
  const int kt = logical / nsp % TK;  // low key tiles see the most queries under causal masking
  const int b = bh / H;
  int kv = N;
  if (kv_len) kv = min(max(kv_len[b], 1), N);

  const size_t base = (size_t)bh * N * D;
  dK += base; dV += base;

  const int grp = G == 1 ? 0 : (int)(threadIdx.x >> 6) / NW;  // query group (G = 2) or 0
  const int w = G == 1 ? (int)(threadIdx.x >> 6) : (int)(threadIdx.x >> 6) % NW, l = lane_id(), half = l >> 5, col = l & 31;
  const int k0 = kt * KT;
  const int kw = k0 + KW * w;  // first key of this wave
  const bool wave_live = kw < kv;
  const unsigned wave_bit = 1u << ((KW * w) / kMaskBlock);  // this wave's mask column within the workgroup

  f32x16 dk[KB][NDA > 0 ? NDA : 1], dv[KB][NDA > 0 ? NDA : 1];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < NDA; ++i) { dk[kb][i] = f32x16{}; dv[kb][i] = f32x16{}; }
  f32x4 dkt[KB][2] = {}, dvt[KB][2] = {};  // T16: dK^T, dV^T columns 32 NDA .. D - 1

  if (k0 < kv) {
    const uint32_t tbytes = (uint32_t)(N * D * sizeof(T));
    const auto rk = make_rsrc(K + base, tbytes);
    const auto rv = make_rsrc(V + base, tbytes);
    const auto rq = make_rsrc(Q + base, tbytes);
    const auto ro = make_rsrc(dO + base, tbytes);
    const auto rl = make_rsrc(Lse + (size_t)bh * N, (uint32_t)(N * sizeof(float)));
    const auto rd = make_rsrc(Dv + (size_t)bh * N, (uint32_t)(N * sizeof(float)));
    typename M::frag kf[KB][KS], vf[KB][VLDS ? 1 : KS];
    lds_t* vt = lds + 2 * STAGE;  // VLDS: V rows k0 .. k0 + KT - 1
    if constexpr (VLDS) {
      TileCopy<T, KT, D, LD, NT> vcp;
      vcp.load(rv, k0);
      vcp.store(vt);
    }
    // STK: the workgroup's K and V rows are copied with contiguous loads into the second stage's
    // Q and dO slots (free until the first stage is consumed), and the fragments read from there.
    TileCopy<T, STK ? KT : 1, STK ? D : 16 / (int)sizeof(T), LD, NT> kst, vst;
    if constexpr (STK) {
      kst.load(rk, k0);
      vst.load(rv, k0);
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kf[kb][ks] = frag_global<T>(rk, kw + 32 * kb + col, D, ks * M::KSTEP);
          if constexpr (!VLDS) vf[kb][ks] = frag_global<T>(rv, kw + 32 * kb + col, D, ks * M::KSTEP);
        }
    }
    const StageReader<T, D> sr(T16);
    // T16: the 16-wide dV and dK products of one 32-query block (weights pf, dS sf as acc_frag c = 0,
    // 1) into key block kb's tail accumulators.
    auto tail_products = [&](int kb, const typename M::frag* pf, const typename M::frag* sf, const lds_t* qtile,
                             const lds_t* otile, int row0) {
      if constexpr (T16) {
        typename M::frag lo, hi;
        M::tail_weights(pf[0], pf[1], lo, hi);
        const typename M::frag ot = sr.trans16(otile, row0, 32 * NDA);
        dvt[kb][0] = M::mma16(ot, lo, dvt[kb][0]);
        dvt[kb][1] = M::mma16(ot, hi, dvt[kb][1]);
        M::tail_weights(sf[0], sf[1], lo, hi);
        const typename M::frag qt = sr.trans16(qtile, row0, 32 * NDA);
        dkt[kb][0] = M::mma16(qt, lo, dkt[kb][0]);
        dkt[kb][1] = M::mma16(qt, hi, dkt[kb][1]);
      }
    };
    auto settle_kv = [&]() {
      if constexpr (STK) {
        kst.template store_to<ST>(lds + STAGE);
        vst.template store_to<ST>(lds + STAGE + TILE);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kf[0][ks] = sr.direct(lds + STAGE, KW * w, ks);
          vf[0][ks] = sr.direct(lds + STAGE + TILE, KW * w, ks);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            settle(kf[kb][ks]);
            if constexpr (!VLDS) settle(vf[kb][ks]);
          }
      }
    };
    // Without DSELF the fragments are waited for here (keeping them out of the first stage's
    // register peak); with DSELF only after the D rows, whose loads then overlap theirs.
    if constexpr (!DSELF) settle_kv();
    const int TQ = (N + BQS - 1) / BQS;
    const int qt0 = causal ? k0 / BQS : 0;
    // This workgroup's query tiles [qt_lo, qt_hi): all from qt0, or one of nsplit equal chunks.
    const int qchunk = (TQ - qt0 + nsp - 1) / nsp;
    const int qt_lo = SPLIT ? min(TQ, qt0 + split * qchunk) : qt0;
    const int qt_hi = SPLIT ? min(TQ, qt_lo + qchunk) : TQ;

    // DSELF: D for rows [qt0*BQS, N), one row per thread at a time, kept in LDS after the stages.
    __attribute__((address_space(3))) float* dself = reinterpret_cast<__attribute__((address_space(3))) float*>(lds + 2 * STAGE);
    if constexpr (DP > D && !T16) {
      zero_pad_stage<ST, T, BQS, D, NT>(lds);
      zero_pad_stage<ST, T, BQS, D, NT>(lds + TILE);
      zero_pad_stage<ST, T, BQS, D, NT>(lds + STAGE);
      zero_pad_stage<ST, T, BQS, D, NT>(lds + STAGE + TILE);
    }
    TileCopy<T, BQS, D, LD, NT> qc, oc;
    // One staged value per thread: L (threads < BQS) or D (threads BQS..2BQS-1).  L is scaled to
    // log2 units and D negated only when written to LDS, so that no arithmetic waits on the load
    // here.  -D is the initial value of the dP accumulator, which then yields dP - D directly.
    float lrd = 0.f;
    auto load_stage = [&](int qt) {
      qc.load(rq, qt * BQS);
      oc.load(ro, qt * BQS);
      const int t = threadIdx.x;
      if (t < (DSELF ? BQS : 2 * BQS))
        lrd = __builtin_bit_cast(float,
                                 __builtin_amdgcn_raw_buffer_load_b32(t < BQS ? rl : rd, (qt * BQS + (t % BQS)) * 4, 0, 0));
    };
    auto store_stage = [&](lds_t* st) {
      qc.template store_to<ST>(st);
      oc.template store_to<ST>(st + TILE);
      if (threadIdx.x < (DSELF ? BQS : 2 * BQS))
        reinterpret_cast<__attribute__((address_space(3))) float*>(st + 2 * TILE)[threadIdx.x] =
            threadIdx.x < BQS ? lrd * kLog2e : -lrd;
    };
    // Query tiles in loop order: all of [qt0, TQ), or (block-sparse) those whose mask row meets one
    // of this workgroup's key blocks; current, next and next-but-one are tracked for the pipeline.
    int cur = qt_lo;
    if constexpr (BSP) {
      build_tile_map(map, bmask, (N + kMaskBlock - 1) / kMaskBlock, k0 / kMaskBlock, KT / kMaskBlock, true, NT);
      __syncthreads();
      cur = next_live_tile(map, qt_lo, qt_hi, SHIFT);
    }
    auto after = [&](int t) { return BSP ? next_live_tile(map, t + 1, qt_hi, SHIFT) : t + 1; };
    if constexpr (DSELF) {
      static_assert(sizeof(T) == 2, "D rows computed in the dK/dV body: bf16 only");
      // The first stage's loads, the D row loads and the K/V fragments are all in flight before
      // the first wait, so this prologue costs one memory latency rather than three.
      if (cur < qt_hi) load_stage(cur);
      // D for rows [qt0 BQS, N): LPR lanes per row, lane j loading 16-byte chunk j of the O and dO
      // rows, so consecutive lanes read consecutive addresses and one load instruction covers whole
      // rows (one thread per row touched a different memory line in every lane).  The sum keeps the
      // fragment order of the dQ kernel and the D pass -- chunk j belongs to half j % 2, each half
      // runs over its chunks in increasing order -- by handing the running sum from lane j - 2 to
      // lane j, so D agrees with theirs bitwise.
      constexpr int C = D * (int)sizeof(T) / 16;                        // 16-byte chunks per row
      constexpr int LPR = C <= 2 ? 2 : C <= 4 ? 4 : C <= 8 ? 8 : 16;  // lanes per row (within a DPP row)
      constexpr int RPP = NT / LPR;                                    // rows per pass
      constexpr int U = 4;                                             // passes in flight
      const int j = (int)threadIdx.x % LPR;
      const int r0 = qt0 * BQS;
      const auto rO = make_rsrc(Oin + base, tbytes);
      for (int p0 = r0; p0 < N; p0 += U * RPP) {
        u32x4 a[U], g[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (p0 + u * RPP < N) {  // uniform: passes with no row are skipped
            const int row = p0 + u * RPP + (int)threadIdx.x / LPR;
            const uint32_t off = (uint32_t)(row * D * (int)sizeof(T) + j * 16);
            const u32x4 zero = {0u, 0u, 0u, 0u};
            const bool ok = j < C && row < N;
            a[u] = ok ? buffer_load16(rO, off) : zero;
            g[u] = ok ? buffer_load16(ro, off) : zero;
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (p0 + u * RPP < N) {
            typename M::frag fa, fg;
            __builtin_memcpy(&fa, &a[u], 16);
            __builtin_memcpy(&fg, &g[u], 16);
            float acc = frag_dot(fa, fg, 0.f);
#pragma unroll
            for (int st = 1; st < C / 2; ++st) {
              // lane j takes the running sum of lane j - 2 (DPP row_shr:2; rows of 16 lanes hold whole
              // groups of LPR lanes), lanes 0 and 1 of a group start from zero
              const float prev = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc), 0x112, 0xf, 0xf, true));
              acc = frag_dot(fa, fg, j >= 2 ? prev : 0.f);
            }
            // lane C - 2 adds the other half's sum from lane C - 1 (DPP row_shl:1)
            const float other = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc), 0x101, 0xf, 0xf, true));
            const int row = p0 + u * RPP + (int)threadIdx.x / LPR;
            if (j == C - 2 && row < N) dself[row - r0] = -(acc + other);
          }
        }
      }
      // Rows [N, N rounded up to a stage) of the last stage are read as the dP accumulators'
      // starting value too; their scores are masked (weight 0), but 0 times a non-finite leftover
      // of this LDS would still be NaN, so they start at 0.
      for (int row = N + (int)threadIdx.x; row < (N + BQS - 1) / BQS * BQS; row += NT) dself[row - r0] = 0.f;
      settle_kv();
      if (cur < qt_hi) store_stage(lds);
    } else if (cur < qt_hi) {
      load_stage(cur);
      store_stage(lds);
    }
    __syncthreads();
    int nxt = cur < qt_hi ? after(cur) : qt_hi;
    if (nxt < qt_hi) load_stage(nxt);

    for (int it = 0; cur < qt_hi; ++it) {
      int nxt2 = qt_hi;
      if constexpr (kBwdStoreEarly && D > 80) {
        // the next stage (loaded one iteration ago) goes to LDS before this stage's products
        nxt2 = nxt < qt_hi ? after(nxt) : qt_hi;
        if (nxt < qt_hi) store_stage(lds + ((it + 1) & 1) * STAGE);
        if (nxt2 < qt_hi) load_stage(nxt2);
      }
      const int q0 = cur * BQS;
      const lds_t* qtile = lds + (it & 1) * STAGE;
      const lds_t* otile = qtile + TILE;
      const __attribute__((address_space(3))) float* lrow =
          reinterpret_cast<const __attribute__((address_space(3))) float*>(qtile + 2 * TILE);
      const __attribute__((address_space(3))) float* drow = DSELF ? dself + (cur - qt0) * BQS : lrow + BQS;
      bool run = wave_live;
      if constexpr (BSP) run = run && (tile_bits(map, cur, SHIFT) & wave_bit);
      // A stage whose rows all see all of this wave's keys (no mask, every query block in range)
      // runs its query blocks as one straight-line block: both blocks' score and dP products first,
      // then each block's weights, dS and dV / dK products, so the second block's products can issue
      // beside the first block's vector work.  Same arithmetic, in the same order per value.  Up to
      // d = 64 only: above, the second block's accumulators do not fit the register file.
      const bool full = kDkdvFull && D <= 64 && NQB > 1 && KB == 1 && G == 1 && q0 + BQS <= N &&
                        kw + 32 <= kv && (!causal || kw + 31 <= q0);
      if (run && full) {
        f32x16 s[NQB], dp[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x4 dd = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(drow + qb * 32 + 8 * m + 4 * half);
#pragma unroll
            for (int r = 0; r < 4; ++r) dp[qb][4 * m + r] = dd[r];
          }
          s[qb] = f32x16{};
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            s[qb] = M::mma(sr.direct(qtile, qb * 32, ks), kf[0][ks], s[qb]);
            if constexpr (VLDS)
              dp[qb] = M::mma(sr.direct(otile, qb * 32, ks), M::frag_direct(vt, LD, (w * KW) * LD + ks * M::KSTEP), dp[qb]);
            else
              dp[qb] = M::mma(sr.direct(otile, qb * 32, ks), vf[0][ks], dp[qb]);
          }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x4 lv = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(lrow + qb * 32 + 8 * m + 4 * half);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int e = 4 * m + r;
              const float p = fast_exp2(__builtin_fmaf(s[qb][e], scale_log2, -lv[r]));
              s[qb][e] = p;
              dp[qb][e] = p * dp[qb][e];
            }
          }
          typename M::frag pf[M::CALLS32], sf[M::CALLS32];
#pragma unroll
          for (int c = 0; c < M::CALLS32; ++c) {
            pf[c] = M::acc_frag(s[qb], c);
            sf[c] = M::acc_frag(dp[qb], c);
#pragma unroll
            for (int db = 0; db < NDA; ++db) {
              dv[0][db] = M::mma(sr.trans(otile, qb * 32, db, c), pf[c], dv[0][db]);
              dk[0][db] = M::mma(sr.trans(qtile, qb * 32, db, c), sf[c], dk[0][db]);
            }
          }
          tail_products(0, pf, sf, qtile, otile, qb * 32);
        }
      } else if (run) {
#pragma unroll
        for (int qbw = 0; qbw < NQB; ++qbw) {
          const int qb = grp * NQB + qbw;  // query block within the stage
          const int qb0 = q0 + qb * 32;
          if (qb0 >= N || (causal && qb0 + 31 < kw)) continue;  // past the end, or before this wave's keys
          // dP accumulators start at -D of their rows (accumulator row order), so after the products
          // they hold dP - D (eq. 17's bracket) with no further subtraction.
          f32x16 nd;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x4 dd = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(drow + qb * 32 + 8 * m + 4 * half);
#pragma unroll
            for (int r = 0; r < 4; ++r) nd[4 * m + r] = dd[r];
          }
          f32x16 s[KB], dp[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) { s[kb] = f32x16{}; dp[kb] = nd; }
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const typename M::frag qa = sr.direct(qtile, qb * 32, ks);
            const typename M::frag oa = sr.direct(otile, qb * 32, ks);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              s[kb] = M::mma(qa, kf[kb][ks], s[kb]);
              if constexpr (VLDS)
                dp[kb] = M::mma(oa, M::frag_direct(vt, LD, (w * KW + 32 * kb) * LD + ks * M::KSTEP), dp[kb]);
              else
                dp[kb] = M::mma(oa, vf[kb][ks], dp[kb]);
            }
          }
          // Mask only blocks that cross the diagonal, the key end or the sequence end: a score
          // whose query row is outside [qmin, N) is pushed to kMaskedScore so exp2 gives 0.  A key
          // block lying wholly above the diagonal comes out all masked (weights exactly 0).
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int kbw = kw + 32 * kb;
            if ((causal && kbw + 31 > qb0) || (kbw + 32 > kv) || (qb0 + 32 > N)) {
              const int key = kbw + col;
              const int qmin = key >= kv ? N : (causal ? key : 0);
              const int lo = qmin - qb0, hi = N - qb0;
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int r = acc_row(e, half);
                s[kb][e] = (r < lo || r >= hi) ? kMaskedScore : s[kb][e];
              }
            }
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int r0 = qb * 32 + 8 * m + 4 * half;
            const f32x4 lv = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(lrow + r0);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int e = 4 * m + r;
                const float p = fast_exp2(__builtin_fmaf(s[kb][e], scale_log2, -lv[r]));
                s[kb][e] = p;
                dp[kb][e] = p * dp[kb][e];
              }
          }
          typename M::frag pf[KB][M::CALLS32], sf[KB][M::CALLS32];
#pragma unroll
          for (int c = 0; c < M::CALLS32; ++c) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              pf[kb][c] = M::acc_frag(s[kb], c);
              sf[kb][c] = M::acc_frag(dp[kb], c);
            }
#pragma unroll
            for (int db = 0; db < NDA; ++db) {
              const typename M::frag ot = sr.trans(otile, qb * 32, db, c);
              const typename M::frag qt = sr.trans(qtile, qb * 32, db, c);
#pragma unroll
              for (int kb = 0; kb < KB; ++kb) {
                dv[kb][db] = M::mma(ot, pf[kb][c], dv[kb][db]);
                dk[kb][db] = M::mma(qt, sf[kb][c], dk[kb][db]);
              }
            }
          }
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) tail_products(kb, pf[kb], sf[kb], qtile, otile, qb * 32);
        }
      }
      if constexpr (kBwdStoreEarly && D > 80) {
        __syncthreads();
      } else {
        nxt2 = nxt < qt_hi ? after(nxt) : qt_hi;
        if (nxt < qt_hi) store_stage(lds + ((it + 1) & 1) * STAGE);
        __syncthreads();
        if (nxt2 < qt_hi) load_stage(nxt2);
      }
      cur = nxt;
      nxt = nxt2;
    }
  }

  if constexpr (G == 2) {
    // Group 1 hands its dK, dV sums to the wave of group 0 that owns the same keys (every wave of
    // the workgroup gets here; the stages are no longer read once the loop's last barrier passed).
    // 16 bytes per lane per access, consecutive lanes at consecutive addresses (conflict-free).
    constexpr int F4A = 2 * KB * NDA * 4;        // float4s per lane: full blocks,
    constexpr int F4 = F4A + (T16 ? 4 * KB : 0);  // then the 16-wide accumulators
    static_assert(NW * 64 * F4 * 16 <= 2 * STAGE, "merge buffer fits in the stages");
    f32x4* mrg = reinterpret_cast<f32x4*>(smem) + w * F4 * 64 + l;
    if (grp == 1) {
      if constexpr (T16)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            mrg[(F4A + 4 * kb + x) * 64] = dkt[kb][x];
            mrg[(F4A + 4 * kb + 2 + x) * 64] = dvt[kb][x];
          }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < NDA; ++i)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x4 k4 = {dk[kb][i][4 * m], dk[kb][i][4 * m + 1], dk[kb][i][4 * m + 2], dk[kb][i][4 * m + 3]};
            const f32x4 v4 = {dv[kb][i][4 * m], dv[kb][i][4 * m + 1], dv[kb][i][4 * m + 2], dv[kb][i][4 * m + 3]};
            mrg[((kb * NDA + i) * 8 + m) * 64] = k4;
            mrg[((kb * NDA + i) * 8 + 4 + m) * 64] = v4;
          }
    }
    __syncthreads();
    if (grp == 1) return;
    if constexpr (T16)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          dkt[kb][x] += mrg[(F4A + 4 * kb + x) * 64];
          dvt[kb][x] += mrg[(F4A + 4 * kb + 2 + x) * 64];
        }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < NDA; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 k4 = mrg[((kb * NDA + i) * 8 + m) * 64];
          const f32x4 v4 = mrg[((kb * NDA + i) * 8 + 4 + m) * 64];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            dk[kb][i][4 * m + r] += k4[r];
            dv[kb][i][4 * m + r] += v4[r];
          }
        }
  }

  // T16: lane l holds columns d16 .. d16 + 3 of keys kw + 32 kb + k16 and k16 + 16.
  const int k16 = l & 15, d16 = 32 * NDA + 4 * (l >> 4);
  if constexpr (SPLIT) {
    if constexpr (T16)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int key = kw + 32 * kb + 16 * x + k16;
          if (key < N) {
            const size_t row = (size_t)split * BH * N + (size_t)bh * N + key;
            *reinterpret_cast<f32x4*>(part + row * D + d16) = dkt[kb][x];
            *reinterpret_cast<f32x4*>(part + (size_t)nsplit * BH * N * D + row * D + d16) = dvt[kb][x];
          }
        }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key = kw + 32 * kb + col;
      if (key < N) {
        const size_t row = (size_t)split * BH * N + (size_t)bh * N + key;
        float* prk = part + row * D;
        float* prv = part + (size_t)nsplit * BH * N * D + row * D;
#pragma unroll
        for (int db = 0; db < NDA; ++db)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int d0 = db * 32 + 8 * m + 4 * half;
            if (D % 32 == 0 || d0 < D) {
              f32x4 k4, v4;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                k4[r] = dk[kb][db][4 * m + r];
                v4[r] = dv[kb][db][4 * m + r];
              }
              *reinterpret_cast<f32x4*>(prk + d0) = k4;
              *reinterpret_cast<f32x4*>(prv + d0) = v4;
            }
          }
      }
    }
    return;
  }
  if constexpr (T16)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int key = kw + 32 * kb + 16 * x + k16;
        if (key < N) {
          T kk[4], vv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kk[r] = (T)(dkt[kb][x][r] * scale);
            vv[r] = (T)dvt[kb][x][r];
          }
          uint2 u;
          __builtin_memcpy(&u, kk, 8);
          *reinterpret_cast<uint2*>(dK + (size_t)key * D + d16) = u;
          __builtin_memcpy(&u, vv, 8);
          *reinterpret_cast<uint2*>(dV + (size_t)key * D + d16) = u;
        }
      }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = kw + 32 * kb + col;
    if (key < N) {
      T* krow = dK + (size_t)key * D;
      T* vrow = dV + (size_t)key * D;
#pragma unroll
      for (int db = 0; db < NDA; ++db)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int d0 = db * 32 + 8 * m + 4 * half;
          if (D % 32 == 0 || d0 < D) {
            T kk[4], vv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              kk[r] = (T)(dk[kb][db][4 * m + r] * scale);
              vv[r] = (T)dv[kb][db][4 * m + r];
            }
            if constexpr (sizeof(T) == 2) {
              uint2 u;
              __builtin_memcpy(&u, kk, 8);
              *reinterpret_cast<uint2*>(krow + d0) = u;
              __builtin_memcpy(&u, vv, 8);
              *reinterpret_cast<uint2*>(vrow + d0) = u;
            } else {
              uint4 u;
              __builtin_memcpy(&u, kk, 16);
              *reinterpret_cast<uint4*>(krow + d0) = u;
              __builtin_memcpy(&u, vv, 16);
              *reinterpret_cast<uint4*>(vrow + d0) = u;
            }
          }
        }
    }
  }
}

template <typename T, int D, int NW, int BQ, int OCC, bool VLDS, int KB, bool BSP, bool SPLIT = false, int G = 1>
__global__ __launch_bounds__(G * NW * 64, OCC) void dkdv_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const float* __restrict__ Lse, const float* __restrict__ Dv, T* __restrict__ dK, T* __restrict__ dV,
    int BH, int H, int N, int causal, float scale, float scale_log2, const int32_t* __restrict__ kv_len,
    const uint8_t* __restrict__ bmask, int nsplit, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) char smem[dkdv_lds_bytes<T, D, NW, BQ, false, VLDS, KB, BSP, G>()];
  dkdv_body<T, D, NW, BQ, false, VLDS, KB, BSP, SPLIT, G, kXcdMap>(smem, blockIdx.x, Q, K, V, dO, nullptr, Lse, Dv, dK, dV,
                                                          BH, H, N, causal, scale, scale_log2, kv_len, bmask, nsplit,
                                                          part);
}

// ------------------------------------------------------------------------------------------
// dQ: one workgroup per (head, 32*NW queries); loop over key tiles of BK rows, double buffered.

template <typename T, int D, int BK, bool BSP = false>
constexpr int dq_lds_bytes() {
  return 4 * StageTile<T, D>::bytes(BK) + (BSP ? kMaxMaskBlocks : 0);
}

// With G = 2 the workgroup has two groups of NW waves over the same queries and key tiles of 2 BK
// keys: group g takes keys [g BK, (g + 1) BK) of every tile, halving each wave's chain; group 1's
// dQ sums are added to group 0's through LDS at the end (as in the forward and dK/dV bodies).
// With STQ the workgroup's rows of Q, dO and O are first copied into LDS after the key stages
// (dq_stq_bytes more bytes) with contiguous 16-byte loads, and each wave reads its operand
// fragments from there: the fragment layout read straight from memory touches 32 rows per load
// instruction, and with G = 2 both groups read the same rows.  Values and reduction order are the
// same either way.
template <typename T, int D, int NW>
constexpr int dq_stq_bytes() {
  return 3 * 32 * NW * lds_pitch<T, (D + 31) / 32 * 32>() * (int)sizeof(T);
}
template <typename T, int D, int NW, int BK, bool BSP = false, bool SPLIT = false, int G = 1, bool STQ = false,
          bool XCD = false>
__device__ __forceinline__ void dq_body(
    char* smem, int block, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const T* __restrict__ Oin, const float* __restrict__ Lse, float* __restrict__ Dv,
    T* __restrict__ dQ, int BH, int H, int N, int causal, float scale, float scale_log2,
    const int32_t* __restrict__ kv_len, const uint8_t* __restrict__ bmask, int nsplit = 1,
    float* __restrict__ part = nullptr) {
  // With Oin != nullptr the kernel first computes D = rowsum(O o dO) for its own query rows (each
  // row belongs to exactly one workgroup) and stores it to Dv for the dK/dV kernel that follows;
  // otherwise it reads D from Dv.
  using M = Mfma<T>;
  constexpr int NT = G * NW * 64;  // threads of the workgroup
  constexpr int QT = 32 * NW;
  constexpr int DP = (D + 31) / 32 * 32;
  constexpr int NDB = DP / 32;
  // bf16 head dims of 16 modulo 32: dQ's last 16 columns on 16-wide products, as in dK/dV.
  constexpr bool T16 = sizeof(T) == 2 && DP - D == 16;
  constexpr int NDA = T16 ? D / 32 : NDB;
  constexpr int KS = D / M::KSTEP;
  constexpr int NB = BK / 32;      // key blocks per wave and tile
  constexpr int BKT = G * BK;      // keys per tile
  constexpr int LD = lds_pitch<T, DP>();  // staged query rows (STQ)
  using ST = StageTile<T, D>;              // K and V tiles
  constexpr int TILE = ST::bytes(BKT);
  constexpr int SHIFT = BK == 64 ? 0 : 1;  // key tiles per mask block = 1 << SHIFT
  static_assert(!BSP || (QT % kMaskBlock == 0 && QT / kMaskBlock <= 8 && (BK == 32 || BK == 64)),
                "block-sparse tiles must nest in the 64 x 64 mask blocks");
  static_assert(G == 1 || (G == 2 && !BSP && !SPLIT), "two key groups: dense and unsplit only");
  static_assert(!STQ || !BSP, "staged query rows: dense masks only");

  lds_t* lds = (lds_t*)smem;
  lds_t* map = lds + 4 * TILE;

  const int TQ = (N + QT - 1) / QT;
  const int nsp = SPLIT ? nsplit : 1;
  const int logical = XCD ? xcd_block(BH, TQ * nsp, block) : rank_major_block(BH, TQ * nsp, block);
  if (logical < 0) return;
  const int split = logical % nsp;
  const int bh = logical / nsp / TQ;
  const int qt = TQ - 1 - logical / nsp % TQ;
  const int b = bh / H;
  int kv = N;
  if (kv_len) kv = min(max(kv_len[b], 1), N);

  const size_t base = (size_t)bh * N * D;
  dQ += base;

  const int grp = G == 1 ? 0 : (int)(threadIdx.x >> 6) / NW;  // key group (G = 2) or 0
  const int w = G == 1 ? (int)(threadIdx.x >> 6) : (int)(threadIdx.x >> 6) % NW, l = lane_id(), half = l >> 5, col = l & 31;
  const int q0 = qt * QT;
  const int qw = q0 + 32 * w;
  const int q = qw + col;
  const int qw_last = min(qw + 31, N - 1);
  const bool wave_live = qw < N;
  const int lim = causal ? min(q, kv - 1) : kv - 1;
  const unsigned wave_bit = 1u << ((32 * w) / kMaskBlock);  // this wave's mask row within the workgroup

  int kend = kv;
  if (causal) kend = min(kend, q0 + QT);
  const int nkt = (kend + BKT - 1) / BKT;
  // This workgroup's key tiles [t_lo, t_hi): all of them, or one of nsplit equal chunks (SPLIT:
  // unscaled float32 partial dQ rows go to part, [nsplit][BH*N][D], for bwd_sum_kernel).
  const int chunk = (nkt + nsp - 1) / nsp;
  const int t_lo = SPLIT ? min(nkt, split * chunk) : 0;
  const int t_hi = SPLIT ? min(nkt, t_lo + chunk) : nkt;

  const uint32_t tbytes = (uint32_t)(N * D * sizeof(T));
  const auto rq = make_rsrc(Q + base, tbytes);
  const auto ro = make_rsrc(dO + base, tbytes);
  const auto rk = make_rsrc(K + base, (uint32_t)(kend * D * sizeof(T)));
  const auto rv = make_rsrc(V + base, (uint32_t)(kend * D * sizeof(T)));

  typename M::frag qf[KS], of[KS];
  if constexpr (!STQ) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = frag_global<T>(rq, q, D, ks * M::KSTEP);
      of[ks] = frag_global<T>(ro, q, D, ks * M::KSTEP);
    }
  }
  const float lq = q < N ? Lse[(size_t)bh * N + q] * kLog2e : 0.f;
  // STQ: rows q0 .. q0 + QT - 1 of Q, dO, O (rows past N read as zero, as the fragments would).
  constexpr int QTILE = QT * LD * (int)sizeof(T);
  lds_t* qs = lds + 4 * TILE;
  TileCopy<T, STQ ? QT : 1, STQ ? D : 16 / (int)sizeof(T), LD, NT> qcp, ocp, ocp2;
  if constexpr (STQ) {
    qcp.load(rq, q0);
    ocp.load(ro, q0);
    if (Oin) ocp2.load(make_rsrc(Oin + base, tbytes), q0);
  }

  f32x16 acc[NDA > 0 ? NDA : 1];
#pragma unroll
  for (int i = 0; i < NDA; ++i) acc[i] = f32x16{};
  f32x4 acct[2] = {};  // T16: dQ^T columns 32 NDA .. D - 1 of queries 0-15 and 16-31

  if constexpr (DP > D && !T16) {
    zero_pad_stage<ST, T, BKT, D, NT>(lds);
    zero_pad_stage<ST, T, BKT, D, NT>(lds + 2 * TILE);
  }
  // Key tiles in loop order (all, or the block-sparse live ones), as in the forward.
  int cur = t_lo;
  if constexpr (BSP) {
    build_tile_map(map, bmask, (N + kMaskBlock - 1) / kMaskBlock, q0 / kMaskBlock, QT / kMaskBlock, false, NT);
    __syncthreads();
    cur = next_live_tile(map, t_lo, t_hi, SHIFT);
  }
  auto after = [&](int t) { return BSP ? next_live_tile(map, t + 1, t_hi, SHIFT) : t + 1; };
  // The first K/V tile's loads are issued before D waits on its O fragments, so the prologue
  // costs one memory latency rather than two.
  TileCopy<T, BKT, D, LD, NT> kc, vc;
  if (cur < t_hi) {
    kc.load(rk, cur * BKT);
    vc.load(rv, cur * BKT);
  }
  if constexpr (STQ) {
    qcp.store(qs);
    ocp.store(qs + QTILE);
    if (Oin) ocp2.store(qs + 2 * QTILE);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = M::frag_direct(qs, LD, 32 * w * LD + ks * M::KSTEP);
      of[ks] = M::frag_direct(qs + QTILE, LD, 32 * w * LD + ks * M::KSTEP);
    }
  }
  float dq_;
  if (Oin) {
    const auto rO = make_rsrc(Oin + base, tbytes);
    float dpart = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const typename M::frag oa = STQ ? M::frag_direct(qs + 2 * QTILE, LD, 32 * w * LD + ks * M::KSTEP)
                                      : frag_global<T>(rO, q, D, ks * M::KSTEP);
      dpart = frag_dot(oa, of[ks], dpart);
    }
    dq_ = dpart + swap_halves(dpart);
    if (half == 0 && q < N && split == 0 && grp == 0) Dv[(size_t)bh * N + q] = dq_;
  } else {
    dq_ = q < N ? Dv[(size_t)bh * N + q] : 0.f;
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    settle(qf[ks]);
    settle(of[ks]);
  }
  settle(lq);
  settle(dq_);
  // bf16 at d = 80: -D enters the dP^T product as one more reduction step, ones (reduction rows 0
  // and 1) against -D rounded to bf16 in two parts, hi + lo (rows 0 and 1 of this lane's query
  // column), so that the accumulators end as dP - D with no subtraction per score.  Lanes 32-63 hold
  // reduction rows 8-15: zero.  Measured on B=4 H=32 N=2048 d=80: 176-177 -> 172-174 us; at d = 64
  // its 8 registers take the kernel past 128 VGPRs, from four waves per SIMD to three (+3%).
  constexpr bool DSTEP = kDqDstep && sizeof(T) == 2 && D == 80;
  typename M::frag ones_f{}, negd_f{};
  if constexpr (DSTEP) {
    if (half == 0) {
      const __bf16 hi = (__bf16)(-dq_);
      ones_f[0] = ones_f[1] = (__bf16)1.0f;
      negd_f[0] = hi;
      negd_f[1] = (__bf16)(-dq_ - (float)hi);
    }
  }
  if (cur < t_hi) {
    kc.template store_to<ST>(lds);
    vc.template store_to<ST>(lds + TILE);
  }
  __syncthreads();
  int nxt = cur < t_hi ? after(cur) : t_hi;
  const StageReader<T, D> sr(T16);
  // T16: the 16-wide dQ products of one 32-key block (dS^T as acc_frag c = 0, 1).
  auto tail_products = [&](const typename M::frag* sf, const lds_t* ktile, int row0) {
    if constexpr (T16) {
      typename M::frag lo, hi;
      M::tail_weights(sf[0], sf[1], lo, hi);
      const typename M::frag kt = sr.trans16(ktile, row0, 32 * NDA);
      acct[0] = M::mma16(kt, lo, acct[0]);
      acct[1] = M::mma16(kt, hi, acct[1]);
    }
  };
  if (nxt < t_hi) {
    kc.load(rk, nxt * BKT);
    vc.load(rv, nxt * BKT);
  }
  for (int it = 0; cur < t_hi; ++it) {
    int nxt2 = t_hi;
    if constexpr (kBwdStoreEarly && D > 80) {
      // the next tile (loaded one iteration ago) goes to LDS before this tile's products
      nxt2 = nxt < t_hi ? after(nxt) : t_hi;
      if (nxt < t_hi) {
        lds_t* st = lds + ((it + 1) & 1) * 2 * TILE;
        kc.template store_to<ST>(st);
        vc.template store_to<ST>(st + TILE);
      }
      if (nxt2 < t_hi) {
        kc.load(rk, nxt2 * BKT);
        vc.load(rv, nxt2 * BKT);
      }
    }
    // This group's keys of the tile: rows grp * BK .. grp * BK + BK - 1 of the staged K and V.
    const lds_t* ktile = lds + (it & 1) * 2 * TILE + ST::block(grp * BK);
    const lds_t* vtile = ktile + TILE;
    bool run = wave_live;
    if constexpr (BSP) run = run && (tile_bits(map, cur, SHIFT) & wave_bit);
    // A tile whose keys are all visible to all of this wave's queries (no mask, every key block
    // in range) runs its key blocks as one straight-line block: both blocks' score and dP products
    // first, then each block's weights, dS and dQ products, so the second block's products can
    // issue beside the first block's vector work.  Same arithmetic, in the same order per value.
    const int kt0 = cur * BKT + grp * BK;
    const bool full = kDqFull && NB > 1 && kt0 + BK <= kend && (!causal || kt0 + BK - 1 <= qw);
    if (run && full) {
      f32x16 s[NB], dp[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        s[nb] = f32x16{};
#pragma unroll
        for (int e = 0; e < 16; ++e) dp[nb][e] = D > 80 ? -dq_ : 0.f;
        if constexpr (DSTEP) dp[nb] = M::mma(ones_f, negd_f, dp[nb]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s[nb] = M::mma(sr.direct(ktile, nb * 32, ks), qf[ks], s[nb]);
          dp[nb] = M::mma(sr.direct(vtile, nb * 32, ks), of[ks], dp[nb]);
        }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[nb][e], scale_log2, -lq));
          dp[nb][e] = D > 80 || DSTEP ? p * dp[nb][e] : p * (dp[nb][e] - dq_);
        }
        typename M::frag sf[M::CALLS32];
#pragma unroll
        for (int c = 0; c < M::CALLS32; ++c) {
          sf[c] = M::acc_frag(dp[nb], c);
#pragma unroll
          for (int db = 0; db < NDA; ++db)
            acc[db] = M::mma(sr.trans(ktile, nb * 32, db, c), sf[c], acc[db]);
        }
        tail_products(sf, ktile, nb * 32);
      }
    } else if (run) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int kb0 = cur * BKT + grp * BK + nb * 32;
        if (kb0 >= kend || (causal && kb0 > qw_last)) continue;
        // At d = 128 the dP^T accumulators start at -D of this lane's query, so they end as dP - D
        // (eq. 17's bracket) with no subtraction per score (2% faster there; at d <= 80 the extra
        // live registers cost more than the subtraction).
        f32x16 s = f32x16{}, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) dp[e] = D > 80 ? -dq_ : 0.f;
        if constexpr (DSTEP) dp = M::mma(ones_f, negd_f, dp);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = M::mma(sr.direct(ktile, nb * 32, ks), qf[ks], s);
          dp = M::mma(sr.direct(vtile, nb * 32, ks), of[ks], dp);
        }
        if ((causal && kb0 + 31 > qw) || (kb0 + 32 > kv)) {
#pragma unroll
          for (int e = 0; e < 16; ++e) s[e] = (kb0 + acc_row(e, half) > lim) ? kMaskedScore : s[e];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[e], scale_log2, -lq));
          dp[e] = D > 80 || DSTEP ? p * dp[e] : p * (dp[e] - dq_);
        }
        typename M::frag sf[M::CALLS32];
#pragma unroll
        for (int c = 0; c < M::CALLS32; ++c) {
          sf[c] = M::acc_frag(dp, c);
#pragma unroll
          for (int db = 0; db < NDA; ++db)
            acc[db] = M::mma(sr.trans(ktile, nb * 32, db, c), sf[c], acc[db]);
        }
        tail_products(sf, ktile, nb * 32);
      }
    }
    if constexpr (kBwdStoreEarly && D > 80) {
      __syncthreads();
    } else {
      nxt2 = nxt < t_hi ? after(nxt) : t_hi;
      if (nxt < t_hi) {
        lds_t* st = lds + ((it + 1) & 1) * 2 * TILE;
        kc.template store_to<ST>(st);
        vc.template store_to<ST>(st + TILE);
      }
      __syncthreads();
      if (nxt2 < t_hi) {
        kc.load(rk, nxt2 * BKT);
        vc.load(rv, nxt2 * BKT);
      }
    }
    cur = nxt;
    nxt = nxt2;
  }

  if constexpr (G == 2) {
    // Group 1 hands its dQ sums to the wave of group 0 that owns the same queries (the tiles are
    // no longer read: the loop ended on a barrier and staged nothing after it).
    // 16 bytes per lane per access, consecutive lanes at consecutive addresses (conflict-free).
    constexpr int F4 = NDA * 4 + (T16 ? 2 : 0);  // float4s per lane (the 16-wide accumulators last)
    static_assert(NW * 64 * F4 * 16 <= 4 * TILE, "merge buffer fits in the tile stages");
    f32x4* mrg = reinterpret_cast<f32x4*>(smem) + w * F4 * 64 + l;
    if (grp == 1) {
      if constexpr (T16) {
        mrg[(4 * NDA) * 64] = acct[0];
        mrg[(4 * NDA + 1) * 64] = acct[1];
      }
#pragma unroll
      for (int i = 0; i < NDA; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 a4 = {acc[i][4 * m], acc[i][4 * m + 1], acc[i][4 * m + 2], acc[i][4 * m + 3]};
          mrg[(4 * i + m) * 64] = a4;
        }
    }
    __syncthreads();
    if (grp == 1) return;
    if constexpr (T16) {
      acct[0] += mrg[(4 * NDA) * 64];
      acct[1] += mrg[(4 * NDA + 1) * 64];
    }
#pragma unroll
    for (int i = 0; i < NDA; ++i)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 a4 = mrg[(4 * i + m) * 64];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][4 * m + r] += a4[r];
      }
  }

  // T16: lane l holds columns d16 .. d16 + 3 of queries q16 and q16 + 16.
  const int q16 = qw + (l & 15), d16 = 32 * NDA + 4 * (l >> 4);
  if constexpr (SPLIT) {
    if constexpr (T16)
#pragma unroll
      for (int x = 0; x < 2; ++x)
        if (q16 + 16 * x < N)
          *reinterpret_cast<f32x4*>(part + ((size_t)split * BH * N + (size_t)bh * N + q16 + 16 * x) * D + d16) = acct[x];
    if (q < N) {
      float* prow = part + ((size_t)split * BH * N + (size_t)bh * N + q) * D;
#pragma unroll
      for (int db = 0; db < NDA; ++db)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int d0 = db * 32 + 8 * m + 4 * half;
          if (D % 32 == 0 || d0 < D) {
            f32x4 v4;
#pragma unroll
            for (int r = 0; r < 4; ++r) v4[r] = acc[db][4 * m + r];
            *reinterpret_cast<f32x4*>(prow + d0) = v4;
          }
        }
    }
    return;
  }
  if constexpr (T16)
#pragma unroll
    for (int x = 0; x < 2; ++x)
      if (q16 + 16 * x < N) {
        T v4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = (T)(acct[x][r] * scale);
        uint2 u;
        __builtin_memcpy(&u, v4, 8);
        *reinterpret_cast<uint2*>(dQ + (size_t)(q16 + 16 * x) * D + d16) = u;
      }
  if (q < N) {
    T* row = dQ + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < NDA; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d0 = db * 32 + 8 * m + 4 * half;
        if (D % 32 == 0 || d0 < D) {
          T v4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v4[r] = (T)(acc[db][4 * m + r] * scale);
          if constexpr (sizeof(T) == 2) {
            uint2 u;
            __builtin_memcpy(&u, v4, 8);
            *reinterpret_cast<uint2*>(row + d0) = u;
          } else {
            uint4 u;
            __builtin_memcpy(&u, v4, 16);
            *reinterpret_cast<uint4*>(row + d0) = u;
          }
        }
      }
  }
}

template <typename T, int D, int NW, int BK, int OCC, bool BSP, bool SPLIT = false, int G = 1>
__global__ __launch_bounds__(G * NW * 64, OCC) void dq_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const T* __restrict__ Oin, const float* __restrict__ Lse, float* __restrict__ Dv, T* __restrict__ dQ, int BH,
    int H, int N, int causal, float scale, float scale_log2, const int32_t* __restrict__ kv_len,
    const uint8_t* __restrict__ bmask, int nsplit, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) char smem[dq_lds_bytes<T, D, G * BK, BSP>()];
  dq_body<T, D, NW, BK, BSP, SPLIT, G, false, kXcdMap>(smem, blockIdx.x, Q, K, V, dO, Oin, Lse, Dv, dQ, BH, H, N, causal, scale,
                                       scale_log2, kv_len, bmask, nsplit, part);
}

// out = scale * sum_s part[s] elementwise (fixed order, so the split backward stays deterministic),
// converted to the output dtype; 4 elements per thread (count is a multiple of 4).
template <typename T>
__global__ __launch_bounds__(256) void bwd_sum_kernel(const float* __restrict__ part, int nsplit, size_t count,
                                                      float scale, T* __restrict__ out) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  for (int sp = 1; sp < nsplit; ++sp) acc += *reinterpret_cast<const f32x4*>(part + (size_t)sp * count + i);
  T v4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v4[r] = (T)(acc[r] * scale);
  if constexpr (sizeof(T) == 2) {
    uint2 u;
    __builtin_memcpy(&u, v4, 8);
    *reinterpret_cast<uint2*>(out + i) = u;
  } else {
    uint4 u;
    __builtin_memcpy(&u, v4, 16);
    *reinterpret_cast<uint4*>(out + i) = u;
  }
}

template <typename T>
static hipError_t launch_sum(const float* part, int nsplit, size_t count, float scale, void* out, hipStream_t s) {
  const unsigned blocks = (unsigned)((count / 4 + 255) / 256);
  hipLaunchKernelGGL((bwd_sum_kernel<T>), dim3(blocks), dim3(256), 0, s, part, nsplit, count, scale, (T*)out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Small problems: dQ and dK/dV in one launch.  The first nq blocks run dQ work items (which also
// store D), the rest run dK/dV work items that compute D themselves, so the two halves have no
// ordering between them and run side by side when the grid would otherwise leave CUs idle.

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename T, int D, bool BSP>
__global__ __launch_bounds__(256, 2) void bwd_small_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const T* __restrict__ O, const float* __restrict__ Lse, float* __restrict__ Dv, T* __restrict__ dQ,
    T* __restrict__ dK, T* __restrict__ dV, int BH, int H, int N, int causal, float scale, float scale_log2,
    const int32_t* __restrict__ kv_len, int nq, const uint8_t* __restrict__ bmask) {
  __shared__ __attribute__((aligned(16))) char
      smem[cmax(dq_lds_bytes<T, D, 32, BSP>(), dkdv_lds_bytes<T, D, 4, 64, true, false, 1, BSP>())];
  if ((int)blockIdx.x < nq)
    dq_body<T, D, 4, 32, BSP>(smem, blockIdx.x, Q, K, V, dO, O, Lse, Dv, dQ, BH, H, N, causal, scale, scale_log2,
                              kv_len, bmask);
  else
    dkdv_body<T, D, 4, 64, true, false, 1, BSP>(smem, blockIdx.x - nq, Q, K, V, dO, O, Lse, Dv, dK, dV, BH, H, N,
                                                causal, scale, scale_log2, kv_len, bmask);
}

// Dense masks: the same two kinds of work item on 8-wave workgroups whose two groups split each
// item's chain (dq_body / dkdv_body with G = 2).  Such workgroups fit one per CU, fewer than the
// items, so the items run longest first: `order` lists the item classes -- bit 7 set for dK/dV,
// low bits the key tile (dK/dV) or the query tile counted from the end (dQ) -- by decreasing
// expected time, and block b runs class b / BH for head b % BH.
struct SmallOrder {
  uint8_t cls[64];
};


template <typename T, int D>
__global__ __launch_bounds__(512, 1) void bwd_small2_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const T* __restrict__ O, const float* __restrict__ Lse, float* __restrict__ Dv, T* __restrict__ dQ,
    T* __restrict__ dK, T* __restrict__ dV, int BH, int H, int N, int causal, float scale, float scale_log2,
    const int32_t* __restrict__ kv_len, SmallOrder order) {
  // dQ items stage their query rows in LDS (STQ) where that fits in the dK/dV items' allocation.
  constexpr bool STQ = D <= 64;
  __shared__ __attribute__((aligned(16))) char
      smem[cmax(dq_lds_bytes<T, D, 64, false>() + (STQ ? dq_stq_bytes<T, D, 4>() : 0),
                dkdv_lds_bytes<T, D, 4, 64, true, false, 1, false, 2>())];
  const int c = order.cls[blockIdx.x / BH];
  // Block of the bodies' rank-major grids: rank (c & 0x7f) of head blockIdx.x % BH.
  const int b = (c & 0x7f) * BH + (int)blockIdx.x % BH;
  if (c & 0x80)
    dkdv_body<T, D, 4, 64, true, false, 1, false, false, 2>(
        smem, b, Q, K, V, dO, O, Lse, Dv, dK, dV, BH, H, N, causal,
        scale, scale_log2, kv_len, nullptr);
  else
    dq_body<T, D, 4, 32, false, false, 2, STQ>(smem, b, Q, K, V, dO, O, Lse, Dv,
                                               dQ, BH, H, N, causal, scale, scale_log2, kv_len, nullptr);
}

// ------------------------------------------------------------------------------------------
// launchers

// Two groups per workgroup in the backward kernels (G = 2 of dq_body and dkdv_body) where the
// merged small-problem launch applies with a dense mask and chains are long enough to gain from
// halving (N >= 512) -- also for the dQ and dK/dV kernels launched on their own, so that attn_bwd
// and its sub-steps stay bitwise equal.  Measured on MI355X (backward launch, bf16): B=4 H=12
// N=512 d=64 26.3 -> 22.7 us, B=2 H=16 N=1024 d=64 45.2 -> 39.2 us; at N=128 and 256 two groups
// were slower (12.9 -> 17.9 us, 20.3 -> 22.1 us): their 8-wave workgroups fit one per CU, so the
// items run in more than one round, which short chains do not pay back.
static bool bwd_two_groups(int dtype, const Problem& p) {
  return !p.bmask && p.N >= 512 && bwd_small_applies(dtype, p);
}

template <typename T, int D>
static hipError_t launch_rowdot_t(const Problem& p, const void* O, const void* dO, float* Dv, hipStream_t s) {
  const int rows = p.B * p.H * p.N;
  const int grid = (rows + kRowdotRows - 1) / kRowdotRows;
  hipLaunchKernelGGL((rowdot_kernel<T, D>), dim3(grid), dim3(256), 0, s, (const T*)O, (const T*)dO, Dv, rows);
  return hipGetLastError();
}

template <typename T, int D, int NW, int BQ, int OCC, bool VLDS = false, int KB = 1>
static hipError_t launch_dkdv_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                const float* L, const float* Dv, void* dK, void* dV, hipStream_t s, int nsplit,
                                float* part) {
  constexpr int KT = 32 * KB * NW;
  const int TK = (p.N + KT - 1) / KT;
  const int BH = p.B * p.H;
  if (nsplit > 1) {
    const int grid = BH * TK * nsplit;
    if (p.bmask)
      hipLaunchKernelGGL((dkdv_kernel<T, D, NW, BQ, OCC, VLDS, KB, true, true>), dim3(grid), dim3(NW * 64), 0, s,
                         (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, (T*)dK, (T*)dV, BH, p.H, p.N,
                         p.causal, p.scale, p.scale * kLog2e, p.kv_len, p.bmask, nsplit, part);
    else
      hipLaunchKernelGGL((dkdv_kernel<T, D, NW, BQ, OCC, VLDS, KB, false, true>), dim3(grid), dim3(NW * 64), 0, s,
                         (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, (T*)dK, (T*)dV, BH, p.H, p.N,
                         p.causal, p.scale, p.scale * kLog2e, p.kv_len, nullptr, nsplit, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t count = (size_t)BH * p.N * D;
    e = launch_sum<T>(part, nsplit, count, p.scale, dK, s);
    if (e != hipSuccess) return e;
    return launch_sum<T>(part + (size_t)nsplit * count, nsplit, count, 1.0f, dV, s);
  }
  const int grid = BH * TK;
  if constexpr (sizeof(T) == 2 && D <= 80 && NW == 4 && BQ == 64 && !VLDS && KB == 1) {
    if (bwd_two_groups(kBF16, p)) {
      hipLaunchKernelGGL((dkdv_kernel<T, D, NW, BQ, 1, VLDS, KB, false, false, 2>), dim3(grid), dim3(2 * NW * 64), 0, s,
                         (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, L, Dv, (T*)dK, (T*)dV, BH, p.H, p.N,
                         p.causal, p.scale, p.scale * kLog2e, p.kv_len, nullptr, 1, nullptr);
      return hipGetLastError();
    }
  }
  if (p.bmask)
    hipLaunchKernelGGL((dkdv_kernel<T, D, NW, BQ, OCC, VLDS, KB, true>), dim3(grid), dim3(NW * 64), 0, s, (const T*)Q,
                       (const T*)K, (const T*)V, (const T*)dO, L, Dv, (T*)dK, (T*)dV, p.B * p.H, p.H, p.N, p.causal,
                       p.scale, p.scale * kLog2e, p.kv_len, p.bmask, 1, nullptr);
  else
    hipLaunchKernelGGL((dkdv_kernel<T, D, NW, BQ, OCC, VLDS, KB, false>), dim3(grid), dim3(NW * 64), 0, s, (const T*)Q,
                       (const T*)K, (const T*)V, (const T*)dO, L, Dv, (T*)dK, (T*)dV, p.B * p.H, p.H, p.N, p.causal,
                       p.scale, p.scale * kLog2e, p.kv_len, nullptr, 1, nullptr);
  return hipGetLastError();
}

template <typename T, int D, int NW, int BK, int OCC>
static hipError_t launch_dq_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                              const void* O, const float* L, float* Dv, void* dQ, hipStream_t s, int nsplit,
                              float* part) {
  constexpr int QT = 32 * NW;
  const int TQ = (p.N + QT - 1) / QT;
  const int BH = p.B * p.H;
  if (nsplit > 1) {
    const int grid = BH * TQ * nsplit;
    if (p.bmask)
      hipLaunchKernelGGL((dq_kernel<T, D, NW, BK, OCC, true, true>), dim3(grid), dim3(NW * 64), 0, s, (const T*)Q,
                         (const T*)K, (const T*)V, (const T*)dO, (const T*)O, L, Dv, (T*)dQ, BH, p.H, p.N, p.causal,
                         p.scale, p.scale * kLog2e, p.kv_len, p.bmask, nsplit, part);
    else
      hipLaunchKernelGGL((dq_kernel<T, D, NW, BK, OCC, false, true>), dim3(grid), dim3(NW * 64), 0, s, (const T*)Q,
                         (const T*)K, (const T*)V, (const T*)dO, (const T*)O, L, Dv, (T*)dQ, BH, p.H, p.N, p.causal,
                         p.scale, p.scale * kLog2e, p.kv_len, nullptr, nsplit, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_sum<T>(part, nsplit, (size_t)BH * p.N * D, p.scale, dQ, s);
  }
  const int grid = BH * TQ;
  if constexpr (sizeof(T) == 2 && D <= 80 && NW == 4 && BK == 32) {
    if (bwd_two_groups(kBF16, p)) {
      hipLaunchKernelGGL((dq_kernel<T, D, NW, BK, 1, false, false, 2>), dim3(grid), dim3(2 * NW * 64), 0, s,
                         (const T*)Q, (const T*)K, (const T*)V, (const T*)dO, (const T*)O, L, Dv, (T*)dQ, BH, p.H,
                         p.N, p.causal, p.scale, p.scale * kLog2e, p.kv_len, nullptr, 1, nullptr);
      return hipGetLastError();
    }
  }
  if (p.bmask)
    hipLaunchKernelGGL((dq_kernel<T, D, NW, BK, OCC, true>), dim3(grid), dim3(NW * 64), 0, s, (const T*)Q,
                       (const T*)K, (const T*)V, (const T*)dO, (const T*)O, L, Dv, (T*)dQ, p.B * p.H, p.H, p.N,
                       p.causal, p.scale, p.scale * kLog2e, p.kv_len, p.bmask, 1, nullptr);
  else
    hipLaunchKernelGGL((dq_kernel<T, D, NW, BK, OCC, false>), dim3(grid), dim3(NW * 64), 0, s, (const T*)Q,
                       (const T*)K, (const T*)V, (const T*)dO, (const T*)O, L, Dv, (T*)dQ, p.B * p.H, p.H, p.N,
                       p.causal, p.scale, p.scale * kLog2e, p.kv_len, nullptr, 1, nullptr);
  return hipGetLastError();
}

bool bwd_supported(int dtype, int d) { return fwd_supported(dtype, d); }

template <typename T, int D>
static hipError_t launch_bwd_small_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                     const void* O, const float* L, float* Dv, void* dQ, void* dK, void* dV,
                                     hipStream_t s) {
  const int BH = p.B * p.H;
  const int nq = BH * ((p.N + 127) / 128);
  const int nk = nq;
  if (!bwd_two_groups(kBF16, p)) {
    if (p.bmask)
      hipLaunchKernelGGL((bwd_small_kernel<T, D, true>), dim3(nq + nk), dim3(256), 0, s, (const T*)Q, (const T*)K,
                         (const T*)V, (const T*)dO, (const T*)O, L, Dv, (T*)dQ, (T*)dK, (T*)dV, BH, p.H, p.N,
                         p.causal, p.scale, p.scale * kLog2e, p.kv_len, nq, p.bmask);
    else
      hipLaunchKernelGGL((bwd_small_kernel<T, D, false>), dim3(nq + nk), dim3(256), 0, s, (const T*)Q, (const T*)K,
                         (const T*)V, (const T*)dO, (const T*)O, L, Dv, (T*)dQ, (T*)dK, (T*)dV, BH, p.H, p.N,
                         p.causal, p.scale, p.scale * kLog2e, p.kv_len, nq, nullptr);
    return hipGetLastError();
  }
  // Item classes, longest expected time first.  Per-item times measured on MI355X (two groups,
  // d = 64): dK/dV about 5 us + 2.7 us per 128-query stage, dQ about 5.2 us + 0.8 us per
  // 64-key tile.  Ties keep dK/dV before dQ and lower tiles first.
  const int T128 = (p.N + 127) / 128;
  if (2 * T128 > 64) return hipErrorInvalidValue;
  struct Cls { float cost; int key; uint8_t code; } cls[64];
  int nc = 0;
  for (int kt = 0; kt < T128; ++kt) {
    const int stages = p.causal ? T128 - kt : T128;
    cls[nc] = {5.0f + 2.7f * stages, nc, (uint8_t)(0x80 | kt)};
    ++nc;
  }
  for (int r = 0; r < T128; ++r) {  // r-th query tile from the end
    const int qt = T128 - 1 - r;
    const int keys = p.causal ? (p.N < 128 * (qt + 1) ? p.N : 128 * (qt + 1)) : p.N;
    cls[nc] = {5.2f + 0.8f * ((keys + 63) / 64), nc, (uint8_t)r};
    ++nc;
  }
  for (int i = 1; i < nc; ++i)  // insertion sort by decreasing cost, stable
    for (int j = i; j > 0 && cls[j].cost > cls[j - 1].cost; --j) {
      const Cls t = cls[j];
      cls[j] = cls[j - 1];
      cls[j - 1] = t;
    }
  SmallOrder order{};
  for (int i = 0; i < nc; ++i) order.cls[i] = cls[i].code;
  hipLaunchKernelGGL((bwd_small2_kernel<T, D>), dim3(nc * BH), dim3(512), 0, s, (const T*)Q, (const T*)K,
                     (const T*)V, (const T*)dO, (const T*)O, L, Dv, (T*)dQ, (T*)dK, (T*)dV, BH, p.H, p.N, p.causal,
                     p.scale, p.scale * kLog2e, p.kv_len, order);
  return hipGetLastError();
}

bool bwd_small_applies(int dtype, const Problem& p) {
  if (dtype != kBF16 || p.d > 80 || p.N > kDselfMaxN) return false;
  // both halves together fit in one pass of two 4-wave workgroups per CU
  return 2L * p.B * p.H * ((p.N + 127) / 128) <= 512;
}

hipError_t launch_bwd_small(int dtype, const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                            const void* O, const float* L, float* Dv, void* dQ, void* dK, void* dV, hipStream_t s) {
  if (!bwd_small_applies(dtype, p)) return hipErrorInvalidValue;
  switch (p.d) {
    case 16: return launch_bwd_small_t<__bf16, 16>(p, Q, K, V, dO, O, L, Dv, dQ, dK, dV, s);
    case 32: return launch_bwd_small_t<__bf16, 32>(p, Q, K, V, dO, O, L, Dv, dQ, dK, dV, s);
    case 64: return launch_bwd_small_t<__bf16, 64>(p, Q, K, V, dO, O, L, Dv, dQ, dK, dV, s);
    case 80: return launch_bwd_small_t<__bf16, 80>(p, Q, K, V, dO, O, L, Dv, dQ, dK, dV, s);
  }
  return hipErrorInvalidValue;
}

#define ATTN_BWD_CASES(X)                                     \
  X(__bf16, kBF16, 16) X(__bf16, kBF16, 32) X(__bf16, kBF16, 64) \
  X(__bf16, kBF16, 80) X(__bf16, kBF16, 128) X(float, kF32, 16) \
  X(float, kF32, 32) X(float, kF32, 64) X(float, kF32, 80) X(float, kF32, 128)

hipError_t launch_rowdot(int dtype, const Problem& p, const void* O, const void* dO, float* Dv, hipStream_t s) {
#define X(T, DT, DD) \
  if (dtype == DT && p.d == DD) return launch_rowdot_t<T, DD>(p, O, dO, Dv, s);
  ATTN_BWD_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

// Tile choices (measured on MI355X): for bf16 head dims up to 80, two 4-wave workgroups per CU with
// 64-query stages (waves of different workgroups share a SIMD, so their MFMA and VALU phases
// interleave).  At d = 128 the register file holds two waves per SIMD only with V in LDS: one
// 8-wave workgroup per CU with 64-query stages for large grids, 4-wave workgroups otherwise.  dQ:
// 4-wave workgroups, two per CU; key tiles of 32 for head dims up to 80, 64 at d = 128.
struct BwdTiles {
  int kt;  // keys per dK/dV workgroup
  int bq;  // query rows per dK/dV stage
  int bk;  // key rows per dQ tile
};
static BwdTiles bwd_tiles(int dtype, const Problem& p) {
  if (dtype == kF32) return {128, 32, 32};
  if (p.d <= 80) return {128, 64, 32};
  if ((long)p.B * p.H * ((p.N + 255) / 256) >= 512) return {256, 64, 64};
  return {128, 64, 64};
}

// Chunks per workgroup chain for the split backward, by the rule the forward uses: split only
// grids with fewer than ~4 workgroups per CU whose chains are long (N >= 2048 in bfloat16, 256
// in float32), into chunks of at least four tiles, at most kMaxSplits.
static int chain_splits(int dtype, const Problem& p, long items, int chain_tiles) {
  if (items >= 1024 || p.N < (dtype == kBF16 ? 2048 : 256)) return 1;
  int s = (int)((1280 + items - 1) / items);
  s = s > kMaxSplits ? kMaxSplits : s;
  s = s > chain_tiles / 4 ? chain_tiles / 4 : s;
  return s >= 2 ? s : 1;
}
static int dq_splits(int dtype, const Problem& p) {
  const BwdTiles t = bwd_tiles(dtype, p);
  return chain_splits(dtype, p, (long)p.B * p.H * ((p.N + 127) / 128), (p.N + t.bk - 1) / t.bk);
}
static int dkdv_splits(int dtype, const Problem& p) {
  const BwdTiles t = bwd_tiles(dtype, p);
  return chain_splits(dtype, p, (long)p.B * p.H * ((p.N + t.kt - 1) / t.kt), (p.N + t.bq - 1) / t.bq);
}
static size_t dq_workspace(int dtype, const Problem& p) {
  const int sq = dq_splits(dtype, p);
  return sq > 1 ? (size_t)sq * p.B * p.H * p.N * p.d * sizeof(float) : 0;
}
static size_t dkdv_workspace(int dtype, const Problem& p) {
  const int sk = dkdv_splits(dtype, p);
  return sk > 1 ? 2 * (size_t)sk * p.B * p.H * p.N * p.d * sizeof(float) : 0;
}

size_t bwd_workspace_bytes(int dtype, const Problem& p) {
  const size_t a = dq_workspace(dtype, p), b = dkdv_workspace(dtype, p);
  return a > b ? a : b;
}

hipError_t launch_dkdv(int dtype, const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                       const float* L, const float* Dv, void* dK, void* dV, hipStream_t s, void* workspace,
                       size_t workspace_bytes) {
  const size_t need = dkdv_workspace(dtype, p);
  const int ns = (need > 0 && workspace && workspace_bytes >= need) ? dkdv_splits(dtype, p) : 1;
  float* part = (float*)workspace;
#define X(T, DT, DD) \
  if (dtype == DT && p.d == DD) {                                                                  \
    if constexpr (DT == kF32) {                                                                     \
      return launch_dkdv_t<T, DD, 4, 32, 1>(p, Q, K, V, dO, L, Dv, dK, dV, s, ns, part);            \
    } else if constexpr (DD <= 80) {                                                                \
      return launch_dkdv_t<T, DD, 4, 64, 2>(p, Q, K, V, dO, L, Dv, dK, dV, s, ns, part);            \
    } else {                                                                                        \
      if (bwd_tiles(dtype, p).kt == 256)                                                            \
        return launch_dkdv_t<T, DD, 8, 64, 1, true>(p, Q, K, V, dO, L, Dv, dK, dV, s, ns, part);    \
      return launch_dkdv_t<T, DD, 4, 64, 1>(p, Q, K, V, dO, L, Dv, dK, dV, s, ns, part);            \
    }                                                                                               \
  }
  ATTN_BWD_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

// dQ tiles: 4 waves x 32 queries with 32-key tiles up to d = 80 (64-key tiles measured slower there);
// at d = 128, 8 waves (256 queries) share each 64-key K/V tile, which halves the K/V reads beyond L2
// per query at the same two waves per SIMD (B=1 H=36 N=16384: 3447 -> 3397 us in a same-box A/B).
hipError_t launch_dq(int dtype, const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                     const void* O, const float* L, float* Dv, void* dQ, hipStream_t s, void* workspace,
                     size_t workspace_bytes) {
  const size_t need = dq_workspace(dtype, p);
  const int ns = (need > 0 && workspace && workspace_bytes >= need) ? dq_splits(dtype, p) : 1;
  float* part = (float*)workspace;
#define X(T, DT, DD) \
  if (dtype == DT && p.d == DD) {                                                                  \
    if constexpr (DT == kF32) return launch_dq_t<T, DD, 4, 32, 1>(p, Q, K, V, dO, O, L, Dv, dQ, s, ns, part); \
    else if constexpr (DD <= 80) return launch_dq_t<T, DD, 4, 32, 2>(p, Q, K, V, dO, O, L, Dv, dQ, s, ns, part); \
    else return launch_dq_t<T, DD, 8, 64, 1>(p, Q, K, V, dO, O, L, Dv, dQ, s, ns, part);            \
  }
  ATTN_BWD_CASES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace attn
