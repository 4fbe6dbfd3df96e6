// Tiled attention forward with online softmax (gfx950).
//
// Computes, per (batch, head), O = softmax(mask(scale * Q K^T)) V and the row logsumexp
// L_i = log sum_j exp(S_ij) of the scaled, masked scores (natural log), following Algorithm 1
// ("FlashAttention-2 forward pass") of the CS336 Assignment 2 (systems) handout, §4.2.2, with
// the causal mask of its Problem (flash_forward)(c) and an optional per-batch key length.
//
// Work decomposition: one workgroup per (head, tile of 32*NW queries); wave w owns 32 queries.
// Each wave computes the transposed score block S^T = K Q^T (keys on MFMA rows, queries on
// columns), so each lane holds one query's scores and the row max / row sum are in-lane
// reductions plus a single exchange with the lane 32 away.  The probabilities are then fed
// straight from the accumulator as the B operand of O^T += V^T P^T, V^T being read from the
// row-major V tile with LDS transpose reads.  The exponentials run in the log2 domain with the
// softmax scale folded into one multiply.
//
// Rescaling is lazy: the running max used for exp2 is only moved when a new row max exceeds it
// by more than kRescaleSlack (log2 units), so most tiles skip the O rescale.  Any stale max is
// used consistently for the numerator and the denominator, so the result is unchanged (the
// largest unnormalised weight is bounded by 2^kRescaleSlack, far from overflow).
#include "attn_device.h"
#include "launch.h"

namespace attn {

constexpr float kRescaleSlack = 8.0f;
constexpr float kSumBound = 256.0f;  // 2^kRescaleSlack
// Head dims up to 64, where the softmax's vector work per key outweighs the matrix products, form
// the weights before taking the row max (see the tile loop); larger ones take the max first.
constexpr int kSumCheckMaxD = 64;
#ifndef ATTN_STORE_EARLY
#define ATTN_STORE_EARLY 1
#endif
constexpr bool kStoreEarly = ATTN_STORE_EARLY;
#ifndef ATTN_XCD_MAP
#define ATTN_XCD_MAP 1
#endif
constexpr bool kXcdMap = ATTN_XCD_MAP;
#ifndef ATTN_PIPELINE
#define ATTN_PIPELINE 1
#endif
constexpr bool kPipeline = ATTN_PIPELINE;

template <int V>
struct Flag {
  static constexpr int value = V;
};

// With SPLIT the key range of every query tile is cut into `nsplit` chunks, one workgroup each;
// a workgroup then writes its unnormalised O rows and their (running max, row sum) to `part`
// (layout: [nsplit][BH*N][D] floats, then [nsplit][BH*N][2] floats) instead of O and L, and
// fwd_combine_kernel merges the chunks with Algorithm 1's rescaling.
//
// With G = 2 the workgroup has two groups of NW waves over the same queries, and key tiles of
// 2 BK keys: group g takes keys [g BK, (g + 1) BK) of every tile, so each wave's chain of tiles is
// half as long (for grids too small to fill the chip, where that chain sets the time).  The two
// groups' (running max, row sum, unnormalised O) are merged through LDS at the end, with the same
// rescaling as between tiles.
template <typename T, int D, int NW, int BK, int OCC, bool BSP, bool SPLIT = false, int G = 1>
__global__ __launch_bounds__(G * NW * 64, OCC) void fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                           const T* __restrict__ V, T* __restrict__ O,
                                                           float* __restrict__ Lse, int BH, int H, int N,
                                                           int causal, float scale_log2,
                                                           const int32_t* __restrict__ kv_len,
                                                           const uint8_t* __restrict__ bmask, int nsplit,
                                                           float* __restrict__ part) {
  using M = Mfma<T>;
  constexpr int NT = G * NW * 64;         // threads of the workgroup
  constexpr int QT = 32 * NW;             // queries per workgroup
  constexpr int DP = (D + 31) / 32 * 32;  // head dim rounded up to a 32-row MFMA block
  constexpr int NDB = DP / 32;
  // bf16 head dims of 16 modulo 32 (16, 80): the last 16 output columns run on 16-wide products
  // (two 16 x 16 accumulators per wave, for its queries 0-15 and 16-31) instead of a 32-row block
  // half of padding; NDA full 32-row blocks precede them.
  constexpr bool T16 = sizeof(T) == 2 && DP - D == 16;
  constexpr int NDA = T16 ? D / 32 : NDB;
  constexpr int KS = D / M::KSTEP;
  constexpr int NB = BK / 32;             // key blocks per wave and tile
  constexpr int BKT = G * BK;             // keys per tile
  // K tiles are only read as 32-row operands (padded rows at lds_pitch, conflict-free for those
  // reads); V tiles only transposed (TransTile, conflict-free for those).
  constexpr int LD = lds_pitch<T, DP>();           // LDS row stride of K tiles (elements)
  using SV = TransTile<T, D>;
  constexpr int TILE = BKT * LD * (int)sizeof(T);  // bytes of one K tile
  constexpr int TILEV = SV::bytes(BKT);            // bytes of one V tile
  constexpr int STG = TILE + TILEV;                // bytes of one stage (K tile, then V tile)
  constexpr int SHIFT = BK == 64 ? 0 : 1;          // key tiles per mask block = 1 << SHIFT
  static_assert(D % M::KSTEP == 0, "head dim must be a multiple of the MFMA reduction depth");
  static_assert(!BSP || (QT % kMaskBlock == 0 && QT / kMaskBlock <= 8 && (BK == 32 || BK == 64)),
                "block-sparse tiles must nest in the 64 x 64 mask blocks");
  static_assert(G == 1 || (G == 2 && BK == 64 && !BSP && !SPLIT), "two key groups: dense, unsplit, BK = 64");

  // Two stages of (K tile, V tile): the next tile is written while the current one is read; then,
  // for block-sparse calls, one byte per mask column (which of this workgroup's rows see it).
  __shared__ __attribute__((aligned(16))) char smem[2 * STG + (BSP ? kMaxMaskBlocks : 0)];
  lds_t* lds = (lds_t*)smem;
  lds_t* map = lds + 2 * STG;

  const int TQ = (N + QT - 1) / QT;
  const int nsp = SPLIT ? nsplit : 1;
  const int logical = kXcdMap ? xcd_block(BH, TQ * nsp, blockIdx.x) : rank_major_block(BH, TQ * nsp, blockIdx.x);
  if (logical < 0) return;
  const int split = logical % nsp;
  const int bh = logical / nsp / TQ;
  const int qt = TQ - 1 - logical / nsp % TQ;  // heaviest (causal) tiles of a head first
  const int b = bh / H;
  int kv = N;
  if (kv_len) kv = min(max(kv_len[b], 1), N);

  const size_t base = (size_t)bh * N * D;
  O += base;
  Lse += (size_t)bh * N;

  const int grp = G == 1 ? 0 : (int)(threadIdx.x >> 6) / NW;  // key group (G = 2) or 0
  const int w = G == 1 ? (int)(threadIdx.x >> 6) : (int)(threadIdx.x >> 6) % NW, l = lane_id(), half = l >> 5, col = l & 31;
  const int q0 = qt * QT;
  const int qw = q0 + 32 * w;  // first query of this wave
  const int q = qw + col;      // this lane's query
  const int qw_last = min(qw + 31, N - 1);
  const bool wave_live = qw < N;
  // Last key this lane's query may see (the mask is "key > lim").
  const int lim = causal ? min(q, kv - 1) : kv - 1;
  const unsigned wave_bit = 1u << ((32 * w) / kMaskBlock);  // this wave's mask row within the workgroup

  int kend = kv;
  if (causal) kend = min(kend, q0 + QT);
  const int nkt = (kend + BKT - 1) / BKT;
  // This workgroup's key tiles [t_lo, t_hi): all of them, or one of nsplit equal chunks.
  const int chunk = (nkt + nsp - 1) / nsp;
  const int t_lo = SPLIT ? min(nkt, split * chunk) : 0;
  const int t_hi = SPLIT ? min(nkt, t_lo + chunk) : nkt;

  const auto rq = make_rsrc(Q + base, (uint32_t)(N * D * sizeof(T)));
  const auto rk = make_rsrc(K + base, (uint32_t)(kend * D * sizeof(T)));  // keys >= kend read as 0
  const auto rv = make_rsrc(V + base, (uint32_t)(kend * D * sizeof(T)));

  // With two key groups both groups need the same Q fragments: the workgroup's Q rows are then
  // copied with contiguous loads into the second stage's K slot (free until the first iteration
  // refills it) and the fragments read from there, rather than each group reading them in fragment
  // layout from memory (16 bytes from each of 32 rows per load instruction).
  constexpr bool STQ = G == 2;
  typename M::frag qf[KS];
  TileCopy<T, STQ ? QT : 1, STQ ? D : 16 / (int)sizeof(T), LD, NT> qst;
  if constexpr (STQ) {
    static_assert(QT <= BKT, "Q rows fit in a K slot");
    qst.load(rq, q0);
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = frag_global<T>(rq, q, D, ks * M::KSTEP);
  }

  f32x16 o[NDA > 0 ? NDA : 1];
#pragma unroll
  for (int i = 0; i < NDA; ++i) o[i] = f32x16{};
  f32x4 ot[2] = {};  // T16: O^T columns 32 NDA .. D - 1 of queries 0-15 and 16-31
  // Rescale the 16-wide accumulators by each query's factor (a: this lane's query's).
  auto scale_tail = [&](float a) {
    if constexpr (T16) {
      float lo, hi;
      split16(a, lo, hi);
      ot[0] *= lo;
      ot[1] *= hi;
    }
  };
  float m_run = -INFINITY, l_part = 0.f;
  bool first = true;  // no tile run yet: the running max starts from the first tile's max

  if constexpr (DP > D && !T16) {
    zero_pad_stage<SV, T, BKT, D, NT>(lds + TILE);
    zero_pad_stage<SV, T, BKT, D, NT>(lds + STG + TILE);
  }
  // Key tiles in loop order: all of [0, nkt), or (block-sparse) those some row of this workgroup
  // may see; the current, next and next-but-one tiles are tracked for the two-stage pipeline.
  int cur = t_lo;
  if constexpr (BSP) {
    build_tile_map(map, bmask, (N + kMaskBlock - 1) / kMaskBlock, q0 / kMaskBlock, QT / kMaskBlock, false, NT);
    __syncthreads();
    cur = next_live_tile(map, t_lo, t_hi, SHIFT);
  }
  auto after = [&](int t) { return BSP ? next_live_tile(map, t + 1, t_hi, SHIFT) : t + 1; };
  TileCopy<T, BKT, D, LD, NT> kc;
  TileCopy<T, BKT, D, SV::LD, NT> vc;
  auto store_v = [&](lds_t* dst) { vc.template store_to<SV>(dst); };
  const TileReader<T, SV> vr(T16);

  // Software-pipelined tiles (bf16, d = 128, dense, unsplit).  The key tiles [0, tp) that no mask
  // touches (every key below the workgroup's first query and below the key length) run with three
  // tiles in flight per straight-line iteration: iteration j forms the scores of tile j + 1, the
  // softmax of tile j (scores from the previous iteration) and the P V product of tile j - 1
  // (weights from the previous iteration).  The three parts are independent, so one wave can
  // issue the vector work of a softmax while its own matrix products run.  K runs one tile ahead
  // of V: iteration j writes K(j + 2) and V(j) into stage j & 1 and reads K(j + 1) and V(j - 1)
  // from stage (j + 1) & 1; the barrier ending an iteration publishes its writes and retires its
  // reads.  O is rescaled for tile j's max after tile j - 1's product, so every value is computed
  // in the same order as in the plain loop below, which takes over at tile tp.
  constexpr bool PIPE = kPipeline && sizeof(T) == 2 && D == 128 && G == 1 && !BSP && !SPLIT;
  int it0 = 0;        // stage parity of the plain loop's first iteration
  bool piped = false;  // the plain loop starts with its first tile staged and the next one loaded
  if constexpr (PIPE) {
    const int tp = min(causal ? q0 / BKT : nkt, kv / BKT);
    if (tp >= 2) {
      piped = true;
      // Two register sets, used alternately by even and odd iterations (unrolled by two, so every
      // index is static): scores of the current / next tile, weights of the current / previous.
      f32x16 sa[2][NB];
      typename M::frag pa[2][NB][M::CALLS32];
      auto scores_at = [&](const lds_t* kt, f32x16* s) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          s[nb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            s[nb] = M::mma(M::frag_direct(kt, LD, nb * 32 * LD + ks * M::KSTEP), qf[ks], s[nb]);
        }
      };
      auto pv_at = [&](const lds_t* vt, const typename M::frag (*pp)[M::CALLS32]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int c = 0; c < M::CALLS32; ++c)
#pragma unroll
            for (int db = 0; db < NDA; ++db) o[db] = M::mma(vr.trans(vt, nb * 32, db, c), pp[nb][c], o[db]);
      };
      // Iteration j (par = j & 1: the loop is unrolled by two, so the register set and the stage
      // each iteration uses are static).
      auto step = [&](int j, auto has_prev, auto has_next, auto par) {
        constexpr int P = decltype(par)::value;
        f32x16* sc = sa[P];
        f32x16* sn = sa[P ^ 1];
        typename M::frag(*pc)[M::CALLS32] = pa[P];
        lds_t* wr = lds + P * STG;
        const lds_t* rd = lds + (P ^ 1) * STG;
        kc.store(wr);        // K(j + 2)
        store_v(wr + TILE);  // V(j)
        kc.load(rk, min(j + 3, tp + 1) * BKT);
        vc.load(rv, (j + 1) * BKT);
        if constexpr (decltype(has_next)::value) scores_at(rd, sn);
        // Softmax of tile j: row max, the running max moved when exceeded by more than the slack.
        float mx = sc[0][0];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int e = (nb == 0 ? 1 : 0); e < 16; ++e) mx = fmaxf(mx, sc[nb][e]);
        mx = fmaxf(mx, swap_halves(mx)) * scale_log2;
        const bool need = mx > m_run + kRescaleSlack;
        const float alpha = fast_exp2(m_run - mx);
        l_part = need ? l_part * alpha : l_part;
        m_run = need ? mx : m_run;
        const float neg_m = -m_run;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int e = 0; e < 16; ++e) sc[nb][e] = fast_exp2(__builtin_fmaf(sc[nb][e], scale_log2, neg_m));
          float lsum = 0.f;
#pragma unroll
          for (int c = 0; c < M::CALLS32; ++c) {
            pc[nb][c] = M::acc_frag(sc[nb], c);
            lsum = M::frag_sum(pc[nb][c], lsum);
          }
          l_part += lsum;
        }
        if constexpr (decltype(has_prev)::value) pv_at(rd + TILE, pa[P ^ 1]);
        // The weights are formed before the rescale branch, so their vector work shares a block
        // with the products.  (The row sums are left to the compiler, which places their dot2s
        // after it: beside busy matrix cores a dot2 costs several times a plain add.)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int c = 0; c < M::CALLS32; ++c) settle(pc[nb][c]);
        if (need) {
#pragma unroll
          for (int i = 0; i < NDA; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
        }
        __syncthreads();
      };
      // Prologue: K(0) and K(1) staged, V(0) and K(2) in registers, tile 0's scores formed.
      TileCopy<T, BKT, D, LD, NT> kc2;
      kc.load(rk, 0);
      kc2.load(rk, BKT);
      vc.load(rv, 0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) settle(qf[ks]);
      kc.store(lds);
      kc2.store(lds + STG);
      kc.load(rk, 2 * BKT);
      __syncthreads();
      scores_at(lds, sa[0]);
      __syncthreads();  // stage 0's K slot is rewritten by iteration 0
      const Flag<1> yes;
      const Flag<0> no;
      // Tile tp - 1's product (its weights and V(tp - 1) in register set / stage P = (tp - 1) & 1);
      // V(tp) completes stage tp & 1 for the plain loop, which finds the next tile (K(tp + 1),
      // V(tp + 1)) in registers.
      auto drain = [&](auto par) {
        constexpr int P = decltype(par)::value;
        store_v(lds + (P ^ 1) * STG + TILE);
        vc.load(rv, (tp + 1) * BKT);
        pv_at(lds + P * STG + TILE, pa[P]);
        __syncthreads();
      };
      step(0, no, yes, no);
      int j = 1;
      for (; j + 2 < tp; j += 2) {
        step(j, yes, yes, yes);
        step(j + 1, yes, yes, no);
      }
      if (j == tp - 1) {
        step(j, yes, no, yes);
        drain(yes);
      } else {
        step(j, yes, yes, yes);
        step(j + 1, yes, no, no);
        drain(no);
      }
      cur = tp;
      it0 = tp;
      first = false;
    }
  }

  if (!piped) {
    if (cur < t_hi) {
      kc.load(rk, cur * BKT);
      vc.load(rv, cur * BKT);
    }
    // The Q fragments (or rows) were requested first: waiting for them here leaves the first K/V
    // tile's loads in flight, so the two memory latencies overlap.
    if constexpr (STQ) {
      qst.store(lds + STG);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) settle(qf[ks]);
    }
    if (cur < t_hi) {
      kc.store(lds);
      store_v(lds + TILE);
    }
    __syncthreads();
    if constexpr (STQ) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = M::frag_direct(lds + STG, LD, 32 * w * LD + ks * M::KSTEP);
      __syncthreads();  // every wave holds its fragments before the first iteration refills the slot
    }
  }
  int nxt = cur < t_hi ? after(cur) : t_hi;
  if (!piped && nxt < t_hi) {
    kc.load(rk, nxt * BKT);
    vc.load(rv, nxt * BKT);
  }
  // Where the next tile is written to LDS: at the start of each iteration (d = 128, where it was
  // measured faster: the writes overlap the tile's products) or right before the barrier.
  constexpr bool EARLY = kStoreEarly && D > 80;

  for (int it = it0; cur < t_hi; ++it) {
    int nxt2 = t_hi;
    if constexpr (EARLY) {
      // The next tile (loaded one iteration ago) goes to LDS at the start of the iteration, into
      // the stage every wave finished reading before the last barrier, so the LDS writes overlap
      // this tile's products instead of stalling every wave right before the barrier.
      nxt2 = nxt < t_hi ? after(nxt) : t_hi;
      if (nxt < t_hi) {
        lds_t* st = lds + ((it + 1) & 1) * STG;
        kc.store(st);
        store_v(st + TILE);
      }
      if (nxt2 < t_hi) {
        kc.load(rk, nxt2 * BKT);
        vc.load(rv, nxt2 * BKT);
      }
    }
    // This group's keys of the tile: rows grp * BK .. grp * BK + BK - 1 of the staged K and V.
    const lds_t* ktile = lds + (it & 1) * STG + grp * BK * LD * (int)sizeof(T);
    const lds_t* vtile = lds + (it & 1) * STG + TILE + SV::block(grp * BK);
    const int k0 = cur * BKT + grp * BK;
    // (k0 is a multiple of 64 and qw of 32, so a wave that runs has key k0 visible in every row.)
    bool run = wave_live && k0 < kend && !(causal && k0 > qw_last);
    if constexpr (BSP) run = run && (tile_bits(map, cur, SHIFT) & wave_bit);
    if (run) {
      // Scores of this wave's keys of the tile (raw, unscaled); masked ones replaced (only on
      // tiles that cross the diagonal or the key end).
      f32x16 s[NB];
      auto scores = [&]() {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          s[nb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            s[nb] = M::mma(M::frag_direct(ktile, LD, nb * 32 * LD + ks * M::KSTEP), qf[ks], s[nb]);
        }
        if ((causal && k0 + BK - 1 > qw) || k0 + BK > kv) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              s[nb][e] = (k0 + nb * 32 + acc_row(e, half) > lim) ? kMaskedScore : s[nb][e];
        }
      };
      // Row max of key blocks [nb0, nb1); the running max moves (and O, l are rescaled) when it
      // exceeds the running max by more than the slack.
      auto move_max = [&](int nb0, int nb1) {
        float mx = s[nb0][0];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          if (nb >= nb0 && nb < nb1)
#pragma unroll
            for (int e = (nb == nb0 ? 1 : 0); e < 16; ++e) mx = fmaxf(mx, s[nb][e]);
        mx = fmaxf(mx, swap_halves(mx)) * scale_log2;
        const bool need = mx > m_run + kRescaleSlack;
        float a = 1.f;
        if (need) {
          const float alpha = fast_exp2(m_run - mx);
#pragma unroll
          for (int i = 0; i < NDA; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
          l_part *= alpha;
          m_run = mx;
          a = alpha;
        }
        // The 16-wide accumulators hold other lanes' queries: rescaled by all lanes together.
        if constexpr (T16)
          if (__ballot(need) != 0) scale_tail(a);
      };
      // Unnormalised weights 2^(s scale_log2 - m_run) of key block nb as MFMA operands, and this
      // lane's part of their row sum (bf16: the sum of the rounded weights the product uses, two
      // per dot2).
      typename M::frag pf[M::CALLS32];
      float lsum;
      auto weights = [&](int nb) {
        const float neg_m = -m_run;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[nb][e] = fast_exp2(__builtin_fmaf(s[nb][e], scale_log2, neg_m));
        lsum = 0.f;
#pragma unroll
        for (int c = 0; c < M::CALLS32; ++c) {
          pf[c] = M::acc_frag(s[nb], c);
          lsum = M::frag_sum(pf[c], lsum);
        }
      };
      scores();
      // Head dims above kSumCheckMaxD, and a wave's first tile, take the tile's row max first.
      // Otherwise each key block's weights are formed with the running max as it stands: a lane
      // whose weights sum to at most 2^kRescaleSlack has every weight within that bound, which is
      // all the running max must guarantee, so the block's max is only taken (and the max moved)
      // when some lane exceeds it or overflowed -- the scores of that block are then recomputed.
      const bool check = !first && D <= kSumCheckMaxD;
      if (first || D > kSumCheckMaxD) {
        move_max(0, NB);
        first = false;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        weights(nb);
        if (check && __ballot(!(lsum <= kSumBound)) != 0) {
          // Re-read the K fragments rather than keep the first reads live through the fast path.
          int fresh = 0;
          asm volatile("" : "+v"(fresh));
          const lds_t* kt = ktile + fresh;
          s[nb] = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            s[nb] = M::mma(M::frag_direct(kt, LD, nb * 32 * LD + ks * M::KSTEP), qf[ks], s[nb]);
          if ((causal && k0 + BK - 1 > qw) || k0 + BK > kv) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              s[nb][e] = (k0 + nb * 32 + acc_row(e, half) > lim) ? kMaskedScore : s[nb][e];
          }
          move_max(nb, nb + 1);
          weights(nb);
        }
        l_part += lsum;
#pragma unroll
        for (int c = 0; c < M::CALLS32; ++c)
#pragma unroll
          for (int db = 0; db < NDA; ++db)
            o[db] = M::mma(vr.trans(vtile, nb * 32, db, c), pf[c], o[db]);
        if constexpr (T16) {
          typename M::frag lo, hi;
          M::tail_weights(pf[0], pf[1], lo, hi);
          const typename M::frag vt = vr.trans16(vtile, nb * 32, 32 * NDA);
          ot[0] = M::mma16(vt, lo, ot[0]);
          ot[1] = M::mma16(vt, hi, ot[1]);
        }
      }
    }
    if constexpr (EARLY) {
      __syncthreads();
    } else {
      nxt2 = nxt < t_hi ? after(nxt) : t_hi;
      if (nxt < t_hi) {
        lds_t* st = lds + ((it + 1) & 1) * STG;
        kc.store(st);
        store_v(st + TILE);
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
    // Group 1 hands (m, l, O) to the wave of group 0 that owns the same queries; the tiles are no
    // longer read (the loop ended on a barrier and staged nothing after it).
    constexpr int F = 2 + 16 * NDA + (T16 ? 8 : 0);  // floats per lane
    static_assert(NW * 64 * F * 4 <= 2 * STG, "merge buffer fits in the tile stages");
    float* mrg = reinterpret_cast<float*>(smem) + w * F * 64 + l;
    if (grp == 1) {
      mrg[0] = m_run;
      mrg[64] = l_part;
#pragma unroll
      for (int i = 0; i < NDA; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) mrg[(2 + 16 * i + e) * 64] = o[i][e];
      if constexpr (T16)
#pragma unroll
        for (int e = 0; e < 8; ++e) mrg[(2 + 16 * NDA + e) * 64] = ot[e >> 2][e & 3];
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = mrg[0], l1 = mrg[64];
    const float m = fmaxf(m_run, m1);
    // A group that saw no key of this row has m = -inf and contributes nothing.
    const float a0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - m);
#pragma unroll
    for (int i = 0; i < NDA; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[i][e] = o[i][e] * a0 + mrg[(2 + 16 * i + e) * 64] * a1;
    if constexpr (T16) {
      float a0l, a0h, a1l, a1h;
      split16(a0, a0l, a0h);
      split16(a1, a1l, a1h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ot[0][e] = ot[0][e] * a0l + mrg[(2 + 16 * NDA + e) * 64] * a1l;
        ot[1][e] = ot[1][e] * a0h + mrg[(2 + 16 * NDA + 4 + e) * 64] * a1h;
      }
    }
    l_part = l_part * a0 + l1 * a1;
    m_run = m;
  }
  const float l_tot = l_part + swap_halves(l_part);
  // T16: lane l holds output columns d16 .. d16 + 3 of queries q16 and q16 + 16.
  const int q16 = qw + (l & 15), d16 = 32 * NDA + 4 * (l >> 4);
  if constexpr (SPLIT) {
    // Unnormalised partial: sum_j exp2(s_j - m) v_j, with m and sum_j exp2(s_j - m) beside it.
    const size_t prow0 = (size_t)split * BH * N + (size_t)bh * N;
    if constexpr (T16) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
        if (q16 + 16 * x < N) *reinterpret_cast<f32x4*>(part + (prow0 + q16 + 16 * x) * D + d16) = ot[x];
    }
    if (q < N) {
      const size_t row = prow0 + q;
      float* prow = part + row * D;
#pragma unroll
      for (int db = 0; db < NDA; ++db)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int d0 = db * 32 + 8 * m + 4 * half;
          if (D % 32 == 0 || d0 < D) {
            f32x4 v4;
#pragma unroll
            for (int r = 0; r < 4; ++r) v4[r] = o[db][4 * m + r];
            *reinterpret_cast<f32x4*>(prow + d0) = v4;
          }
        }
      if (half == 0) {
        float* ml = part + (size_t)nsplit * BH * N * D + row * 2;
        ml[0] = m_run;
        ml[1] = l_tot;
      }
    }
    return;
  }
  // A block-sparse mask can leave a row without keys: O = 0 and L = -inf there.
  const float inv = (BSP && !(l_tot > 0.f)) ? 0.f : 1.0f / l_tot;
  if constexpr (T16) {
    float inv2[2];
    split16(inv, inv2[0], inv2[1]);
#pragma unroll
    for (int x = 0; x < 2; ++x)
      if (q16 + 16 * x < N) {
        T v4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = (T)(ot[x][r] * inv2[x]);
        uint2 u;
        __builtin_memcpy(&u, v4, 8);
        *reinterpret_cast<uint2*>(O + (size_t)(q16 + 16 * x) * D + d16) = u;
      }
  }
  if (q < N) {
    T* orow = O + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < NDA; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d0 = db * 32 + 8 * m + 4 * half;
        if (D % 32 == 0 || d0 < D) {
          T v4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v4[r] = (T)(o[db][4 * m + r] * inv);
          if constexpr (sizeof(T) == 2) {
            uint2 u;
            __builtin_memcpy(&u, v4, 8);
            *reinterpret_cast<uint2*>(orow + d0) = u;
          } else {
            uint4 u;
            __builtin_memcpy(&u, v4, 16);
            *reinterpret_cast<uint4*>(orow + d0) = u;
          }
        }
      }
    if (half == 0) Lse[q] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

// Merge the nsplit partials of every row: with m = max_s m_s, O = sum_s 2^(m_s - m) O_s /
// sum_s 2^(m_s - m) l_s and L = (m + log2 sum_s 2^(m_s - m) l_s) ln 2 -- the same rescaling
// Algorithm 1 applies between key tiles.  Rows whose chunks saw no key give O = 0, L = -inf.
// One thread per 4 consecutive columns of a row.
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(const float* __restrict__ part, int nsplit, int rows,
                                                          T* __restrict__ O, float* __restrict__ Lse) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int t = threadIdx.x;
  if (t >= RPB * TPR) return;
  const int row = blockIdx.x * RPB + t / TPR;
  const int c = 4 * (t % TPR);
  if (row >= rows) return;
  const float* ml = part + (size_t)nsplit * rows * D;
  float m = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, ml[((size_t)sp * rows + row) * 2]);
  float lsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (m > -INFINITY) {
    for (int sp = 0; sp < nsplit; ++sp) {
      const size_t r = (size_t)sp * rows + row;
      const float w = fast_exp2(ml[r * 2] - m);  // 0 for an empty chunk (its m is -inf)
      lsum += w * ml[r * 2 + 1];
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + r * D + c);
      acc += w * v;
    }
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  T v4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v4[r] = (T)(acc[r] * inv);
  if constexpr (sizeof(T) == 2) {
    uint2 u;
    __builtin_memcpy(&u, v4, 8);
    *reinterpret_cast<uint2*>(O + (size_t)row * D + c) = u;
  } else {
    uint4 u;
    __builtin_memcpy(&u, v4, 16);
    *reinterpret_cast<uint4*>(O + (size_t)row * D + c) = u;
  }
  if (c == 0) Lse[row] = lsum > 0.f ? (m + fast_log2(lsum)) * kLn2 : -INFINITY;
}

// Two key groups per workgroup (fwd_kernel's G = 2) when the grid of 128-query workgroups is at
// most one per CU and the longest key chain has at least four 64-key tiles: each CU then runs
// one workgroup, whose chain the second group halves.  Measured on MI355X with the heaviest-first
// work order: B=4 H=12 N=512 d=64 11.1 -> 9.4 us, B=2 H=16 N=1024 d=64 18.1 -> 14.2 us (with
// 64-query workgroups, two per CU, at d <= 64; 128-query ones gave 10.5 and 16.2 us).
static bool fwd_two_groups(const Problem& p, long items) {
  return items <= 256 && p.N >= 256;
}

template <typename T, int D, int NW, int BK, int OCC>
static hipError_t launch_fwd_t(const Problem& p, const void* Q, const void* K, const void* V, void* O,
                               float* L, hipStream_t stream, int nsplit = 1, float* part = nullptr) {
  constexpr int QT = 32 * NW;
  const int TQ = (p.N + QT - 1) / QT;
  const float sl2 = p.scale * kLog2e;
  const int BH = p.B * p.H;
  if (nsplit > 1) {
    // Split grids are small (a few workgroups per CU at most): at most two workgroups per CU are
    // asked for, which leaves the register budget of the d = 64 kernel room to avoid spills.
    constexpr int OCCS = OCC > 2 ? 2 : OCC;
    const int grid = BH * TQ * nsplit;
    if (p.bmask)
      hipLaunchKernelGGL((fwd_kernel<T, D, NW, BK, OCCS, true, true>), dim3(grid), dim3(NW * 64), 0, stream,
                         (const T*)Q, (const T*)K, (const T*)V, (T*)O, L, BH, p.H, p.N, p.causal, sl2, p.kv_len,
                         p.bmask, nsplit, part);
    else
      hipLaunchKernelGGL((fwd_kernel<T, D, NW, BK, OCCS, false, true>), dim3(grid), dim3(NW * 64), 0, stream,
                         (const T*)Q, (const T*)K, (const T*)V, (T*)O, L, BH, p.H, p.N, p.causal, sl2, p.kv_len,
                         nullptr, nsplit, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int RPB = 256 / (D / 4);
    const int rows = BH * p.N;
    hipLaunchKernelGGL((fwd_combine_kernel<T, D>), dim3((rows + RPB - 1) / RPB), dim3(256), 0, stream,
                       (const float*)part, nsplit, rows, (T*)O, L);
    return hipGetLastError();
  }
  const int grid = BH * TQ;
  if constexpr (sizeof(T) == 2 && BK == 64) {
    if (!p.bmask && fwd_two_groups(p, (long)BH * ((p.N + 127) / 128))) {
      // Up to d = 64 two such workgroups fit a CU: 64-query workgroups then spread the heaviest
      // query tiles over twice as many CUs.
      constexpr int NW2 = D <= 64 ? 2 : 4;
      const int grid2 = BH * ((p.N + 32 * NW2 - 1) / (32 * NW2));
      hipLaunchKernelGGL((fwd_kernel<T, D, NW2, BK, D <= 64 ? 2 : 1, false, false, 2>), dim3(grid2),
                         dim3(2 * NW2 * 64), 0, stream, (const T*)Q, (const T*)K, (const T*)V, (T*)O, L, BH, p.H,
                         p.N, p.causal, sl2, p.kv_len, nullptr, 1, nullptr);
      return hipGetLastError();
    }
  }
  if (p.bmask)
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, BK, OCC, true>), dim3(grid), dim3(NW * 64), 0, stream, (const T*)Q,
                       (const T*)K, (const T*)V, (T*)O, L, BH, p.H, p.N, p.causal, sl2, p.kv_len, p.bmask, 1,
                       nullptr);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, BK, OCC, false>), dim3(grid), dim3(NW * 64), 0, stream, (const T*)Q,
                       (const T*)K, (const T*)V, (T*)O, L, BH, p.H, p.N, p.causal, sl2, p.kv_len, nullptr, 1,
                       nullptr);
  return hipGetLastError();
}

// Key chunks per query tile for the split forward.  Measured on MI355X: splitting pays when the
// grid has fewer than ~4 query-tile workgroups per CU and the longest key chain is long (at least
// 32 key tiles in bfloat16, 8 in float32, whose tiles cost about four times as much); below that
// the partial writes and the merge launch cost more than they save (B=4, H=12, N=512 runs 1.6x
// slower split).  Chunks hold at least four key tiles of the longest chain; at most kMaxSplits.
int fwd_splits(int dtype, const Problem& p) {
  const long items = (long)p.B * p.H * ((p.N + 127) / 128);
  const int bk = dtype == kBF16 ? 64 : 32;
  const int nkt_max = (p.N + bk - 1) / bk;
  if (items >= 1024 || nkt_max < (dtype == kBF16 ? 32 : 8)) return 1;
  int s = (int)((1280 + items - 1) / items);
  s = s > kMaxSplits ? kMaxSplits : s;
  s = s > nkt_max / 4 ? nkt_max / 4 : s;
  return s >= 2 ? s : 1;
}

size_t fwd_workspace_bytes(int dtype, const Problem& p) {
  const int s = fwd_splits(dtype, p);
  return s > 1 ? (size_t)s * p.B * p.H * p.N * (p.d + 2) * sizeof(float) : 0;
}

bool fwd_supported(int dtype, int d) {
  (void)dtype;
  return d == 16 || d == 32 || d == 64 || d == 80 || d == 128;
}

hipError_t launch_fwd(int dtype, const Problem& p, const void* Q, const void* K, const void* V, void* O,
                      float* L, hipStream_t s, void* workspace, size_t workspace_bytes) {
  // The split path runs only with a workspace large enough for its partials.
  const size_t need = fwd_workspace_bytes(dtype, p);
  const int ns = (need > 0 && workspace && workspace_bytes >= need) ? fwd_splits(dtype, p) : 1;
  float* part = (float*)workspace;
  if (dtype == kBF16) {
    switch (p.d) {
      case 16: return launch_fwd_t<__bf16, 16, 4, 64, 4>(p, Q, K, V, O, L, s, ns, part);
      case 32: return launch_fwd_t<__bf16, 32, 4, 64, 4>(p, Q, K, V, O, L, s, ns, part);
      case 64: return launch_fwd_t<__bf16, 64, 4, 64, 4>(p, Q, K, V, O, L, s, ns, part);
      case 80: return launch_fwd_t<__bf16, 80, 4, 64, 2>(p, Q, K, V, O, L, s, ns, part);
      // d = 128: 8-wave workgroups (256 queries) share one K/V stream, which halves the K/V reads
      // beyond L2 per query; register use allows 2 waves per SIMD either way.  Measured on the
      // B=1 H=36 N=16384 workload: 2546 -> 2472 us (at d = 80 the same change was slower).
      case 128: return launch_fwd_t<__bf16, 128, 8, 64, 1>(p, Q, K, V, O, L, s, ns, part);
    }
  } else if (dtype == kF32) {
    switch (p.d) {
      case 16: return launch_fwd_t<float, 16, 4, 32, 1>(p, Q, K, V, O, L, s, ns, part);
      case 32: return launch_fwd_t<float, 32, 4, 32, 1>(p, Q, K, V, O, L, s, ns, part);
      case 64: return launch_fwd_t<float, 64, 4, 32, 1>(p, Q, K, V, O, L, s, ns, part);
      case 80: return launch_fwd_t<float, 80, 4, 32, 1>(p, Q, K, V, O, L, s, ns, part);
      case 128: return launch_fwd_t<float, 128, 4, 32, 1>(p, Q, K, V, O, L, s, ns, part);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace attn
