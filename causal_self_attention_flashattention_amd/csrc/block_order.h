// Order in which the workgroups of a launch take their work items (plain constexpr integer
// arithmetic, shared by the kernels and a host-side check).
//
// A launch's grid covers nheads x nranks work items, item h * nranks + r being rank r of head h; a
// head's ranks are numbered heaviest first by the callers (under causal masking, the query tiles
// that see the most keys, the key tiles that see the most queries).  The functions map a block
// index b to its item, or -1 for blocks past the last item.
#pragma once

#if defined(__HIPCC__)
#define ATTN_BO_HD __host__ __device__
#else
#define ATTN_BO_HD
#endif

namespace attn {

// Rank-major: blocks 0 .. nheads - 1 take rank 0 of every head, the next nheads blocks rank 1, and
// so on, so the heavy items of all heads start first and the light ones fill in at the end instead
// of a late head's heaviest tile setting the time.  The 8 XCDs receive blocks round-robin: with
// nheads a multiple of 8 every item of a head lands on one XCD and shares the head's K/V in that
// XCD's L2; otherwise xcd_block below keeps the heads on as few XCDs as the balance allows.
ATTN_BO_HD constexpr int rank_major_block(int nheads, int nranks, int b) {
  return b >= nheads * nranks ? -1 : (b % nheads) * nranks + b / nheads;
}

// As rank_major_block, with each head's items kept on one XCD where that can be balanced.  Block b
// runs on XCD b % 8, in order b / 8 there, and each XCD has its own L2: the items of a head, which
// share its K and V rows, should run on one XCD.  With nheads = 8 hq + hr (0 < hr), XCD x takes
// whole heads x hq .. x hq + hq - 1 and a share of the hr remaining heads by rank: when hr divides
// 8, remaining head j goes to the 8 / hr XCDs j (8 / hr) + (r mod 8 / hr), each holding every
// (8 / hr)-th rank; otherwise rank r of remaining head j goes to XCD (r + j) mod 8.  Every XCD then
// holds the same number of items in every period of that split (8 / hr or 8 consecutive ranks), so
// the XCDs' causal work differs only by rank offsets within a period, and runs them rank-major,
// heaviest first.  (Running an XCD's heads one after another instead cuts the L2
// misses further but starts heavy items late: 8% slower at 36 heads, 14% at 80.)  The split needs
// nranks to be a multiple of its period (8 / hr, or 8); otherwise, and when nheads is a multiple of
// 8 (where rank-major order already keeps each head on one XCD), the order is rank_major_block.
// A bijection from [0, nheads nranks) onto the items.
ATTN_BO_HD constexpr int xcd_block(int nheads, int nranks, int b) {
  constexpr int NX = 8;
  const int hq = nheads / NX, hr = nheads % NX;
  const bool divides = hr > 0 && NX % hr == 0;
  const int T = divides ? NX / hr : NX;  // ranks per period of the split
  if (hr == 0 || nranks % T != 0 || b >= nheads * nranks) return rank_major_block(nheads, nranks, b);
  const int x = b % NX, i = b / NX;
  const int P = T * hq + (divides ? 1 : hr);  // items of XCD x per period
  const int p = i / P;
  int q = i % P;
  for (int rp = 0; rp < T; ++rp) {
    const int r = p * T + rp;
    int j = -1;  // remaining head that XCD x serves at rank r, or -1
    if (divides) {
      j = (r % T == x % T) ? x / T : -1;
    } else {
      j = ((x - r) % NX + NX) % NX;
      if (j >= hr) j = -1;
    }
    const int n = hq + (j >= 0 ? 1 : 0);
    if (q < n) return (q < hq ? x * hq + q : NX * hq + j) * nranks + r;
    q -= n;
  }
  return -1;  // not reached: the P items of a period are enumerated above
}

}  // namespace attn
