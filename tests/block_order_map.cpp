// Block -> work item maps of the attention kernels' launches, printed for the host-side check in
// test_block_order.py.  The maps come from the kernels' own header (csrc/block_order.h).
//
// Usage: block_order_map NHEADS NRANKS  ->  one line "b rank_major xcd" per block index b.
#include <cstdio>
#include <cstdlib>

#include "block_order.h"

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  const int nheads = std::atoi(argv[1]), nranks = std::atoi(argv[2]);
  for (int b = 0; b < nheads * nranks + 8; ++b)  // a few blocks past the end as well
    std::printf("%d %d %d\n", b, attn::rank_major_block(nheads, nranks, b), attn::xcd_block(nheads, nranks, b));
  return 0;
}
