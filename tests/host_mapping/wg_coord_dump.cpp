// Prints, one line per workgroup id, the (request, split, head group) that
// the decode kernels' workgroup order (wg_coord) gives it, for a grid of
// batch * num_splits * n_hg workgroups.  Built for the host only: the test
// that runs it checks the order is a bijection and that the host-side split
// policy counts the same busy workgroups per XCD.
#include <cstdio>
#include <cstdlib>

#include "decode_ws.h"

int main(int argc, char** argv) {
  if (argc != 5) {
    std::fprintf(stderr, "usage: %s batch num_splits n_hg spread\n", argv[0]);
    return 2;
  }
  const int batch = std::atoi(argv[1]), num_splits = std::atoi(argv[2]), n_hg = std::atoi(argv[3]);
  const bool spread = std::atoi(argv[4]) != 0;
  const int n = batch * num_splits * n_hg;
  for (int bid = 0; bid < n; ++bid) {
    const spmla::ws::WgCoord c = spmla::ws::wg_coord(bid, n, num_splits, n_hg, spread);
    std::printf("%d %d %d\n", c.b, c.s, c.hg);
  }
  return 0;
}
