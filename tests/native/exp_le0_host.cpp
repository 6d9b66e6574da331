// Host build of the library's float64 exponential (exp_le0, device.hpp) for
// the CPU test: the table 2^(j/64) from the host's exp2, then one line of
// output per x read from stdin, both as C99 hex floats.
#include <cmath>
#include <cstdio>

#include "../../vocab_row_reductions_amd/csrc/device.hpp"

int main() {
  double e2[64];
  for (int j = 0; j < 64; ++j) e2[j] = std::exp2((double)j / 64.0);
  double x;
  while (std::scanf("%la", &x) == 1) std::printf("%a\n", vsel::exp_le0(x, e2));
  return 0;
}
