// Host driver for the per-block selection header: reads blocks of float
// scores from stdin, writes the keep bits of each block to stdout.
//   input:  m n count, then count*m floats
//   output: count unsigned integers
#include <cstdio>
#include <cstring>
#include <vector>

#include "spa_select.h"

template <int M>
static void run(int n, int count) {
  std::vector<float> f((size_t)count * M);
  for (auto& v : f)
    if (std::scanf("%f", &v) != 1) return;
  for (int b = 0; b < count; ++b) {
    uint32_t s[M];
    for (int j = 0; j < M; ++j) std::memcpy(&s[j], &f[(size_t)b * M + j], 4);
    std::printf("%u\n", spa::topn_keep_bits<M>(s, n));
  }
}

int main() {
  int m, n, count;
  if (std::scanf("%d %d %d", &m, &n, &count) != 3) return 1;
  switch (m) {
    case 4: run<4>(n, count); break;
    case 8: run<8>(n, count); break;
    case 16: run<16>(n, count); break;
    case 32: run<32>(n, count); break;
    default: return 2;
  }
  return 0;
}
