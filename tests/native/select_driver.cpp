// Host driver for the per-block selection header: reads blocks of float
// scores from stdin, writes the keep bits of each block to stdout.
//   input:  m n count, then count*m floats
//   output: count unsigned integers
// With m = 0 it runs the 2:4 tournament instead (n ignored, blocks of 4):
// each line is the keep bits of the returned position code, then the
// positions of the two values it returned (values v[j] = j are passed in).
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

static void run_top2(int count) {
  std::vector<float> f((size_t)count * 4);
  for (auto& v : f)
    if (std::scanf("%f", &v) != 1) return;
  const float pos[4] = {0.f, 1.f, 2.f, 3.f};
  for (int b = 0; b < count; ++b) {
    const float s[4] = {f[4 * b], f[4 * b + 1], f[4 * b + 2], f[4 * b + 3]};
    float lo = -1.f, hi = -1.f;
    const uint32_t code = spa::top2of4(s, pos, lo, hi);
    const uint32_t keep = (1u << (code & 3u)) | (1u << ((code >> 2) & 3u));
    std::printf("%u %d %d %u\n", keep, (int)lo, (int)hi, code);
  }
}

int main() {
  int m, n, count;
  if (std::scanf("%d %d %d", &m, &n, &count) != 3) return 1;
  switch (m) {
    case 0: run_top2(count); break;
    case 4: run<4>(n, count); break;
    case 8: run<8>(n, count); break;
    case 16: run<16>(n, count); break;
    case 32: run<32>(n, count); break;
    default: return 2;
  }
  return 0;
}
