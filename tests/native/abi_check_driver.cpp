// Host-only sweep of the library's argument checks, prefill workspace layout,
// decode plan and per-block selection, meant to be built with AddressSanitizer
// and UndefinedBehaviorSanitizer: every function runs on a fixed pseudo-random
// set of valid and hostile arguments (zero, negative and 2^31 - 1 sizes, null
// and misaligned pointers, out-of-range enums), and the invariants below must
// hold.  Prints "ok <calls>" or the failures, and exits non-zero on any.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "spa.h"
#include "spa_check.h"
#include "spa_plan.h"
#include "spa_select.h"

namespace {

uint64_t g_state = 0x243F6A8885A308D3ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int g_fails = 0;
long g_calls = 0, g_accepted_decode = 0, g_accepted_prefill = 0;
#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond) && g_fails++ < 20) {                        \
      std::printf("fail %s:%d: ", __FILE__, __LINE__);      \
      std::printf(__VA_ARGS__);                             \
      std::printf("\n");                                    \
    }                                                       \
  } while (0)

int32_t pick_dim() {
  static const int32_t edge[] = {0, 1, 4, 15, 16, 32, 36, 64, 776, 4096, 14336, 16384, 262144, 1 << 23,
                                 (1 << 23) + 64, 1 << 24, (1 << 24) + 16, INT32_MAX, -1, -16, INT32_MIN};
  const uint64_t r = next_u64();
  if (r % 3 == 0) return edge[(r >> 8) % (sizeof(edge) / sizeof(edge[0]))];
  return (int32_t)((r >> 8) % 70000) - 16;
}
int32_t pick(int32_t lo, int32_t hi) { return lo + (int32_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

alignas(64) unsigned char g_buf[256];

// pointers: valid and 16-byte aligned, misaligned, or null
const void* pick_ptr() {
  const uint64_t r = next_u64() % 8;
  return r == 0 ? nullptr : r == 1 ? (const void*)(g_buf + 4) : (const void*)(g_buf + 16 * (r % 4));
}

// A valid call, then up to two fields replaced by hostile values.
void sweep_linear() {
  spa_prune_cfg c{};
  spa_weight w{};
  for (int it = 0; it < 300000; ++it) {
    std::memset(&c, 0, sizeof(c));
    const int32_t ms[] = {4, 8, 16, 32};
    c.m = ms[next_u64() % 4];
    c.n = pick(1, c.m);
    c.score = pick(0, 2);
    c.shift = pick(0, 2);
    c.var_rescale = pick(0, 2);
    c.act = pick(0, 1);
    c.var_state = (const float*)(g_buf + 64);
    c.var_state_out = (float*)(g_buf + 128);
    w.dtype = pick(0, 2);
    const int32_t kmax = next_u64() % 4 ? 65536 : (1 << 24);
    w.k = 64 * pick(1, kmax / 64);
    w.n_out = next_u64() % 2 ? 8 * pick(1, 4096) : pick(1, 1 << 24);
    w.w = w.wt = g_buf;
    w.chan_scale = w.row_sum = (const float*)(g_buf + 32);
    const bool decode = next_u64() & 1;
    int32_t t = decode ? pick(1, 32) : (next_u64() % 8 ? pick(0, 5000) : pick(0, 1 << 24));
    const void* x = g_buf;
    const void* y = g_buf + 16;
    const float* eta_in = (const float*)(g_buf + 48);
    const spa_prune_cfg* cp = &c;
    const int nmut = (int)(next_u64() % 3);
    for (int q = 0; q < nmut; ++q) {
      switch (next_u64() % 14) {
        case 0: c.m = pick(-4, 64); break;
        case 1: c.n = pick(-1, 40); break;
        case 2: c.score = pick(-2, 5); c.shift = pick(-2, 5); break;
        case 3: c.var_rescale = pick(-1, 3); c.var_state_out = (float*)c.var_state; break;
        case 4: c.act = pick(-1, 3); break;
        case 5: w.dtype = pick(-1, 4); break;
        case 6: w.k = pick_dim(); break;
        case 7: w.n_out = pick_dim(); break;
        case 8: t = pick_dim(); break;
        case 9: x = pick_ptr(); y = pick_ptr(); break;
        case 10: w.w = pick_ptr(); w.wt = pick_ptr(); break;
        case 11: w.chan_scale = (const float*)pick_ptr(); w.row_sum = (const float*)pick_ptr(); break;
        case 12: eta_in = (const float*)pick_ptr(); c.var_state = (const float*)pick_ptr(); break;
        default: cp = nullptr; break;
      }
    }
    const spa_status st = spa_check::check_linear(x, t, &w, cp, eta_in, y, decode);
    ++g_calls;
    EXPECT(st == SPA_OK || st == SPA_ERR_INVALID || st == SPA_ERR_UNSUPPORTED, "status %d", (int)st);
    if (st != SPA_OK) continue;
    // accepted: the shapes the kernels assume
    EXPECT(spa_check::valid_cfg(&c) && c.n >= 1 && c.n <= c.m, "cfg");
    EXPECT(w.k >= c.m && w.k % c.m == 0 && w.k % 16 == 0 && w.k <= (1 << 24), "k %d m %d", w.k, c.m);
    EXPECT(w.n_out >= 1 && w.n_out <= (1 << 24), "n_out %d", w.n_out);
    if (decode) {
      ++g_accepted_decode;
      EXPECT(t >= 1 && t <= 32, "decode t %d", t);
      const spa::DecodePlan p = spa::plan_decode(t, w.k, w.n_out, w.dtype, c.n, c.m, c.var_rescale);
      ++g_calls;
      EXPECT(p.tiles >= 1 && p.splits >= 1 && p.k_len >= 1, "plan %d %d %d", p.tiles, p.splits, p.k_len);
      if (p.col_tile > 0) EXPECT((long long)p.tiles * p.col_tile >= w.n_out, "columns uncovered");
      EXPECT((long long)p.splits * p.k_len >= w.k, "channels uncovered");
      const size_t offs[] = {p.partial, p.stats, p.counters, p.eta, p.dense};
      for (size_t o : offs) EXPECT(o <= p.bytes && o % 256 == 0, "offset %zu of %zu", o, p.bytes);
    } else {
      ++g_accepted_prefill;
      EXPECT(t >= 0 && t <= (1 << 24) && w.k % 64 == 0, "prefill t %d k %d", t, w.k);
      const spa_check::PrefillPlan p = spa_check::prefill_plan(t, w.k, w.dtype, &c);
      ++g_calls;
      const bool s24 = c.n == 2 && c.m == 4;
      const size_t rows = s24 ? (size_t)spa_check::tiled_rows(t) : (size_t)t;
      const size_t vbytes = rows * (size_t)(s24 ? w.k / 2 : w.k) * (size_t)spa_check::dtype_bytes(w.dtype);
      EXPECT(p.vals == 0 && p.meta >= vbytes, "vals region %zu < %zu", p.meta, vbytes);
      EXPECT(!s24 || p.eta - p.meta >= rows * (size_t)(w.k / 16) * 2, "meta region");
      EXPECT(p.nu - p.eta >= (size_t)t * 4 && p.colnorm - p.nu >= (size_t)t * 4, "eta / nu regions");
      EXPECT(p.sx >= p.colnorm && p.bytes >= p.sx && p.bytes % 256 == 0, "tail regions");
      EXPECT(rows >= (size_t)t && rows % (s24 ? 256 : 1) == 0, "rows %zu", rows);
    }
  }
}

void sweep_meta() {
  for (int it = 0; it < 100000; ++it) {
    const int64_t k = (int64_t)pick_dim() * (next_u64() % 2 ? 1 : 3);
    const bool ok = spa_check::valid_meta(k, pick(-1, 34), pick(-2, 40), pick(-1, 2));
    ++g_calls;
    if (ok) EXPECT(k >= 4 && k <= (1 << 24), "meta k %lld", (long long)k);
  }
}

// Bit patterns of non-negative float scores, often tied.
uint32_t pick_score() {
  static const float levels[] = {0.0f, 1e-42f, 0.5f, 1.0f, 2.0f, 3.0f, 1e30f};
  const uint64_t r = next_u64();
  float f;
  if (r % 2) {
    f = levels[(r >> 8) % 7];
  } else {
    const uint32_t b = (uint32_t)(r >> 16) & 0x7F7FFFFFu;   // finite, non-negative
    std::memcpy(&f, &b, 4);
  }
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

// Keep mask by the rank rule: j is kept when fewer than n positions beat it
// (a larger score, or an equal one at a lower position).
template <int M>
uint32_t rank_rule(const uint32_t (&s)[M], int n) {
  uint32_t keep = 0;
  for (int j = 0; j < M; ++j) {
    int beat = 0;
    for (int q = 0; q < M; ++q) beat += (s[q] > s[j] || (s[q] == s[j] && q < j)) ? 1 : 0;
    if (beat < n) keep |= 1u << j;
  }
  return keep;
}

template <int M>
void sweep_select() {
  for (int it = 0; it < 40000; ++it) {
    uint32_t s[M];
    for (int j = 0; j < M; ++j) s[j] = pick_score();
    const int n = pick(1, M);
    const uint32_t got = spa::topn_keep_bits<M>(s, n);
    ++g_calls;
    EXPECT(got == rank_rule<M>(s, n), "network m %d n %d", M, n);
    if constexpr (M == 4) {
      if (n == 2) {
        float sf[4], v[4] = {0.f, 1.f, 2.f, 3.f}, lo = -1.f, hi = -1.f;
        std::memcpy(sf, s, sizeof(sf));
        const uint32_t code = spa::top2of4(sf, v, lo, hi);
        const uint32_t keep = (1u << (code & 3u)) | (1u << ((code >> 2) & 3u));
        ++g_calls;
        EXPECT(keep == rank_rule<4>(s, 2) && (int)lo == (int)(code & 3u) && (int)hi == (int)(code >> 2) && lo < hi,
               "tournament code %u", code);
      }
    }
  }
}

}  // namespace

int main() {
  sweep_linear();
  sweep_meta();
  sweep_select<4>();
  sweep_select<8>();
  sweep_select<16>();
  sweep_select<32>();
  if (g_fails) {
    std::printf("failures %d of %ld calls\n", g_fails, g_calls);
    return 1;
  }
  std::printf("ok %ld calls, accepted %ld decode and %ld prefill\n", g_calls, g_accepted_decode, g_accepted_prefill);
  return 0;
}
