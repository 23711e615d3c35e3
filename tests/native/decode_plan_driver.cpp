// Host replay of the decode plan and the fused kernel's row list.
//   input: lines "t k n_out dtype n m var rule" (rule 1 = the kernel's slot
//          rule, 0 = base + (pass * threads + tid) * n, the rule that
//          counted the pass offset twice)
//   output per line: "ok <path> <splits> <list_cap> <max_slot> <entries>" or
//          "fail <reason> ..."
// Every workgroup (channel split) of the fused path is replayed pass by pass
// with the kernel's own thread count; each list slot must be written exactly
// once, stay below the workgroup's LDS list capacity, and the entries the
// stream reads ([0, entries)) must all have been written.
#include <cstdio>
#include <vector>

#include "spa_plan.h"

static int replay(int t, int k, int n_out, int dtype, int n, int m, int var, int rule) {
  const spa::DecodePlan p = spa::plan_decode(t, k, n_out, dtype, n, m, var);
  if (spa::t1_kernel(t, dtype, k, n_out)) {
    // one-token kernel: per-wave lists of at most 64 entries; a split covers at most kT1MaxChan channels
    if (p.k_len > spa::kT1MaxChan || p.k_len % m) { std::printf("fail t1_split %d\n", p.k_len); return 1; }
    if ((long long)p.splits * p.k_len < k) { std::printf("fail t1_cover\n"); return 1; }
    std::printf("ok t1 %d 0 0 0\n", p.splits);
    return 0;
  }
  if (spa::decode_on_matrix_cores(t, dtype)) {
    std::printf("ok mm %d 0 0 0\n", p.splits);
    return 0;
  }
  const int tok = spa::fused_tok_of(t);
  const int nt = spa::fused_waves_of(m, tok) * 64;
  const int cap = p.list_cap;
  if ((long long)cap * 4 * (1 + tok) > spa::kFusedListBytes) { std::printf("fail lds %d\n", cap); return 1; }
  if ((long long)p.splits * p.k_len < k || p.k_len % m) { std::printf("fail cover\n"); return 1; }
  const int per_block = m < n * t ? m : n * t;
  int max_slot = -1, max_entries = 0;
  for (int s = 0; s < p.splits; ++s) {
    const int kb = s * p.k_len;
    const int kl = p.k_len < k - kb ? p.k_len : k - kb;
    const int nb = kl / m;
    if (nb * per_block > cap) { std::printf("fail worst_case_union %d %d\n", nb * per_block, cap); return 1; }
    if (t != 1) continue;                       // several tokens: a workgroup prefix scan, bounded above
    std::vector<int> hits(cap + (size_t)nb * n * 4 + 64, 0);
    int base = 0;
    const int npass = (nb + nt - 1) / nt;
    for (int pass = 0; pass < npass; ++pass) {
      for (int tid = 0; tid < nt; ++tid) {
        const int b = pass * nt + tid;
        if (b >= nb) continue;
        const int slot = rule ? spa::one_token_list_slot(base, tid, n) : base + b * n;
        for (int q = 0; q < n; ++q) {
          const int e = slot + q;
          if (e >= (int)hits.size()) { std::printf("fail slot_range %d\n", e); return 1; }
          ++hits[e];
          if (e > max_slot) max_slot = e;
        }
      }
      base += (nt < nb - pass * nt ? nt : nb - pass * nt) * n;
    }
    if (max_slot >= cap) { std::printf("fail slot_past_cap %d %d %d\n", s, max_slot, cap); return 1; }
    for (int e = 0; e < base; ++e)
      if (hits[e] != 1) { std::printf("fail slot_unwritten %d %d %d\n", s, e, hits[e]); return 1; }
    if (base > max_entries) max_entries = base;
  }
  std::printf("ok fused %d %d %d %d\n", p.splits, cap, max_slot, max_entries);
  return 0;
}

int main() {
  int t, k, n_out, dtype, n, m, var, rule;
  int bad = 0;
  while (std::scanf("%d %d %d %d %d %d %d %d", &t, &k, &n_out, &dtype, &n, &m, &var, &rule) == 8)
    bad |= replay(t, k, n_out, dtype, n, m, var, rule);
  std::fflush(stdout);
  return 0 * bad;
}
