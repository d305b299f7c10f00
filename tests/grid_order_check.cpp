// Host-side check of the workgroup-to-tile maps of the attention kernels
// (exact_tiled_attention_36_amd/csrc/common.h): xcd_remap and causal_order<1>,
// causal_order<2>. Built with hipcc's host pass by tests/test_grid_order.py; prints
// "ok" or the first failing case and exits non-zero.
#include <cstdio>
#include <vector>

#include "common.h"

static int fail(const char* what, int a, int b, int c) {
  std::printf("FAIL %s (%d, %d, %d)\n", what, a, b, c);
  return 1;
}

template <int C>
static int check_causal(int nbh, int nqb) {
  const int n = nbh * nqb;
  std::vector<int> seen(n, 0);
  std::vector<int> prev_qb(8, 1 << 30), prev_bh(8, -1);
  for (int hw = 0; hw < n; ++hw) {
    int bh, qb;
    fa::causal_order<C>(hw, n, nqb, bh, qb);
    if (bh < 0 || bh >= nbh || qb < 0 || qb >= nqb) return fail("out of range", C, nbh, nqb);
    if (seen[bh * nqb + qb]++) return fail("tile twice", C, nbh, nqb);
    const int x = hw % 8;  // the XCD this workgroup runs on
    if (nbh % 8 == 0) {
      const int k = nbh / 8;
      if (bh / k != x) return fail("head outside its XCD", C, nbh, nqb);
      // inside a cluster of C heads the row blocks go from the longest down
      // clusters count from the XCD's first head
      const bool same_cluster = prev_bh[x] >= 0 && (prev_bh[x] - x * k) / C == (bh - x * k) / C;
      if (same_cluster && qb > prev_qb[x]) return fail("cluster order", C, nbh, nqb);
    } else if (qb > prev_qb[x]) {
      return fail("level order", C, nbh, nqb);
    }
    prev_qb[x] = qb;
    prev_bh[x] = bh;
  }
  return 0;
}

int main() {
  for (int n = 1; n <= 4096; ++n) {
    std::vector<int> seen(n, 0);
    for (int hw = 0; hw < n; ++hw) {
      const int L = fa::xcd_remap(hw, n);
      if (L < 0 || L >= n || seen[L]++) return fail("xcd_remap", n, hw, L);
    }
  }
  for (int nbh = 1; nbh <= 64; ++nbh)
    for (int nqb = 1; nqb <= 80; ++nqb)
      if (check_causal<1>(nbh, nqb) || check_causal<2>(nbh, nqb)) return 1;
  std::printf("ok\n");
  return 0;
}
