// Host check of the workgroup -> (head, query block) map of the attention
// kernels: a bijection onto Hq x N, ordered KV group by KV group, and within
// a group from the heaviest query block (the last) to the lightest.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../dynamic_sparse_attention_proxy_amd/csrc/common.h"

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  const int hq = atoi(argv[1]), hkv = atoi(argv[2]), nblk = atoi(argv[3]);
  crisp::RowMap m = crisp::make_row_map(hq, hkv, nblk);
  std::vector<int> seen((size_t)hq * nblk, 0);
  int prev_g = 0, prev_qb = nblk;
  for (int id = 0; id < hq * nblk; ++id) {
    int h = -1, qb = -1;
    crisp::map_row(m, id, &h, &qb);
    if (h < 0 || h >= hq || qb < 0 || qb >= nblk) {
      printf("id %d -> (%d, %d) out of range\n", id, h, qb);
      return 1;
    }
    if (seen[(size_t)h * nblk + qb]++) {
      printf("id %d -> (%d, %d) duplicated\n", id, h, qb);
      return 1;
    }
    const int g = h / m.qpg;
    if (g < prev_g || (g == prev_g && qb > prev_qb)) {
      printf("id %d -> group %d qb %d after group %d qb %d\n", id, g, qb, prev_g, prev_qb);
      return 1;
    }
    if (g != prev_g) prev_qb = nblk;
    prev_g = g;
    prev_qb = qb;
  }
  printf("ok\n");
  return 0;
}
