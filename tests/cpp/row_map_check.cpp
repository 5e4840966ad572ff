// Host check of the workgroup -> (head, query block) map used by the
// attention kernels: it must be a bijection onto Hq x N, deal each XCD one
// KV group per die where the shape allows, and hand out heavier (larger qb)
// rows no later than lighter ones on each XCD.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../dynamic_sparse_attention_proxy_amd/csrc/common.h"

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  const int hq = atoi(argv[1]), hkv = atoi(argv[2]), nblk = atoi(argv[3]), want_mode = atoi(argv[4]);
  crisp::RowMap m = crisp::make_row_map(hq, hkv, nblk);
  if (m.mode != want_mode) {
    printf("mode %d, expected %d\n", m.mode, want_mode);
    return 1;
  }
  std::vector<int> seen((size_t)hq * nblk, 0);
  std::vector<int> last_qb(crisp::kNumXcd, 1 << 30);
  std::vector<int> xcd_group(crisp::kNumXcd, -1);
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
    const int x = id % crisp::kNumXcd;
    if (m.mode != 0) {
      if (qb > last_qb[x]) {
        printf("xcd %d: qb %d after %d\n", x, qb, last_qb[x]);
        return 1;
      }
      last_qb[x] = qb;
      const int g = h / m.qpg;
      if (hkv <= crisp::kNumXcd) {
        if (xcd_group[x] >= 0 && xcd_group[x] != g) {
          printf("xcd %d sees groups %d and %d\n", x, xcd_group[x], g);
          return 1;
        }
        xcd_group[x] = g;
      }
    }
  }
  printf("ok mode %d\n", m.mode);
  return 0;
}
