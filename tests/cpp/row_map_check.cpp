// Host check of the workgroup -> (head, query block) map of the attention
// kernels: a bijection onto Hq x N, ordered KV group by KV group, and within
// a group from the heaviest query block (the last) to the lightest.  When N
// is a multiple of 8, the ids dealt to one XCD (id % 8) must visit each
// query block's heads on consecutive slots, blocks in descending order;
// otherwise the heads of a block must take adjacent ids, blocks descending.
// With a fourth argument "runs" (the deal of the one-block attention kernel
// for short lists, N a multiple of 128: runs_of_16 applied to the block)
// the same holds, and the blocks of XCD x come in runs of 16 adjacent
// blocks: 16x .. 16x+15, 16(x+8) .. 16(x+8)+15, ... counted from the last.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../dynamic_sparse_attention_proxy_amd/csrc/common.h"

int main(int argc, char** argv) {
  if (argc != 4 && argc != 5) return 2;
  const int hq = atoi(argv[1]), hkv = atoi(argv[2]), nblk = atoi(argv[3]);
  crisp::RowMap m = crisp::make_row_map(hq, hkv, nblk);
  const int qpg = hq / hkv;
  const bool xcd = nblk % 8 == 0;
  if (m.xcd != (xcd ? 1 : 0)) {
    printf("xcd flag %d for nblk %d\n", m.xcd, nblk);
    return 1;
  }
  const bool runs = argc == 5;
  if (runs && nblk % 128 != 0) return 2;
  std::vector<int> seen((size_t)hq * nblk, 0);
  const int lanes = xcd ? 8 : 1;  // independent id sequences checked for order
  std::vector<int> prev_g(lanes, 0), prev_qb(lanes, nblk), run(lanes, 0);
  for (int id = 0; id < hq * nblk; ++id) {
    int h = -1, qb = -1;
    crisp::map_row(m, id, &h, &qb);
    if (runs) qb = crisp::runs_of_16(qb, nblk);
    if (h < 0 || h >= hq || qb < 0 || qb >= nblk) {
      printf("id %d -> (%d, %d) out of range\n", id, h, qb);
      return 1;
    }
    if (seen[(size_t)h * nblk + qb]++) {
      printf("id %d -> (%d, %d) duplicated\n", id, h, qb);
      return 1;
    }
    const int g = h / qpg;
    const int x = xcd ? id % 8 : 0;
    if (g < prev_g[x]) {
      printf("id %d -> group %d after group %d\n", id, g, prev_g[x]);
      return 1;
    }
    if (g != prev_g[x]) {
      if (run[x] % qpg != 0) {
        printf("id %d: group %d left a block with %d of %d heads\n", id, prev_g[x], run[x] % qpg, qpg);
        return 1;
      }
      prev_qb[x] = nblk;
      run[x] = 0;
    }
    // heads of one block on consecutive positions of this sequence
    if (run[x] % qpg == 0) {
      if (qb >= prev_qb[x]) {
        printf("id %d -> qb %d not below %d\n", id, qb, prev_qb[x]);
        return 1;
      }
    } else if (qb != prev_qb[x]) {
      printf("id %d -> qb %d splits the heads of qb %d\n", id, qb, prev_qb[x]);
      return 1;
    }
    if (runs && ((nblk - 1 - qb) / 16) % 8 != x) {
      printf("id %d -> qb %d outside the runs of XCD %d\n", id, qb, x);
      return 1;
    }
    if (h != g * qpg + run[x] % qpg) {
      printf("id %d -> head %d out of order\n", id, h);
      return 1;
    }
    ++run[x];
    prev_g[x] = g;
    prev_qb[x] = qb;
  }
  printf("ok\n");
  return 0;
}
