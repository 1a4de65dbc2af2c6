// Host driver for the DAG compactor, built with sanitizers by the test-suite.
// Builds many random DAGs (valid and invalid) and walks every plan table,
// checking the structural properties the kernels rely on.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../dag_packed_attention_amd/csrc/plan.hpp"

using namespace dagattn;

static uint64_t rs = 88172645463325252ull;
static uint32_t rnd(uint32_t n) {
  rs ^= rs << 13;
  rs ^= rs >> 7;
  rs ^= rs << 17;
  return (uint32_t)(rs % n);
}

static int check(const Plan& P) {
  const int64_t pages = P.info.pages;
  for (const QPage& q : P.qpages) {
    if (q.phys < 0 || q.phys >= pages || q.nrows <= 0 || q.nrows > 64) return 1;
    if (q.tile_begin < 0 || q.tile_count <= 0 || q.tile_begin + q.tile_count > (int64_t)P.tiles.size()) return 2;
    for (int t = q.tile_begin; t < q.tile_begin + q.tile_count; ++t) {
      const Tile& tl = P.tiles[t];
      const int lo = tl.lohi & 0xff, hi = (tl.lohi >> 8) & 0xff;
      if (tl.page < 0 || tl.page >= pages || lo >= hi || hi > P.page_nrows[tl.page]) return 3;
    }
    if (P.tiles[q.tile_begin + q.tile_count - 1].page != q.phys) return 4;  // diagonal last
  }
  for (int64_t ph = 0; ph < pages; ++ph)
    for (int e = P.kv_off[ph]; e < P.kv_off[ph + 1]; ++e) {
      const KEntry& k = P.kentries[e];
      if (k.lq0 < 0 || k.lq1 <= k.lq0 || k.slot_base < 0) return 5;
      if (k.slot_base + k.lq1 > (int64_t)P.page_table.size()) return 6;
      const int lo = k.lohi_diag & 0xff, hi = (k.lohi_diag >> 8) & 0xff;
      if (lo >= hi || hi > P.page_nrows[ph]) return 7;
    }
  return 0;
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 100;
  int built = 0, rejected = 0;
  for (int it = 0; it < iters; ++it) {
    const int n = 1 + (int)rnd(12);
    std::vector<dag_node> nodes(n);
    std::vector<dag_mount> mounts;
    for (int u = 0; u < n; ++u) {
      nodes[u].parent = u == 0 ? -1 : (rnd(5) == 0 ? -1 : (int)rnd(u));
      if (rnd(50) == 0) nodes[u].parent = u;  // invalid now and then
      nodes[u].length = rnd(8) == 0 ? 0 : 1 + (int)rnd(200);
    }
    for (int u = 0; u < n; ++u) {
      nodes[u].mount_first = (int)mounts.size();
      const int c = rnd(3) == 0 ? 1 + (int)rnd(3) : 0;
      for (int i = 0; i < c; ++i) {
        dag_mount m;
        m.src_node = (int)rnd(n);
        const int len = nodes[m.src_node].length;
        m.begin = len ? (int)rnd(len + 1) : 0;
        m.end = m.begin + (len > m.begin ? (int)rnd(len - m.begin + 1) : 0);
        if (rnd(40) == 0) m.end = len + 3;  // out of range now and then
        mounts.push_back(m);
      }
      nodes[u].mount_count = (int)mounts.size() - nodes[u].mount_first;
    }
    dag_build_opts o{64, 64, (int)rnd(2), (int)rnd(3)};
    Plan P;
    std::string err;
    const dag_status st = build_plan(nodes.data(), n, mounts.data(), (int)mounts.size(), &o, &P, &err);
    if (st != DAG_OK) {
      ++rejected;
      if (err.empty()) return 10;
      continue;
    }
    ++built;
    const int c = check(P);
    if (c) {
      std::printf("table check %d failed at iteration %d\n", c, it);
      return 20 + c;
    }
  }
  std::printf("ok built=%d rejected=%d\n", built, rejected);
  return 0;
}
