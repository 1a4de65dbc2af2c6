// Host driver for the DAG compactor, built with sanitizers by the test-suite.
// Builds many random DAGs (valid and invalid) and walks every plan table,
// checking the structural properties the kernels rely on.
#include <array>
#include <algorithm>
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
  std::vector<int> seen(pages, 0);
  std::vector<int> node_of_page(pages, -1), slot_of_page(pages, -1);
  for (int u = 0; u < P.n_nodes; ++u)
    for (int lp = 0; lp < P.npages[u]; ++lp) {
      node_of_page[P.page_table[P.slot0[u] + lp]] = u;
      slot_of_page[P.page_table[P.slot0[u] + lp]] = lp;
    }
  // one node per page: groups of a node's pages 4 i .. 4 i + 3 (the last may hold fewer);
  // each group's merged steps, projected on each of its pages, are exactly that page's
  // reader entries unrolled into 32-row steps, and the node's own query pages come last,
  // latest first.  Packed plans have no groups.
  const int64_t ngroups = (int64_t)P.kgroups.size() / kGroup;
  if ((int64_t)P.kgroups.size() != ngroups * kGroup) return 70;
  if ((int64_t)P.kgroup_off.size() != ngroups + 1 || P.kgroup_off[0] != 0) return 70;
  if ((int64_t)P.kgsteps.size() != P.kgroup_off[ngroups]) return 71;
  if ((int64_t)P.group_order.size() != ngroups) return 72;
  if (P.packed && ngroups) return 73;
  {
    std::vector<int> cnt(ngroups, 0);
    for (int32_t gr : P.group_order)
      if (gr < 0 || gr >= ngroups || cnt[gr]++) return 72;
  }
  for (int64_t gr = 0; gr < ngroups; ++gr) {
    if (P.kgroup_off[gr + 1] <= P.kgroup_off[gr]) return 74;
    const int ph0 = P.kgroups[kGroup * gr];
    if (ph0 < 0 || ph0 >= pages || slot_of_page[ph0] % kGroup) return 75;
    const int u = node_of_page[ph0];
    int npg = 0;
    for (int side = 0; side < kGroup; ++side) {
      const int ph = P.kgroups[kGroup * gr + side];
      if (ph < 0) {
        for (int64_t i = P.kgroup_off[gr]; i < P.kgroup_off[gr + 1]; ++i)
          if (gvis_of(P.kgsteps[i], side)) return 76;  // a missing page is never read
        continue;
      }
      ++npg;
      if (ph >= pages || seen[ph]++ || npg != side + 1) return 75;  // missing pages last
      if (node_of_page[ph] != u || slot_of_page[ph] != slot_of_page[ph0] + side) return 75;
      std::vector<std::array<int, 5>> want, got;  // qph, rb, lo, hi, diag
      for (int e = P.kv_off[ph]; e < P.kv_off[ph + 1]; ++e) {
        const KEntry& k = P.kentries[e];
        for (int lq = k.lq0; lq < k.lq1; ++lq) {
          const int qph = P.page_table[k.slot_base + lq];
          for (int rb = 0; rb * 32 < P.page_nrows[qph]; ++rb)
            want.push_back({qph, rb, k.lohi_diag & 0xff, (k.lohi_diag >> 8) & 0xff, (k.lohi_diag >> 16) & 1});
        }
      }
      for (int64_t i = P.kgroup_off[gr]; i < P.kgroup_off[gr + 1]; ++i) {
        const GStep& st = P.kgsteps[i];
        if (st.qph < 0 || st.qph >= pages || (st.rb != 0 && st.rb != 1) || st.rb * 32 >= P.page_nrows[st.qph])
          return 77;
        const uint32_t v = gvis_of(st, side);
        if (gvis_lo(v) == gvis_hi(v)) {
          if (v) return 78;  // an empty range carries no other bits
          continue;
        }
        got.push_back({st.qph, st.rb, gvis_lo(v), gvis_hi(v), gvis_diag(v)});
      }
      std::sort(want.begin(), want.end());
      std::sort(got.begin(), got.end());
      if (want != got) return 79;
    }
    // four pages, or the node's last ones
    if (npg != kGroup && slot_of_page[ph0] + npg != P.npages[u]) return 80;
    for (int64_t i = P.kgroup_off[gr]; i < P.kgroup_off[gr + 1]; ++i)
      if (!P.kgsteps[i].vis[0] && !P.kgsteps[i].vis[1]) return 81;  // every step reads a page
    bool in_own = false;
    int prev_slot = 1 << 30;
    for (int64_t i = P.kgroup_off[gr]; i < P.kgroup_off[gr + 1]; ++i) {
      const int qph = P.kgsteps[i].qph;
      if (node_of_page[qph] == u) {
        in_own = true;
        if (slot_of_page[qph] > prev_slot) return 82;
        prev_slot = slot_of_page[qph];
      } else if (in_own) {
        return 82;
      }
    }
  }
  // KV page pairs: a node of one or two pages (packed plans: consecutive pages), or one
  // lone page; each pair's merged steps, projected on each of its pages, are exactly that
  // page's reader entries unrolled into 32-row steps
  const int64_t npairs = (int64_t)P.kpairs.size() / 2;
  if ((int64_t)P.kpair_off.size() != npairs + 1 || P.kpair_off[0] != 0) return 8;
  if ((int64_t)P.kpsteps.size() != P.kpair_off[npairs]) return 13;
  for (int64_t pr = 0; pr < npairs && !P.packed; ++pr) {
    const int pa = P.kpairs[2 * pr];
    if (pa < 0 || pa >= pages || slot_of_page[pa] != 0 || P.npages[node_of_page[pa]] > 2) return 83;
  }
  if (npairs && !P.packed)  // pairs only when small nodes hold most pages, and then all of them
    for (int64_t gr = 0; gr < ngroups; ++gr)
      if (P.npages[node_of_page[P.kgroups[kGroup * gr]]] < 3) return 84;
  for (int64_t pr = 0; pr < npairs; ++pr) {
    for (int side = 0; side < 2; ++side) {
      const int ph = P.kpairs[2 * pr + side];
      if (ph < 0) {
        if (side == 0) return 9;
        for (int64_t i = P.kpair_off[pr]; i < P.kpair_off[pr + 1]; ++i)
          if ((uint32_t)P.kpsteps[i].info >> 16) return 10;  // a missing page is never read
        continue;
      }
      if (ph >= pages || seen[ph]++) return 9;
      if (P.packed) continue;  // packed: checked against the tile lists below
      std::vector<std::array<int, 5>> want, got;  // qph, rb, lo, hi, diag
      for (int e = P.kv_off[ph]; e < P.kv_off[ph + 1]; ++e) {
        const KEntry& k = P.kentries[e];
        for (int lq = k.lq0; lq < k.lq1; ++lq) {
          const int qph = P.page_table[k.slot_base + lq];
          for (int rb = 0; rb * 32 < P.page_nrows[qph]; ++rb)
            want.push_back({qph, rb, k.lohi_diag & 0xff, (k.lohi_diag >> 8) & 0xff, (k.lohi_diag >> 16) & 1});
        }
      }
      for (int64_t i = P.kpair_off[pr]; i < P.kpair_off[pr + 1]; ++i) {
        const KStep& st = P.kpsteps[i];
        const uint32_t inf = ((uint32_t)st.info >> (16 * side)) & 0xffffu;
        const int lo = (inf >> 1) & 0x7f, hi = (inf >> 8) & 0x7f;
        if (lo == hi) continue;
        got.push_back({st.qph, (int)(st.info & 1), lo, hi, (int)((inf >> 15) & 1)});
      }
      std::sort(want.begin(), want.end());
      std::sort(got.begin(), got.end());
      if (want != got) return 11;
    }
    if (P.kpair_off[pr + 1] <= P.kpair_off[pr]) return 14;  // a launched pair has steps
    // the pair's own node's query pages come after every other reader's, latest page first
    if (P.packed) continue;
    const int u = node_of_page[P.kpairs[2 * pr]];
    bool in_own = false;
    int prev_slot = 1 << 30;
    for (int64_t i = P.kpair_off[pr]; i < P.kpair_off[pr + 1]; ++i) {
      const int qph = P.kpsteps[i].qph;
      if (node_of_page[qph] == u) {
        in_own = true;
        if (slot_of_page[qph] > prev_slot) return 16;
        prev_slot = slot_of_page[qph];
      } else if (in_own) {
        return 16;
      }
    }
  }
  for (int64_t ph = 0; ph < pages; ++ph)
    if (!seen[ph] && P.page_nrows[ph] > 0) return 12;  // every page with rows is in a group or a pair
  if ((int64_t)P.pair_order.size() != npairs) return 15;
  if (P.packed) {
    // masks: one id per tile / step side, in range; the key-major half is the transpose of
    // the row-major half; a tile's [lo, hi) spans its mask's keys; padding rows see nothing
    const int64_t nmask = (int64_t)P.masks.size() / 128;
    if ((int64_t)P.masks.size() != nmask * 128 || P.tile_mask.size() != P.tiles.size()) return 50;
    if (P.kstep_mask.size() != P.kpsteps.size()) return 51;
    for (const QPage& q : P.qpages) {
      if (P.tile_mask[q.tile_begin + q.tile_count - 1] < 0) return 52;  // own page last, masked
      for (int t = q.tile_begin; t < q.tile_begin + q.tile_count; ++t) {
        const int mi = P.tile_mask[t];
        if (mi < -1 || mi >= nmask) return 53;
        if (mi < 0) continue;
        const uint64_t* m = &P.masks[(size_t)mi * 128];
        uint64_t any = 0;
        for (int r = 0; r < 64; ++r) {
          if (r >= q.nrows && m[r]) return 54;
          any |= m[r];
          for (int c = 0; c < 64; ++c)
            if (((m[r] >> c) & 1) != ((m[64 + c] >> r) & 1)) return 55;
        }
        const int lo = P.tiles[t].lohi & 0xff, hi = (P.tiles[t].lohi >> 8) & 0xff;
        if (!any || __builtin_ctzll(any) != lo || 64 - __builtin_clzll(any) != hi) return 56;
      }
    }
    for (const KMask& km : P.kstep_mask)
      if (km.a < -1 || km.a >= nmask || km.b < -1 || km.b >= nmask) return 57;
    // every (query page, KV page) tile appears as the pair's steps for that page, with the same
    // range and mask, for each 32-row half of the query page whose rows see it
    std::vector<std::array<int, 5>> want, got;  // kv page, qph, rb, lohi, mask
    for (const QPage& q : P.qpages)
      for (int t = q.tile_begin; t < q.tile_begin + q.tile_count; ++t)
        for (int rb = 0; rb * 32 < q.nrows; ++rb) {
          const int mi = P.tile_mask[t];
          bool sees = mi < 0;
          for (int r = 32 * rb; r < 32 * rb + 32 && !sees; ++r) sees = P.masks[(size_t)mi * 128 + r] != 0;
          if (sees) want.push_back({P.tiles[t].page, q.phys, rb, P.tiles[t].lohi, mi});
        }
    for (int64_t pr = 0; pr < npairs; ++pr)
      for (int64_t i = P.kpair_off[pr]; i < P.kpair_off[pr + 1]; ++i)
        for (int side = 0; side < 2; ++side) {
          const uint32_t inf = ((uint32_t)P.kpsteps[i].info >> (16 * side)) & 0xffffu;
          const int lo = (inf >> 1) & 0x7f, hi = (inf >> 8) & 0x7f;
          if (lo == hi) continue;
          if ((inf >> 15) & 1) return 58;  // packed steps carry no causal rule
          got.push_back({P.kpairs[2 * pr + side], P.kpsteps[i].qph, (int)(P.kpsteps[i].info & 1), lo | (hi << 8),
                         side ? P.kstep_mask[i].b : P.kstep_mask[i].a});
        }
    std::sort(want.begin(), want.end());
    std::sort(got.begin(), got.end());
    if (want != got) return 59;
  }
  {
    std::vector<int> cnt(npairs, 0);
    for (int32_t pr : P.pair_order)
      if (pr < 0 || pr >= npairs || cnt[pr]++) return 15;
  }
  return 0;
}

// Linear-attention schedule: every token row lies in the plan, every own token
// appears once, exports fall inside their producer, consumers and fix-up lists
// index valid entries.
static int check_gdn(const Plan& P) {
  const int B = P.info.gdn_chunk;
  if (B <= 0) return 0;
  const int64_t C = P.info.rows;
  std::vector<int> own(C, 0);
  const int NS = (int)P.gseqs.size();
  const int nslots = (int)P.gslot_off.size() - 1;
  for (int q = 0; q < NS; ++q) {
    const GSeq& g = P.gseqs[q];
    if (g.tok_off < 0 || g.n_tok <= g.n_replay || g.tok_off + g.n_tok > (int64_t)P.grows.size()) return 31;
    if (g.start % B || g.n_replay >= B) return 32;
    for (int j = 0; j < g.n_tok; ++j) {
      const int r = P.grows[g.tok_off + j];
      if (r < 0 || r >= C || P.pos_of_row[r] < 0) return 33;
      if (j >= g.n_replay) own[r]++;
    }
    const int nch = (g.n_tok + B - 1) / B;
    for (int e = g.exp_off; e < g.exp_off + g.exp_cnt; ++e) {
      if (P.gexports[e].chunk < 1 || P.gexports[e].chunk > nch) return 34;
      if (P.gexports[e].slot < 0 || P.gexports[e].slot >= nslots) return 35;
      if (e > g.exp_off && P.gexports[e].chunk <= P.gexports[e - 1].chunk) return 36;
    }
    if ((g.init_slot < 0) != (g.cgrad < 0) || g.init_slot >= nslots || g.cgrad >= P.gdn_ncgrad) return 37;
  }
  for (int64_t r = 0; r < C; ++r)
    if (own[r] != (P.pos_of_row[r] >= 0 ? 1 : 0)) return 38;
  for (int s = 0; s < nslots; ++s)
    for (int i = P.gslot_off[s]; i < P.gslot_off[s + 1]; ++i)
      if (P.gslot_cons[i] < 0 || P.gslot_cons[i] >= P.gdn_ncgrad) return 39;
  std::vector<int> rep_rows;
  for (int q = 0; q < NS; ++q) {
    if (P.gseqs[q].rep_off != (int)rep_rows.size()) return 40;
    for (int j = 0; j < P.gseqs[q].n_replay; ++j) rep_rows.push_back(P.grows[P.gseqs[q].tok_off + j]);
  }
  if ((int64_t)P.grep_slot.size() != C) return 41;
  for (size_t i = 0; i + 1 < P.grep_off.size(); ++i) {
    if (P.grep_slot[P.grep_rows[i]] != (int)i) return 42;
    for (int t = P.grep_off[i]; t < P.grep_off[i + 1]; ++t)
      if (P.grep_tok[t] < 0 || P.grep_tok[t] >= (int)rep_rows.size() || rep_rows[P.grep_tok[t]] != P.grep_rows[i]) return 43;
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
    dag_build_opts o{64, 64, (int)rnd(2), (int)rnd(3), rnd(3) ? 1 + (int)rnd(70) : 0, (int)rnd(3), 0};
    if (o.page_shuffle == 0) o.pack_pages = (int)rnd(2);
    Plan P;
    std::string err;
    const dag_status st = build_plan(nodes.data(), n, mounts.data(), (int)mounts.size(), &o, &P, &err);
    if (st != DAG_OK) {
      ++rejected;
      if (err.empty()) return 10;
      continue;
    }
    ++built;
    int c = check(P);
    if (!c) c = check_gdn(P);
    if (c) {
      std::printf("table check %d failed at iteration %d\n", c, it);
      return 20 + c;
    }
  }
  std::printf("ok built=%d rejected=%d\n", built, rejected);
  return 0;
}
