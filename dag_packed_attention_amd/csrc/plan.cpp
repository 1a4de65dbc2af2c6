// Host-side DAG compactor.
//
// Steps (each tied to the pages' definitions):
//   1. validation of the node and mount tables;
//   2. a dependency order in which every node follows its parent and the
//      sources of its mounts (the execution graph is a DAG: Octopus Sec. 3);
//   3. start positions by monotonic continuation (Octopus Sec. 3.2 Eq. 2):
//      s(u) = max(s(parent) + len(parent), max over u's reads of end position + 1);
//   4. active mounts per node: inherited along the chain, optionally closed
//      over the sources' own active mounts (Octopus Sec. 3.3 item 1);
//   5. non-self visibility as disjoint ranges of source-node offsets: mounted
//      spans first, then the ancestors (Octopus Sec. 3.3 Eq. 4);
//   6. pages: every node starts on a fresh 64-row page; a page table maps the
//      node's page slots to physical pages;
//   7. per-node tile lists (query blocks take a prefix: HARTS Eq. 22's
//      bottom-right causal alignment puts the node's own pages last);
//   8. per-KV-page reader lists in a fixed order (the deterministic order in
//      which the backward sums reader contributions into producer pages,
//      Octopus Sec. 3.4 Eq. 8, HARTS Sec. 3.4);
//   9. launch orders: node-grouped, heaviest first;
//  10. optionally, the chunked linear-attention schedule (gdn_plan.cpp).
#include "plan.hpp"

#include <algorithm>
#include <climits>
#include <cstdio>
#include <numeric>
#include <queue>

namespace dagattn {
namespace {

struct Span {
  int32_t src, b, e;
  bool operator<(const Span& o) const {
    if (src != o.src) return src < o.src;
    if (b != o.b) return b < o.b;
    return e < o.e;
  }
  bool operator==(const Span& o) const { return src == o.src && b == o.b && e == o.e; }
};

dag_status fail(std::string* err, dag_status code, const char* fmt, long long a = 0,
                long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, fmt, a, b, c);
  *err = buf;
  return code;
}

// splitmix64: a small, fully specified generator so shuffled page tables are
// reproducible across compilers and standard libraries.
uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

dag_status build_plan(const dag_node* nodes, int32_t n, const dag_mount* mounts, int32_t nm,
                      const dag_build_opts* opts_in, Plan* P, std::string* err) {
  // ---- options ----------------------------------------------------------
  dag_build_opts opts{64, 64, 1, 0, 0, DAG_VIEW_MOUNTED, 0};
  if (opts_in) opts = *opts_in;
  if (opts.page_size == 0) opts.page_size = kPage;
  if (opts.q_block == 0) opts.q_block = kPage;
  if (opts.page_size != kPage || opts.q_block != kPage)
    return fail(err, DAG_E_UNSUPPORTED, "page_size and q_block must be 64 (got %lld, %lld)",
                opts.page_size, opts.q_block);
  if (opts.transitive != 0 && opts.transitive != 1)
    return fail(err, DAG_E_INVALID, "transitive must be 0 or 1");
  if (opts.view != DAG_VIEW_MOUNTED && opts.view != DAG_VIEW_MOUNT_FREE && opts.view != DAG_VIEW_UNSHIFTED)
    return fail(err, DAG_E_INVALID, "view must be 0, 1 or 2 (got %lld)", opts.view);
  if (opts.gdn_chunk < 0 || opts.gdn_chunk > 4096)
    return fail(err, DAG_E_INVALID, "gdn_chunk must be in [0, 4096] (got %lld)", opts.gdn_chunk);
  if (opts.pack_pages != 0 && opts.pack_pages != 1)
    return fail(err, DAG_E_INVALID, "pack_pages must be 0 or 1 (got %lld)", opts.pack_pages);
  P->opts = opts;

  // ---- 1. validation ------------------------------------------------------
  if (n <= 0 || !nodes) return fail(err, DAG_E_INVALID, "a DAG needs at least one node");
  if (nm < 0 || (nm > 0 && !mounts)) return fail(err, DAG_E_INVALID, "bad mount table");
  for (int32_t u = 0; u < n; ++u) {
    const int32_t p = nodes[u].parent;
    if (p < -1 || p >= n) return fail(err, DAG_E_INVALID, "node %lld: parent %lld out of range", u, p);
    if (p >= u) return fail(err, DAG_E_NOT_TOPO, "node %lld: parent %lld is not earlier", u, p);
    if (nodes[u].length < 0) return fail(err, DAG_E_INVALID, "node %lld: negative length", u);
  }
  for (int32_t u = 0; u < n; ++u) {
    const int64_t f = nodes[u].mount_first, c = nodes[u].mount_count;
    if (c < 0 || f < 0 || f + c > nm)
      return fail(err, DAG_E_INVALID, "node %lld: mount slice out of range", u);
    for (int64_t i = f; i < f + c; ++i) {
      const dag_mount& m = mounts[i];
      if (m.src_node < 0 || m.src_node >= n)
        return fail(err, DAG_E_INVALID, "node %lld: mount source %lld out of range", u, m.src_node);
    }
  }
  P->n_nodes = n;
  P->parent.resize(n);
  P->length.resize(n);
  P->direct.assign(n, {});
  for (int32_t u = 0; u < n; ++u) {
    P->parent[u] = nodes[u].parent;
    P->length[u] = nodes[u].length;
  }
  for (int32_t u = 0; u < n; ++u) {
    for (int64_t i = nodes[u].mount_first; i < nodes[u].mount_first + nodes[u].mount_count; ++i) {
      const dag_mount& m = mounts[i];
      if (!(0 <= m.begin && m.begin <= m.end && m.end <= P->length[m.src_node]))
        return fail(err, DAG_E_MOUNT_RANGE, "node %lld: span [%lld,%lld) outside its source", u,
                    m.begin, m.end);
      if (m.end > m.begin) P->direct[u].push_back(m);
    }
  }
  // reads of the reader's own chain
  for (int32_t u = 0; u < n; ++u) {
    for (const dag_mount& m : P->direct[u]) {
      for (int32_t a = u; a >= 0; a = P->parent[a])
        if (a == m.src_node)
          return fail(err, DAG_E_SELF_ANCESTOR_MOUNT, "node %lld reads its own chain (node %lld)",
                      u, m.src_node);
    }
  }

  // ---- 2. dependency order (Kahn, smallest ready index first) ---------------
  {
    std::vector<int32_t> indeg(n, 0);
    std::vector<std::vector<int32_t>> users(n);
    for (int32_t u = 0; u < n; ++u) {
      std::vector<int32_t> deps;
      if (P->parent[u] >= 0) deps.push_back(P->parent[u]);
      for (const dag_mount& m : P->direct[u]) deps.push_back(m.src_node);
      std::sort(deps.begin(), deps.end());
      deps.erase(std::unique(deps.begin(), deps.end()), deps.end());
      indeg[u] = (int32_t)deps.size();
      for (int32_t s : deps) users[s].push_back(u);
    }
    std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> ready;
    for (int32_t u = 0; u < n; ++u)
      if (indeg[u] == 0) ready.push(u);
    P->order.clear();
    while (!ready.empty()) {
      int32_t u = ready.top();
      ready.pop();
      P->order.push_back(u);
      for (int32_t w : users[u])
        if (--indeg[w] == 0) ready.push(w);
    }
    if ((int32_t)P->order.size() != n)
      return fail(err, DAG_E_MOUNT_CYCLE, "tree and mount edges form a cycle");
  }

  // ---- 3. positions (Octopus Eq. 2) -----------------------------------------
  P->start.assign(n, 0);
  int64_t max_pos = 0;
  for (int32_t u : P->order) {
    const int32_t p = P->parent[u];
    int64_t s = p < 0 ? 0 : (int64_t)P->start[p] + P->length[p];
    if (opts.view != DAG_VIEW_UNSHIFTED) {  // the unshifted regime continues from the parent
      for (const dag_mount& m : P->direct[u]) {
        const int64_t pos_end = (int64_t)P->start[m.src_node] + (m.end - 1);  // last mounted token
        s = std::max(s, pos_end + 1);
      }
    }
    if (s + P->length[u] > INT32_MAX) return fail(err, DAG_E_OVERFLOW, "positions exceed int32");
    P->start[u] = (int32_t)s;
    max_pos = std::max(max_pos, s + std::max(0, P->length[u] - 1));
  }

  // ---- 4. active mounts --------------------------------------------------------
  std::vector<std::vector<Span>> act(n);
  for (int32_t u : P->order) {
    std::vector<Span> s;
    if (P->parent[u] >= 0) s = act[P->parent[u]];
    if (opts.view != DAG_VIEW_MOUNT_FREE) {  // the mount-free view: ancestors only
      for (const dag_mount& m : P->direct[u]) {
        s.push_back({m.src_node, m.begin, m.end});
        if (opts.transitive) s.insert(s.end(), act[m.src_node].begin(), act[m.src_node].end());
      }
    }
    std::sort(s.begin(), s.end());
    s.erase(std::unique(s.begin(), s.end()), s.end());
    act[u] = std::move(s);
  }

  // ---- 5. non-self visibility ranges -------------------------------------------
  P->range_off.assign(n + 1, 0);
  P->ranges.clear();
  std::vector<char> is_anc(n, 0);
  std::vector<int32_t> chain;
  for (int32_t u = 0; u < n; ++u) {
    P->range_off[u] = (int64_t)P->ranges.size() / 3;
    chain.clear();
    for (int32_t a = P->parent[u]; a >= 0; a = P->parent[a]) chain.push_back(a);
    for (int32_t a : chain) is_anc[a] = 1;
    // mounted spans, merged per source (act[u] is sorted by (src, b, e))
    size_t i = 0;
    const std::vector<Span>& s = act[u];
    while (i < s.size()) {
      const int32_t src = s[i].src;
      if (is_anc[src]) {  // an ancestor is visible in full already
        while (i < s.size() && s[i].src == src) ++i;
        continue;
      }
      int32_t lo = s[i].b, hi = s[i].e;
      ++i;
      while (i < s.size() && s[i].src == src) {
        if (s[i].b <= hi) {
          hi = std::max(hi, s[i].e);
        } else {
          P->ranges.insert(P->ranges.end(), {src, lo, hi});
          lo = s[i].b;
          hi = s[i].e;
        }
        ++i;
      }
      P->ranges.insert(P->ranges.end(), {src, lo, hi});
    }
    // ancestors, root first
    for (auto it = chain.rbegin(); it != chain.rend(); ++it)
      if (P->length[*it] > 0) P->ranges.insert(P->ranges.end(), {*it, 0, P->length[*it]});
    for (int32_t a : chain) is_anc[a] = 0;
  }
  P->range_off[n] = (int64_t)P->ranges.size() / 3;

  if (opts.pack_pages) {
    // steps 6-9 for the packed layout (pack_plan.cpp)
    const dag_status pst = build_packed_tables(P, err);
    if (pst != DAG_OK) return pst;
  } else {
    // ---- 6. pages ------------------------------------------------------------------
    P->slot0.assign(n, 0);
    P->npages.assign(n, 0);
    P->tok_off.assign(n, 0);
    int64_t slots = 0, tokens = 0;
    for (int32_t u = 0; u < n; ++u) {
      P->slot0[u] = (int32_t)std::min<int64_t>(slots, INT32_MAX);
      P->npages[u] = (int32_t)(((int64_t)P->length[u] + kPage - 1) / kPage);  // int64: lengths reach 2^31 - 1
      P->tok_off[u] = tokens;
      slots += P->npages[u];
      tokens += P->length[u];
    }
    if (slots * kPage > INT32_MAX) return fail(err, DAG_E_OVERFLOW, "compact rows exceed int32");
    const int32_t n_pages = (int32_t)slots;
    P->page_table.resize(n_pages);
    std::iota(P->page_table.begin(), P->page_table.end(), 0);
    if (opts.page_shuffle) {
      uint64_t st = (uint64_t)(uint32_t)opts.page_shuffle;
      for (int32_t i = n_pages - 1; i > 0; --i) {
        const int32_t j = (int32_t)(splitmix64(st) % (uint64_t)(i + 1));
        std::swap(P->page_table[i], P->page_table[j]);
      }
    }
    const int64_t C = (int64_t)n_pages * kPage;
    P->page_nrows.assign(n_pages, 0);
    P->pos_of_row.assign(C, -1);
    P->row_of_token.assign(tokens, 0);
    for (int32_t u = 0; u < n; ++u) {
      for (int32_t lp = 0; lp < P->npages[u]; ++lp) {
        const int32_t ph = P->page_table[P->slot0[u] + lp];
        const int32_t nr = std::min(kPage, P->length[u] - lp * kPage);
        P->page_nrows[ph] = nr;
        for (int32_t r = 0; r < nr; ++r) {
          const int64_t row = (int64_t)ph * kPage + r;
          P->pos_of_row[row] = P->start[u] + lp * kPage + r;
          P->row_of_token[P->tok_off[u] + lp * kPage + r] = (int32_t)row;
        }
      }
    }

    // ---- 7. tile lists and query pages -----------------------------------------------
    P->tile_off.assign(n + 1, 0);
    P->tile_nonself.assign(n, 0);
    P->tiles.clear();
    P->qpages.clear();
    auto pack = [](int32_t lo, int32_t hi) { return lo | (hi << 8); };
    for (int32_t u = 0; u < n; ++u) {
      if ((int64_t)P->tiles.size() > INT32_MAX / 2) return fail(err, DAG_E_OVERFLOW, "tile lists too long");
      P->tile_off[u] = (int32_t)P->tiles.size();
      if (P->length[u] == 0) continue;
      for (int64_t r = P->range_off[u]; r < P->range_off[u + 1]; ++r) {
        const int32_t src = P->ranges[3 * r], lo = P->ranges[3 * r + 1], hi = P->ranges[3 * r + 2];
        for (int32_t lp = lo / kPage; lp <= (hi - 1) / kPage; ++lp) {
          const int32_t tlo = std::max(lo - lp * kPage, 0), thi = std::min(hi - lp * kPage, kPage);
          P->tiles.push_back({P->page_table[P->slot0[src] + lp], pack(tlo, thi)});
        }
      }
      P->tile_nonself[u] = (int32_t)P->tiles.size() - P->tile_off[u];
      for (int32_t lp = 0; lp < P->npages[u]; ++lp) {
        const int32_t ph = P->page_table[P->slot0[u] + lp];
        P->tiles.push_back({ph, pack(0, P->page_nrows[ph])});
      }
      for (int32_t lp = 0; lp < P->npages[u]; ++lp) {
        const int32_t ph = P->page_table[P->slot0[u] + lp];
        P->qpages.push_back({ph, P->page_nrows[ph], P->tile_off[u], P->tile_nonself[u] + lp + 1});
      }
    }
    P->tile_off[n] = (int32_t)P->tiles.size();

    // ---- 8. reader lists per KV page (fixed order: reader node, then tile order) -------
    std::vector<int64_t> cnt(n_pages + 1, 0);
    auto for_each_entry = [&](auto&& emit) {
      for (int32_t w = 0; w < n; ++w) {
        if (P->length[w] == 0) continue;
        for (int32_t t = P->tile_off[w]; t < P->tile_off[w] + P->tile_nonself[w]; ++t)
          emit(P->tiles[t].page, KEntry{P->slot0[w], 0, P->npages[w], P->tiles[t].lohi});
        for (int32_t lp = 0; lp < P->npages[w]; ++lp) {
          const int32_t ph = P->page_table[P->slot0[w] + lp];
          const int32_t nr = P->page_nrows[ph];
          emit(ph, KEntry{P->slot0[w], lp, lp + 1, pack(0, nr) | (1 << 16)});
          if (lp + 1 < P->npages[w]) emit(ph, KEntry{P->slot0[w], lp + 1, P->npages[w], pack(0, nr)});
        }
      }
    };
    for_each_entry([&](int32_t ph, const KEntry&) { cnt[ph + 1]++; });
    for (int32_t i = 0; i < n_pages; ++i) cnt[i + 1] += cnt[i];
    if (cnt[n_pages] > INT32_MAX) return fail(err, DAG_E_OVERFLOW, "reader lists too long");
    P->kv_off.assign(n_pages + 1, 0);
    for (int32_t i = 0; i <= n_pages; ++i) P->kv_off[i] = (int32_t)cnt[i];
    P->kentries.assign(cnt[n_pages], KEntry{0, 0, 0, 0});
    {
      std::vector<int64_t> fill(cnt.begin(), cnt.end() - 1);
      for_each_entry([&](int32_t ph, const KEntry& e) { P->kentries[fill[ph]++] = e; });
    }

    int64_t small_pages = 0;
    for (int32_t u = 0; u < n; ++u)
      if (P->length[u] > 0 && P->npages[u] <= 2) small_pages += P->npages[u];
    const bool small_in_pairs = 2 * small_pages > n_pages;
    auto in_pair = [&](int32_t u) { return small_in_pairs && P->npages[u] <= 2; };
    // KV pages for the dK/dV kernels: a node's pages in groups of four, 4 i .. 4 i + 3 (its
    // last group may hold fewer).  When nodes of one or two pages hold most of the plan's
    // pages (short segments), those go as pairs (or lone pages) instead, where the pair
    // kernel leaves fewer waves idle; otherwise they stay in groups, so that the one launch
    // takes every unit heaviest first (a second launch would start a long pair only after
    // the last group).  A group's reader steps are its
    // pages' reader lists unrolled into 32-row steps and merged by one logical key: the
    // other nodes' query pages first, by (reader node, query page, occurrence of that
    // query page in the page's list), then the pages' own node's query pages, last page
    // first.  A step carries every page's visible range (empty for a page its rows do not
    // read); a pair's the same, merged over its two pages.  Every key is logical, so the merged order does not depend on the physical
    // page placement.  Every page of a node has the same descendants and (per span) the
    // same mount readers, and the node's own pages come last, latest first, so the groups
    // of one node, which run side by side, walk the shared reader steps in step with each
    // other: a staged Q / dO tile fetched from HBM by one is served to the others from L2.
    {
      std::vector<int32_t> node_of_slot(n_pages, -1);
      for (int32_t w = 0; w < n; ++w)
        if (P->length[w] > 0) node_of_slot[P->slot0[w]] = w;
      struct Item {
        int32_t own, w, lq, k, qph;  // own: the page's own node (sorted last, lq descending)
        int32_t lo, hi, diag;
      };
      auto key_less = [](const Item& a, const Item& b) {
        if (a.own != b.own) return a.own < b.own;
        if (a.w != b.w) return a.w < b.w;
        if (a.lq != b.lq) return a.own ? a.lq > b.lq : a.lq < b.lq;
        return a.k < b.k;
      };
      auto items_of = [&](int32_t ph, int32_t u, std::vector<Item>& out) {
        out.clear();
        for (int32_t e = P->kv_off[ph]; e < P->kv_off[ph + 1]; ++e) {
          const KEntry& k = P->kentries[e];
          const int32_t w = node_of_slot[k.slot_base];
          const int32_t lh = k.lohi_diag;
          for (int32_t lq = k.lq0; lq < k.lq1; ++lq)
            out.push_back(Item{w == u ? 1 : 0, w, lq, 0, P->page_table[k.slot_base + lq], lh & 0xff, (lh >> 8) & 0xff,
                               (lh >> 16) & 1});
        }
        std::stable_sort(out.begin(), out.end(), key_less);  // k is still 0: ties keep list order
        for (size_t i = 1; i < out.size(); ++i)
          if (out[i].w == out[i - 1].w && out[i].lq == out[i - 1].lq) out[i].k = out[i - 1].k + 1;
      };
      // merge the m lists li[0 .. m) by key; emit(qph, rb, item or nullptr per list)
      std::vector<Item> li[kGroup];
      auto merge = [&](int m, auto&& emit) {
        size_t at[kGroup] = {};
        for (;;) {
          int first = -1;
          for (int i = 0; i < m; ++i)
            if (at[i] < li[i].size() && (first < 0 || key_less(li[i][at[i]], li[first][at[first]]))) first = i;
          if (first < 0) break;
          const Item head = li[first][at[first]];
          const Item* x[kGroup] = {};
          for (int i = 0; i < m; ++i)
            if (at[i] < li[i].size() && !key_less(head, li[i][at[i]])) x[i] = &li[i][at[i]++];
          const int32_t nr = P->page_nrows[head.qph];
          for (int32_t rb = 0; rb < (nr > 32 ? 2 : 1); ++rb) emit(head.qph, rb, x);
        }
      };
      P->kgroups.clear();
      P->kgroup_off.assign(1, 0);
      P->kgsteps.clear();
      P->kpairs.clear();
      P->kpair_off.assign(1, 0);
      P->kpsteps.clear();
      for (int32_t u = 0; u < n; ++u) {
        if (P->length[u] == 0) continue;
        const int32_t np = P->npages[u];
        if (in_pair(u)) {
          const int32_t pa = P->page_table[P->slot0[u]];
          const int32_t pb = np == 2 ? P->page_table[P->slot0[u] + 1] : -1;
          items_of(pa, u, li[0]);
          if (pb >= 0) items_of(pb, u, li[1]); else li[1].clear();
          merge(2, [&](int32_t qph, int32_t rb, const Item* const* x) {
            uint32_t info = (uint32_t)rb;
            for (int i = 0; i < 2; ++i)
              if (x[i])
                info |= ((uint32_t)(x[i]->lo << 1) | (uint32_t)(x[i]->hi << 8) | (uint32_t)(x[i]->diag << 15))
                        << (16 * i);
            P->kpsteps.push_back(KStep{qph, (int32_t)info});
          });
          P->kpairs.push_back(pa);
          P->kpairs.push_back(pb);
          P->kpair_off.push_back((int64_t)P->kpsteps.size());
          continue;
        }
        for (int32_t lp = 0; lp < np; lp += kGroup) {
          for (int i = 0; i < kGroup; ++i) {
            const int32_t ph = lp + i < np ? P->page_table[P->slot0[u] + lp + i] : -1;
            P->kgroups.push_back(ph);
            if (ph >= 0) items_of(ph, u, li[i]); else li[i].clear();
          }
          merge(kGroup, [&](int32_t qph, int32_t rb, const Item* const* x) {
            GStep st{qph, rb, {0u, 0u}};
            for (int i = 0; i < kGroup; ++i)
              if (x[i]) st.vis[i >> 1] |= gvis(x[i]->lo, x[i]->hi, x[i]->diag) << (16 * (i & 1));
            P->kgsteps.push_back(st);
          });
          P->kgroup_off.push_back((int64_t)P->kgsteps.size());
        }
      }
    }

    // ---- 9. launch orders -------------------------------------------------------------
    // Node-grouped, heaviest first: nodes sorted by their heaviest page's work, each
    // node's pages listed together (heaviest first).  Neighbouring work-groups then
    // share K/V tiles (forward, dQ: one node's query pages see the same tiles) or
    // reader lists (dK/dV: one node's KV pages are read by the same query pages).
    {
      std::vector<int64_t> wq(P->qpages.size(), 0);
      for (size_t i = 0; i < P->qpages.size(); ++i) {
        const QPage& q = P->qpages[i];
        int64_t keys = 0;
        for (int32_t t = q.tile_begin; t < q.tile_begin + q.tile_count; ++t)
          keys += ((P->tiles[t].lohi >> 8) & 0xff) - (P->tiles[t].lohi & 0xff);
        wq[i] = keys;
      }
      // query pages of node u are contiguous in qpages, lp ascending (heaviest last)
      std::vector<int32_t> qp_first(n + 1, 0);
      for (int32_t u = 0, c = 0; u < n; ++u) {
        qp_first[u] = c;
        c += P->length[u] > 0 ? P->npages[u] : 0;
        qp_first[u + 1] = c;
      }
      std::vector<int32_t> nodes_by(n);
      std::iota(nodes_by.begin(), nodes_by.end(), 0);
      auto node_wq = [&](int32_t u) { return qp_first[u + 1] > qp_first[u] ? wq[qp_first[u + 1] - 1] : -1; };
      std::stable_sort(nodes_by.begin(), nodes_by.end(), [&](int32_t a, int32_t b) { return node_wq(a) > node_wq(b); });
      P->fwd_order.clear();
      for (int32_t u : nodes_by)
        for (int32_t i = qp_first[u + 1] - 1; i >= qp_first[u]; --i) P->fwd_order.push_back(i);

      std::vector<int64_t> wk(n_pages, 0);
      for (int32_t ph = 0; ph < n_pages; ++ph) {
        int64_t w = 0;
        for (int32_t e = P->kv_off[ph]; e < P->kv_off[ph + 1]; ++e) {
          const KEntry& k = P->kentries[e];
          w += (int64_t)(k.lq1 - k.lq0) * (((k.lohi_diag >> 8) & 0xff) - (k.lohi_diag & 0xff));
        }
        wk[ph] = w;
      }
      auto node_wk = [&](int32_t u) {  // a node's first page has the most readers
        return P->length[u] > 0 ? wk[P->page_table[P->slot0[u]]] : -1;
      };
      std::stable_sort(nodes_by.begin(), nodes_by.end(), [&](int32_t a, int32_t b) { return node_wk(a) > node_wk(b); });
      P->bwd_order.clear();
      for (int32_t u : nodes_by)
        if (P->length[u] > 0)
          for (int32_t lp = 0; lp < P->npages[u]; ++lp) P->bwd_order.push_back(P->page_table[P->slot0[u] + lp]);
      // groups and pairs in the same node order (a node's groups are consecutive in
      // kgroups; a node of one or two pages has one pair instead)
      std::vector<int32_t> group0(n + 1, 0), pair0(n + 1, 0);
      for (int32_t u = 0, cg = 0, cp = 0; u < n; ++u) {
        group0[u] = cg;
        pair0[u] = cp;
        if (P->length[u] > 0) {
          if (in_pair(u))
            ++cp;
          else
            cg += (P->npages[u] + kGroup - 1) / kGroup;
        }
        group0[u + 1] = cg;
        pair0[u + 1] = cp;
      }
      P->group_order.clear();
      P->pair_order.clear();
      for (int32_t u : nodes_by) {
        for (int32_t i = group0[u]; i < group0[u + 1]; ++i) P->group_order.push_back(i);
        for (int32_t i = pair0[u]; i < pair0[u + 1]; ++i) P->pair_order.push_back(i);
      }
    }
  }

  // ---- info ------------------------------------------------------------------------
  dag_plan_info& I = P->info;
  I = dag_plan_info{};
  I.rows = (int64_t)P->pos_of_row.size();
  I.tokens = (int64_t)P->row_of_token.size();
  I.pages = (int64_t)P->page_nrows.size();
  I.query_pages = (int64_t)P->qpages.size();
  I.transitive = opts.transitive;
  I.view = opts.view;
  I.max_position = (int32_t)max_pos;
  std::vector<char> has_child(n, 0);
  for (int32_t u = 0; u < n; ++u)
    if (P->parent[u] >= 0) has_child[P->parent[u]] = 1;
  // multiplicity (HARTS Sec. 3.5): a node's tokens belong to every trajectory through it,
  // one per leaf below it; parents precede children, so one backward sweep sums them
  P->leaves_below.assign(n, 0);
  for (int32_t u = n - 1; u >= 0; --u) {
    if (!has_child[u]) P->leaves_below[u] += 1;
    if (P->parent[u] >= 0) P->leaves_below[P->parent[u]] += P->leaves_below[u];
  }
  for (int32_t u = 0; u < n; ++u) I.semantic_tokens += (int64_t)P->length[u] * P->leaves_below[u];
  for (int32_t u = 0; u < n; ++u) {
    int64_t nonself = 0;
    for (int64_t r = P->range_off[u]; r < P->range_off[u + 1]; ++r)
      nonself += P->ranges[3 * r + 2] - P->ranges[3 * r + 1];
    const int64_t L = P->length[u];
    I.visible_pairs += L * nonself + L * (L + 1) / 2;
    if (!has_child[u]) {
      const int64_t T = L + nonself;
      I.n_trajectories += 1;
      I.flat_rows += T;
      I.flat_pairs += T * (T + 1) / 2;
    }
  }
  for (const QPage& q : P->qpages) I.fwd_tiles += q.tile_count;
  I.bwd_entries = P->packed ? (int64_t)P->kpsteps.size() : (int64_t)P->kentries.size();
  I.pack_pages = P->packed ? 1 : 0;
  if (!P->packed) {  // the convolution walks a page's rows as one path: one node per page
    const dag_status cst = build_conv_tables(P, err);
    if (cst != DAG_OK) return cst;
  }
  if (opts.gdn_chunk > 0) return build_gdn_schedule(P, opts.gdn_chunk, err);
  return DAG_OK;
}

}  // namespace dagattn
