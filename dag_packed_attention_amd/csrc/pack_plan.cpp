// Packed page layout for trees of short segments.
//
// With one node per page, a tree whose turns are a few tokens long (HARTS App. A,
// Figs. 6-8: segments of 1-15 tokens) leaves most of every 64-row page empty, and the
// kernels stage and multiply those padding rows like real ones.  Here the nodes are
// laid out in depth-first preorder (children in table order) and share pages: a node
// that fits in the rest of the open page goes there, a longer one starts a fresh page
// and its last page stays open for the nodes after it.  A node's rows stay contiguous
// and a page's valid rows stay a prefix, so row maps, padding and every consumer that
// reads rows by the plan's maps are unchanged.
//
// What a query row sees is the set of Octopus Sec. 3.3 Eq. 4 (ancestors, active mounted
// spans, its own earlier tokens).  Rows of one page can belong to different nodes and
// see a KV page differently; per (query page, KV page) pair the builder forms the 64 x 64
// visibility matrix.  If every valid row sees the same contiguous key range, the tile is
// a plain [lo, hi) range as in the unpacked layout; otherwise it keeps the matrix as a
// mask (row-major for the forward and dQ kernels, where a lane holds a query row, and
// key-major for the dK/dV kernel, where a lane holds a key).  A page's own tile is always
// masked and listed last; a masked tile's mask is exact, so the kernels apply the causal
// rule of an unpacked page's last tile only to unmasked tiles (a mounted span of a node
// that comes later in depth-first order can sit above its reader in the same page).
//
// dK/dV: KV pages are paired in layout order (2i, 2i + 1); a pair's reader steps are the
// query pages that see either page, in page order, 32 rows per step, each step with the
// two pages' ranges and mask ids; a step whose rows see neither page is dropped.
#include <algorithm>
#include <climits>
#include <numeric>

#include "plan.hpp"

namespace dagattn {

namespace {

struct Seg {
  int32_t u;     // node
  int32_t r0;    // first row inside the page
  int32_t r1;    // one past the last row
  int32_t off0;  // node offset of row r0
};

uint64_t bit_range(int a, int b) {  // bits [a, b), 0 <= a <= b <= 64
  if (a >= b) return 0;
  const uint64_t hi = b == 64 ? ~0ull : ((1ull << b) - 1);
  return hi & ~((1ull << a) - 1);
}

}  // namespace

dag_status build_packed_tables(Plan* P, std::string* err) {
  const int32_t n = P->n_nodes;
  if (P->opts.page_shuffle) {
    *err = "pack_pages cannot be combined with page_shuffle";
    return DAG_E_UNSUPPORTED;
  }
  P->packed = true;
  // ---- depth-first preorder, children in table order ------------------------------
  std::vector<std::vector<int32_t>> children(n);
  for (int32_t u = 0; u < n; ++u)
    if (P->parent[u] >= 0) children[P->parent[u]].push_back(u);
  std::vector<int32_t> pre, stack;
  pre.reserve(n);
  for (int32_t r = 0; r < n; ++r) {
    if (P->parent[r] != -1) continue;
    stack.push_back(r);
    while (!stack.empty()) {
      const int32_t u = stack.back();
      stack.pop_back();
      pre.push_back(u);
      for (auto it = children[u].rbegin(); it != children[u].rend(); ++it) stack.push_back(*it);
    }
  }
  // ---- placement ----------------------------------------------------------------
  P->node_row0.assign(n, -1);
  int64_t pages = 0;
  int32_t used = 0;  // rows taken in the open page (page pages - 1); 0: no open page
  for (int32_t u : pre) {
    const int32_t L = P->length[u];
    if (L == 0) continue;
    if (used > 0 && L <= kPage - used) {
      P->node_row0[u] = (pages - 1) * kPage + used;
      used += L;
      if (used == kPage) used = 0;
    } else {
      P->node_row0[u] = pages * kPage;
      pages += ((int64_t)L + kPage - 1) / kPage;
      used = L % kPage;
    }
  }
  if (pages * kPage > INT32_MAX) {
    *err = "compact rows exceed int32";
    return DAG_E_OVERFLOW;
  }
  const int32_t n_pages = (int32_t)pages;
  const int64_t C = pages * kPage;
  int64_t tokens = 0;
  P->tok_off.assign(n, 0);
  for (int32_t u = 0; u < n; ++u) {
    P->tok_off[u] = tokens;
    tokens += P->length[u];
  }
  P->page_nrows.assign(n_pages, 0);
  P->pos_of_row.assign(C, -1);
  P->row_of_token.assign(tokens, 0);
  P->page_table.resize(n_pages);
  std::iota(P->page_table.begin(), P->page_table.end(), 0);
  P->slot0.assign(n, 0);
  P->npages.assign(n, 0);
  std::vector<std::vector<Seg>> segs(n_pages);
  for (int32_t u : pre) {
    const int32_t L = P->length[u];
    if (L == 0) continue;
    const int64_t r0 = P->node_row0[u];
    P->slot0[u] = (int32_t)(r0 / kPage);
    P->npages[u] = (int32_t)((r0 + L - 1) / kPage - r0 / kPage + 1);
    for (int32_t i = 0; i < L; ++i) {
      P->pos_of_row[r0 + i] = P->start[u] + i;
      P->row_of_token[P->tok_off[u] + i] = (int32_t)(r0 + i);
    }
    for (int32_t i = 0; i < L;) {
      const int64_t row = r0 + i;
      const int32_t pg = (int32_t)(row / kPage), r = (int32_t)(row % kPage);
      const int32_t take = std::min(L - i, kPage - r);
      segs[pg].push_back({u, r, r + take, i});
      P->page_nrows[pg] = std::max(P->page_nrows[pg], r + take);
      i += take;
    }
  }
  // ---- per query page: visible KV pages and their tiles -----------------------------
  // visible offsets of src for u: u's non-self ranges (merged per source, disjoint)
  auto ranges_of = [&](int32_t u, int32_t src, auto&& fn) {
    for (int64_t k = P->range_off[u]; k < P->range_off[u + 1]; ++k)
      if (P->ranges[3 * k] == src) fn(P->ranges[3 * k + 1], P->ranges[3 * k + 2]);
  };
  P->tiles.clear();
  P->tile_mask.clear();
  P->masks.clear();
  P->qpages.clear();
  std::vector<int64_t> qwork;
  std::vector<int32_t> cand;
  uint64_t M[kPage];
  auto add_pages = [&](int64_t row_a, int64_t row_b) {  // pages holding rows [row_a, row_b)
    if (row_a >= row_b) return;
    for (int64_t pg = row_a / kPage; pg <= (row_b - 1) / kPage; ++pg) cand.push_back((int32_t)pg);
  };
  for (int32_t Q = 0; Q < n_pages; ++Q) {
    const int32_t nq = P->page_nrows[Q];
    if (nq == 0) continue;
    cand.clear();
    for (const Seg& s : segs[Q]) {
      add_pages(P->node_row0[s.u], P->node_row0[s.u] + s.off0 + (s.r1 - s.r0));
      for (int64_t k = P->range_off[s.u]; k < P->range_off[s.u + 1]; ++k) {
        const int32_t src = P->ranges[3 * k], lo = P->ranges[3 * k + 1], hi = P->ranges[3 * k + 2];
        add_pages(P->node_row0[src] + lo, P->node_row0[src] + hi);
      }
    }
    std::sort(cand.begin(), cand.end());
    cand.erase(std::unique(cand.begin(), cand.end()), cand.end());
    // the page itself last
    cand.erase(std::remove(cand.begin(), cand.end(), Q), cand.end());
    cand.push_back(Q);
    if ((int64_t)P->tiles.size() + (int64_t)cand.size() > INT32_MAX / 2) {
      *err = "tile lists too long";
      return DAG_E_OVERFLOW;
    }
    const int32_t tile_begin = (int32_t)P->tiles.size();
    int64_t work = 0;
    for (int32_t K : cand) {
      std::fill(M, M + kPage, 0ull);
      for (const Seg& s : segs[Q])
        for (const Seg& t : segs[K]) {
          if (t.u == s.u) {  // own tokens: offset j <= i
            for (int32_t r = s.r0; r < s.r1; ++r) {
              const int32_t i = s.off0 + r - s.r0;
              const int32_t c_hi = std::min(t.r1, t.r0 + (i - t.off0) + 1);
              M[r] |= bit_range(t.r0, std::max(c_hi, t.r0));
            }
          } else {
            uint64_t b = 0;
            ranges_of(s.u, t.u, [&](int32_t lo, int32_t hi) {
              const int32_t a = std::max(lo, t.off0), e = std::min(hi, t.off0 + (t.r1 - t.r0));
              if (a < e) b |= bit_range(t.r0 + a - t.off0, t.r0 + e - t.off0);
            });
            if (b)
              for (int32_t r = s.r0; r < s.r1; ++r) M[r] |= b;
          }
        }
      uint64_t any = 0;
      bool same = true;
      for (int32_t r = 0; r < nq; ++r) {
        any |= M[r];
        same = same && M[r] == M[0];
        work += __builtin_popcountll(M[r]);
      }
      if (!any) continue;
      const int lo = __builtin_ctzll(any), hi = 64 - __builtin_clzll(any);
      const bool contiguous = same && M[0] == bit_range(lo, hi);
      P->tiles.push_back({K, lo | (hi << 8)});
      if (contiguous && K != Q) {
        P->tile_mask.push_back(-1);
      } else {
        if (P->masks.size() / (2 * kPage) >= (size_t)INT32_MAX) {
          *err = "too many tile masks";
          return DAG_E_OVERFLOW;
        }
        P->tile_mask.push_back((int32_t)(P->masks.size() / (2 * kPage)));
        for (int32_t r = 0; r < kPage; ++r) P->masks.push_back(r < nq ? M[r] : 0ull);
        for (int32_t c = 0; c < kPage; ++c) {
          uint64_t col = 0;
          for (int32_t r = 0; r < nq; ++r) col |= ((M[r] >> c) & 1ull) << r;
          P->masks.push_back(col);
        }
      }
    }
    P->qpages.push_back({Q, nq, tile_begin, (int32_t)P->tiles.size() - tile_begin});
    qwork.push_back(work);
  }
  // ---- launch order of query pages: heaviest first ---------------------------------
  P->fwd_order.resize(P->qpages.size());
  std::iota(P->fwd_order.begin(), P->fwd_order.end(), 0);
  std::stable_sort(P->fwd_order.begin(), P->fwd_order.end(),
                   [&](int32_t a, int32_t b) { return qwork[a] > qwork[b]; });
  // ---- reader lists per KV page, then pairs ------------------------------------------
  struct Rd {
    int32_t q;     // query page
    int32_t lohi;  // lo | hi << 8
    int32_t mask;  // -1 or mask id
  };
  std::vector<std::vector<Rd>> readers(n_pages);
  for (const QPage& qp : P->qpages)
    for (int32_t t = qp.tile_begin; t < qp.tile_begin + qp.tile_count; ++t)
      readers[P->tiles[t].page].push_back({qp.phys, P->tiles[t].lohi, P->tile_mask[t]});
  // rows [32 rb, 32 rb + 32) of query page q see something of the page through reader x
  auto half_sees = [&](const Rd& x, int rb) {
    if (x.mask < 0) return true;
    const uint64_t* rm = &P->masks[(size_t)x.mask * 2 * kPage];
    for (int r = 32 * rb; r < 32 * rb + 32; ++r)
      if (rm[r]) return true;
    return false;
  };
  P->kentries.clear();
  P->kv_off.assign(n_pages + 1, 0);
  P->bwd_order.clear();
  P->kgroups.clear();  // packed plans run every page in pairs
  P->kgroup_off.assign(1, 0);
  P->kgsteps.clear();
  P->group_order.clear();
  P->kpairs.clear();
  P->kpair_off.assign(1, 0);
  P->kpsteps.clear();
  P->kstep_mask.clear();
  std::vector<int64_t> pwork;
  for (int32_t A = 0; A < n_pages; A += 2) {
    const int32_t B = A + 1 < n_pages ? A + 1 : -1;
    const std::vector<Rd>& la = readers[A];
    static const std::vector<Rd> none;
    const std::vector<Rd>& lb = B >= 0 ? readers[B] : none;
    size_t ia = 0, ib = 0;
    int64_t w = 0;
    while (ia < la.size() || ib < lb.size()) {
      const Rd* xa = nullptr;
      const Rd* xb = nullptr;
      if (ib == lb.size() || (ia < la.size() && la[ia].q < lb[ib].q)) {
        xa = &la[ia++];
      } else if (ia == la.size() || lb[ib].q < la[ia].q) {
        xb = &lb[ib++];
      } else {
        xa = &la[ia++];
        xb = &lb[ib++];
      }
      const int32_t q = xa ? xa->q : xb->q;
      const int32_t nr = P->page_nrows[q];
      for (int32_t rb = 0; rb < (nr > 32 ? 2 : 1); ++rb) {
        const bool sa = xa && half_sees(*xa, rb), sb = xb && half_sees(*xb, rb);
        if (!sa && !sb) continue;
        const uint32_t ia_ = sa ? (uint32_t)(((xa->lohi & 0xff) << 1) | (((xa->lohi >> 8) & 0xff) << 8)) : 0u;
        const uint32_t ib_ = sb ? (uint32_t)(((xb->lohi & 0xff) << 1) | (((xb->lohi >> 8) & 0xff) << 8)) : 0u;
        P->kpsteps.push_back(KStep{q, (int32_t)((uint32_t)rb | ia_ | (ib_ << 16))});
        P->kstep_mask.push_back(KMask{sa ? xa->mask : -1, sb ? xb->mask : -1});
        w += (sa ? 1 : 0) + (sb ? 1 : 0);
      }
    }
    if ((int64_t)P->kpsteps.size() == P->kpair_off.back()) {
      // pages no query row reads (cannot happen: every row reads itself); keep the pair
      // launchable with one empty step
      P->kpsteps.push_back(KStep{A, 0});
      P->kstep_mask.push_back(KMask{-1, -1});
    }
    P->kpairs.push_back(A);
    P->kpairs.push_back(B);
    P->kpair_off.push_back((int64_t)P->kpsteps.size());
    pwork.push_back(w);
  }
  P->pair_order.resize(pwork.size());
  std::iota(P->pair_order.begin(), P->pair_order.end(), 0);
  std::stable_sort(P->pair_order.begin(), P->pair_order.end(),
                   [&](int32_t a, int32_t b) { return pwork[a] > pwork[b]; });
  return DAG_OK;
}

}  // namespace dagattn
