// Tables of the short causal convolution over the rollout tree (HARTS Sec. 4.2:
// a width-w window takes its history from the token's true ancestors only, w <= 4).
//
// The history of own token (u, i) is its root-to-node path with mounted spans
// skipped: the previous token is (u, i - 1), or the last token of the nearest
// ancestor with tokens.  Kernels run one 64-row page at a time, so per physical
// page the plan keeps
//   conv_prev[4p + k]   the row k + 1 steps before the page's first token (-1: none), k < 3
//   conv_ext[...]       every token within 3 steps after the page's last token on
//                       any path (the next page's first rows, or the first tokens of
//                       the children, grandchildren ... at a fork), each as
//                       {row, rows 1, 2 and 3 steps before it}, children in table order;
//                       page p's entries are conv_ext[conv_ext_off[p] .. conv_ext_off[p+1]).
// The backward needs these successors: a token's input gradient sums the taps of
// every output whose window holds it, on every branch.
#include <algorithm>
#include <climits>
#include <string>
#include <vector>

#include "plan.hpp"

namespace dagattn {

namespace {

struct Tok {
  int32_t u, i;
};

}  // namespace

dag_status build_conv_tables(Plan* P, std::string* err) {
  const int32_t n = P->n_nodes;
  std::vector<std::vector<int32_t>> children(n);
  for (int32_t u = 0; u < n; ++u)
    if (P->parent[u] >= 0) children[P->parent[u]].push_back(u);
  auto row = [&](Tok t) { return P->row_of_token[P->tok_off[t.u] + t.i]; };
  // previous token on the path, u/i = -1 if none
  auto pred = [&](Tok t) -> Tok {
    if (t.i > 0) return {t.u, t.i - 1};
    int32_t a = P->parent[t.u];
    while (a >= 0 && P->length[a] == 0) a = P->parent[a];
    return a < 0 ? Tok{-1, -1} : Tok{a, P->length[a] - 1};
  };
  // tokens m steps into the subtree below the end of node v (m >= 1), children in table order
  std::vector<Tok> found;
  auto below = [&](auto&& self, int32_t v, int32_t m) -> void {
    for (int32_t c : children[v]) {
      if (m <= P->length[c])
        found.push_back({c, m - 1});
      else
        self(self, c, m - P->length[c]);
    }
  };
  const int64_t pages = P->info.pages;
  P->conv_prev.assign(4 * pages, -1);
  P->conv_ext_off.assign(pages + 1, 0);
  std::vector<std::vector<ConvExt>> ext(pages);
  for (int32_t u = 0; u < n; ++u) {
    const int32_t L = P->length[u];
    for (int32_t j = 0; j < P->npages[u]; ++j) {
      const int32_t phys = P->page_table[P->slot0[u] + j];
      const int32_t i0 = 64 * j, i1 = std::min(L, i0 + 64) - 1;  // first and last own offsets
      Tok t{u, i0};
      for (int k = 0; k < 3; ++k) {
        t = pred(t);
        if (t.u < 0) break;
        P->conv_prev[4 * phys + k] = row(t);
      }
      found.clear();
      for (int32_t d = 1; d <= 3; ++d) {
        if (i1 + d < L)
          found.push_back({u, i1 + d});
        else
          below(below, u, i1 + d - (L - 1));
      }
      for (const Tok& s : found) {
        ConvExt e{row(s), -1, -1, -1};
        Tok q = s;
        int32_t* p[3] = {&e.p1, &e.p2, &e.p3};
        for (int k = 0; k < 3; ++k) {
          q = pred(q);
          if (q.u < 0) break;
          *p[k] = row(q);
        }
        ext[phys].push_back(e);
      }
    }
  }
  int64_t total = 0;
  for (int64_t p = 0; p < pages; ++p) {
    P->conv_ext_off[p] = total;
    total += (int64_t)ext[p].size();
  }
  P->conv_ext_off[pages] = total;
  if (total > INT32_MAX) {
    *err = "convolution successor table exceeds 2^31 - 1 entries";
    return DAG_E_OVERFLOW;
  }
  P->conv_ext.clear();
  P->conv_ext.reserve(total);
  for (int64_t p = 0; p < pages; ++p) P->conv_ext.insert(P->conv_ext.end(), ext[p].begin(), ext[p].end());
  return DAG_OK;
}

}  // namespace dagattn
