// Semantic position map of the original batch (HARTS Sec. 3.5, Eq. 17): for
// every trajectory, the compact row m(s) and the next token's vocabulary id y_s
// of each own token that has a next token, and the same positions grouped by row.
//
// A trajectory is a root-to-leaf chain, leaves taken depth-first (roots and
// children in table order).  Its flat sequence visits, node by node, the mounted
// tokens that become visible at that node and were not spliced earlier (in
// token order), then the node's own tokens.  Own tokens hold positions; spliced
// tokens are context (Octopus Sec. 3.4: their loss mask is zero), so they hold
// none but can be a target: an own token followed by a splice predicts the
// splice's first token.
#include <algorithm>
#include <climits>
#include <map>
#include <string>
#include <utility>
#include <vector>

#include "plan.hpp"

namespace dagattn {

namespace {

// Disjoint sorted [lo, hi) offsets per source node already spliced into the trajectory.
using Spliced = std::map<int32_t, std::vector<std::pair<int32_t, int32_t>>>;

// First offset in [lo, hi) not covered by the sorted disjoint intervals `have`; hi if none.
int32_t first_uncovered(const std::vector<std::pair<int32_t, int32_t>>& have, int32_t lo, int32_t hi) {
  int32_t x = lo;
  for (const auto& iv : have) {
    if (iv.second <= x) continue;
    if (iv.first > x) break;
    x = iv.second;
    if (x >= hi) break;
  }
  return x < hi ? x : hi;
}

void add_interval(std::vector<std::pair<int32_t, int32_t>>& have, int32_t lo, int32_t hi) {
  have.emplace_back(lo, hi);
  std::sort(have.begin(), have.end());
  std::vector<std::pair<int32_t, int32_t>> out;
  for (const auto& iv : have) {
    if (!out.empty() && iv.first <= out.back().second)
      out.back().second = std::max(out.back().second, iv.second);
    else
      out.push_back(iv);
  }
  have.swap(out);
}

}  // namespace

dag_status build_logprob_map(const Plan& P, const int32_t* labels, std::vector<int32_t>* pos_row,
                             std::vector<int32_t>* pos_target, std::string* err) {
  const int32_t n = P.n_nodes;
  std::vector<std::vector<int32_t>> children(n);
  for (int32_t u = 0; u < n; ++u)
    if (P.parent[u] >= 0) children[P.parent[u]].push_back(u);
  std::vector<int32_t> leaves;
  for (int32_t r = 0; r < n; ++r) {
    if (P.parent[r] != -1) continue;
    std::vector<int32_t> stack{r};
    while (!stack.empty()) {
      const int32_t u = stack.back();
      stack.pop_back();
      if (children[u].empty()) leaves.push_back(u);
      for (auto it = children[u].rbegin(); it != children[u].rend(); ++it) stack.push_back(*it);
    }
  }
  pos_row->clear();
  pos_target->clear();
  std::vector<char> on_chain(n, 0);
  std::vector<int32_t> chain;
  auto label_of = [&](int64_t tok, int32_t* y) -> bool {
    *y = labels[P.row_of_token[tok]];
    return *y >= 0;
  };
  for (int32_t leaf : leaves) {
    chain.clear();
    for (int32_t u = leaf; u >= 0; u = P.parent[u]) chain.push_back(u);
    std::reverse(chain.begin(), chain.end());
    for (int32_t a : chain) on_chain[a] = 1;
    Spliced spliced;
    int32_t pending = -1;  // row of the last own token, waiting for its target
    for (int32_t a : chain) {
      // mounted (non-ancestor) ranges of a: the earliest token not yet spliced
      int64_t first_new = INT64_MAX;
      std::vector<std::pair<int32_t, std::pair<int32_t, int32_t>>> mounted;
      for (int64_t i = P.range_off[a]; i < P.range_off[a + 1]; ++i) {
        const int32_t src = P.ranges[3 * i], lo = P.ranges[3 * i + 1], hi = P.ranges[3 * i + 2];
        if (on_chain[src] || hi <= lo) continue;  // an ancestor: part of the chain itself
        mounted.push_back({src, {lo, hi}});
        const auto it = spliced.find(src);
        const int32_t x = it == spliced.end() ? lo : first_uncovered(it->second, lo, hi);
        if (x < hi) first_new = std::min(first_new, P.tok_off[src] + x);
      }
      for (const auto& m : mounted) add_interval(spliced[m.first], m.second.first, m.second.second);
      if (first_new != INT64_MAX && pending >= 0) {
        int32_t y;
        if (!label_of(first_new, &y)) {
          *err = "negative label on a target row";
          for (int32_t c : chain) on_chain[c] = 0;
          return DAG_E_INVALID;
        }
        pos_row->push_back(pending);
        pos_target->push_back(y);
      }
      if (first_new != INT64_MAX) pending = -1;
      for (int32_t i = 0; i < P.length[a]; ++i) {
        const int64_t tok = P.tok_off[a] + i;
        if (pending >= 0) {
          int32_t y;
          if (!label_of(tok, &y)) {
            *err = "negative label on a target row";
            for (int32_t c : chain) on_chain[c] = 0;
            return DAG_E_INVALID;
          }
          pos_row->push_back(pending);
          pos_target->push_back(y);
        }
        pending = P.row_of_token[tok];
      }
      if (pos_row->size() > (size_t)INT32_MAX) {
        *err = "more than 2^31 - 1 semantic positions";
        for (int32_t c : chain) on_chain[c] = 0;
        return DAG_E_OVERFLOW;
      }
    }
    for (int32_t a : chain) on_chain[a] = 0;
  }
  return DAG_OK;
}

}  // namespace dagattn
