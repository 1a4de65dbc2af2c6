// Trajectory ingestion and prefix-aware microbatch planning, host only
// (HARTS: Hybrid-Attention RL over Tree Structures, Sec. 3.1-3.2).
//
// Ingestion: raw root-to-leaf token sequences become the trie of their shared
// prefixes, as a DAG node table (maximal unbranched runs; every trajectory ends
// at a leaf of its own).  Planning: the trajectories are sorted lexicographically;
// the compact work of a set is its trie's node count (Eq. 5), of a contiguous
// interval a prefix-sum difference, of any set the sum over its sorted members of
// length minus the LCP with the previous member, where LCP of two sorted
// trajectories is the minimum adjacent LCP between them (sparse-table range
// minimum).  Candidates: exact DP over contiguous partitions (N <= N0) or merge /
// split evolution of the natural partition at sampled K (N > N0), one trie-aware
// greedy candidate (best of four orders x two policies with Eq. 10's insertion
// cost, then sparse repair) and, for N > N0, boundary-refined anchors.  Each is
// assigned to replicas and slots and the lexicographically smallest
// (total work, summed slot-critical work, largest replica work) wins (Eq. 4).
// Every tie is broken towards the earliest item in a stated order, so the plan is
// a deterministic function of the input.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <string>
#include <vector>

#include "harts_plan.hpp"

namespace dagattn {

namespace {

constexpr int kQMax = 32, kNear = 8, kRefine = 3;

struct Seqs {
  const int32_t* tok;
  const int64_t* off;
  int64_t len(int32_t i) const { return off[i + 1] - off[i]; }
  bool less(int32_t a, int32_t b) const {
    return std::lexicographical_compare(tok + off[a], tok + off[a + 1], tok + off[b], tok + off[b + 1]);
  }
  int64_t lcp(int32_t a, int32_t b) const {
    const int64_t n = std::min(len(a), len(b));
    const int32_t *x = tok + off[a], *y = tok + off[b];
    int64_t k = 0;
    while (k < n && x[k] == y[k]) ++k;
    return k;
  }
};

std::vector<int32_t> lex_order(const Seqs& S, int32_t n) {
  std::vector<int32_t> ord(n);
  for (int32_t i = 0; i < n; ++i) ord[i] = i;
  std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) { return S.less(a, b); });
  return ord;
}

using Parts = std::vector<std::pair<int32_t, int32_t>>;  // contiguous [a, b] of sorted positions
using Groups = std::vector<std::vector<int32_t>>;         // sets of sorted positions

struct Cand {
  Groups groups;
  std::vector<int64_t> work;
  std::vector<int32_t> replica, slot;
  int64_t J[3];
};

class Planner {
 public:
  Planner(const Seqs& S, int32_t n, int32_t D, int64_t T) : S_(S), N(n), D_(D), T_(T) {
    order = lex_order(S, n);
    len.resize(N);
    L.assign(N, 0);
    for (int32_t p = 0; p < N; ++p) len[p] = S.len(order[p]);
    for (int32_t p = 1; p < N; ++p) L[p] = S.lcp(order[p - 1], order[p]);
    pl.assign(N + 1, 0);
    pL.assign(N + 1, 0);
    for (int32_t p = 0; p < N; ++p) {
      pl[p + 1] = pl[p] + len[p];
      pL[p + 1] = pL[p] + L[p];
    }
    // sparse table over L for LCP of any two sorted positions
    int lg = 1;
    while ((1 << lg) <= N) ++lg;
    rmq.assign(lg, std::vector<int64_t>(N));
    rmq[0] = L;
    for (int k = 1; k < lg; ++k)
      for (int32_t i = 0; i + (1 << k) <= N; ++i) rmq[k][i] = std::min(rmq[k - 1][i], rmq[k - 1][i + (1 << (k - 1))]);
  }

  // LCP of sorted positions i < j: min L[i+1 .. j]
  int64_t lcp(int32_t i, int32_t j) const {
    if (i > j) std::swap(i, j);
    if (i == j) return len[i];
    const int32_t a = i + 1, n = j - a + 1;
    int k = 31 - __builtin_clz((unsigned)n);
    return std::min(rmq[k][a], rmq[k][j - (1 << k) + 1]);
  }
  int64_t W(int32_t a, int32_t b) const { return pl[b + 1] - pl[a] - (pL[b + 1] - pL[a + 1]); }
  // work of a sorted member list
  int64_t C(const std::vector<int32_t>& g) const {
    if (g.empty()) return 0;
    int64_t w = len[g[0]];
    for (size_t i = 1; i < g.size(); ++i) w += len[g[i]] - lcp(g[i - 1], g[i]);
    return w;
  }
  // Eq. 10: increase of C when x joins the sorted list g (x not in g)
  int64_t insert_cost(const std::vector<int32_t>& g, int32_t x) const {
    auto it = std::lower_bound(g.begin(), g.end(), x);
    int64_t d = len[x];
    const bool hp = it != g.begin(), hq = it != g.end();
    if (hp) d -= lcp(*(it - 1), x);
    if (hq) d -= lcp(x, *it);
    if (hp && hq) d += lcp(*(it - 1), *it);
    return d;
  }
  // decrease of C when x (a member) leaves the sorted list g
  int64_t remove_cost(const std::vector<int32_t>& g, int32_t x) const {
    auto it = std::lower_bound(g.begin(), g.end(), x);
    int64_t d = len[x];
    const bool hp = it != g.begin(), hq = it + 1 != g.end();
    if (hp) d -= lcp(*(it - 1), x);
    if (hq) d -= lcp(x, *(it + 1));
    if (hp && hq) d += lcp(*(it - 1), *(it + 1));
    return d;
  }

  bool natural(Parts* out, std::string* err) const {
    // explicit stack: intervals still to examine, leftmost first
    std::vector<std::pair<int32_t, int32_t>> st{{0, N - 1}};
    while (!st.empty()) {
      auto [a, b] = st.back();
      st.pop_back();
      if (W(a, b) <= T_) {
        out->push_back({a, b});
        continue;
      }
      if (a == b) {
        *err = "a trajectory of " + std::to_string(len[a]) + " tokens exceeds the capacity " + std::to_string(T_);
        return false;
      }
      int32_t bt = -1;
      int64_t k0 = 0, k1 = 0, k2 = 0;
      for (int32_t t = a + 1; t <= b; ++t) {
        const int64_t l = W(a, t - 1), r = W(t, b);
        const int64_t c0 = L[t], c1 = std::max(l, r), c2 = l > r ? l - r : r - l;
        if (bt < 0 || c0 < k0 || (c0 == k0 && (c1 < k1 || (c1 == k1 && c2 < k2)))) {
          bt = t;
          k0 = c0;
          k1 = c1;
          k2 = c2;
        }
      }
      st.push_back({bt, b});
      st.push_back({a, bt - 1});
    }
    return true;
  }

  std::vector<int32_t> k_range(int32_t K0) const {
    const int64_t G = W(0, N - 1);
    const int64_t kmin = (int64_t)D_ * std::max<int64_t>(1, (G + T_ * D_ - 1) / (T_ * D_));
    const int64_t kmax = std::max(kmin, std::min<int64_t>((int64_t)D_ * ((K0 + D_ - 1) / D_), (int64_t)D_ * (N / D_)));
    std::vector<int32_t> ks;
    for (int64_t k = kmin; k <= kmax; k += D_) ks.push_back((int32_t)k);
    return ks;
  }

  // exact DP (Eq. 9) for all K <= Kmax at once; F[k][e] = (total, max) or infeasible
  std::vector<Parts> exact(const std::vector<int32_t>& ks) const {
    const int32_t Kmax = ks.empty() ? 0 : ks.back();
    std::vector<Parts> res(ks.size());  // empty: no feasible partition for that K
    const int32_t KK = std::min(Kmax, N);
    const int64_t INF = INT64_MAX;
    std::vector<std::vector<int64_t>> Ft(KK + 1, std::vector<int64_t>(N + 1, INF)), Fm = Ft;
    std::vector<std::vector<int32_t>> arg(KK + 1, std::vector<int32_t>(N + 1, -1));
    Ft[0][0] = 0;
    Fm[0][0] = 0;
    for (int32_t k = 1; k <= KK; ++k)
      for (int32_t e = k; e <= N; ++e) {
        int64_t bt = INF, bm = INF;
        int32_t bs = -1;
        for (int32_t s = k - 1; s < e; ++s) {
          if (Ft[k - 1][s] == INF) continue;
          const int64_t w = W(s, e - 1);
          if (w > T_) continue;
          const int64_t t = Ft[k - 1][s] + w, m = std::max(Fm[k - 1][s], w);
          if (bs < 0 || t < bt || (t == bt && m < bm)) {
            bt = t;
            bm = m;
            bs = s;
          }
        }
        Ft[k][e] = bt;
        Fm[k][e] = bm;
        arg[k][e] = bs;
      }
    for (size_t i = 0; i < ks.size(); ++i) {
      const int32_t K = ks[i];
      if (K > KK || Ft[K][N] == INF) continue;
      Parts p(K);
      int32_t e = N;
      for (int32_t k = K; k >= 1; --k) {
        const int32_t s = arg[k][e];
        p[k - 1] = {s, e - 1};
        e = s;
      }
      res[i] = std::move(p);
    }
    return res;
  }

  std::vector<int32_t> sample_k(const std::vector<int32_t>& ks) const {
    if ((int)ks.size() <= kQMax) return ks;
    std::vector<int32_t> s(ks.begin(), ks.begin() + kQMax / 2);
    const int ns = kQMax - kQMax / 2;
    const int64_t m = (int64_t)ks.size() - 1;
    for (int i = 0; i < ns; ++i) {
      const int64_t num = i * m, q = num / (ns - 1), r = num % (ns - 1);
      s.push_back(ks[q + (2 * r > ns - 1 ? 1 : 0)]);
    }
    std::sort(s.begin(), s.end());
    s.erase(std::unique(s.begin(), s.end()), s.end());
    return s;
  }

  bool evolve(const Parts& P0, int32_t K, Parts* out) const {
    Parts parts = P0;
    while ((int32_t)parts.size() > K) {
      int64_t best = -1;
      int32_t bi = -1;
      for (int32_t i = 0; i + 1 < (int32_t)parts.size(); ++i) {
        if (W(parts[i].first, parts[i + 1].second) > T_) continue;
        const int64_t saving = L[parts[i + 1].first];
        if (bi < 0 || saving > best) {
          best = saving;
          bi = i;
        }
      }
      if (bi < 0) return false;
      parts[bi] = {parts[bi].first, parts[bi + 1].second};
      parts.erase(parts.begin() + bi + 1);
    }
    while ((int32_t)parts.size() < K) {
      int64_t best = 0;
      int32_t bi = -1, bt = -1;
      for (int32_t i = 0; i < (int32_t)parts.size(); ++i)
        for (int32_t t = parts[i].first + 1; t <= parts[i].second; ++t)
          if (bi < 0 || L[t] < best) {
            best = L[t];
            bi = i;
            bt = t;
          }
      if (bi < 0) return false;
      const auto [a, b] = parts[bi];
      parts[bi] = {a, bt - 1};
      parts.insert(parts.begin() + bi + 1, {bt, b});
    }
    *out = parts;
    return true;
  }

  Parts refine(Parts parts) const {
    for (int sweep = 0; sweep < 2; ++sweep) {
      bool changed = false;
      for (size_t i = 0; i + 1 < parts.size(); ++i) {
        const int32_t a = parts[i].first, b = parts[i + 1].second, t0 = parts[i + 1].first;
        int64_t b0 = W(a, t0 - 1) + W(t0, b), b1 = std::max(W(a, t0 - 1), W(t0, b));
        int32_t bt = t0;
        for (int32_t t = std::max(a + 1, t0 - kNear); t <= std::min(b, t0 + kNear); ++t) {
          const int64_t l = W(a, t - 1), r = W(t, b);
          if (l > T_ || r > T_) continue;
          const int64_t c0 = l + r, c1 = std::max(l, r);
          if (c0 < b0 || (c0 == b0 && c1 < b1)) {
            b0 = c0;
            b1 = c1;
            bt = t;
          }
        }
        if (bt != t0) {
          parts[i] = {a, bt - 1};
          parts[i + 1] = {bt, b};
          changed = true;
        }
      }
      if (!changed) break;
    }
    return parts;
  }

  // ---- trie-aware greedy ---------------------------------------------------------
  std::vector<std::vector<int32_t>> orders() const {
    std::vector<int32_t> asc(N);
    for (int32_t i = 0; i < N; ++i) asc[i] = i;
    std::vector<int32_t> desc(asc.rbegin(), asc.rend());
    std::vector<int32_t> by_len = asc, by_u = asc;
    std::stable_sort(by_len.begin(), by_len.end(), [&](int32_t a, int32_t b) { return len[a] > len[b]; });
    auto u = [&](int32_t p) {
      const int64_t l = p > 0 ? L[p] : 0, r = p + 1 < N ? L[p + 1] : 0;
      return len[p] - std::max(l, r);
    };
    std::stable_sort(by_u.begin(), by_u.end(), [&](int32_t a, int32_t b) { return u(a) > u(b); });
    return {asc, desc, by_len, by_u};
  }

  // groups kept sorted, with their work cached
  struct GState {
    Groups g;
    std::vector<int64_t> w;
  };

  int32_t place(const GState& s, int32_t x, bool best_fit, int32_t exclude) const {
    int64_t best = 0;
    int32_t bi = -1;
    for (int32_t gi = 0; gi < (int32_t)s.g.size(); ++gi) {
      if (gi == exclude || s.g[gi].empty()) continue;
      const int64_t d = insert_cost(s.g[gi], x), w = s.w[gi] + d;
      if (w > T_) continue;
      const int64_t key = best_fit ? w : len[x] - d;
      if (bi < 0 || key > best) {
        best = key;
        bi = gi;
      }
    }
    return bi;
  }
  void add(GState& s, int32_t gi, int32_t x) const {
    s.w[gi] += insert_cost(s.g[gi], x);
    s.g[gi].insert(std::lower_bound(s.g[gi].begin(), s.g[gi].end(), x), x);
  }
  void drop(GState& s, int32_t gi, int32_t x) const {
    s.w[gi] -= remove_cost(s.g[gi], x);
    s.g[gi].erase(std::lower_bound(s.g[gi].begin(), s.g[gi].end(), x));
  }

  bool greedy(const std::vector<int32_t>& ord, bool best_fit, Groups* out) const {
    GState s;
    for (int32_t x : ord) {
      const int32_t gi = place(s, x, best_fit, -1);
      if (gi < 0) {
        s.g.push_back({x});
        s.w.push_back(len[x]);
      } else {
        add(s, gi, x);
      }
    }
    // eliminate small microbatches
    while (s.g.size() > 1) {
      int32_t light = 0;
      for (int32_t i = 1; i < (int32_t)s.g.size(); ++i)
        if (s.w[i] < s.w[light]) light = i;
      GState t = s;
      const std::vector<int32_t> moved = t.g[light];
      t.g[light].clear();
      t.w[light] = 0;
      bool ok = true;
      for (int32_t x : moved) {
        const int32_t gi = place(t, x, best_fit, light);
        if (gi < 0) {
          ok = false;
          break;
        }
        add(t, gi, x);
      }
      if (!ok) break;
      t.g.erase(t.g.begin() + light);
      t.w.erase(t.w.begin() + light);
      s = std::move(t);
    }
    // K to a multiple of D by singleton splits
    while (s.g.size() % D_) {
      int64_t best = 0;
      int32_t bg = -1, bx = -1;
      for (int32_t gi = 0; gi < (int32_t)s.g.size(); ++gi) {
        if (s.g[gi].size() < 2) continue;
        for (int32_t x : s.g[gi]) {
          const int64_t inc = len[x] - remove_cost(s.g[gi], x);
          if (bg < 0 || inc < best) {
            best = inc;
            bg = gi;
            bx = x;
          }
        }
      }
      if (bg < 0) return false;
      drop(s, bg, bx);
      s.g.push_back({bx});
      s.w.push_back(len[bx]);
    }
    *out = s.g;
    return true;
  }

  Groups sparse_repair(Groups g) const {
    std::vector<int64_t> w(g.size());
    for (size_t i = 0; i < g.size(); ++i) w[i] = C(g[i]);
    std::vector<int32_t> where(N);
    for (int it = 0; it < 4; ++it) {
      for (int32_t gi = 0; gi < (int32_t)g.size(); ++gi)
        for (int32_t x : g[gi]) where[x] = gi;
      int64_t best = 0;
      int kind = 0;
      int32_t bx = -1, by = -1, bA = -1, bB = -1;
      for (int32_t x = 0; x < N; ++x) {
        const int32_t A = where[x];
        if (g[A].size() < 2) continue;
        const int64_t restA = w[A] - remove_cost(g[A], x);
        for (int32_t B = 0; B < (int32_t)g.size(); ++B) {
          if (B == A) continue;
          bool near = false;
          for (int32_t y : g[B])
            if (y >= x - kNear && y <= x + kNear) {
              near = true;
              break;
            }
          if (!near) continue;
          const int64_t newB = w[B] + insert_cost(g[B], x);
          if (newB > T_) continue;
          const int64_t gain = w[A] + w[B] - restA - newB;
          if (gain > 0 && (kind == 0 || gain > best)) {
            best = gain;
            kind = 1;
            bx = x;
            bA = A;
            bB = B;
          }
        }
      }
      if (kind == 0) {
        for (int32_t x = 0; x < N; ++x)
          for (int32_t y = x + 1; y < std::min(N, x + kNear + 1); ++y) {
            const int32_t A = where[x], B = where[y];
            if (A == B) continue;
            std::vector<int32_t> nA = g[A], nB = g[B];
            nA.erase(std::lower_bound(nA.begin(), nA.end(), x));
            nA.insert(std::lower_bound(nA.begin(), nA.end(), y), y);
            nB.erase(std::lower_bound(nB.begin(), nB.end(), y));
            nB.insert(std::lower_bound(nB.begin(), nB.end(), x), x);
            const int64_t cA = C(nA), cB = C(nB);
            if (cA > T_ || cB > T_) continue;
            const int64_t gain = w[A] + w[B] - cA - cB;
            if (gain > 0 && (kind == 0 || gain > best)) {
              best = gain;
              kind = 2;
              bx = x;
              by = y;
            }
          }
      }
      if (kind == 0) break;
      if (kind == 1) {
        g[bA].erase(std::lower_bound(g[bA].begin(), g[bA].end(), bx));
        g[bB].insert(std::lower_bound(g[bB].begin(), g[bB].end(), bx), bx);
        w[bA] = C(g[bA]);
        w[bB] = C(g[bB]);
      } else {
        const int32_t A = where[bx], B = where[by];
        g[A].erase(std::lower_bound(g[A].begin(), g[A].end(), bx));
        g[A].insert(std::lower_bound(g[A].begin(), g[A].end(), by), by);
        g[B].erase(std::lower_bound(g[B].begin(), g[B].end(), by));
        g[B].insert(std::lower_bound(g[B].begin(), g[B].end(), bx), bx);
        w[A] = C(g[A]);
        w[B] = C(g[B]);
      }
    }
    return g;
  }

  Cand assign(Groups g) const {
    Cand c;
    const int32_t K = (int32_t)g.size();
    c.work.resize(K);
    for (int32_t i = 0; i < K; ++i) c.work[i] = C(g[i]);
    std::vector<int32_t> byw(K);
    for (int32_t i = 0; i < K; ++i) byw[i] = i;
    std::stable_sort(byw.begin(), byw.end(), [&](int32_t a, int32_t b) { return c.work[a] > c.work[b]; });
    c.replica.assign(K, 0);
    c.slot.assign(K, 0);
    std::vector<int64_t> cum(D_, 0);
    int64_t crit = 0;
    for (int32_t j = 0; j < K / D_; ++j) {
      std::vector<char> used(D_, 0);
      int64_t mx = 0;
      for (int32_t q = 0; q < D_; ++q) {
        const int32_t i = byw[j * D_ + q];
        int32_t d = -1;
        for (int32_t r = 0; r < D_; ++r)
          if (!used[r] && (d < 0 || cum[r] < cum[d])) d = r;
        used[d] = 1;
        c.replica[i] = d;
        c.slot[i] = j;
        cum[d] += c.work[i];
        mx = std::max(mx, c.work[i]);
      }
      crit += mx;
    }
    int64_t tot = 0;
    for (int64_t x : c.work) tot += x;
    c.J[0] = tot;
    c.J[1] = crit;
    c.J[2] = *std::max_element(cum.begin(), cum.end());
    c.groups = std::move(g);
    return c;
  }

  static Groups of_parts(const Parts& p) {
    Groups g;
    for (auto [a, b] : p) {
      std::vector<int32_t> m;
      for (int32_t i = a; i <= b; ++i) m.push_back(i);
      g.push_back(std::move(m));
    }
    return g;
  }
  int64_t total(const Groups& g) const {
    int64_t t = 0;
    for (const auto& m : g) t += C(m);
    return t;
  }

  bool plan(int32_t n0, Cand* best, dag_mb_info* info, std::string* err) const {
    Parts P0;
    if (!natural(&P0, err)) return false;
    const std::vector<int32_t> ks = k_range((int32_t)P0.size());
    const bool exact_mode = N <= n0;
    std::vector<Cand> cands;
    std::vector<std::pair<int32_t, Parts>> base;  // K and its contiguous partition, generation order
    if (exact_mode) {
      const std::vector<Parts> ex = exact(ks);
      for (size_t i = 0; i < ks.size(); ++i)
        if (!ex[i].empty()) {
          base.push_back({ks[i], ex[i]});
          cands.push_back(assign(of_parts(ex[i])));
        }
    } else {
      for (int32_t K : sample_k(ks)) {
        Parts p;
        if (!evolve(P0, K, &p)) continue;
        base.push_back({K, p});
        cands.push_back(assign(of_parts(p)));
      }
    }
    const size_t n_base = cands.size();
    int32_t gk = -1;
    {
      Groups bestg;
      int64_t bk = 0, bt = 0;
      bool have = false;
      for (const auto& ord : orders())
        for (bool bf : {true, false}) {
          Groups g;
          if (!greedy(ord, bf, &g)) continue;
          const int64_t k = (int64_t)g.size(), t = total(g);
          if (!have || k < bk || (k == bk && t < bt)) {
            have = true;
            bk = k;
            bt = t;
            bestg = std::move(g);
          }
        }
      if (have) {
        gk = (int32_t)bestg.size();
        cands.push_back(assign(sparse_repair(std::move(bestg))));
      }
    }
    if (!exact_mode && n_base > 0) {
      std::vector<int32_t> anchors;
      auto has = [&](int32_t K) { return std::find(anchors.begin(), anchors.end(), K) != anchors.end(); };
      auto base_of = [&](int32_t K) -> int {
        for (size_t i = 0; i < base.size(); ++i)
          if (base[i].first == K) return (int)i;
        return -1;
      };
      if (gk >= 0 && base_of(gk) >= 0) anchors.push_back(gk);
      int lo = 0;
      for (size_t i = 1; i < base.size(); ++i)
        if (cands[i].J[0] < cands[lo].J[0] || (cands[i].J[0] == cands[lo].J[0] && base[i].first < base[lo].first))
          lo = (int)i;
      if (!has(base[lo].first)) anchors.push_back(base[lo].first);
      if (gk >= 0) {
        int32_t pick = -1;
        for (const auto& b : base) {
          if (has(b.first)) continue;
          const int64_t d = std::abs((int64_t)b.first - gk), dp = pick < 0 ? 0 : std::abs((int64_t)pick - gk);
          if (pick < 0 || d < dp || (d == dp && b.first < pick)) pick = b.first;
        }
        if (pick >= 0) anchors.push_back(pick);
      }
      for (size_t i = 0; i < anchors.size() && (int)i < kRefine; ++i)
        cands.push_back(assign(of_parts(refine(base[base_of(anchors[i])].second))));
    }
    if (cands.empty()) {
      *err = "no feasible plan for this capacity and replica count";
      return false;
    }
    size_t bi = 0;
    for (size_t i = 1; i < cands.size(); ++i) {
      const int64_t* a = cands[i].J;
      const int64_t* b = cands[bi].J;
      if (a[0] < b[0] || (a[0] == b[0] && (a[1] < b[1] || (a[1] == b[1] && a[2] < b[2])))) bi = i;
    }
    *best = std::move(cands[bi]);
    info->microbatches = (int32_t)best->groups.size();
    info->exact = exact_mode ? 1 : 0;
    info->natural_microbatches = (int32_t)P0.size();
    info->candidates = (int32_t)cands.size();
    info->total_work = best->J[0];
    info->slot_critical_work = best->J[1];
    info->max_replica_work = best->J[2];
    info->trie_work = W(0, N - 1);
    return true;
  }

  const Seqs& S_;
  const int32_t N;
  const int32_t D_;
  const int64_t T_;
  std::vector<int32_t> order;
  std::vector<int64_t> len, L, pl, pL;
  std::vector<std::vector<int64_t>> rmq;
};

dag_status check_trajs(const int32_t* tokens, const int64_t* traj_off, int32_t n_traj, std::string* err) {
  if (n_traj < 1 || !traj_off || (!tokens && traj_off[n_traj] > 0)) {
    *err = "need at least one trajectory and its offsets";
    return DAG_E_INVALID;
  }
  if (traj_off[0] != 0) {
    *err = "traj_off[0] must be 0";
    return DAG_E_INVALID;
  }
  for (int32_t i = 0; i < n_traj; ++i)
    if (traj_off[i + 1] < traj_off[i]) {
      *err = "traj_off must be non-decreasing";
      return DAG_E_INVALID;
    }
  return DAG_OK;
}

}  // namespace

dag_status trie_build(const int32_t* tokens, const int64_t* traj_off, int32_t n_traj, TrieOut* out, std::string* err) {
  dag_status st = check_trajs(tokens, traj_off, n_traj, err);
  if (st != DAG_OK) return st;
  const Seqs S{tokens, traj_off};
  const std::vector<int32_t> ord = lex_order(S, n_traj);
  // compressed trie built along the sorted order; temporary node ids, renumbered depth-first at the end
  struct TNode {
    int64_t s, e;   // depth range [s, e)
    int32_t rep;    // a trajectory holding these tokens
    std::vector<int32_t> kids;
    std::vector<int32_t> ends;  // trajectories ending at depth e here
  };
  std::vector<TNode> nd;
  std::vector<int32_t> roots, stack;
  for (int32_t k = 0; k < n_traj; ++k) {
    const int32_t x = ord[k];
    const int64_t l = k ? S.lcp(ord[k - 1], x) : 0, n = S.len(x);
    while (!stack.empty() && nd[stack.back()].s >= l) stack.pop_back();
    if (!stack.empty() && nd[stack.back()].e > l) {  // branch inside the top node: split it at depth l
      const int32_t top = stack.back();
      TNode low{l, nd[top].e, nd[top].rep, std::move(nd[top].kids), std::move(nd[top].ends)};
      nd[top].e = l;
      nd[top].kids.clear();
      nd[top].ends.clear();
      nd.push_back(std::move(low));
      nd[top].kids.push_back((int32_t)nd.size() - 1);
    }
    if (n > l || (stack.empty() && n == l)) {  // new tokens below the branch point (or an empty first root)
      nd.push_back({l, n, x, {}, {x}});
      const int32_t id = (int32_t)nd.size() - 1;
      if (stack.empty())
        roots.push_back(id);
      else
        nd[stack.back()].kids.push_back(id);
      stack.push_back(id);
    } else {
      nd[stack.back()].ends.push_back(x);  // ends where the branch point is
    }
  }
  // depth-first numbering; a node's ending trajectories get zero-length leaves of their own
  // (first among its children: a prefix sorts before its extensions) unless the node is a
  // leaf with exactly one of them
  out->nodes.clear();
  out->tok_off.assign(1, 0);
  out->tokens.clear();
  out->leaf_of_traj.assign(n_traj, -1);
  struct Frame {
    int32_t t, parent;
  };
  std::vector<Frame> st2;
  for (auto it = roots.rbegin(); it != roots.rend(); ++it) st2.push_back({*it, -1});
  while (!st2.empty()) {
    const Frame f = st2.back();
    st2.pop_back();
    const TNode& t = nd[f.t];
    const int32_t id = (int32_t)out->nodes.size();
    out->nodes.push_back({f.parent, (int32_t)(t.e - t.s), 0, 0});
    const int32_t* src = tokens + traj_off[t.rep] + t.s;
    out->tokens.insert(out->tokens.end(), src, src + (t.e - t.s));
    out->tok_off.push_back((int64_t)out->tokens.size());
    if (t.kids.empty() && t.ends.size() == 1) {
      out->leaf_of_traj[t.ends[0]] = id;
    } else {
      for (int32_t x : t.ends) {
        out->leaf_of_traj[x] = (int32_t)out->nodes.size();
        out->nodes.push_back({id, 0, 0, 0});
        out->tok_off.push_back((int64_t)out->tokens.size());
      }
    }
    for (auto it = t.kids.rbegin(); it != t.kids.rend(); ++it) st2.push_back({*it, id});
    if ((int64_t)out->nodes.size() > INT32_MAX - 1 || (int64_t)out->tokens.size() > INT32_MAX) {
      *err = "the trie exceeds 2^31 - 1 nodes or tokens";
      return DAG_E_OVERFLOW;
    }
  }
  return DAG_OK;
}

dag_status microbatch_plan(const int32_t* tokens, const int64_t* traj_off, int32_t n_traj, const dag_mb_opts* o,
                           MbOut* out, std::string* err) {
  dag_status st = check_trajs(tokens, traj_off, n_traj, err);
  if (st != DAG_OK) return st;
  if (!o || o->replicas < 1 || o->capacity < 1 || o->exact_max < 0) {
    *err = "replicas and capacity must be positive, exact_max non-negative";
    return DAG_E_INVALID;
  }
  if (n_traj < o->replicas) {
    *err = "fewer trajectories than replicas";
    return DAG_E_INVALID;
  }
  const Seqs S{tokens, traj_off};
  Planner P(S, n_traj, o->replicas, o->capacity);
  Cand c;
  if (!P.plan(o->exact_max ? o->exact_max : 512, &c, &out->info, err)) return DAG_E_INVALID;
  const int32_t K = (int32_t)c.groups.size();
  out->mb_of_traj.assign(n_traj, -1);
  for (int32_t m = 0; m < K; ++m)
    for (int32_t p : c.groups[m]) out->mb_of_traj[P.order[p]] = m;
  out->replica = c.replica;
  out->slot = c.slot;
  out->work = c.work;
  return DAG_OK;
}

}  // namespace dagattn
