// Chunked linear-attention schedule over the rollout tree.
//
// HARTS: Hybrid-Attention RL over Tree Structures --
//   Sec. 2.2 Eq. 2: a branch that forks at p resumes from the chunk boundary
//     a(p) = B floor(p / B) and re-runs [a(p), p) ("replay");
//   Sec. 3.3: the tree contracted into fork-free segments; Eq. 11 (a side
//     branch can start in its parent's round only if the parent entered with a
//     ready anchor state and crosses no new chunk boundary); Eq. 12-14 (the two
//     minimum call counts T_pre, T_in); Algorithm 1 (recovery of the rounds, as
//     the text describes it); Eq. 15 (mandatory replay).
// The tree is the DAG's parent tree: recurrent layers skip mounted spans
// (Octopus Sec. 3).  Zero-length leaves carry no tokens and are pruned first;
// children are taken in node-table order.
#include <algorithm>
#include <climits>
#include <cstdio>
#include <map>

#include "plan.hpp"

namespace dagattn {
namespace {

struct Seg {
  std::vector<int32_t> nodes;
  int64_t s = 0, e = 0;  // recurrent index of the first token, one past the last
  int32_t parent = -1;
  std::vector<int32_t> ch;
};

struct SeqB {
  int32_t round;
  std::vector<int32_t> segs;
  int64_t start, fork;
  int32_t init_seq;
  int64_t init_b;
};

struct Task {
  bool spawn;      // create a new sequence for v first
  int32_t v;
  bool ready;      // the anchor state of v's entry exists before the round
  int32_t k;       // round budget
  int32_t r;       // round
  int32_t q;       // sequence v joins (when !spawn)
  int32_t init_seq;
  int64_t init_b, start, fork;
};

dag_status gfail(std::string* err, const char* msg, long long a = 0) {
  char buf[200];
  std::snprintf(buf, sizeof buf, msg, a);
  *err = buf;
  return DAG_E_OVERFLOW;
}

}  // namespace

dag_status build_gdn_schedule(Plan* P, int32_t B, std::string* err) {
  const int32_t n = P->n_nodes;
  // -- 1. prune zero-length leaves; children in table order; recurrent depth --------
  std::vector<char> alive(n, 0);
  for (int32_t u = n - 1; u >= 0; --u) {
    if (P->length[u] > 0) alive[u] = 1;
    if (alive[u] && P->parent[u] >= 0) alive[P->parent[u]] = 1;
  }
  std::vector<std::vector<int32_t>> kids(n);
  for (int32_t u = 0; u < n; ++u)
    if (alive[u] && P->parent[u] >= 0) kids[P->parent[u]].push_back(u);
  std::vector<int64_t> depth(n, 0);
  for (int32_t u = 0; u < n; ++u) {
    const int32_t p = P->parent[u];
    depth[u] = p < 0 ? 0 : depth[p] + P->length[p];
  }

  // -- 2. segments, depth-first preorder -------------------------------------------
  std::vector<Seg> segs;
  std::vector<std::pair<int32_t, int32_t>> st;
  for (int32_t root = 0; root < n; ++root) {
    if (P->parent[root] >= 0 || !alive[root]) continue;
    st.push_back({root, -1});
    while (!st.empty()) {
      const auto [u, par] = st.back();
      st.pop_back();
      Seg g;
      g.nodes.push_back(u);
      while (kids[g.nodes.back()].size() == 1) g.nodes.push_back(kids[g.nodes.back()][0]);
      const int32_t last = g.nodes.back();
      g.s = depth[u];
      g.e = depth[last] + P->length[last];
      g.parent = par;
      if (g.e > (int64_t)INT32_MAX - B) return gfail(err, "recurrent index %lld overflows int32", g.e);
      segs.push_back(std::move(g));
      const int32_t me = (int32_t)segs.size() - 1;
      if (par >= 0) segs[par].ch.push_back(me);
      for (auto it = kids[last].rbegin(); it != kids[last].rend(); ++it) st.push_back({*it, me});
    }
  }
  const int32_t S = (int32_t)segs.size();
  auto anchor = [B](int64_t p) { return (p / B) * B; };

  // -- 3. minimum call counts (Eq. 12-14), children before parents ---------------------
  std::vector<int32_t> tpre(S), tin(S);
  for (int32_t v = S - 1; v >= 0; --v) {
    const auto& ch = segs[v].ch;
    if (ch.empty()) {
      tpre[v] = tin[v] = 1;
      continue;
    }
    int32_t m1 = 0, m2 = 0, arg = -1;  // largest and second-largest child T_pre
    for (int32_t u : ch) {
      if (tpre[u] > m1) {
        m2 = m1;
        m1 = tpre[u];
        arg = u;
      } else if (tpre[u] > m2) {
        m2 = tpre[u];
      }
    }
    int32_t best = INT32_MAX;
    for (int32_t o : ch) best = std::min(best, std::max(tin[o], 1 + (o == arg ? m2 : m1)));
    tin[v] = best;
    tpre[v] = segs[v].e < anchor(segs[v].s) + B ? m1 : tin[v];
  }

  // -- 4. recovery (Algorithm 1), iterative; same visiting order as the recursion -----
  std::vector<SeqB> seqs;
  std::vector<Task> ts;
  for (int32_t root = 0; root < S; ++root) {
    if (segs[root].parent >= 0) continue;
    seqs.push_back({1, {}, 0, 0, -1, -1});
    ts.push_back({false, root, true, tpre[root], 1, (int32_t)seqs.size() - 1, -1, -1, 0, 0});
    while (!ts.empty()) {
      Task t = ts.back();
      ts.pop_back();
      if (t.spawn) {
        seqs.push_back({t.r, {}, t.start, t.fork, t.init_seq, t.init_b});
        ts.push_back({false, t.v, true, t.k, t.r, (int32_t)seqs.size() - 1, -1, -1, 0, 0});
        continue;
      }
      seqs[t.q].segs.push_back(t.v);
      const auto& ch = segs[t.v].ch;
      if (ch.empty()) continue;
      const int64_t ev = segs[t.v].e;
      const bool same = t.ready && ev < anchor(segs[t.v].s) + B;
      const int32_t delta = same ? 0 : 1;
      const int32_t kside = t.k - delta;
      int32_t f = 0;
      for (int32_t u : ch) f += tpre[u] > kside;
      int32_t direct = -1;
      for (int32_t o : ch) {
        const int32_t h = same ? tpre[o] : tin[o];
        if (h <= t.k && f - (tpre[o] > kside ? 1 : 0) == 0) {
          direct = o;
          break;
        }
      }
      if (direct < 0) {
        *err = "internal: no feasible direct continuation";
        return DAG_E_INVALID;
      }
      const int64_t b = anchor(ev);
      const int32_t iseq = same ? seqs[t.q].init_seq : t.q;
      const int64_t ib = same ? seqs[t.q].init_b : b;
      for (auto it = ch.rbegin(); it != ch.rend(); ++it)
        if (*it != direct) ts.push_back({true, *it, true, kside, t.r + delta, -1, iseq, ib, b, ev});
      ts.push_back({false, direct, same, t.k, t.r, t.q, -1, -1, 0, 0});
    }
  }
  const int32_t NS = (int32_t)seqs.size();

  // -- 5. token rows: replayed ancestor tokens, then own tokens --------------------------
  P->gseqs.assign(NS, GSeq{});
  P->gseq_info.assign(NS, dag_gdn_seq{});
  P->grows.clear();
  std::vector<std::pair<int32_t, int32_t>> rep;  // (row, replay index) of replayed tokens
  int64_t replay_total = 0, chunks = 0;
  int32_t rounds = 0;
  for (int32_t q = 0; q < NS; ++q) {
    const SeqB& s = seqs[q];
    GSeq& g = P->gseqs[q];
    g.tok_off = (int32_t)P->grows.size();
    g.start = (int32_t)s.start;
    g.n_replay = (int32_t)(s.fork - s.start);
    g.rep_off = (int32_t)replay_total;
    if (g.n_replay > 0) {
      std::vector<int64_t> back;  // token ids, last first
      int32_t x = segs[segs[s.segs[0]].parent].nodes.back();
      int64_t need = g.n_replay;
      while (need > 0) {
        const int64_t len = P->length[x];
        for (int64_t i = len - 1; i >= 0 && need > 0; --i, --need) back.push_back(P->tok_off[x] + i);
        x = P->parent[x];
      }
      for (auto it = back.rbegin(); it != back.rend(); ++it) {
        rep.push_back({P->row_of_token[*it], (int32_t)rep.size()});
        P->grows.push_back(P->row_of_token[*it]);
      }
    }
    int64_t own = 0;
    for (int32_t v : s.segs)
      for (int32_t u : segs[v].nodes) {
        for (int64_t i = 0; i < P->length[u]; ++i) P->grows.push_back(P->row_of_token[P->tok_off[u] + i]);
        own += P->length[u];
      }
    if ((int64_t)P->grows.size() > INT32_MAX) return gfail(err, "schedule tokens %lld overflow int32", (long long)P->grows.size());
    g.n_tok = (int32_t)((int64_t)P->grows.size() - g.tok_off);
    g.round = s.round;
    g.init_slot = -1;
    g.cgrad = -1;
    g.chunk_off = (int32_t)chunks;
    chunks += ((int64_t)g.n_tok + B - 1) / B;
    if (chunks > INT32_MAX) return gfail(err, "schedule chunks %lld overflow int32", chunks);
    replay_total += g.n_replay;
    rounds = std::max(rounds, s.round);
    dag_gdn_seq& info = P->gseq_info[q];
    info.round = s.round;
    info.first_node = segs[s.segs.front()].nodes.front();
    info.last_node = segs[s.segs.back()].nodes.back();
    info.start = (int32_t)s.start;
    info.fork = (int32_t)s.fork;
    info.own_tokens = (int32_t)own;
    info.init_seq = s.init_seq;
    info.init_boundary = s.init_seq >= 0 ? (int32_t)s.init_b : -1;
  }

  // -- 6. boundary-state slots, exports, consumers ---------------------------------------
  std::map<std::pair<int32_t, int64_t>, int32_t> slot_of;
  std::vector<std::vector<GExport>> exps(NS);
  std::vector<std::vector<int32_t>> cons;
  int32_t ncg = 0;
  for (int32_t q = 0; q < NS; ++q) {
    if (seqs[q].init_seq < 0) continue;
    const auto key = std::make_pair(seqs[q].init_seq, seqs[q].init_b);
    auto it = slot_of.find(key);
    if (it == slot_of.end()) {
      const int32_t slot = (int32_t)slot_of.size();
      it = slot_of.emplace(key, slot).first;
      const GSeq& pr = P->gseqs[key.first];
      const int64_t c = (key.second - pr.start) / B;
      if (c < 1 || c > ((int64_t)pr.n_tok + B - 1) / B) {
        *err = "internal: exported boundary outside its producer";
        return DAG_E_INVALID;
      }
      exps[key.first].push_back({(int32_t)c, slot});
      cons.emplace_back();
    }
    P->gseqs[q].init_slot = it->second;
    P->gseqs[q].cgrad = ncg++;
    cons[it->second].push_back(P->gseqs[q].cgrad);
  }
  P->gdn_ncgrad = ncg;
  P->gexports.clear();
  for (int32_t q = 0; q < NS; ++q) {
    std::sort(exps[q].begin(), exps[q].end(), [](const GExport& a, const GExport& b) { return a.chunk < b.chunk; });
    P->gseqs[q].exp_off = (int32_t)P->gexports.size();
    P->gseqs[q].exp_cnt = (int32_t)exps[q].size();
    P->gexports.insert(P->gexports.end(), exps[q].begin(), exps[q].end());
  }
  P->gslot_off.assign(1, 0);
  P->gslot_cons.clear();
  for (const auto& c : cons) {
    P->gslot_cons.insert(P->gslot_cons.end(), c.begin(), c.end());
    P->gslot_off.push_back((int32_t)P->gslot_cons.size());
  }

  // -- 7. rounds: sequences with the most tokens launch first ---------------------------
  P->ground_off.assign(rounds + 1, 0);
  P->ground_seq.clear();
  for (int32_t r = 1; r <= rounds; ++r) {
    std::vector<int32_t> ids;
    for (int32_t q = 0; q < NS; ++q)
      if (seqs[q].round == r) ids.push_back(q);
    std::stable_sort(ids.begin(), ids.end(), [&](int32_t a, int32_t b) { return P->gseqs[a].n_tok > P->gseqs[b].n_tok; });
    P->ground_seq.insert(P->ground_seq.end(), ids.begin(), ids.end());
    P->ground_off[r] = (int32_t)P->ground_seq.size();
  }
  // each round's chunks as independent work items (the chunk-parallel kernels)
  P->gitem_off.assign(rounds + 1, 0);
  P->gitems.clear();
  P->gdn_round_chunks_max = 0;
  for (int32_t r = 0; r < rounds; ++r) {
    const int64_t first = (int64_t)P->gitems.size() / 2;
    for (int32_t i = P->ground_off[r]; i < P->ground_off[r + 1]; ++i) {
      GSeq& g = P->gseqs[P->ground_seq[i]];
      g.item0 = (int32_t)((int64_t)P->gitems.size() / 2);
      const int32_t nch = (int32_t)(((int64_t)g.n_tok + B - 1) / B);
      for (int32_t c = 0; c < nch; ++c) {
        P->gitems.push_back(P->ground_seq[i]);
        P->gitems.push_back(c);
      }
    }
    const int64_t n = (int64_t)P->gitems.size() / 2 - first;
    if (n > INT32_MAX) return gfail(err, "round chunks %lld overflow int32", (long long)n);
    P->gitem_off[r + 1] = (int32_t)((int64_t)P->gitems.size() / 2);
    P->gdn_round_chunks_max = std::max(P->gdn_round_chunks_max, n);
  }

  // -- 8. replay fix-up lists: per row, its replayed occurrences in schedule order ------
  // (replay index = position of the token among all replayed tokens, sequence order)
  std::sort(rep.begin(), rep.end());
  P->grep_slot.assign(P->info.rows, -1);
  P->grep_rows.clear();
  P->grep_off.assign(1, 0);
  P->grep_tok.clear();
  for (size_t i = 0; i < rep.size(); ++i) {
    if (i == 0 || rep[i].first != rep[i - 1].first) {
      if (i) P->grep_off.push_back((int32_t)P->grep_tok.size());
      P->grep_slot[rep[i].first] = (int32_t)P->grep_rows.size();
      P->grep_rows.push_back(rep[i].first);
    }
    P->grep_tok.push_back(rep[i].second);
  }
  if (!rep.empty()) P->grep_off.push_back((int32_t)P->grep_tok.size());

  dag_plan_info& I = P->info;
  I.gdn_chunk = B;
  I.gdn_rounds = rounds;
  I.gdn_sequences = NS;
  I.gdn_replay = replay_total;
  I.gdn_slots = (int64_t)slot_of.size();
  I.gdn_chunks = chunks;
  I.gdn_segments = S;
  return DAG_OK;
}

}  // namespace dagattn
