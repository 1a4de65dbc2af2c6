// Host-side DAG compactor: turns tree and mount edges into an immutable plan.
//
// Plain C++17 with no HIP dependency, so it builds and is tested on a host
// without a GPU (and under the host sanitizers).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/dag_attn.h"

namespace dagattn {

constexpr int kPage = 64;  // rows per KV page and per query block

// One visited KV tile: a physical page and the half-open row range [lo, hi)
// of it that is visible.  Packed so a kernel fetches it with one 8-byte load.
struct Tile {
  int32_t page;
  int32_t lohi;  // lo | (hi << 8)
};

// One query block (= one page of a node's rows).  The tiles it visits are
// the first `tile_count` entries of its node's tile list starting at
// `tile_begin`: the node's visible non-self tiles, then the node's own pages
// 0..lp; the last one is the diagonal page, masked causally.
struct QPage {
  int32_t phys;
  int32_t nrows;
  int32_t tile_begin;
  int32_t tile_count;
};

// One reader-list entry of a KV page: the query pages [lq0, lq1) of the node
// whose page-table slots start at slot_base see rows [lo, hi) of the page;
// `diag` marks the page's own query block (causal mask).
struct KEntry {
  int32_t slot_base;
  int32_t lq0;
  int32_t lq1;
  int32_t lohi_diag;  // lo | (hi << 8) | (diag << 16)
};

// One 32-row step of a KV page pair's merged reader list (a node of one or two pages, or
// consecutive pages of a packed plan), as the pair dK/dV kernel walks it: rows 32 rb .. 32 rb + 31 of physical query page qph see rows [loA, hiA) of
// page A and [loB, hiB) of page B (an empty range: that page is not read by this
// step; diag: the page's own query block, masked causally).  Packed so a kernel
// fetches a step with one 8-byte load.
struct KStep {
  int32_t qph;
  int32_t info;  // rb | loA << 1 | hiA << 8 | diagA << 15 | loB << 17 | hiB << 24 | diagB << 31
};

// Mask ids of one merged reader step's two pages (packed plans): -1 = the step's range
// [lo, hi) alone says what the step's rows see of that page.
struct KMask {
  int32_t a, b;
};

// One 32-row step of a group of up to four KV pages (pages 4 i .. 4 i + 3 of one node),
// as the four-page dK/dV kernel walks it: rows 32 rb .. 32 rb + 31
// of physical query page qph see rows [lo, hi) of each page of the group (empty: not
// read by this step; diag: the page's own query block, masked causally).  Page i's 16
// bits sit in vis[i / 2] >> (16 (i % 2)) as lo | hi << 7 | diag << 14; 16 bytes, one load.
constexpr int kGroup = 4;
struct GStep {
  int32_t qph;
  int32_t rb;
  uint32_t vis[2];
};
inline constexpr uint32_t gvis(int lo, int hi, int diag) {
  return (uint32_t)lo | ((uint32_t)hi << 7) | ((uint32_t)diag << 14);
}
inline constexpr uint32_t gvis_of(const GStep& s, int i) { return (s.vis[i >> 1] >> (16 * (i & 1))) & 0xffffu; }
inline constexpr int gvis_lo(uint32_t v) { return (int)(v & 0x7f); }
inline constexpr int gvis_hi(uint32_t v) { return (int)((v >> 7) & 0x7f); }
inline constexpr int gvis_diag(uint32_t v) { return (int)((v >> 14) & 1); }

// A token within 3 steps after a page's last token on some path, with the rows
// 1, 2 and 3 steps before it on its own path (-1: none); the short convolution's
// backward reads these successors.
struct ConvExt {
  int32_t s, p1, p2, p3;
};

// One packed gated-delta-rule input sequence as the kernels read it.  Its
// tokens are rows[tok_off .. tok_off + n_tok): n_replay replayed ancestor
// tokens (state updates only), then its own tokens.  Token j sits at
// recurrent index start + j; start is a multiple of the chunk, so chunk c of
// the sequence is tokens [c B, c B + B).
struct GSeq {
  int32_t tok_off, n_tok, n_replay, start;
  int32_t init_slot;  // boundary state it starts from; -1: zero
  int32_t cgrad;      // index of its initial-state gradient buffer; -1 when init_slot < 0
  int32_t exp_off, exp_cnt;  // its exported boundary states: gexports[exp_off ..)
  int32_t chunk_off;  // first entry of its per-chunk saved states
  int32_t round;
  int32_t rep_off;    // replay index of its first replayed token (replay gradients)
  int32_t item0;      // index of its chunk 0 among all chunk items (rounds in order)
};
// An exported boundary: the state after `chunk` chunks of the sequence goes to `slot`.
struct GExport {
  int32_t chunk;
  int32_t slot;
};

struct DeviceTables;  // defined by the HIP side
struct Timing;        // defined by the HIP side

struct Plan {
  dag_build_opts opts{};
  int32_t n_nodes = 0;
  std::vector<int32_t> parent, length;
  std::vector<std::vector<dag_mount>> direct;  // non-empty mounts per node
  std::vector<int32_t> order;                  // dependency (topological) order
  std::vector<int32_t> start;                  // Eq. 2 start position per node
  std::vector<int64_t> tok_off;                // first token id per node
  std::vector<int32_t> slot0, npages;          // page-table slots per node
  std::vector<int32_t> page_table;             // slot -> physical page
  std::vector<int32_t> page_nrows;             // physical page -> valid rows
  std::vector<int64_t> range_off;              // node -> offset into ranges (triples)
  std::vector<int32_t> ranges;                 // (src, lo, hi) non-self visibility
  std::vector<int32_t> tile_off, tile_nonself; // node -> tile list
  std::vector<Tile> tiles;
  std::vector<QPage> qpages;
  std::vector<int32_t> fwd_order;              // query-page ids, heaviest first
  std::vector<int32_t> kv_off;                 // physical page -> first reader entry (size pages+1)
  std::vector<KEntry> kentries;
  std::vector<int32_t> bwd_order;              // physical pages with rows, heaviest first
  // dK/dV work: with one node per page, each node's pages in groups of four (its last
  // group may hold fewer), or, when nodes of one or two pages hold most pages, those as
  // pairs; a packed plan's pages in pairs of consecutive pages
  std::vector<int32_t> kgroups;                // kGroup pages per group (-1: none)
  std::vector<int64_t> kgroup_off;             // group -> its first merged reader step (size groups+1)
  std::vector<GStep> kgsteps;                  // merged reader steps of every group
  std::vector<int32_t> group_order;            // group ids, node-grouped, heaviest first
  std::vector<int32_t> kpairs;                 // KV page pairs (A, B; B = -1 for a lone page)
  std::vector<int64_t> kpair_off;              // pair -> its first merged reader step (size pairs+1)
  std::vector<KStep> kpsteps;                  // merged reader steps of every pair
  std::vector<int32_t> pair_order;             // pair ids, node-grouped, heaviest first
  // short causal convolution (see conv_plan.cpp)
  std::vector<int32_t> conv_prev;              // 4 per physical page: rows 1..3 steps before its first token
  std::vector<int64_t> conv_ext_off;           // physical page -> first successor entry (size pages+1)
  std::vector<ConvExt> conv_ext;
  std::vector<int32_t> leaves_below;           // per node: leaves in its subtree (itself if a leaf)
  // packed page layout (opts.pack_pages): several short nodes share a page, so what a
  // query row sees of a KV page can differ from row to row; such a tile carries a mask
  bool packed = false;
  std::vector<int64_t> node_row0;              // first compact row of every node (-1: no tokens)
  std::vector<int32_t> tile_mask;              // per tile: mask id, -1 = [lo, hi) for every row
  std::vector<uint64_t> masks;                 // per mask id: 64 row masks (bit c: key row c), then
                                               // 64 key masks (bit r: query row r)
  std::vector<KMask> kstep_mask;               // per merged reader step
  std::vector<int32_t> pos_of_row;             // C
  std::vector<int32_t> row_of_token;           // U
  // gated-delta-rule schedule (empty when opts.gdn_chunk == 0)
  std::vector<dag_gdn_seq> gseq_info;          // per sequence, for queries
  std::vector<GSeq> gseqs;
  std::vector<int32_t> grows;                  // compact row of each sequence token
  std::vector<GExport> gexports;
  std::vector<int32_t> gslot_off, gslot_cons;  // slot -> consumers' cgrad ids, sequence order
  std::vector<int32_t> ground_off, ground_seq; // round r (0-based) -> sequences, most tokens first
  // round r's chunks, gitems[2 i] = sequence, gitems[2 i + 1] = chunk, for i in
  // [gitem_off[r], gitem_off[r + 1]): the round's sequences in ground_seq order, chunks ascending
  std::vector<int32_t> gitem_off, gitems;
  int64_t gdn_round_chunks_max = 0;            // most chunk items in one round
  // replay fix-up: rows that are replayed somewhere, each with its replay indices
  // (in schedule order); grep_slot maps every row to its position in grep_rows or -1
  std::vector<int32_t> grep_rows, grep_off, grep_tok, grep_slot;
  int32_t gdn_ncgrad = 0;
  dag_plan_info info{};
  DeviceTables* dev = nullptr;
  Timing* timing = nullptr;
};

// Compile; returns DAG_OK or an error code with a message in `err`.
dag_status build_plan(const dag_node* nodes, int32_t n_nodes, const dag_mount* mounts,
                      int32_t n_mounts, const dag_build_opts* opts, Plan* out, std::string* err);

// Packed page layout and its attention tables (steps 6-9 of build_plan for opts.pack_pages).
dag_status build_packed_tables(Plan* P, std::string* err);

// Short-convolution tables (HARTS Sec. 4.2) over the plan's parent tree and rows.
dag_status build_conv_tables(Plan* P, std::string* err);

// Linear-attention schedule (HARTS Sec. 3.3) over the plan's parent tree;
// needs the plan's rows (row_of_token) to be built.
dag_status build_gdn_schedule(Plan* P, int32_t chunk, std::string* err);

// Semantic position map of the original batch (HARTS Sec. 3.5): m(s) and y_s of
// every nonterminal position in batch order.  labels: vocabulary id per compact row.
dag_status build_logprob_map(const Plan& P, const int32_t* labels, std::vector<int32_t>* pos_row,
                             std::vector<int32_t>* pos_target, std::string* err);

}  // namespace dagattn
