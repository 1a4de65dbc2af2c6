// Trajectory ingestion and prefix-aware microbatch planning (harts_plan.cpp), host only.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/dag_attn.h"

namespace dagattn {

struct TrieOut {
  std::vector<dag_node> nodes;       // parent < child, no mounts
  std::vector<int64_t> tok_off;      // node u's tokens: tokens[tok_off[u] .. tok_off[u+1])
  std::vector<int32_t> tokens;       // the compact token sequence, node by node
  std::vector<int32_t> leaf_of_traj;
};

struct MbOut {
  std::vector<int32_t> mb_of_traj, replica, slot;
  std::vector<int64_t> work;
  dag_mb_info info{};
};

dag_status trie_build(const int32_t* tokens, const int64_t* traj_off, int32_t n_traj, TrieOut* out,
                      std::string* err);
dag_status microbatch_plan(const int32_t* tokens, const int64_t* traj_off, int32_t n_traj, const dag_mb_opts* o,
                           MbOut* out, std::string* err);

}  // namespace dagattn
