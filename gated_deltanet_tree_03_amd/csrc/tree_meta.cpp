// Tree metadata: parent pointers -> depth and strict-ancestor bitmasks.
//
// Nodes are laid out in DFS pre-order (review page of "TreeWY: Speculative
// Verification for Gated DeltaNet Hybrids", "Method"), so ancestors precede
// descendants.  In a pre-order every node's parent lies on the path from the
// root to the previous node; that is the check made here, and it is what lets
// the verify kernel keep the current root-to-node path as a depth-indexed
// stack.  One forward pass: anc[t] = anc[p] | (1 << p).
#include <string.h>

#include "../../include/treewy.h"
#include "treewy_internal.h"

namespace treewy {

int build_tree(const int32_t* parent, int n, TreeArgs* out) {
  if (parent == nullptr || out == nullptr) return TREEWY_ERR_ARG;
  if (n < 1 || n > kMaxNodes) return TREEWY_ERR_ARG;
  memset(out, 0, sizeof(*out));
  if (parent[0] != -1) return TREEWY_ERR_TREE;
  out->parent[0] = -1;
  out->depth[0] = 0;
  out->anc[0] = 0;
  // current root-to-(t-1) path as a bitmask
  uint64_t path = 1ull;
  int max_depth = 0;
  for (int t = 1; t < n; ++t) {
    const int p = parent[t];
    if (p < 0 || p >= t) return TREEWY_ERR_TREE;
    if (((path >> p) & 1ull) == 0) return TREEWY_ERR_TREE;  // not pre-order
    out->parent[t] = static_cast<int8_t>(p);
    out->depth[t] = static_cast<int8_t>(out->depth[p] + 1);
    out->anc[t] = out->anc[p] | (1ull << p);
    path = out->anc[t] | (1ull << t);
    if (out->depth[t] > max_depth) max_depth = out->depth[t];
  }
  out->n = n;
  out->max_depth = max_depth;
  return TREEWY_OK;
}

}  // namespace treewy
