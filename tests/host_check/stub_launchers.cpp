// Host-only stand-ins for the kernel launchers, linked with the library's host
// layer (api.cpp, tree_meta.cpp) into a build with no GPU code, so that the
// host layer can run under AddressSanitizer and UndefinedBehaviorSanitizer on
// a machine without a GPU.  Every launcher checks the invariants the kernels
// rely on (node counts, batch sizes, non-null buffers), counts the call and
// returns success; hipGetLastError reports no error.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "treewy_internal.h"

namespace treewy {
namespace {

int g_launches = 0;

void require(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "stub launcher: violated invariant: %s\n", what);
    abort();
  }
}

void check_tree(const TreeArgs& t) {
  require(t.n >= 1 && t.n <= kMaxNodes, "1 <= tree.n <= 64");
  require(t.max_depth >= 0 && t.max_depth < t.n, "0 <= tree.max_depth < tree.n");
}

void check_verify(const VerifyArgs& a) {
  require(a.B > 0 && a.H > 0, "non-empty batch");
  require(a.S0 && a.q && a.k && a.v && a.alpha && a.beta && a.out && a.vtilde && a.gamma,
          "verify buffers");
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, const TreeArgs& tree, hipStream_t) {
  check_verify(a);
  check_tree(tree);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_commit_verify(const VerifyArgs& a, const TreeArgs& tree, const TreeArgs& prev,
                                hipStream_t) {
  check_verify(a);
  check_tree(tree);
  check_tree(prev);
  require(a.S_out && a.vt_prev && a.k_prev && a.gamma_prev, "previous-step buffers");
  require(a.n_prev == prev.n, "n_prev is the previous tree's node count");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_commit_verify_pool_trees(const VerifyArgs& a, const TreeArgs& bound,
                                           const TreeArgs& prev_bound, hipStream_t) {
  check_verify(a);
  require(a.trees && a.trees_prev && a.slots && a.n_slots >= 1, "pool and descriptors");
  require(bound.n >= 1 && bound.n <= kMaxNodes && bound.max_depth < bound.n, "node bound");
  require(prev_bound.n >= 1 && prev_bound.n <= kMaxNodes && prev_bound.max_depth < prev_bound.n,
          "previous node bound");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_commit(const CommitArgs& a, const TreeArgs& tree, hipStream_t) {
  require(a.B > 0 && a.H > 0 && a.S0 && a.vtilde && a.k && a.gamma && a.S_out, "commit buffers");
  check_tree(tree);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_store_all(const StoreAllArgs& a, const TreeArgs& tree, hipStream_t) {
  require(a.B > 0 && a.H > 0 && a.S0 && a.out && a.snapshots, "store_all buffers");
  check_tree(tree);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_store_all_select(const SelectArgs& a, hipStream_t) {
  require(a.B > 0 && a.H > 0 && a.N >= 1 && a.N <= kMaxNodes, "select sizes");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t) {
  require(a.B > 0 && a.H > 0 && a.T > 0 && a.S && a.out, "prefill sizes");
  ++g_launches;
  return hipSuccess;
}

// A fake device scratch (never dereferenced: the launchers above are stand-ins).
hipError_t scratch_buffer(float** ptr, size_t* bytes) {
  *ptr = reinterpret_cast<float*>(uintptr_t(1) << 40);
  *bytes = kScratchBytes;
  return hipSuccess;
}

}  // namespace treewy

extern "C" hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}

extern "C" hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
  *device = 0;
  return hipSuccess;
}

// The number of launcher calls so far (the host-check build's own export).
extern "C" int treewy_hostcheck_launches(void) { return treewy::g_launches; }

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
