// commit-then-verify over a slot-indexed state pool with a tree per sequence:
// one instantiation family of the kernel in verify_kernel.h.
#include "verify_kernel.h"

namespace treewy {

hipError_t launch_commit_verify_pool_trees(const VerifyArgs& a, const TreeArgs& bound,
                                           const TreeArgs& prev_bound, hipStream_t s) {
  if (a.state_bf16) return launch_commit_verify_s16_pool_trees(a, bound, prev_bound, s);
  return a.f32_inputs ? launch_dtype<true, true, true, false, true>(a, bound, prev_bound, s)
                      : launch_dtype<false, true, true, false, true>(a, bound, prev_bound, s);
}

}  // namespace treewy
