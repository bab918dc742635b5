// commit-then-verify over a slot-indexed pool of bf16-stored states with a
// tree per sequence (bf16 inputs): one instantiation family of the kernel in
// verify_kernel.h.
#include "verify_kernel.h"

namespace treewy {

hipError_t launch_commit_verify_s16_pool_trees(const VerifyArgs& a, const TreeArgs& bound,
                                               const TreeArgs& prev_bound, hipStream_t s) {
  return launch_dtype<false, true, true, true, true>(a, bound, prev_bound, s);
}

}  // namespace treewy
