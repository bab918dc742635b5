// commit-then-verify, fp32 state in a batch: one instantiation family of the
// kernel in verify_kernel.h.
#include "verify_kernel.h"

namespace treewy {

hipError_t launch_commit_verify_batch(const VerifyArgs& a, const TreeArgs& tree,
                                      const TreeArgs& prev, hipStream_t s) {
  return a.f32_inputs ? launch_dtype<true, true>(a, tree, prev, s)
                      : launch_dtype<false, true>(a, tree, prev, s);
}

}  // namespace treewy
