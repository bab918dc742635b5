// verify (no commit): one instantiation family of the kernel in verify_kernel.h,
// plus the commit-then-verify dispatcher over the fused families.
#include "verify_kernel.h"

namespace treewy {

hipError_t launch_verify(const VerifyArgs& a, const TreeArgs& tree, hipStream_t s) {
  return a.f32_inputs ? launch_dtype<true, false>(a, tree, tree, s)
                      : launch_dtype<false, false>(a, tree, tree, s);
}

hipError_t launch_commit_verify(const VerifyArgs& a, const TreeArgs& tree, const TreeArgs& prev,
                                hipStream_t s) {
  if (a.state_bf16) {
    return a.slots != nullptr ? launch_commit_verify_s16_pool(a, tree, prev, s)
                              : launch_commit_verify_s16(a, tree, prev, s);
  }
  if (a.slots != nullptr) return launch_commit_verify_pool(a, tree, prev, s);
  return launch_commit_verify_batch(a, tree, prev, s);
}

}  // namespace treewy
