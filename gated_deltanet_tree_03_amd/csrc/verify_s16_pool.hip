// commit-then-verify over a slot-indexed pool of bf16-stored states (bf16
// inputs): one instantiation family of the kernel in verify_kernel.h.
#include "verify_kernel.h"

namespace treewy {

hipError_t launch_commit_verify_s16_pool(const VerifyArgs& a, const TreeArgs& tree,
                                         const TreeArgs& prev, hipStream_t s) {
  return launch_dtype<false, true, true, true>(a, tree, prev, s);
}

}  // namespace treewy
