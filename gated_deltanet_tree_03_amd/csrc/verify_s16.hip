// commit-then-verify over a bf16-stored state (bf16 inputs): one instantiation
// family of the kernel in verify_kernel.h.
#include "verify_kernel.h"

namespace treewy {

hipError_t launch_commit_verify_s16(const VerifyArgs& a, const TreeArgs& tree,
                                    const TreeArgs& prev, hipStream_t s) {
  return launch_dtype<false, true, false, true>(a, tree, prev, s);
}

}  // namespace treewy
