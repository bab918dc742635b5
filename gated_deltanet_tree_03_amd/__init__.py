"""TreeWY verify / commit / store_all through one Gated DeltaNet layer on
MI355X (gfx950): hand-written HIP kernels behind a C ABI (include/treewy.h),
bound here with ctypes."""
from .abi import (treewy_tree_meta, treewy_verify, treewy_commit, treewy_commit_verify,  # noqa: F401
                  treewy_commit_verify_pool, treewy_commit_verify_bf16state, treewy_prefill_chain,
                  prefill_chain, prefill_workspace, treewy_store_all,
                  treewy_store_all_select, status_str, TreewyError, verify, commit, commit_verify,
                  commit_verify_pool, commit_verify_bf16state, store_all,
                  store_all_select, TREEWY_BF16, TREEWY_F32, LIB_PATH)
