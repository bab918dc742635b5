"""CPU oracle (test infrastructure only; see treewy_oracle's header)."""
from .treewy_oracle import (ancestors, path_of, walk, closed_form, commit, chain_wy,  # noqa: F401
                            store_all, gamma_scan, WalkResult, ClosedFormResult)
