"""C ABI checks that need no GPU: the library loads, exports every function
include/treewy.h declares, builds tree metadata, and rejects bad arguments on
the host before any HIP call (so nothing is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from gated_deltanet_tree_03_amd import abi, synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "treewy.h")
pytestmark = pytest.mark.skipif(not os.path.exists(abi.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(treewy_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(abi.EXPORTS)
    L = abi.lib()
    for n in names:
        assert hasattr(L, n), n
    assert abi.status_str(0) == "ok"
    for code in range(-6, 1):
        assert abi.status_str(code) != "unknown status"
    assert abi.status_str(7) == "unknown status"


def _py_meta(parent):
    n = len(parent)
    depth = np.zeros(n, dtype=np.int32)
    anc = np.zeros(n, dtype=np.uint64)
    for t in range(1, n):
        p = parent[t]
        depth[t] = depth[p] + 1
        j = p
        while j >= 0:
            anc[t] |= np.uint64(1) << np.uint64(j)
            j = parent[j]
    return depth, anc


@pytest.mark.parametrize("widths", [(1,), (1, 1, 1), (2, 2, 2), (3, 3, 3), (1, 5, 1)])
def test_tree_meta_full_trees(widths):
    p = synth.tree_from_widths(widths)
    d, a = abi.treewy_tree_meta(p)
    dw, aw = _py_meta(p)
    assert np.array_equal(d, dw) and np.array_equal(a, aw)


def test_tree_meta_random_and_max_chain(rng):
    for n in (1, 2, 17, 63, 64):
        p = synth.random_preorder_tree(n, rng)
        d, a = abi.treewy_tree_meta(p)
        dw, aw = _py_meta(p)
        assert np.array_equal(d, dw) and np.array_equal(a, aw)
    d, a = abi.treewy_tree_meta(synth.chain(64))
    assert d[-1] == 63 and a[-1] == np.uint64(2 ** 63 - 1)


@pytest.mark.parametrize("parent,code", [
    ([0, 0], abi.TREEWY_ERR_TREE),            # root must have parent -1
    ([-1, 1], abi.TREEWY_ERR_TREE),           # parent must precede the child
    ([-1, 0, 1, 0, 2], abi.TREEWY_ERR_TREE),  # node 4's parent 2 left the DFS path
    ([-1, -1], abi.TREEWY_ERR_TREE),          # second root
    ([], abi.TREEWY_ERR_ARG),
    (list(synth.chain(65)), abi.TREEWY_ERR_ARG),
])
def test_tree_meta_rejects(parent, code):
    with pytest.raises(abi.TreewyError) as e:
        abi.treewy_tree_meta(parent)
    assert e.value.status == code


A = 256  # any 16-byte aligned fake address; never dereferenced on rejection


def _verify(**over):
    args = dict(S0=A, q=A, k=A, v=A, alpha=A, beta=A, parent=[-1, 0, 1, 2], B=2, H=3, N=4,
                out=A, vtilde=A, gamma=A, dtype=0)
    args.update(over)
    return abi.treewy_verify(**args, stream=0, check=False)


def test_verify_rejects_before_any_gpu_call():
    assert _verify(S0=None) == abi.TREEWY_ERR_ARG
    assert _verify(out=None) == abi.TREEWY_ERR_ARG
    assert _verify(q=A + 8) == abi.TREEWY_ERR_ALIGN
    assert _verify(gamma=A + 4) == abi.TREEWY_ERR_ALIGN
    assert _verify(dtype=2) == abi.TREEWY_ERR_DTYPE
    assert _verify(B=-1) == abi.TREEWY_ERR_ARG
    assert _verify(N=0, parent=[]) == abi.TREEWY_ERR_ARG
    assert _verify(parent=[-1, 0, 0, 1], N=4) == abi.TREEWY_ERR_TREE
    assert _verify(parent=None) == abi.TREEWY_ERR_ARG
    assert _verify(B=1 << 16, H=1 << 9) == abi.TREEWY_ERR_SIZE


def test_empty_batch_is_a_noop():
    # nothing is enqueued, so even null buffers are accepted
    assert _verify(B=0, S0=None, q=None, out=None) == abi.TREEWY_OK
    assert _verify(H=0, S0=None) == abi.TREEWY_OK
    # but the topology and dtype are still validated
    assert _verify(B=0, parent=[0, 0, 1, 2]) == abi.TREEWY_ERR_TREE
    assert _verify(B=0, dtype=5) == abi.TREEWY_ERR_DTYPE


def test_commit_store_all_select_reject():
    p = [-1, 0, 1, 2]
    c = lambda **o: abi.treewy_commit(**{**dict(S0=A, vtilde=A, k=A, gamma=A, accepted=A, parent=p,
                                                 B=1, H=1, N=4, S_out=A, dtype=0), **o},
                                      stream=0, check=False)
    assert c(accepted=None) == abi.TREEWY_ERR_ARG
    assert c(S_out=A + 2) == abi.TREEWY_ERR_ALIGN
    assert c(parent=[-1, 5, 0, 0]) == abi.TREEWY_ERR_TREE
    assert c(dtype=-1) == abi.TREEWY_ERR_DTYPE
    assert c(B=0) == abi.TREEWY_OK
    s = lambda **o: abi.treewy_store_all(**{**dict(S0=A, q=A, k=A, v=A, alpha=A, beta=A, parent=p,
                                                    B=1, H=1, N=4, out=A, snapshots=A, dtype=1), **o},
                                         stream=0, check=False)
    assert s(snapshots=None) == abi.TREEWY_ERR_ARG
    assert s(v=A + 12) == abi.TREEWY_ERR_ALIGN
    assert s(H=-3) == abi.TREEWY_ERR_ARG
    assert s(H=0) == abi.TREEWY_OK
    sel = lambda **o: abi.treewy_store_all_select(**{**dict(snapshots=A, accepted=A, B=1, H=1, N=4,
                                                            S_out=A), **o}, stream=0, check=False)
    assert sel(N=0) == abi.TREEWY_ERR_ARG
    assert sel(N=65) == abi.TREEWY_ERR_ARG
    assert sel(accepted=None) == abi.TREEWY_ERR_ARG
    assert sel(S_out=A + 1) == abi.TREEWY_ERR_ALIGN
    assert sel(B=0) == abi.TREEWY_OK


def test_commit_verify_rejects_before_any_gpu_call():
    p4, p3 = [-1, 0, 1, 2], [-1, 0, 0]
    base = dict(S0=A, S_out=A, vtilde_prev=A + 4096, k_prev=A, gamma_prev=A + 8192, accepted_prev=A,
                parent_prev=p3, N_prev=3, q=A, k=A, v=A, alpha=A, beta=A, parent=p4, B=2, H=3, N=4,
                out=A, vtilde=A + 16384, gamma=A + 32768, dtype=0)
    cv = lambda **o: abi.treewy_commit_verify(**{**base, **o}, stream=0, check=False)
    assert cv(accepted_prev=None) == abi.TREEWY_ERR_ARG
    assert cv(S_out=None) == abi.TREEWY_ERR_ARG
    assert cv(k_prev=A + 2) == abi.TREEWY_ERR_ALIGN
    assert cv(parent_prev=[-1, 0, 2], N_prev=3) == abi.TREEWY_ERR_TREE
    assert cv(parent_prev=[], N_prev=0) == abi.TREEWY_ERR_ARG
    assert cv(parent=[-1, 1, 0, 0]) == abi.TREEWY_ERR_TREE
    assert cv(dtype=3) == abi.TREEWY_ERR_DTYPE
    # the previous step's pseudo-values / gates are read while the new ones are written
    assert cv(vtilde=A + 4096) == abi.TREEWY_ERR_ARG
    assert cv(gamma=A + 8192) == abi.TREEWY_ERR_ARG
    assert cv(B=0) == abi.TREEWY_OK
    assert cv(H=0, S0=None) == abi.TREEWY_OK


def test_commit_verify_pool_rejects_before_any_gpu_call():
    p4, p3 = [-1, 0, 1, 2], [-1, 0, 0]
    base = dict(pool=A, n_slots=5, slots=A + 64, vtilde_prev=A + 4096, k_prev=A,
                gamma_prev=A + 8192, accepted_prev=A, parent_prev=p3, N_prev=3, q=A, k=A, v=A,
                alpha=A, beta=A, parent=p4, B=2, H=3, N=4, out=A, vtilde=A + 16384,
                gamma=A + 32768, dtype=0)
    cv = lambda **o: abi.treewy_commit_verify_pool(**{**base, **o}, stream=0, check=False)
    assert cv(n_slots=-1) == abi.TREEWY_ERR_ARG
    assert cv(n_slots=0) == abi.TREEWY_ERR_ARG
    assert cv(n_slots=1 << 30) == abi.TREEWY_ERR_SIZE
    assert cv(pool=None) == abi.TREEWY_ERR_ARG
    assert cv(slots=None) == abi.TREEWY_ERR_ARG
    assert cv(slots=A + 4) == abi.TREEWY_ERR_ALIGN
    assert cv(parent_prev=[-1, 0, 2], N_prev=3) == abi.TREEWY_ERR_TREE
    assert cv(parent=[-1, 1, 0, 0]) == abi.TREEWY_ERR_TREE
    assert cv(dtype=3) == abi.TREEWY_ERR_DTYPE
    assert cv(vtilde=A + 4096) == abi.TREEWY_ERR_ARG
    assert cv(gamma=A + 8192) == abi.TREEWY_ERR_ARG
    assert cv(B=0) == abi.TREEWY_OK
    assert cv(H=0, pool=None) == abi.TREEWY_OK


def test_commit_verify_bf16state_rejects_before_any_gpu_call():
    p4, p3 = [-1, 0, 1, 2], [-1, 0, 0]
    base = dict(S0=A, S_out=A, vtilde_prev=A + 4096, k_prev=A, gamma_prev=A + 8192,
                accepted_prev=A, parent_prev=p3, N_prev=3, q=A, k=A, v=A, alpha=A, beta=A,
                parent=p4, B=2, H=3, N=4, out=A, vtilde=A + 16384, gamma=A + 32768,
                dtype=abi.TREEWY_BF16)
    cv = lambda **o: abi.treewy_commit_verify_bf16state(**{**base, **o}, stream=0, check=False)
    assert cv(dtype=abi.TREEWY_F32) == abi.TREEWY_ERR_DTYPE  # bf16 inputs only
    assert cv(S0=None) == abi.TREEWY_ERR_ARG
    assert cv(S_out=A + 8) == abi.TREEWY_ERR_ALIGN
    assert cv(parent=[-1, 1, 0, 0]) == abi.TREEWY_ERR_TREE
    assert cv(vtilde=A + 4096) == abi.TREEWY_ERR_ARG
    assert cv(B=0) == abi.TREEWY_OK


def test_commit_verify_bf16state_pool_rejects_before_any_gpu_call():
    p4, p3 = [-1, 0, 1, 2], [-1, 0, 0]
    base = dict(pool=A, n_slots=5, slots=A + 64, vtilde_prev=A + 4096, k_prev=A,
                gamma_prev=A + 8192, accepted_prev=A, parent_prev=p3, N_prev=3, q=A, k=A, v=A,
                alpha=A, beta=A, parent=p4, B=2, H=3, N=4, out=A, vtilde=A + 16384,
                gamma=A + 32768, dtype=abi.TREEWY_BF16)
    cv = lambda **o: abi.treewy_commit_verify_bf16state_pool(**{**base, **o}, stream=0, check=False)
    assert cv(dtype=abi.TREEWY_F32) == abi.TREEWY_ERR_DTYPE  # bf16 inputs only
    assert cv(n_slots=-1) == abi.TREEWY_ERR_ARG
    assert cv(n_slots=0) == abi.TREEWY_ERR_ARG
    assert cv(n_slots=1 << 30) == abi.TREEWY_ERR_SIZE
    assert cv(pool=None) == abi.TREEWY_ERR_ARG
    assert cv(slots=A + 4) == abi.TREEWY_ERR_ALIGN
    assert cv(parent_prev=[-1, 0, 2], N_prev=3) == abi.TREEWY_ERR_TREE
    assert cv(vtilde=A + 4096) == abi.TREEWY_ERR_ARG
    assert cv(B=0) == abi.TREEWY_OK
    assert cv(H=0, pool=None) == abi.TREEWY_OK


def test_commit_verify_bf16state_pool_trees_rejects_before_any_gpu_call():
    base = dict(pool=A, n_slots=4, slots=A, vtilde_prev=A, k_prev=A, gamma_prev=A, accepted_prev=A,
                trees_prev=A, N_prev=4, depth_prev=3, q=A, k=A, v=A, alpha=A, beta=A, trees=A,
                N=15, depth=3, B=2, H=3, out=A, vtilde=A + 4096, gamma=A + 8192,
                dtype=abi.TREEWY_BF16)
    cv = lambda **o: abi.treewy_commit_verify_bf16state_pool_trees(**{**base, **o}, stream=0,
                                                                   check=False)
    assert cv(dtype=abi.TREEWY_F32) == abi.TREEWY_ERR_DTYPE
    assert cv(N=65) == abi.TREEWY_ERR_ARG
    assert cv(depth=15) == abi.TREEWY_ERR_ARG
    assert cv(n_slots=0) == abi.TREEWY_ERR_ARG
    assert cv(trees=None) == abi.TREEWY_ERR_ARG
    assert cv(trees_prev=A + 8) == abi.TREEWY_ERR_ALIGN
    assert cv(vtilde=A) == abi.TREEWY_ERR_ARG
    assert cv(B=0) == abi.TREEWY_OK


def test_prefill_chain_rejects_before_any_gpu_call():
    base = dict(S=A, q=A, k=A, v=A, alpha=A, beta=A, B=2, T=100, H=3, chunk=64, out=A,
                work_vtilde=A, work_gamma=A, dtype=abi.TREEWY_BF16)
    pf = lambda **o: abi.treewy_prefill_chain(**{**base, **o}, stream=0, check=False)
    assert pf(chunk=0) == abi.TREEWY_ERR_ARG
    assert pf(chunk=65) == abi.TREEWY_ERR_ARG
    assert pf(T=-1) == abi.TREEWY_ERR_ARG
    assert pf(B=-1) == abi.TREEWY_ERR_ARG
    assert pf(dtype=7) == abi.TREEWY_ERR_DTYPE
    assert pf(work_gamma=None) == abi.TREEWY_ERR_ARG
    assert pf(out=A + 4) == abi.TREEWY_ERR_ALIGN
    assert pf(T=0) == abi.TREEWY_OK
    assert pf(B=0) == abi.TREEWY_OK


def test_prefill_rejects_before_any_gpu_call():
    base = dict(S=A, q=A, k=A, v=A, alpha=A, beta=A, B=2, T=100, H=3, out=A,
                dtype=abi.TREEWY_BF16)
    pf = lambda **o: abi.treewy_prefill(**{**base, **o}, stream=0, check=False)
    assert pf(T=-1) == abi.TREEWY_ERR_ARG
    assert pf(B=-1) == abi.TREEWY_ERR_ARG
    assert pf(H=-2) == abi.TREEWY_ERR_ARG
    assert pf(dtype=7) == abi.TREEWY_ERR_DTYPE
    assert pf(S=None) == abi.TREEWY_ERR_ARG
    assert pf(beta=None) == abi.TREEWY_ERR_ARG
    assert pf(out=A + 4) == abi.TREEWY_ERR_ALIGN
    assert pf(q=A + 8) == abi.TREEWY_ERR_ALIGN
    assert pf(B=1 << 13, H=1 << 12) == abi.TREEWY_ERR_SIZE
    assert pf(B=1, H=(1 << 19) + 1) == abi.TREEWY_ERR_SIZE  # 32-bit row offsets in a chunk
    assert pf(T=0) == abi.TREEWY_OK
    assert pf(B=0) == abi.TREEWY_OK


def test_tree_desc_pack_validates_each_request():
    size = abi.treewy_tree_desc_size()
    assert size > 0 and size % 8 == 0
    rng = np.random.default_rng(4)
    trees = [synth.chain(4), synth.tree_from_widths((2, 2, 2)), synth.random_preorder_tree(40, rng)]
    host, n_max, depth = abi.pack_trees(trees)
    assert n_max == 40 and host.size == 3 * size
    assert depth == max(int(synth.node_depths(p).max()) for p in trees)
    # request 1 is not in pre-order (node 3's parent is off the path 0 -> 2)
    par = np.full((3, 4), -1, np.int32)
    for i, p in enumerate([synth.chain(4), [-1, 0, 0, 1], synth.chain(2)]):
        par[i, :len(p)] = p
    buf = np.zeros(3 * size // 8 + 1, np.uint64)
    pk = lambda counts, n_max=4, count=3, addr=buf.ctypes.data: abi.treewy_tree_desc_pack(
        par, counts, count, n_max, addr, check=False)[0]
    assert pk([4, 4, 2]) == abi.TREEWY_ERR_TREE
    assert pk([4, 3, 2]) == abi.TREEWY_OK  # the first 3 nodes of request 1 are a valid tree
    assert pk([5, 3, 2]) == abi.TREEWY_ERR_ARG  # a count above n_max
    assert pk([4, 0, 2]) == abi.TREEWY_ERR_ARG
    assert pk([4, 3, 2], n_max=65) == abi.TREEWY_ERR_ARG
    assert pk([4, 3, 2], addr=buf.ctypes.data + 4) == abi.TREEWY_ERR_ALIGN
    assert pk([], count=0) == abi.TREEWY_OK


def test_commit_verify_pool_trees_rejects_before_any_gpu_call():
    base = dict(pool=A, n_slots=4, slots=A, vtilde_prev=A, k_prev=A, gamma_prev=A, accepted_prev=A,
                trees_prev=A, N_prev=4, depth_prev=3, q=A, k=A, v=A, alpha=A, beta=A, trees=A,
                N=15, depth=3, B=2, H=3, out=A, vtilde=A + 4096, gamma=A + 8192,
                dtype=abi.TREEWY_BF16)
    cv = lambda **o: abi.treewy_commit_verify_pool_trees(**{**base, **o}, stream=0, check=False)
    assert cv(N=0) == abi.TREEWY_ERR_ARG
    assert cv(N=65) == abi.TREEWY_ERR_ARG
    assert cv(N_prev=0) == abi.TREEWY_ERR_ARG
    assert cv(depth=15) == abi.TREEWY_ERR_ARG  # a depth bound must be below the node bound
    assert cv(depth=-1) == abi.TREEWY_ERR_ARG
    assert cv(depth_prev=4) == abi.TREEWY_ERR_ARG
    assert cv(n_slots=0) == abi.TREEWY_ERR_ARG
    assert cv(dtype=7) == abi.TREEWY_ERR_DTYPE
    assert cv(trees=None) == abi.TREEWY_ERR_ARG
    assert cv(trees_prev=A + 8) == abi.TREEWY_ERR_ALIGN
    assert cv(vtilde=A) == abi.TREEWY_ERR_ARG  # the same buffer as vtilde_prev
    assert cv(B=-1) == abi.TREEWY_ERR_ARG
    assert cv(B=0) == abi.TREEWY_OK


# ---------------------------------------------------------------------------
# aliasing: outputs may not overlap one another or any input
# ---------------------------------------------------------------------------

MB = 1 << 20


def _addr(i):
    """Fake, 16-byte aligned, pairwise disjoint buffers (1 MiB apart)."""
    return (i + 1) * MB


# Tests that hand the library a valid, non-overlapping set of fake pointers
# would reach a kernel launch.  They run only in the host-check build, whose
# launchers are stand-ins that never touch a GPU (tests/host_check).
# (decided when a test runs, not at import: importing this module must not
# load the library, since collection on a GPU machine imports it too)
@pytest.fixture
def hostcheck():
    if not hasattr(abi.lib(), "treewy_hostcheck_launches"):
        pytest.skip("needs the host-check build (stand-in launchers)")


needs_hostcheck = pytest.mark.usefixtures("hostcheck")


def _launches():
    return abi.lib().treewy_hostcheck_launches()


def _verify_disjoint(**over):
    args = dict(S0=_addr(0), q=_addr(1), k=_addr(2), v=_addr(3), alpha=_addr(4), beta=_addr(5),
                parent=[-1, 0, 1, 2], B=2, H=3, N=4, out=_addr(6), vtilde=_addr(7), gamma=_addr(8),
                dtype=0)
    args.update(over)
    return abi.treewy_verify(**args, stream=0, check=False)


def test_verify_rejects_partial_overlaps():
    # out is 2*3*4*128*4 = 12288 bytes: a buffer starting inside it overlaps
    assert _verify_disjoint(vtilde=_addr(6) + 12288 - 16) == abi.TREEWY_ERR_ARG
    assert _verify_disjoint(gamma=_addr(7) + 4096) == abi.TREEWY_ERR_ARG
    assert _verify_disjoint(out=_addr(0) + 65536) == abi.TREEWY_ERR_ARG    # inside S0
    assert _verify_disjoint(gamma=_addr(1) + 16) == abi.TREEWY_ERR_ARG     # inside q
    assert _verify_disjoint(out=_addr(4) - 12288 + 16) == abi.TREEWY_ERR_ARG  # runs into alpha


@needs_hostcheck
def test_verify_accepts_adjacent_and_shared_inputs():
    n0 = _launches()
    # out ends exactly where vtilde starts: adjacent, not overlapping
    assert _verify_disjoint(vtilde=_addr(6) + 12288) == abi.TREEWY_OK
    # inputs may overlap one another (q and k the same buffer)
    assert _verify_disjoint(k=_addr(1)) == abi.TREEWY_OK
    assert _launches() == n0 + 2


def _commit_disjoint(**over):
    args = dict(S0=_addr(0), vtilde=_addr(1), k=_addr(2), gamma=_addr(3), accepted=_addr(4),
                parent=[-1, 0, 1, 2], B=2, H=3, N=4, S_out=_addr(5), dtype=0)
    args.update(over)
    return abi.treewy_commit(**args, stream=0, check=False)


def test_commit_rejects_partial_state_overlap():
    assert _commit_disjoint(S_out=_addr(0) + 64) == abi.TREEWY_ERR_ARG   # S0 shifted by 64 B
    assert _commit_disjoint(S_out=_addr(1) - 16) == abi.TREEWY_ERR_ARG   # runs into vtilde
    assert _commit_disjoint(accepted=_addr(5) + 5 * 65536) == abi.TREEWY_ERR_ARG  # in S_out


@needs_hostcheck
def test_commit_in_place_is_accepted():
    n0 = _launches()
    assert _commit_disjoint(S_out=_addr(0)) == abi.TREEWY_OK
    assert _commit_disjoint() == abi.TREEWY_OK
    assert _launches() == n0 + 2


def _cv_disjoint(fn=abi.treewy_commit_verify, **over):
    args = dict(S0=_addr(0), S_out=_addr(0), vtilde_prev=_addr(1), k_prev=_addr(2),
                gamma_prev=_addr(3), accepted_prev=_addr(4), parent_prev=[-1, 0, 0], N_prev=3,
                q=_addr(5), k=_addr(6), v=_addr(7), alpha=_addr(8), beta=_addr(9),
                parent=[-1, 0, 1, 2], B=2, H=3, N=4, out=_addr(10), vtilde=_addr(11),
                gamma=_addr(12), dtype=abi.TREEWY_BF16)
    args.update(over)
    return fn(**args, stream=0, check=False)


@pytest.mark.parametrize("fn", [abi.treewy_commit_verify, abi.treewy_commit_verify_bf16state])
def test_commit_verify_rejects_partial_overlaps(fn):
    # vtilde_prev is 2*3*3*128*4 = 9216 bytes; the new vtilde may not start inside it
    assert _cv_disjoint(fn, vtilde=_addr(1) + 4096) == abi.TREEWY_ERR_ARG
    assert _cv_disjoint(fn, gamma=_addr(3) + 16) == abi.TREEWY_ERR_ARG
    assert _cv_disjoint(fn, S_out=_addr(0) + 16) == abi.TREEWY_ERR_ARG  # partial in-place
    assert _cv_disjoint(fn, out=_addr(5) + 16) == abi.TREEWY_ERR_ARG    # inside q
    assert _cv_disjoint(fn, vtilde=_addr(10) + 16) == abi.TREEWY_ERR_ARG  # inside out


@needs_hostcheck
@pytest.mark.parametrize("fn", [abi.treewy_commit_verify, abi.treewy_commit_verify_bf16state])
def test_commit_verify_accepts_in_place_and_disjoint(fn):
    n0 = _launches()
    assert _cv_disjoint(fn) == abi.TREEWY_OK                          # in place
    assert _cv_disjoint(fn, S_out=_addr(13)) == abi.TREEWY_OK         # out of place
    assert _cv_disjoint(fn, k_prev=_addr(6)) == abi.TREEWY_OK         # inputs may coincide
    assert _launches() == n0 + 3


def _pool_disjoint(fn=None, **over):
    args = dict(pool=_addr(0), n_slots=4, slots=_addr(5), vtilde_prev=_addr(6), k_prev=_addr(7),
                gamma_prev=_addr(8), accepted_prev=_addr(9), parent_prev=[-1, 0, 0], N_prev=3,
                q=_addr(10), k=_addr(11), v=_addr(12), alpha=_addr(13), beta=_addr(14),
                parent=[-1, 0, 1, 2], B=2, H=3, N=4, out=_addr(15), vtilde=_addr(16),
                gamma=_addr(17), dtype=abi.TREEWY_BF16)
    args.update(over)
    return (fn or abi.treewy_commit_verify_pool)(**args, stream=0, check=False)


def test_commit_verify_pool_rejects_overlaps():
    # the pool (4 slots x 3 heads x 64 KiB) is written in place: nothing else may sit inside it
    assert _pool_disjoint(out=_addr(0) + 4 * 3 * 65536 - 16) == abi.TREEWY_ERR_ARG
    assert _pool_disjoint(slots=_addr(0) + 256) == abi.TREEWY_ERR_ARG
    assert _pool_disjoint(vtilde=_addr(6) + 64) == abi.TREEWY_ERR_ARG


@needs_hostcheck
def test_commit_verify_pool_accepts_disjoint():
    n0 = _launches()
    assert _pool_disjoint() == abi.TREEWY_OK
    assert _pool_disjoint(out=_addr(0) + 4 * 3 * 65536) == abi.TREEWY_OK  # right after the pool
    assert _launches() == n0 + 2


def test_bf16state_pool_rejects_overlaps_of_its_half_size_blocks():
    # a bf16 pool of 4 slots x 3 heads holds 4 * 3 * 32 KiB
    f = lambda **o: _pool_disjoint(fn=abi.treewy_commit_verify_bf16state_pool, **o)
    assert f(out=_addr(0) + 4 * 3 * 32768 - 16) == abi.TREEWY_ERR_ARG
    assert f(slots=_addr(0) + 256) == abi.TREEWY_ERR_ARG


@needs_hostcheck
def test_bf16state_pool_accepts_buffers_after_its_half_size_blocks():
    n0 = _launches()
    f = lambda **o: _pool_disjoint(fn=abi.treewy_commit_verify_bf16state_pool, **o)
    assert f() == abi.TREEWY_OK
    assert f(out=_addr(0) + 4 * 3 * 32768) == abi.TREEWY_OK
    assert _launches() == n0 + 2


def _pt_disjoint(fn=None, **over):
    args = dict(pool=_addr(0), n_slots=4, slots=_addr(5), vtilde_prev=_addr(6), k_prev=_addr(7),
                gamma_prev=_addr(8), accepted_prev=_addr(9), trees_prev=_addr(10), N_prev=4,
                depth_prev=3, q=_addr(11), k=_addr(12), v=_addr(13), alpha=_addr(14),
                beta=_addr(15), trees=_addr(16), N=15, depth=3, B=2, H=3, out=_addr(17),
                vtilde=_addr(18), gamma=_addr(19), dtype=abi.TREEWY_BF16)
    args.update(over)
    return (fn or abi.treewy_commit_verify_pool_trees)(**args, stream=0, check=False)


def test_commit_verify_pool_trees_rejects_overlaps():
    assert _pt_disjoint(out=_addr(16) + 1024) == abi.TREEWY_ERR_ARG  # inside the descriptors
    assert _pt_disjoint(gamma=_addr(8) + 16) == abi.TREEWY_ERR_ARG


@needs_hostcheck
def test_commit_verify_pool_trees_accepts_disjoint():
    n0 = _launches()
    assert _pt_disjoint() == abi.TREEWY_OK
    assert _launches() == n0 + 1


def test_bf16state_pool_trees_rejects_overlaps():
    f = lambda **o: _pt_disjoint(fn=abi.treewy_commit_verify_bf16state_pool_trees, **o)
    assert f(out=_addr(0) + 4 * 3 * 32768 - 16) == abi.TREEWY_ERR_ARG
    assert f(gamma=_addr(8) + 16) == abi.TREEWY_ERR_ARG


@needs_hostcheck
def test_bf16state_pool_trees_accepts_disjoint():
    n0 = _launches()
    f = lambda **o: _pt_disjoint(fn=abi.treewy_commit_verify_bf16state_pool_trees, **o)
    assert f() == abi.TREEWY_OK
    assert f(out=_addr(0) + 4 * 3 * 32768) == abi.TREEWY_OK
    assert _launches() == n0 + 2


def test_store_all_select_and_prefills_reject_overlaps():
    sa = dict(S0=_addr(0), q=_addr(1), k=_addr(2), v=_addr(3), alpha=_addr(4), beta=_addr(5),
              parent=[-1, 0, 1, 2], B=1, H=1, N=4, out=_addr(6), snapshots=_addr(7), dtype=0)
    s = lambda **o: abi.treewy_store_all(**{**sa, **o}, stream=0, check=False)
    assert s(out=_addr(7) + 5 * 65536 - 16) == abi.TREEWY_ERR_ARG  # the last snapshot
    assert s(snapshots=_addr(0) + 65536 - 16) == abi.TREEWY_ERR_ARG
    sel = lambda **o: abi.treewy_store_all_select(**{**dict(snapshots=_addr(0), accepted=_addr(1),
                                                            B=1, H=1, N=4, S_out=_addr(2)), **o},
                                                  stream=0, check=False)
    assert sel(S_out=_addr(0) + 3 * 65536) == abi.TREEWY_ERR_ARG
    pf = dict(S=_addr(0), q=_addr(1), k=_addr(2), v=_addr(3), alpha=_addr(4), beta=_addr(5), B=1,
              T=8, H=1, out=_addr(6), dtype=abi.TREEWY_BF16)
    p = lambda **o: abi.treewy_prefill(**{**pf, **o}, stream=0, check=False)
    assert p(out=_addr(0) + 1024) == abi.TREEWY_ERR_ARG
    assert p(S=_addr(1)) == abi.TREEWY_ERR_ARG  # the state is written: it may not sit on q
    pc = lambda **o: abi.treewy_prefill_chain(**{**pf, "chunk": 4, "work_vtilde": _addr(7),
                                                 "work_gamma": _addr(8), **o},
                                              stream=0, check=False)
    assert pc(work_gamma=_addr(7) + 2048) == abi.TREEWY_ERR_ARG
    assert pc(work_vtilde=_addr(6)) == abi.TREEWY_ERR_ARG


@needs_hostcheck
def test_store_all_select_and_prefills_accept_disjoint():
    n0 = _launches()
    assert abi.treewy_store_all(_addr(0), _addr(1), _addr(2), _addr(3), _addr(4), _addr(5),
                                [-1, 0, 1, 0], 1, 1, 4, _addr(6), _addr(7), 0, 0, check=False) == 0
    assert abi.treewy_store_all_select(_addr(0), _addr(1), 1, 1, 4, _addr(2), 0, check=False) == 0
    assert abi.treewy_prefill(_addr(0), _addr(1), _addr(2), _addr(3), _addr(4), _addr(5), 1, 37, 1,
                              _addr(6), abi.TREEWY_BF16, 0, check=False) == 0
    # a chain of 37 tokens in chunks of 16: 3 chunk launches and the final commit
    assert abi.treewy_prefill_chain(_addr(0), _addr(1), _addr(2), _addr(3), _addr(4), _addr(5), 1,
                                    37, 1, 16, _addr(6), _addr(7), _addr(8), abi.TREEWY_BF16, 0,
                                    check=False) == 0
    assert _launches() == n0 + 3 + 4


def test_prefill_chain_noalloc_rejects_before_any_gpu_call():
    base = dict(S=_addr(0), q=_addr(1), k=_addr(2), v=_addr(3), alpha=_addr(4), beta=_addr(5),
                B=2, T=100, H=3, chunk=16, out=_addr(6), dtype=abi.TREEWY_BF16)
    pf = lambda **o: abi.treewy_prefill_chain_noalloc(**{**base, **o}, stream=0, check=False)
    assert pf(chunk=0) == abi.TREEWY_ERR_ARG
    assert pf(chunk=65) == abi.TREEWY_ERR_ARG
    assert pf(T=-1) == abi.TREEWY_ERR_ARG
    assert pf(dtype=7) == abi.TREEWY_ERR_DTYPE
    assert pf(S=None) == abi.TREEWY_ERR_ARG
    assert pf(out=_addr(6) + 4) == abi.TREEWY_ERR_ALIGN
    assert pf(out=_addr(1) + 16) == abi.TREEWY_ERR_ARG  # overlaps q
    # the scratch holds 2 x (B*H*chunk*128 + ceil4(B*H*chunk)) floats at most:
    # 64 MiB fits B*H*chunk = 32768 (16 MiB x 2 + 256 KiB), not 65536
    assert pf(B=512, H=64, chunk=2) == abi.TREEWY_ERR_SIZE
    assert pf(B=256, H=32, chunk=64) == abi.TREEWY_ERR_SIZE
    assert pf(T=0) == abi.TREEWY_OK
    assert pf(B=0) == abi.TREEWY_OK


@needs_hostcheck
def test_prefill_chain_noalloc_accepts_the_largest_fitting_call():
    n0 = _launches()
    # B*H*chunk = 32768: 2 * (32768*128 + 32768) * 4 bytes = 33.8 MB <= 64 MiB
    assert abi.treewy_prefill_chain_noalloc(_addr(0), 1 << 34, 2 << 34, 3 << 34, 4 << 34, 5 << 34,
                                            64, 40, 32, 16, 6 << 34, abi.TREEWY_BF16, 0,
                                            check=False) == abi.TREEWY_OK
    assert _launches() == n0 + 3 + 1  # chunks of 16, 16, 8 and the final commit
