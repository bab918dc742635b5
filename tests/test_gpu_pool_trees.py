"""GPU parity of treewy_commit_verify_pool_trees (commit-then-verify over a
slot-indexed state pool with a draft tree per request), through the C ABI.

Each case runs two steps through the entry point itself:
1. every request has no previous step (accepted_prev = -1): its state is
   verified as it is, with its own tree;
2. each request commits its own accepted node of step 1's tree and verifies a
   new tree of its own.
Both steps are checked against the fp64 oracle walking each request with its
own tree (2e-3): outputs, pseudo-values, gates and the committed pool state.
Rows past a request's node count are checked untouched (NaN-poisoned before).
With one tree shared by every request, the results equal
treewy_commit_verify_pool bit for bit.  At full size (the bench's launch of
this entry point, 128 sequences x 32 heads), sampled pairs of a batch mixing
tree shapes are checked the same way.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
from gpu_cases import TOL, rel_err, to_device  # noqa: E402

import oracle  # noqa: E402
from gated_deltanet_tree_03_amd import abi, synth  # noqa: E402

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(abi.LIB_PATH):
        pytest.fail("libtreewy.so is not built")
    torch.cuda.set_device(0)
    yield


def _err(label, got, ref):
    e = rel_err(got, ref)
    print(f"{label}: {e:.2e}", flush=True)
    assert np.isfinite(e) and e <= TOL, f"{label}: rel err {e:.3e} > {TOL}"


def _trees(sizes, rng, max_depth=None):
    return [synth.random_preorder_tree(int(n), rng, max_depth=max_depth) for n in sizes]


def _descs(parents):
    host, n_max, depth = abi.pack_trees(parents)
    return torch.from_numpy(host.copy()).cuda(), n_max, depth


def _nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _case(label, B, H, sizes1, sizes2, seed, cfg="35b-tree222", dtype=None, max_depth=None):
    rng = np.random.default_rng(seed)
    p1, p2 = _trees(sizes1, rng, max_depth), _trees(sizes2, rng, max_depth)
    t1, N1, md1 = _descs(p1)
    t2, N2, md2 = _descs(p2)
    print(f"case {label}: sizes {list(sizes1)} -> {list(sizes2)}, depth bounds {md1}/{md2}",
          flush=True)
    in1 = synth.make_inputs(cfg, B=B, H=H, seed=seed, parent=synth.chain(N1), dtype=dtype)
    in2 = synth.make_inputs(cfg, B=B, H=H, seed=seed + 1, parent=synth.chain(N2), dtype=dtype)
    d1, d2 = to_device(in1), to_device(in2)
    # the states on distinct random slots of a pool with 3 spare blocks
    n_pool = B + 3
    slot_list = rng.permutation(n_pool)[:B]
    slots = torch.tensor(slot_list, dtype=torch.int32, device="cuda")
    pool = torch.zeros((n_pool, H, 128, 128), dtype=torch.float32, device="cuda")
    pool[slots.long()] = d1["S0"]

    # step 1: no previous step (a one-node previous tree, never read)
    t0, _, _ = _descs([np.array([-1], dtype=np.int32)] * B)
    none = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    vt0 = torch.zeros((B, H, 1, 128), dtype=torch.float32, device="cuda")
    k0 = d1["k"][:, :1].contiguous()
    gm0 = torch.ones((B, H, 1), dtype=torch.float32, device="cuda")
    out1, vt1, gm1 = _nan((B, N1, H, 128)), _nan((B, H, N1, 128)), _nan((B, H, N1))
    abi.commit_verify_pool_trees(pool, slots, vt0, k0, gm0, none, t0, 0, d1["q"], d1["k"], d1["v"],
                                 d1["alpha"], d1["beta"], t1, md1, out=out1, vtilde=vt1, gamma=gm1)
    torch.cuda.synchronize()
    assert torch.equal(pool[slots.long()], d1["S0"]), "step 1 rewrote a state"

    # step 2: commit each request's accepted node of its step-1 tree
    acc = np.array([rng.integers(0, n) for n in sizes1], dtype=np.int32)
    acc_t = torch.from_numpy(acc).cuda()
    out2, vt2, gm2 = _nan((B, N2, H, 128)), _nan((B, H, N2, 128)), _nan((B, H, N2))
    abi.commit_verify_pool_trees(pool, slots, vt1, d1["k"], gm1, acc_t, t1, md1, d2["q"], d2["k"],
                                 d2["v"], d2["alpha"], d2["beta"], t2, md2, out=out2, vtilde=vt2,
                                 gamma=gm2)
    torch.cuda.synchronize()

    got = {k: x.cpu().numpy() for k, x in (("out1", out1), ("vt1", vt1), ("gm1", gm1),
                                           ("out2", out2), ("vt2", vt2), ("gm2", gm2))}
    pool_h = pool.cpu().numpy()
    f64 = lambda x: np.asarray(x, dtype=np.float64)
    ref = {k: [] for k in ("out1", "vt1", "out2", "vt2", "S")}
    mine = {k: [] for k in ref}
    for b in range(B):
        n1, n2 = len(p1[b]), len(p2[b])
        for h in range(H):
            w1 = oracle.walk(f64(in1.S0[b, h])[None], f64(in1.q[b, :n1, h])[None],
                             f64(in1.k[b, :n1, h])[None], f64(in1.v[b, :n1, h])[None],
                             f64(in1.alpha[b, :n1, h])[None], f64(in1.beta[b, :n1, h])[None], p1[b])
            Sa = w1.states[:, acc[b]]
            w2 = oracle.walk(Sa, f64(in2.q[b, :n2, h])[None], f64(in2.k[b, :n2, h])[None],
                             f64(in2.v[b, :n2, h])[None], f64(in2.alpha[b, :n2, h])[None],
                             f64(in2.beta[b, :n2, h])[None], p2[b])
            ref["out1"].append(w1.out[0]); mine["out1"].append(got["out1"][b, :n1, h])
            ref["vt1"].append(w1.vtilde[0]); mine["vt1"].append(got["vt1"][b, h, :n1])
            ref["out2"].append(w2.out[0]); mine["out2"].append(got["out2"][b, :n2, h])
            ref["vt2"].append(w2.vtilde[0]); mine["vt2"].append(got["vt2"][b, h, :n2])
            ref["S"].append(Sa[0]); mine["S"].append(pool_h[slot_list[b], h])
            # gates: the product of alpha along the root path
            for gname, gm, inp, par, n in (("gm1", got["gm1"], in1, p1[b], n1),
                                           ("gm2", got["gm2"], in2, p2[b], n2)):
                g_ref = oracle.gamma_scan(f64(inp.alpha[b, :n, h])[None], par)[0]
                _err(f"{label} {gname} ({b},{h})", gm[b, h, :n], g_ref)
        # rows past the request's own count are not written
        assert np.isnan(got["out1"][b, n1:]).all() and np.isnan(got["vt1"][b, :, n1:]).all()
        assert np.isnan(got["out2"][b, n2:]).all() and np.isnan(got["vt2"][b, :, n2:]).all()
        assert np.isnan(got["gm2"][b, :, n2:]).all()
    for k in ref:
        _err(f"{label} {k}", np.concatenate([m.reshape(-1) for m in mine[k]]),
             np.concatenate([r.reshape(-1) for r in ref[k]]))
    spare = [i for i in range(n_pool) if i not in set(slot_list.tolist())]
    assert not pool[spare].any(), "a pool block no request names was written"


def test_mixed_serving_batch():
    """Chains, (2,2,2)-sized and (3,3,3)-sized trees of depth <= 3 in one batch."""
    _case("mixed depth<=3", B=6, H=3, sizes1=[4, 15, 1, 40, 9, 23], sizes2=[15, 4, 40, 2, 31, 1],
          seed=610, cfg="wide-tree333", max_depth=3)


def test_deep_trees_per_request():
    """Depth classes above 3 (the column-walk tables), one request a 40-node chain."""
    _case("deep", B=5, H=2, sizes1=[40, 12, 30, 5, 20], sizes2=[20, 40, 3, 33, 17], seed=620,
          cfg="wide-tree333")


def test_fp32_inputs_per_request():
    _case("fp32", B=4, H=2, sizes1=[6, 15, 1, 11], sizes2=[9, 2, 15, 7], seed=630, dtype="f32",
          max_depth=4)


def test_single_tree_equals_pool_form_bitwise():
    """Every request on the (2,2,2) tree: the same results as the pool form."""
    B, H = 8, 4
    parent = synth.tree_from_widths((2, 2, 2))
    N = len(parent)
    prev = synth.make_inputs("35b-tree222", B=B, H=H, seed=640, parent=parent)
    new = synth.make_inputs("35b-tree222", B=B, H=H, seed=641, parent=parent)
    pd, nd = to_device(prev), to_device(new)
    _, vt0, gm0 = abi.verify(pd["S0"], pd["q"], pd["k"], pd["v"], pd["alpha"], pd["beta"], parent)
    acc = torch.from_numpy(prev.accepted.astype(np.int32)).cuda()
    slots = torch.tensor(np.random.default_rng(5).permutation(B + 2)[:B], dtype=torch.int32,
                         device="cuda")
    pool_a = torch.zeros((B + 2, H, 128, 128), dtype=torch.float32, device="cuda")
    pool_a[slots.long()] = pd["S0"]
    pool_b = pool_a.clone()
    ra = abi.commit_verify_pool(pool_a, slots, vt0, pd["k"], gm0, acc, parent, nd["q"], nd["k"],
                                nd["v"], nd["alpha"], nd["beta"], parent)
    tr, n_max, depth = _descs([parent] * B)
    assert n_max == N
    rb = abi.commit_verify_pool_trees(pool_b, slots, vt0, pd["k"], gm0, acc, tr, depth, nd["q"],
                                      nd["k"], nd["v"], nd["alpha"], nd["beta"], tr, depth)
    torch.cuda.synchronize()
    assert torch.equal(pool_a, pool_b)
    for x, y, name in zip(ra, rb, ("out", "vtilde", "gamma")):
        assert torch.equal(x, y), f"{name} differs from the pool form"


def test_full_size_mixed_trees_sampled():
    """The bench's pool-with-trees launch at full size (35B-like layer: 128
    sequences x 32 heads, node bound 15), each request on its own tree (a
    chain of 4, the (2,2,2) tree or a random tree of depth <= 3), two steps;
    sampled (request, head) pairs against the oracle."""
    B, H, N = 128, 32, 15
    rng = np.random.default_rng(660)
    kinds = [synth.chain(4), synth.tree_from_widths((2, 2, 2))]
    pick = lambda b: (kinds[b % 2] if b % 3 else
                      synth.random_preorder_tree(int(rng.integers(1, N + 1)), rng, max_depth=3))
    p1 = [pick(b) for b in range(B)]
    p2 = [pick(b + 1) for b in range(B)]
    t1, N1, md1 = _descs(p1)
    t2, N2, md2 = _descs(p2)
    print(f"case full size: node bounds {N1}/{N2}, depth bounds {md1}/{md2}", flush=True)
    in1 = synth.make_inputs("35b-tree222", B=B, H=H, seed=661, parent=synth.chain(N1))
    in2 = synth.make_inputs("35b-tree222", B=B, H=H, seed=662, parent=synth.chain(N2))
    d1, d2 = to_device(in1), to_device(in2)
    slots = torch.from_numpy(rng.permutation(B + 16)[:B].astype(np.int32)).cuda()
    pool = torch.zeros((B + 16, H, 128, 128), dtype=torch.float32, device="cuda")
    pool[slots.long()] = d1["S0"]
    t0, _, _ = _descs([np.array([-1], dtype=np.int32)] * B)
    none = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    _, vt1, gm1 = abi.commit_verify_pool_trees(
        pool, slots, torch.zeros((B, H, 1, 128), device="cuda"), d1["k"][:, :1].contiguous(),
        torch.ones((B, H, 1), device="cuda"), none, t0, 0, d1["q"], d1["k"], d1["v"], d1["alpha"],
        d1["beta"], t1, md1)
    acc = np.array([rng.integers(0, len(p)) for p in p1], dtype=np.int32)
    out2, vt2, _ = abi.commit_verify_pool_trees(
        pool, slots, vt1, d1["k"], gm1, torch.from_numpy(acc).cuda(), t1, md1, d2["q"], d2["k"],
        d2["v"], d2["alpha"], d2["beta"], t2, md2)
    torch.cuda.synchronize()
    f64 = lambda x: np.asarray(x, dtype=np.float64)
    picks = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(6)]
    sl = slots.cpu().numpy()
    for b, h in picks:
        n1, n2 = len(p1[b]), len(p2[b])
        w1 = oracle.walk(f64(in1.S0[b, h])[None], f64(in1.q[b, :n1, h])[None],
                         f64(in1.k[b, :n1, h])[None], f64(in1.v[b, :n1, h])[None],
                         f64(in1.alpha[b, :n1, h])[None], f64(in1.beta[b, :n1, h])[None], p1[b])
        Sa = w1.states[:, acc[b]]
        w2 = oracle.walk(Sa, f64(in2.q[b, :n2, h])[None], f64(in2.k[b, :n2, h])[None],
                         f64(in2.v[b, :n2, h])[None], f64(in2.alpha[b, :n2, h])[None],
                         f64(in2.beta[b, :n2, h])[None], p2[b])
        _err(f"full ({b},{h}) state", pool[int(sl[b]), h].cpu().numpy(), Sa[0])
        _err(f"full ({b},{h}) out", out2[b, :n2, h].cpu().numpy(), w2.out[0])
        _err(f"full ({b},{h}) vtilde", vt2[b, h, :n2].cpu().numpy(), w2.vtilde[0])


def test_graph_replay_takes_new_trees_through_descriptors():
    """One captured launch for a batch bucket (node-count bound 15, depth
    bound 14); before each replay every request gets a new tree, copied into
    the captured descriptor buffer, the way a serving loop reuses one graph
    per bucket.  Each replay equals an eager call on the same descriptors, bit
    for bit (no previous step to commit, so the pool is read only)."""
    B, H, NB, DB = 4, 3, 15, 14
    rng = np.random.default_rng(77)
    inp = synth.make_inputs("35b-tree222", B=B, H=H, seed=77, parent=synth.chain(NB))
    d = to_device(inp)
    n_pool = B + 2
    slots = torch.tensor(rng.permutation(n_pool)[:B], dtype=torch.int32, device="cuda")
    pool = torch.zeros((n_pool, H, 128, 128), dtype=torch.float32, device="cuda")
    pool[slots.long()] = d["S0"]
    before = pool.clone()
    t0, _, _ = _descs([np.array([-1], dtype=np.int32)] * B)
    none = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    vt0 = torch.zeros((B, H, 1, 128), dtype=torch.float32, device="cuda")
    k0 = d["k"][:, :1].contiguous()
    gm0 = torch.ones((B, H, 1), dtype=torch.float32, device="cuda")

    def tree_set():
        sizes = rng.integers(1, NB + 1, size=B)
        parents = _trees(sizes, rng)
        host, _, md = abi.pack_trees(parents, n_max=NB)
        assert md <= DB
        return torch.from_numpy(host.copy()).cuda(), [int(n) for n in sizes]

    def call(trees, out, vt, gm, stream=None):
        abi.commit_verify_pool_trees(pool, slots, vt0, k0, gm0, none, t0, 0, d["q"], d["k"], d["v"],
                                     d["alpha"], d["beta"], trees, DB, stream=stream, out=out,
                                     vtilde=vt, gamma=gm)

    trees, _ = tree_set()
    g_out, g_vt, g_gm = _nan((B, NB, H, 128)), _nan((B, H, NB, 128)), _nan((B, H, NB))
    call(trees, g_out, g_vt, g_gm)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(trees, g_out, g_vt, g_gm, stream=s)
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(torch.nan_to_num(a, nan=7.0), torch.nan_to_num(b, nan=7.0))
    for r in range(3):
        new, sizes = tree_set()
        print(f"replay {r}: tree sizes {sizes}", flush=True)
        e_out, e_vt, e_gm = _nan((B, NB, H, 128)), _nan((B, H, NB, 128)), _nan((B, H, NB))
        call(new, e_out, e_vt, e_gm)
        trees.copy_(new)
        for x in (g_out, g_vt, g_gm):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(g_out, e_out) and same(g_vt, e_vt) and same(g_gm, e_gm), f"replay {r}"
        for b, n in enumerate(sizes):
            assert torch.isfinite(e_out[b, :n]).all() and torch.isnan(e_out[b, n:]).all(), (r, b)
    assert torch.equal(pool, before)
