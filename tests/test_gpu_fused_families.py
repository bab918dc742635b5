"""The three commit-then-verify families on random and deep trees, so that
every (tile count, depth class) instantiation of each is exercised:

* fp32 state in a batch (treewy_commit_verify) against the fp64 oracle
  walking both steps (2e-3);
* the pool form (treewy_commit_verify_pool) against the batch form on the
  same states (1e-5), its committed blocks included;
* the bf16-state form (treewy_commit_verify_bf16state) on the same state
  rounded to bf16: its stored state equals the batch form's committed state
  rounded to bf16 bit for bit, and its outputs equal a plain verify from the
  stored state (1e-5).

Node counts 1..64 cover 1..8 tiles of [K;Q]; the deep cases cover the depth
classes < 4, < 16 and < 64.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
from gpu_cases import TOL, all_pairs, rel_err, to_device  # noqa: E402

import oracle  # noqa: E402
from gated_deltanet_tree_03_amd import abi, synth  # noqa: E402

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TIGHT = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(abi.LIB_PATH):
        pytest.fail("libtreewy.so is not built")
    torch.cuda.set_device(0)
    yield


def _err(label, got, ref, tol):
    e = rel_err(got, ref)
    print(f"{label}: {e:.2e}", flush=True)
    assert np.isfinite(e) and e <= tol, f"{label}: rel err {e:.3e} > {tol}"


def _case(cfg, p_prev, p_new, seed, label, B=2, H=3):
    rng = np.random.default_rng(seed)
    prev = synth.make_inputs(cfg, B=B, H=H, seed=seed, parent=p_prev)
    prev.accepted = rng.integers(0, len(p_prev), size=B).astype(np.int32)
    new = synth.make_inputs(cfg, B=B, H=H, seed=seed + 1, parent=p_new)
    pd, nd = to_device(prev), to_device(new)
    pd["accepted"] = torch.from_numpy(prev.accepted).cuda()
    # a state that is exact in bf16, so all three families start from one value
    S_bf = pd["S0"].to(torch.bfloat16)
    S_f = S_bf.float()
    prev.S0 = S_f.cpu().numpy()
    print(f"case {label}: N_prev={len(p_prev)} N={len(p_new)} "
          f"depths {synth.node_depths(p_prev).max()}/{synth.node_depths(p_new).max()}", flush=True)
    _, vt0, gm0 = abi.verify(S_f, pd["q"], pd["k"], pd["v"], pd["alpha"], pd["beta"], prev.parent)
    args = (vt0, pd["k"], gm0, pd["accepted"], prev.parent, nd["q"], nd["k"], nd["v"],
            nd["alpha"], nd["beta"], new.parent)
    # fp32 state, batch form
    S_b, out_b, vt_b, gm_b = abi.commit_verify(S_f.clone(), *args)
    # pool form: the sequences on distinct random slots of a pool with 3 spare blocks
    n_pool = B + 3
    slot_list = rng.permutation(n_pool)[:B]
    slots = torch.tensor(slot_list, dtype=torch.int32, device="cuda")
    pool = torch.zeros((n_pool, H, 128, 128), dtype=torch.float32, device="cuda")
    pool[slots.long()] = S_f
    out_p, vt_p, gm_p = abi.commit_verify_pool(pool, slots, *args)
    # bf16 state
    S_16, out_16, vt_16, gm_16 = abi.commit_verify_bf16state(S_bf.clone(), *args)
    o_ref, v_ref, _ = abi.verify(S_16.float(), nd["q"], nd["k"], nd["v"], nd["alpha"], nd["beta"],
                                 new.parent)
    torch.cuda.synchronize()
    # batch form against the oracle
    pairs = all_pairs(B, H)
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    f = lambda inp, x: x[bs, :, hs].astype(np.float64)
    w0 = oracle.walk(prev.S0[bs, hs].astype(np.float64), f(prev, prev.q), f(prev, prev.k),
                     f(prev, prev.v), f(prev, prev.alpha), f(prev, prev.beta), prev.parent)
    Sa = w0.states[np.arange(len(pairs)), prev.accepted[bs]]
    w1 = oracle.walk(Sa, f(new, new.q), f(new, new.k), f(new, new.v), f(new, new.alpha),
                     f(new, new.beta), new.parent)
    bsi, hsi = torch.as_tensor(bs, device="cuda"), torch.as_tensor(hs, device="cuda")
    _err(f"{label} batch state", S_b[bsi, hsi].cpu().numpy(), Sa, TOL)
    _err(f"{label} batch out", out_b[bsi, :, hsi].cpu().numpy(), w1.out, TOL)
    _err(f"{label} batch vtilde", vt_b[bsi, hsi].cpu().numpy(), w1.vtilde, TOL)
    # pool form against the batch form
    _err(f"{label} pool state", pool[slots.long()].cpu().numpy(), S_b.cpu().numpy(), TIGHT)
    _err(f"{label} pool out", out_p.cpu().numpy(), out_b.cpu().numpy(), TIGHT)
    _err(f"{label} pool vtilde", vt_p.cpu().numpy(), vt_b.cpu().numpy(), TIGHT)
    assert torch.equal(gm_p, gm_b)
    spare = [i for i in range(n_pool) if i not in set(slot_list.tolist())]
    assert not pool[spare].any(), "a pool block no sequence names was written"
    # bf16 state
    assert torch.equal(S_16, S_b.to(torch.bfloat16)), "stored state != batch state rounded"
    _err(f"{label} bf16-state out", out_16.cpu().numpy(), o_ref.cpu().numpy(), TIGHT)
    _err(f"{label} bf16-state vtilde", vt_16.cpu().numpy(), v_ref.cpu().numpy(), TIGHT)
    assert torch.equal(gm_16, gm_b)


@pytest.mark.parametrize("n", [1, 2, 7, 9, 17, 24, 33, 40, 48, 57, 64])
def test_random_trees_all_families(n):
    rng = np.random.default_rng(2000 + n)
    p_prev = synth.random_preorder_tree(int(rng.integers(1, 65)), rng)
    p_new = synth.random_preorder_tree(n, rng)
    _case("35b-tree222", p_prev, p_new, 300 + n, f"random n={n}")


@pytest.mark.parametrize("n,cap", [(64, None), (12, None), (30, 15), (20, 17)])
def test_deep_trees_all_families(n, cap):
    """Every depth class (gates near 1 keep Gamma in the fp32 normal range)."""
    rng = np.random.default_rng(3000 + n)
    p_new = synth.chain(n) if cap is None else synth.random_preorder_tree(n, rng, max_depth=cap)
    p_prev = synth.chain(24)
    _case("wide-tree333", p_prev, p_new, 400 + n, f"deep n={n} cap={cap}")


def test_wide_tree_xcd_head_order_all_families():
    """Trees of 33+ nodes map workgroups to heads in XCD-contiguous order when
    the grid is a multiple of 8: every head of a 16-head grid, all families."""
    _case("wide-tree333", synth.chain(4), synth.tree_from_widths((3, 3, 3)), 450,
          "(3,3,3) tree, 16 heads", B=4, H=4)
