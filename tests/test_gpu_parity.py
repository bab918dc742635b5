"""GPU parity: the HIP path (called through the C ABI) against the fp64 oracle
on identical seeded inputs, max |diff| / max |ref| <= 2e-3 per tensor (out,
vtilde, committed state; also gamma and the store_all baseline).

Small cases compare every element; full-size workloads (the five shapes the
bench uses) compare sampled (sequence, head) pairs, computed by the oracle one
by one, in the same launch configuration the bench times."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
from gpu_cases import (TOL, all_pairs, full_inputs, gather_device, oracle_heads,  # noqa: E402
                       rel_err, sample_pairs, to_device)

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


def _say(msg):
    print(msg, flush=True)


def run_path(inp, with_store_all=True, poison=True):
    d = to_device(inp)
    B, H, N = inp.B, inp.H, inp.N
    out = torch.full((B, N, H, 128), float("nan"), device="cuda") if poison else None
    vt = torch.full((B, H, N, 128), float("nan"), device="cuda") if poison else None
    gm = torch.full((B, H, N), float("nan"), device="cuda") if poison else None
    out, vt, gm = abi.verify(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], inp.parent,
                             out=out, vtilde=vt, gamma=gm)
    S_out = abi.commit(d["S0"], vt, d["k"], gm, d["accepted"], inp.parent)
    res = dict(dev=d, out=out, vtilde=vt, gamma=gm, S_out=S_out)
    if with_store_all:
        o2, snaps = abi.store_all(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], inp.parent)
        res["sa_out"] = o2
        res["snaps"] = snaps
        res["sa_sel"] = abi.store_all_select(snaps, d["accepted"])
    torch.cuda.synchronize()
    return res


def check_pairs(inp, res, pairs, label):
    ref = oracle_heads(inp, pairs)
    got = gather_device(inp, res["out"], res["vtilde"], res["gamma"], res["S_out"], pairs)
    errs = {
        "out": rel_err(got["out"], ref["out"]),
        "vtilde": rel_err(got["vtilde"], ref["vtilde"]),
        "S_out": rel_err(got["S_out"], ref["S_acc"]),
        "gamma": rel_err(got["gamma"], ref["gamma"]),
    }
    if "sa_out" in res:
        g2 = gather_device(inp, res["sa_out"], res["vtilde"], res["gamma"], res["sa_sel"], pairs)
        errs["store_all.out"] = rel_err(g2["out"], ref["out"])
        errs["store_all.select"] = rel_err(g2["S_out"], ref["S_acc"])
        bs = torch.as_tensor([p[0] for p in pairs], device="cuda")
        hs = torch.as_tensor([p[1] for p in pairs], device="cuda")
        snaps = res["snaps"][bs, hs].cpu().numpy()  # [G, N+1, 128, 128]
        errs["store_all.snap0"] = rel_err(snaps[:, 0], ref["S0"])
        errs["store_all.snaps"] = rel_err(snaps[:, 1:], ref["states"])
    _say(f"{label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert np.isfinite(v) and v <= TOL, f"{label}: {k} rel err {v:.3e} > {TOL}"
    return errs


# ---------------------------------------------------------------------------
# small cases, every element
# ---------------------------------------------------------------------------

def test_c1_fp32_chain_all_heads():
    inp = synth.make_inputs("chain4-f32")
    res = run_path(inp)
    check_pairs(inp, res, all_pairs(inp.B, inp.H), "chain4-f32")


@pytest.mark.parametrize("name", ["35b-chain4", "35b-tree222", "397b-chain4", "397b-tree222", "wide-tree333"])
def test_config_shapes_small_batch_all_heads(name):
    inp = synth.make_inputs(name, B=3, H=5, seed=7)
    res = run_path(inp)
    check_pairs(inp, res, all_pairs(inp.B, inp.H), f"{name}-small")


def test_wide_tree_xcd_head_order_all_heads():
    """A 24-head grid of the (3,3,3) tree: a multiple of 8 heads, so the
    workgroups take heads in XCD-contiguous order; every element checked."""
    inp = synth.make_inputs("wide-tree333", B=4, H=6, seed=11)
    res = run_path(inp)
    check_pairs(inp, res, all_pairs(inp.B, inp.H), "wide-tree333-24-heads")


@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 9, 16, 17, 24, 33, 40, 48, 57, 64])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_random_trees(n, dtype):
    rng = np.random.default_rng(1000 + n)
    parent = synth.random_preorder_tree(n, rng)
    inp = synth.make_inputs("35b-tree222", B=2, H=3, seed=n, parent=parent, dtype=dtype)
    inp.accepted = rng.integers(0, n, size=inp.B).astype(np.int32)
    res = run_path(inp)
    check_pairs(inp, res, all_pairs(inp.B, inp.H), f"random n={n} {dtype} depth={synth.node_depths(parent).max()}")


@pytest.mark.parametrize("n,cap", [(64, None), (40, 5), (30, 15), (20, 17)])
def test_deep_trees_and_long_chains(n, cap):
    """Depths that exercise every register-stack size and the store_all re-read
    of overwritten parents (gates near 1 keep Gamma in the fp32 normal range)."""
    rng = np.random.default_rng(n + (cap or 0))
    parent = synth.chain(n) if cap is None else synth.random_preorder_tree(n, rng, max_depth=cap)
    inp = synth.make_inputs("wide-tree333", B=2, H=2, seed=3, parent=parent)
    inp.accepted = np.array([n - 1, int(rng.integers(0, n))], dtype=np.int32)
    res = run_path(inp)
    check_pairs(inp, res, all_pairs(inp.B, inp.H), f"deep n={n} cap={cap}")


# ---------------------------------------------------------------------------
# full-size workloads (bench shapes), sampled heads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["35b-chain4", "35b-tree222", "397b-chain4", "397b-tree222", "wide-tree333"])
def test_full_size_sampled(name):
    inp = full_inputs(name)
    _say(f"{name}: B={inp.B} H={inp.H} N={inp.N}")
    res = run_path(inp, with_store_all=(name != "wide-tree333"))
    # every output element was written (outputs were NaN-poisoned)
    assert torch.isfinite(res["out"]).all() and torch.isfinite(res["vtilde"]).all()
    assert torch.isfinite(res["S_out"]).all()
    pairs = sample_pairs(inp.B, inp.H, 48, seed=11)
    check_pairs(inp, res, pairs, f"{name}-full")
    # property that holds at any size: S_a q_a reproduces out[a] for every head
    a = res["dev"]["accepted"].long()
    bidx = torch.arange(inp.B, device="cuda")
    qa = res["dev"]["q"][bidx, a].float()                  # [B, H, 128]
    oa = res["out"][bidx, a]                               # [B, H, 128]
    recon = torch.einsum("bhvk,bhk->bhv", res["S_out"], qa)
    err = (recon - oa).abs().max().item() / oa.abs().max().item()
    _say(f"{name}-full: S_a q_a vs out[a] = {err:.2e}")
    assert err <= TOL


def test_c5_store_all_full_size_sampled():
    inp = full_inputs("wide-tree333")
    d = to_device(inp)
    out, snaps = abi.store_all(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], inp.parent)
    sel = abi.store_all_select(snaps, d["accepted"])
    torch.cuda.synchronize()
    pairs = sample_pairs(inp.B, inp.H, 24, seed=5)
    ref = oracle_heads(inp, pairs)
    bs = torch.as_tensor([p[0] for p in pairs], device="cuda")
    hs = torch.as_tensor([p[1] for p in pairs], device="cuda")
    e_out = rel_err(out[bs, :, hs].cpu().numpy(), ref["out"])
    e_sel = rel_err(sel[bs, hs].cpu().numpy(), ref["S_acc"])
    e_snap = rel_err(snaps[bs, hs, 1:].cpu().numpy(), ref["states"])
    _say(f"wide-tree333 store_all full: out={e_out:.2e} select={e_sel:.2e} snaps={e_snap:.2e}")
    assert max(e_out, e_sel, e_snap) <= TOL


# ---------------------------------------------------------------------------
# behaviour
# ---------------------------------------------------------------------------

def test_in_place_commit_and_invalid_accepted():
    inp = synth.make_inputs("35b-tree222", B=4, H=3, seed=21)
    d = to_device(inp)
    out, vt, gm = abi.verify(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], inp.parent)
    ref_S = abi.commit(d["S0"], vt, d["k"], gm, d["accepted"], inp.parent)
    S = d["S0"].clone()
    abi.commit(S, vt, d["k"], gm, d["accepted"], inp.parent, S_out=S)
    torch.cuda.synchronize()
    assert torch.equal(S, ref_S)
    bad = d["accepted"].clone()
    bad[1] = -1
    bad[2] = inp.N
    S2 = abi.commit(d["S0"], vt, d["k"], gm, bad, inp.parent)
    o2, snaps = abi.store_all(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], inp.parent)
    sel = abi.store_all_select(snaps, bad)
    torch.cuda.synchronize()
    for t in (S2, sel):
        assert torch.isnan(t[1]).all() and torch.isnan(t[2]).all()
        assert torch.isfinite(t[0]).all() and torch.isfinite(t[3]).all()
    assert torch.equal(S2[0], ref_S[0]) and torch.equal(S2[3], ref_S[3])


def test_deterministic_repeat():
    inp = synth.make_inputs("wide-tree333", B=4, H=4, seed=2)
    d = to_device(inp)
    r1 = abi.verify(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], inp.parent)
    r2 = abi.verify(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], inp.parent)
    c1 = abi.commit(d["S0"], r1[1], d["k"], r1[2], d["accepted"], inp.parent)
    c2 = abi.commit(d["S0"], r2[1], d["k"], r2[2], d["accepted"], inp.parent)
    torch.cuda.synchronize()
    for x, y in zip(r1 + (c1,), r2 + (c2,)):
        assert torch.equal(x, y)


def test_empty_batch_on_gpu():
    z = torch.zeros(16, device="cuda")
    st = abi.treewy_verify(z, z, z, z, z, z, [-1, 0], 0, 4, 2, z, z, z, abi.TREEWY_BF16, check=False)
    assert st == abi.TREEWY_OK
    torch.cuda.synchronize()


def test_graph_capture_replay_matches_eager():
    inp = synth.make_inputs("35b-tree222", B=8, H=4, seed=9)
    d = to_device(inp)
    B, H, N = inp.B, inp.H, inp.N
    out = torch.empty((B, N, H, 128), device="cuda")
    vt = torch.empty((B, H, N, 128), device="cuda")
    gm = torch.empty((B, H, N), device="cuda")
    S_out = torch.empty_like(d["S0"])
    abi.verify(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], inp.parent, out=out,
               vtilde=vt, gamma=gm)
    abi.commit(d["S0"], vt, d["k"], gm, d["accepted"], inp.parent, S_out=S_out)
    torch.cuda.synchronize()
    eager = [x.clone() for x in (out, vt, gm, S_out)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            abi.verify(d["S0"], d["q"], d["k"], d["v"], d["alpha"], d["beta"], inp.parent, out=out,
                       vtilde=vt, gamma=gm, stream=s)
            abi.commit(d["S0"], vt, d["k"], gm, d["accepted"], inp.parent, S_out=S_out, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (out, vt, gm, S_out):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip((out, vt, gm, S_out), eager):
            assert torch.equal(x, y), f"replay {rep} differs"
