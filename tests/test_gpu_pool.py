"""GPU parity of treewy_commit_verify_pool (commit-then-verify over a
slot-indexed state pool), through the C ABI:

* against the fp64 oracle walking both steps node by node, for states
  scattered over a pool larger than the batch (2e-3);
* against treewy_commit_verify on the same states gathered into a batch
  (same arithmetic: a tight tolerance), with every pool block that no
  sequence names left bit for bit as it was;
* per-sequence cases: a request with no previous step (its block is read
  and not rewritten), an out-of-range accepted index (NaN block), a slot
  outside the pool (no pool memory touched, NaN outputs);
* the full-size 35B-like chain on sampled heads, and HIP-graph replay.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))
from gpu_cases import TOL, all_pairs, rel_err, sample_pairs, to_device  # noqa: E402

import oracle  # noqa: E402
from gated_deltanet_tree_03_amd import abi, synth  # noqa: E402

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TIGHT = 1e-5  # pool form vs the batch form: the same arithmetic


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


def _steps(name, B, H, seed, dtype=None):
    prev = synth.make_inputs(name, B=B, H=H, seed=seed, dtype=dtype)
    new = synth.make_inputs(name, B=B, H=H, seed=seed + 1, dtype=dtype)
    return prev, to_device(prev), new, to_device(new)


def _pool_with(states, n_slots, slots, seed):
    """A pool of n_slots random blocks with states[b] placed at slots[b]."""
    B, H = states.shape[:2]
    g = torch.Generator(device="cpu").manual_seed(seed)
    pool = (torch.randn((n_slots, H, 128, 128), generator=g) * 0.02).cuda()
    for b, s in enumerate(slots):
        if 0 <= s < n_slots:
            pool[s] = states[b]
    return pool


def _prev_verify(prev, prev_dev):
    _, vt0, gm0 = abi.verify(prev_dev["S0"], prev_dev["q"], prev_dev["k"], prev_dev["v"],
                             prev_dev["alpha"], prev_dev["beta"], prev.parent)
    return vt0, gm0


def _run_pool(pool, slots_t, prev, prev_dev, vt0, gm0, acc_t, new, new_dev):
    return abi.commit_verify_pool(pool, slots_t, vt0, prev_dev["k"], gm0, acc_t, prev.parent,
                                  new_dev["q"], new_dev["k"], new_dev["v"], new_dev["alpha"],
                                  new_dev["beta"], new.parent)


def _err(label, got, ref, tol):
    e = rel_err(got, ref)
    _say(f"{label}: {e:.2e}")
    assert np.isfinite(e) and e <= tol, f"{label}: rel err {e:.3e} > {tol}"


@pytest.mark.parametrize("name,dtype", [("35b-chain4", None), ("35b-tree222", None),
                                        ("wide-tree333", None), ("35b-tree222", "f32")])
def test_pool_matches_oracle_and_batch_form(name, dtype):
    B, H, n_slots = 4, 5, 11
    prev, prev_dev, new, new_dev = _steps(name, B, H, 61, dtype)
    slots = [7, 2, 10, 0]
    _say(f"case {name} {dtype} B={B} H={H} slots={slots} of {n_slots}")
    pool = _pool_with(prev_dev["S0"], n_slots, slots, 62)
    before = pool.clone()
    slots_t = torch.tensor(slots, dtype=torch.int32, device="cuda")
    vt0, gm0 = _prev_verify(prev, prev_dev)
    out, vt, gm = _run_pool(pool, slots_t, prev, prev_dev, vt0, gm0, prev_dev["accepted"], new,
                            new_dev)
    # batch form on the same states
    S = prev_dev["S0"].clone()
    S_b, out_b, vt_b, gm_b = abi.commit_verify(S, vt0, prev_dev["k"], gm0, prev_dev["accepted"],
                                               prev.parent, new_dev["q"], new_dev["k"],
                                               new_dev["v"], new_dev["alpha"], new_dev["beta"],
                                               new.parent)
    torch.cuda.synchronize()
    _err("pool vs batch: out", out.cpu().numpy(), out_b.cpu().numpy(), TIGHT)
    _err("pool vs batch: vtilde", vt.cpu().numpy(), vt_b.cpu().numpy(), TIGHT)
    _err("pool vs batch: gamma", gm.cpu().numpy(), gm_b.cpu().numpy(), TIGHT)
    _err("pool vs batch: state", pool[slots_t.long()].cpu().numpy(), S_b.cpu().numpy(), TIGHT)
    untouched = [s for s in range(n_slots) if s not in slots]
    assert torch.equal(pool[untouched], before[untouched]), "a block no sequence names changed"
    # oracle: both steps walked node by node
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
    _err("pool vs oracle: out", out[bsi, :, hsi].cpu().numpy(), w1.out, TOL)
    _err("pool vs oracle: vtilde", vt[bsi, hsi].cpu().numpy(), w1.vtilde, TOL)
    _err("pool vs oracle: state", pool[slots_t.long()[bsi], hsi].cpu().numpy(), Sa, TOL)


def test_pool_new_request_bad_accepted_and_bad_slot():
    B, H, n_slots = 4, 3, 6
    prev, prev_dev, new, new_dev = _steps("35b-tree222", B, H, 71)
    slots = [4, 1, 3, n_slots + 2]          # the last one lies outside the pool
    acc = [-1, int(prev.accepted[1]), prev.N, int(prev.accepted[3])]
    _say(f"case slots={slots} accepted_prev={acc}")
    pool = _pool_with(prev_dev["S0"], n_slots, slots, 72)
    before = pool.clone()
    slots_t = torch.tensor(slots, dtype=torch.int32, device="cuda")
    acc_t = torch.tensor(acc, dtype=torch.int32, device="cuda")
    vt0, gm0 = _prev_verify(prev, prev_dev)
    out, vt, gm = _run_pool(pool, slots_t, prev, prev_dev, vt0, gm0, acc_t, new, new_dev)
    torch.cuda.synchronize()
    # b = 0, no previous step: the block is left as it was and verified as it is
    assert torch.equal(pool[4], before[4])
    o0, v0, _ = abi.verify(before[4:5].contiguous(), new_dev["q"][0:1].contiguous(),
                           new_dev["k"][0:1].contiguous(), new_dev["v"][0:1].contiguous(),
                           new_dev["alpha"][0:1].contiguous(), new_dev["beta"][0:1].contiguous(),
                           new.parent)
    torch.cuda.synchronize()
    _err("new request: out", out[0:1].cpu().numpy(), o0.cpu().numpy(), TIGHT)
    _err("new request: vtilde", vt[0:1].cpu().numpy(), v0.cpu().numpy(), TIGHT)
    # b = 1: an ordinary commit, so the block changed
    assert not torch.equal(pool[1], before[1])
    assert torch.isfinite(pool[1]).all() and torch.isfinite(out[1]).all()
    # b = 2, accepted index out of range: NaN block and outputs
    assert torch.isnan(pool[3]).all()
    assert torch.isnan(out[2]).all() and torch.isnan(vt[2]).all()
    # b = 3, slot outside the pool: NaN outputs, no pool block touched
    assert torch.isnan(out[3]).all() and torch.isnan(vt[3]).all()
    for s in (0, 2, 5):
        assert torch.equal(pool[s], before[s]), f"block {s} changed"


def test_pool_full_size_sampled():
    name = "35b-chain4"
    prev = synth.make_inputs(name)
    new = synth.make_inputs(name, seed=777)
    prev_dev, new_dev = to_device(prev), to_device(new)
    B, H = prev.B, prev.H
    n_slots = 2 * B
    rng = np.random.default_rng(81)
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    _say(f"case {name} full size B={B} H={H} pool {n_slots} slots")
    pool = torch.empty((n_slots, H, 128, 128), dtype=torch.float32, device="cuda")
    pool.fill_(float("nan"))
    slots_t = torch.from_numpy(slots).cuda()
    pool[slots_t.long()] = prev_dev["S0"]
    vt0, gm0 = _prev_verify(prev, prev_dev)
    out, vt, gm = _run_pool(pool, slots_t, prev, prev_dev, vt0, gm0, prev_dev["accepted"], new,
                            new_dev)
    torch.cuda.synchronize()
    pairs = sample_pairs(B, H, 24, seed=82)
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    f = lambda inp, x: x[bs, :, hs].astype(np.float64)
    w0 = oracle.walk(prev.S0[bs, hs].astype(np.float64), f(prev, prev.q), f(prev, prev.k),
                     f(prev, prev.v), f(prev, prev.alpha), f(prev, prev.beta), prev.parent)
    Sa = w0.states[np.arange(len(pairs)), prev.accepted[bs]]
    w1 = oracle.walk(Sa, f(new, new.q), f(new, new.k), f(new, new.v), f(new, new.alpha),
                     f(new, new.beta), new.parent)
    bsi, hsi = torch.as_tensor(bs, device="cuda"), torch.as_tensor(hs, device="cuda")
    _err("full size: out", out[bsi, :, hsi].cpu().numpy(), w1.out, TOL)
    _err("full size: vtilde", vt[bsi, hsi].cpu().numpy(), w1.vtilde, TOL)
    _err("full size: state", pool[slots_t.long()[bsi], hsi].cpu().numpy(), Sa, TOL)
    free = np.setdiff1d(np.arange(n_slots), slots)
    assert torch.isnan(pool[torch.from_numpy(free).cuda()]).all(), "a free block was written"


def test_pool_graph_replay_matches_eager():
    """With no previous step to commit (accepted_prev = -1 everywhere) every
    replay reads the same states, so each must equal the eager call."""
    B, H, n_slots = 3, 4, 5
    prev, prev_dev, new, new_dev = _steps("35b-tree222", B, H, 91)
    slots = [3, 0, 4]
    pool = _pool_with(prev_dev["S0"], n_slots, slots, 92)
    before = pool.clone()
    slots_t = torch.tensor(slots, dtype=torch.int32, device="cuda")
    acc_t = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    vt0, gm0 = _prev_verify(prev, prev_dev)
    out = torch.empty((B, new.N, H, 128), dtype=torch.float32, device="cuda")
    vt = torch.empty((B, H, new.N, 128), dtype=torch.float32, device="cuda")
    gm = torch.empty((B, H, new.N), dtype=torch.float32, device="cuda")
    call = lambda stream: abi.commit_verify_pool(
        pool, slots_t, vt0, prev_dev["k"], gm0, acc_t, prev.parent, new_dev["q"], new_dev["k"],
        new_dev["v"], new_dev["alpha"], new_dev["beta"], new.parent, stream=stream, out=out,
        vtilde=vt, gamma=gm)
    call(None)
    torch.cuda.synchronize()
    ref = (out.clone(), vt.clone(), gm.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(s)
    torch.cuda.synchronize()
    for r in range(3):
        out.zero_()
        vt.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(vt, ref[1]) and torch.equal(gm, ref[2]), r
    assert torch.equal(pool, before)
