"""GPU parity of treewy_commit_verify (the previous step's commit fused into
the next step's verify), through the C ABI:

* against the fp64 oracle walking both steps node by node (2e-3, every element
  on small cases, sampled heads at full size);
* against the two separate calls (commit, then verify on its result), which
  compute the same arithmetic, to a tight tolerance;
* several steps in a row, in place, with differing tree shapes per step, an
  out-of-range accepted index, and HIP-graph replay.
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


def _heads(inp, pairs, with_state=True):
    """Oracle inputs of the listed (b, h) pairs (the state only if asked for:
    a later step starts from the state committed by the one before)."""
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    S = inp.S0[bs, hs].astype(np.float64) if with_state else None
    f = lambda x: x[bs, :, hs].astype(np.float64)
    return S, f(inp.q), f(inp.k), f(inp.v), f(inp.alpha), f(inp.beta), inp.accepted[bs]


def _step_inputs(name, B, H, seed, parent=None, dtype=None):
    inp = synth.make_inputs(name, B=B, H=H, seed=seed, parent=parent, dtype=dtype)
    d = to_device(inp)
    return inp, d


def _fused_step(prev_inp, prev_dev, vt_prev, gm_prev, S, new_inp, new_dev, S_out=None):
    return abi.commit_verify(S, vt_prev, prev_dev["k"], gm_prev, prev_dev["accepted"],
                             prev_inp.parent, new_dev["q"], new_dev["k"], new_dev["v"],
                             new_dev["alpha"], new_dev["beta"], new_inp.parent, S_out=S_out)


def _check(label, got, ref):
    errs = {k: rel_err(got[k], ref[k]) for k in ref}
    _say(f"{label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert np.isfinite(v) and v <= TOL, f"{label}: {k} rel err {v:.3e} > {TOL}"


def _gather(out, vt, gm, S, pairs):
    bs = torch.as_tensor([p[0] for p in pairs], device="cuda")
    hs = torch.as_tensor([p[1] for p in pairs], device="cuda")
    return dict(out=out[bs, :, hs].cpu().numpy(), vtilde=vt[bs, hs].cpu().numpy(),
                gamma=gm[bs, hs].cpu().numpy(), S_out=S[bs, hs].cpu().numpy())


def _two_step_case(prev_inp, prev_dev, new_inp, new_dev, pairs, label):
    # previous step: verify on the GPU (its pseudo-values feed the fused commit)
    _, vt0, gm0 = abi.verify(prev_dev["S0"], prev_dev["q"], prev_dev["k"], prev_dev["v"],
                             prev_dev["alpha"], prev_dev["beta"], prev_inp.parent)
    S = prev_dev["S0"].clone()
    S_out, out1, vt1, gm1 = _fused_step(prev_inp, prev_dev, vt0, gm0, S, new_inp, new_dev)
    torch.cuda.synchronize()
    # oracle: walk the previous step, take the accepted state, walk the new step from it
    S0p, q0, k0, v0, a0, b0, acc0 = _heads(prev_inp, pairs)
    w0 = oracle.walk(S0p, q0, k0, v0, a0, b0, prev_inp.parent)
    Sa = w0.states[np.arange(len(pairs)), acc0]
    _, q1, k1, v1, a1, b1, _ = _heads(new_inp, pairs, with_state=False)
    w1 = oracle.walk(Sa, q1, k1, v1, a1, b1, new_inp.parent)
    ref = dict(out=w1.out, vtilde=w1.vtilde, gamma=oracle.gamma_scan(a1, new_inp.parent), S_out=Sa)
    _check(label, _gather(out1, vt1, gm1, S_out, pairs), ref)
    return vt0, gm0, S_out, out1, vt1, gm1


@pytest.mark.parametrize("name", ["35b-chain4", "35b-tree222", "397b-tree222", "wide-tree333"])
def test_two_steps_against_oracle(name):
    prev_inp, prev_dev = _step_inputs(name, 3, 5, 31)
    new_inp, new_dev = _step_inputs(name, 3, 5, 32)
    _two_step_case(prev_inp, prev_dev, new_inp, new_dev, all_pairs(3, 5), f"{name} two steps")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tree_shape_changes_between_steps(dtype):
    rng = np.random.default_rng(5)
    p_prev = synth.random_preorder_tree(23, rng)
    p_new = synth.random_preorder_tree(9, rng)
    prev_inp, prev_dev = _step_inputs("35b-tree222", 2, 3, 41, parent=p_prev, dtype=dtype)
    prev_inp.accepted = rng.integers(0, 23, size=2).astype(np.int32)
    prev_dev["accepted"] = torch.from_numpy(prev_inp.accepted).cuda()
    new_inp, new_dev = _step_inputs("35b-tree222", 2, 3, 42, parent=p_new, dtype=dtype)
    _two_step_case(prev_inp, prev_dev, new_inp, new_dev, all_pairs(2, 3), f"shape change {dtype}")


def test_deep_previous_path():
    """A 20-node chain before: the committed path spans several staging rounds."""
    p_prev = synth.chain(20)
    prev_inp, prev_dev = _step_inputs("wide-tree333", 2, 2, 51, parent=p_prev)
    prev_inp.accepted = np.array([19, 11], dtype=np.int32)
    prev_dev["accepted"] = torch.from_numpy(prev_inp.accepted).cuda()
    new_inp, new_dev = _step_inputs("wide-tree333", 2, 2, 52)
    _two_step_case(prev_inp, prev_dev, new_inp, new_dev, all_pairs(2, 2), "deep previous path")


def test_equals_separate_calls():
    prev_inp, prev_dev = _step_inputs("35b-tree222", 4, 6, 61)
    new_inp, new_dev = _step_inputs("35b-tree222", 4, 6, 62)
    _, vt0, gm0 = abi.verify(prev_dev["S0"], prev_dev["q"], prev_dev["k"], prev_dev["v"],
                             prev_dev["alpha"], prev_dev["beta"], prev_inp.parent)
    S_seq = abi.commit(prev_dev["S0"], vt0, prev_dev["k"], gm0, prev_dev["accepted"], prev_inp.parent)
    seq = abi.verify(S_seq, new_dev["q"], new_dev["k"], new_dev["v"], new_dev["alpha"],
                     new_dev["beta"], new_inp.parent)
    S_f, *fused = _fused_step(prev_inp, prev_dev, vt0, gm0, prev_dev["S0"].clone(), new_inp, new_dev)
    torch.cuda.synchronize()
    for nm, x, y in zip(("S_out", "out", "vtilde", "gamma"), (S_f, *fused), (S_seq, *seq)):
        err = ((x - y).abs().max() / y.abs().max()).item()
        _say(f"fused vs separate {nm}: {err:.2e}")
        assert err <= 1e-5, nm


def test_three_steps_in_place():
    B, H = 2, 4
    rng = np.random.default_rng(9)
    shapes = [synth.tree_from_widths((2, 2, 2)), synth.chain(4), synth.tree_from_widths((3, 1, 2))]
    inps = [_step_inputs("35b-tree222", B, H, 70 + i, parent=p) for i, p in enumerate(shapes)]
    for inp, d in inps:
        inp.accepted = rng.integers(0, len(inp.parent), size=B).astype(np.int32)
        d["accepted"] = torch.from_numpy(inp.accepted).cuda()
    S = inps[0][1]["S0"].clone()
    _, vt, gm = abi.verify(S, *(inps[0][1][n] for n in ("q", "k", "v", "alpha", "beta")),
                           inps[0][0].parent)
    for i in (1, 2):
        S, out, vt, gm = _fused_step(inps[i - 1][0], inps[i - 1][1], vt, gm, S, *inps[i], S_out=S)
    torch.cuda.synchronize()
    # oracle: walk the three steps, committing the accepted node after the first two
    pairs = all_pairs(B, H)
    Sref = _heads(inps[0][0], pairs)[0]
    for i, (inp, _) in enumerate(inps):
        _, q, k, v, a, b, acc = _heads(inp, pairs, with_state=False)
        w = oracle.walk(Sref, q, k, v, a, b, inp.parent)
        if i < 2:
            Sref = w.states[np.arange(len(pairs)), acc]
    ref = dict(out=w.out, vtilde=w.vtilde, gamma=oracle.gamma_scan(a, inps[2][0].parent), S_out=Sref)
    _check("three steps", _gather(out, vt, gm, S, pairs), ref)


def test_in_place_equals_out_of_place_and_invalid_accepted():
    prev_inp, prev_dev = _step_inputs("35b-chain4", 4, 3, 81)
    new_inp, new_dev = _step_inputs("35b-chain4", 4, 3, 82)
    _, vt0, gm0 = abi.verify(prev_dev["S0"], prev_dev["q"], prev_dev["k"], prev_dev["v"],
                             prev_dev["alpha"], prev_dev["beta"], prev_inp.parent)
    S_oop = torch.empty_like(prev_dev["S0"])
    r_oop = _fused_step(prev_inp, prev_dev, vt0, gm0, prev_dev["S0"], new_inp, new_dev, S_out=S_oop)
    S_in = prev_dev["S0"].clone()
    r_in = _fused_step(prev_inp, prev_dev, vt0, gm0, S_in, new_inp, new_dev, S_out=S_in)
    torch.cuda.synchronize()
    for x, y in zip(r_oop, r_in):
        assert torch.equal(x, y)
    bad = prev_dev["accepted"].clone()
    bad[1] = -1
    bad[2] = 4
    prev_bad = dict(prev_dev, accepted=bad)
    S_b, out_b, vt_b, gm_b = _fused_step(prev_inp, prev_bad, vt0, gm0, prev_dev["S0"], new_inp,
                                         new_dev, S_out=torch.empty_like(prev_dev["S0"]))
    torch.cuda.synchronize()
    for b in (1, 2):
        assert torch.isnan(S_b[b]).all() and torch.isnan(out_b[b]).all() and torch.isnan(vt_b[b]).all()
    for b in (0, 3):
        assert torch.equal(S_b[b], S_oop[b]) and torch.equal(out_b[b], r_oop[1][b])
        assert torch.equal(vt_b[b], r_oop[2][b])


@pytest.mark.parametrize("name", ["35b-chain4", "35b-tree222", "397b-chain4", "397b-tree222",
                                  "wide-tree333"])
def test_full_size_sampled(name):
    prev_inp, prev_dev = _step_inputs(name, None, None, None)
    new_inp = synth.make_inputs(name, seed=synth.CONFIGS[name].seed + 500)
    new_inp.S0 = None  # the new step starts from the committed state
    new_dev = {n: torch.from_numpy(np.ascontiguousarray(new_inp.bits[n]).view(np.int16)).cuda()
               .view(torch.bfloat16) for n in ("q", "k", "v", "alpha", "beta")}
    _say(f"{name}: B={prev_inp.B} H={prev_inp.H} N={prev_inp.N}")
    pairs = sample_pairs(prev_inp.B, prev_inp.H, 32, seed=13)
    _two_step_case(prev_inp, prev_dev, new_inp, new_dev, pairs, f"{name} full size")


def test_graph_capture_replay_matches_eager():
    prev_inp, prev_dev = _step_inputs("35b-tree222", 8, 4, 91)
    new_inp, new_dev = _step_inputs("35b-tree222", 8, 4, 92)
    _, vt0, gm0 = abi.verify(prev_dev["S0"], prev_dev["q"], prev_dev["k"], prev_dev["v"],
                             prev_dev["alpha"], prev_dev["beta"], prev_inp.parent)
    B, H, N = 8, 4, new_inp.N
    S_out = torch.empty_like(prev_dev["S0"])
    out = torch.empty((B, N, H, 128), device="cuda")
    vt = torch.empty((B, H, N, 128), device="cuda")
    gm = torch.empty((B, H, N), device="cuda")
    args = (prev_dev["S0"], vt0, prev_dev["k"], gm0, prev_dev["accepted"], prev_inp.parent,
            new_dev["q"], new_dev["k"], new_dev["v"], new_dev["alpha"], new_dev["beta"], new_inp.parent)
    abi.commit_verify(*args, S_out=S_out, out=out, vtilde=vt, gamma=gm)
    torch.cuda.synchronize()
    eager = [x.clone() for x in (S_out, out, vt, gm)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            abi.commit_verify(*args, S_out=S_out, out=out, vtilde=vt, gamma=gm, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (S_out, out, vt, gm):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip((S_out, out, vt, gm), eager):
            assert torch.equal(x, y), f"replay {rep} differs"
