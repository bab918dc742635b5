"""GPU parity of treewy_commit_verify_bf16state (commit-then-verify over a
bf16-stored state), through the C ABI.

The state is exact in bf16 on input; the committed state is rounded to bf16
once when stored, and the new step is verified from that stored value.  So:

* the stored state against the fp64 oracle: one bf16 rounding, at most
  2^-9 of the element (2^-8 of the largest element is the bound used);
* outputs and pseudo-values against the oracle walking the new step from the
  oracle's committed state rounded to bf16 (2e-3, as everywhere);
* the stored state equals the fp32-state kernel's committed state rounded to
  bf16, bit for bit (the same fp32 arithmetic, one rounding), and the outputs
  equal a plain verify from the stored state (1e-5);
* an out-of-range accepted index (NaN), in place, and the full-size 35B-like
  chain on sampled heads.
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

S16_TOL = 2.0 ** -8  # one bf16 rounding of the stored state (<= 2^-9 of each element)
TIGHT = 1e-5


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


def _err(label, got, ref, tol):
    e = rel_err(got, ref)
    _say(f"{label}: {e:.2e}")
    assert np.isfinite(e) and e <= tol, f"{label}: rel err {e:.3e} > {tol}"


def _bf16_state(inp, dev):
    """The workload's state rounded to bf16 (the stored form), its exact fp32
    widening on the device, and the host copy the oracle uses."""
    S_bf = dev["S0"].to(torch.bfloat16)
    S_f = S_bf.float()
    inp.S0 = S_f.cpu().numpy()
    return S_bf, S_f


def _round_bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def _steps(name, B, H, seed):
    prev = synth.make_inputs(name, B=B, H=H, seed=seed)
    new = synth.make_inputs(name, B=B, H=H, seed=seed + 1)
    return prev, to_device(prev), new, to_device(new)


def _run(prev, prev_dev, new, new_dev, S_bf, S_f):
    _, vt0, gm0 = abi.verify(S_f, prev_dev["q"], prev_dev["k"], prev_dev["v"], prev_dev["alpha"],
                             prev_dev["beta"], prev.parent)
    S = S_bf.clone()
    res = abi.commit_verify_bf16state(S, vt0, prev_dev["k"], gm0, prev_dev["accepted"],
                                      prev.parent, new_dev["q"], new_dev["k"], new_dev["v"],
                                      new_dev["alpha"], new_dev["beta"], new.parent)
    return vt0, gm0, res


def _oracle(prev, new, pairs):
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    f = lambda inp, x: x[bs, :, hs].astype(np.float64)
    w0 = oracle.walk(prev.S0[bs, hs].astype(np.float64), f(prev, prev.q), f(prev, prev.k),
                     f(prev, prev.v), f(prev, prev.alpha), f(prev, prev.beta), prev.parent)
    Sa = w0.states[np.arange(len(pairs)), prev.accepted[bs]]
    w1 = oracle.walk(_round_bf16(Sa), f(new, new.q), f(new, new.k), f(new, new.v),
                     f(new, new.alpha), f(new, new.beta), new.parent)
    return bs, hs, Sa, w1


@pytest.mark.parametrize("name", ["35b-chain4", "35b-tree222", "wide-tree333"])
def test_bf16state_against_oracle_and_fp32_state(name):
    B, H = 3, 5
    prev, prev_dev, new, new_dev = _steps(name, B, H, 111)
    _say(f"case {name} B={B} H={H}")
    S_bf, S_f = _bf16_state(prev, prev_dev)
    vt0, gm0, (S_out, out, vt, gm) = _run(prev, prev_dev, new, new_dev, S_bf, S_f)
    torch.cuda.synchronize()
    bs, hs, Sa, w1 = _oracle(prev, new, all_pairs(B, H))
    bsi, hsi = torch.as_tensor(bs, device="cuda"), torch.as_tensor(hs, device="cuda")
    _err("stored state vs oracle", S_out[bsi, hsi].float().cpu().numpy(), Sa, S16_TOL)
    _err("out vs oracle", out[bsi, :, hsi].cpu().numpy(), w1.out, TOL)
    _err("vtilde vs oracle", vt[bsi, hsi].cpu().numpy(), w1.vtilde, TOL)
    # the fp32-state kernel on the same values: same committed state before rounding
    S32, _, _, _ = abi.commit_verify(S_f.clone(), vt0, prev_dev["k"], gm0, prev_dev["accepted"],
                                     prev.parent, new_dev["q"], new_dev["k"], new_dev["v"],
                                     new_dev["alpha"], new_dev["beta"], new.parent)
    o_ref, v_ref, g_ref = abi.verify(S_out.float(), new_dev["q"], new_dev["k"], new_dev["v"],
                                     new_dev["alpha"], new_dev["beta"], new.parent)
    torch.cuda.synchronize()
    assert torch.equal(S_out, S32.to(torch.bfloat16)), "stored state != fp32 state rounded"
    _err("out vs verify(stored)", out.cpu().numpy(), o_ref.cpu().numpy(), TIGHT)
    _err("vtilde vs verify(stored)", vt.cpu().numpy(), v_ref.cpu().numpy(), TIGHT)
    assert torch.equal(gm, g_ref)


def test_bf16state_invalid_accepted_and_out_of_place():
    B, H = 3, 2
    prev, prev_dev, new, new_dev = _steps("35b-tree222", B, H, 121)
    S_bf, S_f = _bf16_state(prev, prev_dev)
    _, vt0, gm0 = abi.verify(S_f, prev_dev["q"], prev_dev["k"], prev_dev["v"], prev_dev["alpha"],
                             prev_dev["beta"], prev.parent)
    acc = prev_dev["accepted"].clone()
    acc[1] = prev.N  # out of range
    S_in = S_bf.clone()
    S_out = torch.empty_like(S_bf)
    _, out, vt, _ = abi.commit_verify_bf16state(S_in, vt0, prev_dev["k"], gm0, acc, prev.parent,
                                                new_dev["q"], new_dev["k"], new_dev["v"],
                                                new_dev["alpha"], new_dev["beta"], new.parent,
                                                S_out=S_out)
    S_ip = S_bf.clone()
    _, out2, vt2, _ = abi.commit_verify_bf16state(S_ip, vt0, prev_dev["k"], gm0, acc, prev.parent,
                                                  new_dev["q"], new_dev["k"], new_dev["v"],
                                                  new_dev["alpha"], new_dev["beta"], new.parent)
    torch.cuda.synchronize()
    assert torch.equal(S_in, S_bf), "out of place modified its input"
    assert torch.isnan(S_out[1].float()).all() and torch.isnan(out[1]).all()
    ok = [0, 2]
    assert torch.isfinite(S_out[ok].float()).all() and torch.isfinite(out[ok]).all()
    # in place gives the same bits as out of place (NaN blocks included)
    assert torch.equal(S_ip.view(torch.int16), S_out.view(torch.int16))
    assert torch.equal(out2[ok], out[ok]) and torch.equal(vt2[ok], vt[ok])


def test_bf16state_full_size_sampled():
    name = "35b-chain4"
    prev = synth.make_inputs(name)
    new = synth.make_inputs(name, seed=778)
    prev_dev, new_dev = to_device(prev), to_device(new)
    _say(f"case {name} full size B={prev.B} H={prev.H}")
    S_bf, S_f = _bf16_state(prev, prev_dev)
    _, _, (S_out, out, vt, gm) = _run(prev, prev_dev, new, new_dev, S_bf, S_f)
    torch.cuda.synchronize()
    bs, hs, Sa, w1 = _oracle(prev, new, sample_pairs(prev.B, prev.H, 24, seed=113))
    bsi, hsi = torch.as_tensor(bs, device="cuda"), torch.as_tensor(hs, device="cuda")
    _err("full size: stored state", S_out[bsi, hsi].float().cpu().numpy(), Sa, S16_TOL)
    _err("full size: out", out[bsi, :, hsi].cpu().numpy(), w1.out, TOL)
    _err("full size: vtilde", vt[bsi, hsi].cpu().numpy(), w1.vtilde, TOL)
