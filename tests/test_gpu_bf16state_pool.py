"""GPU parity of the bf16-state pool forms, through the C ABI:

* treewy_commit_verify_bf16state_pool against treewy_commit_verify_bf16state
  on the same states: every committed block, output, pseudo-value and gate
  bit for bit (the same arithmetic; only the block addressing differs), on
  random trees of 1..64 nodes and the five workload shapes;
* its per-sequence cases: accepted_prev < 0 leaves the block as it is and
  verifies from it; an accepted index past the previous tree gives a NaN
  block and NaN outputs; a slot outside the pool writes nothing and gives
  NaN outputs; blocks no sequence names are never written;
* treewy_commit_verify_bf16state_pool_trees with one tree shared by every
  request against the pool form, bit for bit; with a tree per request,
  against the fp64 oracle walking each request from its stored bf16 state
  (the stored state within 2^-8 of the largest element of the oracle's
  committed state, the one bf16 rounding of the stored value; outputs and
  pseudo-values within 2e-3 of the oracle verifying from the stored state);
* the full-size 35B-like (2,2,2) tree batch on sampled heads.
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

STATE_TOL = 2.0 ** -8  # one bf16 rounding of the stored state
TIGHT = 1e-5  # two kernels, the same arithmetic up to summation order


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(abi.LIB_PATH):
        pytest.fail("libtreewy.so is not built")
    torch.cuda.set_device(0)
    yield


def _steps(cfg, B, H, seed, p_prev, p_new):
    rng = np.random.default_rng(seed)
    prev = synth.make_inputs(cfg, B=B, H=H, seed=seed, parent=p_prev)
    prev.accepted = rng.integers(0, len(p_prev), size=B).astype(np.int32)
    new = synth.make_inputs(cfg, B=B, H=H, seed=seed + 1, parent=p_new)
    pd, nd = to_device(prev), to_device(new)
    pd["accepted"] = torch.from_numpy(prev.accepted).cuda()
    return rng, prev, new, pd, nd


def _pool_case(label, cfg, p_prev, p_new, seed, B=3, H=4):
    rng, prev, new, pd, nd = _steps(cfg, B, H, seed, p_prev, p_new)
    S16 = pd["S0"].to(torch.bfloat16)
    _, vt0, gm0 = abi.verify(S16.float(), pd["q"], pd["k"], pd["v"], pd["alpha"], pd["beta"], p_prev)
    args = (vt0, pd["k"], gm0, pd["accepted"], p_prev, nd["q"], nd["k"], nd["v"], nd["alpha"],
            nd["beta"], p_new)
    S_b, out_b, vt_b, gm_b = abi.commit_verify_bf16state(S16.clone(), *args)
    n_pool = B + 3
    slot_list = rng.permutation(n_pool)[:B]
    slots = torch.tensor(slot_list, dtype=torch.int32, device="cuda")
    pool = torch.zeros((n_pool, H, 128, 128), dtype=torch.bfloat16, device="cuda")
    pool[slots.long()] = S16
    out_p, vt_p, gm_p = abi.commit_verify_pool(pool, slots, *args)
    torch.cuda.synchronize()
    print(f"case {label}: N_prev={len(p_prev)} N={len(p_new)}", flush=True)
    assert torch.equal(pool[slots.long()], S_b), f"{label}: pooled state != batch form"
    assert torch.equal(out_p, out_b) and torch.equal(vt_p, vt_b) and torch.equal(gm_p, gm_b), label
    spare = [i for i in range(n_pool) if i not in set(slot_list.tolist())]
    assert not pool[spare].float().any(), f"{label}: a block no sequence names was written"


@pytest.mark.parametrize("n", [1, 4, 9, 15, 24, 40, 57, 64])
def test_pool_equals_batch_random_trees(n):
    rng = np.random.default_rng(7000 + n)
    p_prev = synth.random_preorder_tree(int(rng.integers(1, 65)), rng)
    p_new = synth.random_preorder_tree(n, rng)
    _pool_case(f"random n={n}", "35b-tree222", p_prev, p_new, 710 + n)


@pytest.mark.parametrize("name", ["35b-chain4", "35b-tree222", "wide-tree333"])
def test_pool_equals_batch_workload_shapes(name):
    p = synth.CONFIGS[name].parent
    _pool_case(name, name, p, p, 730, B=4, H=4)


def test_pool_no_previous_step_bad_accepted_and_bad_slot():
    B, H = 4, 3
    p = synth.tree_from_widths((2, 2, 2))
    rng, prev, new, pd, nd = _steps("35b-tree222", B, H, 741, p, p)
    S16 = pd["S0"].to(torch.bfloat16)
    _, vt0, gm0 = abi.verify(S16.float(), pd["q"], pd["k"], pd["v"], pd["alpha"], pd["beta"], p)
    acc = pd["accepted"].clone()
    acc[1] = -1                                        # request 1: no previous step
    acc[3] = len(p)                                    # request 3: accepted index out of range
    slots = torch.tensor([2, 0, 9, 4], dtype=torch.int32, device="cuda")  # request 2: outside
    pool = torch.zeros((6, H, 128, 128), dtype=torch.bfloat16, device="cuda")
    for b, s in ((0, 2), (1, 0), (3, 4)):
        pool[s] = S16[b]
    before = pool.clone()
    print(f"case slots={slots.tolist()} accepted_prev={acc.tolist()}", flush=True)
    out, vt, gm = abi.commit_verify_pool(pool, slots, vt0, pd["k"], gm0, acc, p, nd["q"], nd["k"],
                                         nd["v"], nd["alpha"], nd["beta"], p)
    # request 0: an ordinary commit, against the batch form bit for bit
    S_b, out_b, vt_b, _ = abi.commit_verify_bf16state(S16.clone(), vt0, pd["k"], gm0, pd["accepted"],
                                                      p, nd["q"], nd["k"], nd["v"], nd["alpha"],
                                                      nd["beta"], p)
    # request 1: verified from its block as it is
    # (clones: a slice of request 1 starts at an offset the library rejects as misaligned)
    o1, v1, _ = abi.verify(S16[1:2].float(), *(nd[n][1:2].clone()
                                               for n in ("q", "k", "v", "alpha", "beta")), p)
    torch.cuda.synchronize()
    assert torch.equal(pool[2], S_b[0]) and torch.equal(out[0], out_b[0])
    assert torch.equal(vt[0], vt_b[0])
    assert torch.equal(pool[0], before[0]), "no previous step: the block must stay as it is"
    assert rel_err(out[1].cpu().numpy(), o1[0].cpu().numpy()) <= TIGHT
    assert rel_err(vt[1].cpu().numpy(), v1[0].cpu().numpy()) <= TIGHT
    assert torch.isnan(out[2]).all() and torch.isnan(vt[2]).all(), "a bad slot gives NaN outputs"
    assert torch.isnan(pool[4].float()).all(), "a bad accepted index gives a NaN block"
    assert torch.isnan(out[3]).all() and torch.isnan(vt[3]).all()
    assert torch.equal(pool[[1, 3, 5]], before[[1, 3, 5]]), "a block no sequence names was written"


def _descs(parents):
    host, n_max, depth = abi.pack_trees(parents)
    return torch.from_numpy(host.copy()).cuda(), n_max, depth


def test_pool_trees_shared_tree_equals_pool():
    B, H = 4, 4
    p = synth.tree_from_widths((3, 3, 3))
    rng, prev, new, pd, nd = _steps("wide-tree333", B, H, 751, p, p)
    S16 = pd["S0"].to(torch.bfloat16)
    _, vt0, gm0 = abi.verify(S16.float(), pd["q"], pd["k"], pd["v"], pd["alpha"], pd["beta"], p)
    slots = torch.tensor([3, 1, 0, 5], dtype=torch.int32, device="cuda")
    pools = []
    for _ in range(2):
        pool = torch.zeros((6, H, 128, 128), dtype=torch.bfloat16, device="cuda")
        pool[slots.long()] = S16
        pools.append(pool)
    out_p, vt_p, gm_p = abi.commit_verify_pool(pools[0], slots, vt0, pd["k"], gm0, pd["accepted"], p,
                                               nd["q"], nd["k"], nd["v"], nd["alpha"], nd["beta"], p)
    t, _, d = _descs([p] * B)
    out_t, vt_t, gm_t = abi.commit_verify_pool_trees(pools[1], slots, vt0, pd["k"], gm0,
                                                     pd["accepted"], t, d, nd["q"], nd["k"], nd["v"],
                                                     nd["alpha"], nd["beta"], t, d)
    torch.cuda.synchronize()
    assert torch.equal(pools[0], pools[1])
    assert torch.equal(out_p, out_t) and torch.equal(vt_p, vt_t) and torch.equal(gm_p, gm_t)


@pytest.mark.parametrize("seed", [761, 762])
def test_pool_trees_mixed_trees_against_oracle(seed):
    B, H = 5, 3
    rng = np.random.default_rng(seed)
    p1 = [synth.random_preorder_tree(int(n), rng, max_depth=3) for n in rng.integers(1, 41, size=B)]
    p2 = [synth.random_preorder_tree(int(n), rng, max_depth=3) for n in rng.integers(1, 41, size=B)]
    t1, N1, d1 = _descs(p1)
    t2, N2, d2 = _descs(p2)
    in1 = synth.make_inputs("wide-tree333", B=B, H=H, seed=seed, parent=synth.chain(N1))
    in2 = synth.make_inputs("wide-tree333", B=B, H=H, seed=seed + 100, parent=synth.chain(N2))
    dv1, dv2 = to_device(in1), to_device(in2)
    S16 = dv1["S0"].to(torch.bfloat16)
    S_start = S16.float().cpu().numpy().astype(np.float64)
    slots = torch.tensor(rng.permutation(B + 2)[:B], dtype=torch.int32, device="cuda")
    pool = torch.zeros((B + 2, H, 128, 128), dtype=torch.bfloat16, device="cuda")
    pool[slots.long()] = S16
    # step 1: no previous step (a one-node previous tree that is never read)
    t0, _, _ = _descs([np.array([-1], dtype=np.int32)] * B)
    none = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    vt0 = torch.zeros((B, H, 1, 128), device="cuda")
    gm0 = torch.ones((B, H, 1), device="cuda")
    out1, vt1, gm1 = abi.commit_verify_pool_trees(pool, slots, vt0, dv1["k"][:, :1].contiguous(),
                                                  gm0, none, t0, 0, dv1["q"], dv1["k"], dv1["v"],
                                                  dv1["alpha"], dv1["beta"], t1, d1)
    acc = np.array([rng.integers(0, len(p)) for p in p1], dtype=np.int32)
    out2, vt2, gm2 = abi.commit_verify_pool_trees(pool, slots, vt1, dv1["k"], gm1,
                                                  torch.from_numpy(acc).cuda(), t1, d1, dv2["q"],
                                                  dv2["k"], dv2["v"], dv2["alpha"], dv2["beta"], t2, d2)
    torch.cuda.synchronize()
    stored = pool[slots.long()].float().cpu().numpy().astype(np.float64)
    f = lambda x: np.asarray(x, dtype=np.float64)
    errs = {"state": 0.0, "out1": 0.0, "vt1": 0.0, "out2": 0.0, "vt2": 0.0}
    for b in range(B):
        n1, n2 = len(p1[b]), len(p2[b])
        for h in range(H):
            w1 = oracle.walk(S_start[b, h][None], f(in1.q[b, :n1, h])[None], f(in1.k[b, :n1, h])[None],
                             f(in1.v[b, :n1, h])[None], f(in1.alpha[b, :n1, h])[None],
                             f(in1.beta[b, :n1, h])[None], p1[b])
            Sa = w1.states[0, acc[b]]
            errs["state"] = max(errs["state"], rel_err(stored[b, h], Sa))
            w2 = oracle.walk(stored[b, h][None], f(in2.q[b, :n2, h])[None], f(in2.k[b, :n2, h])[None],
                             f(in2.v[b, :n2, h])[None], f(in2.alpha[b, :n2, h])[None],
                             f(in2.beta[b, :n2, h])[None], p2[b])
            errs["out1"] = max(errs["out1"], rel_err(out1[b, :n1, h].cpu().numpy(), w1.out[0]))
            errs["vt1"] = max(errs["vt1"], rel_err(vt1[b, h, :n1].cpu().numpy(), w1.vtilde[0]))
            errs["out2"] = max(errs["out2"], rel_err(out2[b, :n2, h].cpu().numpy(), w2.out[0]))
            errs["vt2"] = max(errs["vt2"], rel_err(vt2[b, h, :n2].cpu().numpy(), w2.vtilde[0]))
    print(f"mixed trees seed {seed}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert errs["state"] <= STATE_TOL
    for k in ("out1", "vt1", "out2", "vt2"):
        assert errs[k] <= TOL, k


def test_pool_full_size_sampled():
    name = "35b-tree222"
    inp = synth.make_inputs(name)
    d = to_device(inp)
    B, H, N = inp.B, inp.H, inp.N
    p = inp.parent
    S16 = d["S0"].to(torch.bfloat16)
    _, vt0, gm0 = abi.verify(S16.float(), d["q"], d["k"], d["v"], d["alpha"], d["beta"], p)
    nxt = synth.make_inputs(name, seed=synth.CONFIGS[name].seed + 500)
    nd = {n: torch.from_numpy(np.ascontiguousarray(nxt.bits[n]).view(np.int16)).cuda()
          .view(torch.bfloat16) for n in ("q", "k", "v", "alpha", "beta")}
    slots = torch.from_numpy(np.random.default_rng(3).permutation(2 * B)[:B].astype(np.int32)).cuda()
    pool = torch.zeros((2 * B, H, 128, 128), dtype=torch.bfloat16, device="cuda")
    pool[slots.long()] = S16
    out, vt, gm = abi.commit_verify_pool(pool, slots, vt0, d["k"], gm0, d["accepted"], p, nd["q"],
                                         nd["k"], nd["v"], nd["alpha"], nd["beta"], p)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    pairs = [(int(i // H), int(i % H)) for i in rng.choice(B * H, size=24, replace=False)]
    S_start = S16.float().cpu().numpy().astype(np.float64)
    stored = pool[slots.long()].float().cpu().numpy().astype(np.float64)
    e = {"state": 0.0, "out": 0.0, "vt": 0.0}
    for b, h in pairs:
        f = lambda inp_, x: x[b, :, h].astype(np.float64)[None]
        w1 = oracle.walk(S_start[b, h][None], f(inp, inp.q), f(inp, inp.k), f(inp, inp.v),
                         f(inp, inp.alpha), f(inp, inp.beta), p)
        e["state"] = max(e["state"], rel_err(stored[b, h], w1.states[0, inp.accepted[b]]))
        w2 = oracle.walk(stored[b, h][None], f(nxt, nxt.q), f(nxt, nxt.k), f(nxt, nxt.v),
                         f(nxt, nxt.alpha), f(nxt, nxt.beta), p)
        e["out"] = max(e["out"], rel_err(out[b, :, h].cpu().numpy(), w2.out[0]))
        e["vt"] = max(e["vt"], rel_err(vt[b, h].cpu().numpy(), w2.vtilde[0]))
    print(f"{name} full size bf16 pool: " + " ".join(f"{k}={v:.2e}" for k, v in e.items()), flush=True)
    assert e["state"] <= STATE_TOL and e["out"] <= TOL and e["vt"] <= TOL
