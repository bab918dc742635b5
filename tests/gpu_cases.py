"""Shared helpers for the GPU parity tests: upload synthetic inputs, run the
library through its C ABI, and build oracle references for chosen
(sequence, head) pairs.  Not collected by pytest (no test_ prefix)."""
from __future__ import annotations

import numpy as np

import oracle
from gated_deltanet_tree_03_amd import abi, synth

TOL = 2e-3  # max |diff| / max |ref| per tensor, against the fp64 oracle


_FULL_CACHE = {}


def full_inputs(name: str) -> synth.Inputs:
    """Full-size inputs of a named workload, generated once per process."""
    if name not in _FULL_CACHE:
        _FULL_CACHE.clear()  # keep at most one large workload on the host
        _FULL_CACHE[name] = synth.make_inputs(name)
    return _FULL_CACHE[name]


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / den) if den > 0 else float(np.max(np.abs(got)))


def committed_state_from_warmup(inp: synth.Inputs) -> np.ndarray:
    """The warmup32 recipe: run the recurrence from a zero state over 32 tokens
    (a 32-node chain) with the oracle; returns fp32 S0 [B,H,128,128]."""
    w = inp.warmup
    B, T, H, d = w["q"].shape
    from conftest import to_heads
    _, q, k, v, a, b = to_heads(None, w["q"], w["k"], w["v"], w["alpha"], w["beta"])
    walk = oracle.walk(np.zeros((B * H, d, d)), q, k, v, a, b, synth.chain(T))
    return walk.states[:, -1].astype(np.float32).reshape(B, H, d, d)


def to_device(inp: synth.Inputs, device="cuda"):
    import torch
    dev = {}
    if inp.S0 is None:
        inp.S0 = committed_state_from_warmup(inp)
    dev["S0"] = torch.from_numpy(np.ascontiguousarray(inp.S0)).to(device)
    for name in ("q", "k", "v", "alpha", "beta"):
        if inp.dtype == "bf16":
            bits = np.ascontiguousarray(inp.bits[name]).view(np.int16)
            dev[name] = torch.from_numpy(bits).to(device).view(torch.bfloat16)
        else:
            dev[name] = torch.from_numpy(np.ascontiguousarray(getattr(inp, name))).to(device)
    dev["accepted"] = torch.from_numpy(inp.accepted.astype(np.int32)).to(device)
    return dev


def oracle_heads(inp: synth.Inputs, pairs):
    """Oracle results for the listed (b, h) pairs (fp64 walk = the definition):
    dict of out [G,N,128], vtilde [G,N,128], S_acc [G,128,128], states [G,N,128,128]."""
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    S0 = inp.S0[bs, hs].astype(np.float64)
    q = inp.q[bs, :, hs].astype(np.float64)
    k = inp.k[bs, :, hs].astype(np.float64)
    v = inp.v[bs, :, hs].astype(np.float64)
    a = inp.alpha[bs, :, hs].astype(np.float64)
    b = inp.beta[bs, :, hs].astype(np.float64)
    w = oracle.walk(S0, q, k, v, a, b, inp.parent)
    acc = inp.accepted[bs]
    S_acc = w.states[np.arange(len(pairs)), acc]
    gam = oracle.gamma_scan(a, inp.parent)
    return dict(out=w.out, vtilde=w.vtilde, S_acc=S_acc, states=w.states, gamma=gam, S0=S0)


def all_pairs(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def sample_pairs(B, H, n, seed=0):
    rng = np.random.default_rng(seed)
    idx = rng.choice(B * H, size=min(n, B * H), replace=False)
    pairs = [(int(i // H), int(i % H)) for i in sorted(idx)]
    # always include the first and last head of the batch
    for p in ((0, 0), (B - 1, H - 1)):
        if p not in pairs:
            pairs.append(p)
    return pairs


def gather_device(inp, out, vtilde, gamma, S_out, pairs):
    """Pull the listed (b,h) pairs of the device results into oracle layout."""
    bs = np.array([p[0] for p in pairs])
    hs = np.array([p[1] for p in pairs])
    import torch
    bsi = torch.as_tensor(bs, device=out.device)
    hsi = torch.as_tensor(hs, device=out.device)
    res = {}
    res["out"] = out[bsi, :, hsi].cpu().numpy()            # [G, N, 128]
    res["vtilde"] = vtilde[bsi, hsi].cpu().numpy()         # [G, N, 128]
    res["gamma"] = gamma[bsi, hsi].cpu().numpy()           # [G, N]
    if S_out is not None:
        res["S_out"] = S_out[bsi, hsi].cpu().numpy()       # [G, 128, 128]
    return res
