"""Seeded synthetic inputs and draft-tree topologies.

This module draws random numbers and builds tree topologies; it contains none
of the gated-delta arithmetic.  Both the HIP path's tests/bench and the CPU
oracle's tests consume what it produces.

Source for the workload shapes: "TreeWY: Speculative Verification for Gated
DeltaNet Hybrids" (paperpeel page), section 2 "The memory problem" (two hybrid
scales with d_k = d_v = 128 and 32 / 64 value heads) and section 4
"Implementation" (draft trees given by a branching factor per level, laid out in
DFS pre-order as section "Method" of the review page describes).

Conventions
-----------
* Node 0 is the root: the last accepted token, whose state update is not yet in
  the committed state ``S0``.  ``parent[0] == -1`` and ``0 <= parent[t] < t``.
* Device layout (row-major):  ``S0 [B,H,dv,dk]`` fp32;  ``q,k [B,N,H,dk]``;
  ``v [B,N,H,dv]``;  ``alpha,beta [B,N,H]``;  ``accepted [B]`` int32.
* bf16 tensors are produced as fp32 values that are exactly representable in
  bf16 (round-to-nearest-even from the fp32 draw) plus their raw uint16 bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

D_HEAD = 128

# --------------------------------------------------------------------------
# Tree topologies
# --------------------------------------------------------------------------


def tree_from_widths(widths: Sequence[int]) -> np.ndarray:
    """Parent array of a full draft tree with ``widths[l]`` children per node at
    level ``l``, in DFS pre-order with children in creation order.

    ``(1,1,1)`` is the chain of three drafts after the root (4 nodes);
    ``(2,2,2)`` has 1+2+4+8 = 15 nodes and ``(3,3,3)`` 1+3+9+27 = 40.
    """
    widths = [int(w) for w in widths]
    if any(w < 1 for w in widths):
        raise ValueError(f"widths must be >= 1, got {widths}")
    parents: List[int] = [-1]

    def grow(node: int, level: int) -> None:
        if level == len(widths):
            return
        for _ in range(widths[level]):
            child = len(parents)
            parents.append(node)
            grow(child, level + 1)

    grow(0, 0)
    return np.asarray(parents, dtype=np.int32)


def chain(n_nodes: int) -> np.ndarray:
    """Parent array of a chain of ``n_nodes`` nodes (root + n_nodes-1 drafts)."""
    if n_nodes < 1:
        raise ValueError("a chain needs at least the root node")
    return np.arange(-1, n_nodes - 1, dtype=np.int32)


def random_preorder_tree(n_nodes: int, rng: np.random.Generator,
                         max_depth: Optional[int] = None) -> np.ndarray:
    """A random tree in DFS pre-order: node t's parent is drawn uniformly from the
    root-to-(t-1) path, which is exactly the set of parents a pre-order allows.
    ``max_depth`` (root = depth 0) caps the depth of every node."""
    parents = [-1]
    depth = [0]
    path = [0]  # root-to-(t-1) path
    for t in range(1, n_nodes):
        choices = path if max_depth is None else [p for p in path if depth[p] < max_depth]
        p = int(choices[rng.integers(0, len(choices))])
        parents.append(p)
        depth.append(depth[p] + 1)
        path = path[: path.index(p) + 1] + [t]
    return np.asarray(parents, dtype=np.int32)


def node_depths(parent: np.ndarray) -> np.ndarray:
    """Depth of every node (root = 0) for a topologically ordered parent array."""
    depth = np.zeros(len(parent), dtype=np.int32)
    for t in range(1, len(parent)):
        depth[t] = depth[parent[t]] + 1
    return depth


def leaves(parent: np.ndarray) -> np.ndarray:
    has_child = np.zeros(len(parent), dtype=bool)
    has_child[parent[parent >= 0]] = True
    return np.nonzero(~has_child)[0].astype(np.int32)


# --------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even), numpy only
# --------------------------------------------------------------------------


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------
# Workload configurations
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    widths: Tuple[int, ...]
    dtype: str             # "f32" or "bf16" for q,k,v,alpha,beta
    seed: int
    alpha_dist: str = "softplus"   # "softplus": exp(-softplus(N(0,1))); "u90": U[0.9,1.0)
    s0_dist: str = "normal002"     # "normal002": N(0, 0.02^2); "warmup32": recurrence over 32 tokens
    accept_rule: str = "path"      # "path": uniform leaf then uniform depth; "deepest": uniform deepest node
    description: str = ""

    @property
    def parent(self) -> np.ndarray:
        return tree_from_widths(self.widths)

    @property
    def N(self) -> int:
        return int(len(self.parent))

    @property
    def heads(self) -> int:
        return self.B * self.H


CONFIGS: Dict[str, Config] = {
    "chain4-f32": Config("chain4-f32", 1, 4, (1, 1, 1), "f32", 101, s0_dist="warmup32",
                         description="chain k=3 (N=4), batch 1, 4 value heads, fp32 throughout, "
                                     "S0 from a 32-token recurrence from zero"),
    "35b-chain4": Config("35b-chain4", 256, 32, (1, 1, 1), "bf16", 102,
                         description="35B-like GDN layer, chain k=3 (N=4), batch 256, 32 value heads"),
    "35b-tree222": Config("35b-tree222", 128, 32, (2, 2, 2), "bf16", 103,
                          description="35B-like layer, tree (2,2,2) (N=15), batch 128, 32 value heads"),
    "397b-chain4": Config("397b-chain4", 128, 64, (1, 1, 1), "bf16", 104,
                          description="397B-like layer, chain k=3 (N=4), batch 128, 64 value heads"),
    "397b-tree222": Config("397b-tree222", 128, 64, (2, 2, 2), "bf16", 105,
                           description="397B-like layer, tree (2,2,2) (N=15), batch 128, 64 value heads"),
    "wide-tree333": Config("wide-tree333", 512, 32, (3, 3, 3), "bf16", 106, alpha_dist="u90", accept_rule="deepest",
                           description="wide-tree stress, tree (3,3,3) (N=40), batch 512, 32 value heads, "
                                       "alpha in [0.9,1.0)"),
}


@dataclass
class Inputs:
    """One batch of synthetic inputs in device layout.

    ``*_f32`` are the values the kernels see (bf16-exact for bf16 configs);
    ``*_bits`` are the raw bf16 patterns (None for fp32 configs).  For the
    ``warmup32`` S0 recipe, ``S0`` is None and ``warmup`` holds the 32 warm-up
    tokens; the committed state is the result of running them from zero.
    """
    cfg_name: str
    B: int
    H: int
    N: int
    dtype: str
    parent: np.ndarray
    S0: Optional[np.ndarray]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    accepted: np.ndarray
    bits: Dict[str, np.ndarray] = field(default_factory=dict)
    warmup: Optional[Dict[str, np.ndarray]] = None


def _unit_normal_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _alpha(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "softplus":
        x = rng.standard_normal(shape, dtype=np.float32)
        return np.exp(-np.logaddexp(np.float32(0), x)).astype(np.float32)
    if dist == "u90":
        u = rng.random(shape, dtype=np.float32)
        return (np.float32(0.9) + np.float32(0.1) * u).astype(np.float32)
    raise ValueError(dist)


def _beta(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return (np.float32(1) / (np.float32(1) + np.exp(-x))).astype(np.float32)


def _token_draws(rng, B, N, H, d, alpha_dist):
    q = _unit_normal_rows(rng, (B, N, H, d))
    k = _unit_normal_rows(rng, (B, N, H, d))
    v = rng.standard_normal((B, N, H, d), dtype=np.float32)
    a = _alpha(rng, (B, N, H), alpha_dist)
    b = _beta(rng, (B, N, H))
    return q, k, v, a, b


def choose_accepted(parent: np.ndarray, B: int, rule: str,
                    rng: np.random.Generator) -> np.ndarray:
    depth = node_depths(parent)
    lv = leaves(parent)
    out = np.empty(B, dtype=np.int32)
    if rule == "path":
        for b in range(B):
            leaf = int(lv[rng.integers(0, len(lv))])
            d = int(rng.integers(0, depth[leaf] + 1))
            node = leaf
            while depth[node] > d:
                node = int(parent[node])
            out[b] = node
        return out
    if rule == "deepest":
        deepest = np.nonzero(depth == depth.max())[0]
        return deepest[rng.integers(0, len(deepest), size=B)].astype(np.int32)
    raise ValueError(rule)


def make_inputs(cfg: Config | str, seed: Optional[int] = None, B: Optional[int] = None,
                H: Optional[int] = None, parent: Optional[np.ndarray] = None,
                dtype: Optional[str] = None) -> Inputs:
    """Draw one batch for ``cfg`` (overrides allowed for small test cases).

    Draw order, one PCG64 stream: S0 (or the 32 warm-up tokens) -> q -> k -> v
    -> alpha -> beta -> accepted.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.seed if seed is None else seed
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    dtype = cfg.dtype if dtype is None else dtype
    parent = cfg.parent if parent is None else np.asarray(parent, dtype=np.int32)
    N = len(parent)
    d = D_HEAD
    rng = np.random.Generator(np.random.PCG64(seed))

    warmup = None
    if cfg.s0_dist == "normal002":
        S0 = (rng.standard_normal((B, H, d, d), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    elif cfg.s0_dist == "warmup32":
        wq, wk, wv, wa, wb = _token_draws(rng, B, 32, H, d, cfg.alpha_dist)
        warmup = dict(q=wq, k=wk, v=wv, alpha=wa, beta=wb)
        S0 = None
    else:
        raise ValueError(cfg.s0_dist)

    q, k, v, a, b = _token_draws(rng, B, N, H, d, cfg.alpha_dist)
    accepted = choose_accepted(parent, B, cfg.accept_rule, rng)

    bits: Dict[str, np.ndarray] = {}
    if dtype == "bf16":
        for name, arr in (("q", q), ("k", k), ("v", v), ("alpha", a), ("beta", b)):
            bits[name] = bf16_bits(arr)
        q, k, v, a, b = (bf16_to_f32(bits[n]) for n in ("q", "k", "v", "alpha", "beta"))
    elif dtype != "f32":
        raise ValueError(dtype)

    return Inputs(cfg.name, B, H, N, dtype, parent, S0, q, k, v, a, b, accepted,
                  bits, warmup)
