"""fp64 CPU oracle for TreeWY verify / commit / store_all through one Gated
DeltaNet layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
bench's ``cpu_baseline`` leg may import this module.  It shares no code with the
HIP library (no kernels, headers, tables or helpers) and never imports it.  It
is plain and slow on purpose: every step is the definition written out, with
numpy's matmul / dense solve as the only library primitives.

Sources (all from "TreeWY: Speculative Verification for Gated DeltaNet
Hybrids"):
* paperpeel page, section 3 "Method: TreeWY", the "Key rewrite" paragraph: the
  gated delta rule written as decayed additive attention,
  ``S_t = alpha_t S_{t-1} + vt_t k_t^T`` with pseudo-value
  ``vt_t = beta_t (v_t - alpha_t S_{t-1} k_t)``.  Equation (1) itself is not
  printed; the reading used is the gated delta rule of the Gated Delta Networks
  paper (reference [4] there): ``S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T)
  + beta_t v_t k_t^T``, which expands to exactly the printed form.
* the same page, section 2 (paragraph after the prior-work list) and the
  abstract on the mlsanity page: one triangular solve yields every node's
  pseudo-value; only the accepted state is rebuilt on commit; the tree form is
  the strict-ancestor generalisation of DeltaNet's chain WY transform
  (reference [13] there).
* review page, "Method": nodes are laid out in DFS pre-order so that ancestors
  precede descendants and the system is lower triangular.
* paperpeel section 2, first bullet pair: full-state snapshotting keeps one
  state per draft position and rolls back by indexing ("store_all").

Readings taken where the pages are silent (each also listed in the design
notes): the output is ``o_t = S_t q_t`` with the post-update state and no
scale; node 0 is the root (last accepted token, update not yet in S0) so
``Gamma_0 = alpha_0``; the path gate is inclusive, ``Gamma_t = alpha_t
Gamma_{parent(t)}``.

Array layout (one row per (sequence, head) pair, ``G`` rows):
``S0 [G, dv, dk]``, ``q, k [G, N, dk]``, ``v [G, N, dv]``,
``alpha, beta [G, N]``, ``parent [N]`` (``parent[0] == -1``, ``parent[t] < t``).
Any topological order is accepted here; the DFS pre-order requirement belongs
to the fast path, not to the definition.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

__all__ = [
    "ancestors", "path_of", "walk", "closed_form", "commit", "chain_wy",
    "store_all", "gamma_scan", "WalkResult", "ClosedFormResult",
]


# --------------------------------------------------------------------------
# Tree bookkeeping (sets of nodes, not bitmasks)
# --------------------------------------------------------------------------

def _check_parent(parent: Sequence[int]) -> np.ndarray:
    parent = np.asarray(parent, dtype=np.int64)
    if parent.ndim != 1 or len(parent) == 0:
        raise ValueError("parent must be a non-empty 1-D array")
    if parent[0] != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    for t in range(1, len(parent)):
        if not (0 <= parent[t] < t):
            raise ValueError(f"parent[{t}]={parent[t]} must lie in [0, {t})")
    return parent


def ancestors(parent: Sequence[int]) -> List[List[int]]:
    """Strict ancestors of each node, ordered root first, found by following
    parent pointers upward."""
    parent = _check_parent(parent)
    result = []
    for t in range(len(parent)):
        chain_up = []
        j = parent[t]
        while j >= 0:
            chain_up.append(int(j))
            j = parent[j]
        result.append(chain_up[::-1])
    return result


def path_of(parent: Sequence[int], t: int) -> List[int]:
    """Ancestor-or-self set of node t, root first."""
    return ancestors(parent)[t] + [int(t)]


def _f64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


# --------------------------------------------------------------------------
# 1. The definition: walk the recurrence node by node
# --------------------------------------------------------------------------

@dataclass
class WalkResult:
    out: np.ndarray      # [G, N, dv]   o_t = S_t q_t
    vtilde: np.ndarray   # [G, N, dv]   pseudo-values
    states: np.ndarray   # [G, N, dv, dk]  S_t after node t


def walk(S0, q, k, v, alpha, beta, parent) -> WalkResult:
    """Run the gated delta rule along every root-to-node path.

    For t in index order (a parent always precedes its children):
        S_p  = S0 if t is the root else S_{parent(t)}
        vt_t = beta_t * (v_t - alpha_t * S_p k_t)
        S_t  = alpha_t * S_p + vt_t k_t^T
        o_t  = S_t q_t
    """
    parent = _check_parent(parent)
    S0, q, k, v, alpha, beta = _f64(S0, q, k, v, alpha, beta)
    G, N = alpha.shape
    dv, dk = S0.shape[1], S0.shape[2]
    states = np.empty((G, N, dv, dk))
    out = np.empty((G, N, dv))
    vt = np.empty((G, N, dv))
    for t in range(N):
        Sp = S0 if parent[t] < 0 else states[:, parent[t]]
        a = alpha[:, t][:, None]
        b = beta[:, t][:, None]
        Sp_k = np.einsum("gvk,gk->gv", Sp, k[:, t])
        vt[:, t] = b * (v[:, t] - a * Sp_k)
        states[:, t] = a[:, :, None] * Sp + vt[:, t][:, :, None] * k[:, t][:, None, :]
        out[:, t] = np.einsum("gvk,gk->gv", states[:, t], q[:, t])
    return WalkResult(out, vt, states)


def store_all(S0, q, k, v, alpha, beta, parent):
    """Full-state snapshotting: the walk's outputs plus the snapshot list
    ``[S0, S_0, ..., S_{N-1}]`` (N+1 blocks).  Rolling back to node ``a`` is
    indexing snapshot ``a+1``."""
    w = walk(S0, q, k, v, alpha, beta, parent)
    S0 = np.asarray(S0, dtype=np.float64)
    snaps = np.concatenate([S0[:, None], w.states], axis=1)
    return w.out, snaps


# --------------------------------------------------------------------------
# 2. The closed form: one triangular solve over the tree
# --------------------------------------------------------------------------

@dataclass
class ClosedFormResult:
    out: np.ndarray      # [G, N, dv]
    vtilde: np.ndarray   # [G, N, dv]
    gamma: np.ndarray    # [G, N]


def gamma_scan(alpha, parent) -> np.ndarray:
    """Cumulative path gate: Gamma_t = alpha_t * Gamma_{parent(t)}, with the
    empty product 1 above the root."""
    parent = _check_parent(parent)
    (alpha,) = _f64(alpha)
    G, N = alpha.shape
    gam = np.empty((G, N))
    for t in range(N):
        above = 1.0 if parent[t] < 0 else gam[:, parent[t]]
        gam[:, t] = alpha[:, t] * above
    return gam


def decay(gam, t, j):
    """Decay weight from node j down to its descendant-or-self t: Gamma_t / Gamma_j."""
    return gam[:, t] / gam[:, j]


def build_system(S0, k, v, beta, gam, anc):
    """(I + A) Vt = B with, for j a strict ancestor of t,
        A[t, j] = beta_t * Gamma_t / Gamma_j * (k_t . k_j)
    and zero elsewhere, and
        B[t]    = beta_t * (v_t - Gamma_t * S0 k_t).
    """
    G, N, _ = k.shape
    A = np.zeros((G, N, N))
    for t in range(N):
        for j in anc[t]:
            A[:, t, j] = beta[:, t] * decay(gam, t, j) * np.einsum("gd,gd->g", k[:, t], k[:, j])
    S0_k = np.einsum("gvk,gnk->gnv", S0, k)
    Bm = beta[:, :, None] * (v - gam[:, :, None] * S0_k)
    return A, Bm


def solve_pseudo_values(A, Bm):
    """Dense library solve of (I + A) Vt = B (I + A is unit lower triangular in
    any topological node order, so the solution is unique)."""
    G, N, _ = A.shape
    return np.linalg.solve(np.eye(N)[None] + A, Bm)


def outputs(S0, q, k, vt, gam, parent_paths):
    """o_t = Gamma_t S0 q_t + sum over j ancestor-or-self of t of
    (Gamma_t / Gamma_j) (k_j . q_t) vt_j."""
    G, N, _ = q.shape
    S0_q = np.einsum("gvk,gnk->gnv", S0, q)
    out = gam[:, :, None] * S0_q
    for t in range(N):
        for j in parent_paths[t]:
            coef = decay(gam, t, j) * np.einsum("gd,gd->g", k[:, j], q[:, t])
            out[:, t] += coef[:, None] * vt[:, j]
    return out


def closed_form(S0, q, k, v, alpha, beta, parent) -> ClosedFormResult:
    """Every node's pseudo-value from one triangular solve, then every output
    as a decay-weighted sum over its ancestor-or-self set."""
    parent = _check_parent(parent)
    S0, q, k, v, alpha, beta = _f64(S0, q, k, v, alpha, beta)
    anc = ancestors(parent)
    paths = [a + [t] for t, a in enumerate(anc)]
    gam = gamma_scan(alpha, parent)
    A, Bm = build_system(S0, k, v, beta, gam, anc)
    vt = solve_pseudo_values(A, Bm)
    out = outputs(S0, q, k, vt, gam, paths)
    return ClosedFormResult(out, vt, gam)


def commit(S0, vtilde, k, gamma, parent, accepted):
    """Rebuild the accepted state only:
        S_a = Gamma_a S0 + sum over j ancestor-or-self of a of
              (Gamma_a / Gamma_j) vt_j k_j^T.
    ``accepted`` holds one node index per row of the batch ([G])."""
    parent = _check_parent(parent)
    S0, vtilde, k, gamma = _f64(S0, vtilde, k, gamma)
    accepted = np.asarray(accepted, dtype=np.int64)
    G = S0.shape[0]
    anc = ancestors(parent)
    S_out = np.empty_like(S0)
    for g in range(G):
        a = int(accepted[g])
        Sa = gamma[g, a] * S0[g]
        for j in anc[a] + [a]:
            Sa = Sa + (gamma[g, a] / gamma[g, j]) * np.outer(vtilde[g, j], k[g, j])
        S_out[g] = Sa
    return S_out


# --------------------------------------------------------------------------
# 3. Chain WY / UT form (DeltaNet's chunk transform with gating)
# --------------------------------------------------------------------------

def chain_wy(S0, q, k, v, alpha, beta):
    """Chain-only cross-check in the chunked WY/UT form of DeltaNet with
    per-token decay (the Gated DeltaNet chunk form).  For a chain every earlier
    token is an ancestor, so the mask is the full strictly-lower triangle:

        g_t   = prod_{i<=t} alpha_i             (np.cumprod)
        L     = strictly-lower( diag(beta) (D * K K^T) ),  D[t,j] = g_t / g_j
        T     = (I + L)^{-1} diag(beta)          (the UT transform)
        U     = T V,   W = T diag(g) K           (the WY factors)
        Vt    = U - W S0^T
        O     = diag(g) Q S0^T + lower-incl( D * Q K^T ) Vt
        S_end = g_N S0 + sum_t (g_N / g_t) vt_t k_t^T

    Returns (out [G,N,dv], vtilde [G,N,dv], S_end [G,dv,dk]).
    """
    S0, q, k, v, alpha, beta = _f64(S0, q, k, v, alpha, beta)
    G, N = alpha.shape
    g = np.cumprod(alpha, axis=1)                        # [G, N]
    D = g[:, :, None] / g[:, None, :]                    # [G, N, N]
    strict = np.tril(np.ones((N, N)), -1)[None]
    incl = np.tril(np.ones((N, N)), 0)[None]
    KK = np.matmul(k, np.swapaxes(k, 1, 2))
    QK = np.matmul(q, np.swapaxes(k, 1, 2))
    L = beta[:, :, None] * D * KK * strict
    T = np.matmul(np.linalg.inv(np.eye(N)[None] + L), beta[:, :, None] * np.eye(N)[None])
    U = np.matmul(T, v)
    W = np.matmul(T, g[:, :, None] * k)
    S0T = np.swapaxes(S0, 1, 2)
    vt = U - np.matmul(W, S0T)
    out = g[:, :, None] * np.matmul(q, S0T) + np.matmul(D * QK * incl, vt)
    wN = g[:, -1][:, None] / g                           # g_N / g_t
    S_end = g[:, -1][:, None, None] * S0 + np.einsum("gt,gtv,gtk->gvk", wN, vt, k)
    return out, vt, S_end
