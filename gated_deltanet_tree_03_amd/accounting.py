"""Memory accounting for speculative verification of GDN state.

Source: "TreeWY: Speculative Verification for Gated DeltaNet Hybrids"
(paperpeel page), section 2 "The memory problem": the softmax KV cache per
token is 2 (K and V) x softmax layers x KV heads x head dim x bytes per element;
the GDN state per sequence is GDN layers x value heads x d_v x d_k x bytes per
element; full-state snapshotting keeps one block per verified token.  The review
page ("Key idea") notes the pseudo-value matrix is d_k times smaller than one
state per node.
"""
from __future__ import annotations

from dataclasses import dataclass

KiB, MiB, GiB = 1024, 1024 ** 2, 1024 ** 3


@dataclass(frozen=True)
class HybridShape:
    n_gdn: int
    n_vheads: int
    n_softmax: int
    n_kv_heads: int = 2
    d_head: int = 256
    d_k: int = 128
    d_v: int = 128


# the two hybrid scales of section 2 (3:1 GDN-to-softmax)
SCALE_35B = HybridShape(n_gdn=30, n_vheads=32, n_softmax=10)
SCALE_397B = HybridShape(n_gdn=45, n_vheads=64, n_softmax=15)


def kv_bytes_per_token(m: HybridShape, elem_bytes: int = 2) -> int:
    return 2 * m.n_softmax * m.n_kv_heads * m.d_head * elem_bytes


def gdn_state_bytes_per_seq(m: HybridShape, elem_bytes: int = 2) -> int:
    return m.n_gdn * m.n_vheads * m.d_v * m.d_k * elem_bytes


def state_block_bytes(d_v: int = 128, d_k: int = 128, elem_bytes: int = 4) -> int:
    """One (sequence, head) state block."""
    return d_v * d_k * elem_bytes


def snapshot_blocks_per_request(n_nodes: int) -> int:
    """Blocks held by full-state snapshotting when n_nodes tokens (root + drafts)
    are verified: one per verified token (k+1 for a chain of k drafts)."""
    return n_nodes


def store_all_buffer_blocks(n_nodes: int) -> int:
    """Blocks in this library's store_all snapshot buffer: S0 plus one state
    per node, i.e. N+1."""
    return n_nodes + 1


def treewy_state_blocks(n_nodes: int) -> int:
    """TreeWY keeps the committed state only, whatever the tree."""
    return 1


def pseudo_value_bytes(n_nodes: int, d_v: int = 128, elem_bytes: int = 4) -> int:
    """Transient pseudo-value matrix per (sequence, head) between verify and commit."""
    return n_nodes * d_v * elem_bytes
