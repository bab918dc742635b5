"""Host-side helpers pinned against numbers the pages print (see the golden
file's _source) and against the tree layout rules."""
import json
import os

import numpy as np
import pytest

from gated_deltanet_tree_03_amd import accounting as acc
from gated_deltanet_tree_03_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "memory_accounting.json")))


def test_kv_and_state_sizes_match_pages():
    for name, m in (("35B", acc.SCALE_35B), ("397B", acc.SCALE_397B)):
        assert acc.kv_bytes_per_token(m) == GOLD["kv_per_token_KiB"][name] * acc.KiB
        per_seq = acc.kv_bytes_per_token(m) * 32768 / acc.GiB
        assert per_seq == pytest.approx(GOLD["kv_per_seq_GiB_at_32K"][name], abs=0.005)
        assert acc.gdn_state_bytes_per_seq(m) == GOLD["gdn_state_per_seq_MiB"][name] * acc.MiB
        blocks = acc.snapshot_blocks_per_request(len(synth.chain(4)))
        assert blocks * acc.gdn_state_bytes_per_seq(m) == GOLD["snapshot_k3_per_seq_MiB"][name] * acc.MiB


def test_block_counts_match_pages():
    for key, want in GOLD["storeall_blocks_by_widths"].items():
        widths = tuple(int(x) for x in key.split(","))
        n = len(synth.tree_from_widths(widths))
        assert acc.snapshot_blocks_per_request(n) == want
        assert acc.store_all_buffer_blocks(n) == want + 1
        assert acc.treewy_state_blocks(n) == GOLD["treewy_blocks"]
    assert acc.state_block_bytes() // acc.pseudo_value_bytes(1) == GOLD["pseudo_value_smaller_by"]


@pytest.mark.parametrize("widths,n", [((1, 1, 1), 4), ((2, 2, 2), 15), ((3, 3, 3), 40), ((2,), 3), ((1, 3), 5)])
def test_tree_from_widths_counts_and_preorder(widths, n):
    p = synth.tree_from_widths(widths)
    assert len(p) == n == 1 + sum(int(np.prod(widths[: i + 1])) for i in range(len(widths)))
    assert p[0] == -1 and all(0 <= p[t] < t for t in range(1, n))
    # pre-order: each node's parent lies on the root-to-previous-node path
    path = [0]
    for t in range(1, n):
        assert p[t] in path
        path = path[: path.index(p[t]) + 1] + [t]
    d = synth.node_depths(p)
    assert d.max() == len(widths)
    assert np.all(np.bincount(d) == [1] + [int(np.prod(widths[: i + 1])) for i in range(len(widths))])


def test_chain_layout():
    assert synth.chain(4).tolist() == [-1, 0, 1, 2] == synth.tree_from_widths((1, 1, 1)).tolist()


def test_random_preorder_tree_is_preorder(rng):
    for n in (1, 2, 10, 64):
        p = synth.random_preorder_tree(n, rng)
        path = [0]
        for t in range(1, n):
            assert p[t] in path
            path = path[: path.index(p[t]) + 1] + [t]
        capped = synth.random_preorder_tree(n, rng, max_depth=3)
        assert synth.node_depths(capped).max() <= 3


def test_bf16_rounding_is_rne():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 10
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]  # ties both ways
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(synth.round_bf16(x), want)


def test_inputs_are_seeded_and_shaped():
    a = synth.make_inputs("35b-tree222", B=2, H=3)
    b = synth.make_inputs("35b-tree222", B=2, H=3)
    assert a.q.shape == (2, 15, 3, 128) and a.alpha.shape == (2, 15, 3) and a.S0.shape == (2, 3, 128, 128)
    for name in ("S0", "q", "k", "v", "alpha", "beta", "accepted"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert np.all((a.alpha > 0) & (a.alpha <= 1)) and np.all((a.beta > 0) & (a.beta < 1))
    assert np.allclose(np.linalg.norm(a.k, axis=-1), 1, atol=2e-2)
    assert np.array_equal(synth.round_bf16(a.q), a.q)
    wide = synth.make_inputs("wide-tree333", B=4, H=2)
    assert np.all(wide.alpha >= 0.9) and np.all(wide.alpha <= 1.0)
    d = synth.node_depths(wide.parent)
    assert np.all(d[wide.accepted] == 3)
    small = synth.make_inputs("chain4-f32")
    assert small.S0 is None and small.warmup["q"].shape == (1, 32, 4, 128) and small.q.dtype == np.float32
