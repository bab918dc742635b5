"""GPU parity of treewy_prefill_chain (chunked prefill of a chain through the
commit-then-verify kernels), through the C ABI, against the fp64 oracle
walking the whole chain token by token: every token's output and the final
state (2e-3).  Chunk sizes from 7 to 64 tokens, ragged last chunks, one
token, fp32 and bf16 inputs."""
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(abi.LIB_PATH):
        pytest.fail("libtreewy.so is not built")
    torch.cuda.set_device(0)
    yield


def _err(label, got, ref):
    e = rel_err(got, ref)
    print(f"{label}: {e:.2e}", flush=True)
    assert np.isfinite(e) and e <= TOL, f"{label}: rel err {e:.3e} > {TOL}"


# long chunks take the long-memory gates (alpha in [0.9, 1)) so that a chunk's
# gate product stays in the fp32 normal range
@pytest.mark.parametrize("T,chunk,cfg,dtype", [
    (1, 64, "wide-tree333", None), (5, 64, "wide-tree333", None), (64, 64, "wide-tree333", None),
    (257, 64, "wide-tree333", None), (100, 16, "35b-tree222", None), (70, 7, "35b-tree222", None),
    (130, 32, "wide-tree333", "f32")])
def test_prefill_against_oracle(T, chunk, cfg, dtype):
    B, H = 2, 3
    inp = synth.make_inputs(cfg, B=B, H=H, seed=500 + T, parent=synth.chain(T), dtype=dtype)
    dev = to_device(inp)
    print(f"case T={T} chunk={chunk} {cfg} {inp.dtype}", flush=True)
    S = dev["S0"].clone()
    out = abi.prefill_chain(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], chunk=chunk)
    torch.cuda.synchronize()
    G = B * H
    heads = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3)).reshape(G, T, 128)
    gates = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1)).reshape(G, T)
    w = oracle.walk(inp.S0.reshape(G, 128, 128).astype(np.float64),
                    heads(inp.q).astype(np.float64), heads(inp.k).astype(np.float64),
                    heads(inp.v).astype(np.float64), gates(inp.alpha).astype(np.float64),
                    gates(inp.beta).astype(np.float64), synth.chain(T))
    got_out = heads(out.cpu().numpy())
    _err(f"T={T} chunk={chunk} out", got_out, w.out)
    _err(f"T={T} chunk={chunk} state", S.cpu().numpy().reshape(G, 128, 128), w.states[:, -1])


def test_prefill_empty_sequence_leaves_state():
    inp = synth.make_inputs("35b-tree222", B=2, H=2, seed=9, parent=synth.chain(3))
    dev = to_device(inp)
    S = dev["S0"].clone()
    q = dev["q"][:, :0].contiguous()
    k, v = dev["k"][:, :0].contiguous(), dev["v"][:, :0].contiguous()
    a, b = dev["alpha"][:, :0].contiguous(), dev["beta"][:, :0].contiguous()
    out = abi.prefill_chain(S, q, k, v, a, b)
    torch.cuda.synchronize()
    assert out.shape[1] == 0 and torch.equal(S, dev["S0"])
