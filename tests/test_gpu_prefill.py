"""GPU parity of the two prefill entry points, through the C ABI, against
the fp64 oracle walking the whole chain token by token: every token's output
and the final state (2e-3).
- treewy_prefill_chain (chunked prefill through the commit-then-verify
  kernels): chunk sizes from 7 to 64 tokens, ragged last chunks, one token,
  fp32 and bf16 inputs;
- treewy_prefill (one launch, the state on chip): ragged sequence lengths
  around the 16-token chunk, both gate distributions, fp32 and bf16 inputs,
  agreement with the chunked form, and sampled heads at the full size of the
  batched prompt workload (256 sequences x 256 tokens x 32 heads)."""
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


# ---- treewy_prefill: one launch, the state on chip across chunks of 16 ----

def _walk_heads(inp, T):
    G = inp.B * inp.H
    heads = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3)).reshape(G, T, 128)
    gates = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1)).reshape(G, T)
    w = oracle.walk(inp.S0.reshape(G, 128, 128).astype(np.float64),
                    heads(inp.q).astype(np.float64), heads(inp.k).astype(np.float64),
                    heads(inp.v).astype(np.float64), gates(inp.alpha).astype(np.float64),
                    gates(inp.beta).astype(np.float64), synth.chain(T))
    return w, heads


# T covers one token, a short chunk, exactly one chunk, one chunk plus one
# token, several full chunks and a ragged tail; both gate distributions
@pytest.mark.parametrize("T,cfg,dtype", [
    (1, "35b-tree222", None), (5, "35b-tree222", None), (16, "35b-tree222", None),
    (17, "35b-tree222", None), (64, "wide-tree333", None), (100, "35b-tree222", None),
    (257, "wide-tree333", None), (37, "35b-tree222", "f32"), (130, "wide-tree333", "f32")])
def test_prefill_one_launch_against_oracle(T, cfg, dtype):
    B, H = 2, 3
    inp = synth.make_inputs(cfg, B=B, H=H, seed=700 + T, parent=synth.chain(T), dtype=dtype)
    dev = to_device(inp)
    print(f"case treewy_prefill T={T} {cfg} {inp.dtype}", flush=True)
    S = dev["S0"].clone()
    out = abi.prefill(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"])
    torch.cuda.synchronize()
    w, heads = _walk_heads(inp, T)
    _err(f"prefill T={T} out", heads(out.cpu().numpy()), w.out)
    _err(f"prefill T={T} state", S.cpu().numpy().reshape(B * H, 128, 128), w.states[:, -1])


# Every length of the last chunk, after one full chunk: the chunk tables are
# built in two 8 x 8 blocks, so lengths 1..8 leave the second block empty and
# 9..15 fill it in part; fp32 inputs at two of them
@pytest.mark.parametrize("tail,dtype", [(n, None) for n in range(1, 17)] + [(12, "f32"), (15, "f32")])
def test_prefill_one_launch_every_tail_length(tail, dtype):
    T = 16 + tail
    B, H = 2, 2
    inp = synth.make_inputs("35b-tree222", B=B, H=H, seed=900 + tail, parent=synth.chain(T), dtype=dtype)
    dev = to_device(inp)
    print(f"case treewy_prefill T={T} (last chunk {tail}) {inp.dtype}", flush=True)
    S = dev["S0"].clone()
    out = abi.prefill(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"])
    torch.cuda.synchronize()
    w, heads = _walk_heads(inp, T)
    _err(f"prefill T={T} out", heads(out.cpu().numpy()), w.out)
    _err(f"prefill T={T} state", S.cpu().numpy().reshape(B * H, 128, 128), w.states[:, -1])


# The one-launch kernel keeps the state divided by a running decay and
# applies that decay to the state registers only when it leaves
# [2^-100, 2^100]: strong decay (a restart every other chunk), gates of exactly
# zero (the decay becomes 0 inside a chunk, at a chunk's last token and at a
# chunk's first), gates of exactly one (no decay at all), and one gate of
# 1e-35 (a restart forced by a single token)
@pytest.mark.parametrize("mode,dtype", [("strong", None), ("zero", None), ("one", None), ("tiny", None),
                                        ("strong", "f32"), ("zero", "f32"), ("tiny", "f32")])
def test_prefill_one_launch_decay_extremes(mode, dtype):
    T, B, H = 100, 2, 2
    inp = synth.make_inputs("35b-tree222", B=B, H=H, seed=1300, parent=synth.chain(T), dtype=dtype)
    a = inp.alpha.astype(np.float32)
    if mode == "strong":
        a = np.float32(0.02) + np.float32(0.1) * a
    elif mode == "zero":
        a[:, [7, 31, 47, 64], :] = 0.0
    elif mode == "one":
        a[:] = 1.0
    else:
        a[:, 20, :] = 1e-35
    if inp.dtype == "bf16":
        inp.bits["alpha"] = synth.bf16_bits(a)
        a = synth.bf16_to_f32(inp.bits["alpha"])
    inp.alpha = a.astype(np.float32)
    dev = to_device(inp)
    print(f"case treewy_prefill T={T} decay {mode} {inp.dtype}", flush=True)
    S = dev["S0"].clone()
    out = abi.prefill(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"])
    torch.cuda.synchronize()
    w, heads = _walk_heads(inp, T)
    _err(f"prefill decay {mode} out", heads(out.cpu().numpy()), w.out)
    _err(f"prefill decay {mode} state", S.cpu().numpy().reshape(B * H, 128, 128), w.states[:, -1])


# A long prompt, 64 chunks: rounding carried through many state updates.
# With the 35B-like workloads' gates (alpha in [0.09, 0.9]) the running decay
# is applied to the state registers about every 80 tokens; with the wide
# tree's long-memory gates (alpha in [0.9, 1)) never in 1024 tokens.
@pytest.mark.parametrize("cfg", ["35b-tree222", "wide-tree333"])
def test_prefill_one_launch_long_prompt(cfg):
    T, B, H = 1024, 1, 2
    inp = synth.make_inputs(cfg, B=B, H=H, seed=1400, parent=synth.chain(T))
    dev = to_device(inp)
    print(f"case treewy_prefill T={T} {cfg} gates", flush=True)
    S = dev["S0"].clone()
    out = abi.prefill(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"])
    torch.cuda.synchronize()
    w, heads = _walk_heads(inp, T)
    _err(f"prefill long {cfg} out", heads(out.cpu().numpy()), w.out)
    _err(f"prefill long {cfg} state", S.cpu().numpy().reshape(B * H, 128, 128), w.states[:, -1])


@pytest.mark.parametrize("T", [29, 40])
def test_prefill_one_launch_near_identical_keys(T):
    """A repeated token: the keys of a head are one unit vector plus 5% noise
    and beta is near 1, so the entries of A approach beta and the chunk
    tables are at their least benign (bf16 inputs, rounded as loaded)."""
    B, H = 2, 2
    inp = synth.make_inputs("35b-tree222", B=B, H=H, seed=950 + T, parent=synth.chain(T))
    rng = np.random.default_rng(951 + T)
    k0 = rng.standard_normal((B, 1, H, 128))
    k = k0 + 0.05 * rng.standard_normal((B, T, H, 128))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = 0.9 + 0.1 * rng.random((B, T, H))
    for name, arr in (("k", k), ("beta", beta)):
        bits = synth.bf16_bits(arr.astype(np.float32))
        inp.bits[name] = bits
        setattr(inp, name, synth.bf16_to_f32(bits))
    dev = to_device(inp)
    print(f"case treewy_prefill near-identical keys T={T}", flush=True)
    S = dev["S0"].clone()
    out = abi.prefill(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"])
    torch.cuda.synchronize()
    w, heads = _walk_heads(inp, T)
    _err(f"prefill near-identical keys T={T} out", heads(out.cpu().numpy()), w.out)
    _err(f"prefill near-identical keys T={T} state", S.cpu().numpy().reshape(B * H, 128, 128),
         w.states[:, -1])


@pytest.mark.parametrize("T", [33, 200])
def test_prefill_one_launch_matches_chunked(T):
    """Two different computations of the same result: the one-launch kernel
    (MFMA state update) and the chunked verify/commit composition."""
    inp = synth.make_inputs("35b-tree222", B=3, H=4, seed=800 + T, parent=synth.chain(T))
    dev = to_device(inp)
    print(f"case prefill vs prefill_chain T={T}", flush=True)
    S1, S2 = dev["S0"].clone(), dev["S0"].clone()
    o1 = abi.prefill(S1, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"])
    o2 = abi.prefill_chain(S2, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], chunk=16)
    torch.cuda.synchronize()
    for label, a, b in (("out", o1, o2), ("state", S1, S2)):
        e = rel_err(a.cpu().numpy(), b.cpu().numpy().astype(np.float64))
        print(f"T={T} {label}: {e:.2e}", flush=True)
        assert e <= 1e-4, f"{label}: {e:.3e}"


def test_prefill_one_launch_full_size_sampled():
    """The bench's prefill launch: 256 sequences x 256 tokens x 32 heads, bf16,
    long-memory gates; sampled (sequence, head) pairs against the oracle walk."""
    B, T, H = 256, 256, 32
    dev = torch.device("cuda:0")
    print(f"case treewy_prefill full size B={B} T={T} H={H}", flush=True)
    g = torch.Generator(device=dev).manual_seed(17)
    rnd = lambda *shape: torch.randn(shape, generator=g, device=dev)
    unit = lambda x: torch.nn.functional.normalize(x, dim=-1)
    q = unit(rnd(B, T, H, 128)).to(torch.bfloat16)
    k = unit(rnd(B, T, H, 128)).to(torch.bfloat16)
    v = rnd(B, T, H, 128).to(torch.bfloat16)
    a = (0.9 + 0.1 * torch.rand((B, T, H), generator=g, device=dev)).to(torch.bfloat16)
    b = torch.sigmoid(rnd(B, T, H)).to(torch.bfloat16)
    S0 = rnd(B, H, 128, 128) * 0.02
    S = S0.clone()
    out = abi.prefill(S, q, k, v, a, b)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    picks = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(4)]
    f64 = lambda x: x.float().cpu().numpy().astype(np.float64)
    for bb, hh in picks:
        w = oracle.walk(f64(S0[bb, hh])[None], f64(q[bb, :, hh])[None], f64(k[bb, :, hh])[None],
                        f64(v[bb, :, hh])[None], f64(a[bb, :, hh])[None], f64(b[bb, :, hh])[None],
                        synth.chain(T))
        _err(f"({bb},{hh}) out", out[bb, :, hh].cpu().numpy()[None], w.out)
        _err(f"({bb},{hh}) state", S[bb, hh].cpu().numpy()[None], w.states[:, -1])


def test_prefill_one_launch_empty_sequence():
    inp = synth.make_inputs("35b-tree222", B=2, H=2, seed=9, parent=synth.chain(3))
    dev = to_device(inp)
    S = dev["S0"].clone()
    cut = lambda x: x[:, :0].contiguous()
    out = abi.prefill(S, cut(dev["q"]), cut(dev["k"]), cut(dev["v"]), cut(dev["alpha"]),
                      cut(dev["beta"]))
    torch.cuda.synchronize()
    assert out.shape[1] == 0 and torch.equal(S, dev["S0"])


def test_prefill_one_launch_graph_replay_matches_eager():
    """treewy_prefill is one launch that allocates nothing: captured in a HIP
    graph, each replay (from the same starting state) equals the eager call
    bit for bit."""
    T = 45
    inp = synth.make_inputs("35b-tree222", B=4, H=4, seed=901, parent=synth.chain(T))
    dev = to_device(inp)
    S = dev["S0"].clone()
    out = torch.empty((inp.B, T, inp.H, 128), device="cuda")
    abi.prefill(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], out=out)
    torch.cuda.synchronize()
    eager = (out.clone(), S.clone())
    S.copy_(dev["S0"])
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            abi.prefill(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], out=out, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        S.copy_(dev["S0"])
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0]), f"replay {rep}: outputs differ"
        assert torch.equal(S, eager[1]), f"replay {rep}: state differs"
