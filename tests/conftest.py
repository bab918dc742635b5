import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def to_heads(S0, q, k, v, alpha, beta):
    """Device layout ([B,N,H,d] tokens, [B,H,d,d] state) -> one row per
    (sequence, head): S0 [G,dv,dk], q/k/v [G,N,d], alpha/beta [G,N]."""
    B, N, H, _ = q.shape
    G = B * H
    S = None if S0 is None else np.asarray(S0).reshape(G, S0.shape[2], S0.shape[3])
    tok = lambda x: np.ascontiguousarray(np.asarray(x).transpose(0, 2, 1, 3)).reshape(G, N, x.shape[-1])
    gate = lambda x: np.ascontiguousarray(np.asarray(x).transpose(0, 2, 1)).reshape(G, N)
    return S, tok(q), tok(k), tok(v), gate(alpha), gate(beta)


@pytest.fixture
def rng():
    return np.random.default_rng(1234)
